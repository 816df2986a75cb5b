"""GPU checks of the one-function Python entry ``split_kv_flash_amd.decode``:
it plans, sizes the workspace and runs ``attn_decode`` exactly as the
``DecodeCall`` wrapper does, so its output is the same bits, for GQA and for
the shared latent; a short workspace is refused before any launch."""

import pytest

import synthetic
from harness import oracle_out, assert_parity
from synthetic.torch_io import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import split_kv_flash_amd.binding as B

    B.lib()  # fail loudly if the HIP library is missing


@pytest.mark.parametrize("which", ["gqa-f16", "paged-bf16", "latent-f16"])
def test_decode_function_equals_the_call_object(which):
    import torch
    import split_kv_flash_amd as skf

    if which == "gqa-f16":
        case = synthetic.gqa_case("api-gqa", seq_lens=[3000, 17], num_q_heads=16, num_kv_heads=4,
                                  head_dim=256, kv_dtype="f16", capacity=3100, seed=501)
    elif which == "paged-bf16":
        case = synthetic.gqa_case("api-paged", seq_lens=[900, 33, 1], num_q_heads=8,
                                  num_kv_heads=2, head_dim=128, q_dtype="bf16", kv_dtype="bf16",
                                  layout="paged", capacity=1024, seed=502)
    else:
        case = synthetic.latent_case("api-lat", seq_len=2000, kv_dtype="f16", capacity=2048,
                                     seed=503, scale=1 / 24)
    t = to_device(case)
    vcols = case.head_dim_v if case.kv_shared else None
    call = skf.DecodeCall(t["q"], t["k"], t["v"], t["seq_lens"], case.seq_lens, scale=case.scale,
                          block_table=t["block_table"], page_size=case.page_size, v_cols=vcols)
    ref_out, ref_lse = (x.clone() for x in call.decode())
    out, lse = skf.decode(t["q"], t["k"], t["v"], seq_lens=t["seq_lens"], scale=case.scale,
                          block_table=t["block_table"], page_size=case.page_size, v_cols=vcols,
                          lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    ref, _ = oracle_out(case)
    assert_parity(case, out.double().cpu().numpy(), ref, tight=not case.kv_shared,
                  label=f"decode() {which}")
    # host lengths given, caller's buffers, no lse
    o2 = torch.empty_like(out)
    ws = torch.empty(call.ws_bytes, dtype=torch.uint8, device="cuda")
    r, no_lse = skf.decode(t["q"], t["k"], t["v"], seq_lens=t["seq_lens"], scale=case.scale,
                           block_table=t["block_table"], page_size=case.page_size, v_cols=vcols,
                           host_seq_lens=case.seq_lens, out=o2, workspace=ws)
    torch.cuda.synchronize()
    assert r is o2 and no_lse is None and torch.equal(o2, ref_out)


def test_decode_function_refuses_a_short_workspace():
    import torch
    import split_kv_flash_amd as skf
    from split_kv_flash_amd.binding import SK_ERR_WORKSPACE_TOO_SMALL

    case = synthetic.tiny_gqa(1000)
    t = to_device(case)
    with pytest.raises(skf.SplitKVError) as e:
        skf.decode(t["q"], t["k"], t["v"], seq_lens=t["seq_lens"], scale=case.scale,
                   workspace=torch.empty(64, dtype=torch.uint8, device="cuda"))
    assert e.value.status == SK_ERR_WORKSPACE_TOO_SMALL
