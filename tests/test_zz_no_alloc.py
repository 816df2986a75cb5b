"""attn_decode_no_alloc: the whole decode call with the partials in the
library's per-device scratch instead of a caller workspace, for callers that
cannot allocate.

On the GPU it must give attn_decode's result bit for bit (the same kernels and
plan on the same inputs) on two calls in a row, the second with a smaller
input, and meet the oracle gate. A plan whose partials exceed the scratch is
refused before any HIP call (checked without a GPU).
"""

import numpy as np
import pytest

import synthetic
from harness import assert_parity, decode_call, oracle_out
from synthetic.torch_io import to_device


def _desc_plan(n_splits):
    import split_kv_flash_amd.binding as B

    desc = B.SkDesc(batch=1, num_q_heads=96, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                    kv_shared=1, scale=1.0 / 24.0, q_dtype=B.SK_F32, kv_dtype=B.SK_F16,
                    layout=B.SK_KV_CONTIGUOUS, max_seq_len=131072, page_size=0,
                    max_pages_per_seq=0, num_pages=0, stride_seq=131072 * 576, stride_pos=576,
                    stride_head=0)
    return desc, B.SkPlan(n_splits=n_splits, chunk=-(-131072 // n_splits))


def test_no_alloc_refuses_partials_beyond_the_scratch_before_any_hip_call():
    # 96 heads x 512 splits x 514 floats = 101 MB > 64 MiB: refused with the
    # workspace status and a message naming the limit, with null buffers (a
    # HIP call or launch would fault or fail differently).
    import split_kv_flash_amd.binding as B

    desc, plan = _desc_plan(512)
    assert B.attn_decode_workspace_bytes(desc, plan) > B.SK_NO_ALLOC_SCRATCH_BYTES
    with pytest.raises(B.SplitKVError) as e:
        B.attn_decode_no_alloc(desc, plan, 1 << 20, 1 << 20, None, None, 1 << 20, 1 << 20, None, 0)
    assert e.value.status == B.SK_ERR_WORKSPACE_TOO_SMALL
    assert "static scratch holds 67108864" in e.value.message
    # Within the limit the same call moves on to the pointer checks (v must be NULL
    # for a shared latent, so a non-NULL v is refused), still before any HIP call.
    desc, plan = _desc_plan(256)
    assert B.attn_decode_workspace_bytes(desc, plan) <= B.SK_NO_ALLOC_SCRATCH_BYTES
    with pytest.raises(B.SplitKVError) as e:
        B.attn_decode_no_alloc(desc, plan, 1 << 20, 1 << 20, 1 << 20, None, 1 << 20, 1 << 20, None, 0)
    assert e.value.status == B.SK_ERR_INVALID_ARG


def _pair(kind):
    # (first, second) cases of one family; the second is smaller (fewer
    # sequences, shorter, fewer partials).
    if kind == "f32-gqa":
        mk = lambda name, lens, cap, seed: synthetic.gqa_case(
            name, seq_lens=lens, num_q_heads=16, num_kv_heads=4, head_dim=256, kv_dtype="f32",
            capacity=cap, seed=seed)
        return mk("no-alloc-f32-a", [20480, 4097, 33], 20480, 31), mk("no-alloc-f32-b", [900], 900, 32)
    if kind == "f16-query-tile":
        mk = lambda name, lens, cap, seed: synthetic.gqa_case(
            name, seq_lens=lens, num_q_heads=24, num_kv_heads=4, head_dim=256, kv_dtype="f16",
            capacity=cap, seed=seed)
        return mk("no-alloc-f16-a", [8192, 1, 700], 8192, 33), mk("no-alloc-f16-b", [300, 77], 300, 34)
    if kind == "bf16-paged":
        mk = lambda name, lens, seed: synthetic.gqa_case(
            name, seq_lens=lens, num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16",
            kv_dtype="bf16", layout="paged", seed=seed)
        return mk("no-alloc-paged-a", [3000, 1500, 17, 2048], 35), mk("no-alloc-paged-b", [500], 36)
    mk = lambda name, L, seed: synthetic.latent_case(name, seq_len=L, kv_dtype="f16", seed=seed,
                                                     scale=1.0 / 24.0)
    return mk("no-alloc-latent-a", 8192, 37), mk("no-alloc-latent-b", 300, 38)


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["f32-gqa", "f16-query-tile", "bf16-paged", "latent-f16"])
def test_no_alloc_matches_attn_decode_on_two_calls(kind):
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    for case in _pair(kind):
        t = to_device(case)
        call = decode_call(case, t)
        call.workspace.view(torch.uint8).fill_(0xFF)
        ref_out, ref_lse = call()
        ref_out, ref_lse = ref_out.clone(), ref_lse.clone()
        call.out.fill_(float("nan"))
        call.lse.fill_(float("nan"))
        call.decode_no_alloc()
        torch.cuda.synchronize()
        out, lse = call.out.double().cpu().numpy(), call.lse.double().cpu().numpy()
        assert np.array_equal(out, ref_out.double().cpu().numpy()), f"{case.name}: out differs"
        assert np.array_equal(lse, ref_lse.double().cpu().numpy()), f"{case.name}: lse differs"
        ref, _ = oracle_out(case)
        assert_parity(case, out, ref, label=case.name, tight=case.kv_shared == 0)
