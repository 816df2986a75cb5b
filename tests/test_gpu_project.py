"""GPU parity of the combine with the per-head output projection
(attn_decode_combine_project) against the float64 oracle.

Lecture 06 section 2: the value up-projection wv_b needs the merged latent, so
it runs in the combine, after the merge. The oracle is project_heads_f64 over
the definition's output (float64); the weights are seeded N(0,1)/sqrt(Dv)
matrices, so the projected outputs are unit-scale like the attention outputs
and the same gates apply (max abs 1e-4 for f32 KV, 2e-3 for f16/bf16 KV).
"""

import numpy as np
import pytest

import oracle
import synthetic
from harness import ABS_GATE, REL_L2_GATE, decode_call, errors, oracle_out
from synthetic.torch_io import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import split_kv_flash_amd.binding as B

    B.lib()  # fail loudly if the HIP library is missing


def weights_tensor(w, w_dtype):
    import torch

    if w_dtype == "bf16":
        return torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(w).cuda()


def run_project(case, w, w_dtype, *, n_splits=0, tensors=None):
    """Split kernel, then the combine-project kernel, with NaN-filled workspace
    and outputs beforehand. Returns (y, lse, plain combine out, call)."""
    import torch

    t = to_device(case) if tensors is None else tensors
    call = decode_call(case, t, n_splits=n_splits)
    call.workspace.fill_(0xFF)
    call.splitk()
    wt = weights_tensor(w, w_dtype)
    y = torch.full((case.batch, case.num_q_heads, w.shape[1]), float("nan"), device="cuda")
    call.lse.fill_(float("nan"))
    call.combine_project(wt, y)
    torch.cuda.synchronize()
    lse = call.lse.double().cpu().numpy()
    call.combine()
    torch.cuda.synchronize()
    return y.double().cpu().numpy(), lse, call.out.double().cpu().numpy(), call


def check(case, y, w, w_dtype, label):
    ref, rlse = oracle_out(case)
    want = oracle.project_heads_f64(ref, w, w_dtype)
    assert np.all(np.isfinite(y)), f"{label}: non-finite"
    ea, er, _ = errors(y, want)
    assert ea <= ABS_GATE[case.kv_dtype], f"{label}: max abs err {ea:.3e}"
    assert er <= REL_L2_GATE[case.kv_dtype], f"{label}: relL2 {er:.3e}"
    return rlse


@pytest.mark.parametrize("kv", ["f32", "f16"])
@pytest.mark.parametrize("L", [64, 8192, 131072])
@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
def test_latent_combine_project_matches_oracle(kv, L, w_dtype):
    """96 heads, merged 512-column latent projected to 128 per head, with the
    heuristic plan the bench uses."""
    case = synthetic.latent_decode(L, kv, seed=3000 + L)
    w = synthetic.projection_weights(96, 128, 512, w_dtype, seed=6100 + L)
    y, lse, _, call = run_project(case, w, w_dtype)
    rlse = check(case, y, w, w_dtype, f"latent {kv} L={L} W {w_dtype} plan={call.plan}")
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=ABS_GATE[kv])
    del call


@pytest.mark.parametrize("L,S", [(1, 8), (33, 8), (1000, 7), (4097, 3)])
def test_latent_explicit_splits_with_empty_tails(L, S):
    case = synthetic.latent_case(f"proj-{L}", seq_len=L, kv_dtype="f32", capacity=L + 5,
                                 seed=L + S, scale=1 / 24)
    w = synthetic.projection_weights(96, 128, 512, "f16", seed=L)
    y, _, _, call = run_project(case, w, "f16", n_splits=S)
    check(case, y, w, "f16", f"latent L={L} S={S}")


def test_identity_projection_returns_the_merged_output():
    """W_h = I (P = Dv = 512): the projection returns the combine's output."""
    case = synthetic.latent_decode(8192, "f32", seed=77)
    w = np.broadcast_to(np.eye(512, dtype=np.float32), (96, 512, 512)).copy()
    y, _, plain, _ = run_project(case, w, "f32")
    assert np.abs(y - plain).max() <= 1e-6 * max(1.0, np.abs(plain).max())


@pytest.mark.parametrize("wd", ["f32", "f16", "bf16"])
def test_gqa_layer_per_head_projection(wd):
    """A GQA layer (16/4 heads, head_dim 256) with per-head 256 -> 64 matrices."""
    case = synthetic.qwen9b_like(4096, "f16", seed=88)
    w = synthetic.projection_weights(16, 64, 256, wd, seed=89)
    y, _, _, _ = run_project(case, w, wd)
    check(case, y, w, wd, f"gqa W {wd}")


def test_ragged_paged_batch_projection():
    """32 sequences of the ragged bf16 batch, per-head 128 -> 96 (bf16)."""
    case = synthetic.ragged_paged()
    w = synthetic.projection_weights(32, 96, 128, "bf16", seed=90)
    y, _, _, _ = run_project(case, w, "bf16")
    check(case, y, w, "bf16", "ragged")


def test_tiny_head_width_and_odd_row_count():
    case = synthetic.tiny_gqa(1000, seed=91, capacity=1003)
    w = synthetic.projection_weights(4, 37, 64, "f32", seed=92)
    y, _, _, _ = run_project(case, w, "f32", n_splits=3)
    check(case, y, w, "f32", "tiny D64 P37")


def test_invalid_length_gives_nan():
    import torch

    case = synthetic.gqa_case("bad", seq_lens=[50, 40], num_q_heads=8, num_kv_heads=2,
                              head_dim=64, capacity=64, seed=3)
    t = to_device(case)
    call = decode_call(case, t, n_splits=2)
    t["seq_lens"].copy_(torch.tensor([50, 0], dtype=torch.int32))
    call.splitk()
    w = synthetic.projection_weights(8, 16, 64, "f32", seed=4)
    y = torch.zeros(2, 8, 16, device="cuda")
    call.combine_project(weights_tensor(w, "f32"), y)
    torch.cuda.synchronize()
    yy = y.cpu().numpy()
    assert np.all(np.isnan(yy[1])) and np.all(np.isfinite(yy[0]))
    case.seq_lens = np.array([50, 40], dtype=np.int32)
    ref, _ = oracle_out(case)
    want = oracle.project_heads_f64(ref, w, "f32")
    assert np.abs(yy[0] - want[0]).max() <= 1e-4
