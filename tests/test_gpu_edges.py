"""Edge cases at the limits: a million-position context, a large ragged batch
of short sequences, and split counts beyond what one combine pass covers.

At a million positions the float64 oracle would need the whole cache widened
(17 GB), so those cases use closed forms the definition fixes exactly: with
q = 0 every score is equal and the output is the mean of the value rows; with
one key made dominant the output is that key's value row.
"""

import numpy as np
import pytest

import synthetic
from harness import assert_parity, oracle_out, run_gpu, run_gpu_fused
from synthetic.torch_io import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import split_kv_flash_amd.binding as B

    B.lib()  # fail loudly if the HIP library is missing


def free():
    import torch

    torch.cuda.synchronize()
    torch.cuda.empty_cache()


MILLION = 1 << 20


def test_million_positions_equal_scores_give_the_mean_of_v():
    """9B-like layer (16/4 heads, head_dim 256, f16 KV) at 1,048,576 positions
    with q = 0, launched with the heuristic plan (two launches and one)."""
    case = synthetic.qwen9b_like(MILLION, "f16", seed=12001)
    case.q[:] = 0.0
    t = to_device(case)
    mean = np.stack([case.v[0, :, g].astype(np.float64).mean(axis=0) for g in range(4)])
    want = np.repeat(mean, 4, axis=0)  # head h reads KV head h // 4
    out, _, call = run_gpu(case, tensors=t)
    assert call.plan.n_splits * call.plan.chunk >= MILLION
    assert np.abs(out[0] - want).max() <= 1e-5
    out1, _, _ = run_gpu_fused(case, tensors=t)
    assert np.abs(out1[0] - want).max() <= 1e-5
    del t, call
    free()


def test_million_positions_dominant_last_key_returns_its_row():
    case = synthetic.qwen9b_like(MILLION, "f16", seed=12002)
    j = MILLION - 1
    qd = case.q[0, 0].astype(np.float64)
    case.q[0, :] = case.q[0, 0]
    for g in range(4):  # every KV head's last key aligned with q (score ~ 60)
        case.k[0, j, g] = (qd / np.linalg.norm(qd) * 16 * 60 / np.linalg.norm(qd)).astype(np.float16)
    out, _, _ = run_gpu(case)
    for h in range(16):
        np.testing.assert_allclose(out[0, h], case.v[0, j, h // 4].astype(np.float64), rtol=0, atol=2e-3)
    free()


def test_million_position_latent_equal_scores():
    """96-head latent (f16 cache, 1.2 GB) at 1,048,576 positions, q = 0."""
    case = synthetic.latent_decode(MILLION, "f16", seed=12003)
    case.q[:] = 0.0
    out, _, call = run_gpu(case)
    mean = case.k[0, :, 0, :512].astype(np.float64).mean(axis=0)
    assert np.abs(out[0] - mean[None, :]).max() <= 1e-4
    free()


def test_large_ragged_paged_batch_of_short_sequences():
    """512 sequences of 1 to 2048 positions (bf16, 16-token pages, shuffled
    table): the serving shape with many short requests."""
    rng = np.random.default_rng(12004)
    lens = rng.integers(1, 2048, endpoint=True, size=512)
    case = synthetic.gqa_case("ragged512", seq_lens=lens.tolist(), num_q_heads=32, num_kv_heads=8,
                              head_dim=128, q_dtype="bf16", kv_dtype="bf16", layout="paged",
                              page_size=16, seed=12004)
    out, _, call = run_gpu(case)
    heads = [(b, h) for b in range(0, 512, 37) for h in (0, 13, 31)]
    ref, _ = oracle_out(case, heads=heads)
    mask = np.zeros(out.shape, dtype=bool)
    for b, h in heads:
        mask[b, h] = True
    got = np.where(mask, out, np.nan)
    assert_parity(case, got, ref, label=f"ragged512 plan={call.plan}")
    assert np.all(np.isfinite(out))
    free()


@pytest.mark.parametrize("B", [2, 64, 65])
def test_work_ordered_pairs_at_the_batch_limits(B):
    """Batches of 2 to 64 sequences start their (split, sequence) pairs in
    order of work (full slices, partial slices longest first, empty ones);
    65 sequences keep the grid's own order. Lengths give every kind of slice:
    whole chunks only, a partial last slice, one position, and sequences
    with empty slices. Both entry points, against the oracle on sampled
    heads of every sequence."""
    rng = np.random.default_rng(12010 + B)
    S = 5
    lens = rng.integers(1, 5 * 96, endpoint=True, size=B)
    lens[0] = 5 * 96           # every slice full (chunk 96)
    lens[1] = 1
    if B > 2:
        lens[2] = 96 * 2       # two full slices, three empty ones
    case = synthetic.gqa_case(f"wo{B}", seq_lens=lens.tolist(), num_q_heads=8, num_kv_heads=2,
                              head_dim=64, kv_dtype="f32", seed=12010 + B)
    out, lse, call = run_gpu(case, n_splits=S)
    assert (call.plan.n_splits, call.plan.chunk) == (S, 96)
    heads = [(b, h) for b in range(B) for h in (0, 5)]
    ref, rlse = oracle_out(case, heads=heads)
    mask = np.zeros(out.shape, dtype=bool)
    for b, h in heads:
        mask[b, h] = True
    assert_parity(case, np.where(mask, out, np.nan), ref, label=f"B={B}")
    out1, lse1, _ = run_gpu_fused(case, n_splits=S)
    assert_parity(case, np.where(mask, out1, np.nan), ref, label=f"B={B} one-launch")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(out1))
    free()


@pytest.mark.parametrize("S", [257, 1000, 4096])
def test_combine_with_many_splits(S):
    """Split counts beyond one 64-split pass and beyond the combine's four
    waves (every split holds positions: 100,000 / S >= 24)."""
    case = synthetic.tiny_gqa(100000, seed=12005 + S, capacity=100003)
    out, lse, call = run_gpu(case, n_splits=S)
    assert call.plan.n_splits == S
    ref, rlse = oracle_out(case)
    assert_parity(case, out, ref, label=f"S={S}")
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-4)
    out1, _, _ = run_gpu_fused(case, n_splits=S)
    assert_parity(case, out1, ref, label=f"S={S} one launch")
