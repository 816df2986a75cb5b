"""GPU parity of the split + combine path against the float64 oracle.

Every call goes through the C ABI (libsplitkv.so) with a workspace filled with
NaN first (so the combine can only read partials the split kernel wrote) and
with KV padding past each sequence's end filled with NaN (so an over-read
poisons the output). Gates: max |gpu - oracle| <= 1e-4 for f32 KV and 2e-3 for
f16/bf16 KV, plus a relative-L2 bound; the oracle reads the same stored values.
"""

import math

import numpy as np
import pytest

import oracle
import synthetic
from harness import (ABS_GATE, assert_parity, decode_call, errors, oracle_out, run_gpu, run_gpu_fused)
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


# --------------------------------------------------------------- tiny GQA


@pytest.mark.parametrize("L", [1, 33, 1000, 4096])
@pytest.mark.parametrize("S", [1, 3, 8, 0])
def test_tiny_gqa_matches_oracle(L, S):
    case = synthetic.tiny_gqa(L, seed=1000 + L, capacity=L + 7)  # NaN rows past the end
    out, lse, call = run_gpu(case, n_splits=S)
    ref, rlse = oracle_out(case)
    assert_parity(case, out, ref, label=f"L={L} S={S} plan={call.plan}")
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-5)


@pytest.mark.parametrize("S", [1, 3, 8])
def test_single_position_returns_its_value_row_bit_exactly(S):
    import torch

    case = synthetic.tiny_gqa(1, seed=7, capacity=9)
    out, lse, call = run_gpu(case, n_splits=S)
    v0 = case.v[0, 0, 0].astype(np.float32)
    for h in range(4):
        assert np.array_equal(out[0, h].astype(np.float32), v0)
    acc, m, l = (x.cpu() for x in call.partials())
    # Splits past the only position hold the neutral partial (m = -inf, l = 0).
    if S > 1:
        assert torch.all(torch.isneginf(m[0, :, 1:])) and torch.all(l[0, :, 1:] == 0)
        assert torch.all(acc[0, :, 1:] == 0)
    s0 = case.scale * (case.q[0].astype(np.float64) @ case.k[0, 0, 0].astype(np.float64))
    np.testing.assert_allclose(lse[0], s0, rtol=0, atol=1e-5)


@pytest.mark.parametrize("L", [33, 1000, 4096])
def test_equal_scores_give_the_mean_of_v(L):
    case = synthetic.tiny_gqa(L, seed=11)
    case.q[:] = 0.0
    out, _, _ = run_gpu(case, n_splits=3)
    mean = case.v[0, :L, 0].astype(np.float64).mean(axis=0)
    for h in range(4):
        assert np.abs(out[0, h] - mean).max() <= 1e-5


@pytest.mark.parametrize("jstar", [0, 32, 517, 999])
def test_one_dominant_score_returns_that_row(jstar):
    """Position 32 is the first row of the second 32-row tile; 517 sits in the
    middle split and 999 in the last one (S = 3)."""
    L = 1000
    case = synthetic.tiny_gqa(L, seed=jstar)
    q = case.q[0, 0].astype(np.float64)
    case.q[0, :] = case.q[0, 0]
    qn = q / np.linalg.norm(q)
    case.k[0, jstar, 0] = (qn * 8 * 70 / np.linalg.norm(q)).astype(np.float32)  # score ~ 70
    ref, _ = oracle_out(case)
    out, _, _ = run_gpu(case, n_splits=3)
    assert_parity(case, out, ref, label=f"dominant at {jstar}")
    for h in range(4):
        np.testing.assert_allclose(out[0, h], case.v[0, jstar, 0], rtol=0, atol=1e-4)


def test_tile_boundary_length_33_with_the_max_in_the_second_tile():
    case = synthetic.tiny_gqa(33, seed=5)
    q = case.q[0, 0].astype(np.float64)
    case.k[0, 32, 0] = (q / np.linalg.norm(q) * 8 * 6 / np.linalg.norm(q)).astype(np.float32)
    ref, _ = oracle_out(case)
    for S in (1, 2, 0):
        out, _, _ = run_gpu(case, n_splits=S)
        assert_parity(case, out, ref, label=f"L=33 S={S}")


@pytest.mark.parametrize("L,S", [(65, 0), (4097, 0), (12289, 0), (12289, 333), (4097, 111), (1000, 27)])
def test_boundary_lengths_and_odd_chunks(L, S):
    """Lengths just past a multiple (65, 4097, 12289) and chunks that are not a
    multiple of the workgroup's row count (4097/111 -> 37 rows per split)."""
    case = synthetic.tiny_gqa(L, seed=L + S, capacity=L + 3)
    out, _, call = run_gpu(case, n_splits=S)
    ref, _ = oracle_out(case)
    assert_parity(case, out, ref, label=f"L={L} S={S} plan={call.plan}")


def test_split_partials_match_the_oracle_schedule():
    """The split kernel alone: every (head, split) partial (m, l, acc) against
    the oracle's schedule model with the same chunk."""
    for case, S in [(synthetic.tiny_gqa(1000, seed=3), 3),
                    (synthetic.qwen9b_like(4096, "f32", seed=4), 8),
                    (synthetic.qwen9b_like(4096, "f16", seed=5), 5)]:
        _, _, call = run_gpu(case, n_splits=S)
        acc, m, l = (x.double().cpu().numpy() for x in call.partials())
        rm, rl, racc = oracle.split_partials_f64(
            case.q, case.k_rows(), case.v_rows(), case.seq_lens, case.scale, call.plan.chunk,
            call.plan.n_splits, q_dtype=case.q_dtype, kv_dtype=case.kv_dtype)
        np.testing.assert_allclose(m, rm, rtol=0, atol=2e-5)
        np.testing.assert_allclose(l, rl, rtol=2e-5, atol=0)
        scale = np.abs(racc).max()
        assert np.abs(acc - racc).max() <= 2e-5 * scale


def test_combine_on_the_worked_merge_example():
    """Write the Lecture 07 worked-example partials straight into a workspace
    and combine them (1 head, 2 splits, every value column equal)."""
    import os

    import torch

    rows = []
    with open(os.path.join(os.path.dirname(__file__), "golden", "merge_worked_example.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([float(t) for t in line.split()])
    (m1, l1, a1), (m2, l2, a2) = rows
    case = synthetic.gqa_case("merge", seq_lens=[2], num_q_heads=1, num_kv_heads=1, head_dim=64, seed=0)
    t = to_device(case)
    call = decode_call(case, t, n_splits=2)
    assert (call.plan.n_splits, call.plan.chunk) == (2, 1)
    call.workspace.fill_(0xFF)
    acc, m, l = call.partials()
    acc[0, 0, 0, :] = a1
    acc[0, 0, 1, :] = a2
    m[0, 0, :] = torch.tensor([m1, m2])
    l[0, 0, :] = torch.tensor([l1, l2])
    call.combine()
    torch.cuda.synchronize()
    # The same partials arise from 8 scores equal to 2 with values 0.5 and 6
    # scores equal to 3 with values 3; their full softmax is the expected merge.
    s = [m1] * int(l1) + [m2] * int(l2)
    vals = [a1 / l1] * int(l1) + [a2 / l2] * int(l2)
    w = [math.exp(x - max(s)) for x in s]
    want = math.fsum(wi * vi for wi, vi in zip(w, vals)) / math.fsum(w)
    want_lse = max(s) + math.log(math.fsum(w))
    np.testing.assert_allclose(call.out[0, 0].cpu().numpy(), want, rtol=1e-6, atol=0)
    assert abs(call.lse[0, 0].item() - want_lse) <= 2e-6


# ------------------------------------------------------------ 9B-like layer


@pytest.mark.parametrize("kv", ["f32", "f16"])
@pytest.mark.parametrize("L", [4096, 20480])
def test_nine_b_like_full_outputs(kv, L):
    case = synthetic.qwen9b_like(L, kv, seed=2000 + L)
    out, lse, call = run_gpu(case)
    ref, rlse = oracle_out(case)
    assert_parity(case, out, ref, label=f"9B-like {kv} L={L} plan={call.plan}")
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-4)
    free()


@pytest.mark.parametrize("kv", ["f32", "f16"])
@pytest.mark.parametrize("L", [61440, 151552, 262144])
def test_nine_b_like_long_context_sampled_heads(kv, L):
    """Full size, launched exactly as the bench launches it (heuristic plan);
    the oracle computes one query head of every KV group."""
    case = synthetic.qwen9b_like(L, kv, seed=2000 + L)
    out, _, call = run_gpu(case)
    heads = [(0, 0), (0, 5), (0, 10), (0, 15)]
    ref, _ = oracle_out(case, heads=heads)
    assert_parity(case, out, ref, label=f"9B-like {kv} L={L} plan={call.plan}")
    del call
    free()


def test_splitting_is_independent_of_S_and_does_not_lose_accuracy():
    """Lecture 06 section 2.1: split partials act like pairwise summation, so
    accuracy should not degrade with splitting."""
    case = synthetic.qwen9b_like(20480, "f32", seed=9)
    ref, _ = oracle_out(case)
    t = to_device(case)
    outs = {}
    for S in (0, 1, 3, 8, 64):
        out, _, _ = run_gpu(case, n_splits=S, tensors=t)
        assert_parity(case, out, ref, label=f"S={S}")
        outs[S] = out
    for a in outs:
        for b in outs:
            assert np.abs(outs[a] - outs[b]).max() <= 2 * ABS_GATE["f32"]
    rel_split = errors(outs[0], ref)[1]
    rel_one = errors(outs[1], ref)[1]
    assert rel_split <= 1.5 * rel_one, (rel_split, rel_one)


# --------------------------------------------------------------- ragged, paged


def test_ragged_paged_bf16_batch():
    case = synthetic.ragged_paged()
    out, lse, call = run_gpu(case)
    ref, rlse = oracle_out(case)
    assert_parity(case, out, ref, label=f"ragged plan={call.plan}")
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-4)
    free()


def test_paged_result_ignores_where_pages_live():
    """Moving every page to another pool slot and rewriting the table gives
    the same bits."""
    case = synthetic.gqa_case("pg", seq_lens=[300, 17, 1024, 1], num_q_heads=8, num_kv_heads=2,
                              head_dim=128, q_dtype="bf16", kv_dtype="bf16", layout="paged",
                              page_size=16, seed=21)
    out1, _, _ = run_gpu(case, n_splits=5)
    P = case.k.shape[0]
    perm = np.random.default_rng(1).permutation(P)
    inv = np.argsort(perm)
    case.k, case.v = case.k[perm].copy(), case.v[perm].copy()
    case.block_table = np.where(case.block_table >= 0, inv[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    out2, _, _ = run_gpu(case, n_splits=5)
    assert np.array_equal(out1, out2)
    ref, _ = oracle_out(case)
    assert_parity(case, out2, ref)


# ------------------------------------------------------------ 27B-like peaky


def test_wide_group_peaky_heuristic_and_sweep():
    case = synthetic.wide_group_peaky(262144)
    t = to_device(case)
    heads = [(0, 0), (0, 7), (0, 13), (0, 23)]
    ref, _ = oracle_out(case, heads=heads)
    for S in (0, 64, 128, 256, 512):
        out, _, call = run_gpu(case, n_splits=S, tensors=t)
        assert_parity(case, out, ref, label=f"peaky S={S} plan={call.plan}")
        del call
    del t
    free()


# ------------------------------------------------------------ contract checks


LDS_FAMILIES = {
    # GQA vector split kernel
    "9b-f32": lambda: synthetic.qwen9b_like(64, "f32", seed=1),
    "9b-f16": lambda: synthetic.qwen9b_like(64, "f16", seed=1),
    # decode on the query-tile kernel (wide f16 group, narrow bf16 heads)
    "27b-f16-query-tile": lambda: synthetic.gqa_case("lds-27b", seq_lens=[64], num_q_heads=24,
                                                     num_kv_heads=4, head_dim=256, kv_dtype="f16",
                                                     seed=1),
    "d64-bf16-query-tile": lambda: synthetic.gqa_case("lds-d64", seq_lens=[64], num_q_heads=8,
                                                      num_kv_heads=8, head_dim=64, kv_dtype="bf16",
                                                      seed=1),
    # paged bf16 (the ragged batch's geometry)
    "paged-bf16": lambda: synthetic.gqa_case("lds-paged", seq_lens=[64, 64], num_q_heads=32,
                                             num_kv_heads=8, head_dim=128, q_dtype="bf16",
                                             kv_dtype="bf16", layout="paged", seed=1),
    # shared-latent kernels (f32 caches as f16 parts, f16 caches)
    "latent-f32": lambda: synthetic.latent_case("lds-l32", seq_len=64, kv_dtype="f32", seed=1,
                                                scale=1.0 / 24.0),
    "latent-f16": lambda: synthetic.latent_case("lds-l16", seq_len=64, kv_dtype="f16", seed=1,
                                                scale=1.0 / 24.0),
}


@pytest.mark.parametrize("family", sorted(LDS_FAMILIES))
def test_lds_does_not_depend_on_context_length(family):
    """Lecture 06 section 2: shared memory is O(key width + tile), never
    O(context). For each kernel family the kernel a descriptor selects, from
    64 to 1,048,576 positions, uses at most 160 KB (one compute unit's LDS)
    and at most two static sizes (short contexts may select a variant with
    fewer rows or heads per workgroup), and the longest context uses exactly
    the LDS of 131,072 positions."""
    from split_kv_flash_amd import attn_decode_kernel_info, attn_decode_plan

    case = LDS_FAMILIES[family]()
    call = decode_call(case, to_device(case))
    seen = {}
    for L in (64, 4096, 131072, 262144, 1048576):
        call.desc.max_seq_len = L
        if call.desc.layout == 1:  # paged: the table row must cover L positions
            call.desc.max_pages_per_seq = -(-L // call.desc.page_size)
        plan = attn_decode_plan(call.desc, L, L * case.batch, 256, 0)
        info = attn_decode_kernel_info(call.desc, plan)
        assert info.block >= 64 and 0 < info.lds_bytes <= 160 * 1024, (L, info.lds_bytes)
        seen[L] = info.lds_bytes
    assert len(set(seen.values())) <= 2, seen
    assert seen[1048576] == seen[131072] == seen[262144], seen


@pytest.mark.parametrize("kv", ["f32", "f16"])  # f16 at width 64 runs on the query-tile kernel
def test_invalid_lengths_give_nan_for_that_sequence_only(kv):
    import torch

    case = synthetic.gqa_case("bad", seq_lens=[50, 40, 30], num_q_heads=8, num_kv_heads=2,
                              head_dim=64, capacity=64, seed=3, kv_dtype=kv)
    t = to_device(case)
    call = decode_call(case, t, n_splits=2)
    t["seq_lens"].copy_(torch.tensor([50, 0, 100], dtype=torch.int32))  # 0 and > capacity
    call.workspace.fill_(0xFF)
    call()
    torch.cuda.synchronize()
    out = call.out.cpu().numpy()
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[2]))
    case.seq_lens = np.array([50, 40, 30], dtype=np.int32)
    ref, _ = oracle_out(case)
    assert np.abs(out[0] - ref[0]).max() <= 1e-4


# ------------------------------------------------------------ shared latent


@pytest.mark.parametrize("kv", ["f32", "f16"])
@pytest.mark.parametrize("L", [64, 8192, 131072])
def test_latent_matches_oracle(kv, L):
    """96 heads on one 576-column latent, values = first 512 columns, launched
    as the bench launches it (heuristic plan)."""
    case = synthetic.latent_decode(L, kv, seed=3000 + L)
    out, lse, call = run_gpu(case)
    ref, rlse = oracle_out(case)
    assert_parity(case, out, ref, tight=(kv == "f32"), label=f"latent {kv} L={L} plan={call.plan}")
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=ABS_GATE[kv])
    del call
    free()


def _latent_batch(name, lens, cap, hq, seed):
    """Sequences of one latent geometry stacked into a batch (f16 cache, NaN
    rows past each length)."""
    import dataclasses

    parts = [synthetic.latent_case(f"{name}-{i}", seq_len=L, kv_dtype="f16", num_q_heads=hq,
                                   capacity=cap, seed=seed + i, scale=1.0 / 24.0)
             for i, L in enumerate(lens)]
    return dataclasses.replace(parts[0], name=name, batch=len(lens),
                               q=np.concatenate([p.q for p in parts]),
                               k=np.concatenate([p.k for p in parts]),
                               seq_lens=np.asarray(lens, dtype=np.int32))


@pytest.mark.parametrize("hq", [64, 96])
@pytest.mark.parametrize("lens,S", [((4097,), 130), ((20000,), 150), ((5000, 300), 129),
                                    ((33, 2000), 200)])
def test_latent_f16_dedicated_role_kernel(hq, lens, S):
    """64 and 96 f16 heads with more than 128 (split, sequence) pairs run the
    dedicated-role kernel (8 waves of 512 threads; hq/32 scoring waves of 32
    heads, the other waves own the value columns and multiply all blocks'
    weights; four tile buffers; the query staged through the tile buffers):
    one-tile slices with a one-row tail (4097 at S = 130), slices of
    134 rows (four tiles and a 6-row tail), a batch of two whose short
    sequence leaves empty slices, and a batch whose first sequence has fewer
    rows than one tile. NaN rows past every length."""
    from split_kv_flash_amd import attn_decode_kernel_info

    case = _latent_batch(f"lat16d-{hq}-{'-'.join(map(str, lens))}", list(lens), max(lens) + 7, hq,
                         seed=7700 + hq + S)
    out, lse, call = run_gpu(case, n_splits=S)
    info = attn_decode_kernel_info(call.desc, call.plan)
    assert info.block == 512 and (info.grid_x, info.grid_z) == (S, 1), (info.block, info.grid_x)
    ref, rlse = oracle_out(case)
    assert_parity(case, out, ref, tight=False, label=f"{case.name} S={S}")
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=ABS_GATE["f16"])
    free()


def test_latent_f16_dedicated_role_kernel_dominant_key_in_second_tile():
    """Position 32, the first row of the first slice's second tile, holds a
    key that dominates every head's scores: each head returns that row's
    values, so a slip in a block's scores, in the published weights, in the
    output waves' column blocks or in the tile buffers' rotation shows."""
    L, S = 8300, 129  # chunk 65: slice 0 is tiles [0, 32), [32, 64), [64, 65)
    case = synthetic.latent_case("lat16d-dom", seq_len=L, kv_dtype="f32", seed=19, scale=1 / 24)
    q = case.q[0, 0].astype(np.float64)
    case.q[0, :] = case.q[0, 0]
    row = q / np.linalg.norm(q) * 24 * 30 / np.linalg.norm(q)  # score ~ 30
    case.k[0, 32, 0] = row.astype(np.float32)
    case.k = case.k.astype(np.float16)
    case.kv_dtype = "f16"
    out, _, call = run_gpu(case, n_splits=S)
    ref, _ = oracle_out(case)
    assert_parity(case, out, ref, tight=False, label="latent f16 dominant, dedicated roles")
    for h in (0, 17, 50, 95):
        np.testing.assert_allclose(out[0, h], ref[0, h], rtol=0, atol=ABS_GATE["f16"])


@pytest.mark.parametrize("kv", ["f32", "f16"])
@pytest.mark.parametrize("L,S", [(1, 1), (1, 8), (33, 2), (1000, 3), (1000, 7)])
def test_latent_explicit_splits_and_padding(kv, L, S):
    case = synthetic.latent_case(f"lat-{kv}-{L}", seq_len=L, kv_dtype=kv, capacity=L + 5,
                                 seed=L * 10 + S, scale=1 / 24)
    out, _, call = run_gpu(case, n_splits=S)
    ref, _ = oracle_out(case)
    assert_parity(case, out, ref, tight=(kv == "f32"), label=f"latent {kv} L={L} S={S}")
    if L == 1:
        # One position: the output is its value row. f16 values are used as
        # stored (exact); f32 values enter the products as two f16 parts,
        # 22 significant bits (within 2^-22 |v| + 2^-36).
        v0 = case.k[0, 0, 0, :512].astype(np.float32)
        for h in range(case.num_q_heads):
            o = out[0, h].astype(np.float32)
            if kv == "f16":
                assert np.array_equal(o, v0)
            else:
                assert np.all(np.abs(o.astype(np.float64) - v0) <= 2.0**-22 * np.abs(v0) + 2.0**-36 + 2.0**-24 * np.abs(v0))


@pytest.mark.parametrize("where", ["cache", "query"])
def test_latent_f32_operands_beyond_f16_range_give_nan(where):
    # An f32 latent cache enters the products as f16 parts: a cache entry or a
    # scaled query value of magnitude 65,520 or more has an infinite hi part
    # and the opposite infinity as lo part, so the outputs of the heads whose
    # products it enters come out NaN (every head for a cache entry, its own
    # head for a query value), as the header says. Values just inside the
    # range stay finite and in parity.
    case = synthetic.latent_case("lat-f32-range", seq_len=100, kv_dtype="f32", capacity=104,
                                 seed=77, scale=1 / 24)
    if where == "cache":
        case.k[0, 40, 0, 7] = 1.0e5
    else:
        case.q[0, 5, 100] = 1.0e7  # times 1/24 log2(e): about 6e5
    for fused in (False, True):
        out, _, _ = (run_gpu_fused if fused else run_gpu)(case, n_splits=2)
        assert np.all(np.isnan(out[0] if where == "cache" else out[0, 5])), (where, fused)
        if where == "query":
            others = np.delete(out[0], 5, axis=0)
            assert np.all(np.isfinite(others)), (where, fused)
    case = synthetic.latent_case("lat-f32-edge", seq_len=100, kv_dtype="f32", capacity=104,
                                 seed=78, scale=1 / 24)
    case.k[0, 40, 0, 7] = 60000.0
    out, _, _ = run_gpu(case, n_splits=2)
    ref, _ = oracle_out(case)
    assert np.all(np.isfinite(out))
    _, er, _ = errors(out, ref)  # outputs near 6e4: a relative gate
    assert er <= 1e-5, er


@pytest.mark.parametrize("kv", ["f32", "f16"])
def test_latent_dominant_key_in_the_second_tile(kv):
    """Position 32 is the first row of the second f16 tile (third f32 tile)."""
    L = 40
    case = synthetic.latent_case("lat-dom", seq_len=L, kv_dtype="f32", seed=9, scale=1 / 24)
    q = case.q[0, 0].astype(np.float64)
    case.q[0, :] = case.q[0, 0]
    row = (q / np.linalg.norm(q) * 24 * 30 / np.linalg.norm(q))  # score ~ 30
    case.k[0, 32, 0] = row.astype(np.float32)
    if kv == "f16":
        case.k = case.k.astype(np.float16)
        case.kv_dtype = "f16"
    ref, _ = oracle_out(case)
    out, _, _ = run_gpu(case, n_splits=1)
    assert_parity(case, out, ref, tight=False, label=f"latent dominant {kv}")
    for h in (0, 50, 95):
        np.testing.assert_allclose(out[0, h], ref[0, h], rtol=0, atol=ABS_GATE[kv])


@pytest.mark.parametrize("kv", ["f32", "f16"])
def test_latent_split_partials_match_the_oracle_schedule(kv):
    case = synthetic.latent_decode(1000, kv, seed=31)
    _, _, call = run_gpu(case, n_splits=4)
    acc, m, l = (x.double().cpu().numpy() for x in call.partials())
    rm, rl, racc = oracle.split_partials_f64(
        case.q, case.k_rows(), None, case.seq_lens, case.scale, call.plan.chunk,
        call.plan.n_splits, q_dtype=case.q_dtype, kv_dtype=case.kv_dtype, v_cols=512)
    tol = 2e-5 if kv == "f32" else 2e-3
    # m is the slice maximum, or (where a kernel moves it lazily) at most 8 ln 2
    # below it; l and acc are taken against that m, so the slice's log-sum-exp
    # m + ln l and its normalised output acc / l are fixed whatever m is.
    assert np.all(m <= rm + tol) and np.all(m >= rm - 8 * np.log(2) - tol)
    np.testing.assert_allclose(m + np.log(l), rm + np.log(rl), rtol=0, atol=tol)
    assert np.abs(acc / l[..., None] - racc / rl[..., None]).max() <= tol
