"""GPU parity of the one-launch decode (attn_decode_one_launch) and of the
whole-call entry point attn_decode against the float64 oracle.

attn_decode_one_launch is one launch of the split kernel in which the last
workgroup of each (sequence, KV head) to finish merges the group's partials
(Lecture 06 section 2's combine); for a shared latent it is a cooperative
launch whose workgroups meet at a grid barrier and then all merge. Every case runs with a workspace
whose partial rows are NaN beforehand (so the merge can only use partials
written in this launch) and checks that the completion counters are back at
zero afterwards, so the next call needs no preparation. Gates as for the
two-launch path.
"""

import itertools

import numpy as np
import pytest

import synthetic
from harness import (ABS_GATE, LSE_F32_ARITH, assert_parity, decode_call, oracle_out, run_gpu,
                     run_gpu_fused)
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


GROUPS = [1, 2, 4, 6, 8]
WIDTHS = [64, 128, 256]
STORAGE = ["f32", "f16", "bf16"]
LAYOUTS = ["contiguous", "paged"]


@pytest.mark.parametrize("G,D,kv,layout", list(itertools.product(GROUPS, WIDTHS, STORAGE, LAYOUTS)))
def test_every_variant_one_launch_matches_oracle(G, D, kv, layout):
    q_dtype = STORAGE[(G + D // 64 + 1) % 3]
    seed = 9000 + G * 100 + D + STORAGE.index(kv) * 7 + LAYOUTS.index(layout)
    case = synthetic.gqa_case(
        f"fused-G{G}-D{D}-{kv}-{layout}", seq_lens=[1000, 77, 1], num_q_heads=2 * G,
        num_kv_heads=2, head_dim=D, q_dtype=q_dtype, kv_dtype=kv, layout=layout, capacity=1040,
        seed=seed)
    ref, rlse = oracle_out(case)
    for S in (0, 7):
        out, lse, call = run_gpu_fused(case, n_splits=S)
        assert_parity(case, out, ref, label=f"G={G} D={D} {kv} {layout} plan={call.plan}")
        np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("L", [1, 33, 1000, 4096])
@pytest.mark.parametrize("S", [1, 3, 8, 0])
def test_tiny_gqa_one_launch(L, S):
    case = synthetic.tiny_gqa(L, seed=1000 + L, capacity=L + 7)
    out, lse, call = run_gpu_fused(case, n_splits=S)
    ref, rlse = oracle_out(case)
    assert_parity(case, out, ref, label=f"L={L} S={S} plan={call.plan}")
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-5)
    if L == 1:  # one position: its value row, bit for bit, whatever S
        v0 = case.v[0, 0, 0].astype(np.float32)
        for h in range(4):
            assert np.array_equal(out[0, h].astype(np.float32), v0)


def test_dominant_key_in_the_last_split_and_second_tile():
    L = 1000
    for jstar in (32, 999):
        case = synthetic.tiny_gqa(L, seed=jstar + 5)
        q = case.q[0, 0].astype(np.float64)
        case.q[0, :] = case.q[0, 0]
        case.k[0, jstar, 0] = (q / np.linalg.norm(q) * 8 * 70 / np.linalg.norm(q)).astype(np.float32)
        ref, _ = oracle_out(case)
        out, _, _ = run_gpu_fused(case, n_splits=3)
        assert_parity(case, out, ref, label=f"dominant at {jstar}")
        for h in range(4):
            np.testing.assert_allclose(out[0, h], case.v[0, jstar, 0], rtol=0, atol=1e-4)


@pytest.mark.parametrize("kv", ["f32", "f16"])
@pytest.mark.parametrize("L", [4096, 20480])
def test_nine_b_like_one_launch_full_outputs(kv, L):
    case = synthetic.qwen9b_like(L, kv, seed=2000 + L)
    out, lse, call = run_gpu_fused(case)
    ref, rlse = oracle_out(case)
    assert_parity(case, out, ref, label=f"9B-like {kv} L={L} plan={call.plan}")
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-4)
    free()


@pytest.mark.parametrize("kv,L", [("f32", 131072), ("f32", 262144), ("f16", 151552), ("f16", 262144)])
def test_nine_b_like_one_launch_long_context_sampled_heads(kv, L):
    """Full size with the heuristic plan, as the bench launches it; one query
    head of every KV group against the oracle, and the whole output against
    the two-launch path."""
    case = synthetic.qwen9b_like(L, kv, seed=2000 + L)
    t = to_device(case)
    call = decode_call(case, t)
    out, _, _ = run_gpu_fused(case, tensors=t, call=call)
    heads = [(0, 0), (0, 5), (0, 10), (0, 15)]
    ref, _ = oracle_out(case, heads=heads)
    assert_parity(case, out, ref, label=f"9B-like {kv} L={L} plan={call.plan}")
    two, _, _ = run_gpu(case, tensors=t, call=call)
    assert np.abs(out - two).max() <= ABS_GATE[kv] / 10
    del call, t
    free()


def test_wide_group_peaky_one_launch_heuristic_and_sweep():
    case = synthetic.wide_group_peaky(262144)
    t = to_device(case)
    heads = [(0, 0), (0, 7), (0, 13), (0, 23)]
    ref, _ = oracle_out(case, heads=heads)
    for S in (0, 64, 512):
        out, _, call = run_gpu_fused(case, n_splits=S, tensors=t)
        assert_parity(case, out, ref, label=f"peaky S={S} plan={call.plan}")
        del call
    del t
    free()


def test_ragged_paged_bf16_batch_one_launch():
    case = synthetic.ragged_paged()
    out, lse, call = run_gpu_fused(case)
    ref, rlse = oracle_out(case)
    assert_parity(case, out, ref, label=f"ragged plan={call.plan}")
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-4)
    free()


def test_repeated_calls_need_no_preparation_and_agree_with_two_launches():
    """Three calls in a row on one workspace (no re-initialisation), then a
    two-launch call, then a one-launch call again: the counters return to zero
    after every call and the one-launch results are identical bits."""
    import torch

    case = synthetic.gqa_case("repeat", seq_lens=[5000, 64, 1300, 4097], num_q_heads=16,
                              num_kv_heads=4, head_dim=128, kv_dtype="f16", capacity=5100, seed=77)
    t = to_device(case)
    call = decode_call(case, t, n_splits=11)
    first, _, _ = run_gpu_fused(case, tensors=t, call=call)
    for _ in range(2):
        call.out.fill_(float("nan"))
        call.decode_one_launch()
        torch.cuda.synchronize()
        assert int(call.counters().abs().sum().item()) == 0
        assert np.array_equal(call.out.double().cpu().numpy(), first)
    call()  # two launches on the same workspace
    torch.cuda.synchronize()
    two = call.out.double().cpu().numpy()
    call.out.fill_(float("nan"))
    call.decode_one_launch()
    torch.cuda.synchronize()
    assert np.array_equal(call.out.double().cpu().numpy(), first)
    ref, _ = oracle_out(case)
    assert_parity(case, first, ref)
    assert np.abs(first - two).max() <= ABS_GATE["f16"] / 100


def test_invalid_lengths_give_nan_for_that_sequence_only():
    import torch

    case = synthetic.gqa_case("bad", seq_lens=[50, 40, 30, 20], num_q_heads=8, num_kv_heads=2,
                              head_dim=64, capacity=64, seed=3)
    t = to_device(case)
    call = decode_call(case, t, n_splits=2)
    # 0, beyond the capacity, and beyond n_splits*chunk (2*25 = 50 < 60 <= 64)
    t["seq_lens"].copy_(torch.tensor([50, 0, 100, 60], dtype=torch.int32))
    call.workspace.fill_(0xFF)
    call.init_workspace()
    call.decode_one_launch()
    torch.cuda.synchronize()
    out, lse = call.out.cpu().numpy(), call.lse.cpu().numpy()
    for b in (1, 2, 3):
        assert np.all(np.isnan(out[b])) and np.all(np.isnan(lse[b]))
    assert int(call.counters().abs().sum().item()) == 0
    case.seq_lens = np.array([50, 40, 30, 20], dtype=np.int32)
    ref, _ = oracle_out(case)
    assert np.abs(out[0] - ref[0]).max() <= 1e-4


def test_without_lse():
    import torch

    case = synthetic.tiny_gqa(1000, seed=12)
    t = to_device(case)
    call = decode_call(case, t, n_splits=5)
    call.lse.fill_(-7.0)
    call.decode_one_launch(with_lse=False)
    torch.cuda.synchronize()
    assert torch.all(call.lse == -7.0)
    ref, _ = oracle_out(case)
    assert_parity(case, call.out.double().cpu().numpy(), ref)


def test_whole_call_entry_point_equals_the_two_launches():
    """attn_decode is the split kernel then the combine kernel: the same bits
    as calling the two entry points, for GQA and for both latent types."""
    import torch

    cases = [synthetic.qwen9b_like(4096, "f16", seed=61),
             synthetic.latent_case("lat-f32", seq_len=3000, kv_dtype="f32", capacity=3005, seed=51,
                                   scale=1 / 24),
             synthetic.latent_case("lat-f16", seq_len=3000, kv_dtype="f16", capacity=3005, seed=52,
                                   scale=1 / 24)]
    for case in cases:
        t = to_device(case)
        call = decode_call(case, t)
        two, two_lse, _ = run_gpu(case, tensors=t, call=call)
        call.workspace.fill_(0xFF)
        call.out.fill_(float("nan"))
        call.decode()
        torch.cuda.synchronize()
        assert np.array_equal(call.out.double().cpu().numpy(), two), case.name
        assert np.array_equal(call.lse.double().cpu().numpy(), two_lse), case.name
        ref, _ = oracle_out(case)
        assert_parity(case, two, ref, tight=(case.kv_dtype == "f32"), label=case.name)


# ------------------------------------------------------------ shared latent
# One cooperative launch: each workgroup writes its partial, all meet at a grid
# barrier, then every workgroup merges a share of the (sequence, head) rows.


def _latent_one_launch_twice(case, t, call):
    """One-launch result on a poisoned workspace, then a second call on the
    same workspace: identical bits, counters back at zero."""
    import torch

    out, lse, _ = run_gpu_fused(case, tensors=t, call=call)
    call.out.fill_(float("nan"))
    call.decode_one_launch()
    torch.cuda.synchronize()
    assert np.array_equal(call.out.double().cpu().numpy(), out, equal_nan=True)
    assert int(call.counters().abs().sum().item()) == 0
    return out, lse


@pytest.mark.parametrize("kv", ["f32", "f16"])
@pytest.mark.parametrize("L", [64, 8192])
def test_latent_one_launch_matches_oracle(kv, L):
    """96 heads, heuristic plan (as the bench launches it)."""
    case = synthetic.latent_decode(L, kv, seed=3000 + L)
    t = to_device(case)
    call = decode_call(case, t)
    out, lse = _latent_one_launch_twice(case, t, call)
    ref, rlse = oracle_out(case)
    assert_parity(case, out, ref, tight=(kv == "f32"), label=f"latent one-launch {kv} L={L} plan={call.plan}")
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=ABS_GATE[kv])
    two, _, _ = run_gpu(case, tensors=t, call=call)
    assert np.abs(out - two).max() <= ABS_GATE[kv] / 10
    del call, t
    free()


@pytest.mark.parametrize("kv", ["f32", "f16"])
def test_latent_one_launch_full_size_sampled_heads(kv):
    """131,072 positions with the heuristic plan (256 resident workgroups):
    three heads against the oracle, every head against the two-launch path."""
    case = synthetic.latent_decode(131072, kv, seed=3000 + 131072)
    t = to_device(case)
    call = decode_call(case, t)
    out, _ = _latent_one_launch_twice(case, t, call)
    heads = [(0, 0), (0, 47), (0, 95)]
    ref, _ = oracle_out(case, heads=heads)
    assert_parity(case, out, ref, tight=(kv == "f32"), label=f"latent one-launch {kv} plan={call.plan}")
    two, _, _ = run_gpu(case, tensors=t, call=call)
    assert np.abs(out - two).max() <= ABS_GATE[kv] / 10
    del call, t
    free()


@pytest.mark.parametrize("kv", ["f32", "f16"])
@pytest.mark.parametrize("hq", [32, 64, 128])
def test_latent_one_launch_head_counts_and_empty_splits(kv, hq):
    """Other head counts, with an explicit plan over a 3,005-row capacity for
    a 1,500-row sequence: half the splits are empty (their workgroups write
    nothing but still meet at the barrier and merge)."""
    case = synthetic.latent_case(f"lat1l-{hq}-{kv}", seq_len=1500, kv_dtype=kv, num_q_heads=hq,
                                 capacity=3005, seed=54 + hq, scale=1 / 24)
    t = to_device(case)
    call = decode_call(case, t, n_splits=16)
    out, _ = _latent_one_launch_twice(case, t, call)
    ref, _ = oracle_out(case)
    assert_parity(case, out, ref, tight=(kv == "f32"), label=f"latent one-launch hq={hq} {kv}")
    del call, t
    free()


@pytest.mark.parametrize("kv", ["f32", "f16"])
def test_latent_one_launch_index_lists_and_invalid_lengths(kv):
    """Index lists (top-k rows of a pool) for a batch of three, one of them
    with a length past n_splits*chunk: NaN for that sequence only."""
    import torch

    case = synthetic.indexed_case(f"dsa-one-{kv}", pool_rows=6000, seq_lens=[2048, 700, 1500],
                                  num_q_heads=96, num_kv_heads=1, head_dim=576, kv_dtype=kv,
                                  latent_value_dim=512, seed=71, scale=1.0 / 24.0)
    t = to_device(case)
    call = decode_call(case, t, n_splits=8)
    out, _ = _latent_one_launch_twice(case, t, call)
    ref, _ = oracle_out(case)
    assert_parity(case, out, ref, tight=(kv == "f32"), label=f"indexed latent one-launch {kv}")
    t["seq_lens"].copy_(torch.tensor([2048, 0, 1500], dtype=torch.int32))
    call.out.fill_(0.0)
    call.decode_one_launch()
    torch.cuda.synchronize()
    got, lse = call.out.double().cpu().numpy(), call.lse.double().cpu().numpy()
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(lse[1]))
    assert np.array_equal(got[[0, 2]], out[[0, 2]])
    assert int(call.counters().abs().sum().item()) == 0
    del call, t
    free()


@pytest.mark.parametrize("kv,hq,hkv,D", [("f16", 24, 4, 256), ("bf16", 32, 4, 256),
                                         ("f16", 32, 8, 128), ("bf16", 8, 8, 64)])
def test_one_launch_on_query_tiles_repeats_and_isolates_invalid_lengths(kv, hq, hkv, D):
    # Descriptors whose decode runs on the query-tile kernel merge in that
    # kernel's grid. A second call without preparation (the kernel resets the
    # counters) gives the same bits, since the merge folds the splits in
    # order whichever workgroup performs it; lengths 0 and past the capacity
    # make those sequences NaN and leave the valid one untouched.
    import torch

    case = synthetic.gqa_case(f"qt-one-launch-{hq}x{hkv}-d{D}-{kv}", seq_lens=[3000, 1, 700],
                              num_q_heads=hq, num_kv_heads=hkv, head_dim=D, kv_dtype=kv,
                              capacity=3001, seed=9500 + D + hq)
    t = to_device(case)
    out1, lse1, call = run_gpu_fused(case, tensors=t)
    ref, rlse = oracle_out(case)
    assert_parity(case, out1, ref, label=case.name)
    # q and the weights in 16-bit parts keep f32 arithmetic: a one-position
    # sequence's lse is its score
    np.testing.assert_allclose(lse1, rlse, rtol=0, atol=LSE_F32_ARITH)
    call.decode_one_launch()
    torch.cuda.synchronize()
    assert np.array_equal(call.out.double().cpu().numpy(), out1)
    assert int(call.counters().abs().sum().item()) == 0
    t["seq_lens"].copy_(torch.tensor([3000, 0, 5000], dtype=torch.int32))
    call.decode_one_launch()
    torch.cuda.synchronize()
    out = call.out.double().cpu().numpy()
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[2]))
    assert np.array_equal(out[0], out1[0])
    assert int(call.counters().abs().sum().item()) == 0
