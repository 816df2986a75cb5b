"""GPU parity of query-tile attention (attn_query_tiles: several query
positions per sequence, causal) against the float64 oracle.

Query t of a sequence of L positions sits at L - q_len + t and attends
positions [0, L - q_len + t] ("Decoder Block 6: Online Attention, the
Capstone"). K/V padding past each length is NaN, so an over-read poisons the
output; the workspace is NaN beforehand. Gates as for decode (max abs 2e-3
and relL2 1e-3 for 16-bit KV); q and the weights are split into 16-bit parts
(two f16 or three bf16), so both paths also meet the tight f32-arithmetic
bound.
"""

import itertools
import math

import numpy as np
import pytest

import oracle
import synthetic
from harness import ABS_GATE, LSE_F32_ARITH, REL_L2_F32_ARITH, REL_L2_GATE, errors
from synthetic.torch_io import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import split_kv_flash_amd.binding as B

    B.lib()  # fail loudly if the HIP library is missing


def run_qt(case, *, n_splits=0, tensors=None):
    import torch
    from split_kv_flash_amd import QueryTileCall

    t = to_device(case) if tensors is None else tensors
    call = QueryTileCall(t["q"], t["k"], t["v"], t["seq_lens"], case.seq_lens, scale=case.scale,
                         n_splits=n_splits)
    call.workspace.fill_(0xFF)
    call.out.fill_(float("nan"))
    call.lse.fill_(float("nan"))
    call()
    torch.cuda.synchronize()
    return call.out.double().cpu().numpy(), call.lse.double().cpu().numpy(), call


def ref_qt(case, heads=None):
    return oracle.attend_multiquery_f64(case.q, case.k, case.v, case.seq_lens, case.scale,
                                        q_dtype=case.q_dtype, kv_dtype=case.kv_dtype, heads=heads)


def check(case, out, ref, label, tight=True):
    mask = ~np.isnan(ref)
    assert np.all(np.isfinite(out[mask])), f"{label}: non-finite output"
    ea, er, _ = errors(out, ref)
    assert ea <= ABS_GATE[case.kv_dtype], f"{label}: max abs err {ea:.3e}"
    assert er <= REL_L2_GATE[case.kv_dtype], f"{label}: relL2 {er:.3e}"
    if tight:
        assert er <= REL_L2_F32_ARITH, f"{label}: relL2 {er:.3e} (hi/lo products)"


@pytest.mark.parametrize("L,Q", [(1, 1), (33, 1), (33, 33), (33, 5), (100, 40), (64, 64), (2, 3)])
@pytest.mark.parametrize("kv", ["f16", "bf16"])
def test_small_causal_cases(L, Q, kv):
    case = synthetic.multiquery_case(f"qt-{L}-{Q}", seq_lens=[L], q_len=Q, num_q_heads=4,
                                     num_kv_heads=1, head_dim=64, kv_dtype=kv, capacity=L + 5,
                                     seed=L * 100 + Q)
    ref, rlse = ref_qt(case)
    for S in (0, 1, 3):
        out, lse, call = run_qt(case, n_splits=S)
        check(case, out, ref, f"L={L} Q={Q} S={S} plan={call.plan}")
        m = ~np.isnan(rlse)
        np.testing.assert_allclose(lse[m], rlse[m], rtol=0, atol=1e-4)
        # queries that see no position (L < Q) give NaN
        assert np.all(np.isnan(out[np.isnan(ref)]))


def test_length_33_with_the_maximum_in_the_second_tile():
    """Position 32 opens the second 32-position tile and holds every row's
    dominant key: rows that see it must rescale what they gathered in tile 1."""
    case = synthetic.multiquery_case("qt33", seq_lens=[33], q_len=33, num_q_heads=4,
                                     num_kv_heads=1, head_dim=64, kv_dtype="f16", seed=3333)
    qd = case.q[0, 32, 0].astype(np.float64)
    case.q[0, :, :] = case.q[0, 32, 0]
    case.k[0, 32, 0] = (qd / np.linalg.norm(qd) * 8 * 6 / np.linalg.norm(qd)).astype(np.float16)
    ref, _ = ref_qt(case)
    out, _, _ = run_qt(case, n_splits=1)
    check(case, out, ref, "L=33 dominant at 32")


@pytest.mark.parametrize("Q,G,D,kv", [(4, 4, 256, "f16"), (2, 8, 128, "bf16"), (8, 4, 128, "f16"),
                                        (3, 4, 64, "bf16"), (1, 16, 256, "bf16")])
def test_head_width_split_with_a_late_dominant_key(Q, G, D, kv):
    """16 or 32 query rows per KV group: the waves of a row block share the
    head width, their partial scores summed in LDS. A key that dominates
    every row sits in the slice's third tile, so each row must rescale what
    it gathered before it (and the partial sums must agree across waves for
    the softmax to be consistent)."""
    L = 200
    case = synthetic.multiquery_case(f"qt-ds-Q{Q}-G{G}-D{D}", seq_lens=[L, 150], q_len=Q,
                                     num_q_heads=2 * G, num_kv_heads=2, head_dim=D, kv_dtype=kv,
                                     capacity=L + 8, seed=9100 + Q * 100 + D)
    qd = case.q[0, 0, 0].astype(np.float64)
    case.q[0, :, :] = case.q[0, 0, 0]
    dom = (qd / np.linalg.norm(qd) * 10 * math.sqrt(D) / np.linalg.norm(qd))
    case.k[0, 70, :] = synthetic.to_storage(dom.astype(np.float32), kv)
    ref, _ = ref_qt(case)
    for S in (1, 2):
        out, _, call = run_qt(case, n_splits=S)
        check(case, out, ref, f"Q={Q} G={G} D={D} {kv} S={S} plan={call.plan}")


@pytest.mark.parametrize("G,D,kv", list(itertools.product([1, 2, 4, 6, 8], [64, 128, 256], ["f16", "bf16"])))
def test_every_group_and_width(G, D, kv):
    q_dtype = ["f32", "f16", "bf16"][(G + D // 64) % 3]
    case = synthetic.multiquery_case(f"qt-G{G}-D{D}-{kv}", seq_lens=[300, 77], q_len=5,
                                     num_q_heads=2 * G, num_kv_heads=2, head_dim=D, kv_dtype=kv,
                                     q_dtype=q_dtype, capacity=310, seed=7700 + G * 10 + D)
    ref, _ = ref_qt(case)
    for S in (0, 4):
        out, _, call = run_qt(case, n_splits=S)
        check(case, out, ref, f"G={G} D={D} {kv} q={q_dtype} plan={call.plan}")


def test_one_query_equals_the_decode_path():
    case = synthetic.multiquery_case("qt1", seq_lens=[5000, 1200], q_len=1, num_q_heads=16,
                                     num_kv_heads=4, head_dim=128, kv_dtype="f16", seed=41)
    out, _, _ = run_qt(case)
    import torch
    from split_kv_flash_amd import DecodeCall

    t = to_device(case)
    dc = DecodeCall(t["q"][:, 0].contiguous(), t["k"], t["v"], t["seq_lens"], case.seq_lens,
                    scale=case.scale)
    dc()
    torch.cuda.synchronize()
    dec = dc.out.double().cpu().numpy()
    assert np.abs(out[:, 0] - dec).max() <= 1e-5


def test_causal_self_attention_block_2048():
    """Decoder Block 6's shape: 4 heads of 64, 2048 tokens, every position a
    query (q_len = L), checked on a sample of query positions."""
    case = synthetic.causal_block(2048, kv_dtype="f16", seed=8101)
    out, _, call = run_qt(case)
    ts = [0, 1, 31, 32, 33, 511, 1024, 2047]
    ref, _ = ref_qt(case, heads=[(0, t, h) for t in ts for h in range(4)])
    check(case, out[:, ts], ref[:, ts], f"causal block plan={call.plan}")


def test_speculative_verify_at_131072():
    case = synthetic.spec_verify(131072, 4, kv_dtype="f16")
    out, _, call = run_qt(case)
    heads = [(0, t, h) for t in range(4) for h in (0, 5, 10, 15)]
    ref, _ = ref_qt(case, heads=heads)
    check(case, out, ref, f"verify plan={call.plan}")
    import torch

    torch.cuda.empty_cache()


def test_chunked_prefill_512_of_8192_bf16():
    case = synthetic.chunked_prefill(8192, 512, kv_dtype="bf16")
    out, _, call = run_qt(case)
    heads = [(0, t, h) for t in (0, 100, 255, 256, 511) for h in (0, 7, 15)]
    ref, _ = ref_qt(case, heads=heads)
    check(case, out, ref, f"prefill plan={call.plan}")


def test_ragged_batch_and_invalid_length():
    import torch

    case = synthetic.multiquery_case("qt-rag", seq_lens=[900, 40, 3], q_len=8, num_q_heads=8,
                                     num_kv_heads=2, head_dim=128, kv_dtype="bf16", capacity=1000,
                                     seed=42)
    t = to_device(case)
    out, _, call = run_qt(case, n_splits=3, tensors=t)
    ref, _ = ref_qt(case)
    check(case, out, ref, "ragged")
    t["seq_lens"][1] = 5000  # beyond the capacity: that sequence's outputs are NaN
    call.workspace.fill_(0xFF)
    call()
    torch.cuda.synchronize()
    o2 = call.out.double().cpu().numpy()
    assert np.all(np.isnan(o2[1]))
    assert np.array_equal(o2[0], out[0])


@pytest.mark.parametrize("kv", ["f16", "bf16"])
@pytest.mark.parametrize("hq,hkv,D", [(24, 4, 256), (32, 8, 128), (8, 8, 64)])
def test_routed_decode_scores_keep_f32_accuracy(hq, hkv, D, kv):
    # 256 one-position sequences: each lse is that head's score, so this
    # measures the score products alone, over 2,048-8,192 scores. q in 16-bit
    # parts (two f16, the second scaled by 2^11, or three bf16) carries 22-24
    # bits, so the error is f32 rounding: about 1e-7, and below 1e-6 for every
    # score (scores reach about 5 here, where an f32 step is 4.8e-7).
    case = synthetic.gqa_case(f"scores-{hq}x{hkv}-d{D}-{kv}", seq_lens=[1] * 256,
                              num_q_heads=hq, num_kv_heads=hkv, head_dim=D, kv_dtype=kv,
                              capacity=1, seed=777 + D)
    from harness import oracle_out, run_gpu

    _, lse, _ = run_gpu(case)
    _, rlse = oracle_out(case)
    err = np.abs(lse - rlse)
    assert err.max() <= 1e-6, f"max score error {err.max():.3e} (median {np.median(err):.2e})"
    assert np.median(err) <= 2e-7, f"median score error {np.median(err):.3e}"


@pytest.mark.parametrize("kv", ["f16", "bf16"])
@pytest.mark.parametrize("hq,hkv,D", [(24, 4, 256), (32, 4, 256), (32, 8, 128), (8, 8, 64), (48, 8, 64)])
def test_decode_on_query_tiles_is_the_one_query_call(hq, hkv, D, kv):
    # 16-bit groups that single-query decode runs on the query-tile kernel:
    # attn_decode's output and lse equal those of attn_query_tiles with one
    # query bit for bit (same plan, kernel and combine), the kernel report
    # names that kernel (its LDS holds the 4-buffer K/V ring), and the result
    # meets the oracle with the f32-arithmetic bound. Lengths: ragged, one
    # position, and a tail that is not a multiple of the 32-position tile.
    import split_kv_flash_amd.binding as B
    from harness import assert_parity, oracle_out, run_gpu

    case = synthetic.gqa_case(f"routed-{hq}x{hkv}-d{D}-{kv}", seq_lens=[5000, 1, 70, 4097],
                              num_q_heads=hq, num_kv_heads=hkv, head_dim=D, kv_dtype=kv,
                              seed=9100 + D + hq)
    t = to_device(case)
    out, lse, call = run_gpu(case, tensors=t)
    info = B.attn_decode_kernel_info(call.desc, call.plan)
    assert info.lds_bytes >= 4 * 2 * 32 * D * 2, info.lds_bytes
    assert (info.grid_x, info.grid_y, info.grid_z) == (hkv, call.plan.n_splits, 4)
    q1 = t["q"].unsqueeze(1).contiguous()
    qo, ql, qcall = run_qt(case, tensors={**t, "q": q1})
    assert (qcall.plan.n_splits, qcall.plan.chunk) == (call.plan.n_splits, call.plan.chunk)
    assert np.array_equal(qo[:, 0], out, equal_nan=True)
    assert np.array_equal(ql[:, 0], lse, equal_nan=True)
    ref, rlse = oracle_out(case)
    assert_parity(case, out, ref, label=case.name)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=LSE_F32_ARITH)


@pytest.mark.parametrize("kv,hq,hkv,D", [("f16", 8, 8, 64), ("bf16", 24, 4, 256), ("f16", 32, 8, 128)])
@pytest.mark.parametrize("S", [1, 3, 200])
def test_decode_on_query_tiles_with_explicit_splits(kv, hq, hkv, D, S):
    # Explicit split counts on routed descriptors: one slice, uneven slices,
    # and 200 slices of 25 positions (shorter than a 32-position tile; most
    # are empty for the short sequences and write the neutral partial).
    from harness import assert_parity, oracle_out, run_gpu

    case = synthetic.gqa_case(f"routed-S{S}-{hq}x{hkv}-d{D}-{kv}", seq_lens=[5000, 1, 333],
                              num_q_heads=hq, num_kv_heads=hkv, head_dim=D, kv_dtype=kv,
                              capacity=5003, seed=9300 + S + D)
    t = to_device(case)
    out, lse, call = run_gpu(case, n_splits=S, tensors=t)
    assert call.plan.n_splits == S
    qo, ql, _ = run_qt(case, n_splits=S, tensors={**t, "q": t["q"].unsqueeze(1).contiguous()})
    assert np.array_equal(qo[:, 0], out, equal_nan=True)
    assert np.array_equal(ql[:, 0], lse, equal_nan=True)
    ref, rlse = oracle_out(case)
    assert_parity(case, out, ref, label=case.name)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=LSE_F32_ARITH)
