"""Pins for the float64 oracle: checks against things other than itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a wrong group map, a missing
rescale) fails at least one test here:

* brute force with exact summation (``math.fsum``) in plain Python loops;
* torch's float64 CPU scaled-dot-product attention (a library routine), with
  each KV head repeated for its group;
* closed forms: one position returns its value row; equal scores return the
  mean of the values; one dominant score returns that row;
* invariants: linearity in V, permutation of positions, paged vs contiguous;
* the worked merge example of Lecture 07 (tests/golden/), checked against a
  full softmax over a sequence that has exactly those partials;
* negative controls from Lecture 06 section 6 and the Decoder Block 6 lesson.
"""

import math
import os

import numpy as np
import pytest

import oracle
import synthetic

HERE = os.path.dirname(os.path.abspath(__file__))


def brute_force(q, k, v, lens, scale):
    """Plain-Python decode attention with exact summation (no numpy maths)."""
    B, Hq, Dk = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k[0][0])
    G = Hq // Hkv
    out, lse = [], []
    for b in range(B):
        ob, lb = [], []
        for h in range(Hq):
            g = h // G
            s = [scale * math.fsum(float(q[b][h][d]) * float(k[b][j][g][d]) for d in range(Dk))
                 for j in range(lens[b])]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            den = math.fsum(w)
            dv = len(v[b][0][g])
            ob.append([math.fsum(w[j] * float(v[b][j][g][e]) for j in range(lens[b])) / den
                       for e in range(dv)])
            lb.append(m + math.log(den))
        out.append(ob)
        lse.append(lb)
    return np.array(out), np.array(lse)


def rand_case(rng, B, Hq, Hkv, Dk, Dv, lens):
    q = rng.standard_normal((B, Hq, Dk))
    cap = max(lens)
    k = rng.standard_normal((B, cap, Hkv, Dk))
    v = rng.standard_normal((B, cap, Hkv, Dv))
    return q, k, v


# ---------------------------------------------------------------- definition


@pytest.mark.parametrize("lens", [[1, 1], [2, 7], [8, 3], [5, 5]])
def test_definition_matches_exact_brute_force(lens):
    rng = np.random.default_rng(sum(lens))
    q, k, v = rand_case(rng, 2, 6, 2, 4, 3, lens)
    scale = 0.7
    out, lse = oracle.attend_f64(q, k, v, lens, scale, q_dtype="f64", kv_dtype="f64")
    bo, bl = brute_force(q, k, v, lens, scale)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-13)


@pytest.mark.parametrize("G,Hkv,D,L", [(4, 1, 64, 50), (4, 4, 32, 77), (6, 2, 16, 33)])
def test_definition_matches_torch_sdpa_f64(G, Hkv, D, L):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(G * 100 + L)
    B = 2
    Hq = G * Hkv
    q, k, v = rand_case(rng, B, Hq, Hkv, D, D, [L, L])
    scale = 1.0 / math.sqrt(D)
    out, _ = oracle.attend_f64(q, k, v, [L, L], scale, q_dtype="f64", kv_dtype="f64")
    tq = torch.from_numpy(q).unsqueeze(2)                                 # [B][Hq][1][D]
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, 1)  # [B][Hq][L][D]
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    np.testing.assert_allclose(out, ref[:, :, 0].numpy(), rtol=0, atol=1e-12)


def test_latent_definition_matches_torch_sdpa_f64():
    """Shared latent: keys are the 576-column rows, values their first 512."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    L, Hq = 40, 96
    q = rng.standard_normal((1, Hq, 576))
    c = rng.standard_normal((1, L, 1, 576))
    out, _ = oracle.attend_f64(q, c, None, [L], 1 / 24, q_dtype="f64", kv_dtype="f64", v_cols=512)
    tk = torch.from_numpy(c[0, :, 0]).expand(1, Hq, L, 576)
    tv = torch.from_numpy(c[0, :, 0, :512]).expand(1, Hq, L, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).unsqueeze(2), tk, tv, scale=1 / 24)
    np.testing.assert_allclose(out[0], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


def test_single_position_returns_its_value_row_exactly():
    rng = np.random.default_rng(1)
    q, k, v = rand_case(rng, 1, 4, 1, 64, 64, [1])
    out, lse = oracle.attend_f64(q, k, v, [1], 0.125, q_dtype="f64", kv_dtype="f64")
    for h in range(4):
        assert np.array_equal(out[0, h], v[0, 0, 0])
        assert lse[0, h] == pytest.approx(0.125 * float(q[0, h] @ k[0, 0, 0]), abs=1e-14)


@pytest.mark.parametrize("L", [33, 1000, 4096])
def test_equal_scores_give_the_mean_of_v(L):
    rng = np.random.default_rng(L)
    q, k, v = rand_case(rng, 1, 4, 1, 64, 64, [L])
    q[:] = 0.0
    out, lse = oracle.attend_f64(q, k, v, [L], 0.125, q_dtype="f64", kv_dtype="f64")
    mean = np.array([math.fsum(v[0, :L, 0, e]) / L for e in range(64)])
    for h in range(4):
        np.testing.assert_allclose(out[0, h], mean, rtol=0, atol=1e-13)
        assert lse[0, h] == pytest.approx(math.log(L), abs=1e-12)


@pytest.mark.parametrize("jstar", [0, 32, 517, 999])
def test_one_dominant_score_returns_that_row(jstar):
    """Score gap >= 60 (and large absolute scores, which overflow exp unless
    the maximum is subtracted first)."""
    L, D = 1000, 64
    rng = np.random.default_rng(jstar)
    q, k, v = rand_case(rng, 1, 4, 1, D, D, [L])
    q[0, :] = q[0, 0]
    qn = q[0, 0] / np.linalg.norm(q[0, 0])
    k[0, :, 0] = k[0, :, 0] - np.outer(k[0, :, 0] @ qn, qn)  # keys orthogonal to q
    k[0, :, 0] += 400.0 * qn                                 # every score large
    k[0, jstar, 0] += 480.0 * qn                             # one much larger
    scale = 1.0 / np.linalg.norm(q[0, 0])
    out, _ = oracle.attend_f64(q, k, v, [L], scale, q_dtype="f64", kv_dtype="f64")
    assert np.all(np.isfinite(out))
    for h in range(4):
        np.testing.assert_allclose(out[0, h], v[0, jstar, 0], rtol=0, atol=L * math.exp(-60) * 10)


def test_linear_in_v():
    rng = np.random.default_rng(3)
    q, k, v = rand_case(rng, 2, 8, 2, 16, 16, [30, 19])
    a, c = -2.5, 0.75
    o1, _ = oracle.attend_f64(q, k, v, [30, 19], 0.25, q_dtype="f64", kv_dtype="f64")
    o2, _ = oracle.attend_f64(q, k, a * v + c, [30, 19], 0.25, q_dtype="f64", kv_dtype="f64")
    np.testing.assert_allclose(o2, a * o1 + c, rtol=0, atol=1e-13)


def test_position_permutation_invariance():
    rng = np.random.default_rng(4)
    L = 257
    q, k, v = rand_case(rng, 1, 8, 2, 32, 32, [L])
    perm = rng.permutation(L)
    o1, l1 = oracle.attend_f64(q, k, v, [L], 0.2, q_dtype="f64", kv_dtype="f64")
    o2, l2 = oracle.attend_f64(q, k[:, perm], v[:, perm], [L], 0.2, q_dtype="f64", kv_dtype="f64")
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_group_map_is_contiguous():
    """Query head h reads KV head h // G: swapping KV heads must permute outputs."""
    rng = np.random.default_rng(5)
    q, k, v = rand_case(rng, 1, 8, 2, 16, 16, [20])
    o1, _ = oracle.attend_f64(q, k, v, [20], 0.3, q_dtype="f64", kv_dtype="f64")
    o2, _ = oracle.attend_f64(q[:, [4, 5, 6, 7, 0, 1, 2, 3]], k[:, :, ::-1], v[:, :, ::-1], [20],
                              0.3, q_dtype="f64", kv_dtype="f64")
    np.testing.assert_allclose(o2, o1[:, [4, 5, 6, 7, 0, 1, 2, 3]], rtol=0, atol=1e-14)


# ------------------------------------------------------------------ storage


def test_bf16_widening_is_exact():
    import torch

    x = torch.tensor([1.0, -2.5, 3.140625, 1e-3, 65504.0, -1e30, 0.0], dtype=torch.float32)
    bits = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = x.to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), ref)
    # Hand-checked patterns: 0x3F80 = 1.0, 0xC000 = -2.0, 0x4049 = 3.140625.
    got = oracle.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x4049], dtype=np.uint16))
    assert list(got) == [1.0, -2.0, 3.140625]


def test_f16_widening_reads_stored_values():
    x = np.array([0.1, 1 / 3, -7.25], dtype=np.float32)
    h = x.astype(np.float16)
    w = oracle.widen(h, "f16")
    assert list(w) == [float(t) for t in h]
    assert w[0] != 0.1  # the stored, rounded value, not the float32 draw


# -------------------------------------------------------------------- paged


def test_paged_gather_equals_contiguous_and_ignores_table_shuffle():
    case = synthetic.gqa_case("paged", seq_lens=[37, 16, 5], num_q_heads=8, num_kv_heads=2,
                              head_dim=16, layout="paged", page_size=4, seed=11)
    ks = [oracle.gather_paged(case.k, case.block_table[b], int(L), 4)
          for b, L in enumerate(case.seq_lens)]
    vs = [oracle.gather_paged(case.v, case.block_table[b], int(L), 4)
          for b, L in enumerate(case.seq_lens)]
    # The gathered rows are exactly the ones the table names, in order.
    b, j = 0, 13
    assert np.array_equal(ks[b][j], case.k[case.block_table[b][j // 4], j % 4])
    o1, _ = oracle.attend_f64(case.q, ks, vs, case.seq_lens, case.scale)
    # Move every page to a new slot of the pool and rewrite the table.
    P = case.k.shape[0]
    perm = np.random.default_rng(0).permutation(P)
    inv = np.argsort(perm)
    k2, v2 = case.k[perm], case.v[perm]
    t2 = np.where(case.block_table >= 0, inv[np.maximum(case.block_table, 0)], -1)
    ks2 = [oracle.gather_paged(k2, t2[b], int(L), 4) for b, L in enumerate(case.seq_lens)]
    vs2 = [oracle.gather_paged(v2, t2[b], int(L), 4) for b, L in enumerate(case.seq_lens)]
    o2, _ = oracle.attend_f64(case.q, ks2, vs2, case.seq_lens, case.scale)
    assert np.array_equal(o1, o2)
    assert np.all(np.isfinite(o1))


# -------------------------------------------------------------------- merge


def load_worked_example():
    rows = []
    with open(os.path.join(HERE, "golden", "merge_worked_example.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(t) for t in line.split()])
    return np.array(rows)


def test_worked_merge_example_equals_full_softmax():
    """Build a score/value sequence whose two blocks have exactly the page's
    partials, and compare the merge with the softmax over the whole sequence."""
    ex = load_worked_example()
    (m1, l1, a1), (m2, l2, a2) = ex
    # Block 1: 8 scores equal to 2 (max 2, sum exp(s-2) = 8), values 0.5 (sum 4).
    # Block 2: 6 scores equal to 3 (sum 6), values 3 (sum 18).
    s = [m1] * int(l1) + [m2] * int(l2)
    vals = [a1 / l1] * int(l1) + [a2 / l2] * int(l2)
    top = max(s)
    w = [math.exp(x - top) for x in s]
    want_out = math.fsum(wi * vi for wi, vi in zip(w, vals)) / math.fsum(w)
    want_lse = top + math.log(math.fsum(w))
    out, lse = oracle.merge_partials_f64(ex[:, 0], ex[:, 1], ex[:, 2:3])
    assert out[0] == pytest.approx(want_out, rel=0, abs=1e-15)
    assert lse == pytest.approx(want_lse, rel=0, abs=1e-15)
    out2, lse2 = oracle.merge_partials_lse_f64(ex[:, 0], ex[:, 1], ex[:, 2:3])
    assert out2[0] == pytest.approx(want_out, rel=0, abs=1e-15)
    assert lse2 == pytest.approx(want_lse, rel=0, abs=1e-15)
    # Partials taken from the recurrence over that sequence match the page.
    sv = np.array(s)
    vv = np.array(vals)[:, None]
    p1 = oracle.online_partial_f64(sv[:8], vv[:8], tile=3)
    p2 = oracle.online_partial_f64(sv[8:], vv[8:], tile=4)
    assert p1[0] == m1 and p1[1] == pytest.approx(l1) and p1[2][0] == pytest.approx(a1)
    assert p2[0] == m2 and p2[1] == pytest.approx(l2) and p2[2][0] == pytest.approx(a2)


def test_lse_form_equals_rescale_form():
    """The two forms of the merge agree to ~1e-16 (Lecture 07 reports 6e-16)."""
    rng = np.random.default_rng(9)
    worst = 0.0
    for _ in range(200):
        n = int(rng.integers(1, 12))
        m = rng.normal(0, 5, n)
        l = rng.uniform(0.5, 50, n)
        acc = rng.normal(0, 10, (n, 7))
        o1, e1 = oracle.merge_partials_f64(m, l, acc)
        o2, e2 = oracle.merge_partials_lse_f64(m, l, acc)
        worst = max(worst, np.abs(o1 - o2).max() / max(1.0, np.abs(o1).max()), abs(e1 - e2) / max(1.0, abs(e1)))
    assert worst <= 1e-14


def test_neutral_partial_has_zero_weight():
    m = np.array([1.5, -np.inf, 0.25])
    l = np.array([3.0, 0.0, 2.0])
    acc = np.array([[1.0], [0.0], [4.0]])
    o, _ = oracle.merge_partials_f64(m, l, acc)
    o2, _ = oracle.merge_partials_f64(m[[0, 2]], l[[0, 2]], acc[[0, 2]])
    assert o[0] == o2[0]
    em = oracle.online_partial_f64(np.zeros(0), np.zeros((0, 3)), tile=8)
    assert em[0] == -math.inf and em[1] == 0.0 and np.array_equal(em[2], np.zeros(3))


# -------------------------------------------------------------- split twin


@pytest.mark.parametrize("L", [1, 33, 1000, 4097])
@pytest.mark.parametrize("S", [1, 2, 3, 8, 64])
def test_twin_equals_definition(L, S):
    case = synthetic.tiny_gqa(L, seed=L)
    ref, rl = oracle.attend_f64(case.q, case.k_rows(), case.v_rows(), case.seq_lens, case.scale)
    chunk = -(-L // S)
    for tile in (1, 7, 32, 64):
        out, lse = oracle.split_twin_f64(case.q, case.k_rows(), case.v_rows(), case.seq_lens,
                                         case.scale, chunk, S, tile=tile)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_twin_with_empty_trailing_splits():
    """L = 33, S = 8: chunk 5, split 7 starts at 35 and is empty."""
    case = synthetic.tiny_gqa(33, seed=2)
    chunk = -(-33 // 8)
    assert oracle.split_ranges(33, chunk, 8)[7] == (33, 33)
    m, l, acc = oracle.split_partials_f64(case.q, case.k_rows(), case.v_rows(), case.seq_lens,
                                          case.scale, chunk, 8)
    assert np.all(m[0, :, 7] == -np.inf) and np.all(l[0, :, 7] == 0) and np.all(acc[0, :, 7] == 0)
    assert np.all(np.isfinite(m[0, :, :7]))


# --------------------------------------------------------- negative controls

GATES = (1e-4, 2e-3)


def _err(a, b):
    return float(np.abs(a - b).max())


@pytest.mark.parametrize("L", [1000, 20480])
def test_negative_control_no_merge_rescale_fails(L):
    case = synthetic.qwen9b_like(L, "f32", seed=L)
    ref, _ = oracle.attend_f64(case.q, case.k_rows(), case.v_rows(), case.seq_lens, case.scale)
    S = 8
    bad, _ = oracle.split_twin_f64(case.q, case.k_rows(), case.v_rows(), case.seq_lens,
                                   case.scale, -(-L // S), S, rescale=False)
    assert _err(bad, ref) > 5 * max(GATES)


def test_negative_control_no_alpha_fails_at_tile_boundary():
    """L = 33 with a 32-position tile; position 32 carries the largest score
    for every head, so the running max moves in the second tile."""
    case = synthetic.tiny_gqa(33, seed=3)
    qn = case.q[0, 0] / np.linalg.norm(case.q[0, 0])
    case.q[0, :] = case.q[0, 0]
    case.k[0, 32, 0] = (qn * 40.0).astype(np.float32)  # score about |q| * 40 / 8
    ks, vs = case.k_rows(), case.v_rows()
    ref, _ = oracle.attend_f64(case.q, ks, vs, case.seq_lens, case.scale)
    good, _ = oracle.split_twin_f64(case.q, ks, vs, case.seq_lens, case.scale, 33, 1, tile=32)
    bad, _ = oracle.split_twin_f64(case.q, ks, vs, case.seq_lens, case.scale, 33, 1, tile=32, alpha=False)
    assert _err(good, ref) < 1e-12
    assert _err(bad, ref) > 5 * max(GATES)


@pytest.mark.parametrize("L", [1000, 20480])
def test_negative_control_no_alpha_fails_at_length(L):
    case = synthetic.qwen9b_like(L, "f32", seed=L + 1)
    ref, _ = oracle.attend_f64(case.q, case.k_rows(), case.v_rows(), case.seq_lens, case.scale)
    bad, _ = oracle.split_twin_f64(case.q, case.k_rows(), case.v_rows(), case.seq_lens,
                                   case.scale, L, 1, tile=64, alpha=False)
    assert _err(bad, ref) > 5 * max(GATES)


def test_negative_controls_group_map_scale_zero_fail():
    case = synthetic.qwen9b_like(1000, "f32", seed=77)
    args = (case.q, case.k_rows(), case.v_rows(), case.seq_lens, case.scale)
    ref, _ = oracle.attend_f64(*args)
    wrong_map, _ = oracle.attend_f64(*args, group_map="modulo")
    no_scale, _ = oracle.attend_f64(*args, apply_scale=False)
    assert _err(wrong_map, ref) > 5 * max(GATES)
    assert _err(no_scale, ref) > 5 * max(GATES)
    assert _err(np.zeros_like(ref), ref) > 5 * max(GATES)


# ------------------------------------------------------------------ planner


def test_plan_explicit_splits_are_honoured():
    assert oracle.plan_splits([1], 1, 256, 8) == (8, 1)
    assert oracle.plan_splits([33], 1, 256, 8) == (8, 5)
    assert oracle.plan_splits([4096], 1, 256, 3) == (3, 1366)


def test_plan_heuristic_matches_the_single_sequence_rule():
    """At batch 1 the product budget reduces to the design note's rule:
    chunk = max(64, ceil(L / S_target)), S = ceil(L / chunk), S_target = 4*CUs/Hkv."""
    for L in (4096, 20480, 61440, 151552, 262144):
        for hkv in (1, 2, 4, 8):
            s_target = 4 * 256 // hkv
            chunk = max(64, -(-L // s_target))
            chunk = -(-chunk // 64) * 64
            assert oracle.plan_splits([L], hkv, 256) == (-(-L // chunk), chunk)
    assert oracle.plan_splits([262144], 4, 256) == (256, 1024)


def test_plan_heuristic_never_leaves_an_empty_split():
    rng = np.random.default_rng(0)
    for _ in range(200):
        lens = rng.integers(1, 300000, size=int(rng.integers(1, 40)))
        S, chunk = oracle.plan_splits(lens, int(rng.choice([1, 4, 8])), 256)
        for L in lens:
            n = -(-int(L) // chunk)
            assert n <= S
            assert (n - 1) * chunk < L  # the last used split holds positions


def test_plan_ragged_batch_is_budgeted_on_the_product():
    lens = synthetic.ragged_lengths()
    S, chunk = oracle.plan_splits(lens, 8, 256)
    blocks = sum(8 * -(-int(L) // chunk) for L in lens)
    assert chunk % 16 == 0
    assert 0.75 * 1024 <= blocks <= 1.5 * 1024


def test_plan_minimum_context_gate():
    assert oracle.plan_splits([4000], 4, 256, min_ctx=4096) == (1, 4000)
    assert oracle.plan_splits([4096], 4, 256, min_ctx=4096)[0] > 1


# ------------------------------------------------- projection after the merge


def _brute_project(out, w):
    B, Hq, Dv = len(out), len(out[0]), len(out[0][0])
    P = len(w[0])
    return np.array([[[math.fsum(float(w[h][r][c]) * float(out[b][h][c]) for c in range(Dv))
                       for r in range(P)] for h in range(Hq)] for b in range(B)])


def test_projection_matches_exact_brute_force():
    rng = np.random.default_rng(5)
    out = rng.standard_normal((2, 3, 7))
    w = rng.standard_normal((3, 4, 7))
    got = oracle.project_heads_f64(out, w, "f64")
    assert np.abs(got - _brute_project(out, w)).max() <= 1e-14


def test_projection_identity_and_one_hot_rows_are_exact():
    rng = np.random.default_rng(6)
    out = rng.standard_normal((2, 4, 16))
    eye = np.broadcast_to(np.eye(16), (4, 16, 16)).copy()
    assert np.array_equal(oracle.project_heads_f64(out, eye, "f64"), out)
    cols = [3, 0, 15, 7, 7]
    onehot = np.zeros((4, len(cols), 16))
    for r, c in enumerate(cols):
        onehot[:, r, c] = 1.0
    assert np.array_equal(oracle.project_heads_f64(out, onehot, "f64"), out[:, :, cols])
    # each head uses its own matrix: scaling one head's W scales only that head
    w = rng.standard_normal((4, 5, 16))
    w2 = w.copy()
    w2[2] *= 3.0
    a, b = oracle.project_heads_f64(out, w, "f64"), oracle.project_heads_f64(out, w2, "f64")
    assert np.abs(b[:, 2] - 3 * a[:, 2]).max() <= 1e-12
    assert np.array_equal(np.delete(a, 2, axis=1), np.delete(b, 2, axis=1))


def test_projection_is_linear_in_the_output():
    rng = np.random.default_rng(7)
    o1, o2 = rng.standard_normal((2, 1, 3, 9))
    w = rng.standard_normal((3, 5, 9))
    lhs = oracle.project_heads_f64(2.5 * o1 - o2, w, "f64")
    rhs = 2.5 * oracle.project_heads_f64(o1, w, "f64") - oracle.project_heads_f64(o2, w, "f64")
    assert np.abs(lhs - rhs).max() <= 1e-12


def test_projection_storage_widening_reads_stored_weights():
    w32 = synthetic.projection_weights(2, 3, 8, "f32", seed=1)
    w16 = synthetic.projection_weights(2, 3, 8, "f16", seed=1)
    wbf = synthetic.projection_weights(2, 3, 8, "bf16", seed=1)
    out = np.ones((1, 2, 8))
    assert np.array_equal(oracle.project_heads_f64(out, w16, "f16")[0],
                          w16.astype(np.float64).sum(axis=2))
    got = oracle.project_heads_f64(out, wbf, "bf16")[0]
    assert np.array_equal(got, oracle.bf16_bits_to_f64(wbf).sum(axis=2))
    assert np.abs(got - w32.astype(np.float64).sum(axis=2)).max() < 0.05


def _latent_partials(L, S, seed):
    case = synthetic.latent_case("proj", seq_len=L, kv_dtype="f32", seed=seed, scale=1 / 24)
    chunk = -(-L // S)
    m, l, acc = oracle.split_partials_f64(case.q, case.k_rows(), None, case.seq_lens, case.scale,
                                          chunk, S, v_cols=512)
    ref, _ = oracle.attend_f64(case.q, case.k_rows(), None, case.seq_lens, case.scale, v_cols=512)
    return case, m, l, acc, ref


def test_projection_commutes_with_the_rescaled_merge():
    """W is linear, so projecting each slice's un-normalised accumulator and
    merging with the combine's own weights equals projecting the merged output
    (at S times the projection work): the projection of the definition is the
    unique correct result."""
    case, m, l, acc, ref = _latent_partials(1000, 4, 11)
    w = synthetic.projection_weights(96, 128, 512, "f32", seed=2)
    want = oracle.project_heads_f64(ref, w, "f32")
    for h in (0, 37, 95):
        got = oracle.project_per_slice_f64(m[0, h], l[0, h], acc[0, h], 4, w[h], "f32")
        assert np.abs(got - want[0, h]).max() <= 1e-12


@pytest.mark.parametrize("L,S", [(1000, 3), (8192, 16)])
def test_negative_control_projecting_normalised_slices_fails(L, S):
    """[L06] section 2: the projection is a function of the merged latent.
    Projecting each slice's normalised output and averaging the slices with
    equal weights must miss the f32 gate by far (test power)."""
    case, m, l, acc, ref = _latent_partials(L, S, 12)
    w = synthetic.projection_weights(96, 128, 512, "f32", seed=3)
    want = oracle.project_heads_f64(ref, w, "f32")
    bad = np.stack([oracle.project_per_slice_f64(m[0, h], l[0, h], acc[0, h], S, w[h], "f32",
                                                 normalised_mean=True) for h in range(96)])
    err = float(np.abs(bad - want[0]).max())
    rel = float(np.linalg.norm(bad - want[0]) / np.linalg.norm(want[0]))
    assert err > 10 * GATES[0] and rel > 100 * 1e-5, (err, rel)


# ------------------------------------------------------- sparse (index-list)


def test_index_list_gather_of_every_row_in_order_is_the_contiguous_cache():
    rng = np.random.default_rng(21)
    pool = rng.standard_normal((50, 2, 8))
    assert np.array_equal(oracle.gather_indexed(pool, np.arange(50), 50), pool)
    assert np.array_equal(oracle.gather_indexed(pool, np.arange(50), 17), pool[:17])
    # the same rows through a block table of one-row pages
    table = rng.permutation(50)
    got = oracle.gather_indexed(pool, table, 30)
    paged = oracle.gather_paged(pool[:, None], table, 30, 1)
    assert np.array_equal(got, paged)
    with pytest.raises(ValueError):
        oracle.gather_indexed(pool, [3, 50], 2)
    with pytest.raises(ValueError):
        oracle.gather_indexed(pool, [-1, 0], 2)


def test_sparse_attention_matches_exact_brute_force_over_the_listed_rows():
    case = synthetic.indexed_case("sp", pool_rows=40, seq_lens=[5, 1, 9], num_q_heads=4,
                                  num_kv_heads=2, head_dim=6, seed=22)
    got, glse = oracle.attend_f64(case.q, case.k_rows(), case.v_rows(), case.seq_lens, case.scale)
    q = case.q.astype(np.float64).tolist()
    for b, L in enumerate(case.seq_lens):
        idx = case.block_table[b, :L]
        k = [[case.k[r].astype(np.float64).tolist() for r in idx]]
        v = [[case.v[r].astype(np.float64).tolist() for r in idx]]
        want, wlse = brute_force([q[b]], k, v, [int(L)], case.scale)
        assert np.abs(got[b] - want[0]).max() <= 1e-14
        assert np.abs(glse[b] - wlse[0]).max() <= 1e-13


def test_sparse_attention_does_not_depend_on_the_order_of_the_list():
    case = synthetic.indexed_case("sp", pool_rows=3000, seq_lens=[2048, 700], num_q_heads=8,
                                  num_kv_heads=2, head_dim=64, kv_dtype="f16", seed=23)
    a, _ = oracle.attend_f64(case.q, case.k_rows(), case.v_rows(), case.seq_lens, case.scale,
                             kv_dtype="f16")
    rng = np.random.default_rng(1)
    for b, L in enumerate(case.seq_lens):
        case.block_table[b, :L] = rng.permutation(case.block_table[b, :L])
    bb, _ = oracle.attend_f64(case.q, case.k_rows(), case.v_rows(), case.seq_lens, case.scale,
                              kv_dtype="f16")
    assert np.abs(a - bb).max() <= 1e-13


def test_negative_control_ignoring_the_index_list_fails():
    """Attending the first L pool rows instead of the listed ones must miss the
    gates by far (so a kernel that drops the indirection cannot pass)."""
    case = synthetic.dsa_latent(topk=2048, pool_rows=16384, kv_dtype="f32", seed=24)
    want, _ = oracle.attend_f64(case.q, case.k_rows(), None, case.seq_lens, case.scale, v_cols=512)
    first = [case.k[: int(case.seq_lens[0])]]
    bad, _ = oracle.attend_f64(case.q, first, None, case.seq_lens, case.scale, v_cols=512)
    assert _err(bad, want) > 5 * max(GATES)


# ------------------------------------------------- several queries (query tiles)


def _brute_causal(case):
    """Plain-Python causal attention with exact summation."""
    B, Q, Hq, D = case.q.shape
    G = Hq // case.num_kv_heads
    out = np.full((B, Q, Hq, D), np.nan)
    for b in range(B):
        L = int(case.seq_lens[b])
        for t in range(Q):
            lim = L - Q + t + 1
            if lim < 1:
                continue
            for h in range(Hq):
                g = h // G
                qv = [float(x) for x in case.q[b, t, h]]
                s = [case.scale * math.fsum(qv[d] * float(case.k[b, j, g, d]) for d in range(D))
                     for j in range(lim)]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                den = math.fsum(w)
                out[b, t, h] = [math.fsum(w[j] * float(case.v[b, j, g, e]) for j in range(lim)) / den
                                for e in range(D)]
    return out


def test_multiquery_definition_matches_exact_brute_force():
    case = synthetic.multiquery_case("mq", seq_lens=[9, 4, 2], q_len=3, num_q_heads=4,
                                     num_kv_heads=2, head_dim=5, kv_dtype="f32", seed=31)
    got, _ = oracle.attend_multiquery_f64(case.q, case.k, case.v, case.seq_lens, case.scale)
    want = _brute_causal(case)
    assert np.array_equal(np.isnan(got), np.isnan(want))  # L=2 < Q=3: query 0 sees nothing
    assert np.nanmax(np.abs(got - want)) <= 1e-14


def test_multiquery_is_causal():
    """Changing the key and value rows at position p changes exactly the
    queries that can see p (lim > p) and leaves every other bit unchanged."""
    case = synthetic.multiquery_case("mq", seq_lens=[40], q_len=16, num_q_heads=4,
                                     num_kv_heads=1, head_dim=8, kv_dtype="f32", seed=32)
    a, _ = oracle.attend_multiquery_f64(case.q, case.k, case.v, case.seq_lens, case.scale)
    p = 30
    case.k[0, p] += 1.0
    case.v[0, p] -= 2.0
    b, _ = oracle.attend_multiquery_f64(case.q, case.k, case.v, case.seq_lens, case.scale)
    lims = oracle.causal_limits(40, 16)
    for t in range(16):
        if lims[t] > p:
            assert np.abs(a[0, t] - b[0, t]).max() > 1e-6
        else:
            assert np.array_equal(a[0, t], b[0, t])


def test_full_self_attention_first_query_sees_only_position_zero():
    case = synthetic.causal_block(64, kv_dtype="f32", seed=33)
    out, _ = oracle.attend_multiquery_f64(case.q, case.k, case.v, case.seq_lens, case.scale)
    for h in range(4):
        assert np.array_equal(out[0, 0, h], case.v[0, 0, h].astype(np.float64))


@pytest.mark.parametrize("L,Q", [(33, 33), (33, 5), (1000, 40)])
def test_query_tile_twin_equals_definition(L, Q):
    case = synthetic.multiquery_case("mq", seq_lens=[L], q_len=Q, num_q_heads=4, num_kv_heads=2,
                                     head_dim=16, kv_dtype="f16", seed=L + Q)
    want, _ = oracle.attend_multiquery_f64(case.q, case.k, case.v, case.seq_lens, case.scale,
                                           kv_dtype="f16")
    for tile in (1, 7, 32):
        got = oracle.query_tile_twin_f64(case.q, case.k, case.v, case.seq_lens, case.scale,
                                         tile=tile, kv_dtype="f16")
        assert np.abs(got - want).max() <= 1e-12


def test_negative_control_query_tiles_without_alpha_fail_at_length_33():
    """[DB6]: without the rescale the block is wrong once the running maximum
    moves between tiles; length 33 puts the rows past 32 in two tiles. Make
    position 32 the dominant key so the maximum moves for every row that sees it."""
    case = synthetic.multiquery_case("mq33", seq_lens=[33], q_len=33, num_q_heads=4,
                                     num_kv_heads=1, head_dim=64, kv_dtype="f32", seed=34)
    qd = case.q[0, 32, 0].astype(np.float64)
    case.q[0, :, :] = case.q[0, 32, 0]
    case.k[0, 32, 0] = (qd / np.linalg.norm(qd) * 8 * 6 / np.linalg.norm(qd)).astype(np.float32)
    want, _ = oracle.attend_multiquery_f64(case.q, case.k, case.v, case.seq_lens, case.scale)
    bad = oracle.query_tile_twin_f64(case.q, case.k, case.v, case.seq_lens, case.scale,
                                     tile=32, alpha=False)
    assert _err(bad[0, 32], want[0, 32]) > 5 * max(GATES)
    assert _err(bad[0, :32], want[0, :32]) <= 1e-12  # one tile: no rescale needed


def test_negative_control_without_the_causal_mask_fails():
    case = synthetic.chunked_prefill(2048, 64, kv_dtype="f32", seed=35)
    want, _ = oracle.attend_multiquery_f64(case.q, case.k, case.v, case.seq_lens, case.scale,
                                           heads=[(0, t, 0) for t in range(64)])
    bad, _ = oracle.attend_multiquery_f64(case.q, case.k, case.v, case.seq_lens, case.scale,
                                          causal=False, heads=[(0, t, 0) for t in range(64)])
    assert np.nanmax(np.abs(bad - want)) > 5 * max(GATES)
