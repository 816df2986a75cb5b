"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, plans splits exactly as the oracle's reading of the pages,
sizes the workspace as documented, and rejects bad arguments before any HIP
call."""

import ctypes
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic
from split_kv_flash_amd import binding as B


def lib():
    try:
        return B.lib()
    except RuntimeError as e:  # the library is built by __graft_entry__.build()
        pytest.fail(str(e))


def gqa_desc(Hq=16, Hkv=4, D=256, cap=4096, kv="f32", q="f32", batch=1, layout="contiguous",
             page=16, max_pages=None, num_pages=1000):
    d = B.SkDesc()
    d.batch, d.num_q_heads, d.num_kv_heads = batch, Hq, Hkv
    d.head_dim_qk = d.head_dim_v = D
    d.kv_shared = 0
    d.scale = 1.0 / D ** 0.5
    d.q_dtype, d.kv_dtype = B.DTYPES[q], B.DTYPES[kv]
    if layout == "contiguous":
        d.layout = B.SK_KV_CONTIGUOUS
        d.max_seq_len = cap
        d.stride_head = D
        d.stride_pos = Hkv * D
        d.stride_seq = cap * Hkv * D
    else:
        d.layout = B.SK_KV_PAGED
        d.page_size = page
        d.max_pages_per_seq = max_pages or -(-cap // page)
        d.num_pages = num_pages
        d.max_seq_len = cap
    return d


def latent_desc(cap=8192, kv="f32", Hq=96):
    d = B.SkDesc()
    d.batch, d.num_q_heads, d.num_kv_heads = 1, Hq, 1
    d.head_dim_qk, d.head_dim_v, d.kv_shared = 576, 512, 1
    d.scale = 1 / 24
    d.q_dtype, d.kv_dtype = B.SK_F32, B.DTYPES[kv]
    d.layout = B.SK_KV_CONTIGUOUS
    d.max_seq_len = cap
    d.stride_head, d.stride_pos, d.stride_seq = 576, 576, cap * 576
    return d


def test_library_loads_and_exports_every_header_function():
    L = lib()
    names = B.header_functions()
    assert {"attn_decode_splitk", "attn_decode_combine", "attn_decode_plan",
            "attn_decode_workspace_bytes", "attn_decode", "attn_decode_one_launch",
            "attn_decode_workspace_init", "attn_decode_combine_project", "attn_query_tiles",
            "attn_query_tiles_plan", "attn_query_tiles_workspace_bytes",
            "attn_decode_read_probe"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"libsplitkv.so does not export {n}"


def test_status_strings():
    lib()
    for s in range(6):
        assert B.attn_decode_status_string(s)
    assert B.attn_decode_status_string(0) == "ok"


@pytest.mark.parametrize("hkv", [1, 4, 8])
def test_plan_matches_oracle_reading(hkv):
    lib()
    rng = np.random.default_rng(hkv)
    for _ in range(300):
        batch = int(rng.integers(1, 40))
        lens = rng.integers(1, 300000, size=batch)
        cu = int(rng.choice([80, 132, 256, 304]))
        req = int(rng.choice([0, 0, 0, 1, 3, 8, 64, 512]))
        d = gqa_desc(Hq=4 * hkv, Hkv=hkv, D=128, cap=int(lens.max()), batch=batch)
        p = B.attn_decode_plan(d, int(lens.max()), int(lens.sum()), cu, req)
        budget = 8 if int(lens.sum()) < batch * int(lens.max()) else 1  # ragged batches: 8 per CU
        want = oracle.plan_splits(lens, hkv, cu, req, blocks_per_cu=budget)
        if req == 0 and budget == 1 and -(-hkv * int(lens.sum()) // cu) >= 1024:
            # long slices: three quarters of the compute units
            want = oracle.plan_splits(lens, hkv, cu, req, blocks_per_cu=Fraction(3, 4))
        assert (p.n_splits, p.chunk) == want


def test_plan_keeps_the_pages_split_properties_whatever_the_budget():
    """What the pages fix about a plan, independent of the library's tuned
    budget (aprender issue #3725 design note section 2; Lecture 06 sections 2
    and 5.1): an explicit split count is honoured with chunk = ceil(L_max/S);
    otherwise every sequence is covered (ceil(L_b/chunk) <= S), the longest
    sequence's last split is not empty ((S-1)*chunk < L_max), a slice is at
    least 64 positions and a whole number of 64-position tiles, and the
    blocks (KV heads x slices over the batch) stay within a few tiles' worth of
    one to eight per compute unit, the range the budgets span."""
    lib()
    rng = np.random.default_rng(11)
    for _ in range(400):
        hkv = int(rng.choice([1, 2, 4, 8]))
        batch = int(rng.integers(1, 33))
        lens = rng.integers(1, 400000, size=batch)
        cu = int(rng.choice([80, 132, 256, 304]))
        req = int(rng.choice([0, 0, 0, 2, 7, 64]))
        d = gqa_desc(Hq=4 * hkv, Hkv=hkv, D=128, cap=int(lens.max()), batch=batch)
        p = B.attn_decode_plan(d, int(lens.max()), int(lens.sum()), cu, req)
        l_max = int(lens.max())
        if req:
            assert (p.n_splits, p.chunk) == (req, -(-l_max // req))
            continue
        assert p.chunk >= 64 and p.chunk % 64 == 0
        assert all(-(-int(L) // p.chunk) <= p.n_splits for L in lens)
        assert (p.n_splits - 1) * p.chunk < l_max
        blocks = hkv * sum(-(-int(L) // p.chunk) for L in lens)
        if p.chunk > 64:  # not held at the minimum slice
            # chunk is the smallest granule multiple at or above the budget's
            # slice, so one granule less would have exceeded the budget
            assert hkv * sum(-(-int(L) // (p.chunk - 64)) for L in lens) > 0.75 * cu
            assert blocks <= 8 * cu + hkv * batch


def test_plan_latent_matches_oracle_reading():
    lib()
    # f16 latents: one workgroup per split up to 96 heads, two of 64 heads at
    # 128; f32 latents spread a split's heads over Hq/48 (or Hq/32)
    # workgroups of 16-head blocks.
    groups = {("f16", 96): 1, ("f16", 32): 1, ("f16", 64): 1, ("f16", 128): 2, ("f32", 96): 2,
              ("f32", 32): 1, ("f32", 64): 2, ("f32", 128): 4}
    for (kv, hq), g in groups.items():
        for L in (1, 64, 65, 8192, 131072, 262144):
            for cu in (132, 256):
                p = B.attn_decode_plan(latent_desc(cap=L, kv=kv, Hq=hq), L, L, cu, 0)
                want = oracle.plan_splits([L], 1, cu, kv_shared=True, latent_groups=g)
                assert (p.n_splits, p.chunk) == want, (kv, hq, L, cu)


def test_plan_for_the_nine_b_like_layer_at_262144():
    lib()
    p = B.attn_decode_plan(gqa_desc(cap=262144), 262144, 262144, 256, 0)
    # 4 KV heads x 48 splits = 192 workgroups: three quarters of the compute units
    assert (p.n_splits, p.chunk) == (48, 5504)
    p = B.attn_decode_plan(gqa_desc(cap=20480), 20480, 20480, 256, 0)
    assert (p.n_splits, p.chunk) == (64, 320)  # short slices keep one workgroup per CU


def test_plan_for_the_wide_f16_group_keeps_every_compute_unit():
    lib()
    d = gqa_desc(Hq=24, Hkv=4, D=256, cap=262144, kv="f16")
    p = B.attn_decode_plan(d, 262144, 262144, 256, 0)
    assert (p.n_splits, p.chunk) == (64, 4096)  # 4 x 64 = 256 workgroups, one per CU
    assert (p.n_splits, p.chunk) == oracle.plan_splits([262144], 4, 256, blocks_per_cu=1)
    d = gqa_desc(Hq=24, Hkv=4, D=256, cap=262144, kv="f32")  # the f32 kernel streams from 3/4
    p = B.attn_decode_plan(d, 262144, 262144, 256, 0)
    assert (p.n_splits, p.chunk) == (48, 5504)


def test_plan_for_decode_on_query_tiles_counts_resident_workgroups():
    lib()
    # 16-bit groups decoded by the query-tile kernel (all of width 64, width 128
    # from 4 heads per KV head, width 256 from 6): one round of the 1, 2 or 4
    # workgroups a compute unit holds at width 256, 128 or 64, over KV heads x
    # slices (a ragged batch: 8 per compute unit, as on the split kernel);
    # attn_query_tiles_plan with one query gives the same plan.
    for hq, hkv, D, res in [(24, 4, 256, 1), (32, 4, 256, 1), (64, 8, 256, 1), (32, 8, 128, 2),
                            (48, 8, 128, 2), (8, 8, 64, 4), (64, 8, 64, 4)]:
        for lens, kv in itertools.product(([1000], [32768], [131072], [16384] * 8, [300, 5000, 70000]),
                                          ("f16", "bf16")):
            for cu in (80, 256):
                d = gqa_desc(Hq=hq, Hkv=hkv, D=D, cap=max(lens), kv=kv, batch=len(lens))
                p = B.attn_decode_plan(d, max(lens), sum(lens), cu, 0)
                ragged = sum(lens) < len(lens) * max(lens)  # the ragged budget: 8 per CU
                want = oracle.plan_splits(lens, hkv, cu, blocks_per_cu=8 if ragged else res)
                assert (p.n_splits, p.chunk) == want, (hq, hkv, D, lens, cu)
                pq = B.attn_query_tiles_plan(d, 1, max(lens), sum(lens), cu, 0)
                assert (pq.n_splits, pq.chunk) == want
    # f32 storage and the narrower 16-bit groups keep the split kernel's rule
    p = B.attn_decode_plan(gqa_desc(Hq=24, Hkv=4, D=256, cap=262144, kv="f32"), 262144, 262144, 256, 0)
    assert (p.n_splits, p.chunk) == (48, 5504)
    p = B.attn_decode_plan(gqa_desc(Hq=16, Hkv=4, D=256, cap=262144, kv="bf16"), 262144, 262144, 256, 0)
    assert (p.n_splits, p.chunk) == (48, 5504)
    p = B.attn_decode_plan(gqa_desc(Hq=16, Hkv=4, D=256, cap=262144, kv="f16"), 262144, 262144, 256, 0)
    assert (p.n_splits, p.chunk) == (48, 5504)
    p = B.attn_decode_plan(gqa_desc(Hq=16, Hkv=8, D=128, cap=131072, kv="f16"), 131072, 131072, 256, 0)
    assert (p.n_splits, p.chunk) == oracle.plan_splits([131072], 8, 256, blocks_per_cu=Fraction(3, 4))


def test_query_tile_plan_counts_resident_workgroups():
    lib()
    # several queries: the tiles of 64 (query, head) rows per KV head times
    # the KV heads, over the workgroups a compute unit holds
    for q_len, hq, hkv, D, res in [(4, 16, 4, 256, 1), (512, 16, 4, 256, 1), (2048, 4, 4, 64, 4),
                                   (8, 32, 8, 128, 2)]:
        L = 8192
        d = gqa_desc(Hq=hq, Hkv=hkv, D=D, cap=L, kv="f16")
        p = B.attn_query_tiles_plan(d, q_len, L, L, 256, 0)
        tiles = hkv * -(-(q_len * (hq // hkv)) // 64)
        assert (p.n_splits, p.chunk) == oracle.plan_splits([L], tiles, 256, blocks_per_cu=res)


def test_workspace_bytes_follow_the_documented_layout():
    lib()
    for (bsz, hq, s, dv) in [(1, 16, 256, 256), (32, 32, 9, 128), (1, 4, 3, 64), (1, 96, 256, 512)]:
        if dv == 512:
            d = latent_desc()
        else:
            d = gqa_desc(Hq=hq, Hkv=hq // 4 if hq >= 4 else 1, D=dv, batch=bsz)
        p = B.SkPlan(s, 64)
        rows = bsz * hq * s
        a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
        # per (sequence, KV head): the merge tree's chunk count, then one count per
        # chunk of 16 splits
        counters = a256(bsz * d.num_kv_heads * (1 + (s + 15) // 16) * 4)
        want = a256(rows * dv * 4) + a256(rows * 4) + a256(rows * 4) + counters
        assert B.attn_decode_workspace_bytes(d, p) == want


def _split(d, p, q=4096, k=4096, v=4096, bt=None, lens=4096, ws=4096, wsb=1 << 40):
    L = lib()
    s = L.attn_decode_splitk(ctypes.byref(d), ctypes.byref(p), q, k, v, bt, lens, ws, wsb, None)
    return s, B.attn_decode_last_error()


def _combine(d, p, lens=4096, ws=4096, wsb=1 << 40, out=4096, lse=None):
    L = lib()
    s = L.attn_decode_combine(ctypes.byref(d), ctypes.byref(p), lens, ws, wsb, out, lse, None)
    return s, B.attn_decode_last_error()


def _decode(d, p, q=4096, k=4096, v=4096, bt=None, lens=4096, ws=4096, wsb=1 << 40, out=4096,
            lse=None):
    L = lib()
    s = L.attn_decode(ctypes.byref(d), ctypes.byref(p), q, k, v, bt, lens, ws, wsb, out, lse, None)
    return s, B.attn_decode_last_error()


def _one(d, p, q=4096, k=4096, v=4096, bt=None, lens=4096, ws=4096, wsb=1 << 40, out=4096,
         lse=None):
    L = lib()
    s = L.attn_decode_one_launch(ctypes.byref(d), ctypes.byref(p), q, k, v, bt, lens, ws, wsb, out,
                                 lse, None)
    return s, B.attn_decode_last_error()


def _proj(d, p, lens=4096, ws=4096, wsb=1 << 40, w=4096, wdt=0, P=128, out=4096, lse=None):
    L = lib()
    s = L.attn_decode_combine_project(ctypes.byref(d), ctypes.byref(p), lens, ws, wsb, w, wdt, P,
                                      out, lse, None)
    return s, B.attn_decode_last_error()


def _init(d, p, ws=4096, wsb=1 << 40):
    L = lib()
    s = L.attn_decode_workspace_init(ctypes.byref(d), ctypes.byref(p), ws, wsb, None)
    return s, B.attn_decode_last_error()


def test_argument_errors_are_reported_before_any_launch():
    """Every case below is rejected by host validation (fake device addresses
    are never dereferenced), with its own status and a detail message."""
    lib()
    good = gqa_desc()
    plan = B.SkPlan(8, 512)
    cases = []

    d = gqa_desc(Hq=10, Hkv=4)
    cases.append(("heads not a multiple", _split(d, plan), B.SK_ERR_INVALID_ARG))
    d = gqa_desc(D=96)
    cases.append(("unsupported head dim", _split(d, plan), B.SK_ERR_UNSUPPORTED))
    d = gqa_desc(Hq=12, Hkv=4)
    cases.append(("unsupported group size 3", _split(d, plan), B.SK_ERR_UNSUPPORTED))
    cases.append(("zero splits", _split(good, B.SkPlan(0, 512)), B.SK_ERR_INVALID_ARG))
    cases.append(("zero chunk", _split(good, B.SkPlan(8, 0)), B.SK_ERR_INVALID_ARG))
    cases.append(("NULL seq_lens", _split(good, plan, lens=None), B.SK_ERR_INVALID_ARG))
    cases.append(("NULL q", _split(good, plan, q=None), B.SK_ERR_INVALID_ARG))
    cases.append(("NULL v for separate K/V", _split(good, plan, v=None), B.SK_ERR_INVALID_ARG))
    cases.append(("NULL workspace", _split(good, plan, ws=None), B.SK_ERR_INVALID_ARG))
    cases.append(("misaligned workspace", _split(good, plan, ws=4096 + 16), B.SK_ERR_INVALID_ARG))
    cases.append(("misaligned K", _split(good, plan, k=4096 + 4), B.SK_ERR_INVALID_ARG))
    cases.append(("misaligned q", _split(good, plan, q=4096 + 8), B.SK_ERR_INVALID_ARG))
    cases.append(("workspace too small", _split(good, plan, wsb=1024), B.SK_ERR_WORKSPACE_TOO_SMALL))
    cases.append(("table for contiguous", _split(good, plan, bt=4096), B.SK_ERR_INVALID_ARG))
    d = gqa_desc(layout="paged", D=128, Hq=32, Hkv=8, cap=32768)
    cases.append(("paged without table", _split(d, plan), B.SK_ERR_INVALID_ARG))
    d = gqa_desc(layout="paged", D=128, Hq=32, Hkv=8, cap=32768, page=12)
    cases.append(("page size not a power of two", _split(d, plan, bt=4096), B.SK_ERR_INVALID_ARG))
    d = gqa_desc(layout="paged", D=128, Hq=32, Hkv=8, cap=32768, max_pages=4)
    cases.append(("capacity beyond the table", _split(d, plan, bt=4096), B.SK_ERR_INVALID_ARG))
    d = gqa_desc()
    d.kv_dtype = 7
    cases.append(("unknown dtype", _split(d, plan), B.SK_ERR_INVALID_ARG))
    d = gqa_desc()
    d.layout = 5
    cases.append(("unknown layout", _split(d, plan), B.SK_ERR_INVALID_ARG))
    d = gqa_desc()
    d.scale = float("inf")
    cases.append(("infinite scale", _split(d, plan), B.SK_ERR_INVALID_ARG))
    d = gqa_desc()
    d.batch = 0
    cases.append(("zero batch", _split(d, plan), B.SK_ERR_INVALID_ARG))
    d = gqa_desc()
    d.stride_pos = 6
    cases.append(("stride not a 16-byte multiple", _split(d, plan), B.SK_ERR_UNSUPPORTED))
    d = gqa_desc()
    d.stride_pos = 128  # positions overlap (head_dim 256)
    cases.append(("overlapping positions", _split(d, plan), B.SK_ERR_INVALID_ARG))
    d = gqa_desc()
    d.stride_pos = (1 << 22) + 4  # f32: just over 16 MiB between positions
    cases.append(("position step beyond 32-bit tile offsets", _split(d, plan), B.SK_ERR_UNSUPPORTED))
    d = gqa_desc()
    d.layout, d.max_pages_per_seq, d.num_pages = B.SK_KV_INDEXED, 4096, 100000
    cases.append(("indexed without table", _split(d, plan), B.SK_ERR_INVALID_ARG))
    d.max_pages_per_seq = 100
    cases.append(("indexed: capacity beyond the table", _split(d, plan, bt=4096), B.SK_ERR_INVALID_ARG))
    d.max_pages_per_seq, d.num_pages = 4096, 0
    cases.append(("indexed: empty pool", _split(d, plan, bt=4096), B.SK_ERR_INVALID_ARG))
    d = latent_desc()
    cases.append(("v given with a shared latent", _split(d, plan, v=4096), B.SK_ERR_INVALID_ARG))
    d = latent_desc()
    d.num_kv_heads = 2
    d.num_q_heads = 96
    cases.append(("shared latent with 2 KV heads", _split(d, plan, v=None), B.SK_ERR_INVALID_ARG))
    d = latent_desc(Hq=100)
    cases.append(("latent head count", _split(d, plan, v=None), B.SK_ERR_UNSUPPORTED))
    cases.append(("combine: NULL out", _combine(good, plan, out=None), B.SK_ERR_INVALID_ARG))
    cases.append(("combine: small workspace", _combine(good, plan, wsb=64), B.SK_ERR_WORKSPACE_TOO_SMALL))
    cases.append(("combine: misaligned out", _combine(good, plan, out=4096 + 4), B.SK_ERR_INVALID_ARG))
    cases.append(("combine: zero splits", _combine(good, B.SkPlan(0, 1)), B.SK_ERR_INVALID_ARG))
    cases.append(("decode: NULL out", _decode(good, plan, out=None), B.SK_ERR_INVALID_ARG))
    cases.append(("decode: misaligned out", _decode(good, plan, out=4096 + 8), B.SK_ERR_INVALID_ARG))
    cases.append(("decode: NULL q", _decode(good, plan, q=None), B.SK_ERR_INVALID_ARG))
    cases.append(("decode: small workspace", _decode(good, plan, wsb=64), B.SK_ERR_WORKSPACE_TOO_SMALL))
    cases.append(("decode: group size 3", _decode(gqa_desc(Hq=12, Hkv=4), plan), B.SK_ERR_UNSUPPORTED))
    cases.append(("decode: latent NULL out", _decode(latent_desc(), plan, v=None, out=None),
                  B.SK_ERR_INVALID_ARG))
    cases.append(("one launch: NULL out", _one(good, plan, out=None), B.SK_ERR_INVALID_ARG))
    cases.append(("one launch: misaligned out", _one(good, plan, out=4100), B.SK_ERR_INVALID_ARG))
    cases.append(("one launch: shared latent, NULL out", _one(latent_desc(), plan, v=None, out=None),
                  B.SK_ERR_INVALID_ARG))
    cases.append(("one launch: small workspace", _one(good, plan, wsb=64), B.SK_ERR_WORKSPACE_TOO_SMALL))
    lat = latent_desc()
    cases.append(("project: NULL weights", _proj(lat, plan, w=None), B.SK_ERR_INVALID_ARG))
    cases.append(("project: misaligned weights", _proj(lat, plan, w=4096 + 4), B.SK_ERR_INVALID_ARG))
    cases.append(("project: zero rows", _proj(lat, plan, P=0), B.SK_ERR_INVALID_ARG))
    cases.append(("project: unknown weight dtype", _proj(lat, plan, wdt=9), B.SK_ERR_INVALID_ARG))
    cases.append(("project: NULL out", _proj(lat, plan, out=None), B.SK_ERR_INVALID_ARG))
    cases.append(("project: small workspace", _proj(lat, plan, wsb=64), B.SK_ERR_WORKSPACE_TOO_SMALL))
    d = latent_desc()
    d.head_dim_v = 320
    cases.append(("project: value width 320", _proj(d, plan), B.SK_ERR_UNSUPPORTED))
    L = lib()
    for name, args in (("probe: NULL buffer", (None, 1 << 20, 64, 4096, None)),
                       ("probe: misaligned buffer", (4100, 1 << 20, 64, 4096, None)),
                       ("probe: zero workgroups", (4096, 1 << 20, 0, 4096, None)),
                       ("probe: buffer too small", (4096, 64, 64, 4096, None))):
        cases.append((name, (L.attn_decode_read_probe(*args), B.attn_decode_last_error()),
                      B.SK_ERR_INVALID_ARG))
    cases.append(("init: NULL workspace", _init(good, plan, ws=None), B.SK_ERR_INVALID_ARG))
    cases.append(("init: misaligned workspace", _init(good, plan, ws=4096 + 64), B.SK_ERR_INVALID_ARG))
    cases.append(("init: small workspace", _init(good, plan, wsb=64), B.SK_ERR_WORKSPACE_TOO_SMALL))
    cases.append(("init: zero splits", _init(good, B.SkPlan(0, 1)), B.SK_ERR_INVALID_ARG))
    for name, (got, msg), want in cases:
        assert got == want, f"{name}: status {got}, expected {want} ({msg})"
        assert msg, f"{name}: no detail message"

def test_plan_argument_errors():
    lib()
    d = gqa_desc(cap=4096)
    with pytest.raises(B.SplitKVError) as e:
        B.attn_decode_plan(d, 5000, 5000, 256, 0)  # longer than the capacity
    assert e.value.status == B.SK_ERR_INVALID_ARG
    with pytest.raises(B.SplitKVError):
        B.attn_decode_plan(d, 0, 0, 256, 0)
    with pytest.raises(B.SplitKVError):
        B.attn_decode_plan(d, 100, 50, 256, 0)  # total below the maximum
    with pytest.raises(B.SplitKVError):
        B.attn_decode_plan(d, 100, 100, 0, 0)   # no compute units
    with pytest.raises(B.SplitKVError):
        B.attn_decode_plan(d, 100, 100, 256, -1)
    assert lib().attn_decode_workspace_bytes(None, None) == 0


def test_synthetic_case_descriptor_fields_round_trip():
    """The torch-side descriptor builder reads shapes and strides as documented."""
    torch = pytest.importorskip("torch")
    from split_kv_flash_amd import make_desc
    from synthetic.torch_io import to_device

    case = synthetic.gqa_case("t", seq_lens=[37, 20], num_q_heads=8, num_kv_heads=2, head_dim=64,
                              kv_dtype="f16", capacity=40, seed=1)
    t = to_device(case, "cpu")
    d = make_desc(t["q"], t["k"], t["v"], scale=case.scale)
    assert (d.batch, d.num_q_heads, d.num_kv_heads, d.head_dim_qk, d.kv_dtype) == (2, 8, 2, 64, B.SK_F16)
    assert (d.stride_seq, d.stride_pos, d.stride_head, d.max_seq_len) == (40 * 2 * 64, 128, 64, 40)
    case = synthetic.gqa_case("p", seq_lens=[37, 20], num_q_heads=8, num_kv_heads=2, head_dim=64,
                              kv_dtype="bf16", q_dtype="bf16", layout="paged", page_size=16, seed=1)
    t = to_device(case, "cpu")
    assert t["k"].dtype == torch.bfloat16
    d = make_desc(t["q"], t["k"], t["v"], scale=case.scale, block_table=t["block_table"], page_size=16)
    assert (d.layout, d.page_size, d.max_pages_per_seq, d.num_pages) == (B.SK_KV_PAGED, 16, 3, 5)


def test_host_tensors_are_refused_before_the_library_is_called():
    """The binding passes device addresses only: a host tensor raises before
    any entry point runs (a kernel would fault on a host address)."""
    import torch

    lib()
    d = gqa_desc()
    plan = B.attn_decode_plan(d, 4096, 4096, 256, 0)
    q = torch.zeros(1, 16, 256)
    with pytest.raises(B.SplitKVError) as e:
        B.attn_decode_splitk(d, plan, q, 4096, 4096, None, 4096, 4096, 1 << 30, 0)
    assert e.value.status == B.SK_ERR_INVALID_ARG and "GPU" in e.value.message
    import split_kv_flash_amd as skf

    with pytest.raises(B.SplitKVError):
        skf.decode(q, torch.zeros(1, 4096, 4, 256), torch.zeros(1, 4096, 4, 256),
                   seq_lens=torch.full((1,), 4096, dtype=torch.int32), scale=1 / 16,
                   host_seq_lens=[4096], out=torch.zeros(1, 16, 256))


# ------------------------------------------------- kernels' private memory
def _gfx950_kernels(path):
    """Kernel metadata (the AMDGPU metadata note, msgpack) of every gfx950
    code object bundled in the built library's .hip_fatbin section."""
    import struct

    import msgpack

    def sections(b):
        assert b[:4] == b"\x7fELF" and b[4] == 2
        shoff, = struct.unpack_from("<Q", b, 0x28)
        shentsize, shnum, shstrndx = struct.unpack_from("<HHH", b, 0x3A)
        raw = [struct.unpack_from("<IIQQQQ", b, shoff + i * shentsize) for i in range(shnum)]
        names = raw[shstrndx][4]
        return {b[names + r[0]:b.index(b"\0", names + r[0])].decode(): (r[1], r[4], r[5]) for r in raw}

    so = open(path, "rb").read()
    _, off, size = sections(so)[".hip_fatbin"]
    fat = so[off:off + size]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    kernels, pos = [], fat.find(magic)
    while pos >= 0:
        n, = struct.unpack_from("<Q", fat, pos + len(magic))
        p = pos + len(magic) + 8
        for _ in range(n):
            eo, es, ts = struct.unpack_from("<QQQ", fat, p)
            triple = fat[p + 24:p + 24 + ts].decode()
            p += 24 + ts
            if not triple.endswith("gfx950"):
                continue
            dev = fat[pos + eo:pos + eo + es]
            for typ, o, sz in sections(dev).values():
                q = o
                while typ == 7 and q < o + sz:  # SHT_NOTE
                    namesz, descsz, ntype = struct.unpack_from("<III", dev, q)
                    owner = dev[q + 12:q + 12 + namesz]
                    desc_at = q + 12 + ((namesz + 3) & ~3)
                    if ntype == 32 and owner.startswith(b"AMDGPU"):  # NT_AMDGPU_METADATA
                        kernels += msgpack.unpackb(dev[desc_at:desc_at + descsz], raw=False)["amdhsa.kernels"]
                    q = desc_at + ((descsz + 3) & ~3)
        pos = fat.find(magic, pos + 1)
    return kernels


# Kernels allowed a private segment, with the reason: the 96-head f16
# index-list kernel runs 12 waves (168 registers each) and spills a few of
# them; it serves only 96-head index lists beyond 128 (split, sequence)
# pairs (contiguous caches there take the dedicated-role kernel).
_SPILLS_ALLOWED = ("_ZN2sk18mla16_split_kernelILi6ELb1ELb0EEEvNS_7MlaArgsE",
                   "_ZN2sk18mla16_split_kernelILi6ELb1ELb1EEEvNS_7MlaArgsE")


def test_kernels_keep_their_state_out_of_scratch_memory():
    """Every kernel of the built library holds its state in registers and LDS:
    no private (scratch) segment and no dynamic stack. A helper the compiler
    leaves as a call puts the kernel's arguments and live registers in
    scratch for the whole kernel (the shared-latent one-launch kernel ran 142
    instead of 76 us that way), and so does a register spill."""
    lib()
    kernels = _gfx950_kernels(B.LIB_PATH)
    assert len(kernels) > 100, len(kernels)
    names = {k[".name"] for k in kernels}
    assert any("mla16d_split_kernel" in n for n in names) and any("gqa_split_kernel" in n for n in names)
    bad = [(k[".name"], k.get(".private_segment_fixed_size"), k.get(".vgpr_spill_count"))
           for k in kernels
           if (k.get(".private_segment_fixed_size", 0) or k.get(".uses_dynamic_stack"))
           and k[".name"] not in _SPILLS_ALLOWED]
    assert not bad, bad
