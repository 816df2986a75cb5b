"""Float64 reference for single-token (decode) attention and its split schedule.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the bench's
CPU-baseline leg, never by the product path. Shares no code with the HIP
library. Page keys ([L06], [I3725], [DB6], [L07]) are listed in the package
docstring.

Two layers live here:

* ``attend_f64`` is the plain definition of the result: for every sequence
  b, query head h and its KV group g, scores s_j = scale * <q_h, k_j> over the
  L_b stored positions, then softmax-weighted values, computed two-pass in
  float64 (scores and their max first, then weights, normaliser and weighted
  sum). [L07] section "Decode Starves the SMs: Split-KV, the LSE Merge, and One
  Latent for 128 Heads" states that the split merge equals full-KV softmax, so
  this definition is what the split method must reproduce up to reassociation;
  [L06] section 6 ("Testing a path your gate cannot reach") describes exactly
  such a float64 two-pass reference.
* ``split_partials_f64`` / ``merge_partials_f64`` / ``split_twin_f64`` follow
  the method's own steps in the pages' order: partition the positions into
  contiguous slices, run the online-softmax recurrence over each slice in
  tiles, emit the partial triple (m, l, acc), then rescale every partial to the
  common maximum and sum. They model the schedule, not any kernel, and exist to
  test the schedule's arithmetic and the negative controls the pages ask for.

Inputs are the *stored* values: float16 and bfloat16 arrays are widened to
float64 exactly before any arithmetic, so a comparison isolates the kernel's
arithmetic from storage rounding ([I3725] design note, section 4,
"Verification": the f16 case reads the same f16 values widened).
"""

from __future__ import annotations

import math
from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# Storage widening
# --------------------------------------------------------------------------


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen stored bfloat16 values (given as their 16-bit patterns) to float64.

    A bfloat16 value is the upper half of an IEEE-754 binary32 word, so the
    widening is exact: put the 16 stored bits into the top of a 32-bit word,
    read that word as binary32, then convert binary32 to binary64.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        b = b.view(np.uint16)
    word = b.astype(np.uint32) << np.uint32(16)
    return word.view(np.float32).astype(np.float64)


def widen(x, dtype: str) -> np.ndarray:
    """Return the stored values of ``x`` as float64.

    ``dtype`` names the storage: "f32", "f16", "f64" (numpy arrays of that
    type) or "bf16" (an array of 16-bit patterns).
    """
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype in ("f32", "f16", "f64"):
        return np.asarray(x).astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# --------------------------------------------------------------------------
# Paged addressing
# --------------------------------------------------------------------------


def gather_paged(pool, table_row: Sequence[int], length: int, page_size: int) -> np.ndarray:
    """Logical rows [0, length) of one sequence stored in a paged pool.

    [L07] section "Decode Starves the SMs ...": the kernel reaches KV through
    the block table, so position j of a sequence lives in page
    ``table_row[j // page_size]`` at slot ``j % page_size``. ``pool`` is shaped
    [pages][page_size][kv_heads][dim]; the result is [length][kv_heads][dim]
    in the pool's storage type (no arithmetic happens here).
    """
    j = np.arange(length)
    pages = np.asarray(table_row, dtype=np.int64)[j // page_size]
    if length and pages.min() < 0:
        raise ValueError("block table names an unused (negative) page inside the sequence")
    return np.asarray(pool)[pages, j % page_size]


def gather_indexed(pool, index_row: Sequence[int], length: int) -> np.ndarray:
    """Rows of one sequence named by an index list: position j is pool row
    ``index_row[j]`` for j < length.

    [L07] section "Decode Starves the SMs ..." (sparsity): the sparse decode
    path takes an indices tensor (batch, qlen, top-k) and gathers the selected
    tokens straight from the KV pool by index, materialising nothing. ``pool``
    is [rows][kv_heads][dim]; the result is [length][kv_heads][dim] in the
    pool's storage type (no arithmetic happens here).
    """
    idx = np.asarray(index_row, dtype=np.int64)[:length]
    if length and (idx.min() < 0 or idx.max() >= np.asarray(pool).shape[0]):
        raise ValueError("index list names a row outside the pool")
    return np.asarray(pool)[idx]


# --------------------------------------------------------------------------
# The definition
# --------------------------------------------------------------------------


def _group_of(h: int, num_q_heads: int, num_kv_heads: int, group_map: str) -> int:
    g = num_q_heads // num_kv_heads
    if group_map == "contiguous":
        # Query heads g*G .. g*G+G-1 share KV head g ([I3725] design note,
        # section 2: one block serves "ALL G query heads of its group").
        return h // g
    if group_map == "modulo":  # negative control only
        return h % num_kv_heads
    raise ValueError(group_map)


def _seq_rows(x, b: int, length: int, dtype: str) -> np.ndarray:
    return widen(np.asarray(x[b])[:length], dtype)


def attend_f64(
    q,
    k,
    v,
    seq_lens: Sequence[int],
    scale: float,
    *,
    q_dtype: str = "f32",
    kv_dtype: str = "f32",
    v_cols: Optional[int] = None,
    heads: Optional[Sequence[Tuple[int, int]]] = None,
    group_map: str = "contiguous",
    apply_scale: bool = True,
) -> Tuple[np.ndarray, np.ndarray]:
    """Decode attention by its definition, two-pass, in float64.

    Arguments
      q        [B][Hq][Dk] stored query values.
      k        indexable by sequence: k[b] is [>= L_b][Hkv][Dk] stored keys.
      v        like k with Dv columns, or None when keys and values share one
               latent row (multi-head latent attention in absorbed form, where
               the values are the first ``v_cols`` columns of each cached row:
               [L07] section "Decode Starves the SMs ...", 512 latent columns
               followed by 64 rotary columns).
      seq_lens L_b >= 1 for every sequence (the softmax over an empty set is
               undefined).
      scale    multiplies q.k.
      heads    optional list of (b, h) pairs to compute; other outputs stay NaN.
      group_map, apply_scale: negative-control switches only.

    Returns (out [B][Hq][Dv], lse [B][Hq]) where lse = ln sum_j exp(s_j).
    """
    qa = np.asarray(q)
    B, Hq, Dk = qa.shape
    k0 = np.asarray(k[0])
    Hkv = k0.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    if v is None:
        if v_cols is None:
            raise ValueError("v_cols is required when v is None")
        Dv = v_cols
    else:
        Dv = np.asarray(v[0]).shape[-1]
    out = np.full((B, Hq, Dv), np.nan)
    lse = np.full((B, Hq), np.nan)
    want = None if heads is None else set((int(b), int(h)) for b, h in heads)

    for b in range(B):
        L = int(seq_lens[b])
        if L < 1:
            raise ValueError("every sequence needs at least one position")
        kb = _seq_rows(k, b, L, kv_dtype)                       # [L][Hkv][Dk]
        vb = kb[..., :Dv] if v is None else _seq_rows(v, b, L, kv_dtype)
        qb = widen(qa[b], q_dtype)                               # [Hq][Dk]
        for h in range(Hq):
            if want is not None and (b, h) not in want:
                continue
            g = _group_of(h, Hq, Hkv, group_map)
            kg = np.ascontiguousarray(kb[:, g, :])
            vg = np.ascontiguousarray(vb[:, g, :])
            # Pass 1: every score, then their maximum.
            s = kg @ qb[h]
            if apply_scale:
                s = s * scale
            m = s.max()
            # Pass 2: weights relative to the maximum, normaliser, weighted sum.
            w = np.exp(s - m)
            l = w.sum()
            out[b, h] = (w @ vg) / l
            lse[b, h] = m + math.log(l)
    return out, lse


# --------------------------------------------------------------------------
# The split schedule (method steps)
# --------------------------------------------------------------------------


def plan_splits(
    seq_lens: Sequence[int],
    num_kv_heads: int,
    cu_count: int,
    n_splits: int = 0,
    *,
    kv_shared: bool = False,
    granule: int = 64,
    min_chunk: int = 64,
    blocks_per_cu=4,
    min_ctx: int = 0,
    latent_groups: int = 1,
) -> Tuple[int, int]:
    """Split count S and slice length ``chunk`` for one decode call.

    Returns (S, chunk); sequence b uses splits i = 0 .. ceil(L_b/chunk) - 1,
    split i covering positions [i*chunk, min(L_b, (i+1)*chunk)).

    * An explicit ``n_splits`` > 0 is honoured: chunk = ceil(L_max / S).
      Trailing splits may then be empty (e.g. L = 1, S = 8).
    * Below ``min_ctx`` positions no split happens (S = 1): [L06] section 2
      gates the split below a minimum context because the extra combine launch
      and global round trip cost more than the parallelism gains.
    * Otherwise the rule of [I3725] design note section 2 — chunk =
      max(64, ceil(L / S_target)), S = ceil(L / chunk) so that no split is
      empty, with S_target about 4 blocks per multiprocessor divided among the
      KV heads — is budgeted on the product of blocks, as [L06] section 5.1
      asks (KV heads x splits, summed over the sequences of a batch): chunk =
      max(min_chunk, ceil(Hkv * sum(L_b) / (blocks_per_cu * cu_count))),
      rounded up to a multiple of ``granule``. ``blocks_per_cu`` may be a
      fraction (an int or ``fractions.Fraction``; the ceiling is exact).
    * Latent attention (``kv_shared``): one block serves every query head of
      the latent (or ``latent_groups`` blocks share a split, each serving a
      slice of the heads), so the budget is one block per compute unit rather
      than four: chunk = max(min_chunk, ceil(latent_groups * sum(L_b) /
      cu_count)), rounded up to ``granule``. Each split costs a partial of all
      query heads, so fewer, longer splits keep that traffic small against the
      cache read.
    """
    lens = [int(x) for x in seq_lens]
    if not lens or min(lens) < 1:
        raise ValueError("every sequence needs at least one position")
    l_max = max(lens)
    if n_splits > 0:
        return n_splits, -(-l_max // n_splits)
    if l_max < min_ctx:
        return 1, l_max
    total = sum(lens)
    if kv_shared:
        chunk = max(min_chunk, -(-(latent_groups * total) // cu_count))
    else:
        budget = Fraction(blocks_per_cu) * cu_count
        chunk = max(min_chunk, math.ceil(Fraction(num_kv_heads * total) / budget))
    chunk = -(-chunk // granule) * granule
    return -(-l_max // chunk), chunk


def split_ranges(length: int, chunk: int, n_splits: int) -> List[Tuple[int, int]]:
    """Contiguous slices [i*chunk, min(L, (i+1)*chunk)), empty past the end.

    [L06] section 2 keeps the slices contiguous rather than strided so each
    block's walk stays sequential.
    """
    out = []
    for i in range(n_splits):
        lo = min(length, i * chunk)
        hi = min(length, (i + 1) * chunk)
        out.append((lo, hi))
    return out


def online_partial_f64(s: np.ndarray, vrows: np.ndarray, tile: int, *, alpha: bool = True):
    """Online-softmax recurrence over one slice, ``tile`` positions at a time.

    State starts at m = -inf, l = 0, acc = 0 and, for every tile, follows
    [DB6] and [L07] section "But Softmax Wants the Whole Row...":
    m_new = max(m, tile max); a = exp(m - m_new); l = a*l + sum exp(s - m_new);
    acc = a*acc + sum exp(s - m_new) v; m = m_new. The accumulator stays
    un-normalised. An empty slice returns the neutral partial
    (m = -inf, l = 0, acc = 0), whose merge weight is exactly zero ([L06]
    section 2 asks empty slices to be neutral, not NaN).

    ``alpha=False`` drops the rescale factor: a negative control only.
    """
    dv = vrows.shape[-1]
    m = -math.inf
    l = 0.0
    acc = np.zeros(dv)
    for t0 in range(0, len(s), tile):
        st = s[t0:t0 + tile]
        vt = vrows[t0:t0 + tile]
        m_new = max(m, float(st.max()))
        a = math.exp(m - m_new) if alpha else 1.0
        p = np.exp(st - m_new)
        l = a * l + p.sum()
        acc = a * acc + p @ vt
        m = m_new
    return m, l, acc


def merge_partials_f64(m, l, acc, *, rescale: bool = True):
    """Merge split partials: the combine step.

    [L06] section 2 and [I3725] design note section 2 (kernel B):
    M = max_i m_i, w_i = exp(m_i - M), l* = sum_i w_i l_i,
    out = sum_i w_i acc_i / l*. Also returns lse = M + ln l*.
    Neutral partials (m = -inf, l = 0) get weight 0.
    ``rescale=False`` drops w_i: the negative control of [L06] section 6.
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    acc = np.asarray(acc, dtype=np.float64)
    M = m.max()
    w = np.exp(m - M) if rescale else np.ones_like(m)
    lstar = (w * l).sum()
    num = (w[:, None] * acc).sum(axis=0)
    return num / lstar, M + math.log(lstar)


def merge_partials_lse_f64(m, l, acc):
    """The log-sum-exp form of the merge ([L07] section "Decode Starves the SMs").

    LSE_s = m_s + ln l_s; the weight of slice s is exp(LSE_s - LSE*) with
    LSE* = ln sum_s exp(LSE_s), applied to the normalised partial acc_s / l_s.
    Empty slices (l_s = 0) carry no mass and are left out.
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    acc = np.asarray(acc, dtype=np.float64)
    keep = l > 0
    lse_s = m[keep] + np.log(l[keep])
    top = lse_s.max()
    lse_star = top + math.log(np.exp(lse_s - top).sum())
    wt = np.exp(lse_s - lse_star)
    onorm = acc[keep] / l[keep][:, None]
    return (wt[:, None] * onorm).sum(axis=0), lse_star


def split_partials_f64(
    q,
    k,
    v,
    seq_lens: Sequence[int],
    scale: float,
    chunk: int,
    n_splits: int,
    *,
    tile: int = 32,
    q_dtype: str = "f32",
    kv_dtype: str = "f32",
    v_cols: Optional[int] = None,
    heads: Optional[Sequence[Tuple[int, int]]] = None,
    alpha: bool = True,
):
    """Per-split partial triples (m, l, acc) of the split schedule.

    Returns m, l of shape [B][Hq][S] and acc of shape [B][Hq][S][Dv]; m is the
    slice's maximum score in natural-log units (the score itself), l and acc
    are relative to that maximum. Splits past the end hold the neutral partial.
    Heads not listed in ``heads`` stay NaN.
    """
    qa = np.asarray(q)
    B, Hq, _ = qa.shape
    Hkv = np.asarray(k[0]).shape[1]
    G = Hq // Hkv
    Dv = v_cols if v is None else np.asarray(v[0]).shape[-1]
    m = np.full((B, Hq, n_splits), np.nan)
    l = np.full((B, Hq, n_splits), np.nan)
    acc = np.full((B, Hq, n_splits, Dv), np.nan)
    want = None if heads is None else set((int(b), int(h)) for b, h in heads)
    for b in range(B):
        L = int(seq_lens[b])
        kb = _seq_rows(k, b, L, kv_dtype)
        vb = kb[..., :Dv] if v is None else _seq_rows(v, b, L, kv_dtype)
        qb = widen(qa[b], q_dtype)
        for h in range(Hq):
            if want is not None and (b, h) not in want:
                continue
            g = h // G
            s = (np.ascontiguousarray(kb[:, g, :]) @ qb[h]) * scale
            vg = np.ascontiguousarray(vb[:, g, :])
            for i, (lo, hi) in enumerate(split_ranges(L, chunk, n_splits)):
                mi, li, ai = online_partial_f64(s[lo:hi], vg[lo:hi], tile, alpha=alpha)
                m[b, h, i], l[b, h, i], acc[b, h, i] = mi, li, ai
    return m, l, acc


def split_twin_f64(
    q,
    k,
    v,
    seq_lens: Sequence[int],
    scale: float,
    chunk: int,
    n_splits: int,
    *,
    tile: int = 32,
    q_dtype: str = "f32",
    kv_dtype: str = "f32",
    v_cols: Optional[int] = None,
    heads: Optional[Sequence[Tuple[int, int]]] = None,
    rescale: bool = True,
    alpha: bool = True,
):
    """Split schedule end to end: partials per slice, then the merge.

    [L06] section 6 models the split schedule on the CPU against a float64
    two-pass reference, with a negative control that removes the merge
    rescale; ``rescale`` and ``alpha`` are those switches. Only the splits that
    hold positions (the first ceil(L_b/chunk)) are merged.
    Returns (out [B][Hq][Dv], lse [B][Hq]).
    """
    m, l, acc = split_partials_f64(
        q, k, v, seq_lens, scale, chunk, n_splits, tile=tile, q_dtype=q_dtype,
        kv_dtype=kv_dtype, v_cols=v_cols, heads=heads, alpha=alpha)
    B, Hq, _ = m.shape
    out = np.full((B, Hq, acc.shape[-1]), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b in range(B):
        n_b = min(n_splits, -(-int(seq_lens[b]) // chunk))
        for h in range(Hq):
            if np.isnan(m[b, h, 0]):
                continue
            out[b, h], lse[b, h] = merge_partials_f64(
                m[b, h, :n_b], l[b, h, :n_b], acc[b, h, :n_b], rescale=rescale)
    return out, lse


# --------------------------------------------------------------------------
# Per-head output projection after the merge
# --------------------------------------------------------------------------


def project_heads_f64(out, w, w_dtype: str = "f32") -> np.ndarray:
    """Per-head projection of merged attention outputs.

    [L06] section 2 ("The output projection moves into the combine"): the
    value up-projection wv_b acts on the *merged* latent of each head, so it
    runs after the combine, never per slice. With W_h of shape [P][Dv] for
    head h, the result is y[b, h, :] = W_h @ out[b, h, :] for every sequence
    b and head h (the latent geometry of [L06] section 6 is Dv = 512, P = 128).

    ``out`` is [B][Hq][Dv] (float64), ``w`` is [Hq][P][Dv] in the named
    storage type (widened exactly). Returns [B][Hq][P] float64.
    """
    o = np.asarray(out, dtype=np.float64)
    W = widen(w, w_dtype)
    B, Hq, Dv = o.shape
    if W.shape[0] != Hq or W.shape[2] != Dv:
        raise ValueError(f"weights {W.shape} do not match outputs {o.shape}")
    y = np.empty((B, Hq, W.shape[1]))
    for h in range(Hq):
        y[:, h, :] = o[:, h, :] @ W[h].T
    return y


def project_per_slice_f64(m, l, acc, n_used: int, w_h, w_dtype: str = "f32",
                          *, normalised_mean: bool = False) -> np.ndarray:
    """Projection applied to each slice's partial before the merge, for one head.

    With ``normalised_mean=False`` each slice's un-normalised accumulator is
    projected and the projected partials are merged with the combine's own
    weights exp(m_i - M) and normaliser: because W is linear this equals the
    projection of the merged output exactly (up to rounding), at n_used times
    the projection work. ``normalised_mean=True`` is the mistake [L06] section
    2 warns about: project each slice's normalised output acc_i / l_i and
    average the slices with equal weights, ignoring their maxima and masses.
    """
    m = np.asarray(m, dtype=np.float64)[:n_used]
    l = np.asarray(l, dtype=np.float64)[:n_used]
    acc = np.asarray(acc, dtype=np.float64)[:n_used]
    W = widen(w_h, w_dtype)
    proj = acc @ W.T  # [n_used][P]
    if normalised_mean:
        return (proj / l[:, None]).mean(axis=0)
    M = m.max()
    wt = np.exp(m - M)
    return (wt[:, None] * proj).sum(axis=0) / (wt * l).sum()


# --------------------------------------------------------------------------
# Several query positions per sequence (query tiles)
# --------------------------------------------------------------------------


def causal_limits(seq_len: int, q_len: int) -> np.ndarray:
    """Positions visible to each of the q_len newest queries of a sequence of
    seq_len positions: query t sits at position seq_len - q_len + t and sees
    positions [0, seq_len - q_len + t] (causal attention, [DB6])."""
    return np.asarray([seq_len - q_len + t + 1 for t in range(q_len)], dtype=np.int64)


def attend_multiquery_f64(q, k, v, seq_lens: Sequence[int], scale: float, *,
                          q_dtype: str = "f32", kv_dtype: str = "f32", causal: bool = True,
                          heads: Optional[Sequence[Tuple[int, int, int]]] = None):
    """Causal attention of the q_len newest positions of every sequence.

    q is [B][Q][Hq][Dk]; query t of sequence b attends positions
    [0, L_b - Q + t] by the definition (``attend_f64`` with that length), so
    Q = 1 is single-token decode and Q = L_b is causal self-attention over the
    whole sequence ([DB6]: every query row carries its own running max,
    normaliser and accumulator over the tiles it can see). ``causal=False``
    (every query sees all L_b positions) is a negative control only.
    ``heads`` optionally lists (b, t, h) triples to compute. Returns
    (out [B][Q][Hq][Dv], lse [B][Q][Hq]).
    """
    qa = np.asarray(q)
    B, Q, Hq, _ = qa.shape
    Dv = np.asarray(v[0]).shape[-1]
    out = np.full((B, Q, Hq, Dv), np.nan)
    lse = np.full((B, Q, Hq), np.nan)
    want = None if heads is None else set((int(b), int(t), int(h)) for b, t, h in heads)
    for b in range(B):
        L = int(seq_lens[b])
        lims = causal_limits(L, Q) if causal else np.full(Q, L)
        for t in range(Q):
            if lims[t] < 1:
                continue  # no visible position: undefined, left NaN
            hs = [h for h in range(Hq) if want is None or (b, t, h) in want]
            if not hs:
                continue
            o, s = attend_f64(qa[b:b + 1, t], [np.asarray(k[b])], [np.asarray(v[b])],
                              [int(lims[t])], scale, q_dtype=q_dtype, kv_dtype=kv_dtype,
                              heads=[(0, h) for h in hs])
            out[b, t, hs] = o[0, hs]
            lse[b, t, hs] = s[0, hs]
    return out, lse


def query_tile_twin_f64(q, k, v, seq_lens: Sequence[int], scale: float, *, tile: int = 32,
                        q_dtype: str = "f32", kv_dtype: str = "f32", alpha: bool = True):
    """The query-tile schedule of [DB6] for one call: every query row walks the
    K/V tiles of ``tile`` positions it can see, carrying (m, l, acc) with the
    per-tile rescale alpha = exp(m_old - m_new), and divides by l at the end.
    ``alpha=False`` drops the rescale (the negative control [DB6] names: wrong
    as soon as the running maximum moves between tiles). Returns out
    [B][Q][Hq][Dv]."""
    qa = np.asarray(q)
    B, Q, Hq, _ = qa.shape
    Hkv = np.asarray(k[0]).shape[1]
    G = Hq // Hkv
    Dv = np.asarray(v[0]).shape[-1]
    out = np.full((B, Q, Hq, Dv), np.nan)
    for b in range(B):
        L = int(seq_lens[b])
        kb = widen(np.asarray(k[b])[:L], kv_dtype)
        vb = widen(np.asarray(v[b])[:L], kv_dtype)
        qb = widen(qa[b], q_dtype)
        for t, lim in enumerate(causal_limits(L, Q)):
            if lim < 1:
                continue
            for h in range(Hq):
                g = h // G
                s = (kb[:lim, g, :] @ qb[t, h]) * scale
                m, l, acc = online_partial_f64(s, vb[:lim, g, :], tile, alpha=alpha)
                out[b, t, h] = acc / l
    return out
