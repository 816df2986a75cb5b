"""Seeded synthetic decode-attention workloads.

The one module that both sides of a parity check read: the tests, the bench
and the smoke check draw their inputs here, then hand the same stored arrays
to the HIP library and to the float64 oracle. It holds none of the method's
arithmetic: it draws normal numbers, rounds them to the storage type, and
lays them out (contiguous token-major rows, or a paged pool behind a
shuffled block table).

Recipe (the shapes are the ones the pages discuss; no dataset is involved):

* ``numpy.random.SeedSequence(seed)`` spawns one child stream per role
  (q, K, V, lengths, page permutation, peaked positions); a large tensor is
  drawn in fixed row chunks, each from its own grandchild stream, so the
  values depend only on (seed, shape) and can be drawn on several threads.
* Values are float32 standard normals, rounded to the storage type with
  round-to-nearest-even (torch's ``.to``); bfloat16 arrays are kept as their
  16-bit patterns (numpy has no bfloat16).
* Positions past a sequence's length (contiguous padding, unused slots of a
  sequence's last page) are filled with NaN, so any read past the end turns
  into a NaN in the output.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

ROLE_Q, ROLE_K, ROLE_V, ROLE_LENS, ROLE_PERM, ROLE_PEAKS = range(6)
_CHUNK_ELEMS = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rows_split(shape: Sequence[int]):
    """Rows are the leading axes down to the last two (positions); each holds
    prod(shape[-2:]) elements. Chunks hold about 4M elements."""
    shape = tuple(int(s) for s in shape)
    lead = int(np.prod(shape[:-2])) if len(shape) > 2 else shape[0]
    inner = int(np.prod(shape)) // max(1, lead)
    per = max(1, _CHUNK_ELEMS // max(1, inner))
    return shape, lead, inner, list(range(0, lead, per)), per


def draw(ss: np.random.SeedSequence, shape: Sequence[int], dtype: str = "f32",
         row_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """N(0,1) float32 draws rounded to ``dtype``, in fixed row chunks.

    Each chunk of rows comes from its own child stream of ``ss``, so the values
    depend only on (seed, shape) and chunks can be drawn on several threads.
    ``row_scale`` (one float32 per row) multiplies rows before rounding.
    """
    shape, lead, inner, starts, per = _rows_split(shape)
    np_dtype = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    out = np.empty(shape, dtype=np_dtype)
    if out.size == 0:
        return out
    flat = out.reshape(lead, inner)
    kids = ss.spawn(len(starts))

    def fill(i):
        r0 = starts[i]
        r1 = min(lead, r0 + per)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        x = g.standard_normal(size=(r1 - r0, inner), dtype=np.float32)
        if row_scale is not None:
            x *= row_scale[r0:r1, None]
        flat[r0:r1] = to_storage(x, dtype)

    if len(starts) == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(len(starts))))
    return out


def normal_f32(ss: np.random.SeedSequence, shape: Sequence[int]) -> np.ndarray:
    """float32 N(0,1) array (see ``draw``)."""
    return draw(ss, shape, "f32")


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage type (nearest even)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def nan_value(dtype: str):
    """The NaN used to poison padding, in the storage type's representation."""
    if dtype == "bf16":
        return np.uint16(0x7FC0)
    return np.nan


@dataclass
class Case:
    """One decode-attention call's inputs, as stored arrays on the host.

    Layouts (all row-major):
      q           [B][Hq][Dk]
      contiguous  k, v: [B][cap][Hkv][D] (token-major); v is None when the
                  values are the first ``head_dim_v`` columns of k
      paged       k, v: pools [pages][page_size][Hkv][D]; block_table
                  [B][max_pages] int32 (-1 = unused)
    """

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    kv_shared: bool
    scale: float
    q_dtype: str
    kv_dtype: str
    layout: str
    q: np.ndarray
    k: np.ndarray
    v: Optional[np.ndarray]
    seq_lens: np.ndarray
    block_table: Optional[np.ndarray] = None
    page_size: int = 0
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def capacity(self) -> int:
        if self.layout == "paged":
            return self.block_table.shape[1] * self.page_size
        if self.layout == "indexed":
            return self.block_table.shape[1]
        return self.k.shape[1]

    def kv_bytes(self) -> int:
        """Bytes of K and V the call must read once (positions < L_b only)."""
        b = 4 if self.kv_dtype == "f32" else 2
        per_pos = self.num_kv_heads * (self.head_dim_qk + (0 if self.kv_shared else self.head_dim_v)) * b
        return int(self.seq_lens.astype(np.int64).sum()) * per_pos

    def k_rows(self) -> List[np.ndarray]:
        """Per-sequence [L_b][Hkv][Dk] stored keys, gathered through the block table."""
        return self._rows(self.k)

    def v_rows(self) -> Optional[List[np.ndarray]]:
        return None if self.v is None else self._rows(self.v)

    def _rows(self, x) -> List[np.ndarray]:
        rows = []
        for b in range(self.batch):
            L = int(self.seq_lens[b])
            if self.layout == "paged":
                ps = self.page_size
                j = np.arange(L)
                rows.append(x[self.block_table[b][j // ps], j % ps])
            elif self.layout == "indexed":
                rows.append(x[self.block_table[b][:L]])
            else:
                rows.append(x[b, :L])
        return rows


def _spawn(seed: int):
    return np.random.SeedSequence(seed).spawn(6)


def gqa_case(
    name: str,
    *,
    seq_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    q_dtype: str = "f32",
    kv_dtype: str = "f32",
    layout: str = "contiguous",
    page_size: int = 16,
    capacity: Optional[int] = None,
    seed: int = 0,
    scale: Optional[float] = None,
    peaky_fraction: float = 0.0,
    peaky_factor: float = 8.0,
) -> Case:
    """A grouped-query decode call: q, K, V ~ N(0,1), optional peaked keys.

    ``peaky_fraction`` > 0 picks floor(fraction * L) positions per sequence
    without replacement and multiplies their key rows (all KV heads) by
    ``peaky_factor`` in float32, before rounding to the storage type.
    """
    lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(lens)
    kids = _spawn(seed)
    D = head_dim
    q = draw(kids[ROLE_Q], (B, num_q_heads, D), q_dtype)
    l_max = int(lens.max())
    peaks = np.random.Generator(np.random.PCG64(kids[ROLE_PEAKS]))
    if layout == "contiguous":
        cap = l_max if capacity is None else int(capacity)
        assert cap >= l_max
        row_scale = None
        if peaky_fraction > 0:
            row_scale = np.ones(B * cap, dtype=np.float32)
            for b in range(B):
                L = int(lens[b])
                pos = peaks.choice(L, size=int(math.floor(peaky_fraction * L)), replace=False)
                row_scale[b * cap + pos] = np.float32(peaky_factor)
        k = draw(kids[ROLE_K], (B, cap, num_kv_heads, D), kv_dtype, row_scale)
        v = draw(kids[ROLE_V], (B, cap, num_kv_heads, D), kv_dtype)
        for b in range(B):
            k[b, lens[b]:] = nan_value(kv_dtype)
            v[b, lens[b]:] = nan_value(kv_dtype)
        table = None
        ps = 0
    elif layout == "paged":
        ps = int(page_size)
        n_pages = [-(-int(L) // ps) for L in lens]
        P = int(sum(n_pages))
        cap = l_max if capacity is None else int(capacity)
        max_pages = -(-cap // ps)
        perm = np.random.Generator(np.random.PCG64(kids[ROLE_PERM])).permutation(P)
        table = np.full((B, max_pages), -1, dtype=np.int32)
        off = 0
        for b in range(B):
            table[b, :n_pages[b]] = perm[off:off + n_pages[b]]
            off += n_pages[b]
        row_scale = None
        if peaky_fraction > 0:
            row_scale = np.ones(P * ps, dtype=np.float32)
            for b in range(B):
                L = int(lens[b])
                pos = peaks.choice(L, size=int(math.floor(peaky_fraction * L)), replace=False)
                row_scale[table[b][pos // ps].astype(np.int64) * ps + pos % ps] = np.float32(peaky_factor)
        k = draw(kids[ROLE_K], (P, ps, num_kv_heads, D), kv_dtype, row_scale)
        v = draw(kids[ROLE_V], (P, ps, num_kv_heads, D), kv_dtype)
        for b in range(B):
            L = int(lens[b])
            if L % ps:
                last = table[b][n_pages[b] - 1]
                k[last, L % ps:] = nan_value(kv_dtype)
                v[last, L % ps:] = nan_value(kv_dtype)
    else:
        raise ValueError(layout)
    return Case(
        name=name, batch=B, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim_qk=D, head_dim_v=D, kv_shared=False,
        scale=(1.0 / math.sqrt(D)) if scale is None else float(scale),
        q_dtype=q_dtype, kv_dtype=kv_dtype, layout=layout, q=q, k=k, v=v,
        seq_lens=lens, block_table=table, page_size=ps, seed=seed,
        meta={"peaky_fraction": peaky_fraction},
    )


def latent_case(
    name: str,
    *,
    seq_len: int,
    kv_dtype: str = "f32",
    num_q_heads: int = 96,
    latent_dim: int = 576,
    value_dim: int = 512,
    capacity: Optional[int] = None,
    seed: int = 0,
    scale: Optional[float] = None,
) -> Case:
    """Latent (MLA-as-MQA) decode: every query head attends one shared row of
    ``latent_dim`` columns per position; values are its first ``value_dim``."""
    kids = _spawn(seed)
    cap = seq_len if capacity is None else int(capacity)
    q = draw(kids[ROLE_Q], (1, num_q_heads, latent_dim), "f32")
    c = draw(kids[ROLE_K], (1, cap, 1, latent_dim), kv_dtype)
    c[0, seq_len:] = nan_value(kv_dtype)
    return Case(
        name=name, batch=1, num_q_heads=num_q_heads, num_kv_heads=1,
        head_dim_qk=latent_dim, head_dim_v=value_dim, kv_shared=True,
        scale=(1.0 / math.sqrt(latent_dim)) if scale is None else float(scale),
        q_dtype="f32", kv_dtype=kv_dtype, layout="contiguous", q=q, k=c, v=None,
        seq_lens=np.asarray([seq_len], dtype=np.int32), seed=seed,
    )


# ----- The five workloads, by what they are ----------------------------------


def tiny_gqa(seq_len: int, seed: int = 1000, capacity: Optional[int] = None) -> Case:
    """Tiny GQA: batch 1, 4 query heads on 1 KV head, head_dim 64, f32."""
    return gqa_case(f"tiny-gqa-L{seq_len}", seq_lens=[seq_len], num_q_heads=4,
                    num_kv_heads=1, head_dim=64, seed=seed, capacity=capacity)


def qwen9b_like(seq_len: int, kv_dtype: str = "f32", seed: int = 2000,
                capacity: Optional[int] = None) -> Case:
    """9B-like full-attention layer: 16 query / 4 KV heads, head_dim 256,
    q f32, K/V stored f32 or f16."""
    return gqa_case(f"gqa16x4-d256-{kv_dtype}-L{seq_len}", seq_lens=[seq_len],
                    num_q_heads=16, num_kv_heads=4, head_dim=256, kv_dtype=kv_dtype,
                    seed=seed, capacity=capacity)


def latent_decode(seq_len: int, kv_dtype: str = "f32", seed: int = 3000) -> Case:
    """Latent attention: 96 query heads, one 576-column latent, 512 value columns."""
    return latent_case(f"mla96-576-{kv_dtype}-L{seq_len}", seq_len=seq_len,
                       kv_dtype=kv_dtype, seed=seed, scale=1.0 / 24.0)


def ragged_lengths(seed: int = 4000, batch: int = 32, lo: int = 1024, hi: int = 32768) -> np.ndarray:
    """Integer lengths uniform on [lo, hi], both ends inclusive."""
    g = np.random.Generator(np.random.PCG64(_spawn(seed)[ROLE_LENS]))
    return g.integers(lo, hi, endpoint=True, size=batch).astype(np.int32)


def ragged_paged(seed: int = 4000, batch: int = 32, lo: int = 1024, hi: int = 32768) -> Case:
    """Ragged batch: 32 sequences, lengths uniform on [lo, hi] (both ends
    inclusive), 32 query / 8 KV heads, head_dim 128, bf16 q and KV in
    16-token pages behind a shuffled block table."""
    lens = ragged_lengths(seed, batch, lo, hi)
    return gqa_case(f"ragged{batch}-gqa32x8-d128-bf16-paged16", seq_lens=lens,
                    num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16",
                    kv_dtype="bf16", layout="paged", page_size=16, capacity=hi,
                    seed=seed)


def wide_group_peaky(seq_len: int = 262144, seed: int = 5000) -> Case:
    """27B-like wide group: 24 query / 4 KV heads, head_dim 256, f16 KV with
    1% of positions' keys scaled by 8 (peaked softmax), q f32."""
    return gqa_case(f"gqa24x4-d256-f16-peaky-L{seq_len}", seq_lens=[seq_len],
                    num_q_heads=24, num_kv_heads=4, head_dim=256, kv_dtype="f16",
                    seed=seed, peaky_fraction=0.01)


def projection_weights(num_heads: int, out_dim: int, in_dim: int, dtype: str = "f32",
                       seed: int = 6000) -> np.ndarray:
    """Per-head projection matrices [num_heads][out_dim][in_dim]: float32
    N(0,1) draws times 1/sqrt(in_dim) (so that a unit-scale input gives a
    unit-scale output), rounded to ``dtype``. The latent geometry uses
    in_dim = 512 (the merged latent) and out_dim = 128."""
    w = normal_f32(np.random.SeedSequence(seed), (num_heads, out_dim, in_dim))
    return to_storage(w * np.float32(1.0 / math.sqrt(in_dim)), dtype)


def indexed_case(
    name: str,
    *,
    pool_rows: int,
    seq_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    kv_dtype: str = "f32",
    q_dtype: str = "f32",
    latent_value_dim: Optional[int] = None,
    max_indices: Optional[int] = None,
    seed: int = 0,
    scale: Optional[float] = None,
) -> Case:
    """Sparse (top-k) decode: every sequence attends the pool rows named by its
    index list. The pool holds ``pool_rows`` rows [rows][Hkv][D] (the whole
    cache of one request, or a paged pool of physical slots); sequence b's list
    has seq_lens[b] distinct rows in random order (a top-k selection is not
    sorted), padded with -1 to ``max_indices``. With ``latent_value_dim`` the
    pool is a shared latent (one row of ``head_dim`` columns, values are its
    first ``latent_value_dim``)."""
    kids = _spawn(seed)
    lens = np.asarray(seq_lens, dtype=np.int32)
    width = int(max_indices or lens.max())
    latent = latent_value_dim is not None
    hkv = 1 if latent else num_kv_heads
    q = draw(kids[ROLE_Q], (len(lens), num_q_heads, head_dim), q_dtype)
    k = draw(kids[ROLE_K], (pool_rows, hkv, head_dim), kv_dtype)
    v = None if latent else draw(kids[ROLE_V], (pool_rows, hkv, head_dim), kv_dtype)
    rng = np.random.default_rng(kids[ROLE_PERM])
    table = np.full((len(lens), width), -1, dtype=np.int32)
    for b, L in enumerate(lens):
        table[b, :L] = rng.choice(pool_rows, size=int(L), replace=False)
    return Case(
        name=name, batch=len(lens), num_q_heads=num_q_heads, num_kv_heads=hkv,
        head_dim_qk=head_dim, head_dim_v=latent_value_dim if latent else head_dim,
        kv_shared=latent,
        scale=(1.0 / math.sqrt(head_dim)) if scale is None else float(scale),
        q_dtype=q_dtype, kv_dtype=kv_dtype, layout="indexed", q=q, k=k, v=v, seq_lens=lens,
        block_table=table, page_size=1, seed=seed,
    )


def dsa_latent(topk: int = 2048, pool_rows: int = 131072, kv_dtype: str = "f16",
               seed: int = 8000) -> Case:
    """Sparse latent decode as the DSA chain runs it: 96 query heads over one
    576-column latent row per position (512 value columns), the top-k rows of
    a 131,072-row cache selected by an index list."""
    return indexed_case(f"dsa-latent96-{kv_dtype}-top{topk}-of{pool_rows}", pool_rows=pool_rows,
                        seq_lens=[topk], num_q_heads=96, num_kv_heads=1, head_dim=576,
                        kv_dtype=kv_dtype, latent_value_dim=512, seed=seed, scale=1.0 / 24.0)


def multiquery_case(
    name: str,
    *,
    seq_lens: Sequence[int],
    q_len: int,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    kv_dtype: str = "f16",
    q_dtype: str = "f32",
    capacity: Optional[int] = None,
    seed: int = 0,
) -> Case:
    """The q_len newest positions of every sequence query its cache at once
    (speculative verify, chunked prefill, causal self-attention when
    q_len = L): q is [B][q_len][Hq][D]; K/V are token-major [B][cap][Hkv][D]
    with NaN past each length."""
    kids = _spawn(seed)
    lens = np.asarray(seq_lens, dtype=np.int32)
    cap = int(capacity or lens.max())
    B = len(lens)
    q = draw(kids[ROLE_Q], (B, q_len, num_q_heads, head_dim), q_dtype)
    k = draw(kids[ROLE_K], (B, cap, num_kv_heads, head_dim), kv_dtype)
    v = draw(kids[ROLE_V], (B, cap, num_kv_heads, head_dim), kv_dtype)
    for b, L in enumerate(lens):
        k[b, L:] = nan_value(kv_dtype)
        v[b, L:] = nan_value(kv_dtype)
    return Case(
        name=name, batch=B, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim_qk=head_dim, head_dim_v=head_dim, kv_shared=False,
        scale=1.0 / math.sqrt(head_dim), q_dtype=q_dtype, kv_dtype=kv_dtype,
        layout="contiguous", q=q, k=k, v=v, seq_lens=lens, seed=seed, meta={"q_len": q_len},
    )


def causal_block(seq_len: int = 2048, kv_dtype: str = "f16", seed: int = 8100) -> Case:
    """Causal self-attention over a whole sequence with head_dim 64, the
    teaching decoder block's shape (4 heads of 64, 2048 tokens)."""
    return multiquery_case(f"causal-block4x64-{kv_dtype}-L{seq_len}", seq_lens=[seq_len],
                           q_len=seq_len, num_q_heads=4, num_kv_heads=4, head_dim=64,
                           kv_dtype=kv_dtype, seed=seed)


def spec_verify(seq_len: int = 131072, q_len: int = 4, kv_dtype: str = "f16",
                seed: int = 8200) -> Case:
    """Speculative verify on the 9B-like layer: q_len drafted tokens at the end
    of a seq_len-position cache (16 query / 4 KV heads, head_dim 256)."""
    return multiquery_case(f"verify{q_len}-gqa16x4-d256-{kv_dtype}-L{seq_len}", seq_lens=[seq_len],
                           q_len=q_len, num_q_heads=16, num_kv_heads=4, head_dim=256,
                           kv_dtype=kv_dtype, seed=seed)


def chunked_prefill(seq_len: int = 8192, q_len: int = 512, kv_dtype: str = "f16",
                    seed: int = 8300) -> Case:
    """Chunked prefill on the 9B-like layer: the last q_len positions of a
    seq_len-position sequence (16 query / 4 KV heads, head_dim 256)."""
    return multiquery_case(f"prefill{q_len}-gqa16x4-d256-{kv_dtype}-L{seq_len}", seq_lens=[seq_len],
                           q_len=q_len, num_q_heads=16, num_kv_heads=4, head_dim=256,
                           kv_dtype=kv_dtype, seed=seed)
