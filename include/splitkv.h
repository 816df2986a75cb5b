/*
 * splitkv.h — C ABI of a split-KV ("flash-decoding") decode-attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * One decode call computes, for every sequence b and query head h (reading
 * KV head g = h / (num_q_heads / num_kv_heads)), single-token attention over
 * the L_b cached positions:
 *
 *     s_j = scale * <q[b,h,:], K[b,g,j,:]>          j = 0 .. L_b - 1
 *     out[b,h,:] = sum_j exp(s_j - m) V[b,g,j,:] / sum_j exp(s_j - m),
 *     m = max_j s_j,   lse[b,h] = m + ln sum_j exp(s_j - m)
 *
 * either in two launches, as the pages describe the method, or in one:
 *
 *   attn_decode_splitk   One workgroup per (sequence, KV head or shared
 *                        latent, context split) runs the online-softmax
 *                        recurrence over one contiguous slice of positions
 *                        and writes the partial triple (m, l, acc) of every
 *                        query head it serves ("Part 4 · Lecture 06 —
 *                        Attention at 128k", section 2 "Split over context";
 *                        aprender issue #3725 design note, section 2, kernel
 *                        A; "The Kernel Level: Attention and MoE", section
 *                        "Decode Starves the SMs: Split-KV, the LSE Merge, and
 *                        One Latent for 128 Heads").
 *   attn_decode_combine  Rescales the partials of each (sequence, query head)
 *                        to their common maximum and sums them (Lecture 06
 *                        section 2: M = max m_i, l = sum l_i exp(m_i - M),
 *                        acc = sum acc_i exp(m_i - M); issue #3725 design
 *                        note section 2, kernel B).
 *   attn_decode          Both steps in one call (the two kernels back to back).
 *   attn_decode_one_launch
 *                        Both steps in one launch, for separate K and V: the
 *                        last workgroup of each (sequence, KV head) to finish
 *                        performs the combine of that group's query heads.
 *                        It exists for callers that need one kernel per call;
 *                        on MI355X it measured slower than the two launches
 *                        enqueued back to back (the combine's launch overlaps
 *                        the split kernel, while the in-grid merge waits for
 *                        device-scope round trips at the end of the grid).
 *   attn_decode_no_alloc attn_decode with the partials in a scratch array the
 *                        library holds per device, for callers that cannot
 *                        allocate.
 *
 * Conventions shared by every call
 *   - Pointers named "device" are device memory on the device that owns
 *     `stream`; the library never dereferences them on the host.
 *   - The caller owns every buffer, including the workspace. The library
 *     allocates nothing and keeps no global or per-device state, so calls are
 *     re-entrant and safe from several host threads and devices (Lecture 06
 *     section 2 explains why scratch must be per device, never one static
 *     pointer shared by several devices). The one exception is
 *     attn_decode_no_alloc, which keeps its partials in a fixed array of its
 *     own on each device.
 *   - Arguments are validated before any HIP call. A failed validation
 *     returns SK_ERR_INVALID_ARG, SK_ERR_UNSUPPORTED or
 *     SK_ERR_WORKSPACE_TOO_SMALL and launches nothing.
 *   - Every launch is followed by hipGetLastError(); a failure returns
 *     SK_ERR_LAUNCH, so a bad launch is reported by the call that made it
 *     and not by some later call (Lecture 06 section 5.3, "The launch guard").
 *     attn_decode_last_error() returns the detail text for the calling thread.
 *   - Launches are asynchronous on `stream`; results are valid once the stream
 *     has completed them. Nothing synchronises inside the library.
 *   - Plan-time inputs are two host integers; lengths are read on the device,
 *     so pointers and shapes stay fixed across decode steps.
 */
#ifndef SPLITKV_H
#define SPLITKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SK_OK = 0,
  SK_ERR_INVALID_ARG = 1,         /* null pointer, bad size, inconsistent descriptor or plan */
  SK_ERR_UNSUPPORTED = 2,         /* valid request with no kernel for it; nothing runs       */
  SK_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < attn_decode_workspace_bytes(...)       */
  SK_ERR_LAUNCH = 4,              /* hipGetLastError() failed right after a launch            */
  SK_ERR_HIP = 5                  /* another HIP runtime call failed                           */
} sk_status_t;

/* Element types. q and KV may be any of them; out, lse and the workspace are f32. */
typedef enum { SK_F32 = 0, SK_F16 = 1, SK_BF16 = 2 } sk_dtype_t;

/* KV cache layouts. */
typedef enum {
  /* K and V are separate buffers addressed as
   *   base + b*stride_seq + j*stride_pos + g*stride_head + d      (elements),
   * d contiguous. The usual token-major cache [batch][capacity][Hkv][D] has
   * stride_seq = capacity*Hkv*D, stride_pos = Hkv*D, stride_head = D
   * (issue #3725 design note section 1 reads this layout). Strides are
   * multiples of 16 bytes and stride_pos spans at most 16 MiB.                 */
  SK_KV_CONTIGUOUS = 0,
  /* K and V are pools [num_pages][page_size][Hkv][D]; position j of sequence b
   * lives in page block_table[b*max_pages_per_seq + j/page_size], slot
   * j % page_size ("The Kernel Level: Attention and MoE": the kernel indexes
   * KV through the block table; the table pointer stays fixed across steps). */
  SK_KV_PAGED = 1,
  /* Sparse (top-k) decode over an index list: K and V (or the shared latent) are row
   * pools of num_pages rows, row r of KV head g at base + r*stride_pos + g*stride_head
   * + d (elements; strides as for SK_KV_CONTIGUOUS, stride_seq unused); position j of
   * sequence b is row block_table[b*max_pages_per_seq + j], j < L_b ("The Kernel Level:
   * Attention and MoE", sparsity: the decode kernel takes an indices tensor (batch,
   * qlen, top-k) and gathers the selected tokens from the pool by index). page_size is
   * unused; max_seq_len <= max_pages_per_seq. An index outside [0, num_pages) is never
   * followed: its position scores NaN, so that head's output is NaN.                   */
  SK_KV_INDEXED = 2
} sk_kv_layout_t;

/* Shape and layout of one decode call. Plain data; the caller fills it. */
typedef struct {
  int32_t batch;            /* B >= 1                                                   */
  int32_t num_q_heads;      /* Hq >= 1, a multiple of num_kv_heads                       */
  int32_t num_kv_heads;     /* Hkv >= 1; 1 when kv_shared                                */
  int32_t head_dim_qk;      /* Dk: key width (GQA: 64, 128, 256; latent: 576)            */
  int32_t head_dim_v;       /* Dv: value width (GQA: equal to Dk; latent: <= Dk, e.g. 512) */
  int32_t kv_shared;        /* 1: values are columns [0, Dv) of the key rows (multi-head
                               latent attention in absorbed form, "The Kernel Level:
                               Attention and MoE": a 512-column latent followed by 64
                               rotary columns); `v` must then be NULL                    */
  float scale;              /* multiplies q.k (usually 1/sqrt(Dk))                       */
  int32_t q_dtype;          /* sk_dtype_t of q                                          */
  int32_t kv_dtype;         /* sk_dtype_t of K and V                                     */
  int32_t layout;           /* sk_kv_layout_t                                           */
  int32_t max_seq_len;      /* capacity per sequence in positions: contiguous rows
                               readable per sequence; paged: <= max_pages_per_seq*page_size */
  int32_t page_size;        /* paged: positions per page, a power of two                 */
  int32_t max_pages_per_seq;/* paged: row length of block_table                          */
  int64_t num_pages;        /* paged: pages in each pool                                 */
  int64_t stride_seq;       /* contiguous: elements between sequences                    */
  int64_t stride_pos;       /* contiguous: elements between consecutive positions       */
  int64_t stride_head;      /* contiguous: elements between KV heads                     */
} sk_desc_t;

/* How the context axis is cut. Split i of sequence b covers positions
 * [i*chunk, min(L_b, (i+1)*chunk)); sequence b uses splits 0 .. ceil(L_b/chunk)-1
 * and splits past those are empty (their workgroups write the neutral partial
 * m = -inf, l = 0, acc = 0 and read nothing). */
typedef struct {
  int32_t n_splits; /* S: split slots per (sequence, KV head); workspace is sized by it */
  int32_t chunk;    /* positions per split                                                */
} sk_plan_t;

/* Choose S and chunk (host only; no HIP call).
 *   max_seq_len         longest L_b of this call (>= 1)
 *   total_tokens        sum of L_b over the batch (>= max_seq_len)
 *   cu_count            compute units of the device (hipDeviceProp_t.multiProcessorCount)
 *   n_splits_requested  > 0: honoured exactly, chunk = ceil(max_seq_len / S) (trailing
 *                       splits may be empty); 0: heuristic.
 * Heuristic (issue #3725 design note section 2: chunk = max(64, ceil(L/S_target)) and
 * S = ceil(L/chunk) so that no split is empty; budgeted on the product of KV heads and
 * splits summed over the batch, as Lecture 06 section 5.1 asks):
 *   GQA:    chunk = max(64, ceil(Hkv * total_tokens / (k * cu_count))), where k is the
 *           number of workgroups per compute unit measured best on MI355X: 1 (one
 *           round of one workgroup per compute unit), 8 for a ragged batch
 *           (total_tokens < batch * max_seq_len). For a batch that is not ragged,
 *           when that chunk is at least 1024 positions, k becomes 3/4 (192
 *           concurrent sequential readers stream HBM faster than 256), except
 *           for the f16 6-head group of width 256, whose VALU-heavy loop needs
 *           every compute unit. The note's own S_target is about 4 per
 *           multiprocessor of its GPU.
 *   GQA on the query-tile kernel (f16/bf16 KV: head width 64; width 128 with at least 4
 *           query heads per KV head; width 256 with at least 6; see
 *           attn_decode_splitk): the attn_query_tiles_plan rule with one query,
 *           k = 1, 2 or 4 workgroups per compute unit at width 256, 128 or 64, and
 *           8 for a ragged batch.
 *   latent: chunk = max(64, ceil(g * total_tokens / cu_count)) with g workgroups per
 *           split, each serving a slice of the query heads: for f16 caches 1 up to
 *           96 heads and 2 (of 64 heads) at 128; for f32 caches Hq/48 (Hq/32 when
 *           48 does not divide Hq), whose kernel holds fewer heads per workgroup.
 *           Each split costs a partial of every head, so splits stay long.
 *   chunk is rounded up to a multiple of 64 and S = ceil(max_seq_len / chunk).
 * Below SK_MIN_SPLIT_CONTEXT positions the heuristic returns S = 1 (Lecture 06
 * section 2 gates the split below a minimum context).
 * Errors: SK_ERR_INVALID_ARG for null pointers or non-positive sizes. */
#define SK_MIN_SPLIT_CONTEXT 0
sk_status_t attn_decode_plan(const sk_desc_t* desc, int32_t max_seq_len, int64_t total_tokens,
                             int32_t cu_count, int32_t n_splits_requested, sk_plan_t* plan);

/* Bytes of workspace a call with (desc, plan) needs; 0 if the pair is invalid.
 * Layout (f32, each section starting at a multiple of 256 bytes):
 *   acc [batch][num_q_heads][n_splits][head_dim_v]   sum over the slice of exp(s_j - m) V_j
 *   m   [batch][num_q_heads][n_splits]               the slice's reference score (natural-log
 *                                                    units), -inf for an empty slice
 *   l   [batch][num_q_heads][n_splits]               sum over the slice of exp(s_j - m)
 *   cnt [batch][num_kv_heads][1 + ceil(n_splits/16)] uint32
 *                                                    completion counters of
 *                                                    attn_decode_one_launch (chunks done,
 *                                                    then splits done per chunk of 16)
 * (issue #3725 design note section 2: partials of (m, s, acc[D]) per query head and split,
 * acc left un-normalised.) m is the slice maximum of s_j, except on the shared-latent
 * kernels of f32 caches and, for 64 and 96 heads at more than 128 (split, sequence) pairs,
 * of f16 caches, whose m can lie up to 8 ln 2 below it (it moves only when a tile's maximum
 * exceeds it by more than that, which spares rescaling the accumulators); the combine and
 * the result are the same for any m that l and acc are taken against. */
size_t attn_decode_workspace_bytes(const sk_desc_t* desc, const sk_plan_t* plan);

/* Split kernel: writes the partial triple of every (b, h, split) into `workspace`.
 *   q            device, [batch][num_q_heads][head_dim_qk] of q_dtype, contiguous,
 *                16-byte aligned
 *   k, v         device, KV cache of kv_dtype in `layout`; v is NULL iff kv_shared
 *   block_table  device int32 [batch][max_pages_per_seq] when paged (page numbers) or
 *                indexed (pool rows), else NULL
 *   seq_lens     device int32 [batch]; 1 <= L_b <= min(max_seq_len, n_splits*chunk)
 *   workspace    device, >= attn_decode_workspace_bytes(desc, plan) bytes, 256-byte aligned
 *   stream       HIP stream of the device holding every buffer
 * A length outside its range is a caller error: the kernels never read outside
 * [0, max_seq_len) nor outside the pools, and the combine then writes NaN for that
 * sequence. A block-table entry outside [0, num_pages) is likewise never followed;
 * the rows it names poison that head's output with NaN.
 * Supported: GQA with head_dim_qk == head_dim_v in {64, 128, 256}, group size
 * num_q_heads/num_kv_heads in {1, 2, 4, 6, 8}, any q/KV dtype, every layout; latent
 * (kv_shared) with num_kv_heads == 1, head_dim_qk == 576, head_dim_v == 512, num_q_heads
 * in {32, 64, 96, 128}, q f32, KV f32 or f16, contiguous or indexed. Latent f16 caches run on f16
 * MFMA: q and the softmax weights are rounded to f16 there (f32 accumulation). Latent f32
 * caches run on f16 MFMA too, with every operand (cache entries, q * scale * log2 e, the
 * weights) split into two f16 parts, hi and (x - hi) * 2^11, and three part products per
 * product (22 significant bits: each operand within 2^-22 |x| + 2^-36; f32 accumulation);
 * a cache entry or scaled query value of magnitude 65,520 or more, past f16's range, makes
 * NaN the outputs of the heads whose products it enters (every head of the sequence for a
 * cache entry, its own head for a query value).
 * Anything else returns SK_ERR_UNSUPPORTED without launching.
 * Kernel: contiguous f16/bf16 caches of head width 64, of width 128 with at least 4
 * query heads per KV head, and of width 256 with at least 6, run on the query-tile
 * kernel of attn_query_tiles with one query (its partials have this layout): MFMA
 * scores and outputs with q and the weights split into two f16 or three bf16 parts
 * (22 or 24 significant bits; scores within 1e-6 of exact on unit-scale data), which
 * holds wide groups at the memory rate where the vector split kernel runs out of ALU
 * issue. Every other GQA descriptor runs the vector split kernel. */
sk_status_t attn_decode_splitk(const sk_desc_t* desc, const sk_plan_t* plan,
                               const void* q, const void* k, const void* v,
                               const int32_t* block_table, const int32_t* seq_lens,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Combine kernel: merges the first ceil(L_b/chunk) partials of each (b, h) — the only
 * non-empty ones — into
 *   out  device f32 [batch][num_q_heads][head_dim_v]
 *   lse  device f32 [batch][num_q_heads], or NULL to skip (natural log of sum_j exp(s_j))
 * reading `workspace` as written by attn_decode_splitk with the same desc and plan,
 * earlier on the same stream. */
sk_status_t attn_decode_combine(const sk_desc_t* desc, const sk_plan_t* plan,
                                const int32_t* seq_lens, const void* workspace,
                                size_t workspace_bytes, float* out, float* lse,
                                hipStream_t stream);

/* Zeroes the counter section (cnt) of a workspace with a fill kernel on `stream` (no
 * memset, so the call may be captured in a graph). attn_decode_one_launch needs the
 * counters at zero when it starts and leaves them at zero when it completes, so this
 * runs once after the workspace is allocated, or after anything else has written over it.
 * Errors: SK_ERR_INVALID_ARG, SK_ERR_WORKSPACE_TOO_SMALL (nothing launched), SK_ERR_LAUNCH. */
sk_status_t attn_decode_workspace_init(const sk_desc_t* desc, const sk_plan_t* plan,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* The whole decode call: attn_decode_splitk followed by attn_decode_combine on `stream`,
 * with the same arguments, layouts and contract, every argument checked before the
 * first launch.
 *   out  device f32 [batch][num_q_heads][head_dim_v], 16-byte aligned
 *   lse  device f32 [batch][num_q_heads], or NULL to skip
 * Errors: as attn_decode_splitk, plus SK_ERR_INVALID_ARG for a NULL or misaligned out. */
sk_status_t attn_decode(const sk_desc_t* desc, const sk_plan_t* plan, const void* q,
                        const void* k, const void* v, const int32_t* block_table,
                        const int32_t* seq_lens, void* workspace, size_t workspace_bytes,
                        float* out, float* lse, hipStream_t stream);

/* For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. The whole decode call as attn_decode
 * (the same kernels, plan, results and error behaviour), but with no workspace argument:
 * the partials go to a scratch array the library holds on each device, of
 * SK_NO_ALLOC_SCRATCH_BYTES bytes (64 MiB, the attn_decode_workspace_bytes layout).
 * The array exists once per device the library runs on and is held until the process
 * ends; its device address is looked up on the first call on a device (with that
 * device current) and kept. The call allocates nothing and frees nothing.
 *   stream  must belong to the current device (the scratch used is that device's)
 * Nothing in the scratch needs to start at zero: the combine reads only the partials
 * this call's split step wrote. Every call on a device shares that device's array, and
 * each call overwrites what the last one left, so calls that overlap in time on one
 * device (two streams, two threads) race and must not be made.
 * Errors: as attn_decode; SK_ERR_WORKSPACE_TOO_SMALL, before any HIP call, when
 * attn_decode_workspace_bytes(desc, plan) exceeds SK_NO_ALLOC_SCRATCH_BYTES (plan fewer
 * splits, or use attn_decode with a workspace); SK_ERR_INVALID_ARG when `stream` belongs
 * to another device; SK_ERR_HIP when the scratch address cannot be looked up. */
#define SK_NO_ALLOC_SCRATCH_BYTES ((size_t)64 << 20)
sk_status_t attn_decode_no_alloc(const sk_desc_t* desc, const sk_plan_t* plan, const void* q,
                                 const void* k, const void* v, const int32_t* block_table,
                                 const int32_t* seq_lens, float* out, float* lse,
                                 hipStream_t stream);

/* The whole decode call in one launch, same arguments and results as attn_decode.
 * Separate K and V: every workgroup holding positions writes its partial to the workspace
 * with device-scope stores, waits for them to complete and counts it (device-scope
 * atomics). The merge (Lecture 06 section 2: M = max m_i, l = sum l_i exp(m_i - M),
 * out = sum acc_i exp(m_i - M) / l) is a two-level tree over the n = ceil(L_b/chunk)
 * non-empty splits of (b, g): the workgroup whose count completes a chunk of 16
 * consecutive splits reads the chunk's partials back with device-scope loads and writes
 * their merge into the chunk's first partial row; the one whose count completes the
 * chunks merges those rows into out and lse of the group's query heads (with n <= 16 the
 * chunk's merge goes to out directly). Each count is set back to zero by its last
 * arrival. No workgroup waits for another. Workgroups of empty slices exit at once and
 * write no workspace row. A length outside [1, min(max_seq_len, n_splits*chunk)] makes
 * that sequence's out and lse NaN. The counter section must be zero when the call starts
 * (attn_decode_workspace_init); a call that completes leaves it zero. Calls that share a workspace must not overlap in
 * time (for example on two streams). The descriptors attn_decode_splitk serves with the
 * query-tile kernel run its one-launch form (the same count and merge); the others the
 * vector split kernel's.
 * Shared latent (kv_shared): a split's partial row covers every head (96 x 512 floats
 * for 96 heads), far more than one workgroup merges quickly, so the latent split kernel
 * is started as a cooperative launch (every workgroup resident at once): each workgroup
 * writes its partial with device-scope stores and meets the others at a grid barrier on
 * the first two words of the counter section (arrivals, then departures: the last
 * workgroup to depart sets both back to zero); every workgroup then merges its share of
 * the (sequence, head, half of the value columns) rows, reading the non-empty splits
 * back with device-scope loads. The barrier's wait is bounded (about 2^24 sleeps) so
 * that no launch can hang on it. The same zero-counter contract holds.
 * Errors: as attn_decode; SK_ERR_UNSUPPORTED for a shared latent whose grid (n_splits x
 * batch x workgroups per split) does not fit on the device at once; SK_ERR_LAUNCH when
 * the runtime refuses the cooperative launch. */
sk_status_t attn_decode_one_launch(const sk_desc_t* desc, const sk_plan_t* plan, const void* q,
                                   const void* k, const void* v, const int32_t* block_table,
                                   const int32_t* seq_lens, void* workspace,
                                   size_t workspace_bytes, float* out, float* lse,
                                   hipStream_t stream);

/* Combine followed by a per-head output projection, in one kernel: for every sequence b
 * and query head h, the merged output o[b][h] (as attn_decode_combine computes it) is
 * multiplied by that head's matrix, out[b][h][r] = sum_c w_proj[h][r][c] * o[b][h][c]
 * ("Part 4 · Lecture 06 — Attention at 128k", section 2: the value up-projection wv_b is a
 * function of the merged latent, so it runs after the merge, never per slice).
 *   w_proj    device, [num_q_heads][proj_dim][head_dim_v] of w_dtype, row-major,
 *             16-byte aligned; widened to f32, f32 accumulation
 *   proj_dim  P >= 1 (the latent geometry of the pages: head_dim_v 512, P 128)
 *   out       device f32 [batch][num_q_heads][proj_dim]
 *   lse       device f32 [batch][num_q_heads], or NULL to skip
 * The workspace must hold partials written by attn_decode_splitk with the same desc and
 * plan, earlier on the same stream. An invalid length makes that sequence's out and lse
 * NaN. Supported: head_dim_v in {64, 128, 256, 512}, w_dtype f32, f16 or bf16.
 * Errors: SK_ERR_INVALID_ARG (NULL or misaligned pointers, proj_dim < 1, unknown dtype),
 * SK_ERR_UNSUPPORTED, SK_ERR_WORKSPACE_TOO_SMALL (nothing launched), SK_ERR_LAUNCH. */
sk_status_t attn_decode_combine_project(const sk_desc_t* desc, const sk_plan_t* plan,
                                        const int32_t* seq_lens, const void* workspace,
                                        size_t workspace_bytes, const void* w_proj,
                                        int32_t w_dtype, int32_t proj_dim, float* out, float* lse,
                                        hipStream_t stream);

/* Several query positions per sequence (speculative verify, chunked prefill, causal
 * self-attention): the q_len newest positions of every sequence attend their cache
 * causally. Query t (0 <= t < q_len) of sequence b sits at position L_b - q_len + t and
 * attends positions [0, L_b - q_len + t] ("Decoder Block 6: Online Attention, the
 * Capstone": a tile of query rows stays resident while each K/V tile is staged on chip
 * once, every row carrying its own running max, normaliser and accumulator). The context
 * is split as for single queries and the same combine merges the slices.
 *   q         device, [batch][q_len][num_q_heads][head_dim_qk] of q_dtype, contiguous
 *   k, v      device, contiguous caches as for SK_KV_CONTIGUOUS, f16 or bf16
 *   seq_lens  device int32 [batch]: L_b, the positions in the cache including the q_len
 *             newest; 1 <= L_b <= min(max_seq_len, n_splits*chunk)
 *   workspace >= attn_query_tiles_workspace_bytes(desc, plan, q_len) bytes, 256-byte aligned;
 *             partials of the (query, head) rows, row t*num_q_heads + h
 *   out       device f32 [batch][q_len][num_q_heads][head_dim_v]
 *   lse       device f32 [batch][q_len][num_q_heads], or NULL
 * Two launches (the query-tile split kernel, then the combine). A query with no visible
 * position (L_b < q_len) gets NaN. Products run on 16-bit MFMA with q and the softmax
 * weights each split into 16-bit parts (two f16 parts, 22 bits; three bf16 parts, 24
 * bits), f32 accumulation.
 * Supported: separate K and V, contiguous, f16/bf16 KV, head_dim 64/128/256, any group size.
 * Errors: SK_ERR_INVALID_ARG, SK_ERR_UNSUPPORTED, SK_ERR_WORKSPACE_TOO_SMALL (nothing
 * launched), SK_ERR_LAUNCH. */
sk_status_t attn_query_tiles(const sk_desc_t* desc, const sk_plan_t* plan, int32_t q_len,
                             const void* q, const void* k, const void* v,
                             const int32_t* seq_lens, void* workspace, size_t workspace_bytes,
                             float* out, float* lse, hipStream_t stream);

/* Split plan for attn_query_tiles (host only): as attn_decode_plan with the workgroup
 * budget counted over (KV head, 64-row query tile, slice): chunk = max(64,
 * ceil(Hkv * tiles * total_tokens / (k * cu_count))), rounded up to a multiple of 64,
 * with k = 1, 2 or 4 workgroups per compute unit at head width 256, 128 or 64 (the
 * LDS tile ring bounds how many a compute unit holds), and k = 8 for a ragged batch
 * (total_tokens < batch * max_seq_len), as attn_decode_plan; an explicit n_splits is
 * honoured with chunk = ceil(max_seq_len / n_splits). */
sk_status_t attn_query_tiles_plan(const sk_desc_t* desc, int32_t q_len, int32_t max_seq_len,
                                  int64_t total_tokens, int32_t cu_count,
                                  int32_t n_splits_requested, sk_plan_t* plan);

/* Workspace bytes attn_query_tiles needs (0 if the arguments are invalid). */
size_t attn_query_tiles_workspace_bytes(const sk_desc_t* desc, const sk_plan_t* plan,
                                        int32_t q_len);

/* Measurement aid (not part of a decode call): reads the first
 * (bytes/16/workgroups)*workgroups*16 bytes of `buf` once with 16-byte vector loads,
 * each of `workgroups` workgroups of 512 threads streaming one contiguous slice, and
 * writes nothing unless the data sum to an impossible value (scratch: device, >=
 * workgroups floats). Timed by the caller, it gives the device's achievable streaming
 * read rate, the practical ceiling beside the published HBM peak for the split kernel's
 * roofline. Errors: SK_ERR_INVALID_ARG (NULL or misaligned buf, workgroups outside
 * [1, 65535], buffer smaller than one 16-byte load per workgroup), SK_ERR_LAUNCH. */
sk_status_t attn_decode_read_probe(const void* buf, size_t bytes, int32_t workgroups,
                                   float* scratch, hipStream_t stream);

/* Static text for a status code. */
const char* attn_decode_status_string(sk_status_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* attn_decode_last_error(void);

/* Properties of the split kernel a (desc, plan) pair selects for attn_decode_splitk
 * (the query-tile kernel where that entry point names it; needs a GPU: it asks
 * the HIP runtime for the kernel's attributes).
 *   lds_bytes    static LDS per workgroup (independent of the context length: Lecture 06
 *                section 2 requires shared memory of O(key width + tile), never O(n_ctx))
 *   vgprs        vector registers per lane (arch + accumulation), as the runtime reports
 *   block        threads per workgroup; grid_x/y/z the launch grid */
typedef struct {
  int32_t lds_bytes;
  int32_t vgprs;
  int32_t block;
  int32_t grid_x, grid_y, grid_z;
} sk_kernel_info_t;
sk_status_t attn_decode_kernel_info(const sk_desc_t* desc, const sk_plan_t* plan,
                                    sk_kernel_info_t* info);

#ifdef __cplusplus
}
#endif

#endif /* SPLITKV_H */
