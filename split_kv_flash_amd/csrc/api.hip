// C ABI entry points: validation, split planning, workspace layout, launches.
//
// Everything before the first HIP call is plain host logic, so argument errors
// are reported (and testable) on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "sk_internal.h"
#include "splitkv.h"

namespace {

thread_local std::string g_last_error;

sk_status_t fail(sk_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sk_status_t fail(sk_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

sk_status_t ok() {
  g_last_error.clear();
  return SK_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

constexpr int32_t kMinChunk = 64;
constexpr int32_t kChunkGranule = 64;
// Ragged batches (total_tokens < batch * max_seq_len) plan this many times
// more workgroups: their slices differ in length, and more, shorter blocks
// balance the compute units.
constexpr int32_t kRaggedBlockFactor = 8;
// Slices of at least this many positions (at one workgroup per compute unit)
// are planned for three quarters of the compute units instead: on MI355X 192
// concurrent sequential readers stream HBM faster than 256 (9B-like layer at
// 262,144 positions, f16: 0.759 vs 0.724 of peak per call; f32 at 131,072:
// 0.735 vs 0.728), while short slices gain nothing from it.
constexpr int64_t kLongSlice = 1024;
constexpr int32_t kMaxGridYZ = 65535;
// Largest step between consecutive positions of a contiguous cache: a split
// kernel tile (at most 64 rows) is addressed with 32-bit byte offsets.
constexpr int64_t kMaxRowStepBytes = int64_t(1) << 24;

// Shape checks shared by every entry point (no pointer checks).
sk_status_t check_desc(const sk_desc_t* d) {
  if (!d) return fail(SK_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 1) return fail(SK_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", d->batch);
  if (d->batch > kMaxGridYZ) return fail(SK_ERR_INVALID_ARG, "batch %d exceeds %d", d->batch, kMaxGridYZ);
  if (d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(SK_ERR_INVALID_ARG, "head counts must be >= 1 (q %d, kv %d)", d->num_q_heads,
                d->num_kv_heads);
  if (d->num_q_heads % d->num_kv_heads)
    return fail(SK_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                d->num_q_heads, d->num_kv_heads);
  if (d->head_dim_qk < 1 || d->head_dim_v < 1)
    return fail(SK_ERR_INVALID_ARG, "head dims must be >= 1 (qk %d, v %d)", d->head_dim_qk,
                d->head_dim_v);
  if (d->head_dim_v % 4)
    return fail(SK_ERR_INVALID_ARG, "head_dim_v %d is not a multiple of 4", d->head_dim_v);
  if (d->kv_shared != 0 && d->kv_shared != 1)
    return fail(SK_ERR_INVALID_ARG, "kv_shared must be 0 or 1");
  if (d->kv_shared && d->head_dim_v > d->head_dim_qk)
    return fail(SK_ERR_INVALID_ARG, "shared latent: head_dim_v %d exceeds head_dim_qk %d",
                d->head_dim_v, d->head_dim_qk);
  if (d->kv_shared && d->num_kv_heads != 1)
    return fail(SK_ERR_INVALID_ARG, "shared latent needs num_kv_heads == 1");
  if (!d->kv_shared && d->head_dim_v != d->head_dim_qk)
    return fail(SK_ERR_UNSUPPORTED, "separate K and V need head_dim_qk == head_dim_v");
  if (!(d->scale == d->scale) || d->scale == __builtin_inff() || d->scale == -__builtin_inff())
    return fail(SK_ERR_INVALID_ARG, "scale must be finite");
  if (d->q_dtype < SK_F32 || d->q_dtype > SK_BF16 || d->kv_dtype < SK_F32 || d->kv_dtype > SK_BF16)
    return fail(SK_ERR_INVALID_ARG, "unknown dtype (q %d, kv %d)", d->q_dtype, d->kv_dtype);
  if (d->max_seq_len < 1) return fail(SK_ERR_INVALID_ARG, "max_seq_len must be >= 1");
  if (d->layout == SK_KV_CONTIGUOUS || d->layout == SK_KV_INDEXED) {
    if (d->layout == SK_KV_INDEXED) {
      if (d->max_pages_per_seq < 1 || d->num_pages < 1)
        return fail(SK_ERR_INVALID_ARG, "indexed: max_pages_per_seq and num_pages must be >= 1");
      if (d->max_seq_len > d->max_pages_per_seq)
        return fail(SK_ERR_INVALID_ARG, "indexed: max_seq_len %d exceeds the index row length %d",
                    d->max_seq_len, d->max_pages_per_seq);
    }
    if (d->stride_pos < 1 || d->stride_head < 0 || d->stride_seq < 0)
      return fail(SK_ERR_INVALID_ARG, "contiguous strides must be non-negative (stride_pos >= 1)");
    if (d->num_kv_heads > 1 && d->stride_head < d->head_dim_qk)
      return fail(SK_ERR_INVALID_ARG, "stride_head %lld overlaps KV heads of width %d",
                  (long long)d->stride_head, d->head_dim_qk);
    const int64_t vec = d->kv_dtype == SK_F32 ? 4 : 8;  // elements per 16-byte load
    if (d->stride_pos % vec || d->stride_head % vec || d->stride_seq % vec)
      return fail(SK_ERR_UNSUPPORTED, "strides must be multiples of 16 bytes (vector loads)");
    if (d->stride_pos < d->head_dim_qk)
      return fail(SK_ERR_INVALID_ARG, "stride_pos %lld overlaps positions of width %d",
                  (long long)d->stride_pos, d->head_dim_qk);
    const int64_t esize = d->kv_dtype == SK_F32 ? 4 : 2;
    if (d->stride_pos * esize > kMaxRowStepBytes)
      return fail(SK_ERR_UNSUPPORTED, "stride_pos of %lld bytes exceeds %lld (32-bit tile offsets)",
                  (long long)(d->stride_pos * esize), (long long)kMaxRowStepBytes);
  } else if (d->layout == SK_KV_PAGED) {
    if (d->kv_shared) return fail(SK_ERR_UNSUPPORTED, "paged shared latent is not supported");
    if (!is_pow2(d->page_size))
      return fail(SK_ERR_INVALID_ARG, "page_size %d is not a power of two", d->page_size);
    if (d->max_pages_per_seq < 1 || d->num_pages < 1)
      return fail(SK_ERR_INVALID_ARG, "paged: max_pages_per_seq and num_pages must be >= 1");
    if ((int64_t)d->max_seq_len > (int64_t)d->max_pages_per_seq * d->page_size)
      return fail(SK_ERR_INVALID_ARG, "max_seq_len %d exceeds max_pages_per_seq*page_size",
                  d->max_seq_len);
  } else {
    return fail(SK_ERR_INVALID_ARG, "unknown layout %d", d->layout);
  }
  return SK_OK;
}

sk_status_t check_plan(const sk_desc_t* d, const sk_plan_t* p) {
  if (!p) return fail(SK_ERR_INVALID_ARG, "plan is NULL");
  if (p->n_splits < 1 || p->chunk < 1)
    return fail(SK_ERR_INVALID_ARG, "plan needs n_splits >= 1 and chunk >= 1 (got %d, %d)",
                p->n_splits, p->chunk);
  if (p->n_splits > kMaxGridYZ)
    return fail(SK_ERR_INVALID_ARG, "n_splits %d exceeds %d", p->n_splits, kMaxGridYZ);
  return SK_OK;
}

sk_status_t check_support(const sk_desc_t* d) {
  if (d->kv_shared) {
    if (!sk::latent_supported(*d))
      return fail(SK_ERR_UNSUPPORTED,
                  "shared latent supports Hkv 1, Dk 576, Dv 512, Hq 32/64/96/128, q f32, "
                  "KV f32/f16, contiguous or indexed (f16 indexed: Hq 32/96)");
  } else if (!sk::gqa_supported(*d)) {
    return fail(SK_ERR_UNSUPPORTED,
                "GQA supports head_dim 64/128/256 (qk == v) and group size 1/2/4/6/8");
  }
  return SK_OK;
}

}  // namespace

namespace sk {

WsLayout ws_layout(const sk_desc_t& d, const sk_plan_t& p) {
  WsLayout w;
  const size_t rows = (size_t)d.batch * d.num_q_heads * p.n_splits;
  w.acc_off = 0;
  w.m_off = align256(rows * d.head_dim_v * sizeof(float));
  w.l_off = w.m_off + align256(rows * sizeof(float));
  w.cnt_off = w.l_off + align256(rows * sizeof(float));
  w.total = w.cnt_off + align256((size_t)d.batch * d.num_kv_heads * merge_counter_words(p.n_splits) *
                                  sizeof(uint32_t));
  return w;
}

}  // namespace sk

namespace {

// Rounds a slice length to the planner's granule and derives the split count.
sk_status_t finish_plan(int64_t chunk, int32_t max_seq_len, sk_plan_t* plan) {
  if (chunk < kMinChunk) chunk = kMinChunk;
  chunk = ceil_div(chunk, kChunkGranule) * kChunkGranule;
  int64_t n = ceil_div(max_seq_len, chunk);
  if (n > kMaxGridYZ) {  // unreachable for 32-bit lengths and chunk >= 64; kept as a guard
    n = kMaxGridYZ;
    chunk = ceil_div(max_seq_len, n);
  }
  plan->n_splits = (int32_t)n;
  plan->chunk = (int32_t)chunk;
  return ok();
}

// One round of resident query-tile workgroups over (KV head, query tile,
// slice): [I3725] section 2's one-round rule, counted over query tiles and
// the workgroups a compute unit holds. A ragged batch takes the split
// kernel's ragged budget instead (kRaggedBlockFactor per compute unit): its
// short sequences leave long-sequence slices as the tail. On the seeded
// ragged batch of 32 (bf16, 8 KV heads of width 128, 4 heads each, 545,012
// positions) one round gave 4 splits and 673 us, the ragged budget 14
// splits and 400 us.
int64_t query_tile_chunk(const sk_desc_t& d, int32_t q_len, int32_t max_seq_len,
                         int64_t total_tokens, int32_t cu_count) {
  const int64_t tiles = (int64_t)d.num_kv_heads * sk::query_tile_rows_tiles(d, q_len);
  const bool ragged = total_tokens < (int64_t)max_seq_len * d.batch;
  const int64_t per_cu = ragged ? kRaggedBlockFactor : sk::query_tile_resident(d);
  return ceil_div(tiles * total_tokens, per_cu * cu_count);
}

}  // namespace

extern "C" {

sk_status_t attn_decode_plan(const sk_desc_t* desc, int32_t max_seq_len, int64_t total_tokens,
                             int32_t cu_count, int32_t n_splits_requested, sk_plan_t* plan) {
  sk_status_t s = check_desc(desc);
  if (s != SK_OK) return s;
  if (!plan) return fail(SK_ERR_INVALID_ARG, "plan is NULL");
  if (max_seq_len < 1) return fail(SK_ERR_INVALID_ARG, "max_seq_len must be >= 1");
  if (max_seq_len > desc->max_seq_len)
    return fail(SK_ERR_INVALID_ARG, "max_seq_len %d exceeds the capacity %d", max_seq_len,
                desc->max_seq_len);
  if (total_tokens < max_seq_len || total_tokens > (int64_t)max_seq_len * desc->batch)
    return fail(SK_ERR_INVALID_ARG, "total_tokens %lld is inconsistent with max_seq_len and batch",
                (long long)total_tokens);
  if (cu_count < 1) return fail(SK_ERR_INVALID_ARG, "cu_count must be >= 1");
  if (n_splits_requested < 0) return fail(SK_ERR_INVALID_ARG, "n_splits_requested must be >= 0");
  if (n_splits_requested > kMaxGridYZ)
    return fail(SK_ERR_INVALID_ARG, "n_splits_requested %d exceeds %d", n_splits_requested,
                kMaxGridYZ);
  if (n_splits_requested > 0) {
    plan->n_splits = n_splits_requested;
    plan->chunk = (int32_t)ceil_div(max_seq_len, n_splits_requested);
    return ok();
  }
  if (max_seq_len < SK_MIN_SPLIT_CONTEXT) {
    plan->n_splits = 1;
    plan->chunk = max_seq_len;
    return ok();
  }
  int64_t chunk;
  if (desc->kv_shared) {
    chunk = ceil_div(total_tokens * sk::latent_blocks_per_split(*desc), (int64_t)cu_count);
  } else if (sk::decode_on_query_tiles(*desc)) {
    chunk = query_tile_chunk(*desc, 1, max_seq_len, total_tokens, cu_count);
  } else {
    const bool ragged = total_tokens < (int64_t)max_seq_len * desc->batch;
    const int64_t per_cu = (int64_t)sk::gqa_resident_blocks(*desc) * (ragged ? kRaggedBlockFactor : 1);
    const int64_t work = (int64_t)desc->num_kv_heads * total_tokens;
    chunk = ceil_div(work, per_cu * cu_count);
    if (!ragged && chunk >= kLongSlice && sk::gqa_prefers_fewer_streams(*desc))
      chunk = ceil_div(4 * work, 3 * per_cu * cu_count);
  }
  return finish_plan(chunk, max_seq_len, plan);
}

size_t attn_decode_workspace_bytes(const sk_desc_t* desc, const sk_plan_t* plan) {
  if (check_desc(desc) != SK_OK) return 0;
  if (check_plan(desc, plan) != SK_OK) return 0;
  return sk::ws_layout(*desc, *plan).total;
}

static sk_status_t prepare_split(const sk_desc_t* desc, const sk_plan_t* plan, const void* q,
                                 const void* k, const void* v, const int32_t* block_table,
                                 const int32_t* seq_lens, void* workspace, size_t workspace_bytes,
                                 bool need_pointers, sk::SplitLaunch* out) {
  sk_status_t s = check_desc(desc);
  if (s != SK_OK) return s;
  if ((s = check_plan(desc, plan)) != SK_OK) return s;
  if (need_pointers) {
    if (!q || !k || !seq_lens || !workspace)
      return fail(SK_ERR_INVALID_ARG, "q, k, seq_lens and workspace must be non-NULL");
    if (desc->kv_shared && v)
      return fail(SK_ERR_INVALID_ARG, "v must be NULL when keys and values share the latent");
    if (!desc->kv_shared && !v) return fail(SK_ERR_INVALID_ARG, "v is NULL");
    if (desc->layout != SK_KV_CONTIGUOUS && !block_table)
      return fail(SK_ERR_INVALID_ARG, "paged and indexed layouts need block_table");
    if (desc->layout == SK_KV_CONTIGUOUS && block_table)
      return fail(SK_ERR_INVALID_ARG, "contiguous layout takes no block_table");
    if ((uintptr_t)workspace % 256) return fail(SK_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    if ((uintptr_t)k % 16 || (v && (uintptr_t)v % 16))
      return fail(SK_ERR_INVALID_ARG, "K and V must be 16-byte aligned");
    if ((uintptr_t)q % 16) return fail(SK_ERR_INVALID_ARG, "q must be 16-byte aligned");
    const size_t need = sk::ws_layout(*desc, *plan).total;
    if (workspace_bytes < need)
      return fail(SK_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes,
                  need);
  }
  if ((s = check_support(desc)) != SK_OK) return s;
  const sk::WsLayout w = sk::ws_layout(*desc, *plan);
  char* ws = static_cast<char*>(workspace);
  out->d = desc;
  out->p = plan;
  out->q = q;
  out->k = k;
  out->v = v;
  out->block_table = block_table;
  out->seq_lens = seq_lens;
  out->ws_acc = reinterpret_cast<float*>(ws + w.acc_off);
  out->ws_m = reinterpret_cast<float*>(ws + w.m_off);
  out->ws_l = reinterpret_cast<float*>(ws + w.l_off);
  out->counters = reinterpret_cast<uint32_t*>(ws + w.cnt_off);
  out->stream = nullptr;
  return SK_OK;
}

// Single-query decode as a query-tile launch (q_len = 1): the rows are the
// group's heads and the partials take the split kernel's layout.
static sk::QueryTileLaunch one_query_tiles(const sk::SplitLaunch& a) {
  sk::QueryTileLaunch t;
  t.d = a.d;
  t.p = a.p;
  t.q_len = 1;
  t.q = a.q;
  t.k = a.k;
  t.v = a.v;
  t.seq_lens = a.seq_lens;
  t.ws_acc = a.ws_acc;
  t.ws_m = a.ws_m;
  t.ws_l = a.ws_l;
  t.stream = a.stream;
  t.fused = a.fused;
  t.counters = a.counters;
  t.out = a.out;
  t.lse = a.lse;
  return t;
}

// The split step of two-launch decode: the shared-latent kernel, the GQA split
// kernel, or the query-tile kernel with one query (whose partials and grid
// have the same layout) for the descriptors it serves faster.
static sk_status_t split_dispatch(const sk::SplitLaunch& a, bool launch, const void** fn,
                                  int grid[3], int* block) {
  if (a.d->kv_shared) return sk::latent_split_launch(a, launch, fn, grid, block);
  if (sk::decode_on_query_tiles(*a.d))
    return sk::query_tile_launch(one_query_tiles(a), launch, fn, grid, block);
  return sk::gqa_split_launch(a, launch, fn, grid, block);
}

sk_status_t attn_decode_splitk(const sk_desc_t* desc, const sk_plan_t* plan, const void* q,
                               const void* k, const void* v, const int32_t* block_table,
                               const int32_t* seq_lens, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  sk::SplitLaunch a;
  sk_status_t s = prepare_split(desc, plan, q, k, v, block_table, seq_lens, workspace,
                                workspace_bytes, true, &a);
  if (s != SK_OK) return s;
  a.stream = stream;
  int grid[3], block;
  s = split_dispatch(a, true, nullptr, grid, &block);
  if (s != SK_OK) return fail(s, "no split kernel for this descriptor");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(SK_ERR_LAUNCH, "split kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

sk_status_t attn_decode_combine(const sk_desc_t* desc, const sk_plan_t* plan,
                                const int32_t* seq_lens, const void* workspace,
                                size_t workspace_bytes, float* out, float* lse,
                                hipStream_t stream) {
  sk_status_t s = check_desc(desc);
  if (s != SK_OK) return s;
  if ((s = check_plan(desc, plan)) != SK_OK) return s;
  if (!seq_lens || !workspace || !out)
    return fail(SK_ERR_INVALID_ARG, "seq_lens, workspace and out must be non-NULL");
  if ((uintptr_t)workspace % 256) return fail(SK_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if ((uintptr_t)out % 16) return fail(SK_ERR_INVALID_ARG, "out must be 16-byte aligned");
  const sk::WsLayout w = sk::ws_layout(*desc, *plan);
  if (workspace_bytes < w.total)
    return fail(SK_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes,
                w.total);
  const char* ws = static_cast<const char*>(workspace);
  sk::CombineLaunch c;
  c.d = desc;
  c.p = plan;
  c.seq_lens = seq_lens;
  c.ws_acc = reinterpret_cast<const float*>(ws + w.acc_off);
  c.ws_m = reinterpret_cast<const float*>(ws + w.m_off);
  c.ws_l = reinterpret_cast<const float*>(ws + w.l_off);
  c.out = out;
  c.lse = lse;
  c.stream = stream;
  s = sk::combine_launch(c);
  if (s != SK_OK) return fail(s, "combine launch rejected");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(SK_ERR_LAUNCH, "combine kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

sk_status_t attn_decode_combine_project(const sk_desc_t* desc, const sk_plan_t* plan,
                                        const int32_t* seq_lens, const void* workspace,
                                        size_t workspace_bytes, const void* w_proj,
                                        int32_t w_dtype, int32_t proj_dim, float* out, float* lse,
                                        hipStream_t stream) {
  sk_status_t s = check_desc(desc);
  if (s != SK_OK) return s;
  if ((s = check_plan(desc, plan)) != SK_OK) return s;
  if (!seq_lens || !workspace || !w_proj || !out)
    return fail(SK_ERR_INVALID_ARG, "seq_lens, workspace, w_proj and out must be non-NULL");
  if ((uintptr_t)workspace % 256) return fail(SK_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if ((uintptr_t)w_proj % 16) return fail(SK_ERR_INVALID_ARG, "w_proj must be 16-byte aligned");
  if (w_dtype < SK_F32 || w_dtype > SK_BF16)
    return fail(SK_ERR_INVALID_ARG, "unknown weight dtype %d", w_dtype);
  if (proj_dim < 1) return fail(SK_ERR_INVALID_ARG, "proj_dim must be >= 1 (got %d)", proj_dim);
  if (!sk::project_supported(*desc, w_dtype))
    return fail(SK_ERR_UNSUPPORTED, "the projection supports head_dim_v 64/128/256/512");
  const sk::WsLayout w = sk::ws_layout(*desc, *plan);
  if (workspace_bytes < w.total)
    return fail(SK_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes,
                w.total);
  const char* ws = static_cast<const char*>(workspace);
  sk::ProjectLaunch c;
  c.d = desc;
  c.p = plan;
  c.seq_lens = seq_lens;
  c.ws_acc = reinterpret_cast<const float*>(ws + w.acc_off);
  c.ws_m = reinterpret_cast<const float*>(ws + w.m_off);
  c.ws_l = reinterpret_cast<const float*>(ws + w.l_off);
  c.w = w_proj;
  c.w_dtype = w_dtype;
  c.proj_dim = proj_dim;
  c.out = out;
  c.lse = lse;
  c.stream = stream;
  s = sk::combine_project_launch(c);
  if (s != SK_OK) return fail(s, "combine-project launch rejected");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(SK_ERR_LAUNCH, "combine-project kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Several queries per sequence: the combine sees q_len * num_q_heads rows per
// sequence ((query position, head) pairs), as if they were heads.
static sk_desc_t rows_desc(const sk_desc_t& d, int32_t q_len) {
  sk_desc_t r = d;
  r.num_q_heads = d.num_q_heads * q_len;
  return r;
}

static sk_status_t check_query_tiles(const sk_desc_t* desc, int32_t q_len) {
  sk_status_t s = check_desc(desc);
  if (s != SK_OK) return s;
  if (q_len < 1) return fail(SK_ERR_INVALID_ARG, "q_len must be >= 1 (got %d)", q_len);
  if ((int64_t)q_len * desc->num_q_heads > (1 << 24))
    return fail(SK_ERR_INVALID_ARG, "q_len * num_q_heads exceeds 2^24");
  if ((int64_t)desc->num_kv_heads * sk::query_tile_rows_tiles(*desc, q_len) > 0x7fffffff)
    return fail(SK_ERR_INVALID_ARG, "too many query tiles");
  if (!sk::query_tile_supported(*desc))
    return fail(SK_ERR_UNSUPPORTED,
                "query tiles support separate K and V, contiguous, f16/bf16 KV, head_dim 64/128/256");
  return SK_OK;
}

sk_status_t attn_query_tiles_plan(const sk_desc_t* desc, int32_t q_len, int32_t max_seq_len,
                                  int64_t total_tokens, int32_t cu_count,
                                  int32_t n_splits_requested, sk_plan_t* plan) {
  sk_status_t s = check_query_tiles(desc, q_len);
  if (s != SK_OK) return s;
  if (!plan) return fail(SK_ERR_INVALID_ARG, "plan is NULL");
  if (max_seq_len < 1 || max_seq_len > desc->max_seq_len)
    return fail(SK_ERR_INVALID_ARG, "max_seq_len %d outside [1, %d]", max_seq_len, desc->max_seq_len);
  if (total_tokens < max_seq_len || total_tokens > (int64_t)max_seq_len * desc->batch)
    return fail(SK_ERR_INVALID_ARG, "total_tokens %lld is inconsistent with max_seq_len and batch",
                (long long)total_tokens);
  if (cu_count < 1) return fail(SK_ERR_INVALID_ARG, "cu_count must be >= 1");
  if (n_splits_requested < 0 || n_splits_requested > kMaxGridYZ)
    return fail(SK_ERR_INVALID_ARG, "n_splits_requested %d out of range", n_splits_requested);
  if (n_splits_requested > 0) {
    plan->n_splits = n_splits_requested;
    plan->chunk = (int32_t)ceil_div(max_seq_len, n_splits_requested);
    return ok();
  }
  return finish_plan(query_tile_chunk(*desc, q_len, max_seq_len, total_tokens, cu_count),
                     max_seq_len, plan);
}

size_t attn_query_tiles_workspace_bytes(const sk_desc_t* desc, const sk_plan_t* plan,
                                        int32_t q_len) {
  if (check_desc(desc) != SK_OK || check_plan(desc, plan) != SK_OK || q_len < 1) return 0;
  const sk_desc_t r = rows_desc(*desc, q_len);
  return sk::ws_layout(r, *plan).total;
}

sk_status_t attn_query_tiles(const sk_desc_t* desc, const sk_plan_t* plan, int32_t q_len,
                             const void* q, const void* k, const void* v,
                             const int32_t* seq_lens, void* workspace, size_t workspace_bytes,
                             float* out, float* lse, hipStream_t stream) {
  sk_status_t s = check_query_tiles(desc, q_len);
  if (s != SK_OK) return s;
  if ((s = check_plan(desc, plan)) != SK_OK) return s;
  if (!q || !k || !v || !seq_lens || !workspace || !out)
    return fail(SK_ERR_INVALID_ARG, "q, k, v, seq_lens, workspace and out must be non-NULL");
  if ((uintptr_t)workspace % 256) return fail(SK_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if ((uintptr_t)k % 16 || (uintptr_t)v % 16 || (uintptr_t)q % 16 || (uintptr_t)out % 16)
    return fail(SK_ERR_INVALID_ARG, "q, K, V and out must be 16-byte aligned");
  const sk_desc_t r = rows_desc(*desc, q_len);
  const sk::WsLayout w = sk::ws_layout(r, *plan);
  if (workspace_bytes < w.total)
    return fail(SK_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes,
                w.total);
  char* ws = static_cast<char*>(workspace);
  sk::QueryTileLaunch a;
  a.d = desc;
  a.p = plan;
  a.q_len = q_len;
  a.q = q;
  a.k = k;
  a.v = v;
  a.seq_lens = seq_lens;
  a.ws_acc = reinterpret_cast<float*>(ws + w.acc_off);
  a.ws_m = reinterpret_cast<float*>(ws + w.m_off);
  a.ws_l = reinterpret_cast<float*>(ws + w.l_off);
  a.stream = stream;
  s = sk::query_tile_launch(a);
  if (s != SK_OK) return fail(s, "no query-tile kernel for this descriptor");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(SK_ERR_LAUNCH, "query-tile kernel launch failed: %s", hipGetErrorString(e));
  sk::CombineLaunch c;
  c.d = &r;
  c.p = plan;
  c.seq_lens = seq_lens;
  c.ws_acc = a.ws_acc;
  c.ws_m = a.ws_m;
  c.ws_l = a.ws_l;
  c.out = out;
  c.lse = lse;
  c.stream = stream;
  s = sk::combine_launch(c);
  if (s != SK_OK) return fail(s, "combine launch rejected");
  e = hipGetLastError();
  if (e != hipSuccess)
    return fail(SK_ERR_LAUNCH, "combine kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

sk_status_t attn_decode_workspace_init(const sk_desc_t* desc, const sk_plan_t* plan,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  sk_status_t s = check_desc(desc);
  if (s != SK_OK) return s;
  if ((s = check_plan(desc, plan)) != SK_OK) return s;
  if (!workspace) return fail(SK_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)workspace % 256) return fail(SK_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  const sk::WsLayout w = sk::ws_layout(*desc, *plan);
  if (workspace_bytes < w.total)
    return fail(SK_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes,
                w.total);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + w.cnt_off);
  sk::zero_words_launch(cnt, (size_t)desc->batch * desc->num_kv_heads * sk::merge_counter_words(plan->n_splits),
                       stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(SK_ERR_LAUNCH, "workspace init launch failed: %s", hipGetErrorString(e));
  return ok();
}

sk_status_t attn_decode(const sk_desc_t* desc, const sk_plan_t* plan, const void* q,
                        const void* k, const void* v, const int32_t* block_table,
                        const int32_t* seq_lens, void* workspace, size_t workspace_bytes,
                        float* out, float* lse, hipStream_t stream) {
  // Every check runs before the first launch.
  sk::SplitLaunch a;
  sk_status_t s = prepare_split(desc, plan, q, k, v, block_table, seq_lens, workspace,
                                workspace_bytes, true, &a);
  if (s != SK_OK) return s;
  if (!out) return fail(SK_ERR_INVALID_ARG, "out must be non-NULL");
  if ((uintptr_t)out % 16) return fail(SK_ERR_INVALID_ARG, "out must be 16-byte aligned");
  s = attn_decode_splitk(desc, plan, q, k, v, block_table, seq_lens, workspace, workspace_bytes,
                         stream);
  if (s != SK_OK) return s;
  return attn_decode_combine(desc, plan, seq_lens, workspace, workspace_bytes, out, lse, stream);
}

// Partials of attn_decode_no_alloc, for callers that cannot allocate: one
// array per device, held by the loaded library until the process ends. Host
// code never names it except to look up its device address: in host code the
// name stands for a host-side shadow, not for device memory.
static __device__ __align__(256) char scratch[SK_NO_ALLOC_SCRATCH_BYTES];

}  // extern "C"

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch`, per device

// The current device's scratch address, looked up with that device current on
// its first use and kept.
sk_status_t device_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SK_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(SK_ERR_UNSUPPORTED, "device %d is past the %d devices the scratch table covers", dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SK_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return SK_OK;
}

}  // namespace

extern "C" {

sk_status_t attn_decode_no_alloc(const sk_desc_t* desc, const sk_plan_t* plan, const void* q,
                                 const void* k, const void* v, const int32_t* block_table,
                                 const int32_t* seq_lens, float* out, float* lse,
                                 hipStream_t stream) {
  // Every argument check runs before the first HIP call: the descriptor and plan,
  // the scratch size, then the pointers (against a stand-in, aligned workspace
  // address, since the real one is looked up only afterwards).
  sk_status_t s = check_desc(desc);
  if (s != SK_OK) return s;
  if ((s = check_plan(desc, plan)) != SK_OK) return s;
  const size_t need = sk::ws_layout(*desc, *plan).total;
  if (need > SK_NO_ALLOC_SCRATCH_BYTES)
    return fail(SK_ERR_WORKSPACE_TOO_SMALL,
                "this call needs %zu bytes of partials; the static scratch holds %zu "
                "(plan fewer splits, or pass a workspace to attn_decode)",
                need, (size_t)SK_NO_ALLOC_SCRATCH_BYTES);
  sk::SplitLaunch a;
  void* const stand_in = reinterpret_cast<void*>((uintptr_t)256);
  s = prepare_split(desc, plan, q, k, v, block_table, seq_lens, stand_in, SK_NO_ALLOC_SCRATCH_BYTES,
                    true, &a);
  if (s != SK_OK) return s;
  if (!out) return fail(SK_ERR_INVALID_ARG, "out must be non-NULL");
  if ((uintptr_t)out % 16) return fail(SK_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if (stream) {
    int cur = -1, sdev = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(SK_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
    if (sdev != cur)
      return fail(SK_ERR_INVALID_ARG, "stream belongs to device %d, but device %d is current", sdev,
                  cur);
  }
  void* ws = nullptr;
  if ((s = device_scratch(&ws)) != SK_OK) return s;
  s = attn_decode_splitk(desc, plan, q, k, v, block_table, seq_lens, ws, SK_NO_ALLOC_SCRATCH_BYTES,
                         stream);
  if (s != SK_OK) return s;
  return attn_decode_combine(desc, plan, seq_lens, ws, SK_NO_ALLOC_SCRATCH_BYTES, out, lse, stream);
}

sk_status_t attn_decode_one_launch(const sk_desc_t* desc, const sk_plan_t* plan, const void* q,
                                   const void* k, const void* v, const int32_t* block_table,
                                   const int32_t* seq_lens, void* workspace,
                                   size_t workspace_bytes, float* out, float* lse,
                                   hipStream_t stream) {
  sk::SplitLaunch a;
  sk_status_t s = prepare_split(desc, plan, q, k, v, block_table, seq_lens, workspace,
                                workspace_bytes, true, &a);
  if (s != SK_OK) return s;
  if (!out) return fail(SK_ERR_INVALID_ARG, "out must be non-NULL");
  if ((uintptr_t)out % 16) return fail(SK_ERR_INVALID_ARG, "out must be 16-byte aligned");
  a.stream = stream;
  a.fused = true;
  a.out = out;
  a.lse = lse;
  int grid[3], block;
  s = split_dispatch(a, true, nullptr, grid, &block);
  if (s == SK_ERR_UNSUPPORTED && desc->kv_shared)
    return fail(s, "the one-launch latent decode needs its %d x %d x %d workgroups resident at once "
                   "(a cooperative launch): use fewer splits", grid[0], grid[1], grid[2]);
  if (s == SK_ERR_HIP) return fail(s, "could not query the device for the cooperative launch");
  if (s == SK_ERR_LAUNCH)
    return fail(s, "one-launch latent decode failed to launch: %s", hipGetErrorString(hipGetLastError()));
  if (s != SK_OK) return fail(s, "no split kernel for this descriptor");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(SK_ERR_LAUNCH, "one-launch decode kernel failed to launch: %s", hipGetErrorString(e));
  return ok();
}

sk_status_t attn_decode_read_probe(const void* buf, size_t bytes, int32_t workgroups,
                                   float* scratch, hipStream_t stream) {
  if (!buf || !scratch) return fail(SK_ERR_INVALID_ARG, "buf and scratch must be non-NULL");
  if ((uintptr_t)buf % 16) return fail(SK_ERR_INVALID_ARG, "buf must be 16-byte aligned");
  if (workgroups < 1 || workgroups > kMaxGridYZ)
    return fail(SK_ERR_INVALID_ARG, "workgroups must lie in [1, %d]", kMaxGridYZ);
  if (bytes / 16 < (size_t)workgroups)
    return fail(SK_ERR_INVALID_ARG, "buffer of %zu bytes is too small for %d workgroups", bytes,
                workgroups);
  sk::read_probe_launch(buf, bytes, workgroups, scratch, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(SK_ERR_LAUNCH, "read probe launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* attn_decode_status_string(sk_status_t status) {
  switch (status) {
    case SK_OK: return "ok";
    case SK_ERR_INVALID_ARG: return "invalid argument";
    case SK_ERR_UNSUPPORTED: return "unsupported combination";
    case SK_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SK_ERR_LAUNCH: return "kernel launch failed";
    case SK_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* attn_decode_last_error(void) { return g_last_error.c_str(); }

sk_status_t attn_decode_kernel_info(const sk_desc_t* desc, const sk_plan_t* plan,
                                    sk_kernel_info_t* info) {
  if (!info) return fail(SK_ERR_INVALID_ARG, "info is NULL");
  sk::SplitLaunch a;
  sk_status_t s = prepare_split(desc, plan, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                0, false, &a);
  if (s != SK_OK) return s;
  const void* fn = nullptr;
  int grid[3], block;
  s = split_dispatch(a, false, &fn, grid, &block);
  if (s != SK_OK) return fail(s, "no split kernel for this descriptor");
  hipFuncAttributes attr;
  hipError_t e = hipFuncGetAttributes(&attr, fn);
  if (e != hipSuccess) return fail(SK_ERR_HIP, "hipFuncGetAttributes: %s", hipGetErrorString(e));
  info->lds_bytes = (int32_t)attr.sharedSizeBytes;
  info->vgprs = attr.numRegs;
  info->block = block;
  info->grid_x = grid[0];
  info->grid_y = grid[1];
  info->grid_z = grid[2];
  return ok();
}

}  // extern "C"
