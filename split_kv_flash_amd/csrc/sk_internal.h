// Host-side interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "splitkv.h"

namespace sk {

// Splits per chunk of the one-launch decode's merge tree, and the counter
// words it keeps per (sequence, KV head): chunks done, then one per chunk.
constexpr int kMergeChunk = 16;
inline constexpr int merge_counter_words(int n_splits) {
  return 1 + (n_splits + kMergeChunk - 1) / kMergeChunk;
}

// Workspace section offsets (bytes), each a multiple of 256. The counter
// section (merge_counter_words(S) uint32 per (sequence, KV head)) is used by
// the one-launch decode only.
struct WsLayout {
  size_t acc_off, m_off, l_off, cnt_off, total;
};
WsLayout ws_layout(const sk_desc_t& d, const sk_plan_t& p);

// Everything a launcher needs; validated by the caller.
struct SplitLaunch {
  const sk_desc_t* d;
  const sk_plan_t* p;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* ws_acc;
  float* ws_m;
  float* ws_l;
  hipStream_t stream;
  // One-launch decode (separate K and V): the last workgroup of each (sequence, KV
  // head) to finish merges the partials into out/lse.
  bool fused = false;
  uint32_t* counters = nullptr;
  float* out = nullptr;
  float* lse = nullptr;
};

struct CombineLaunch {
  const sk_desc_t* d;
  const sk_plan_t* p;
  const int32_t* seq_lens;
  const float* ws_acc;
  const float* ws_m;
  const float* ws_l;
  float* out;
  float* lse;
  hipStream_t stream;
};

struct ProjectLaunch {
  const sk_desc_t* d;
  const sk_plan_t* p;
  const int32_t* seq_lens;
  const float* ws_acc;
  const float* ws_m;
  const float* ws_l;
  const void* w;
  int32_t w_dtype;
  int32_t proj_dim;
  float* out;
  float* lse;
  hipStream_t stream;
};

struct QueryTileLaunch {
  const sk_desc_t* d;
  const sk_plan_t* p;
  int32_t q_len;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  float* ws_acc;
  float* ws_m;
  float* ws_l;
  hipStream_t stream;
  // One-launch decode (q_len = 1 only): merge in the grid into out and lse.
  bool fused = false;
  uint32_t* counters = nullptr;
  float* out = nullptr;
  float* lse = nullptr;
};

// Host-only capability checks (no HIP calls).
bool gqa_supported(const sk_desc_t& d);
// Workgroups per compute unit the split heuristic plans for a uniform batch.
int gqa_resident_blocks(const sk_desc_t& d);
// Whether long slices are planned for three quarters of the compute units.
bool gqa_prefers_fewer_streams(const sk_desc_t& d);
bool latent_supported(const sk_desc_t& d);
// Workgroups that share one split of a shared latent (the f32 kernel spreads
// the heads of a split over several).
int latent_blocks_per_split(const sk_desc_t& d);

// Launchers: return the kernel function pointer they use through `fn` when
// non-null (for attribute queries) and launch only when `launch` is true.
// Grid dimensions are written to grid[3].
sk_status_t gqa_split_launch(const SplitLaunch& a, bool launch, const void** fn, int grid[3],
                             int* block);
sk_status_t latent_split_launch(const SplitLaunch& a, bool launch, const void** fn, int grid[3],
                                int* block);
sk_status_t combine_launch(const CombineLaunch& a);
bool project_supported(const sk_desc_t& d, int w_dtype);
bool query_tile_supported(const sk_desc_t& d);
// 64-row query tiles per KV head for q_len queries.
int query_tile_rows_tiles(const sk_desc_t& d, int q_len);
// Query-tile workgroups resident per compute unit (LDS-bound).
int query_tile_resident(const sk_desc_t& d);
// Whether single-query decode of this descriptor runs on the query-tile
// kernel (q_len = 1) instead of the GQA split kernel.
bool decode_on_query_tiles(const sk_desc_t& d);
// Launches (when `launch`) the query-tile kernel; reports its function, grid
// and block like the split launchers.
sk_status_t query_tile_launch(const QueryTileLaunch& a, bool launch = true, const void** fn = nullptr,
                              int grid[3] = nullptr, int* block = nullptr);
sk_status_t combine_project_launch(const ProjectLaunch& a);
// Zeroes n 32-bit words with a fill kernel (no memset node, so a captured
// graph may hold it).
sk_status_t zero_words_launch(uint32_t* p, size_t n, hipStream_t stream);
sk_status_t read_probe_launch(const void* buf, size_t bytes, int32_t workgroups, float* out,
                              hipStream_t stream);

}  // namespace sk
