// Device-scope partials and the in-grid merge of the one-launch decode
// kernels (the GQA split kernel and the query-tile kernel with one query).
//
// Lecture 06 section 2: M = max m_i, l = sum l_i exp(m_i - M),
// out = sum acc_i exp(m_i - M) / l, lse = M + ln l. Args is a kernel argument
// struct with ws_acc [B][Hq][S][D], ws_m and ws_l [B][Hq][S], out [B][Hq][D],
// lse [B][Hq] (or null), Hq and S.
#pragma once

#include "sk_device.h"
#include "sk_internal.h"

namespace sk {

// Device-scope (all XCDs) relaxed accesses for the one-launch kernels'
// partials: the stores write through to the coherence point and the loads read
// from it, so no cache maintenance is needed between workgroups on different
// XCDs. The 16-byte loads are raw buffer loads with the device-scope cache
// policy bit (sc1).
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr int kCachePolicyDevice = 16;  // sc1
__device__ __forceinline__ float4 ld_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicyDevice));
}

// Merges k partial rows of query heads h0 .. h0+G-1 of sequence b (rows
// first, first + stride, ..., first + (k-1)*stride of each head's S rows), in
// passes of P rows: the pass's m and l values of every head are read once
// into LDS (s_ml, 2*G*P floats), then thread t takes four consecutive columns
// of one head, finds the pass maximum from LDS, rescales its running sums if
// it grew, and folds the pass's accumulator rows, K per chunk, with the next
// chunk's loads in flight. Rows past the pass are clamped to its last row (a
// written partial) and weighted zero, so every read is in range.
// to_out: the result goes to out and lse (out = acc / l, lse = M + ln l);
// otherwise it is written back, un-normalised, as partial row `first`
// (m = M, l, acc), with device-scope stores: that row's own values were read
// by the thread that overwrites them, before it does.
template <int D, int NT, int P, int K = 16, typename Args>
__device__ __forceinline__ void merge_rows(const Args& a, int G, int b, int h0, int first, int k,
                                           int stride, bool to_out, int tid, float* s_ml) {
  constexpr int C4 = D / 4;
  const int64_t row0 = ((int64_t)b * a.Hq + h0) * a.S;  // head hh's row r: row0 + hh*S + r
  const auto racc = raw_rsrc(a.ws_acc + row0 * D, (uint32_t)((int64_t)G * a.S * D * 4));
  // The column loop's trip count is the same for every thread (the passes
  // below hold barriers); threads past the last column do no work in it.
  for (int base = 0; base < G * C4; base += NT) {
    const int idx = base + tid;
    const bool active = idx < G * C4;
    const int hh = active ? idx / C4 : 0;
    const int c = active ? (idx - hh * C4) * 4 : 0;
    const uint32_t col_off = (uint32_t)(((int64_t)hh * a.S * D + c) * 4);
    float M = -INFINITY, ls = 0.0f;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p0 = 0; p0 < k; p0 += P) {
      const int np = min(P, k - p0);
      float4 x0[K], x1[K];
      auto fetch = [&](float4 (&x)[K], int i0) {
#pragma unroll
        for (int kk = 0; kk < K; ++kk) {
          const int i = first + (p0 + min(i0 + kk, np - 1)) * stride;
          x[kk] = ld_dev4(racc, col_off + (uint32_t)i * (uint32_t)(D * 4));
        }
      };
      // The pass's first accumulator rows do not depend on m and l: they are
      // requested before the m and l values, so both travel in one round trip.
      fetch(x0, 0);
      __syncthreads();  // the previous pass (or column) is done with s_ml
      for (int j = tid; j < G * np; j += NT) {
        const int jh = j / np, i = j - (j / np) * np;
        const int64_t r = row0 + (int64_t)jh * a.S + first + (int64_t)(p0 + i) * stride;
        s_ml[2 * (jh * P + i)] = ld_dev(a.ws_m + r);
        s_ml[2 * (jh * P + i) + 1] = ld_dev(a.ws_l + r);
      }
      __syncthreads();
      if (!active) continue;
      const float* ml = s_ml + 2 * hh * P;
      float mc = M;
      for (int i = 0; i < np; ++i) mc = fmaxf(mc, ml[2 * i]);
      const float mu = (mc == -INFINITY) ? 0.0f : mc;  // guard: no finite maximum yet
      const float al = fast_exp2((M - mu) * kLog2e);
      ls *= al;
      A.x *= al;
      A.y *= al;
      A.z *= al;
      A.w *= al;
      M = mc;
      auto fold = [&](const float4 (&x)[K], int i0) {
#pragma unroll
        for (int kk = 0; kk < K; ++kk) {
          const int i = min(i0 + kk, np - 1);
          const float w = (i0 + kk < np) ? fast_exp2((ml[2 * i] - mu) * kLog2e) : 0.0f;
          ls = fmaf(w, ml[2 * i + 1], ls);
          A.x = fmaf(w, x[kk].x, A.x);
          A.y = fmaf(w, x[kk].y, A.y);
          A.z = fmaf(w, x[kk].z, A.z);
          A.w = fmaf(w, x[kk].w, A.w);
        }
      };
      for (int i0 = 0;;) {
        if (i0 + K < np) fetch(x1, i0 + K);
        fold(x0, i0);
        i0 += K;
        if (i0 >= np) break;
        if (i0 + K < np) fetch(x0, i0 + K);
        fold(x1, i0);
        i0 += K;
        if (i0 >= np) break;
      }
    }
    if (!active) continue;
    if (to_out) {
      const float inv = 1.0f / ls;
      float* o = a.out + ((int64_t)b * a.Hq + h0 + hh) * D + c;
      *reinterpret_cast<float4*>(o) = make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
      if (a.lse && c == 0) a.lse[(int64_t)b * a.Hq + h0 + hh] = M + logf(ls);
    } else {
      const int64_t r = row0 + (int64_t)hh * a.S + first;
      float* o = a.ws_acc + r * D + c;
      st_dev(o, A.x);
      st_dev(o + 1, A.y);
      st_dev(o + 2, A.z);
      st_dev(o + 3, A.w);
      if (c == 0) {
        st_dev(a.ws_m + r, M);
        st_dev(a.ws_l + r, ls);
      }
    }
  }
}

// The one-launch merge as a two-level tree. The n non-empty splits of a
// (sequence, KV head) form chunks of kMergeChunk consecutive splits; the
// workgroup whose count completes a chunk merges the chunk's partials into
// its first row, and the one whose count completes the chunks merges those
// rows into out and lse (a single chunk goes to out directly). Every merge
// step then reads at most kMergeChunk rows (one round of loads in flight),
// and the chunks merge in parallel, where one workgroup reading all n rows
// in sequence made the tail of the grid. Counts are device-scope atomics on
// cnt[0] (chunks done) and cnt[1 + c] (splits of chunk c done); the last
// arrival resets each to zero. The caller has written its partial (split
// `split`) with device-scope stores and waited for them (s_waitcnt 0) in
// every thread; s_flag is a word of LDS.
template <int D, int NT, int P, int K = 16, typename Args>
__device__ __forceinline__ void merge_tree(const Args& a, int G, int b, int h0, int split, int n,
                                           uint32_t* cnt, int tid, int* s_flag, float* s_ml) {
  const int nc = (n + kMergeChunk - 1) / kMergeChunk;
  const int ch = split / kMergeChunk;
  const int kc = min(kMergeChunk, n - ch * kMergeChunk);
  __syncthreads();  // every thread's partial stores have completed
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(cnt + 1 + ch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev + 1 == (uint32_t)kc;
    if (last) __hip_atomic_store(cnt + 1 + ch, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last;
  }
  __syncthreads();
  if (!*s_flag) return;
  if (nc == 1) {
    merge_rows<D, NT, P, K>(a, G, b, h0, 0, kc, 1, true, tid, s_ml);
    return;
  }
  merge_rows<D, NT, P, K>(a, G, b, h0, ch * kMergeChunk, kc, 1, false, tid, s_ml);
  __builtin_amdgcn_s_waitcnt(0);  // the chunk's row is stored
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev + 1 == (uint32_t)nc;
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last;
  }
  __syncthreads();
  if (!*s_flag) return;
  merge_rows<D, NT, P, K>(a, G, b, h0, 0, nc, kMergeChunk, true, tid, s_ml);
}

}  // namespace sk
