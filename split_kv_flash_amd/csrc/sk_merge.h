// Device-scope partials and the in-grid merge of the one-launch decode
// kernels: the last-arrival tree of the GQA split kernel and the query-tile
// kernel with one query, and the grid barrier and distributed merge of the
// shared-latent kernels.
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
__device__ __forceinline__ void st_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCachePolicyDevice);
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

// Grid-wide barrier of a cooperative launch (every workgroup of the grid is
// resident, so every workgroup reaches it), on two device-scope counters that
// are zero before the launch and zero again after it. Arrival: each workgroup
// adds one to `arrived` (after its device-scope stores have completed) and
// waits until the count reaches n. Departure, once the workgroup no longer
// needs the barrier: it adds one to `departed`, and the last to depart sets
// both back to zero; every workgroup has then seen the full count, so none is
// still waiting. The wait is bounded: after about 2^24 sleeps a workgroup
// stops waiting and proceeds (its results may then be wrong), so no launch can
// hang on it.
__device__ __forceinline__ void grid_arrive_and_wait(uint32_t* arrived, uint32_t n) {
  __builtin_amdgcn_s_waitcnt(0);  // this thread's device-scope stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev + 1 < n) {
      for (uint32_t spins = 0; spins < (1u << 24); ++spins) {
        if (__hip_atomic_load(arrived, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) break;
        __builtin_amdgcn_s_sleep(2);
      }
    }
  }
  __syncthreads();
}
__device__ __forceinline__ void grid_depart(uint32_t* arrived, uint32_t* departed, uint32_t n) {
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(departed, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev + 1 == n) {
      __hip_atomic_store(arrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(departed, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The merge of the shared-latent one-launch decode, run by every workgroup of
// the cooperative grid after the barrier (Lecture 06 section 2: M = max m_i,
// l = sum l_i exp(m_i - M), out = sum acc_i exp(m_i - M) / l, lse = M + ln l).
// A task is (sequence b, head h, half of the Dv = 512 value columns): lane j
// of the wave that takes it holds columns 4j .. 4j+3 of the half. Only the
// n_b = ceil(L_b / chunk) non-empty splits are read (device-scope loads); a
// length outside [1, min(cap, S*chunk)] gives NaN for that sequence, as the
// combine kernel does. Args: ws_acc [B][Hq][S][512], ws_m, ws_l [B][Hq][S],
// out [B][Hq][512], lse [B][Hq] or null, seq_lens, Hq, S, chunk, cap.
struct LatentTask {
  int64_t row0;  // partial row of split 0 of (b, h)
  int bh, half, n;
  bool valid;
};
template <typename Args>
__device__ __forceinline__ LatentTask latent_task_of(const Args& a, int task, int Lraw) {
  LatentTask t;
  t.half = task & 1;
  t.bh = task >> 1;
  // Every lane read the same length: kept in scalar registers, so the
  // addressing built from it stays wave-uniform.
  const int L = __builtin_amdgcn_readfirstlane(Lraw);
  t.valid = L >= 1 && L <= a.cap && (int64_t)L <= (int64_t)a.S * a.chunk;
  t.n = t.valid ? (int)((L + (int64_t)a.chunk - 1) / a.chunk) : 0;
  t.row0 = (int64_t)t.bh * a.S;
  return t;
}
template <typename Args>
__device__ __forceinline__ LatentTask latent_task(const Args& a, int task) {
  return latent_task_of(a, task, a.seq_lens[(task >> 1) / a.Hq]);
}
template <typename Args>
__device__ __forceinline__ void latent_store(const Args& a, const LatentTask& t, int lane, float M,
                                             float ls, float4 A) {
  const float inv = t.valid ? 1.0f / ls : __builtin_nanf("");
  float* o = a.out + (int64_t)t.bh * 512 + t.half * 256 + lane * 4;
  *reinterpret_cast<float4*>(o) = make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
  if (a.lse && t.half == 0 && lane == 0) a.lse[t.bh] = t.valid ? M + logf(ls) : __builtin_nanf("");
}
// Folds loaded partials (m, l, acc) of one task into its running (M, ls, A):
// slot k of the NS given holds split i0 + k; only splits below n count (the
// others may be rows this call did not write, so they are skipped by select,
// not weighted by zero).
template <int NS>
__device__ __forceinline__ void latent_fold(const float4* x, const float* mi, const float* li, int i0,
                                            int n, float& M, float& ls, float4& A) {
  float mb = M;
#pragma unroll
  for (int k = 0; k < NS; ++k) mb = (i0 + k < n) ? fmaxf(mb, mi[k]) : mb;
  const float mu = (mb == -INFINITY) ? 0.0f : mb;  // guard: no finite maximum yet
  const float al = fast_exp2((M - mu) * kLog2e);
  ls *= al;
  A.x *= al;
  A.y *= al;
  A.z *= al;
  A.w *= al;
  M = mb;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    if (i0 + k < n) {
      const float w = fast_exp2((mi[k] - mu) * kLog2e);
      ls = fmaf(w, li[k], ls);
      A.x = fmaf(w, x[k].x, A.x);
      A.y = fmaf(w, x[k].y, A.y);
      A.z = fmaf(w, x[k].z, A.z);
      A.w = fmaf(w, x[k].w, A.w);
    }
  }
}

// Workgroup mode (long slices): the workgroups take tasks in turn; wave r of
// the R = NT/64 waves folds splits r, r + R, ... (16 in flight per lane), and
// the waves' sums meet in LDS (s_lds: at least NT*4 + 2*R floats), where wave 0
// finishes the task.
template <int NT, typename Args>
__device__ void latent_merge_by_workgroup(const Args& a, int tasks, float* s_lds) {
  constexpr int R = NT / 64;
  constexpr int K = 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int r = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwg = (int)(gridDim.x * gridDim.y * gridDim.z);
  const int wg = (int)((blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x);
  float4* s_a = reinterpret_cast<float4*>(s_lds);  // [R][64]
  float* s_ml = s_lds + NT * 4;                    // [R][2]
  for (int task = wg; task < tasks; task += nwg) {
    const LatentTask t = latent_task(a, task);
    const auto racc = raw_rsrc(a.ws_acc + t.row0 * 512, (uint32_t)((int64_t)a.S * 512 * 4));
    const uint32_t col_off = (uint32_t)((t.half * 64 + lane) * 16);
    float M = -INFINITY, ls = 0.0f;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
    // The first batch's rows are clamped to the plan's splits, not to the
    // length, so its loads need not wait for the length.
    for (int i0 = r; i0 == r || i0 < t.n; i0 += R * K) {
      float4 x[K];
      float mi[K], li[K];
#pragma unroll
      for (int kk = 0; kk < K; ++kk) {
        const int i = min(i0 + kk * R, a.S - 1);  // slots past n are skipped by the fold
        x[kk] = ld_dev4(racc, col_off + (uint32_t)i * 2048u);
        mi[kk] = ld_dev(a.ws_m + t.row0 + i);
        li[kk] = ld_dev(a.ws_l + t.row0 + i);
      }
      // Slot kk holds split i0 + kk*R: fold with a stride-R view of n.
      const int nr = (t.n - i0 + R - 1) / R;  // slots of this batch that count
      latent_fold<K>(x, mi, li, 0, nr, M, ls, A);
    }
    s_a[r * 64 + lane] = A;
    if (lane == 0) {
      s_ml[2 * r] = M;
      s_ml[2 * r + 1] = ls;
    }
    __syncthreads();
    if (r == 0) {
      float Mt = -INFINITY;
#pragma unroll
      for (int w = 0; w < R; ++w) Mt = fmaxf(Mt, s_ml[2 * w]);
      const float mu = (Mt == -INFINITY) ? 0.0f : Mt;
      float lt = 0.0f;
      float4 At = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < R; ++w) {
        const float f = fast_exp2((s_ml[2 * w] - mu) * kLog2e);
        const float4 x = s_a[w * 64 + lane];
        lt = fmaf(f, s_ml[2 * w + 1], lt);
        At.x = fmaf(f, x.x, At.x);
        At.y = fmaf(f, x.y, At.y);
        At.z = fmaf(f, x.z, At.z);
        At.w = fmaf(f, x.w, At.w);
      }
      latent_store(a, t, lane, Mt, lt, At);
    }
    __syncthreads();  // s_a and s_ml are free for the next task
  }
}

// Wave mode (short slices, few workgroups): tasks [t_begin, t_end) go to W
// waves (this one is number w), J = 8/NP tasks at a time, with NP split slots
// each (NP >= S for NP < 8; NP = 8 walks the splits in batches of 8), all 8
// slots' loads in flight together; no LDS and no barrier. A task's addressing
// is wave-uniform (scalar registers). POL is the loads' cache policy:
// kCachePolicyDevice for partials other workgroups wrote with device-scope
// stores, 0 for the workgroup's own plain stores (complete before a workgroup
// barrier; the waves of a workgroup share one CU and its caches).
template <int NP, int POL, typename Args>
__device__ void latent_merge_by_wave(const Args& a, int t_begin, int t_end, int w, int W) {
  constexpr int K = 8;
  constexpr int J = K / NP;
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)gridDim.y * a.Hq * a.S;
  const auto rm = raw_rsrc(a.ws_m, (uint32_t)(rows * 4));
  const auto rl = raw_rsrc(a.ws_l, (uint32_t)(rows * 4));
  for (int t0 = t_begin + w * J; t0 < t_end; t0 += W * J) {
    float4 x[K];
    float mi[K], li[K];
    // Batch i0: slot k holds split i0 + k % NP of task t0 + k / NP (rows
    // clamped to the plan's splits, so no load waits for a length).
    auto load = [&](int i0) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int task = min(t0 + k / NP, t_end - 1);  // past the last task: read, not written
        const int64_t row = (int64_t)(task >> 1) * a.S + min(i0 + k % NP, a.S - 1);
        x[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                              raw_rsrc(a.ws_acc + row * 512, 2048u),
                                              (uint32_t)(((task & 1) * 256 + lane * 4) * 4), 0, POL));
        mi[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, (uint32_t)(row * 4), 0, POL));
        li[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)(row * 4), 0, POL));
      }
    };
    int Lraw[J];  // the lengths, then the first batch, requested before either is used
#pragma unroll
    for (int j = 0; j < J; ++j) Lraw[j] = a.seq_lens[(min(t0 + j, t_end - 1) >> 1) / a.Hq];
    load(0);
    LatentTask t[J];
    float M[J], ls[J];
    float4 A[J];
    int nmax = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      t[j] = latent_task_of(a, min(t0 + j, t_end - 1), Lraw[j]);
      nmax = max(nmax, t[j].n);
      M[j] = -INFINITY;
      ls[j] = 0.0f;
      A[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int i0 = 0;;) {
#pragma unroll
      for (int j = 0; j < J; ++j) latent_fold<NP>(x + j * NP, mi + j * NP, li + j * NP, i0, t[j].n, M[j], ls[j], A[j]);
      i0 += NP;
      if (i0 >= nmax) break;
      load(i0);
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (t0 + j < t_end) latent_store(a, t[j], lane, M[j], ls[j], A[j]);
  }
}

// Chooses the mode with the fewer rounds of dependent loads (the same choice
// in every workgroup: it depends only on the grid, S and the task count).
template <int NT, typename Args>
__device__ void latent_grid_merge(const Args& a, int batch, float* s_lds) {
  constexpr int R = NT / 64;
  const int tasks = batch * a.Hq * 2;
  const int nwg = (int)(gridDim.x * gridDim.y * gridDim.z);
  const int wg = (int)((blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x);
  const int rounds_wg = ((tasks + nwg - 1) / nwg) * ((a.S + R * 16 - 1) / (R * 16));
  const int slots = nwg * R;
  const int rounds_wave = ((tasks + slots - 1) / slots) * ((a.S + 7) / 8);
  if (rounds_wg <= rounds_wave)
    latent_merge_by_workgroup<NT>(a, tasks, s_lds);
  else
    latent_merge_by_wave<8, kCachePolicyDevice>(
        a, 0, tasks, wg * R + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), slots);
}

}  // namespace sk
