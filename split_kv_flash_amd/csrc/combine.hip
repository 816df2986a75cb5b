// Combine kernel: merges the split partials of each (sequence, query head).
//
// Lecture 06 section 2 and issue #3725 design note section 2 (kernel B): with
// M = max_i m_i and w_i = exp(m_i - M), l* = sum_i w_i l_i and
// out = sum_i w_i acc_i / l*. Only the first ceil(L_b/chunk) splits of a
// sequence hold positions; they are the only ones read. lse = M + ln l*
// (the log-sum-exp of the scores, "The Kernel Level: Attention and MoE").
//
// Launch: grid (ceil(Dv/64), Hq, B), 256 threads. A workgroup owns 64 output
// columns of one (b, h): 16 lanes cover the 64 columns with float4 loads and
// the 16 lane-groups take every 16th split, so each split row of the partials
// is read once, coalesced, and the Dv/64 column blocks multiply the parallelism
// of small-head problems.
#include "sk_device.h"
#include "sk_internal.h"

namespace sk {

struct CombineArgs {
  const int32_t* seq_lens;
  const float* ws_acc;
  const float* ws_m;
  const float* ws_l;
  float* out;
  float* lse;
  int32_t Hq, S, chunk, Dv, cap;
};

constexpr int kCombCols = 64;
constexpr int kCombThreads = 256;

__device__ __forceinline__ float block_reduce(float x, float* scratch, bool is_max) {
  // wave reduction through DPP rows, then across the 16-lane rows, then waves.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (is_max) {
    x = fmaxf(x, dpp<kDppRowRor8>(x));
    x = fmaxf(x, dpp<kDppRowRor4>(x));
    x = fmaxf(x, dpp<kDppQuadXor2>(x));
    x = fmaxf(x, dpp<kDppQuadXor1>(x));
    x = fmaxf(x, xor16(x));
    x = fmaxf(x, xor32(x));
  } else {
    x = row16_sum(x);
    x += xor16(x);
    x += xor32(x);
  }
  __syncthreads();
  if (lane == 0) scratch[wave] = x;
  __syncthreads();
  float r = scratch[0];
  for (int w = 1; w < kCombThreads / 64; ++w) r = is_max ? fmaxf(r, scratch[w]) : r + scratch[w];
  return r;
}

// Splits handled per pass: each of the 16 lane-groups owns every 16th split of
// the pass and issues all its loads before using any of them.
constexpr int kPass = kCombThreads;
constexpr int kPerThread = kPass / 16;

__global__ __launch_bounds__(kCombThreads) void combine_kernel(CombineArgs a) {
  __shared__ float s_w[kPass];
  __shared__ float4 s_part[kCombThreads / 16][16];
  __shared__ float s_red[kCombThreads / 64];

  const int cb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int Lraw = a.seq_lens[b];
  const bool valid = Lraw >= 1 && Lraw <= a.cap && (int64_t)Lraw <= (int64_t)a.S * a.chunk;
  const int n = valid ? (int)min((int64_t)a.S, ((int64_t)Lraw + a.chunk - 1) / a.chunk) : 0;
  const int64_t row0 = ((int64_t)b * a.Hq + h) * a.S;
  const float* __restrict__ mrow = a.ws_m + row0;
  const float* __restrict__ lrow = a.ws_l + row0;

  const int c4 = tid & 15;  // which float4 of the 64 columns
  const int rg = tid >> 4;  // which residue of the split index
  const int col = cb * kCombCols + c4 * 4;
  const bool col_ok = col < a.Dv;
  const float* accp = a.ws_acc + row0 * a.Dv + col;

  // First pass: the partial accumulators, and m and l of the pass's splits,
  // all requested before anything waits on them.
  float4 x[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int i = rg + 16 * k;
    x[k] = (i < n && col_ok) ? *reinterpret_cast<const float4*>(accp + (int64_t)i * a.Dv)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float mi = tid < n ? mrow[tid] : -INFINITY;
  float li = tid < n ? lrow[tid] : 0.0f;

  float mx = mi;
  for (int i = tid + kPass; i < n; i += kPass) mx = fmaxf(mx, mrow[i]);  // only when n > kPass
  mx = block_reduce(mx, s_red, true);
  const float mu = (mx == -INFINITY) ? 0.0f : mx;

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lsum = 0.0f;
  for (int i0 = 0; i0 < n; i0 += kPass) {
    if (i0 > 0) {
      const int i = i0 + tid;
      mi = i < n ? mrow[i] : -INFINITY;
      li = i < n ? lrow[i] : 0.0f;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) {
        const int j = i0 + rg + 16 * k;
        x[k] = (j < n && col_ok) ? *reinterpret_cast<const float4*>(accp + (int64_t)j * a.Dv)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    const float w = i0 + tid < n ? fast_exp2((mi - mu) * kLog2e) : 0.0f;
    lsum = fmaf(w, li, lsum);
    __syncthreads();
    s_w[tid] = w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const float wk = s_w[rg + 16 * k];
      acc.x = fmaf(wk, x[k].x, acc.x);
      acc.y = fmaf(wk, x[k].y, acc.y);
      acc.z = fmaf(wk, x[k].z, acc.z);
      acc.w = fmaf(wk, x[k].w, acc.w);
    }
  }
  const float lstar = block_reduce(lsum, s_red, false);

  s_part[rg][c4] = acc;
  __syncthreads();
  if (tid < 16 && col_ok) {
    float4 t = s_part[0][tid];
    for (int r = 1; r < kCombThreads / 16; ++r) {
      const float4 u = s_part[r][tid];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    float* o = a.out + ((int64_t)b * a.Hq + h) * a.Dv + col;
    if (valid) {
      const float inv = 1.0f / lstar;
      *reinterpret_cast<float4*>(o) = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
    } else {
      const float nan = __builtin_nanf("");
      *reinterpret_cast<float4*>(o) = make_float4(nan, nan, nan, nan);
    }
  }
  if (a.lse && cb == 0 && tid == 0)
    a.lse[(int64_t)b * a.Hq + h] = valid ? mx + logf(lstar) : __builtin_nanf("");
}

sk_status_t combine_launch(const CombineLaunch& c) {
  const sk_desc_t& d = *c.d;
  CombineArgs a;
  a.seq_lens = c.seq_lens;
  a.ws_acc = c.ws_acc;
  a.ws_m = c.ws_m;
  a.ws_l = c.ws_l;
  a.out = c.out;
  a.lse = c.lse;
  a.Hq = d.num_q_heads;
  a.S = c.p->n_splits;
  a.chunk = c.p->chunk;
  a.Dv = d.head_dim_v;
  a.cap = d.max_seq_len;
  const dim3 grid((d.head_dim_v + kCombCols - 1) / kCombCols, d.num_q_heads, d.batch);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(kCombThreads), 0, c.stream, a);
  return SK_OK;
}

}  // namespace sk
