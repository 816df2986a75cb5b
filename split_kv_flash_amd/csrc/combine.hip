// Combine kernel: merges the split partials of each (sequence, query head).
//
// Lecture 06 section 2 and issue #3725 design note section 2 (kernel B): with
// M = max_i m_i and w_i = exp(m_i - M), l* = sum_i w_i l_i and
// out = sum_i w_i acc_i / l*. Only the first n = ceil(L_b/chunk) splits of a
// sequence hold positions; only their values are used. lse = M + ln l* (the
// log-sum-exp of the scores, "The Kernel Level: Attention and MoE").
//
// Launch: grid (ceil(Dv/64), Hq, B); a workgroup of NWC = min(4, ceil(S/64))
// waves owns 64 output columns of one (b, h). Splits are taken 64 at a time
// (wave w takes passes w, w + NWC, ...): lane i holds m and l of split i of
// the pass, and the 16-lane quarters of the wave each read every 4th split's
// 64 columns as float4 rows, so every partial row is read once, coalesced.
// Every split block of the grid writes its partial (empty slices write the
// neutral one), so a pass's rows are all requested at once, together with the
// sequence length; the rows at or past n are then dropped by selection, never
// by arithmetic, so their values cannot reach the result. Within a wave the
// maximum and the sums are wave reductions; the waves' (m, l, acc) are merged
// once through LDS with the same rescaling.
#include <algorithm>

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
constexpr int kPass = 64;             // splits per pass: one per lane
constexpr int kRowsPerQuarter = kPass / 4;

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kDppRowRor8>(x));
  x = fmaxf(x, dpp<kDppRowRor4>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, xor16(x));
  return fmaxf(x, xor32(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  x += xor16(x);
  return x + xor32(x);
}
// Value of x held by lane `src` (0..63).
__device__ __forceinline__ float from_lane(float x, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}

constexpr int kMaxCombWaves = 4;

__global__ __launch_bounds__(64 * kMaxCombWaves) void combine_kernel(CombineArgs a) {
  __shared__ float4 s_acc[kMaxCombWaves][16];
  __shared__ float s_ml[kMaxCombWaves][2];

  const int cb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwc = blockDim.x >> 6;
  const int c4 = lane & 15;  // which float4 of the 64 columns
  const int qt = lane >> 4;  // quarter: splits qt, qt+4, qt+8, ... of a pass
  const int col = cb * kCombCols + c4 * 4;
  const bool col_ok = col < a.Dv;
  const int64_t row0 = ((int64_t)b * a.Hq + h) * a.S;
  const float* __restrict__ mrow = a.ws_m + row0;
  const float* __restrict__ lrow = a.ws_l + row0;
  const float* __restrict__ accp = a.ws_acc + row0 * a.Dv + col;

  const int Lraw = a.seq_lens[b];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float mrun = -INFINITY, lrun = 0.0f;
  const bool valid = Lraw >= 1 && Lraw <= a.cap && (int64_t)Lraw <= (int64_t)a.S * a.chunk;
  int n = a.S;  // replaced by ceil(L/chunk) once the length has arrived
  bool first = true;
  for (int i0 = wave * kPass; i0 < a.S; i0 += nwc * kPass) {
    // Requests first: this pass's m, l and accumulator rows.
    const bool in_s = i0 + lane < a.S;
    float mi = in_s ? mrow[i0 + lane] : -INFINITY;
    float li = in_s ? lrow[i0 + lane] : 0.0f;
    float4 x[kRowsPerQuarter];
#pragma unroll
    for (int k = 0; k < kRowsPerQuarter; ++k) {
      const int i = i0 + qt + 4 * k;
      x[k] = (i < a.S && col_ok) ? *reinterpret_cast<const float4*>(accp + (int64_t)i * a.Dv)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (first) {
      n = valid ? (int)min((int64_t)a.S, ((int64_t)Lraw + a.chunk - 1) / a.chunk) : 0;
      first = false;
    }
    if (i0 >= n) break;  // uniform: no used split left for this wave
    // Keep only the splits that hold positions.
    const bool use = i0 + lane < n;
    mi = use ? mi : -INFINITY;
    li = use ? li : 0.0f;
    const float mn = fmaxf(mrun, wave_max(mi));
    const float mu = (mn == -INFINITY) ? 0.0f : mn;  // guard: no finite maximum yet
    const float al = fast_exp2((mrun - mu) * kLog2e);  // 0 on the first pass
    const float w = use ? fast_exp2((mi - mu) * kLog2e) : 0.0f;
    lrun = fmaf(lrun, al, wave_sum(w * li));
    acc.x *= al;
    acc.y *= al;
    acc.z *= al;
    acc.w *= al;
#pragma unroll
    for (int k = 0; k < kRowsPerQuarter; ++k) {
      const int i = i0 + qt + 4 * k;
      const float wk = from_lane(w, qt + 4 * k);
      if (i < n) {
        acc.x = fmaf(wk, x[k].x, acc.x);
        acc.y = fmaf(wk, x[k].y, acc.y);
        acc.z = fmaf(wk, x[k].z, acc.z);
        acc.w = fmaf(wk, x[k].w, acc.w);
      }
    }
    mrun = mn;
  }
  // Sum the four quarters (lanes c4, c4+16, c4+32, c4+48).
  acc.x += xor16(acc.x);
  acc.y += xor16(acc.y);
  acc.z += xor16(acc.z);
  acc.w += xor16(acc.w);
  acc.x += xor32(acc.x);
  acc.y += xor32(acc.y);
  acc.z += xor32(acc.z);
  acc.w += xor32(acc.w);
  if (nwc > 1) {
    // Merge the waves: rescale each wave's (l, acc) to the common maximum.
    if (qt == 0) s_acc[wave][c4] = acc;
    if (lane == 0) {
      s_ml[wave][0] = mrun;
      s_ml[wave][1] = lrun;
    }
    __syncthreads();
    if (wave != 0) return;
    float M = s_ml[0][0];
    for (int w = 1; w < nwc; ++w) M = fmaxf(M, s_ml[w][0]);
    const float Mu = (M == -INFINITY) ? 0.0f : M;
    acc = make_float4(0.f, 0.f, 0.f, 0.f);
    lrun = 0.0f;
    for (int w = 0; w < nwc; ++w) {
      const float f = fast_exp2((s_ml[w][0] - Mu) * kLog2e);  // 0 for a wave without splits
      const float4 v = s_acc[w][c4];
      lrun = fmaf(f, s_ml[w][1], lrun);
      acc.x = fmaf(f, v.x, acc.x);
      acc.y = fmaf(f, v.y, acc.y);
      acc.z = fmaf(f, v.z, acc.z);
      acc.w = fmaf(f, v.w, acc.w);
    }
    mrun = M;
  }
  if (qt == 0 && col_ok) {
    float* o = a.out + ((int64_t)b * a.Hq + h) * a.Dv + col;
    if (valid) {
      const float inv = 1.0f / lrun;
      *reinterpret_cast<float4*>(o) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    } else {
      const float nan = __builtin_nanf("");
      *reinterpret_cast<float4*>(o) = make_float4(nan, nan, nan, nan);
    }
  }
  if (a.lse && cb == 0 && lane == 0)
    a.lse[(int64_t)b * a.Hq + h] = valid ? mrun + logf(lrun) : __builtin_nanf("");
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

sk_status_t zero_words_launch(uint32_t* p, size_t n, hipStream_t stream) {
  if (n == 0) return SK_OK;
  const int64_t blocks = std::min<int64_t>(1024, ((int64_t)n + 255) / 256);
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, (int64_t)n);
  return SK_OK;
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
  const int waves = (int)std::min<int64_t>(kMaxCombWaves, (a.S + kPass - 1) / kPass);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(64 * waves), 0, c.stream, a);
  return SK_OK;
}

}  // namespace sk
