// Combine with the per-head output projection: merges the split partials of
// each (sequence, query head) and multiplies the merged output by that head's
// projection matrix, in one kernel.
//
// Lecture 06 section 2 ("The output projection moves into the combine"): the
// value up-projection wv_b is a function of the merged latent, so it cannot
// run per slice; it runs where the merged output first exists. For head h with
// matrix W_h [P][Dv]:
//
//     o   = sum_i w_i acc_i / sum_i w_i l_i,   w_i = exp(m_i - M),  M = max m_i
//     y   = W_h o                                   (P outputs)
//     lse = M + ln sum_i w_i l_i
//
// Launch: one workgroup of 1024 threads (16 waves) per (head, sequence).
//   Phase 1: the threads form NSG = 1024 / (Dv/4) split groups of Dv/4
//     threads; group j folds splits j, j + NSG, ... of the n = ceil(L/chunk)
//     that hold positions, each thread four consecutive columns (float4 rows,
//     coalesced across the group), 8 splits per chunk with the next chunk's
//     loads in flight, rescaling its running sums when the maximum grows.
//   Phase 2: the groups' (m, l, acc) meet in LDS and are rescaled to the
//     common maximum; o = acc / l goes to LDS.
//   Phase 3: wave w computes rows w, w + 16, ... of W_h o: lane i holds
//     columns [i*Dv/64, (i+1)*Dv/64) of o and of the row (one vector load of
//     the weights), and a DPP / swizzle reduction sums the 64 lanes.
#include <algorithm>

#include "sk_device.h"
#include "sk_internal.h"

namespace sk {

struct ProjArgs {
  const int32_t* seq_lens;
  const float* ws_acc;
  const float* ws_m;
  const float* ws_l;
  const void* w;  // [Hq][P][Dv] of the weight type
  float* out;     // [B][Hq][P]
  float* lse;     // [B][Hq] or null
  int32_t Hq, S, chunk, cap, P;
};

constexpr int kProjThreads = 1024;
constexpr int kProjWaves = kProjThreads / 64;

template <typename WT, int DV>
__global__ __launch_bounds__(kProjThreads) void combine_project_kernel(ProjArgs a) {
  constexpr int C4 = DV / 4;               // float4 columns
  constexpr int NSG = kProjThreads / C4;   // split groups
  constexpr int CPL = DV / 64;             // columns per lane in the projection
  constexpr int K = 8;                     // splits per chunk
  static_assert(kProjThreads % C4 == 0 && DV % 64 == 0, "column layout");

  __shared__ float s_acc[NSG][DV];
  __shared__ float s_m[NSG], s_l[NSG];
  __shared__ float s_o[DV];

  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = tid / C4, c4 = tid - (tid / C4) * C4;
  const int64_t row0 = ((int64_t)b * a.Hq + h) * a.S;

  const int Lraw = a.seq_lens[b];
  const bool valid = Lraw >= 1 && Lraw <= a.cap && (int64_t)Lraw <= (int64_t)a.S * a.chunk;
  float* y = a.out + ((int64_t)b * a.Hq + h) * a.P;
  if (!valid) {
    for (int r = tid; r < a.P; r += kProjThreads) y[r] = __builtin_nanf("");
    if (a.lse && tid == 0) a.lse[(int64_t)b * a.Hq + h] = __builtin_nanf("");
    return;
  }
  const int n = (int)(((int64_t)Lraw + a.chunk - 1) / a.chunk);

  // ---- phase 1: this group's splits grp, grp + NSG, ... < n.
  const float* __restrict__ mp = a.ws_m + row0;
  const float* __restrict__ lp = a.ws_l + row0;
  const float* __restrict__ ap = a.ws_acc + row0 * DV + c4 * 4;
  const int mine = n > grp ? (n - grp + NSG - 1) / NSG : 0;  // splits of this group
  struct Chunk {
    float m[K], l[K];
    float4 acc[K];
  };
  auto fetch = [&](Chunk& ch, int k0) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i = grp + NSG * min(k0 + k, max(mine - 1, 0));  // clamped: always a split < n
      const int ii = min(i, n - 1);
      ch.m[k] = mp[ii];
      ch.l[k] = lp[ii];
      ch.acc[k] = *reinterpret_cast<const float4*>(ap + (int64_t)ii * DV);
    }
  };
  float M = -INFINITY, ls = 0.0f;
  float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fold = [&](const Chunk& ch, int k0) {
    float mk[K];
    float mc = M;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      mk[k] = (k0 + k < mine) ? ch.m[k] : -INFINITY;
      mc = fmaxf(mc, mk[k]);
    }
    const float mu = (mc == -INFINITY) ? 0.0f : mc;  // guard: no finite maximum yet
    const float al = fast_exp2((M - mu) * kLog2e);
    ls *= al;
    A.x *= al;
    A.y *= al;
    A.z *= al;
    A.w *= al;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const float wgt = (k0 + k < mine) ? fast_exp2((mk[k] - mu) * kLog2e) : 0.0f;
      ls = fmaf(wgt, ch.l[k], ls);
      A.x = fmaf(wgt, ch.acc[k].x, A.x);
      A.y = fmaf(wgt, ch.acc[k].y, A.y);
      A.z = fmaf(wgt, ch.acc[k].z, A.z);
      A.w = fmaf(wgt, ch.acc[k].w, A.w);
    }
    M = mc;
  };
  if (mine > 0) {
    Chunk c0, c1;
    fetch(c0, 0);
    for (int k0 = 0;;) {
      if (k0 + K < mine) fetch(c1, k0 + K);
      fold(c0, k0);
      k0 += K;
      if (k0 >= mine) break;
      if (k0 + K < mine) fetch(c0, k0 + K);
      fold(c1, k0);
      k0 += K;
      if (k0 >= mine) break;
    }
  }

  // ---- phase 2: merge the groups to the common maximum.
  *reinterpret_cast<float4*>(&s_acc[grp][c4 * 4]) = A;
  if (c4 == 0) {
    s_m[grp] = M;
    s_l[grp] = ls;
  }
  __syncthreads();
  float Mx = s_m[0];
#pragma unroll
  for (int g = 1; g < NSG; ++g) Mx = fmaxf(Mx, s_m[g]);
  const float Mu = (Mx == -INFINITY) ? 0.0f : Mx;
  if (tid < DV) {
    float t = 0.0f, lt = 0.0f;
#pragma unroll
    for (int g = 0; g < NSG; ++g) {
      const float f = fast_exp2((s_m[g] - Mu) * kLog2e);  // 0 for a group without splits
      t = fmaf(f, s_acc[g][tid], t);
      lt = fmaf(f, s_l[g], lt);
    }
    s_o[tid] = t / lt;
    if (tid == 0 && a.lse) a.lse[(int64_t)b * a.Hq + h] = Mx + logf(lt);
  }
  __syncthreads();

  // ---- phase 3: y = W_h o, rows wave, wave + 16, ...
  float o[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) o[e] = s_o[lane * CPL + e];
  const WT* __restrict__ wh = reinterpret_cast<const WT*>(a.w) + (int64_t)h * a.P * DV + lane * CPL;
  for (int r0 = wave; r0 < a.P; r0 += 4 * kProjWaves) {
    // Four rows per wave per pass, their loads issued together.
    Vec<WT, CPL> wr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = min(r0 + u * kProjWaves, a.P - 1);
      wr[u] = load_vec<WT, CPL>(wh + (int64_t)r * DV);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float p = 0.0f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) p = fmaf(to_f32(wr[u].v[e]), o[e], p);
      p = row_sum<64>(p);
      const int r = r0 + u * kProjWaves;
      if (lane == 0 && r < a.P) y[r] = p;
    }
  }
}

template <typename WT>
static sk_status_t launch_by_dv(const ProjectLaunch& c, const ProjArgs& a) {
  const dim3 grid(c.d->num_q_heads, c.d->batch);
  switch (c.d->head_dim_v) {
    case 64: hipLaunchKernelGGL((combine_project_kernel<WT, 64>), grid, dim3(kProjThreads), 0, c.stream, a); break;
    case 128: hipLaunchKernelGGL((combine_project_kernel<WT, 128>), grid, dim3(kProjThreads), 0, c.stream, a); break;
    case 256: hipLaunchKernelGGL((combine_project_kernel<WT, 256>), grid, dim3(kProjThreads), 0, c.stream, a); break;
    case 512: hipLaunchKernelGGL((combine_project_kernel<WT, 512>), grid, dim3(kProjThreads), 0, c.stream, a); break;
    default: return SK_ERR_UNSUPPORTED;
  }
  return SK_OK;
}

bool project_supported(const sk_desc_t& d, int w_dtype) {
  const int dv = d.head_dim_v;
  return (dv == 64 || dv == 128 || dv == 256 || dv == 512) &&
         (w_dtype == SK_F32 || w_dtype == SK_F16 || w_dtype == SK_BF16);
}

sk_status_t combine_project_launch(const ProjectLaunch& c) {
  ProjArgs a;
  a.seq_lens = c.seq_lens;
  a.ws_acc = c.ws_acc;
  a.ws_m = c.ws_m;
  a.ws_l = c.ws_l;
  a.w = c.w;
  a.out = c.out;
  a.lse = c.lse;
  a.Hq = c.d->num_q_heads;
  a.S = c.p->n_splits;
  a.chunk = c.p->chunk;
  a.cap = c.d->max_seq_len;
  a.P = c.proj_dim;
  switch (c.w_dtype) {
    case SK_F32: return launch_by_dv<float>(c, a);
    case SK_F16: return launch_by_dv<_Float16>(c, a);
    case SK_BF16: return launch_by_dv<bf16_t>(c, a);
    default: return SK_ERR_UNSUPPORTED;
  }
}

}  // namespace sk
