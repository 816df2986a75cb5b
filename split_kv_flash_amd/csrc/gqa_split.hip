// Grouped-query split kernel for gfx950.
//
// One workgroup per (sequence b, KV head g, context split i) serves all G query
// heads of the group, so each K and V row crosses HBM once per decode step
// (aprender issue #3725 design note, section 2, kernel A: one block per (KV head,
// split) serving all G query heads; Lecture 06 section 2: each block runs the
// online softmax over one contiguous slice and writes a partial (m, l, acc)).
//
// Work decomposition (MI355X-first rather than the pages' 32-lane warps):
//   * 256 threads = 4 waves of 64 lanes. A KV row is held by RL consecutive lanes
//     (RL = 16 or 32), so a wave holds 64/RL rows at once and one vector load
//     instruction reads 64/RL contiguous row segments of RL*16 bytes.
//   * Each lane keeps its D/RL dimensions of the G query vectors and of the G
//     accumulators in registers; a dot product is a per-lane partial followed by
//     a 16-lane DPP reduction (plus one swizzle when RL = 32).
//   * The workgroup's NG = 4*64/RL row groups take interleaved positions
//     base + r*NG + group, R rows per group per tile, and each group carries its
//     own online-softmax state (m, l, acc) per head; tile-level rescaling follows
//     the recurrence of "Decoder Block 6" and Lecture 07 ("But Softmax Wants the
//     Whole Row..."): m' = max(m, tile max), a = exp(m - m'), l = a l + sum p,
//     acc = a acc + sum p v.
//   * Scores are kept in base-2 units (q is pre-multiplied by scale*log2 e) so
//     every exponential is one exp2; the stored m is converted back to natural
//     units.
//   * At the end the row groups merge by cross-lane exchange, the waves merge
//     through LDS (4*G*D floats, independent of the context length), and the
//     workgroup writes one partial per query head.
#include "sk_device.h"
#include "sk_internal.h"

namespace sk {

struct GqaArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* ws_acc;
  float* ws_m;
  float* ws_l;
  int64_t stride_seq, stride_pos, stride_head;
  int64_t num_pages;
  int32_t q_dtype;
  int32_t Hq, S, chunk, cap;
  int32_t page_shift, max_pages;
  float qscale;
};

template <typename KV, int D, int RL_, int R_>
struct GqaShape {
  static constexpr int RL = RL_;
  static constexpr int R = R_;
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kGroupsPerWave = 64 / RL;
  static constexpr int kGroups = kGroupsPerWave * kWaves;
  static constexpr int kDpl = D / RL;
  static constexpr int kVecMax = 16 / (int)sizeof(KV);
  static constexpr int kVec = kVecMax < kDpl ? kVecMax : kDpl;
  static constexpr int kLoads = kDpl / kVec;
  static_assert(D % RL == 0, "row width must split evenly over the row's lanes");
  static_assert(kDpl % kVec == 0, "lane slice must be whole vector loads");
};

template <typename KV, int G, int D, bool PAGED, int RL, int R>
__global__ __launch_bounds__(256) void gqa_split_kernel(GqaArgs a) {
  using Sh = GqaShape<KV, D, RL, R>;
  constexpr int DPL = Sh::kDpl;
  constexpr int VEC = Sh::kVec;
  constexpr int NL = Sh::kLoads;
  constexpr int NG = Sh::kGroups;
  constexpr int NW = Sh::kWaves;

  __shared__ float s_acc[NW][G][D];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];

  const int g = blockIdx.x;
  const int split = blockIdx.y;
  const int b = blockIdx.z;
  const int Hkv = gridDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & (RL - 1);
  const int grp = wave * Sh::kGroupsPerWave + lane / RL;
  const int h0 = g * G;

  const int L = min(a.seq_lens[b], a.cap);
  const int64_t start = (int64_t)split * a.chunk;
  const int64_t end = min((int64_t)L, start + a.chunk);
  const int64_t ws0 = ((int64_t)b * a.Hq + h0) * a.S + split;

  if (start >= end) {
    // Empty slice (or an invalid length): the neutral partial, weight zero.
    for (int idx = tid; idx < G * D; idx += Sh::kThreads) {
      const int h = idx / D, e = idx - (idx / D) * D;
      a.ws_acc[(ws0 + (int64_t)h * a.S) * D + e] = 0.0f;
    }
    if (tid < G) {
      a.ws_m[ws0 + (int64_t)tid * a.S] = -INFINITY;
      a.ws_l[ws0 + (int64_t)tid * a.S] = 0.0f;
    }
    return;
  }

  // This lane's slice of the G query vectors, pre-scaled into base-2 units.
  float qr[G][DPL];
  const int64_t qbase = ((int64_t)b * a.Hq + h0) * D;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < NL; ++j)
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        qr[h][j * VEC + e] =
            load_q(a.q, a.q_dtype, qbase + h * D + j * RL * VEC + li * VEC + e) * a.qscale;

  float m[G], l[G], acc[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[h][d] = 0.0f;
  }

  const KV* __restrict__ kp = reinterpret_cast<const KV*>(a.k);
  const KV* __restrict__ vp = reinterpret_cast<const KV*>(a.v);
  const int64_t seq_base = (int64_t)b * a.stride_seq + (int64_t)g * a.stride_head;
  const int lane_col = li * VEC;

  for (int64_t base = start; base < end; base += NG * R) {
    Vec<KV, VEC> kr[R][NL], vr[R][NL];
    bool ok[R];
    bool bad[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int64_t pos = base + r * NG + grp;
      ok[r] = pos < end;
      pos = ok[r] ? pos : end - 1;
      int64_t off;
      if constexpr (PAGED) {
        int page = a.block_table[(int64_t)b * a.max_pages + (pos >> a.page_shift)];
        bad[r] = page < 0 || (int64_t)page >= a.num_pages;
        page = bad[r] ? 0 : page;
        const int64_t slot = pos & ((1 << a.page_shift) - 1);
        off = ((((int64_t)page << a.page_shift) + slot) * Hkv + g) * D;
      } else {
        bad[r] = false;
        off = seq_base + pos * a.stride_pos;
      }
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        kr[r][j] = load_vec<KV, VEC>(kp + off + j * RL * VEC + lane_col);
        vr[r][j] = load_vec<KV, VEC>(vp + off + j * RL * VEC + lane_col);
      }
    }

    float s[G][R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float p = 0.0f;
#pragma unroll
        for (int j = 0; j < NL; ++j)
#pragma unroll
          for (int e = 0; e < VEC; ++e) p = fmaf(qr[h][j * VEC + e], to_f32(kr[r][j].v[e]), p);
        p = row_sum<RL>(p);
        s[h][r] = ok[r] ? (bad[r] ? __builtin_nanf("") : p) : -INFINITY;
      }
    }

#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mt = s[h][0];
#pragma unroll
      for (int r = 1; r < R; ++r) mt = fmaxf(mt, s[h][r]);
      const float mn = fmaxf(m[h], mt);
      const float mu = (mn == -INFINITY) ? 0.0f : mn;
      const float al = fast_exp2(m[h] - mu);
      float p[R];
      float ls = 0.0f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        p[r] = fast_exp2(s[h][r] - mu);
        ls += p[r];
      }
      l[h] = fmaf(l[h], al, ls);
#pragma unroll
      for (int j = 0; j < NL; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float t = acc[h][j * VEC + e] * al;
#pragma unroll
          for (int r = 0; r < R; ++r) t = fmaf(p[r], to_f32(vr[r][j].v[e]), t);
          acc[h][j * VEC + e] = t;
        }
      m[h] = mn;
    }
  }

  // Merge the row groups of each wave, then the waves through LDS.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mw = groups_max<RL>(m[h]);
    const float mwu = (mw == -INFINITY) ? 0.0f : mw;
    const float f = fast_exp2(m[h] - mwu);
    const float lw = groups_sum<RL>(l[h] * f);
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[h][d] = groups_sum<RL>(acc[h][d] * f);
    if (lane == 0) {
      s_m[wave][h] = mw;
      s_l[wave][h] = lw;
    }
    if (lane < RL) {
#pragma unroll
      for (int j = 0; j < NL; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) s_acc[wave][h][j * RL * VEC + lane_col + e] = acc[h][j * VEC + e];
    }
  }
  __syncthreads();

  for (int idx = tid; idx < G * D; idx += Sh::kThreads) {
    const int h = idx / D, e = idx - (idx / D) * D;
    float mb = s_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) mb = fmaxf(mb, s_m[w][h]);
    const float mbu = (mb == -INFINITY) ? 0.0f : mb;
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t = fmaf(s_acc[w][h][e], fast_exp2(s_m[w][h] - mbu), t);
    a.ws_acc[(ws0 + (int64_t)h * a.S) * D + e] = t;
  }
  if (tid < G) {
    const int h = tid;
    float mb = s_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) mb = fmaxf(mb, s_m[w][h]);
    const float mbu = (mb == -INFINITY) ? 0.0f : mb;
    float lt = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) lt = fmaf(s_l[w][h], fast_exp2(s_m[w][h] - mbu), lt);
    a.ws_m[ws0 + (int64_t)h * a.S] = mb * kLn2;
    a.ws_l[ws0 + (int64_t)h * a.S] = lt;
  }
}

// Lane-per-row width and rows per group per tile for each (storage, width).
// These are the tuning knobs; the values are the ones measured best on MI355X.
#ifndef SK_GQA_RL256
#define SK_GQA_RL256 32
#endif
#ifndef SK_GQA_R256
#define SK_GQA_R256 4
#endif
#ifndef SK_GQA_RL128
#define SK_GQA_RL128 16
#endif
#ifndef SK_GQA_R128
#define SK_GQA_R128 2
#endif
#ifndef SK_GQA_RL64
#define SK_GQA_RL64 16
#endif
#ifndef SK_GQA_R64
#define SK_GQA_R64 2
#endif

template <int D>
struct Tune;
template <>
struct Tune<256> {
  static constexpr int RL = SK_GQA_RL256, R = SK_GQA_R256;
};
template <>
struct Tune<128> {
  static constexpr int RL = SK_GQA_RL128, R = SK_GQA_R128;
};
template <>
struct Tune<64> {
  static constexpr int RL = SK_GQA_RL64, R = SK_GQA_R64;
};

template <typename KV, int G, int D, bool PAGED>
static sk_status_t launch_variant(const SplitLaunch& s, bool launch, const void** fn, int grid[3],
                                  int* block) {
  const sk_desc_t& d = *s.d;
  auto kern = gqa_split_kernel<KV, G, D, PAGED, Tune<D>::RL, Tune<D>::R>;
  const dim3 gr(d.num_kv_heads, s.p->n_splits, d.batch);
  grid[0] = gr.x;
  grid[1] = gr.y;
  grid[2] = gr.z;
  *block = 256;
  if (fn) *fn = reinterpret_cast<const void*>(kern);
  if (!launch) return SK_OK;
  GqaArgs a;
  a.q = s.q;
  a.k = s.k;
  a.v = s.v;
  a.block_table = s.block_table;
  a.seq_lens = s.seq_lens;
  a.ws_acc = s.ws_acc;
  a.ws_m = s.ws_m;
  a.ws_l = s.ws_l;
  a.stride_seq = d.stride_seq;
  a.stride_pos = d.stride_pos;
  a.stride_head = d.stride_head;
  a.num_pages = d.num_pages;
  a.q_dtype = d.q_dtype;
  a.Hq = d.num_q_heads;
  a.S = s.p->n_splits;
  a.chunk = s.p->chunk;
  a.cap = d.max_seq_len;
  a.page_shift = 0;
  if (PAGED) {
    while ((1 << a.page_shift) < d.page_size) ++a.page_shift;
  }
  a.max_pages = d.max_pages_per_seq;
  a.qscale = d.scale * kLog2e;
  hipLaunchKernelGGL(kern, gr, dim3(256), 0, s.stream, a);
  return SK_OK;
}

template <typename KV, int G, int D>
static sk_status_t by_layout(const SplitLaunch& s, bool launch, const void** fn, int grid[3],
                             int* block) {
  if (s.d->layout == SK_KV_PAGED) return launch_variant<KV, G, D, true>(s, launch, fn, grid, block);
  return launch_variant<KV, G, D, false>(s, launch, fn, grid, block);
}

template <typename KV, int G>
static sk_status_t by_dim(const SplitLaunch& s, bool launch, const void** fn, int grid[3],
                          int* block) {
  switch (s.d->head_dim_qk) {
    case 64: return by_layout<KV, G, 64>(s, launch, fn, grid, block);
    case 128: return by_layout<KV, G, 128>(s, launch, fn, grid, block);
    case 256: return by_layout<KV, G, 256>(s, launch, fn, grid, block);
    default: return SK_ERR_UNSUPPORTED;
  }
}

template <typename KV>
static sk_status_t by_group(const SplitLaunch& s, bool launch, const void** fn, int grid[3],
                            int* block) {
  switch (s.d->num_q_heads / s.d->num_kv_heads) {
    case 1: return by_dim<KV, 1>(s, launch, fn, grid, block);
    case 2: return by_dim<KV, 2>(s, launch, fn, grid, block);
    case 4: return by_dim<KV, 4>(s, launch, fn, grid, block);
    case 6: return by_dim<KV, 6>(s, launch, fn, grid, block);
    case 8: return by_dim<KV, 8>(s, launch, fn, grid, block);
    default: return SK_ERR_UNSUPPORTED;
  }
}

bool gqa_supported(const sk_desc_t& d) {
  if (d.kv_shared) return false;
  if (d.head_dim_qk != d.head_dim_v) return false;
  if (d.head_dim_qk != 64 && d.head_dim_qk != 128 && d.head_dim_qk != 256) return false;
  const int G = d.num_q_heads / d.num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 6 && G != 8) return false;
  return d.kv_dtype == SK_F32 || d.kv_dtype == SK_F16 || d.kv_dtype == SK_BF16;
}

sk_status_t gqa_split_launch(const SplitLaunch& s, bool launch, const void** fn, int grid[3],
                             int* block) {
  if (!gqa_supported(*s.d)) return SK_ERR_UNSUPPORTED;
  switch (s.d->kv_dtype) {
    case SK_F32: return by_group<float>(s, launch, fn, grid, block);
    case SK_F16: return by_group<_Float16>(s, launch, fn, grid, block);
    case SK_BF16: return by_group<bf16_t>(s, launch, fn, grid, block);
    default: return SK_ERR_UNSUPPORTED;
  }
}

}  // namespace sk
