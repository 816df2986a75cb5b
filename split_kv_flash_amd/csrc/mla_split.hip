// Shared-latent split kernel (multi-head latent attention in absorbed form).
//
// Every query head attends one shared row of 576 latent columns per position
// (512 value columns followed by 64 rotary columns); the values are the first
// 512 columns of the same row ("The Kernel Level: Attention and MoE", section
// "Decode Starves the SMs ...": 128 heads packed as GEMM rows against one
// K-dim-576 cache, each latent block loaded from HBM once for all heads;
// Lecture 06 section 1.1: one block per head streams the same cache once per
// head). One workgroup per context split therefore serves ALL query heads, and
// each cache row crosses HBM once per decode step.
//
// The two products are dense contractions, so both run on MFMA:
//   scores  S[h][j] = sum_d Q[h][d] C[j][d]    (heads x positions, K = 576)
//   output  acc[h][e] += sum_j P[h][j] C[j][e] (heads x values,    K = positions)
// with the online-softmax update between them. f16 caches use
// v_mfma_f32_16x16x16_f16 (q and the probabilities rounded to f16, f32
// accumulation); f32 caches use v_mfma_f32_16x16x4_f32 (no rounding).
//
// Workgroup: 512 threads = 8 waves, one per split. Per tile of T positions:
//   1. the tile of cache rows (T x 576) is staged in LDS (row-padded); the next
//      tile's global loads are already in flight;
//   2. score phase: wave w = (head half, column quarter) computes the partial
//      scores of its heads over its 144 columns (split K); Q stays in registers
//      for f16 caches and is read through the cache hierarchy for f32 caches;
//   3. softmax phase: partials are summed from LDS, each wave updates the
//      running max / normaliser of 1/8 of the heads and writes the tile's
//      probabilities and rescale factors to LDS;
//   4. output phase: wave w owns 64 value columns for every head; it rescales
//      its accumulators and adds P (from LDS) times the tile's value columns.
// LDS use depends only on T and the head count, never on the context length.
#include "sk_device.h"
#include "sk_internal.h"

namespace sk {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kLatDk = 576;
constexpr int kLatDv = 512;
constexpr int kMlaWaves = 8;
constexpr int kMlaThreads = 64 * kMlaWaves;
constexpr int kDimSplit = 4;                   // score phase: 2 head halves x 4 column quarters
constexpr int kDimQ = kLatDk / kDimSplit;      // 144 columns per quarter
constexpr int kColsPerWave = kLatDv / kMlaWaves;  // 64 value columns per wave

struct MlaArgs {
  const float* q;
  const void* c;
  const int32_t* seq_lens;
  float* ws_acc;
  float* ws_m;
  float* ws_l;
  int64_t stride_seq, stride_pos;
  int32_t Hq, S, chunk, cap;
  float qscale;  // scale * log2(e): scores are kept in base-2 units
};

template <typename CT>
struct MlaCfg;
template <>
struct MlaCfg<_Float16> {
  static constexpr int T = 32;     // positions per tile
  static constexpr int KW = 16;    // MFMA K per instruction
  static constexpr int ROW = 584;  // LDS row stride (elements): 576 + 8
  using PT = _Float16;
};
template <>
struct MlaCfg<float> {
  static constexpr int T = 16;
  static constexpr int KW = 4;
  static constexpr int ROW = 596;  // 576 + 20: conflict-free score-phase reads
  using PT = float;
};

__device__ __forceinline__ float4_t mfma(half4_t a, half4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma(float a, float b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Max / sum over the T consecutive lanes that hold one head's tile (T = 16: a
// DPP row; T = 32: two rows joined by a swizzle).
template <int T>
__device__ __forceinline__ float seg_max(float x) {
  x = fmaxf(x, dpp<kDppRowRor8>(x));
  x = fmaxf(x, dpp<kDppRowRor4>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  if constexpr (T == 32) x = fmaxf(x, xor16(x));
  return x;
}
template <int T>
__device__ __forceinline__ float seg_sum(float x) {
  x = row16_sum(x);
  if constexpr (T == 32) x += xor16(x);
  return x;
}

template <typename CT, int NHB>
__global__ __launch_bounds__(kMlaThreads) void mla_split_kernel(MlaArgs a) {
  using Cfg = MlaCfg<CT>;
  using PT = typename Cfg::PT;
  constexpr int T = Cfg::T, KW = Cfg::KW, ROW = Cfg::ROW;
  constexpr int H = NHB * 16;           // query heads
  constexpr int HBW = NHB / 2;          // head blocks per wave in the score phase
  constexpr int KSTEPS = kDimQ / KW;    // MFMA steps over a column quarter
  constexpr int PB = T / 16;            // 16-position blocks per tile
  constexpr int PROW = T + 4;           // LDS row stride of P (elements)
  constexpr int EPC = 16 / (int)sizeof(CT);            // elements per 16-byte chunk
  constexpr int CPR = kLatDk / EPC;                    // chunks per cache row
  constexpr int CHUNKS = T * CPR;                      // chunks per tile
  constexpr int CPT = (CHUNKS + kMlaThreads - 1) / kMlaThreads;
  constexpr int HPI = 64 / T;                          // heads per softmax step per wave
  constexpr int ITER = H / kMlaWaves / HPI;            // softmax steps per wave
  constexpr bool kQInRegs = sizeof(CT) == 2;
  static_assert(H % (kMlaWaves * HPI) == 0, "head count must split over the waves");
  using CV = Vec<CT, EPC>;

  __shared__ __align__(16) CT s_c[T * ROW];
  __shared__ float s_sp[kDimSplit][H][T + 1];
  __shared__ __align__(16) PT s_p[H * PROW];
  __shared__ float s_alpha[H];

  const int split = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lq = lane >> 4;

  const int L = min(a.seq_lens[b], a.cap);
  const int64_t start = (int64_t)split * a.chunk;
  const int64_t end = min((int64_t)L, start + a.chunk);
  const int64_t ws0 = (int64_t)b * a.Hq * a.S + split;  // + h*S for head h

  if (start >= end) {
    for (int idx = tid; idx < H * kLatDv; idx += kMlaThreads) {
      const int h = idx / kLatDv, e = idx - (idx / kLatDv) * kLatDv;
      a.ws_acc[(ws0 + (int64_t)h * a.S) * kLatDv + e] = 0.0f;
    }
    for (int h = tid; h < H; h += kMlaThreads) {
      a.ws_m[ws0 + (int64_t)h * a.S] = -INFINITY;
      a.ws_l[ws0 + (int64_t)h * a.S] = 0.0f;
    }
    return;
  }

  const CT* __restrict__ cbase = reinterpret_cast<const CT*>(a.c) + (int64_t)b * a.stride_seq;
  const float* __restrict__ qb = a.q + (int64_t)b * a.Hq * kLatDk;

  // Staging of one tile: rows past the end re-read row end-1 (a cache hit).
  CV stage[CPT];
  auto load_tile = [&](int64_t tb) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * kMlaThreads;
      if (CHUNKS % kMlaThreads == 0 || idx < CHUNKS) {
        const int r = idx / CPR, cc = idx - (idx / CPR) * CPR;
        int64_t pos = tb + r;
        pos = pos < end ? pos : end - 1;
        stage[c] = load_vec<CT, EPC>(cbase + pos * a.stride_pos + cc * EPC);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * kMlaThreads;
      if (CHUNKS % kMlaThreads == 0 || idx < CHUNKS) {
        const int r = idx / CPR, cc = idx - (idx / CPR) * CPR;
        *reinterpret_cast<CV*>(&s_c[r * ROW + cc * EPC]) = stage[c];
      }
    }
  };

  // Score-phase role and the f16 query fragments (rounded once).
  const int hh = wave >> 2;  // head half
  const int dq = wave & 3;   // column quarter
  half4_t qf[kQInRegs ? HBW : 1][kQInRegs ? KSTEPS : 1];
  if constexpr (kQInRegs) {
#pragma unroll
    for (int hbl = 0; hbl < HBW; ++hbl)
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int head = (hh * HBW + hbl) * 16 + l16;
          const int dim = dq * kDimQ + ks * KW + lq * 4 + e;
          qf[hbl][ks][e] = (_Float16)qb[head * kLatDk + dim];
        }
  }

  // Softmax-phase state: this lane's head for step `it` is
  // wave + 8 * (it * HPI + lane / T), position lane % T.
  const int hsub = lane / T;
  const int spos = lane % T;
  float m_r[ITER], l_r[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    m_r[it] = -INFINITY;
    l_r[it] = 0.0f;
  }

  // Output-phase accumulators: heads hb*16 + 4*lq + e, columns
  // 64*wave + 16*cb + l16.
  float4_t acc[NHB][4];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[hb][cb] = float4_t{0.f, 0.f, 0.f, 0.f};

  load_tile(start);
  for (int64_t tb = start; tb < end; tb += T) {
    __syncthreads();  // the previous tile's readers of s_c and s_p are done
    store_tile();
    if constexpr (kQInRegs) load_tile(tb + T);
    __syncthreads();

    // ---- scores: partial over this wave's 144 columns ----
    float4_t sacc[HBW][PB];
#pragma unroll
    for (int hbl = 0; hbl < HBW; ++hbl)
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) sacc[hbl][pb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) {
        const int prow = pb * 16 + l16;
        if constexpr (kQInRegs) {
          const int dim = dq * kDimQ + ks * KW + lq * 4;
          const half4_t bv = *reinterpret_cast<const half4_t*>(&s_c[prow * ROW + dim]);
#pragma unroll
          for (int hbl = 0; hbl < HBW; ++hbl) sacc[hbl][pb] = mfma(qf[hbl][ks], bv, sacc[hbl][pb]);
        } else {
          const int dim = dq * kDimQ + ks * KW + lq;
          const float bv = (float)s_c[prow * ROW + dim];
#pragma unroll
          for (int hbl = 0; hbl < HBW; ++hbl) {
            const int head = (hh * HBW + hbl) * 16 + l16;
            const float av = qb[head * kLatDk + dim];
            sacc[hbl][pb] = mfma(av, bv, sacc[hbl][pb]);
          }
        }
      }
    }
#pragma unroll
    for (int hbl = 0; hbl < HBW; ++hbl)
#pragma unroll
      for (int pb = 0; pb < PB; ++pb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s_sp[dq][(hh * HBW + hbl) * 16 + lq * 4 + e][pb * 16 + l16] = sacc[hbl][pb][e];
    if constexpr (!kQInRegs) load_tile(tb + T);
    __syncthreads();

    // ---- online softmax over the tile, 1/8 of the heads per wave ----
    {
      const bool ok = tb + spos < end;
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        const int h = wave + kMlaWaves * (it * HPI + hsub);
        float s = (s_sp[0][h][spos] + s_sp[1][h][spos]) + (s_sp[2][h][spos] + s_sp[3][h][spos]);
        s = ok ? s * a.qscale : -INFINITY;
        const float mn = fmaxf(m_r[it], seg_max<T>(s));
        const float mu = (mn == -INFINITY) ? 0.0f : mn;
        const float al = fast_exp2(m_r[it] - mu);
        const PT pr = (PT)fast_exp2(s - mu);
        l_r[it] = fmaf(l_r[it], al, seg_sum<T>((float)pr));
        m_r[it] = mn;
        s_p[h * PROW + spos] = pr;
        if (spos == 0) s_alpha[h] = al;
      }
    }
    __syncthreads();

    // ---- output: rescale, then acc += P x V for this wave's 64 columns ----
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      float al[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) al[e] = s_alpha[hb * 16 + lq * 4 + e];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[hb][cb][e] *= al[e];
    }
    const int col0 = wave * kColsPerWave + l16;
#pragma unroll
    for (int ks = 0; ks < T / KW; ++ks) {
      if constexpr (kQInRegs) {
        half4_t vb[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int e = 0; e < 4; ++e) vb[cb][e] = s_c[(ks * KW + lq * 4 + e) * ROW + col0 + cb * 16];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          const half4_t pa =
              *reinterpret_cast<const half4_t*>(&s_p[(hb * 16 + l16) * PROW + ks * KW + lq * 4]);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) acc[hb][cb] = mfma(pa, vb[cb], acc[hb][cb]);
        }
      } else {
        float vb[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) vb[cb] = (float)s_c[(ks * KW + lq) * ROW + col0 + cb * 16];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          const float pa = (float)s_p[(hb * 16 + l16) * PROW + ks * KW + lq];
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) acc[hb][cb] = mfma(pa, vb[cb], acc[hb][cb]);
        }
      }
    }
  }

  // Partials: accumulators by the column owner, (m, l) by the softmax owner.
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int head = hb * 16 + lq * 4 + e;
        const int col = wave * kColsPerWave + cb * 16 + l16;
        a.ws_acc[(ws0 + (int64_t)head * a.S) * kLatDv + col] = acc[hb][cb][e];
      }
  if (spos == 0) {
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int h = wave + kMlaWaves * (it * HPI + hsub);
      a.ws_m[ws0 + (int64_t)h * a.S] = m_r[it] * kLn2;
      a.ws_l[ws0 + (int64_t)h * a.S] = l_r[it];
    }
  }
}

bool latent_supported(const sk_desc_t& d) {
  return d.kv_shared == 1 && d.num_kv_heads == 1 && d.head_dim_qk == kLatDk &&
         d.head_dim_v == kLatDv && d.layout == SK_KV_CONTIGUOUS && d.q_dtype == SK_F32 &&
         (d.kv_dtype == SK_F32 || d.kv_dtype == SK_F16) &&
         (d.num_q_heads == 32 || d.num_q_heads == 64 || d.num_q_heads == 96 ||
          d.num_q_heads == 128);
}

template <typename CT, int NHB>
static sk_status_t latent_variant(const SplitLaunch& s, bool launch, const void** fn, int grid[3],
                                  int* block) {
  const sk_desc_t& d = *s.d;
  auto kern = mla_split_kernel<CT, NHB>;
  const dim3 gr(s.p->n_splits, d.batch, 1);
  grid[0] = gr.x;
  grid[1] = gr.y;
  grid[2] = gr.z;
  *block = kMlaThreads;
  if (fn) *fn = reinterpret_cast<const void*>(kern);
  if (!launch) return SK_OK;
  MlaArgs a;
  a.q = reinterpret_cast<const float*>(s.q);
  a.c = s.k;
  a.seq_lens = s.seq_lens;
  a.ws_acc = s.ws_acc;
  a.ws_m = s.ws_m;
  a.ws_l = s.ws_l;
  a.stride_seq = d.stride_seq;
  a.stride_pos = d.stride_pos;
  a.Hq = d.num_q_heads;
  a.S = s.p->n_splits;
  a.chunk = s.p->chunk;
  a.cap = d.max_seq_len;
  a.qscale = d.scale * kLog2e;
  hipLaunchKernelGGL(kern, gr, dim3(kMlaThreads), 0, s.stream, a);
  return SK_OK;
}

template <typename CT>
static sk_status_t latent_by_heads(const SplitLaunch& s, bool launch, const void** fn, int grid[3],
                                   int* block) {
  switch (s.d->num_q_heads) {
    case 32: return latent_variant<CT, 2>(s, launch, fn, grid, block);
    case 64: return latent_variant<CT, 4>(s, launch, fn, grid, block);
    case 96: return latent_variant<CT, 6>(s, launch, fn, grid, block);
    case 128: return latent_variant<CT, 8>(s, launch, fn, grid, block);
    default: return SK_ERR_UNSUPPORTED;
  }
}

sk_status_t latent_split_launch(const SplitLaunch& s, bool launch, const void** fn, int grid[3],
                                int* block) {
  if (!latent_supported(*s.d)) return SK_ERR_UNSUPPORTED;
  if (s.d->kv_dtype == SK_F16) return latent_by_heads<_Float16>(s, launch, fn, grid, block);
  return latent_by_heads<float>(s, launch, fn, grid, block);
}

}  // namespace sk
