// Query-tile online attention: several query positions per sequence, causal.
//
// "Decoder Block 6: Online Attention, the Capstone": keep a tile of query rows
// resident, stage each K/V tile on chip once and let every row of the tile
// consume it; each row carries its running maximum m, normaliser l and
// unnormalised accumulator, and at every K/V tile
//     m' = max(m, tile max), alpha = exp(m - m'),
//     l  = alpha l + sum_j exp(s_j - m'),  acc = alpha acc + sum_j exp(s_j - m') v_j.
// The query rows here are the (query position, head) pairs of one KV group:
// query t of a sequence of L positions sits at position L - q_len + t and sees
// positions [0, L - q_len + t] (q_len = 1 is decode, q_len = L is causal
// self-attention). The context is also split (Lecture 06 section 2): a
// workgroup covers one slice and writes the partial (m, l, acc) of each of its
// rows, and the combine kernel merges the slices, so a few query rows over a
// long context (speculative verify) still fill the GPU.
//
// Work decomposition (MI355X-first):
//   * One workgroup (4 waves) per (sequence, KV head, query tile, context
//     slice), rows ordered (position t, head) so a tile's rows have
//     neighbouring causal limits. A tile is 64 rows, wave w owning rows
//     16w .. 16w+15; when a KV head has only 16 or 32 query rows the tile
//     shrinks to them and the waves of a 16-row block share out the head
//     width instead (see the DS parameter).
//   * K/V tiles of 32 positions go from HBM straight into LDS
//     (global_load_lds_dwordx4) in a ring of four buffers, three tiles in
//     flight while one is consumed; rows unpadded, 16-byte chunks XOR-swizzled
//     by row & 7; one barrier per tile (two with the score exchange).
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_16x16x32_{f16,bf16}: the K rows are the A operand and the
//     query rows (held in registers) the B operand. The result leaves lane
//     (row l16, quarter lq) holding positions 4lq+i and 16+4lq+i of its row,
//     which, with the contraction index ordered the same way, is exactly that
//     lane's A operand of the output product P V; the V operands come from the
//     gfx950 transpose read ds_read_b64_tr_b16 in the same position order. P
//     never goes through LDS.
//   * Precision: the MFMA inputs are 16-bit, so q and P are each split into
//     16-bit parts, one product per part: two f16 parts (22 bits) or three
//     bf16 parts (24 bits), so scores and weights keep close to f32 accuracy
//     while K and V are used exactly as stored. f16's second part of q is
//     taken times 2^11, which keeps it out of f16's subnormal range, and its
//     products go to an accumulator of their own that is added back times
//     2^-11.
#include "sk_device.h"
#include "sk_internal.h"
#include "sk_merge.h"

namespace sk {

typedef _Float16 qt_half8 __attribute__((ext_vector_type(8)));
typedef __bf16 qt_bf8 __attribute__((ext_vector_type(8)));
typedef float qt_f4 __attribute__((ext_vector_type(4)));
typedef short qt_s4 __attribute__((ext_vector_type(4)));
typedef short qt_s8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) qt_s4 qt_lds_s4;
typedef uint32_t qt_u4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk

struct QtArgs {
  const void* q;  // [B][Q][Hq][D]
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  float* ws_acc;  // [B][Q*Hq][S][D], row (t, h) = t*Hq + h
  float* ws_m;
  float* ws_l;
  int64_t stride_seq, stride_pos, stride_head;
  int32_t q_dtype;
  int32_t Q, Hq, G, S, chunk, cap, nqt;  // nqt: 64-row query tiles per KV head
  float qscale;                          // scale * log2(e)
  // One-launch decode only (Q = 1).
  uint32_t* counters;  // [B][Hkv], zero between calls
  float* out;          // [B][Hq][D]
  float* lse;          // [B][Hq] or null
};

// Splits of one merge pass of the one-launch kernel (its m and l values sit in
// the freed K/V ring).
constexpr int kQtMergePass = 64;

// 16-bit storage types: round-to-nearest-even conversion from f32, widening,
// and the 16x16x32 MFMA of that type.
template <typename KT>
struct QtType;
template <>
struct QtType<_Float16> {
  static constexpr int kParts = 2;  // 11 + 11 significand bits
  // The second part of q is stored times 2^11: what the first part leaves is
  // below 2^-11 of it, and for query values near 0.1 (q scale/sqrt(D) log2 e)
  // that would be an f16 subnormal with a few significant bits.
  static constexpr float kLoScale = 2048.0f;
  static __device__ __forceinline__ short from(float x) { return __builtin_bit_cast(short, (_Float16)x); }
  static __device__ __forceinline__ float to(short b) { return (float)__builtin_bit_cast(_Float16, b); }
  static __device__ __forceinline__ qt_f4 mma(qt_s8 a, qt_s8 b, qt_f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(qt_half8, a),
                                                  __builtin_bit_cast(qt_half8, b), c, 0, 0, 0);
  }
};
template <>
struct QtType<bf16_t> {
  static constexpr int kParts = 3;  // 8 + 8 + 8 significand bits
  static constexpr float kLoScale = 1.0f;  // bf16 has f32's exponent range
  static __device__ __forceinline__ short from(float x) { return __builtin_bit_cast(short, (__bf16)x); }
  static __device__ __forceinline__ float to(short b) {
    return __uint_as_float(((uint32_t)(uint16_t)b) << 16);
  }
  static __device__ __forceinline__ qt_f4 mma(qt_s8 a, qt_s8 b, qt_f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(qt_bf8, a),
                                                   __builtin_bit_cast(qt_bf8, b), c, 0, 0, 0);
  }
};

// The value itself, hidden from the optimiser: what is computed from it
// starts from this rounded f32 value and cannot be fused with its producer.
__device__ __forceinline__ float opaque_f32(float x) {
  asm("" : "+v"(x));
  return x;
}

__device__ __forceinline__ qt_s4 qt_read_tr(const short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((qt_lds_s4*)(p));
}

// DS: waves sharing one 16-row block. With DS > 1, wave w takes row block
// w / DS and the column part w % DS of the head width: it forms the partial
// scores over its columns, the DS partials meet in LDS and are summed in a
// fixed order (so every wave of the block derives the same softmax), and it
// accumulates its own output columns. Few query rows (speculative verify) then
// keep all four waves busy instead of one.
//
// FUSED (one query per sequence: the one-launch decode): partials are
// written with device-scope stores, and the workgroup that completes the
// (sequence, KV head)'s count merges them into out and lse, as the GQA split
// kernel's one-launch variant does; empty slices take no part, and an invalid
// length makes that sequence's outputs NaN.
template <typename KT, int D, int DS, bool FUSED>
__global__ __launch_bounds__(256) void query_tile_kernel(QtArgs a) {
  using TT = QtType<KT>;
  constexpr int NP = TT::kParts;  // parts of q and of the softmax weights
  constexpr int T = 32;         // positions per K/V tile
  constexpr int KS = D / 32;    // score MFMA steps over the head width
  constexpr int CB = D / 16;    // output column blocks over the head width
  constexpr int KSW = KS / DS;  // score steps of one wave
  constexpr int CBW = CB / DS;  // output column blocks of one wave
  constexpr int RB = 4 / DS;    // row blocks per workgroup
  constexpr int RW = 16 * RB;   // query rows per workgroup
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int NB = 4;         // LDS tile buffers: three tiles in flight while one is consumed
  constexpr int WLH = T * CPR / 64;  // wave-loads of 64 chunks per tile half (K or V)
  constexpr int DPW = 2 * WLH / 4;   // wave-loads per wave per tile (half K, then half V)
  static_assert(D % 64 == 0 && KS % DS == 0 && (DS == 1 || DS == 2 || DS == 4), "head width / split");
  static_assert(DPW % 2 == 0 && CPR >= 8, "even split of a wave's loads; 8-chunk swizzle");

  // [buffer][K, V][row * D + column], rows unpadded, the 16-byte chunk index of
  // row r stored XOR-ed with r & 7 (conflict-free score and transpose reads).
  __shared__ __align__(16) short s_kv[NB][2][T * D];
  __shared__ __align__(16) float s_sc[DS > 1 ? 4 : 1][64][8];  // partial scores per wave and lane

  const int g = blockIdx.x / a.nqt;
  const int qt = blockIdx.x - g * a.nqt;
  const int split = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lq = lane >> 4;
  const int rb = wave / DS;       // row block
  const int dq = wave - rb * DS;  // column part
  const int QG = a.Q * a.G;
  const int QH = a.Q * a.Hq;

  const int Lraw = a.seq_lens[b];
  if constexpr (FUSED) {
    const bool valid = Lraw >= 1 && Lraw <= a.cap && (int64_t)Lraw <= (int64_t)a.S * a.chunk;
    if (!valid) {
      if (split == 0) {
        for (int idx = tid; idx < a.G * D; idx += 256)
          a.out[((int64_t)b * a.Hq + g * a.G) * D + idx] = __builtin_nanf("");
        if (a.lse && tid < a.G) a.lse[(int64_t)b * a.Hq + g * a.G + tid] = __builtin_nanf("");
      }
      return;
    }
    if ((int64_t)split * a.chunk >= Lraw) return;  // an empty slice takes no part in the merge
  }
  const int L = min(Lraw, a.cap);
  const int64_t start = (int64_t)split * a.chunk;
  const int64_t end = min((int64_t)L, start + a.chunk);

  // This lane's query row (scores and softmax): row l16 of the row block.
  const int rho = qt * RW + rb * 16 + l16;
  const bool rvalid = rho < QG;
  const int t = rvalid ? rho / a.G : 0;
  const int hh = rvalid ? rho - t * a.G : 0;
  const int64_t lim = rvalid ? (int64_t)L - a.Q + t + 1 : 0;  // visible: positions < lim
  // The tile's rows are ordered by position, so its last row sees the most.
  const int rho_last = min(qt * RW + RW - 1, QG - 1);
  const int64_t lim_max = (int64_t)L - a.Q + rho_last / a.G + 1;
  const int64_t stop = min(end, lim_max);  // this workgroup reads positions [start, stop)

  float m = -INFINITY, l = 0.0f;  // row l16 (replicated over the quarters), base-2 units
  qt_f4 acc[CBW];  // output columns 16 (dq CBW + c) + l16
#pragma unroll
  for (int c = 0; c < CBW; ++c) acc[c] = qt_f4{0.f, 0.f, 0.f, 0.f};

  if (start < stop) {
    // Query row as B operands: lane (l16, lq) holds columns 32ks + 8lq .. +7 of
    // row l16 (ks over this wave's column part), pre-scaled into base-2 units
    // and split into NP parts, each the rounding of what the previous ones
    // left (their sum carries 22 bits for f16 and 24 for bf16).
    qt_s8 qp[NP][KSW];
    {
      const int64_t qbase = (((int64_t)b * a.Q + t) * a.Hq + g * a.G + hh) * D + 32 * KSW * dq;
      // Eight consecutive elements per step, widened to f32: every load is
      // issued before the first conversion, under uniform branches on the
      // run-time type (0 f32, 1 f16, 2 bf16).
      float qv[KSW][8];
#pragma unroll
      for (int ks = 0; ks < KSW; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[ks][e] = 0.0f;
      if (rvalid) {
        const int64_t q0 = qbase + 8 * lq;
        if (a.q_dtype == 0) {
          float4 w[KSW][2];
#pragma unroll
          for (int ks = 0; ks < KSW; ++ks) {
            w[ks][0] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.q) + q0 + 32 * ks);
            w[ks][1] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.q) + q0 + 32 * ks + 4);
          }
#pragma unroll
          for (int ks = 0; ks < KSW; ++ks) {
            qv[ks][0] = w[ks][0].x; qv[ks][1] = w[ks][0].y; qv[ks][2] = w[ks][0].z; qv[ks][3] = w[ks][0].w;
            qv[ks][4] = w[ks][1].x; qv[ks][5] = w[ks][1].y; qv[ks][6] = w[ks][1].z; qv[ks][7] = w[ks][1].w;
          }
        } else {
          qt_u4 w[KSW];
#pragma unroll
          for (int ks = 0; ks < KSW; ++ks)
            w[ks] = *reinterpret_cast<const qt_u4*>(reinterpret_cast<const uint16_t*>(a.q) + q0 + 32 * ks);
          if (a.q_dtype == 1) {
#pragma unroll
            for (int ks = 0; ks < KSW; ++ks)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                qv[ks][2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[ks][e] & 0xffffu));
                qv[ks][2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[ks][e] >> 16));
              }
          } else {
#pragma unroll
            for (int ks = 0; ks < KSW; ++ks)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                qv[ks][2 * e] = __uint_as_float(w[ks][e] << 16);
                qv[ks][2 * e + 1] = __uint_as_float(w[ks][e] & 0xffff0000u);
              }
          }
        }
      }
      {
        // Each part must be the rounding of the very f32 value its residual is
        // taken from. Left to itself the compiler rounds the exact product
        // q*qscale straight to f16 (a mixed-precision fma) where it forms the
        // residual, but rounds it to f32 first where it forms the MFMA
        // operand; where the two roundings differ (about once in 2^14
        // elements) the parts then miss x by a whole f16 step. The product is
        // therefore made opaque, and contraction is off for the split.
#pragma clang fp contract(off)
#pragma unroll
        for (int ks = 0; ks < KSW; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float x = opaque_f32(qv[ks][e] * a.qscale);
#pragma unroll
            for (int i = 0; i < NP; ++i) {
              const short part = TT::from(i == 1 ? x * TT::kLoScale : x);
              qp[i][ks][e] = part;
              x -= (i == 1 ? TT::to(part) / TT::kLoScale : TT::to(part));
            }
          }
      }
    }

    const KT* __restrict__ kp = reinterpret_cast<const KT*>(a.k) + (int64_t)b * a.stride_seq + (int64_t)g * a.stride_head;
    const KT* __restrict__ vp = reinterpret_cast<const KT*>(a.v) + (int64_t)b * a.stride_seq + (int64_t)g * a.stride_head;
    // Tile staging by direct global-to-LDS loads: wave-load wh of a tile half
    // (0 .. WLH-1, for K and again for V) fills 1 KB of the half's LDS rows; lane
    // slot s of it is row s / CPR, physical chunk p = s % CPR, which holds
    // logical chunk p ^ (row & 7). Rows past `stop` re-read row stop-1 (in
    // range; their scores are masked). With DS > 1 the KV group's query rows
    // fit one workgroup, the only reader of its rows: non-temporal loads,
    // which stream HBM faster on MI355X. Otherwise several query tiles read
    // the same rows and the plain policy lets the later reads hit the caches.
    const uint32_t lds_kv = (uint32_t)(size_t)(const __attribute__((address_space(3))) short*)(&s_kv[0][0][0]);
    // Every wave issues DPW/2 wave-loads of K, then the same of V: the whole
    // K half is requested before any V row, the order the scores need it in.
    const int wq0 = __builtin_amdgcn_readfirstlane(wave * (DPW / 2));
    // One wave-uniform base per tile and half, 32-bit lane offsets (the host
    // bounds a row step to 16 MB, so 32 rows stay below 2^32 bytes).
    const uint32_t row_bytes = (uint32_t)(a.stride_pos * (int64_t)sizeof(KT));
    auto issue = [&](int buf, int64_t tb) {
      const int64_t tbc = min(tb, stop - 1);
      const int last = (int)(stop - 1 - tbc);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint64_t bu = reinterpret_cast<uint64_t>((half ? vp : kp) + tbc * a.stride_pos);
        const void* base = reinterpret_cast<const void*>(
            ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(bu >> 32)) << 32) |
            (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bu));
#pragma unroll
        for (int c = 0; c < DPW / 2; ++c) {
          const int wh = wq0 + c;  // wave-load within the half
          const int sl = wh * 64 + lane;
          const int row = sl / CPR, p = sl - (sl / CPR) * CPR;
          const uint32_t off = (uint32_t)min(row, last) * row_bytes + (uint32_t)((p ^ (row & 7)) * 16);
          const uint32_t dst = lds_kv + (uint32_t)(((buf * 2 + half) * T * D + wh * 512) * 2);
          dma16s(off, base, __builtin_amdgcn_readfirstlane(dst), DS > 1);
        }
      }
    };

    // Uniform over the workgroup; said so, the loop exits on a scalar branch
    // instead of an exec-masked one (whose merged paths cost the loads' overlap).
    const int ntiles = __builtin_amdgcn_readfirstlane((int)((stop - start + T - 1) / T));
    // Consumes tile i from LDS buffer i % NB: scores, online softmax, output.
    auto consume = [&](int i) {
      const int64_t tb = start + (int64_t)i * T;
      const short* kb = s_kv[i % NB][0];
      const short* vb = s_kv[i % NB][1];

      // ---- scores S^T: two blocks of 16 positions, this block's 16 rows ----
      // sp: the products of q's unscaled parts; sl: those of its scaled second
      // part (f16), added back times 2^-11.
      constexpr bool kScaledLo = TT::kLoScale != 1.0f;
      qt_f4 sp[2] = {qt_f4{0.f, 0.f, 0.f, 0.f}, qt_f4{0.f, 0.f, 0.f, 0.f}};
      qt_f4 sl[2] = {qt_f4{0.f, 0.f, 0.f, 0.f}, qt_f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
#pragma unroll
        for (int ks = 0; ks < KSW; ++ks) {
          // row 16 pb + l16 (swizzle l16 & 7), logical chunk 4 (KSW dq + ks) + lq
          const qt_s8 av = *reinterpret_cast<const qt_s8*>(
              kb + (16 * pb + l16) * D + (((4 * (KSW * dq + ks) + lq) ^ (l16 & 7)) << 3));
#pragma unroll
          for (int i = 0; i < NP; ++i) {
            if (kScaledLo && i == 1)
              sl[pb] = TT::mma(av, qp[i][ks], sl[pb]);
            else
              sp[pb] = TT::mma(av, qp[i][ks], sp[pb]);
          }
        }
        if constexpr (kScaledLo) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sp[pb][e] = fmaf(sl[pb][e], 1.0f / TT::kLoScale, sp[pb][e]);
        }
      }
      if constexpr (DS > 1) {
        // Partial scores of the block's DS waves: same lane layout, summed in
        // wave order. The buffer is rewritten only after the tile's closing
        // barrier, which every wave reaches after this read.
        qt_f4* mine = reinterpret_cast<qt_f4*>(&s_sc[wave][lane][0]);
        mine[0] = sp[0];
        mine[1] = sp[1];
        wait_vm_lgkm0<63>();  // this wave's LDS writes done; tile loads stay in flight
        raw_barrier();
        const qt_f4* p0 = reinterpret_cast<const qt_f4*>(&s_sc[rb * DS][lane][0]);
        sp[0] = p0[0];
        sp[1] = p0[1];
#pragma unroll
        for (int j = 1; j < DS; ++j) {
          const qt_f4* pj = reinterpret_cast<const qt_f4*>(&s_sc[rb * DS + j][lane][0]);
          sp[0] += pj[0];
          sp[1] += pj[1];
        }
      }

      // ---- online softmax of row l16 over the tile's visible positions ----
      float s[8];
      float mx = -INFINITY;
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t pos = tb + 16 * pb + 4 * lq + e;
          s[4 * pb + e] = (pos < stop && pos < lim) ? sp[pb][e] : -INFINITY;
          mx = fmaxf(mx, s[4 * pb + e]);
        }
      mx = fmaxf(mx, xor16(mx));
      mx = fmaxf(mx, xor32(mx));
      const float mn = fmaxf(m, mx);
      const float mu = (mn == -INFINITY) ? 0.0f : mn;
      const float al = fast_exp2(m - mu);
      float ls = 0.0f;
      qt_s8 pp[NP];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float p = fast_exp2(s[j] - mu);
        ls += p;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const short part = TT::from(p);
          pp[i][j] = part;
          p -= TT::to(part);
        }
      }
      ls += xor16(ls);
      ls += xor32(ls);
      l = fmaf(l, al, ls);
      m = mn;
      // Accumulator item e is row 4lq + e, whose factor lane 4lq + e holds.
      if (__any(al != 1.0f)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ae = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * lq + e) << 2, __float_as_int(al)));
#pragma unroll
          for (int c = 0; c < CBW; ++c) acc[c][e] *= ae;
        }
      }

      // ---- output: acc += P V over this wave's columns, positions in the scores' order ----
      // Rows rv = 4 lq + l16/4 and rv + 16 (same swizzle rv & 7), columns
      // 16 (CBW dq + c) + 4 (l16 & 3): logical chunk 2 (CBW dq + c) + (l16 & 3)/2,
      // at half 4 (l16 & 1) within it.
      const int rv = 4 * lq + (l16 >> 2);
      const short* vrow = vb + rv * D + 4 * (l16 & 1);
#pragma unroll
      for (int c = 0; c < CBW; ++c) {
        const int vch = ((2 * (CBW * dq + c) + ((l16 & 3) >> 1)) ^ (rv & 7)) << 3;
        const qt_s4 v0 = qt_read_tr(vrow + vch);
        const qt_s4 v1 = qt_read_tr(vrow + 16 * D + vch);
        const qt_s8 vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int i = 0; i < NP; ++i) acc[c] = TT::mma(pp[i], vv, acc[c]);
      }
    };
    // Ring of NB = 4 buffers: tiles i+1 .. i+3 are in flight while tile i is
    // consumed. Tile i+3 goes to the buffer tile i-1 used, which every wave
    // left at the previous barrier; each wave then waits for its own loads of
    // tile i+1 (at most 2 DPW of its loads, tiles i+2 and i+3, remain) and the
    // barrier publishes the tile. Loads past the end re-read row stop-1.
    issue(0, start);
    issue(1, start + T);
    issue(2, start + 2 * T);
    wait_vm_lgkm0<2 * DPW>();
    raw_barrier();
    for (int i = 0; i < ntiles; ++i) {
      issue((i + 3) % NB, start + (int64_t)(i + 3) * T);
      consume(i);
      wait_vm_lgkm0<2 * DPW>();
      raw_barrier();
    }
    wait_vm_lgkm0<0>();  // no load into LDS outlives the workgroup
  }

  // ---- partials of this wave's rows and columns (rows with nothing visible: neutral) ----
  if constexpr (!FUSED) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int re = qt * RW + rb * 16 + 4 * lq + e;
      if (re < QG) {
        const int te = re / a.G;
        const int w = te * a.Hq + g * a.G + (re - te * a.G);
        float* dst = a.ws_acc + (((int64_t)b * QH + w) * a.S + split) * D + 16 * CBW * dq + l16;
#pragma unroll
        for (int c = 0; c < CBW; ++c) dst[16 * c] = acc[c][e];
      }
    }
  } else {
    // Device-scope stores in whole lines: the wave's 16 x 16*CBW block goes
    // through its own rows of the K/V ring (free: every wave has passed the
    // loop's last barrier; rows padded by four floats, so the writes of the
    // four row quarters fall in distinct banks) and out as 16-byte stores,
    // 4*CBW of them per row, from a wave-uniform base (one query per
    // sequence: the block's rows are consecutive partial rows). Scalar
    // device-scope stores of 64-byte row pieces cost this form about 10 us
    // at 262,144 positions.
    constexpr int WCOL = 16 * CBW;
    constexpr int PITCH = WCOL + 4;
    static_assert(4 * 16 * PITCH * (int)sizeof(float) <= (int)sizeof(s_kv), "the block fits the ring");
    float* tw = reinterpret_cast<float*>(&s_kv[0][0][0]) + wave * 16 * PITCH;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int c = 0; c < CBW; ++c) tw[(4 * lq + e) * PITCH + 16 * c + l16] = acc[c][e];
    wait_vm_lgkm0<0>();
    const int re0 = qt * RW + rb * 16;  // the block's first row (a head of the group)
    const int nrow = min(16, QG - re0);
    if (nrow > 0) {
      const int64_t rowstep = (int64_t)a.S * D;  // floats between consecutive heads' partial rows
      const float* base = a.ws_acc + (((int64_t)b * QH + g * a.G + re0) * a.S + split) * D + WCOL * dq;
      const auto rs = raw_rsrc(base, (uint32_t)((((int64_t)nrow - 1) * rowstep + WCOL) * 4));
#pragma unroll
      for (int k = 0; k < CBW; ++k) {
        const int j = k * 64 + lane;
        const int r = j / (WCOL / 4), c4 = j - (j / (WCOL / 4)) * (WCOL / 4);
        if (r < nrow) {
          st_dev4(rs, (uint32_t)(((int64_t)r * rowstep + 4 * c4) * 4),
                  *reinterpret_cast<const float4*>(tw + r * PITCH + 4 * c4));
        }
      }
    }
  }
  if (lq == 0 && rvalid && dq == 0) {
    const int64_t r = ((int64_t)b * QH + t * a.Hq + g * a.G + hh) * a.S + split;
    if constexpr (FUSED) {
      st_dev(a.ws_m + r, m * kLn2);
      st_dev(a.ws_l + r, l);
    } else {
      a.ws_m[r] = m * kLn2;
      a.ws_l[r] = l;
    }
  }

  if constexpr (FUSED) {
    // Every thread waits until its device-scope stores have completed; the
    // count then tells the last workgroup of the group that every partial is
    // in place, and it merges them (the K/V ring is free again).
    // The flag lives in the score exchange buffer, free by now: a separate
    // word would take width 64 past 40 KB and four workgroups per CU.
    int* s_last = reinterpret_cast<int*>(&s_sc[0][0][0]);
    __builtin_amdgcn_s_waitcnt(0);
    const int n = (int)((L + (int64_t)a.chunk - 1) / a.chunk);
    uint32_t* cnt = a.counters + ((int64_t)b * (a.Hq / a.G) + g) * merge_counter_words(a.S);
    static_assert(2 * 8 * kQtMergePass * 4 <= (int)sizeof(s_kv), "m, l of 8 heads per pass fit the ring");
    // Sixteen accumulator rows in flight per chunk at width 256 (one
    // workgroup per CU either way), four below it, which keeps the merge
    // within the registers of the resident count (16 took 200 at width 64).
    constexpr int MK = D >= 256 ? 16 : 4;
    merge_tree<D, 256, kQtMergePass, MK>(a, a.G, b, g * a.G, split, n, cnt, tid, s_last,
                                         reinterpret_cast<float*>(&s_kv[0][0][0]));
  }
}

bool query_tile_supported(const sk_desc_t& d) {
  return !d.kv_shared && d.layout == SK_KV_CONTIGUOUS && d.head_dim_qk == d.head_dim_v &&
         (d.head_dim_qk == 64 || d.head_dim_qk == 128 || d.head_dim_qk == 256) &&
         (d.kv_dtype == SK_F16 || d.kv_dtype == SK_BF16);
}

int query_tile_rows_tiles(const sk_desc_t& d, int q_len) {
  const int G = d.num_q_heads / d.num_kv_heads;
  return (q_len * G + 63) / 64;
}

// Waves per 16-row block: the head width is shared out when the query rows of
// a KV head fill only one or two row blocks (every choice keeps
// ceil(rows / 64) workgroups per KV head and slice).
static int query_tile_ways(int rows, int D) {
  if (rows <= 16 && D >= 128) return 4;
  if (rows <= 32) return 2;
  return 1;
}

// Workgroups one compute unit holds: the LDS tile ring with the score
// exchange is 136, 72 and 40 KB at head width 256, 128 and 64, of 160 KB per
// compute unit (registers allow more). A plan for fewer leaves the narrow
// widths with too few tiles in flight: with one per compute unit, decode at
// width 128 took 126 us where two per unit take 93 us (8 KV heads, 131,072
// f16 positions), and width 64 took 113 us where four take 60 us.
int query_tile_resident(const sk_desc_t& d) {
  return d.head_dim_qk >= 256 ? 1 : (d.head_dim_qk >= 128 ? 2 : 4);
}

// Single-query decode on the query-tile kernel (q_len = 1: the rows are the
// group's heads, and its partials have the split kernel's layout) where that
// measured faster on MI355X: the MFMA score and output products keep wide
// groups and narrow heads at the memory rate, while the vector split kernel
// runs out of ALU issue with more heads per KV row (at 131,072 f16 positions,
// 8 heads of width 256 per KV head: 355 vs 160 us; width 128, 4 heads: 100 vs
// 93 us; width 64, one head: 75 vs 60 us). q and the weights in two f16 or
// three bf16 parts (22 or 24 bits) keep the scores within f32 rounding.
bool decode_on_query_tiles(const sk_desc_t& d) {
  if (!query_tile_supported(d) || d.num_kv_heads < 1) return false;
  const int G = d.num_q_heads / d.num_kv_heads;
  switch (d.head_dim_qk) {
    case 64: return true;
    case 128: return G >= 4;
    default: return G >= 6;
  }
}

template <typename KT, int D, int DS, bool FUSED>
static void qt_go(bool launch, const void** fn, dim3 grid, hipStream_t stream, const QtArgs& a) {
  auto kern = query_tile_kernel<KT, D, DS, FUSED>;
  if (fn) *fn = reinterpret_cast<const void*>(kern);
  if (launch) hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, a);
}

// The one-launch kernel exists for one query per sequence, whose group of at
// most 8 rows takes 4 ways at width 128 and 256 and 2 at width 64.
template <typename KT, int D>
static sk_status_t qt_launch(int ways, bool fused, bool launch, const void** fn, dim3 grid,
                             hipStream_t stream, const QtArgs& a) {
  if (fused) {
    if (a.Q != 1 || a.G > 8 || ways != (D >= 128 ? 4 : 2)) return SK_ERR_UNSUPPORTED;
    if constexpr (D >= 128)
      qt_go<KT, D, 4, true>(launch, fn, grid, stream, a);
    else
      qt_go<KT, D, 2, true>(launch, fn, grid, stream, a);
  } else if (ways == 4) {
    if constexpr (D >= 128) qt_go<KT, D, 4, false>(launch, fn, grid, stream, a);
  } else if (ways == 2) {
    qt_go<KT, D, 2, false>(launch, fn, grid, stream, a);
  } else {
    qt_go<KT, D, 1, false>(launch, fn, grid, stream, a);
  }
  return SK_OK;
}

template <typename KT>
static sk_status_t qt_by_dim(const QueryTileLaunch& s, const QtArgs& a, dim3 grid, bool launch,
                             const void** fn) {
  const int D = s.d->head_dim_qk;
  const int ways = query_tile_ways(a.Q * a.G, D);
  switch (D) {
    case 64: return qt_launch<KT, 64>(ways, s.fused, launch, fn, grid, s.stream, a);
    case 128: return qt_launch<KT, 128>(ways, s.fused, launch, fn, grid, s.stream, a);
    case 256: return qt_launch<KT, 256>(ways, s.fused, launch, fn, grid, s.stream, a);
    default: return SK_ERR_UNSUPPORTED;
  }
}

sk_status_t query_tile_launch(const QueryTileLaunch& s, bool launch, const void** fn, int grid3[3],
                              int* block) {
  const sk_desc_t& d = *s.d;
  if (!query_tile_supported(d)) return SK_ERR_UNSUPPORTED;
  QtArgs a;
  a.q = s.q;
  a.k = s.k;
  a.v = s.v;
  a.seq_lens = s.seq_lens;
  a.ws_acc = s.ws_acc;
  a.ws_m = s.ws_m;
  a.ws_l = s.ws_l;
  a.stride_seq = d.stride_seq;
  a.stride_pos = d.stride_pos;
  a.stride_head = d.stride_head;
  a.q_dtype = d.q_dtype;
  a.Q = s.q_len;
  a.Hq = d.num_q_heads;
  a.G = d.num_q_heads / d.num_kv_heads;
  a.S = s.p->n_splits;
  a.chunk = s.p->chunk;
  a.cap = d.max_seq_len;
  a.nqt = query_tile_rows_tiles(d, s.q_len);
  a.qscale = d.scale * kLog2e;
  a.counters = s.counters;
  a.out = s.out;
  a.lse = s.lse;
  const dim3 grid(d.num_kv_heads * a.nqt, s.p->n_splits, d.batch);
  if (grid3) {
    grid3[0] = grid.x;
    grid3[1] = grid.y;
    grid3[2] = grid.z;
  }
  if (block) *block = 256;
  if (d.kv_dtype == SK_F16) return qt_by_dim<_Float16>(s, a, grid, launch, fn);
  return qt_by_dim<bf16_t>(s, a, grid, launch, fn);
}

}  // namespace sk
