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
// with the online-softmax update between them. f16 caches use f16 MFMA (q and
// the probabilities rounded to f16, f32 accumulation); f32 caches use f16 MFMA
// on two f16 parts of every operand (22 significant bits, three part products
// per product, f32 accumulation). Three kernels live here, each described at
// its definition:
//   * mla16_split_kernel (f16 caches): two waves per 16-head block, x32 MFMA,
//     scores transposed, one barrier per tile; 32, 64 and 96 heads in one
//     workgroup per split, 128 heads as two workgroups of 64;
//   * mla16d_split_kernel (f16 caches, 64 and 96 heads when every compute
//     unit gets a split): eight waves in two roles, scoring waves of 32 heads
//     (scores and softmax in registers) and output waves that own the value
//     columns and multiply every block's weights by them;
//   * mla32_split_kernel (f32 caches): four waves per 16-head block, tiles
//     turned into f16 parts in LDS as they land, scores transposed so P stays
//     in registers, heads over one or more workgroups per split.
// Each has a FUSED instantiation for the one-launch decode: the partials go
// out with device-scope stores and the workgroups merge them in the same
// grid (latent_fused_tail).
#include "sk_device.h"
#include "sk_internal.h"
#include "sk_merge.h"

namespace sk {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kLatDk = 576;
constexpr int kLatDv = 512;

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
  // Index-list layout: position j of sequence b is pool row
  // table[b * max_idx + j]; rows outside [0, num_rows) are never read.
  const int32_t* table;
  int32_t max_idx;
  int64_t num_rows;
  int32_t nt;  // 1: this workgroup is its rows' only reader (non-temporal tile loads)
  // One-launch decode (the FUSED kernels): partials go out with device-scope
  // stores, then every workgroup meets at a grid barrier (arrival and
  // departure counts in counters[0] and [1]) and merges a share of the
  // (sequence, head) rows into out and lse.
  uint32_t* counters;
  float* out;
  float* lse;
};

// A partial value: a device-scope store where workgroups on other XCDs read it
// back after the grid barrier (the one-launch decode with more than one
// split), a plain store otherwise.
__device__ __forceinline__ void put_partial(float* p, float v, bool dev) {
  if (dev)
    st_dev(p, v);
  else
    *p = v;
}

// The one-launch tail of every latent split kernel; heads [h0, h0 + H) of
// sequence blockIdx.y are this workgroup's. With one split a workgroup's own
// partial is all its heads have: it merges them itself, with no grid barrier
// (its plain stores have completed after the wait and the workgroup barrier). Otherwise every
// workgroup meets the others at the grid barrier and merges a share of all
// rows (s_lds: the kernel's tile buffers, free once the barrier has passed).
template <int NT>
__device__ __forceinline__ void latent_fused_tail(const MlaArgs& a, float* s_lds, int h0, int H) {
  if (a.S == 1) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int t = ((int)blockIdx.y * a.Hq + h0) * 2;
    // Inlined here: a call would put the kernel's arguments in scratch
    // memory for the whole kernel.
    [[clang::always_inline]] latent_merge_by_wave<1, 0>(a, t, t + 2 * H,
                                                        __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), NT / 64);
    return;
  }
  const uint32_t n = gridDim.x * gridDim.y * gridDim.z;
  grid_arrive_and_wait(a.counters, n);
  latent_grid_merge<NT>(a, (int)gridDim.y, s_lds);
  grid_depart(a.counters, a.counters + 1, n);
}
// Index-list tiles (IDX kernels): lane r < T of every wave holds the pool row
// of tile row r (positions past the split's end repeat the last one), loaded
// one tile ahead of the tile's own loads. A row outside the pool is replaced
// by row 0 for the load and its bit in the tile's mask makes its scores NaN.
__device__ __forceinline__ int32_t load_tile_index(const MlaArgs& a, int b, int64_t tb,
                                                   int64_t end, int T) {
  const int lane = threadIdx.x & 63;
  if (lane >= T) return 0;
  const int64_t pos = (tb + lane < end) ? tb + lane : end - 1;
  return a.table[(int64_t)b * a.max_idx + pos];
}
__device__ __forceinline__ bool index_bad(const MlaArgs& a, int32_t r) {
  return r < 0 || (int64_t)r >= a.num_rows;
}
// The tile mask of bad rows (bit r: tile row r) and the row each lane reads
// for tile row `row` (taken from lane `row`).
__device__ __forceinline__ uint32_t tile_bad_mask(const MlaArgs& a, int32_t idx, int T) {
  const int lane = threadIdx.x & 63;
  return (uint32_t)__ballot(lane < T && index_bad(a, idx));
}
__device__ __forceinline__ int32_t row_of(const MlaArgs& a, int32_t idx, int row) {
  const int32_t safe = index_bad(a, idx) ? 0 : idx;
  return __builtin_amdgcn_ds_bpermute(row << 2, safe);
}

// ---------------------------------------------------------------------------
// How the latent kernels stage tiles (the direct-to-LDS load, its explicit
// wait and the raw barrier live in sk_device.h) and read them:
//  * global_load_lds_dwordx4 puts each lane's 16 bytes at M0 + 16*lane, so a
//    tile goes straight from HBM into LDS with no registers holding staged
//    data; rows are stored unpadded with their 16-byte chunk index XOR-ed by
//    the row, and a lane chooses which global chunk to fetch so that its fixed
//    LDS slot holds the swizzled layout.
//  * ds_read_b64_tr_b16: within a 16-lane group, lane i's item t is element
//    i%4 of the 8-byte chunk addressed by lane 4t + i/4.
//  * Each wave waits for its own tile loads with an explicit vmcnt before the
//    barrier that publishes them (a workgroup fence would wait for every load
//    in flight).
// ---------------------------------------------------------------------------
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __attribute__((address_space(3))) _Float16 lds_half_t;

__device__ __forceinline__ uint32_t lds_addr_of(const _Float16* p) {
  return (uint32_t)(size_t)(const lds_half_t*)(p);
}

__device__ __forceinline__ float4_t mfma32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half4_t lds_read_tr(const _Float16* p) {
  // p points into LDS; the C-style cast is the generic-to-LDS address-space cast.
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(p));
  return __builtin_bit_cast(half4_t, v);
}


constexpr int kT16 = 32;     // positions per tile
constexpr int kCpr16 = kLatDk / 8;   // 72 chunks of 16 bytes per cache row

// LDS offset (halves) of logical chunk cc of tile row r.
__device__ __forceinline__ int tile_off(int r, int cc) { return r * kLatDk + ((cc ^ (r & 7)) << 3); }

// ---------------------------------------------------------------------------
// f16 caches: two waves per 16-head block (workgroup of 2*NHB waves, wave
// w = 2*hb + dh), tiles of 32 rows staged by direct global-to-LDS loads three
// deep (chunks XOR-swizzled by row & 7), scores computed transposed, one
// barrier per tile.
//  * Wave (hb, dh) computes partial scores of its 16 heads over latent columns
//    [288*dh, 288*dh + 288) with v_mfma_f32_16x16x32_f16, its query rows held
//    in registers as B operands; the two waves of a block add each other's
//    partials through LDS, so both hold the block's full scores and run the
//    online softmax in registers. The same wave owns value columns
//    [256*dh, 256*dh + 256).
//  * Scores S^T[position][head] = C . Q^T: the cache tile is the A operand and
//    the query rows the B operand of v_mfma_f32_16x16x32_f16, so lane (head
//    l16, quarter lq) ends with positions 4*lq + i (first 16-position block)
//    and 16 + 4*lq + i (second). After the two partials of the block are
//    added and the softmax runs, those eight weights, in that order, are the
//    lane's A operand for the output product over the tile's 32 positions; the
//    value operands are read in the same position order (two transpose reads
//    of four rows each). P stays in registers.
//  * Software pipeline: iteration i computes the output product of tile i-1
//    and the scores of tile i, then one barrier publishes the partial scores
//    (double-buffered by parity) and the next tile; after it tile i+2 is
//    requested into the buffer tile i-1 used and the softmax of tile i runs.
//  * A tile is 36 wave-loads of 64 chunks; wave w issues loads
//    [w*base + min(w, extra), ...) of them, base + (w < extra) in all
//    (base = 36 / NW, extra = 36 % NW: 9, 4 + 1 for waves 0-3, or 3 per wave
//    for 4, 8 or 12 waves).
//  * Heads: one workgroup per split holds NHB blocks; a split's heads are
//    spread over gridDim.z workgroups of NHB*16 (two for 128 heads, whose
//    eight blocks would not fit the registers of 16 waves), each streaming
//    the split's rows.
// ---------------------------------------------------------------------------
// f16: 16-head blocks per workgroup and workgroups per split (128 heads: two
// workgroups of 64, whose 8 waves keep two waves per SIMD).
__host__ __device__ constexpr int mla16_blocks(int Hq) { return Hq == 128 ? 4 : Hq / 16; }
__host__ __device__ constexpr int mla16_groups(int Hq) { return Hq / (16 * mla16_blocks(Hq)); }
constexpr int64_t kHalveHeadsAt = 128;  // (split, sequence) pairs, half of MI355X's CUs

template <int NHB, bool IDX, bool FUSED>
__global__ __launch_bounds__(NHB * 128) void mla16_split_kernel(MlaArgs a) {
  constexpr int H = NHB * 16;
  constexpr int NW = 2 * NHB;
  constexpr int KH = kLatDk / 2;                  // 288 latent columns per wave
  constexpr int KS = KH / 32;                     // 9 MFMA steps
  constexpr int SLOTS = kT16 * kCpr16;            // 2304 chunks per tile
  constexpr int WLOADS = SLOTS / 64;              // 36 wave-loads per tile
  constexpr int LBASE = WLOADS / NW, LEXTRA = WLOADS % NW;
  constexpr int DPW = LBASE + (LEXTRA > 0 ? 1 : 0);  // most loads one wave issues per tile
  static_assert(SLOTS % 64 == 0, "a tile is whole wave-loads");
  constexpr int NCB = 16;                         // 16-column blocks per half (256 columns)
  constexpr int TILE = kT16 * kLatDk;             // halves per tile buffer

  __shared__ __align__(16) _Float16 s_c[3 * TILE];
  __shared__ __align__(16) float4_t s_sx[2][NW][2][64];

  const int split = blockIdx.x;
  const int b = blockIdx.y;
  const int h0 = blockIdx.z * H;  // first head of this workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hb = wave >> 1;
  const int dh = wave & 1;
  const int l16 = lane & 15;
  const int lq = lane >> 4;
  const int wl0 = wave * LBASE + min(wave, LEXTRA);       // this wave's first wave-load
  const int nwl = LBASE + (wave < LEXTRA ? 1 : 0);        // and their count

  const int L = min(a.seq_lens[b], a.cap);
  const int64_t start = (int64_t)split * a.chunk;
  const int64_t end = min((int64_t)L, start + a.chunk);
  const int64_t ws0 = ((int64_t)b * a.Hq + h0) * a.S + split;

  if (start >= end) {
    // One-launch decode: an empty slice takes no part in the merge, but its
    // workgroup still meets the others at the grid barrier and merges.
    if constexpr (FUSED) {
      latent_fused_tail<NW * 64>(a, reinterpret_cast<float*>(s_c), h0, H);
      return;
    }
    for (int idx = tid; idx < H * kLatDv; idx += NW * 64) {
      const int h = idx / kLatDv, e = idx - (idx / kLatDv) * kLatDv;
      a.ws_acc[(ws0 + (int64_t)h * a.S) * kLatDv + e] = 0.0f;
    }
    for (int h = tid; h < H; h += NW * 64) {
      a.ws_m[ws0 + (int64_t)h * a.S] = -INFINITY;
      a.ws_l[ws0 + (int64_t)h * a.S] = 0.0f;
    }
    return;
  }

  const _Float16* __restrict__ cbase =
      reinterpret_cast<const _Float16*>(a.c) + (IDX ? 0 : (int64_t)b * a.stride_seq);
  const float* __restrict__ qb = a.q + ((int64_t)b * a.Hq + h0) * kLatDk;

  // Tile staging: this wave's wave-loads per tile; slot s holds tile row s/72,
  // logical chunk (s%72) ^ (row & 7). Rows past the end re-read row end-1.
  // The slot coordinates are recomputed per tile (a few integer operations)
  // rather than held in registers across the loop.
  // The tile base (clamped to the last row) is wave-uniform; a lane's offset
  // is its row (clamped to the last row) times the row stride plus its chunk.
  const uint32_t lds0 = lds_addr_of(s_c);
  const uint32_t row_bytes = (uint32_t)(a.stride_pos * 2);
  // Index-list layout: the next tile's rows (lane r < 32) and the bad-row
  // masks of the tiles in the three buffers.
  int32_t nidx = 0;
  uint32_t bad0 = 0, bad1 = 0, bad2 = 0;
  auto issue_tile = [&](int bi, int64_t tb) {
    if constexpr (IDX) {
      const uint32_t bad = tile_bad_mask(a, nidx, kT16);
      bad0 = bi == 0 ? bad : bad0;
      bad1 = bi == 1 ? bad : bad1;
      bad2 = bi == 2 ? bad : bad2;
#pragma unroll
      for (int c = 0; c < DPW; ++c) {
        if (LEXTRA != 0 && c >= nwl) break;  // wave-uniform
        const int sl = (wl0 + c) * 64 + lane;
        const int srow = sl / kCpr16;
        const int scol = ((sl - srow * kCpr16) ^ (srow & 7)) * 8;
        const int32_t r = row_of(a, nidx, srow);
        const uint32_t dst = lds0 + (uint32_t)((bi * TILE + (wl0 + c) * 64 * 8) * 2);
        dma16(cbase + (int64_t)r * a.stride_pos + scol, __builtin_amdgcn_readfirstlane(dst), a.nt);
      }
      nidx = load_tile_index(a, b, tb + kT16, end, kT16);  // the next tile's rows
    } else {
      const int64_t tbc = tb < end ? tb : end - 1;
      const int last = (int)(end - 1 - tbc);  // >= 0
      const _Float16* tbase = cbase + tbc * a.stride_pos;
#pragma unroll
      for (int c = 0; c < DPW; ++c) {
        if (LEXTRA != 0 && c >= nwl) break;  // wave-uniform
        const int sl = (wl0 + c) * 64 + lane;
        const int srow = sl / kCpr16;
        const int scol = ((sl - srow * kCpr16) ^ (srow & 7)) * 8;
        const uint32_t off = (uint32_t)min(srow, last) * row_bytes + (uint32_t)(scol * 2);
        const uint32_t dst = lds0 + (uint32_t)((bi * TILE + (wl0 + c) * 64 * 8) * 2);
        dma16s(off, tbase, __builtin_amdgcn_readfirstlane(dst), a.nt);
      }
    }
  };

  // Running max (base 2) and normaliser of head hb*16 + l16 (replicated over
  // the quarters); output accumulators: heads 4*lq + e (items), columns
  // 256*dh + 16*cb + l16.
  float m = -INFINITY, l = 0.0f;
  float4_t acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = float4_t{0.f, 0.f, 0.f, 0.f};

  // Per-lane LDS offsets (halves) inside a tile buffer.
  //  * score reads, rows l16 (+16 for the second block), logical chunk
  //    36*dh + lq + 4*ks: sb[ks & 1] + 32*ks (+ 16 rows);
  //  * transpose reads, rows 4*lq + l16/4 (+16), logical chunk
  //    32*dh + 2*cb + (l16&3)/2: bv[cb & 3] + 64*(cb >> 2) (+ 16 rows), plus
  //    4 halves for odd l16.
  const int c0 = dh * 36 + lq;
  const int sw = l16 & 7;
  const int sb0 = l16 * kLatDk + ((c0 ^ sw) << 3);
  const int sb1 = l16 * kLatDk + (((c0 + 4) ^ sw) << 3) - 32;
  const int r0 = 4 * lq + (l16 >> 2);
  const int jv = (l16 & 3) >> 1;
  const int hoff = (l16 & 1) * 4;
  int bv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) bv[u] = r0 * kLatDk + ((dh * 32 + ((2 * u + jv) ^ (r0 & 7))) << 3) + hoff;
  constexpr int kRow16 = 16 * kLatDk;  // 16 rows further down (same swizzle)

  const int ntiles = (int)((end - start + kT16 - 1) / kT16);
  if constexpr (IDX) {
    nidx = load_tile_index(a, b, start, end, kT16);
    wait_vm_lgkm0<0>();
  }
  issue_tile(0, start);
  // Query rows of this head block as B operands: lane holds head hb*16 + l16,
  // columns 288*dh + 32*ks + 8*lq .. +7 (rounded to f16 once).
  half8_t qf[KS];
  if constexpr (NHB <= 4) {
    // Up to 64 heads: the rows are staged in f16 through tile buffers 1-2
    // (64 rows of 576 halves fill them) with whole-line loads by the whole
    // workgroup, then tile 1 is requested; iteration 0 waits for it only at
    // its end. A wave's own fragments (16 rows, 32 bytes apart in each)
    // would touch sixteen lines per load instruction.
    constexpr int QV = H * (kLatDk / 4) / (NW * 64);  // float4 per thread
    static_assert(H * (kLatDk / 4) % (NW * 64) == 0 && H * kLatDk <= 2 * TILE, "staged rows fit");
    _Float16* const sq = s_c + TILE;
    {
      float4 qv[QV];
#pragma unroll
      for (int k = 0; k < QV; ++k) qv[k] = *reinterpret_cast<const float4*>(qb + 4 * (tid + NW * 64 * k));
      // Row h keeps chunk c (8 halves) at chunk position c ^ (h & 7).
#pragma unroll
      for (int k = 0; k < QV; ++k) {
        const int f = tid + NW * 64 * k;
        const int h = f / (kLatDk / 4);
        const int c4 = f - h * (kLatDk / 4);
        *reinterpret_cast<half4_t*>(sq + h * kLatDk + (((c4 >> 1) ^ (h & 7)) << 3) + (c4 & 1) * 4) =
            half4_t{(_Float16)qv[k].x, (_Float16)qv[k].y, (_Float16)qv[k].z, (_Float16)qv[k].w};
      }
    }
    wait_vm_lgkm0<0>();  // tile 0 (and the next tile's rows of an index list)
    raw_barrier();
    const _Float16* qrow = sq + (hb * 16 + l16) * kLatDk;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = *reinterpret_cast<const half8_t*>(qrow + (((dh * 36 + 4 * ks + lq) ^ (l16 & 7)) << 3));
    wait_vm_lgkm0<0>();
    raw_barrier();  // the staged rows are read before tile 1 overwrites them
    issue_tile(1, start + kT16);
  } else {
    if constexpr (IDX) wait_vm_lgkm0<0>();  // the second tile's rows
    issue_tile(1, start + kT16);
    // (requested after the first tiles, so their latency overlaps)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        qf[ks][e] = (_Float16)qb[(hb * 16 + l16) * kLatDk + dh * KH + ks * 32 + lq * 8 + e];
    wait_vm_lgkm0<0>();  // both tiles and the query rows landed
    raw_barrier();
  }

  half8_t pp = half8_t{};  // weights of the previous tile (A operand)
  float alp = 1.0f;        // its rescale factor, head hb*16 + l16
  bool movedp = false;
  for (int i = 0;; ++i) {
    // ---- output of tile i-1: acc = alp * acc + P x V ----
    if (i > 0) {
      const _Float16* prv = s_c + ((i - 1) % 3) * TILE;
      if (__any(movedp)) {
        // Accumulator item e is head 4*lq + e, whose factor lane 4*lq + e holds.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ae = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * lq + e) << 2, __float_as_int(alp)));
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) acc[cb][e] *= ae;
        }
      }
      auto vread = [&](int cb) {
        const _Float16* vp = prv + bv[cb & 3] + 64 * (cb >> 2);
        const half4_t v0 = lds_read_tr(vp);
        const half4_t v1 = lds_read_tr(vp + kRow16);
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      half8_t vn = vread(0);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const half8_t vb = vn;
        if (cb + 1 < NCB) vn = vread(cb + 1);
        acc[cb] = mfma32(pp, vb, acc[cb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (i == ntiles) break;
    const int64_t tb = start + (int64_t)i * kT16;
    const int rel = (int)(end - tb);  // positions of this tile before the end (> 0)
    const _Float16* cur = s_c + (i % 3) * TILE;

    // ---- partial scores S^T over this wave's 288 columns, both blocks ----
    float4_t sp0 = float4_t{0.f, 0.f, 0.f, 0.f}, sp1 = sp0;
    const _Float16* sbp0 = cur + sb0;
    const _Float16* sbp1 = cur + sb1;
    auto bread = [&](int ks, int rows) {
      const _Float16* bp = (ks & 1) ? sbp1 : sbp0;
      return *reinterpret_cast<const half8_t*>(bp + rows + 32 * ks);
    };
    half8_t n0 = bread(0, 0), n1 = bread(0, kRow16);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const half8_t b0 = n0, b1 = n1;
      if (ks + 1 < KS) {
        n0 = bread(ks + 1, 0);
        n1 = bread(ks + 1, kRow16);
      }
      sp0 = mfma32(b0, qf[ks], sp0);
      sp1 = mfma32(b1, qf[ks], sp1);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int par = i & 1;
    s_sx[par][wave][0][lane] = sp0;
    s_sx[par][wave][1][lane] = sp1;
    // Tile i+1 (requested one iteration ago, or in the prologue) is the only
    // tile load still in flight: wait for it, then publish it and the partials.
    wait_vm_lgkm0<0>();
    raw_barrier();
    // Every wave has finished the output product of tile i-1: its buffer takes
    // tile i+2 now, so the load overlaps the softmax as well.
    issue_tile((i + 2) % 3, tb + 2 * kT16);

    // ---- full scores (own + partner), online softmax over the 32 positions ----
    const float4_t q0 = s_sx[par][wave ^ 1][0][lane];
    const float4_t q1 = s_sx[par][wave ^ 1][1][lane];
    float v[8];
    float mx = -INFINITY;
    uint32_t badt = 0;  // rows of this tile whose index lies outside the pool
    if constexpr (IDX) badt = (i % 3 == 0) ? bad0 : ((i % 3 == 1) ? bad1 : bad2);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = 4 * lq + e < rel ? (sp0[e] + q0[e]) * a.qscale : -INFINITY;
      v[4 + e] = 16 + 4 * lq + e < rel ? (sp1[e] + q1[e]) * a.qscale : -INFINITY;
      if constexpr (IDX) {
        v[e] = ((badt >> (4 * lq + e)) & 1) ? __builtin_nanf("") : v[e];
        v[4 + e] = ((badt >> (16 + 4 * lq + e)) & 1) ? __builtin_nanf("") : v[4 + e];
      }
      mx = fmaxf(mx, fmaxf(v[e], v[4 + e]));
    }
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx));
    const float mn = fmaxf(m, mx);
    const float mu = (mn == -INFINITY) ? 0.0f : mn;
    alp = fast_exp2(m - mu);
    movedp = alp != 1.0f;
    float ls = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const _Float16 pj = (_Float16)fast_exp2(v[j] - mu);
      pp[j] = pj;
      ls += (float)pj;
    }
    ls += xor16(ls);
    ls += xor32(ls);
    l = fmaf(l, alp, ls);
    m = mn;
  }
  // Drain the tile loads still in flight before the workgroup can retire.
  wait_vm_lgkm0<0>();

  // Partials: both waves of a block hold the same m and l.
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int head = hb * 16 + lq * 4 + e;
      const int col = dh * 256 + cb * 16 + l16;
      put_partial(a.ws_acc + (ws0 + (int64_t)head * a.S) * kLatDv + col, acc[cb][e], FUSED && a.S > 1);
    }
  if (dh == 0 && lq == 0) {
    put_partial(a.ws_m + ws0 + (int64_t)(hb * 16 + l16) * a.S, m * kLn2, FUSED && a.S > 1);
    put_partial(a.ws_l + ws0 + (int64_t)(hb * 16 + l16) * a.S, l, FUSED && a.S > 1);
  }
  if constexpr (FUSED) latent_fused_tail<NW * 64>(a, reinterpret_cast<float*>(s_c), h0, H);
}

// How far (base 2) a tile's maximum may exceed the running value the weights
// are taken against before that value moves (weights stay below 2^8).
constexpr float kLazyMax = 8.0f;

// ---------------------------------------------------------------------------
// f32 caches: f16 MFMA on f16 parts, four waves per 16-head block, heads of a
// split spread over HG workgroups.
//
// Every f32 operand x (cache entries, q * scale * log2 e, the weights P) is
// taken as two f16 parts, hi = round(x) and lo = round((x - hi) * 2^11), which
// hold x within 2^-22 |x| + 2^-36, and a product of two split operands as
// a_hi b_hi + 2^-11 (a_hi b_lo + a_lo b_hi) (the dropped a_lo b_lo is below
// 2^-22 of it). Per flop, v_mfma_f32_16x16x32_f16 issues 16 times as fast
// as v_mfma_f32_16x16x4_f32 (and the x16 form at least 8 times), so three
// part products still cost well under one f32 product. f16's range ends at
// 65,504: an operand of magnitude 65,520 or more makes the scores or outputs
// it enters NaN (f16_parts).
//
// The query parts of 16 heads x 576 columns and the 16 x 512 output
// accumulators do not fit one wave's share of the register file at three waves
// per SIMD, so each 16-head block has four waves: wave (hb, dq) computes the
// partial scores over latent columns [144*dq, 144*dq + 144) and owns value
// columns [128*dq, 128*dq + 128). A workgroup holds NHBB blocks (12 waves for
// NHBB = 3) and a split's heads are spread over HG = Hq / (16*NHBB)
// workgroups on one XCD, each streaming the split's cache rows (the L2 serves
// the second reader).
//  * Tiles of 16 cache rows go straight from HBM into LDS with
//    global_load_lds_dwordx4, three tiles deep; each row's 144 chunks of 16
//    bytes are stored with the chunk index XOR-ed by the row (0..15). Once its
//    own loads have landed, each wave rewrites its slots in place as parts:
//    the 16 bytes of four f32 values become four hi halves and four lo halves.
//  * Scores are computed transposed, S^T[position][head] = C[position][:] .
//    Q^T, with v_mfma_f32_16x16x32_f16 (chunks t and t+1 of the lane: columns
//    4*(36*dq + lq + 4t) .. +3 and the next chunk's; the ninth chunk's
//    products as one x16 and one x32 over (column, part) pairs), so the
//    result leaves lane (head l16, quarter lq) holding the scores of
//    positions 4*lq + i: after the four partials of the block are added
//    (through LDS, in a fixed order, so all four waves hold identical values)
//    and the softmax runs in registers, those four weights are exactly the
//    lane's A operand of the output products over the tile's 16 positions
//    (an x32 over (position, part) pairs and an x16); the value parts come
//    through the gfx950 transpose read ds_read_b64_tr_b16. P never goes
//    through LDS.
//  * One barrier per tile (below).
// ---------------------------------------------------------------------------
constexpr int kT32 = 16;              // positions per tile
constexpr int kCpr32 = kLatDk / 4;    // 144 chunks of 16 bytes per f32 cache row
constexpr int kSlots32 = kT32 * kCpr32;

// Dedicated-role f16 latent kernel (64 or 96 heads of a split in one
// workgroup of eight waves). NS = NHB/2 scoring waves own 32 heads each (two
// 16-head blocks): every K fragment read from LDS feeds both blocks, so the
// scores take the tile out of LDS NS times rather than NHB times. A scoring
// wave runs its two blocks' online softmax in registers and publishes P (f16)
// and the rescale factors. The other 8 - NS output waves own the 32 16-column
// value blocks (Mla16dRoles shares them out so every SIMD carries about the
// same MFMA work; wave w runs on SIMD w % 4), multiply the P of all blocks by
// them and request the tiles. One barrier per tile and four tile buffers:
// iteration i scores tile i, runs the output product of tile i-1 and requests
// tile i+2 (two tiles of look-ahead).
template <int NHB>
struct Mla16dRoles {
  static constexpr int NS = NHB / 2;               // scoring waves
  static constexpr int NO = 8 - NS;                // output waves
  static constexpr int kShared = NHB == 6 ? 6 : 4; // column blocks of an output wave beside a scoring wave
  static constexpr int kAlone = NHB == 6 ? 7 : 6;  // ... of one on a SIMD without a scoring wave
  static constexpr bool shared(int w) { return w >= 4 && (w & 3) < NS; }
  static constexpr int ncb(int w) { return w < NS ? 0 : (shared(w) ? kShared : kAlone); }
  static constexpr int cb0(int w) {
    int s = 0;
    for (int v = NS; v < w; ++v) s += ncb(v);
    return s;
  }
  static constexpr int kLoads = kT16 * kCpr16 / 64;  // 36 wave-loads per tile
  static constexpr int LB = kLoads / NO, LX = kLoads % NO;
  static constexpr int DPW = LB + (LX > 0 ? 1 : 0);
};

struct Mla16dShared {
  _Float16* c;          // NBUF tile buffers
  half8_t* p;           // [2][NHB][64]: P of a tile (f16), A-operand lane order
  float* alpha;         // [2][NHB][16]: rescale factors of a tile
  int* moved;           // [2]: last tile whose factors were not all 1
};

// One role of the dedicated-role kernel: NCB == 0 scores, else the output
// product over NCB column blocks. Every role passes the same barriers.
template <int NHB, int NCB, bool FUSED>
__device__ __forceinline__ void mla16d_role(const MlaArgs& a, const Mla16dShared& sh, int64_t start, int64_t end,
                                            int64_t ws0, int b) {
  using R = Mla16dRoles<NHB>;
  constexpr int H = 16 * NHB;
  constexpr int NW = 8;
  constexpr int KS = kLatDk / 32;  // 18 x32 score steps
  constexpr int NBUF = 4;
  constexpr int TILE = kT16 * kLatDk;
  constexpr int kRow16 = 16 * kLatDk;
  constexpr bool SCORER = NCB == 0;
  static_assert(R::cb0(8) == kLatDv / 16, "the output waves cover the value columns");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int lq = lane >> 4;
  _Float16* const s_c = sh.c;

  const _Float16* __restrict__ cbase = reinterpret_cast<const _Float16*>(a.c) + (int64_t)b * a.stride_seq;
  const float* __restrict__ qb = a.q + (int64_t)b * a.Hq * kLatDk;

  // Tile staging as in the other f16 kernels: slot s of a tile holds row
  // s/72, logical chunk (s%72) ^ (row & 7); rows past the end re-read row
  // end-1. The 36 wave-loads of a tile are the output waves' (the workgroup
  // is its rows' only reader: non-temporal loads).
  const int ow = wave - R::NS;  // output wave index (negative for a scoring wave)
  const int wl0 = SCORER ? 0 : ow * R::LB + min(ow, R::LX);
  const int nwl = SCORER ? 0 : R::LB + (ow < R::LX ? 1 : 0);
  const uint32_t lds0 = lds_addr_of(s_c);
  const uint32_t row_bytes = (uint32_t)(a.stride_pos * 2);
  struct TileAt {
    const _Float16* base;
    int last;  // rows past base before the end (>= 0)
  };
  auto tile_at = [&](int64_t tb) {
    const int64_t tbc = tb < end ? tb : end - 1;
    return TileAt{cbase + tbc * a.stride_pos, (int)(end - 1 - tbc)};
  };
  auto issue_tile = [&](int bi, int64_t tb) {
    if constexpr (!SCORER) {
      const TileAt t = tile_at(tb);
      // The base is wave-uniform; say so, for the scalar operand of the load.
      const uint64_t bu = reinterpret_cast<uint64_t>(t.base);
      const void* base = reinterpret_cast<const void*>(
          ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(bu >> 32)) << 32) |
          (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bu));
#pragma unroll
      for (int cc = 0; cc < R::DPW; ++cc) {
        if (R::LX != 0 && cc >= nwl) continue;
        const int sl = (wl0 + cc) * 64 + lane;
        const int srow = sl / kCpr16;
        const int scol = ((sl - srow * kCpr16) ^ (srow & 7)) * 8;
        const uint32_t off = (uint32_t)min(srow, t.last) * row_bytes + (uint32_t)(scol * 2);
        const uint32_t dst = lds0 + (uint32_t)((bi * TILE + (wl0 + cc) * 64 * 8) * 2);
        dma16s(off, base, __builtin_amdgcn_readfirstlane(dst), true);
      }
    }
  };
  // Everything of this wave but its loads of the newest tile has landed.
  auto wait_but_newest = [&]() {
    if constexpr (SCORER) {
      wait_vm_lgkm0<0>();
    } else if constexpr (R::LX == 0) {
      wait_vm_lgkm0<R::DPW>();
    } else {
      if (nwl == R::DPW)
        wait_vm_lgkm0<R::DPW>();
      else
        wait_vm_lgkm0<R::DPW - 1>();
    }
  };

  const int ntiles = (int)((end - start + kT16 - 1) / kT16);
  if (tid < 2) sh.moved[tid] = -1;
  // Prologue: tile 0; the query rows, rounded to f16 once and staged through
  // the last NHB/2 tile buffers (H rows of 576 halves fill them exactly) with
  // whole-line loads by the whole workgroup; tile 1 (before the staging when
  // its buffer is not among them, else after).
  constexpr int QB0 = NBUF - NHB / 2;
  constexpr int QV = H * (kLatDk / 4) / (NW * 64);  // float4 per thread
  static_assert(H * (kLatDk / 4) % (NW * 64) == 0, "whole float4 rounds");
  static_assert(H * kLatDk <= (NBUF - QB0) * TILE, "the staged rows fit");
  _Float16* const sq = s_c + QB0 * TILE;
  issue_tile(0, start);
  {
    float4 qv[QV];
#pragma unroll
    for (int k = 0; k < QV; ++k) qv[k] = *reinterpret_cast<const float4*>(qb + 4 * (tid + NW * 64 * k));
    if constexpr (QB0 >= 2) issue_tile(1, start + kT16);
    // Row h keeps chunk c (8 halves) at chunk position c ^ (h & 7), so the 16
    // rows a fragment read touches fall in distinct banks.
#pragma unroll
    for (int k = 0; k < QV; ++k) {
      const int f = tid + NW * 64 * k;
      const int h = f / (kLatDk / 4);
      const int c4 = f - h * (kLatDk / 4);
      *reinterpret_cast<half4_t*>(sq + h * kLatDk + (((c4 >> 1) ^ (h & 7)) << 3) + (c4 & 1) * 4) =
          half4_t{(_Float16)qv[k].x, (_Float16)qv[k].y, (_Float16)qv[k].z, (_Float16)qv[k].w};
    }
  }
  if constexpr (QB0 >= 2)
    wait_but_newest();
  else
    wait_vm_lgkm0<0>();
  raw_barrier();
  // A scoring wave's heads 32w + 16hb + l16, columns 32t + 8lq .. +7.
  half8_t qf[SCORER ? 2 : 1][SCORER ? KS : 1];
  if constexpr (SCORER) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const _Float16* qrow = sq + (32 * wave + 16 * hb + l16) * kLatDk;
#pragma unroll
      for (int t = 0; t < KS; ++t)
        qf[hb][t] = *reinterpret_cast<const half8_t*>(qrow + (((4 * t + lq) ^ (l16 & 7)) << 3));
    }
  }
  // The staged rows are read before any tile load may overwrite them; tile 0
  // (and the query) landed, at most this wave's loads of tile 1 remain.
  if constexpr (QB0 >= 2) {
    wait_but_newest();
    raw_barrier();
  } else {
    wait_vm_lgkm0<0>();
    raw_barrier();
    issue_tile(1, start + kT16);
  }

  if constexpr (SCORER) {
    // Score fragments of step t (logical chunk 4t + lq of rows l16 and
    // l16 + 16): the XOR touches bits 0-2 only, so even and odd steps have one
    // base each.
    const int sb0 = l16 * kLatDk + ((lq ^ (l16 & 7)) << 3);
    const int sb1 = l16 * kLatDk + (((4 + lq) ^ (l16 & 7)) << 3);
    auto soff = [&](int t) { return ((t & 1) ? sb1 : sb0) + 64 * (t >> 1); };
    float m[2] = {-INFINITY, -INFINITY}, ll[2] = {0.0f, 0.0f};  // heads 32w + 16hb + l16; ll this lane's share
    for (int i = 0; i < ntiles; ++i) {
      const int64_t tb = start + (int64_t)i * kT16;
      const _Float16* cur = s_c + (i % NBUF) * TILE;
      float4_t s[2][2];  // [block][rows 0-15, 16-31]
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) s[hb][0] = s[hb][1] = float4_t{0.f, 0.f, 0.f, 0.f};
      // Operands two steps ahead.
      half8_t k0[3], k1[3];
      k0[0] = *reinterpret_cast<const half8_t*>(cur + soff(0));
      k1[0] = *reinterpret_cast<const half8_t*>(cur + soff(0) + kRow16);
      k0[1] = *reinterpret_cast<const half8_t*>(cur + soff(1));
      k1[1] = *reinterpret_cast<const half8_t*>(cur + soff(1) + kRow16);
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        if (t + 2 < KS) {
          k0[(t + 2) % 3] = *reinterpret_cast<const half8_t*>(cur + soff(t + 2));
          k1[(t + 2) % 3] = *reinterpret_cast<const half8_t*>(cur + soff(t + 2) + kRow16);
        }
        const half8_t a0 = k0[t % 3], a1 = k1[t % 3];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          s[hb][0] = mfma32(a0, qf[hb][t], s[hb][0]);
          s[hb][1] = mfma32(a1, qf[hb][t], s[hb][1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const int rel = (int)(end - tb);  // positions of tile i before the end (> 0)
      const int par = i & 1;
      bool moved = false;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float v[8];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = 4 * lq + e < rel ? s[hb][0][e] * a.qscale : -INFINITY;
          v[4 + e] = 16 + 4 * lq + e < rel ? s[hb][1][e] * a.qscale : -INFINITY;
          mx = fmaxf(mx, fmaxf(v[e], v[4 + e]));
        }
        mx = max_xor32(max_xor16(mx));
        // m moves to the tile's maximum only when that exceeds it by more than
        // kLazyMax (base 2): the weights stay below 2^kLazyMax (f16 holds
        // them), and most tiles keep m, so nothing is rescaled.
        const float mn = mx > m[hb] + kLazyMax ? mx : m[hb];
        const float mu = (mn == -INFINITY) ? 0.0f : mn;
        const float al = fast_exp2(m[hb] - mu);
        half8_t pw;
        float ls = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const _Float16 pj = (_Float16)fast_exp2(v[j] - mu);
          pw[j] = pj;
          ls += (float)pj;
        }
        ll[hb] = fmaf(ll[hb], al, ls);
        m[hb] = mn;
        moved = moved || al != 1.0f;
        sh.p[(par * NHB + 2 * wave + hb) * 64 + lane] = pw;
        if (lq == 0) sh.alpha[(par * NHB + 2 * wave + hb) * 16 + l16] = al;
      }
      // Several scoring waves may report the same tile: an LDS atomic max
      // (the flag only ever rises to the newest tile index).
      if (__any(moved) && lane == 0) atomicMax(&sh.moved[par], i);
      wait_vm_lgkm0<0>();
      raw_barrier();  // P and factors of tile i; tile i+1
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float l = sum_xor32(sum_xor16(ll[hb]));
      if (lq == 0) {
        const int head = 32 * wave + 16 * hb + l16;
        put_partial(a.ws_m + ws0 + (int64_t)head * a.S, m[hb] * kLn2, FUSED && a.S > 1);
        put_partial(a.ws_l + ws0 + (int64_t)head * a.S, l, FUSED && a.S > 1);
      }
    }
  } else {
    const int cb0 = R::cb0(wave);
    // Value fragments (transpose reads): rows 4*lq + l16/4 (+16), logical
    // chunk 2c + (l16&3)/2 of column block c, plus 4 halves for odd l16 (the
    // position order of P's layout).
    const int r0 = 4 * lq + (l16 >> 2);
    const int jv = (l16 & 3) >> 1;
    const int hoff = (l16 & 1) * 4;
    auto voff = [&](int u) { return r0 * kLatDk + (((2 * (cb0 + u) + jv) ^ (r0 & 7)) << 3) + hoff; };
    float4_t acc[NHB][NCB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[hb][cb] = float4_t{0.f, 0.f, 0.f, 0.f};
    auto output = [&](int j) {
      const _Float16* prv = s_c + (j % NBUF) * TILE;
      const int par = j & 1;
      if (sh.moved[par] == j) {
        // Accumulator items are heads 4*lq + e of each block.
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          const float4_t alp = *reinterpret_cast<const float4_t*>(&sh.alpha[(par * NHB + hb) * 16 + 4 * lq]);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[hb][cb][e] *= alp[e];
        }
      }
      half8_t pp[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) pp[hb] = sh.p[(par * NHB + hb) * 64 + lane];
      auto vread = [&](int u) {
        const _Float16* vp = prv + voff(u);
        const half4_t v0 = lds_read_tr(vp);
        const half4_t v1 = lds_read_tr(vp + kRow16);
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      half8_t vn = vread(0);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const half8_t vv = vn;
        if (cb + 1 < NCB) vn = vread(cb + 1);
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) acc[hb][cb] = mfma32(pp[hb], vv, acc[hb][cb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int i = 0;; ++i) {
      const bool more = i < ntiles;  // tile i exists (else only tile i-1's output remains)
      const int64_t tb = start + (int64_t)i * kT16;
      // Tile i+2 goes into the buffer of tile i-2, whose output product ran
      // before the last barrier; tiles past the end are not requested.
      const bool load_next = more && tb + 2 * kT16 < end;
      if (load_next) issue_tile((i + 2) % NBUF, tb + 2 * kT16);
      if (i > 0) output(i - 1);
      if (!more) break;
      // Tile i+1 (requested one iteration ago, or in the prologue) must have
      // landed; tile i+2's loads, if any, stay in flight.
      if (load_next)
        wait_but_newest();
      else
        wait_vm_lgkm0<0>();
      raw_barrier();
    }
    // Drain the tile loads still in flight before the workgroup can retire.
    wait_vm_lgkm0<0>();
    // Partials: heads 16hb + 4*lq + e, columns 16(cb0 + cb) + l16.
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int head = 16 * hb + 4 * lq + e;
          const int col = 16 * (cb0 + cb) + l16;
          put_partial(a.ws_acc + (ws0 + (int64_t)head * a.S) * kLatDv + col, acc[hb][cb][e], FUSED && a.S > 1);
        }
  }
}

template <int NHB, bool FUSED>
__global__ __launch_bounds__(512) void mla16d_split_kernel(MlaArgs a) {
  constexpr int H = 16 * NHB;
  constexpr int NBUF = 4;
  constexpr int TILE = kT16 * kLatDk;
  using R = Mla16dRoles<NHB>;
  static_assert(NHB == 4 || NHB == 6, "64 or 96 heads");
  __shared__ __align__(16) _Float16 s_c[NBUF * TILE];
  __shared__ __align__(16) half8_t s_p[2 * NHB * 64];
  __shared__ __align__(16) float s_alpha[2 * NHB * 16];
  __shared__ int s_moved[2];

  const int split = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int L = min(a.seq_lens[b], a.cap);
  const int64_t start = (int64_t)split * a.chunk;
  const int64_t end = min((int64_t)L, start + a.chunk);
  const int64_t ws0 = (int64_t)b * a.Hq * a.S + split;
  if (start >= end) {
    if constexpr (FUSED) {
      latent_fused_tail<512>(a, reinterpret_cast<float*>(s_c), 0, H);
      return;
    }
    for (int idx = tid; idx < H * kLatDv; idx += 512) {
      const int h = idx / kLatDv, e = idx - (idx / kLatDv) * kLatDv;
      a.ws_acc[(ws0 + (int64_t)h * a.S) * kLatDv + e] = 0.0f;
    }
    for (int h = tid; h < H; h += 512) {
      a.ws_m[ws0 + (int64_t)h * a.S] = -INFINITY;
      a.ws_l[ws0 + (int64_t)h * a.S] = 0.0f;
    }
    return;
  }
  const Mla16dShared sh{s_c, s_p, s_alpha, s_moved};
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave < R::NS)
    mla16d_role<NHB, 0, FUSED>(a, sh, start, end, ws0, b);
  else if (R::shared(wave))
    mla16d_role<NHB, R::kShared, FUSED>(a, sh, start, end, ws0, b);
  else
    mla16d_role<NHB, R::kAlone, FUSED>(a, sh, start, end, ws0, b);
  if constexpr (FUSED) latent_fused_tail<512>(a, reinterpret_cast<float*>(s_c), 0, H);
}

typedef __attribute__((address_space(3))) float lds_float_t;
__device__ __forceinline__ uint32_t lds_addr_of(const float* p) {
  return (uint32_t)(size_t)(const lds_float_t*)(p);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float4_t mfma16(half4_t a, half4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

typedef float float2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2_t;

// Lazy-maximum threshold (base 2) of the f32-cache kernel: its weights, at
// most 2^kLazyMax32, times 2^11 must stay finite in f16.
constexpr float kLazyMax32 = 4.0f;

// Four f32 values as two f16 parts, packed [hi0 hi1 hi2 hi3 | lo0 lo1 lo2 lo3]:
// hi = x rounded to f16, lo = (x - hi) * 2^11 rounded to f16. x - hi is exact
// and at most 2^-11 |x|, so hi + lo * 2^-11 equals x within 2^-22 |x| + 2^-36
// (the scaling keeps lo clear of f16's subnormals). The residual is one fused
// step from the packed hi (exact: (x - hi) 2^11 is an f32 value). Past f16's
// range (|x| >= 65,520) hi is an infinity and lo the opposite infinity (or
// NaN): every product x enters then sums an infinity with its negation, so
// the scores or outputs it touches come out NaN.
__device__ __forceinline__ u32x4_t f16_parts(float4_t x) {
#pragma clang fp contract(off)
  const half2_t h0 = __builtin_convertvector(float2_t{x[0], x[1]}, half2_t);
  const half2_t h1 = __builtin_convertvector(float2_t{x[2], x[3]}, half2_t);
  const float r0 = __builtin_fmaf((float)h0[0], -2048.0f, x[0] * 2048.0f);
  const float r1 = __builtin_fmaf((float)h0[1], -2048.0f, x[1] * 2048.0f);
  const float r2 = __builtin_fmaf((float)h1[0], -2048.0f, x[2] * 2048.0f);
  const float r3 = __builtin_fmaf((float)h1[1], -2048.0f, x[3] * 2048.0f);
  const half2_t l0 = __builtin_convertvector(float2_t{r0, r1}, half2_t);
  const half2_t l1 = __builtin_convertvector(float2_t{r2, r3}, half2_t);
  return u32x4_t{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1),
                 __builtin_bit_cast(uint32_t, l0), __builtin_bit_cast(uint32_t, l1)};
}

// LDS reads at a byte address (a wave-uniform buffer base plus a lane offset;
// the constant parts go into the instructions' offset fields).
__device__ __forceinline__ u32x4_t lds_ld16(uint32_t addr) { return *(const lds_u32x4_t*)(size_t)addr; }
// (volatile: two reads of one chunk must not be merged into one, whose
// registers would then have to be moved into the operands.)
__device__ __forceinline__ u32x2_t lds_ld8(uint32_t addr) { return *(volatile const lds_u32x2_t*)(size_t)addr; }
__device__ __forceinline__ half4_t lds_tr16(uint32_t addr) {
  return __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(size_t)addr));
}

// 16-head blocks per workgroup for an f32 latent with Hq heads, and the
// workgroups that share one split.
__host__ __device__ constexpr int mla32_blocks(int Hq) { return Hq % 48 == 0 ? 3 : 2; }
__host__ __device__ constexpr int mla32_groups(int Hq) { return Hq / (16 * mla32_blocks(Hq)); }

template <int NHBB, bool IDX, bool FUSED>
__global__ __launch_bounds__(NHBB * 256) void mla32_split_kernel(MlaArgs a) {
  constexpr int NW = 4 * NHBB;
  constexpr int NT = NW * 64;
  constexpr int HW = 16 * NHBB;                    // heads per workgroup
  constexpr int KT = kLatDk / 4 / 16;              // 9 chunks of 4 columns per lane over the wave's 144
  constexpr int DPW = (kSlots32 + NT - 1) / NT;    // tile loads per lane
  constexpr int TSTRIDE = DPW * NT * 4;            // floats per tile buffer (padded slots included)

  __shared__ __align__(16) float s_c[3 * TSTRIDE];
  __shared__ __align__(16) float4_t s_sx[2][NW][64];

  const int split = blockIdx.x;
  const int b = blockIdx.y;
  const int hg = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hb = wave >> 2;
  const int dq = wave & 3;
  const int l16 = lane & 15;
  const int lq = lane >> 4;
  const int head0 = hg * HW + hb * 16;

  const int L = min(a.seq_lens[b], a.cap);
  const int64_t start = (int64_t)split * a.chunk;
  const int64_t end = min((int64_t)L, start + a.chunk);
  const int64_t ws0 = (int64_t)b * a.Hq * a.S + split;

  if (start >= end) {
    if constexpr (FUSED) {
      latent_fused_tail<NT>(a, s_c, hg * HW, HW);
      return;
    }
    for (int idx = tid; idx < HW * kLatDv; idx += NT) {
      const int h = hg * HW + idx / kLatDv, e = idx - (idx / kLatDv) * kLatDv;
      a.ws_acc[(ws0 + (int64_t)h * a.S) * kLatDv + e] = 0.0f;
    }
    for (int h = tid; h < HW; h += NT) {
      a.ws_m[ws0 + (int64_t)(hg * HW + h) * a.S] = -INFINITY;
      a.ws_l[ws0 + (int64_t)(hg * HW + h) * a.S] = 0.0f;
    }
    return;
  }

  const float* __restrict__ cbase =
      reinterpret_cast<const float*>(a.c) + (IDX ? 0 : (int64_t)b * a.stride_seq);
  const float* __restrict__ qb = a.q + (int64_t)b * a.Hq * kLatDk;

  // Tile staging: slot s of a buffer holds tile row s/144, stored chunk s%144,
  // i.e. logical chunk (s%144) ^ row. Padding slots (s >= 2304, only when the
  // slots do not divide evenly over the waves) re-read the split's first row
  // into the buffer's tail, which nothing reads.
  int srow[DPW], scol[DPW];
#pragma unroll
  for (int c = 0; c < DPW; ++c) {
    const int sl = (wave * DPW + c) * 64 + lane;
    const bool real = sl < kSlots32;
    srow[c] = real ? sl / kCpr32 : -1;
    scol[c] = real ? ((sl - (sl / kCpr32) * kCpr32) ^ (sl / kCpr32)) * 4 : 0;
  }
  const uint32_t lds0 = lds_addr_of(s_c);
  const uint32_t row_bytes32 = (uint32_t)(a.stride_pos * 4);  // a tile spans 16 rows: offsets fit 32 bits
  // Index-list layout: the next tile's rows (lane r < 16) and the bad-row
  // masks of the tiles in the three buffers. Padding slots read tile row 0.
  int32_t nidx = 0;
  uint32_t bad0 = 0, bad1 = 0, bad2 = 0;
  auto issue_tile = [&](int bi, int64_t tb) {
    if constexpr (IDX) {
      const uint32_t bad = tile_bad_mask(a, nidx, kT32);
      bad0 = bi == 0 ? bad : bad0;
      bad1 = bi == 1 ? bad : bad1;
      bad2 = bi == 2 ? bad : bad2;
#pragma unroll
      for (int c = 0; c < DPW; ++c) {
        const int32_t r = row_of(a, nidx, srow[c] < 0 ? 0 : srow[c]);
        const uint32_t dst = lds0 + (uint32_t)((bi * TSTRIDE + (wave * DPW + c) * 64 * 4) * 4);
        dma16(cbase + (int64_t)r * a.stride_pos + scol[c], __builtin_amdgcn_readfirstlane(dst), a.nt);
      }
      nidx = load_tile_index(a, b, tb + kT32, end, kT32);  // the next tile's rows
    } else {
      // One wave-uniform base per tile (rows past the end re-read row end-1;
      // padding slots re-read the tile's first row) and 32-bit lane offsets.
      const int64_t tbc = tb < end ? tb : end - 1;
      const uint64_t bu = reinterpret_cast<uint64_t>(cbase + tbc * a.stride_pos);
      const void* tbase = reinterpret_cast<const void*>(
          ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(bu >> 32)) << 32) |
          (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bu));
      const int last = (int)(end - 1 - tbc);
#pragma unroll
      for (int c = 0; c < DPW; ++c) {
        const int row = srow[c] < 0 ? 0 : min(srow[c], last);
        const uint32_t off = (uint32_t)row * row_bytes32 + (uint32_t)(scol[c] * 4);
        const uint32_t dst = lds0 + (uint32_t)((bi * TSTRIDE + (wave * DPW + c) * 64 * 4) * 4);
        dma16s(off, tbase, __builtin_amdgcn_readfirstlane(dst), a.nt);
      }
    }
  };

  // Running max (base 2) of head head0 + l16, replicated over the four
  // quarters; ll is this lane's share of the normaliser (its positions of
  // every tile), summed over the quarters at the end. Accumulator acc[cb]
  // holds heads 4*lq + e (items) at column 128*dq + 16*cb + l16.
  float m = -INFINITY, ll = 0.0f;
  float4_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = float4_t{0.f, 0.f, 0.f, 0.f};

  // Per-lane LDS offsets (floats) inside a tile buffer. Score reads: row l16,
  // logical chunk 36*dq + lq + 4*t (t = 0..8), i.e. soff(t). Value reads
  // (transposed, 16 columns by 4 rows per 16 lanes): lane l16 = 4*rho + sg of
  // quarter lq gives row 4*lq + rho, columns 4*sg .. +3 of 16-column block cb
  // of the wave's 128, i.e. logical chunk 32*dq + 4*cb + sg, at
  // vb[cb & 3] + 64*(cb >> 2) (the row swizzle only touches the low four bits
  // of the chunk).
  int sb[4], vb[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    sb[v] = l16 * kLatDk + (((36 * dq + lq + 4 * v) ^ l16) << 2);
    const int r = 4 * lq + (l16 >> 2);
    vb[v] = r * kLatDk + ((32 * dq + ((4 * v + (l16 & 3)) ^ r)) << 2);
  }
  auto soff = [&](int t) { return sb[t & 3] + 64 * (t >> 2); };
  // Each wave turns the slots it loaded into f16 parts in place once they have
  // landed (16 bytes of f32 become 8 bytes of hi parts and 8 of lo parts), so
  // every read of the tile after the barrier that publishes it takes parts.
  // Rows of odd index keep the lo halves first: the 16 lanes of a read that
  // meet in one 16-byte chunk position then split evenly over its two
  // halves, which keeps the 8-byte operand reads free of bank conflicts.
  auto split_own = [&](int bi) {
#pragma unroll
    for (int c = 0; c < DPW; ++c) {
      u32x4_t* p = reinterpret_cast<u32x4_t*>(s_c + bi * TSTRIDE + ((wave * DPW + c) * 64 + lane) * 4);
      const u32x4_t v = f16_parts(__builtin_bit_cast(float4_t, *p));
      *p = (srow[c] & 1) ? u32x4_t{v.z, v.w, v.x, v.y} : v;
    }
  };

  const int ntiles = (int)((end - start + kT32 - 1) / kT32);
  if constexpr (IDX) {
    nidx = load_tile_index(a, b, start, end, kT32);
    wait_vm_lgkm0<0>();
  }
  issue_tile(0, start);
  if constexpr (IDX) wait_vm_lgkm0<0>();  // the second tile's rows
  issue_tile(1, start + kT32);
  // Query block as B operands (requested after the first tiles, so their
  // latency overlaps), pre-scaled into base-2 units and split into f16
  // parts: chunk t of this wave is columns 4*(36*dq + lq + 4*t) .. +3 of head
  // head0 + l16; step s of the x32 score products takes chunks 2s and 2s+1,
  // the last step chunk 8. The workgroup loads every block's rows as
  // consecutive float4s (whole lines per instruction; a wave's own
  // fragments, 16 rows 64 bytes apart, touch sixteen lines) and stages one
  // block at a time through tile buffer 2, which one block's 16 x 576 floats
  // fill; row h keeps float4 chunk c at position c ^ h, as the tiles do.
  half8_t qh[4], ql[4];
  half4_t qh8, ql8;
  {
    constexpr int QF = 16 * kLatDk / 4;      // float4 per block
    constexpr int QV = (QF + NT - 1) / NT;    // per thread and block (the last one partial)
    static_assert(16 * kLatDk <= TSTRIDE, "one block fits buffer 2");
    float4 qs[NHBB][QV];
    const float* qblk = qb + (int64_t)hg * HW * kLatDk;
#pragma unroll
    for (int r = 0; r < NHBB; ++r)
#pragma unroll
      for (int k = 0; k < QV; ++k)
        if (QF % NT == 0 || tid + NT * k < QF)
          qs[r][k] = *reinterpret_cast<const float4*>(qblk + (int64_t)r * 16 * kLatDk + 4 * (tid + NT * k));
    float* const sq = s_c + 2 * TSTRIDE;
#pragma unroll
    for (int r = 0; r < NHBB; ++r) {
      if (r > 0) {
        wait_vm_lgkm0<0>();
        raw_barrier();  // the previous block's fragments are read
      }
#pragma unroll
      for (int k = 0; k < QV; ++k) {
        const int f = tid + NT * k;
        if (QF % NT != 0 && f >= QF) continue;
        const int h = f / (kLatDk / 4);
        const int c = f - h * (kLatDk / 4);
        *reinterpret_cast<float4_t*>(sq + h * kLatDk + ((c ^ h) << 2)) =
            float4_t{qs[r][k].x * a.qscale, qs[r][k].y * a.qscale, qs[r][k].z * a.qscale, qs[r][k].w * a.qscale};
      }
      wait_vm_lgkm0<0>();
      raw_barrier();
      if (hb == r) {
        u32x4_t qc[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) qc[t] = f16_parts(*reinterpret_cast<const float4_t*>(sq + soff(t)));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          qh[u] = __builtin_bit_cast(half8_t, u32x4_t{qc[2 * u].x, qc[2 * u].y, qc[2 * u + 1].x, qc[2 * u + 1].y});
          ql[u] = __builtin_bit_cast(half8_t, u32x4_t{qc[2 * u].z, qc[2 * u].w, qc[2 * u + 1].z, qc[2 * u + 1].w});
        }
        qh8 = __builtin_bit_cast(half4_t, u32x2_t{qc[8].x, qc[8].y});
        ql8 = __builtin_bit_cast(half4_t, u32x2_t{qc[8].z, qc[8].w});
      }
    }
  }

  wait_vm_lgkm0<0>();  // both tiles and the query block landed
  split_own(0);
  split_own(1);
  wait_vm_lgkm0<0>();
  raw_barrier();

  // Partial scores S^T of the tile at LDS address `cur` over this wave's 144
  // columns: four x32 steps (chunks 2s, 2s+1) and a step for chunk 8, three
  // products each (C_hi q_hi into one accumulator; C_hi q_lo and C_lo q_hi,
  // whose lo parts carry 2^11, into another), each step's
  // operands read from LDS one step ahead. After steps 0-2, stage(s) of the
  // previous tile's softmax runs (a constant after unrolling), so the
  // softmax's VALU and cross-lane work issues while the matrix pipe works
  // through the products. Accumulators by step parity keep consecutive
  // products independent; they are summed at the end in a fixed order.
  auto scores = [&](uint32_t cur, auto&& stage) -> float4_t {
    const float4_t z = float4_t{0.f, 0.f, 0.f, 0.f};
    float4_t sp[2] = {z, z}, sa[2] = {z, z};
    // Lane addresses of chunks 0-3 in this buffer, made opaque so the other
    // chunks' reads add constants in the instructions' offset fields instead
    // of keeping an address register per read.
    // (Row l16's hi halves sit at byte 8 * (l16 & 1) of a chunk, lo at the
    // other: the lo address is the hi address with bit 3 flipped.)
    uint32_t ab[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ab[u] = cur + 4 * sb[u] + 8 * (l16 & 1);
      asm volatile("" : "+v"(ab[u]));
    }
    auto addr = [&](int t, int part) { return (ab[t & 3] ^ (8u * part)) + 256 * (t >> 2); };
    // hi (part 0) or lo (part 1) halves of chunks t and t+1, read straight
    // into the operand's register pairs.
    auto opnd = [&](int t, int part) {
      const u32x2_t x0 = lds_ld8(addr(t, part)), x1 = lds_ld8(addr(t + 1, part));
      return __builtin_bit_cast(half8_t, u32x4_t{x0.x, x0.y, x1.x, x1.y});
    };
    half8_t nh = opnd(0, 0), nl = opnd(0, 1);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const half8_t ah = nh, al = nl;
      if (st < 3) {
        nh = opnd(2 * st + 2, 0);
        nl = opnd(2 * st + 2, 1);
      }
      sa[st & 1] = mfma32(ah, ql[st], sa[st & 1]);
      sp[st & 1] = mfma32(ah, qh[st], sp[st & 1]);
      sa[st & 1] = mfma32(al, qh[st], sa[st & 1]);
      if (st < 3) stage(st);
      __builtin_amdgcn_sched_barrier(0);
    }
    const half4_t ah = __builtin_bit_cast(half4_t, lds_ld8(addr(8, 0)));
    const half4_t al = __builtin_bit_cast(half4_t, lds_ld8(addr(8, 1)));
    // The ninth chunk's two mixed products as one x32 product over
    // (column, part) pairs: [C_hi | C_lo] against [q_lo | q_hi].
    sp[0] = mfma16(ah, qh8, sp[0]);
    sa[0] = mfma32(__builtin_shufflevector(ah, al, 0, 1, 2, 3, 4, 5, 6, 7),
                   __builtin_shufflevector(ql8, qh8, 0, 1, 2, 3, 4, 5, 6, 7), sa[0]);
    const float4_t lo = sa[0] + sa[1];
    const float4_t hi = sp[0] + sp[1];
    float4_t r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = fmaf(lo[e], 1.0f / 2048.0f, hi[e]);
    return r;
  };

  // Software pipeline, one barrier per tile. Before iteration i the barrier
  // has published the partial scores of tile i (double-buffered by parity)
  // and tile i+1, and tile i+2 is in flight. Iteration i computes the partial
  // scores of tile i+1 with the softmax of tile i interleaved, then the output
  // product of tile i (acc = alpha * acc + P[16 heads][16 positions] x V);
  // after the next barrier tile i+3 goes into tile i's buffer.
  {
    const float4_t sp0 = scores(lds0, [](int) {});
    s_sx[0][wave][lane] = sp0;
    raw_barrier();
    if (start + 2 * kT32 < end) issue_tile(2, start + 2 * kT32);
  }
  for (int i = 0;; ++i) {
    const int par = i & 1;
    const bool next = i + 1 < ntiles;
    const int rel = (int)(end - (start + (int64_t)i * kT32));  // positions of tile i before the end (> 0)
    uint32_t badt = 0;  // rows of tile i whose index lies outside the pool
    if constexpr (IDX) badt = (i % 3 == 0) ? bad0 : ((i % 3 == 1) ? bad1 : bad2);

    // ---- softmax of tile i (the block's four partials summed in a fixed order) ----
    const float4_t x0 = s_sx[par][hb * 4 + 0][lane], x1 = s_sx[par][hb * 4 + 1][lane];
    const float4_t x2 = s_sx[par][hb * 4 + 2][lane], x3 = s_sx[par][hb * 4 + 3][lane];
    float pp[4], lmx = -INFINITY, mu = 0.0f, alp = 1.0f;
    bool moved = false;
    auto stage = [&](int t) {
      if (t == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pp[e] = 4 * lq + e < rel ? (x0[e] + x1[e]) + (x2[e] + x3[e]) : -INFINITY;
          if constexpr (IDX) pp[e] = ((badt >> (4 * lq + e)) & 1) ? __builtin_nanf("") : pp[e];
          lmx = fmaxf(lmx, pp[e]);
        }
      } else if (t == 1) {
        // m moves to the tile's maximum only when that exceeds it by more than
        // kLazyMax (base 2): the weights stay below 2^kLazyMax. Most tiles keep
        // m, which this lane's own four scores decide without any cross-lane
        // step; only a wave where some lane sees a larger score finds the
        // heads' maxima and rescales.
        if (__any(lmx > m + kLazyMax32)) {
          const float mx = max_xor32(max_xor16(lmx));
          const float mn = mx > m + kLazyMax32 ? mx : m;
          alp = fast_exp2(m - ((mn == -INFINITY) ? 0.0f : mn));
          ll *= alp;
          m = mn;
          moved = true;
        }
        mu = (m == -INFINITY) ? 0.0f : m;
      } else if (t == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) pp[e] = fast_exp2(pp[e] - mu);
        ll += (pp[0] + pp[1]) + (pp[2] + pp[3]);
      }
    };
    if (next) {
      const float4_t sp = scores(lds0 + (uint32_t)(((i + 1) % 3) * TSTRIDE * 4), stage);
      s_sx[par ^ 1][wave][lane] = sp;
    } else {
#pragma unroll
      for (int t = 0; t < 3; ++t) stage(t);
    }

    // ---- output of tile i ----
    if (moved) {
      // Accumulator item e is head 4*lq + e, whose factor lane 4*lq + e holds.
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ae = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * lq + e) << 2, __float_as_int(alp)));
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c][e] *= ae;
      }
    }
    // P as f16 parts over the tile's 16 positions (lane: head l16, positions
    // 4*lq + e). Each 16-column block accumulates 2^11 P V as P_hi 2^11 V_hi +
    // P_hi V_lo + P_lo V_hi (V_lo and P_lo carry 2^11) into one accumulator:
    // the first two as one x32 product whose contraction runs over (position,
    // part) pairs, A = [P_hi 2^11 | P_hi] against B = [V_hi | V_lo] (the
    // lane's two transpose reads side by side), the third as an x16 product.
    // P_hi 2^11 is exact in f16 because the weights stay at or below
    // 2^kLazyMax32.
    half4_t ph, phs, pl;
    {
#pragma clang fp contract(off)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ph[e] = (_Float16)pp[e];
        phs[e] = (_Float16)((float)ph[e] * 2048.0f);
        pl[e] = (_Float16)__builtin_fmaf((float)ph[e], -2048.0f, pp[e] * 2048.0f);
      }
    }
    const uint32_t prv = lds0 + (uint32_t)((i % 3) * TSTRIDE * 4);
    // Opaque lane addresses of blocks 0-3, as for the score reads; this lane's
    // row 4*lq + (l16 >> 2) keeps its hi halves at byte 8 * ((l16 >> 2) & 1).
    uint32_t vab[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      vab[u] = prv + 4 * vb[u] + 8 * ((l16 >> 2) & 1);
      asm volatile("" : "+v"(vab[u]));
    }
    auto vread = [&](int cb, int part) { return lds_tr16((vab[cb & 3] ^ (8u * part)) + 256 * (cb >> 2)); };
    // Two halves of four blocks; within a half the two products of a block
    // are four MFMAs apart.
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      half4_t vh[4], vl[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        vh[c] = vread(4 * hf + c, 0);
        vl[c] = vread(4 * hf + c, 1);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[4 * hf + c] = mfma32(__builtin_shufflevector(phs, ph, 0, 1, 2, 3, 4, 5, 6, 7),
                                 __builtin_shufflevector(vh[c], vl[c], 0, 1, 2, 3, 4, 5, 6, 7), acc[4 * hf + c]);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[4 * hf + c] = mfma16(pl, vh[c], acc[4 * hf + c]);
    }
    if (!next) break;
    // Tile i+2 (requested after the previous barrier) is the only tile load
    // in flight: wait for it, turn this wave's slots of it into f16 parts, then
    // publish it and the partials of tile i+1.
    wait_vm_lgkm0<0>();
    if (i + 2 < ntiles) {
      split_own((i + 2) % 3);
      wait_vm_lgkm0<0>();
    }
    raw_barrier();
    // Every wave has finished the output product of tile i: its buffer takes
    // tile i+3.
    const int64_t tn = start + (int64_t)(i + 3) * kT32;
    if (tn < end) issue_tile(i % 3, tn);
  }
  // Drain the tile loads still in flight before the workgroup can retire.
  wait_vm_lgkm0<0>();

  // Partials: lane (column l16 of block cb, quarter lq) holds heads 4*lq + i.
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = head0 + 4 * lq + i;
      const int col = dq * 128 + 16 * cb + l16;
      put_partial(a.ws_acc + (ws0 + (int64_t)head * a.S) * kLatDv + col, acc[cb][i] * (1.0f / 2048.0f),
                  FUSED && a.S > 1);
    }
  const float l = sum_xor32(sum_xor16(ll));
  if (dq == 0 && lq == 0) {
    put_partial(a.ws_m + ws0 + (int64_t)(head0 + l16) * a.S, m * kLn2, FUSED && a.S > 1);
    put_partial(a.ws_l + ws0 + (int64_t)(head0 + l16) * a.S, l, FUSED && a.S > 1);
  }
  if constexpr (FUSED) latent_fused_tail<NT>(a, s_c, hg * HW, HW);
}

// Dedicated-role f32 latent kernel: 48 heads of a split per workgroup of
// eight waves (two workgroups per split, as mla32_split_kernel), on the same
// f16 parts. Three scoring waves each own one 16-head block over all 576
// columns (no partial-score exchange), run its online softmax in registers and
// publish P's parts and the rescale factors. Five output waves own the 32
// 16-column value blocks (six each beside a scoring wave on SIMDs 0-2, seven
// each for the two on SIMD 3), multiply every block's P by them, so each
// value block leaves LDS once per tile rather than once per head block. Every
// wave requests its share of the tiles and splits it into parts in place as it
// lands. Four tile buffers and
// one barrier per tile: iteration i scores tile i, runs the output product of
// tile i-1 and requests tile i+2.
struct Mla32dRoles {
  static constexpr int NS = 3;  // scoring waves (one per head block)
  static constexpr int NO = 5;  // output waves
  static constexpr int kShared = 6, kAlone = 7;
  static constexpr bool shared(int w) { return w >= 4 && (w & 3) < NS; }
  static constexpr int ncb(int w) { return w < NS ? 0 : (shared(w) ? kShared : kAlone); }
  static constexpr int cb0(int w) {
    int s = 0;
    for (int v = NS; v < w; ++v) s += ncb(v);
    return s;
  }
  static constexpr int kLoads = kSlots32 / 64;  // 36 wave-loads per tile, over all eight waves
  static constexpr int kScoreLoads = 2;  // wave-loads per scoring wave (the output waves take the rest)
  static constexpr int LB = (kLoads - NS * kScoreLoads) / NO, LX = (kLoads - NS * kScoreLoads) % NO;
  static constexpr int DPW = LB + (LX > 0 ? 1 : 0);
};

struct Mla32dShared {
  float* c;      // four tile buffers
  half4_t* p;    // [2][3 blocks][3 parts][64]: P_hi 2^11, P_hi, P_lo 2^11 (A-operand lane order)
  float* alpha;  // [2][3][16]: rescale factors of a tile
  int* moved;    // [2]: last tile whose factors were not all 1
};

// One role: NCB == 0 scores, else the output product over NCB column blocks.
// Every role passes the same barriers.
template <int NCB, bool FUSED>
__device__ __forceinline__ void mla32d_role(const MlaArgs& a, const Mla32dShared& sh, int64_t start,
                                            int64_t end, int64_t ws0, int b, int hg) {
  using R = Mla32dRoles;
  constexpr int HW = 48, NW = 8, NBUF = 4;
  constexpr int TSTR = kSlots32 * 4;  // floats per tile buffer
  constexpr int KS = kLatDk / 32;     // 18 x32 score steps
  constexpr bool SCORER = NCB == 0;
  static_assert(R::cb0(8) == kLatDv / 16, "the output waves cover the value columns");
  static_assert(R::kLoads * 64 == kSlots32, "whole wave-loads");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int lq = lane >> 4;
  float* const s_c = sh.c;

  const float* __restrict__ cbase = reinterpret_cast<const float*>(a.c) + (int64_t)b * a.stride_seq;
  const float* __restrict__ qb = a.q + ((int64_t)b * a.Hq + hg * HW) * kLatDk;

  // Tile staging as in mla32_split_kernel (slot s: row s / 144, logical chunk
  // (s % 144) ^ row); every wave issues and splits its share of the 36
  // wave-loads of a tile.
  const int ow = wave - R::NS;
  const int wl0 = SCORER ? wave * R::kScoreLoads : R::NS * R::kScoreLoads + ow * R::LB + min(ow, R::LX);
  const int nwl = SCORER ? R::kScoreLoads : R::LB + (ow < R::LX ? 1 : 0);
  const uint32_t lds0 = lds_addr_of(s_c);
  const uint32_t row_bytes = (uint32_t)(a.stride_pos * 4);  // 16 rows: offsets fit 32 bits
  auto issue_tile = [&](int bi, int64_t tb) {
    {
      const int64_t tbc = tb < end ? tb : end - 1;
      const uint64_t bu = reinterpret_cast<uint64_t>(cbase + tbc * a.stride_pos);
      const void* base = reinterpret_cast<const void*>(
          ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(bu >> 32)) << 32) |
          (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bu));
      const int last = (int)(end - 1 - tbc);
#pragma unroll
      for (int cc = 0; cc < R::DPW; ++cc) {
        if (cc >= nwl) continue;  // scoring and output waves take different shares
        const int sl = (wl0 + cc) * 64 + lane;
        const int srow = sl / kCpr32;
        const int scol = (sl - srow * kCpr32) ^ srow;
        const uint32_t off = (uint32_t)min(srow, last) * row_bytes + (uint32_t)(scol * 16);
        const uint32_t dst = lds0 + (uint32_t)((bi * TSTR + (wl0 + cc) * 256) * 4);
        dma16s(off, base, __builtin_amdgcn_readfirstlane(dst), a.nt);
      }
    }
  };
  // The slots this wave loaded, as f16 parts in place; odd rows keep lo first.
  auto split_own = [&](int bi) {
    {
#pragma unroll
      for (int cc = 0; cc < R::DPW; ++cc) {
        if (cc >= nwl) continue;  // scoring and output waves take different shares
        const int sl = (wl0 + cc) * 64 + lane;
        u32x4_t* p = reinterpret_cast<u32x4_t*>(s_c + bi * TSTR + sl * 4);
        const u32x4_t v = f16_parts(__builtin_bit_cast(float4_t, *p));
        *p = ((sl / kCpr32) & 1) ? u32x4_t{v.z, v.w, v.x, v.y} : v;
      }
    }
  };
  // Everything of this wave but its loads of the newest tile has landed.
  auto wait_but_newest = [&]() {
    if constexpr (SCORER) {
      wait_vm_lgkm0<R::kScoreLoads>();
    } else if constexpr (R::LX == 0) {
      wait_vm_lgkm0<R::DPW>();
    } else {
      if (nwl == R::DPW)
        wait_vm_lgkm0<R::DPW>();
      else
        wait_vm_lgkm0<R::DPW - 1>();
    }
  };

  const int ntiles = (int)((end - start + kT32 - 1) / kT32);
  // Prologue: tile 0; the query rows (48 x 576 f32, times scale log2 e)
  // staged through tile buffers 1-3, which they fill, with whole-line loads by
  // the whole workgroup (row h keeps chunk c at position c ^ (h & 15)); each
  // scoring wave splits its block's fragments into parts; then tile 1.
  constexpr int QF = HW * kLatDk / 4;
  constexpr int QV = (QF + NW * 64 - 1) / (NW * 64);
  static_assert(HW * kLatDk <= 3 * TSTR, "the staged rows fit");
  float* const sq = s_c + TSTR;
  issue_tile(0, start);
  {
    float4 qv[QV];
#pragma unroll
    for (int k = 0; k < QV; ++k)
      if (QF % (NW * 64) == 0 || tid + NW * 64 * k < QF)
        qv[k] = *reinterpret_cast<const float4*>(qb + 4 * (tid + NW * 64 * k));
#pragma unroll
    for (int k = 0; k < QV; ++k) {
      const int f = tid + NW * 64 * k;
      if (QF % (NW * 64) != 0 && f >= QF) continue;
      const int h = f / (kLatDk / 4);
      const int c = f - h * (kLatDk / 4);
      *reinterpret_cast<float4_t*>(sq + h * kLatDk + ((c ^ (h & 15)) << 2)) =
          float4_t{qv[k].x * a.qscale, qv[k].y * a.qscale, qv[k].z * a.qscale, qv[k].w * a.qscale};
    }
  }
  wait_vm_lgkm0<0>();  // the staged rows and tile 0
  raw_barrier();
  // Score chunk t of a scoring wave (t = 0..35): logical chunk lq + 4t of row
  // (head) l16, at sb[t & 3] + 64 (t >> 2) floats; step s takes chunks 2s and
  // 2s + 1.
  int sb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) sb[u] = l16 * kLatDk + (((lq + 4 * u) ^ l16) << 2);
  auto soff = [&](int t) { return sb[t & 3] + 64 * (t >> 2); };
  half8_t qh[SCORER ? KS : 1], ql[SCORER ? KS : 1];
  if constexpr (SCORER) {
    const float* qrow = sq + 16 * wave * kLatDk;  // rows 16w + l16 (swizzle l16)
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const u32x4_t p0 = f16_parts(*reinterpret_cast<const float4_t*>(qrow + soff(2 * st)));
      const u32x4_t p1 = f16_parts(*reinterpret_cast<const float4_t*>(qrow + soff(2 * st + 1)));
      qh[st] = __builtin_bit_cast(half8_t, u32x4_t{p0.x, p0.y, p1.x, p1.y});
      ql[st] = __builtin_bit_cast(half8_t, u32x4_t{p0.z, p0.w, p1.z, p1.w});
    }
  }
  raw_barrier();  // the staged rows are read: buffers 1-3 are free
  issue_tile(1, start + kT32);
  split_own(0);
  wait_but_newest();
  raw_barrier();  // tile 0's parts

  if constexpr (SCORER) {
    float m = -INFINITY, ll = 0.0f;  // head 16w + l16 (replicated over quarters); ll: this lane's share
    for (int i = 0; i < ntiles; ++i) {
      const int64_t tb = start + (int64_t)i * kT32;
      const bool load_next = tb + 2 * kT32 < end;
      if (load_next) issue_tile((i + 2) % NBUF, tb + 2 * kT32);
      const uint32_t cur = lds0 + (uint32_t)((i % NBUF) * TSTR * 4);
      // Lane addresses of chunks 0-3 (hi halves: byte 8 (l16 & 1) of a
      // chunk; lo: bit 3 flipped), opaque so the other chunks' reads use the
      // instructions' offset fields.
      uint32_t ab[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ab[u] = cur + 4 * sb[u] + 8 * (l16 & 1);
        asm volatile("" : "+v"(ab[u]));
      }
      auto opnd = [&](int st, int part) {
        const u32x2_t x0 = lds_ld8((ab[(2 * st) & 3] ^ (8u * part)) + 256 * ((2 * st) >> 2));
        const u32x2_t x1 = lds_ld8((ab[(2 * st + 1) & 3] ^ (8u * part)) + 256 * ((2 * st + 1) >> 2));
        return __builtin_bit_cast(half8_t, u32x4_t{x0.x, x0.y, x1.x, x1.y});
      };
      const float4_t z = float4_t{0.f, 0.f, 0.f, 0.f};
      float4_t sp[2] = {z, z}, sa[2] = {z, z}, sc[2] = {z, z};
      half8_t nh = opnd(0, 0), nl = opnd(0, 1);
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const half8_t ah = nh, al = nl;
        if (st + 1 < KS) {
          nh = opnd(st + 1, 0);
          nl = opnd(st + 1, 1);
        }
        sa[st & 1] = mfma32(ah, ql[st], sa[st & 1]);
        sp[st & 1] = mfma32(ah, qh[st], sp[st & 1]);
        sc[st & 1] = mfma32(al, qh[st], sc[st & 1]);
        if (st & 1) __builtin_amdgcn_sched_barrier(0);
      }
      const float4_t lo = (sa[0] + sa[1]) + (sc[0] + sc[1]);
      const float4_t hi = sp[0] + sp[1];
      const int rel = (int)(end - tb);  // positions of tile i before the end (> 0)
      float v[4], lmx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = 4 * lq + e < rel ? fmaf(lo[e], 1.0f / 2048.0f, hi[e]) : -INFINITY;
        lmx = fmaxf(lmx, v[e]);
      }
      // Lazy running maximum (threshold kLazyMax32, base 2), as in
      // mla32_split_kernel.
      float al = 1.0f;
      bool moved = false;
      if (__any(lmx > m + kLazyMax32)) {
        const float mx = max_xor32(max_xor16(lmx));
        const float mn = mx > m + kLazyMax32 ? mx : m;
        al = fast_exp2(m - ((mn == -INFINITY) ? 0.0f : mn));
        ll *= al;
        m = mn;
        moved = true;
      }
      const float mu = (m == -INFINITY) ? 0.0f : m;
      half4_t phs, ph, pl;
      {
#pragma clang fp contract(off)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = fast_exp2(v[e] - mu);
          ll += pe;
          ph[e] = (_Float16)pe;
          phs[e] = (_Float16)((float)ph[e] * 2048.0f);
          pl[e] = (_Float16)__builtin_fmaf((float)ph[e], -2048.0f, pe * 2048.0f);
        }
      }
      const int par = i & 1;
      half4_t* pw = sh.p + (par * 3 + wave) * 3 * 64 + lane;
      pw[0] = phs;
      pw[64] = ph;
      pw[128] = pl;
      if (lq == 0) sh.alpha[(par * 3 + wave) * 16 + l16] = al;
      // Several scoring waves may report the same tile: an LDS atomic max
      // (the flag only ever rises to the newest tile index).
      if (__any(moved) && lane == 0) atomicMax(&sh.moved[par], i);
      // Tile i+1 must have landed: split this wave's slots of it.
      if (load_next)
        wait_but_newest();
      else
        wait_vm_lgkm0<0>();
      if (i + 1 < ntiles) {
        split_own((i + 1) % NBUF);
        if (load_next)
          wait_but_newest();
        else
          wait_vm_lgkm0<0>();
      }
      raw_barrier();  // P and factors of tile i; tile i+1's parts
    }
    wait_vm_lgkm0<0>();
    const float l = sum_xor32(sum_xor16(ll));
    if (lq == 0) {
      const int head = hg * HW + 16 * wave + l16;
      put_partial(a.ws_m + ws0 + (int64_t)head * a.S, m * kLn2, FUSED && a.S > 1);
      put_partial(a.ws_l + ws0 + (int64_t)head * a.S, l, FUSED && a.S > 1);
    }
  } else {
    const int cb0 = R::cb0(wave);
    // Value reads (transposed, 16 columns by 4 rows per 16 lanes): lane
    // l16 = 4 rho + sg of quarter lq takes row r = 4 lq + rho, columns
    // 4 sg .. +3 of block cb0 + u: logical chunk 4 (cb0 + u) + sg, at
    // (chunk ^ r); its hi halves at byte 8 (r & 1).
    const int r = 4 * lq + (l16 >> 2);
    uint32_t vo[NCB];
#pragma unroll
    for (int u = 0; u < NCB; ++u)
      vo[u] = (uint32_t)((r * kLatDk + (((4 * (cb0 + u) + (l16 & 3)) ^ r) << 2)) * 4 + 8 * (r & 1));
    float4_t acc[3][NCB];
#pragma unroll
    for (int hb = 0; hb < 3; ++hb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[hb][cb] = float4_t{0.f, 0.f, 0.f, 0.f};
    auto output = [&](int j) {
      const uint32_t prv = lds0 + (uint32_t)((j % NBUF) * TSTR * 4);
      const int par = j & 1;
      if (sh.moved[par] == j) {
        // Accumulator items are heads 4 lq + e of each block.
#pragma unroll
        for (int hb = 0; hb < 3; ++hb) {
          const float4_t alp = *reinterpret_cast<const float4_t*>(&sh.alpha[(par * 3 + hb) * 16 + 4 * lq]);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[hb][cb][e] *= alp[e];
        }
      }
      half4_t pp[3][3];
#pragma unroll
      for (int hb = 0; hb < 3; ++hb)
#pragma unroll
        for (int part = 0; part < 3; ++part) pp[hb][part] = sh.p[((par * 3 + hb) * 3 + part) * 64 + lane];
      half4_t vh = lds_tr16(prv + vo[0]), vl = lds_tr16((prv + vo[0]) ^ 8u);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const half4_t bh = vh, bl = vl;
        if (cb + 1 < NCB) {
          vh = lds_tr16(prv + vo[cb + 1]);
          vl = lds_tr16((prv + vo[cb + 1]) ^ 8u);
        }
        const half8_t bb = __builtin_shufflevector(bh, bl, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int hb = 0; hb < 3; ++hb)
          acc[hb][cb] = mfma32(__builtin_shufflevector(pp[hb][0], pp[hb][1], 0, 1, 2, 3, 4, 5, 6, 7), bb, acc[hb][cb]);
#pragma unroll
        for (int hb = 0; hb < 3; ++hb) acc[hb][cb] = mfma16(pp[hb][2], bh, acc[hb][cb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int i = 0;; ++i) {
      const bool more = i < ntiles;  // tile i exists (else only tile i-1's output remains)
      const int64_t tb = start + (int64_t)i * kT32;
      // Tile i+2 goes into the buffer of tile i-2, whose output product ran
      // before the last barrier; tiles past the end are not requested.
      const bool load_next = more && tb + 2 * kT32 < end;
      if (load_next) issue_tile((i + 2) % NBUF, tb + 2 * kT32);
      if (i > 0) output(i - 1);
      if (!more) break;
      // Tile i+1 (requested one iteration ago, or in the prologue) must have
      // landed: split it into parts; tile i+2's loads, if any, stay in flight.
      if (load_next)
        wait_but_newest();
      else
        wait_vm_lgkm0<0>();
      if (i + 1 < ntiles) {
        split_own((i + 1) % NBUF);
        if (load_next)
          wait_but_newest();
        else
          wait_vm_lgkm0<0>();
      }
      raw_barrier();
    }
    // Drain the tile loads still in flight before the workgroup can retire.
    wait_vm_lgkm0<0>();
    // Partials: heads 16 hb + 4 lq + e, columns 16 (cb0 + cb) + l16.
#pragma unroll
    for (int hb = 0; hb < 3; ++hb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int head = hg * HW + 16 * hb + 4 * lq + e;
          const int col = 16 * (cb0 + cb) + l16;
          put_partial(a.ws_acc + (ws0 + (int64_t)head * a.S) * kLatDv + col, acc[hb][cb][e] * (1.0f / 2048.0f),
                      FUSED && a.S > 1);
        }
  }
}

template <bool FUSED>
__global__ __launch_bounds__(512) void mla32d_split_kernel(MlaArgs a) {
  constexpr int HW = 48, NBUF = 4;
  using R = Mla32dRoles;
  __shared__ __align__(16) float s_c[NBUF * kSlots32 * 4];
  __shared__ __align__(16) half4_t s_p[2 * 3 * 3 * 64];
  __shared__ __align__(16) float s_alpha[2 * 3 * 16];
  __shared__ int s_moved[2];

  const int split = blockIdx.x;
  const int b = blockIdx.y;
  const int hg = blockIdx.z;
  const int tid = threadIdx.x;
  const int L = min(a.seq_lens[b], a.cap);
  const int64_t start = (int64_t)split * a.chunk;
  const int64_t end = min((int64_t)L, start + a.chunk);
  const int64_t ws0 = (int64_t)b * a.Hq * a.S + split;
  if (start >= end) {
    if constexpr (FUSED) {
      latent_fused_tail<512>(a, s_c, hg * HW, HW);
      return;
    }
    for (int idx = tid; idx < HW * kLatDv; idx += 512) {
      const int h = hg * HW + idx / kLatDv, e = idx - (idx / kLatDv) * kLatDv;
      a.ws_acc[(ws0 + (int64_t)h * a.S) * kLatDv + e] = 0.0f;
    }
    for (int h = tid; h < HW; h += 512) {
      a.ws_m[ws0 + (int64_t)(hg * HW + h) * a.S] = -INFINITY;
      a.ws_l[ws0 + (int64_t)(hg * HW + h) * a.S] = 0.0f;
    }
    return;
  }
  if (tid < 2) s_moved[tid] = -1;
  const Mla32dShared sh{s_c, s_p, s_alpha, s_moved};
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave < R::NS)
    mla32d_role<0, FUSED>(a, sh, start, end, ws0, b, hg);
  else if (R::shared(wave))
    mla32d_role<R::kShared, FUSED>(a, sh, start, end, ws0, b, hg);
  else
    mla32d_role<R::kAlone, FUSED>(a, sh, start, end, ws0, b, hg);
  if constexpr (FUSED) latent_fused_tail<512>(a, s_c, hg * HW, HW);
}

int latent_blocks_per_split(const sk_desc_t& d) {
  return d.kv_dtype == SK_F32 ? mla32_groups(d.num_q_heads) : mla16_groups(d.num_q_heads);
}

bool latent_supported(const sk_desc_t& d) {
  const bool heads_ok = d.num_q_heads == 32 || d.num_q_heads == 64 || d.num_q_heads == 96 ||
                        d.num_q_heads == 128;
  const bool layout_ok = d.layout == SK_KV_CONTIGUOUS || d.layout == SK_KV_INDEXED;
  return d.kv_shared == 1 && d.num_kv_heads == 1 && d.head_dim_qk == kLatDk &&
         d.head_dim_v == kLatDv && layout_ok && d.q_dtype == SK_F32 &&
         (d.kv_dtype == SK_F32 || d.kv_dtype == SK_F16) && heads_ok;
}

template <typename CT, int NHB>
static sk_status_t latent_variant(const SplitLaunch& s, bool launch, const void** fn, int grid[3],
                                  int* block) {
  const sk_desc_t& d = *s.d;
  // f32 caches take the f16-part kernel, f16 caches the x32 f16 kernels; each
  // spreads a split's heads over one or more workgroups (mla32_groups,
  // mla16_groups).
  constexpr int H = NHB * 16;
  constexpr bool kF32 = sizeof(CT) == 4;
  void (*kern)(MlaArgs);
  int threads, groups;
  const bool idx = d.layout == SK_KV_INDEXED;
  if constexpr (kF32) {
    kern = idx ? (s.fused ? mla32_split_kernel<mla32_blocks(H), true, true> : mla32_split_kernel<mla32_blocks(H), true, false>)
               : (s.fused ? mla32_split_kernel<mla32_blocks(H), false, true> : mla32_split_kernel<mla32_blocks(H), false, false>);
    threads = mla32_blocks(H) * 256;
    groups = mla32_groups(H);
    if constexpr (H == 96) {
      if (!idx && (int64_t)s.p->n_splits * d.batch >= 64) {
        // Contiguous caches, once the grid (two workgroups per (split,
        // sequence) pair) fills half the compute units: the dedicated-role
        // form. Shorter grids keep the four-wave form, the one the
        // index-list path shares tile for tile.
        kern = s.fused ? mla32d_split_kernel<true> : mla32d_split_kernel<false>;
        threads = 512;
      }
    }
  } else {
    if constexpr (H == 64 || H == 96) {
      // (Contiguous caches never take the whole-head form of this kernel
      // for these head counts, so it is not built for them.)
      kern = s.fused ? mla16_split_kernel<mla16_blocks(H), true, true> : mla16_split_kernel<mla16_blocks(H), true, false>;
    } else {
      kern = idx ? (s.fused ? mla16_split_kernel<mla16_blocks(H), true, true> : mla16_split_kernel<mla16_blocks(H), true, false>)
                 : (s.fused ? mla16_split_kernel<mla16_blocks(H), false, true> : mla16_split_kernel<mla16_blocks(H), false, false>);
    }
    threads = mla16_blocks(H) * 128;
    groups = mla16_groups(H);
    if constexpr (H == 64 || H == 96) {
      if ((int64_t)s.p->n_splits * d.batch <= kHalveHeadsAt) {
        // A short context leaves most of the 256 compute units idle with one
        // workgroup per split: up to 128 (split, sequence) pairs, the heads go
        // to two workgroups of half as many (results unchanged: each head's
        // arithmetic does not depend on its workgroup).
        kern = idx ? (s.fused ? mla16_split_kernel<H / 32, true, true> : mla16_split_kernel<H / 32, true, false>)
                   : (s.fused ? mla16_split_kernel<H / 32, false, true> : mla16_split_kernel<H / 32, false, false>);
        threads = (H / 32) * 128;
        groups = 2;
      } else if (!idx) {
        // Contiguous caches at longer contexts: the dedicated-role form.
        kern = s.fused ? mla16d_split_kernel<H / 16, true> : mla16d_split_kernel<H / 16, false>;
        threads = 512;
        groups = 1;
      }
    }
  }
  const dim3 gr(s.p->n_splits, d.batch, groups);
  grid[0] = gr.x;
  grid[1] = gr.y;
  grid[2] = gr.z;
  *block = threads;
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
  a.table = s.block_table;
  a.max_idx = d.max_pages_per_seq;
  a.num_rows = d.num_pages;
  a.nt = groups == 1;
  a.counters = s.counters;
  a.out = s.out;
  a.lse = s.lse;
  if (!s.fused || s.p->n_splits == 1) {
    hipLaunchKernelGGL(kern, gr, dim3(threads), 0, s.stream, a);
    return SK_OK;
  }
  // With more than one split the one-launch form waits at a grid barrier, so
  // every workgroup must be resident at once: a cooperative launch, which the
  // runtime refuses rather than start a grid that does not fit; it is checked
  // here first.
  int per_cu = 0, cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), threads, 0) !=
          hipSuccess)
    return SK_ERR_HIP;
  if ((int64_t)gr.x * gr.y * gr.z > (int64_t)per_cu * cus) return SK_ERR_UNSUPPORTED;
  void* args[] = {&a};
  if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), gr, dim3(threads), args, 0, s.stream) !=
      hipSuccess)
    return SK_ERR_LAUNCH;
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
