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
//     (RL = 16 or 32), so one vector load instruction reads whole contiguous
//     row segments of RL*16 bytes.
//   * Each lane keeps its D/RL dimensions of its query vectors and accumulators
//     in registers; a dot product is a per-lane partial followed by a 16-lane
//     DPP reduction (plus one swizzle when RL = 32). With HS head slices, HS
//     sets of RL lanes read the same row and each serves G/HS of the heads,
//     which divides the per-lane reductions and exponentials by HS.
//   * The workgroup's NG = 256/(RL*HS) row groups take interleaved positions
//     base + r*NG + group, R rows per group per tile, and each group carries its
//     own online-softmax state (m, l, acc) per head; tile-level rescaling follows
//     the recurrence of "Decoder Block 6" and Lecture 07 ("But Softmax Wants the
//     Whole Row..."): m' = max(m, tile max), a = exp(m - m'), l = a l + sum p,
//     acc = a acc + sum p v. The multiply by a is skipped when no head's
//     maximum moved anywhere in the wave (a is then exactly 1).
//   * Contiguous caches are read with raw buffer loads: one resource per tile
//     bounds the reads to the split, so the tail of the last tile and the
//     pipeline's look-ahead past the end read nothing from memory. Every K/V
//     load carries the non-temporal policy (the rows are read once), and a
//     contiguous tile's K loads all go out before its V loads.
//   * Scores are kept in base-2 units (q is pre-multiplied by scale*log2 e) so
//     every exponential is one exp2; the stored m is converted back to natural
//     units.
//   * At the end the row groups merge by cross-lane exchange, the waves merge
//     through LDS (4*G*D floats, independent of the context length), and the
//     workgroup writes one partial per query head.
//   * One-launch variant (FUSED): the combine step runs inside the same grid.
//     Each workgroup that holds positions writes its partial with device-scope
//     stores (they write through this XCD's L2 to the device's coherence
//     point), waits until they have completed, and counts itself in a
//     per-(sequence, KV head) counter; the workgroup whose count completes the
//     set merges the group's partials with device-scope loads (Lecture 06
//     section 2: M = max m_i, l = sum l_i exp(m_i - M), out = sum acc_i
//     exp(m_i - M) / l) and resets the counter to zero for the next call. No
//     workgroup waits for another, and no cache is flushed or invalidated: a
//     device-scope fence per workgroup writes back or drops a whole L2 and
//     measured tens of microseconds per launch.
#include <type_traits>

#include "sk_device.h"
#include "sk_internal.h"
#include "sk_merge.h"

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
  int32_t paged_fast;  // page size, tile span and split chunk line up (see the tile loop)
  float qscale;
  // One-launch decode only.
  uint32_t* counters;  // [B][Hkv], zero between calls
  float* out;          // [B][Hq][D]
  float* lse;          // [B][Hq] or null
};

// Addressing modes of the tile loop.
constexpr int kContig = 0, kPagedFast = 1, kPagedAny = 2;

template <typename KV, int D, int RL_, int R_, int HS_>
struct GqaShape {
  static constexpr int RL = RL_;
  static constexpr int R = R_;
  static constexpr int HS = HS_;  // head slices: lane sets that share a row, each with G/HS heads
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kGroupLanes = RL * HS;
  static constexpr int kGroupsPerWave = 64 / kGroupLanes;
  static constexpr int kGroups = kGroupsPerWave * kWaves;
  static constexpr int kDpl = D / RL;
  static constexpr int kVecMax = 16 / (int)sizeof(KV);
  static constexpr int kVec = kVecMax < kDpl ? kVecMax : kDpl;
  static constexpr int kLoads = kDpl / kVec;
  static_assert(D % RL == 0, "row width must split evenly over the row's lanes");
  static_assert(kDpl % kVec == 0, "lane slice must be whole vector loads");
};

// Loads this lane's slice of the G query vectors of one group, scaled into
// base-2 units. q's storage type is uniform, so the branch is taken once.
template <int G, int D, int RL, int VEC, int NL, typename QT>
__device__ __forceinline__ void load_q_slice(float (&qr)[G][D / RL], const QT* q, int li,
                                             float qscale) {
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < NL; ++j)
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        qr[h][j * VEC + e] = to_f32(q[h * D + j * RL * VEC + li * VEC + e]) * qscale;
}

// Largest slices first, for a batch of 2 to 64 sequences. Workgroups start
// in the order of their pair index k = blockIdx.y + S * blockIdx.z, so k is
// mapped to the (split, sequence) pairs ordered by work: every full-chunk
// slice first (sequence by sequence), then the partial last slices, longest
// first, then the empty ones. Short slices then fill the grid's tail instead
// of full ones starting last (list scheduling, largest job first); what each
// pair computes and where it writes are unchanged. Wave 0 finds the pair
// (lane t holds sequence t) and publishes it in LDS. Lengths are clamped as
// the slices use them; in the one-launch form a rejected length counts as
// empty, so that sequence's split-0 pair still writes its NaN result.
__device__ __forceinline__ void work_ordered_pair(const GqaArgs& a, bool fused, int* s_pair, int& split,
                                                  int& b) {
  const int B = gridDim.z;
  split = blockIdx.y;
  b = blockIdx.z;
  if (B == 1 || B > 64) return;
  if (threadIdx.x < 64) {
    const int t = threadIdx.x;
    const int S = a.S;
    const int64_t span = (int64_t)S * a.chunk;
    int64_t le = 0;
    if (t < B) {
      const int lraw = a.seq_lens[t];
      const bool ok = !fused || (lraw >= 1 && lraw <= a.cap && (int64_t)lraw <= span);
      le = ok ? max((int64_t)0, min((int64_t)min(lraw, a.cap), span)) : 0;
    }
    const int nf = (int)(le / a.chunk);                 // full-chunk slices
    const int r = (int)(le - (int64_t)nf * a.chunk);    // rows of the partial last slice (0: none)
    const int n = nf + (r > 0 ? 1 : 0);
    const int e = t < B ? S - n : 0;                    // empty slices
    int pf = 0, pe = 0, rk = 0, F = 0, P = 0;
    for (int u = 0; u < B; ++u) {
      const int nfu = __builtin_amdgcn_readlane(nf, u);
      const int ru = __builtin_amdgcn_readlane(r, u);
      const int eu = __builtin_amdgcn_readlane(e, u);
      pf += u < t ? nfu : 0;
      pe += u < t ? eu : 0;
      rk += (ru > r || (ru == r && u < t)) ? 1 : 0;  // rank among the partial slices (r > 0)
      F += nfu;
      P += ru > 0 ? 1 : 0;
    }
    const int k = (int)blockIdx.y + S * (int)blockIdx.z;
    bool mine;
    int sp;
    if (k < F) {
      mine = t < B && k >= pf && k < pf + nf;
      sp = k - pf;
    } else if (k < F + P) {
      mine = t < B && r > 0 && rk == k - F;
      sp = nf;
    } else {
      const int q = k - F - P;
      mine = t < B && q >= pe && q < pe + e;
      sp = n + (q - pe);
    }
    // Exactly one lane owns k (the map is a bijection). One lane writes: the
    // owner, or lane 0 with the unmapped pair should none match, so the pair
    // read below is always in range.
    const uint64_t own = __builtin_amdgcn_ballot_w64(mine && sp >= 0 && sp < S);
    const int src = own ? (int)__builtin_ctzll(own) : 0;
    if (t == src) {
      s_pair[0] = own ? sp : split;
      s_pair[1] = own ? t : b;
    }
  }
  __syncthreads();
  split = s_pair[0];
  b = s_pair[1];
}

template <typename KV, int G, int D, bool PAGED, int RL, int R, int HS, int WPE, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE))) void gqa_split_kernel(
    GqaArgs a) {
  using Sh = GqaShape<KV, D, RL, R, HS>;
  static_assert(G % HS == 0, "head slices must split the group evenly");
  constexpr int GH = G / HS;  // query heads per lane
  constexpr int DPL = Sh::kDpl;
  constexpr int VEC = Sh::kVec;
  constexpr int NL = Sh::kLoads;
  constexpr int NG = Sh::kGroups;
  constexpr int NW = Sh::kWaves;
  constexpr int TR = NG * R;  // positions per tile
  using V = Vec<KV, VEC>;

  __shared__ float s_acc[NW][G][D];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];

  __shared__ int s_pair[2];
  const int g = blockIdx.x;
  int split, b;
  work_ordered_pair(a, FUSED, s_pair, split, b);
  const int Hkv = gridDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & (RL - 1);
  const int hs = (lane / RL) % HS;
  const int grp = wave * Sh::kGroupsPerWave + lane / Sh::kGroupLanes;
  const int h0 = g * G;

  const int Lraw = a.seq_lens[b];
  if constexpr (FUSED) {
    // A length outside [1, min(cap, S*chunk)] is a caller error: that
    // sequence's outputs become NaN and nothing of it is read or counted.
    const bool valid = Lraw >= 1 && Lraw <= a.cap && (int64_t)Lraw <= (int64_t)a.S * a.chunk;
    if (!valid) {
      if (split == 0) {
        for (int idx = tid; idx < G * D; idx += Sh::kThreads)
          a.out[((int64_t)b * a.Hq + h0) * D + idx] = __builtin_nanf("");
        if (a.lse && tid < G) a.lse[(int64_t)b * a.Hq + h0 + tid] = __builtin_nanf("");
      }
      return;
    }
  }
  const int L = min(Lraw, a.cap);
  const int64_t start = (int64_t)split * a.chunk;
  const int64_t end = min((int64_t)L, start + a.chunk);
  const int64_t ws0 = ((int64_t)b * a.Hq + h0) * a.S + split;

  if (start >= end) {
    // One-launch variant: an empty slice takes no part in the merge.
    if constexpr (FUSED) return;
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

  // This lane's slice of its GH query vectors (heads h0 + hs*GH ...),
  // pre-scaled into base-2 units; loaded after the first tile is requested,
  // so the query's memory latency overlaps the first K/V loads.
  float qr[GH][DPL];
  // Inlined at both paged modes' call sites: a call would put the kernel's
  // state in scratch memory.
  auto load_q = [&]() __attribute__((always_inline)) {
    const int64_t qbase = ((int64_t)b * a.Hq + h0 + hs * GH) * D;
    if (a.q_dtype == 0)
      load_q_slice<GH, D, RL, VEC, NL>(qr, reinterpret_cast<const float*>(a.q) + qbase, li, a.qscale);
    else if (a.q_dtype == 1)
      load_q_slice<GH, D, RL, VEC, NL>(qr, reinterpret_cast<const _Float16*>(a.q) + qbase, li, a.qscale);
    else
      load_q_slice<GH, D, RL, VEC, NL>(qr, reinterpret_cast<const bf16_t*>(a.q) + qbase, li, a.qscale);
  };

  float m[GH], l[GH], acc[GH][DPL];
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[h][d] = 0.0f;
  }

  // Row addressing. Contiguous: a tile's rows sit at fixed 32-bit byte
  // offsets from the tile's first row, whose address is uniform across the
  // workgroup (scalar registers). Paged: (page*page_size + slot)*Hkv*D elements from this head's column
  // of the pool, page indices from the block table.
  const int lane_col = li * VEC;
  const int64_t head_off =
      PAGED ? (int64_t)g * a.stride_head : (int64_t)b * a.stride_seq + (int64_t)g * a.stride_head;
  const KV* __restrict__ kb = reinterpret_cast<const KV*>(a.k) + head_off + lane_col;
  const KV* __restrict__ vb = reinterpret_cast<const KV*>(a.v) + head_off + lane_col;
  const KV* __restrict__ kh = reinterpret_cast<const KV*>(a.k) + head_off;
  const KV* __restrict__ vh = reinterpret_cast<const KV*>(a.v) + head_off;
  const int64_t row_stride = a.stride_pos;  // paged: Hkv*D (pool rows); indexed: the caller's
  const int ps_mask = (1 << a.page_shift) - 1;
  const int32_t* __restrict__ table = a.block_table + (int64_t)b * a.max_pages;
  const uint32_t row_bytes = (uint32_t)(row_stride * (int64_t)sizeof(KV));  // host-checked < 2^31 / TR
  uint32_t loff[R];
#pragma unroll
  for (int r = 0; r < R; ++r) loff[r] = (uint32_t)(r * NG + grp) * row_bytes + (uint32_t)(lane_col * sizeof(KV));

  // The tile loop, instantiated per addressing mode:
  //  * kContig: one buffer resource per tile (rows before `end` only);
  //  * kPagedFast: every row set r of a tile (rows r*NG + group) lies in one
  //    page, the same for the whole workgroup (the host guarantees that page
  //    size, tile span and split chunk line up), so its page index is one
  //    scalar table load and its rows are one buffer resource covering the
  //    page's rows before `end`; lane offsets are loop-invariant;
  //  * kPagedAny: per-lane page lookups, rows past `end` re-read row end-1.
  const uint32_t lofp = (uint32_t)grp * row_bytes + (uint32_t)(lane_col * sizeof(KV));
  auto run = [&](auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;

    // kPagedAny: rows past `end` read row end-1 instead (in bounds, a cache
    // hit); their scores are masked to -inf.
    auto table_page = [&](int64_t pos) -> int {
      return table[pos >> a.page_shift];
    };
    int64_t last_off = 0;
    if constexpr (MODE == kPagedAny) {
      int pg = table_page(end - 1);
      pg = (pg < 0 || (int64_t)pg >= a.num_pages) ? 0 : pg;
      last_off = (((int64_t)pg << a.page_shift) + ((end - 1) & ps_mask)) * row_stride;
    }

    // Page indices of a tile. kPagedAny: per lane, one per row (rows past the
    // end look up row end-1's page). kPagedFast: one per row set, uniform.
    // The table is never read out of range.
    auto load_pages = [&](int (&pg)[R], int64_t tb) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if constexpr (MODE == kPagedFast) {
          const int64_t pos0 = tb + r * NG;
          pg[r] = __builtin_amdgcn_readfirstlane(table_page(pos0 < end ? pos0 : end - 1));
        } else {
          const int64_t pos = tb + r * NG + grp;
          pg[r] = table_page(pos < end ? pos : end - 1);
        }
      }
    };

    auto issue = [&](V (&kt)[R][NL], V (&vt)[R][NL], int64_t tb, const int (&pg)[R]) {
      if constexpr (MODE == kPagedAny) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int64_t pos = tb + r * NG + grp;
          const int p = (pg[r] < 0 || (int64_t)pg[r] >= a.num_pages) ? 0 : pg[r];
          int64_t off = (((int64_t)p << a.page_shift) + (pos & ps_mask)) * row_stride;
          off = pos < end ? off : last_off;
#pragma unroll
          for (int j = 0; j < NL; ++j) {
            kt[r][j] = load_vec_stream<KV, VEC>(kb + off + j * RL * VEC);
            vt[r][j] = load_vec_stream<KV, VEC>(vb + off + j * RL * VEC);
          }
        }
      } else if constexpr (MODE == kPagedFast) {
        // Each K load beside the V load of the same row: for 16-token pages this
        // measured faster than the contiguous path's K-then-V order.
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int64_t pos0 = tb + r * NG;
          const int64_t left = end - pos0;
          const bool bad = pg[r] < 0 || (int64_t)pg[r] >= a.num_pages;
          const uint32_t nbytes =
              (bad || left <= 0) ? 0u : (uint32_t)(left < NG ? left : NG) * row_bytes;
          const int64_t row0 = ((int64_t)(bad ? 0 : pg[r]) << a.page_shift) + (pos0 & ps_mask);
          const auto rk = raw_rsrc(kh + row0 * row_stride, nbytes);
          const auto rv = raw_rsrc(vh + row0 * row_stride, nbytes);
#pragma unroll
          for (int j = 0; j < NL; ++j) {
            const uint32_t o = lofp + (uint32_t)(j * RL * VEC * sizeof(KV));
            kt[r][j] = load_vec_stream<KV, VEC>(rk, o);
            vt[r][j] = load_vec_stream<KV, VEC>(rv, o);
          }
        }
      } else {
        // One buffer resource per tile, based at the tile's first row and
        // covering the rows before `end`: rows past it (the last tile's tail,
        // or a whole tile past the end) read as zero without a memory access,
        // and the lane offsets stay loop-invariant.
        const int64_t left = end - tb;
        const uint32_t nbytes = left <= 0 ? 0u : (uint32_t)(left < TR ? left : TR) * row_bytes;
        const auto rk = raw_rsrc(kh + tb * row_stride, nbytes);
        const auto rv = raw_rsrc(vh + tb * row_stride, nbytes);
        // All of the tile's K loads, then all of its V loads: pairing each K
        // load with the V load of the same row measured up to 3% slower here,
        // depending on where K and V sit relative to each other in HBM.
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int j = 0; j < NL; ++j)
            kt[r][j] = load_vec_stream<KV, VEC>(rk, loff[r] + (uint32_t)(j * RL * VEC * sizeof(KV)));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int j = 0; j < NL; ++j)
            vt[r][j] = load_vec_stream<KV, VEC>(rv, loff[r] + (uint32_t)(j * RL * VEC * sizeof(KV)));
      }
    };

    auto compute = [&](const V (&kt)[R][NL], const V (&vt)[R][NL], int64_t tb, const int (&pg)[R]) {
      float s[GH][R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int h = 0; h < GH; ++h) {
          float p = 0.0f;
#pragma unroll
          for (int j = 0; j < NL; ++j)
#pragma unroll
            for (int e = 0; e < VEC; ++e) p = fmaf(qr[h][j * VEC + e], to_f32(kt[r][j].v[e]), p);
          s[h][r] = row_sum<RL>(p);
        }
      }
      if constexpr (MODE == kPagedAny) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const bool ok = tb + r * NG + grp < end;
          const bool bad = pg[r] < 0 || (int64_t)pg[r] >= a.num_pages;
#pragma unroll
          for (int h = 0; h < GH; ++h) s[h][r] = ok ? (bad ? __builtin_nanf("") : s[h][r]) : -INFINITY;
        }
      } else {
        // Rows past `end` (last tile only) are masked; a row set whose page
        // entry is invalid poisons its rows with NaN (paged only).
        bool anybad = false;
        if constexpr (MODE == kPagedFast) {
#pragma unroll
          for (int r = 0; r < R; ++r) anybad |= pg[r] < 0 || (int64_t)pg[r] >= a.num_pages;
        }
        if (tb + TR > end || anybad) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const bool ok = tb + r * NG + grp < end;
            bool bad = false;
            if constexpr (MODE == kPagedFast) bad = pg[r] < 0 || (int64_t)pg[r] >= a.num_pages;
#pragma unroll
            for (int h = 0; h < GH; ++h) s[h][r] = ok ? (bad ? __builtin_nanf("") : s[h][r]) : -INFINITY;
          }
        }
      }
      // Running max per head. The accumulators and l are rescaled only when
      // some head's max moved somewhere in the wave (otherwise the factor is
      // exp2(0) = 1).
      float mn[GH];
      bool moved = false;
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        float mt = s[h][0];
#pragma unroll
        for (int r = 1; r < R; ++r) mt = fmaxf(mt, s[h][r]);
        mn[h] = fmaxf(m[h], mt);
        moved |= mn[h] != m[h];
      }
      if (__any(moved)) {
#pragma unroll
        for (int h = 0; h < GH; ++h) {
          const float al = fast_exp2(m[h] - ((mn[h] == -INFINITY) ? 0.0f : mn[h]));
          l[h] *= al;
#pragma unroll
          for (int d = 0; d < DPL; ++d) acc[h][d] *= al;
          m[h] = mn[h];
        }
      }
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        const float mu = (m[h] == -INFINITY) ? 0.0f : m[h];
        float p[R];
        float ls = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          p[r] = fast_exp2(s[h][r] - mu);
          ls += p[r];
        }
        l[h] += ls;
#pragma unroll
        for (int j = 0; j < NL; ++j)
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            float t = acc[h][j * VEC + e];
#pragma unroll
            for (int r = 0; r < R; ++r) t = fmaf(p[r], to_f32(vt[r][j].v[e]), t);
            acc[h][j * VEC + e] = t;
          }
      }
    };

    // Software pipeline: the loads of tile t+1 are issued before tile t's
    // arithmetic, so every wave keeps a tile of K/V in flight while it
    // computes. With paging, page indices run one tile further ahead (pc: this
    // tile, pn: next, pnn: the one after), so a table read never waits behind
    // K/V loads. The tile after the last one reads nothing (contiguous, fast
    // paged: its resources are empty) or re-reads row end-1 (a cache hit).
    V kA[R][NL], vA[R][NL], kB[R][NL], vB[R][NL];
    int pc[R], pn[R], pnn[R];
#pragma unroll
    for (int r = 0; r < R; ++r) pc[r] = pn[r] = pnn[r] = 0;
    if constexpr (MODE != kContig) {
      load_pages(pc, start);
      load_pages(pn, start + TR);
    }
    issue(kA, vA, start, pc);
    load_q();
    auto rotate = [&]() {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        pc[r] = pn[r];
        pn[r] = pnn[r];
      }
    };
    for (int64_t tb = start;;) {
      if constexpr (MODE != kContig) load_pages(pnn, tb + 2 * TR);
      issue(kB, vB, tb + TR, pn);
      __builtin_amdgcn_sched_barrier(0);
      compute(kA, vA, tb, pc);
      tb += TR;
      if (tb >= end) break;
      if constexpr (MODE != kContig) rotate();
      if constexpr (MODE != kContig) load_pages(pnn, tb + 2 * TR);
      issue(kA, vA, tb + TR, pn);
      __builtin_amdgcn_sched_barrier(0);
      compute(kB, vB, tb, pc);
      tb += TR;
      if (tb >= end) break;
      if constexpr (MODE != kContig) rotate();
    }
  };
  if constexpr (!PAGED) {
    run(std::integral_constant<int, kContig>{});
  } else {
    if (a.paged_fast)
      run(std::integral_constant<int, kPagedFast>{});
    else
      run(std::integral_constant<int, kPagedAny>{});
  }

  // Merge the row groups of each wave, then the waves through LDS.
  constexpr int GL = Sh::kGroupLanes;
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    const float mw = groups_max<GL>(m[h]);
    const float mwu = (mw == -INFINITY) ? 0.0f : mw;
    const float f = fast_exp2(m[h] - mwu);
    const float lw = groups_sum<GL>(l[h] * f);
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[h][d] = groups_sum<GL>(acc[h][d] * f);
    if (lane < GL) {
      const int hh = hs * GH + h;
      if (li == 0) {
        s_m[wave][hh] = mw;
        s_l[wave][hh] = lw;
      }
#pragma unroll
      for (int j = 0; j < NL; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) s_acc[wave][hh][j * RL * VEC + lane_col + e] = acc[h][j * VEC + e];
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
    float* dst = a.ws_acc + (ws0 + (int64_t)h * a.S) * D + e;
    if constexpr (FUSED)
      st_dev(dst, t);
    else
      *dst = t;
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
    if constexpr (FUSED) {
      st_dev(a.ws_m + ws0 + (int64_t)h * a.S, mb * kLn2);
      st_dev(a.ws_l + ws0 + (int64_t)h * a.S, lt);
    } else {
      a.ws_m[ws0 + (int64_t)h * a.S] = mb * kLn2;
      a.ws_l[ws0 + (int64_t)h * a.S] = lt;
    }
  }

  if constexpr (FUSED) {
    // Every thread waits until its device-scope stores have completed, then
    // the workgroup counts its partial. Counts are device-scope atomics, so
    // the workgroup that brings the count to n is the last of the group, and
    // every other partial was complete before its count: it reads them all.
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);
    const int n = (int)((L + (int64_t)a.chunk - 1) / a.chunk);
    uint32_t* cnt = a.counters + ((int64_t)b * Hkv + g) * merge_counter_words(a.S);
    // The epilogue's LDS is free again: it holds the merge's m and l values.
    merge_tree<D, Sh::kThreads, NW * D / 2>(a, G, b, h0, split, n, cnt, tid, &s_last, &s_acc[0][0][0]);
  }
}

// Lanes per KV row segment (RL), head slices (HS), rows per row group per
// tile (R) and the waves per SIMD the registers are held to (WPE), for each
// storage type, group size and width: the values measured best on MI355X.
// Wider groups carry more query and accumulator registers per lane; the
// 6-head f16 group splits its heads over two 16-lane slices of each row,
// which halves its per-lane reductions and exponentials.
constexpr bool sliced_variant(bool f16, int D, int G) { return f16 && D == 256 && G == 6; }

template <typename KV, int G, int D, bool PAGED>
struct Tune {
  static constexpr bool kWideGroup = G > 4;
  static constexpr bool kSliced = sliced_variant(std::is_same<KV, _Float16>::value, D, G);
  static constexpr int RL = kSliced ? 16 : ((D == 256 && kWideGroup) ? 32 : 16);
  static constexpr int HS = kSliced ? 2 : 1;
  // Rows per tile and row group.
  static constexpr int R =
      kSliced ? (PAGED ? 2 : 4) : (D == 128 ? 4 : ((D == 256 && kWideGroup && sizeof(KV) == 2) ? 4 : 2));
  // Rows for slices of at least kLongRowsFrom positions. The contiguous 4-head
  // width-256 layer takes four there: same-tensor A/B against two measured
  // 165.9 vs 168.8 us (f32, 131,072 positions) and 165.8 vs 170.5 us (f16,
  // 262,144), while slices of 64-960 positions lost 3-13% with four.
  static constexpr int RLong = (D == 256 && !PAGED && G == 4) ? 4 : R;
  // Two waves per SIMD where the query, accumulator and two in-flight tiles
  // fit 256 registers without spilling (checked against the compiler's
  // resource report), else one.
  static constexpr int WPE = kSliced ? 2 : ((sizeof(KV) == 2 && D == 128 && G <= 4) ? 2 : 1);
};

constexpr int kLongRowsFrom = 2048;

template <typename KV, int G, int D, bool PAGED, int R>
static sk_status_t launch_rows(const SplitLaunch& s, bool launch, const void** fn, int grid[3],
                               int* block) {
  const sk_desc_t& d = *s.d;
  using T = Tune<KV, G, D, PAGED>;
  auto kern = s.fused ? gqa_split_kernel<KV, G, D, PAGED, T::RL, R, T::HS, T::WPE, true>
                      : gqa_split_kernel<KV, G, D, PAGED, T::RL, R, T::HS, T::WPE, false>;
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
  if (d.layout == SK_KV_PAGED) {  // pools [pages][page_size][Hkv][D]
    a.stride_pos = (int64_t)d.num_kv_heads * D;
    a.stride_head = D;
  }
  a.num_pages = d.num_pages;
  a.q_dtype = d.q_dtype;
  a.Hq = d.num_q_heads;
  a.S = s.p->n_splits;
  a.chunk = s.p->chunk;
  a.cap = d.max_seq_len;
  a.page_shift = 0;  // indexed: pages of one row, the table names rows
  if (d.layout == SK_KV_PAGED) {
    while ((1 << a.page_shift) < d.page_size) ++a.page_shift;
  }
  a.max_pages = d.max_pages_per_seq;
  {
    using Sh = GqaShape<KV, D, T::RL, R, T::HS>;
    constexpr int NG = Sh::kGroups;
    constexpr int TR = NG * R;
    const int P = d.page_size;
    a.paged_fast = d.layout == SK_KV_PAGED && P % NG == 0 && TR % P == 0 && s.p->chunk % P == 0;
  }
  a.qscale = d.scale * kLog2e;
  a.counters = s.counters;
  a.out = s.out;
  a.lse = s.lse;
  hipLaunchKernelGGL(kern, gr, dim3(256), 0, s.stream, a);
  return SK_OK;
}

template <typename KV, int G, int D, bool PAGED>
static sk_status_t launch_variant(const SplitLaunch& s, bool launch, const void** fn, int grid[3],
                                  int* block) {
  using T = Tune<KV, G, D, PAGED>;
  if constexpr (T::RLong != T::R) {
    if (s.p->chunk >= kLongRowsFrom) return launch_rows<KV, G, D, PAGED, T::RLong>(s, launch, fn, grid, block);
  }
  return launch_rows<KV, G, D, PAGED, T::R>(s, launch, fn, grid, block);
}

template <typename KV, int G, int D>
static sk_status_t by_layout(const SplitLaunch& s, bool launch, const void** fn, int grid[3],
                             int* block) {
  if (s.d->layout != SK_KV_CONTIGUOUS) return launch_variant<KV, G, D, true>(s, launch, fn, grid, block);
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

int gqa_resident_blocks(const sk_desc_t&) {
  // One round of one workgroup per compute unit (measured best on MI355X for
  // every variant, the 6-head f16 one included: 0.737 of peak per call at
  // 64 splits against 0.710 at 128 for the 27B-like layer).
  return 1;
}

bool gqa_prefers_fewer_streams(const sk_desc_t& d) {
  // The memory-bound variants stream long slices faster from three quarters
  // of the compute units; the 6-head f16 kernel's VALU-heavy loop needs all.
  const int G = d.num_kv_heads > 0 ? d.num_q_heads / d.num_kv_heads : 0;
  return !sliced_variant(d.kv_dtype == SK_F16, d.head_dim_qk, G);
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
