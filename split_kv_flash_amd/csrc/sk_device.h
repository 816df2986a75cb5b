// Device-side helpers shared by the split and combine kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sk {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Storage types. bf16 is carried as its 16-bit pattern: the upper half of an
// IEEE binary32 word, so widening is a shift.
// ---------------------------------------------------------------------------
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float(((uint32_t)x.bits) << 16);
}

// A vector of N storage elements loaded with one instruction (4, 8 or 16 bytes).
template <typename T, int N>
struct alignas(sizeof(T) * N) Vec {
  T v[N];
};

template <typename T, int N>
__device__ __forceinline__ Vec<T, N> load_vec(const T* p) {
  return *reinterpret_cast<const Vec<T, N>*>(p);
}

// Raw buffer loads. A buffer resource carries a base address and a byte count;
// a load whose offset (lane offset plus immediate) lies at or past the count
// returns zero and touches no memory, which makes the rows past a split's end
// free to skip. Word 3 of a gfx9 resource: 32-bit data format, raw (unswizzled,
// no index stride) addressing.
constexpr int kRawBufferWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRawBufferWord3);
}
// Streaming loads for data read once (the K/V cache): the non-temporal cache
// policy (the nt bit, cache-policy operand 2 of the buffer load; the
// nontemporal builtin for a plain address). On MI355X a stream of 16-byte
// loads reads HBM at about 7.0 TB/s with it and about 6.2 TB/s without.
constexpr int kCacheStream = 2;
template <typename T, int N>
__device__ __forceinline__ Vec<T, N> load_vec_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  static_assert(sizeof(T) * N == 16 || sizeof(T) * N == 8, "buffer loads of 8 or 16 bytes");
  if constexpr (sizeof(T) * N == 16)
    return __builtin_bit_cast(Vec<T, N>, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCacheStream));
  else
    return __builtin_bit_cast(Vec<T, N>, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCacheStream));
}
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <typename T, int N>
__device__ __forceinline__ Vec<T, N> load_vec_stream(const T* p) {
  static_assert(sizeof(T) * N == 16 || sizeof(T) * N == 8, "loads of 8 or 16 bytes");
  if constexpr (sizeof(T) * N == 16)
    return __builtin_bit_cast(Vec<T, N>, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
  else
    return __builtin_bit_cast(Vec<T, N>, __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p)));
}

// ---------------------------------------------------------------------------
// Direct global-to-LDS tile loads and the explicit waits they need.
// ---------------------------------------------------------------------------
// One global_load_lds_dwordx4: each lane's 16 bytes at `g` land in LDS at
// lds_addr + 16*lane (lds_addr must be wave-uniform; it goes through M0).
// `nt` (wave-uniform) selects the non-temporal policy: used when the workgroup
// is the only reader of its rows, with which MI355X streams HBM measurably
// faster; when several workgroups re-read the same rows, the plain policy
// lets the later reads hit the caches.
// Issued as inline assembly so the compiler's wait-count tracking does not
// treat every later LDS read as possibly aliasing it (it would then wait for
// all loads in flight); the kernel waits for these loads explicitly. The
// kernels that use it do not otherwise use M0 (the asm declares it clobbered).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr, bool nt) {
  if (nt)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(g), "s"(lds_addr)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds_addr)
                 : "memory", "m0");
}
// The same load with a wave-uniform 64-bit base in scalar registers and a
// 32-bit per-lane byte offset (global address = base + offset).
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, uint32_t lds_addr, bool nt) {
  if (nt)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds_addr)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds_addr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt with vmcnt = VM (no wait on exp), lgkmcnt = 0: this wave's LDS
// writes are done and at most VM of its vector-memory operations remain.
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
}
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Cross-lane reductions. A row of 16 lanes is the unit DPP works in on gfx9:
// row_ror:8, row_ror:4 and two quad permutations give every lane the sum of
// its 16-lane row in four VALU operations.
// ---------------------------------------------------------------------------
// bound_ctrl set: every source lane these patterns name exists, and the flag
// lets the compiler fold the move into the consuming add (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]

__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kDppRowRor8>(x);
  x += dpp<kDppRowRor4>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppQuadXor1>(x);
  return x;
}

// Exchange with lane ^ 16 (within each 32-lane half): ds_swizzle in bit mode,
// and_mask 0x1F, xor_mask 0x10. Uses the LDS crossbar, no LDS memory.
__device__ __forceinline__ float xor16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}
// Exchange with lane ^ 32 through ds_bpermute (byte address of the source lane).
__device__ __forceinline__ float xor32(float x) {
  const int src = ((int)(threadIdx.x & 63) ^ 32) << 2;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(x)));
}

// The same combinations (a value with that of lane ^ 16, or of lane ^ 32)
// through gfx950's v_permlane16_swap / v_permlane32_swap: VALU instructions,
// where ds_swizzle and ds_bpermute take a round trip through the LDS
// crossbar. With both operands x, permlane16_swap leaves row 2k's values in
// rows 2k and 2k+1 of its first result and row 2k+1's in both rows of its
// second; permlane32_swap does the same with the two 32-lane halves. Every
// lane then combines its own value with its partner's, in one order or the
// other (max and + are commutative, so both lanes get the same bits).
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the RL consecutive lanes that hold one KV row (RL in {16, 32, 64});
// every lane of the group receives the total.
template <int RL>
__device__ __forceinline__ float row_sum(float x) {
  x = row16_sum(x);
  if constexpr (RL >= 32) x += xor16(x);
  if constexpr (RL >= 64) x += xor32(x);
  return x;
}

// Combine values across the row groups of a wave, GL lanes apart (lanes l,
// l+GL, l+2GL, ...).
template <int GL>
__device__ __forceinline__ float groups_max(float x) {
  if constexpr (GL <= 16) x = fmaxf(x, xor16(x));
  if constexpr (GL <= 32) x = fmaxf(x, xor32(x));
  return x;
}
template <int GL>
__device__ __forceinline__ float groups_sum(float x) {
  if constexpr (GL <= 16) x += xor16(x);
  if constexpr (GL <= 32) x += xor32(x);
  return x;
}

// exp2 as the single hardware instruction v_exp_f32 (compiler builtin). Results
// below the normal range may flush to zero; every use here is exp2 of a
// non-positive difference, where such terms are below 2^-126 of the largest.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace sk
