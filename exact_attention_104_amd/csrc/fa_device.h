// Device-side helpers shared by the gfx950 attention kernels: vector types,
// MFMA wrappers, LDS transpose reads, lane exchange, bf16/fp8 conversion.
//
// Register layouts used throughout (measured on gfx950 with a layout probe):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[m = l%32][k = 8*(l/32) + j], j = 0..7 (one bf16x8)
//     B: lane l holds B[k = 8*(l/32) + j][n = l%32]
//     D: lane l, element i holds D[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32]
//   ds_read_b64_tr_b16: in each group of 16 lanes, lane i supplies the address
//     of 4 consecutive 16-bit values; the group reads a 4 x 16 block whose row r
//     comes from lanes 4r..4r+3, and lane i receives column i (rows 0..3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// e4m3 x e4m3 -> fp32, 32x32x64; A/B: 32 bytes per lane. Any k permutation that
// is the same for A and B gives the same product, so only the pairing matters.
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(FA_LDS_PTR(i16x4, p));
}

__device__ __forceinline__ i32x2 lds_read_tr8(const void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(FA_LDS_PTR(i32x2, p));
}

// Value of x held by lane l ^ 32 (the other half of the wave), via v_permlane32_swap.
__device__ __forceinline__ float other_half(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // r[0] = (lanes <32: own, >=32: lane-32), r[1] = (lanes <32: lane+32, >=32: own)
  const bool upper = (threadIdx.x & 32) != 0;
  return __builtin_bit_cast(float, upper ? r[0] : r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Direct global->LDS loads (global_load_lds_dword[x4]): lane l's 4 or 16 bytes
// from `src` land at lds_wave_base + size * l; lds_wave_base must be the same
// for the whole wave. Issued through inline asm on purpose: the compiler then
// does not track them, so it does not hold every LDS read of the other buffer
// behind a wait for these loads (it cannot tell the buffers apart once the
// buffer is chosen at run time). Every caller waits explicitly with
// wait_vmem_all() and a barrier before reading what they wrote. M0 (the LDS
// base operand) is saved and restored around the load: M0 is a reserved
// register, which a clobber list cannot name (the compiler warns that such a
// clobber is not honoured), and the "s" / "=&s" operands come from the
// allocatable SGPRs, which exclude M0. The kernels here never use M0
// otherwise (checked in the generated code).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// LDS reads at a byte address (lds_addr of a __shared__ object plus an offset).
__device__ __forceinline__ u32x4 lds_load16(uint32_t a) {
  return *(const __attribute__((address_space(3))) u32x4*)(size_t)a;
}
__device__ __forceinline__ i16x4 lds_read_tr16_at(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(size_t)a);
}
__device__ __forceinline__ void lds_dma16(void* lds_wave_base, const void* src) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(m0) : "memory");
}
__device__ __forceinline__ void lds_dma4(void* lds_wave_base, const void* src) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(m0) : "memory");
}
// As lds_dma16, with the global address formed by the load itself from a
// wave-uniform 64-bit base (SGPRs) plus this lane's 32-bit byte offset, so
// that no per-lane 64-bit address arithmetic precedes it. lds_wave_addr is the
// wave's LDS byte address (lane l lands at +16 l).
__device__ __forceinline__ void lds_dma16_sbase(uint32_t lds_wave_addr, const void* sbase, uint32_t voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_wave_addr);
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(m0) : "memory");
}
// vmcnt(0), other counters untouched: every vector memory operation of this
// wave, including the loads above, has completed.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Two fp32 -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) { return __builtin_bit_cast(bf16x8, u); }

// Maximum of the 32 values of two accumulator blocks as a tree of three-input
// maxima (v_max3_f32: 16 instructions where pairwise maxima need 31).
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
__device__ __forceinline__ float max_of_32(const f32x16& a, const f32x16& b) {
  float t[11];
#pragma unroll
  for (int i = 0; i < 5; ++i) t[i] = max3f(a[3 * i], a[3 * i + 1], a[3 * i + 2]);
  t[5] = max3f(a[15], b[0], b[1]);
#pragma unroll
  for (int i = 0; i < 4; ++i) t[6 + i] = max3f(b[2 + 3 * i], b[3 + 3 * i], b[4 + 3 * i]);
  t[10] = fmaxf(b[14], b[15]);
  return max3f(max3f(t[0], t[1], t[2]), max3f(t[3], t[4], t[5]), max3f(t[6], t[7], max3f(t[8], t[9], t[10])));
}

// XOR swizzles of 16-byte chunks inside an LDS row of a [rows][D] bf16 tile
// (the banks repeat every 256 bytes, i.e. every 16 chunks; rows of D >= 128
// span whole bank periods, rows of D = 64 half of one).
// K tile: read as 32 rows x one chunk per 16 lanes -> chunk ^ f(row) spreads
// 16 consecutive rows over 16 distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D >= 128 ? (row & 15) : ((row >> 1) & 7);
}
// V tile: read transposed, 4 rows x 4 chunks per 16-lane group.
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D >= 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

}  // namespace fa
