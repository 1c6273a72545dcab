// LDS tile helpers shared by the backward kernels (fa_bwd.hip, fa_bwd_dq.hip):
// the XOR-swizzled bf16 tile layout, direct global->LDS tile loads, the
// transposed-read pair, and the XCD-aware work-id remap.
#pragma once

#include "fa_device.h"

namespace fa {
namespace bwd {

// 16-byte chunk swizzle of a [rows][D] bf16 tile that is conflict-free both for
// 16-lane row reads (16 consecutive rows, one chunk) and for transposed reads
// (4 aligned consecutive rows x 64 bytes).
template <int D>
__device__ __forceinline__ int swz2(int row) {
  return D >= 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int toff(int row, int col) {
  return row * D + ((((col >> 3) ^ swz2<D>(row))) << 3) + (col & 7);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// Direct global->LDS loads of a [ROWS x D] bf16 tile (row stride rs elements,
// rows clamped to N-1) by
// THREADS threads into the layout of toff<D> (TR) or of the forward's K tile.
// Thread `tid` fills the 16-byte LDS chunks n * THREADS + tid; the source chunk
// is chosen so that LDS holds the swizzled layout.
template <int D, int ROWS, int THREADS, bool TR>
__device__ __forceinline__ void load_tile_async(uint16_t* lds_tile, const uint16_t* head, long long rs, int r0, int N,
                                                int tid) {
  constexpr int CH = D / 8;
  const int w = tid >> 6;
#pragma unroll
  for (int n = 0; n < (ROWS * CH) / THREADS; ++n) {
    const int e = n * THREADS + tid;
    const int r = e / CH, p = e % CH;
    const int c = p ^ (TR ? swz2<D>(r) : swz_k<D>(r));
    const int row = min(r0 + r, N - 1);
    const uint16_t* src = head + (uint64_t)(uint32_t)row * (uint32_t)rs + c * 8;  // rs < 2^31
    lds_dma16(lds_tile + (n * THREADS + w * 64) * 8, src);  // lane l lands at +16 l bytes
  }
}

// L (lanes 0..31) and D (lanes 32..63) of 32 rows, by one wave.
__device__ __forceinline__ void load_ld_async(float* lds_ld, const float* lse_h, const float* d_h, int q0, int N,
                                              int lane) {
  const int r = min(q0 + (lane & 31), N - 1);
  const float* src = (lane < 32) ? lse_h + r : d_h + r;
  lds_dma4(lds_ld, src);
}

__device__ __forceinline__ void wait_loads_and_sync() {
  wait_vmem_all();
  __syncthreads();
}

__device__ __forceinline__ u32x4 tr_pair(const uint16_t* p0, const uint16_t* p1) {
  const i16x4 t0 = lds_read_tr16(p0);
  const i16x4 t1 = lds_read_tr16(p1);
  return u32x4{__builtin_bit_cast(u32x2, t0)[0], __builtin_bit_cast(u32x2, t0)[1],
               __builtin_bit_cast(u32x2, t1)[0], __builtin_bit_cast(u32x2, t1)[1]};
}

// Work-id remap: blocks are dispatched round-robin over the 8 XCDs; give each
// XCD a contiguous range of work ids so that one head's blocks share its L2.
__device__ __forceinline__ int xcd_work_id(int total) {
  const int b = (int)blockIdx.x;
  return (total & 7) == 0 ? (b & 7) * (total >> 3) + (b >> 3) : b;
}

}  // namespace bwd
}  // namespace fa
