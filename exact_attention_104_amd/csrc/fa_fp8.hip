// fp8 (OCP e4m3) input path for gfx950: block quantiser with optional
// random-sign Hadamard rotation, and the e4m3 MFMA forward.
//
// [LIB] "FA3 — the Hopper moment", pillar 3, and [LIN] "FA3 (2024)", idea 3:
// e4m3 attention inputs, one scale per tile of rows instead of per tensor
// (block quantisation), and an orthogonal random Hadamard-based rotation that
// spreads outliers before quantising ("incoherent processing").
//
// Quantiser: one workgroup per (batch, head, 128-row block). Rotation along d
// (d = 128): x' = H_128 (s o x) / sqrt(128) in fp32 with butterflies at
// strides 1, 2, 4 inside a lane's 8 values and 8, 16, 32, 64 across lanes;
// then scale = fl32(amax / 448), codes = e4m3(clamp(fl32(x' * fl32(448 / amax)))).
//
// Forward: as the bf16 forward (split-Q waves of 32 query rows, S^T =
// K Q^T so lanes own queries, online exp2 softmax with threshold rescale,
// direct global->LDS double-buffered tiles, one barrier per tile), on
// v_mfma_f32_32x32x64 e4m3 products with fp32 accumulation. Block scales are
// applied after the products: S = sq * sk * (Q8 K8^T). P is quantised to e4m3
// for the P V product with the V block scale folded in: p' = p * sv_j * R with
// R = 32 / max_j sv_j, where p is taken against a running max that is moved
// only when some row's maximum exceeds it by more than 3 (log2 units), so
// p' <= 256; the row sum keeps the unscaled p, and the final division removes R.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

// 4 floats -> 4 e4m3 bytes (RNE); the inputs are already clamped to +-448.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

// Block quantiser without rotation: one workgroup per 128-row block, 8
// values per lane, the block's amax reduced across the workgroup, then the
// codes (fl32 amax / 448 the scale, x * fl32(448 / amax) clamped and rounded
// to e4m3).
template <int D>
__global__ void __launch_bounds__(256)
quant_kernel(const uint16_t* __restrict__ X, uint8_t* __restrict__ X8, float* __restrict__ scales, int N, int nb) {
  constexpr int LPR = D / 8;         // lanes per row, 8 values each
  constexpr int RPP = 256 / LPR;     // rows per pass
  constexpr int PASSES = 128 / RPP;  // passes over the 128-row block
  __shared__ float wmax[4];

  const int blk = (int)(blockIdx.x % nb);
  const size_t bh = blockIdx.x / nb;
  const int tid = threadIdx.x, c = tid % LPR, rr = tid / LPR;
  const size_t base = bh * (size_t)N * D;

  float x[PASSES][8];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = blk * 128 + p * RPP + rr;
    u32x4 u = {0, 0, 0, 0};
    if (row < N) u = *(const u32x4*)(X + base + (size_t)row * D + c * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[p][2 * j] = __builtin_bit_cast(float, u[j] << 16);
      x[p][2 * j + 1] = __builtin_bit_cast(float, u[j] & 0xffff0000u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[p][i]));  // rows past N hold zeros
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const bool zero = amax == 0.f;
  const float scale = zero ? 1.f : __fdiv_rn(amax, 448.f);
  const float factor = zero ? 1.f : __fdiv_rn(448.f, amax);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = blk * 128 + p * RPP + rr;
    if (row < N) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = fminf(fmaxf(x[p][i] * factor, -448.f), 448.f);
      const u32x2 out = {pack_e4m3x4(v[0], v[1], v[2], v[3]), pack_e4m3x4(v[4], v[5], v[6], v[7])};
      *(u32x2*)(X8 + base + (size_t)row * D + c * 8) = out;
    }
  }
  if (tid == 0) scales[bh * nb + blk] = scale;
}

// Block quantiser with the random-sign Hadamard rotation (d = 128): x' =
// H_128 (s o x) / sqrt(128) in fp32, as radix-2 butterflies (a, b) -> (a + b,
// a - b) at strides 1, 2, 4, ..., 64 in that order, then the multiply by
// fl32(1 / sqrt(128)). Four lanes per row: lane 4r + e holds columns 32 e ..
// 32 e + 31 of row r of the block, so strides 1 .. 16 pair values inside the
// lane, and strides 32 and 64 pair lanes e ^ 1 and e ^ 2 of the same quad
// (DPP quad permutations). In each cross-lane stage the lower lane keeps the
// sum and the upper the difference, its partner's value minus its own, as
// fma(own, +-1, partner): own * (+-1) is exact, so each is the one rounding of
// the sum or the difference (a - b itself: b - a negated would turn an exact
// zero into -0). So every value takes the same roundings as in the stated
// order. 32 values per lane keep the kernel near 64 VGPRs, eight waves per
// SIMD: its loads, butterflies and stores then overlap across more
// workgroups than with 64 values per lane.
__global__ void __launch_bounds__(512)
quant_rot_kernel(const uint16_t* __restrict__ X, uint8_t* __restrict__ X8, float* __restrict__ scales,
                 const int8_t* __restrict__ signs, int N, int nb) {
  constexpr int D = 128;
  __shared__ float wmax[8];

  const int blk = (int)(blockIdx.x % nb);
  const size_t bh = blockIdx.x / nb;
  const int tid = threadIdx.x, e = tid & 3, row = blk * 128 + (tid >> 2);
  const size_t base = bh * (size_t)N * D;
  u32x4 u[4];
  const uint16_t* src = X + base + (size_t)row * D + 32 * e;
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = u32x4{0, 0, 0, 0};
  if (row < N) {
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = *(const u32x4*)(src + 8 * i);
  }
  // the random signs of this lane's 32 columns, loaded after the values (one
  // wait covers both) and by every lane: a table in LDS behind a barrier
  // held each workgroup back by the latency of one wave's load
  const u32x4 sg[2] = {*(const u32x4*)(signs + 32 * e), *(const u32x4*)(signs + 32 * e + 16)};
  float x[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // negation is a sign-bit flip: the sign bits (bit 7) of the pair's two
      // int8 signs, moved to bits 15 and 31 of the packed bf16 pair
      const uint32_t sw = sg[i >> 1][2 * (i & 1) + (j >> 1)];
      const uint32_t m = (j & 1) ? (((sw >> 8) & 0x8000u) | (sw & 0x80000000u))
                                 : (((sw << 8) & 0x8000u) | ((sw << 16) & 0x80000000u));
      const uint32_t w = u[i][j] ^ m;
      x[8 * i + 2 * j] = __builtin_bit_cast(float, w << 16);
      x[8 * i + 2 * j + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
    }
  }
#pragma unroll
  for (int h = 1; h < 32; h *= 2)
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
  // stride 32: lanes e, e ^ 1 (quad_perm [1,0,3,2]); stride 64: lanes e, e ^ 2
  // (quad_perm [2,3,0,1])
  const float s32 = (e & 1) ? -1.f : 1.f, s64 = (e & 2) ? -1.f : 1.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float p = __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x[i]), 0xB1, 0xF, 0xF, false));
    x[i] = __builtin_fmaf(x[i], s32, p);
  }
  const float inv_sqrt128 = 0x1.6a09e6p-4f;  // fl32(1 / sqrt(128))
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float p = __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x[i]), 0x4E, 0xF, 0xF, false));
    x[i] = __builtin_fmaf(x[i], s64, p) * inv_sqrt128;
    amax = fmaxf(amax, fabsf(x[i]));  // rows past N hold zeros
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])),
               fmaxf(fmaxf(wmax[4], wmax[5]), fmaxf(wmax[6], wmax[7])));
  const bool zero = amax == 0.f;
  const float scale = zero ? 1.f : __fdiv_rn(amax, 448.f);
  const float factor = zero ? 1.f : __fdiv_rn(448.f, amax);
  if (row < N) {
    uint8_t* dst = X8 + base + (size_t)row * D + 32 * e;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float v[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) v[t] = fminf(fmaxf(x[16 * i + t] * factor, -448.f), 448.f);
      const u32x4 out = {pack_e4m3x4(v[0], v[1], v[2], v[3]), pack_e4m3x4(v[4], v[5], v[6], v[7]),
                         pack_e4m3x4(v[8], v[9], v[10], v[11]), pack_e4m3x4(v[12], v[13], v[14], v[15])};
      *(u32x4*)(dst + 16 * i) = out;
    }
  }
  if (tid == 0) scales[bh * nb + blk] = scale;
}

// 16-byte chunk swizzle of a [64 keys][D bytes] e4m3 tile: conflict-free for
// 16-lane row reads (16 consecutive rows, one chunk: the 8 row pairs take 8
// distinct chunks) and for the transposed byte reads of V, which at d = 128
// take two adjacent chunks of rows {0, 2, 8, 10} (+ const) in one pass: with
// bits 0 and 1 of (row >> 1) swapped those rows map to disjoint chunk pairs
// (plain (row >> 1) & 7 pairs rows 0 / 2 and 8 / 10 on the same banks).
template <int D>
__device__ __forceinline__ int swz8(int row) {
  const int x = (row >> 1) & 7;
  return D == 128 ? (((x & 1) << 1) | ((x >> 1) & 1) | (x & 4)) : ((row >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int toff8(int row, int byte) {
  return row * D + ((((byte >> 4) ^ swz8<D>(row))) << 4) + (byte & 15);
}

namespace {

// Workgroups of NW wavefronts (8: 256 query rows, one per CU; 4: 128 rows,
// two per CU, which balance short and causal rows better).
constexpr int kF8QW = 32;             // query rows per wavefront
constexpr int kF8BC = 64;             // keys per tile
constexpr float kF8Lazy = 3.f;        // rescale threshold (log2 units) of the running max

// Direct global->LDS loads of one [64 x D] e4m3 tile into the swizzled layout
// of toff8 (rows past the end read row N-1; they are masked or meet P = 0),
// 16-byte chunk i by thread i mod (64 NW), whole wavefronts at a time. A
// full tile is loaded from its first row (a uniform base) plus each lane's
// byte offset inside the tile, formed once (tile8_offsets): no per-lane
// address arithmetic per tile. The ragged last tile clamps each row. The
// causal instances use this (FAST; 2.9% faster at N = 8192, d = 128); without
// a mask it measured 1-2% slower, and those keep the per-row form.
template <int D, int NW>
struct Tile8Lanes {
  static constexpr int kN = (kF8BC * (D / 16) + NW * 64 - 1) / (NW * 64);
  uint32_t off[kN];
};
template <int D, int NW>
__device__ __forceinline__ Tile8Lanes<D, NW> tile8_offsets(int tid) {
  constexpr int CHB = D / 16;
  Tile8Lanes<D, NW> t;
#pragma unroll
  for (int n = 0; n < Tile8Lanes<D, NW>::kN; ++n) {
    const int i = n * NW * 64 + tid;
    const int r = i / CHB, p = i % CHB;
    t.off[n] = (uint32_t)(r * D + (p ^ swz8<D>(r)) * 16);
  }
  return t;
}
template <int D, int NW, bool FAST>
__device__ __forceinline__ void load_tile8_async(uint8_t* lds_tile, const uint8_t* head, int k0, int N, int tid,
                                                 const Tile8Lanes<D, NW>& tl) {
  constexpr int CHB = D / 16;
  constexpr int CHUNKS = kF8BC * CHB;  // 512 (D = 128) or 256 (D = 64)
  constexpr int T = NW * 64;
  if (FAST && k0 + kF8BC <= N) {
    const uint8_t* base = head + (size_t)k0 * D;
    const uint32_t lds = lds_addr(lds_tile) + (uint32_t)__builtin_amdgcn_readfirstlane(tid >> 6) * 1024u;
#pragma unroll
    for (int n = 0; n < Tile8Lanes<D, NW>::kN; ++n) {
      if (CHUNKS - n * T < T && n * T + tid >= CHUNKS) return;  // whole wavefronts
      lds_dma16_sbase(lds + n * T * 16, base, tl.off[n]);
    }
    return;
  }
#pragma unroll
  for (int i0 = 0; i0 < CHUNKS; i0 += T) {
    const int i = i0 + tid;
    if (CHUNKS - i0 < T && i >= CHUNKS) return;  // whole wavefronts (CHUNKS is a multiple of 64)
    const int r = i / CHB, p = i % CHB;
    const int c = p ^ swz8<D>(r);
    const int row = min(k0 + r, N - 1);
    const uint8_t* src = head + (size_t)row * D + c * 16;
    lds_dma16(lds_tile + (i - (tid & 63)) * 16, src);  // lane l lands at +16 l bytes
  }
}

}  // namespace

// 2^x on the FMA units, the software exponential of [LIB] "FA4 — Blackwell's
// asymmetry" (idea 1) and [LIN] "FA4 (2026)" (change 2), for x <= 8: x = n + f
// with n = rint(x) (adding 1.5 * 2^23 leaves n in the low mantissa bits) and
// f in [-1/2, 1/2]; 2^f by a degree-4 polynomial whose coefficients are a
// weighted least-squares fit of 2^f on [-1/2, 1/2] (relative error at most
// 2.7e-6 over x in [-125.5, 8]); 2^n added into the exponent field. Between
// -126 and -125.5 that sum leaves the normal range (values below 2^-125,
// nothing next to a row's largest p, which is at least 1); below -126
// (masked scores are -inf) it returns 0. Nine vector
// instructions per value against one v_exp_f32, so it pays only where the
// transcendental unit binds; here it does not (measured, see fa_fwd_fp8_ext).
__device__ __forceinline__ float soft_exp2(float x) {
  const float xc = fmaxf(x, -126.f);
  const float t = xc + 12582912.f;
  const float f = xc - (t - 12582912.f);
  float p = __builtin_fmaf(0.009560510516166687f, f, 0.05591703951358795f);
  p = __builtin_fmaf(p, f, 0.24024981260299683f);
  p = __builtin_fmaf(p, f, 0.6931219696998596f);
  p = __builtin_fmaf(p, f, 0.9999991655349731f);
  const float r = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, p) + (__builtin_bit_cast(uint32_t, t) << 23));
  return x < -126.f ? 0.f : r;
}

// XCD (causal d = 128, chosen by the host when every round holds whole heads): the
// grid holds one workgroup per resident slot, and XCD x (workgroup j runs on
// XCD j % 8) takes heads x, x + 8, ..., all Q-blocks of a head per round,
// the Q-block order reversed on odd rounds, as in the bf16 forward.
// Otherwise one workgroup per (head, Q-block): the loop below runs once.
// SEXP: which exponentials of the softmax run as soft_exp2 (0 none, 1 one
// value in four, 2 all); d = 128 only.
template <int D, bool CAUSAL, int NW, bool XCD = false, int SEXP = 0>
__global__ void __launch_bounds__(NW * 64, NW == 4 ? 2 : 1)
fwd_fp8_kernel(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8, const uint8_t* __restrict__ V8,
               const float* __restrict__ QS, const float* __restrict__ KSc, const float* __restrict__ VS,
               uint16_t* __restrict__ Og, float* __restrict__ LSEg, int BH, int N, int nqb, int nsb,
               float scale_log2) {
  constexpr int KS = D / 64;      // k-steps of the S product (64 bytes each)
  constexpr int DB = D / 32;      // 32-row d blocks of O^T
  constexpr int TILE = kF8BC * D; // bytes of one K or V tile

  __shared__ __attribute__((aligned(16))) uint8_t sK0[TILE];
  __shared__ __attribute__((aligned(16))) uint8_t sK1[TILE];
  __shared__ __attribute__((aligned(16))) uint8_t sV0[TILE];
  __shared__ __attribute__((aligned(16))) uint8_t sV1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int g = lane >> 4, i16 = lane & 15;

  const int total = nqb * BH;
  const int xj = (int)blockIdx.x, xx = xj & 7, xGx = (int)gridDim.x >> 3;
  const int xitems = (BH >> 3) * nqb;  // items of this XCD (XCD dealing)
  for (int xu = xj >> 3, xk = 0;; xu += xGx, ++xk) {
  int wid;
  if constexpr (XCD) {
    if (xu >= xitems) break;
    const int qb = (xk & 1) ? nqb - 1 - xu % nqb : xu % nqb;
    wid = ((xu / nqb) * 8 + xx) * nqb + qb;  // Q-block nqb - 1 - qb (causal)
  } else {
    wid = (int)blockIdx.x;
    if ((total & 7) == 0) wid = (wid & 7) * (total >> 3) + (wid >> 3);
  }
  const int bh = wid / nqb;
  const int qblk = CAUSAL ? nqb - 1 - (wid % nqb) : (wid % nqb);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint8_t* Kh = K8 + head;
  const uint8_t* Vh = V8 + head;
  constexpr int BR = NW * kF8QW;  // query rows per workgroup
  const int qw0 = qblk * BR + w * kF8QW;
  const int qrow = qw0 + l32;
  const float* qs_h = QS + (size_t)bh * nsb;
  const float* ks_h = KSc + (size_t)bh * nsb;
  const float* vs_h = VS + (size_t)bh * nsb;

  const int kend = CAUSAL ? min(N, qblk * BR + BR) : N;
  const int ntiles = (kend + kF8BC - 1) / kF8BC;
  const int wlast = CAUSAL ? min(ntiles - 1, (qw0 + kF8QW - 1) / kF8BC) : ntiles - 1;

  Tile8Lanes<D, NW> lanes8;  // used by the causal instances only
  if constexpr (CAUSAL) lanes8 = tile8_offsets<D, NW>(tid);
  load_tile8_async<D, NW, CAUSAL>(sK0, Kh, 0, N, tid, lanes8);
  load_tile8_async<D, NW, CAUSAL>(sV0, Vh, 0, N, tid, lanes8);

  // R = 32 / max_j sv_j over the head: with the running max at most kF8Lazy
  // below a row's true maximum, every quantised p' = p sv_j R <= 32 * 8 = 256
  float svm = 0.f;
  for (int i = lane; i < nsb; i += 64) svm = fmaxf(svm, vs_h[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) svm = fmaxf(svm, __shfl_xor(svm, o));
  const float R = 32.f / svm;
  const float sq = qs_h[min(qw0, N - 1) / 128];  // the wave's 32 rows share one scale block

  // Q8 as the B operand of S^T = K Q^T: lane holds Q8[q][64 ks + 32 hi .. +31]
  i32x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    i32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (qrow < N) {
      const uint8_t* p = Q8 + head + (size_t)qrow * D + ks * 64 + hi * 32;
      a = *(const i32x4*)p;
      b = *(const i32x4*)(p + 16);
    }
    qf[ks] = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  auto tile = [&](int t, const uint8_t* sK, const uint8_t* sV, uint8_t* nK, uint8_t* nV,
                  auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int k0 = t * kF8BC;
    const float sk = ks_h[k0 / 128], sv = vs_h[k0 / 128];
    const float ct = sq * sk * scale_log2;  // exp2-domain scale of this tile's scores
    const float ft = sv * R;                // factor folded into p' for the P V product
    const float tt = __log2f(ft);
    // 1 / ft only rescales the row sum back to p: the hardware reciprocal
    // (within 1 ulp) instead of an IEEE division (about ten instructions)
    const float inv_ft = __builtin_amdgcn_rcpf(ft);

    // ---- S^T = K8 Q8^T (fp32 accumulation; unscaled)
    f32x16 s[2];
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r = kb * 32 + l32;
        const i32x4 a0 = *(const i32x4*)(sK + toff8<D>(r, ks * 64 + hi * 32));
        const i32x4 a1 = *(const i32x4*)(sK + toff8<D>(r, ks * 64 + hi * 32 + 16));
        const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        s[kb] = mfma_fp8_32x32x64(a, qf[ks], s[kb]);
      }
    }

    // ---- online softmax; p' = p * ft quantised to e4m3 (bytes in accumulator order)
    if constexpr (MASKED) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + 8 * (i / 4) + 4 * hi + (i % 4);
          if ((CAUSAL && key > qrow) || key >= N) s[kb][i] = -INFINITY;
        }
    }
    float mx = max_of_32(s[0], s[1]);
    mx = fmaxf(mx, other_half(mx)) * ct;
    // lazy rescale: the running max moves only once some row's tile maximum
    // exceeds it by more than kF8Lazy (log2 units)
    if (__any(mx > m + kF8Lazy)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      m = m_new;
    }
    const float off = tt - m;
    float rs = 0.f;
    i32x8 pb;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = __builtin_fmaf(s[kb][4 * q4 + e], ct, off);
          const bool sw = SEXP == 2 || (SEXP == 1 && e == 0);
          p[e] = sw ? soft_exp2(x) : fast_exp2(x);
          rs += p[e];
        }
        // no clamp needed: m >= this tile's scaled maximum - kF8Lazy, so
        // p' <= 8 ft <= 256 (up to rounding), inside the e4m3 range of +-448
        pb[kb * 4 + q4] = (int)pack_e4m3x4(p[0], p[1], p[2], p[3]);
      }
    }
    l += rs * inv_ft;

    // ---- O^T += V8^T P8^T: one 64-key MFMA per 32-row d block
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int byte = db * 32 + 16 * (g & 1) + 8 * (i16 & 1);
      const int c = i16 >> 1;  // row of the 8 x 16 byte block this lane addresses
      i32x8 a;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = 32 * (rr >> 1) + 8 * (2 * (rr & 1) + (c >> 2)) + 4 * hi + (c & 3);
        const i32x2 t2 = lds_read_tr8(sV + toff8<D>(key, byte));
        a[2 * rr] = t2[0];
        a[2 * rr + 1] = t2[1];
      }
      acc[db] = mfma_fp8_32x32x64(a, pb, acc[db]);
    }
  };

  // One tile per step: wait for its loads, barrier, issue the next tile's
  // loads, then compute. A tile needs the mask when it crosses the causal
  // diagonal of the wave's rows or runs past N; without causality only the
  // last tile can, so it is peeled off the unrolled loop.
  auto step = [&](int t, const uint8_t* sK, const uint8_t* sV, uint8_t* nK, uint8_t* nV,
                  auto last_tag) __attribute__((always_inline)) {
    constexpr bool LAST = decltype(last_tag)::value;
    wait_vmem_all();
    __syncthreads();  // tile t landed; every wave finished tile t-1
    if (!LAST && t + 1 < ntiles) {
      load_tile8_async<D, NW, CAUSAL>(nK, Kh, (t + 1) * kF8BC, N, tid, lanes8);
      load_tile8_async<D, NW, CAUSAL>(nV, Vh, (t + 1) * kF8BC, N, tid, lanes8);
    }
    if (t > wlast) return;
    const int k0 = t * kF8BC;
    if constexpr (CAUSAL) {
      if (k0 + kF8BC - 1 > qw0 || k0 + kF8BC > N)
        tile(t, sK, sV, nK, nV, std::true_type{});
      else
        tile(t, sK, sV, nK, nV, std::false_type{});
    } else {
      tile(t, sK, sV, nK, nV, std::integral_constant<bool, LAST>{});
    }
  };

  int t = 0;
  for (; t + 2 < ntiles; t += 2) {
    step(t, sK0, sV0, sK1, sV1, std::false_type{});
    step(t + 1, sK1, sV1, sK0, sV0, std::false_type{});
  }
  if (t + 1 < ntiles) {
    step(t, sK0, sV0, sK1, sV1, std::false_type{});
    step(t + 1, sK1, sV1, sK0, sV0, std::true_type{});
  } else {
    step(t, sK0, sV0, sK1, sV1, std::true_type{});
  }

  const float lt = l + other_half(l);
  const float inv = 1.0f / (lt * R);
  if (qrow < N) {
    uint16_t* orow = Og + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hi;
        const u32x2 pk = {pack_bf16x2(acc[db][4 * g4 + 0] * inv, acc[db][4 * g4 + 1] * inv),
                          pack_bf16x2(acc[db][4 * g4 + 2] * inv, acc[db][4 * g4 + 3] * inv)};
        *(u32x2*)(orow + d) = pk;
      }
    if (hi == 0) LSEg[(size_t)bh * N + qrow] = (m + __log2f(lt)) * kLn2;
  }
  if constexpr (!XCD) break;
  __syncthreads();  // every wave is done with the LDS tiles before the next item's loads
  }  // items
}

// Workgroups of fwd_fp8_kernel<D, true, NW, true, SEXP> resident on the
// current device at once, looked up once per device and instance.
template <int D, int NW, int SEXP>
static int f8_resident_slots() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fwd_fp8_kernel<D, true, NW, true, SEXP>, NW * 64, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    v = per_cu * cus;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

int launch_quant_fp8(const QuantArgs& a) {
  const int nb = (a.N + 127) / 128;
  const dim3 grid((unsigned)(a.B * a.H * nb)), block(256);
  hipStream_t st = (hipStream_t)a.stream;
  if (a.d == 128) {
    if (a.signs)
      hipLaunchKernelGGL(quant_rot_kernel, grid, dim3(512), 0, st, a.x, a.x8, a.scales, a.signs, a.N, nb);
    else
      hipLaunchKernelGGL((quant_kernel<128>), grid, block, 0, st, a.x, a.x8, a.scales, a.N, nb);
  } else {
    hipLaunchKernelGGL((quant_kernel<64>), grid, block, 0, st, a.x, a.x8, a.scales, a.N, nb);
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <int D, bool CAUSAL, int NW, int SEXP>
static int launch_f8_nw(const Fp8FwdArgs& a) {
  constexpr int BR = NW * kF8QW;
  const int nqb = (a.N + BR - 1) / BR, nsb = (a.N + 127) / 128;
  const int BH = a.B * a.H;
  const int blocks = nqb * BH;
  // Causal d = 128: persistent (2.7% faster at N = 8192, 15-18% at 1024 -
  // 2048). Not at d = 64, where the loop's registers cost a workgroup per CU.
  if constexpr (CAUSAL && D == 128) {
    const int slots = f8_resident_slots<D, NW, SEXP>();
    const int g = slots > 0 ? std::min(blocks, slots) : blocks;
    if (g % 8 == 0 && BH % 8 == 0 && (g / 8) % nqb == 0) {
      hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, NW, true, SEXP>), dim3((unsigned)g), dim3(NW * 64), 0,
                         (hipStream_t)a.stream, a.q8, a.k8, a.v8, a.qs, a.ks, a.vs, a.o, a.lse, BH, a.N, nqb,
                         nsb, a.scale * kLog2e);
      return hipGetLastError() == hipSuccess ? 0 : 1;
    }
  }
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, NW, false, SEXP>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                     (hipStream_t)a.stream, a.q8, a.k8, a.v8, a.qs, a.ks, a.vs, a.o, a.lse, BH, a.N, nqb,
                     nsb, a.scale * kLog2e);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Four-wave workgroups (two per CU) were faster for every causal length and
// at d = 64 (2-24%), and for non-causal d = 128 up to N = 2048; above that
// the eight-wave workgroup was 2-4% faster.
constexpr int kF8WideKeys = 2048;
template <int D, bool CAUSAL, int SEXP>
static int launch_f8(const Fp8FwdArgs& a) {
  if constexpr (D == 128 && !CAUSAL) {
    if (a.N > kF8WideKeys) return launch_f8_nw<D, CAUSAL, 8, SEXP>(a);
  }
  return launch_f8_nw<D, CAUSAL, 4, SEXP>(a);
}

template <int SEXP>
static int launch_f8_128(const Fp8FwdArgs& a) {
  return a.causal ? launch_f8<128, true, SEXP>(a) : launch_f8<128, false, SEXP>(a);
}

int launch_fwd_fp8(const Fp8FwdArgs& a) {
  if (a.d == 128) {
    if (a.exp_mode == 1) return launch_f8_128<1>(a);
    if (a.exp_mode == 2) return launch_f8_128<2>(a);
    return launch_f8_128<0>(a);
  }
  return a.causal ? launch_f8<64, true, 0>(a) : launch_f8<64, false, 0>(a);
}

}  // namespace fa
