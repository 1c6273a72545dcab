// fa_fwd: bf16 exact attention forward for gfx950 (MI355X).
//
// Method ([HUB] "How it works"; [LIB] "The trick that made it all possible:
// online softmax"; [LIN] "FA2 (2023)"): one workgroup per (batch, head,
// Q-block); every wavefront owns its own query rows (split-Q), streams K/V
// tiles through LDS, forms the score tile on chip with bf16 MFMA (fp32
// accumulation), keeps the running max m and sum l per query in registers,
// rescales the output accumulator only when some row's max changed, and
// divides by l once at the end, saving LSE = m + log l.
//
// Orientation: each wave computes S^T = K Q^T so that MFMA accumulator
// columns are queries: a lane owns one query, the row max and row sum are
// lane-local apart from one exchange with the other half of the wave, and the
// per-query rescale of O^T = V^T P^T is lane-local too. P^T leaves the
// accumulators already in the B-operand layout of the P V product; V^T comes
// from LDS through transposed 16-bit reads.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

template <int D, int QW, bool CAUSAL>
__global__ void __launch_bounds__(256, 1)
fwd_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
           const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og, float* __restrict__ LSEg,
           int BH, int N, int nqb, float scale_log2) {
  constexpr int NW = 4;            // wavefronts per workgroup
  constexpr int BR = NW * QW;      // query rows per workgroup
  constexpr int BC = 64;           // keys per tile
  constexpr int QB = QW / 32;      // 32-query MFMA blocks per wave
  constexpr int KS = D / 16;       // k-steps of the S product
  constexpr int DB = D / 32;       // 32-row d blocks of O^T
  constexpr int CH = D / 8;        // 16-byte chunks per row

  __shared__ __attribute__((aligned(16))) uint16_t sK[BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, hi = lane >> 5;

  // Heaviest Q-blocks first (they have the most causal tiles).
  const int qblk = nqb - 1 - (int)(blockIdx.x / BH);
  const int bh = (int)(blockIdx.x % BH);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Qg + head;
  const uint16_t* Kh = Kg + head;
  const uint16_t* Vh = Vg + head;
  const int qw0 = qblk * BR + w * QW;  // first query row of this wave

  // Q as the B operand of S^T = K Q^T: lane holds Q[q][16 ks + 8 hi .. +7].
  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + qb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 u = {0, 0, 0, 0};
      if (row < N) u = *(const u32x4*)(Qh + (size_t)row * D + ks * 16 + hi * 8);
      qf[qb][ks] = as_bf16x8(u);
    }
  }

  f32x16 acc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = f32x16{};
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m[qb] = -INFINITY; l[qb] = 0.f; }

  const int kend = CAUSAL ? min(N, qblk * BR + BR) : N;
  const int ntiles = (kend + BC - 1) / BC;

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * BC;
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int n = 0; n < (BC * CH) / 256; ++n) {
      const int u = tid + 256 * n;
      const int r = u / CH, c = u % CH;
      const int key = k0 + r;
      u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (key < N) {
        kv = *(const u32x4*)(Kh + (size_t)key * D + c * 8);
        vv = *(const u32x4*)(Vh + (size_t)key * D + c * 8);
      }
      *(u32x4*)(sK + r * D + ((c ^ swz_k<D>(r)) * 8)) = kv;
      *(u32x4*)(sV + r * D + ((c ^ swz_v<D>(r)) * 8)) = vv;
    }
    __syncthreads();

    // Tiles entirely above the diagonal for this wave's rows: nothing to add.
    if (CAUSAL && k0 > qw0 + QW - 1) continue;

    // ---- S^T = K Q^T (two 32-key blocks x QB query blocks)
    f32x16 s[2][QB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r = kb * 32 + l32;
        const int c = ks * 2 + hi;
        const bf16x8 a = as_bf16x8(*(const u32x4*)(sK + r * D + ((c ^ swz_k<D>(r)) * 8)));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma_bf16_32x32x16(a, qf[qb][ks], s[kb][qb]);
      }
    }

    // ---- online softmax per query (lane-local plus one half-wave exchange)
    u32x4 pb[2][2][QB];  // [kb][16-key step within kb][qb]: bf16x8 B operands of P V
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = qw0 + qb * 32 + l32;
      const bool need_mask = (CAUSAL && k0 + BC - 1 > qw0 + qb * 32) || (k0 + BC > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + kb * 32 + 8 * (i / 4) + 4 * hi + (i % 4);
            const bool masked = (CAUSAL && key > qrow) || key >= N;
            if (masked) s[kb][qb][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][qb][i]);
      mx = fmaxf(mx, other_half(mx));
      const float m_new = fmaxf(m[qb], mx * scale_log2);
      // m_new is finite: key 0 is visible to every row and sits in tile 0.
      if (__any(m_new > m[qb])) {
        const float alpha = fast_exp2(m[qb] - m_new);
        l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[qb][db] *= alpha;
      }
      m[qb] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          float p[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            p[j] = fast_exp2(__builtin_fmaf(s[kb][qb][8 * h2 + j], scale_log2, -m_new));
            rs += p[j];
          }
          pb[kb][h2][qb] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                 pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        }
      }
      l[qb] += rs;
    }

    // ---- O^T += V^T P^T over four 16-key steps
    const int g = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = db * 32 + 16 * (g & 1) + 4 * (i16 & 3);
          const int c = d >> 3, within = d & 7;
          const int r0 = kb * 32 + 16 * h2 + 4 * hi + (i16 >> 2);
          const int r1 = r0 + 8;
          const i16x4 t0 = lds_read_tr16(sV + r0 * D + ((c ^ swz_v<D>(r0)) * 8) + within);
          const i16x4 t1 = lds_read_tr16(sV + r1 * D + ((c ^ swz_v<D>(r1)) * 8) + within);
          const u32x4 au = {__builtin_bit_cast(u32x2, t0)[0], __builtin_bit_cast(u32x2, t0)[1],
                            __builtin_bit_cast(u32x2, t1)[0], __builtin_bit_cast(u32x2, t1)[1]};
          const bf16x8 a = as_bf16x8(au);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            acc[qb][db] = mfma_bf16_32x32x16(a, as_bf16x8(pb[kb][h2][qb]), acc[qb][db]);
        }
      }
    }
  }

  // ---- epilogue: divide once by l, store O (bf16) and LSE (natural log)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l[qb] + other_half(l[qb]);
    const float inv = 1.0f / lt;
    const int row = qw0 + qb * 32 + l32;
    if (row < N) {
      uint16_t* orow = Og + head + (size_t)row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4 + 4 * hi;
          const u32x2 pk = {pack_bf16x2(acc[qb][db][4 * g4 + 0] * inv, acc[qb][db][4 * g4 + 1] * inv),
                            pack_bf16x2(acc[qb][db][4 * g4 + 2] * inv, acc[qb][db][4 * g4 + 3] * inv)};
          *(u32x2*)(orow + d) = pk;
        }
      if (hi == 0) LSEg[(size_t)bh * N + row] = (m[qb] + __log2f(lt)) * kLn2;
    }
  }
}

template <int D, int QW, bool CAUSAL>
static int launch(const FwdArgs& a) {
  constexpr int BR = 4 * QW;
  const int nqb = (a.N + BR - 1) / BR;
  const int BH = a.B * a.H;
  const dim3 grid((unsigned)(nqb * BH)), block(256);
  hipLaunchKernelGGL((fwd_kernel<D, QW, CAUSAL>), grid, block, 0, (hipStream_t)a.stream,
                     a.q, a.k, a.v, a.o, a.lse, BH, a.N, nqb, a.scale * kLog2e);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

int launch_fwd(const FwdArgs& a) {
  if (a.d == 128) return a.causal ? launch<128, 64, true>(a) : launch<128, 64, false>(a);
  return a.causal ? launch<64, 64, true>(a) : launch<64, 64, false>(a);
}

}  // namespace fa
