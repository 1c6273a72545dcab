// fa_bwd: bf16 attention backward for gfx950 by recomputation.
//
// Method ([HUB] "How it works": store only L_i = m_i + log l_i and recompute
// P_ij = exp(S_ij - L_i) tile by tile; [LIB] "FA1 — changing the order of the
// operations": recomputation in the backward pass). The gradients are those
// of the forward definition: dV = P^T dO, dP = dO V^T, D = rowsum(dO o O),
// dS = P o (dP - D), dQ = scale dS K, dK = scale dS^T Q.
//
// Three launches on the caller's stream, none with atomics:
//   1. pre_kernel  : D = rowsum(dO o O) in fp32.
//   2. dkdv_kernel : one workgroup per (batch, head, 128-key block); four waves
//                    own 32 keys each and keep K, V (MFMA operands) and the dK,
//                    dV accumulators in registers for the whole pass. For every
//                    32-row Q block: S = Q K^T and dP = dO V^T (lane = key),
//                    P and dS lane-locally, dV += P^T dO and dK += dS^T Q with
//                    dO / Q read transposed from LDS. Q, dO, L and D of the next
//                    block arrive by direct global->LDS loads meanwhile.
//   3. dq_kernel   : one workgroup per (batch, head, 256-row Q block), eight
//                    waves of 32 query rows that keep Q, dO (MFMA operands) and
//                    the dQ accumulator in registers, and stream 64-key K / V
//                    tiles: S^T = K Q^T and dP^T = V dO^T (lane = query), P and
//                    dS lane-locally, dQ^T += K^T dS^T with K read transposed.
// Splitting dQ from dK/dV recomputes S and dP once more (7 instead of 5
// matrix products) but needs no fp32 atomics: on this chip an fp32 atomic add
// retires about ten times slower than a store, and one dQ partial per
// (key block, query block) pair would cost more than the extra products.
// Every output is written once by one wave, so the results are deterministic.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kBKC = 128;  // dkdv: keys per workgroup (4 waves x 32)
constexpr int kBQ = 32;    // dkdv: query rows per step
constexpr int kQNW = 8;    // dq: waves per workgroup
constexpr int kQBR = kQNW * 32;  // dq: query rows per workgroup
constexpr int kQBC = 64;   // dq: keys per tile
constexpr int kQThreads = kQNW * 64;

// 16-byte chunk swizzle of a [rows][D] bf16 tile that is conflict-free both for
// 16-lane row reads (16 consecutive rows, one chunk) and for transposed reads
// (4 aligned consecutive rows x 64 bytes).
template <int D>
__device__ __forceinline__ int swz2(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int toff(int row, int col) {
  return row * D + ((((col >> 3) ^ swz2<D>(row))) << 3) + (col & 7);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// Direct global->LDS loads of a [ROWS x D] bf16 tile (rows clamped to N-1) by
// THREADS threads into the layout of toff<D> (TR) or of the forward's K tile.
// Thread `tid`
// fills the 16-byte LDS chunks n * THREADS + tid; the source chunk is chosen so
// that LDS holds the swizzled layout.
template <int D, int ROWS, int THREADS, bool TR>
__device__ __forceinline__ void load_tile_async(uint16_t* lds_tile, const uint16_t* head, int r0, int N, int tid) {
  constexpr int CH = D / 8;
  const int w = tid >> 6;
#pragma unroll
  for (int n = 0; n < (ROWS * CH) / THREADS; ++n) {
    const int e = n * THREADS + tid;
    const int r = e / CH, p = e % CH;
    const int c = p ^ (TR ? swz2<D>(r) : swz_k<D>(r));
    const int row = min(r0 + r, N - 1);
    const uint16_t* src = head + (size_t)row * D + c * 8;
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

// dK / dV accumulation into AGPR-resident accumulators. With the compiler's
// own MFMA the register allocator moved these 128 registers between AGPRs and
// VGPRs on every step; the "a" constraint pins them. The compiler inserts no
// wait states in front of inline asm: s_nop 1 gives the two that an MFMA needs
// after a VALU write of its A/B operands (back-to-back accumulation into the
// same registers needs none).
__device__ __forceinline__ void mfma_acc_agpr(f32x16& acc, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last MFMA writes of two accumulators and the reads
// that follow (at least 18 are needed after a 32x32 MFMA); the operands tie the
// reads to this point.
__device__ __forceinline__ void agpr_settle(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(x), "+a"(y));
}

// Work-id remap: blocks are dispatched round-robin over the 8 XCDs; give each
// XCD a contiguous range of work ids so that one head's blocks share its L2.
__device__ __forceinline__ int xcd_work_id(int total) {
  const int b = (int)blockIdx.x;
  return (total & 7) == 0 ? (b & 7) * (total >> 3) + (b >> 3) : b;
}

}  // namespace

template <int D>
__global__ void __launch_bounds__(256)
pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, float* __restrict__ delta,
           long long rows) {
  constexpr int LPR = D / 8;        // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;    // rows per block
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float s = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + c * 8;
    const u32x4 a = *(const u32x4*)(O + off);
    const u32x4 b = *(const u32x4*)(dO + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) s += bf16_lo(a[j]) * bf16_lo(b[j]) + bf16_hi(a[j]) * bf16_hi(b[j]);
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (row < rows && c == 0) delta[row] = s;
}

// ---------------------------------------------------------------------------
// dK, dV: key-stationary
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 1)
dkdv_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg,
            const uint16_t* __restrict__ dOg, const float* __restrict__ LSEg, const float* __restrict__ Dg,
            uint16_t* __restrict__ dKg, uint16_t* __restrict__ dVg, int BH, int N, int nkb, float scale,
            float scale_log2) {
  constexpr int KS = D / 16;    // k-steps over d
  constexpr int DB = D / 32;    // 32-wide d blocks
  constexpr int QT = kBQ * D;   // elements of a Q or dO tile

  // separate arrays per buffer so the compiler can tell filled from read buffers
  __shared__ __attribute__((aligned(16))) uint16_t sQ0[QT];
  __shared__ __attribute__((aligned(16))) uint16_t sQ1[QT];
  __shared__ __attribute__((aligned(16))) uint16_t sO0[QT];
  __shared__ __attribute__((aligned(16))) uint16_t sO1[QT];
  __shared__ __attribute__((aligned(16))) float sLD0[2 * kBQ];
  __shared__ __attribute__((aligned(16))) float sLD1[2 * kBQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int g = lane >> 4, i16 = lane & 15;

  // One head's key blocks run together on one XCD, heaviest causal block first.
  const int wid = xcd_work_id(nkb * BH);
  const int bh = wid / nkb;
  const int kblk = wid % nkb;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Qg + head;
  const uint16_t* dOh = dOg + head;
  const float* lse_h = LSEg + (size_t)bh * N;
  const float* d_h = Dg + (size_t)bh * N;
  const int kb0 = kblk * kBKC;
  const int kw0 = kb0 + w * 32;
  const int key_l = kw0 + l32;  // this lane's key in S / dP

  // Query blocks from the last down, so that the concurrent key blocks of a
  // head read the same Q / dO tiles at about the same time.
  const int nqs = (N + kBQ - 1) / kBQ;
  const int qs_lo = CAUSAL ? kb0 / kBQ : 0;

  load_tile_async<D, kBQ, 256, true>(sQ0, Qh, (nqs - 1) * kBQ, N, tid);
  load_tile_async<D, kBQ, 256, true>(sO0, dOh, (nqs - 1) * kBQ, N, tid);
  if (w == 0) load_ld_async(sLD0, lse_h, d_h, (nqs - 1) * kBQ, N, lane);

  // per-wave K and V as B operands of S = Q K^T and dP = dO V^T
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (key_l < N) {
      a = *(const u32x4*)(Kg + head + (size_t)key_l * D + ks * 16 + hi * 8);
      b = *(const u32x4*)(Vg + head + (size_t)key_l * D + ks * 16 + hi * 8);
    }
    kf[ks] = as_bf16x8(a);
    vf[ks] = as_bf16x8(b);
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) { dk[db] = f32x16{}; dv[db] = f32x16{}; }

  auto step = [&](int qs, const uint16_t* sQ, const uint16_t* sO, const float* sLD, uint16_t* nQ, uint16_t* nO,
                  float* nLD) __attribute__((always_inline)) {
    const int q0 = qs * kBQ;
    wait_loads_and_sync();  // this block's Q, dO, L, D landed; every wave is done with the other buffers
    if (qs > qs_lo) {
      load_tile_async<D, kBQ, 256, true>(nQ, Qh, q0 - kBQ, N, tid);
      load_tile_async<D, kBQ, 256, true>(nO, dOh, q0 - kBQ, N, tid);
      if (w == 0) load_ld_async(nLD, lse_h, d_h, q0 - kBQ, N, lane);
    }
    // (Causal steps whose queries all precede this wave's keys run through the
    // masked path and add zeros: skipping them costs more in register moves.)
    // lane index through an empty asm: LDS addresses are formed here, not hoisted
    int lp = lane;
    asm volatile("" : "+v"(lp));
    const int l32 = lp & 31, hi = lp >> 5, g = lp >> 4, i16 = lp & 15;

    // ---- S = Q K^T and dP = dO V^T (lane = key, 16 queries per lane); the
    // Q / dO operands are read one k-step ahead
    f32x16 s = f32x16{}, dp = f32x16{};
    u32x4 aq = *(const u32x4*)(sQ + toff<D>(l32, hi * 8));
    u32x4 ao = *(const u32x4*)(sO + toff<D>(l32, hi * 8));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 nq, no;
      if (ks + 1 < KS) {
        const int col = (ks + 1) * 16 + hi * 8;
        nq = *(const u32x4*)(sQ + toff<D>(l32, col));
        no = *(const u32x4*)(sO + toff<D>(l32, col));
      }
      s = mfma_bf16_32x32x16(as_bf16x8(aq), kf[ks], s);
      dp = mfma_bf16_32x32x16(as_bf16x8(ao), vf[ks], dp);
      if (ks + 1 < KS) {
        aq = nq;
        ao = no;
      }
    }

    // ---- P = exp2(S c - L log2 e), dS = P (dP - D); masked entries give P = 0.
    // The masked variant is a separate instantiation so that unmasked blocks
    // carry no compare/select code.
    u32x4 pP[2], pS[2];
    auto p_ds = [&](auto masked_tag) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int qi = 8 * g4 + 4 * hi;
        const f32x4 L4 = *(const f32x4*)(sLD + qi);
        const f32x4 D4 = *(const f32x4*)(sLD + kBQ + qi);
        float p[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g4 + e;
          float arg = __builtin_fmaf(s[i], scale_log2, -L4[e] * kLog2e);
          if constexpr (MASKED) {
            const int q = q0 + qi + e;
            arg = ((CAUSAL && key_l > q) || key_l >= N || q >= N) ? -INFINITY : arg;
          }
          const float pv = fast_exp2(arg);
          p[e] = pv;
          ds[e] = pv * (dp[i] - D4[e]);
        }
        pP[g4 >> 1][2 * (g4 & 1)] = pack_bf16x2(p[0], p[1]);
        pP[g4 >> 1][2 * (g4 & 1) + 1] = pack_bf16x2(p[2], p[3]);
        pS[g4 >> 1][2 * (g4 & 1)] = pack_bf16x2(ds[0], ds[1]);
        pS[g4 >> 1][2 * (g4 & 1) + 1] = pack_bf16x2(ds[2], ds[3]);
      }
    };
    if ((CAUSAL && q0 < kw0 + 31) || (kw0 + 32 > N) || (q0 + kBQ > N))
      p_ds(std::true_type{});
    else
      p_ds(std::false_type{});

    // ---- dV += P^T dO and dK += dS^T Q (dO, Q read transposed). The query
    // order inside a k-step follows the accumulator layout of S: slot 8 hi + j
    // holds query 16 s2 + 8 (j / 4) + 4 hi + j % 4.
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int r0 = 16 * s2 + 4 * hi + (i16 >> 2);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 32 + 16 * (g & 1) + 4 * (i16 & 3);
        const u32x4 bo = tr_pair(sO + toff<D>(r0, d), sO + toff<D>(r0 + 8, d));
        const u32x4 bq = tr_pair(sQ + toff<D>(r0, d), sQ + toff<D>(r0 + 8, d));
        mfma_acc_agpr(dv[db], pP[s2], bo);
        mfma_acc_agpr(dk[db], pS[s2], bq);
      }
    }
  };

  // Buffers alternate by step parity (not unrolled: the swizzled LDS addresses
  // of one step then stay in few registers).
  for (int qs = nqs - 1; qs >= qs_lo; --qs) {
    const bool odd = (nqs - 1 - qs) & 1;
    step(qs, odd ? sQ1 : sQ0, odd ? sO1 : sO0, odd ? sLD1 : sLD0, odd ? sQ0 : sQ1, odd ? sO0 : sO1,
         odd ? sLD0 : sLD1);
  }

  // ---- dK (times scale) and dV, bf16 (lane = d column, 16 keys per lane)
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    agpr_settle(dk[db], dv[db]);
    const int d = db * 32 + l32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw0 + 8 * (i / 4) + 4 * hi + (i % 4);
      if (key < N) {
        const size_t off = head + (size_t)key * D + d;
        dKg[off] = (uint16_t)(pack_bf16x2(dk[db][i] * scale, 0.f) & 0xffffu);
        dVg[off] = (uint16_t)(pack_bf16x2(dv[db][i], 0.f) & 0xffffu);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: query-stationary
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kQThreads, 1)
dq_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg,
          const uint16_t* __restrict__ dOg, const float* __restrict__ LSEg, const float* __restrict__ Dg,
          uint16_t* __restrict__ dQg, int BH, int N, int nqb, float scale, float scale_log2) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = kQBC * D;

  __shared__ __attribute__((aligned(16))) uint16_t sK0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int g = lane >> 4, i16 = lane & 15;

  const int wid = xcd_work_id(nqb * BH);
  const int bh = wid / nqb;
  const int qblk = CAUSAL ? nqb - 1 - (wid % nqb) : (wid % nqb);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Kh = Kg + head;
  const uint16_t* Vh = Vg + head;
  const int qw0 = qblk * kQBR + w * 32;
  const int qrow = qw0 + l32;

  const int kend = CAUSAL ? min(N, qblk * kQBR + kQBR) : N;
  const int ntiles = (kend + kQBC - 1) / kQBC;
  const int wlast = CAUSAL ? min(ntiles - 1, (qw0 + 31) / kQBC) : ntiles - 1;

  load_tile_async<D, kQBC, kQThreads, true>(sK0, Kh, 0, N, tid);
  load_tile_async<D, kQBC, kQThreads, true>(sV0, Vh, 0, N, tid);

  // Q and dO as B operands of S^T = K Q^T and dP^T = V dO^T
  bf16x8 qf[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (qrow < N) {
      a = *(const u32x4*)(Qg + head + (size_t)qrow * D + ks * 16 + hi * 8);
      b = *(const u32x4*)(dOg + head + (size_t)qrow * D + ks * 16 + hi * 8);
    }
    qf[ks] = as_bf16x8(a);
    of[ks] = as_bf16x8(b);
  }
  // rows past N: L = +inf gives P = 0
  const float Lq = qrow < N ? LSEg[(size_t)bh * N + qrow] * kLog2e : INFINITY;
  const float Dq = qrow < N ? Dg[(size_t)bh * N + qrow] : 0.f;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  auto tile = [&](int t, const uint16_t* sK, const uint16_t* sV, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int k0 = t * kQBC;
    // The lane index passes through an empty asm so that the LDS addresses
    // derived from it are formed inside the tile rather than hoisted out of
    // the loop for both tile variants (which would not fit in registers).
    int lp = lane;
    asm volatile("" : "+v"(lp));
    const int l32 = lp & 31, hi = lp >> 5, g = lp >> 4, i16 = lp & 15;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // ---- S^T and dP^T for 32 keys (lane = query)
      const int r = kb * 32 + l32;
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int col = ks * 16 + hi * 8;
        const bf16x8 ak = as_bf16x8(*(const u32x4*)(sK + toff<D>(r, col)));
        const bf16x8 av = as_bf16x8(*(const u32x4*)(sV + toff<D>(r, col)));
        s = mfma_bf16_32x32x16(ak, qf[ks], s);
        dp = mfma_bf16_32x32x16(av, of[ks], dp);
      }
      // ---- dS^T = P^T o (dP^T - D), packed as the B operands of K^T dS^T
      u32x4 dsb[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        float ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * h2 + j;
          float pv = fast_exp2(__builtin_fmaf(s[i], scale_log2, -Lq));
          if constexpr (MASKED) {
            const int key = k0 + kb * 32 + 8 * (i / 4) + 4 * hi + (i % 4);
            if ((CAUSAL && key > qrow) || key >= N) pv = 0.f;
          }
          ds[j] = pv * (dp[i] - Dq);
        }
        dsb[h2] = u32x4{pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]), pack_bf16x2(ds[4], ds[5]),
                        pack_bf16x2(ds[6], ds[7])};
      }
      // ---- dQ^T += K^T dS^T over two 16-key steps (K read transposed)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int r0 = kb * 32 + 16 * h2 + 4 * hi + (i16 >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = db * 32 + 16 * (g & 1) + 4 * (i16 & 3);
          const u32x4 au = tr_pair(sK + toff<D>(r0, d), sK + toff<D>(r0 + 8, d));
          acc[db] = mfma_bf16_32x32x16(as_bf16x8(au), as_bf16x8(dsb[h2]), acc[db]);
        }
      }
    }
  };

  // Buffers alternate by tile parity (not unrolled, for the same reason).
  for (int t = 0; t < ntiles; ++t) {
    const bool odd = t & 1;
    wait_loads_and_sync();  // tile t landed; every wave finished tile t-1
    if (t + 1 < ntiles) {
      load_tile_async<D, kQBC, kQThreads, true>(odd ? sK0 : sK1, Kh, (t + 1) * kQBC, N, tid);
      load_tile_async<D, kQBC, kQThreads, true>(odd ? sV0 : sV1, Vh, (t + 1) * kQBC, N, tid);
    }
    if (t > wlast) continue;  // this wave's rows see none of these keys
    const int k0 = t * kQBC;
    const uint16_t* sK = odd ? sK1 : sK0;
    const uint16_t* sV = odd ? sV1 : sV0;
    if ((CAUSAL && k0 + kQBC - 1 > qw0) || k0 + kQBC > N)
      tile(t, sK, sV, std::true_type{});
    else
      tile(t, sK, sV, std::false_type{});
  }

  // ---- dQ = scale dQ^T^T, bf16 (lane = query, d over the accumulator rows)
  if (qrow < N) {
    uint16_t* row = dQg + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hi;
        const u32x2 pk = {pack_bf16x2(acc[db][4 * g4 + 0] * scale, acc[db][4 * g4 + 1] * scale),
                          pack_bf16x2(acc[db][4 * g4 + 2] * scale, acc[db][4 * g4 + 3] * scale)};
        *(u32x2*)(row + d) = pk;
      }
  }
}

template <int D, bool CAUSAL>
static int launch(const BwdArgs& a) {
  hipStream_t st = (hipStream_t)a.stream;
  const int BH = a.B * a.H;
  const long long rows = (long long)BH * a.N;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st, a.o, a.dO,
                     a.delta, rows);
  const int nkb = (a.N + kBKC - 1) / kBKC;
  hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL>), dim3((unsigned)(nkb * BH)), dim3(256), 0, st, a.q, a.k, a.v,
                     a.dO, a.lse, a.delta, a.dk, a.dv, BH, a.N, nkb, a.scale, a.scale * kLog2e);
  const int nqb = (a.N + kQBR - 1) / kQBR;
  hipLaunchKernelGGL((dq_kernel<D, CAUSAL>), dim3((unsigned)(nqb * BH)), dim3(kQThreads), 0, st, a.q, a.k, a.v,
                     a.dO, a.lse, a.delta, a.dq, BH, a.N, nqb, a.scale, a.scale * kLog2e);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

int launch_bwd(const BwdArgs& a) {
  if (a.d == 128) return a.causal ? launch<128, true>(a) : launch<128, false>(a);
  return a.causal ? launch<64, true>(a) : launch<64, false>(a);
}

}  // namespace fa
