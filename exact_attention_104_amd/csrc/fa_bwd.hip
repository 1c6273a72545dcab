// fa_bwd: bf16 attention backward for gfx950 by recomputation.
//
// Method ([HUB] "How it works": store only L_i = m_i + log l_i and recompute
// P_ij = exp(S_ij - L_i) tile by tile; [LIB] "FA1 — changing the order of the
// operations": recomputation in the backward pass). The gradients are those
// of the forward definition: dV = P^T dO, dP = dO V^T, D = rowsum(dO o O),
// dS = P o (dP - D), dQ = scale dS K, dK = scale dS^T Q.
//
// Three launches on the caller's stream:
//   1. bwd_pre_kernel  : D = rowsum(dO o O) (fp32) and zero the fp32 dQ accumulator
//   2. bwd_kernel      : one workgroup per (batch, head, 128-key block); four
//                        waves own 32 keys each and keep K, V (MFMA operands)
//                        and the dK, dV accumulators in registers for the whole
//                        pass (no atomics for dK, dV). For every 32-row Q block:
//                        S = Q K^T and dP = dO V^T (lane = key), P and dS
//                        lane-locally, dV += P^T dO and dK += dS^T Q with dO / Q
//                        read transposed from LDS, dS staged in LDS, then
//                        dQ += dS K for the block, added to the fp32 accumulator
//                        with atomics. Q, dO, L and D of the next block arrive by
//                        direct global->LDS loads while the current one is used.
//   3. bwd_convert_kernel : dQ = scale * accumulator -> bf16
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kBKC = 128;  // keys per workgroup (4 waves x 32)
constexpr int kBQ = 32;    // query rows per step

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
// dS tile [128 keys][32 queries] bf16 (64-byte rows) in 8-byte chunks: the
// 8-byte row writes (32 consecutive keys) and the transposed reads (4 keys x
// 32 bytes per 16 lanes) both spread over all banks.
__device__ __forceinline__ int ds_off(int key, int q) {
  const int c8 = (q >> 2) ^ ((key >> 2) & 7);
  return key * kBQ + c8 * 4 + (q & 3);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// Direct global->LDS loads of a [32 x D] bf16 row tile (rows clamped to N-1)
// into the swizzled layout of toff<D>.
template <int D>
__device__ __forceinline__ void load_rows_async(uint16_t* lds_tile, const uint16_t* head, int q0, int N, int tid) {
  constexpr int CH = D / 8;
  const int w = tid >> 6;
#pragma unroll
  for (int n = 0; n < (kBQ * CH) / 256; ++n) {
    const int e = n * 256 + tid;
    const int r = e / CH, p = e % CH;
    const int c = p ^ swz2<D>(r);
    const int row = min(q0 + r, N - 1);
    const uint16_t* src = head + (size_t)row * D + c * 8;
    uint16_t* dst = lds_tile + (n * 256 + w * 64) * 8;
    __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  }
}

// L (lanes 0..31) and D (lanes 32..63) of 32 rows, by wave 0 only.
__device__ __forceinline__ void load_ld_async(float* lds_ld, const float* lse_h, const float* d_h, int q0, int N,
                                              int lane) {
  const int r = min(q0 + (lane & 31), N - 1);
  const float* src = (lane < 32) ? lse_h + r : d_h + r;
  __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)lds_ld, 4, 0, 0);
}

__device__ __forceinline__ void wait_loads_and_sync() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

__device__ __forceinline__ u32x4 tr_pair(const uint16_t* p0, const uint16_t* p1) {
  const i16x4 t0 = lds_read_tr16(p0);
  const i16x4 t1 = lds_read_tr16(p1);
  return u32x4{__builtin_bit_cast(u32x2, t0)[0], __builtin_bit_cast(u32x2, t0)[1],
               __builtin_bit_cast(u32x2, t1)[0], __builtin_bit_cast(u32x2, t1)[1]};
}

}  // namespace

template <int D>
__global__ void __launch_bounds__(256)
bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, float* __restrict__ delta,
               float* __restrict__ dq_acc, long long rows) {
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
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *(f32x4*)(dq_acc + off) = z;
    *(f32x4*)(dq_acc + off + 4) = z;
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (row < rows && c == 0) delta[row] = s;
}

__global__ void __launch_bounds__(256)
bwd_convert_kernel(const float* __restrict__ acc, uint16_t* __restrict__ dq, long long n8, float scale) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *(const f32x4*)(acc + i * 8);
  const f32x4 b = *(const f32x4*)(acc + i * 8 + 4);
  const u32x4 o = {pack_bf16x2(a[0] * scale, a[1] * scale), pack_bf16x2(a[2] * scale, a[3] * scale),
                   pack_bf16x2(b[0] * scale, b[1] * scale), pack_bf16x2(b[2] * scale, b[3] * scale)};
  *(u32x4*)(dq + i * 8) = o;
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 1)
bwd_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg,
           const uint16_t* __restrict__ dOg, const float* __restrict__ LSEg, const float* __restrict__ Dg,
           float* __restrict__ dQacc, uint16_t* __restrict__ dKg, uint16_t* __restrict__ dVg,
           int BH, int N, float scale, float scale_log2) {
  constexpr int KS = D / 16;    // k-steps over d
  constexpr int DB = D / 32;    // 32-wide d blocks
  constexpr int CH = D / 8;     // 16-byte chunks per row
  constexpr int QT = kBQ * D;   // elements of a Q or dO tile

  // separate arrays per buffer so the compiler can tell filled from read buffers
  __shared__ __attribute__((aligned(16))) uint16_t sQ0[QT];
  __shared__ __attribute__((aligned(16))) uint16_t sQ1[QT];
  __shared__ __attribute__((aligned(16))) uint16_t sO0[QT];
  __shared__ __attribute__((aligned(16))) uint16_t sO1[QT];
  __shared__ __attribute__((aligned(16))) float sLD0[2 * kBQ];
  __shared__ __attribute__((aligned(16))) float sLD1[2 * kBQ];
  __shared__ __attribute__((aligned(16))) uint16_t sK[kBKC * D];
  __shared__ __attribute__((aligned(16))) uint16_t sdS[kBKC * kBQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int g = lane >> 4, i16 = lane & 15;

  const int kblk = (int)(blockIdx.x / BH);  // ascending: most causal work first
  const int bh = (int)(blockIdx.x % BH);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Qg + head;
  const uint16_t* dOh = dOg + head;
  const float* lse_h = LSEg + (size_t)bh * N;
  const float* d_h = Dg + (size_t)bh * N;
  const int kb0 = kblk * kBKC;
  const int kw0 = kb0 + w * 32;
  const int key_l = kw0 + l32;  // this lane's key in S / dP

  const int nqs = (N + kBQ - 1) / kBQ;
  const int qs0 = CAUSAL ? kb0 / kBQ : 0;

  // first Q block's loads, then the stationary K block
  load_rows_async<D>(sQ0, Qh, qs0 * kBQ, N, tid);
  load_rows_async<D>(sO0, dOh, qs0 * kBQ, N, tid);
  if (w == 0) load_ld_async(sLD0, lse_h, d_h, qs0 * kBQ, N, lane);
#pragma unroll
  for (int n = 0; n < (kBKC * CH) / 256; ++n) {
    const int u = tid + 256 * n;
    const int r = u / CH, c = u % CH;
    u32x4 kv = {0, 0, 0, 0};
    if (kb0 + r < N) kv = *(const u32x4*)(Kg + head + (size_t)(kb0 + r) * D + c * 8);
    *(u32x4*)(sK + toff<D>(r, c * 8)) = kv;
  }
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
                  float* nLD) {
    const int q0 = qs * kBQ;
    wait_loads_and_sync();  // this block's Q, dO, L, D landed; previous step done with sdS
    if (qs + 1 < nqs) {
      load_rows_async<D>(nQ, Qh, q0 + kBQ, N, tid);
      load_rows_async<D>(nO, dOh, q0 + kBQ, N, tid);
      if (w == 0) load_ld_async(nLD, lse_h, d_h, q0 + kBQ, N, lane);
    }

    // ---- S = Q K^T and dP = dO V^T (lane = key, 16 queries per lane)
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int col = ks * 16 + hi * 8;
      const bf16x8 aq = as_bf16x8(*(const u32x4*)(sQ + toff<D>(l32, col)));
      const bf16x8 ao = as_bf16x8(*(const u32x4*)(sO + toff<D>(l32, col)));
      s = mfma_bf16_32x32x16(aq, kf[ks], s);
      dp = mfma_bf16_32x32x16(ao, vf[ks], dp);
    }

    // ---- P = exp2(S c - L log2 e), dS = P (dP - D); masked entries give P = 0.
    // The masked variant is a separate instantiation so that unmasked blocks
    // carry no compare/select code.
    u32x4 pP[2], pS[2];
    auto p_ds = [&](auto masked_tag) {
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
          float pv = fast_exp2(__builtin_fmaf(s[i], scale_log2, -L4[e] * kLog2e));
          if constexpr (MASKED) {
            const int q = q0 + qi + e;
            if ((CAUSAL && key_l > q) || key_l >= N || q >= N) pv = 0.f;
          }
          p[e] = pv;
          ds[e] = pv * (dp[i] - D4[e]);
        }
        const uint32_t p01 = pack_bf16x2(p[0], p[1]), p23 = pack_bf16x2(p[2], p[3]);
        const uint32_t d01 = pack_bf16x2(ds[0], ds[1]), d23 = pack_bf16x2(ds[2], ds[3]);
        pP[g4 >> 1][2 * (g4 & 1)] = p01;
        pP[g4 >> 1][2 * (g4 & 1) + 1] = p23;
        pS[g4 >> 1][2 * (g4 & 1)] = d01;
        pS[g4 >> 1][2 * (g4 & 1) + 1] = d23;
        *(u32x2*)(sdS + ds_off(w * 32 + l32, qi)) = u32x2{d01, d23};
      }
    };
    if ((CAUSAL && q0 < kw0 + 31) || (kw0 + 32 > N) || (q0 + kBQ > N))
      p_ds(std::true_type{});
    else
      p_ds(std::false_type{});

    // ---- dV += P^T dO and dK += dS^T Q (dO, Q read transposed)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int r0 = 16 * s2 + 4 * hi + (i16 >> 2);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 32 + 16 * (g & 1) + 4 * (i16 & 3);
        const u32x4 bo = tr_pair(sO + toff<D>(r0, d), sO + toff<D>(r0 + 8, d));
        const u32x4 bq = tr_pair(sQ + toff<D>(r0, d), sQ + toff<D>(r0 + 8, d));
        dv[db] = mfma_bf16_32x32x16(as_bf16x8(pP[s2]), as_bf16x8(bo), dv[db]);
        dk[db] = mfma_bf16_32x32x16(as_bf16x8(pS[s2]), as_bf16x8(bq), dk[db]);
      }
    }
    __syncthreads();  // dS tile complete

    // ---- dQ += dS K for this block: wave w owns d block w (DB = 4) or d/q
    // halves (DB = 2); atomics into the fp32 accumulator
    if (w < DB) {
      f32x16 dq = f32x16{};
      const int db = w;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int kr = 16 * st + 8 * hi + (i16 >> 2);
        const int qc = 16 * (g & 1) + 4 * (i16 & 3);
        const int d = db * 32 + 16 * (g & 1) + 4 * (i16 & 3);
        const u32x4 au = tr_pair(sdS + ds_off(kr, qc), sdS + ds_off(kr + 4, qc));
        const u32x4 bu = tr_pair(sK + toff<D>(kr, d), sK + toff<D>(kr + 4, d));
        dq = mfma_bf16_32x32x16(as_bf16x8(au), as_bf16x8(bu), dq);
      }
      const int d = db * 32 + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = q0 + 8 * (i / 4) + 4 * hi + (i % 4);
        if (q < N) unsafeAtomicAdd(dQacc + head + (size_t)q * D + d, dq[i]);
      }
    }
  };

  // Buffers alternate by step parity (not unrolled: the swizzled LDS addresses
  // of one step then stay in few registers).
  for (int qs = qs0; qs < nqs; ++qs) {
    const bool odd = (qs - qs0) & 1;
    step(qs, odd ? sQ1 : sQ0, odd ? sO1 : sO0, odd ? sLD1 : sLD0, odd ? sQ0 : sQ1, odd ? sO0 : sO1,
         odd ? sLD0 : sLD1);
  }

  // ---- dK (times scale) and dV, bf16 (lane = d column, 16 keys per lane)
#pragma unroll
  for (int db = 0; db < DB; ++db) {
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

template <int D, bool CAUSAL>
static int launch(const BwdArgs& a) {
  hipStream_t st = (hipStream_t)a.stream;
  const int BH = a.B * a.H;
  const long long rows = (long long)BH * a.N;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st,
                     a.o, a.dO, a.delta, a.dq_acc, rows);
  const int nkb = (a.N + kBKC - 1) / kBKC;
  hipLaunchKernelGGL((bwd_kernel<D, CAUSAL>), dim3((unsigned)(nkb * BH)), dim3(256), 0, st,
                     a.q, a.k, a.v, a.dO, a.lse, a.delta, a.dq_acc, a.dk, a.dv, BH, a.N, a.scale,
                     a.scale * kLog2e);
  const long long n8 = rows * D / 8;
  hipLaunchKernelGGL(bwd_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                     a.dq_acc, a.dq, n8, a.scale);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

int launch_bwd(const BwdArgs& a) {
  if (a.d == 128) return a.causal ? launch<128, true>(a) : launch<128, false>(a);
  return a.causal ? launch<64, true>(a) : launch<64, false>(a);
}

}  // namespace fa
