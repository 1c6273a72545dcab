// dQ of the bf16 attention backward (first launch of fa_bwd; the method and
// the second launch are described in fa_bwd.hip).
//
// One workgroup per (batch, head, 256-row Q block): eight waves of 32 query
// rows keep Q and dO (MFMA operands) and the dQ accumulator in registers,
// form D = rowsum(dO o O) of their rows (written to the workspace for the
// dK/dV launch that follows), and stream 64-key K / V tiles: S^T = K Q^T and dP^T = V dO^T (lane = query),
// P = exp2(S c - L log2 e) and dS = P o (dP - D) lane-locally, then
// dQ^T += K^T dS^T with K read transposed ([HUB] "How it works": dQ = scale
// dS K). Kept in its own file because it compiles best with MFMAs that write
// VGPRs (the key-stationary kernel wants the opposite).
#include <type_traits>

#include <algorithm>
#include <atomic>

#include "fa_bwd_tiles.h"
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

// dq: waves per workgroup (four at d = 256, where a wave needs more than the
// 256 registers of two-per-SIMD residency), query rows per workgroup
template <int D>
constexpr int kQNWof = D == 256 ? 4 : 8;
constexpr int kQBC = 64;   // dq: keys per tile
// Shorter key ranges use four-wave workgroups at d <= 128 (two per CU, each
// wave still at two per SIMD): one workgroup's start and end overlap
// another's tiles, and causal work splits more evenly. Measured on the whole
// backward: 3-8% faster up to 2048 keys, 1-3% at 4096 causal, 1-2% slower at
// 8192. Only the no-mask and causal instances: the general-band instance
// spills registers at four waves.
constexpr int kQShortKeys = 1024;        // four-wave workgroups up to this many keys without a mask,
constexpr int kQShortKeysCausal = 4096;  // and up to this many under the causal mask

}  // namespace

using namespace bwd;

// Masks as in the forward (the band of keys i + off - wl .. i + off + wr of
// 0 .. Nk - 1; kMaskBandAlibi adds -slope_h |i + off - j| to the scaled
// scores; kMaskNone and kMaskCausal keep the fixed arithmetic).
//
// XCD: the grid holds one workgroup per resident slot, and XCD x (workgroup
// j runs on XCD j % 8) takes heads x, x + 8, ..., its workgroups taking all
// Q-blocks of a head at once, with the Q-block order reversed on odd rounds
// (the forward's head-major dealing; the host uses it for the causal d = 128
// instances, four or eight waves, when every round holds whole heads; the
// four-wave one spills 29 VGPRs there and is still 1-2% faster at
// N = 1024 - 4096). Otherwise one workgroup per
// (head, Q-block): the loop below then runs once.
template <int D, int MASK, int NW, bool XCD = false>
__global__ void __launch_bounds__(NW * 64, (D <= 128 && NW == 4) ? 2 : 1)
dq_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg,
          const uint16_t* __restrict__ dOg, const float* __restrict__ LSEg, const uint16_t* __restrict__ Og,
          float* __restrict__ Dg, uint16_t* __restrict__ dQg, int BH, int H, int group, int Nq, int Nk, int nqb,
          float scale, float scale_log2, Band band, const float* __restrict__ slopes, Strides sq, Strides sk,
          Strides sv, Strides sdo, Strides so, Strides sdq) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = kQBC * D;
  constexpr bool BAND = MASK >= kMaskBand, CAUSAL = MASK == kMaskCausal, ALIBI = MASK == kMaskBandAlibi;
  constexpr int kQBR = NW * 32, kQThreads = NW * 64;

  // K(t) and V(t) tiles, double-buffered, in one array so that each V tile
  // sits a fixed 2 TILE elements after its K tile (one address serves both).
  __shared__ __attribute__((aligned(16))) uint16_t sKV[4 * TILE];
  uint16_t* const sK0 = sKV;
  uint16_t* const sK1 = sKV + TILE;
  uint16_t* const sV0 = sKV + 2 * TILE;
  uint16_t* const sV1 = sKV + 3 * TILE;

  const int tid = threadIdx.x;
  // The wave index is uniform. Under a general band, readfirstlane lets the
  // per-wave bounds live in scalar registers (else they spill); the fixed
  // masks schedule better without it.
  const int lane = tid & 63, w = BAND ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6, l32 = lane & 31,
            hi = lane >> 5;

  const int xj = (int)blockIdx.x, xx = xj & 7, xGx = (int)gridDim.x >> 3;
  const int xitems = (BH >> 3) * nqb;  // items of this XCD (XCD dealing)
  for (int xu = xj >> 3, xk = 0;; xu += xGx, ++xk) {
  int wid;
  if constexpr (XCD) {
    if (xu >= xitems) break;
    const int qb = (xk & 1) ? nqb - 1 - xu % nqb : xu % nqb;
    wid = ((xu / nqb) * 8 + xx) * nqb + qb;  // under a mask: Q-block nqb - 1 - qb
  } else {
    wid = xcd_work_id(nqb * BH);
  }
  const int bh = wid / nqb;
  const int qblk = MASK != kMaskNone ? nqb - 1 - (wid % nqb) : (wid % nqb);
  const int b = bh / H, h = bh % H, hk = h / group;  // query head h reads K/V head h / group
  const uint16_t* Kh = Kg + b * sk.b + hk * sk.h;
  const uint16_t* Vh = Vg + b * sv.b + hk * sv.h;
  const int q0 = qblk * kQBR;
  const int qw0 = q0 + w * 32;
  const int qrow = qw0 + l32;

  // key tiles t0 .. t1 - 1 cover the band of the block's rows, wfirst .. wlast
  // that of this wave's rows (none when they are all past Nq)
  int t0 = 0, t1, wfirst = 0, wlast;
  if constexpr (BAND) {
    const int qlast = min(q0 + kQBR, Nq) - 1;
    const int blo = max(0, q0 + band.off - band.wl);
    const int bhi = min(Nk - 1, qlast + band.off + band.wr);
    t0 = blo / kQBC;
    t1 = bhi >= blo ? bhi / kQBC + 1 : t0;
    const int wqlast = min(qw0 + 32, Nq) - 1;
    const int wlo = max(0, qw0 + band.off - band.wl);
    const int whi = min(Nk - 1, wqlast + band.off + band.wr);
    wfirst = wlo / kQBC;
    wlast = (wqlast >= qw0 && whi >= wlo) ? whi / kQBC : -1;
  } else {
    const int kend = CAUSAL ? min(Nk, q0 + kQBR) : Nk;
    t1 = (kend + kQBC - 1) / kQBC;
    wlast = CAUSAL ? min(t1 - 1, (qw0 + 31) / kQBC) : t1 - 1;
  }
  float nslope = 0.f;
  if constexpr (ALIBI) nslope = -slopes[h] * kLog2e;

  if (t1 > t0) {
    load_tile_async<D, kQBC, kQThreads, true>(sK0, Kh, sk.n, t0 * kQBC, Nk, tid);
    load_tile_async<D, kQBC, kQThreads, true>(sV0, Vh, sv.n, t0 * kQBC, Nk, tid);
  }

  // Q and dO as B operands of S^T = K Q^T and dP^T = V dO^T
  bf16x8 qf[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 a = {0, 0, 0, 0}, e = {0, 0, 0, 0};
    if (qrow < Nq) {
      a = *(const u32x4*)(Qg + b * sq.b + h * sq.h + (size_t)qrow * sq.n + ks * 16 + hi * 8);
      e = *(const u32x4*)(dOg + b * sdo.b + h * sdo.h + (size_t)qrow * sdo.n + ks * 16 + hi * 8);
    }
    qf[ks] = as_bf16x8(a);
    of[ks] = as_bf16x8(e);
  }
  // rows past Nq: L = +inf gives P = 0 (rows that see no key have L = -inf and
  // lie only in masked tiles, where P is set to 0)
  const float Lq = qrow < Nq ? LSEg[(size_t)bh * Nq + qrow] * kLog2e : INFINITY;
  // D = rowsum(dO o O) of this lane's row, from the half row of dO it holds
  // (lanes l and l + 32 hold the two halves); written for the dK/dV kernel,
  // which runs after this one
  float dpart = 0.f;
  if (qrow < Nq) {
    const uint16_t* orow = Og + b * so.b + h * so.h + (size_t)qrow * so.n + hi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 o = *(const u32x4*)(orow + ks * 16);
      const u32x4 e = __builtin_bit_cast(u32x4, of[ks]);
#pragma unroll
      for (int j = 0; j < 4; ++j) dpart += bf16_lo(o[j]) * bf16_lo(e[j]) + bf16_hi(o[j]) * bf16_hi(e[j]);
    }
  }
  const float Dq = dpart + __shfl_xor(dpart, 32);
  if (hi == 0 && qrow < Nq) Dg[(size_t)bh * Nq + qrow] = Dq;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  // LDS byte offsets of this lane's operands inside a tile. The swizzle of
  // toff<D> only flips bits that depend on the lane, so every operand address
  // is a tile base plus (lane offset XOR a constant of the loop indices):
  //   K / V operand (kb, ks): kb 64 D + (pk ^ 32 ks)
  //   K^T reads (kb, h2, db): (kb 32 + 16 h2) 2 D + (pt ^ 64 db), and for the
  //   rows 8 further: + 16 D + ((pt ^ 32) ^ 64 db)
  // (both identical to toff<D> for every lane and index; one instruction per
  // address instead of re-deriving the swizzle in every tile).
  auto lane_offsets = [](int ln, uint32_t& pk, uint32_t& pt) __attribute__((always_inline)) {
    const int l32_ = ln & 31, hi_ = ln >> 5, g_ = ln >> 4, i16_ = ln & 15;
    pk = 2u * (uint32_t)(l32_ * D + ((hi_ ^ swz2<D>(l32_)) << 3));
    const int z = 2 * (g_ & 1) + ((i16_ & 3) >> 1);
    const int wv = z ^ swz2<D>(4 * hi_ + (i16_ >> 2));
    pt = 2u * (uint32_t)((4 * hi_ + (i16_ >> 2)) * D + 4 * (i16_ & 1) + (wv << 3));
  };

  auto tile = [&](int t, const uint16_t* sK, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const uint32_t kbase = lds_addr(sK);  // V(t) sits 2 TILE elements after K(t)
    const int k0 = t * kQBC;
    // The lane index passes through an empty asm so that the LDS addresses
    // derived from it are formed inside the tile rather than hoisted out of
    // the loop for both tile variants (which would not fit in registers).
    // The causal instances up to d = 128 fit without it and run faster (the
    // addresses are then formed once, not per tile).
    constexpr bool PIN = !(CAUSAL && D <= 128);
    int lp = lane;
    if constexpr (PIN) asm volatile("" : "+v"(lp));
    const int l32 = lp & 31, hi = lp >> 5;
    uint32_t pk, pt;
    lane_offsets(lp, pk, pt);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // ---- S^T and dP^T for 32 keys (lane = query)
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t ka = kbase + kb * 64 * D + (pk ^ (32u * ks));
        const bf16x8 ak = as_bf16x8(lds_load16(ka));
        const bf16x8 av = as_bf16x8(lds_load16(ka + 4 * TILE));
        s = mfma_bf16_32x32x16(ak, qf[ks], s);
        dp = mfma_bf16_32x32x16(av, of[ks], dp);
      }
      // issue order: four operand reads ahead of their products
      if constexpr (D == 64 || (CAUSAL && D == 128)) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 2 * KS - 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
      // ---- dS^T = P^T o (dP^T - D), packed as the B operands of K^T dS^T
      u32x4 dsb[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        float ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * h2 + j;
          float arg = __builtin_fmaf(s[i], scale_log2, -Lq);
          if constexpr (ALIBI) {
            const float dist = (float)(k0 + kb * 32 + 4 * hi - qrow - band.off) + (float)(8 * (i / 4) + (i % 4));
            arg = __builtin_fmaf(nslope, __builtin_fabsf(dist), arg);
          }
          float pv = fast_exp2(arg);
          if constexpr (MASKED) {
            const int key = k0 + kb * 32 + 8 * (i / 4) + 4 * hi + (i % 4);
            if constexpr (BAND) {
              // this lane's visible keys are qr + off - wl .. qr + off + wr
              const int qr = qw0 + l32;
              if (key < qr + band.off - band.wl || key > qr + band.off + band.wr || key >= Nk) pv = 0.f;
            } else {
              if ((CAUSAL && key > qrow) || key >= Nk) pv = 0.f;
            }
          }
          ds[j] = pv * (dp[i] - Dq);
        }
        dsb[h2] = u32x4{pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]), pack_bf16x2(ds[4], ds[5]),
                        pack_bf16x2(ds[6], ds[7])};
      }
      // ---- dQ^T += K^T dS^T over two 16-key steps (K read transposed)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const uint32_t rb = kbase + (kb * 32 + 16 * h2) * 2 * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const i16x4 t0 = lds_read_tr16_at(rb + (pt ^ (64u * db)));
          const i16x4 t1 = lds_read_tr16_at(rb + 16 * D + ((pt ^ 32u) ^ (64u * db)));
          const u32x4 au = {__builtin_bit_cast(u32x2, t0)[0], __builtin_bit_cast(u32x2, t0)[1],
                            __builtin_bit_cast(u32x2, t1)[0], __builtin_bit_cast(u32x2, t1)[1]};
          acc[db] = mfma_bf16_32x32x16(as_bf16x8(au), as_bf16x8(dsb[h2]), acc[db]);
        }
      }
    }
  };

  // Tile t reads buffer (t - t0) % 2 and loads tile t+1 into the other.
  // Where registers allow (d = 64, and the causal instance at d = 128), the
  // loop is unrolled by two so that each buffer's base is a constant that
  // folds into the LDS instructions' offsets; elsewhere the base is chosen at
  // run time (one add per address: the unrolled form spills there).
  auto step = [&](int t, const uint16_t* sK, uint16_t* nK, uint16_t* nV) __attribute__((always_inline)) {
    wait_loads_and_sync();  // tile t landed; every wave finished tile t-1
    if (t + 1 < t1) {
      load_tile_async<D, kQBC, kQThreads, true>(nK, Kh, sk.n, (t + 1) * kQBC, Nk, tid);
      load_tile_async<D, kQBC, kQThreads, true>(nV, Vh, sv.n, (t + 1) * kQBC, Nk, tid);
    }
    if ((BAND && t < wfirst) || t > wlast) return;  // this wave's rows see none of these keys
    const int k0 = t * kQBC;
    // mask unless every row of this wave sees the whole tile
    bool masked;
    if constexpr (BAND)
      masked = !(k0 >= qw0 + 31 + band.off - band.wl && k0 + kQBC - 1 <= qw0 + band.off + band.wr && k0 + kQBC <= Nk);
    else
      masked = (CAUSAL && k0 + kQBC - 1 > qw0) || k0 + kQBC > Nk;
    if (masked)
      tile(t, sK, std::true_type{});
    else
      tile(t, sK, std::false_type{});
  };
  if constexpr (D == 64 || (CAUSAL && D == 128)) {
    int t = t0;
    for (; t + 1 < t1; t += 2) {
      step(t, sK0, sK1, sV1);
      step(t + 1, sK1, sK0, sV0);
    }
    if (t < t1) step(t, sK0, sK1, sV1);
  } else {
    for (int t = t0; t < t1; ++t) {
      const bool odd = (t - t0) & 1;
      step(t, odd ? sK1 : sK0, odd ? sK0 : sK1, odd ? sV0 : sV1);
    }
  }

  // ---- dQ = scale dQ^T^T, bf16 (lane = query, d over the accumulator rows)
  if (qrow < Nq) {
    uint16_t* row = dQg + b * sdq.b + h * sdq.h + (size_t)qrow * sdq.n;
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
  if constexpr (!XCD) break;
  __syncthreads();  // every wave is done with the LDS tiles before the next item's loads
  }  // items
}

// Workgroups of dq_kernel<D, MASK, NW, true> resident on the current device
// at once, looked up once per device.
template <int D, int MASK, int NW>
static int dq_resident_slots() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dq_kernel<D, MASK, NW, true>, NW * 64, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    v = per_cu * cus;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int D, int MASK, int NW>
static int launch_dq_nw(const BwdArgs& a) {
  const int BH = a.B * a.H;
  const int nqb = (a.Nq + NW * 32 - 1) / (NW * 32);
  const int blocks = nqb * BH;
  if constexpr (D == 128 && MASK == kMaskCausal) {
    const int slots = dq_resident_slots<D, MASK, NW>();
    const int g = slots > 0 ? std::min(blocks, slots) : blocks;
    if (g % 8 == 0 && BH % 8 == 0 && (g / 8) % nqb == 0) {
      hipLaunchKernelGGL((dq_kernel<D, MASK, NW, true>), dim3((unsigned)g), dim3(NW * 64), 0, (hipStream_t)a.stream,
                         a.q, a.k, a.v, a.dO, a.lse, a.o, a.delta, a.dq, BH, a.H, a.H / a.Hkv, a.Nq, a.Nk, nqb, a.scale,
                         a.scale * kLog2e, a.band, a.slopes, a.sq, a.sk, a.sv, a.sdo, a.so, a.sdq);
      return hipGetLastError() == hipSuccess ? 0 : 1;
    }
  }
  hipLaunchKernelGGL((dq_kernel<D, MASK, NW>), dim3((unsigned)blocks), dim3(NW * 64), 0, (hipStream_t)a.stream,
                     a.q, a.k, a.v, a.dO, a.lse, a.o, a.delta, a.dq, BH, a.H, a.H / a.Hkv, a.Nq, a.Nk, nqb, a.scale,
                     a.scale * kLog2e, a.band, a.slopes, a.sq, a.sk, a.sv, a.sdo, a.so, a.sdq);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <int D, int MASK>
static int launch_dq(const BwdArgs& a) {
  if constexpr (kQNWof<D> == 8 && MASK <= kMaskCausal) {
    if (a.Nk <= (MASK == kMaskNone ? kQShortKeys : kQShortKeysCausal)) return launch_dq_nw<D, MASK, 4>(a);
  }
  return launch_dq_nw<D, MASK, kQNWof<D>>(a);
}

template <int D>
static int launch_dq_d(const BwdArgs& a) {
  switch (mask_mode(a.band, a.slopes)) {
    case kMaskNone: return launch_dq<D, kMaskNone>(a);
    case kMaskCausal: return launch_dq<D, kMaskCausal>(a);
    case kMaskBand: return launch_dq<D, kMaskBand>(a);
    default: return launch_dq<D, kMaskBandAlibi>(a);
  }
}

int launch_bwd_dq(const BwdArgs& a) {
  if (a.d == 256) return launch_dq_d<256>(a);
  return a.d == 128 ? launch_dq_d<128>(a) : launch_dq_d<64>(a);
}

}  // namespace fa
