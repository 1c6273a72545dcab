// Kernels and launch templates of the bf16 backward (included by fa_bwd.hip,
// which instantiates d = 64 and 128, and by fa_bwd_d256.hip, which
// instantiates d = 256 and is built with the VGPR form of the MFMAs; see the
// register placement in dkdv_kernel). The method and the launch sequence are
// described at the top of fa_bwd.hip.
#pragma once

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "fa_bwd_tiles.h"
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kBKC = 128;  // dkdv: keys per workgroup (4 waves x 32)
constexpr int kBQ = 32;    // dkdv: query rows per step
constexpr int kKeyBlocksPersistent = 8;  // dkdv: persistent grid up to this many key blocks (1024 keys)

}  // namespace

using namespace bwd;

// ---------------------------------------------------------------------------
// dK, dV: key-stationary
// ---------------------------------------------------------------------------
// Masks as in the forward: query i sees keys i + off - wl .. i + off + wr of
// 0 .. Nk - 1; a key block visits only the query blocks whose band reaches it,
// and masks only steps that cut the band's edges. kMaskBandAlibi adds
// -slope_h |i + off - j| to the scaled scores; kMaskNone keeps the fixed
// arithmetic. (Causal runs as a band here: a causal-only instance compiled to
// a worse register allocation.)
//
// XCD (d = 128, no split, a causal-like band): the grid holds one workgroup
// per resident slot, and XCD x (workgroup j runs on XCD j % 8) takes the K/V
// heads x, x + 8, ...; its workgroups take a head's key blocks together, in
// chunks of min(key blocks, workgroups) per round, the chunk order reversed
// on odd rounds, so that each workgroup pairs a heavy (early) key block with
// a light one and the key blocks of a head read the same Q / dO tiles at
// about the same time. Otherwise one workgroup per key block: the loop below
// then runs once.
//
// Up to d = 64 a wave fits in 256 VGPRs with no AGPRs (two workgroups per
// CU). The launch bound says so: the compiler then gives every MFMA its VGPR
// form, and S and dP need no copies out of AGPRs before the vector work.
template <int D, int MASK, bool XCD = false>
__global__ void __launch_bounds__(256, D <= 64 ? 2 : 1)
dkdv_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg,
            const uint16_t* __restrict__ dOg, const float* __restrict__ LSEg, const float* __restrict__ Dg,
            uint16_t* __restrict__ dKg, uint16_t* __restrict__ dVg, float* __restrict__ part, int BHkv, int H,
            int group, int split, int Nq, int Nk, int nkb, float scale, float scale_log2, Band band,
            const float* __restrict__ slopes, Strides sq, Strides sk, Strides sv, Strides sdo, Strides sdk,
            Strides sdv) {
  constexpr int KS = D / 16;    // k-steps over d
  // dK / dV columns per workgroup: all of d up to 128; at d = 256 two
  // workgroups share a key block, each accumulating one half of the columns
  // (S and dP, which contract over all of d, are formed by both), so that the
  // accumulators and the K / V operands still fit in the 256 AGPRs.
  constexpr int DC = D == 256 ? 128 : D;
  constexpr int NH = D / DC;    // column halves per key block
  constexpr int DB = DC / 32;   // 32-wide d blocks of the accumulators
  constexpr int QT = kBQ * D;   // elements of a Q or dO tile
  static_assert(MASK != kMaskCausal, "causal runs as a band");
  constexpr bool BAND = MASK >= kMaskBand, ALIBI = MASK == kMaskBandAlibi;

  // Three buffers: while step j's dV / dK products read buffer j % 3 and step
  // j+1's S / dP products read buffer (j+1) % 3, step j+2 loads into the third.
  __shared__ __attribute__((aligned(16))) uint16_t sQ0[QT];
  __shared__ __attribute__((aligned(16))) uint16_t sQ1[QT];
  __shared__ __attribute__((aligned(16))) uint16_t sQ2[QT];
  __shared__ __attribute__((aligned(16))) uint16_t sO0[QT];
  __shared__ __attribute__((aligned(16))) uint16_t sO1[QT];
  __shared__ __attribute__((aligned(16))) uint16_t sO2[QT];
  __shared__ __attribute__((aligned(16))) float sLD0[2 * kBQ];
  __shared__ __attribute__((aligned(16))) float sLD1[2 * kBQ];
  __shared__ __attribute__((aligned(16))) float sLD2[2 * kBQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;

  // One K/V head's key blocks run together on one XCD, heaviest causal block
  // first. The block's keys serve the group's query heads hk * group + g;
  // with split > 1, workgroup si of the key block takes the gs = group / split
  // heads from hk * group + si * gs and leaves fp32 partials.
  const int xj = (int)blockIdx.x, xx = xj & 7, xGx = (int)gridDim.x >> 3;
  const int xitems = (BHkv >> 3) * nkb, xc = min(nkb, xGx);  // items of this XCD; a head's items per round
  for (int xu = xj >> 3, xk = 0;; xu += xGx, ++xk) {
  int wid;
  if constexpr (XCD) {  // split = 1, NH = 1: wid = bhk nkb + kblk
    if (xu >= xitems) break;
    const int r = xu % nkb, lc = xu % xc;
    wid = ((xu / nkb) * 8 + xx) * nkb + ((xk & 1) ? r - lc + (xc - 1 - lc) : r);
  } else {
    wid = xcd_work_id(nkb * BHkv * split * NH);
  }
  const int hc = wid % NH;        // column half
  const int dc0 = hc * DC;        // first dK / dV column of this workgroup
  const int unit = wid / NH / nkb;  // (bhk, si)
  const int kblk = (wid / NH) % nkb;
  const int bhk = unit / split, si = unit % split;
  const int Hkv = H / group, gs = group / split;
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int h0 = hk * group + si * gs;  // first query head of this workgroup
  const uint16_t* Kh = Kg + b * sk.b + hk * sk.h;
  const uint16_t* Vh = Vg + b * sv.b + hk * sv.h;
  const int kb0 = kblk * kBKC;
  const int kw0 = kb0 + w * 32;
  const int key_l = kw0 + (lane & 31);  // this lane's key in S / dP

  // Steps run over the query heads h0 .. h0 + gs - 1 in turn; within a head,
  // over the query blocks whose band reaches this key block, from the last
  // down (so that the concurrent key blocks of a head read the same Q / dO
  // tiles at about the same time).
  int qs_lo, nsq;  // first query block, query blocks per head
  if constexpr (BAND) {
    const int kblast = min(kb0 + kBKC, Nk) - 1;
    const int qa = max(0, kb0 - band.off - band.wr);          // first query seeing a key of the block
    const int qz = min(Nq - 1, kblast - band.off + band.wl);  // last such query
    qs_lo = qa / kBQ;
    nsq = qz >= qa ? qz / kBQ - qs_lo + 1 : 0;
  } else {
    qs_lo = 0;
    nsq = (Nq + kBQ - 1) / kBQ;
  }
  const int nsteps = nsq * gs;
  const int q_hi = (qs_lo + nsq - 1) * kBQ, q_lo = qs_lo * kBQ;

  if (BAND && nsteps == 0) {  // no query sees these keys: dK = dV = 0
    constexpr int CH = D / 8;
    constexpr int CC = DC / 8;
    for (int e = tid; e < kBKC * CC; e += 256) {
      const int key = kb0 + e / CC, c = dc0 + (e % CC) * 8;
      if (key >= Nk) continue;
      if (split == 1) {
        *(u32x4*)(dKg + b * sdk.b + hk * sdk.h + (size_t)key * sdk.n + c) = u32x4{0, 0, 0, 0};
        *(u32x4*)(dVg + b * sdv.b + hk * sdv.h + (size_t)key * sdv.n + c) = u32x4{0, 0, 0, 0};
      } else {
        float* pk = part + ((size_t)unit * Nk + key) * D + c;
        float* pv = pk + (size_t)BHkv * split * Nk * D;
        *(f32x4*)pk = f32x4{0.f, 0.f, 0.f, 0.f};
        *(f32x4*)(pk + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
        *(f32x4*)pv = f32x4{0.f, 0.f, 0.f, 0.f};
        *(f32x4*)(pv + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    if constexpr (XCD) continue;  // this item used no LDS; the next may load at once
    return;
  }
  // query block after q0 in step order (wrapping to the next head's last)
  auto next_q0 = [&](int q0) { return q0 == q_lo ? q_hi : q0 - kBQ; };
  // Buffer j % 3 of the three (chosen at run time: one set of lane offsets
  // then serves all three buffers).
  auto bufQ = [&](int j) -> uint16_t* { const int b = j % 3; return b == 0 ? sQ0 : (b == 1 ? sQ1 : sQ2); };
  auto bufO = [&](int j) -> uint16_t* { const int b = j % 3; return b == 0 ? sO0 : (b == 1 ? sO1 : sO2); };
  auto bufLD = [&](int j) -> float* { const int b = j % 3; return b == 0 ? sLD0 : (b == 1 ? sLD1 : sLD2); };
  // The loads walk the steps with a cursor (query block, head bases), which
  // spares a division per step.
  int ld_q0 = q_hi;
  const uint16_t* ld_q = Qg + b * sq.b + (long long)h0 * sq.h;
  const uint16_t* ld_o = dOg + b * sdo.b + (long long)h0 * sdo.h;
  size_t ld_row = ((size_t)b * H + h0) * Nq;  // LSE / D row of the head
  auto issue_loads = [&](int j) __attribute__((always_inline)) {
    load_tile_async<D, kBQ, 256, true>(bufQ(j), ld_q, sq.n, ld_q0, Nq, tid);
    load_tile_async<D, kBQ, 256, true>(bufO(j), ld_o, sdo.n, ld_q0, Nq, tid);
    if (w == 0) load_ld_async(bufLD(j), LSEg + ld_row, Dg + ld_row, ld_q0, Nq, lane);
    if (ld_q0 == q_lo) {
      ld_q += sq.h;
      ld_o += sdo.h;
      ld_row += Nq;
    }
    ld_q0 = next_q0(ld_q0);
  };
  // A step needs the mask when some (key, query) pair of this wave is not
  // visible: a band edge, a ragged query block, a ragged key block.
  auto needs_mask = [&](int q0) {
    if constexpr (BAND)
      return !(kw0 - band.off >= q0 + kBQ - 1 - band.wl && kw0 + 31 - band.off <= q0 + band.wr &&
               kw0 + 32 <= Nk && q0 + kBQ <= Nq);
    else
      return (kw0 + 32 > Nk) || (q0 + kBQ > Nq);
  };
  // the queries that see this lane's key: qmin_l .. qmax_l
  int qmin_l, qmax_l;
  if constexpr (BAND) {
    qmin_l = key_l - band.off - band.wr;
    qmax_l = key_l < Nk ? min(Nq - 1, key_l - band.off + band.wl) : -1;
  } else {
    qmin_l = 0;
    qmax_l = key_l < Nk ? Nq - 1 : -1;
  }

  issue_loads(0);
  if (nsteps > 1) issue_loads(1);

  // per-wave K and V as B operands of S = Q K^T and dP = dO V^T
  const int l32 = lane & 31, hi = lane >> 5, g = lane >> 4, i16 = lane & 15;
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 a = {0, 0, 0, 0}, c = {0, 0, 0, 0};
    if (key_l < Nk) {
      a = *(const u32x4*)(Kh + (size_t)key_l * sk.n + ks * 16 + hi * 8);
      c = *(const u32x4*)(Vh + (size_t)key_l * sv.n + ks * 16 + hi * 8);
    }
    kf[ks] = as_bf16x8(a);
    vf[ks] = as_bf16x8(c);
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) { dk[db] = f32x16{}; dv[db] = f32x16{}; }
  u32x4 pP[2], pS[2];  // P^T, dS^T of the step whose dV / dK products are next

  // ---- S = Q K^T and dP = dO V^T (lane = key, 16 queries per lane); the Q /
  // dO operands are read one k-step ahead
  auto s_dp = [&](const uint16_t* sQ, const uint16_t* sO, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
    s = f32x16{};
    dp = f32x16{};
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
  };
  // ---- P = exp2(S c - L log2 e) (ALiBi: minus slope |i + off - j| log2 e),
  // dS = P (dP - D), packed bf16 (masked entries: exponent -inf, P = 0); 4
  // queries (one g4 group) at a time
  auto p_ds_part = [&](const f32x16& s, const f32x16& dp, const float* sLD, int q0, float nslope, int g4,
                       u32x4* oP, u32x4* oS, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int qi = 8 * g4 + 4 * hi;
    const f32x4 L4 = *(const f32x4*)(sLD + qi);
    const f32x4 D4 = *(const f32x4*)(sLD + kBQ + qi);
    float p[4], ds[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * g4 + e;
      float arg = __builtin_fmaf(s[i], scale_log2, -L4[e] * kLog2e);
      if constexpr (ALIBI) {
        const float dist = (float)(q0 + qi + band.off - key_l) + (float)e;  // i + off - j
        arg = __builtin_fmaf(nslope, __builtin_fabsf(dist), arg);
      }
      if constexpr (MASKED) {
        const int q = q0 + qi + e;
        arg = (q < qmin_l || q > qmax_l) ? -INFINITY : arg;
      }
      p[e] = fast_exp2(arg);
      ds[e] = p[e] * (dp[i] - D4[e]);
    }
    oP[g4 >> 1][2 * (g4 & 1)] = pack_bf16x2(p[0], p[1]);
    oP[g4 >> 1][2 * (g4 & 1) + 1] = pack_bf16x2(p[2], p[3]);
    oS[g4 >> 1][2 * (g4 & 1)] = pack_bf16x2(ds[0], ds[1]);
    oS[g4 >> 1][2 * (g4 & 1) + 1] = pack_bf16x2(ds[2], ds[3]);
  };
  // ---- dV += P^T dO and dK += dS^T Q for one (s2, db): dO, Q read
  // transposed; the query order inside a k-step follows the accumulator layout
  // of S (slot 8 hi + j holds query 16 s2 + 8 (j / 4) + 4 hi + j % 4)
  auto dvdk_part = [&](const uint16_t* sQ, const uint16_t* sO, int s2, int db) __attribute__((always_inline)) {
    const int r0 = 16 * s2 + 4 * hi + (i16 >> 2);
    const int d = dc0 + db * 32 + 16 * (g & 1) + 4 * (i16 & 3);
    const u32x4 bo = tr_pair(sO + toff<D>(r0, d), sO + toff<D>(r0 + 8, d));
    const u32x4 bq = tr_pair(sQ + toff<D>(r0, d), sQ + toff<D>(r0 + 8, d));
    dv[db] = mfma_bf16_32x32x16(as_bf16x8(pP[s2]), as_bf16x8(bo), dv[db]);
    dk[db] = mfma_bf16_32x32x16(as_bf16x8(pS[s2]), as_bf16x8(bq), dk[db]);
  };
  // Register placement: the loop-invariant K / V operands and the dK / dV
  // accumulators are pinned at the loop boundaries. At d = 128 they go to
  // AGPRs (an MFMA reads its B operand and accumulator there directly); left
  // to itself the compiler moved the accumulators through VGPRs on every step
  // and kept no VGPRs free for reading LDS ahead. Up to d = 64 everything
  // stays in VGPRs (an AGPR constraint would switch every MFMA of the kernel
  // to its AGPR form and bring back the copies of S and dP). At d = 256 the
  // instances are built with every MFMA in its VGPR form (fa_bwd_d256.hip):
  // the accumulators, S and dP stay in VGPRs (no copies of S and dP), and the
  // K / V operands, which an MFMA also reads from AGPRs, are pinned there.
  auto pin_acc = [&]() __attribute__((always_inline)) {
    if constexpr (D == 256) {
#pragma unroll
      for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(dk[db]), "+v"(dv[db]));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+a"(kf[ks]), "+a"(vf[ks]));
    } else if constexpr (D <= 64) {
#pragma unroll
      for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(dk[db]), "+v"(dv[db]));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(kf[ks]), "+v"(vf[ks]));
    } else {
#pragma unroll
      for (int db = 0; db < DB; ++db) asm volatile("" : "+a"(dk[db]), "+a"(dv[db]));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+a"(kf[ks]), "+a"(vf[ks]));
    }
  };

  // ALiBi slope (negated, times log2 e) of the query head of a step
  auto slope_of = [&](int h) { return ALIBI ? -slopes[h] * kLog2e : 0.f; };

  // prologue: P, dS of step 0
  wait_loads_and_sync();
  {
    f32x16 s, dp;
    s_dp(sQ0, sO0, s, dp);
    const float ns = slope_of(h0);
    if (needs_mask(q_hi)) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) p_ds_part(s, dp, sLD0, q_hi, ns, g4, pP, pS, std::true_type{});
    } else {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) p_ds_part(s, dp, sLD0, q_hi, ns, g4, pP, pS, std::false_type{});
    }
  }

  // Iteration j: S / dP of step j+1, then the dV / dK products of step j with
  // the P / dS work of step j+1 interleaved between them (matrix core and
  // vector ALU busy at once); the loads of step j+2 go to the third buffer
  // meanwhile.
  auto iteration = [&](int j, int nq0, float ns, auto masked_tag) __attribute__((always_inline)) {
    f32x16 s, dp;
    s_dp(bufQ(j + 1), bufO(j + 1), s, dp);
    u32x4 nP[2], nS[2];
    const float* nLD = bufLD(j + 1);
    const uint16_t* cQ = bufQ(j);
    const uint16_t* cO = bufO(j);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dvdk_part(cQ, cO, s2, db);
        const int part = s2 * DB + db;  // spread the four P / dS groups evenly
        if (part % (2 * DB / 4) == 0) p_ds_part(s, dp, nLD, nq0, ns, part / (2 * DB / 4), nP, nS, masked_tag);
      }
    }
    pP[0] = nP[0];
    pP[1] = nP[1];
    pS[0] = nS[0];
    pS[1] = nS[1];
    // Issue order (one wave per SIMD, so the order is the overlap): the S / dP
    // products each with up to three LDS reads (their operand and the
    // transposed reads of the dV / dK products, read well ahead of use), then
    // the dV / dK products with seven vector instructions of P / dS work after
    // each.
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);   // VALU
    }
  };
  int nq0 = q_hi;  // query block and head of step j + 1 (after the update below)
  int nh = h0;
  for (int j = 0; j + 1 < nsteps; ++j) {
    pin_acc();
    wait_loads_and_sync();  // step j+1 landed; every wave is done with step j-1's buffer
    if (j + 2 < nsteps) issue_loads(j + 2);
    if (ALIBI && nq0 == q_lo) ++nh;
    nq0 = next_q0(nq0);
    const float ns = slope_of(nh);
    if (needs_mask(nq0))
      iteration(j, nq0, ns, std::true_type{});
    else
      iteration(j, nq0, ns, std::false_type{});
    pin_acc();
  }
  // last step: dV / dK only
  wait_loads_and_sync();
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int db = 0; db < DB; ++db) dvdk_part(bufQ(nsteps - 1), bufO(nsteps - 1), s2, db);

  // ---- dK (times scale) and dV, bf16 (lane = d column, 16 keys per lane);
  // with split > 1, the unscaled fp32 sums into this workgroup's partials
  if (split == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = dc0 + db * 32 + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kw0 + 8 * (i / 4) + 4 * hi + (i % 4);
        if (key < Nk) {
          dKg[b * sdk.b + hk * sdk.h + (size_t)key * sdk.n + d] =
              (uint16_t)(pack_bf16x2(dk[db][i] * scale, 0.f) & 0xffffu);
          dVg[b * sdv.b + hk * sdv.h + (size_t)key * sdv.n + d] = (uint16_t)(pack_bf16x2(dv[db][i], 0.f) & 0xffffu);
        }
      }
    }
  } else {
    float* pk = part + (size_t)unit * Nk * D;
    float* pv = pk + (size_t)BHkv * split * Nk * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = dc0 + db * 32 + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kw0 + 8 * (i / 4) + 4 * hi + (i % 4);
        if (key < Nk) {
          pk[(size_t)key * D + d] = dk[db][i];
          pv[(size_t)key * D + d] = dv[db][i];
        }
      }
    }
  }
  if constexpr (!XCD) break;
  __syncthreads();  // every wave is done with the LDS tiles before the next item's loads
  }  // items
}

// Workgroups of dkdv_kernel<D, MASK, true> resident on the current device at
// once, looked up once per device.
template <int D, int MASK>
static int dkdv_resident_slots() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dkdv_kernel<D, MASK, true>, 256, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    v = per_cu * cus;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// dK = scale * (sum of the split partials), dV = sum, to bf16 views. One
// thread per 8 consecutive elements of a (batch, K/V head, key) row.
template <int D>
__global__ void __launch_bounds__(256)
kv_reduce_kernel(const float* __restrict__ part, uint16_t* __restrict__ dKg, uint16_t* __restrict__ dVg,
                 long long rows, int Hkv, int split, int N, float scale, Strides sdk, Strides sdv) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  if (row >= rows) return;
  const int c = threadIdx.x % LPR;
  const long long bhk = row / N;
  const int n = (int)(row % N), b = (int)(bhk / Hkv), hk = (int)(bhk % Hkv);
  const size_t half = (size_t)rows * split * D;  // dV partials follow the dK partials
  float sk[8] = {}, sv[8] = {};
  for (int si = 0; si < split; ++si) {
    const float* src = part + ((size_t)(bhk * split + si) * N + n) * D + c * 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 a = *(const f32x4*)(src + 4 * h);
      const f32x4 e = *(const f32x4*)(src + half + 4 * h);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sk[4 * h + j] += a[j];
        sv[4 * h + j] += e[j];
      }
    }
  }
  u32x4 ok, ov;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ok[j] = pack_bf16x2(sk[2 * j] * scale, sk[2 * j + 1] * scale);
    ov[j] = pack_bf16x2(sv[2 * j], sv[2 * j + 1]);
  }
  *(u32x4*)(dKg + b * sdk.b + hk * sdk.h + (long long)n * sdk.n + c * 8) = ok;
  *(u32x4*)(dVg + b * sdv.b + hk * sdv.h + (long long)n * sdv.n + c * 8) = ov;
}



template <int D, int MASK>
static int launch(const BwdArgs& a) {
  hipStream_t st = (hipStream_t)a.stream;
  constexpr int RPB = 256 / (D / 8);
  // dQ first: its kernel also forms D = rowsum(dO o O) of every query row and
  // writes it to the workspace, where the dK/dV kernel reads it
  if (launch_bwd_dq(a) != 0) return 1;
  const int nkb = bwd_key_blocks(a.Nk);
  static_assert(kBKC == 128, "bwd_key_blocks assumes 128-key blocks");
  const int BHkv = a.B * a.Hkv;
  const int blocks = nkb * BHkv * a.split * (D == 256 ? 2 : 1);
  bool launched = false;
  if constexpr (D == 128 && MASK != kMaskNone) {
    // Short keys under a causal-like band (each query sees every earlier key):
    // key blocks differ in cost, and each workgroup has few steps. Measured
    // (causal, whole fa_bwd): 9.5% faster at N = 512, 5% at 1024, but 2.5%
    // slower at 2048 and 10% at 4096 (the loop's live state puts the kernel at
    // 256 VGPRs with spilled SGPRs); at d = 64 it would cost the second
    // workgroup per CU.
    if (a.split == 1 && nkb <= kKeyBlocksPersistent && a.band.wl >= a.Nk && a.band.wr < a.Nk) {
      const int slots = dkdv_resident_slots<D, MASK>();
      const int g = slots > 0 ? std::min(blocks, slots) : blocks, gx = g / 8;
      if (g % 8 == 0 && BHkv % 8 == 0 && gx > 0 && (nkb % gx == 0 || gx % nkb == 0)) {
        hipLaunchKernelGGL((dkdv_kernel<D, MASK, true>), dim3((unsigned)g), dim3(256), 0, st, a.q, a.k, a.v, a.dO,
                           a.lse, a.delta, a.dk, a.dv, a.part, BHkv, a.H, a.H / a.Hkv, a.split, a.Nq, a.Nk, nkb,
                           a.scale, a.scale * kLog2e, a.band, a.slopes, a.sq, a.sk, a.sv, a.sdo, a.sdk, a.sdv);
        launched = true;
      }
    }
  }
  if (!launched)
    hipLaunchKernelGGL((dkdv_kernel<D, MASK>), dim3((unsigned)blocks), dim3(256), 0, st, a.q, a.k, a.v, a.dO,
                       a.lse, a.delta, a.dk, a.dv, a.part, BHkv, a.H, a.H / a.Hkv, a.split, a.Nq, a.Nk, nkb,
                       a.scale, a.scale * kLog2e, a.band, a.slopes, a.sq, a.sk, a.sv, a.sdo, a.sdk, a.sdv);
  if (hipGetLastError() != hipSuccess) return 1;
  if (a.split > 1) {
    const long long kv_rows = (long long)BHkv * a.Nk;
    hipLaunchKernelGGL((kv_reduce_kernel<D>), dim3((unsigned)((kv_rows + RPB - 1) / RPB)), dim3(256), 0, st,
                       a.part, a.dk, a.dv, kv_rows, a.Hkv, a.split, a.Nk, a.scale, a.sdk, a.sdv);
    if (hipGetLastError() != hipSuccess) return 1;
  }
  return 0;
}

template <int D>
static int launch_d(const BwdArgs& a) {
  switch (mask_mode(a.band, a.slopes)) {
    case kMaskNone: return launch<D, kMaskNone>(a);
    case kMaskCausal:  // the band instance (see dkdv_kernel)
    case kMaskBand: return launch<D, kMaskBand>(a);
    default: return launch<D, kMaskBandAlibi>(a);
  }
}

}  // namespace fa
