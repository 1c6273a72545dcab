// fa_fwd: bf16 exact attention forward for gfx950 (MI355X).
//
// Method ([HUB] "How it works"; [LIB] "The trick that made it all possible:
// online softmax"; [LIN] "FA2 (2023)"): one workgroup per (batch, head,
// 256-row Q-block); each of its eight wavefronts owns 32 query rows
// (split-Q), streams 64-key K/V tiles through LDS, forms the score tile on
// chip with bf16 MFMA (fp32 accumulation), keeps the running max m and sum l
// per query in registers, rescales the output accumulator only when some
// row's max grew by more than a fixed slack ([LIB] "FA4": skip the rescale
// unless the max changes significantly; exact, since O and l share the same
// stale max), and divides by l once at the end, saving LSE = m + log l.
//
// Orientation: each wave computes S^T = K Q^T so that MFMA accumulator
// columns are queries: a lane owns one query, the row max and row sum are
// lane-local apart from one exchange with the other half of the wave, and the
// per-query rescale of O^T = V^T P^T is lane-local too. P^T leaves the
// accumulators already in the B-operand layout of the P V product; V^T comes
// from LDS through transposed 16-bit reads.
//
// Overlap: two wavefronts per SIMD, so one wave's softmax (VALU) runs while
// the other's products occupy the matrix core; K/V tiles arrive by direct
// global->LDS loads into double buffers while the current tile is consumed,
// with one barrier per tile.
#include <algorithm>
#include <atomic>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

// Wavefronts per workgroup: eight (two per SIMD, so that one wave's softmax
// overlaps another's products) up to d = 128; four at d = 256, where a wave
// needs more than the 256 registers of two-per-SIMD residency. At d <= 128
// shorter key ranges use four-wave workgroups too (two workgroups per CU,
// each wave still at two per SIMD): when every workgroup has only a few
// tiles, one workgroup's loads, prologue and epilogue overlap another's
// tiles, and under a mask the smaller Q-blocks split the uneven work more
// evenly. These four-wave grids are persistent (see DEAL below). Measured:
// faster up to 1024 keys without a mask and up to 4096 with one, and at
// d = 64 under a mask at every length; slower beyond at d = 128 (the
// eight-wave blocks read each K/V tile from HBM or L2 for twice as many
// rows).
template <int D>
constexpr int kNWof = D == 256 ? 4 : 8;
constexpr int kQW = 32;   // query rows per wavefront
constexpr int kShortKeys = 1024;        // four-wave workgroups up to this many keys without a mask,
constexpr int kShortKeysMasked = 4096;  // and up to this many under a mask
constexpr int kBC = 64;   // keys per tile
// Work dealing of the forward grid: one item per workgroup, or persistent
// workgroups with a fixed list of items each (see the kernel).
constexpr int kDealOne = 0, kDealFalling = 1, kDealByXcd = 2;
#ifndef FA_RESCALE_SLACK
#define FA_RESCALE_SLACK 8.0f
#endif
constexpr float kRescaleSlack = FA_RESCALE_SLACK;  // log2 units; P stays <= 256 in bf16

// Direct global->LDS loads of one [64 x D] bf16 tile. Thread `tid` fills the
// 16-byte LDS chunks n * 64 NW + tid of the tile; the source chunk is chosen
// so that LDS holds the XOR-swizzled layout. Rows past the end are read from
// row N-1 (finite values that are masked, or multiplied by P = 0).
//
// Up to d = 128 a thread's byte offsets (r rs + 8 c) 2 inside a tile are
// formed once (TileLanes), and a full tile is loaded from the uniform base
// head + k0 rs with those offsets: one load instruction per chunk and no
// per-lane address arithmetic. That needs 64 rs 2 < 2^32 (row strides below
// 2^25 elements); the last, ragged tile and larger strides take the general
// form, which clamps each row and forms its 64-bit address.
template <int D, bool IS_V, int NW>
struct TileLanes {
  static constexpr bool kOn = D <= 128;
  static constexpr int kN = kOn ? (kBC * (D / 8)) / (NW * 64) : 1;
  uint32_t off[kN];
  __device__ __forceinline__ void init(long long rs, int tid) {
    if constexpr (kOn) {
      constexpr int CH = D / 8;
#pragma unroll
      for (int n = 0; n < kN; ++n) {
        const int e = n * NW * 64 + tid;
        const int r = e / CH, p = e % CH;
        const int c = p ^ (IS_V ? swz_v<D>(r) : swz_k<D>(r));
        off[n] = (uint32_t)(((uint64_t)r * (uint64_t)rs + (uint64_t)(c * 8)) * 2u);
      }
    }
  }
};

template <int D, bool IS_V, int NW>
__device__ __forceinline__ void load_tile_async(uint16_t* lds_tile, const uint16_t* head, long long rs, int k0,
                                                int N, int tid, const TileLanes<D, IS_V, NW>& tl, bool small_rs) {
  constexpr int CH = D / 8;
  const int w = tid >> 6;
  constexpr int kThreads = NW * 64;
  if (TileLanes<D, IS_V, NW>::kOn && small_rs && k0 + kBC <= N) {
    const uint16_t* base = head + (uint64_t)(uint32_t)k0 * (uint32_t)rs;  // the tile's first row
    const uint32_t lds = lds_addr(lds_tile) + (uint32_t)__builtin_amdgcn_readfirstlane(w) * 1024u;
#pragma unroll
    for (int n = 0; n < TileLanes<D, IS_V, NW>::kN; ++n) lds_dma16_sbase(lds + n * kThreads * 16, base, tl.off[n]);
    return;
  }
#pragma unroll
  for (int n = 0; n < (kBC * CH) / kThreads; ++n) {
    const int e = n * kThreads + tid;  // 16-byte chunk index inside the tile
    const int r = e / CH, p = e % CH;
    const int c = p ^ (IS_V ? swz_v<D>(r) : swz_k<D>(r));
    const int row = min(k0 + r, N - 1);
    const uint16_t* src = head + (uint64_t)(uint32_t)row * (uint32_t)rs + c * 8;  // rs < 2^31
    lds_dma16(lds_tile + (n * kThreads + w * 64) * 8, src);  // lane l lands at +16 l bytes
  }
}

__device__ __forceinline__ void wait_loads_and_sync() {
  wait_vmem_all();
  __syncthreads();
}

}  // namespace

// Masks: query i sees keys i + off - wl .. i + off + wr of 0 .. Nk - 1 (the
// band; causal, sliding windows and cross-attention are all bands). Tiles
// outside a Q-block's band are never loaded, tiles outside a wave's band are
// skipped, and only tiles that cut the band's edges (or the end of the keys)
// are masked element by element. With ALiBi (kMaskBandAlibi) the scaled
// score of query i and key j gets -slope_h |i + off - j|. kMaskNone and
// kMaskCausal are the no-mask and plain causal bands with fixed arithmetic.
//
// DEAL: kDealOne launches one workgroup per item (one Q-block of one head).
// At d <= 128 the four-wave instances (short key ranges) and the eight-wave
// instances under a mask are persistent: the grid holds only as many
// workgroups as fit on the chip at once, and each runs a fixed list of items
// one after another (a barrier between them, before the next item's loads
// reuse the LDS buffers). With one workgroup per item the dispatcher starts
// items of mixed cost as slots free up and, at short lengths, the slots sit
// idle a third of the time; the fixed lists even out the causal costs, and
// kDealByXcd keeps the Q-blocks of a head together in time on one XCD, so
// that their K / V re-reads hit its L2 (kDealFalling where it cannot).
template <int D, int MASK, int NW, int DEAL>
__global__ void __launch_bounds__(NW * 64, (D <= 128 && NW == 4) ? 2 : 1)
fwd_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
           const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og, float* __restrict__ LSEg,
           int BH, int H, int group, int Nq, int Nk, int nqb, float scale_log2, Band band,
           const float* __restrict__ slopes, Strides sq, Strides sk, Strides sv, Strides so) {
  constexpr int KS = D / 16;        // k-steps of the S product
  constexpr int DB = D / 32;        // 32-row d blocks of O^T
  constexpr int TILE = kBC * D;     // elements of one K or V tile
  constexpr bool BAND = MASK >= kMaskBand, CAUSAL = MASK == kMaskCausal, ALIBI = MASK == kMaskBandAlibi;
  constexpr int kBR = NW * kQW;  // query rows per workgroup

  // Four separate arrays so that the compiler can tell the buffer being filled
  // by the direct loads from the one being read.
  __shared__ __attribute__((aligned(16))) uint16_t sK0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[TILE];

  const int tid = threadIdx.x;
  // the wave index is uniform: readfirstlane lets every per-wave bound live in
  // scalar registers and keeps the per-tile branches uniform
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), l32 = lane & 31, hi = lane >> 5;
  const int g = lane >> 4, i16 = lane & 15;

  // Work id: one head's Q-blocks run together on one XCD (blocks are dispatched
  // round-robin over the 8 XCDs) so its K/V stay in that XCD's L2; inside a
  // head, the last Q-blocks (the heaviest under a causal band) go first.
  const int total = nqb * BH;
  // lane offsets of the K / V tile loads, and whether the row strides allow them
  TileLanes<D, false, NW> klanes;
  TileLanes<D, true, NW> vlanes;
  klanes.init(sk.n, tid);
  vlanes.init(sv.n, tid);
  const bool small_rs = sk.n < (1LL << 25) && sv.n < (1LL << 25);
  // Key tiles t0 .. t1 - 1 that hold the band of the rows of Q-block qblk.
  auto block_tiles = [&](int qblk, int& t0, int& t1) __attribute__((always_inline)) {
    const int q0 = qblk * kBR;
    if constexpr (BAND) {
      const int qlast = min(q0 + kBR, Nq) - 1;
      const int blo = max(0, q0 + band.off - band.wl);
      const int bhi = min(Nk - 1, qlast + band.off + band.wr);
      t0 = blo / kBC;
      t1 = bhi >= blo ? bhi / kBC + 1 : t0;
    } else {
      const int kend = CAUSAL ? min(Nk, q0 + kBR) : Nk;
      t0 = 0;
      t1 = (kend + kBC - 1) / kBC;
    }
  };
  auto item_qblk = [&](int wid) { return MASK != kMaskNone ? nqb - 1 - (wid % nqb) : (wid % nqb); };
  // One work item: Q-block item_qblk(wid) of head wid / nqb.
  auto run_item = [&](int wid) __attribute__((always_inline)) {
  const int bh = wid / nqb;
  const int qblk = item_qblk(wid);
  const int b = bh / H, h = bh % H, hk = h / group;  // query head h reads K/V head h / group
  const uint16_t* Qh = Qg + b * sq.b + h * sq.h;
  const uint16_t* Kh = Kg + b * sk.b + hk * sk.h;
  const uint16_t* Vh = Vg + b * sv.b + hk * sv.h;
  const int q0 = qblk * kBR;
  const int qw0 = q0 + w * kQW;  // first query row of this wave
  const int qrow = qw0 + l32;    // this lane's query

  // Key tiles t0 .. t1 - 1 hold the band of the block's rows; this wave's rows
  // need tiles wfirst .. wlast of them (none when its rows are all past Nq).
  int t0, t1, wfirst = 0, wlast, klo = 0, khi = 0;
  block_tiles(qblk, t0, t1);
  if constexpr (BAND) {
    const int wqlast = min(qw0 + kQW, Nq) - 1;
    const int wlo = max(0, qw0 + band.off - band.wl);
    const int whi = min(Nk - 1, wqlast + band.off + band.wr);
    wfirst = wlo / kBC;
    wlast = (wqlast >= qw0 && whi >= wlo) ? whi / kBC : -1;
    klo = qrow + band.off - band.wl;  // this lane's visible keys
    khi = min(Nk - 1, qrow + band.off + band.wr);
  } else {
    wlast = CAUSAL ? min(t1 - 1, (qw0 + kQW - 1) / kBC) : t1 - 1;  // causal: the diagonal tile
  }
  float nslope = 0.f;  // ALiBi slope times log2 e, negated
  if constexpr (ALIBI) nslope = -slopes[h] * kLog2e;

  if (t1 > t0) {
    load_tile_async<D, false, NW>(sK0, Kh, sk.n, t0 * kBC, Nk, tid, klanes, small_rs);
    load_tile_async<D, true, NW>(sV0, Vh, sv.n, t0 * kBC, Nk, tid, vlanes, small_rs);
  }


  // Q as the B operand of S^T = K Q^T: lane holds Q[q][16 ks + 8 hi .. +7].
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 u = {0, 0, 0, 0};
    if (qrow < Nq) u = *(const u32x4*)(Qh + (size_t)qrow * sq.n + ks * 16 + hi * 8);
    qf[ks] = as_bf16x8(u);
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  // Under a general band m starts finite so that a row whose first tiles are
  // all masked keeps p = exp2(-inf - m) = 0 (no inf - inf) until it sees a
  // key; otherwise every row sees a key in its first tile.
  float m = BAND ? -1e30f : -INFINITY, l = 0.f;

  // One tile: K(t), V(t) are in (sK, sV); the loads of tile t+1 go to (nK, nV).
  const int lane_l32 = l32, lane_hi = hi, lane_g = g, lane_i16 = i16;
  // Up to d = 128, the LDS byte offsets of this lane's operand reads inside a
  // tile, computed once: the swizzles depend only on lane bits once the row
  // offsets of the 32-key blocks and 16-key steps (multiples of 16 rows) are
  // taken out, so every read in the tile is a buffer constant plus one of
  // these (K: one per k-step; V^T: one per 32-row d block, the row 8 further
  // down at a constant distance).
  constexpr bool HOIST = D <= 128;
  uint32_t koff[HOIST ? KS : 1], voff[HOIST ? DB : 1];
  if constexpr (HOIST) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = (uint32_t)(l32 * D + (((2 * ks + hi) ^ swz_k<D>(l32)) * 8)) * 2u;
    const int rv = 4 * hi + (i16 >> 2);  // row of the V^T read within its 16-key step
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = db * 32 + 16 * (g & 1) + 4 * (i16 & 3);
      voff[db] = (uint32_t)(rv * D + (((d >> 3) ^ swz_v<D>(rv)) * 8) + (d & 7)) * 2u;
    }
  }
  auto tile = [&](int t, const uint16_t* sK, const uint16_t* sV, uint16_t* nK, uint16_t* nV) {
    wait_loads_and_sync();  // tile t landed; every wave finished tile t-1
    if (t + 1 < t1) {
      load_tile_async<D, false, NW>(nK, Kh, sk.n, (t + 1) * kBC, Nk, tid, klanes, small_rs);
      load_tile_async<D, true, NW>(nV, Vh, sv.n, (t + 1) * kBC, Nk, tid, vlanes, small_rs);
    }
    if ((BAND && t < wfirst) || t > wlast) return;  // this wave's rows see none of these keys
    const int k0 = t * kBC;
    // At d = 256 the lane index passes through an empty asm so that the LDS
    // addresses derived from it are formed here rather than hoisted out of the
    // tile loop (64 of them would not fit in registers). Not in the ALiBi
    // instance: built that way, its element mask came out wrong on band-edge
    // tiles handled by the second of the two unrolled copies of this body,
    // only with a window and ALiBi together (the source is equivalent; the
    // generated code is at fault). Without the asm it is right, at the cost
    // of a few spilled registers.
    constexpr bool PIN = D == 256 && !ALIBI;
    int lp = lane;
    if constexpr (PIN) asm volatile("" : "+v"(lp));
    const int l32 = PIN ? (lp & 31) : lane_l32, hi = PIN ? (lp >> 5) : lane_hi;
    const int g = PIN ? (lp >> 4) : lane_g, i16 = PIN ? (lp & 15) : lane_i16;

    // ---- S^T = K Q^T: two 32-key blocks (K operands read one k-step ahead)
    f32x16 s[2];
    s[0] = f32x16{};
    s[1] = f32x16{};
    bf16x8 a[2], an[2];
    const uint32_t kbase = lds_addr(sK), vbase = lds_addr(sV);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int r = kb * 32 + l32;
      if constexpr (HOIST)
        a[kb] = as_bf16x8(lds_load16(kbase + kb * 32 * D * 2 + koff[0]));
      else
        a[kb] = as_bf16x8(*(const u32x4*)(sK + r * D + ((hi ^ swz_k<D>(r)) * 8)));
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int r = kb * 32 + l32;
          const int c = (ks + 1) * 2 + hi;
          if constexpr (HOIST)
            an[kb] = as_bf16x8(lds_load16(kbase + kb * 32 * D * 2 + koff[ks + 1]));
          else
            an[kb] = as_bf16x8(*(const u32x4*)(sK + r * D + ((c ^ swz_k<D>(r)) * 8)));
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma_bf16_32x32x16(a[kb], qf[ks], s[kb]);
      if (ks + 1 < KS) {
        a[0] = an[0];
        a[1] = an[1];
      }
    }
    // issue order: four K operand reads ahead of their products
    {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * KS - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    // ---- ALiBi: scores to the exp2 domain with the bias, -slope |i + off - j|
    if constexpr (ALIBI) {
      const float fb = (float)(k0 + 4 * hi - qrow - band.off);  // j - (i + off) of element 0
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[kb][i] = __builtin_fmaf(s[kb][i], scale_log2,
                                    nslope * __builtin_fabsf(fb + (float)(kb * 32 + 8 * (i / 4) + (i % 4))));
    }
    // ---- online softmax (lane-local plus one half-wave exchange); mask only
    // tiles that some row of this wave does not see whole
    bool masked;
    if constexpr (BAND)
      masked = !(k0 >= qw0 + kQW - 1 + band.off - band.wl && k0 + kBC - 1 <= qw0 + band.off + band.wr &&
                 k0 + kBC <= Nk);
    else
      masked = (CAUSAL && k0 + kBC - 1 > qw0) || (k0 + kBC > Nk);
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + 8 * (i / 4) + 4 * hi + (i % 4);
          if (BAND ? (key < klo || key > khi) : ((CAUSAL && key > qrow) || key >= Nk)) s[kb][i] = -INFINITY;
        }
    }
    float mx = max_of_32(s[0], s[1]);
    mx = fmaxf(mx, other_half(mx));
    if constexpr (!ALIBI) mx *= scale_log2;
    // The running max is replaced (and O, l rescaled) only when some row's max
    // exceeds it by more than kRescaleSlack: until then p <= 2^kRescaleSlack,
    // and O and l share the same stale max, so O / l and the LSE are unchanged.
    // A row that has seen no key yet has mx = -inf and keeps m.
    if (__any(mx > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);
      l *= alpha;
      // At d = 256, O^T lives in AGPRs. The pin keeps the copies out to VGPRs
      // (and back) that the multiply needs inside this rarely taken branch;
      // without it the compiler read all 128 registers out on every tile.
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if constexpr (D == 256) asm volatile("" : "+a"(acc[db]));
        acc[db] *= alpha;
      }
      m = m_new;
    }
    float rs4[4] = {0.f, 0.f, 0.f, 0.f};  // row sum in four chains (shorter dependences)
    u32x4 pb[2][2];  // [kb][16-key step]: bf16x8 B operands of P V
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if constexpr (ALIBI)
            p[j] = fast_exp2(s[kb][8 * h2 + j] - m);
          else
            p[j] = fast_exp2(__builtin_fmaf(s[kb][8 * h2 + j], scale_log2, -m));
          rs4[j & 3] += p[j];
        }
        pb[kb][h2] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                           pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
      }
    }
    l += (rs4[0] + rs4[1]) + (rs4[2] + rs4[3]);

    // ---- O^T += V^T P^T over four 16-key steps
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int r0 = kb * 32 + 16 * h2 + 4 * hi + (i16 >> 2);
        const int r1 = r0 + 8;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = db * 32 + 16 * (g & 1) + 4 * (i16 & 3);
          const int c = d >> 3, within = d & 7;
          i16x4 t0, t1;
          if constexpr (HOIST) {
            const uint32_t a0 = vbase + (kb * 32 + 16 * h2) * D * 2 + voff[db];
            t0 = lds_read_tr16_at(a0);
            t1 = lds_read_tr16_at(a0 + 8 * D * 2);
          } else {
            t0 = lds_read_tr16(sV + r0 * D + ((c ^ swz_v<D>(r0)) * 8) + within);
            t1 = lds_read_tr16(sV + r1 * D + ((c ^ swz_v<D>(r1)) * 8) + within);
          }
          const u32x4 au = {__builtin_bit_cast(u32x2, t0)[0], __builtin_bit_cast(u32x2, t0)[1],
                            __builtin_bit_cast(u32x2, t1)[0], __builtin_bit_cast(u32x2, t1)[1]};
          acc[db] = mfma_bf16_32x32x16(as_bf16x8(au), as_bf16x8(pb[kb][h2]), acc[db]);
        }
      }
    }
  };

  int t = t0;
  for (; t + 1 < t1; t += 2) {
    tile(t, sK0, sV0, sK1, sV1);
    tile(t + 1, sK1, sV1, sK0, sV0);
  }
  if (t < t1) tile(t, sK0, sV0, sK1, sV1);

  // ---- epilogue: divide once by l, store O (bf16) and LSE (natural log); a
  // row that saw no key stores O = 0 and LSE = -inf
  const float lt = l + other_half(l);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (qrow < Nq) {
    uint16_t* orow = Og + b * so.b + h * so.h + (size_t)qrow * so.n;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hi;
        const u32x2 pk = {pack_bf16x2(acc[db][4 * g4 + 0] * inv, acc[db][4 * g4 + 1] * inv),
                          pack_bf16x2(acc[db][4 * g4 + 2] * inv, acc[db][4 * g4 + 3] * inv)};
        *(u32x2*)(orow + d) = pk;
      }
    if (hi == 0) LSEg[(size_t)bh * Nq + qrow] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  }
  };  // run_item

  if constexpr (DEAL == kDealByXcd) {
    // XCD x (workgroup j runs on XCD j % 8) takes heads x, x + 8, ..., and
    // its G / 8 workgroups take them nqb items at a time, so all Q-blocks of
    // a head run at once on one XCD and read each K / V tile from its L2 at
    // about the same time. Odd rounds reverse the Q-block order inside each
    // head, so that over two rounds every workgroup does one heavy and one
    // light block under a causal band. The host picks this dealing only when
    // every round holds whole heads (nqb divides G / 8) and every XCD as many
    // heads (8 divides BH, G a multiple of 8).
    const int j = (int)blockIdx.x, x = j & 7, s = j >> 3, Gx = (int)gridDim.x >> 3;
    const int items = (BH >> 3) * nqb;  // items of this XCD
    for (int u = s, k = 0; u < items; u += Gx, ++k) {
      const int qb = (k & 1) ? nqb - 1 - u % nqb : u % nqb;
      run_item(((u / nqb) * 8 + x) * nqb + qb);  // under a mask: Q-block nqb - 1 - qb
      __syncthreads();  // every wave is done with the LDS tiles before the next item's loads
    }
  } else if constexpr (DEAL == kDealFalling) {
    // Items in falling cost (Q-block major across heads under a mask), dealt
    // in rounds of G: even rounds to workgroups 0 .. G-1, odd rounds in
    // reverse by groups of 8 (a workgroup keeps its place in its group, i.e.
    // its XCD), which evens out the sums; odd workgroups take their rounds
    // from the last, so that workgroups sharing a CU are not in one phase.
    const int G = (int)gridDim.x, j = (int)blockIdx.x;
    const int R = (total + G - 1) / G;
    for (int k = 0; k < R; ++k) {
      const int r = (j & 1) ? R - 1 - k : k;
      const int jj = (r & 1) && (G & 7) == 0 ? ((G >> 3) - 1 - (j >> 3)) * 8 + (j & 7) : j;
      const int i = r * G + jj;
      if (i >= total) continue;
      const int qb = MASK != kMaskNone ? i / BH : i % nqb;  // position in falling cost
      const int bhh = MASK != kMaskNone ? i % BH : i / nqb;
      run_item(bhh * nqb + qb);  // under a mask: Q-block nqb - 1 - qb
      __syncthreads();
    }
  } else {
    int wid = (int)blockIdx.x;
    if ((total & 7) == 0) wid = (wid & 7) * (total >> 3) + (wid >> 3);
    run_item(wid);
  }
}

// Workgroups of one kernel instance resident on the current device at once
// (CUs times blocks per CU), looked up once per device and instance (the
// cache is a static of the instance: all instances share one pointer type).
template <int D, int MASK, int NW, int DEAL>
static int resident_slots() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fwd_kernel<D, MASK, NW, DEAL>, NW * 64, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    v = per_cu * cus;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int D, int MASK, int NW, int DEAL>
static int launch_deal(const FwdArgs& a, int nqb, int blocks) {
  const dim3 grid((unsigned)blocks), block(NW * 64);
  hipLaunchKernelGGL((fwd_kernel<D, MASK, NW, DEAL>), grid, block, 0, (hipStream_t)a.stream,
                     a.q, a.k, a.v, a.o, a.lse, a.B * a.H, a.H, a.H / a.Hkv, a.Nq, a.Nk, nqb, a.scale * kLog2e, a.band,
                     a.slopes, a.sq, a.sk, a.sv, a.so);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <int D, int MASK, int NW>
static int launch_nw(const FwdArgs& a) {
  constexpr int kBR = NW * kQW;
  const int nqb = (a.Nq + kBR - 1) / kBR;
  const int BH = a.B * a.H;
  const int blocks = nqb * BH;
  // persistent: at most one workgroup per resident slot (a generic lambda, so
  // that only the instances that call it compile the persistent kernels)
  auto persistent = [&](auto) {
    const int sx = resident_slots<D, MASK, NW, kDealByXcd>();
    const int gx = sx > 0 ? std::min(blocks, sx) : blocks;
    if (gx % 8 == 0 && BH % 8 == 0 && (gx / 8) % nqb == 0) return launch_deal<D, MASK, NW, kDealByXcd>(a, nqb, gx);
    const int sf = resident_slots<D, MASK, NW, kDealFalling>();
    return launch_deal<D, MASK, NW, kDealFalling>(a, nqb, sf > 0 ? std::min(blocks, sf) : blocks);
  };
  if constexpr (D <= 128 && NW == 4) {
    return persistent(0);
  } else if constexpr (D == 128 && MASK != kMaskNone) {  // (masked d = 64 runs four waves)
    // Eight waves under a mask: persistent when the band runs from the first
    // key to a bound that moves with the row (causal-like), so that the
    // Q-blocks differ in cost; a band bounded on the left (a sliding window)
    // gives every Q-block about the same work and runs one workgroup per item
    // (measured: the persistent grid 2.4% faster causal at N = 8192, 2-3%
    // slower with windows).
    if (a.band.wl >= a.Nk && a.band.wr < a.Nk) return persistent(0);
    return launch_deal<D, MASK, NW, kDealOne>(a, nqb, blocks);
  } else {
    return launch_deal<D, MASK, NW, kDealOne>(a, nqb, blocks);
  }
}

template <int D, int MASK>
static int launch(const FwdArgs& a) {
  if constexpr (kNWof<D> == 8) {
    if (a.Nk <= (MASK == kMaskNone ? kShortKeys : kShortKeysMasked) || (D == 64 && MASK != kMaskNone))
      return launch_nw<D, MASK, 4>(a);
  }
  return launch_nw<D, MASK, kNWof<D>>(a);
}

template <int D>
static int launch_d(const FwdArgs& a) {
  switch (mask_mode(a.band, a.slopes)) {
    case kMaskNone: return launch<D, kMaskNone>(a);
    case kMaskCausal: return launch<D, kMaskCausal>(a);
    case kMaskBand: return launch<D, kMaskBand>(a);
    default: return launch<D, kMaskBandAlibi>(a);
  }
}

int launch_fwd(const FwdArgs& a) {
  if (a.d == 256) return launch_d<256>(a);
  return a.d == 128 ? launch_d<128>(a) : launch_d<64>(a);
}

}  // namespace fa
