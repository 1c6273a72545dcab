// Host-side launch interface between the C ABI (fa_api.hip) and the kernel
// files. Arguments arrive here already validated.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fa {

// Element strides of a [B, H, N, d] tensor view whose d elements are contiguous.
struct Strides {
  long long b, h, n;
};
inline Strides contiguous_strides(int H, int N, int d) {
  return Strides{(long long)H * N * d, (long long)N * d, (long long)d};
}

// Keys visible to query i (of Nq, against Nk keys): i + off - wl ..
// i + off + wr, intersected with 0 .. Nk - 1. off = Nk - Nq aligns the last
// query with the last key; causal is wr = 0; kOpen leaves a side unbounded.
constexpr int kOpen = 1 << 30;
struct Band {
  int off, wl, wr;
};

// Kernel instances by mask: no mask, causal with Nq = Nk (the band (open, 0),
// off = 0), any band, any band with ALiBi. The first two keep the simplest
// index arithmetic (their kernels run at the register limit, where every
// extra live value costs).
enum MaskMode { kMaskNone = 0, kMaskCausal = 1, kMaskBand = 2, kMaskBandAlibi = 3 };
inline MaskMode mask_mode(const Band& b, const float* slopes) {
  if (slopes) return kMaskBandAlibi;
  if (b.wl == kOpen && b.wr == kOpen) return kMaskNone;
  if (b.wl == kOpen && b.wr == 0 && b.off == 0) return kMaskCausal;
  return kMaskBand;
}

// H query heads share Hkv key/value heads: query head h reads K/V head
// h / (H / Hkv) (Hkv divides H; Hkv = H is plain multi-head attention).
struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;  // contiguous [B, H, Nq]
  int B, H, Hkv, Nq, Nk, d;
  Band band;
  const float* slopes;  // ALiBi slopes [H] (device), or null
  float scale;
  Strides sq, sk, sv, so;
  void* stream;
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dO;
  const float* lse;  // contiguous [B, H, Nq]
  uint16_t* dq;
  uint16_t* dk;      // [B, Hkv, N, d] view: the sum over the query heads of each group
  uint16_t* dv;
  float* delta;      // workspace: fp32 D [B, H, Nq]
  int B, H, Hkv, Nq, Nk, d;
  Band band;
  const float* slopes;  // ALiBi slopes [H] (device), or null
  float scale;
  Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
  void* stream;
  float* part = nullptr;  // workspace after D: fp32 partial dK, dV when split > 1
  int split = 1;          // bwd_kv_split
};

struct QuantArgs {
  const uint16_t* x;
  uint8_t* x8;
  float* scales;
  const int8_t* signs;  // NULL: no rotation
  int B, H, N, d;
  void* stream;
};

struct Fp8FwdArgs {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8;
  const float* qs;
  const float* ks;
  const float* vs;
  uint16_t* o;
  float* lse;
  int B, H, N, d, causal;
  float scale;
  void* stream;
  int exp_mode = 0;  // exponentials of the softmax in software: 0 none, 1 one in four, 2 all (d = 128)
};

// Each returns 0 on a successful launch, nonzero if hipGetLastError reports one.
int launch_fwd(const FwdArgs& a);
int launch_bwd(const BwdArgs& a);     // all three backward launches
int launch_bwd_d256(const BwdArgs& a);  // the same at d = 256 (fa_bwd_d256.hip)
int launch_bwd_dq(const BwdArgs& a);  // the dQ launch (it also writes D for the dK/dV launch)
int launch_quant_fp8(const QuantArgs& a);
int launch_fwd_fp8(const Fp8FwdArgs& a);

// Workspace of the backward pass: D = rowsum(dO o O), rounded to 256 bytes,
// then (grouped heads split over workgroups only) fp32 partial dK, dV.
inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t bwd_delta_bytes(int B, int H, int N) { return round256((size_t)B * H * N * sizeof(float)); }

// Key blocks per (batch, K/V head) in the dK/dV kernel (128 keys each).
inline int bwd_key_blocks(int N) { return (N + 127) / 128; }

// How many workgroups share one (batch, K/V head, key block) of grouped
// heads: each sums the gradients of group / split query heads and, for
// split > 1, writes fp32 partials that a reduction adds up. The smallest
// divisor of the group that gives at least 256 workgroups (one per CU), or
// 1024 when the band is bounded (so that uneven key blocks balance), else the
// whole group.
inline int bwd_kv_split(int B, int H_kv, int group, int N, bool uneven) {
  const long long units = (long long)bwd_key_blocks(N) * B * H_kv;
  const long long want = uneven ? 1024 : 256;
  for (int s = 1; s < group; ++s)
    if (group % s == 0 && units * s >= want) return s;
  return group;
}

inline size_t bwd_partial_bytes(int B, int H_kv, int N, int d, int split) {
  return split > 1 ? round256((size_t)2 * B * H_kv * split * N * d * sizeof(float)) : 0;
}

}  // namespace fa
