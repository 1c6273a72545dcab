// C ABI of the attention library: argument validation, device check, dispatch.
// Validation runs entirely on the host and touches no HIP API, so a bad call
// returns its status on any machine; the device check is the last step before
// a launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <utility>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_DEVICE;
  int st = g_device_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return FA_ERR_DEVICE;
    st = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_ok[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? FA_OK : FA_ERR_DEVICE;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;
};
Range span(const void* p, size_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Every output range must be disjoint from every other range.
bool any_alias(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

bool shape_ok(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return false;
  const double elems = (double)B * H * N * d;
  return elems < 1099511627776.0 && (double)B * H < 2147483647.0 && N <= (1 << 24);
}

bool scalars_ok(int causal, float scale) {
  return (causal == 0 || causal == 1) && std::isfinite(scale) && scale > 0.f;
}

bool scale_ok(float scale) { return std::isfinite(scale) && scale > 0.f; }

// head dims of the bf16 kernels (the fp8 path takes 64 and 128)
bool bf16_head_dim(int d) { return d == 64 || d == 128 || d == 256; }

constexpr int kMaxLen = 1 << 24;

// A mask is valid with causal 0 / 1 and each window side -1 (unbounded) or
// 0 .. 2^24; NULL means no mask.
bool mask_ok(const fa_mask* m) {
  if (!m) return true;
  return (m->causal == 0 || m->causal == 1) && m->window_left >= -1 && m->window_left <= kMaxLen &&
         m->window_right >= -1 && m->window_right <= kMaxLen;
}

// The band of visible keys (fa_internal.h) for a mask and the two lengths.
fa::Band band_of(const fa_mask* m, int N_q, int N_k) {
  fa::Band b{N_k - N_q, fa::kOpen, fa::kOpen};
  if (!m) return b;
  if (m->window_left >= 0) b.wl = m->window_left;
  if (m->window_right >= 0) b.wr = m->window_right;
  if (m->causal) b.wr = std::min(b.wr, 0);
  return b;
}

// Work per key block is uneven when the band is bounded on either side.
bool uneven(const fa_mask* m) {
  return m && (m->causal || m->window_left >= 0 || m->window_right >= 0);
}

// A [B, Hx, N, d] view with element strides st and contiguous d.
struct View {
  const void* p;
  long long B, H, N, d;
  fa_strides st;
  // bytes from p to one past the last element
  size_t bytes() const {
    return 2u * (size_t)((B - 1) * st.batch + (H - 1) * st.head + (N - 1) * st.row + d);
  }
  Range range() const { return span(p, bytes()); }
  // rows start on 16-byte boundaries (the kernels load 16-byte chunks)
  bool aligned() const {
    return aligned16(p) && st.batch % 8 == 0 && st.head % 8 == 0 && st.row % 8 == 0;
  }
  // row strides stay below 2^31 elements: the kernels form row offsets with
  // one 32 x 32 -> 64-bit multiply
  bool strides_ok() const { return st.batch > 0 && st.head > 0 && st.row > 0 && st.row <= 0x7fffffffLL; }
  // no two elements share an address: with dims of extent > 1 sorted by stride,
  // each stride exceeds the span of all finer dims (d counts as stride 1)
  bool injective() const {
    long long ext[3] = {B, H, N}, str[3] = {st.batch, st.head, st.row};
    for (int i = 0; i < 3; ++i)
      for (int j = i + 1; j < 3; ++j)
        if (str[j] < str[i]) {
          std::swap(str[i], str[j]);
          std::swap(ext[i], ext[j]);
        }
    long long reach = d;  // elements spanned by the finer dims
    for (int i = 0; i < 3; ++i) {
      if (ext[i] == 1) continue;
      if (str[i] < reach) return false;
      reach = str[i] * (ext[i] - 1) + reach;
    }
    return true;
  }
};

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: B, H or N out of range";
    case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM: unsupported head dim";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: tensor pointer not 16-byte aligned";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace NULL, misaligned or too small";
    case FA_ERR_DEVICE: return "FA_ERR_DEVICE: no gfx950 device current";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: an output overlaps another tensor";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: kernel launch failed";
    case FA_ERR_ARG: return "FA_ERR_ARG: bad causal flag, window, scale or stride";
    case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH: B*H*N exceeds the static scratch of fa_bwd_noalloc";
    default: return "FA_ERR_UNKNOWN";
  }
}

int fa_abi_version(void) { return FA_ABI_VERSION; }

int fa_fwd_ext(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
               int B, int H, int H_kv, int N_q, int N_k, int d, const fa_strides* st, const fa_mask* mask,
               float scale, void* stream) {
  if (!scale_ok(scale) || !mask_ok(mask)) return FA_ERR_ARG;
  if (!q || !k || !v || !o || !lse || !st) return FA_ERR_NULL;
  if (!bf16_head_dim(d)) return FA_ERR_HEADDIM;
  if (!shape_ok(B, H, N_q, d) || !shape_ok(B, H_kv, N_k, d) || H_kv < 1 || H % H_kv != 0) return FA_ERR_SHAPE;
  const View vq{q, B, H, N_q, d, st[0]}, vk{k, B, H_kv, N_k, d, st[1]}, vv{v, B, H_kv, N_k, d, st[2]},
      vo{o, B, H, N_q, d, st[3]};
  if (!vq.strides_ok() || !vk.strides_ok() || !vv.strides_ok() || !vo.strides_ok()) return FA_ERR_ARG;
  const float* slopes = mask ? mask->alibi_slopes : nullptr;
  if (!vq.aligned() || !vk.aligned() || !vv.aligned() || !vo.aligned() || !aligned16(lse) ||
      ((uintptr_t)slopes & 3u))
    return FA_ERR_ALIGN;
  const size_t lb = (size_t)B * H * N_q * 4;
  const Range ins[4] = {vq.range(), vk.range(), vv.range(), span(slopes, slopes ? (size_t)H * 4 : 0)};
  const Range outs[2] = {vo.range(), span(lse, lb)};
  if (!vo.injective() || any_alias(outs, 2, ins, 4)) return FA_ERR_ALIAS;
  if (int s = check_device()) return s;
  auto S = [&](int i) { return fa::Strides{st[i].batch, st[i].head, st[i].row}; };
  fa::FwdArgs a{q, k, v, o, lse, B, H, H_kv, N_q, N_k, d, band_of(mask, N_q, N_k), slopes, scale,
                S(0), S(1), S(2), S(3), stream};
  return fa::launch_fwd(a) ? FA_ERR_LAUNCH : FA_OK;
}

int fa_fwd_strided(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                   int B, int H, int H_kv, int N, int d, const fa_strides* st, int causal, float scale,
                   void* stream) {
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  const fa_mask m{causal, -1, -1, nullptr};
  return fa_fwd_ext(q, k, v, o, lse, B, H, H_kv, N, N, d, st, &m, scale, stream);
}

int fa_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
           int B, int H, int N, int d, int causal, float scale, void* stream) {
  const fa_strides c{(int64_t)H * N * d, (int64_t)N * d, (int64_t)d};
  const fa_strides st[4] = {c, c, c, c};
  return fa_fwd_strided(q, k, v, o, lse, B, H, H, N, d, st, causal, scale, stream);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (!bf16_head_dim(d) || !shape_ok(B, H, N, d)) return 0;
  return fa::bwd_delta_bytes(B, H, N);
}

size_t fa_bwd_ext_workspace_bytes(int B, int H, int H_kv, int N_q, int N_k, int d, const fa_mask* mask) {
  if (!bf16_head_dim(d) || !shape_ok(B, H, N_q, d) || !shape_ok(B, H_kv, N_k, d) || H_kv < 1 ||
      H % H_kv != 0 || !mask_ok(mask))
    return 0;
  const int split = fa::bwd_kv_split(B, H_kv, H / H_kv, N_k, uneven(mask));
  return fa::bwd_delta_bytes(B, H, N_q) + fa::bwd_partial_bytes(B, H_kv, N_k, d, split);
}

size_t fa_bwd_strided_workspace_bytes(int B, int H, int H_kv, int N, int d, int causal) {
  if (causal != 0 && causal != 1) return 0;
  const fa_mask m{causal, -1, -1, nullptr};
  return fa_bwd_ext_workspace_bytes(B, H, H_kv, N, N, d, &m);
}

}  // extern "C"

namespace {

// Static scratch of fa_bwd_noalloc: the fp32 row vector D (the only
// workspace fa_bwd needs when H_kv = H). Each GPU the library runs on holds
// its own copy until the process ends. In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = FA_BWD_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch (the current device), or NULL.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return nullptr;
    p = a;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

// The backward of fa_bwd_ext. With noalloc the workspace comes from the
// static scratch instead of (ws, ws_bytes), which are then ignored.
int bwd_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o, const uint16_t* dO,
             const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv, int B, int H, int H_kv, int N_q, int N_k,
             int d, const fa_strides* st, const fa_mask* mask, float scale, void* ws, size_t ws_bytes,
             void* stream, bool noalloc) {
  if (!scale_ok(scale) || !mask_ok(mask)) return FA_ERR_ARG;
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv || !st) return FA_ERR_NULL;
  if (!bf16_head_dim(d)) return FA_ERR_HEADDIM;
  if (!shape_ok(B, H, N_q, d) || !shape_ok(B, H_kv, N_k, d) || H_kv < 1 || H % H_kv != 0) return FA_ERR_SHAPE;
  const View vq{q, B, H, N_q, d, st[0]}, vk{k, B, H_kv, N_k, d, st[1]}, vv{v, B, H_kv, N_k, d, st[2]},
      vo{o, B, H, N_q, d, st[3]}, vdo{dO, B, H, N_q, d, st[4]}, vdq{dq, B, H, N_q, d, st[5]},
      vdk{dk, B, H_kv, N_k, d, st[6]}, vdv{dv, B, H_kv, N_k, d, st[7]};
  const View* all[8] = {&vq, &vk, &vv, &vo, &vdo, &vdq, &vdk, &vdv};
  for (const View* x : all)
    if (!x->strides_ok()) return FA_ERR_ARG;
  for (const View* x : all)
    if (!x->aligned()) return FA_ERR_ALIGN;
  const float* slopes = mask ? mask->alibi_slopes : nullptr;
  if (!aligned16(lse) || ((uintptr_t)slopes & 3u)) return FA_ERR_ALIGN;
  const size_t need = fa_bwd_ext_workspace_bytes(B, H, H_kv, N_q, N_k, d, mask);
  if (noalloc) {
    if (need > kNoAllocScratchBytes) return FA_ERR_SCRATCH;
  } else if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < need) {
    return FA_ERR_WORKSPACE;
  }
  const size_t lb = (size_t)B * H * N_q * 4;
  const Range ins[7] = {vq.range(), vk.range(), vv.range(), vo.range(), vdo.range(), span(lse, lb),
                        span(slopes, slopes ? (size_t)H * 4 : 0)};
  const Range outs[4] = {vdq.range(), vdk.range(), vdv.range(), span(noalloc ? nullptr : ws, noalloc ? 0 : need)};
  if (!vdq.injective() || !vdk.injective() || !vdv.injective() || any_alias(outs, 4, ins, 7)) return FA_ERR_ALIAS;
  if (int s = check_device()) return s;
  if (noalloc) {
    ws = scratch_ptr();
    if (!ws) return FA_ERR_DEVICE;
  }
  auto S = [&](int i) { return fa::Strides{st[i].batch, st[i].head, st[i].row}; };
  fa::BwdArgs a{q, k, v, o, dO, lse, dq, dk, dv, (float*)ws, B, H, H_kv, N_q, N_k, d,
                band_of(mask, N_q, N_k), slopes, scale, S(0), S(1), S(2), S(3), S(4), S(5), S(6), S(7), stream};
  a.split = fa::bwd_kv_split(B, H_kv, H / H_kv, N_k, uneven(mask));
  a.part = a.split > 1 ? (float*)((char*)ws + fa::bwd_delta_bytes(B, H, N_q)) : nullptr;
  return fa::launch_bwd(a) ? FA_ERR_LAUNCH : FA_OK;
}

}  // namespace

extern "C" {

int fa_bwd_ext(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
               const uint16_t* dO, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
               int B, int H, int H_kv, int N_q, int N_k, int d, const fa_strides* st, const fa_mask* mask,
               float scale, void* ws, size_t ws_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, H_kv, N_q, N_k, d, st, mask, scale, ws, ws_bytes, stream,
                  false);
}

int fa_bwd_strided(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                   const uint16_t* dO, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                   int B, int H, int H_kv, int N, int d, const fa_strides* st, int causal, float scale,
                   void* ws, size_t ws_bytes, void* stream) {
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  const fa_mask m{causal, -1, -1, nullptr};
  return fa_bwd_ext(q, k, v, o, dO, lse, dq, dk, dv, B, H, H_kv, N, N, d, st, &m, scale, ws, ws_bytes, stream);
}

int fa_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
           const uint16_t* dO, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
           int B, int H, int N, int d, int causal, float scale, void* ws, size_t ws_bytes,
           void* stream) {
  const fa_strides c{(int64_t)H * N * d, (int64_t)N * d, (int64_t)d};
  const fa_strides st[8] = {c, c, c, c, c, c, c, c};
  return fa_bwd_strided(q, k, v, o, dO, lse, dq, dk, dv, B, H, H, N, d, st, causal, scale, ws, ws_bytes, stream);
}

int fa_bwd_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                   const uint16_t* dO, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                   int B, int H, int N, int d, int causal, float scale, void* stream) {
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  const fa_strides c{(int64_t)H * N * d, (int64_t)N * d, (int64_t)d};
  const fa_strides st[8] = {c, c, c, c, c, c, c, c};
  const fa_mask m{causal, -1, -1, nullptr};
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, H, N, N, d, st, &m, scale, nullptr, 0, stream, true);
}

int fa_quant_fp8(const uint16_t* x, uint8_t* x8, float* scales, const int8_t* signs_or_null,
                 int B, int H, int N, int d, void* stream) {
  if (!x || !x8 || !scales) return FA_ERR_NULL;
  if ((d != 64 && d != 128) || (signs_or_null && d != 128)) return FA_ERR_HEADDIM;
  if (!shape_ok(B, H, N, d)) return FA_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(x8) || !aligned16(scales) || (signs_or_null && !aligned16(signs_or_null)))
    return FA_ERR_ALIGN;
  const size_t n = (size_t)B * H * N * d, nb = (size_t)B * H * ((N + 127) / 128) * 4;
  const Range ins[2] = {span(x, 2 * n), span(signs_or_null, signs_or_null ? 128 : 0)};
  const Range outs[2] = {span(x8, n), span(scales, nb)};
  if (any_alias(outs, 2, ins, signs_or_null ? 2 : 1)) return FA_ERR_ALIAS;
  if (int st = check_device()) return st;
  fa::QuantArgs a{x, x8, scales, signs_or_null, B, H, N, d, stream};
  return fa::launch_quant_fp8(a) ? FA_ERR_LAUNCH : FA_OK;
}

int fa_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
               const float* k_scale, const float* v_scale, uint16_t* o, float* lse,
               int B, int H, int N, int d, int causal, float scale, void* stream) {
  return fa_fwd_fp8_ext(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, H, N, d, causal, scale, 0, stream);
}

int fa_fwd_fp8_ext(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
                   const float* k_scale, const float* v_scale, uint16_t* o, float* lse,
                   int B, int H, int N, int d, int causal, float scale, int exp_mode, void* stream) {
  if (!scalars_ok(causal, scale) || exp_mode < 0 || exp_mode > 2) return FA_ERR_ARG;
  if (!q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale || !o || !lse) return FA_ERR_NULL;
  if ((d != 64 && d != 128) || (exp_mode != 0 && d != 128)) return FA_ERR_HEADDIM;
  if (!shape_ok(B, H, N, d)) return FA_ERR_SHAPE;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(q_scale) ||
      !aligned16(k_scale) || !aligned16(v_scale) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const size_t n = (size_t)B * H * N * d, nb = (size_t)B * H * ((N + 127) / 128) * 4;
  const Range ins[6] = {span(q8, n), span(k8, n), span(v8, n), span(q_scale, nb), span(k_scale, nb),
                        span(v_scale, nb)};
  const Range outs[2] = {span(o, 2 * n), span(lse, (size_t)B * H * N * 4)};
  if (any_alias(outs, 2, ins, 6)) return FA_ERR_ALIAS;
  if (int st = check_device()) return st;
  fa::Fp8FwdArgs a{q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, H, N, d, causal, scale, stream, exp_mode};
  return fa::launch_fwd_fp8(a) ? FA_ERR_LAUNCH : FA_OK;
}

}  // extern "C"
