/*
 * fa.h — C ABI of the MI355X (gfx950) exact-attention library (libfa_mi355x.so).
 *
 * Exact scaled-dot-product attention computed the FlashAttention way: score
 * tiles S = Q K^T are formed and consumed on chip, the softmax is applied
 * online with a running (m, l) state, the output is normalised once at the
 * end, a per-row logsumexp is saved, and the backward pass recomputes P from it.
 *
 * Sources (web pages):
 *   [LIB] "FlashAttention v1/v2/v3/v4: the librarian who never clears the desk"
 *   [HUB] research-hub concept page "FlashAttention"
 *   [LIN] "The FlashAttention lineage — FA1 / FA2 / FA3 / FA4"
 *
 * Conventions for every call
 * --------------------------
 * - Tensors are [B, H, N, d] row-major (d fastest), the (batch, heads, tokens,
 *   head dim) order of PyTorch's scaled_dot_product_attention. Per-row vectors
 *   (LSE) are [B, H, N] float32. bf16 values travel as their uint16_t bits.
 * - Every tensor pointer is a DEVICE pointer owned by the caller, 16-byte
 *   aligned, on the current HIP device. The library never allocates or frees
 *   device memory; the backward workspace comes from the caller. The only
 *   device memory it holds is the static scratch array of fa_bwd_noalloc.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream). All
 *   calls are asynchronous on that stream; a device fault surfaces at the
 *   caller's next synchronisation.
 * - Supported: d in {64, 128, 256} (the fp8 calls: {64, 128}); B, H, N >= 1 with
 *   B*H*N*d < 2^40; causal in {0, 1};
 *   scale finite and > 0. Causal means query i sees key j iff j <= i.
 * - Arguments are validated before anything is launched. On error nothing is
 *   written and a status below is returned; the library never prints or aborts.
 * - Forward calls are bitwise deterministic for fixed inputs and shape.
 * - Inputs are finite: NaN or infinite values in q, k, v, o, dO, lse (except
 *   the -inf LSE of a query that sees no key) or the fp8 scales are outside the
 *   contract. The kernels are built assuming no NaN operands (maxima compile to
 *   plain v_max), so such inputs give unspecified outputs, not an error status
 *   and not necessarily NaN.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 4

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,     /* B, H or N < 1, the tensor is too large, or H_kv does not divide H */
  FA_ERR_HEADDIM = 3,   /* d not 64, 128 or 256 (fp8: 64 or 128; rotation and exp_mode 1, 2: 128) */
  FA_ERR_ALIGN = 4,     /* a tensor pointer is not 16-byte aligned, or a stride not a multiple of 8 */
  FA_ERR_WORKSPACE = 5, /* backward workspace NULL, misaligned or too small */
  FA_ERR_DEVICE = 6,    /* no HIP device, or the current device is not gfx950 */
  FA_ERR_ALIAS = 7,     /* an output overlaps an input, another output or itself */
  FA_ERR_LAUNCH = 8,    /* the kernel launch failed (hipGetLastError) */
  FA_ERR_ARG = 9,       /* causal not 0/1, a window side < -1 or > 2^24, scale not finite and positive,
                           a stride < 1, a row stride >= 2^31, or exp_mode not 0, 1 or 2 */
  FA_ERR_SCRATCH = 10   /* fa_bwd_noalloc: 4 * B * H * N bytes exceed FA_BWD_NOALLOC_SCRATCH_BYTES */
};

/*
 * Element strides of one [B, H, N, d] tensor view whose d elements are
 * contiguous: element (b, h, n, j) is at base + b*batch + h*head + n*row + j.
 * Contiguous [B, H, N, d] is {H*N*d, N*d, d}; [B, N, H, d] viewed as
 * [B, H, N, d] is {N*H*d, d, H*d}.
 */
typedef struct fa_strides {
  int64_t batch, head, row;
} fa_strides;

/* Human-readable name of a status (static string, never NULL). */
const char* fa_status_string(int status);

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

/*
 * Forward: O = softmax(scale * Q K^T [+ causal mask]) V and
 * LSE_i = log sum_j exp(scale * q_i . k_j) over the visible keys (natural log).
 * [HUB] "How it works" (definition, fusion, saved L_i = m_i + log l_i);
 * [LIB] "The trick that made it all possible: online softmax" (recurrence);
 * [LIN] "FA2 (2023)" (sequence-parallel grid, split-Q, deferred division).
 *   q, k, v : in,  bf16 [B, H, N, d]
 *   o       : out, bf16 [B, H, N, d] (round to nearest even from fp32)
 *   lse     : out, fp32 [B, H, N]
 */
int fa_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
           int B, int H, int N, int d, int causal, float scale, void* stream);

/*
 * fa_fwd on strided views, with grouped key/value heads (GQA; MQA when
 * H_kv = 1): query head h attends to key/value head h / (H / H_kv)
 * ([LIB] "Cases where FlashAttention does not help": GQA/MQA natively
 * supported; [LIB] "FA2": models with aggressive GQA). fa_fwd is the case
 * H_kv = H with contiguous strides.
 *   q, o  : [B, H, N, d] views;  k, v : [B, H_kv, N, d] views
 *   lse   : out, fp32 contiguous [B, H, N]
 *   st    : host array of 4 views' strides, in order q, k, v, o; every
 *           stride >= 1 and a multiple of 8 elements (rows start on 16-byte
 *           boundaries), row strides below 2^31 (else FA_ERR_ARG); o must
 *           not overlap itself (FA_ERR_ALIAS)
 *   H_kv  : divides H (else FA_ERR_SHAPE)
 */
int fa_fwd_strided(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                   int B, int H, int H_kv, int N, int d, const fa_strides* st, int causal, float scale,
                   void* stream);

/*
 * Bytes of device workspace fa_bwd needs: the fp32 row vector
 * D = rowsum(dO o O) [B, H, N], rounded up to 256 bytes. Returns 0 for
 * invalid shapes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Bytes of device workspace fa_bwd_strided needs: D as above, then, when the
 * key/value heads are grouped (H_kv < H) and one workgroup per (batch, K/V
 * head, 128-key block) would leave the GPU under-filled or, causal, unevenly
 * loaded, fp32 partial dK and dV of the workgroups that share a key block:
 * 2 x B x H_kv x s x N x d x 4 bytes for a split s dividing H / H_kv (at most
 * 2 x B x H x N x d x 4). Equals fa_bwd_workspace_bytes when H_kv = H.
 * Returns 0 for invalid arguments.
 */
size_t fa_bwd_strided_workspace_bytes(int B, int H, int H_kv, int N, int d, int causal);

/*
 * Backward by recomputation: P_ij = exp(scale q_i.k_j - LSE_i) is rebuilt tile
 * by tile from the saved LSE ([HUB] "How it works"; [LIB] "FA1 — changing the
 * order of the operations"); dV = P^T dO, dP = dO V^T, D = rowsum(dO o O),
 * dS = P o (dP - D), dQ = scale dS K, dK = scale dS^T Q.
 *   q, k, v, o, dO : in, bf16 [B, H, N, d] (o and lse as produced by fa_fwd)
 *   lse            : in, fp32 [B, H, N]
 *   dq, dk, dv     : out, bf16 [B, H, N, d]
 *   ws, ws_bytes   : caller-owned device workspace, >= fa_bwd_workspace_bytes,
 *                    256-byte aligned; its contents on entry are ignored.
 * No atomics: each output element is produced by one wave, so all three
 * gradients are bitwise deterministic across runs.
 */
int fa_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
           const uint16_t* dO, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
           int B, int H, int N, int d, int causal, float scale, void* ws, size_t ws_bytes,
           void* stream);

/*
 * fa_bwd without a workspace argument and without any allocation, for callers
 * that cannot allocate device memory at the point of the call: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * library calls no hipMalloc, hipFree or allocating routine here; the fp32
 * D = rowsum(dO o O) vector that fa_bwd keeps in the caller's workspace lives
 * instead in a static device array of FA_BWD_NOALLOC_SCRATCH_BYTES (8 MiB, so
 * B * H * N <= 2^21 rows), one per GPU, held until the process ends.
 * Arguments, layouts, results and determinism are those of fa_bwd; the
 * results are bitwise identical to fa_bwd's (the same kernels run).
 *   returns FA_ERR_SCRATCH when 4 * B * H * N > FA_BWD_NOALLOC_SCRATCH_BYTES,
 *   checked on the host before anything is launched.
 * Every call on one GPU shares that GPU's array and leaves its D there (the
 * next call overwrites all of it before reading it; nothing needs clearing).
 * Calls that overlap in time on one GPU (two streams, or two host threads)
 * race on the array and give wrong gradients: serialise them.
 */
#define FA_BWD_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int fa_bwd_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                   const uint16_t* dO, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                   int B, int H, int N, int d, int causal, float scale, void* stream);

/*
 * fa_bwd on strided views with grouped key/value heads (see fa_fwd_strided):
 * dK and dV of key/value head g are the sums over the H / H_kv query heads
 * that read it (the chain rule through the shared head). fa_bwd is the case
 * H_kv = H with contiguous strides. The workspace is
 * fa_bwd_strided_workspace_bytes(B, H, H_kv, N, d, causal).
 *   q, o, dO, dq : [B, H, N, d] views;  k, v, dk, dv : [B, H_kv, N, d] views
 *   lse          : in, fp32 contiguous [B, H, N]
 *   st           : host array of 8 views' strides, in order q, k, v, o, dO,
 *                  dq, dk, dv (rules as in fa_fwd_strided; dq, dk, dv must
 *                  not overlap themselves)
 */
int fa_bwd_strided(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                   const uint16_t* dO, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                   int B, int H, int H_kv, int N, int d, const fa_strides* st, int causal, float scale,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * Masks beyond causal, and queries and keys of different lengths ([LIB]
 * "Cases where FlashAttention does not help": the kernels ship causal,
 * sliding-window and ALiBi masks; cross-attention is supported). Query i of
 * N_q is aligned with key c_i = i + N_k - N_q (the last query with the last
 * key; c_i = i when N_q = N_k). Key j is visible to query i iff
 *   causal = 0 or j <= c_i, and
 *   window_left  = -1 or j >= c_i - window_left, and
 *   window_right = -1 or j <= c_i + window_right.
 * alibi_slopes, when not NULL, is a device fp32 [H] array (one slope per query
 * head, finite; 4-byte aligned): the scaled score of (i, j) in head h gets
 * -alibi_slopes[h] * |c_i - j| added before the softmax (no gradient flows to
 * the slopes). A query with no visible key gets O = 0 and LSE = -inf, and
 * zero gradients. A NULL mask is causal = 0, both windows -1, no ALiBi.
 */
typedef struct fa_mask {
  int causal;                /* 0 or 1 */
  int window_left;           /* -1 (unbounded) or 0 .. 2^24 */
  int window_right;          /* -1 (unbounded) or 0 .. 2^24 */
  const float* alibi_slopes; /* NULL or device fp32 [H] */
} fa_mask;

/*
 * The general forward: fa_fwd_strided with N_q queries against N_k keys and
 * a mask (above). fa_fwd_strided is the case N_q = N_k = N with
 * {causal, -1, -1, NULL}.
 *   q, o  : [B, H, N_q, d] views;  k, v : [B, H_kv, N_k, d] views
 *   lse   : out, fp32 contiguous [B, H, N_q]
 *   st    : host array of 4 views' strides (q, k, v, o), rules of fa_fwd_strided
 *   mask  : host pointer, or NULL
 */
int fa_fwd_ext(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
               int B, int H, int H_kv, int N_q, int N_k, int d, const fa_strides* st, const fa_mask* mask,
               float scale, void* stream);

/*
 * Workspace bytes of fa_bwd_ext: fp32 D [B, H, N_q] rounded to 256 bytes,
 * then for grouped heads split over workgroups the fp32 partial dK, dV
 * (2 x B x H_kv x s x N_k x d x 4 bytes, s dividing H / H_kv; see
 * fa_bwd_strided_workspace_bytes). 0 for invalid arguments.
 */
size_t fa_bwd_ext_workspace_bytes(int B, int H, int H_kv, int N_q, int N_k, int d, const fa_mask* mask);

/*
 * The general backward, matching fa_fwd_ext (o and lse as it produced them).
 *   q, o, dO, dq : [B, H, N_q, d] views;  k, v, dk, dv : [B, H_kv, N_k, d] views
 *   st           : host array of 8 views' strides (q, k, v, o, dO, dq, dk, dv)
 *   ws, ws_bytes : >= fa_bwd_ext_workspace_bytes(B, H, H_kv, N_q, N_k, d, mask)
 * Keys no query sees get dK = dV = 0. Deterministic, as fa_bwd.
 */
int fa_bwd_ext(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
               const uint16_t* dO, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
               int B, int H, int H_kv, int N_q, int N_k, int d, const fa_strides* st, const fa_mask* mask,
               float scale, void* ws, size_t ws_bytes, void* stream);

/*
 * FP8 input path ([LIB] "FA3 — the Hopper moment", pillar 3; [LIN] "FA3
 * (2024)", idea 3): optional random-sign Hadamard rotation along d, then block
 * quantisation to OCP E4M3FN with one fp32 scale per 128 token rows of a
 * (batch, head).
 *   x             : in,  bf16 [B, H, N, d]
 *   x8            : out, e4m3 codes [B, H, N, d]
 *   scales        : out, fp32 [B, H, ceil(N / 128)]; scale = fl32(amax / 448),
 *                   1 for an all-zero block
 *   signs_or_null : in, device int8 [128] of +-1 (rotation x' = H_128 (s o x) /
 *                   sqrt(128), d must be 128; 16-byte aligned like every
 *                   tensor here, else FA_ERR_ALIGN), or NULL for no rotation
 * Codes: e4m3_rne_saturating(fl32(x' * fl32(448 / amax))). Rotation order:
 * multiply by s, butterflies (a, b) -> (a + b, a - b) at strides 1, 2, ..., 64,
 * multiply by fl32(1 / sqrt(128)), all in fp32.
 */
int fa_quant_fp8(const uint16_t* x, uint8_t* x8, float* scales, const int8_t* signs_or_null,
                 int B, int H, int N, int d, void* stream);

/*
 * FP8 forward on block-quantised inputs (as produced by fa_quant_fp8; Q and K
 * rotated with the same signs or not at all, V never rotated). Computes the
 * forward above on the dequantised values x8 * scale: e4m3 MFMA for Q K^T and
 * P V with fp32 accumulation; P is quantised to e4m3 for the P V product.
 *   q8, k8, v8                  : in, e4m3 [B, H, N, d]
 *   q_scale, k_scale, v_scale   : in, fp32 [B, H, ceil(N / 128)]
 *   o                           : out, bf16 [B, H, N, d]
 *   lse                         : out, fp32 [B, H, N]
 */
int fa_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
               const float* k_scale, const float* v_scale, uint16_t* o, float* lse,
               int B, int H, int N, int d, int causal, float scale, void* stream);

/*
 * fa_fwd_fp8 with the softmax's exponentials chosen by exp_mode: the software
 * 2^x of [LIB] "FA4 — Blackwell's asymmetry" (idea 1) and [LIN] "FA4 (2026)"
 * (change 2), a polynomial on the FMA units (range reduction to n + f,
 * 2^f by a degree-4 polynomial, 2^n into the exponent field; relative error
 * at most 2.7e-6), in place of the transcendental instruction.
 *   exp_mode : 0 the hardware exponential for every value (what fa_fwd_fp8
 *              runs); 1 the software 2^x for one value in four; 2 for all.
 *              Other values: FA_ERR_ARG. Modes 1 and 2 need d = 128
 *              (else FA_ERR_HEADDIM).
 * Other arguments, checks and outputs as fa_fwd_fp8. On this chip the
 * software form costs more vector instructions than it saves, so mode 0 is
 * the fast one; the others are for measuring that trade.
 */
int fa_fwd_fp8_ext(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
                   const float* k_scale, const float* v_scale, uint16_t* o, float* lse,
                   int B, int H, int N, int d, int causal, float scale, int exp_mode, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
