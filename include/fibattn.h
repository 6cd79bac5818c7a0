/*
 * fibattn.h - C ABI of the Fibonacci-offset dilated sparse attention library (gfx950).
 *
 * The operation is the attention layer of "Depth-Staggered Fibonacci Spacing for Sparse
 * Attention: Static Schedules Beat Learned Dilation and Extrapolate Where Dense Attention
 * Fails" (arXiv 2606.28560; gist.science technical summaries, Korean and Spanish pages),
 * cited below as [FIB]:
 *   - Method > Architecture and attention mechanism: query i attends a dense local window
 *     of W keys plus one key per base offset f_k (fib = 1, 2, 3, 5, ..., 987) placed at
 *     distance d_k = alpha * f_k, alpha a per-layer scalar in [0.5, 1.5]; non-integer
 *     offsets linearly interpolate the key/value rows so that a gradient reaches alpha;
 *     RoPE is applied before the gather.
 *   - Results 2 (efficiency): static schedules use integer offsets (a fused boolean-mask
 *     path), learned ones the interpolated gather.
 *   - Method > Experimental variables: the Fixed, Staggered-linear and Staggered-coprime
 *     (l -> 7l mod L) per-layer schedules.
 *
 * Conventions fixed by this library where the pages are silent:
 *   - causal; window = distances 0..W-1 (the query itself included);
 *   - integer mode (FIB_INT): r_k = round-half-to-even(alpha * f_k) computed exactly
 *     (fp32 alpha times an integer, in fp64); offsets r_k < W are dropped; equal offsets
 *     collapse; offset r is used by query i when r <= i;
 *   - interpolated mode (FIB_INTERP): entries with d_k >= W are kept, c_k = ceil(d_k),
 *     w_k = c_k - d_k; query i (when c_k <= i) attends the virtual key
 *     (1 - w_k) * K^[i - c_k] + w_k * K^[i - c_k + 1] with the same blend of V rows;
 *   - RoPE: rotate-half pairs (j, j + D/2), omega_j = theta^(-2j/D), positions 0..N-1,
 *     applied to Q and K inside the call (inputs are un-rotated); V is not rotated;
 *   - softmax scale 1/sqrt(D); fp32 accumulation; O, dQ, dK, dV in the input dtype
 *     (round to nearest even for bf16); LSE natural log, fp32.
 *
 * Memory layout: every tensor is [B, H, N, D] row-major and contiguous (D fastest); LSE is
 * [B, H, N]. Device pointers must be 16-byte aligned. D = 64 is the supported head size.
 *
 * Ownership: the caller allocates and owns all device buffers (outputs and backward
 * workspace included); the library never allocates or frees device memory. Host arrays
 * (base, out_* of the table helper) are read or written during the call only. The library
 * keeps no state between calls that affects results (it only records, per device, that a
 * kernel's LDS limit has been raised, so the setting is made once) and is reentrant. Device work is enqueued on `stream`
 * (a hipStream_t; NULL = the null stream) and the call returns without synchronizing.
 *
 * Errors: every call returns FIB_OK (0) or a negative FIB_ERR_* status. On an argument
 * error nothing is launched and no output is touched. Device faults surface at the
 * caller's next synchronization (HIP semantics). No C++ exception crosses this ABI.
 */
#ifndef FIBATTN_H
#define FIBATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define FIB_OK 0
#define FIB_ERR_NULL (-1)        /* a required pointer is NULL */
#define FIB_ERR_SHAPE (-2)       /* B, H or N < 1, or B*H*N*D does not fit the index range */
#define FIB_ERR_HEAD_DIM (-3)    /* D is not 64 */
#define FIB_ERR_DTYPE (-4)       /* dtype is not FIB_F32 or FIB_BF16 */
#define FIB_ERR_WINDOW (-5)      /* W < 1 */
#define FIB_ERR_ALPHA (-6)       /* alpha not finite or <= 0 */
#define FIB_ERR_BASE (-7)        /* n_base outside [1, 32], or base not strictly increasing in [1, 2^24] */
#define FIB_ERR_THETA (-8)       /* rope_theta not finite or <= 0 */
#define FIB_ERR_MODE (-9)        /* mode is not FIB_INT or FIB_INTERP */
#define FIB_ERR_ALIGN (-10)      /* a device pointer is not 16-byte aligned */
#define FIB_ERR_WORKSPACE (-11)  /* backward workspace NULL or smaller than required */
#define FIB_ERR_LAUNCH (-12)     /* the HIP runtime reported an error at launch */
#define FIB_ERR_SCHEDULE (-13)   /* bad schedule kind, layer or layer count */
#define FIB_ERR_CAPACITY (-14)   /* an output array is too small */
#define FIB_ERR_SCRATCH (-15)    /* fib_sparse_attn_bwd_noalloc: the call needs more workspace than the
                                    library's fixed scratch (FIB_NOALLOC_SCRATCH_BYTES) */

/* element types of Q, K, V, O, dO, dQ, dK, dV */
#define FIB_F32 0
#define FIB_BF16 1

/* offset modes */
#define FIB_INT 0     /* rounded integer offsets ([FIB] Results 2, static schedules) */
#define FIB_INTERP 1  /* interpolated K/V rows at non-integer offsets ([FIB] Method) */

/* per-layer schedules of alpha ([FIB] Method > Experimental variables) */
#define FIB_SCHED_FIXED 0    /* alpha = 1 for every layer */
#define FIB_SCHED_LINEAR 1   /* fp32 nearest to 0.5 + l / (L - 1) */
#define FIB_SCHED_COPRIME 2  /* linear value at index (7 l) mod L; needs gcd(7, L) = 1 */

#define FIB_MAX_BASE 32

/*
 * Forward ([FIB] Method > Architecture and attention mechanism).
 *   q, k, v  device, [B, H, N, D] of `dtype`, un-rotated (RoPE is applied inside).
 *   o        device, [B, H, N, D] of `dtype`, written.
 *   lse      device, [B, H, N] fp32 log-sum-exp of the scaled logits, written; may be NULL.
 *   W        window size >= 1.
 *   alpha    per-layer dilation (> 0, finite; the pages use [0.5, 1.5]).
 *   base     host, n_base strictly increasing offsets in [1, 2^24] (e.g. 1, 2, 3, 5, ..., 987).
 *   rope_theta  RoPE base (e.g. 10000).
 *   mode     FIB_INT or FIB_INTERP.
 *   stream   hipStream_t (NULL = null stream).
 * Returns FIB_OK or FIB_ERR_*.
 */
int fib_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                        int W, float alpha, const int32_t* base, int n_base,
                        float rope_theta, int mode, void* stream);

/*
 * Backward of the forward above with respect to q, k, v and alpha, given dO
 * ([FIB] Method: interpolation lets the gradient reach alpha; Learned schedule).
 *   o, lse   device, the forward's outputs for the same arguments (lse must not be NULL).
 *   dout     device, [B, H, N, D] of `dtype`, gradient of the loss w.r.t. O.
 *   dq, dk, dv  device, [B, H, N, D] of `dtype`, overwritten with the gradients w.r.t.
 *            the un-rotated inputs.
 *   dalpha   device, 1 fp32, overwritten with dL/dalpha (0 in FIB_INT mode, where the
 *            offsets are piecewise constant in alpha); may be NULL to skip it.
 *   workspace  device scratch of at least fib_sparse_attn_bwd_workspace_size(...) bytes,
 *            16-byte aligned; its contents on entry are ignored.
 * The result is deterministic (no floating-point atomics).
 */
int fib_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse,
                        void* dq, void* dk, void* dv, float* dalpha,
                        int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                        int W, float alpha, const int32_t* base, int n_base,
                        float rope_theta, int mode,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * fib_sparse_attn_bwd without a workspace argument, for callers that cannot allocate device
 * memory around the call (code under HIP graph capture, tight training loops, harnesses that
 * forbid allocation). The workspace lives in a fixed device array inside the library,
 * FIB_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held from the first call on that GPU until the
 * process ends; the call allocates and frees nothing. Arguments, results and errors are those
 * of fib_sparse_attn_bwd, plus FIB_ERR_SCRATCH (nothing launched) when
 * fib_sparse_attn_bwd_workspace_size_for(B, H, N, D, dtype, mode, W, alpha, base, n_base)
 * exceeds the scratch: e.g. every FIB_INT call up to about 16M (b, h, n) rows, and FIB_INTERP
 * bf16 calls up to 64 MiB / (264 + 4 x entries) bytes per row (about 220K rows with 11
 * entries).
 * All calls on one GPU share the array: calls that overlap in time on that GPU (different
 * streams, or host threads) race and must be serialized by the caller.
 */
#define FIB_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fib_sparse_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse,
                                void* dq, void* dk, void* dv, float* dalpha,
                                int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                                int W, float alpha, const int32_t* base, int n_base,
                                float rope_theta, int mode, void* stream);

/* Bytes of device workspace fib_sparse_attn_bwd needs for these sizes (0 on bad sizes),
 * enough for any base and alpha: about 4 bytes per (b, h, n) row for Delta = <dO, O> and the
 * d(alpha) partials; for bf16 inputs in FIB_INTERP mode also 4 * D bytes per row, where the
 * query side leaves the RoPE-rotated q and k rows (bf16) for the key side, and 4 bytes per
 * row and possible table entry (FIB_MAX_BASE of them) in which it hands each (query, entry)
 * pair's softmax weight and dS to the key side. */
size_t fib_sparse_attn_bwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D,
                                          int dtype, int mode);

/* The same for calls with this W and base and every alpha <= alpha_max (a host alpha, the
 * top of a device alpha's declared range, or the largest alpha of a layer stack): the
 * (query, entry) words then cover only the base entries with alpha_max * f >= W, the entries
 * such a call can keep (interpolated mode keeps d = alpha f >= W). 0 on bad arguments. A
 * backward call checks its workspace against this size for its own alphas. */
size_t fib_sparse_attn_bwd_workspace_size_for(int64_t B, int64_t H, int64_t N, int64_t D, int dtype, int mode,
                                              int W, float alpha_max, const int32_t* base, int n_base);

/*
 * Decode step: the newest position of a key/value cache attends its window and offset keys
 * ([FIB] Method > Architecture and attention mechanism; Results 2 compares the inference
 * cost of the integer and interpolated gathers). The result equals row N - 1 of
 * fib_sparse_attn_fwd over the cache with this query at position N - 1.
 *   q        device, [B, H, D] of `dtype`: the query of position N - 1, un-rotated.
 *   k_cache, v_cache  device, [B, H, N, D] of `dtype`: keys and values of positions
 *            0..N-1 (the new position's included), un-rotated.
 *   o        device, [B, H, D] of `dtype`, written.
 *   lse      device, [B, H] fp32, written; may be NULL.
 * The other arguments, the errors and the ownership rules are those of fib_sparse_attn_fwd.
 */
int fib_sparse_attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                           int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                           int W, float alpha, const int32_t* base, int n_base,
                           float rope_theta, int mode, void* stream);

/*
 * alpha in device memory (the Learned schedule of [FIB] Method > Experimental variables
 * trains alpha on the device): the same operations with alpha read from `alpha` (device,
 * one fp32) instead of a host value, so a call needs no device-to-host copy and no stream
 * synchronization. The offset table is built on the device, by a small kernel enqueued on
 * `stream` ahead of the attention kernels, into `plan` (device, at least
 * fib_sparse_attn_plan_bytes() bytes, 16-byte aligned, overwritten; its contents on entry
 * are ignored; it must not be shared by calls that overlap). Kernel instances are chosen on
 * the host to fit every alpha in [alpha_lo, alpha_hi] (0 < alpha_lo <= alpha_hi, finite);
 * the device value is clamped into that range (a NaN becomes alpha_lo). A wide range can
 * select slower instances than the exact alpha would. Results equal the host-alpha calls'
 * up to floating-point summation order.
 * Errors as for the host-alpha calls, plus FIB_ERR_NULL for a NULL alpha or plan,
 * FIB_ERR_ALPHA for a bad range, FIB_ERR_ALIGN for a misaligned alpha or plan and
 * FIB_ERR_WORKSPACE for plan_bytes below fib_sparse_attn_plan_bytes().
 */
size_t fib_sparse_attn_plan_bytes(void);

int fib_sparse_attn_fwd_dev(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                            int W, const float* alpha, float alpha_lo, float alpha_hi,
                            const int32_t* base, int n_base, float rope_theta, int mode,
                            void* plan, size_t plan_bytes, void* stream);

int fib_sparse_attn_bwd_dev(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse,
                            void* dq, void* dk, void* dv, float* dalpha,
                            int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                            int W, const float* alpha, float alpha_lo, float alpha_hi,
                            const int32_t* base, int n_base, float rope_theta, int mode,
                            void* workspace, size_t workspace_bytes, void* plan, size_t plan_bytes,
                            void* stream);

int fib_sparse_attn_decode_dev(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                               int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                               int W, const float* alpha, float alpha_lo, float alpha_hi,
                               const int32_t* base, int n_base, float rope_theta, int mode,
                               void* plan, size_t plan_bytes, void* stream);

/*
 * Several layers in one call (one launch per kernel for the whole stack of layers; each
 * layer has its own alpha, e.g. the Staggered-linear, Staggered-coprime or Learned
 * schedules of [FIB] Method > Experimental variables, which assign one alpha per layer).
 * Layer l computes exactly what the single-layer call with alpha[l] computes, on the l-th
 * [B, H, N, D] block of the inputs:
 *   q, k, v, o, dout, dq, dk, dv: [L, B, H, N, D] contiguous; lse: [L, B, H, N];
 *   dalpha (backward, may be NULL): device float[L], dL/dalpha of each layer;
 *   alpha: fib_sparse_attn_fwd_layers / _bwd_layers: host float[L], read during the call
 *          (each finite and > 0); the kernels are planned for [min alpha, max alpha];
 *          ..._dev: device float[L], clamped into [alpha_lo, alpha_hi] as in the
 *          device-alpha calls above;
 *   plan: device buffer of fib_sparse_attn_layers_plan_bytes(L) bytes, 16-byte aligned,
 *         overwritten (one offset table per layer, built on the device); calls that
 *         overlap must not share it;
 *   workspace (backward): fib_sparse_attn_bwd_workspace_size(L * B, H, N, D, dtype, mode)
 *         bytes.
 * Decode over a stack (fib_sparse_attn_decode_layers, ..._dev): q and o [L, B, H, D], the
 * caches [L, B, H, N, D], lse [L, B, H]; layer l is fib_sparse_attn_decode with alpha[l]
 * (one launch for the whole stack).
 * 1 <= L <= 256. Errors as for the single-layer calls; FIB_ERR_SHAPE for L outside
 * [1, 256]; FIB_ERR_WORKSPACE for a plan smaller than fib_sparse_attn_layers_plan_bytes(L).
 * fib_sparse_attn_layers_plan_bytes returns 0 for L outside [1, 256].
 */
size_t fib_sparse_attn_layers_plan_bytes(int64_t n_layers);

int fib_sparse_attn_fwd_layers(const void* q, const void* k, const void* v, void* o, float* lse,
                               int64_t L, int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                               int W, const float* alpha, const int32_t* base, int n_base,
                               float rope_theta, int mode, void* plan, size_t plan_bytes, void* stream);

int fib_sparse_attn_decode_layers(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                  int64_t L, int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                                  int W, const float* alpha, const int32_t* base, int n_base,
                                  float rope_theta, int mode, void* plan, size_t plan_bytes, void* stream);

int fib_sparse_attn_decode_layers_dev(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                      int64_t L, int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                                      int W, const float* alpha, float alpha_lo, float alpha_hi,
                                      const int32_t* base, int n_base, float rope_theta, int mode,
                                      void* plan, size_t plan_bytes, void* stream);

int fib_sparse_attn_fwd_layers_dev(const void* q, const void* k, const void* v, void* o, float* lse,
                                   int64_t L, int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                                   int W, const float* alpha, float alpha_lo, float alpha_hi,
                                   const int32_t* base, int n_base, float rope_theta, int mode,
                                   void* plan, size_t plan_bytes, void* stream);

int fib_sparse_attn_bwd_layers(const void* q, const void* k, const void* v, const void* o,
                               const void* dout, const float* lse,
                               void* dq, void* dk, void* dv, float* dalpha,
                               int64_t L, int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                               int W, const float* alpha, const int32_t* base, int n_base,
                               float rope_theta, int mode, void* workspace, size_t workspace_bytes,
                               void* plan, size_t plan_bytes, void* stream);

int fib_sparse_attn_bwd_layers_dev(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse,
                                   void* dq, void* dk, void* dv, float* dalpha,
                                   int64_t L, int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                                   int W, const float* alpha, float alpha_lo, float alpha_hi,
                                   const int32_t* base, int n_base, float rope_theta, int mode,
                                   void* workspace, size_t workspace_bytes, void* plan, size_t plan_bytes,
                                   void* stream);

/*
 * Dropped attention mass (diagnostic): the softmax weight that dense causal attention puts
 * on keys outside the sparse set, the attention-gap measure of "SSA: Sparse Sparse
 * Attention" (arXiv 2511.20102, gist.science summary, 1. Problem definition, item 1)
 * applied to this pattern. For query i with integer offsets:
 *   dropped[i] = 1 - exp(lse_sparse[i] - lse_dense[i]),
 * lse_sparse from fib_sparse_attn_fwd (mode FIB_INT) and lse_dense from
 * fib_dense_causal_lse on the same q, k and rope_theta.
 *
 * fib_dense_causal_lse: lse [B, H, N] (natural log, fp32) of the dense causal logits
 * <R_i q_i, R_j k_j> / sqrt(D), j <= i. O(N^2) work per head on bf16 MFMA: q and k are
 * rotated in fp32 and rounded to bf16 (fp32 inputs too) into the workspace
 * (fib_dense_lse_workspace_size bytes, caller-owned, 16-byte aligned), products accumulate
 * in fp32. Errors: FIB_ERR_NULL, FIB_ERR_SHAPE, FIB_ERR_HEAD_DIM, FIB_ERR_DTYPE,
 * FIB_ERR_THETA, FIB_ERR_WORKSPACE, FIB_ERR_ALIGN, FIB_ERR_LAUNCH.
 * fib_sparse_attn_dropped_mass: the elementwise map above over `count` device floats.
 * fib_dense_lse_workspace_size returns 0 for a bad shape.
 */
size_t fib_dense_lse_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D, int dtype);

int fib_dense_causal_lse(const void* q, const void* k, float* lse, int64_t B, int64_t H, int64_t N, int64_t D,
                         int dtype, float rope_theta, void* workspace, size_t workspace_bytes, void* stream);

int fib_sparse_attn_dropped_mass(const float* lse_sparse, const float* lse_dense, float* dropped, int64_t count,
                                 void* stream);

/* Static, human-readable text of a status code. */
const char* fib_status_string(int status);

/*
 * Host-only: the per-layer offset table the kernels use ([FIB] Method: d_k = alpha * f_k).
 *   FIB_INT:    out_dist[e] = kept offsets r (ascending), out_w[e] = 0, out_f[e] = 0.
 *   FIB_INTERP: out_dist[e] = c_k = ceil(alpha f_k), out_w[e] = fp32(c_k - alpha f_k),
 *               out_f[e] = f_k, for kept entries in base order.
 * Entries whose distance does not fit in int32 are dropped (no query can use them).
 * out_* are host arrays of capacity >= n_base; *out_n receives the entry count.
 */
int fib_sparse_attn_offset_table(float alpha, const int32_t* base, int n_base, int W, int mode,
                                 int32_t* out_dist, float* out_w, int32_t* out_f, int* out_n);

/*
 * Device debug export of the attended rows ([FIB] Method > Architecture and attention
 * mechanism: window of W keys plus one row, or one interpolated row pair, per kept offset).
 * It is built from the device offset table and the per-query validity rule of the general
 * (non-ring) kernels; the LDS-ring kernels apply the same table with their own masking and
 * ring addressing, so this export pins the table and the general kernels, not the ring
 * kernels (their attended sets are checked through their outputs). out: device int32
 * [N, out_cols], out_cols must equal W + (entry count of fib_sparse_attn_offset_table), i.e.
 * W plus the kept entries (at most n_base); column s < W holds the window key i - s, column
 * W + e the row i - dist[e] (interpolated: the lower row i - c_e), and -1 where the key does
 * not exist (before position 0).
 */
int fib_sparse_attn_index_set(int64_t N, int W, float alpha, const int32_t* base, int n_base,
                              int mode, int32_t* out, int64_t out_cols, void* stream);

/* Host-only: alpha of layer `layer` of an n_layers schedule (FIB_SCHED_*), as fp32. */
int fib_schedule_alpha(int schedule, int layer, int n_layers, float* out_alpha);

#ifdef __cplusplus
}
#endif

#endif /* FIBATTN_H */
