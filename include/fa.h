/*
 * fa.h -- C ABI of the exact-attention library for AMD Instinct MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention with an online
 * softmax (forward) and its gradient with recomputation (backward), as
 * described in "Flash Attention 2 -- forward pass notes" (section "The
 * algorithm" and "Loop (per (b, h, Q-tile))") and "Flash Attention 2 --
 * backward pass notes" (section "The math (FA2 backward with recompute)").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.   q, k, v, dO, o, dq, dk, dv are dense row-major [B, T, H, hd]
 *           tensors (the [B, T, C] activations with C = H * hd of the forward
 *           notes).  lse and delta are dense [B, H, T] float32 vectors.
 * Dtypes.   Inputs q, k, v, dO are FA_F32 (float32), FA_BF16 (bfloat16
 *           bits) or FA_F16 (IEEE binary16 bits).  Every output and
 *           workspace is float32.
 * Mask.     causal != 0 keeps key j for query i iff j <= i (diagonal kept);
 *           causal == 0 keeps every key.  Self-attention only (one T).
 * Scale.    Scores are scale * <q_i, k_j>; scale must be finite and > 0
 *           (1/sqrt(hd) in the usual case).
 * Memory.   Every pointer is a device pointer allocated by the caller,
 *           16-byte aligned.  The library only enqueues kernels on `stream`
 *           (a hipStream_t, NULL for the default stream), in order, and
 *           returns; it allocates, frees or synchronises in one case only:
 *           fa_forward's own key split (its workspace, described there).
 *           fa_backward_nows uses a static device array instead.  Inputs are
 *           read-only.  Outputs are fully overwritten (no pre-zeroing, nothing
 *           accumulates).  Outputs must not overlap each other or any input.
 * Errors.   0 on success, a negative FA_ERR_* code otherwise.  All argument
 *           checks happen before the first launch, so a failing call writes
 *           nothing.  A launch failure reports FA_ERR_LAUNCH; kernels already
 *           enqueued by that call may have run.
 * Sizes.    B, H, T >= 1; B * H * T < 2^31 rows; B * H * T * hd < 2^40
 *           elements; H * hd < 2^25 (the row stride, in elements: the 16-bit
 *           forward addresses the rows of a key block with 32-bit byte
 *           offsets).  Larger sizes return FA_ERR_ARG.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_BF16 = 1, FA_F16 = 2 } fa_dtype;

/*
 * Operand precision of the two products whose left factor is computed inside
 * the kernel (P in P.V and dV, dS in dQ and dK).  Only meaningful for FA_BF16
 * inputs; FA_F32 inputs accept FA_PREC_DEFAULT only and compute every product
 * in float32; FA_F16 inputs accept FA_PREC_DEFAULT only and round P and dS to
 * binary16 for their products.
 *   FA_PREC_DEFAULT  same as FA_PREC_BF16 for bfloat16 inputs
 *   FA_PREC_BF16     P and dS rounded to bfloat16 before the matrix product
 *   FA_PREC_BF16X2   P and dS split into a bfloat16 value and a bfloat16
 *                    residual, two products (about 16 significant bits)
 * Accumulation is float32 in every mode.
 */
typedef enum { FA_PREC_DEFAULT = 0, FA_PREC_BF16 = 1, FA_PREC_BF16X2 = 2 } fa_precision;

enum {
  FA_OK = 0,
  FA_ERR_ARG = -1,         /* null pointer, B/H/T < 1, bad scale/causal/enum, size overflow */
  FA_ERR_ALIGN = -2,       /* a pointer is not 16-byte aligned */
  FA_ERR_UNSUPPORTED = -3, /* (hd, dtype, precision) not built */
  FA_ERR_ALIAS = -4,       /* an output overlaps an input or another output */
  FA_ERR_LAUNCH = -5,      /* the runtime rejected a kernel launch */
  FA_ERR_TOO_LARGE = -6    /* larger than fa_backward_nows's static workspace */
};

/*
 * Forward pass: o = softmax(mask(scale * q k^T)) v per (batch, head), and
 * lse[b, h, i] = m_i + ln(l_i), the natural-log log-sum-exp of row i's
 * visible scores (forward notes, "Loop (per (b, h, Q-tile))" and "What's
 * still needed for full FA2" item 1).  A row with no visible key would get
 * o = 0 and lse = -inf; with T >= 1 every row sees key 0.
 *   q, k, v   [B, T, H, hd] inputs of `dtype`
 *   o         [B, T, H, hd] float32 output
 *   lse       [B, H, T] float32 output
 * When the plain forward's work items (query tiles of 128 rows, per batch and
 * head) would fill at most half of the workgroups the GPU holds at once (few
 * (batch, head) pairs, long rows), fa_forward runs the split-key forward of
 * fa_forward_splitkv instead, with nsplit = min(64, resident workgroups /
 * work items, T / 128); the results then equal the unsplit ones up to
 * rounding, as described there.  Its workspace is one device buffer per
 * (device, stream) that the library allocates on first use and keeps until
 * the process ends; a call that needs a larger one waits for `stream`, frees
 * the old buffer and allocates a new one.  If the stream is being captured
 * into a graph and the buffer would have to grow, or an allocation fails,
 * fa_forward runs unsplit (so capture after one call of the same size).
 * Concurrent calls on one stream from several host threads are serialised
 * by the stream; they share the buffer safely only because the stream runs
 * their kernels in order.  fa_forward_splitkv with nsplit = 1 and
 * ws = NULL always runs the plain forward and allocates nothing.
 */
int fa_forward(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H, int T, int hd,
               float scale, int causal, fa_dtype dtype, fa_precision prec, void* stream);

/*
 * Split-key forward: the same outputs as fa_forward (o, lse), computed by
 * splitting each row's keys into nsplit contiguous ranges processed by
 * separate workgroups, each writing a partial (o_s, lse_s) to `ws`, followed
 * by a merge kernel that combines the partials with the associative merge of
 * the online normaliser (forward notes, the merge identity after the loop;
 * the fused-attention lesson, block "sources.onlineSoftmax", claim that the
 * merge is associative and commutative).  More workgroups per query tile:
 * for few (batch, head) pairs and long T.  Results equal fa_forward's up to
 * rounding (not bit for bit): float32 summation order, and for 16-bit inputs
 * the rounding of P, which each split takes against its own running max.
 *   ws      float32 workspace of nsplit * (B*T*H*hd + B*H*T) elements,
 *           caller-allocated; overwritten.  May be NULL when nsplit = 1:
 *           then the plain forward runs (no split, no workspace, results
 *           bit for bit those of an unsplit fa_forward)
 *   nsplit  1 .. 64
 * Other arguments and the contract as fa_forward.  Extra limit: B*H <=
 * 65535.
 */
int fa_forward_splitkv(const void* q, const void* k, const void* v, float* o, float* lse, float* ws, int B, int H,
                       int T, int hd, float scale, int causal, int nsplit, fa_dtype dtype, fa_precision prec,
                       void* stream);

/*
 * The key-split count fa_forward uses for these sizes on the current device
 * (1: no split), as described at fa_forward.  Returns a count >= 1, or a
 * negative status for invalid or unsupported arguments.  Launches nothing.
 */
int fa_forward_auto_splits(int B, int H, int T, int hd, int causal, fa_dtype dtype, fa_precision prec);

/*
 * Unfused forward (float32 inputs only), the comparator of the fused-attention
 * lesson ("Lesson K23, fused attention", blocks "sources" -- Algorithm 0 of
 * the FlashAttention paper -- and "lab"): three kernels in order on `stream`,
 * a scores kernel writing S = scale * q k^T to `scores`, a row softmax
 * kernel overwriting S with P (masked keys get P = 0), and a kernel writing
 * o = P v.  The score matrix makes 4 T^2 floats per head of extra global
 * traffic against fa_forward.  No lse is produced.
 *   q, k, v   [B, T, H, hd] float32 inputs
 *   o         [B, T, H, hd] float32 output
 *   scores    [B, H, T, T] float32 caller-provided workspace; on return it
 *             holds P
 * Extra limits: B * H <= 65535 and B * H * T * T < 2^40.  Returns
 * FA_ERR_UNSUPPORTED for bfloat16 inputs.
 */
int fa_forward_unfused(const void* q, const void* k, const void* v, float* o, float* scores, int B, int H, int T,
                       int hd, float scale, int causal, fa_dtype dtype, void* stream);

/*
 * Control variant of fa_forward (float32 inputs only), deliberately WRONG:
 * when a key block raises a row's running max, the running sum l and the
 * accumulated output are not rescaled by alpha = exp(m_old - m_new) (the
 * "broken" kernel of the fused-attention lesson, blocks "controls" and
 * "correctness"; the rescale is step 3 of "Loop (per (b, h, Q-tile))" in the
 * forward notes).  It agrees with fa_forward only while every row's max is
 * set by its first key block (T <= 32 keys for float32, 64 for half here),
 * and exists so that error checkers can be shown to reject it.  Same
 * arguments and contract as fa_forward (precision FA_PREC_DEFAULT); float32
 * and half inputs; FA_ERR_UNSUPPORTED for bfloat16.
 */
int fa_forward_norescale(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H, int T,
                         int hd, float scale, int causal, fa_dtype dtype, void* stream);

/*
 * Control variant of fa_forward, deliberately UNSAFE: the softmax without the
 * max subtracted, p = exp(s) (the naive softmax of the fused-attention
 * lesson, block "overflow"; the max subtraction is step 3 of "Loop (per (b,
 * h, Q-tile))" in the forward notes).  With FA_F16 inputs the weights enter
 * the P.V product as binary16, so any visible score s >= ln 65520 = 11.09
 * becomes an infinite weight and its row of o is not finite; with FA_F32
 * inputs the same happens only above ln(float max) = 88.7.  lse = ln(sum p).
 * Same arguments and contract as fa_forward_norescale.
 */
int fa_forward_nomax(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H, int T, int hd,
                     float scale, int causal, fa_dtype dtype, void* stream);

/*
 * Backward pass with recomputation (backward notes, "The math (FA2 backward
 * with recompute)"): from the forward's o and lse and the upstream gradient
 * dO = d loss / d o, writes dq, dk, dv.  Runs fa_backward_dq_delta, then
 * fa_backward_dkv, in order on `stream`.
 *   q, k, v, dO  [B, T, H, hd] inputs of `dtype`
 *   o            [B, T, H, hd] float32, the forward output for these inputs
 *   lse          [B, H, T] float32, the forward log-sum-exp
 *   dq, dk, dv   [B, T, H, hd] float32 outputs
 *   delta        [B, H, T] float32 caller-provided workspace; on return it
 *                holds D_i = <dO_i, o_i>
 */
int fa_backward(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dO,
                float* dq, float* dk, float* dv, float* delta, int B, int H, int T, int hd, float scale, int causal,
                fa_dtype dtype, fa_precision prec, void* stream);

/*
 * The backward stages, for callers that schedule them separately.
 * fa_backward == fa_backward_dq_delta; fa_backward_dkv, and
 * fa_backward_dq_delta == fa_backward_delta; fa_backward_dq.
 *
 * fa_backward_delta: delta[b, h, i] = <dO[b, i, h, :], o[b, i, h, :]>, the
 * pre-pass of the backward notes ("Why the WGSL kernel isn't shipped this
 * turn", option 1).
 */
int fa_backward_delta(const float* o, const void* dO, float* delta, int B, int H, int T, int hd, fa_dtype dtype,
                      void* stream);

/*
 * fa_backward_dq: one workgroup per query tile (backward notes, option 3,
 * the dQ kernel); needs lse and delta.  Writes dq only.
 */
int fa_backward_dq(const void* q, const void* k, const void* v, const float* lse, const void* dO,
                   const float* delta, float* dq, int B, int H, int T, int hd, float scale, int causal,
                   fa_dtype dtype, fa_precision prec, void* stream);

/*
 * fa_backward_dq_delta: fa_backward_delta and fa_backward_dq in one pass: each
 * query tile computes D for its rows from o and dO (the pre-pass of the
 * backward notes), writes it to delta, and produces dq (the dQ kernel of
 * option 3).  Outputs: dq and delta.
 */
int fa_backward_dq_delta(const void* q, const void* k, const void* v, const float* o, const float* lse,
                         const void* dO, float* dq, float* delta, int B, int H, int T, int hd, float scale,
                         int causal, fa_dtype dtype, fa_precision prec, void* stream);

/*
 * fa_backward_dkv: one workgroup per key tile, walking every query that can
 * see it (backward notes, option 3, the dK/dV kernel); needs lse and delta.
 * Writes dk and dv only.
 */
int fa_backward_dkv(const void* q, const void* k, const void* v, const float* lse, const void* dO,
                    const float* delta, float* dk, float* dv, int B, int H, int T, int hd, float scale,
                    int causal, fa_dtype dtype, fa_precision prec, void* stream);

/*
 * fa_backward without the delta workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Neither this call nor anything it runs
 * allocates or frees memory.  D lives in a static device array of the library
 * (4,194,304 floats = 16 MiB, one copy on each GPU the library runs on, held
 * until the process ends): B * H * T must be <= 4194304, else the call returns
 * FA_ERR_TOO_LARGE before launching anything.  The array keeps the last
 * call's D; nothing in it needs clearing (every row is written before it is
 * read).  Calls that overlap in time on one GPU share the array and race:
 * serialise them (one stream, or events).  The array's device address is
 * looked up once per device, on the first call that runs there.  Other
 * arguments, results and errors as fa_backward.
 */
int fa_backward_nows(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dO,
                     float* dq, float* dk, float* dv, int B, int H, int T, int hd, float scale, int causal,
                     fa_dtype dtype, fa_precision prec, void* stream);

/* 1 if (hd, dtype) is built (f32: hd in {8,16,32,64,128}; bf16 and f16: {64,128}), else 0. */
int fa_is_supported(int hd, fa_dtype dtype);

/* Static string naming a status code; never NULL. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
