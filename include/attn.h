/*
 * attn.h -- C ABI of the MI355X (gfx950) fused exact-attention forward library.
 *
 * Operation (the attention that the FlashAttention-3 deep dive (techknowgenie)
 * introduces and computes with I/O-aware tiling plus an online softmax, so
 * that the S_q x S_k score matrix never reaches HBM; section 2 lists the
 * per-key-block steps: scores, running max/sum update, output accumulation):
 *
 *   O[b,h,i,:] = sum_j softmax_j( scale * q[b,h,i,:] . k[b,h,j,:] ) * v[b,h,j,:]
 *   LSE[b,h,i] = log sum_j exp( scale * q[b,h,i,:] . k[b,h,j,:] )      (natural log)
 *
 * with j over all keys, or, when causal != 0, over the keys j <= i only
 * (top-left aligned: query i sees keys 0..i whatever S_q and S_k are).
 *
 * Layout: q and o are [B][H][S_q][d]; k and v are [B][H][S_k][d]; lse is
 * [B][H][S_q] fp32.  All dense, row-major, d fastest.  All pointers are
 * device pointers on the current HIP device, where the kernels are launched;
 * `stream` must belong to that device.
 *
 * Ownership: the caller allocates and owns every buffer.  The library keeps no
 * per-call state, allocates nothing and is re-entrant.  Calls are asynchronous
 * on `stream` (a hipStream_t; NULL means the default stream); the results are
 * ready when that stream has reached the launch.  With a given build the
 * results are deterministic (no atomics).
 *
 * Errors: every argument is checked on the host before anything is enqueued;
 * on any error nothing is launched and o/lse are untouched.
 *
 * Empty inputs: sizes may be 0.  A call with no query rows (B, H or S_q = 0)
 * checks d, dtype and scale, then returns ATTN_OK without launching, reading
 * or writing anything (its pointers may then be NULL).  S_k = 0 while there
 * are query rows is ATTN_ERR_SHAPE: a softmax over no keys is undefined.  The
 * quantisers and the RMSNorm likewise do nothing for a tensor with no rows.  The guards follow
 * the host-side checks that the FlashInfer KDA write-up (blog.secrett2633)
 * describes in its section 3 (16-byte base alignment, 32-bit index range).
 */
#ifndef EXACT_ATTENTION_32_AMD_ATTN_H
#define EXACT_ATTENTION_32_AMD_ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_F16 = 0,       /* q, k, v, o are IEEE binary16 */
    ATTN_BF16 = 1,      /* q, k, v, o are bfloat16 */
    ATTN_FP8_E4M3 = 2,  /* q, k, v are OCP E4M3 codes (unit descales), o is bfloat16 */
    ATTN_F32 = 3,       /* IEEE binary32: an input type of the quantisers only */
    ATTN_FP8_E5M2 = 4   /* q, k, v are OCP E5M2 codes (unit descales), o is bfloat16 */
} attn_dtype;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,         /* q, k, v or o is NULL (lse may be NULL: then it is not written) */
    ATTN_ERR_SHAPE = 2,        /* a size < 0, or S_k = 0 while there are query rows */
    ATTN_ERR_UNSUPPORTED = 3,  /* d not 64 or 128, or unknown dtype */
    ATTN_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned */
    ATTN_ERR_OVERFLOW = 5,     /* S*d or the grid size exceeds the 32-bit index range */
    ATTN_ERR_LAUNCH = 6,       /* the HIP runtime refused the launch (no device, bad stream, ...) */
    /* codes past the six of the original plan, for checks it did not foresee: */
    ATTN_ERR_VALUE = 7,        /* scale (or the RMSNorm's eps) is not finite or out of range */
    ATTN_ERR_DESCALE = 8       /* fp8 path: a descale pointer is NULL or misaligned (4 bytes) */
} attn_status;

/*
 * Exact-attention forward for fp16 / bf16 (and unit-descale fp8) inputs.
 *   q, k, v : device pointers, layout above, element type per `dtype`
 *   o       : device pointer, [B][H][S_q][d]; f16 for ATTN_F16, bf16 otherwise
 *   lse     : device pointer to [B][H][S_q] fp32, natural-log LSE; may be NULL
 *   scale   : multiplies q.k before the softmax (finite, > 0), e.g. 1/sqrt(d)
 *   causal  : 0 = all keys, otherwise key j visible to query i iff j <= i
 *   stream  : hipStream_t or NULL
 * Returns an attn_status.
 */
int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int S_q, int S_k,
             int d, int causal, float scale, int dtype, void *stream);

/*
 * attn_fwd of RMSNorm(q) with k and v, the RMSNorm folded into the loads of
 * the Q operands (the QKNorm-across-heads write-up's norm, Q side): every Q
 * value the kernel uses is q[b,h,s,t] * q_rstd[b*S_q + s] * w_q[h*d + t],
 * computed in fp32 and rounded to nearest even in dtype, which is bit for bit
 * what attn_qk_rmsnorm stores, so O and LSE are those of attn_fwd on
 * attn_qk_rmsnorm's output.  q: the raw queries; q_rstd: [B][S_q] floats from
 * attn_qk_rmsnorm_split (4-byte aligned); w_q: [H*d] weights in dtype
 * (16-byte aligned); k: normalised keys (attn_qk_rmsnorm_split's k_out).
 * dtype: ATTN_BF16 or ATTN_F16 only (else ATTN_ERR_UNSUPPORTED); other
 * arguments, checks and the empty cases as attn_fwd; ATTN_ERR_NULL when q_rstd
 * or w_q is NULL with work to do.  Returns an attn_status.
 */
int attn_fwd_qnorm(const void *q, const void *k, const void *v, const float *q_rstd, const void *w_q, void *o,
                   float *lse, int B, int H, int S_q, int S_k, int d, int causal, float scale, int dtype,
                   void *stream);

/*
 * Exact-attention forward for block-scaled fp8 inputs (the FlashAttention-3
 * deep dive, section 4: per-block scale factors from each block's local
 * maximum; the score product in FP8, the softmax and the output accumulated
 * in FP32).  q, k, v hold OCP E4M3 codes; the real value of element
 * [b,h,r,t] is e4m3(code) * descale[b,h,r/128].
 *   q_descale : fp32 [B][H][ceil(S_q/128)]
 *   k_descale : fp32 [B][H][ceil(S_k/128)]
 *   v_descale : fp32 [B][H][ceil(S_k/128)]
 *   o         : bf16 [B][H][S_q][d]
 * Other arguments as for attn_fwd.  Descales must be finite and > 0.
 */
int attn_fwd_fp8(const void *q, const void *k, const void *v, const float *q_descale, const float *k_descale,
                 const float *v_descale, void *o, float *lse, int B, int H, int S_q, int S_k, int d, int causal,
                 float scale, void *stream);

/*
 * As attn_fwd_fp8 for OCP E5M2 codes (the deep dive's section 4 names E5M2
 * beside E4M3: two mantissa bits, a range up to 57344): the real value of
 * element [b,h,r,t] is e5m2(code) * descale[b,h,r/128].  The probabilities
 * are still rounded to E4M3 for the P.V product.  Arguments, layout, errors
 * and ownership as for attn_fwd_fp8.
 */
int attn_fwd_fp8_e5m2(const void *q, const void *k, const void *v, const float *q_descale,
                      const float *k_descale, const float *v_descale, void *o, float *lse, int B, int H, int S_q,
                      int S_k, int d, int causal, float scale, void *stream);

/*
 * Block quantisation to OCP E4M3, the input preparation of attn_fwd_fp8 (the
 * FlashAttention-3 deep dive, section 4: one scale per block, from the block's
 * largest magnitude).  For every (b, h) and block of 128 rows of
 * x[B][H][S][d] (the last block may be shorter):
 *   amax       = max |x| over the block
 *   descale    = amax / 448 in fp32 (448 = largest finite E4M3), 1 if amax == 0
 *   codes[...] = the E4M3 code nearest to x / descale (exact quotient), ties
 *                to even, saturating at +-448; the sign of x is kept (-0 -> 0x80)
 *   x       : device pointer, dtype ATTN_F32, ATTN_BF16 or ATTN_F16, 16-byte aligned
 *   codes   : device pointer, uint8 [B][H][S][d], 16-byte aligned
 *   descale : device pointer, fp32 [B][H][ceil(S/128)], 4-byte aligned
 *   d       : 64 or 128; stream: hipStream_t or NULL
 * The outputs are exactly what attn_fwd_fp8 takes.  x must be finite.
 * Returns an attn_status (ATTN_ERR_DESCALE for a NULL or misaligned descale).
 */
int attn_quantize_e4m3(const void *x, int dtype, void *codes, float *descale, int B, int H, int S, int d,
                       void *stream);

/*
 * Block quantisation to OCP E5M2, the input preparation of attn_fwd_fp8_e5m2:
 * as attn_quantize_e4m3 with 57344 (the largest finite E5M2) in place of 448,
 * and the E5M2 code nearest to x / descale (ties to even, saturating at
 * +-57344).  Arguments, layout, errors and ownership as for attn_quantize_e4m3.
 */
int attn_quantize_e5m2(const void *x, int dtype, void *codes, float *descale, int B, int H, int S, int d,
                       void *stream);

/*
 * The block quantisation of attn_quantize_e4m3 / attn_quantize_e5m2 for Q, K
 * and V in one launch (the three inputs of attn_fwd_fp8 / attn_fwd_fp8_e5m2).
 *   fmt      : ATTN_FP8_E4M3 or ATTN_FP8_E5M2
 *   q        : [B][H][S_q][d], k and v: [B][H][S_k][d], all of type dtype
 *   *_codes  : uint8, the inputs' shapes; *_descale: fp32 [B][H][ceil(S/128)]
 * Results are bit-identical to the three single-tensor calls.  Argument
 * checks, errors and ownership as for attn_quantize_e4m3; a tensor with no
 * rows (S_q = 0, or S_k = 0) is skipped and its pointers may be NULL.
 */
int attn_quantize_qkv(const void *q, const void *k, const void *v, int dtype, int fmt, void *q_codes, void *k_codes,
                      void *v_codes, float *q_descale, float *k_descale, float *v_descale, int B, int H, int S_q,
                      int S_k, int d, void *stream);

/*
 * RMSNorm of Q and K across heads, the step before attention in the sglang
 * QKNorm-across-heads write-up (blog.secrett2633): for every token, one RMS
 * over its whole hidden vector (the H*d values of all heads), then
 *   out[b,h,s,t] = x[b,h,s,t] * rsqrt(eps + sum_{h',t'} x[b,h',s,t']^2 / (H*d)) * w[h*d + t]
 * computed in fp32 and stored rounded to nearest even in the tensor's type.
 *   q, q_out  : device pointers, [B][H][S_q][d]; k, k_out: [B][H][S_k][d]
 *   w_q, w_k  : device pointers, [H*d] per-channel weights
 *   dtype     : ATTN_BF16 or ATTN_F16 for all six tensors
 *   eps       : finite, >= 0;  d: 64 or 128;  H*d <= 8192
 * In place is allowed (q_out == q and/or k_out == k); other overlaps are
 * undefined.  All pointers 16-byte aligned.  The outputs are attn_fwd's q and
 * k.  A tensor with no tokens (S_q = 0, or S_k = 0) is not touched and its
 * three pointers may be NULL.  Returns an attn_status.
 */
int attn_qk_rmsnorm(const void *q, const void *k, const void *w_q, const void *w_k, void *q_out, void *k_out,
                    int B, int H, int S_q, int S_k, int d, float eps, int dtype, void *stream);

/*
 * The same step with Q's normalisation left to attention (the fused prologue
 * of the QKNorm-across-heads write-up, Q side): K is normalised exactly as
 * attn_qk_rmsnorm does it (k_out, in place allowed); for Q only the per-token
 * factor is written,
 *   q_rstd[b*S_q + s] = rsqrt(eps + sum_{h,t} q[b,h,s,t]^2 / (H*d))   (fp32),
 * the same value attn_qk_rmsnorm multiplies by.  q_rstd: device pointer,
 * [B][S_q] floats, 4-byte aligned; w_q is not needed here (attn_fwd_qnorm
 * takes it).  Other arguments, checks and the empty cases as
 * attn_qk_rmsnorm; q_rstd may be NULL when S_q = 0.  Returns an attn_status.
 */
int attn_qk_rmsnorm_split(const void *q, const void *k, const void *w_k, float *q_rstd, void *k_out, int B, int H,
                          int S_q, int S_k, int d, float eps, int dtype, void *stream);

/*
 * Tile policy.  attn_fwd picks a compiled kernel variant (schedule and tile shape) at run time from
 * a table measured on MI355X, keyed on the shape (d, causal, dtype, S_q, B*H) and on the device's
 * compute-unit count, the runtime policy that the FlashInfer KDA write-up (blog.secrett2633)
 * describes in its section 1 and its closing lessons.  The entry points below report that choice
 * and override it (for tuning and tests); none of them touches device memory.
 */

/* Schedules of the f16/bf16 kernel (attn_fwd_set_policy). */
typedef enum {
    ATTN_SCHED_DEFAULT = 0,   /* the library's measured policy table */
    ATTN_SCHED_CLASSIC = 1,   /* all waves: S = QK^T, softmax, O += PV per tile */
    ATTN_SCHED_PINGPONG = 2,  /* wave groups alternate barrier-separated MFMA and softmax intervals */
    ATTN_SCHED_DEPHASED = 3   /* the SIMD partner waves run one softmax behind */
} attn_schedule;

/*
 * Tuning and test hook: makes every later f16/bf16 attn_fwd call of this
 * process use one compiled schedule and tile shape (qb 32-query blocks per
 * wave, nw waves per workgroup, ns LDS stages, bk keys per tile) instead of
 * the measured policy table.  Compiled, as (qb, nw, ns, bk):
 *   CLASSIC   (1,8,3,64) (1,8,4,64) (2,4,3,64) (2,4,4,64) (1,4,2,64)
 *             (1,4,3,64) (1,8,2,128), and for d = 64 only (2,8,3,64)
 *             (2,8,4,64) (1,4,3,192) (1,4,2,256) (attn_fwd returns
 *             ATTN_ERR_UNSUPPORTED for these at d = 128);
 *   PINGPONG  (1,8,3,64);  DEPHASED (1,8,4,64).
 * schedule = ATTN_SCHED_DEFAULT restores the table (the other arguments are
 * then ignored).  The environment variable ATTN_FWD_POLICY =
 * "schedule,qb,nw,ns,bk", read at the first call, sets the same override.
 * Process-wide, not tied to a stream: calls in flight keep the shape they
 * were launched with.  Returns ATTN_OK, or ATTN_ERR_UNSUPPORTED for a shape
 * that is not compiled (the setting is then unchanged).
 */
int attn_fwd_set_policy(int schedule, int qb, int nw, int ns, int bk);

/*
 * The schedule that attn_fwd launches for head dimension d, causal flag and
 * dtype under the current policy (for reports and profiles): an attn_schedule
 * value for ATTN_F16 / ATTN_BF16; ATTN_SCHED_DEFAULT (0) for the fp8 dtypes,
 * which have one kernel; minus an attn_status for bad arguments.
 */
int attn_fwd_schedule(int d, int causal, int dtype);

/* Human-readable text of a status code (static storage, never NULL). */
const char *attn_status_string(int status);

/*
 * Tile shape the library launches for a problem (for reports and tests):
 * writes queries per workgroup, keys per tile, waves per workgroup and the
 * workgroup count (0 when there are no query rows).  With n query tiles of
 * block_q rows per (batch, head), the count is B*H*n, except for causal f16 /
 * bf16 problems on the classic schedule whose tiles pair up into whole rounds
 * of the device's CUs (the pairs' estimated time within 2% of single tiles
 * taken heaviest first): a workgroup then takes the query tiles n-1-j and j of
 * one head (their keys cost n+1 tiles between them), B*H*ceil(n/2) in all.
 * Returns an attn_status
 * (argument checks as attn_fwd; the CU count is queried once per device).
 */
int attn_fwd_plan(int B, int H, int S_q, int S_k, int d, int causal, int dtype, int *block_q, int *block_k,
                  int *waves, int *workgroups);

#ifdef __cplusplus
}
#endif

#endif
