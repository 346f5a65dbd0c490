/*
 * attn_oracle.c -- fp64 CPU oracle for the exact-attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call this code:
 * it exists so that tests, the smoke check and the benchmark's CPU-baseline
 * leg can check the GPU kernels against a plain, slow, obviously correct
 * definition.  It shares no code, header, table or helper with the GPU
 * library.
 *
 * What it computes (the plain definition of softmax attention that the
 * FlashAttention-3 deep dive (techknowgenie) introduces as "standard
 * attention" in its introduction, i.e. the result that I/O-aware tiling
 * with an online softmax reproduces without writing the score matrix to HBM):
 *
 *   for every batch b, head h, query row i:
 *     vis(i)  = { j < S_k : !causal  or  j <= i }      (causal: key j is visible
 *                                                      to query i iff j <= i)
 *     s_ij    = scale * sum_t q[b,h,i,t] * k[b,h,j,t]   (j in vis(i))
 *     m_i     = max_j s_ij
 *     e_ij    = exp(s_ij - m_i),   l_i = sum_j e_ij
 *     P_ij    = e_ij / l_i          (explicit softmax matrix; 0 where masked)
 *     O[b,h,i,:] = sum_j P_ij * v[b,h,j,:]
 *     LSE[b,h,i] = m_i + log(l_i)   (natural log)
 *
 * All arithmetic is fp64.  Inputs are fp64 arrays holding the exact decoded
 * values of the low-precision tensors (fp16/bf16 are exact in fp64; e4m3
 * codes times an fp32 descale are exact too, see oracle_decode_e4m3_blocks).
 *
 * Layout: q, o are [B][H][S_q][d]; k, v are [B][H][S_k][d]; lse is
 * [B][H][S_q]; all dense row-major with d fastest.
 *
 * Three entry points:
 *   oracle_attn_explicit  -- the definition above, one explicit P block of
 *                            up to ORACLE_ROWS query rows at a time.
 *   oracle_attn_rows      -- the same definition for a caller-chosen list of
 *                            (b*H + h, i) query rows (sampled checks at full
 *                            size).
 *   oracle_attn_online    -- the key-block loop of the deep dive's section 2
 *                            ("3-stage asynchronous software pipelining",
 *                            the FlashAttention-2 per-block steps): per key
 *                            block, scores, running max/sum update, output
 *                            accumulation; used to show that the two-pass
 *                            and the online forms agree.
 * plus oracle_decode_e4m3_blocks (fp8 input decoding, OCP E4M3 "fn" format
 * with per-(b, h, 128-row block) fp32 descale; the deep dive's section 4
 * block quantisation; oracle_decode_fp8_blocks also for OCP E5M2),
 * oracle_quantize_fp8_blocks (the block quantisation itself: per-block |max|,
 * descale, nearest code, E4M3 or E5M2), oracle_rmsnorm_across_heads (the
 * QK-RMSNorm that precedes attention in the sglang QKNorm-across-heads
 * write-up: one RMS per token over all heads) and oracle_softmax_block
 * (exposes one explicit P block so tests can check that softmax rows sum to
 * one).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_ROWS 64

typedef struct {
    const double *q, *k, *v;
    double *o, *lse;
    int B, H, Sq, Sk, d, causal;
    double scale;
    /* explicit / online work split */
    int bc;                       /* online: key block size */
    const int64_t *rows;          /* rows mode: pairs (bh, i) */
    int64_t nrows;
    /* work queue */
    int64_t nitems;
    int64_t next;
    pthread_mutex_t mu;
    int mode;                     /* 0 explicit, 1 rows, 2 online */
} job_t;

static job_t make_job(const double *q, const double *k, const double *v, double *o, double *lse, int B, int H,
                      int Sq, int Sk, int d, int causal, double scale, int mode) {
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.o = o; J.lse = lse;
    J.B = B; J.H = H; J.Sq = Sq; J.Sk = Sk; J.d = d; J.causal = causal;
    J.scale = scale;
    J.mode = mode;
    return J;
}

static int visible(int causal, int i, int j) { return !causal || j <= i; }

/* Number of keys visible to query row i. */
static int n_visible(const job_t *J, int i) {
    if (!J->causal) return J->Sk;
    return (i + 1 < J->Sk) ? i + 1 : J->Sk;
}

/* Explicit softmax for query rows [i0, i0+nr) of head bh.  P is nr x Sk. */
static void explicit_block(const job_t *J, int64_t bh, int i0, int nr, double *P, double *lse_out) {
    const int Sk = J->Sk, d = J->d;
    const double *Q = J->q + (bh * J->Sq) * (int64_t)d;
    const double *K = J->k + (bh * Sk) * (int64_t)d;
    for (int r = 0; r < nr; ++r) {
        const int i = i0 + r;
        double *p = P + (int64_t)r * Sk;
        /* scores */
        for (int j = 0; j < Sk; ++j) {
            if (!visible(J->causal, i, j)) { p[j] = 0.0; continue; }
            double acc = 0.0;
            for (int t = 0; t < d; ++t) acc += Q[(int64_t)i * d + t] * K[(int64_t)j * d + t];
            p[j] = J->scale * acc;
        }
        /* row max over visible keys */
        double m = -INFINITY;
        for (int j = 0; j < Sk; ++j)
            if (visible(J->causal, i, j) && p[j] > m) m = p[j];
        /* exponentials and row sum */
        double l = 0.0;
        for (int j = 0; j < Sk; ++j) {
            if (!visible(J->causal, i, j)) continue;
            p[j] = exp(p[j] - m);
            l += p[j];
        }
        /* normalise: explicit softmax row */
        for (int j = 0; j < Sk; ++j)
            if (visible(J->causal, i, j)) p[j] /= l;
        if (lse_out) lse_out[r] = m + log(l);
    }
}

/* O rows = P . V for the block; out is [nr][d]. */
static void apply_pv(const job_t *J, int64_t bh, int i0, int nr, const double *P, double *o_out) {
    const int Sk = J->Sk, d = J->d;
    const double *V = J->v + (bh * Sk) * (int64_t)d;
    for (int r = 0; r < nr; ++r) {
        const int i = i0 + r;
        double *out = o_out + (int64_t)r * d;
        for (int t = 0; t < d; ++t) out[t] = 0.0;
        const double *p = P + (int64_t)r * Sk;
        for (int j = 0; j < Sk; ++j) {
            if (!visible(J->causal, i, j)) continue;
            for (int t = 0; t < d; ++t) out[t] += p[j] * V[(int64_t)j * d + t];
        }
    }
}

/* Online softmax over key blocks of size bc, for one query row. */
static void online_row(const job_t *J, int64_t bh, int i) {
    const int Sk = J->Sk, d = J->d, bc = J->bc;
    const double *Q = J->q + (bh * J->Sq + i) * (int64_t)d;
    const double *K = J->k + (bh * Sk) * (int64_t)d;
    const double *V = J->v + (bh * Sk) * (int64_t)d;
    double *acc = J->o + (bh * J->Sq + i) * (int64_t)d;
    double *s = (double *)malloc(sizeof(double) * (size_t)bc);
    double m = -INFINITY, l = 0.0;
    for (int t = 0; t < d; ++t) acc[t] = 0.0;
    const int nvis = n_visible(J, i);
    for (int j0 = 0; j0 < nvis; j0 += bc) {
        const int nb = (nvis - j0 < bc) ? nvis - j0 : bc;
        /* scores of this key block */
        double mb = -INFINITY;
        for (int c = 0; c < nb; ++c) {
            const double *kr = K + (int64_t)(j0 + c) * d;
            double a = 0.0;
            for (int t = 0; t < d; ++t) a += Q[t] * kr[t];
            s[c] = J->scale * a;
            if (s[c] > mb) mb = s[c];
        }
        /* running statistics: new max, rescale factor for what is accumulated */
        const double mnew = (mb > m) ? mb : m;
        const double alpha = (m == -INFINITY) ? 0.0 : exp(m - mnew);
        l *= alpha;
        for (int t = 0; t < d; ++t) acc[t] *= alpha;
        /* accumulate this block's unnormalised probabilities times V */
        for (int c = 0; c < nb; ++c) {
            const double p = exp(s[c] - mnew);
            l += p;
            const double *vr = V + (int64_t)(j0 + c) * d;
            for (int t = 0; t < d; ++t) acc[t] += p * vr[t];
        }
        m = mnew;
    }
    for (int t = 0; t < d; ++t) acc[t] /= l;
    if (J->lse) J->lse[bh * J->Sq + i] = m + log(l);
    free(s);
}

static void *worker(void *arg) {
    job_t *J = (job_t *)arg;
    double *P = NULL;
    if (J->mode == 0 || J->mode == 1) P = (double *)malloc(sizeof(double) * (size_t)ORACLE_ROWS * (size_t)J->Sk);
    const int64_t nblk = (J->Sq + ORACLE_ROWS - 1) / ORACLE_ROWS;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t it = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (it >= J->nitems) break;
        if (J->mode == 0) {
            const int64_t bh = it / nblk;
            const int i0 = (int)(it % nblk) * ORACLE_ROWS;
            const int nr = (J->Sq - i0 < ORACLE_ROWS) ? J->Sq - i0 : ORACLE_ROWS;
            const int64_t row0 = bh * J->Sq + i0;
            explicit_block(J, bh, i0, nr, P, J->lse ? J->lse + row0 : NULL);
            apply_pv(J, bh, i0, nr, P, J->o + row0 * (int64_t)J->d);
        } else if (J->mode == 1) {
            const int64_t bh = J->rows[2 * it], i = J->rows[2 * it + 1];
            /* one explicit softmax row, written to output slot `it` */
            explicit_block(J, bh, (int)i, 1, P, J->lse ? J->lse + it : NULL);
            apply_pv(J, bh, (int)i, 1, P, J->o + it * (int64_t)J->d);
        } else {
            const int64_t bh = it / J->Sq;
            const int i = (int)(it % J->Sq);
            online_row(J, bh, i);
        }
    }
    free(P);
    return NULL;
}

static int run(job_t *J, int nthreads) {
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    pthread_mutex_init(&J->mu, NULL);
    J->next = 0;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, worker, J) != 0) break;
        ++started;
    }
    if (started == 0) worker(J);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    pthread_mutex_destroy(&J->mu);
    return started > 0 ? started : 1;
}

/* Returns the number of threads used (>= 1), or -1 on bad arguments. */
int oracle_attn_explicit(const double *q, const double *k, const double *v, double *o, double *lse,
                         int B, int H, int Sq, int Sk, int d, int causal, double scale, int nthreads) {
    if (!q || !k || !v || !o || B < 1 || H < 1 || Sq < 1 || Sk < 1 || d < 1) return -1;
    job_t J = make_job(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, 0);
    J.nitems = (int64_t)B * H * ((Sq + ORACLE_ROWS - 1) / ORACLE_ROWS);
    return run(&J, nthreads);
}

/* rows: nrows pairs (bh, i) with bh = b*H + h.  o is [nrows][d], lse [nrows]. */
int oracle_attn_rows(const double *q, const double *k, const double *v, double *o, double *lse,
                     int B, int H, int Sq, int Sk, int d, int causal, double scale,
                     const int64_t *rows, int64_t nrows, int nthreads) {
    if (!q || !k || !v || !o || !rows || B < 1 || H < 1 || Sq < 1 || Sk < 1 || d < 1) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[2 * r] < 0 || rows[2 * r] >= (int64_t)B * H || rows[2 * r + 1] < 0 || rows[2 * r + 1] >= Sq)
            return -1;
    job_t J = make_job(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, 1);
    J.rows = rows;
    J.nrows = nrows;
    J.nitems = nrows;
    return run(&J, nthreads);
}

int oracle_attn_online(const double *q, const double *k, const double *v, double *o, double *lse,
                       int B, int H, int Sq, int Sk, int d, int causal, double scale, int bc, int nthreads) {
    if (!q || !k || !v || !o || B < 1 || H < 1 || Sq < 1 || Sk < 1 || d < 1 || bc < 1) return -1;
    job_t J = make_job(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, 2);
    J.bc = bc;
    J.nitems = (int64_t)B * H * Sq;
    return run(&J, nthreads);
}

/* Explicit softmax rows [i0, i0+nr) of head bh (P is nr x S_k, 0 where masked). */
int oracle_softmax_block(const double *q, const double *k, double *P, int B, int H, int Sq, int Sk, int d,
                         int causal, double scale, int64_t bh, int i0, int nr) {
    if (!q || !k || !P || bh < 0 || bh >= (int64_t)B * H || i0 < 0 || nr < 1 || i0 + nr > Sq) return -1;
    job_t J = make_job(q, k, NULL, NULL, NULL, B, H, Sq, Sk, d, causal, scale, 0);
    explicit_block(&J, bh, i0, nr, P, NULL);
    return 0;
}

/*
 * OCP 8-bit floating point, E4M3 ("fn": no infinities, one NaN pattern per
 * sign): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
 *   e == 0            : (-1)^s * 2^-6 * (m / 8)        (subnormal)
 *   e == 15 && m == 7 : NaN
 *   otherwise         : (-1)^s * 2^(e-7) * (1 + m / 8)  (max finite 448)
 */
double oracle_e4m3_value(uint8_t code) {
    const int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/*
 * OCP 8-bit floating point, E5M2: 1 sign bit, 5 exponent bits with bias 15,
 * 2 mantissa bits, IEEE-like specials.
 *   e == 0            : (-1)^s * 2^-14 * (m / 4)        (subnormal)
 *   e == 31, m == 0   : infinity;  e == 31, m != 0 : NaN
 *   otherwise         : (-1)^s * 2^(e-15) * (1 + m / 4)  (max finite 57344)
 */
double oracle_e5m2_value(uint8_t code) {
    const int s = code >> 7, e = (code >> 2) & 31, m = code & 3;
    double mag;
    if (e == 31) return m == 0 ? (s ? -INFINITY : INFINITY) : NAN;
    if (e == 0) mag = ldexp((double)m / 4.0, -14);
    else mag = ldexp(1.0 + (double)m / 4.0, e - 15);
    return s ? -mag : mag;
}

/* value of a code of format fmt (0: E4M3, 1: E5M2) */
static double fp8_value(uint8_t code, int fmt) { return fmt ? oracle_e5m2_value(code) : oracle_e4m3_value(code); }

/* x[b,h,r,:] = e4m3(codes[b,h,r,:]) * descale[b,h,r/blk] for a [B][H][S][d] tensor. */
int oracle_decode_fp8_blocks(const uint8_t *codes, const float *descale, int B, int H, int S, int d, int blk,
                             int fmt, double *out) {
    if (!codes || !descale || !out || blk < 1 || fmt < 0 || fmt > 1) return -1;
    const int nblk = (S + blk - 1) / blk;
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh)
        for (int r = 0; r < S; ++r) {
            const double ds = (double)descale[bh * nblk + r / blk];
            for (int t = 0; t < d; ++t) {
                const int64_t idx = (bh * S + r) * (int64_t)d + t;
                out[idx] = fp8_value(codes[idx], fmt) * ds;
            }
        }
    return 0;
}

int oracle_decode_e4m3_blocks(const uint8_t *codes, const float *descale, int B, int H, int S, int d, int blk,
                              double *out) {
    return oracle_decode_fp8_blocks(codes, descale, B, H, S, d, blk, 0, out);
}

/*
 * The finite code of format fmt (0: E4M3, 1: E5M2) nearest to the real value
 * x, ties to the even code (round to nearest even), found by scanning every
 * finite non-negative code (E4M3 0x00 .. 0x7e, E5M2 0x00 .. 0x7b).
 * Magnitudes above the largest finite value (448, 57344) get that value, i.e.
 * the encoding saturates.  The sign bit is x's sign bit (-0 -> 0x80).
 */
uint8_t oracle_fp8_encode(double x, int fmt) {
    const double a = fabs(x);
    const int top = fmt ? 0x7b : 0x7e;   /* largest finite code: 57344 (E5M2), 448 (E4M3) */
    int best = 0;
    double best_err = a;   /* code 0 has value 0 */
    for (int c = 1; c <= top; ++c) {
        const double err = fabs(fp8_value((uint8_t)c, fmt) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(best | (signbit(x) ? 0x80 : 0));
}

uint8_t oracle_e4m3_encode(double x) { return oracle_fp8_encode(x, 0); }

/*
 * Block quantisation of a [B][H][S][d] fp32 tensor (the deep dive's section 4:
 * one scale per block from the block's local maximum): for each (b, h, block
 * of blk rows), amax = max |x| over the block (rows past S do not exist),
 * descale = amax / fmax as a float (fmax = largest finite value: 448 for
 * E4M3, 57344 for E5M2), or 1 when amax = 0; code = oracle_fp8_encode(
 * x / descale, fmt).  The quotient is taken in double: the exact quotient of
 * two floats that is not exactly a midpoint between codes lies at least 2^-29
 * (relative) away from every midpoint, far beyond the 2^-53 of the double
 * rounding, so the code is that of the exact quotient.
 */
int oracle_quantize_fp8_blocks(const float *x, int B, int H, int S, int d, int blk, int fmt, uint8_t *codes,
                               float *descale) {
    if (!x || !codes || !descale || B < 1 || H < 1 || S < 1 || d < 1 || blk < 1 || fmt < 0 || fmt > 1) return -1;
    const float fmax = fmt ? 57344.0f : 448.0f;   /* largest finite value of the format */
    const int nblk = (S + blk - 1) / blk;
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh)
        for (int j = 0; j < nblk; ++j) {
            const int r0 = j * blk, r1 = (r0 + blk < S) ? r0 + blk : S;
            float amax = 0.0f;
            for (int r = r0; r < r1; ++r)
                for (int t = 0; t < d; ++t) {
                    const float v = fabsf(x[(bh * S + r) * (int64_t)d + t]);
                    if (v > amax) amax = v;
                }
            const float ds = amax > 0.0f ? amax / fmax : 1.0f;
            descale[bh * nblk + j] = ds;
            for (int r = r0; r < r1; ++r)
                for (int t = 0; t < d; ++t) {
                    const int64_t idx = (bh * S + r) * (int64_t)d + t;
                    codes[idx] = oracle_fp8_encode((double)x[idx] / (double)ds, fmt);
                }
        }
    return 0;
}

int oracle_quantize_e4m3_blocks(const float *x, int B, int H, int S, int d, int blk, uint8_t *codes, float *descale) {
    return oracle_quantize_fp8_blocks(x, B, H, S, d, blk, 0, codes, descale);
}

/*
 * RMSNorm across heads (sglang QKNorm-across-heads write-up (blog.secrett2633),
 * its key-code section: one reduction per token over the whole hidden vector,
 * then rsqrt(eps + sum of squares / hidden size), times a per-channel weight).
 * The hidden vector of token (b, s) is the H*d values x[b][h][s][t] of all
 * heads h; hidden channel h*d + t has weight w[h*d + t]:
 *
 *   ms         = (1 / (H*d)) * sum_{h,t} x[b][h][s][t]^2
 *   out[b][h][s][t] = x[b][h][s][t] / sqrt(eps + ms) * w[h*d + t]
 *
 * x, out: [B][H][S][d] fp64 (may alias); w: [H*d] fp64.  All fp64.
 */
int oracle_rmsnorm_across_heads(const double *x, const double *w, int B, int H, int S, int d, double eps,
                                double *out) {
    if (!x || !w || !out || B < 1 || H < 1 || S < 1 || d < 1 || !(eps >= 0.0)) return -1;
    const int64_t hs = (int64_t)S * d;   /* stride between heads of one token */
    for (int b = 0; b < B; ++b)
        for (int s = 0; s < S; ++s) {
            const int64_t base = (int64_t)b * H * hs + (int64_t)s * d;
            double ss = 0.0;
            for (int h = 0; h < H; ++h)
                for (int t = 0; t < d; ++t) {
                    const double v = x[base + h * hs + t];
                    ss += v * v;
                }
            const double ms = ss / ((double)H * d);
            const double r = 1.0 / sqrt(eps + ms);
            for (int h = 0; h < H; ++h)
                for (int t = 0; t < d; ++t) out[base + h * hs + t] = x[base + h * hs + t] * r * w[h * d + t];
        }
    return 0;
}
