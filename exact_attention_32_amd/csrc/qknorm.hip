// qknorm.hip -- RMSNorm of Q and K across heads on MI355X (gfx950).
//
// The step before attention in the sglang QKNorm-across-heads write-up (blog.secrett2633): for
// every token, one RMS over its whole hidden vector (all heads), then
//   out = x * rsqrt(eps + sum(x^2) / (H * d)) * w[channel]
// with a per-channel weight, and the result stored in the tensor's own type.  As on that page,
// the grid is two-dimensional (token blocks x {Q, K}), so a workgroup handles one tensor only.
//
// The path is HBM-bound (2 bytes in and 2 out per element), so the kernel is one read of each
// token into registers, one wave reduction, one write: one wave owns one token.  Q and K are
// [B][H][S][d], so a token's hidden vector is H rows of d values, S * d elements apart; lanes
// 16 l' .. 16 l' + 15 (d = 128) read one 256-byte row, and one wave load covers 4 heads (8 at
// d = 64).  Holding the token in registers makes the in-place call safe: every value of a token
// is read before any is written.
//
// The split form (attn_qk_rmsnorm_split) normalises K the same way but writes, for Q, only the
// factor r of each token (4 bytes instead of the 2 H d bytes of the normalised row); attention
// then applies q * r * w_q to its Q operands as it loads them (attn_fwd_qnorm), with the same
// arithmetic, so the result is the same bits as normalising Q here first.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "attn.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int QN_WAVES = 4;      // tokens per workgroup
constexpr int QN_MAXG = 16;      // wave loads per token held in registers: H * d <= 64 * 8 * 16
// the kernel is compiled for NG = 1, 2, 4, 8, 16 wave loads per token (registers: 4 NG VGPRs of
// data), so a small hidden size keeps more waves, and more loads in flight, per SIMD

struct Bf16 {};
struct F16 {};

// two 16-bit values of one dword -> floats
template <class T> __device__ __forceinline__ void unpack2(uint32_t u, float &a, float &b);
template <> __device__ __forceinline__ void unpack2<Bf16>(uint32_t u, float &a, float &b) {
    a = __uint_as_float(u << 16);
    b = __uint_as_float(u & 0xFFFF0000u);
}
template <> __device__ __forceinline__ void unpack2<F16>(uint32_t u, float &a, float &b) {
    const f16x2 h = __builtin_bit_cast(f16x2, u);
    a = (float)h[0];
    b = (float)h[1];
}
// two floats -> two 16-bit values (round to nearest even), first in the low half
template <class T> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<Bf16>(float a, float b) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
template <> __device__ __forceinline__ uint32_t pack2<F16>(float a, float b) {
    const f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

struct QnParams {
    const uint16_t *x[2], *w[2];   // [0]: Q, [1]: K
    uint16_t *out[2];
    int S[2];
    int B, H;
    float eps;
    float *rstd;   // non-null: Q's factor r per token goes here instead of the normalised Q
};

template <class T, int D, int NG>
__global__ __launch_bounds__(QN_WAVES * 64) void qk_rmsnorm_kernel(QnParams p) {
    constexpr int LPR = D / 8;          // lanes per row of d values (16 bytes each)
    constexpr int HPL = 64 / LPR;       // rows (heads) per wave load
    const int which = blockIdx.y;       // 0: Q, 1: K
    const int S = p.S[which], H = p.H;
    const int lane = threadIdx.x & 63;
    const int tok = blockIdx.x * QN_WAVES + (threadIdx.x >> 6);
    if (tok >= p.B * S) return;         // wave-uniform: no barrier in this kernel
    const int b = tok / S, s = tok - b * S;
    const int hsub = lane / LPR, col = (lane % LPR) * 8;
    const int ng = (H + HPL - 1) / HPL;
    const size_t hstride = (size_t)S * D;
    const uint16_t *__restrict__ x = p.x[which] + ((size_t)b * H * S + s) * D + col;
    const uint16_t *__restrict__ w = p.w[which] + col;
    uint16_t *__restrict__ out = p.out[which] + ((size_t)b * H * S + s) * D + col;

    u32x4 v[NG];
    float ss = 0.f;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const int h = gi * HPL + hsub;
        v[gi] = u32x4{0u, 0u, 0u, 0u};
        if (gi < ng && h < H) {
            v[gi] = *reinterpret_cast<const u32x4 *>(x + h * hstride);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float a, c;
                unpack2<T>(v[gi][e], a, c);
                ss = fmaf(a, a, ss);
                ss = fmaf(c, c, ss);
            }
        }
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(p.eps + ss / (float)(H * D));
    if (which == 0 && p.rstd) {
        if (lane == 0) p.rstd[tok] = r;   // tok = b * S + s
        return;
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const int h = gi * HPL + hsub;
        if (gi < ng && h < H) {
            const u32x4 wv = *reinterpret_cast<const u32x4 *>(w + h * D);
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float a, c, wa, wc;
                unpack2<T>(v[gi][e], a, c);
                unpack2<T>(wv[e], wa, wc);
                o[e] = pack2<T>(a * r * wa, c * r * wc);
            }
            *reinterpret_cast<u32x4 *>(out + h * hstride) = o;
        }
    }
}

template <class T, int D, int NG>
void launch_qn_ng(const QnParams &p, int nwg, hipStream_t s) {
    hipLaunchKernelGGL((qk_rmsnorm_kernel<T, D, NG>), dim3(nwg, 2), dim3(QN_WAVES * 64), 0, s, p);
}

template <class T, int D>
void launch_qn_d(const QnParams &p, int nwg, hipStream_t s) {
    constexpr int HPL = 64 / (D / 8);
    const int ng = (p.H + HPL - 1) / HPL;
    if (ng <= 1) launch_qn_ng<T, D, 1>(p, nwg, s);
    else if (ng <= 2) launch_qn_ng<T, D, 2>(p, nwg, s);
    else if (ng <= 4) launch_qn_ng<T, D, 4>(p, nwg, s);
    else if (ng <= 8) launch_qn_ng<T, D, 8>(p, nwg, s);
    else launch_qn_ng<T, D, 16>(p, nwg, s);
}

template <class T>
int launch_qn(const QnParams &p, int d, int nwg, hipStream_t s) {
    if (d == 128) launch_qn_d<T, 128>(p, nwg, s);
    else launch_qn_d<T, 64>(p, nwg, s);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

namespace {

// split false: Q and K normalised; true: K normalised and Q's factor r written to q_rstd
int run_qn(const void *q, const void *k, const void *w_q, const void *w_k, void *q_out, void *k_out, float *q_rstd,
           bool split, int B, int H, int S_q, int S_k, int d, float eps, int dtype, void *stream) {
    if (B < 0 || H < 0 || S_q < 0 || S_k < 0) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_UNSUPPORTED;
    if ((long long)H * d > 64LL * 8 * QN_MAXG) return ATTN_ERR_UNSUPPORTED;
    if (!std::isfinite(eps) || eps < 0.f) return ATTN_ERR_VALUE;
    if (B == 0 || H == 0 || (S_q == 0 && S_k == 0)) return ATTN_OK;   // no tokens: nothing to do
    // a tensor with no tokens is not read or written: its pointers may be NULL
    if (S_q > 0 && (!q || (split ? !q_rstd : (!w_q || !q_out)))) return ATTN_ERR_NULL;
    if (S_k > 0 && (!k || !w_k || !k_out)) return ATTN_ERR_NULL;
    const uintptr_t mis = (reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                           reinterpret_cast<uintptr_t>(w_q) | reinterpret_cast<uintptr_t>(w_k) |
                           reinterpret_cast<uintptr_t>(q_out) | reinterpret_cast<uintptr_t>(k_out)) & 15u;
    if (mis || (reinterpret_cast<uintptr_t>(q_rstd) & 3u)) return ATTN_ERR_ALIGN;
    const long long tq = (long long)B * S_q, tk = (long long)B * S_k;
    const long long tmax = tq > tk ? tq : tk;
    if (tmax > INT_MAX || (long long)B * H > INT_MAX || (long long)S_q * d > INT_MAX || (long long)S_k * d > INT_MAX)
        return ATTN_ERR_OVERFLOW;
    const long long nwg = (tmax + QN_WAVES - 1) / QN_WAVES;
    QnParams p;
    p.x[0] = static_cast<const uint16_t *>(q);
    p.x[1] = static_cast<const uint16_t *>(k);
    p.w[0] = static_cast<const uint16_t *>(w_q);
    p.w[1] = static_cast<const uint16_t *>(w_k);
    p.out[0] = static_cast<uint16_t *>(q_out);
    p.out[1] = static_cast<uint16_t *>(k_out);
    p.S[0] = S_q;
    p.S[1] = S_k;
    p.B = B;
    p.H = H;
    p.eps = eps;
    p.rstd = q_rstd;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return dtype == ATTN_BF16 ? launch_qn<Bf16>(p, d, (int)nwg, s) : launch_qn<F16>(p, d, (int)nwg, s);
}

}  // namespace

extern "C" int attn_qk_rmsnorm(const void *q, const void *k, const void *w_q, const void *w_k, void *q_out,
                               void *k_out, int B, int H, int S_q, int S_k, int d, float eps, int dtype,
                               void *stream) {
    return run_qn(q, k, w_q, w_k, q_out, k_out, nullptr, false, B, H, S_q, S_k, d, eps, dtype, stream);
}

extern "C" int attn_qk_rmsnorm_split(const void *q, const void *k, const void *w_k, float *q_rstd, void *k_out,
                                     int B, int H, int S_q, int S_k, int d, float eps, int dtype, void *stream) {
    return run_qn(q, k, nullptr, w_k, nullptr, k_out, q_rstd, true, B, H, S_q, S_k, d, eps, dtype, stream);
}
