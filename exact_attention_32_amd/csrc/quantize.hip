// quantize.hip -- per-block fp8 (E4M3 or E5M2) quantisation on MI355X (gfx950).
//
// The step before the block-scaled fp8 attention: one fp32 scale per
// (batch, head, 128-row block) taken from the block's largest |x|
// (FlashAttention-3 deep dive (techknowgenie), section 4, block quantisation),
// descale = amax / fmax (fmax = largest finite value: 448 for E4M3, 57344 for
// E5M2; 1 for an all-zero block), code = the fp8 value nearest to
// x / descale, ties to even, saturating at +-fmax.
//
// The path is HBM-bound (4, 2 or 2 bytes in and 1 byte out per element), so the
// kernel is one read of the block into registers, one reduction, one write:
// a workgroup of 4 d threads owns one 128-row block (128 x d elements), each
// thread holds 8 groups of 4 consecutive elements (coalesced 16- or 8-byte
// loads, 4-byte code stores); 32 data registers per thread leave room for 8
// waves per SIMD, so many loads are in flight.
//
// Exact rounding: the fp32 quotient q = RN(x / descale) and the exact quotient
// lie on the same side of every code midpoint unless q is itself a midpoint
// (a midpoint between them would be a closer float), so only then is the exact
// residual x - q * descale (one FMA, exact for a correctly rounded quotient)
// consulted, and q is moved one float towards the exact quotient before the
// hardware's round-to-nearest-even conversion.  The correctly rounded division
// is a long instruction sequence, so the common case takes x * RN(1 / descale)
// instead: that product is within 2 floats of the exact quotient, so its code is
// the exact quotient's unless a midpoint lies within 4 floats of it; only those
// elements (and the subnormal range) take the exact path.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "attn.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int QBLK = 128;    // rows per scale block
constexpr int QPER = 8;      // groups of 4 elements per thread
template <int D> constexpr int qthreads() { return QBLK * D / 4 / QPER; }   // 512 (d = 128), 256 (d = 64)

template <class In> __device__ __forceinline__ f32x4 load4(const In *p);
template <> __device__ __forceinline__ f32x4 load4<float>(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}
// 16-bit storage types (2 bytes, so that pointer arithmetic counts elements); a bfloat16 value
// is the upper half of a float
struct bf16_t {
    uint16_t bits;
};
struct f16_t {
    uint16_t bits;
};
static_assert(sizeof(bf16_t) == 2 && sizeof(f16_t) == 2, "16-bit element types");
template <> __device__ __forceinline__ f32x4 load4<bf16_t>(const bf16_t *p) {
    const u16x4 v = *reinterpret_cast<const u16x4 *>(p);
    return f32x4{__uint_as_float((uint32_t)v[0] << 16), __uint_as_float((uint32_t)v[1] << 16),
                 __uint_as_float((uint32_t)v[2] << 16), __uint_as_float((uint32_t)v[3] << 16)};
}
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
template <> __device__ __forceinline__ f32x4 load4<f16_t>(const f16_t *p) {
    const f16x4 v = *reinterpret_cast<const f16x4 *>(p);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// Format constants: largest finite value, smallest normal, the float mantissa bits below the
// kept ones (mask and the midpoint pattern), and 1 / half the subnormal spacing.
template <int FMT> struct Fp8Fmt;
template <> struct Fp8Fmt<0> {   // E4M3: 3 mantissa bits, subnormal spacing 2^-9
    static constexpr float fmax = 448.0f, min_normal = 0x1p-6f, inv_half_ulp_sub = 1024.0f;
    static constexpr uint32_t low_mask = 0xFFFFFu, half = 0x80000u;
};
template <> struct Fp8Fmt<1> {   // E5M2: 2 mantissa bits, subnormal spacing 2^-16
    static constexpr float fmax = 57344.0f, min_normal = 0x1p-14f, inv_half_ulp_sub = 131072.0f;
    static constexpr uint32_t low_mask = 0x1FFFFFu, half = 0x100000u;
};

// x / ds as the float that the hardware's nearest-even conversion maps to the code of the exact
// quotient (see the file comment); |result| <= fmax
template <int FMT> __device__ __forceinline__ float quotient_exact(float x, float ds) {
    using F = Fp8Fmt<FMT>;
    float q = x / ds;   // correctly rounded division
    const float a = fabsf(q);
    if (a >= F::fmax) return copysignf(F::fmax, q);
    bool mid;
    if (a >= F::min_normal) {
        // normal range: the kept mantissa bits, the next one set, the rest zero
        mid = (__float_as_uint(a) & F::low_mask) == F::half;
    } else {
        // subnormal range: midpoints are the odd multiples of half the spacing
        const float t = a * F::inv_half_ulp_sub;
        mid = (t == truncf(t)) && (((int)t & 1) != 0);
    }
    if (mid) {
        const float r = fmaf(-q, ds, x);   // exact residual
        if (r != 0.0f)
            q = __uint_as_float(__float_as_uint(q) + (((r > 0.0f) == (q > 0.0f)) ? 1u : 0xFFFFFFFFu));
    }
    return q;
}

// The same result, with inv = RN(1 / ds): the product when no code midpoint can lie between it
// and the exact quotient, else quotient_exact
template <int FMT> __device__ __forceinline__ float quotient(float x, float ds, float inv) {
    using F = Fp8Fmt<FMT>;
    const float q = x * inv;
    const float a = fabsf(q);
    if (a >= F::fmax) return copysignf(F::fmax, q);
    bool near = true;   // subnormal range: always the exact path
    if (a >= F::min_normal) near = (__float_as_uint(a) & F::low_mask) - (F::half - 4u) <= 8u;
    return near ? quotient_exact<FMT>(x, ds) : q;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// four quotients -> four codes (nearest even), first value in the low byte
template <int FMT> __device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d);
template <> __device__ __forceinline__ uint32_t pack4<0>(float a, float b, float c, float d) {
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}
template <> __device__ __forceinline__ uint32_t pack4<1>(float a, float b, float c, float d) {
    const int w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
}

// Up to three tensors (Q, K, V) per launch: blockIdx.y selects the tensor, blockIdx.x the
// (b, h, 128-row block).
struct QuantParams {
    const void *x[3];
    uint32_t *codes[3];
    float *descale[3];
    int S[3], nblk[3], nwg[3];
};

template <int D, class In, int FMT>
__global__ __launch_bounds__(qthreads<D>()) void quantize_fp8_kernel(QuantParams qp) {
    constexpr int QTHREADS = qthreads<D>(), PER = QPER;
    static_assert(PER * 4 * QTHREADS == QBLK * D, "block shape");
    const int which = blockIdx.y;
    const int blk = blockIdx.x;
    if (blk >= qp.nwg[which]) return;   // the whole workgroup leaves before its barrier
    const In *__restrict__ x = static_cast<const In *>(qp.x[which]);
    uint32_t *__restrict__ codes = qp.codes[which];
    float *__restrict__ descale = qp.descale[which];
    const int S = qp.S[which], nblk = qp.nblk[which];
    const int tid = threadIdx.x;
    const int bh = blk / nblk, j = blk - bh * nblk;
    const int r0 = j * QBLK;
    const int rows = min(QBLK, S - r0);
    const size_t base = ((size_t)bh * S + r0) * D;   // first element of the block

    f32x4 v[PER];
    float amax = 0.0f;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int g = tid + p * QTHREADS;   // group index inside the block
        if ((4 * g) / D < rows) {
            v[p] = load4<In>(x + base + 4 * g);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[p][0]), fabsf(v[p][1])), fmaxf(fabsf(v[p][2]), fabsf(v[p][3]))));
        } else {
            v[p] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    __shared__ float red[QTHREADS / 64];
    amax = wave_max(amax);
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int i = 1; i < QTHREADS / 64; ++i) amax = fmaxf(amax, red[i]);
    const float ds = amax > 0.0f ? amax / Fp8Fmt<FMT>::fmax : 1.0f;
    const float inv = 1.0f / ds;
    if (tid == 0) descale[blk] = ds;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
        const int g = tid + p * QTHREADS;
        if ((4 * g) / D < rows) {
            codes[(base + 4 * g) / 4] = pack4<FMT>(quotient<FMT>(v[p][0], ds, inv), quotient<FMT>(v[p][1], ds, inv),
                                                   quotient<FMT>(v[p][2], ds, inv), quotient<FMT>(v[p][3], ds, inv));
        }
    }
}

template <int D, int FMT>
int launch_quant(const QuantParams &qp, int ntensors, int dtype, hipStream_t s) {
    constexpr int QTHREADS = qthreads<D>();
    int gx = 0;
    for (int i = 0; i < ntensors; ++i) gx = qp.nwg[i] > gx ? qp.nwg[i] : gx;
    const dim3 grid(gx, ntensors);
    if (dtype == ATTN_F32)
        hipLaunchKernelGGL((quantize_fp8_kernel<D, float, FMT>), grid, dim3(QTHREADS), 0, s, qp);
    else if (dtype == ATTN_BF16)
        hipLaunchKernelGGL((quantize_fp8_kernel<D, bf16_t, FMT>), grid, dim3(QTHREADS), 0, s, qp);
    else
        hipLaunchKernelGGL((quantize_fp8_kernel<D, f16_t, FMT>), grid, dim3(QTHREADS), 0, s, qp);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// argument checks of one tensor; fills slot i of qp (an empty tensor, B, H or S = 0, leaves the
// slot with no workgroups, and its pointers are not used)
int check_tensor(const void *x, void *codes, float *descale, int B, int H, int S, QuantParams *qp, int i) {
    if (B < 0 || H < 0 || S < 0) return ATTN_ERR_SHAPE;
    if (B == 0 || H == 0 || S == 0) return ATTN_OK;
    if (!x || !codes) return ATTN_ERR_NULL;
    if (!descale) return ATTN_ERR_DESCALE;
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(codes)) & 15u) return ATTN_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(descale) & 3u) return ATTN_ERR_DESCALE;
    const long long nblk = (S + QBLK - 1) / QBLK;
    const long long nwg = (long long)B * H * nblk;
    if (nwg > INT_MAX || (long long)B * H > INT_MAX / S) return ATTN_ERR_OVERFLOW;
    qp->x[i] = x;
    qp->codes[i] = static_cast<uint32_t *>(codes);
    qp->descale[i] = descale;
    qp->S[i] = S;
    qp->nblk[i] = (int)nblk;
    qp->nwg[i] = (int)nwg;
    return ATTN_OK;
}

int check_types(int dtype, int d) {
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_F16) return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

int launch_checked(const QuantParams &qp, int ntensors, int dtype, int d, int fmt, void *stream) {
    int any = 0;
    for (int i = 0; i < ntensors; ++i) any |= qp.nwg[i];
    if (!any) return ATTN_OK;   // every tensor is empty: nothing to launch
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fmt == 0)
        return d == 128 ? launch_quant<128, 0>(qp, ntensors, dtype, s) : launch_quant<64, 0>(qp, ntensors, dtype, s);
    return d == 128 ? launch_quant<128, 1>(qp, ntensors, dtype, s) : launch_quant<64, 1>(qp, ntensors, dtype, s);
}

template <int FMT>
int quantize(const void *x, int dtype, void *codes, float *descale, int B, int H, int S, int d, void *stream) {
    int st = check_types(dtype, d);
    if (st != ATTN_OK) return st;
    QuantParams qp = {};
    st = check_tensor(x, codes, descale, B, H, S, &qp, 0);
    if (st != ATTN_OK) return st;
    return launch_checked(qp, 1, dtype, d, FMT, stream);
}

}  // namespace

extern "C" int attn_quantize_e4m3(const void *x, int dtype, void *codes, float *descale, int B, int H, int S, int d,
                                  void *stream) {
    return quantize<0>(x, dtype, codes, descale, B, H, S, d, stream);
}

extern "C" int attn_quantize_e5m2(const void *x, int dtype, void *codes, float *descale, int B, int H, int S, int d,
                                  void *stream) {
    return quantize<1>(x, dtype, codes, descale, B, H, S, d, stream);
}

extern "C" int attn_quantize_qkv(const void *q, const void *k, const void *v, int dtype, int fmt, void *q_codes,
                                 void *k_codes, void *v_codes, float *q_descale, float *k_descale, float *v_descale,
                                 int B, int H, int S_q, int S_k, int d, void *stream) {
    if (fmt != ATTN_FP8_E4M3 && fmt != ATTN_FP8_E5M2) return ATTN_ERR_UNSUPPORTED;
    int st = check_types(dtype, d);
    if (st != ATTN_OK) return st;
    QuantParams qp = {};
    st = check_tensor(q, q_codes, q_descale, B, H, S_q, &qp, 0);
    if (st == ATTN_OK) st = check_tensor(k, k_codes, k_descale, B, H, S_k, &qp, 1);
    if (st == ATTN_OK) st = check_tensor(v, v_codes, v_descale, B, H, S_k, &qp, 2);
    if (st != ATTN_OK) return st;
    return launch_checked(qp, 3, dtype, d, fmt == ATTN_FP8_E5M2 ? 1 : 0, stream);
}
