// attn_fwd.hip -- fused exact-attention forward for MI355X (gfx950, CDNA4).
//
// Computes O = softmax(scale * Q K^T [causal mask]) V and the natural-log LSE
// with I/O-aware tiling and an online softmax (FlashAttention-3 deep dive
// (techknowgenie), introduction and section 2): the score matrix lives only in
// registers, K/V tiles are streamed through LDS, and the running row max and
// sum are updated per key tile.
//
// gfx950 mapping (not the page's Hopper design):
//   * one workgroup per (batch*head, tile of BR queries); NW waves, each wave
//     owns QB blocks of 32 queries for the whole key loop;
//   * the wave computes S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16}:
//     K rows come from LDS as the A operand, Q^T is the B operand and stays in
//     VGPRs for the whole loop.  In the 32x32 accumulator every lane then holds
//     16 scores of ONE query (its column), so the row max / row sum are
//     in-lane reductions plus a single v_permlane32_swap between the two lane
//     halves;
//   * O^T = V^T P^T with the same MFMA: the S^T accumulator, rounded to the
//     input type, is already the B operand (P never leaves registers); V^T is
//     the A operand, read from an LDS copy of the V tile that is stored
//     transposed with the key order of the accumulator layout;
//   * K/V tiles are double-buffered in LDS: the global loads of tile t+1 are
//     issued before the MFMA work on tile t and written to the other LDS buffer
//     after it, one barrier per tile;
//   * exp2 with log2(e) folded into the scale (the page's section 4 computes the
//     exponent in base 2);
//   * causal: tiles wholly above the diagonal are never loaded; the mask is
//     applied only on diagonal and tail tiles; query tiles are dispatched
//     heaviest first and all tiles of one head land on one XCD.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "attn.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// clang vector types (not HIP's u32x4 struct, whose copies go through memory)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct BF16 {};
struct F16 {};

template <class T> __device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c);
template <> __device__ __forceinline__ f32x16 mfma_32x32x16<BF16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mfma_32x32x16<F16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
}

// Two floats -> two 16-bit values of type T in one dword (round to nearest even).
template <class T> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<BF16>(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
template <> __device__ __forceinline__ uint32_t pack2<F16>(float a, float b) {
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Row max between lane l and lane l^32 (the two halves of a 32x32 accumulator column).
__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct Params {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int Sq, Sk;
    int nqt;         // query tiles per (b, h)
    int num_wg;      // total workgroups
    int xcd_remap;   // 1: map workgroups so each XCD gets a contiguous range of heads
    float c;         // scale * log2(e)
};

// Position of key r (0 <= r < BC) in a transposed V row: within each group of
// 16 keys, keys 4..7 and 8..11 trade places, so that the 8 keys lane half g
// feeds to one 32x32x16 MFMA step (keys 4g..4g+3 and 8+4g..8+4g+3 of the
// accumulator layout) are contiguous.
// Dword i (compile-time after unrolling) of a 16-byte register group.
__device__ __forceinline__ uint32_t word(u32x4 v, int i) { return v[i]; }

__device__ __forceinline__ int vt_pos(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <class T, int D, int QB, int NW, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(Params p) {
    constexpr int NT = NW * 64;                // threads
    constexpr int BR = NW * QB * 32;           // queries per workgroup
    constexpr int KSTR = D * 2 + 16;           // bytes per K row in LDS (padded)
    constexpr int VSTR = BC * 2 + 16;          // bytes per V^T row in LDS (padded)
    constexpr int KBUF = BC * KSTR;
    constexpr int VBUF = D * VSTR;
    constexpr int KCHUNKS = BC * D / 8;        // 16-byte chunks in a K tile
    constexpr int KPT = KCHUNKS / NT;
    constexpr int VTASKS = (D / 8) * (BC / 4); // 4 keys x 8 columns per task
    constexpr int VPT = VTASKS / NT;
    static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
    static_assert(KCHUNKS % NT == 0 && VTASKS % NT == 0 && KPT >= 1 && VPT >= 1, "tile loads must split evenly");
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * (KBUF + VBUF)];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;

    int L = blockIdx.x;
    if (p.xcd_remap) L = (blockIdx.x & 7) * (p.num_wg >> 3) + (blockIdx.x >> 3);
    const int bh = L / p.nqt;
    int qt = L - bh * p.nqt;
    if (CAUSAL) qt = p.nqt - 1 - qt;   // heaviest query tiles first
    const int q0 = qt * BR;
    const int Sq = p.Sq, Sk = p.Sk;

    const uint16_t *__restrict__ Qh = p.q + (size_t)bh * Sq * D;
    const uint16_t *__restrict__ Kh = p.k + (size_t)bh * Sk * D;
    const uint16_t *__restrict__ Vh = p.v + (size_t)bh * Sk * D;

    const int qw0 = q0 + wave * QB * 32;   // first query of this wave

    // Q^T operands, resident for the whole key loop.
    u32x4 qf[QB][D / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = min(qw0 + qb * 32 + l32, Sq - 1);   // rows past S_q are computed, never stored
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            qf[qb][ks] = *reinterpret_cast<const u32x4 *>(Qh + (size_t)row * D + ks * 16 + g * 8);
    }

    f32x16 oacc[QB][D / 32];
    float mrow[QB], lrow[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        mrow[qb] = -INFINITY;
        lrow[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[qb][db][i] = 0.f;
    }

    int nt = (Sk + BC - 1) / BC;
    if (CAUSAL) {
        const int qlast = min(q0 + BR, Sq) - 1;
        nt = min(nt, qlast / BC + 1);
    }

    u32x4 kst[KPT];
    u32x4 vst[VPT][4];

    auto load_tile = [&](int t) __attribute__((always_inline)) {
        const int k0 = t * BC;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int c = tid + j * NT;
            {
                const int r = c / (D / 8), col = c % (D / 8);
                // rows past S_k are clamped onto the last key: their scores are masked to -inf
                // and their P is exactly 0, so any finite value is harmless
                const int key = min(k0 + r, Sk - 1);
                kst[j] = *reinterpret_cast<const u32x4 *>(Kh + (size_t)key * D + col * 8);
            }
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int tk = tid + j * NT;
            {
                const int rg = tk % (BC / 4), cg = tk / (BC / 4);   // key groups across lanes: conflict-free V^T writes
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = min(k0 + rg * 4 + r, Sk - 1);
                    vst[j][r] = *reinterpret_cast<const u32x4 *>(Vh + (size_t)key * D + cg * 8);
                }
            }
        }
    };

    auto store_tile = [&](int buf) __attribute__((always_inline)) {
        unsigned char *kb = smem + buf * (KBUF + VBUF);
        unsigned char *vb = kb + KBUF;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int c = tid + j * NT;
            {
                const int r = c / (D / 8), col = c % (D / 8);
                *reinterpret_cast<u32x4 *>(kb + r * KSTR + col * 16) = kst[j];
            }
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int tk = tid + j * NT;
            {
                const int rg = tk % (BC / 4), cg = tk / (BC / 4);   // key groups across lanes: conflict-free V^T writes
                const int pos = vt_pos(rg * 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // column e of the 4 staged rows -> 4 consecutive keys of V^T row (cg*8 + e)
                    const uint32_t w0 = word(vst[j][0], e >> 1), w1 = word(vst[j][1], e >> 1);
                    const uint32_t w2 = word(vst[j][2], e >> 1), w3 = word(vst[j][3], e >> 1);
                    u32x2 val;
                    if (e & 1) {
                        val = u32x2{(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
                    } else {
                        val = u32x2{(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
                    }
                    *reinterpret_cast<u32x2 *>(vb + (cg * 8 + e) * VSTR + pos * 2) = val;
                }
            }
        }
    };

    load_tile(0);
    store_tile(0);
    // Drain every outstanding load (the Q fragments included) before the key loop: the memory
    // counter is in order, so a first wait on Q inside the loop would also wait on the
    // prefetch of the next K/V tile.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const float c = p.c;
    for (int t = 0; t < nt; ++t) {
        const int buf = t & 1;
        if (t + 1 < nt) load_tile(t + 1);
        const int k0 = t * BC;
        const unsigned char *kb = smem + buf * (KBUF + VBUF);
        const unsigned char *vb = kb + KBUF;
        const bool active = !CAUSAL || k0 <= qw0 + QB * 32 - 1;
        if (active) {
            // S^T = K Q^T for this tile
            f32x16 s[QB][BC / 32];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                    for (int i = 0; i < 16; ++i) s[qb][kb2][i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
                for (int kb2 = 0; kb2 < BC / 32; ++kb2) {
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(kb + (kb2 * 32 + l32) * KSTR + ks * 32 + g * 16);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) s[qb][kb2] = mfma_32x32x16<T>(a, qf[qb][ks], s[qb][kb2]);
                }
            }
            // mask: keys past S_k, and (causal) keys after the query
            const bool need_mask = (k0 + BC > Sk) || (CAUSAL && k0 + BC - 1 > qw0);
            if (need_mask) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int qrow = qw0 + qb * 32 + l32;
#pragma unroll
                    for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int key = k0 + kb2 * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                            if (key >= Sk || (CAUSAL && key > qrow)) s[qb][kb2][i] = -INFINITY;
                        }
                }
            }
            // online softmax (base 2), P packed to T as the B operand of P.V
            u32x4 pf[QB][BC / 16];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float mx = -INFINITY;
#pragma unroll
                for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qb][kb2][i]);
                mx = xhalf_max(mx) * c;
                // O and l are rescaled only when some row of the wave raises its max (wave-uniform
                // branch; rows whose max did not move get alpha = 1).
                if (__builtin_amdgcn_ballot_w64(mx > mrow[qb]) != 0) {
                    const float mnew = fmaxf(mrow[qb], mx);
                    const float alpha = __builtin_amdgcn_exp2f(mrow[qb] - (mnew == -INFINITY ? 0.f : mnew));
                    mrow[qb] = mnew;
                    lrow[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) oacc[qb][db][i] *= alpha;
                }
                const float mbase = (mrow[qb] == -INFINITY) ? 0.f : mrow[qb];
#pragma unroll
                for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        s[qb][kb2][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb2][i], c, -mbase));
                // l: fp32 sum of p.  The running max is exact, so the largest p of a row is exactly 1
                // and survives the rounding of P to T unchanged.
                float ls = lrow[qb];
#pragma unroll
                for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                    for (int i = 0; i < 16; ++i) ls += s[qb][kb2][i];
                lrow[qb] = ls;
#pragma unroll
                for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int o = h * 8;
                        pf[qb][kb2 * 2 + h] = u32x4{pack2<T>(s[qb][kb2][o + 0], s[qb][kb2][o + 1]),
                                                    pack2<T>(s[qb][kb2][o + 2], s[qb][kb2][o + 3]),
                                                    pack2<T>(s[qb][kb2][o + 4], s[qb][kb2][o + 5]),
                                                    pack2<T>(s[qb][kb2][o + 6], s[qb][kb2][o + 7])};
                    }
            }
            // O^T += V^T P^T
#pragma unroll
            for (int ks = 0; ks < BC / 16; ++ks) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(vb + (db * 32 + l32) * VSTR + ks * 32 + g * 16);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = mfma_32x32x16<T>(a, pf[qb][ks], oacc[qb][db]);
                }
            }
        }
        if (t + 1 < nt) store_tile(buf ^ 1);
        __syncthreads();
    }

    // epilogue: O = O^T / l, LSE = ln2 * (m + log2 l)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = xhalf_sum(lrow[qb]);
        const float inv = 1.0f / lt;
        const int qrow = qw0 + qb * 32 + l32;
        if (qrow < Sq) {
            uint16_t *orow = p.o + ((size_t)bh * Sq + qrow) * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int gi = 0; gi < 4; ++gi) {
                    const int dv = db * 32 + 8 * gi + 4 * g;
                    u32x2 val = u32x2{pack2<T>(oacc[qb][db][gi * 4 + 0] * inv, oacc[qb][db][gi * 4 + 1] * inv),
                                           pack2<T>(oacc[qb][db][gi * 4 + 2] * inv, oacc[qb][db][gi * 4 + 3] * inv)};
                    *reinterpret_cast<u32x2 *>(orow + dv) = val;
                }
            if (p.lse && g == 0) p.lse[(size_t)bh * Sq + qrow] = (mrow[qb] + log2f(lt)) * 0.69314718055994530942f;
        }
    }
}

// ---------------------------------------------------------------------------
// host side

struct Plan {
    int block_q, block_k, waves, nqt, num_wg;
};

int check_common(const void *q, const void *k, const void *v, const void *o, const void *lse, int B, int H, int Sq,
                 int Sk, int d, float scale) {
    if (!q || !k || !v || !o) return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    const uintptr_t mis = (reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                           reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o)) & 15u;
    if (mis || (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_ALIGN;
    if ((long long)Sq * d > INT_MAX || (long long)Sk * d > INT_MAX || (long long)B * H > INT_MAX)
        return ATTN_ERR_OVERFLOW;
    if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_VALUE;
    return ATTN_OK;
}

int make_plan(int B, int H, int Sq, int d, Plan *pl) {
    // first policy: 4 waves x 32 queries; 64 keys per tile at d = 128, 128 at d = 64
    pl->waves = 4;
    pl->block_q = 4 * 32;
    pl->block_k = (d == 128) ? 64 : 128;
    pl->nqt = (Sq + pl->block_q - 1) / pl->block_q;
    const long long wg = (long long)pl->nqt * B * H;
    if (wg > INT_MAX) return ATTN_ERR_OVERFLOW;
    pl->num_wg = (int)wg;
    return ATTN_OK;
}

template <class T, int D, bool CAUSAL>
int launch(const Params &p, const Plan &pl, hipStream_t stream) {
    constexpr int BC = (D == 128) ? 64 : 128;
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, 1, 4, BC, CAUSAL>), dim3(pl.num_wg), dim3(4 * 64), 0, stream, p);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

template <class T>
int dispatch(const Params &p, const Plan &pl, int d, int causal, hipStream_t s) {
    if (d == 128) return causal ? launch<T, 128, true>(p, pl, s) : launch<T, 128, false>(p, pl, s);
    return causal ? launch<T, 64, true>(p, pl, s) : launch<T, 64, false>(p, pl, s);
}

}  // namespace

extern "C" int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int S_q,
                        int S_k, int d, int causal, float scale, int dtype, void *stream) {
    int st = check_common(q, k, v, o, lse, B, H, S_q, S_k, d, scale);
    if (st != ATTN_OK) return st;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    Plan pl;
    st = make_plan(B, H, S_q, d, &pl);
    if (st != ATTN_OK) return st;
    Params p;
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.o = static_cast<uint16_t *>(o);
    p.lse = lse;
    p.Sq = S_q;
    p.Sk = S_k;
    p.nqt = pl.nqt;
    p.num_wg = pl.num_wg;
    p.xcd_remap = (pl.num_wg % 8 == 0) ? 1 : 0;
    p.c = scale * 1.44269504088896340736f;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == ATTN_BF16) return dispatch<BF16>(p, pl, d, causal, s);
    return dispatch<F16>(p, pl, d, causal, s);
}

extern "C" int attn_fwd_fp8(const void *q, const void *k, const void *v, const float *q_descale,
                            const float *k_descale, const float *v_descale, void *o, float *lse, int B, int H,
                            int S_q, int S_k, int d, int causal, float scale, void *stream) {
    int st = check_common(q, k, v, o, lse, B, H, S_q, S_k, d, scale);
    if (st != ATTN_OK) return st;
    if (!q_descale || !k_descale || !v_descale) return ATTN_ERR_DESCALE;
    if ((reinterpret_cast<uintptr_t>(q_descale) | reinterpret_cast<uintptr_t>(k_descale) |
         reinterpret_cast<uintptr_t>(v_descale)) & 3u)
        return ATTN_ERR_DESCALE;
    (void)causal;
    (void)stream;
    return ATTN_ERR_UNSUPPORTED;
}

extern "C" int attn_fwd_plan(int B, int H, int S_q, int S_k, int d, int causal, int dtype, int *block_q,
                             int *block_k, int *waves, int *workgroups) {
    (void)causal;
    if (B < 1 || H < 1 || S_q < 1 || S_k < 1) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
    Plan pl;
    const int st = make_plan(B, H, S_q, d, &pl);
    if (st != ATTN_OK) return st;
    if (block_q) *block_q = pl.block_q;
    if (block_k) *block_k = pl.block_k;
    if (waves) *waves = pl.waves;
    if (workgroups) *workgroups = pl.num_wg;
    return ATTN_OK;
}

extern "C" const char *attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer (q, k, v or o) is NULL";
        case ATTN_ERR_SHAPE: return "B, H, S_q and S_k must be >= 1";
        case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension (64 or 128) or dtype";
        case ATTN_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
        case ATTN_ERR_OVERFLOW: return "S*d or the workgroup count exceeds the 32-bit index range";
        case ATTN_ERR_VALUE: return "scale must be finite and > 0";
        case ATTN_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
        case ATTN_ERR_DESCALE: return "fp8 descale pointers must be non-NULL and 4-byte aligned";
        default: return "unknown status";
    }
}
