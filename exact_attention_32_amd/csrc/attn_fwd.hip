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
//     the A operand, fetched from the row-major V tile in LDS with transposing
//     reads (ds_read_b64_tr_b16);
//   * K/V tiles reach LDS by direct-to-LDS loads (global_load_lds_dwordx4) into
//     a ring of NS stages, NS-1 tiles ahead, with one explicit memory-counter
//     wait and one barrier per tile;
//   * each MFMA stream (S^T, then P.V) issues in a fixed order, one MFMA per
//     scheduling fence, with the LDS operand fetches of the next few MFMAs in
//     flight;
//   * exp2 with log2(e) folded into the scale (the page's section 4 computes the
//     exponent in base 2); lazy rescaling of O;
//   * causal: tiles wholly above the diagonal are never loaded; the mask is
//     applied only on diagonal and tail tiles; all query tiles of one head land
//     on one XCD, taken in pairs (n-1-j, j) per workgroup when there are enough
//     of them (else heaviest first);
//   * the Q operands can carry the RMSNorm of the QKNorm-across-heads step,
//     applied as they are loaded (attn_fwd_qnorm).
//
// Kernels: attn_fwd_kernel (the schedule above; the policy table's choice at both
// head dims), attn_fwd_dp_kernel (SIMD partner waves one softmax apart) and
// attn_fwd_pp_kernel (barrier-separated ping-pong), both opt-in; attn_fwd_fp8_kernel
// (block-scaled E4M3 / E5M2).  The host side at the end holds the policy table.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

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
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

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

// The two 16-bit values of type T in one dword -> floats (low half first).
template <class T> __device__ __forceinline__ void unpack2(uint32_t u, float &a, float &b);
template <> __device__ __forceinline__ void unpack2<BF16>(uint32_t u, float &a, float &b) {
    a = __uint_as_float(u << 16);
    b = __uint_as_float(u & 0xFFFF0000u);
}
template <> __device__ __forceinline__ void unpack2<F16>(uint32_t u, float &a, float &b) {
    const f16x2 h = __builtin_bit_cast(f16x2, u);
    a = (float)h[0];
    b = (float)h[1];
}

// acc + a.lo + a.hi for a dword holding two 16-bit values of type T (one v_dot2 against ones).
template <class T> __device__ __forceinline__ float sum2(uint32_t a, float acc);
template <> __device__ __forceinline__ float sum2<BF16>(uint32_t a, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), one, acc, false);
}
template <> __device__ __forceinline__ float sum2<F16>(uint32_t a, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), one, acc, false);
}

// The running max moves only when a row's max would grow by more than RESCALE_LOG2 (base 2);
// until then p = exp2(s*c - m) <= 2^RESCALE_LOG2 and the O rescale is skipped.  (The classic
// kernel bounds the row sums instead, which it forms anyway.)
constexpr float RESCALE_LOG2 = 8.0f;

// Row max between lane l and lane l^32 (the two halves of a 32x32 accumulator column).
__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroups are dispatched round-robin over the XCDs (workgroup b to XCD b % nx).  With num_wg a
// multiple of nx, work item L = (b % nx) * (num_wg / nx) + b / nx gives each XCD a contiguous range
// of items, so all query tiles of one (b, h) share one XCD's L2 (they read the same K and V).
__device__ __forceinline__ int xcd_order(int b, int num_wg, int nx) {
    return (b % nx) * (num_wg / nx) + b / nx;
}

struct Params {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int Sq, Sk;
    int nqt;         // query tiles per (b, h)
    int num_wg;      // total workgroups
    int xcd_remap;   // XCD count nx: map workgroups so each XCD gets a contiguous range of heads; 0: off
    float c;         // scale * log2(e)
    int pair;        // causal, classic schedule: a workgroup takes query tiles nqt-1-j and j (see there)
    // RMSNorm of Q folded into the Q operand loads (null qr: q is used as it is): qr [B][S_q] the
    // per-token factor, wq [H*d] the per-channel weight
    const float *qr;
    const uint16_t *wq;
    int H;
};

// One Q^T operand: the 8 values of query row `row`, channels 16 ks + 8 half .. + 7, of head bh.
// With p.qr set they are RMSNorm(q) as the QKNorm-across-heads step forms it (the sglang write-up,
// blog.secrett2633): q * r[b][row] * w_q[h*d + channel] in fp32, rounded to nearest even in T, the
// same operations in the same order as attn_qk_rmsnorm, so the operand is bit for bit the one that
// attn_qk_rmsnorm would have stored.
template <class T, int D>
__device__ __forceinline__ u32x4 load_q_frag(const Params &p, const uint16_t *Qh, int bh, int row, int ks, int half) {
    u32x4 v = *reinterpret_cast<const u32x4 *>(Qh + (size_t)row * D + ks * 16 + half * 8);
    if (p.qr) {
        const int b = bh / p.H, h = bh - b * p.H;
        const float r = p.qr[(size_t)b * p.Sq + row];
        const u32x4 w = *reinterpret_cast<const u32x4 *>(p.wq + (size_t)h * D + ks * 16 + half * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float a, c, wa, wc;
            unpack2<T>(v[e], a, c);
            unpack2<T>(w[e], wa, wc);
            v[e] = pack2<T>(a * r * wa, c * r * wc);
        }
    }
    return v;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// K and V tiles sit in LDS row-major (one key per row, 2*D bytes, no padding).  The 16-byte
// chunk c of row r is stored at chunk position c ^ swz(r): the XOR spreads the rows read by
// one MFMA operand fetch over all LDS banks, both for the K fetch (32 consecutive rows, one
// chunk each) and for the transposed V fetch (8 rows, 4 consecutive chunks each).
template <int D> __device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Wait until at most N of this wave's vector-memory loads are outstanding (they complete in
// order): s_waitcnt with the vmcnt field (bits 3:0 and 15:14) set to N and the expcnt and
// lgkmcnt fields at "no wait".
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}

// Workgroup barrier without a memory fence (a fence would drain the in-flight direct-to-LDS
// loads of later tiles).  The LDS data a wave needs is covered by its explicit memory-counter
// wait before the barrier; the empty asm statements keep the compiler from moving memory
// accesses across it.
// The lane id, formed where it is used: the compiler can neither hoist it out of a loop nor keep
// it (or an address made from it) in a register across one.
__device__ __forceinline__ int fresh_lane_id() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

__device__ __forceinline__ void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <int I, int N, class F> __device__ __forceinline__ void static_for_impl(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_impl<I + 1, N>(f);
    }
}
template <int N, class F> __device__ __forceinline__ void static_for(F &&f) { static_for_impl<0, N>(f); }

// ds_read_b64_tr_b16: inside each group of 16 lanes, lane j receives element (j % 4) of the
// 8-byte words addressed by lanes 4k + j/4, for k = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char *ptr) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(ptr));
    return __builtin_bit_cast(u32x2, v);
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// Direct-to-LDS load of 16 bytes per lane from sbase + voff (a wave-uniform 64-bit base in SGPRs
// and a 32-bit per-lane byte offset); lane l's bytes land at LDS address lds + 16 l.  Written as
// asm so that the compiler's own memory-counter bookkeeping does not see it (it would otherwise
// wait for these loads before any later LDS read it cannot tell apart); every wait for them is
// explicit.  The address registers are read when the load issues.
__device__ __forceinline__ void dma16s(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const unsigned char *p) {
    return (uint32_t)(uintptr_t)(const lds_u8 *)p;
}

// Direct-to-LDS loads of this wave's share of one K tile and one V tile: rows [k0, k0 + ROWS) of
// a head, ROWB bytes per row, into LDS at kst and vst.  Block j (1 KiB) of the wave: lane l's 16
// bytes come from byte goff[j] of a full tile: row goff[j] / ROWB, byte column goff[j] % ROWB.  In
// the S_k tail, rows past S_k are clamped onto the last key: their scores are masked to -inf and
// their P is exactly 0, so any finite value is harmless.  (The row and column are derived from
// goff where needed, so they take no registers through the key loop.)
template <int BPW, int ROWS, int ROWB>
__device__ __forceinline__ void load_kv_tile(const unsigned char *kh, const unsigned char *vh, int k0, int Sk,
                                             const uint32_t (&goff)[BPW], uint32_t kst, uint32_t vst, int wave) {
    const unsigned char *kt = kh + (size_t)k0 * ROWB, *vt = vh + (size_t)k0 * ROWB;
    if (k0 + ROWS <= Sk) {
#pragma unroll
        for (int j = 0; j < BPW; ++j) {
            const uint32_t off = (uint32_t)((wave * BPW + j) * 1024);
            dma16s(kt, goff[j], kst + off);
            dma16s(vt, goff[j], vst + off);
        }
    } else {
#pragma unroll
        for (int j = 0; j < BPW; ++j) {
            uint32_t g = goff[j];
            asm volatile("" : "+v"(g));   // derived here, not hoisted out of the key loop
            const int row = (int)(g / ROWB), colb = (int)(g % ROWB);
            const uint32_t o = (uint32_t)((min(k0 + row, Sk - 1) - k0) * ROWB + colb);
            const uint32_t off = (uint32_t)((wave * BPW + j) * 1024);
            dma16s(kt, o, kst + off);
            dma16s(vt, o, vst + off);
        }
    }
}

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
// LDS reads at a 32-bit LDS byte address; OFF is a compile-time offset that the instruction's
// immediate field absorbs
template <int OFF> __device__ __forceinline__ u32x4 lds_load_b128(uint32_t addr) {
    return *(const lds_u32x4 *)(uintptr_t)(addr + OFF);
}
template <int OFF> __device__ __forceinline__ u32x2 lds_load_tr16(uint32_t addr) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)(addr + OFF));
    return __builtin_bit_cast(u32x2, v);
}

template <class T, int D, int QB, int NW, int BC, int NS, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(Params p) {
    constexpr int BR = NW * QB * 32;     // queries per workgroup
    constexpr int ROWB = 2 * D;          // bytes per K/V row in LDS
    constexpr int TILEB = BC * ROWB;     // bytes per K (or V) tile
    constexpr int NBLK = TILEB / 1024;   // 1 KiB direct-to-LDS blocks per tile
    constexpr int BPW = NBLK / NW;       // blocks per wave
    static_assert(BC % 32 == 0 && D % 32 == 0 && NBLK % NW == 0 && BPW >= 1, "tile shape");
    // NS stages: tile t is read while tiles t+1 .. t+NS-2 are in flight
    static_assert(NS >= 2 && NS <= 4, "stages");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NS][2][TILEB];   // [stage][K, V]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;

    // Work item L: one query tile, or (causal, p.pair) the pair of tiles nqt-1-j and j of one head,
    // the heavy one first with the key tiles in order, then the light one with them in reverse
    // order.  Both passes of a pair together take the same number N of key-tile steps for every j,
    // so the workgroups of a head that start together finish together, and at step u all of them
    // read the same key tile: tile u in the first pass, tile N-1-u in the second.  Unpaired, the
    // causal tiles run heaviest first, and a tile that starts when another ends reads its keys one
    // query tile's worth of steps behind the tile that started before it on that XCD.  A key tile
    // that the first and the second pass both read is still fetched twice when the two reads lie
    // far apart (bf16 causal B=1 H=32 S=8192 d=128: FETCH_SIZE 1.25x the algorithmic bytes paired,
    // 1.43x unpaired).
    int L = blockIdx.x;
    if (p.xcd_remap) L = xcd_order(blockIdx.x, p.num_wg, p.xcd_remap);
    const int np = (CAUSAL && p.pair) ? (p.nqt + 1) >> 1 : p.nqt;
    const int bh = L / np;
    const int jq = L - bh * np;
    const int npass = (CAUSAL && p.pair && 2 * jq + 1 != p.nqt) ? 2 : 1;
    const int Sq = p.Sq, Sk = p.Sk;

    const uint16_t *__restrict__ Qh = p.q + (size_t)bh * Sq * D;
    const uint16_t *__restrict__ Kh = p.k + (size_t)bh * Sk * D;
    const uint16_t *__restrict__ Vh = p.v + (size_t)bh * Sk * D;

    // per-lane LDS offsets of the MFMA operand fetches (the swizzle only sees row bits 0..3)
    int koff[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) koff[ks] = l32 * ROWB + (((2 * ks + g) ^ swz<D>(l32)) << 4);
    int voff[2][D / 32];
    {
        const int i = lane & 15, g2 = (lane >> 4) & 1;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = h * 8 + 4 * g + (i >> 2);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const int dv = db * 32 + 16 * g2 + 4 * (i & 3);
                voff[h][db] = r * ROWB + (((dv >> 3) ^ swz<D>(r)) << 4) + ((dv >> 2) & 1) * 8;
            }
        }
    }
    // direct-to-LDS loads: block b of a tile is LDS bytes [1024 b, 1024 b + 1024); lane l fills
    // 16 bytes at 1024 b + 16 l, i.e. row `grow`, chunk position `pch`, with global chunk
    // pch ^ swz(row)
    int grow[BPW], gcolb[BPW];
    uint32_t goff[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int off = (wave * BPW + j) * 1024 + lane * 16;
        grow[j] = off / ROWB;
        gcolb[j] = ((off % ROWB) >> 4 ^ swz<D>(grow[j])) << 4;
        goff[j] = (uint32_t)(grow[j] * ROWB + gcolb[j]);
    }

    for (int pass = 0; pass < npass; ++pass) {
    const int qt = CAUSAL ? (pass == 0 ? p.nqt - 1 - jq : jq) : jq;   // causal: heaviest tiles first
    const bool rev = CAUSAL && pass == 1;                             // keys in reverse order
    const int q0 = qt * BR;
    const int qw0 = q0 + wave * QB * 32;   // first query of this wave

    u32x4 qf[QB][D / 16];   // Q^T operands, loaded after the first K/V loads are issued

    f32x16 oacc[QB][D / 32];
    float mrow[QB], lrow[QB], lrnd[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        mrow[qb] = -INFINITY;
        lrow[qb] = 0.f;
        lrnd[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[qb][db][i] = 0.f;
    }

    // tiles [0, n_full) need no mask; [n_full, n_total) hold the causal diagonal or the S_k tail
    int n_total = (Sk + BC - 1) / BC;
    int n_full = Sk / BC;
    if (CAUSAL) {
        n_total = min(n_total, (min(q0 + BR, Sq) - 1) / BC + 1);
        n_full = min(n_full, (q0 + 1) / BC);
    }
    n_full = min(n_full, n_total);
    // step u takes key tile tile_of(u) from LDS stage u % NS
    auto tile_of = [&](int u) __attribute__((always_inline)) { return rev ? n_total - 1 - u : u; };
    // the step that sets the running max: the wave's first tile with keys for it (in reverse order,
    // the last tile it sees at all; its rows each see at least the key of their own position there)
    const int u_first = rev ? n_total - 1 - min(n_total - 1, (qw0 + QB * 32 - 1) / BC) : 0;

    const uint32_t smem0 = lds_addr(&smem[0][0][0]);
    auto dma = [&](int u) __attribute__((always_inline)) {
        const uint32_t st = smem0 + (uint32_t)((u % NS) * 2 * TILEB);
        load_kv_tile<BPW, BC, ROWB>((const unsigned char *)Kh, (const unsigned char *)Vh, tile_of(u) * BC, Sk, goff,
                                    st, st + TILEB, wave);
    };

    const float c = p.c;
    auto compute = [&](int t, bool first, const unsigned char *kb, const unsigned char *vb, bool masked)
                       __attribute__((always_inline)) {
        const int k0 = t * BC;
        // S^T = K Q^T
        f32x16 s[QB][BC / 32];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[qb][kb2][i] = 0.f;
        // S^T MFMAs in a fixed order, each fenced, with the K operand fetches of the next RING
        // MFMAs in flight (measured 1.6% faster on B=2 H=16 S=4096 and 3.6% causal at d=128
        // than leaving the order to the compiler; the P.V stream below is built the same way)
        {
            constexpr int NQK = (D / 16) * (BC / 32), RING = 4;
            auto kread = [&](auto J) __attribute__((always_inline)) {
                constexpr int jj = decltype(J)::value, ks = jj / (BC / 32), kb2 = jj % (BC / 32);
                return *reinterpret_cast<const u32x4 *>(kb + kb2 * 32 * ROWB + koff[ks]);
            };
            u32x4 ring[RING];
            static_for<RING>([&](auto J) { ring[decltype(J)::value] = kread(J); });
            __builtin_amdgcn_sched_barrier(0);
            static_for<NQK>([&](auto J) {
                constexpr int jj = decltype(J)::value, ks = jj / (BC / 32), kb2 = jj % (BC / 32);
                const u32x4 a = ring[jj % RING];
                if constexpr (jj + RING < NQK) ring[jj % RING] = kread(std::integral_constant<int, jj + RING>{});
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) s[qb][kb2] = mfma_32x32x16<T>(a, qf[qb][ks], s[qb][kb2]);
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        if (masked && (k0 + BC > Sk || (CAUSAL && k0 + BC - 1 > qw0))) {
            // element i of block kb2 holds key k0 + 4g + c with c = 32 kb2 + 8 (i / 4) + i % 4 (a
            // constant); it is visible iff c < lim
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int base = k0 + 4 * g;
                int lim = Sk - base;
                if (CAUSAL) lim = min(lim, qw0 + qb * 32 + l32 + 1 - base);
#pragma unroll
                for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (kb2 * 32 + 8 * (i >> 2) + (i & 3) >= lim) s[qb][kb2][i] = -INFINITY;
            }
        }
        // online softmax (base 2); P rounded to T is the B operand of P.V.  The tile's row max is
        // taken only on the first tile, which sets the running max m.  Past it, x = s*c - m is
        // formed in place and p = exp2(x) taken at once: every p of a lane is at most the lane's
        // sum, which is formed anyway.  While each lane's sum stays within SUMMAX, m stays.  Past
        // that, the wave takes the row max from x and moves m up to it: after P.V when every sum
        // is still within PLIMIT (P as formed is representable, and O and the sums take the factor
        // after this tile's products), else before it, with P formed again.  A stale m costs no
        // precision in floating point; the bounds keep P within f16's range and O within fp32's
        // (|O| grows to at most SUMMAX * S_k / 64 times max |V| before m moves, and a deferred
        // bf16 tile adds at most 2^64 * 64 * max |V|: finite for |V| below 2^56).  The bf16 bound
        // is high because forming P again is the costly branch: on the long-context workload with
        // outliers (1% of Q and K entries x10) a bound of 2^32 sent about 3% of the wave tiles
        // there, 3% of the time.
        constexpr bool HALF = std::is_same<T, F16>::value;
        constexpr float SUMMAX = HALF ? 4096.f : 65536.f;                   // 2^12, 2^16
        constexpr float PLIMIT = HALF ? 32768.f : 18446744073709551616.f;   // 2^15, 2^64
        u32x4 pf[QB][BC / 16];
        float ps[QB], pr[QB], dl[QB];
        auto exp_pack = [&](int qb) __attribute__((always_inline)) {
            float sum = 0.f, lr = 0.f;
#pragma unroll
            for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        e[j] = __builtin_amdgcn_exp2f(s[qb][kb2][h * 8 + j]);
                        sum += e[j];
                    }
                    const u32x4 pk = u32x4{pack2<T>(e[0], e[1]), pack2<T>(e[2], e[3]), pack2<T>(e[4], e[5]),
                                           pack2<T>(e[6], e[7])};
                    pf[qb][kb2 * 2 + h] = pk;
                    lr = sum2<T>(pk[0], sum2<T>(pk[1], sum2<T>(pk[2], sum2<T>(pk[3], lr))));
                }
            ps[qb] = sum;
            pr[qb] = lr;
        };
        // new running max mnew >= m for row qb; O and the sums take alpha = exp2(m - mnew)
        auto raise_max = [&](int qb, float mnew) __attribute__((always_inline)) {
            const float alpha = __builtin_amdgcn_exp2f(mrow[qb] - (mnew == -INFINITY ? 0.f : mnew));
            mrow[qb] = mnew;
            lrow[qb] *= alpha;
            lrnd[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[qb][db][i] *= alpha;
        };
        auto row_max = [&](int qb) __attribute__((always_inline)) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qb][kb2][i]);
            return xhalf_max(mx);
        };
        if (first) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) raise_max(qb, fmaxf(mrow[qb], row_max(qb) * c));
        }
        bool over = false, big = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float mb = (mrow[qb] == -INFINITY) ? 0.f : mrow[qb];
#pragma unroll
            for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[qb][kb2][i] = __builtin_fmaf(s[qb][kb2][i], c, -mb);
            exp_pack(qb);
            over |= __builtin_amdgcn_ballot_w64(!(ps[qb] <= SUMMAX)) != 0;
            big |= __builtin_amdgcn_ballot_w64(!(ps[qb] <= PLIMIT)) != 0;
        }
        bool defer = false;
        if (over) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) dl[qb] = fmaxf(row_max(qb), 0.f);   // rows without keys: 0
            if (big) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    if (__builtin_amdgcn_ballot_w64(dl[qb] > 0.f) != 0) {
                        raise_max(qb, mrow[qb] + dl[qb]);
#pragma unroll
                        for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                            for (int i = 0; i < 16; ++i) s[qb][kb2][i] -= dl[qb];
                        exp_pack(qb);
                    }
            } else {
                defer = true;
            }
        }
        // lrow: fp32 sum of p, for the LSE.  lrnd: sum of p rounded to T (the values P.V uses),
        // for the normalisation of O: with a stale max the largest p of a row is not 1, and its
        // rounding cancels only if numerator and denominator see the same value.  Both take the
        // tile's sum, formed from zero, with one rounding per tile (chained into the running sum,
        // every dot2 would round against the row's whole sum: about 3% of O lost over 16.7 million
        // keys of a repeating pattern).
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            lrow[qb] += ps[qb];
            lrnd[qb] += pr[qb];
        }
        // O^T += V^T P^T; V^T is fetched with two transposing LDS reads per operand
        {
            constexpr int NPV = (BC / 16) * (D / 32), RING = 4;
            auto vread = [&](auto J) __attribute__((always_inline)) {
                constexpr int jj = decltype(J)::value, ks = jj / (D / 32), db = jj % (D / 32);
                const u32x2 lo = lds_read_tr16(vb + ks * 16 * ROWB + voff[0][db]);
                const u32x2 hi = lds_read_tr16(vb + ks * 16 * ROWB + voff[1][db]);
                return u32x4{lo[0], lo[1], hi[0], hi[1]};
            };
            u32x4 ring[RING];
            static_for<RING>([&](auto J) { ring[decltype(J)::value] = vread(J); });
            __builtin_amdgcn_sched_barrier(0);
            static_for<NPV>([&](auto J) {
                constexpr int jj = decltype(J)::value, ks = jj / (D / 32), db = jj % (D / 32);
                const u32x4 a = ring[jj % RING];
                if constexpr (jj + RING < NPV) ring[jj % RING] = vread(std::integral_constant<int, jj + RING>{});
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = mfma_32x32x16<T>(a, pf[qb][ks], oacc[qb][db]);
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        if (defer) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                if (__builtin_amdgcn_ballot_w64(dl[qb] > 0.f) != 0) raise_max(qb, mrow[qb] + dl[qb]);
        }
    };

    constexpr int LPT = 2 * BPW;   // direct-to-LDS loads per tile per wave

    // step u: wait until its tile is in LDS for every wave (this wave's loads of the next tiles
    // may still be in flight), which also means every wave is done with step u-1, whose stage
    // then receives the tile of step u+NS-1; compute on the tile
    auto step = [&](int u, bool masked) __attribute__((always_inline)) {
        const int ahead = min(NS - 2, n_total - 1 - u);   // tiles issued after this one
        if (NS >= 4 && ahead >= 2)
            wait_vmcnt<2 * LPT>();
        else if (NS >= 3 && ahead >= 1)
            wait_vmcnt<LPT>();
        else
            wait_vmcnt<0>();
        wg_barrier();
        if (u + NS - 1 < n_total) dma(u + NS - 1);
        // causal: a wave whose queries all precede the tile has nothing to add
        const int t = tile_of(u);
        if (!masked || !CAUSAL || t * BC <= qw0 + QB * 32 - 1)
            compute(t, u == u_first, &smem[u % NS][0][0], &smem[u % NS][1][0], masked);
    };

    // the second pass: every wave is done with the first pass's last tile before its stages refill
    if (pass) wg_barrier();
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
        if (u < n_total) dma(u);
    // Q^T operands (B of the S^T MFMA), resident for the whole key loop.  Rows past S_q are
    // clamped: they are computed and never stored.
    {
        const int lq = fresh_lane_id();
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int row = min(qw0 + qb * 32 + (lq & 31), Sq - 1);
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                qf[qb][ks] = load_q_frag<T, D>(p, Qh, bh, row, ks, lq >> 5);
        }
    }

    // the Q fragments are the newest loads; draining them here keeps the in-order memory
    // counter free of them inside the key loop
    __builtin_amdgcn_s_waitcnt(0);

    // the tiles without a mask, then those with one (the causal diagonal or the S_k tail); in
    // reverse order every step takes the masked form, which skips the mask where the tile needs none
    int u = 0;
    for (; u < (rev ? 0 : n_full); ++u) step(u, false);
    for (; u < n_total; ++u) step(u, true);

    // epilogue: O = O^T / l, LSE = ln2 * (m + log2 l)
    const int lane_e = fresh_lane_id();
    const int ge = lane_e >> 5;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = xhalf_sum(lrow[qb]);
        const float inv = 1.0f / xhalf_sum(lrnd[qb]);
        const int qrow = qw0 + qb * 32 + (lane_e & 31);
        if (qrow < Sq) {
            uint16_t *orow = p.o + ((size_t)bh * Sq + qrow) * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int gi = 0; gi < 4; ++gi) {
                    const int dv = db * 32 + 8 * gi + 4 * ge;
                    u32x2 val = u32x2{pack2<T>(oacc[qb][db][gi * 4 + 0] * inv, oacc[qb][db][gi * 4 + 1] * inv),
                                      pack2<T>(oacc[qb][db][gi * 4 + 2] * inv, oacc[qb][db][gi * 4 + 3] * inv)};
                    *reinterpret_cast<u32x2 *>(orow + dv) = val;
                }
            if (p.lse && ge == 0) p.lse[(size_t)bh * Sq + qrow] = (mrow[qb] + log2f(lt)) * 0.69314718055994530942f;
        }
    }
    }   // pass
}

// De-phased schedule for two waves per SIMD: 8 waves of 32 queries, 64-key tiles, 4 LDS stages,
// one barrier per tile.  After the barrier of tile t, waves 0-3 run S^T(t), softmax(t) and
// O^T += V^T P^T (t), while their SIMD partners, waves 4-7, run softmax(t-1), O^T += V^T P^T (t-1)
// and S^T(t): right after each barrier one wave of every SIMD starts on the matrix core and the
// other on the VALU (a wave overlaps its own MFMAs only with VALU work that does not wait on
// them, and the softmax of a tile waits on its scores).  This is the
// overlap of GEMM and softmax across warpgroups of the FlashAttention-3 deep dive
// (techknowgenie), section 3, with the wave pairs of a SIMD in the role of the warpgroups.
// Waves 4-7 keep the scores of tile t-1 across the barrier and read V(t-1) during tile t, so the
// loads run two tiles ahead (tile t+2 goes into the stage of tile t-2).
template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(512) void attn_fwd_dp_kernel(Params p) {
    constexpr int NW = 8, BC = 64, NS = 4, BR = NW * 32;
    constexpr int ROWB = 2 * D, TILEB = BC * ROWB, NBLK = TILEB / 1024, BPW = NBLK / NW;
    static_assert(NBLK % NW == 0 && BPW >= 1, "tile shape");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NS][2][TILEB];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool lag = wave >= NW / 2;
    const int g = lane >> 5, l32 = lane & 31;
    int L = blockIdx.x;
    if (p.xcd_remap) L = xcd_order(blockIdx.x, p.num_wg, p.xcd_remap);
    const int bh = L / p.nqt;
    int qt = L - bh * p.nqt;
    if (CAUSAL) qt = p.nqt - 1 - qt;
    const int q0 = qt * BR;
    const int Sq = p.Sq, Sk = p.Sk;
    const uint16_t *__restrict__ Qh = p.q + (size_t)bh * Sq * D;
    const uint16_t *__restrict__ Kh = p.k + (size_t)bh * Sk * D;
    const uint16_t *__restrict__ Vh = p.v + (size_t)bh * Sk * D;
    const int qw0 = q0 + wave * 32;

    int koff[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) koff[ks] = l32 * ROWB + (((2 * ks + g) ^ swz<D>(l32)) << 4);
    int voff[2][D / 32];
    {
        const int i = lane & 15, g2 = (lane >> 4) & 1;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = h * 8 + 4 * g + (i >> 2);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const int dv = db * 32 + 16 * g2 + 4 * (i & 3);
                voff[h][db] = r * ROWB + (((dv >> 3) ^ swz<D>(r)) << 4) + ((dv >> 2) & 1) * 8;
            }
        }
    }
    int grow[BPW], gcolb[BPW];
    uint32_t goff[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int off = (wave * BPW + j) * 1024 + lane * 16;
        grow[j] = off / ROWB;
        gcolb[j] = ((off % ROWB) >> 4 ^ swz<D>(grow[j])) << 4;
        goff[j] = (uint32_t)(grow[j] * ROWB + gcolb[j]);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float mrow = -INFINITY, lrow = 0.f, lrnd = 0.f;

    int n_total = (Sk + BC - 1) / BC;
    int n_full = Sk / BC;
    if (CAUSAL) {
        n_total = min(n_total, (min(q0 + BR, Sq) - 1) / BC + 1);
        n_full = min(n_full, (q0 + 1) / BC);
    }
    n_full = min(n_full, n_total);

    const uint32_t smem0 = lds_addr(&smem[0][0][0]);
    auto dma = [&](int t) __attribute__((always_inline)) {
        const uint32_t st = smem0 + (uint32_t)((t % NS) * 2 * TILEB);
        load_kv_tile<BPW, BC, ROWB>((const unsigned char *)Kh, (const unsigned char *)Vh, t * BC, Sk, goff, st,
                                    st + TILEB, wave);
    };

    u32x4 qf[D / 16];
    const float c = p.c;
    f32x16 s[BC / 32];

    // S^T = K Q^T of tile t (the first k-step starts from a zero accumulator)
    auto qk = [&](int t) __attribute__((always_inline)) {
        const unsigned char *kb = &smem[t % NS][0][0];
        const f32x16 zero = {};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
            for (int kb2 = 0; kb2 < BC / 32; ++kb2) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(kb + kb2 * 32 * ROWB + koff[ks]);
                s[kb2] = mfma_32x32x16<T>(a, qf[ks], ks == 0 ? zero : s[kb2]);
            }
    };
    // mask, online softmax (base 2, lazy rescale) and O^T += V^T P^T of tile t, whose scores are in s
    auto smpv = [&](int t, bool masked) __attribute__((always_inline)) {
        const int k0 = t * BC;
        if (masked) {
            const int base = k0 + 4 * g;
            int lim = Sk - base;
            if (CAUSAL) lim = min(lim, qw0 + l32 + 1 - base);
#pragma unroll
            for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (kb2 * 32 + 8 * (i >> 2) + (i & 3) >= lim) s[kb2][i] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb2][i]);
        mx = xhalf_max(mx) * c;
        if (__builtin_amdgcn_ballot_w64(mx > mrow + RESCALE_LOG2) != 0) {
            const float mnew = fmaxf(mrow, mx);
            const float alpha = __builtin_amdgcn_exp2f(mrow - (mnew == -INFINITY ? 0.f : mnew));
            mrow = mnew;
            lrow *= alpha;
            lrnd *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        }
        const float mbase = (mrow == -INFINITY) ? 0.f : mrow;
        // the tile's sums from zero, one rounding each into the running sums
        float ls = 0.f, lr = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s[kb2][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb2][i], c, -mbase));
                ls += s[kb2][i];
            }
        lrow += ls;
        u32x4 pf[BC / 16];
#pragma unroll
        for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int o = h * 8;
                const u32x4 pk = u32x4{pack2<T>(s[kb2][o + 0], s[kb2][o + 1]), pack2<T>(s[kb2][o + 2], s[kb2][o + 3]),
                                       pack2<T>(s[kb2][o + 4], s[kb2][o + 5]), pack2<T>(s[kb2][o + 6], s[kb2][o + 7])};
                pf[kb2 * 2 + h] = pk;
                lr = sum2<T>(pk[0], sum2<T>(pk[1], sum2<T>(pk[2], sum2<T>(pk[3], lr))));
            }
        lrnd += lr;
        const unsigned char *vb = &smem[t % NS][1][0];
#pragma unroll
        for (int ks = 0; ks < BC / 16; ++ks)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const u32x2 lo = lds_read_tr16(vb + ks * 16 * ROWB + voff[0][db]);
                const u32x2 hi = lds_read_tr16(vb + ks * 16 * ROWB + voff[1][db]);
                oacc[db] = mfma_32x32x16<T>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[ks], oacc[db]);
            }
    };
    // a wave whose 32 queries all precede tile t (causal) has nothing to add from it
    auto active = [&](int t) __attribute__((always_inline)) { return !CAUSAL || t * BC <= qw0 + 31; };

    constexpr int LPT = 2 * BPW;
    // barrier of tile t: tile t in LDS for every wave, every wave done with tile t-1 (group A)
    // and t-2 (group B), so stage (t+2) % NS = (t-2) % NS takes tile t+2
    auto sync = [&](int t) __attribute__((always_inline)) {
        if (t + 1 < n_total) wait_vmcnt<LPT>();
        else wait_vmcnt<0>();
        wg_barrier();
        if (t + 2 < n_total) dma(t + 2);
    };

    dma(0);
    if (n_total > 1) dma(1);
    {
        const int row = min(qw0 + l32, Sq - 1);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qf[ks] = load_q_frag<T, D>(p, Qh, bh, row, ks, g);
    }
    // the Q fragments are the newest loads; draining them here keeps the memory counter free of
    // them inside the key loop.  Both branches pass n_total barriers.
    __builtin_amdgcn_s_waitcnt(0);

    if (!lag) {
        int t = 0;
        for (; t < n_full; ++t) {
            sync(t);
            qk(t);
            smpv(t, false);
        }
        for (; t < n_total; ++t) {
            sync(t);
            if (active(t)) {
                qk(t);
                smpv(t, true);
            }
        }
    } else {
        sync(0);
        if (active(0)) qk(0);
        int t = 1;
        for (; t < n_full; ++t) {
            sync(t);
            smpv(t - 1, false);
            qk(t);
        }
        for (; t < n_total; ++t) {
            sync(t);
            if (active(t - 1)) smpv(t - 1, t - 1 >= n_full);
            if (active(t)) qk(t);
        }
        if (active(n_total - 1)) smpv(n_total - 1, n_total - 1 >= n_full);
    }

    const float lt = xhalf_sum(lrow);
    const float inv = 1.0f / xhalf_sum(lrnd);
    const int qrow = qw0 + l32;
    if (qrow < Sq) {
        uint16_t *orow = p.o + ((size_t)bh * Sq + qrow) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int dv = db * 32 + 8 * gi + 4 * g;
                *reinterpret_cast<u32x2 *>(orow + dv) =
                    u32x2{pack2<T>(oacc[db][gi * 4 + 0] * inv, oacc[db][gi * 4 + 1] * inv),
                          pack2<T>(oacc[db][gi * 4 + 2] * inv, oacc[db][gi * 4 + 3] * inv)};
            }
        if (p.lse && g == 0) p.lse[(size_t)bh * Sq + qrow] = (mrow + log2f(lt)) * 0.69314718055994530942f;
    }
}

// Ping-pong schedule for two waves per SIMD.  Eight waves per workgroup, 32 queries each; the
// waves are split into group A (waves 0-3) and group B (waves 4-7); wave w and wave w+4 share a
// SIMD.  The key loop runs in barrier-separated intervals.  In its MFMA interval a wave does
// O^T += V^T P^T for tile t-1 and S^T = K Q^T for tile t; in its VALU interval it runs the online
// softmax of tile t.  Group B runs one interval behind group A, so in every interval one wave of
// each SIMD keeps the matrix core busy while the other one does the softmax: the overlap of
// GEMM and softmax that the FlashAttention-3 deep dive (techknowgenie), sections 2 and 3,
// obtains with asynchronous warpgroups, here obtained with the barrier that the K/V pipeline
// needs anyway.
//
// LDS per stage: K (row-major, swizzled) and V (row-major, swizzled), both filled by
// direct-to-LDS loads, three stages.  While group A runs the MFMA interval of tile t, group B
// also rewrites V(t) as V^T (two V^T buffers), so that the MFMA intervals fetch every operand
// with full 16-byte reads: one wave's LDS throughput is bounded by its outstanding requests, and
// 16-byte requests carry twice the data of the transposing 8-byte reads.
template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(512) void attn_fwd_pp_kernel(Params p) {
    constexpr int NW = 8, BC = 64, NS = 3;
    constexpr int BR = NW * 32;          // queries per workgroup
    constexpr int ROWB = 2 * D;          // bytes per K/V row in LDS
    constexpr int TILEB = BC * ROWB;     // bytes per K (or V, or V^T) tile
    constexpr int VTROWB = 2 * BC;       // bytes per V^T row (one dv, BC keys)
    constexpr int NBLK = TILEB / 1024;   // 1 KiB direct-to-LDS blocks per tile
    constexpr int BPW = NBLK / NW;       // blocks per wave
    static_assert(NBLK % NW == 0 && BPW >= 1, "tile shape");
    static_assert((D / 32) * (BC / 16) % 8 == 0, "V^T chunks split over the eight waves");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NS][2][TILEB];   // [stage][K, V]
    __shared__ __attribute__((aligned(1024))) unsigned char svt[2][TILEB];        // V^T, [tile % 2]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int g = lane >> 5, l32 = lane & 31;

    int L = blockIdx.x;
    if (p.xcd_remap) L = xcd_order(blockIdx.x, p.num_wg, p.xcd_remap);
    const int bh = L / p.nqt;
    int qt = L - bh * p.nqt;
    if (CAUSAL) qt = p.nqt - 1 - qt;   // heaviest query tiles first
    const int q0 = qt * BR;
    const int Sq = p.Sq, Sk = p.Sk;
    const uint16_t *__restrict__ Qh = p.q + (size_t)bh * Sq * D;
    const uint16_t *__restrict__ Kh = p.k + (size_t)bh * Sk * D;
    const uint16_t *__restrict__ Vh = p.v + (size_t)bh * Sk * D;
    const int qw0 = q0 + wave * 32;   // first query of this wave

    int n_total = (Sk + BC - 1) / BC;
    int n_full = Sk / BC;
    if (CAUSAL) {
        n_total = min(n_total, (min(q0 + BR, Sq) - 1) / BC + 1);
        n_full = min(n_full, (q0 + 1) / BC);
    }
    n_full = min(n_full, n_total);

    // V^T row dv = 32 db + l32 holds chunk kc (8 keys of k-step kc / 2, lane half kc % 2) at chunk
    // position kc ^ ((dv >> 1) & 7): conflict-free for both the writes and the MFMA reads
    int grow[BPW], gcolb[BPW];
    uint32_t goff[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int off = (wave * BPW + j) * 1024 + lane * 16;
        grow[j] = off / ROWB;
        gcolb[j] = ((off % ROWB) >> 4 ^ swz<D>(grow[j])) << 4;
        goff[j] = (uint32_t)(grow[j] * ROWB + gcolb[j]);
    }
    const uint32_t smem0 = lds_addr(&smem[0][0][0]);
    const uint32_t svt0 = lds_addr(&svt[0][0]);

    auto dma = [&](int t) __attribute__((always_inline)) {
        const uint32_t st = smem0 + (uint32_t)((t % NS) * 2 * TILEB);
        load_kv_tile<BPW, BC, ROWB>((const unsigned char *)Kh, (const unsigned char *)Vh, t * BC, Sk, goff, st,
                                    st + TILEB, wave);
    };

    // V(t) -> V^T(t): the (dv block, k-step) chunks are split over the 8 waves; each call does
    // the share of this wave's group (half of the chunks)
    auto transpose_v = [&](int t) __attribute__((always_inline)) {
        const uint32_t vr = smem0 + (uint32_t)((t % NS) * 2 * TILEB + TILEB);
        const uint32_t vt = svt0 + (uint32_t)((t % 2) * TILEB);
        constexpr int NCH = (D / 32) * (BC / 16);   // (db, ks) pairs
        const int i = lane & 15, g2 = (lane >> 4) & 1;
#pragma unroll
        for (int cc = 0; cc < NCH / 8; ++cc) {
            const int idx = wave * (NCH / 8) + cc;  // wave-uniform
            const int db = idx / (BC / 16), ks = idx % (BC / 16);
            // transposing fetches of two 8-key halves of k-step ks, dv block db (see swz)
            const int dv = db * 32 + 16 * g2 + 4 * (i & 3);
            const int r0 = 4 * g + (i >> 2), r1 = r0 + 8;
            const uint32_t a0 = vr + (ks * 16 + r0) * ROWB + ((((dv >> 3) ^ swz<D>(r0)) << 4) | (((dv >> 2) & 1) << 3));
            const uint32_t a1 = vr + (ks * 16 + r1) * ROWB + ((((dv >> 3) ^ swz<D>(r1)) << 4) | (((dv >> 2) & 1) << 3));
            const u32x2 lo = lds_load_tr16<0>(a0);
            const u32x2 hi = lds_load_tr16<0>(a1);
            const uint32_t w = vt + (db * 32 + l32) * VTROWB + (((2 * ks + g) ^ ((l32 >> 1) & 7)) << 4);
            *(__attribute__((address_space(3))) u32x4 *)(uintptr_t)w = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    };

    // prologue: tiles 0 and 1 in flight, then Q^T operands; wait for all; V^T(0)
    dma(0);
    if (n_total > 1) dma(1);
    u32x4 qf[D / 16];
    {
        const int row = min(qw0 + l32, Sq - 1);   // rows past S_q: computed, never stored
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            qf[ks] = load_q_frag<T, D>(p, Qh, bh, row, ks, g);
    }
    __builtin_amdgcn_s_waitcnt(0);
    wg_barrier();
    transpose_v(0);
    // V^T buffer 1 stands for "tile -1" in the first MFMA interval: zeros
    static_assert(TILEB % (512 * 16) == 0, "V^T zero fill");
#pragma unroll
    for (int j = 0; j < TILEB / (512 * 16); ++j)
        *(__attribute__((address_space(3))) u32x4 *)(uintptr_t)(svt0 + TILEB + (uint32_t)((j * 512 + tid) * 16)) =
            u32x4{0u, 0u, 0u, 0u};
    __builtin_amdgcn_s_waitcnt(0);
    wg_barrier();

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float mrow = -INFINITY, lrow = 0.f, lrnd = 0.f;
    f32x16 s[BC / 32];
    u32x4 pf[BC / 16];
#pragma unroll
    for (int ks = 0; ks < BC / 16; ++ks) pf[ks] = u32x4{0u, 0u, 0u, 0u};
    const float c = p.c;

    // a wave whose queries all precede tile t (causal) has nothing to do for it
    auto active = [&](int t) __attribute__((always_inline)) { return !CAUSAL || t * BC <= qw0 + 31; };

    // The MFMA interval as one operand stream: operations [0, PV_OPS) are O^T += V^T P^T for tile
    // t-1 (k-step major, 16-byte V^T fetches), operations [PV_OPS, N_OPS) are S^T = K Q^T for tile
    // t.  READ_AHEAD fetches stay in flight ahead of the MFMA that consumes them (one wave's LDS
    // throughput is its outstanding fetches over their latency); a scheduling fence after every
    // operation keeps the compiler to exactly that order and register footprint.
    constexpr int PV_OPS = (BC / 16) * (D / 32), N_OPS = PV_OPS + (D / 16) * (BC / 32);
    constexpr int READ_AHEAD = 12;
    // per-lane parts of the fetch addresses: row base and the swizzled chunk of k-step 0; the
    // chunk of k-step ks is that chunk XOR 2 ks (k-step ks covers chunks 2 ks and 2 ks + 1)
    const uint32_t k_row = l32 * ROWB, k_chunk = (uint32_t)((g ^ swz<D>(l32)) << 4);
    const uint32_t vt_row = l32 * VTROWB, vt_chunk = (uint32_t)((g ^ ((l32 >> 1) & 7)) << 4);
    auto op_fetch = [&](auto I, uint32_t vt, uint32_t kbase, uint32_t kr, uint32_t kc, uint32_t vr,
                        uint32_t vc) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        if constexpr (i < PV_OPS) {
            constexpr int ks = i / (D / 32), db = i % (D / 32);
            return lds_load_b128<db * 32 * VTROWB>(vt + vr + (vc ^ (uint32_t)(ks << 5)));
        } else {
            constexpr int ks = (i - PV_OPS) / (BC / 32), kb2 = (i - PV_OPS) % (BC / 32);
            return lds_load_b128<kb2 * 32 * ROWB>(kbase + kr + (kc ^ (uint32_t)(ks << 5)));
        }
    };
    auto op_mfma = [&](auto I, const u32x4 &a) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        if constexpr (i < PV_OPS) {
            constexpr int ks = i / (D / 32), db = i % (D / 32);
            oacc[db] = mfma_32x32x16<T>(a, pf[ks], oacc[db]);
        } else {
            constexpr int ks = (i - PV_OPS) / (BC / 32), kb2 = (i - PV_OPS) % (BC / 32);
            s[kb2] = mfma_32x32x16<T>(a, qf[ks], s[kb2]);
        }
    };
    // Every MFMA interval runs both products, so that the register allocator sees one path: for
    // t = 0 the V^T buffer of "tile -1" holds zeros and P^T is zero; for t = n_total the scores
    // are computed from a stale stage and never used; a wave with nothing to add for tile t
    // (causal) has P^T = 0.
    auto mfma_phase = [&](int t) __attribute__((always_inline)) {
        constexpr int R = READ_AHEAD;
        const uint32_t vt = svt0 + (uint32_t)(((t + 1) % 2) * TILEB);   // V^T of tile t-1
        const uint32_t kbase = smem0 + (uint32_t)((t % NS) * 2 * TILEB);
#pragma unroll
        for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb2][i] = 0.f;
        // the lane parts pass through an empty asm so that the compiler derives every address
        // here instead of keeping all of them live across the loop
        uint32_t kr = k_row, kc = k_chunk, vr = vt_row, vc = vt_chunk;
        asm volatile("" : "+v"(kr), "+v"(kc), "+v"(vr), "+v"(vc));
        u32x4 ring[R];
        static_for<R>([&](auto J) {
            ring[decltype(J)::value] = op_fetch(J, vt, kbase, kr, kc, vr, vc);
        });
        __builtin_amdgcn_sched_barrier(0);
        static_for<N_OPS>([&](auto J) {
            constexpr int j = decltype(J)::value;
            const u32x4 a = ring[j % R];
            if constexpr (j + R < N_OPS)
                ring[j % R] = op_fetch(std::integral_constant<int, j + R>{}, vt, kbase, kr, kc, vr, vc);
            op_mfma(J, a);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    auto valu_phase = [&](int t) __attribute__((always_inline)) {
        if (t >= n_total) return;
        if (!active(t)) {
#pragma unroll
            for (int ks = 0; ks < BC / 16; ++ks) pf[ks] = u32x4{0u, 0u, 0u, 0u};
            return;
        }
        if (t >= n_full) {
            // element i of block kb2 holds key k0 + 4g + c with c = 32 kb2 + 8 (i / 4) + i % 4 (a
            // constant); it is visible iff c < lim
            const int base = t * BC + 4 * g;
            int lim = Sk - base;
            if (CAUSAL) lim = min(lim, qw0 + l32 + 1 - base);
#pragma unroll
            for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (kb2 * 32 + 8 * (i >> 2) + (i & 3) >= lim) s[kb2][i] = -INFINITY;
        }
        // row max as a tree of independent v_max3 chains
        float mq[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int kb2 = (k * 8) / 16 % (BC / 32), o = (k * 8) % 16;
            float m0 = fmaxf(s[kb2][o], s[kb2][o + 1]);
#pragma unroll
            for (int i = 2; i < 8; ++i) m0 = fmaxf(m0, s[kb2][o + i]);
            mq[k] = m0;
        }
        float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
#pragma unroll
        for (int kb2 = 2; kb2 < BC / 32; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb2][i]);
        mx = xhalf_max(mx) * c;
        if (__builtin_amdgcn_ballot_w64(mx > mrow + RESCALE_LOG2) != 0) {
            const float mnew = fmaxf(mrow, mx);
            const float alpha = __builtin_amdgcn_exp2f(mrow - (mnew == -INFINITY ? 0.f : mnew));
            mrow = mnew;
            lrow *= alpha;
            lrnd *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        }
        const float mbase = (mrow == -INFINITY) ? 0.f : mrow;
        // exponentials, the fp32 row sum as four independent partial sums
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s[kb2][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb2][i], c, -mbase));
                ls[i & 3] += s[kb2][i];
            }
        float lr[2] = {0.f, 0.f};
#pragma unroll
        for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int o = h * 8;
                const u32x4 pk = u32x4{pack2<T>(s[kb2][o + 0], s[kb2][o + 1]), pack2<T>(s[kb2][o + 2], s[kb2][o + 3]),
                                       pack2<T>(s[kb2][o + 4], s[kb2][o + 5]), pack2<T>(s[kb2][o + 6], s[kb2][o + 7])};
                pf[kb2 * 2 + h] = pk;
                lr[h] = sum2<T>(pk[0], sum2<T>(pk[1], sum2<T>(pk[2], sum2<T>(pk[3], lr[h]))));
            }
        lrow += (ls[0] + ls[1]) + (ls[2] + ls[3]);
        lrnd += lr[0] + lr[1];
    };

    // Global interval 2t: A does the MFMA work of tile t, B the softmax of tile t-1 and the V^T of
    // tile t; interval 2t+1: A the softmax of tile t, B the MFMA work of tile t.  Tile t+1 is
    // loaded from the start of interval 2t and waited for at the end of interval 2t+1, so it is
    // in LDS when interval 2t+2 needs its K (QK) and its V (the V^T rewrite).  Both groups pass
    // the same number of barriers (2 n_total + 3).
    // (tiles 0 and 1 come from the prologue, so the loads start with tile 2 in interval 2.)
    if (grp == 0) {
        for (int t = 0; t <= n_total; ++t) {
            if (t >= 1 && t + 1 < n_total) dma(t + 1);
            mfma_phase(t);
            wg_barrier();
            if (t >= 1 && t < n_total) transpose_v(t);
            valu_phase(t);
            __builtin_amdgcn_s_waitcnt(0);
            wg_barrier();
        }
        wg_barrier();
    } else {
        wg_barrier();
        for (int t = 0; t <= n_total; ++t) {
            mfma_phase(t);
            __builtin_amdgcn_s_waitcnt(0);
            wg_barrier();
            if (t + 2 < n_total) dma(t + 2);
            if (t + 1 < n_total) transpose_v(t + 1);
            valu_phase(t);
            wg_barrier();
        }
    }

    // epilogue: O = O^T / l, LSE = ln2 * (m + log2 l)
    const float lt = xhalf_sum(lrow);
    const float inv = 1.0f / xhalf_sum(lrnd);
    const int qrow = qw0 + l32;
    if (qrow < Sq) {
        uint16_t *orow = p.o + ((size_t)bh * Sq + qrow) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int dv = db * 32 + 8 * gi + 4 * g;
                *reinterpret_cast<u32x2 *>(orow + dv) =
                    u32x2{pack2<T>(oacc[db][gi * 4 + 0] * inv, oacc[db][gi * 4 + 1] * inv),
                          pack2<T>(oacc[db][gi * 4 + 2] * inv, oacc[db][gi * 4 + 3] * inv)};
            }
        if (p.lse && g == 0) p.lse[(size_t)bh * Sq + qrow] = (mrow + log2f(lt)) * 0.69314718055994530942f;
    }
}

// ---------------------------------------------------------------------------
// Block-scaled fp8 path (the FlashAttention-3 deep dive (techknowgenie), section 4: per-block
// scale factors, both products in FP8, softmax and accumulation in FP32).
//
// Q, K, V hold OCP fp8 codes, all three E4M3 or all three E5M2 (the template argument FMT; the
// deep dive's section 4 names both formats); the value of row r of a head is
// code * descale[r / 128].  One key tile is one descale block (128 keys).  With raw = Q_code . K_code
// (exact in the fp32 MFMA accumulator), the base-2 score is x = raw * c_t with
// c_t = scale * log2(e) * qd * kd_t.
//
// P' for the P.V product is rounded to E4M3 (for either input format: the matrix core takes a
// format per operand, and E4M3 keeps one more mantissa bit of the probabilities than E5M2).  Its
// range is kept away from both ends of E4M3:
//   * headroom: the running offset m is set to the row max of the exponents (below) minus 5, so
//     the largest P' of the tile that sets it is exactly 2^5 = 32 (its weight carries no rounding
//     error, which matters for rows with few keys), keys 11 binades below it are still normal and
//     14 binades below still representable (E4M3's smallest normal is 2^-6, its smallest subnormal
//     2^-9).  m moves only when a later tile's P' leaves E4M3's range: a value above 464 converts
//     to NaN, which the matrix core's row sum of P' (formed anyway) carries, and only then is the
//     tile redone with its max put back at 2^5.  The slack of 2^3.86 (less up to one binade of the
//     V mantissa below) is passed by about 3% of wave-tiles on N(0,1) scores; with 2^8 instead,
//     the first tile's max (about 1.5 binades below a row's final max) left too little slack and
//     half of all wave-tiles had to be redone.
//   * V's descale never shifts P': vd_t = f_t * 2^e_t with f_t in [0.5, 1).  2^e_t is the E8M0
//     block scale of the V^T operand of the scaled MFMA (the matrix core applies it exactly), and
//     only log2(f_t), in [-1, 0), enters the exponent of P'.  So P' = exp2(x + log2 f_t - m), the
//     weights P.V applies are round(P') / f_t, and the row sums add (sum P') / f_t per tile.
//     (A descale below 2^-126 is taken as 2^-126 with f_t = 1: such a block's V values are below
//     448 * 2^-126 in magnitude, so the difference is below 6e-36.)

// MFMA: v_mfma_scale_f32_32x32x64_f8f6f4 (operand format 0 = E4M3, 1 = E5M2; block scales 2^0
// except on the V^T operand, which carries the power of two of V's descale).  It sums
// A[i][k] B[k][j] over
// the pairs (lane half, byte) that A and B share, so any key order that both operands use is
// valid.  The order used here is the one of the S^T accumulator: byte b of lane half g of
// k-step kk is key 64 kk + 32 (b / 16) + 8 ((b % 16) / 4) + 4 g + b % 4, so P^T is packed
// from the accumulator in place, and V^T is fetched with ds_read_b64_tr_b8 (inside each group
// of 16 lanes, lane j receives byte j % 8 of the 8-byte words addressed by lanes 2 k + j / 8,
// for k = 0..7).

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

struct ParamsF8 {
    const uint8_t *q, *k, *v;
    const float *qd, *kd, *vd;   // descales [b*h][block]; NULL: all ones
    uint16_t *o;                 // bf16
    float *lse;
    int Sq, Sk;
    int nqb, nkb;                // 128-row blocks of Q and of K/V per head
    int nqt, num_wg, xcd_remap;
    float c;                     // scale * log2(e)
};

// operand formats FA (of A) and FB (of B): 0 = E4M3, 1 = E5M2; block scale exponents 127 (2^0)
template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma_f8(const i32x8 &a, const i32x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 127, 0, 127);
}
// the same with A scaled by 2^(sa - 127) (sa: an E8M0 exponent byte, 0..254, uniform over the wave)
template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma_f8_sa(const i32x8 &a, const i32x8 &b, const f32x16 &c, int sa) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, sa, 0, 127);
}

// P' headroom: the tile that sets the running offset m puts its largest P' at 2^P8_HEAD (E4M3's
// largest finite value is 448 = 2^8.81, its smallest subnormal 2^-9)
constexpr float P8_HEAD = 5.0f;
// the descale of a tensor passed without descales: its loads read this instead, so that the key
// loop takes no branch on whether descales were given
__constant__ float kUnitDescale = 1.0f;

// four floats -> four E4M3 bytes (round to nearest even), first value in the low byte.  The
// first conversion's "old" operand only supplies bytes 2-3, which the second one overwrites, so
// any register does (a's bits: no zero has to be materialised).
__device__ __forceinline__ int pack4_e4m3(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// fp8 tiles sit in LDS row-major (D bytes per key).  The 16-byte chunk c of row r is stored at
// position c ^ swz8(r).  Every K operand fetch (32 rows x one chunk, two lane halves) and every
// transposing V fetch (16 rows x 32 bytes) then spreads evenly over the LDS banks.
template <int D> __device__ __forceinline__ int swz8(int row) {
    if constexpr (D == 128) return (row >> 1) & 7;
    else return (row >> 2) & 3;
}

template <int OFF> __device__ __forceinline__ u32x2 lds_load_tr8(uint32_t addr) {
    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(uintptr_t)(addr + OFF));
    return __builtin_bit_cast(u32x2, v);
}

template <int D, int NS, bool CAUSAL, int FMT>
__global__ __launch_bounds__(512) void attn_fwd_fp8_kernel(ParamsF8 p) {
    constexpr int NW = 8, BC = 128, BR = NW * 32;
    constexpr int ROWB = D;              // bytes per K/V row
    constexpr int TILEB = BC * ROWB;     // bytes per K (or V) tile
    constexpr int NBLK = TILEB / 1024;   // 1 KiB direct-to-LDS blocks per tile
    constexpr int BPW = NBLK / NW;
    constexpr int KSTEPS = D / 64;       // k-steps of S^T = K Q^T
    static_assert(NBLK % NW == 0 && BPW >= 1, "tile shape");
    static_assert(NS >= 2 && NS <= 4, "stages");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NS][2][TILEB];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;

    int L = blockIdx.x;
    if (p.xcd_remap) L = xcd_order(blockIdx.x, p.num_wg, p.xcd_remap);
    const int bh = L / p.nqt;
    int qt = L - bh * p.nqt;
    if (CAUSAL) qt = p.nqt - 1 - qt;
    const int q0 = qt * BR;
    const int Sq = p.Sq, Sk = p.Sk;
    const uint8_t *__restrict__ Qh = p.q + (size_t)bh * Sq * D;
    const uint8_t *__restrict__ Kh = p.k + (size_t)bh * Sk * D;
    const uint8_t *__restrict__ Vh = p.v + (size_t)bh * Sk * D;
    const int qw0 = q0 + wave * 32;
    const float qd = p.qd ? p.qd[(size_t)bh * p.nqb + min(qw0, Sq - 1) / 128] : 1.f;
    const float cq = p.c * qd;

    // K operand: row l32 of a 32-key block, chunks 4 ks + 2 g and 4 ks + 2 g + 1
    int koff[2 * KSTEPS];
#pragma unroll
    for (int j = 0; j < 2 * KSTEPS; ++j)
        koff[j] = l32 * ROWB + (((4 * (j >> 1) + 2 * g + (j & 1)) ^ swz8<D>(l32)) << 4);
    // V^T operand of dv block db: lane m of its 16-lane group fetches 8 bytes of row
    // 8 (m / 8) + 4 g + (m / 2) % 4 (+ 16 r' per fetch), columns 32 db + 16 ((lane / 16) % 2) + 8 (m % 2)
    int vlane[D / 32];
    {
        const int m = lane & 15, h1 = (lane >> 4) & 1;
        const int r0 = 8 * (m >> 3) + 4 * g + ((m >> 1) & 3);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            vlane[db] = r0 * ROWB + (((2 * db + h1) ^ swz8<D>(r0)) << 4) + 8 * (m & 1);
    }
    int grow[BPW], gcolb[BPW];
    uint32_t goff[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int off = (wave * BPW + j) * 1024 + lane * 16;
        grow[j] = off / ROWB;
        gcolb[j] = (((off % ROWB) >> 4) ^ swz8<D>(grow[j])) << 4;
        goff[j] = (uint32_t)(grow[j] * ROWB + gcolb[j]);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    float mrow = -INFINITY, lrow = 0.f, lrnd = 0.f;

    int n_total = (Sk + BC - 1) / BC;
    int n_full = Sk / BC;
    if (CAUSAL) {
        n_total = min(n_total, (min(q0 + BR, Sq) - 1) / BC + 1);
        n_full = min(n_full, (q0 + 1) / BC);
    }
    n_full = min(n_full, n_total);

    const uint32_t smem0 = lds_addr(&smem[0][0][0]);
    auto stage = [&](int t) __attribute__((always_inline)) { return smem0 + (uint32_t)((t % NS) * 2 * TILEB); };
    auto dma = [&](int t) __attribute__((always_inline)) {
        const uint32_t st = stage(t);
        load_kv_tile<BPW, BC, ROWB>(Kh, Vh, t * BC, Sk, goff, st, st + TILEB, wave);
    };

    i32x8 qf[KSTEPS];
    const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                        0x38383838, 0x38383838, 0x38383838, 0x38383838};   // E4M3 1.0

    // descales through the constant address space: wave-uniform scalar loads, which the
    // vector-memory counter that paces the K/V pipeline does not see.  Tile t+1's are loaded at the
    // end of tile t: a scalar load still in flight when the next K operand fetches are waited for
    // would make that wait cover every LDS read too (scalar loads return out of order).
    typedef const __attribute__((address_space(4))) float cfloat;
    auto load_descales = [&](int t, float &kd, float &vd) __attribute__((always_inline)) {
        const int tt = min(t, p.nkb - 1);
        const size_t i = (size_t)bh * p.nkb + tt;
        cfloat *kp = p.kd ? (cfloat *)p.kd + i : (cfloat *)&kUnitDescale;
        cfloat *vp = p.vd ? (cfloat *)p.vd + i : (cfloat *)&kUnitDescale;
        kd = *kp;
        vd = *vp;
    };
    float kd_cur, vd_cur;

    // The key loop is software-pipelined by one tile: iteration t forms S^T(t) and P'(t), and
    // multiplies P'(t-1) into O.  The P'(t-1) products do not depend on tile t's softmax, so the
    // matrix core runs them while the VALU forms P'(t); and the range check of P'(t-1) (below)
    // reads a row sum that finished during the previous iteration.  The V tile of t-1 is still read
    // in iteration t, so tiles are loaded two iterations ahead into four LDS stages.
    static_assert(NS == 4, "the pipelined key loop needs four stages");

    // per-tile scale terms: ct multiplies the raw code products; vsc / vf split V's descale
    struct TileScale {
        float ct, lvf, ivf;
        int vsc;
    };
    auto decode = [&](float kdt, float vdt) __attribute__((always_inline)) {
        // vd_t = vf * 2^(vsc - 127) with vf in [0.5, 1) (see the header above)
        const uint32_t vbits = __float_as_uint(vdt);
        const int vexp = (int)((vbits >> 23) & 0xff);
        TileScale ts;
        ts.vsc = vexp == 0 ? 1 : min(vexp + 1, 254);
        const float vf = __uint_as_float(
            vexp == 0 ? 0x3f800000u : ((vbits & 0x807fffffu) | (vexp >= 254 ? (127u << 23) : (126u << 23))));
        ts.ct = cq * kdt;
        ts.lvf = __builtin_amdgcn_logf(vf);   // log2(vf), in [-1, 0]
        ts.ivf = __builtin_amdgcn_rcpf(vf);
        return ts;
    };

    // S^T = K Q^T (codes) of the tile at LDS address kt, masked on diagonal and tail tiles
    auto qk = [&](f32x16 (&s)[BC / 32], uint32_t kt, int t, bool masked) __attribute__((always_inline)) {
        // one address per lane offset (stage base + lane offset), passed through an empty asm so
        // that each fetch is that address + an immediate
        uint32_t ka[2 * KSTEPS];
#pragma unroll
        for (int j = 0; j < 2 * KSTEPS; ++j) {
            ka[j] = kt + (uint32_t)koff[j];
            asm volatile("" : "+v"(ka[j]));
        }
#pragma unroll
        for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb2][i] = 0.f;
        // S^T MFMAs in a fixed order, each fenced, with the K fetches of the next two in flight
        constexpr int NQK = KSTEPS * (BC / 32), RING = 2;
        auto kread = [&](auto J) __attribute__((always_inline)) {
            constexpr int jj = decltype(J)::value, ks = jj / (BC / 32), kb2 = jj % (BC / 32);
            const u32x4 lo = lds_load_b128<kb2 * 32 * ROWB>(ka[2 * ks]);
            const u32x4 hi = lds_load_b128<kb2 * 32 * ROWB>(ka[2 * ks + 1]);
            return __builtin_bit_cast(i32x8, (u32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        };
        i32x8 ring[RING];
        static_for<RING>([&](auto J) { ring[decltype(J)::value] = kread(J); });
        __builtin_amdgcn_sched_barrier(0);
        static_for<NQK>([&](auto J) {
            constexpr int jj = decltype(J)::value, ks = jj / (BC / 32), kb2 = jj % (BC / 32);
            const i32x8 a = ring[jj % RING];
            if constexpr (jj + RING < NQK) ring[jj % RING] = kread(std::integral_constant<int, jj + RING>{});
            s[kb2] = mfma_f8<FMT, FMT>(a, qf[ks], s[kb2]);
            __builtin_amdgcn_sched_barrier(0);
        });
        if (masked) {
            const int base = t * BC + 4 * g;
            int lim = Sk - base;
            if (CAUSAL) lim = min(lim, qw0 + l32 + 1 - base);
#pragma unroll
            for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (kb2 * 32 + 8 * (i >> 2) + (i & 3) >= lim) s[kb2][i] = -INFINITY;
        }
    };
    auto raise_max = [&](float mnew) __attribute__((always_inline)) {
        const float alpha = __builtin_amdgcn_exp2f(mrow - (mnew == -INFINITY ? 0.f : mnew));
        mrow = mnew;
        lrow *= alpha;
        lrnd *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    };
    // four independent chains from -inf (a max3 chain with no canonicalising first step)
    auto lane_max = [&](const f32x16 (&s)[BC / 32]) __attribute__((always_inline)) {
        float mq[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float m0 = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) m0 = fmaxf(m0, s[k][i]);
            mq[k] = m0;
        }
        return fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
    };
    // x = raw * ct + log2(vf) - m in place
    auto to_exponents = [&](f32x16 (&s)[BC / 32], const TileScale &ts) __attribute__((always_inline)) {
        const float off = ts.lvf - ((mrow == -INFINITY) ? 0.f : mrow);
#pragma unroll
        for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb2][i] = __builtin_fmaf(s[kb2][i], ts.ct, off);
    };
    // P'^T in E4M3 from x: dword w of k-step kk = keys of s[2 kk + w / 4][4 (w % 4) .. + 3]; returns
    // this lane's fp32 sum of p'
    auto exp_pack = [&](const f32x16 (&s)[BC / 32], i32x8 (&pf)[BC / 64]) __attribute__((always_inline)) {
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < BC / 64; ++kk)
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const f32x16 &sv = s[2 * kk + (w >> 2)];
                const int o = 4 * (w & 3);
                float e[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    e[j] = __builtin_amdgcn_exp2f(sv[o + j]);
                    ls[j] += e[j];
                }
                pf[kk][w] = pack4_e4m3(e[0], e[1], e[2], e[3]);
            }
        return (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };
    // sum of the rounded p' (the weights P.V uses) of each query: ones x P'^T on the matrix core
    auto row_sum = [&](const i32x8 (&pf)[BC / 64]) __attribute__((always_inline)) {
        f32x16 r = {};
#pragma unroll
        for (int kk = 0; kk < BC / 64; ++kk) r = mfma_f8<0, 0>(ones, pf[kk], r);
        return r[0];   // every row of ones x P'^T holds the same sums
    };
    // O^T += V^T P'^T for the V tile at LDS address vt: op (kk, db) needs four transposing fetches,
    // issued PV_AHEAD ops ahead of their MFMA
    auto pv = [&](const i32x8 (&pf)[BC / 64], uint32_t vt, int vsc) __attribute__((always_inline)) {
        uint32_t va[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            va[db] = vt + (uint32_t)vlane[db];
            asm volatile("" : "+v"(va[db]));
        }
        constexpr int NPV = (BC / 64) * (D / 32), PV_AHEAD = 2;
        auto pv_fetch = [&](auto I) __attribute__((always_inline)) {
            constexpr int i = decltype(I)::value, kk = i / (D / 32), db = i % (D / 32);
            const u32x2 r0 = lds_load_tr8<(64 * kk + 0) * ROWB>(va[db]);
            const u32x2 r1 = lds_load_tr8<(64 * kk + 16) * ROWB>(va[db]);
            const u32x2 r2 = lds_load_tr8<(64 * kk + 32) * ROWB>(va[db]);
            const u32x2 r3 = lds_load_tr8<(64 * kk + 48) * ROWB>(va[db]);
            return __builtin_bit_cast(i32x8, (u32x8){r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]});
        };
        i32x8 ring[PV_AHEAD];
        static_for<PV_AHEAD>([&](auto J) { ring[decltype(J)::value] = pv_fetch(J); });
        static_for<NPV>([&](auto J) {
            constexpr int j = decltype(J)::value, kk = j / (D / 32), db = j % (D / 32);
            const i32x8 a = ring[j % PV_AHEAD];
            if constexpr (j + PV_AHEAD < NPV) ring[j % PV_AHEAD] = pv_fetch(std::integral_constant<int, j + PV_AHEAD>{});
            oacc[db] = mfma_f8_sa<FMT, 0>(a, pf[kk], oacc[db], vsc);
        });
    };

    // the tile waiting for its P.V product: its P'^T, sums and scale terms
    i32x8 pprev[BC / 64];
    float ls_prev = 0.f, rs_prev = 0.f;
    TileScale ts_prev = {0.f, 0.f, 1.f, 127};
    int t_prev = -1;

    // Check the waiting tile: a NaN row sum means some P' passed E4M3's range (values above 464
    // convert to NaN); then the tile's scores are formed again from its K tile (still in LDS), m
    // moves up so that the tile's row max is at P8_HEAD, and P' is formed again.  O has not yet
    // received this tile's products, so rescaling it and the sums is all the correction needs.
    auto check_prev = [&]() __attribute__((always_inline)) {
        if (__builtin_amdgcn_ballot_w64(rs_prev != rs_prev) != 0) {
            f32x16 s[BC / 32];
            qk(s, stage(t_prev), t_prev, true);   // the mask changes nothing on a full tile
            to_exponents(s, ts_prev);
            const float d = fmaxf(xhalf_max(lane_max(s)) - P8_HEAD, 0.f);
            raise_max(mrow + d);
#pragma unroll
            for (int kb2 = 0; kb2 < BC / 32; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb2][i] -= d;
            ls_prev = exp_pack(s, pprev);
            rs_prev = row_sum(pprev);
        }
        lrow += ls_prev * ts_prev.ivf;
        lrnd += rs_prev * ts_prev.ivf;
    };
    auto pv_prev = [&]() __attribute__((always_inline)) {
        pv(pprev, stage(t_prev) + TILEB, ts_prev.vsc);
        t_prev = -1;
    };

    // Tile t: the waiting tile's check, S^T(t), then P'(t-1) into O (the matrix core) while P'(t)
    // is formed (the VALU).  The first tile of a row sets m from its row max.  A causal wave whose
    // queries all precede the tile only finishes the waiting tile.
    auto tile = [&](int t, bool masked, bool work) __attribute__((always_inline)) {
        const bool waiting = t_prev >= 0;
        if (waiting) check_prev();
        const TileScale ts = decode(kd_cur, vd_cur);
        f32x16 s[BC / 32];
        if (work) {
            qk(s, stage(t), t, masked);
            if (t == 0) raise_max(__builtin_fmaf(xhalf_max(lane_max(s)), ts.ct, ts.lvf) - P8_HEAD);
        }
        if (waiting) pv_prev();
        if (work) {
            to_exponents(s, ts);
            ls_prev = exp_pack(s, pprev);
            rs_prev = row_sum(pprev);
            ts_prev = ts;
            t_prev = t;
        }
    };

    // P'(t-1) into O on the matrix core, interleaved in program order with the forming of P'(t)
    // from the scores s of tile t (the VALU): P.V op j is issued after the j-th share of the
    // exponentials, while the next share runs, and a scheduling fence after each keeps the pairs in
    // that order.  Returns this lane's fp32 sum of p'(t); P'(t) goes to pnew.
    auto pv_softmax = [&](const i32x8 (&pold)[BC / 64], uint32_t vt, int vsc, const f32x16 (&s)[BC / 32],
                          const TileScale &ts, i32x8 (&pnew)[BC / 64]) __attribute__((always_inline)) {
        uint32_t va[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            va[db] = vt + (uint32_t)vlane[db];
            asm volatile("" : "+v"(va[db]));
        }
        constexpr int NPV = (BC / 64) * (D / 32), PV_AHEAD = 2;
        constexpr int NGRP = (BC / 64) * 8, GPER = NGRP / NPV;   // groups of 4 scores per P.V op
        static_assert(NGRP % NPV == 0, "shares");
        auto pv_fetch = [&](auto I) __attribute__((always_inline)) {
            constexpr int i = decltype(I)::value, kk = i / (D / 32), db = i % (D / 32);
            const u32x2 r0 = lds_load_tr8<(64 * kk + 0) * ROWB>(va[db]);
            const u32x2 r1 = lds_load_tr8<(64 * kk + 16) * ROWB>(va[db]);
            const u32x2 r2 = lds_load_tr8<(64 * kk + 32) * ROWB>(va[db]);
            const u32x2 r3 = lds_load_tr8<(64 * kk + 48) * ROWB>(va[db]);
            return __builtin_bit_cast(i32x8, (u32x8){r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]});
        };
        const float off = ts.lvf - ((mrow == -INFINITY) ? 0.f : mrow);
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
        i32x8 ring[PV_AHEAD];
        static_for<PV_AHEAD>([&](auto J) { ring[decltype(J)::value] = pv_fetch(J); });
        __builtin_amdgcn_sched_barrier(0);
        static_for<NPV>([&](auto J) {
            constexpr int j = decltype(J)::value, kk = j / (D / 32), db = j % (D / 32);
#pragma unroll
            for (int gi = 0; gi < GPER; ++gi) {
                const int grp = j * GPER + gi, k2 = grp >> 3, w = grp & 7;
                const f32x16 &sv = s[2 * k2 + (w >> 2)];
                const int o = 4 * (w & 3);
                float e[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    e[q] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[o + q], ts.ct, off));
                    ls[q] += e[q];
                }
                pnew[k2][w] = pack4_e4m3(e[0], e[1], e[2], e[3]);
            }
            const i32x8 a = ring[j % PV_AHEAD];
            if constexpr (j + PV_AHEAD < NPV) ring[j % PV_AHEAD] = pv_fetch(std::integral_constant<int, j + PV_AHEAD>{});
            oacc[db] = mfma_f8_sa<FMT, 0>(a, pold[kk], oacc[db], vsc);
            __builtin_amdgcn_sched_barrier(0);
        });
        return (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };

    // A full tile past the first, with a tile waiting: the same steps with nothing left to decide
    // at run time after the waiting tile's check, so that S^T(t), P'(t-1) into O and the forming of
    // P'(t) fall in one basic block, with the P.V products interleaved into the softmax.
    auto tile_steady = [&](int t) __attribute__((always_inline)) {
        check_prev();
        const TileScale ts = decode(kd_cur, vd_cur);
        f32x16 s[BC / 32];
        qk(s, stage(t), t, false);
        i32x8 pnew[BC / 64];
        ls_prev = pv_softmax(pprev, stage(t_prev) + TILEB, ts_prev.vsc, s, ts, pnew);
        rs_prev = row_sum(pnew);
#pragma unroll
        for (int kk = 0; kk < BC / 64; ++kk) pprev[kk] = pnew[kk];
        ts_prev = ts;
        t_prev = t;
    };

    // one iteration: wait until tile t has landed for every wave (this wave's loads of tile t+1 may
    // still be in flight), which also means every wave is done with iteration t-1 and so with tile
    // t-2, whose stage then receives tile t+2
    auto step_begin = [&](int t) __attribute__((always_inline)) {
        constexpr int LPT = 2 * BPW;   // direct-to-LDS loads per tile per wave
        if (t + 1 < n_total)
            wait_vmcnt<LPT>();
        else
            wait_vmcnt<0>();
        wg_barrier();
        if (t + 2 < n_total) dma(t + 2);
    };

    dma(0);
    if (n_total > 1) dma(1);
    {
        const int row = min(qw0 + l32, Sq - 1);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(Qh + (size_t)row * D + 64 * ks + 32 * g);
            const u32x4 lo = src[0], hi = src[1];
            qf[ks] = __builtin_bit_cast(i32x8, (u32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        }
    }
    load_descales(0, kd_cur, vd_cur);
    __builtin_amdgcn_s_waitcnt(0);

    int t = 0;
    if (n_full > 0) {
        step_begin(0);
        tile(0, false, true);
        load_descales(1, kd_cur, vd_cur);
        t = 1;
    }
    for (; t < n_full; ++t) {
        step_begin(t);
        tile_steady(t);
        load_descales(t + 1, kd_cur, vd_cur);
    }
    // diagonal and tail tiles: a causal wave whose queries all precede the tile has nothing to add
    for (; t < n_total; ++t) {
        step_begin(t);
        tile(t, true, !CAUSAL || t * BC <= qw0 + 31);
        load_descales(t + 1, kd_cur, vd_cur);
    }
    // the last tile's K and V stay in their stage: no load follows them
    if (t_prev >= 0) {
        check_prev();
        pv_prev();
    }

    // lrow holds this lane half's keys; lrnd already sums both halves (the MFMA reduces over k)
    const float lt = xhalf_sum(lrow);
    const float inv = 1.0f / lrnd;
    const int qrow = qw0 + l32;
    if (qrow < Sq) {
        uint16_t *orow = p.o + ((size_t)bh * Sq + qrow) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int dv = db * 32 + 8 * gi + 4 * g;
                *reinterpret_cast<u32x2 *>(orow + dv) =
                    u32x2{pack2<BF16>(oacc[db][gi * 4 + 0] * inv, oacc[db][gi * 4 + 1] * inv),
                          pack2<BF16>(oacc[db][gi * 4 + 2] * inv, oacc[db][gi * 4 + 3] * inv)};
            }
        if (p.lse && g == 0) p.lse[(size_t)bh * Sq + qrow] = (mrow + log2f(lt)) * 0.69314718055994530942f;
    }
}

// ---------------------------------------------------------------------------
// host side

struct Plan {
    int sched;                   // ATTN_SCHED_CLASSIC, _PINGPONG or _DEPHASED (f16/bf16); 0 for fp8
    int qb, nw, ns, bk;          // 32-query blocks per wave, waves, LDS stages, keys per tile
    int block_q, block_k, nqt, num_wg;
    int pair;                    // causal classic schedule: one workgroup per pair of query tiles
};

// Internal status of check_common: no query rows (B, H or S_q = 0), so nothing to compute.
constexpr int kEmpty = -1;

int check_common(const void *q, const void *k, const void *v, const void *o, const void *lse, int B, int H, int Sq,
                 int Sk, int d, float scale) {
    if (B < 0 || H < 0 || Sq < 0 || Sk < 0) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_VALUE;
    if (B == 0 || H == 0 || Sq == 0) return kEmpty;
    if (Sk == 0) return ATTN_ERR_SHAPE;   // a softmax over no keys is undefined
    if (!q || !k || !v || !o) return ATTN_ERR_NULL;
    const uintptr_t mis = (reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                           reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o)) & 15u;
    if (mis || (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_ALIGN;
    if ((long long)Sq * d > INT_MAX || (long long)Sk * d > INT_MAX || (long long)B * H > INT_MAX)
        return ATTN_ERR_OVERFLOW;
    return ATTN_OK;
}

// CU and XCD counts of the current device, queried once per device (the policy table below was
// measured on 256 CUs in 8 XCDs; those are also the values taken when no device answers, e.g. for
// a plan asked for on a host without one).
struct DevInfo {
    int cus, xcds;
};
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
DevInfo g_dev_info[kMaxDevices];

DevInfo device_info() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return {256, 8};
    }
    std::call_once(g_dev_once[dev], [dev] {
        int cus = 0, xcds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
        if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds < 1) xcds = 8;
        (void)hipGetLastError();
        g_dev_info[dev] = {cus, xcds};
    });
    return g_dev_info[dev];
}

// XCD count to order workgroups by (see xcd_order), or 0 when the grid does not split evenly
int xcd_remap_for(int num_wg) {
    const int nx = device_info().xcds;
    return (nx > 1 && num_wg % nx == 0) ? nx : 0;
}

// Schedules and tile shapes that are compiled: (schedule, query blocks per wave, waves, stages,
// keys per tile).
constexpr int kShapes[][5] = {
    {ATTN_SCHED_CLASSIC, 1, 8, 3, 64},  {ATTN_SCHED_CLASSIC, 1, 8, 4, 64},  {ATTN_SCHED_CLASSIC, 2, 4, 3, 64},
    {ATTN_SCHED_CLASSIC, 2, 4, 4, 64},  {ATTN_SCHED_CLASSIC, 1, 4, 2, 64},  {ATTN_SCHED_CLASSIC, 1, 4, 3, 64},
    {ATTN_SCHED_CLASSIC, 2, 8, 3, 64},  {ATTN_SCHED_CLASSIC, 2, 8, 4, 64},  {ATTN_SCHED_CLASSIC, 1, 8, 2, 128},
    {ATTN_SCHED_CLASSIC, 1, 4, 3, 192}, {ATTN_SCHED_CLASSIC, 1, 4, 2, 256}, {ATTN_SCHED_PINGPONG, 1, 8, 3, 64},
    {ATTN_SCHED_DEPHASED, 1, 8, 4, 64}};
// (2, 8, *) holds 64 queries per wave at two waves per SIMD, which fits the registers at d = 64
// only; at d = 128 plans and launches with it return ATTN_ERR_UNSUPPORTED.  128-key tiles take
// 64 KiB of LDS per stage at d = 128, so two stages.  192 and 256 keys per tile (d = 64 only, the
// same error at d = 128, where one stage would take 96 or 128 KiB) run one wave per SIMD: their
// scores alone take 96 or 128 registers a lane, which two waves per SIMD cannot hold (they
// spill 172-396 bytes a lane there); one wave has the matrix-core registers of the SIMD to itself.

bool compiled_shape(int sched, int qb, int nw, int ns, int bk) {
    for (const auto &sh : kShapes)
        if (sh[0] == sched && sh[1] == qb && sh[2] == nw && sh[3] == ns && sh[4] == bk) return true;
    return false;
}

int pack_policy(int sched, int qb, int nw, int ns, int bk) {
    return sched | (qb << 4) | (nw << 8) | (ns << 12) | ((bk / 64) << 16);
}

// Process-wide override of the policy table (attn_fwd_set_policy, or ATTN_FWD_POLICY =
// "sched,qb,nw,ns,bk" read once at the first call); 0 means none, -1 not read yet.
std::atomic<int> g_override{-1};

int policy_override() {
    int v = g_override.load(std::memory_order_relaxed);
    if (v != -1) return v;
    int packed = 0;
    const char *e = std::getenv("ATTN_FWD_POLICY");
    int a = 0, b = 0, c = 0, d = 0, k = 0;
    if (e && std::sscanf(e, "%d,%d,%d,%d,%d", &a, &b, &c, &d, &k) == 5 && compiled_shape(a, b, c, d, k))
        packed = pack_policy(a, b, c, d, k);
    int expected = -1;
    g_override.compare_exchange_strong(expected, packed);
    return g_override.load(std::memory_order_relaxed);
}

// Tile policy, measured on MI355X (bf16 B=2 H=16 S=4096, B=4 H=16 S=2048 and causal B=1 H=32
// S=8192 at d=128; B=1..4, H=8..40, S=2048..16384 causal and not, and B=1 H=2 S=128 at d=64).
// d=128: the classic schedule with 128-key tiles and two stages is 1.4-2.1% faster than the
// de-phased schedule on 64-key tiles, which in turn is 1.5-2% faster than the classic schedule on
// 64-key tiles (causal S=8192 with paired tiles: 495 us against 524 for (1, 8, 4, 64) and 564
// de-phased).  d=64: see the rule below; the de-phased schedule is not faster there, nor are
// 192- or 256-key tiles (one wave per SIMD: 27-38% slower).  Choosing the kernel variant at run
// time from a table measured per shape and keyed on the device's compute-unit count is the
// runtime policy of the FlashInfer KDA write-up (blog.secrett2633), its section 1 and its closing
// lessons.
// Causal query tiles of a head cost 1, 2, .., n key-tile rows of work; paired (n-1-j, j) they cost
// n+1 each (the middle tile of an odd n alone (n+1)/2).  Equal items fill the CUs in whole rounds,
// so pairing pays only where its rounds come out full: the makespan estimate of the pairs (rounds
// of n+1, two middle tiles to a slot) against that of single tiles taken heaviest first (the
// longest tile or the work per CU, whichever is larger), within 2% (what the shared K/V reads
// gain: bf16 causal B=1 H=32 S=8192 d=128, 497 -> 482 us at equal balance).
bool pairs_well(long long bh, int n, int cus) {
    if (n < 2) return false;
    const long long slots = bh * (n / 2) + ((n & 1) ? (bh + 1) / 2 : 0);
    const long long paired = (slots + cus - 1) / cus * (n + 1);
    const long long total = bh * n * (long long)(n + 1) / 2;
    const long long single = std::max<long long>(n, (total + cus - 1) / cus);
    return paired * 50 <= single * 51;
}

void choose_policy(int B, int H, int Sq, int d, int causal, Plan *pl) {
    pl->sched = ATTN_SCHED_CLASSIC;
    pl->qb = 1;
    pl->nw = 8;
    if (d == 128) {
        pl->ns = 2;
        pl->bk = 128;
    } else {
        // d = 64: 128-key tiles with 32 queries per wave, (1, 8, 2, 128), or 64-key tiles with 64
        // queries per wave, (2, 8, 4, 64), 4% faster per query tile but half as many tiles, so it
        // wins only where its rounds of workgroups come out as full (non-causal: rounds times the
        // tile's cost; B=2 H=16 S=4096 147.6 against 154.3 us, B=1 H=20 S=8192 525.3 against
        // 423.5 us, its 320 tiles taking 2 rounds of 512 queries where (1, 8, 2, 128)'s 640 take 3
        // rounds of 256).  Causal,
        // it wins on long sequences with its tiles paired (B=1 H=16 S=16384: 586 against 606 us)
        // and loses on short ones (B=4 H=32 S=2048: 104.9 against 97.6 us).  (1, 8, 4, 64) measured
        // slower than (1, 8, 2, 128) on every d = 64 shape timed (B=1 H=8..40, S=2048..8192).
        pl->ns = 2;
        pl->bk = 128;
        const long long bh = (long long)B * H, cus = device_info().cus;
        const long long n512 = (Sq + 511) / 512, n256 = (Sq + 255) / 256;
        bool wide;
        if (!causal) {
            const double t512 = (double)((bh * n512 + cus - 1) / cus) * 512.0;
            const double t256 = (double)((bh * n256 + cus - 1) / cus) * 256.0 / 0.96;
            wide = t512 <= t256;
        } else {
            wide = Sq >= 8192 && pairs_well(bh, (int)n512, (int)cus);
        }
        if (wide) {
            pl->qb = 2;
            pl->ns = 4;
            pl->bk = 64;
        }
    }
    // at most 128 query rows: 256-query workgroups would compute as many clamped rows as real
    // ones; 4 waves of 32 queries compute none (B=1 H=2 S=128 d=64: 7.4 vs 7.8 us per launch)
    if (Sq <= 128) {
        pl->qb = 1;
        pl->nw = 4;
        pl->ns = 2;
        pl->bk = 64;
    }
    const int ov = policy_override();
    if (ov > 0) {
        pl->sched = ov & 15;
        pl->qb = (ov >> 4) & 15;
        pl->nw = (ov >> 8) & 15;
        pl->ns = (ov >> 12) & 15;
        pl->bk = ((ov >> 16) & 15) * 64;
    }
}

int make_plan(int B, int H, int Sq, int d, int causal, Plan *pl) {
    choose_policy(B, H, Sq, d, causal, pl);
    if (pl->qb == 2 && pl->nw == 8 && d != 64) return ATTN_ERR_UNSUPPORTED;   // registers: d = 64 only
    if (pl->bk > 128 && d != 64) return ATTN_ERR_UNSUPPORTED;                 // LDS: d = 64 only
    pl->block_q = pl->nw * pl->qb * 32;
    pl->block_k = pl->bk;
    pl->nqt = (Sq + pl->block_q - 1) / pl->block_q;
    // Causal tiles go in pairs (nqt-1-j, j) where that keeps the CUs as busy (pairs_well): the key
    // tiles are then fetched about once per head instead of up to twice (bf16 causal B=1 H=32
    // S=8192 d=128: FETCH_SIZE 1.43x the algorithmic bytes unpaired, 1.25x paired).
    const long long npair = (long long)B * H * ((pl->nqt + 1) / 2);
    pl->pair = causal && pl->sched == ATTN_SCHED_CLASSIC && pairs_well((long long)B * H, pl->nqt, device_info().cus);
    const long long wg = pl->pair ? npair : (long long)pl->nqt * B * H;
    if (wg > INT_MAX) return ATTN_ERR_OVERFLOW;
    pl->num_wg = (int)wg;
    return ATTN_OK;
}

template <class T, int D, bool CAUSAL, int QB, int NW, int NS, int BC = 64>
int launch(const Params &p, const Plan &pl, hipStream_t stream) {
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, QB, NW, BC, NS, CAUSAL>), dim3(pl.num_wg), dim3(NW * 64), 0, stream, p);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

template <class T, int D, bool CAUSAL>
int launch_shape(const Params &p, const Plan &pl, hipStream_t s) {
    if (pl.sched == ATTN_SCHED_PINGPONG) {
        hipLaunchKernelGGL((attn_fwd_pp_kernel<T, D, CAUSAL>), dim3(pl.num_wg), dim3(512), 0, s, p);
        return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
    }
    if (pl.sched == ATTN_SCHED_DEPHASED) {
        hipLaunchKernelGGL((attn_fwd_dp_kernel<T, D, CAUSAL>), dim3(pl.num_wg), dim3(512), 0, s, p);
        return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
    }
    if (pl.bk == 128) {
        if (pl.qb == 1 && pl.nw == 8 && pl.ns == 2) return launch<T, D, CAUSAL, 1, 8, 2, 128>(p, pl, s);
        return ATTN_ERR_UNSUPPORTED;
    }
    if (pl.bk == 192 || pl.bk == 256) {
        if constexpr (D == 64) {
            if (pl.bk == 192 && pl.qb == 1 && pl.nw == 4 && pl.ns == 3)
                return launch<T, D, CAUSAL, 1, 4, 3, 192>(p, pl, s);
            if (pl.bk == 256 && pl.qb == 1 && pl.nw == 4 && pl.ns == 2)
                return launch<T, D, CAUSAL, 1, 4, 2, 256>(p, pl, s);
        }
        return ATTN_ERR_UNSUPPORTED;
    }
    const int key = pl.qb * 100 + pl.nw * 10 + pl.ns;
    switch (key) {
        case 183: return launch<T, D, CAUSAL, 1, 8, 3>(p, pl, s);
        case 184: return launch<T, D, CAUSAL, 1, 8, 4>(p, pl, s);
        case 243: return launch<T, D, CAUSAL, 2, 4, 3>(p, pl, s);
        case 244: return launch<T, D, CAUSAL, 2, 4, 4>(p, pl, s);
        case 142: return launch<T, D, CAUSAL, 1, 4, 2>(p, pl, s);
        case 143: return launch<T, D, CAUSAL, 1, 4, 3>(p, pl, s);
        case 283:
            if constexpr (D == 64) return launch<T, D, CAUSAL, 2, 8, 3>(p, pl, s);
            return ATTN_ERR_UNSUPPORTED;
        case 284:
            if constexpr (D == 64) return launch<T, D, CAUSAL, 2, 8, 4>(p, pl, s);
            return ATTN_ERR_UNSUPPORTED;
        default: return ATTN_ERR_UNSUPPORTED;
    }
}

template <class T>
int dispatch(const Params &p, const Plan &pl, int d, int causal, hipStream_t s) {
    if (d == 128) return causal ? launch_shape<T, 128, true>(p, pl, s) : launch_shape<T, 128, false>(p, pl, s);
    return causal ? launch_shape<T, 64, true>(p, pl, s) : launch_shape<T, 64, false>(p, pl, s);
}

// fp8: 8 waves x 32 queries, 128-key tiles (one descale block), four stages: step t reads the V
// tile of t-1 (its P.V runs one step late) and the K tile of t while tiles t+1 and t+2 load
constexpr int kFp8Stages = 4;

void make_plan_fp8(int B, int H, int Sq, Plan *pl) {
    pl->sched = 0;
    pl->bk = 128;
    pl->qb = 1;
    pl->nw = 8;
    pl->ns = kFp8Stages;
    pl->pair = 0;
    pl->block_q = 256;
    pl->block_k = 128;
    pl->nqt = (Sq + pl->block_q - 1) / pl->block_q;
    pl->num_wg = 0;
    const long long wg = (long long)pl->nqt * B * H;
    if (wg <= INT_MAX) pl->num_wg = (int)wg;
}

template <int D, bool CAUSAL, int FMT>
int launch_fp8(const ParamsF8 &p, const Plan &pl, hipStream_t s) {
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, kFp8Stages, CAUSAL, FMT>), dim3(pl.num_wg), dim3(512), 0, s, p);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

template <int FMT>
int launch_fp8_d(const ParamsF8 &p, const Plan &pl, int d, int causal, hipStream_t s) {
    if (d == 128) return causal ? launch_fp8<128, true, FMT>(p, pl, s) : launch_fp8<128, false, FMT>(p, pl, s);
    return causal ? launch_fp8<64, true, FMT>(p, pl, s) : launch_fp8<64, false, FMT>(p, pl, s);
}

// fmt: 0 = E4M3 codes, 1 = E5M2 codes
int run_fp8(const void *q, const void *k, const void *v, const float *q_descale, const float *k_descale,
            const float *v_descale, void *o, float *lse, int B, int H, int S_q, int S_k, int d, int causal,
            float scale, int fmt, void *stream) {
    Plan pl;
    make_plan_fp8(B, H, S_q, &pl);
    if (pl.num_wg == 0) return ATTN_ERR_OVERFLOW;
    ParamsF8 p;
    p.q = static_cast<const uint8_t *>(q);
    p.k = static_cast<const uint8_t *>(k);
    p.v = static_cast<const uint8_t *>(v);
    p.qd = q_descale;
    p.kd = k_descale;
    p.vd = v_descale;
    p.o = static_cast<uint16_t *>(o);
    p.lse = lse;
    p.Sq = S_q;
    p.Sk = S_k;
    p.nqb = (S_q + 127) / 128;
    p.nkb = (S_k + 127) / 128;
    p.nqt = pl.nqt;
    p.num_wg = pl.num_wg;
    p.xcd_remap = xcd_remap_for(pl.num_wg);
    p.c = scale * 1.44269504088896340736f;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return fmt ? launch_fp8_d<1>(p, pl, d, causal, s) : launch_fp8_d<0>(p, pl, d, causal, s);
}

int check_descales(const float *q_descale, const float *k_descale, const float *v_descale) {
    if (!q_descale || !k_descale || !v_descale) return ATTN_ERR_DESCALE;
    if ((reinterpret_cast<uintptr_t>(q_descale) | reinterpret_cast<uintptr_t>(k_descale) |
         reinterpret_cast<uintptr_t>(v_descale)) & 3u)
        return ATTN_ERR_DESCALE;
    return ATTN_OK;
}

// f16 / bf16 attention (arguments checked); q_rstd and w_q non-null fold RMSNorm into Q
int run_half(const void *q, const void *k, const void *v, const float *q_rstd, const void *w_q, void *o, float *lse,
             int B, int H, int S_q, int S_k, int d, int causal, float scale, int dtype, void *stream) {
    Plan pl;
    int st = make_plan(B, H, S_q, d, causal, &pl);
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
    p.xcd_remap = xcd_remap_for(pl.num_wg);
    p.c = scale * 1.44269504088896340736f;
    p.pair = pl.pair;
    p.qr = q_rstd;
    p.wq = static_cast<const uint16_t *>(w_q);
    p.H = H;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == ATTN_BF16) return dispatch<BF16>(p, pl, d, causal, s);
    return dispatch<F16>(p, pl, d, causal, s);
}

}  // namespace

extern "C" int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int S_q,
                        int S_k, int d, int causal, float scale, int dtype, void *stream) {
    if (dtype != ATTN_F16 && dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3 && dtype != ATTN_FP8_E5M2)
        return ATTN_ERR_UNSUPPORTED;
    int st = check_common(q, k, v, o, lse, B, H, S_q, S_k, d, scale);
    if (st == kEmpty) return ATTN_OK;
    if (st != ATTN_OK) return st;
    if (dtype == ATTN_FP8_E4M3 || dtype == ATTN_FP8_E5M2)
        return run_fp8(q, k, v, nullptr, nullptr, nullptr, o, lse, B, H, S_q, S_k, d, causal, scale,
                       dtype == ATTN_FP8_E5M2 ? 1 : 0, stream);
    return run_half(q, k, v, nullptr, nullptr, o, lse, B, H, S_q, S_k, d, causal, scale, dtype, stream);
}

extern "C" int attn_fwd_qnorm(const void *q, const void *k, const void *v, const float *q_rstd, const void *w_q,
                              void *o, float *lse, int B, int H, int S_q, int S_k, int d, int causal, float scale,
                              int dtype, void *stream) {
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    int st = check_common(q, k, v, o, lse, B, H, S_q, S_k, d, scale);
    if (st == kEmpty) return ATTN_OK;
    if (st != ATTN_OK) return st;
    if (!q_rstd || !w_q) return ATTN_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(q_rstd) & 3u) || (reinterpret_cast<uintptr_t>(w_q) & 15u)) return ATTN_ERR_ALIGN;
    if ((long long)B * S_q > INT_MAX || (long long)H * d > INT_MAX) return ATTN_ERR_OVERFLOW;
    return run_half(q, k, v, q_rstd, w_q, o, lse, B, H, S_q, S_k, d, causal, scale, dtype, stream);
}

extern "C" int attn_fwd_fp8(const void *q, const void *k, const void *v, const float *q_descale,
                            const float *k_descale, const float *v_descale, void *o, float *lse, int B, int H,
                            int S_q, int S_k, int d, int causal, float scale, void *stream) {
    int st = check_common(q, k, v, o, lse, B, H, S_q, S_k, d, scale);
    if (st == kEmpty) return ATTN_OK;
    if (st != ATTN_OK) return st;
    st = check_descales(q_descale, k_descale, v_descale);
    if (st != ATTN_OK) return st;
    return run_fp8(q, k, v, q_descale, k_descale, v_descale, o, lse, B, H, S_q, S_k, d, causal, scale, 0, stream);
}

extern "C" int attn_fwd_fp8_e5m2(const void *q, const void *k, const void *v, const float *q_descale,
                                 const float *k_descale, const float *v_descale, void *o, float *lse, int B, int H,
                                 int S_q, int S_k, int d, int causal, float scale, void *stream) {
    int st = check_common(q, k, v, o, lse, B, H, S_q, S_k, d, scale);
    if (st == kEmpty) return ATTN_OK;
    if (st != ATTN_OK) return st;
    st = check_descales(q_descale, k_descale, v_descale);
    if (st != ATTN_OK) return st;
    return run_fp8(q, k, v, q_descale, k_descale, v_descale, o, lse, B, H, S_q, S_k, d, causal, scale, 1, stream);
}

extern "C" int attn_fwd_plan(int B, int H, int S_q, int S_k, int d, int causal, int dtype, int *block_q,
                             int *block_k, int *waves, int *workgroups) {
    if (B < 0 || H < 0 || S_q < 0 || S_k < 0) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3 && dtype != ATTN_FP8_E5M2)
        return ATTN_ERR_UNSUPPORTED;
    const bool empty = B == 0 || H == 0 || S_q == 0;   // no query rows: a plan with no workgroups
    if (!empty && S_k == 0) return ATTN_ERR_SHAPE;
    Plan pl;
    if (empty) {
        if (dtype == ATTN_FP8_E4M3 || dtype == ATTN_FP8_E5M2) {
            make_plan_fp8(1, 1, 1, &pl);
        } else {
            const int st = make_plan(1, 1, 1, d, causal, &pl);
            if (st != ATTN_OK) return st;
        }
        pl.num_wg = 0;
    } else if (dtype == ATTN_FP8_E4M3 || dtype == ATTN_FP8_E5M2) {
        make_plan_fp8(B, H, S_q, &pl);
        if (pl.num_wg == 0) return ATTN_ERR_OVERFLOW;
    } else {
        const int st = make_plan(B, H, S_q, d, causal, &pl);
        if (st != ATTN_OK) return st;
    }
    if (block_q) *block_q = pl.block_q;
    if (block_k) *block_k = pl.block_k;
    if (waves) *waves = pl.nw;
    if (workgroups) *workgroups = pl.num_wg;
    return ATTN_OK;
}

extern "C" int attn_fwd_schedule(int d, int causal, int dtype) {
    if (d != 64 && d != 128) return -ATTN_ERR_UNSUPPORTED;
    if (dtype == ATTN_FP8_E4M3 || dtype == ATTN_FP8_E5M2) return ATTN_SCHED_DEFAULT;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return -ATTN_ERR_UNSUPPORTED;
    Plan pl;
    choose_policy(1, 1, 1, d, causal, &pl);
    return pl.sched;
}

extern "C" int attn_fwd_set_policy(int schedule, int qb, int nw, int ns, int bk) {
    if (schedule == 0) {
        policy_override();   // consume the environment once, then clear
        g_override.store(0, std::memory_order_relaxed);
        return ATTN_OK;
    }
    if (!compiled_shape(schedule, qb, nw, ns, bk)) return ATTN_ERR_UNSUPPORTED;
    policy_override();
    g_override.store(pack_policy(schedule, qb, nw, ns, bk), std::memory_order_relaxed);
    return ATTN_OK;
}

extern "C" const char *attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer (q, k, v or o) is NULL";
        case ATTN_ERR_SHAPE: return "a size is negative, or S_k is 0 while there are queries";
        case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension (64 or 128) or dtype";
        case ATTN_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
        case ATTN_ERR_OVERFLOW: return "S*d or the workgroup count exceeds the 32-bit index range";
        case ATTN_ERR_VALUE: return "scale must be finite and > 0";
        case ATTN_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
        case ATTN_ERR_DESCALE: return "fp8 descale pointers must be non-NULL and 4-byte aligned";
        default: return "unknown status";
    }
}
