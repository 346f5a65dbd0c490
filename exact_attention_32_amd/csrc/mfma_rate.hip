// mfma_rate.hip -- calibration kernels: the dense matrix-core rate that MI355X sustains on random
// operands under its power limit (the roofline's practical ceiling for the attention kernels, which
// run the same instructions).
//
// Each workgroup holds 8 waves (two per SIMD, as the attention kernels run).  Every wave issues
// MFMAs back to back into four independent accumulators; the A operand of each MFMA is a fresh
// LDS read from a 64 KiB table of random values (as the attention kernels read K and V^T), the B
// operand cycles through eight register fragments (as the query fragments do).
//   bf16: v_mfma_f32_32x32x16_bf16, 16-byte A fragments; FLOP per MFMA = 32 * 32 * 16 * 2.
//   fp8:  v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands and unit block scales (the fp8
//         attention kernel's instruction), 32-byte A fragments; FLOP per MFMA = 32 * 32 * 64 * 2.
//   A in registers (bf16 or fp8): the same kernels with the A operand cycling through four
//         register fragments (random values from the same table) instead of LDS reads, so that the
//         rate with and without the attention kernels' LDS operand reads can be told apart.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mfma_rate.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 512;
constexpr int kTableBytes = 65536;
constexpr int kTable16 = kTableBytes / 16;   // 16-byte entries

template <bool FP8> __device__ __forceinline__ f32x16 mfma_step(const u32x4 &a0, const u32x4 &a1, const u32x4 &b0,
                                                                const u32x4 &b1, const f32x16 &c) {
    if constexpr (FP8) {
        const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    } else {
        (void)a1;
        (void)b1;
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0), __builtin_bit_cast(bf16x8, b0), c,
                                                       0, 0, 0);
    }
}

template <bool FP8, bool AREG = false>
__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(const u32x4 *__restrict__ table, int iters,
                                                             float *__restrict__ out) {
    // 96 KiB of LDS (the table in the first 64 KiB) keeps one workgroup per CU
    __shared__ __attribute__((aligned(1024))) u32x4 lds[3 * kTableBytes / 32];
    for (int i = threadIdx.x; i < kTable16; i += kThreads) lds[i] = table[i];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    u32x4 bq[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) bq[j] = table[(blockIdx.x * 64 + j * 512 + threadIdx.x) & (kTable16 - 1)];
    u32x4 ar[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ar[j] = table[(blockIdx.x * 64 + j * 256 + 77 + threadIdx.x) & (kTable16 - 1)];
    __syncthreads();
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
    // each wave walks its own offset through the table; 16 MFMAs per iteration
    int base = (wave * 16 + (blockIdx.x & 15)) * 64 + lane;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const u32x4 a0 = AREG ? ar[u & 3] : lds[(base + u * 64) & (kTable16 - 1)];
            u32x4 a1 = a0;
            if constexpr (FP8) a1 = AREG ? ar[(u + 1) & 3] : lds[(base + u * 64 + 32) & (kTable16 - 1)];
            acc[u & 3] = mfma_step<FP8>(a0, a1, bq[u & 7], bq[(u + 1) & 7], acc[u & 3]);
        }
        base += 1024;
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[j][i];
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

// The entry points of include/mfma_rate.h.  table: device pointer to 64 KiB of operand values (bf16
// values, or E4M3 codes for the fp8 kernel);
// out: device float[grid * 512]; 16 * iters MFMAs per wave; grid = the CU count gives one
// workgroup (two waves per SIMD) per CU.  Returns 0, 1 for bad arguments, or the hipError_t of
// the launch.
extern "C" int attn_mfma_rate(const void *table, int grid, int iters, float *out, void *stream) {
    if (!table || !out || grid < 1 || iters < 1) return 1;
    hipLaunchKernelGGL(mfma_rate_kernel<false>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4 *)table, iters, out);
    return (int)hipGetLastError();
}

extern "C" int attn_mfma_rate_regs(const void *table, int grid, int iters, float *out, void *stream) {
    if (!table || !out || grid < 1 || iters < 1) return 1;
    hipLaunchKernelGGL((mfma_rate_kernel<false, true>), dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4 *)table, iters, out);
    return (int)hipGetLastError();
}

extern "C" int attn_mfma_rate_fp8(const void *table, int grid, int iters, float *out, void *stream) {
    if (!table || !out || grid < 1 || iters < 1) return 1;
    hipLaunchKernelGGL(mfma_rate_kernel<true>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4 *)table, iters, out);
    return (int)hipGetLastError();
}

extern "C" int attn_mfma_rate_fp8_regs(const void *table, int grid, int iters, float *out, void *stream) {
    if (!table || !out || grid < 1 || iters < 1) return 1;
    hipLaunchKernelGGL((mfma_rate_kernel<true, true>), dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4 *)table, iters, out);
    return (int)hipGetLastError();
}
