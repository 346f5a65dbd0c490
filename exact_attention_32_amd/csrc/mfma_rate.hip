// mfma_rate.hip -- calibration kernel: the dense bf16 matrix-core rate that MI355X sustains on
// random operands under its power limit (the roofline's practical ceiling for the attention
// kernels, which run the same instruction).
//
// Each workgroup holds 8 waves (two per SIMD, as the attention kernels run).  Every wave issues
// v_mfma_f32_32x32x16_bf16 back to back into four independent accumulators; the A operand of each
// MFMA is a fresh 16-byte LDS read from a 64 KiB table of N(0,1) bf16 values (as the attention
// kernels read K and V^T), the B operand cycles through eight register fragments (as the query
// fragments do).  FLOP per launch = 32 * 32 * 16 * 2 * MFMAs.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kTableBytes = 65536;

__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(const u32x4 *__restrict__ table, int iters,
                                                             float *__restrict__ out) {
    // 96 KiB of LDS (the table in the first 64 KiB) keeps one workgroup per CU
    __shared__ __attribute__((aligned(1024))) u32x4 lds[3 * kTableBytes / 32];
    for (int i = threadIdx.x; i < kTableBytes / 16; i += kThreads) lds[i] = table[i];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    u32x4 bq[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) bq[j] = table[(blockIdx.x * 64 + j * 512 + threadIdx.x) & (kTableBytes / 16 - 1)];
    __syncthreads();
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
    // each wave walks its own offset through the table; 16 reads of 1 KiB per iteration
    int base = (wave * 16 + (blockIdx.x & 15)) * 64 + lane;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const u32x4 a = lds[(base + u * 64) & (kTableBytes / 16 - 1)];
            acc[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                                 __builtin_bit_cast(bf16x8, bq[u & 7]), acc[u & 3], 0,
                                                                 0, 0);
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

// table: device pointer to 64 KiB of bf16 operand values; out: device float[grid * 512];
// 16 * iters MFMAs per wave; grid = the CU count gives one workgroup (two waves per SIMD) per CU.
// Returns 0, or the hipError_t of the launch.
extern "C" int attn_mfma_rate(const void *table, int grid, int iters, float *out, void *stream) {
    if (!table || !out || grid < 1 || iters < 1) return 1;
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, (const u32x4 *)table,
                       iters, out);
    return (int)hipGetLastError();
}
