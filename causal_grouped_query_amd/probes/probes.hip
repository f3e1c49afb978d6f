// probes.hip -- measurement aids for the roofline context of the attention
// kernels (libgqa_probes.so; not part of the attention library's ABI).
//
//  * gqa_probe_mfma_bf16: every wave runs independent chains of
//    v_mfma_f32_32x32x16_bf16 on operands it loads once from a caller buffer
//    (seeded N(0,1) bf16 values: MFMA power, and hence the clock the board
//    sustains, depends on the operand bits).  FLOP = 32768 per MFMA.
//  * gqa_probe_stream_lds: every workgroup streams its share of a buffer
//    HBM -> LDS with global_load_lds_dwordx4 through a ring, with no
//    arithmetic: the read bandwidth the attention kernels' copies can reach.
//
// Both record, per workgroup, the shader clock counter (s_memtime) and the
// constant 100 MHz counter (s_memrealtime) at start and end, so the host can
// report the shader clock the chip actually ran at under that load.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define GQA_PROBE_API extern "C" __attribute__((visibility("default")))

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;  // independent accumulators per wave

// clk[4 * block + 0..3] = memtime start, memtime end, realtime start, realtime end
__device__ __forceinline__ void stamp(unsigned long long *clk, int slot)
{
    const unsigned long long t = __builtin_amdgcn_s_memtime();
    const unsigned long long r = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        clk[4 * blockIdx.x + slot] = t;
        clk[4 * blockIdx.x + 2 + slot] = r;
    }
}

__global__ __launch_bounds__(512) void mfma_probe_kernel(const u32x4 *ops, float *out, unsigned long long *clk,
                                                         int iters, int n_ops)
{
    const int gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    u32x4 a[kChains], b[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) {
        a[j] = ops[((gw * 2 * kChains + 2 * j) % n_ops) * 64 + lane];
        b[j] = ops[((gw * 2 * kChains + 2 * j + 1) % n_ops) * 64 + lane];
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    __syncthreads();
    stamp(clk, 0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[j]),
                                                             __builtin_bit_cast(bf16x8, b[j]), acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    __syncthreads();
    stamp(clk, 1);
    out[(size_t)gw * 64 + lane] = s;  // keeps every chain live
}

// Ring of kStreamStages slots of (waves x 64 lanes x 16 B); each wave waits
// for its own copies before reusing a slot (no cross-wave hand-off: the data
// is never read).
constexpr int kStreamStages = 8;

__global__ __launch_bounds__(256) void stream_probe_kernel(const char *src, size_t bytes_per_block, int reps,
                                                           unsigned long long *clk)
{
    __shared__ __attribute__((aligned(1024))) char ring[kStreamStages][256 * 16];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const char *base = src + (size_t)blockIdx.x * bytes_per_block;
    const size_t steps = bytes_per_block / (256 * 16);
    stamp(clk, 0);
    for (int r = 0; r < reps; ++r) {
        for (size_t s = 0; s < steps; ++s) {
            const char *g = base + s * 4096 + (size_t)w * 1024 + (size_t)lane * 16;
            const unsigned lds = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)&ring[s % kStreamStages][w * 1024];
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved: the clobber records the write
            asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off\n\ts_waitcnt vmcnt(6)" ::"v"(g),
                         "s"(__builtin_amdgcn_readfirstlane(lds))
                         : "memory", "m0");
#pragma clang diagnostic pop
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    stamp(clk, 1);
}

} // namespace

// grid workgroups of waves_per_block (1..8) waves; ops: n_ops >= 1 operand
// registers of 64 lanes x 16 B (bf16); out: grid * waves_per_block * 64
// floats; clk: grid * 4 counters.  Returns 0 or -1 (bad argument / launch).
GQA_PROBE_API int gqa_probe_mfma_bf16(const void *ops, int n_ops, float *out, unsigned long long *clk, int grid,
                                      int waves_per_block, int iters, void *stream)
{
    if (!ops || !out || !clk || n_ops < 1 || grid < 1 || waves_per_block < 1 || waves_per_block > 8 || iters < 1)
        return -1;
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(grid), dim3(64 * waves_per_block), 0, (hipStream_t)stream,
                       (const u32x4 *)ops, out, clk, iters, n_ops);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// grid workgroups of 4 waves each read bytes_per_block bytes (a multiple of
// 4096) of src, reps times; src holds grid * bytes_per_block bytes, 16-byte
// aligned; clk: grid * 4 counters.
GQA_PROBE_API int gqa_probe_stream_lds(const void *src, size_t bytes_per_block, int grid, int reps,
                                       unsigned long long *clk, void *stream)
{
    if (!src || !clk || grid < 1 || reps < 1 || bytes_per_block < 4096 || bytes_per_block % 4096 != 0 ||
        ((uintptr_t)src % 16) != 0)
        return -1;
    hipLaunchKernelGGL(stream_probe_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const char *)src,
                       bytes_per_block, reps, clk);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
