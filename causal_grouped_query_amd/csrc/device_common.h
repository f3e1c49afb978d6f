// device_common.h -- small gfx950 building blocks shared by the attention
// kernels of libgqa_attn.so: MFMA wrapper, bf16 packing, the key permutation
// that lets the score accumulator feed the PV product without a shuffle, and
// the register transpose that stages V as V^T in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define GQA_LDS __attribute__((address_space(3)))
#define GQA_GLOBAL __attribute__((address_space(1)))

// 32x32x16 bf16 MFMA, fp32 accumulate.  Operand lane layout (both A and B):
// lane l holds row/column (l & 31) and 8 contraction slots owned by lane
// half (l >> 5); A and B are always filled with the same slot -> index map,
// so the hardware's slot order inside a lane never matters.  Accumulator:
// lane l holds column (l & 31), element e is row 8*(e>>2) + 4*(l>>5) + (e&3).
__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4 &a, const u32x4 &b, const f32x16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA, fp32 accumulate.  Lane l holds row/column (l & 15)
// and contraction slots 8*(l>>4) .. +7 of A and B; accumulator element i is
// row 4*(l>>4) + i, column (l & 15).
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4 &a, const u32x4 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Round-to-nearest-even fp32 -> bf16 for two values, packed lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2 p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

// acc + sum of the 8 bf16 values packed in p (v_dot2c_f32_bf16 against 1.0).
// Summing the rounded weights makes the normaliser match the weights the PV
// product actually applies.
__device__ __forceinline__ float sum_bf16x8(const u32x4 &p, float acc)
{
    // Note: bit-cast the whole vector.  This clang miscompiles
    // __builtin_bit_cast applied to a single ext-vector element (it reads
    // element 0 whatever the index).
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    const bf16x8 v = __builtin_bit_cast(bf16x8, p);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[0], v[1]}, one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2], v[3]}, one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[4], v[5]}, one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[6], v[7]}, one, acc, false);
    return acc;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Key permutation inside a 32-key block.  Accumulator row m of a score
// tile S^T = K Q^T is produced by A-operand row m, which we load from key
// kperm(m).  With kperm(m) = 16*(m>>4) + 8*((m>>2)&1) + 4*((m>>3)&1) + (m&3)
// the 8 accumulator elements a lane holds for PV step s are the 8
// consecutive keys 16*s + 8*(l>>5) + 0..7, i.e. the B operand of P^T V-step
// s is the lane's own accumulator slice, and the matching A operand (V^T)
// is one contiguous 16-byte LDS read.
__device__ __forceinline__ int kperm(int m)
{
    return ((m >> 4) << 4) + (((m >> 2) & 1) << 3) + (((m >> 3) & 1) << 2) + (m & 3);
}

// Key (within a 64-key tile) of accumulator element e of score tile t held
// by lane half `hi`.
__device__ __forceinline__ int acc_key(int t, int e, int hi)
{
    return 32 * t + 16 * (e >> 3) + 8 * hi + (e & 7);
}

// Transpose a 4-key x 8-dim block of bf16 (rows r[0..3], 8 dims each) into
// 8 dim-rows of 4 keys: out[e] holds keys 0..3 of dim e as two packed dwords.
__device__ __forceinline__ void transpose4x8(const u32x4 r[4], u32x2 out[8])
{
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        // dims 2w (low halves) and 2w+1 (high halves) of dword w
        out[2 * w].x = __builtin_amdgcn_perm(r[1][w], r[0][w], 0x05040100u);
        out[2 * w].y = __builtin_amdgcn_perm(r[3][w], r[2][w], 0x05040100u);
        out[2 * w + 1].x = __builtin_amdgcn_perm(r[1][w], r[0][w], 0x07060302u);
        out[2 * w + 1].y = __builtin_amdgcn_perm(r[3][w], r[2][w], 0x07060302u);
    }
}

// LDS tile layout ("planes").  A tile of R rows x CPR 16-byte chunks is
// stored plane-major: plane p holds chunks 4p..4p+3 of every row (64 bytes
// per row), and chunk c of row r sits at position (c & 3) ^ pswz(r) of its
// row inside the plane, with pswz(r) = r3 | (r1 ^ r2) << 1 (row bits).
// Bank groups are 16-byte positions inside a 128-byte (32-bank) or 256-byte
// (64-bank) window.  With this swizzle
//  * an MFMA A-operand read (one chunk of rows kperm(0..31): rows
//    16a + {0..3, 8..11} per 8 lanes, rows 16a + 0..15 per 16 lanes) and
//  * a ds_read_b64_tr_b16 read (rows r0 + 0..3, chunks {c0, c0 + 1} per 16
//    lanes; all four chunks of a plane per 32 lanes)
// touch distinct bank groups in both window sizes, and every per-lane
// address of a tile loop is a base register plus an immediate.
#ifndef GQA_PSWZ
#define GQA_PSWZ 1
#endif
__device__ __forceinline__ int pswz(int r)
{
#if GQA_PSWZ
    return ((r >> 3) & 1) | ((((r >> 1) ^ (r >> 2)) & 1) << 1);
#else
    return ((r >> 3) & 1) | (((r >> 1) & 1) << 1);
#endif
}

// Swizzle used by the 16x16x32 operand reads of the absorbed-MLA kernel
// (A rows 16 t + (l & 15), chunk l >> 4; V^T transpose rows 4 (l >> 4) + r):
// measured free of LDS bank conflicts for both read shapes; pswz is not.
__device__ __forceinline__ int pswz16(int r)
{
    return (__builtin_popcount(r & 7) & 1) | ((__builtin_popcount(r & 5) & 1) << 1);
}

template <int R, bool SW16 = false>
struct PlaneTile {
    static constexpr int PLANE_BYTES = R * 64;
    static __device__ __forceinline__ int swz(int r) { return SW16 ? pswz16(r) : pswz(r); }
    // byte offset of chunk c of row r
    static __device__ __forceinline__ int offset(int r, int c)
    {
        return (c >> 2) * PLANE_BYTES + r * 64 + (((c & 3) ^ swz(r)) << 4);
    }
    // The 16-byte slot a copy lane fills: slot = 64 * copy + lane (copies
    // write 1 KiB blocks in order).  Returns the (row, chunk) it must fetch.
    static __device__ __forceinline__ void slot_source(int slot, int &r, int &c)
    {
        const int plane = slot / (R * 4), rem = slot % (R * 4);
        r = rem >> 2;
        c = plane * 4 + ((rem & 3) ^ swz(r));
    }
};

// Asynchronous global -> LDS copy of 16 bytes per lane (gfx950
// global_load_lds_dwordx4).  Lane l's bytes land at lds_wave_base + 16*l;
// lds_wave_base must be the same for the whole wave.
//
// The copies are written as inline assembly on purpose.  Seen as builtins,
// the compiler treats every later LDS transpose read and every workgroup
// barrier as depending on all copies still in flight and drains them
// (s_waitcnt vmcnt(0)), which turns a multi-stage K/V ring into a single
// stage.  Here the compiler knows nothing of the copies: every wait on them
// is explicit (wait_vmem / wait_vmem_le before lds_barrier).  The
// instructions have no register results; they only read their address
// operands at issue.  M0 carries the LDS base (1 wait state before the copy).
//
// NT = true marks the copy non-temporal (the `nt` cache policy): for data a
// kernel reads once per call, such as a decode's KV stream, so that those
// lines do not push other data (the dirty output lines of a preceding
// kernel, say) out of the caches.  Data that other workgroups read again,
// like the forward kernel's K/V tiles, keeps the default policy.
//
// Every one of these statements writes M0 and names it in its clobber list.
// M0 is a reserved register of the AMDGPU backend (the compiler sets it
// right before each of its own uses and never keeps a value in it); clang
// warns that a reserved register is not preserved across the statement,
// which is exactly what the clobber says, so that warning is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ unsigned lds_u32(const void *lds_ptr)
{
    return __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(GQA_LDS const void *)lds_ptr);
}

template <bool NT = false>
__device__ __forceinline__ void g2lds16(const void *gptr, void *lds_wave_base)
{
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(gptr),
                     "s"(lds_u32(lds_wave_base))
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr),
                     "s"(lds_u32(lds_wave_base))
                     : "memory", "m0");
}

// 4 bytes per lane (global_load_lds_dword): lane l's word lands at
// lds_wave_base + 4*l.
template <bool NT = false>
__device__ __forceinline__ void g2lds4(const void *gptr, void *lds_wave_base)
{
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off nt" ::"v"(gptr),
                     "s"(lds_u32(lds_wave_base))
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gptr),
                     "s"(lds_u32(lds_wave_base))
                     : "memory", "m0");
}

// Same copy from a workgroup-uniform base plus a per-lane unsigned byte
// offset (scalar-base form: no per-lane 64-bit address arithmetic).
template <bool NT = false>
__device__ __forceinline__ void g2lds16(const void *uniform_base, unsigned byte_off, void *lds_wave_base)
{
    const unsigned long long a = (unsigned long long)uniform_base;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
    const unsigned long long base = ((unsigned long long)hi << 32) | lo;
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(byte_off), "s"(base),
                     "s"(lds_u32(lds_wave_base))
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(byte_off), "s"(base),
                     "s"(lds_u32(lds_wave_base))
                     : "memory", "m0");
}

// Same copy with the LDS destination given as a workgroup-uniform LDS byte
// address (no generic-pointer round trip, whose null check costs scalar
// instructions per copy).
template <bool NT = false>
__device__ __forceinline__ void g2lds16_at(const void *uniform_base, unsigned byte_off, unsigned lds_addr)
{
    const unsigned long long a = (unsigned long long)uniform_base;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
    const unsigned long long base = ((unsigned long long)hi << 32) | lo;
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(byte_off), "s"(base),
                     "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(byte_off), "s"(base),
                     "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                     : "memory", "m0");
}

template <bool NT = false>
__device__ __forceinline__ void g2lds16_at(const void *gptr, unsigned lds_addr)
{
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(gptr),
                     "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr),
                     "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                     : "memory", "m0");
}

#pragma clang diagnostic pop

// Complete a register's pending global load here: the compiler waits for it
// before an asm statement that reads the register.  Without this, a value
// loaded before a loop whose copies are issued as inline assembly can leave a
// (needlessly full) vmcnt wait inside the loop body.
template <typename T>
__device__ __forceinline__ void hold_reg(const T &x)
{
    asm volatile("" ::"v"(x));
}

// Debug builds (GQA_DEBUG_NANFILL=1) fill a kernel's LDS buffers with NaN
// bit patterns (0xffff in every bf16 half, 0xffffffff as fp32) before first
// use, so any read of a slot no copy or store wrote turns the result into
// NaN.  Called by every thread at kernel entry; ends with a barrier.  A
// no-op in normal builds.
#ifndef GQA_DEBUG_NANFILL
#define GQA_DEBUG_NANFILL 0
#endif
template <typename T>
__device__ __forceinline__ void debug_nanfill(T &lds_obj)
{
#if GQA_DEBUG_NANFILL
    unsigned *w = (unsigned *)&lds_obj;
    for (unsigned i = threadIdx.x; i < sizeof(T) / 4; i += blockDim.x) w[i] = 0xffffffffu;
    __syncthreads();
#else
    (void)lds_obj;
#endif
}

// Workgroup barrier for LDS hand-off: this wave's LDS reads and writes are
// complete (lgkmcnt(0)) before it arrives.  Unlike __syncthreads it does not
// drain outstanding vector-memory operations, so copies for later tiles stay
// in flight across it; the copies a reader needs must be waited for (by every
// wave, for its own copies) before the barrier.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait for this wave's outstanding vector-memory operations (including
// global -> LDS copies).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N of this wave's vector-memory operations are
// outstanding (loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_le()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each 16-lane group, lane
// i receives, for r = 0..3, the 16-bit element (i & 3) of the 8-byte chunk
// addressed by lane 4r + (i >> 2) of the same group.  If lane 4r + q points
// at row R0 + r, columns C0 + 4q .. C0 + 4q + 3 of a row-major 16-bit
// matrix, lane i therefore receives column C0 + i of rows R0 .. R0 + 3.
__device__ __forceinline__ u32x2 lds_read_tr16(const void *lds_addr)
{
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GQA_LDS i16x4 *)lds_addr);
    return __builtin_bit_cast(u32x2, r);
}

// Combine a value with the one held by lane l ^ 32 (same accumulator
// column, other half of the key rows) using gfx950 v_permlane32_swap: after
// the swap the two results hold the low and the high half-wave's values in
// every lane, so max / sum of the pair is the same in both lanes.
__device__ __forceinline__ float halves_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max of finite or -inf values with one VALU instruction each.  fmaxf
// follows IEEE maxNum, for which the compiler first quiets every input it
// cannot prove canonical (one extra v_max_f32 x, x per input); the softmax
// max runs on MFMA results and -inf, where that is never needed.
__device__ __forceinline__ float vmax3(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float vmax(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
// max over lanes l and l ^ 32 of finite or -inf values (see halves_max)
__device__ __forceinline__ float halves_vmax(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Max / sum over the four lanes l, l^16, l^32, l^48 (one 16x16 accumulator
// column) with v_permlane16_swap and v_permlane32_swap; every lane of the
// column gets the same result.
__device__ __forceinline__ float quarters_max(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return halves_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float quarters_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return halves_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

} // namespace gqa
