// Device-side helpers shared by the gfx950 kernels of the block library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 storage (upper half of an fp32)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define LLB_DEV __device__ __forceinline__

LLB_DEV float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
LLB_DEV bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

LLB_DEV uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// 8 fp32 -> one MFMA bf16x8 operand (element 0 in the low half of word 0).
LLB_DEV bf16x8 to_bf16x8(const float* v) {
    uint4 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    u.z = pack_bf16x2(v[4], v[5]);
    u.w = pack_bf16x2(v[6], v[7]);
    return __builtin_bit_cast(bf16x8, u);
}

LLB_DEV bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

LLB_DEV void unpack_bf16x8(uint4 u, float* v) {
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
    v[4] = __uint_as_float(u.z << 16); v[5] = __uint_as_float(u.z & 0xffff0000u);
    v[6] = __uint_as_float(u.w << 16); v[7] = __uint_as_float(u.w & 0xffff0000u);
}

// D(32x32) += A(32x16) B(16x32); lane l supplies A row l%32 and B column l%32,
// k-elements 8*(l/32)..+8.  D: lane l holds column l%32, register r holds row
// 8*(r/4) + 4*(l/32) + r%4.
LLB_DEV f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x32) B(32x16); lane l supplies A row l%16 and B column l%16,
// k-elements 8*(l/16)..+8.  D: lane l holds column l%16, register r holds row
// 4*(l/16) + r.
LLB_DEV f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

LLB_DEV float warp_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

LLB_DEV float warp_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

LLB_DEV float silu_f(float z) { return z / (1.0f + expf(-z)); }

// SiLU for bf16 results: the hardware exp2 and reciprocal (about 1 ulp each in
// fp32, far below bf16's half-ulp of 2^-9).  Large |z| behave: exp2 -> inf
// gives 0 (z < 0), exp2 -> 0 gives z (z > 0).
LLB_DEV float silu_bf16(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// Inverse RMS of a row from its fp32 sum of squares (eps inside the square root).
LLB_DEV float inv_rms(float sumsq, int n, float eps) {
    return 1.0f / sqrtf(sumsq / (float)n + eps);
}

// Workgroup id -> tile id such that consecutive tile ids run on the same XCD.
// Workgroups are dispatched round-robin over the 8 XCDs; tiles that share
// operand panels should share an XCD's L2.
LLB_DEV int xcd_remap(int bid, int nblocks) {
    constexpr int XCD = 8;
    if (nblocks % XCD != 0) return bid;
    return (bid % XCD) * (nblocks / XCD) + bid / XCD;
}

// One 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4): lane i's
// 16 bytes land at LDS byte address lds + 16 * i.  Issued from inline assembly
// so that the compiler does not treat every later LDS read as depending on it
// (it would otherwise wait for all copies in flight before each read); the
// kernel retires the copies itself with s_waitcnt vmcnt.
LLB_DEV void dma16(const void* gptr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(lds)
                 : "memory", "m0");
}

// The same copy with a scalar base: lane i's 16 bytes come from sbase + voff
// (voff a per-lane 32-bit byte offset, sbase uniform), so a loop that moves
// the base by a uniform amount per step needs no per-lane address arithmetic.
LLB_DEV void dma16_s(uint32_t voff, const void* sbase, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}

// Four bytes per lane from gptr into LDS at lds + 4 * lane (one 256-byte
// block per wave), counted by vmcnt like dma16.
LLB_DEV void dma4(const void* gptr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(gptr), "s"(lds)
                 : "memory", "m0");
}

LLB_DEV uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding, expcnt left at its maximum):
// this wave's copies older than the n most recent have landed in LDS, and its
// own LDS reads have completed.
template <int N>
LLB_DEV void wait_vm_lgkm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70);
}

// s_waitcnt vmcnt(n) alone (lgkmcnt and expcnt left at their maxima).
template <int N>
LLB_DEV void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding DMA copy); the empty asm keeps the compiler from
// moving LDS accesses across it.
LLB_DEV void barrier() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
