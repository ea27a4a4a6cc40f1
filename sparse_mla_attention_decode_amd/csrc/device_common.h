// Device helpers shared by the gfx950 kernels of libmla: vector types, LDS
// access, the FP8 dequant conversion, register-class-pinned MFMAs and their
// hazard fences, direct-to-LDS copies and explicit memory-counter waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int TILE = 32;                   // keys per tile
constexpr float INIT_MAX = -1e30f;         // "no reference max yet"

__device__ __forceinline__ u32x4 lds_read16(const LDS_AS uint8_t* base, int off) {
    return *(const LDS_AS u32x4*)(base + off);
}
__device__ __forceinline__ u32x2 lds_read8(const LDS_AS uint8_t* base, int off) {
    return *(const LDS_AS u32x2*)(base + off);
}
__device__ __forceinline__ void lds_write16(LDS_AS uint8_t* base, int off, u32x4 v) {
    *(LDS_AS u32x4*)(base + off) = v;
}

// Transposing LDS read: in each group of 16 lanes, lane 4b+c receives column c
// (16-bit) of the 8-byte rows addressed by lanes b, b+4, b+8, b+12.
__device__ __forceinline__ u32x2 lds_read_tr16(const LDS_AS uint8_t* base, int off) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(base + off));
    return __builtin_bit_cast(u32x2, v);
}

// two e4m3fn codes (bytes 2*HI, 2*HI+1 of w) times a power-of-two scale -> two
// bf16 packed in a dword (low half = lower byte); the product is exact.
template <bool HI>
__device__ __forceinline__ uint32_t dequant2(uint32_t w, float scale) {
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2 r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

// MFMA helpers with explicit register classes.  At occupancy 1 a wave owns
// 256 VGPRs + 256 AGPRs: the output accumulator takes all AGPRs; Q, the score
// accumulators and everything else live in VGPRs.  Without the constraints the
// compiler puts every accumulator in AGPRs and spills.
// GUARD: two wait states before the MFMA.  When spare AGPRs exist (a kernel
// whose accumulators leave some free) the compiler may park an operand there
// and reload it into its VGPR right before the asm; that VALU write followed
// by the MFMA's read needs two wait states, and the compiler's hazard
// recognizer does not insert them for inline asm.
template <bool GUARD = false>
__device__ __forceinline__ void mfma_qk_first(f32x16& s, const bf16x8& a, const bf16x8& q) {
    if (GUARD) asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "v"(q));
    else asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "v"(q));
}
template <bool GUARD = false>
__device__ __forceinline__ void mfma_qk(f32x16& s, const bf16x8& a, const bf16x8& q) {
    if (GUARD) asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(q));
    else asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(q));
}
__device__ __forceinline__ void mfma_pv(f32x16& o, const bf16x8& a, const bf16x8& pm) {
    o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pm, o, 0, 0, 0);
}
// The hazard recognizer does not look inside inline asm.  These fences wait
// out the MFMA result latency before VALU reads an accumulator, and the VALU
// write -> MFMA operand read latency before freshly computed P is consumed.
__device__ __forceinline__ void mfma_result_fence2(f32x16& s, f32x16& t) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(s), "+v"(t));
}
__device__ __forceinline__ void valu_to_mfma_fence(bf16x8& a, bf16x8& b) {
    asm volatile("s_nop 4" : "+v"(a), "+v"(b));
}

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Direct-to-LDS copies: lane i's bytes land at lds_addr + 16 i (dwordx4) or
// lds_addr + 4 i (dword).  Written as inline asm so the compiler's wait-count
// pass neither counts them nor treats later LDS reads as aliasing them (it
// would drain every copy in flight); the kernels order them with explicit
// vmcnt waits.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(lds_addr), "v"(src) : "memory", "m0");
}
// Destination = scalar base + constant, added straight into M0.
__device__ __forceinline__ void dma16_at(const void* src, uint32_t base, int off) {
    asm volatile("s_add_u32 m0, %0, %2\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(base), "v"(src), "i"(off) : "memory", "m0", "scc");
}
// Scalar row base + per-lane 32-bit offset (every lane reads 16 bytes of one
// row), destination given as a scalar LDS address.
__device__ __forceinline__ void dma16_row(uint64_t row, uint32_t lane_off, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds_addr), "v"(lane_off), "s"(row) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                 :: "s"(lds_addr), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ void dma4_at(const void* src, uint32_t base, int off) {
    asm volatile("s_add_u32 m0, %0, %2\n\tglobal_load_lds_dword %1, off"
                 :: "s"(base), "v"(src), "i"(off) : "memory", "m0", "scc");
}

// s_waitcnt on vmcnt only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ uint32_t lds_u32(const LDS_AS uint8_t* p) {
    return (uint32_t)(uintptr_t)p;
}

}  // namespace mla
