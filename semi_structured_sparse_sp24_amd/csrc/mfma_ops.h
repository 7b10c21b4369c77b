// mfma_ops.h -- thin wrappers over the gfx950 sparse and dense matrix
// instructions, with the operand layouts measured on the hardware.
//
// Sparse (the paper's section 2 "Sparse tensor cores": the compressed first
// operand A carries two kept values and a 2-bit position per group of four;
// the positions select the matching elements of the dense operand B):
//
//   v_smfmac_f32_16x16x64_{bf16,f16}   (one "step" = 64 dense K)
//     A, lane l: row l%16; 8 compressed values = the 4 groups of dense K
//        [16*(l/16), +16), values 2j and 2j+1 belonging to group j;
//     index: 16 bits per lane, slot s reading bits [2s, 2s+1] -- that is,
//        group j's nibble p0 | p1 << 2 at bits [4j, 4j+3]; `abid` picks the
//        low (0) or high (1) half of the 32-bit index register;
//     B, lane l: column l%16; 16 values = dense K [8*(l/16), +8) followed by
//        dense K [32 + 8*(l/16), +8);
//     D, lane l: D[4*(l/16) + i][l%16], i = 0..3.
//   v_smfmac_f32_16x16x128_fp8_fp8, v_smfmac_i32_16x16x128_i8  (one step = 128 dense K)
//     A, lane l: row l%16; 16 compressed bytes = the 8 groups of dense K
//        [32*(l/16), +32); index: all 32 bits, group j's nibble at [4j, 4j+3];
//     B, lane l: column l%16; 32 bytes = dense K [16*(l/16), +16) then
//        [64 + 16*(l/16), +16);
//     D as above.
// With the metadata format of this library (nibble per group, 8 groups per
// little-endian uint32), lane group kg of a 16-bit step needs the half
// (kg & 1) of word (2*step + kg/2) of its row: one shift per lane.  An fp8
// step's lane group kg needs word (4*step + kg) unchanged.
//
// Dense:
//   v_mfma_f32_32x32x16_{bf16,f16}: A/B lane l: row/column l%32, dense K
//     [8*(l/32), +8); D lane l: D[8*(i/4) + 4*(l/32) + i%4][l%32], i=0..15.
//   v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 both sides, unit E8M0 scales):
//     A/B lane l: row/column l%32, 32 bytes of dense K [32*(l/32), +32).
#pragma once

#include "sp24_internal.h"

namespace sp24 {

// Raw buffer access over one operand.  The descriptor's size is the operand's
// byte size, and the hardware returns zeros for any offset at or past it, so
// rows past the end of a matrix and chunks masked with kOOB read as zeros
// without branches.  Operands are limited to 2 GiB each (checked on the host).
constexpr uint32_t kOOB = 0x80000000u;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

struct Buf {
    __amdgpu_buffer_rsrc_t r;
    u32x4 d;   // the same descriptor as four scalar words, for the LDS DMA load below
    __device__ __forceinline__ Buf(const void* p, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000)) {
        const uint64_t a = (uint64_t)(uintptr_t)p;
        d = (u32x4){(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) & 0xffffu,
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), 0x00020000u};
    }
    __device__ __forceinline__ uint4 ld16(uint32_t off) const {
        u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
        return make_uint4(v[0], v[1], v[2], v[3]);
    }
    __device__ __forceinline__ uint32_t ld4(uint32_t off) const {
        return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    }
};

// Global -> LDS load of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane
// l's 16 bytes at byte offset voff + soff of the buffer land at LDS address
// lds + 16 l.  Rows past the buffer's size read as zeros.
//
// Written as inline assembly, not with the compiler's LDS-DMA builtin, on
// purpose: the compiler cannot tell which LDS bytes a DMA load writes, so
// before every LDS read that follows one it waits for every DMA load still in
// flight (s_waitcnt vmcnt(0)), including those that fill later pipeline
// stages, which drains the software pipeline at every step.  The kernels
// order their DMA loads and LDS reads themselves: each waits with an explicit
// s_waitcnt vmcnt(n) for its own loads of a stage, and a barrier then makes
// every wave's loads of that stage visible before any wave reads it.  The
// instruction has no register results (nothing to wait on for registers).
// M0 holds the LDS address; gfx9 needs one wait state between writing M0 and
// an LDS DMA load that reads it (the s_nop).
__device__ __forceinline__ void dma16_lds(const Buf& b, void* lds, uint32_t voff, uint32_t soff) {
    typedef __attribute__((address_space(3))) void lds_t;
    const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_t*)lds);
    const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane((int)soff);
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(b.d), "s"(so), "s"(m)
                 : "m0");
}

// s_barrier, then a compiler fence: the DMA loads above are invisible to the
// compiler as LDS writes, so without the fence it may hoist LDS reads of the
// next stage above the barrier that makes that stage's data visible.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <sp24_dtype DT>
struct SparseOp;

template <>
struct SparseOp<SP24_BF16> {
    static constexpr int KSTEP = 64;        // dense K per instruction
    static constexpr int ELEM = 2;          // bytes per element
    __device__ static __forceinline__ f32x4 mma(uint4 a, uint4 b0, uint4 b1, uint32_t idx, f32x4 c) {
        bf16x8 av = __builtin_bit_cast(bf16x8, a);
        struct { uint4 x, y; } bb = {b0, b1};
        bf16x16 bv = __builtin_bit_cast(bf16x16, bb);
        return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(av, bv, c, (int)idx, 0, 0);
    }
};

template <>
struct SparseOp<SP24_F16> {
    static constexpr int KSTEP = 64;
    static constexpr int ELEM = 2;
    __device__ static __forceinline__ f32x4 mma(uint4 a, uint4 b0, uint4 b1, uint32_t idx, f32x4 c) {
        f16x8 av = __builtin_bit_cast(f16x8, a);
        struct { uint4 x, y; } bb = {b0, b1};
        f16x16 bv = __builtin_bit_cast(f16x16, bb);
        return __builtin_amdgcn_smfmac_f32_16x16x64_f16(av, bv, c, (int)idx, 0, 0);
    }
};

template <>
struct SparseOp<SP24_E4M3> {
    static constexpr int KSTEP = 128;
    static constexpr int ELEM = 1;
    __device__ static __forceinline__ f32x4 mma(uint4 a, uint4 b0, uint4 b1, uint32_t idx, f32x4 c) {
        i32x4 av = __builtin_bit_cast(i32x4, a);
        struct { uint4 x, y; } bb = {b0, b1};
        i32x8 bv = __builtin_bit_cast(i32x8, bb);
        return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(av, bv, c, (int)idx, 0, 0);
    }
};

// The int8 form: the same operand layout as fp8, int32 accumulation.  The
// accumulator registers hold the int32 bits (exact: at most K * 128 * 127 in
// magnitude); acc_to_f32 converts them once, after the K loop.
template <>
struct SparseOp<SP24_I8> {
    static constexpr int KSTEP = 128;
    static constexpr int ELEM = 1;
    __device__ static __forceinline__ f32x4 mma(uint4 a, uint4 b0, uint4 b1, uint32_t idx, f32x4 c) {
        i32x4 av = __builtin_bit_cast(i32x4, a);
        struct { uint4 x, y; } bb = {b0, b1};
        i32x8 bv = __builtin_bit_cast(i32x8, bb);
        i32x4 ci = __builtin_bit_cast(i32x4, c);
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_smfmac_i32_16x16x128_i8(av, bv, ci, (int)idx, 0, 0));
    }
};

// Accumulators as fp32 values: int8 accumulates int32 bits in the same
// registers, every other input dtype fp32 already.
template <sp24_dtype DT>
__device__ __forceinline__ f32x4 acc_to_f32(f32x4 v) {
    if constexpr (DT == SP24_I8)
        return __builtin_convertvector(__builtin_bit_cast(i32x4, v), f32x4);
    return v;
}
template <sp24_dtype DT>
__device__ __forceinline__ f32x16 acc_to_f32(f32x16 v) {
    typedef __attribute__((ext_vector_type(16))) int i32x16;
    if constexpr (DT == SP24_I8)
        return __builtin_convertvector(__builtin_bit_cast(i32x16, v), f32x16);
    return v;
}

// Byte offsets, within one step of one row, of what lane group kg loads.
//   A values: 16 bytes at a_off(kg) of the row's compressed step (KSTEP/2 values)
//   B: 16 bytes at b_off0(kg) and 16 at b_off1(kg) of the row's dense step
template <sp24_dtype DT>
struct StepLayout {
    static constexpr int KSTEP = SparseOp<DT>::KSTEP;
    static constexpr int ELEM = SparseOp<DT>::ELEM;
    static constexpr int A_STEP_BYTES = KSTEP / 2 * ELEM;     // 64 B
    static constexpr int B_STEP_BYTES = KSTEP * ELEM;         // 128 B
    static constexpr int META_WORDS = KSTEP / 32;             // 2 or 4 words per step
    __device__ static __forceinline__ int a_off(int kg) { return 16 * kg; }
    __device__ static __forceinline__ int b_off0(int kg) { return 16 * kg; }
    __device__ static __forceinline__ int b_off1(int kg) { return B_STEP_BYTES / 2 + 16 * kg; }
    // metadata word of this step used by lane group kg, and the shift to
    // bring its 16 (or 32) bits to the bottom
    __device__ static __forceinline__ int meta_word(int kg) { return ELEM == 2 ? kg >> 1 : kg; }
    __device__ static __forceinline__ int meta_shift(int kg) { return ELEM == 2 ? 16 * (kg & 1) : 0; }
};

// fp32 -> output element, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);     // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
    _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
}

template <sp24_dtype OUT>
__device__ __forceinline__ void store_out(void* Y, int64_t off, float v) {
    if constexpr (OUT == SP24_F32)
        reinterpret_cast<float*>(Y)[off] = v;
    else if constexpr (OUT == SP24_BF16)
        reinterpret_cast<uint16_t*>(Y)[off] = f32_to_bf16_rne(v);
    else
        reinterpret_cast<uint16_t*>(Y)[off] = f32_to_f16_rne(v);
}

// 16 bytes written with the non-temporal hint (output the kernel never reads back).
__device__ __forceinline__ void store_stream(void* p, uint4 d) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, d), reinterpret_cast<u32x4*>(p));
}

// Four consecutive outputs (offset off .. off+3), vectorized when aligned.
template <sp24_dtype OUT>
__device__ __forceinline__ void store_out4(void* Y, int64_t off, f32x4 v) {
    if constexpr (OUT == SP24_F32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(Y) + off) = v;
    } else {
        uint16_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            h[i] = OUT == SP24_BF16 ? f32_to_bf16_rne(v[i]) : f32_to_f16_rne(v[i]);
        uint2 p = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(Y) + off) = p;
    }
}

}  // namespace sp24
