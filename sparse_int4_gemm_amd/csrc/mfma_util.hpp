// gfx950 matrix-core helpers shared by the slim_linear kernel families.
//
// Lane layouts (wave64; measured on gfx950 with an in-bounds probe):
//  v_mfma_f32_16x16x32_f16   A: lane l holds row l%16, k = 8*(l/16) + [0,8)
//                            B: lane l holds col l%16, k = 8*(l/16) + [0,8)
//                            D: lane l holds col l%16, rows 4*(l/16) + [0,4)
//  v_smfmac_f32_16x16x64_f16 A (2:4 compressed): lane l holds row l%16 and the
//                            8 kept values of dense k = 16*(l/16) + [0,16)
//                            (4 groups of 4, two kept values each, in group
//                            order), their 2-bit positions in a 16-bit field of
//                            the index VGPR selected by abid;
//                            B: lane l holds col l%16, k = 8*(l/16) + [0,8)
//                            in elements 0..7 and k = 32 + 8*(l/16) + [0,8)
//                            in elements 8..15;
//                            D: as the dense 16x16 layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace slim {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16 __attribute__((ext_vector_type(16)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Dequantise one packed values word: 8 kept int4 codes of 4 groups (bits
// [4j,4j+4) = lower-index value of group j, bits [16+4j,..) = higher-index
// value) times the group scale, in smfmac A order (lo0, hi0, lo1, hi1, ...).
// Each fp16 pair is built as 1024 + (q + 8) with an exact fp16 subtraction of
// 1032, then one fp16 multiply by the scale (the only rounding).
__device__ __forceinline__ h8 dequant_word(uint32_t w, h2 s2) {
    const uint32_t u = w ^ 0x88888888u;              // two's complement nibble -> q + 8
    const uint32_t d0 = (u & 0x000F000Fu) | 0x64006400u;
    const uint32_t d1 = ((u >> 4) & 0x000F000Fu) | 0x64006400u;
    const uint32_t d2 = ((u >> 8) & 0x000F000Fu) | 0x64006400u;
    const uint32_t d3 = ((u >> 12) & 0x000F000Fu) | 0x64006400u;
    const h2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 p0 = (__builtin_bit_cast(h2, d0) - bias) * s2;
    const h2 p1 = (__builtin_bit_cast(h2, d1) - bias) * s2;
    const h2 p2 = (__builtin_bit_cast(h2, d2) - bias) * s2;
    const h2 p3 = (__builtin_bit_cast(h2, d3) - bias) * s2;
    h8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// One int4 values word -> 8 fp16 weights in smfmac A order (lo0, hi0, lo1, hi1,
// ...).  Nibbles 0 and 2 of each half become 1024 + (q + 8), nibbles 1 and 3
// 64 + (q + 8) (the nibble lands in mantissa bits 4..7 under exponent 6), so
// only one shift is needed; the subtraction is exact and the scale multiply is
// the only rounding.
__device__ __forceinline__ void dequant_word_fast(uint32_t w, h2 s2, h8& out) {
    const uint32_t lo = ((w ^ 0x00080008u) & 0x000F000Fu) | 0x64006400u;
    const uint32_t hi = ((w ^ 0x00800080u) & 0x00F000F0u) | 0x54005400u;
    const uint32_t w8 = w >> 8;
    const uint32_t lo2 = ((w8 ^ 0x00080008u) & 0x000F000Fu) | 0x64006400u;
    const uint32_t hi2 = ((w8 ^ 0x00800080u) & 0x00F000F0u) | 0x54005400u;
    const h2 b0 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 b1 = {(_Float16)72.0f, (_Float16)72.0f};
    const h2 p0 = (__builtin_bit_cast(h2, lo) - b0) * s2;
    const h2 p1 = (__builtin_bit_cast(h2, hi) - b1) * s2;
    const h2 p2 = (__builtin_bit_cast(h2, lo2) - b0) * s2;
    const h2 p3 = (__builtin_bit_cast(h2, hi2) - b1) * s2;
    out[0] = p0[0]; out[1] = p0[1]; out[2] = p1[0]; out[3] = p1[1];
    out[4] = p2[0]; out[5] = p2[1]; out[6] = p3[0]; out[7] = p3[1];
}

__device__ __forceinline__ h16 concat8(h8 a, h8 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
}

template <int ABID>
__device__ __forceinline__ f4 smfmac(h8 a, h16 b, f4 c, uint32_t idx) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, b, c, (int)idx, 0, ABID);
}

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h8 load_h8(const uint16_t* p) {
    return *reinterpret_cast<const h8*>(p);
}

// Raw buffer resource over [base, base + bytes): loads at a byte offset at or
// past `bytes` return zero without touching memory (no partial loads occur
// when offsets and sizes are multiples of the load width).  Word 3 is the
// gfx9-family raw-buffer format.
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr int kOOB = 0x7FFFFFF0;                 // an offset past every buffer made here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int n = bytes <= 0 ? 0 : (bytes > kOOB ? kOOB : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, (int)kRsrcWord3);
}

__device__ __forceinline__ h8 buffer_load_h8(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// Direct-to-LDS 16-byte load per lane (buffer_load_dwordx4 ... lds): lane l's
// 16 bytes from rsrc at voff + soff land at LDS byte lds + 16 l (lanes whose
// offset is past the buffer write zero; lanes masked off write nothing).
// Written as asm: the compiler cannot tell which LDS bytes such a load writes
// and would wait for every load in flight before any LDS read; callers order
// them with wait_vmem_below.  No register outputs.
__device__ __forceinline__ void lds_load16(u4 rsrc, const unsigned char* lds, int voff, int soff) {
    const uint32_t l = (uint32_t)(size_t)(const __attribute__((address_space(3))) unsigned char*)lds;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(l)), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// LDS byte addresses as 32-bit integers: the address of a __shared__ object,
// a load at an address, and the direct-to-LDS load of lds_load16 at an
// address (uniform).  Adding compile-time constants to such an address lets
// the compiler use the 16-bit offset field of the LDS instructions.
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) unsigned char*)p;
}
template <class T>
__device__ __forceinline__ T lds_ld(uint32_t a) {
    return *(const __attribute__((address_space(3))) T*)(size_t)a;
}
__device__ __forceinline__ void lds_load16_at(u4 rsrc, uint32_t lds, int voff, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// Raw buffer descriptor words (gfx9 family) over [base, base + bytes); see make_rsrc.
__device__ __forceinline__ u4 rsrc_words(const void* base, int64_t bytes) {
    const uint64_t p = (uint64_t)base;
    const uint32_t n = bytes <= 0 ? 0u : (bytes > kOOB ? (uint32_t)kOOB : (uint32_t)bytes);
    return u4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p),
              (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32)),
              (uint32_t)__builtin_amdgcn_readfirstlane((int)n), kRsrcWord3};
}

// Wait until at most N vector-memory loads of this wave are in flight
// (vmcnt(N): bits 3..0 and 15..14 of the count; expcnt and lgkmcnt left free).
template <int N>
__device__ __forceinline__ void wait_vmem_below() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Sum of v over the 64 lanes of the wave, complete in lanes 48..63 (DPP
// steps, no LDS): partners lane^1 and lane^2 (quad permutes), then the
// mirrored half row and row (8, then 16 lanes), then rows 1 and 3 add the
// last lane of the row below (row_bcast:15) and rows 2 and 3 add lane 31
// (row_bcast:31).  Rows not enabled by a step's row mask receive 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xF, false);
    return x + __builtin_bit_cast(float, t);
}

__device__ __forceinline__ float wave_sum_hi(float v) {
    v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_add<0x140, 0xF>(v);  // row_mirror
    v = dpp_add<0x142, 0xA>(v);  // row_bcast:15
    v = dpp_add<0x143, 0xC>(v);  // row_bcast:31
    return v;
}

// XCD-aware block order: workgroup i runs on XCD i % 8; give each XCD a
// contiguous range of logical blocks so neighbouring tiles share its L2.
__device__ __forceinline__ int xcd_remap(int i, int nblocks) {
    const int x = i & 7, local = i >> 3;
    const int q = nblocks >> 3, rem = nblocks & 7;
    return x * q + (x < rem ? x : rem) + local;
}

}  // namespace slim
