// One-shot quantise -> 2:4 prune -> pack of a fp32 weight W [N][K].
//
// Method: Compression Trinity thesis, Fig. 7.1 caption (quantise W
// symmetrically, then sparsify the quantised weights), §1.2.2 (per-group
// quantisation) and §2.2.3 "Sparse Tensor Core Acceleration" (2:4 along the
// reduction dimension, kept values stored packed next to position indices);
// group size 128 from the developinglight.com summary of the thesis.
//
// Layout of the work: the packed format has one 32-bit values word and one
// 16-bit metadata half-word per 16 consecutive k of a row, and K is a multiple
// of 128.  Lane t reads floats [16t, 16t+16) of W flattened row-major (the
// 16-k block t % (K/16) of row t / (K/16)); eight consecutive lanes form one
// 128-wide group and reduce its absmax with cross-lane shuffles.  Outputs go
// to the memory order of the format: rows in blocks of 16 (the last block
// holds N mod 16 rows if that is not 0), inside a block group by group,
// inside a group row by row, so the eight lanes of a group write 32
// contiguous bytes of values and 16 of metadata, and one scale.  The kernel is
// HBM-bound on reading W (4 B read, 25/64 B written per weight); no LDS.
#include "internal.hpp"

namespace slim {
namespace {

__device__ inline int quantize_one(float w, float s) {
    // fp32 division (correctly rounded: this file is built without fast-math),
    // round half to even, clamp to the symmetric int4 range.
    float t = rintf(w / s);
    t = fminf(fmaxf(t, -7.0f), 7.0f);
    return (int)t;
}

// HYBRID: dense / 2:4 tiles (flags int32 [ceil(N/16)][K/128], nonzero = dense): a dense
// tile keeps every code, the pair at positions 0, 1 of each group of 4 in
// `values` (metadata 0, 1) and the pair at positions 2, 3 in `dvalues`; a 2:4
// tile is pruned as usual and its dvalues word is 0.
template <bool HYBRID>
__global__ __launch_bounds__(256) void pack_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                   uint32_t* __restrict__ values,
                                                   uint16_t* __restrict__ meta,
                                                   uint16_t* __restrict__ scales,
                                                   const int32_t* __restrict__ flags,
                                                   uint32_t* __restrict__ dvalues) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t KB = K / 16;                   // 16-k blocks per row
    const bool live = t < N * KB;

    float w[16];
    if (live) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4* src = reinterpret_cast<const f32x4*>(W) + t * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 v = __builtin_nontemporal_load(src + i);
            w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) w[i] = 0.0f;
    }

    // absmax of the 128-group: 16 values here, then across the 8 lanes.
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(w[i]));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));

    const float s32 = a / 7.0f;
    const _Float16 s16 = (_Float16)s32;          // round to nearest even
    const float sf = (float)s16;

    int q[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = (sf > 0.0f) ? quantize_one(w[i], sf) : 0;

    uint32_t word = 0;
    uint32_t half = 0;
    uint32_t dword = 0;
    bool dense = false;
    if constexpr (HYBRID) {
        if (live) {
            const int64_t n = t / KB, kb = t - n * KB;
            dense = flags[(n >> 4) * (K / 128) + (kb >> 3)] != 0;
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // Rank key: larger |q| first, then lower index; keys are distinct.
        int key[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int m = q[4 * j + i] < 0 ? -q[4 * j + i] : q[4 * j + i];
            key[i] = (m << 2) | (3 - i);
        }
        int lo = -1, hi = -1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int beaten = 0;
#pragma unroll
            for (int o = 0; o < 4; ++o) beaten += (o != i) && (key[o] > key[i]);
            const bool keep = beaten < 2;
            if (keep && lo < 0) lo = i;
            else if (keep) hi = i;
        }
        if (HYBRID && dense) {
            lo = 0;
            hi = 1;
            dword |= ((uint32_t)q[4 * j + 2] & 0xFu) << (4 * j);
            dword |= ((uint32_t)q[4 * j + 3] & 0xFu) << (16 + 4 * j);
        }
        const uint32_t nlo = (uint32_t)q[4 * j + lo] & 0xFu;
        const uint32_t nhi = (uint32_t)q[4 * j + hi] & 0xFu;
        word |= nlo << (4 * j);
        word |= nhi << (16 + 4 * j);
        half |= ((uint32_t)lo | ((uint32_t)hi << 2)) << (4 * j);
    }

    if (live) {
        const int64_t n = t / KB, kb = t - n * KB;
        const int64_t gb = n >> 4, ri = n & 15;
        const int64_t RB = N - 16 * gb < 16 ? N - 16 * gb : 16;     // rows in this block
        const int64_t pc = kb >> 3, j = kb & 7;                     // 128-k group, 16-k block in it
        const int64_t o = gb * 16 * KB + (pc * RB + ri) * 8 + j;    // word / half-word index
        values[o] = word;
        meta[o] = (uint16_t)half;
        if constexpr (HYBRID) dvalues[o] = dword;
        if (j == 0) scales[gb * 16 * (K / 128) + pc * RB + ri] = __builtin_bit_cast(uint16_t, s16);
    }
}

}  // namespace

hipError_t launch_pack(const float* W, int64_t N, int64_t K, uint8_t* values, uint8_t* meta,
                       uint16_t* scales, hipStream_t stream) {
    const int64_t nblocks = N * (K / 16);
    const int64_t grid = (nblocks + 255) / 256;
    hipLaunchKernelGGL(pack_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, W, N, K,
                       reinterpret_cast<uint32_t*>(values), reinterpret_cast<uint16_t*>(meta),
                       scales, nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_pack_hybrid(const float* W, int64_t N, int64_t K, const int32_t* flags, uint8_t* values,
                              uint8_t* meta, uint16_t* scales, uint8_t* dvalues, hipStream_t stream) {
    const int64_t nblocks = N * (K / 16);
    const int64_t grid = (nblocks + 255) / 256;
    hipLaunchKernelGGL(pack_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, W, N, K,
                       reinterpret_cast<uint32_t*>(values), reinterpret_cast<uint16_t*>(meta),
                       scales, flags, reinterpret_cast<uint32_t*>(dvalues));
    return hipGetLastError();
}

}  // namespace slim
