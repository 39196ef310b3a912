// Quantised low-rank adapters ("Quantized SLiM": the thesis' Tables E.13 and
// E.14 quantise the adapters as well; the pages give no adapter quantiser,
// so the one of W is used, without pruning).
//
// A factor is stored output-major (rows: outputs of the product it feeds,
// columns: its reduction dimension): Lt = L^T [r][K] in groups of 128 along
// K, Rt = R^T [N][r] in groups of 32 along r.  Codes are symmetric int4,
// s16 = fp16(absmax / 7), q = clamp(rint(w / s16), -7, 7) (fp32 division,
// half to even; q = 0 where s16 = 0).  Packing: per row, per 8 consecutive
// elements one little-endian uint32 in which element e sits in nibble
// (0, 4, 1, 5, 2, 6, 3, 7)[e], so that the in-register int4 -> fp16 step of
// the decode kernels yields the 8 elements in order.  Scales fp16 [rows][cols
// / group], row-major.
//
// adapter_pack_kernel<RUNS>: one lane per 8-element run (RUNS = group / 8
//   consecutive lanes form a group and reduce its absmax with shuffles).
// adapter_dequant_kernel: q * s16 in fp16 (one rounding), one lane per run,
//   16-byte stores, both factors in one launch; used by the shapes whose
//   kernels read fp16 adapters.
#include "internal.hpp"

namespace slim {
namespace {

constexpr int kNibPos[8] = {0, 4, 1, 5, 2, 6, 3, 7};

template <int RUNS>
__global__ __launch_bounds__(256) void adapter_pack_kernel(const float* __restrict__ A, int64_t rows, int64_t cols,
                                                           uint32_t* __restrict__ q, uint16_t* __restrict__ scales) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t runs = rows * (cols / 8);
    const bool live = t < runs;
    float w[8];
    if (live) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4* src = reinterpret_cast<const f32x4*>(A) + t * 2;
        const f32x4 a = __builtin_nontemporal_load(src), b = __builtin_nontemporal_load(src + 1);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(w[i]));
#pragma unroll
    for (int d = 1; d < RUNS; d <<= 1) m = fmaxf(m, __shfl_xor(m, d));
    const _Float16 s16 = (_Float16)(m / 7.0f);             // fp32 division, round to nearest even
    const float sf = (float)s16;
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        int c = 0;
        if (sf > 0.0f) c = (int)fminf(fmaxf(rintf(w[e] / sf), -7.0f), 7.0f);
        word |= ((uint32_t)c & 0xFu) << (4 * kNibPos[e]);
    }
    if (live) {
        q[t] = word;
        if ((t & (RUNS - 1)) == 0) scales[t / RUNS] = __builtin_bit_cast(uint16_t, s16);
    }
}

// Two factors in one launch: workgroups [0, nb0) take factor 0, the rest factor 1.
struct DequantJob {
    const uint32_t* q;
    const uint16_t* scales;
    int64_t runs;
    int runs_per_group;
    uint16_t* out;
};

__global__ __launch_bounds__(256) void adapter_dequant_kernel(DequantJob j0, DequantJob j1, unsigned nb0) {
    const bool second = blockIdx.x >= nb0;              // uniform
    const uint32_t* __restrict__ q = second ? j1.q : j0.q;
    const uint16_t* __restrict__ scales = second ? j1.scales : j0.scales;
    const int runs_per_group = second ? j1.runs_per_group : j0.runs_per_group;
    uint16_t* __restrict__ out = second ? j1.out : j0.out;
    const int64_t t = (int64_t)(second ? blockIdx.x - nb0 : blockIdx.x) * 256 + threadIdx.x;
    if (t >= (second ? j1.runs : j0.runs)) return;
    const uint32_t w = q[t];
    const _Float16 s = __builtin_bit_cast(_Float16, scales[t / runs_per_group]);
    _Float16 v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int nib = (int)((w >> (4 * kNibPos[e])) & 0xFu);
        v[e] = (_Float16)(nib >= 8 ? nib - 16 : nib) * s;
    }
    typedef _Float16 h8v __attribute__((ext_vector_type(8)));
    const h8v o = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
    *reinterpret_cast<h8v*>(out + 8 * t) = o;
}

}  // namespace

hipError_t launch_adapter_pack(const float* A, int64_t rows, int64_t cols, int64_t group, uint8_t* q,
                               uint16_t* scales, hipStream_t stream) {
    const int64_t runs = rows * (cols / 8);
    const unsigned grid = (unsigned)((runs + 255) / 256);
    uint32_t* qw = reinterpret_cast<uint32_t*>(q);
    if (group == 32)
        hipLaunchKernelGGL(adapter_pack_kernel<4>, dim3(grid), dim3(256), 0, stream, A, rows, cols, qw, scales);
    else
        hipLaunchKernelGGL(adapter_pack_kernel<16>, dim3(grid), dim3(256), 0, stream, A, rows, cols, qw, scales);
    return hipGetLastError();
}

hipError_t launch_adapter_dequant2(const uint8_t* q0, const uint16_t* s0, int64_t rows0, int64_t cols0, int64_t group0,
                                   uint16_t* out0, const uint8_t* q1, const uint16_t* s1, int64_t rows1, int64_t cols1,
                                   int64_t group1, uint16_t* out1, hipStream_t stream) {
    const DequantJob j0{reinterpret_cast<const uint32_t*>(q0), s0, rows0 * (cols0 / 8), (int)(group0 / 8), out0};
    const DequantJob j1{reinterpret_cast<const uint32_t*>(q1), s1, rows1 * (cols1 / 8), (int)(group1 / 8), out1};
    const unsigned nb0 = (unsigned)((j0.runs + 255) / 256), nb1 = (unsigned)((j1.runs + 255) / 256);
    if (nb0 + nb1 == 0) return hipSuccess;
    hipLaunchKernelGGL(adapter_dequant_kernel, dim3(nb0 + nb1), dim3(256), 0, stream, j0, j1, nb0);
    return hipGetLastError();
}

}  // namespace slim
