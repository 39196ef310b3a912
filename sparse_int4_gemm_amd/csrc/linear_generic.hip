// Generic slim_linear kernels: one thread per output element, fp32
// accumulation.  Correct for every legal shape; used where no tuned kernel
// family fits the shape.
//
//   T[m][j] = sum_k X[m][k] L[k][j]                         (adapter down)
//   Y[m][n] = sum_k X[m][k] q[n][k] s[n][k/128] + sum_j T[m][j] R[j][n]
// with the adapter stored output-major: Lt = L^T [r][K], Rt = R^T [N][r].
//
// Layer definition: Compression Trinity thesis §2.1 (Y = X W^T) and the Ch. 4
// introduction (sparse weights and the dense adapter as parallel paths).
#include "internal.hpp"

namespace slim {
namespace {

__device__ inline float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__global__ __launch_bounds__(256) void adapter_down_generic(LinearArgs a, float* __restrict__ T) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t m = blockIdx.y;
    const int64_t b = blockIdx.z;
    if (j >= a.r) return;
    const uint16_t* X = a.X + b * a.sX + m * a.K;
    const uint16_t* Lt = a.Lt + b * a.sLt + j * a.K;
    float acc = 0.0f;
    for (int64_t k = 0; k < a.K; ++k) acc = fmaf(h2f(X[k]), h2f(Lt[k]), acc);
    float* Tb = reinterpret_cast<float*>(a.ws + b * a.ws_per_problem + kCounterRegion);
    Tb[m * a.r + j] = acc;
}

__global__ __launch_bounds__(256) void main_generic(LinearArgs a) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t m = blockIdx.y;
    const int64_t b = blockIdx.z;
    if (n >= a.N) return;
    const uint16_t* X = a.X + b * a.sX + m * a.K;
    // Packed format in 16-row blocks, group by group (N is a multiple of 16):
    // row n's 8 words (half-words) of group g at (16 (n / 16) (K/128) + 16 g
    // + n % 16) * 8, its scale at 16 (n / 16) (K/128) + 16 g + n % 16.
    const int64_t rb = 16 * (n >> 4) * (a.K / kGroup), ri = n & 15;
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(a.values + b * a.sV);
    const uint16_t* mh = reinterpret_cast<const uint16_t*>(a.meta + b * a.sMeta);
    const uint16_t* sc = a.scales + b * a.sS;
    // Hybrid dense / 2:4 tiles: a dense tile's second pair of codes sits at
    // positions 2 and 3 of every group of 4, in dvalues (same arrangement).
    const uint32_t* dw = a.dvalues ? reinterpret_cast<const uint32_t*>(a.dvalues) : nullptr;
    const int32_t* fl = a.dflags ? reinterpret_cast<const int32_t*>(a.dflags) : nullptr;
    float acc = 0.0f;
    for (int64_t g = 0; g < a.K / kGroup; ++g) {
        float part = 0.0f;
        const int64_t rg = rb + 16 * g + ri;
        const bool dense = dw && fl[(n >> 4) * (a.K / kGroup) + g] != 0;
        for (int blk = 0; blk < kGroup / 16; ++blk) {
            const int64_t bi = g * (kGroup / 16) + blk;
            const uint32_t word = vw[rg * 8 + blk];
            const uint32_t half = mh[rg * 8 + blk];
            const uint32_t word2 = dense ? dw[rg * 8 + blk] : 0u;
            for (int j = 0; j < 4; ++j) {
                for (int h = 0; h < 2; ++h) {
                    int nib = (int)((word >> (16 * h + 4 * j)) & 0xFu);
                    int q = nib >= 8 ? nib - 16 : nib;
                    int pos = (int)((half >> (4 * j + 2 * h)) & 0x3u);
                    part = fmaf(h2f(X[bi * 16 + 4 * j + pos]), (float)q, part);
                    int nib2 = (int)((word2 >> (16 * h + 4 * j)) & 0xFu);
                    int q2 = nib2 >= 8 ? nib2 - 16 : nib2;
                    part = fmaf(h2f(X[bi * 16 + 4 * j + 2 + h]), (float)q2, part);
                }
            }
        }
        acc = fmaf(part, h2f(sc[rg]), acc);
    }
    if (a.r > 0) {
        const float* T = reinterpret_cast<const float*>(a.ws + b * a.ws_per_problem + kCounterRegion) + m * a.r;
        const uint16_t* Rt = a.Rt + b * a.sRt + n * a.r;
        for (int64_t j = 0; j < a.r; ++j) acc = fmaf(T[j], h2f(Rt[j]), acc);
    }
    a.Y[b * a.sY + m * a.N + n] = __builtin_bit_cast(uint16_t, (_Float16)acc);
}

}  // namespace

hipError_t launch_linear_generic(const LinearArgs& a, hipStream_t stream) {
    if (a.r > 0) {
        dim3 grid((unsigned)((a.r + 255) / 256), (unsigned)a.M, (unsigned)a.batch);
        hipLaunchKernelGGL(adapter_down_generic, grid, dim3(256), 0, stream, a, nullptr);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dim3 grid((unsigned)((a.N + 255) / 256), (unsigned)a.M, (unsigned)a.batch);
    hipLaunchKernelGGL(main_generic, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace slim
