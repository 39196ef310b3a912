// slim_linear for decode-shaped problems (M <= 16 tokens): HBM-bound.
//
//   T = X . L                                   (adapter down, dense MFMA)
//   Y = X . deq(W_c)^T + T . R                  (2:4 sparse MFMA + dense MFMA)
//
// Layer: Compression Trinity thesis §2.1 (Y = X W^T) with the sparse weight
// and the low-rank adapter as parallel paths (Ch. 4 introduction); decode is
// the memory-bound regime (§2.5.2), so both kernels are built to read every
// HBM byte once with wide coalesced loads.
//
// adapter_partial_kernel: grid = (r/32 column chunks) x S splits of K.  A
//   workgroup multiplies X[:, k-range] by L[k-range, 32 columns] with
//   v_mfma_f32_16x16x32_f16 (tokens are the MFMA N side, zero-padded to 16),
//   reduces its 4 waves in LDS and writes an fp32 partial to the workspace.
// adapter_reduce_kernel: T = sum of the S partials in a fixed order
//   (deterministic, no atomics), stored in fp16.
// decode_main_kernel: one workgroup of 16 waves per 16 rows of W (XCD-aware
//   order).  The waves split K into 256-wide chunks; per chunk and lane: 16 B
//   of packed values, 8 B of metadata and one scale of its row, and 2 x 4 x
//   16 B of X.  Each 64-k step dequantises one values word in registers and
//   issues one v_smfmac_f32_16x16x64_f16 (W rows are the sparse A side,
//   tokens the B side).  The epilogue adds T . R with dense MFMA into the
//   same accumulators (one 32-wide slice of r per wave), reduces the waves in
//   LDS and stores fp16 Y.
// All loads are unconditional (clamped addresses, values masked after the
// load) so that every wave has its whole share of HBM traffic in flight
// before it first waits.
#include "internal.hpp"
#include "mfma_util.hpp"

namespace slim {
namespace {

constexpr int kDecodeMaxM = 16;

struct DecodeWs {
    size_t t_off, p_off, total;
    int splits;
};

__host__ __device__ inline int decode_splits(int64_t K) {
    const int64_t steps = K / 32;
    return (int)(steps < 16 ? steps : 16);
}

DecodeWs decode_ws_layout(int64_t N, int64_t K, int64_t r) {
    (void)N;
    DecodeWs w;
    w.splits = decode_splits(K);
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    w.t_off = kCounterRegion;   // up to 256 column-chunk tickets before it
    w.p_off = w.t_off + al((size_t)kDecodeMaxM * (size_t)r * 2);
    w.total = w.p_off + al((size_t)w.splits * kDecodeMaxM * (size_t)r * sizeof(float));
    return w;
}

// ----------------------------------------------------------------- T = X L
// Partial T over one K split for 32 columns: P[s][m][c*32 + j] (fp32).
// Every load is unconditional (clamped address, value masked afterwards), and
// a wave issues the loads of U steps before its first MFMA.
template <int U>
__global__ __launch_bounds__(256) void adapter_partial_kernel(LinearArgs a, int splits, size_t p_off) {
    const int b = blockIdx.y;
    const int nR = (int)(a.r / 32);
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int c = logical % nR;                // 32-column chunk of T
    const int s = logical / nR;                // K split
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int jl = lane & 15, G = lane >> 4;
    const int m = jl;                          // token column of the B operand
    const bool mval = m < a.M;
    const int64_t K = a.K, r = a.r;

    const uint16_t* X = a.X + b * a.sX + (int64_t)(mval ? m : 0) * K;
    const uint16_t* L = a.L + b * a.sL + 32 * c + jl;

    const int nsteps = (int)(K / 32);
    const int st0 = (int)((int64_t)s * nsteps / splits);
    const int st1 = (int)((int64_t)(s + 1) * nsteps / splits);

    f4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
    for (int base = st0 + wave; base < st1; base += 4 * U) {
        h8 xb[U], l0[U], l1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int st = base + 4 * u;
            const int sc = st < st1 ? st : st0;                 // clamp: always a valid row
            const int64_t k0 = (int64_t)sc * 32 + 8 * G;
            xb[u] = load_h8(X + k0);
            const uint16_t* lp = L + k0 * r;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                l0[u][e] = __builtin_bit_cast(_Float16, lp[e * r]);
                l1[u][e] = __builtin_bit_cast(_Float16, lp[e * r + 16]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool live = mval && (base + 4 * u < st1);
            const h8 xv = live ? xb[u] : h8{};
            acc0 = mfma16(l0[u], xv, acc0);    // rows j = 4G+v of the chunk, col m
            acc1 = mfma16(l1[u], xv, acc1);    // rows j = 16+4G+v
        }
    }

    __shared__ f4 red[4][2][64];
    red[wave][0][lane] = acc0;
    red[wave][1][lane] = acc1;
    __syncthreads();
    float* P = reinterpret_cast<float*>(a.ws + b * a.ws_per_problem + p_off) +
               (size_t)s * kDecodeMaxM * r;                     // [m 16][r]
    const int half = threadIdx.x >> 7;
    const int ln = (threadIdx.x >> 1) & 63;
    const int v0 = (threadIdx.x & 1) * 2;
    const f4 sum = red[0][half][ln] + red[1][half][ln] + red[2][half][ln] + red[3][half][ln];
    const int mm = ln & 15;
    const int j = 32 * c + 16 * half + 4 * (ln >> 4) + v0;
    P[(int64_t)mm * r + j] = sum[v0];
    P[(int64_t)mm * r + j + 1] = sum[v0 + 1];
}

// T[m][j] = sum over splits of P[s][m][j], fixed order, stored as fp16.
__global__ __launch_bounds__(256) void adapter_reduce_kernel(LinearArgs a, int splits, size_t t_off,
                                                             size_t p_off) {
    const int b = blockIdx.y;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;     // over M*r
    const int64_t total = a.M * a.r;
    const int64_t ec = e < total ? e : 0;
    const float* P = reinterpret_cast<const float*>(a.ws + b * a.ws_per_problem + p_off);
    const int64_t stride = (int64_t)kDecodeMaxM * a.r;
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = P[(q < splits ? q : 0) * stride + ec];
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q) sum += (q < splits) ? v[q] : 0.0f;
    if (e < total) reinterpret_cast<_Float16*>(a.ws + b * a.ws_per_problem + t_off)[e] = (_Float16)sum;
}

// ------------------------------------------------- Y = X deq(W)^T + T R
// Template parameters: NW waves per workgroup, CPW 256-k chunk slots per wave
// (wave w owns chunks w, w+NW, ...), ADAPTER = (r > 0).
template <int NW, int CPW, bool ADAPTER>
__global__ __launch_bounds__(64 * NW) void decode_main_kernel(LinearArgs a, size_t t_off) {
    const int b = blockIdx.y;
    const int nb = xcd_remap(blockIdx.x, gridDim.x);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nl = lane & 15, G = lane >> 4;
    const int64_t K = a.K, N = a.N;
    const int64_t n0 = (int64_t)nb * 16;
    const int Kb = (int)(K / 16);                         // 16-k blocks per row
    const int nch = (int)((K + 255) / 256);               // 256-k chunks (last may be half)

    const uint8_t* vrow = a.values + b * a.sV + (n0 + nl) * (K / 4);
    const uint8_t* mrow = a.meta + b * a.sMeta + (n0 + nl) * (K / 8);
    const uint16_t* srow = a.scales + b * a.sS + (n0 + nl) * (K / kGroup);
    const int m = nl;
    const bool mval = m < a.M;
    const uint16_t* xrow = a.X + b * a.sX + (int64_t)(mval ? m : 0) * K;
    const int gA1 = G >> 1, gA2 = 2 + (G >> 1), hoff = 8 * (G & 1);

    // X operand of one chunk slot: L2-resident, 8 x 16 B per lane; an
    // invalid part reads the row start and is masked at use.
    auto load_x = [&](int i, h8* x1, h8* x2) {
        const int c = wave + NW * i;
        const bool b1 = c < nch && 16 * c + 4 * gA1 < Kb;
        const bool b2 = c < nch && 16 * c + 4 * gA2 < Kb;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            x1[t] = load_h8(xrow + (b1 ? 16 * (16 * c + 4 * gA1 + t) + hoff : 0));
            x2[t] = load_h8(xrow + (b2 ? 16 * (16 * c + 4 * gA2 + t) + hoff : 0));
        }
    };
    h8 xa[4], xb[4], xc[4], xd[4];
    load_x(0, xa, xb);

    // 1. All packed-W loads of this wave (the HBM stream), unconditional:
    //    an invalid slot reads the row's first block and is masked later.
    u4 vw[CPW];
    u2 mw[CPW];
    uint32_t sh[CPW];
    bool aval[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int c = wave + NW * i;
        aval[i] = c < nch && 16 * c + 4 * G < Kb;
        vw[i] = *reinterpret_cast<const u4*>(vrow + (aval[i] ? 64 * c + 16 * G : 0));
        mw[i] = *reinterpret_cast<const u2*>(mrow + (aval[i] ? 32 * c + 8 * G : 0));
        sh[i] = srow[aval[i] ? 2 * c + (G >> 1) : 0];
    }

    // 2. Adapter operands: one 32-wide slice of r per wave.
    const int nR = (int)(a.r / 32);
    const uint16_t* Rb = a.R + b * a.sR;
    const uint16_t* Tb = reinterpret_cast<const uint16_t*>(a.ws + b * a.ws_per_problem + t_off);
    h8 ra = {}, tb = {};
    if constexpr (ADAPTER) {
        const int jb = wave < nR ? wave : nR - 1;
        const uint16_t* rp = Rb + (int64_t)(32 * jb + 8 * G) * N + n0 + nl;
#pragma unroll
        for (int e = 0; e < 8; ++e) ra[e] = __builtin_bit_cast(_Float16, rp[e * N]);
        tb = load_h8(Tb + (int64_t)(mval ? m : 0) * a.r + 32 * jb + 8 * G);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep every load above ahead of the first wait

    // 3. Per chunk slot: 4 smfmac steps; the next slot's X loads go out first.
    f4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        h8* x1 = (i & 1) ? xc : xa;
        h8* x2 = (i & 1) ? xd : xb;
        if (i + 1 < CPW) load_x(i + 1, (i & 1) ? xa : xc, (i & 1) ? xb : xd);
        const int c = wave + NW * i;
        const bool u1 = mval && c < nch && 16 * c + 4 * gA1 < Kb;
        const bool u2b = mval && c < nch && 16 * c + 4 * gA2 < Kb;
        const u4 v = aval[i] ? vw[i] : u4{0, 0, 0, 0};
        const u2 mm = aval[i] ? mw[i] : u2{0, 0};
        const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)(aval[i] ? sh[i] : 0u));
        const h2 s2 = {sv, sv};
        acc = smfmac<0>(dequant_word(v[0], s2), concat8(u1 ? x1[0] : h8{}, u2b ? x2[0] : h8{}), acc, mm[0]);
        acc = smfmac<1>(dequant_word(v[1], s2), concat8(u1 ? x1[1] : h8{}, u2b ? x2[1] : h8{}), acc, mm[0]);
        acc = smfmac<0>(dequant_word(v[2], s2), concat8(u1 ? x1[2] : h8{}, u2b ? x2[2] : h8{}), acc, mm[1]);
        acc = smfmac<1>(dequant_word(v[3], s2), concat8(u1 ? x1[3] : h8{}, u2b ? x2[3] : h8{}), acc, mm[1]);
    }

    // 4. Epilogue: acc[n][m] += sum_j R[j][n] T[m][j] (dense MFMA, same layout).
    if constexpr (ADAPTER) {
        acc = mfma16(wave < nR ? ra : h8{}, mval ? tb : h8{}, acc);
        for (int jb = wave + NW; jb < nR; jb += NW) {      // only when r > 32*NW
            h8 r2, t2;
            const uint16_t* rp = Rb + (int64_t)(32 * jb + 8 * G) * N + n0 + nl;
#pragma unroll
            for (int e = 0; e < 8; ++e) r2[e] = __builtin_bit_cast(_Float16, rp[e * N]);
            t2 = load_h8(Tb + (int64_t)(mval ? m : 0) * a.r + 32 * jb + 8 * G);
            acc = mfma16(r2, mval ? t2 : h8{}, acc);
        }
    }

    // 5. Reduce the waves' partial sums and store fp16 Y.
    __shared__ f4 red[NW][64];
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        f4 sum = red[0][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) sum += red[w][lane];
        if (mval) {
            h4 out = {(_Float16)sum[0], (_Float16)sum[1], (_Float16)sum[2], (_Float16)sum[3]};
            *reinterpret_cast<h4*>(a.Y + b * a.sY + (int64_t)m * N + n0 + 4 * G) = out;
        }
    }
}

constexpr int kDecodeWaves = 16;
constexpr int kDecodeMaxCPW = 4;

template <int CPW>
hipError_t launch_main(const LinearArgs& a, size_t t_off, hipStream_t stream) {
    dim3 grid((unsigned)(a.N / 16), (unsigned)a.batch);
    if (a.r > 0)
        hipLaunchKernelGGL((decode_main_kernel<kDecodeWaves, CPW, true>), grid, dim3(64 * kDecodeWaves), 0,
                           stream, a, t_off);
    else
        hipLaunchKernelGGL((decode_main_kernel<kDecodeWaves, CPW, false>), grid, dim3(64 * kDecodeWaves), 0,
                           stream, a, t_off);
    return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int64_t N, int64_t K, int64_t r) { return decode_ws_layout(N, K, r).total; }

bool decode_fits(const LinearArgs& a) {
    const int64_t nch = (a.K + 255) / 256;
    return a.M >= 1 && a.M <= kDecodeMaxM && nch <= (int64_t)kDecodeWaves * kDecodeMaxCPW;
}

hipError_t launch_linear_decode(const LinearArgs& a, hipStream_t stream) {
    const DecodeWs w = decode_ws_layout(a.N, a.K, a.r);
    if (a.r > 0) {
        dim3 grid((unsigned)((a.r / 32) * w.splits), (unsigned)a.batch);
        hipLaunchKernelGGL(adapter_partial_kernel<2>, grid, dim3(256), 0, stream, a, w.splits, w.p_off);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        dim3 g2((unsigned)((a.M * a.r + 255) / 256), (unsigned)a.batch);
        hipLaunchKernelGGL(adapter_reduce_kernel, g2, dim3(256), 0, stream, a, w.splits, w.t_off, w.p_off);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int cpw = (int)(((a.K + 255) / 256 + kDecodeWaves - 1) / kDecodeWaves);
    switch (cpw) {
        case 1: return launch_main<1>(a, w.t_off, stream);
        case 2: return launch_main<2>(a, w.t_off, stream);
        case 3: return launch_main<3>(a, w.t_off, stream);
        default: return launch_main<4>(a, w.t_off, stream);
    }
}

}  // namespace slim
