// slim_linear for a few tokens (decode, M <= 16) with K split over
// workgroups: HBM-bound.
//
//   Y = X . deq(W_c)^T + (X . L) . R
//
// Layer: Compression Trinity thesis §2.1 (Y = X W^T) with the sparse weight
// and the low-rank adapter as parallel paths (Ch. 4 introduction); decode is
// the memory-bound regime (§2.5.2).
//
// A workgroup that owns 16 rows of W over all of K reads all of X from L2:
// at 16 tokens that is 128 KB per workgroup for 25 KB of packed W, and the
// X reads, not HBM, set the time.  Here a workgroup owns 64 rows of W and one
// K slice, so X is read once per 64 rows, and the adapter-down T = X L is
// split the same way.  Two launches, in stream order:
//
// decode_split_kernel: one 8-wave workgroup per (64 rows of W, K slice s).
//   Every operand of the slice goes straight from HBM (or L2) into LDS, 1 KB
//   per wave instruction: the M rows of X, the R8b blocks of the 64 rows
//   (values, metadata, scales: a block's data of consecutive groups is
//   contiguous), and the slice of the workgroup's share of Lt rows (row group
//   g owns T columns [g r / NG, (g + 1) r / NG)).  Then wave w runs the main
//   term of block w & 3 over half the slice's 256-k chunks (dequant +
//   v_smfmac_f32_16x16x64_f16, W rows the sparse A side, tokens B) and an
//   eighth of the slice's 32-k steps of T (v_mfma_f32_16x16x32_f16, Lt rows
//   A, tokens B).  Stores fp32 partials Yp[s][M][N] and Tp[s][M][r].
// decode_finish_kernel<S>: one 8-wave workgroup per 16 rows of W.
//   Y = sum_s Yp[s] + (sum_s Tp[s]) . R: wave w takes the 32-column blocks
//   jb = w, w + 8, ... of r (A: rows of Rt, B: T summed over the slices and
//   rounded to fp16), then the waves are joined in LDS.
#include "internal.hpp"
#include "mfma_util.hpp"

namespace slim {
namespace {

constexpr int kSpThreads = 512;
constexpr int kSpWaves = kSpThreads / 64;
constexpr int kSpLds = 150 * 1024;       // one workgroup per CU at most this
constexpr int kSpMaxM = 16;
constexpr int kSpMaxJ = 16;              // T columns per row group: one MFMA tile
constexpr int kSpMaxS = 16;
constexpr int kSpMinGrid = 256;          // workgroups wanted for the split launch

struct SplitPlan {
    int S;                               // K slices (1, 2, 4, 8 or 16)
    int nG;                              // 128-k groups of K
    int gps;                             // groups per slice, at most
    int NG;                              // row groups of 64 rows
    int jmax;                            // T columns per row group, at most
    int xp;                              // LDS pitch of X and Lt rows (bytes)
    int x_off, v_off, m_off, s_off, l_off, red_off, total;   // LDS bytes
    size_t yp_off, tp_off, ws_total;     // workspace bytes of one problem
};

SplitPlan split_plan(int64_t M, int64_t N, int64_t K, int64_t r) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    auto kb = [](int x) { return (x + 1023) & ~1023; };
    SplitPlan p{};
    p.nG = (int)(K / kGroup);
    p.NG = (int)((N + 63) / 64);
    p.jmax = r > 0 ? (int)((r + p.NG - 1) / p.NG) : 0;
    int S = 1;
    while (S < kSpMaxS && (int64_t)p.NG * S < kSpMinGrid && 2 * S <= p.nG) S *= 2;
    for (;;) {
        p.S = S;
        p.gps = (p.nG + S - 1) / S;
        p.xp = 256 * p.gps + 16;         // + 16 B: the 16 rows of an operand read fall on distinct banks
        int o = 0;
        p.x_off = o; o = kb(o + (int)M * p.xp);
        p.v_off = o; o += 4 * p.gps * 512;
        p.m_off = o; o += 4 * p.gps * 256;
        p.s_off = o; o = kb(o + 4 * p.gps * 32);
        p.l_off = o; o = kb(o + p.jmax * p.xp);
        p.red_off = o; o += 12 * 64 * 16;
        p.total = o;
        if (p.total <= kSpLds || 2 * S > kSpMaxS || 2 * S > p.nG) break;
        S *= 2;
    }
    p.yp_off = kCounterRegion;
    p.tp_off = p.yp_off + al((size_t)p.S * M * N * 4);
    p.ws_total = p.tp_off + al((size_t)p.S * M * r * 4);
    return p;
}

// Lanes of one wave copy `bytes` (a multiple of 16) from buffer offset `off`
// to LDS at `dst`, 1 KB per instruction; lanes past the end are masked off.
__device__ __forceinline__ void dma_copy(u4 rsrc, int off, unsigned char* dst, int bytes, int lane) {
    for (int q = 0; 1024 * q < bytes; ++q)
        if (16 * lane + 1024 * q < bytes) lds_load16(rsrc, dst + 1024 * q, off + 16 * lane, 1024 * q);
}

__global__ __launch_bounds__(kSpThreads) void decode_split_kernel(LinearArgs a, SplitPlan p) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kSpLds];
    const int b = blockIdx.y;
    const int S = p.S;
    const int g = __builtin_amdgcn_readfirstlane((int)blockIdx.x / S);
    const int s = __builtin_amdgcn_readfirstlane((int)blockIdx.x - g * S);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nl = lane & 15, G = lane >> 4;
    const int K = (int)a.K, M = (int)a.M, r = (int)a.r, N = (int)a.N, nG = p.nG;
    const int G0 = s * nG / S, ns = (s + 1) * nG / S - G0;     // groups [G0, G0 + ns) of this slice
    const int nblk = min(4, N / 16 - 4 * g);                   // 16-row blocks of this row group
    const int j0 = (int)((int64_t)g * r / p.NG), nj = (int)((int64_t)(g + 1) * r / p.NG) - j0;
    const int64_t n0 = (int64_t)g * 64;

    // 1. Operands of the slice into LDS.  X rows m = wave, wave + 8, ...;
    //    waves 0..3: values of block wave; waves 4..7: metadata and scales of
    //    block wave - 4; Lt rows j0 + j for j = wave, wave + 8, ...
    const u4 rx = rsrc_words(a.X + b * a.sX, (int64_t)M * K * 2);
    for (int m = wave; m < M; m += kSpWaves)
        dma_copy(rx, (m * K + G0 * kGroup) * 2, lds + p.x_off + m * p.xp, ns * 256, lane);
    if (wave < 4) {
        const u4 rv = rsrc_words(a.values + b * a.sV + n0 * (K / 4), (int64_t)nblk * 16 * (K / 4));
        if (wave < nblk) dma_copy(rv, wave * 16 * (K / 4) + G0 * 512, lds + p.v_off + wave * p.gps * 512, ns * 512, lane);
    } else {
        const int f = wave - 4;
        const u4 rm = rsrc_words(a.meta + b * a.sMeta + n0 * (K / 8), (int64_t)nblk * 16 * (K / 8));
        const u4 rs = rsrc_words(a.scales + b * a.sS + n0 * nG, (int64_t)nblk * 16 * nG * 2);
        if (f < nblk) {
            dma_copy(rm, f * 16 * (K / 8) + G0 * 256, lds + p.m_off + f * p.gps * 256, ns * 256, lane);
            dma_copy(rs, (f * 16 * nG + G0 * 16) * 2, lds + p.s_off + f * p.gps * 32, ns * 32, lane);
        }
    }
    if (nj > 0) {
        const u4 rl = rsrc_words(a.Lt + b * a.sLt + (int64_t)j0 * K, (int64_t)nj * K * 2);
        for (int j = wave; j < nj; j += kSpWaves)
            dma_copy(rl, (j * K + G0 * kGroup) * 2, lds + p.l_off + j * p.xp, ns * 256, lane);
    }
    wait_vmem_below<0>();
    __syncthreads();

    // 2. Main term: block f = wave & 3, 256-k chunks of half h = wave >> 2.
    //    Lane (row or token nl, G): values of group 2c + G / 2, words for the
    //    chunk blocks 4G .. 4G + 3 (one per 64-k step); B elements 0..7 at
    //    chunk k 64 (G / 2) + 16 t + 8 (G & 1), elements 8..15 at 128 more.
    const int f = wave & 3, h = wave >> 2;
    const int nchk = (ns + 1) / 2, c_mid = (nchk + 1) / 2;
    f4 acc = {0, 0, 0, 0};
    if (f < nblk) {
        const bool mval = nl < M;
        for (int c = h ? c_mid : 0; c < (h ? nchk : c_mid); ++c) {
            const int gl = 2 * c + (G >> 1);
            const bool av = gl < ns;
            const int blk = (f * p.gps + (av ? gl : 0));
            const u4 v = av ? *reinterpret_cast<const u4*>(lds + p.v_off + blk * 512 + nl * 32 + 16 * (G & 1)) : u4{0, 0, 0, 0};
            const u2 mm = av ? *reinterpret_cast<const u2*>(lds + p.m_off + blk * 256 + nl * 16 + 8 * (G & 1)) : u2{0, 0};
            const _Float16 sv = av ? *reinterpret_cast<const _Float16*>(lds + p.s_off + blk * 32 + 2 * nl) : (_Float16)0.0f;
            const h2 s2 = {sv, sv};
            const bool b1 = mval && 2 * c < ns, b2 = mval && 2 * c + 1 < ns;
            const unsigned char* xr = lds + p.x_off + (mval ? nl : 0) * p.xp + 2 * (256 * c + 64 * (G >> 1) + 8 * (G & 1));
            h8 x1[4], x2[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                x1[t] = b1 ? *reinterpret_cast<const h8*>(xr + 32 * t) : h8{};
                x2[t] = b2 ? *reinterpret_cast<const h8*>(xr + 256 + 32 * t) : h8{};
            }
            acc = smfmac<0>(dequant_word(v[0], s2), concat8(x1[0], x2[0]), acc, mm[0]);
            acc = smfmac<1>(dequant_word(v[1], s2), concat8(x1[1], x2[1]), acc, mm[0]);
            acc = smfmac<0>(dequant_word(v[2], s2), concat8(x1[2], x2[2]), acc, mm[1]);
            acc = smfmac<1>(dequant_word(v[3], s2), concat8(x1[3], x2[3]), acc, mm[1]);
        }
    }

    // 3. Partial T of the slice: 32-k steps st = wave, wave + 8, ... (A: Lt
    //    row j0 + nl, B: token nl).
    f4 tacc = {0, 0, 0, 0};
    for (int st = wave; st < 4 * ns && nj > 0; st += kSpWaves) {
        const h8 la = nl < nj ? *reinterpret_cast<const h8*>(lds + p.l_off + nl * p.xp + 2 * (32 * st + 8 * G)) : h8{};
        const h8 xb = nl < M ? *reinterpret_cast<const h8*>(lds + p.x_off + nl * p.xp + 2 * (32 * st + 8 * G)) : h8{};
        tacc = mfma16(la, xb, tacc);
    }

    // 4. Join the halves and the eight T partials; store fp32 partials (lane:
    //    token nl, rows or T columns 4G .. 4G + 3).
    f4* red = reinterpret_cast<f4*>(lds + p.red_off);
    if (h == 1) red[f * 64 + lane] = acc;
    red[(4 + wave) * 64 + lane] = tacc;
    __syncthreads();
    unsigned char* ws = a.ws + b * a.ws_per_problem;
    if (h == 0 && f < nblk && nl < M) {
        acc += red[f * 64 + lane];
        float* Yp = reinterpret_cast<float*>(ws + p.yp_off);
        *reinterpret_cast<f4*>(Yp + ((int64_t)s * M + nl) * N + n0 + 16 * f + 4 * G) = acc;
    }
    if (wave == 4 && nj > 0 && nl < M) {
        f4 t = red[4 * 64 + lane];
#pragma unroll
        for (int w = 1; w < kSpWaves; ++w) t += red[(4 + w) * 64 + lane];
        float* Tp = reinterpret_cast<float*>(ws + p.tp_off) + ((int64_t)s * M + nl) * r + j0;
#pragma unroll
        for (int v = 0; v < 4; ++v)
            if (4 * G + v < nj) Tp[4 * G + v] = t[v];
    }
}

// S: K slices of the split launch.
template <int S>
__global__ __launch_bounds__(kSpThreads) void decode_finish_kernel(LinearArgs a, SplitPlan p) {
    __shared__ f4 red[kSpWaves][64];
    const int b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nl = lane & 15, G = lane >> 4;
    const int M = (int)a.M, r = (int)a.r, N = (int)a.N;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const unsigned char* ws = a.ws + b * a.ws_per_problem;
    const bool mval = nl < M;

    // acc += Rt-slice . T over the 32-column blocks of this wave.
    f4 acc = {0, 0, 0, 0};
    const int nR = r / 32;
    if (wave < nR) {
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.Rt + b * a.sRt + n0 * r, (int64_t)16 * r * 2);
        const __amdgpu_buffer_rsrc_t rt = make_rsrc(ws + p.tp_off, (int64_t)S * M * r * 4);
        for (int jb = wave; jb < nR; jb += kSpWaves) {
            const h8 ra = buffer_load_h8(rr, (nl * r + 32 * jb + 8 * G) * 2);
            f4 lo[S], hi[S];
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int off = mval ? ((s * M + nl) * r + 32 * jb + 8 * G) * 4 : kOOB;
                lo[s] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rt, off, 0, 0));
                hi[s] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rt, mval ? off + 16 : kOOB, 0, 0));
            }
            f4 tl = lo[0], th = hi[0];
#pragma unroll
            for (int s = 1; s < S; ++s) {
                tl += lo[s];
                th += hi[s];
            }
            const h8 tb = {(_Float16)tl[0], (_Float16)tl[1], (_Float16)tl[2], (_Float16)tl[3],
                           (_Float16)th[0], (_Float16)th[1], (_Float16)th[2], (_Float16)th[3]};
            acc = mfma16(ra, tb, acc);
        }
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && mval) {
        const float* Yp = reinterpret_cast<const float*>(ws + p.yp_off);
        f4 y[S];
#pragma unroll
        for (int s = 0; s < S; ++s) y[s] = *reinterpret_cast<const f4*>(Yp + ((int64_t)s * M + nl) * N + n0 + 4 * G);
        f4 sum = red[0][lane];
#pragma unroll
        for (int w = 1; w < kSpWaves; ++w) sum += red[w][lane];
#pragma unroll
        for (int s = 0; s < S; ++s) sum += y[s];
        const h4 out = {(_Float16)sum[0], (_Float16)sum[1], (_Float16)sum[2], (_Float16)sum[3]};
        *reinterpret_cast<h4*>(a.Y + b * a.sY + (int64_t)nl * N + n0 + 4 * G) = out;
    }
}

}  // namespace

size_t split_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
    if (M < 1 || M > kSpMaxM || K < kGroup) return 0;
    return split_plan(M, N, K, r).ws_total;
}

bool split_fits(const LinearArgs& a) {
    if (a.M < 1 || a.M > kSpMaxM || a.K < kGroup) return false;
    const SplitPlan p = split_plan(a.M, a.N, a.K, a.r);
    // 32-bit buffer offsets: a row group's packed W, X and the partials.
    const int64_t lim = 0x7FFFFFF0;
    return p.jmax <= kSpMaxJ && p.total <= kSpLds && 64 * (a.K / 4) < lim && a.M * a.K * 2 < lim &&
           (int64_t)p.S * a.M * a.N * 4 < lim && (int64_t)p.S * a.M * a.r * 4 < lim;
}

hipError_t launch_linear_split(const LinearArgs& a, hipStream_t stream) {
    const SplitPlan p = split_plan(a.M, a.N, a.K, a.r);
    hipLaunchKernelGGL(decode_split_kernel, dim3((unsigned)(p.NG * p.S), (unsigned)a.batch), dim3(kSpThreads), 0,
                       stream, a, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(a.N / 16), (unsigned)a.batch), block(kSpThreads);
    switch (p.S) {
        case 1: hipLaunchKernelGGL(decode_finish_kernel<1>, grid, block, 0, stream, a, p); break;
        case 2: hipLaunchKernelGGL(decode_finish_kernel<2>, grid, block, 0, stream, a, p); break;
        case 4: hipLaunchKernelGGL(decode_finish_kernel<4>, grid, block, 0, stream, a, p); break;
        case 8: hipLaunchKernelGGL(decode_finish_kernel<8>, grid, block, 0, stream, a, p); break;
        default: hipLaunchKernelGGL(decode_finish_kernel<16>, grid, block, 0, stream, a, p); break;
    }
    return hipGetLastError();
}

}  // namespace slim
