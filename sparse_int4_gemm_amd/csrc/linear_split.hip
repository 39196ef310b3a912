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
// X reads, not HBM, set the time.  Here a workgroup owns a row group of 64
// rows of W (96 or 128 when that brings the items into one round) and one K
// slice, so X is read once per row group, and the adapter-down T = X L is
// split the same way.  Two launches, in stream order:
//
// decode_split_kernel<QA, NBI>: 8-wave workgroups, at most one per CU, each
//   taking the items (16 NBI rows of W, K slice s) i = blockIdx, blockIdx +
//   gridDim, ... in turn (one round of workgroups whatever the item count).
//   Per item, every operand of the slice goes straight from HBM (or L2) into
//   LDS, 1 KB per wave instruction: the M rows of X, the R8b blocks of the
//   row group (values, metadata, scales: a block's data of consecutive groups
//   is contiguous), and, with NBI = 4, the slice of the row group's share of
//   Lt rows (row group g owns T columns [g r / NG, (g + 1) r / NG)); with
//   NBI = 6 or 8 the Lt operands of each wave's T steps go straight into
//   registers instead.  Then the waves take the work units (256-k chunk,
//   64-k step pair) in turn, each applying one X operand read to all NBI
//   blocks (dequant + v_smfmac_f32_16x16x64_f16, W rows the sparse A side,
//   tokens B), and an eighth of the slice's 32-k steps of T each
//   (v_mfma_f32_16x16x32_f16, Lt rows A, tokens B).  Stores fp32 partials
//   Yp[s][M][N] and Tp[s][M][r].
// decode_finish_kernel<S, QA>: one 8-wave workgroup per 16 rows of W.
//   Y = sum_s Yp[s] + (sum_s Tp[s]) . R: wave w takes the 32-column blocks
//   jb = w, w + 8, ... of r (A: rows of Rt, B: T summed over the slices and
//   rounded to fp16), then the waves are joined in LDS.
#include <atomic>

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
    int nbi;                             // 16-row blocks per row group: 4, or 6 or 8 (Lt then read into registers)
    int NG;                              // row groups of 16 nbi rows
    int jmax;                            // T columns per row group, at most
    int xp;                              // LDS pitch of X and Lt rows (bytes)
    int x_off, v_off, m_off, s_off, l_off, red_off, total;   // LDS bytes (red over the operands)
    size_t yp_off, tp_off, ws_total;     // workspace bytes of one problem
};

SplitPlan split_plan_nb(int64_t M, int64_t N, int64_t K, int64_t r, int nbi, int s_fixed = 0) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    auto kb = [](int x) { return (x + 1023) & ~1023; };
    SplitPlan p{};
    p.nbi = nbi;
    p.nG = (int)(K / kGroup);
    p.NG = (int)((N / 16 + nbi - 1) / nbi);
    p.jmax = r > 0 ? (int)((r + p.NG - 1) / p.NG) : 0;
    int S = 1;
    while (S < kSpMaxS && (int64_t)p.NG * S < kSpMinGrid && 2 * S <= p.nG) S *= 2;
    if (s_fixed > 0) S = s_fixed;
    for (;;) {
        p.S = S;
        p.gps = (p.nG + S - 1) / S;
        p.xp = 256 * p.gps + 16;         // + 16 B: the 16 rows of an operand read fall on distinct banks
        int o = 0;
        p.x_off = o; o = kb(o + (int)M * p.xp);
        p.v_off = o; o += nbi * p.gps * 512;
        p.m_off = o; o += nbi * p.gps * 256;
        p.s_off = o; o = kb(o + nbi * p.gps * 32);
        p.l_off = o; o = nbi == 4 ? kb(o + p.jmax * p.xp) : o;
        p.red_off = 0;                   // after the compute, over the operands
        const int red = kSpWaves * (nbi + 1) * 64 * 16;
        p.total = o > red ? o : red;
        if (p.total <= kSpLds || s_fixed > 0 || 2 * S > kSpMaxS || 2 * S > p.nG) break;
        S *= 2;
    }
    p.yp_off = kCounterRegion;
    p.tp_off = p.yp_off + al((size_t)p.S * M * N * 4);
    p.ws_total = p.tp_off + al((size_t)p.S * M * r * 4);
    return p;
}

// Row groups of 4 blocks; of 6 or 8 when that brings more than one round of
// items into one with the same K split (gate/up at 16 tokens: 344 items of 4
// blocks, 230 of 6; down: 512 of 4, 256 of 8) and the layout fits (Lt not in
// LDS: at most 64 steps of T per item, 8 per wave).
SplitPlan split_plan(int64_t M, int64_t N, int64_t K, int64_t r, bool qa = false) {
    (void)qa;
    const SplitPlan p4 = split_plan_nb(M, N, K, r, 4);
    if ((int64_t)p4.NG * p4.S <= kSpMinGrid) return p4;
    for (int nbi : {6, 8}) {
        const SplitPlan q = split_plan_nb(M, N, K, r, nbi, p4.S);
        if ((int64_t)q.NG * q.S <= kSpMinGrid && q.total <= kSpLds && q.jmax <= kSpMaxJ && 4 * q.gps <= 8 * kSpWaves)
            return q;
    }
    return p4;
}

// Lanes of one wave copy `bytes` (a multiple of 16) from buffer offset `off`
// to LDS at `dst`, 1 KB per instruction; lanes past the end are masked off.
__device__ __forceinline__ void dma_copy(u4 rsrc, int off, unsigned char* dst, int bytes, int lane) {
    for (int q = 0; 1024 * q < bytes; ++q)
        if (16 * lane + 1024 * q < bytes) lds_load16(rsrc, dst + 1024 * q, off + 16 * lane, 1024 * q);
}

// QA: the adapter factors are int4 codes with fp16 group scales (Lt: one per
// 128 k, Rt: one per 32 r); a slice's Lt codes go to LDS like the fp16 rows
// (pitch 64 gps + 16 bytes), their scales after them ([jmax][gps] fp16).
// NBI: 16-row blocks per row group (p.nbi).  With 6 or 8 the Lt operand of the T
// steps is loaded straight into registers (8 steps per wave at most) so that
// X and the six blocks fit in LDS.
template <bool QA, int NBI>
__global__ __launch_bounds__(kSpThreads) void decode_split_kernel(LinearArgs a, SplitPlan p) {
    static_assert(NBI == 4 || NBI == 6 || NBI == 8, "row groups of 4, 6 or 8 blocks");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kSpLds];
    const int b = blockIdx.y;
    const int S = p.S;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nl = lane & 15, G = lane >> 4;
    const int K = (int)a.K, M = (int)a.M, r = (int)a.r, N = (int)a.N, nG = p.nG;
    for (int item = blockIdx.x; item < p.NG * S; item += gridDim.x) {
        const int g = __builtin_amdgcn_readfirstlane(item / S);
        const int s = __builtin_amdgcn_readfirstlane(item - g * S);
        const int G0 = s * nG / S, ns = (s + 1) * nG / S - G0;     // groups [G0, G0 + ns) of this slice
        const int nblk = min(NBI, N / 16 - NBI * g);               // 16-row blocks of this row group
        const int j0 = (int)((int64_t)g * r / p.NG), nj = (int)((int64_t)(g + 1) * r / p.NG) - j0;
        const int64_t n0 = (int64_t)g * 16 * NBI;

        // 1. Operands of the slice into LDS.  X rows m = wave, wave + 8, ...;
        //    values of block f by wave f, its metadata and scales by wave
        //    (f + NBI) % 8; Lt rows j0 + j for j = wave, wave + 8, ... (NBI = 4).
        const u4 rx = rsrc_words(a.X + b * a.sX, (int64_t)M * K * 2);
        for (int m = wave; m < M; m += kSpWaves)
            dma_copy(rx, (m * K + G0 * kGroup) * 2, lds + p.x_off + m * p.xp, ns * 256, lane);
        {
            const u4 rv = rsrc_words(a.values + b * a.sV + n0 * (K / 4), (int64_t)nblk * 16 * (K / 4));
            const u4 rm = rsrc_words(a.meta + b * a.sMeta + n0 * (K / 8), (int64_t)nblk * 16 * (K / 8));
            const u4 rs = rsrc_words(a.scales + b * a.sS + n0 * nG, (int64_t)nblk * 16 * nG * 2);
#pragma unroll
            for (int f = 0; f < NBI; ++f) {
                if (f < nblk && wave == f % kSpWaves)
                    dma_copy(rv, f * 16 * (K / 4) + G0 * 512, lds + p.v_off + f * p.gps * 512, ns * 512, lane);
                if (f < nblk && wave == (f + NBI) % kSpWaves) {
                    dma_copy(rm, f * 16 * (K / 8) + G0 * 256, lds + p.m_off + f * p.gps * 256, ns * 256, lane);
                    dma_copy(rs, (f * 16 * nG + G0 * 16) * 2, lds + p.s_off + f * p.gps * 32, ns * 32, lane);
                }
            }
        }
        const int lqp = 64 * p.gps + 16, ls_off = p.l_off + ((p.jmax * lqp + 15) & ~15);
        if (nj > 0) {
            if constexpr (QA && NBI == 4) {
                const u4 rl = rsrc_words(a.Lq + (int64_t)j0 * (K / 2), (int64_t)nj * (K / 2));
                for (int j = wave; j < nj; j += kSpWaves)
                    dma_copy(rl, j * (K / 2) + G0 * 64, lds + p.l_off + j * lqp, ns * 64, lane);
                // Scales: one plain load per thread (nj ns <= 16 gps halves).
                for (int e = tid; e < nj * ns; e += kSpThreads) {
                    const int j = e / ns, gg = e - j * ns;
                    const uint16_t sc = reinterpret_cast<const uint16_t*>(a.Ls)[(int64_t)(j0 + j) * nG + G0 + gg];
                    *reinterpret_cast<uint16_t*>(lds + ls_off + 2 * (j * p.gps + gg)) = sc;
                }
            } else if constexpr (!QA && NBI == 4) {
                const u4 rl = rsrc_words(a.Lt + b * a.sLt + (int64_t)j0 * K, (int64_t)nj * K * 2);
                for (int j = wave; j < nj; j += kSpWaves)
                    dma_copy(rl, (j * K + G0 * kGroup) * 2, lds + p.l_off + j * p.xp, ns * 256, lane);
            }
        }
        // NBI = 6: the A operands of this wave's T steps st = wave + 8 i (Lt row
        // j0 + nl, k = 128 G0 + 32 st + 8 G .. +8); rows past nj and steps past
        // the slice read zero.
        //      Quantised adapters: the codes word (8 k) and the group scale
        //      of each step, turned into fp16 at the step.
        h8 lreg[NBI == 4 || QA ? 1 : 8];
        uint32_t qw[NBI != 4 && QA ? 8 : 1], qs[NBI != 4 && QA ? 8 : 1];
        if constexpr (NBI != 4 && !QA) {
            const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.Lt + b * a.sLt + (int64_t)j0 * K, (int64_t)nj * K * 2);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int st = wave + kSpWaves * i;
                const bool ok = nl < nj && st < 4 * ns;
                lreg[i] = buffer_load_h8(rl, ok ? (nl * K + G0 * kGroup + 32 * st + 8 * G) * 2 : kOOB);
            }
        } else if constexpr (NBI != 4) {
            const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.Lq + (int64_t)j0 * (K / 2), (int64_t)nj * (K / 2));
            const __amdgpu_buffer_rsrc_t rqs = make_rsrc(a.Ls + (int64_t)j0 * nG, (int64_t)nj * nG * 2);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int st = wave + kSpWaves * i;
                const bool ok = nl < nj && st < 4 * ns;
                qw[i] = __builtin_amdgcn_raw_buffer_load_b32(rq, ok ? nl * (K / 2) + G0 * 64 + 16 * st + 4 * G : kOOB, 0, 0);
                qs[i] = __builtin_amdgcn_raw_buffer_load_b16(rqs, ok ? 2 * (nl * nG + G0 + st / 4) : kOOB, 0, 0);
            }
        }
        wait_vmem_below<0>();
        __syncthreads();

        // 2. Main term.  Work units (256-k chunk c, 64-k step pair q): wave w
        //    takes units w, w + 8, ..., reads the X operand of its two steps
        //    once and applies it to all four blocks.  Lane (row or token nl,
        //    G): values of group 2c + G / 2, words 2q, 2q + 1 of the chunk
        //    blocks 4G .. 4G + 3 (one word per 64-k step); B elements 0..7 at
        //    chunk k 64 (G / 2) + 16 t + 8 (G & 1), elements 8..15 at 128 more.
        //    Every LDS read is unconditional (clamped to data of this item)
        //    and zeroed afterwards, so a unit's reads go out together.
        const int nchk = (ns + 1) / 2;
        f4 acc[NBI];
#pragma unroll
        for (int f = 0; f < NBI; ++f) acc[f] = f4{0, 0, 0, 0};
        const bool mval = nl < M;
        for (int u = wave; u < 2 * nchk; u += kSpWaves) {
            const int c = u >> 1, q = u & 1;
            const int gl = 2 * c + (G >> 1);
            const bool av = gl < ns;
            const int glc = av ? gl : 0;
            const bool b1 = mval && 2 * c < ns, b2 = mval && 2 * c + 1 < ns;
            const unsigned char* xr =
                lds + p.x_off + (mval ? nl : 0) * p.xp + 2 * (256 * c + 64 * (G >> 1) + 8 * (G & 1) + 32 * q);
            h8 x1[2], x2[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                x1[t] = *reinterpret_cast<const h8*>(xr + 32 * t);
                x2[t] = *reinterpret_cast<const h8*>(xr + 256 + 32 * t);
            }
            u2 v[NBI];
            uint32_t mm[NBI];
            _Float16 sv[NBI];
#pragma unroll
            for (int f = 0; f < NBI; ++f) {
                const int blk = f * p.gps + glc;
                v[f] = *reinterpret_cast<const u2*>(lds + p.v_off + blk * 512 + nl * 32 + 16 * (G & 1) + 8 * q);
                mm[f] = *reinterpret_cast<const uint32_t*>(lds + p.m_off + blk * 256 + nl * 16 + 8 * (G & 1) + 4 * q);
                sv[f] = *reinterpret_cast<const _Float16*>(lds + p.s_off + blk * 32 + 2 * nl);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                x1[t] = b1 ? x1[t] : h8{};
                x2[t] = b2 ? x2[t] : h8{};
            }
            const h16 xb0 = concat8(x1[0], x2[0]), xb1 = concat8(x1[1], x2[1]);
#pragma unroll
            for (int f = 0; f < NBI; ++f) {
                const u2 vf = av ? v[f] : u2{0, 0};
                const uint32_t mf = av ? mm[f] : 0u;
                const _Float16 sf = av ? sv[f] : (_Float16)0.0f;
                const h2 s2 = {sf, sf};
                acc[f] = smfmac<0>(dequant_word(vf[0], s2), xb0, acc[f], mf);
                acc[f] = smfmac<1>(dequant_word(vf[1], s2), xb1, acc[f], mf);
            }
        }

        // 3. Partial T of the slice: 32-k steps st = wave, wave + 8, ... (A: Lt
        //    row j0 + nl, B: token nl).
        f4 tacc = {0, 0, 0, 0};
        if constexpr (NBI != 4) {
            if (nj > 0) {
                const unsigned char* xr = lds + p.x_off + (nl < M ? nl : 0) * p.xp + 16 * G;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int st = wave + kSpWaves * i;
                    if (st >= 4 * ns) break;                       // uniform
                    const h8 xb = *reinterpret_cast<const h8*>(xr + 64 * st);
                    h8 la;
                    if constexpr (QA) {
                        const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)qs[i]);
                        la = dequant_word(qw[i], h2{sc, sc});
                    } else {
                        la = lreg[i];
                    }
                    tacc = mfma16(la, nl < M ? xb : h8{}, tacc);
                }
            }
        } else if (nj > 0) {
            const int jl = nl < nj ? nl : 0;
            const unsigned char* lr = lds + p.l_off + jl * (QA ? lqp : p.xp) + (QA ? 4 : 16) * G;
            const unsigned char* xr = lds + p.x_off + (nl < M ? nl : 0) * p.xp + 16 * G;
            for (int st = wave; st < 4 * ns; st += kSpWaves) {
                h8 la;
                if constexpr (QA) {     // 32-k step st: codes word 4 st + G of the row, scale of group st / 4
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(lr + 16 * st);
                    const _Float16 sc = *reinterpret_cast<const _Float16*>(lds + ls_off + 2 * (jl * p.gps + st / 4));
                    la = dequant_word(w, h2{sc, sc});
                } else {
                    la = *reinterpret_cast<const h8*>(lr + 64 * st);
                }
                const h8 xb = *reinterpret_cast<const h8*>(xr + 64 * st);
                tacc = mfma16(nl < nj ? la : h8{}, nl < M ? xb : h8{}, tacc);
            }
        }

        // 4. Join the waves' partial sums (block f: wave f sums the eight) and
        //    the eight T partials (wave NBI); store fp32 partials (lane: token
        //    nl, rows or T columns 4G .. 4G + 3).
        constexpr int kR = NBI + 1;                                // slots per wave
        f4* red = reinterpret_cast<f4*>(lds + p.red_off);        // [kSpWaves][kR][64]
        __syncthreads();                                           // operands no longer read
#pragma unroll
        for (int f = 0; f < NBI; ++f) red[(wave * kR + f) * 64 + lane] = acc[f];
        red[(wave * kR + NBI) * 64 + lane] = tacc;
        __syncthreads();
        unsigned char* ws = a.ws + b * a.ws_per_problem;
        if (wave < NBI && wave < nblk && nl < M) {
            f4 y = red[wave * 64 + lane];
#pragma unroll
            for (int w = 1; w < kSpWaves; ++w) y += red[(w * kR + wave) * 64 + lane];
            float* Yp = reinterpret_cast<float*>(ws + p.yp_off);
            *reinterpret_cast<f4*>(Yp + ((int64_t)s * M + nl) * N + n0 + 16 * wave + 4 * G) = y;
        }
        if (wave == NBI % kSpWaves && nj > 0 && nl < M) {
            f4 t = red[NBI * 64 + lane];
#pragma unroll
            for (int w = 1; w < kSpWaves; ++w) t += red[(w * kR + NBI) * 64 + lane];
            float* Tp = reinterpret_cast<float*>(ws + p.tp_off) + ((int64_t)s * M + nl) * r + j0;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (4 * G + v < nj) Tp[4 * G + v] = t[v];
        }
        __syncthreads();                     // the next item's loads overwrite LDS
    }
}

// S: K slices of the split launch.  T = sum_s Tp[s] is formed once per
// workgroup from contiguous 16-byte pieces (thread t: pieces t, t + 512, ...,
// all slices' loads in flight together) into an fp16 tile in LDS, and the
// workgroup's NB blocks of 16 rows of Rt go straight into LDS; the MFMA
// operands are then read from LDS.  NB = 3 when the N / 16 blocks would
// take more than one round of the 256 CUs (gate/up: 688 blocks, 230
// workgroups), so that T is summed once for three blocks.
constexpr int kFinMaxR = 512;            // T tile and Rt rows fit the LDS for M <= 16
constexpr int kFinPitch = 2 * kFinMaxR + 16;
constexpr int kFinLds(int nb) { return ((kSpMaxM * kFinPitch + 1023) & ~1023) + nb * 16 * kFinPitch; }

// QA: the rows' Rt codes (r / 2 bytes each) and scales (r / 32 fp16 each)
// are two contiguous blocks, copied as they are.
template <int S, bool QA, int NB>
__global__ __launch_bounds__(kSpThreads) void decode_finish_kernel(LinearArgs a, SplitPlan p) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kFinLds(NB)];
    __shared__ f4 red[NB][kSpWaves][64];
    const int b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nl = lane & 15, G = lane >> 4;
    const int M = (int)a.M, r = (int)a.r, N = (int)a.N;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * NB;
    const int left = N / 16 - (int)blockIdx.x * NB;
    const int nbk = NB == 1 ? 1 : (left < NB ? left : NB);      // blocks of this workgroup (uniform)
    const unsigned char* ws = a.ws + b * a.ws_per_problem;
    const bool mval = nl < M;
    const int rp = 2 * r + 16;                                  // LDS row pitch (bytes) of T and Rt
    unsigned char* tt = lds;                                    // T [M][r] fp16
    unsigned char* rt = lds + ((M * rp + 1023) & ~1023);        // Rt rows [16 nbk][r] fp16

    // 1. Rt rows n0 + q (q = wave, wave + 8, ...) into LDS; the partials of Y
    //    (wave j: block j); T summed over the slices into the fp16 tile.
    if (QA && r > 0) {
        const int cb = 8 * r * nbk;                             // codes bytes
        const u4 rq = rsrc_words(a.Rq + n0 * (r / 2), (int64_t)cb);
        const u4 rs = rsrc_words(a.Rs + n0 * (r / 32), (int64_t)r * nbk);
        if (wave < kSpWaves - 1) {
            if (2048 * wave < cb) dma_copy(rq, 2048 * wave, rt + 2048 * wave, min(2048, cb - 2048 * wave), lane);
        } else {
            dma_copy(rs, 0, rt + cb, r * nbk, lane);
        }
    } else if (r > 0) {
        const u4 rr = rsrc_words(a.Rt + b * a.sRt + n0 * r, (int64_t)16 * nbk * r * 2);
        for (int q = wave; q < 16 * nbk; q += kSpWaves)
            for (int i = 0; 1024 * i < 2 * r; ++i)
                if (16 * lane + 1024 * i < 2 * r) lds_load16(rr, rt + q * rp + 1024 * i, q * 2 * r + 16 * lane, 1024 * i);
    }
    f4 y[S];
    if (wave < nbk) {
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(ws + p.yp_off, (int64_t)S * M * N * 4);
#pragma unroll
        for (int s = 0; s < S; ++s)
            y[s] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(
                       ry, mval ? (int)((((int64_t)s * M + nl) * N + n0 + 16 * wave + 4 * G) * 4) : kOOB, 0, 0));
    }
    const __amdgpu_buffer_rsrc_t rtp = make_rsrc(ws + p.tp_off, (int64_t)S * M * r * 4);
    constexpr int U = S <= 8 ? 4 : 2;                           // pieces per thread in flight
    const int nq = M * r / 4;                                   // 16-byte pieces of one slice's T
    for (int q0 = tid; q0 < nq; q0 += U * kSpThreads) {
        f4 v[U][S];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = q0 + u * kSpThreads;
#pragma unroll
            for (int s = 0; s < S; ++s)
                v[u][s] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rtp, q < nq ? (s * nq + q) * 16 : kOOB, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = q0 + u * kSpThreads;
            if (q >= nq) break;
            f4 t = v[u][0];
#pragma unroll
            for (int s = 1; s < S; ++s) t += v[u][s];
            const int m = 4 * q / r, j = 4 * q - m * r;
            const h4 th = {(_Float16)t[0], (_Float16)t[1], (_Float16)t[2], (_Float16)t[3]};
            *reinterpret_cast<h4*>(tt + m * rp + 2 * j) = th;
        }
    }
    wait_vmem_below<0>();
    __syncthreads();

    // 2. acc[j] += Rt-slice of block j . T over the 32-column blocks jb =
    //    wave, wave + 8, ...
    f4 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = f4{0, 0, 0, 0};
    for (int jb = wave; jb < r / 32; jb += kSpWaves) {
        const h8 tb = mval ? *reinterpret_cast<const h8*>(tt + nl * rp + 2 * (32 * jb + 8 * G)) : h8{};
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if (j >= nbk) break;                                // uniform: the last workgroup
            const int q = 16 * j + nl;                          // Rt row in LDS
            h8 ra;
            if constexpr (QA) {  // row q, r-columns 32 jb + 8 G .. +8: one codes word, scale of group jb
                const uint32_t w = *reinterpret_cast<const uint32_t*>(rt + q * (r / 2) + 16 * jb + 4 * G);
                const _Float16 sc = *reinterpret_cast<const _Float16*>(rt + 8 * r * nbk + 2 * (q * (r / 32) + jb));
                ra = dequant_word(w, h2{sc, sc});
            } else {
                ra = *reinterpret_cast<const h8*>(rt + q * rp + 2 * (32 * jb + 8 * G));
            }
            acc[j] = mfma16(ra, tb, acc[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) red[j][wave][lane] = acc[j];
    __syncthreads();
    if (wave < nbk && mval) {
        const int j = wave;
        f4 sum = red[j][0][lane];
#pragma unroll
        for (int w = 1; w < kSpWaves; ++w) sum += red[j][w][lane];
#pragma unroll
        for (int s = 0; s < S; ++s) sum += y[s];
        const h4 out = {(_Float16)sum[0], (_Float16)sum[1], (_Float16)sum[2], (_Float16)sum[3]};
        *reinterpret_cast<h4*>(a.Y + b * a.sY + (int64_t)nl * N + n0 + 16 * j + 4 * G) = out;
    }
}

}  // namespace

size_t split_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
    if (M < 1 || M > kSpMaxM || K < kGroup) return 0;
    return split_plan(M, N, K, r).ws_total;
}

bool split_fits(const LinearArgs& a) {
    if (a.M < 1 || a.M > kSpMaxM || a.K < kGroup) return false;
    const SplitPlan p = split_plan(a.M, a.N, a.K, a.r, a.Lq != nullptr);
    // 32-bit buffer offsets: a row group's packed W, X and the partials.
    const int64_t lim = 0x7FFFFFF0;
    return p.jmax <= kSpMaxJ && p.total <= kSpLds && a.r <= kFinMaxR && 64 * (a.K / 4) < lim && a.M * a.K * 2 < lim &&
           (int64_t)p.S * a.M * a.N * 4 < lim && (int64_t)p.S * a.M * a.r * 4 < lim;
}

// Workgroups of decode_split_kernel resident at once on the current device
// (one per CU); 0 if it cannot be determined.
int64_t split_capacity() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int64_t> cache[kMaxDevices];              // 0: not yet known
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int64_t c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<false, 4>, kSpThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    c = (int64_t)per_cu * cus;
    cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

hipError_t launch_linear_split(const LinearArgs& a, hipStream_t stream) {
    const SplitPlan p = split_plan(a.M, a.N, a.K, a.r, a.Lq != nullptr);
    // One round of workgroups shared by the batch's problems.
    const int64_t items = (int64_t)p.NG * p.S, cap = split_capacity();
    int64_t per = cap > 0 ? cap / a.batch : items;
    if (per < 1) per = 1;
    if (per > items) per = items;
    // Quantised adapters when the int4 factors are given (one problem).
    const bool qa = a.Lq != nullptr;
    if (qa && a.batch != 1) return hipErrorInvalidValue;
    if (qa && p.nbi == 6)
        hipLaunchKernelGGL((decode_split_kernel<true, 6>), dim3((unsigned)per, 1u), dim3(kSpThreads), 0, stream, a, p);
    else if (qa && p.nbi == 8)
        hipLaunchKernelGGL((decode_split_kernel<true, 8>), dim3((unsigned)per, 1u), dim3(kSpThreads), 0, stream, a, p);
    else if (qa)
        hipLaunchKernelGGL((decode_split_kernel<true, 4>), dim3((unsigned)per, 1u), dim3(kSpThreads), 0, stream, a, p);
    else if (p.nbi == 6)
        hipLaunchKernelGGL((decode_split_kernel<false, 6>), dim3((unsigned)per, (unsigned)a.batch), dim3(kSpThreads), 0, stream, a, p);
    else if (p.nbi == 8)
        hipLaunchKernelGGL((decode_split_kernel<false, 8>), dim3((unsigned)per, (unsigned)a.batch), dim3(kSpThreads), 0, stream, a, p);
    else
        hipLaunchKernelGGL((decode_split_kernel<false, 4>), dim3((unsigned)per, (unsigned)a.batch), dim3(kSpThreads), 0, stream, a, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // Three 16-row blocks per finishing workgroup when one block each would
    // take more than one round of the 256 CUs.
    const bool fin3 = a.N / 16 > 256;
    const dim3 grid((unsigned)(fin3 ? (a.N / 16 + 2) / 3 : a.N / 16), (unsigned)a.batch), block(kSpThreads);
#define SLIM_FIN(S_)                                                                                          \
    do {                                                                                                      \
        if (fin3) {                                                                                           \
            if (qa) hipLaunchKernelGGL((decode_finish_kernel<S_, true, 3>), grid, block, 0, stream, a, p);    \
            else    hipLaunchKernelGGL((decode_finish_kernel<S_, false, 3>), grid, block, 0, stream, a, p);   \
        } else {                                                                                              \
            if (qa) hipLaunchKernelGGL((decode_finish_kernel<S_, true, 1>), grid, block, 0, stream, a, p);    \
            else    hipLaunchKernelGGL((decode_finish_kernel<S_, false, 1>), grid, block, 0, stream, a, p);   \
        }                                                                                                     \
    } while (0)
    switch (p.S) {
        case 1: SLIM_FIN(1); break;
        case 2: SLIM_FIN(2); break;
        case 4: SLIM_FIN(4); break;
        case 8: SLIM_FIN(8); break;
        default: SLIM_FIN(16); break;
    }
#undef SLIM_FIN
    return hipGetLastError();
}

}  // namespace slim
