// slim_linear for prefill-shaped problems (M > 16 tokens): MFMA-bound.
//
//   Y = X . deq(W_c)^T + (X . L) . R
//
// Layer: Compression Trinity thesis §2.1 (Y = X W^T) with the sparse weight
// and the low-rank adapter as parallel paths (Ch. 4 introduction); prefill is
// the compute-bound regime (§2.5.1), so the work goes to the matrix cores:
// 2:4 sparse MFMA for the main term (§2.2.3: only the kept half of W is
// multiplied), dense MFMA for the adapter.
//
// prefill_main_kernel: one 8-wave workgroup per 256 rows of W x 128 tokens
//   (each wave 64 rows x 64 tokens, two waves per SIMD).  K advances in
//   128-wide chunks (one scale group); a chunk's X tile, packed W and Lt tile
//   are staged through LDS two chunks ahead.  Each wave dequantises its W
//   fragments in registers and issues v_smfmac_f32_16x16x64_f16 with 4 row
//   fragments x 4 token fragments.
//   Workgroups of the first r/32 column blocks also compute a 128 x 32 block
//   of T = X . L from the same LDS tile with dense v_mfma_f32_16x16x32_f16
//   (Lt rows are the A operand).  Stores Y_main (fp16) and T (fp16).
// prefill_adapter_up_kernel: Y += T . R with dense MFMA, 128 x 128 output
//   tiles, the operands (rows of Rt and T) read with 16-byte loads.
#include "internal.hpp"
#include "mfma_util.hpp"

namespace slim {
namespace {

constexpr int kPN = 256;                 // W rows per workgroup
constexpr int kPM = 128;                 // tokens per workgroup
constexpr int kPK = 128;                 // k per chunk (one scale group)
constexpr int kPThreads = 256;           // 4 waves, one per SIMD: wave w owns W rows 64w..64w+63
constexpr int kLRows = 32;               // Lt rows (adapter columns) per T block
constexpr int kGroupM = 4;               // m-blocks per XCD group of tiles

// LDS stage (bytes).  Row pitches keep every read pattern bank-conflict free:
// X / Lt rows 272 B (16-byte reads of 8 consecutive rows hit 8 distinct bank
// quads), values rows 40 B (8-byte reads of 16 rows: distinct bank pairs),
// metadata rows 24 B (4-byte reads of 16 rows x 2 columns: distinct banks).
constexpr int kXPitch = kPK + 8;                               // halfs
constexpr int kVPitch = 40, kMPitch = 24;                      // bytes
constexpr int kXOff = 0, kXBytes = kPM * kXPitch * 2;
constexpr int kLOff = kXOff + kXBytes, kLBytes = kLRows * kXPitch * 2;
constexpr int kVOff = kLOff + kLBytes, kVBytes = kPN * kVPitch;
constexpr int kMOff = kVOff + kVBytes, kMBytes = kPN * kMPitch;
constexpr int kSOff = kMOff + kMBytes, kSBytes = kPN * 2;
constexpr int kStageBytes = kSOff + kSBytes;
static_assert(2 * kStageBytes <= 160 * 1024, "two stages must fit in LDS");

// Global pieces per thread and chunk: X 8 x 16 B, Lt 2 x 16 B, values 2 x 16 B,
// metadata 16 B, one scale.
constexpr int kXPieces = kPM * kPK * 2 / 16 / kPThreads;       // 8
constexpr int kLPieces = kLRows * kPK * 2 / 16 / kPThreads;    // 2
constexpr int kVPieces = kPN * kPK / 4 / 16 / kPThreads;       // 2
static_assert(kXPieces == 8 && kLPieces == 2 && kVPieces == 2, "piece counts");

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit elements (gfx9 family)

struct PrefillPlan {
    size_t t_off, total;
};

PrefillPlan prefill_plan(int64_t M, int64_t r) {
    PrefillPlan p;
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    p.t_off = kCounterRegion;
    p.total = p.t_off + al((size_t)M * (size_t)r * 2);
    return p;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    // Accesses at or past `bytes` read zero without touching memory.
    const int n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, (int)kRsrcWord3);
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

// ------------------------------------------------------------ main kernel
// Software pipeline per 128-k chunk ch with two LDS stages and two register
// sets: iteration ch issues the buffer loads of chunk ch+2 into one register
// set, computes chunk ch from LDS, writes the other register set (chunk ch+1,
// issued one iteration earlier) to the other stage, then synchronises.  A
// chunk's loads have two iterations to land.  Loads are raw buffer loads: the
// per-thread offsets are fixed, the chunk moves a scalar offset, and rows past
// M or N (or the Lt tile of a workgroup without a T block) read zero.
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_main_kernel(LinearArgs a, size_t t_off) {
    const int b = blockIdx.y;
    const int64_t K = a.K, N = a.N, M = a.M;
    const int nNB = (int)((N + kPN - 1) / kPN), nMB = (int)((M + kPM - 1) / kPM);
    // XCD-aware tile order: each XCD runs a contiguous range of logical tiles,
    // grouped kGroupM m-blocks at a time so that X and W tiles are shared in L2.
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int gsize = kGroupM * nNB, gid = L / gsize, fm = gid * kGroupM;
    const int gm = nMB - fm < kGroupM ? nMB - fm : kGroupM;
    const int mb = fm + (L % gsize) % gm, nb = (L % gsize) / gm;
    const int64_t n0 = (int64_t)nb * kPN, m0 = (int64_t)mb * kPM;
    const int nchunks = (int)(K / kPK);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nl = lane & 15, G = lane >> 4;
    const int nR = (int)(a.r / kLRows);
    const bool do_t = nb < nR;

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStageBytes];

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X + b * a.sX + m0 * K, (M - m0) * K * 2);
    const __amdgpu_buffer_rsrc_t rl =
        make_rsrc(do_t ? a.Lt + b * a.sLt + (int64_t)kLRows * nb * K : a.X, do_t ? (int64_t)kLRows * K * 2 : 0);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.values + b * a.sV + n0 * (K / 4), (N - n0) * (K / 4));
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.meta + b * a.sMeta + n0 * (K / 8), (N - n0) * (K / 8));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales + b * a.sS + n0 * (K / kGroup), (N - n0) * (K / kGroup) * 2);

    // Fixed per-thread byte offsets (piece c = tid + 256 i).
    int ox[kXPieces], ol[kLPieces], ov[kVPieces];
#pragma unroll
    for (int i = 0; i < kXPieces; ++i) {
        const int c = tid + kPThreads * i;
        ox[i] = (int)(((c >> 4) * K + 8 * (c & 15)) * 2);
    }
#pragma unroll
    for (int i = 0; i < kLPieces; ++i) {
        const int c = tid + kPThreads * i;
        ol[i] = (int)(((c >> 4) * K + 8 * (c & 15)) * 2);
    }
#pragma unroll
    for (int i = 0; i < kVPieces; ++i) {
        const int c = tid + kPThreads * i;
        ov[i] = (int)((c >> 1) * (K / 4) + 16 * (c & 1));
    }
    const int om = (int)(tid * (K / 8));
    const int os = (int)(tid * (K / kGroup) * 2);

    struct Stage {
        h8 x[kXPieces], l[kLPieces], v[kVPieces], m;
        uint32_t s;
    };
    auto load_stage = [&](int ch, Stage& st) {
        ch = ch < nchunks ? ch : nchunks - 1;
#pragma unroll
        for (int i = 0; i < kXPieces; ++i)
            st.x[i] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rx, ox[i], ch * kPK * 2, 0));
#pragma unroll
        for (int i = 0; i < kLPieces; ++i)
            st.l[i] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rl, ol[i], ch * kPK * 2, 0));
#pragma unroll
        for (int i = 0; i < kVPieces; ++i)
            st.v[i] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rv, ov[i], ch * (kPK / 4), 0));
        st.m = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rm, om, ch * (kPK / 8), 0));
        st.s = __builtin_amdgcn_raw_buffer_load_b16(rs, os, ch * 2, 0);
    };
    auto store_stage = [&](int buf, const Stage& st) {
        unsigned char* sm = smem + buf * kStageBytes;
        _Float16* xs = reinterpret_cast<_Float16*>(sm + kXOff);
        _Float16* ls = reinterpret_cast<_Float16*>(sm + kLOff);
#pragma unroll
        for (int i = 0; i < kXPieces; ++i) {
            const int c = tid + kPThreads * i;
            *reinterpret_cast<h8*>(xs + (c >> 4) * kXPitch + 8 * (c & 15)) = st.x[i];
        }
        if (do_t) {
#pragma unroll
            for (int i = 0; i < kLPieces; ++i) {
                const int c = tid + kPThreads * i;
                *reinterpret_cast<h8*>(ls + (c >> 4) * kXPitch + 8 * (c & 15)) = st.l[i];
            }
        }
#pragma unroll
        for (int i = 0; i < kVPieces; ++i) {
            const int c = tid + kPThreads * i;
            u2* dst = reinterpret_cast<u2*>(sm + kVOff + (c >> 1) * kVPitch + 16 * (c & 1));
            const u4 v = __builtin_bit_cast(u4, st.v[i]);
            dst[0] = u2{v[0], v[1]};
            dst[1] = u2{v[2], v[3]};
        }
        {
            u2* dst = reinterpret_cast<u2*>(sm + kMOff + tid * kMPitch);
            const u4 m = __builtin_bit_cast(u4, st.m);
            dst[0] = u2{m[0], m[1]};
            dst[1] = u2{m[2], m[3]};
        }
        reinterpret_cast<uint16_t*>(sm + kSOff)[tid] = (uint16_t)st.s;
    };

    f4 acc[4][8];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 8; ++g) acc[f][g] = f4{0, 0, 0, 0};
    f4 acct[2][2] = {{{0, 0, 0, 0}, {0, 0, 0, 0}}, {{0, 0, 0, 0}, {0, 0, 0, 0}}};

    const int gA1 = G >> 1, gA2 = 2 + (G >> 1), hoff = 8 * (G & 1);
    auto compute = [&](int buf) {
        const unsigned char* sm = smem + buf * kStageBytes;
        const _Float16* xt = reinterpret_cast<const _Float16*>(sm + kXOff);
        // This lane's W rows 64*wave + 16f + nl, blocks 2G (t = 0) and 2G+1 (t = 1).
        h8 A[4][2];
        uint32_t mw[4];
        h8 TL[4][2], TX[4][2];
        if (do_t) {
            const _Float16* lt = reinterpret_cast<const _Float16*>(sm + kLOff);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                TL[s][0] = *reinterpret_cast<const h8*>(lt + nl * kXPitch + 32 * s + 8 * G);
                TL[s][1] = *reinterpret_cast<const h8*>(lt + (16 + nl) * kXPitch + 32 * s + 8 * G);
#pragma unroll
                for (int mf = 0; mf < 2; ++mf)
                    TX[s][mf] = *reinterpret_cast<const h8*>(xt + (32 * wave + 16 * mf + nl) * kXPitch + 32 * s + 8 * G);
            }
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int rr = 64 * wave + 16 * f + nl;
            const u2 vw = *reinterpret_cast<const u2*>(sm + kVOff + rr * kVPitch + 8 * G);
            mw[f] = *reinterpret_cast<const uint32_t*>(sm + kMOff + rr * kMPitch + 4 * G);
            const _Float16 sv = reinterpret_cast<const _Float16*>(sm + kSOff)[rr];
            const h2 s2 = {sv, sv};
            dequant_word_fast(vw[0], s2, A[f][0]);
            dequant_word_fast(vw[1], s2, A[f][1]);
        }
        // 16 steps q = 8t + g (t: k-half, g: token fragment); the B operand of
        // step q + 2 is read from LDS while step q's four smfmac run.
        auto readB = [&](int q) {
            const int t = q >> 3, g = q & 7;
            const _Float16* xrow = xt + (16 * g + nl) * kXPitch;
            return concat8(*reinterpret_cast<const h8*>(xrow + 16 * (2 * gA1 + t) + hoff),
                           *reinterpret_cast<const h8*>(xrow + 16 * (2 * gA2 + t) + hoff));
        };
        h16 Bq[3];
        Bq[0] = readB(0);
        Bq[1] = readB(1);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            if (q + 2 < 16) Bq[(q + 2) % 3] = readB(q + 2);
            const h16 B = Bq[q % 3];
            const int g = q & 7;
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                if (q < 8) acc[f][g] = smfmac<0>(A[f][0], B, acc[f][g], mw[f]);
                else       acc[f][g] = smfmac<1>(A[f][1], B, acc[f][g], mw[f]);
            }
        }
        if (do_t) {
            // T^T[j][m] += Lt[j][k] X[m][k] for this wave's tokens 32*wave + 16*mf + nl;
            // the 16 operands were read with the W words at the top.
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int mf = 0; mf < 2; ++mf) {
                    acct[0][mf] = mfma16(TL[s][0], TX[s][mf], acct[0][mf]);
                    acct[1][mf] = mfma16(TL[s][1], TX[s][mf], acct[1][mf]);
                }
        }
    };

    Stage s0, s1;
    load_stage(0, s0);
    load_stage(1, s1);
    store_stage(0, s0);
    __syncthreads();
    auto step = [&](int ch, Stage& issue, const Stage& ready) {
        load_stage(ch + 2, issue);
        __builtin_amdgcn_sched_barrier(0);             // the prefetch goes out before the compute
        if (ch < nchunks) compute(ch & 1);
        store_stage((ch + 1) & 1, ready);
        __syncthreads();
    };
    for (int ch = 0; ch < nchunks; ch += 2) {
        step(ch, s0, s1);
        step(ch + 1, s1, s0);
    }

    // Y_main: lane holds rows n = 4G+v of fragment f, token 16g + nl.
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        const int64_t m = m0 + 16 * g + nl;
        if (m >= M) continue;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int64_t n = n0 + 64 * wave + 16 * f + 4 * G;
            if (n >= N) continue;
            const h4 out = {(_Float16)acc[f][g][0], (_Float16)acc[f][g][1], (_Float16)acc[f][g][2],
                            (_Float16)acc[f][g][3]};
            *reinterpret_cast<h4*>(a.Y + b * a.sY + m * N + n) = out;
        }
    }
    if (do_t) {
        _Float16* T = reinterpret_cast<_Float16*>(a.ws + b * a.ws_per_problem + t_off);
#pragma unroll
        for (int mf = 0; mf < 2; ++mf) {
            const int64_t m = m0 + 32 * wave + 16 * mf + nl;
            if (m >= M) continue;
#pragma unroll
            for (int jf = 0; jf < 2; ++jf) {
                const int64_t j = (int64_t)kLRows * nb + 16 * jf + 4 * G;
                const h4 out = {(_Float16)acct[jf][mf][0], (_Float16)acct[jf][mf][1], (_Float16)acct[jf][mf][2],
                                (_Float16)acct[jf][mf][3]};
                *reinterpret_cast<h4*>(T + m * a.r + j) = out;
            }
        }
    }
}

// ------------------------------------------------------- Y += T . R
// prefill_adapter_up_kernel: a 256 (rows of Rt) x 128 (tokens) output tile
// per workgroup of 4 waves (wave w: 64 rows x 128 tokens, 4 x 8 fragments of
// v_mfma_f32_16x16x32_f16).  T [M][r] (fp16, from the main kernel) and Rt
// [N][r] stream through LDS 64 columns of r at a time (columns past r read
// zero), with kUDepth chunks of loads in flight.  Y is read and written in
// whole 16-byte pieces of token rows: after the product, its tile is fetched
// while the fp32 product goes through LDS (half the tokens at a time), so that
// each thread adds and stores contiguous pieces.
constexpr int kUCols = 64;                       // columns of r per chunk
constexpr int kUPitch = kUCols + 8;              // halfs per LDS row (144 B: 16-byte reads of 8 rows are conflict free)
constexpr int kUTBytes = kPM * kUPitch * 2, kURBytes = kPN * kUPitch * 2;
constexpr int kUStage = kUTBytes + kURBytes;
constexpr int kUDepth = 2;                       // chunks whose loads are in flight
constexpr int kUTPieces = kPM * kUCols * 2 / 16 / kPThreads;     // 4
constexpr int kURPieces = kPN * kUCols * 2 / 16 / kPThreads;     // 8
constexpr int kUOutPitch = kPN + 4;              // floats per token row of the LDS output tile
constexpr int kUOutBytes = kPM / 2 * kUOutPitch * 4;
static_assert(kUOutBytes <= 2 * kUStage, "output half-tile reuses the stage buffers");

__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_adapter_up_kernel(LinearArgs a, size_t t_off) {
    const int b = blockIdx.y;
    const int64_t N = a.N, M = a.M, r = a.r;
    const int nNB = (int)((N + kPN - 1) / kPN), nMB = (int)((M + kPM - 1) / kPM);
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int gsize = kGroupM * nNB, gid = L / gsize, fm = gid * kGroupM;
    const int gm = nMB - fm < kGroupM ? nMB - fm : kGroupM;
    const int mb = fm + (L % gsize) % gm, nb = (L % gsize) / gm;
    const int64_t n0 = (int64_t)nb * kPN, m0 = (int64_t)mb * kPM;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nl = lane & 15, G = lane >> 4;
    const int nch = (int)((r + kUCols - 1) / kUCols);

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kUStage];
    const uint16_t* Tg = reinterpret_cast<const uint16_t*>(a.ws + b * a.ws_per_problem + t_off);
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(Tg + m0 * r, (M - m0) * r * 2);
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.Rt + b * a.sRt + n0 * r, (N - n0) * r * 2);
    // Pieces of a 64-column chunk: 8 per row; piece i of this thread is row
    // (tid >> 3) + 32 i, columns 8 (tid & 7) .. +8 of the chunk.  The row is
    // part of the per-lane offset (the buffer range check applies to it, so
    // rows past M or N read zero); the chunk's column is the scalar offset.  A
    // piece whose columns lie past r (only in the last chunk) is read at an
    // offset past the buffer: zero.
    constexpr int kOOB = 0x7FFFFFF0;
    const int pcol = 8 * (tid & 7);
    int pt[kUTPieces], pr[kURPieces];
#pragma unroll
    for (int i = 0; i < kUTPieces; ++i) pt[i] = (int)((((tid >> 3) + 32 * i) * r + pcol) * 2);
#pragma unroll
    for (int i = 0; i < kURPieces; ++i) pr[i] = (int)((((tid >> 3) + 32 * i) * r + pcol) * 2);
    struct UStage {
        h8 t[kUTPieces], r[kURPieces];
    };
    auto load_stage = [&](int ch, UStage& st) {
        ch = ch < nch ? ch : nch - 1;
        const int col0 = ch * kUCols;
        const bool cok = col0 + pcol < r;
#pragma unroll
        for (int i = 0; i < kUTPieces; ++i)
            st.t[i] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rt, cok ? pt[i] : kOOB, col0 * 2, 0));
#pragma unroll
        for (int i = 0; i < kURPieces; ++i)
            st.r[i] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rr, cok ? pr[i] : kOOB, col0 * 2, 0));
    };
    auto store_stage = [&](int buf, const UStage& st) {
        _Float16* ts = reinterpret_cast<_Float16*>(smem + buf * kUStage);
        _Float16* rs = reinterpret_cast<_Float16*>(smem + buf * kUStage + kUTBytes);
#pragma unroll
        for (int i = 0; i < kUTPieces; ++i) {
            const int c = tid + kPThreads * i;
            *reinterpret_cast<h8*>(ts + (c >> 3) * kUPitch + 8 * (c & 7)) = st.t[i];
        }
#pragma unroll
        for (int i = 0; i < kURPieces; ++i) {
            const int c = tid + kPThreads * i;
            *reinterpret_cast<h8*>(rs + (c >> 3) * kUPitch + 8 * (c & 7)) = st.r[i];
        }
    };

    f4 acc[4][8];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 8; ++g) acc[f][g] = f4{0, 0, 0, 0};
    auto compute = [&](int buf) {
        const _Float16* ts = reinterpret_cast<const _Float16*>(smem + buf * kUStage);
        const _Float16* rs = reinterpret_cast<const _Float16*>(smem + buf * kUStage + kUTBytes);
#pragma unroll
        for (int s = 0; s < kUCols / 32; ++s) {
            h8 A[4], B[8];
#pragma unroll
            for (int f = 0; f < 4; ++f)
                A[f] = *reinterpret_cast<const h8*>(rs + (64 * wave + 16 * f + nl) * kUPitch + 32 * s + 8 * G);
#pragma unroll
            for (int g = 0; g < 8; ++g) B[g] = *reinterpret_cast<const h8*>(ts + (16 * g + nl) * kUPitch + 32 * s + 8 * G);
#pragma unroll
            for (int g = 0; g < 8; ++g)
#pragma unroll
                for (int f = 0; f < 4; ++f) acc[f][g] = mfma16(A[f], B[g], acc[f][g]);
        }
    };

    // Register stage ring: set i % kUDepth holds chunk i from its load (issued
    // kUDepth - 1 iterations ahead) until it is written to LDS buffer i % 2.
    UStage ring[kUDepth];
#pragma unroll
    for (int i = 0; i < kUDepth; ++i) load_stage(i, ring[i]);

    store_stage(0, ring[0]);
    __syncthreads();
    for (int base = 0; base < nch; base += kUDepth) {
#pragma unroll
        for (int u = 0; u < kUDepth; ++u) {
            const int ch = base + u;
            if (ch >= nch) break;                      // uniform: every thread leaves together
            // ring[u] (chunk ch) went to LDS one iteration ago: reuse it for chunk ch + kUDepth.
            load_stage(ch + kUDepth, ring[u]);
            __builtin_amdgcn_sched_barrier(0);
            compute(ch & 1);
            store_stage((ch + 1) & 1, ring[(u + 1) % kUDepth]);
            __syncthreads();
        }
    }

    // This thread's pieces of the Y tile: token row (tid >> 2) + 64 h of the
    // tile, 64 consecutive columns starting at 64 (tid & 3), as 8 x 16 B,
    // fetched now (their latency overlaps the first LDS transpose).
    // Columns past N or tokens past M are not read (zero) and not stored.
    const int orow = tid >> 2, ocol = 64 * (tid & 3);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.Y + b * a.sY + m0 * N, (M - m0) * N * 2);
    h8 yv[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int64_t n = n0 + ocol + 8 * q;
            const int off = n < N ? (int)(((orow + 64 * h) * N + n) * 2) : kOOB;
            yv[h][q] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(ry, off, 0, 0));
        }

    // Output, half the tokens at a time: the accumulators (token 16g + nl, rows
    // 64 wave + 16f + 4G + v) go to an fp32 LDS tile, then each thread adds its
    // 64 contiguous columns of one token row to Y and stores them.
    float* ot_lds = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int f = 0; f < 4; ++f)
                *reinterpret_cast<f4*>(ot_lds + (16 * g + nl) * kUOutPitch + 64 * wave + 16 * f + 4 * G) = acc[f][4 * h + g];
        __syncthreads();
        const int64_t m = m0 + orow + 64 * h;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int64_t n = n0 + ocol + 8 * q;
            const f4 lo = *reinterpret_cast<const f4*>(ot_lds + orow * kUOutPitch + ocol + 8 * q);
            const f4 hi = *reinterpret_cast<const f4*>(ot_lds + orow * kUOutPitch + ocol + 8 * q + 4);
            const h8 y = yv[h][q];
            h8 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                out[e] = (_Float16)((float)y[e] + lo[e]);
                out[4 + e] = (_Float16)((float)y[4 + e] + hi[e]);
            }
            if (m < M && n < N) *reinterpret_cast<h8*>(a.Y + b * a.sY + m * N + n) = out;
        }
        __syncthreads();
    }
}

}  // namespace

size_t prefill_workspace_bytes(int64_t M, int64_t r) { return prefill_plan(M, r).total; }

bool prefill_fits(const LinearArgs& a) {
    // The T blocks are produced by the first r/32 column blocks of W; every
    // buffer that a workgroup addresses with 32-bit offsets stays below 2 GiB.
    const int64_t lim = 0x7FFFFFF0;
    return a.M > 16 && (a.r / kLRows) <= (a.N + kPN - 1) / kPN && a.M * a.K * 2 < lim &&
           (int64_t)kLRows * a.K * 2 < lim && a.N * (a.K / 4) < lim && a.M < (1LL << 31) / kPM;
}

hipError_t launch_linear_prefill(const LinearArgs& a, hipStream_t stream) {
    const PrefillPlan p = prefill_plan(a.M, a.r);
    const unsigned tiles = (unsigned)(((a.N + kPN - 1) / kPN) * ((a.M + kPM - 1) / kPM));
    hipLaunchKernelGGL(prefill_main_kernel, dim3(tiles, (unsigned)a.batch), dim3(kPThreads), 0, stream, a, p.t_off);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.r == 0) return e;
    hipLaunchKernelGGL(prefill_adapter_up_kernel, dim3(tiles, (unsigned)a.batch), dim3(kPThreads), 0, stream, a, p.t_off);
    return hipGetLastError();
}

}  // namespace slim
