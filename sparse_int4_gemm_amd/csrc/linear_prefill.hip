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
constexpr int kPK = 128;                 // k per chunk
constexpr int kPWaves = 8;                 // 4 along W rows x 2 along tokens
constexpr int kXPitch = kPK + 8;         // LDS row pitch in halfs (272 B: rows shift banks)

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

// ------------------------------------------------------------ main kernel
// Software pipeline per 128-k chunk ch, LDS holding 2 stage buffers.  A stage
// is the chunk's X tile (128 tokens x 128 k), the Lt tile of the workgroup's
// T block (32 x 128 k) and the packed W of its 256 rows (values, metadata,
// scales).  Iteration ch: issue the global loads of stage ch+2 into register
// set ch%2; compute chunk ch from LDS; write register set (ch+1)%2 (stage
// ch+1, issued one iteration earlier) to the other buffer; barrier.  Every
// global load has about two chunks of compute to land.
constexpr int kRows = kPM + 32;                    // X rows then Lt rows
constexpr int kXHalfs = kRows * kXPitch;
constexpr int kVBytes = kPN * 32;                  // values of 256 rows, 128 k
constexpr int kMBytes = kPN * 16;                  // metadata
constexpr int kSBytes = kPN * 2;                   // scales
constexpr int kStageBytes = kXHalfs * 2 + kVBytes + kMBytes + kSBytes;

__global__ __launch_bounds__(64 * kPWaves) void prefill_main_kernel(LinearArgs a, size_t t_off) {
    const int b = blockIdx.z;
    const int nb = blockIdx.x, mb = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave & 3, wm = wave >> 2;           // 64 W rows x 64 tokens per wave
    const int nl = lane & 15, G = lane >> 4;
    const int64_t K = a.K, N = a.N, M = a.M;
    const int64_t n0 = (int64_t)nb * kPN, m0 = (int64_t)mb * kPM;
    const int nchunks = (int)(K / kPK);
    const int tid = threadIdx.x;

    __shared__ __attribute__((aligned(16))) unsigned char smem[2][kStageBytes];

    const int nR = (int)(a.r / 32);
    const bool do_t = nb < nR;
    const bool have_lt = nR > 0;
    const uint16_t* Xb = a.X + b * a.sX;
    // With no adapter, the Lt pieces are read from X (any valid address) and
    // never used: every stage load stays unconditional.
    const uint16_t* Ltb = have_lt ? a.Lt + b * a.sLt + (int64_t)32 * (do_t ? nb : 0) * K : a.X + b * a.sX;
    const int64_t lt_rows = have_lt ? 32 : 1;
    const uint8_t* Vb = a.values + b * a.sV;
    const uint8_t* Mb = a.meta + b * a.sMeta;
    const uint16_t* Sb = a.scales + b * a.sS;

    // 16-byte pieces of a stage for this thread (512 threads):
    //  p0..3 : X row (c>>4), 16-byte column (c&15), c = tid + 512 i
    //  p4    : Lt row (tid>>4)  (Lt rows 0..31)
    //  p5    : values, W row (tid>>1), half (tid&1)
    //  p6    : metadata of W row tid            (tid < 256)
    //  sc    : scale of W row tid               (tid < 256)
    struct Stage {
        h8 p[7];
        uint32_t sc;
    };
    const bool wthr = tid < kPN;
    auto wrow = [&](int rr) {
        int64_t row = n0 + rr;
        return row < N ? row : N - 1;                  // rows past N: clamped, never stored
    };
    auto load_stage = [&](int ch, Stage& st) {
        ch = ch < nchunks ? ch : nchunks - 1;
        const int64_t k0 = (int64_t)ch * kPK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 512 * i;
            int64_t m = m0 + (c >> 4);
            m = m < M ? m : M - 1;                     // tokens past M: clamped, never stored
            st.p[i] = load_h8(Xb + m * K + k0 + 8 * (c & 15));
        }
        st.p[4] = load_h8(Ltb + (int64_t)((tid >> 4) % lt_rows) * K + k0 + 8 * (tid & 15));
        st.p[5] = *reinterpret_cast<const h8*>(Vb + wrow(tid >> 1) * (K / 4) + k0 / 4 + 16 * (tid & 1));
        const int wr = wthr ? tid : 0;
        st.p[6] = *reinterpret_cast<const h8*>(Mb + wrow(wr) * (K / 8) + k0 / 8);
        st.sc = Sb[wrow(wr) * (K / kGroup) + ch];
    };
    auto store_stage = [&](int buf, const Stage& st) {
        unsigned char* sm = smem[buf];
        _Float16* xs = reinterpret_cast<_Float16*>(sm);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 512 * i;
            *reinterpret_cast<h8*>(xs + (c >> 4) * kXPitch + 8 * (c & 15)) = st.p[i];
        }
        if (have_lt) *reinterpret_cast<h8*>(xs + (kPM + (tid >> 4)) * kXPitch + 8 * (tid & 15)) = st.p[4];
        unsigned char* vs = sm + kXHalfs * 2;
        *reinterpret_cast<h8*>(vs + 16 * tid) = st.p[5];               // row tid>>1: 32 bytes
        if (wthr) {
            *reinterpret_cast<h8*>(vs + kVBytes + 16 * tid) = st.p[6];
            reinterpret_cast<uint16_t*>(vs + kVBytes + kMBytes)[tid] = (uint16_t)st.sc;
        }
    };

    f4 acc[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[f][g] = f4{0, 0, 0, 0};
    f4 acct[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};

    const int gA1 = G >> 1, gA2 = 2 + (G >> 1), hoff = 8 * (G & 1);
    auto compute = [&](int buf) {
        const unsigned char* sm = smem[buf];
        const _Float16* xt = reinterpret_cast<const _Float16*>(sm);
        const unsigned char* vs = sm + kXHalfs * 2;
        // This lane's W data: rows 64*wn + 16f + nl, blocks 2G and 2G+1.
        u2 vw[4];
        uint32_t mw[4];
        h2 s2[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int rr = 64 * wn + 16 * f + nl;
            vw[f] = *reinterpret_cast<const u2*>(vs + 32 * rr + 8 * G);
            mw[f] = *reinterpret_cast<const uint32_t*>(vs + kVBytes + 16 * rr + 4 * G);
            const _Float16 sv = reinterpret_cast<const _Float16*>(vs + kVBytes + kMBytes)[rr];
            s2[f] = h2{sv, sv};
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            h8 A[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) A[f] = dequant_word(vw[f][t], s2[f]);
            // B operand (tokens 64wm + 16g + nl): window k 8G'.. of A-group
            // G'/2 and 32 + 8G'.. of A-group 2 + G'/2; A-group q holds block 2q + t.
            const int k1 = 16 * (2 * gA1 + t) + hoff;
            const int k2 = 16 * (2 * gA2 + t) + hoff;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const _Float16* xrow = xt + (64 * wm + 16 * g + nl) * kXPitch;
                const h16 B = concat8(*reinterpret_cast<const h8*>(xrow + k1),
                                      *reinterpret_cast<const h8*>(xrow + k2));
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    if (t == 0) acc[f][g] = smfmac<0>(A[f], B, acc[f][g], mw[f]);
                    else        acc[f][g] = smfmac<1>(A[f], B, acc[f][g], mw[f]);
                }
            }
        }
        if (do_t) {
            // T^T[j][m] += Lt[j][k] X[m][k]; this wave's token fragment is 16*wave.
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const h8 L0 = *reinterpret_cast<const h8*>(xt + (kPM + nl) * kXPitch + 32 * s + 8 * G);
                const h8 L1 = *reinterpret_cast<const h8*>(xt + (kPM + 16 + nl) * kXPitch + 32 * s + 8 * G);
                const h8 Bx = *reinterpret_cast<const h8*>(xt + (16 * wave + nl) * kXPitch + 32 * s + 8 * G);
                acct[0] = mfma16(L0, Bx, acct[0]);
                acct[1] = mfma16(L1, Bx, acct[1]);
            }
        }
    };

    Stage s0, s1;
    load_stage(0, s0);
    load_stage(1, s1);
    store_stage(0, s0);
    __syncthreads();
    // Global loads are never under a branch (the chunk index is clamped), so
    // the compiler's memory-counter waits only cover the stage being stored
    // and the prefetch stays in flight.  Only compute is guarded.
    auto step = [&](int ch, Stage& issue, const Stage& ready) {
        load_stage(ch + 2, issue);
        if (ch < nchunks) compute(ch & 1);
        store_stage((ch + 1) & 1, ready);
        __syncthreads();
    };
    for (int ch = 0; ch < nchunks; ch += 2) {
        step(ch, s0, s1);
        step(ch + 1, s1, s0);
    }

    // Y_main: lane holds rows n = 4G+v of fragment f, token 64wm + 16g + nl.
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int64_t m = m0 + 64 * wm + 16 * g + nl;
        if (m >= M) continue;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int64_t n = n0 + 64 * wn + 16 * f + 4 * G;
            if (n >= N) continue;
            const h4 out = {(_Float16)acc[f][g][0], (_Float16)acc[f][g][1], (_Float16)acc[f][g][2],
                            (_Float16)acc[f][g][3]};
            *reinterpret_cast<h4*>(a.Y + b * a.sY + m * N + n) = out;
        }
    }
    if (do_t) {
        _Float16* T = reinterpret_cast<_Float16*>(a.ws + b * a.ws_per_problem + t_off);
        const int64_t m = m0 + 16 * wave + nl;
        if (m < M) {
#pragma unroll
            for (int jf = 0; jf < 2; ++jf) {
                const int64_t j = 32 * nb + 16 * jf + 4 * G;
                const h4 out = {(_Float16)acct[jf][0], (_Float16)acct[jf][1], (_Float16)acct[jf][2],
                                (_Float16)acct[jf][3]};
                *reinterpret_cast<h4*>(T + m * a.r + j) = out;
            }
        }
    }
}

// ------------------------------------------------------- Y += T . R
constexpr int kUN = 128, kUM = 128;

__global__ __launch_bounds__(256) void prefill_adapter_up_kernel(LinearArgs a, size_t t_off) {
    const int b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nl = lane & 15, G = lane >> 4;
    const int wn = wave & 1, wm = wave >> 1;
    const int64_t N = a.N, M = a.M, r = a.r;
    const int64_t n0 = (int64_t)blockIdx.x * kUN + 64 * wn, m0 = (int64_t)blockIdx.y * kUM + 64 * wm;
    const uint16_t* Rt = a.Rt + b * a.sRt;
    const uint16_t* T = reinterpret_cast<const uint16_t*>(a.ws + b * a.ws_per_problem + t_off);
    const uint16_t* ap[4];
    const uint16_t* bp[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        int64_t n = n0 + 16 * f + nl;
        n = n < N ? n : N - 1;
        ap[f] = Rt + n * r + 8 * G;
        int64_t m = m0 + 16 * f + nl;
        m = m < M ? m : M - 1;
        bp[f] = T + m * r + 8 * G;
    }
    f4 acc[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[f][g] = f4{0, 0, 0, 0};
    const int nR = (int)(r / 32);
    h8 A[4], B[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        A[f] = load_h8(ap[f]);
        B[f] = load_h8(bp[f]);
    }
    for (int jb = 0; jb < nR; ++jb) {
        h8 An[4], Bn[4];
        const int jn = jb + 1 < nR ? jb + 1 : jb;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            An[f] = load_h8(ap[f] + 32 * jn);
            Bn[f] = load_h8(bp[f] + 32 * jn);
        }
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int g = 0; g < 4; ++g) acc[f][g] = mfma16(A[f], B[g], acc[f][g]);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            A[f] = An[f];
            B[f] = Bn[f];
        }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int64_t m = m0 + 16 * g + nl;
        if (m >= M) continue;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int64_t n = n0 + 16 * f + 4 * G;
            if (n >= N) continue;
            h4* yp = reinterpret_cast<h4*>(a.Y + b * a.sY + m * N + n);
            const h4 y = *yp;
            const h4 out = {(_Float16)((float)y[0] + acc[f][g][0]), (_Float16)((float)y[1] + acc[f][g][1]),
                            (_Float16)((float)y[2] + acc[f][g][2]), (_Float16)((float)y[3] + acc[f][g][3])};
            *yp = out;
        }
    }
}

}  // namespace

size_t prefill_workspace_bytes(int64_t M, int64_t r) { return prefill_plan(M, r).total; }

bool prefill_fits(const LinearArgs& a) {
    // The T blocks are produced by the first r/32 column blocks of W.
    return a.M > 16 && (a.r / 32) <= (a.N + kPN - 1) / kPN && a.M < (1LL << 31) / kPM;
}

hipError_t launch_linear_prefill(const LinearArgs& a, hipStream_t stream) {
    const PrefillPlan p = prefill_plan(a.M, a.r);
    dim3 grid((unsigned)((a.N + kPN - 1) / kPN), (unsigned)((a.M + kPM - 1) / kPM), (unsigned)a.batch);
    hipLaunchKernelGGL(prefill_main_kernel, grid, dim3(64 * kPWaves), 0, stream, a, p.t_off);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.r == 0) return e;
    dim3 g2((unsigned)((a.N + kUN - 1) / kUN), (unsigned)((a.M + kUM - 1) / kUM), (unsigned)a.batch);
    hipLaunchKernelGGL(prefill_adapter_up_kernel, g2, dim3(256), 0, stream, a, p.t_off);
    return hipGetLastError();
}

}  // namespace slim
