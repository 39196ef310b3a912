// slim_linear for decode-shaped problems (M <= 16 tokens): HBM-bound.
//
//   T = X . L                                   (adapter down)
//   Y = X . deq(W_c)^T + T . R                  (2:4 sparse MFMA + dense MFMA)
//
// Layer: Compression Trinity thesis §2.1 (Y = X W^T) with the sparse weight
// and the low-rank adapter as parallel paths (Ch. 4 introduction).  Decode is
// the memory-bound regime (§2.5.2): the kernels read every HBM byte once with
// wide loads and issue all of a wave's loads before its first wait.
//
// One or two tokens, one problem, workgroups all resident: ONE launch.  Each
// workgroup of decode_kernel<..., FUSED> also computes one or two rows of T
// (a dot product over all of K, reduced in the workgroup) and publishes them
// as tagged 64-bit entries in the reserved workspace bytes; once its main
// term is done it polls T until every entry carries this call's tag, then
// adds T . R.  Measured on MI355X: stores or atomics of many workgroups to
// one word are served one after another (tens of ns each), and a device-wide
// fence costs microseconds, so the hand-off uses neither: one 64-bit
// device-scope store per row of T, polled by one wave per workgroup.
// Otherwise two launches (adapter-down, then the main kernel).
//
// The adapter factors come output-major (Lt = L^T [r][K], Rt = R^T [N][r]), so
// every MFMA operand below is one contiguous 16-byte load per lane.
//
// adapter_down_gemv_kernel (M <= 2, two launches): T = X L as a
//   matrix-vector product.  One 256-thread workgroup per 2 columns of r over
//   all of K; each thread loads 16-byte pieces of both Lt rows and of the
//   token rows, forms fp32 dot products (v_dot2), and the workgroup reduces
//   them; T is stored complete (one "split").
// adapter_down_kernel (M > 2): one 16-wave workgroup per (16 columns of r, K split).
//   Waves take 32-k steps; per step the lane loads 8 k of one row of Lt (the
//   MFMA A operand) and 8 k of X, and issues one v_mfma_f32_16x16x32_f16
//   (tokens are the MFMA N side, zero-padded to 16).  The waves are reduced
//   in LDS and the fp32 partial of T is stored with plain stores.
// decode_kernel<NW, CPW, ADAPTER, KS, FUSED>: one workgroup of NW waves per 16
//   rows of W (XCD-aware order).  The waves split K into 256-wide chunks
//   (wave w owns chunks w, w+NW, ...).  Per chunk and lane: 16 B of packed
//   values, 8 B of metadata and one scale of its row, and 2 x 4 x 16 B of X
//   (buffer loads: lanes of padding tokens read zero without a memory
//   access).  Each 64-k step dequantises one values word in registers and
//   issues one v_smfmac_f32_16x16x64_f16 (W rows are the sparse A side,
//   tokens the B side).  The epilogue takes T for one 32-wide slice of r per
//   wave (the sum of KS partials, or the tagged entries) and adds T . R with
//   dense MFMA into the same accumulators (R was loaded at the start),
//   reduces the waves in LDS and stores fp16 Y.
#include <atomic>

#include "internal.hpp"
#include "mfma_util.hpp"

namespace slim {
namespace {

constexpr int kDecodeMaxM = 16;
constexpr int kDecodeWaves = 16;
constexpr int kDecodeMaxCPW = 4;
constexpr int kDownWaves = 16;
constexpr int kDownSPW = 4;              // 32-k steps per wave whose loads go out together
constexpr int kMaxKSplits = 4;
constexpr int kGemvMaxM = 2;             // tokens handled by the matrix-vector adapter-down
constexpr int kGemvCols = 2;             // columns of r per workgroup
constexpr int kGemvThreads = 256;
constexpr int kGemvUnroll = 4;           // 8-k pieces per thread and row in flight together
constexpr int kFusedTRows = 2;           // fused launch: rows of Lt per workgroup, at most
constexpr int kFusedPieces = 4;          // fused launch: 16-byte Lt pieces per thread, at most
constexpr int kMaxTagged = (int)((kCounterRegion - kTagBase) / 8);   // M * r entries, at most
constexpr int kPollUnroll = 8;           // tagged entries per lane and poll pass, loaded together

// ------------------------------------------------ hand-off of T (one launch)
// State in the reserved workspace bytes: the 64-bit epoch E at byte 0, the
// 64-bit give-up count at byte kGiveupOffset, and T as tagged 64-bit entries,
// entry (t, j) at byte kTagBase + 8 (t r + j): the fp16 value of T[t][j] in
// bits [0, 16) (T enters the T . R product in fp16, so rounding it here
// gives the same product) and the 48-bit tag E + 1 of the writing workgroup
// above it.  Every workgroup reads E, stores its rows of T tagged E + 1 and
// waits, bounded, until every entry carries E + 1.  At the end of its wait a
// workgroup that saw every entry and is workgroup 0, or that gave up, raises
// the epoch to its tag (atomic max: the epoch never decreases); one that
// gave up also counts itself and writes NaN to its rows of Y.
// Invariant: after every launch each tag ever written is at most the epoch,
// so no entry of an earlier call can carry the tag a later call waits for.
// (A workgroup that gives up raised the epoch to its own tag; one that saw
// every entry tagged E + 1 saw workgroup 0's, so workgroup 0 read the same E
// and raises the epoch to E + 1 whether it succeeds or gives up.)
constexpr unsigned long long kTagMask = (1ull << 48) - 1;

__device__ __forceinline__ unsigned long long tag_entry(unsigned long long want, float v) {
    return ((want & kTagMask) << 16) | (unsigned long long)__builtin_bit_cast(uint16_t, (_Float16)v);
}
__device__ __forceinline__ bool entry_tagged(unsigned long long e, unsigned long long want) {
    return (e >> 16) == (want & kTagMask);
}
__device__ __forceinline__ float entry_value(unsigned long long e) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(e & 0xFFFFu));
}
// End of one workgroup's wait (one lane calls it).
__device__ __forceinline__ void handoff_finish(unsigned char* ws, unsigned long long want, bool ok, bool first) {
    unsigned long long* epoch = reinterpret_cast<unsigned long long*>(ws);
    if (ok && !first) return;
    __hip_atomic_fetch_max(epoch, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!ok)
        __hip_atomic_fetch_add(reinterpret_cast<unsigned long long*>(ws + kGiveupOffset), 1ull, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}

struct DecodePlan {
    size_t t_off, total;
    int ksplits;                         // K splits of the adapter-down kernel
    bool fused = false;                  // T = X L inside the main launch
};

DecodePlan decode_plan(int64_t M, int64_t N, int64_t K, int64_t r) {
    (void)M;
    (void)N;
    DecodePlan p;
    int64_t S = M <= kGemvMaxM ? 1 : kMaxKSplits;  // adapter-down workgroups: (r/16) x S, or r/2
    const int64_t nsteps = K / 32;
    if (S > nsteps) S = nsteps;
    if (S < 1) S = 1;
    p.ksplits = (int)S;
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    p.t_off = kCounterRegion;
    p.total = p.t_off + al((size_t)S * kDecodeMaxM * (size_t)r * sizeof(float));
    return p;
}

// ----------------------------------------------------------------- T = X L
// Partial T of K split s for columns [16c, 16c+16): Tp[s][m][j] (fp32).
// T^T = Lt . X^T: the MFMA A operand is a 16 x 32 tile of Lt (rows j), the B
// operand 32 k of X per token; both are contiguous 16-byte loads.
__global__ __launch_bounds__(64 * kDownWaves) void adapter_down_kernel(LinearArgs a, int ksplits, size_t t_off) {
    const int b = blockIdx.y;
    const int nJ = (int)(a.r / 16);
    const int c = blockIdx.x % nJ;
    const int s = blockIdx.x / nJ;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int jl = lane & 15, G = lane >> 4;
    const bool mval = jl < a.M;
    const int64_t K = a.K;
    const uint16_t* X = a.X + b * a.sX + (int64_t)(mval ? jl : 0) * K + 8 * G;
    const uint16_t* Lt = a.Lt + b * a.sLt + (int64_t)(16 * c + jl) * K + 8 * G;

    const int nsteps = (int)(K / 32);
    const int st0 = (int)((int64_t)s * nsteps / ksplits);
    const int st1 = (int)((int64_t)(s + 1) * nsteps / ksplits);

    f4 acc = {0, 0, 0, 0};
    for (int base = st0 + wave; base < st1; base += kDownWaves * kDownSPW) {
        h8 xs[kDownSPW], ls[kDownSPW];
#pragma unroll
        for (int u = 0; u < kDownSPW; ++u) {
            const int st = base + kDownWaves * u;
            const int64_t k0 = (int64_t)(st < st1 ? st : st0) * 32;   // clamp: always valid
            xs[u] = load_h8(X + k0);
            ls[u] = load_h8(Lt + k0);
        }
#pragma unroll
        for (int u = 0; u < kDownSPW; ++u) {
            // A clamped duplicate step contributes zero.  Token columns m >= M
            // read row 0 of X; they are never stored and MFMA columns do not mix.
            const bool live = base + kDownWaves * u < st1;
            acc = mfma16(live ? ls[u] : h8{}, xs[u], acc);     // rows j = 4G+v, col m
        }
    }

    __shared__ f4 lds[kDownWaves * 64];
    lds[wave * 64 + lane] = acc;
    __syncthreads();
    const int t = threadIdx.x;
    if (t < 256) {
        const int ln = t >> 2, v = t & 3;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kDownWaves; ++w) sum += lds[w * 64 + ln][v];
        const int mm = ln & 15, j = 16 * c + 4 * (ln >> 4) + v;
        if (mm < a.M) {
            float* Tp = reinterpret_cast<float*>(a.ws + b * a.ws_per_problem + t_off);
            Tp[((size_t)s * kDecodeMaxM + mm) * a.r + j] = sum;
        }
    }
}

// ------------------------------------------- T = X L, one or two tokens
// QA: Lt given as int4 codes (per 8 k one uint32) with one fp16 scale per
// 128 k; the piece's codes are turned into fp16 and scaled in registers.
template <bool QA>
__global__ __launch_bounds__(kGemvThreads) void adapter_down_gemv_kernel(LinearArgs a, size_t t_off) {
    const int b = blockIdx.y;
    const int j0 = blockIdx.x * kGemvCols;
    const int tid = threadIdx.x;
    const int64_t K = a.K;
    const int npieces = (int)(K / 8);                  // 8-k pieces per row
    const uint16_t* X = a.X + b * a.sX;
    const uint16_t* L0 = QA ? nullptr : a.Lt + b * a.sLt + (int64_t)j0 * K;
    const uint16_t* L1 = QA ? nullptr : L0 + K;
    const bool two = a.M > 1;                          // uniform: a second token row
    float acc[kGemvMaxM][kGemvCols] = {};
    auto dot8 = [](const h8& u, const h8& v, float c) {
        c = __builtin_amdgcn_fdot2(h2{u[0], u[1]}, h2{v[0], v[1]}, c, false);
        c = __builtin_amdgcn_fdot2(h2{u[2], u[3]}, h2{v[2], v[3]}, c, false);
        c = __builtin_amdgcn_fdot2(h2{u[4], u[5]}, h2{v[4], v[5]}, c, false);
        return __builtin_amdgcn_fdot2(h2{u[6], u[7]}, h2{v[6], v[7]}, c, false);
    };
    const uint32_t* Q0 = QA ? reinterpret_cast<const uint32_t*>(a.Lq) + (int64_t)j0 * npieces : nullptr;
    const _Float16* S0 = QA ? reinterpret_cast<const _Float16*>(a.Ls) + (int64_t)j0 * (K / kGroup) : nullptr;
    for (int base = tid; base < npieces; base += kGemvThreads * kGemvUnroll) {
        h8 l0[kGemvUnroll], l1[kGemvUnroll], x0[kGemvUnroll], x1[kGemvUnroll];
#pragma unroll
        for (int u = 0; u < kGemvUnroll; ++u) {        // clamped: always in bounds
            const int c = base + kGemvThreads * u;
            const int cc = c < npieces ? c : base;
            const int64_t k = 8 * (int64_t)cc;
            if constexpr (QA) {
                const _Float16 s0 = S0[cc / 16], s1 = S0[K / kGroup + cc / 16];
                l0[u] = dequant_word(Q0[cc], h2{s0, s0});
                l1[u] = dequant_word(Q0[npieces + cc], h2{s1, s1});
            } else {
                l0[u] = load_h8(L0 + k);
                l1[u] = load_h8(L1 + k);
            }
            x0[u] = load_h8(X + k);
            x1[u] = two ? load_h8(X + K + k) : x0[u];
        }
#pragma unroll
        for (int u = 0; u < kGemvUnroll; ++u) {
            if (base + kGemvThreads * u < npieces) {
                acc[0][0] = dot8(l0[u], x0[u], acc[0][0]);
                acc[0][1] = dot8(l1[u], x0[u], acc[0][1]);
                acc[1][0] = dot8(l0[u], x1[u], acc[1][0]);
                acc[1][1] = dot8(l1[u], x1[u], acc[1][1]);
            }
        }
    }
    // Reduce the 256 threads: within each wave by shuffles, then over waves.
#pragma unroll
    for (int m = 0; m < kGemvMaxM; ++m)
#pragma unroll
        for (int c = 0; c < kGemvCols; ++c)
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) acc[m][c] += __shfl_xor(acc[m][c], off, 64);
    __shared__ float red[kGemvThreads / 64][kGemvMaxM * kGemvCols];
    const int lane = tid & 63, wave = tid >> 6;
    if (lane == 0) {
#pragma unroll
        for (int m = 0; m < kGemvMaxM; ++m)
#pragma unroll
            for (int c = 0; c < kGemvCols; ++c) red[wave][m * kGemvCols + c] = acc[m][c];
    }
    __syncthreads();
    if (tid < kGemvMaxM * kGemvCols) {
        const int m = tid / kGemvCols, c = tid % kGemvCols;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kGemvThreads / 64; ++w) sum += red[w][tid];
        if (m < a.M) {
            float* T = reinterpret_cast<float*>(a.ws + b * a.ws_per_problem + t_off);
            T[(size_t)m * a.r + j0 + c] = sum;           // the single split: Tp[0][m][j]
        }
    }
}

// ------------------------------------------------- Y = X deq(W)^T + T R
// QA: Rt given as int4 codes (per 8 r one uint32) with one fp16 scale per 32 r.
// HYB: hybrid dense / 2:4 tiles (a.dvalues, a.dflags): for a dense tile the
// lane also loads the second pair of codes (positions 2 and 3 of each group
// of 4, metadata implied) and issues a second smfmac per 64-k step; a 2:4
// tile's lane reads zero there without a memory access.
template <int NW, int CPW, bool ADAPTER, int KS, bool FUSED, bool QA = false, bool HYB = false>
__global__ __launch_bounds__(64 * NW) void decode_kernel(LinearArgs a, size_t t_off) {
    static_assert(!FUSED || (ADAPTER && KS == 1), "the fused launch computes the complete T itself");
    static_assert(!QA || (ADAPTER && !FUSED), "quantised adapters: the two-launch form only");
    static_assert(!HYB || (!FUSED && !QA), "hybrid tiles: the two-launch form with fp16 adapters");
    const int b = blockIdx.y;
    const int nb = xcd_remap(blockIdx.x, gridDim.x);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nl = lane & 15, G = lane >> 4;
    const int64_t K = a.K, N = a.N;
    const int64_t n0 = (int64_t)nb * 16;
    const int Kb = (int)(K / 16);                         // 16-k blocks per row
    const int nch = (int)((K + 255) / 256);               // 256-k chunks (last may be half)

    // This workgroup's 16-row block of the packed format (group by group, row
    // by row inside a group: 32 B of values, 16 B of metadata, one scale).
    const uint8_t* vblk = a.values + b * a.sV + n0 * (K / 4);
    const uint8_t* mblk = a.meta + b * a.sMeta + n0 * (K / 8);
    const uint16_t* sblk = a.scales + b * a.sS + n0 * (K / kGroup);
    const int m = nl;
    const bool mval = m < a.M;
    const int gA1 = G >> 1, gA2 = 2 + (G >> 1), hoff = 8 * (G & 1);

    // X operand of one chunk slot: L2-resident, 8 x 16 B per lane, as buffer
    // loads over the M real token rows: the lanes of padding tokens (rows past
    // M) and k ranges past K read zero without a memory access, so with one
    // token only 4 of 64 lanes move data through the CU's vector memory path.
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X + b * a.sX, a.M * K * 2);
    const int xo = (int)(((int64_t)m * K + hoff) * 2);
    auto load_x = [&](int i, h8* x1, h8* x2) {
        const int c = wave + NW * i;
        const bool b1 = c < nch && 16 * c + 4 * gA1 < Kb;
        const bool b2 = c < nch && 16 * c + 4 * gA2 < Kb;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            x1[t] = buffer_load_h8(rx, b1 ? xo + 32 * (16 * c + 4 * gA1 + t) : kOOB);
            x2[t] = buffer_load_h8(rx, b2 ? xo + 32 * (16 * c + 4 * gA2 + t) : kOOB);
        }
    };
    // 0. Fused launch (one or two tokens): this workgroup's share of T = X L,
    //    rows [fj0, fj0 + fnr) of Lt over all of K, loaded before everything
    //    else so that T is published as early as possible.  Piece f of the
    //    flattened rows: row f / (K/8), k = 8 (f % (K/8)).
    const int npr = (int)(K / 8);
    const bool two = a.M > 1;                                // uniform
    int fj0 = 0, fnr = 0;
    h8 fl[kFusedPieces], fx0[kFusedPieces], fx1[kFusedPieces];
    // Hand-off state (see tag_entry): entries are written and read as single
    // 64-bit device-scope atomics (coherent across the XCDs' L2 caches): one
    // hop, no flags, no fences.
    unsigned long long* sync = reinterpret_cast<unsigned long long*>(a.ws);
    unsigned long long* tagged = reinterpret_cast<unsigned long long*>(a.ws + kTagBase);
    unsigned long long epoch = 0;
    if constexpr (FUSED) {
        // Read by every wave (no branch, so nothing waits for it before use).
        epoch = __hip_atomic_load(sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int P = (int)gridDim.x;
        fj0 = (int)((int64_t)blockIdx.x * a.r / P);
        fnr = (int)((int64_t)(blockIdx.x + 1) * a.r / P) - fj0;
        const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.Lt + b * a.sLt, a.r * K * 2);
#pragma unroll
        for (int i = 0; i < kFusedPieces; ++i) {
            const int f = (int)threadIdx.x + 64 * NW * i;
            const bool ok = f < fnr * npr;
            const int u = f >= npr ? 1 : 0, p = f - u * npr;
            fl[i] = buffer_load_h8(rl, ok ? (int)(((int64_t)(fj0 + u) * K + 8 * p) * 2) : kOOB);
            fx0[i] = buffer_load_h8(rx, ok ? 16 * p : kOOB);
            fx1[i] = two ? buffer_load_h8(rx, ok ? (int)((K + 8 * p) * 2) : kOOB) : h8{};
        }
    }

    // The Lt loads of every wave go out before any main-term load of the CU
    // (a barrier on issue only, no wait for data): T is on the critical path.
    if constexpr (FUSED) __builtin_amdgcn_s_barrier();

    h8 xa[4], xb[4], xc[4], xd[4];
    load_x(0, xa, xb);

    // 1. All packed-W loads of this wave (the HBM stream); hybrid tiles: the
    //    tile flags go out first.
    const int nG = (int)(K / kGroup);
    uint32_t tflag[CPW];
    if constexpr (HYB) {
        const __amdgpu_buffer_rsrc_t rf = make_rsrc(a.dflags + (int64_t)nb * nG * 4, nG * 4);
#pragma unroll
        for (int i = 0; i < CPW; ++i)
            tflag[i] = __builtin_amdgcn_raw_buffer_load_b32(rf, 4 * (2 * (wave + NW * i) + (G >> 1)), 0, 0);
    }
    u4 vw[CPW];
    u2 mw[CPW];
    uint32_t sh[CPW];
    bool aval[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int c = wave + NW * i;
        aval[i] = c < nch && 16 * c + 4 * G < Kb;
        const int rg = aval[i] ? 16 * (2 * c + (G >> 1)) + nl : 0;   // (group, row) of this lane's 64 k
        vw[i] = *reinterpret_cast<const u4*>(vblk + 32 * rg + 16 * (G & 1));
        mw[i] = *reinterpret_cast<const u2*>(mblk + 16 * rg + 8 * (G & 1));
        sh[i] = sblk[rg];
    }
    u4 dv[HYB ? CPW : 1];
    if constexpr (HYB) {
        const __amdgpu_buffer_rsrc_t rdv = make_rsrc(a.dvalues + n0 * (K / 4), 16 * (K / 4));
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int c = wave + NW * i;
            const int rg = 16 * (2 * c + (G >> 1)) + nl;
            const bool ld = aval[i] && tflag[i] != 0;
            dv[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rdv, ld ? 32 * rg + 16 * (G & 1) : kOOB, 0, 0));
        }
    }

    // 2. Adapter operands of this wave's 32-wide slice of r: R (HBM) and the
    //    partials of T (L2-resident, written by the previous launch).
    const int nR = (int)(a.r / 32);
    const __amdgpu_buffer_rsrc_t rt =
        make_rsrc(a.ws + b * a.ws_per_problem + t_off, (int64_t)KS * kDecodeMaxM * a.r * 4);
    auto load_r = [&](int jb) {      // Rt[n0 + nl][32jb + 8G .. +8]: the A operand of T . R
        if constexpr (QA) {
            const uint32_t w = reinterpret_cast<const uint32_t*>(a.Rq)[((n0 + nl) * a.r + 32 * jb + 8 * G) / 8];
            const _Float16 sc = reinterpret_cast<const _Float16*>(a.Rs)[(n0 + nl) * (a.r / 32) + jb];
            return dequant_word(w, h2{sc, sc});
        } else {
            return load_h8(a.Rt + b * a.sRt + (n0 + nl) * a.r + 32 * jb + 8 * G);
        }
    };
    auto load_t = [&](int jb) {
        // T[m][32jb + 8G .. +8] = sum over the KS K splits of the fp32
        // partials; lanes of padding tokens read zero without a memory access.
        f4 pl[KS], ph[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {                     // all loads in flight together
            const int off = mval ? (int)((((int64_t)s * kDecodeMaxM + m) * a.r + 32 * jb + 8 * G) * 4) : kOOB;
            pl[s] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rt, off, 0, 0));
            ph[s] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rt, off + 16, 0, 0));
        }
        f4 lo = pl[0], hi = ph[0];
#pragma unroll
        for (int s = 1; s < KS; ++s) {
            lo += pl[s];
            hi += ph[s];
        }
        h8 tv = {(_Float16)lo[0], (_Float16)lo[1], (_Float16)lo[2], (_Float16)lo[3],
                 (_Float16)hi[0], (_Float16)hi[1], (_Float16)hi[2], (_Float16)hi[3]};
        return tv;
    };
    h8 ra = {}, tb = {};
    const int jb0 = wave < nR ? wave : nR - 1;
    if constexpr (ADAPTER) {
        ra = load_r(jb0);
        if constexpr (!FUSED) tb = load_t(jb0);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load above is issued before the first wait
    const unsigned long long want = epoch + 1u;    // the tag of this call (fused launch)

    // Fused launch: finish this workgroup's rows of T (fp32 dot products, the
    // workgroup reduced in LDS), store them and raise this workgroup's flag;
    // the release orders the T stores before the flag.
    if constexpr (FUSED) {
        auto dot8 = [](const h8& x, const h8& y, float c) {
            c = __builtin_amdgcn_fdot2(h2{x[0], x[1]}, h2{y[0], y[1]}, c, false);
            c = __builtin_amdgcn_fdot2(h2{x[2], x[3]}, h2{y[2], y[3]}, c, false);
            c = __builtin_amdgcn_fdot2(h2{x[4], x[5]}, h2{y[4], y[5]}, c, false);
            return __builtin_amdgcn_fdot2(h2{x[6], x[7]}, h2{y[6], y[7]}, c, false);
        };
        float tp[kFusedTRows][2] = {};                       // [row u][token]
#pragma unroll
        for (int i = 0; i < kFusedPieces; ++i) {
            const int f = (int)threadIdx.x + 64 * NW * i;
            const float d0 = dot8(fl[i], fx0[i], 0.0f), d1 = dot8(fl[i], fx1[i], 0.0f);
            const bool hi = f >= npr;                          // invalid pieces loaded zeros
            tp[0][0] += hi ? 0.0f : d0;
            tp[0][1] += hi ? 0.0f : d1;
            tp[1][0] += hi ? d0 : 0.0f;
            tp[1][1] += hi ? d1 : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kFusedTRows; ++u)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) tp[u][t] += __shfl_xor(tp[u][t], off, 64);
        __shared__ float tred[NW][kFusedTRows * 2];
        if (lane == 0) {
#pragma unroll
            for (int u = 0; u < kFusedTRows; ++u)
#pragma unroll
                for (int t = 0; t < 2; ++t) tred[wave][2 * u + t] = tp[u][t];
        }
        __syncthreads();
        if (wave == 0) {
            if (lane < kFusedTRows * 2) {
                float v = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; ++w) v += tred[w][lane];
                const int u = lane >> 1, t = lane & 1;
                if (u < fnr && t < a.M) {
                    __hip_atomic_store(tagged + (int64_t)t * a.r + fj0 + u, tag_entry(want, v), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    }

    // 3. Main term: per chunk slot, 4 smfmac steps; the next slot's X goes out first.
    f4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        h8* x1 = (i & 1) ? xc : xa;
        h8* x2 = (i & 1) ? xd : xb;
        if (i + 1 < CPW) load_x(i + 1, (i & 1) ? xa : xc, (i & 1) ? xb : xd);
        const int c = wave + NW * i;
        const u4 v = aval[i] ? vw[i] : u4{0, 0, 0, 0};
        const u2 mm = aval[i] ? mw[i] : u2{0, 0};
        const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)(aval[i] ? sh[i] : 0u));
        const h2 s2 = {sv, sv};
        acc = smfmac<0>(dequant_word(v[0], s2), concat8(x1[0], x2[0]), acc, mm[0]);
        acc = smfmac<1>(dequant_word(v[1], s2), concat8(x1[1], x2[1]), acc, mm[0]);
        acc = smfmac<0>(dequant_word(v[2], s2), concat8(x1[2], x2[2]), acc, mm[1]);
        acc = smfmac<1>(dequant_word(v[3], s2), concat8(x1[3], x2[3]), acc, mm[1]);
        if constexpr (HYB) {
            // second pair of a dense tile: positions 2, 3 of every group (index 0xE)
            const u4 d = aval[i] ? dv[i] : u4{0, 0, 0, 0};
            acc = smfmac<0>(dequant_word(d[0], s2), concat8(x1[0], x2[0]), acc, 0xEEEEEEEEu);
            acc = smfmac<1>(dequant_word(d[1], s2), concat8(x1[1], x2[1]), acc, 0xEEEEEEEEu);
            acc = smfmac<0>(dequant_word(d[2], s2), concat8(x1[2], x2[2]), acc, 0xEEEEEEEEu);
            acc = smfmac<1>(dequant_word(d[3], s2), concat8(x1[3], x2[3]), acc, 0xEEEEEEEEu);
        }
    }

    // Fused launch: wave 0 polls all M r tagged entries (entry lane + 64 i;
    // one poll is a few load instructions for the workgroup, not one per
    // wave) until every one carries this call's tag, and hands the values
    // to the other waves through LDS.  Workgroup 0 then advances the epoch
    // (stores of many workgroups to one word would queue one after another
    // at the memory).  A bounded wait: on giving up (workgroups not all
    // resident) the workgroup's partial sums become NaN, so its rows of Y
    // read NaN (handoff_finish).
    if constexpr (FUSED) {
        __shared__ float tlds[kMaxTagged];
        __shared__ int tok;
        const int E = (int)(a.M * a.r);
        if (wave == 0) {
            bool ok = false;
            for (int it = 0; it < a.wait_limit && !ok; ++it) {
                bool mine = true;
                for (int i0 = 0; i0 < E; i0 += 64 * kPollUnroll) {
                    unsigned long long e[kPollUnroll];
#pragma unroll
                    for (int q = 0; q < kPollUnroll; ++q) {
                        const int i = i0 + lane + 64 * q;
                        e[q] = __hip_atomic_load(tagged + (i < E ? i : E - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
#pragma unroll
                    for (int q = 0; q < kPollUnroll; ++q) {
                        const int i = i0 + lane + 64 * q;
                        mine &= entry_tagged(e[q], want);
                        if (i < E) tlds[i] = entry_value(e[q]);
                    }
                }
                ok = __all(mine) != 0;
                if (!ok) __builtin_amdgcn_s_sleep(2);
            }
            if (lane == 0) {
                tok = ok;
                handoff_finish(a.ws, want, ok, blockIdx.x == 0);
            }
        }
        __syncthreads();
        if (tok) {
            if (mval && wave < nR) {
#pragma unroll
                for (int i = 0; i < 8; ++i) tb[i] = (_Float16)tlds[m * a.r + 32 * wave + 8 * G + i];
            }
        } else {
            acc = f4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
        }
    }

    // 4. Epilogue: acc[n][m] += sum_j R[j][n] T[m][j] (dense MFMA, same layout).
    if constexpr (ADAPTER) {
        acc = mfma16(wave < nR ? ra : h8{}, tb, acc);
        for (int jb = wave + NW; jb < nR; jb += NW) {      // only when r > 32*NW
            const h8 r2 = load_r(jb);
            const h8 t2 = load_t(jb);
            acc = mfma16(r2, t2, acc);
        }
    }

    // 5. Reduce the waves' partial sums and store fp16 Y.
    __shared__ f4 lds[NW * 64];
    lds[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave == 0) {
        f4 sum = lds[lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) sum += lds[w * 64 + lane];
        if (mval) {
            h4 out = {(_Float16)sum[0], (_Float16)sum[1], (_Float16)sum[2], (_Float16)sum[3]};
            *reinterpret_cast<h4*>(a.Y + b * a.sY + (int64_t)m * N + n0 + 4 * G) = out;
        }
    }
}

// --------------------------------- one launch, one or two tokens, a T wave
// decode_twave_kernel: the one-launch path with the rows of T on their own
// wave.  On this GPU a CU keeps only a few tens of KB of loads in flight and
// serves them in issue order; a wave whose next load cannot issue stalls, so
// a workgroup barrier waits for the slowest wave's loads.  Hence:
//   wave 0 issues the loads of the workgroup's one or two rows of Lt and of
//     X (straight into LDS) before any other wave issues a load (first
//     barrier), forms the rows of T (fp32 dot products summed with DPP) and
//     publishes them as tagged entries, loads the workgroup's 16 NB rows of
//     Rt into LDS, and polls all tagged entries with two passes in flight;
//   waves 1..7 meanwhile load their own 256-k chunks of the workgroup's NB
//     R8b blocks (values: one full 1 KB wave load per chunk and block;
//     metadata; scales) and of X straight into registers and run the main
//     term (dequant + smfmac), one X operand read per chunk for all NB
//     blocks; X of a chunk is put in B-operand order through a wave-private
//     LDS slot.
// After the second barrier (T and Rt in LDS) every wave adds its share of
// T . R (dense MFMA); a third barrier joins the eight partial sums (wave j
// joins block j).  NB = 1 when the N / 16 blocks fit the resident
// workgroups, else 3 (three blocks per workgroup, the last may hold fewer).
// With quantised adapters (QA) the factors are int4 codes with fp16 group
// scales, turned into fp16 where they are read.
constexpr int kTwThreads = 512;
constexpr int kTwWaves = kTwThreads / 64;
constexpr int kTwMain = kTwWaves - 1;    // waves of the main term
constexpr int kTwLds = 150 * 1024;       // one workgroup per CU

struct TwLayout {                        // LDS byte offsets
    int lt_off;                          // Lt rows [fnr][K] fp16, or their int4 codes [fnr][K/2] (wave 0)
    int ls_off;                          // quantised adapters: scales of those rows [fnr][K/128] fp16
    int x_off;                           // X [M][K] fp16 (wave 0)
    int rt_off, rtp;                     // Rt rows [16 NB][r] fp16, row pitch rtp, or codes [16 NB][r/2] (wave 0)
    int rs_off;                          // quantised adapters: scales of the Rt rows [16 NB][r/32] fp16
    int t_off;                           // T [M][r] fp32 (wave 0)
    int xs_off;                          // one 1 KB X slot per main wave
    int red_off;                         // partial sums: f4 [NB][kTwWaves][64]
    int total;
};

TwLayout tw_layout(int64_t M, int64_t K, int64_t r, bool qa = false, int nb = 1, int tw = kTwThreads) {
    auto kb = [](int64_t x) { return (int)((x + 1023) & ~int64_t(1023)); };
    TwLayout L{};
    int o = 0;
    L.lt_off = o; o += kb((int64_t)kFusedTRows * K * (qa ? 1 : 4) / 2);
    L.ls_off = o; o += qa ? kb((int64_t)kFusedTRows * (K / kGroup) * 2 + 32) : 0;
    L.x_off = o; o += kb(M * K * 2);
    L.rtp = (int)(qa ? r / 2 : 2 * r + 16);
    L.rt_off = o; o += kb(16 * nb * (int64_t)L.rtp);
    L.rs_off = o; o += qa ? kb(16 * nb * (r / 32) * 2) : 0;
    L.t_off = o; o += kb(M * r * 4);
    L.xs_off = o; o += (tw / 64 - 1) * 1024;
    L.red_off = o; o += nb * (tw / 64) * 64 * 16;
    L.total = o;
    return L;
}

// CPW: 256-k chunks per main wave (chunk c of wave w: c = w - 1 + 7 i).
// PS: tagged entries per lane and poll pass (M r <= 64 PS), loaded
// unconditionally (indexes past M r re-read the last entry) so that the
// compiler counts every pass exactly and waits for the older pass only.
// QA: the adapter factors are int4 codes with fp16 group scales (Lt: groups
// of 128 along K, Rt: groups of 32 along r; per 8 consecutive elements one
// uint32 whose nibbles the int4 -> fp16 step returns in element order).
// NB: 16-row blocks of W per workgroup (the last workgroup may hold fewer),
// so that N / 16 above the resident-workgroup count still runs in one launch;
// each main wave applies one X operand read to all NB blocks.
// TW: threads per workgroup, 512 or 1024 (15 main waves, so that long K
// leaves each main wave fewer chunks in sequence).
// HOLD: the main waves issue the loads of their last chunk slot only once
// wave 0 has issued the stores of its T entries (an LDS flag), and start
// their main term after that.
template <int CPW, int PS, bool QA, int NB, int TW = kTwThreads, bool HOLD = (TW == kTwThreads)>
__global__ __launch_bounds__(TW) void decode_twave_kernel(LinearArgs a, TwLayout L) {
    constexpr int kW = TW / 64, kMn = kW - 1;                   // waves, main waves
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kTwLds];
    __shared__ int tok;
    __shared__ int tpub;                                        // wave 0 has issued its T entries' stores
    const int P = (int)gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nl = lane & 15, G = lane >> 4;
    const int K = (int)a.K, M = (int)a.M, r = (int)a.r;
    const int nb = xcd_remap(blockIdx.x, P);
    const int64_t N = a.N, n0 = (int64_t)nb * 16 * NB;
    const int64_t left = N / 16 - (int64_t)nb * NB;
    const int nbk = NB == 1 ? 1 : (left < NB ? (int)left : NB);                // blocks held
    unsigned long long* sync = reinterpret_cast<unsigned long long*>(a.ws);
    unsigned long long* tagged = reinterpret_cast<unsigned long long*>(a.ws + kTagBase);
    float* tl = reinterpret_cast<float*>(lds + L.t_off);
    const unsigned bx = blockIdx.x;
    const int fj0 = (int)(bx * (unsigned)r / (unsigned)P);
    const int fnr = (int)((bx + 1u) * (unsigned)r / (unsigned)P) - fj0;
    f4 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = f4{0, 0, 0, 0};
    // Poll passes of wave 0.  The pass still in flight when the poll ends is
    // used once more at the very end (a test that never holds) so that its
    // registers are not reused before it has landed.
    unsigned long long ea[PS] = {}, eb[PS] = {};
    unsigned long long epoch = 0;
    // Quantised adapters: the rows' scales are copied from the 16-byte
    // boundary at or below the first one (a row holds K / 128 of them, not
    // always a multiple of 8), so they sit ls_d bytes into their LDS area.
    const int64_t ls_first = QA ? (int64_t)fj0 * (K / kGroup) * 2 : 0;
    const int ls_d = (int)(ls_first & 15);

    if (tid == 0) {
        __hip_atomic_store(&tpub, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    // 1. Wave 0: the epoch, then Lt rows [fj0, fj0 + fnr) and X (both
    //    contiguous) into LDS, 1 KB per instruction (pieces past the rows
    //    read zero); no other wave has a load in flight yet.
    if (wave == 0) {
        __builtin_amdgcn_s_setprio(3);
        epoch = __hip_atomic_load(sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const u4 rx = rsrc_words(a.X, (int64_t)M * K * 2);
        const int nIX = (M * K + 511) / 512;
        if constexpr (QA) {
            const u4 rl = rsrc_words(a.Lq + (int64_t)fj0 * (K / 2), (int64_t)fnr * (K / 2));
            // Whole 16-byte pieces: the range check drops a piece that
            // crosses the end of the range.  Both ends stay inside the
            // scales array (16-byte aligned, r K / 64 bytes, r % 32 == 0).
            const int sbytes = (ls_d + fnr * (K / kGroup) * 2 + 15) & ~15;
            const u4 rls = rsrc_words(reinterpret_cast<const unsigned char*>(a.Ls) + (ls_first - ls_d), sbytes);
            const int nIL = (fnr * K + 2047) / 2048, nIS = (sbytes + 1023) / 1024;
            for (int i = 0; i < nIL; ++i) lds_load16(rl, lds + L.lt_off + 1024 * i, 16 * lane, 1024 * i);
            for (int i = 0; i < nIS; ++i) lds_load16(rls, lds + L.ls_off + 1024 * i, 16 * lane, 1024 * i);
        } else {
            const u4 rl = rsrc_words(a.Lt + (int64_t)fj0 * K, (int64_t)fnr * K * 2);
            const int nIL = (fnr * K + 511) / 512;
            for (int i = 0; i < nIL; ++i) lds_load16(rl, lds + L.lt_off + 1024 * i, 16 * lane, 1024 * i);
        }
        for (int i = 0; i < nIX; ++i) lds_load16(rx, lds + L.x_off + 1024 * i, 16 * lane, 1024 * i);
    }
    __builtin_amdgcn_s_barrier();

    if (wave == 0) {
        // 2. Rows of T (the second token's products only when M = 2).
        wait_vmem_below<0>();
        // Keep every use of the epoch load below the barrier: the compiler
        // would otherwise wait for it, and so for all loads in flight, above.
        asm volatile("" : "+v"(epoch));
        const unsigned long long want = epoch + 1u;
        auto dot8 = [](const h8& x, const h8& y, float c) {
            c = __builtin_amdgcn_fdot2(h2{x[0], x[1]}, h2{y[0], y[1]}, c, false);
            c = __builtin_amdgcn_fdot2(h2{x[2], x[3]}, h2{y[2], y[3]}, c, false);
            c = __builtin_amdgcn_fdot2(h2{x[4], x[5]}, h2{y[4], y[5]}, c, false);
            return __builtin_amdgcn_fdot2(h2{x[6], x[7]}, h2{y[6], y[7]}, c, false);
        };
        const int npr = K / 8;
        float t00 = 0.0f, t01 = 0.0f, t10 = 0.0f, t11 = 0.0f;       // [row u][token m]
        if constexpr (QA) {
            // Units of 32 k (one 16-byte codes read per row, one scale): lane
            // l takes the units l, l + 64, ..., two in flight; the unit's dot
            // products of the unscaled codes are scaled once.
            const int nun = K / 32;
            const int rs1 = fnr > 1 ? K / 2 : 0, ss1 = fnr > 1 ? 2 * (K / kGroup) : 0;
            for (int u0 = lane; u0 < nun; u0 += 128) {
                u4 c0[2], c1[2];
                _Float16 s0[2], s1[2];
                h8 x0[2][4], x1[2][4];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int u = u0 + 64 * j;
                    const bool ok = u < nun;
                    const int uu = ok ? u : 0;
                    c0[j] = *reinterpret_cast<const u4*>(lds + L.lt_off + 16 * uu);
                    c1[j] = *reinterpret_cast<const u4*>(lds + L.lt_off + rs1 + 16 * uu);
                    s0[j] = ok ? *reinterpret_cast<const _Float16*>(lds + L.ls_off + ls_d + 2 * (uu / 4)) : (_Float16)0.0f;
                    s1[j] = ok && fnr > 1 ? *reinterpret_cast<const _Float16*>(lds + L.ls_off + ls_d + ss1 + 2 * (uu / 4))
                                          : (_Float16)0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) x0[j][i] = *reinterpret_cast<const h8*>(lds + L.x_off + 64 * uu + 16 * i);
                    if (M > 1) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            x1[j][i] = *reinterpret_cast<const h8*>(lds + L.x_off + 2 * K + 64 * uu + 16 * i);
                    }
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float a00 = 0.0f, a10 = 0.0f, a01 = 0.0f, a11 = 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const h8 q0 = dequant_word(c0[j][i], h2{(_Float16)1.0f, (_Float16)1.0f});
                        const h8 q1 = dequant_word(c1[j][i], h2{(_Float16)1.0f, (_Float16)1.0f});
                        a00 = dot8(q0, x0[j][i], a00);
                        a10 = dot8(q1, x0[j][i], a10);
                        if (M > 1) {
                            a01 = dot8(q0, x1[j][i], a01);
                            a11 = dot8(q1, x1[j][i], a11);
                        }
                    }
                    t00 = fmaf((float)s0[j], a00, t00);
                    t10 = fmaf((float)s1[j], a10, t10);
                    t01 = fmaf((float)s0[j], a01, t01);
                    t11 = fmaf((float)s1[j], a11, t11);
                }
            }
        } else {
            // Lane l takes the 16-byte pieces l, l + 64, ... of each row, four
            // pieces per row and token in flight together.
            for (int p0 = lane; p0 < npr; p0 += 256) {
                h8 l0[4], l1[4], x0[4], x1[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int p = p0 + 64 * j;
                    const bool ok = p < npr;
                    l0[j] = ok ? *reinterpret_cast<const h8*>(lds + L.lt_off + 16 * p) : h8{};
                    l1[j] = ok && fnr > 1 ? *reinterpret_cast<const h8*>(lds + L.lt_off + 16 * (npr + p)) : h8{};
                    x0[j] = ok ? *reinterpret_cast<const h8*>(lds + L.x_off + 16 * p) : h8{};
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    t00 = dot8(l0[j], x0[j], t00);
                    t10 = dot8(l1[j], x0[j], t10);
                }
                if (M > 1) {           // second token (uniform branch)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int p = p0 + 64 * j;
                        x1[j] = p < npr ? *reinterpret_cast<const h8*>(lds + L.x_off + 16 * (npr + p)) : h8{};
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        t01 = dot8(l0[j], x1[j], t01);
                        t11 = dot8(l1[j], x1[j], t11);
                    }
                }
            }
        }
        t00 = wave_sum_hi(t00);
        t01 = wave_sum_hi(t01);
        t10 = wave_sum_hi(t10);
        t11 = wave_sum_hi(t11);
        if (lane >= 60) {
            const int u = (lane - 60) >> 1, m = lane & 1;
            const float v = u ? (m ? t11 : t10) : (m ? t01 : t00);
            if (u < fnr && m < M)
                __hip_atomic_store(tagged + (int64_t)m * r + fj0 + u, tag_entry(want, v), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        if (lane == 0) __hip_atomic_store(&tpub, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);

        // 3. Rt rows n0 .. n0 + 16 NB - 1 into LDS, one instruction per row
        //    (lanes past the row's 2r bytes are masked off; rows past N read
        //    zero).  These loads are older than every poll pass, so the wait
        //    for the first checked pass covers them.
        if constexpr (QA) {
            // The rows' codes and scales are contiguous: 1 KB per instruction.
            const int cb = 16 * NB * (r / 2), sb = 16 * NB * (r / 32) * 2;
            const u4 rr = rsrc_words(a.Rq + n0 * (r / 2), (int64_t)16 * nbk * (r / 2));
            const u4 rrs = rsrc_words(a.Rs + n0 * (r / 32), (int64_t)16 * nbk * (r / 32) * 2);
            for (int i = 0; 1024 * i < cb; ++i)
                if (16 * lane + 1024 * i < cb) lds_load16(rr, lds + L.rt_off + 1024 * i, 16 * lane, 1024 * i);
            for (int i = 0; 1024 * i < sb; ++i)
                if (16 * lane + 1024 * i < sb) lds_load16(rrs, lds + L.rs_off + 1024 * i, 16 * lane, 1024 * i);
        } else {
            const u4 rr = rsrc_words(a.Rt + n0 * r, (int64_t)16 * nbk * r * 2);
            if (lane < r / 8) {
#pragma unroll
                for (int q = 0; q < 16 * NB; ++q) lds_load16(rr, lds + L.rt_off + q * L.rtp, 16 * lane, q * 2 * r);
            }
        }

        // 4. Poll the M r tagged entries (entry lane + 64 q), two passes in
        //    flight; each pass writes its values to LDS, the last one complete.
        const int E = M * r;
        auto issue = [&](unsigned long long (&e)[PS]) __attribute__((always_inline)) {
#pragma unroll
            for (int q = 0; q < PS; ++q) {
                const int i = lane + 64 * q;
                e[q] = __hip_atomic_load(tagged + (i < E ? i : E - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        };
        auto check = [&](const unsigned long long (&e)[PS]) __attribute__((always_inline)) {
            bool mine = true;
#pragma unroll
            for (int q = 0; q < PS; ++q) {
                const int i = lane + 64 * q;
                mine &= entry_tagged(e[q], want);
                if (i < E) tl[i] = entry_value(e[q]);
            }
            return __all(mine) != 0;
        };
        bool ok = false;
        issue(ea);
        for (int it = 0; it < a.wait_limit; it += 2) {
            issue(eb);
            if (check(ea)) { ok = true; break; }
            __builtin_amdgcn_s_sleep(1);
            issue(ea);
            if (check(eb)) { ok = true; break; }
            __builtin_amdgcn_s_sleep(1);
        }
        if (lane == 0) {
            tok = ok;
            handoff_finish(a.ws, want, ok, blockIdx.x == 0);
        }
    } else {
        // 2'. Main term.  Block-local (group, row) index rg = 16 (2c + G / 2)
        //    + nl: values at 32 rg + 16 (G & 1) (4 words: chunk blocks 4G ..
        //    4G + 3), metadata at 16 rg + 8 (G & 1), scale at 2 rg; offsets
        //    past the block (half chunk at the end of K, chunks past K) read
        //    zero.
        // Block j of the workgroup starts 16 j rows after n0.
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.values + n0 * (K / 4), (int64_t)16 * nbk * (K / 4));
        const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.meta + n0 * (K / 8), (int64_t)16 * nbk * (K / 8));
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales + n0 * (K / kGroup), (int64_t)16 * nbk * (K / kGroup) * 2);
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X, (int64_t)M * K * 2);
        const int nch = (K + 255) / 256;
        u4 vv[CPW][NB];
        u2 mv[CPW][NB];
        uint32_t sv[CPW][NB];
        h8 xv[CPW];
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            if (HOLD && i == CPW - 1) {
                while (__hip_atomic_load(&tpub, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
                    __builtin_amdgcn_s_sleep(2);
            }
            const int c = wave - 1 + kMn * i;
            const int rg = 16 * (2 * c + (G >> 1)) + nl;
            const bool cv = c < nch;
            // X of the chunk: lane l < 32 M takes 8 k of token l / 32.
            const int k = 256 * c + 8 * (lane & 31);
            const bool xok = cv && lane < 32 * M && k < K;
            xv[i] = buffer_load_h8(rx, xok ? ((lane >> 5) * K + k) * 2 : kOOB);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const bool bv = cv && j < nbk;
                vv[i][j] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                               rv, bv ? 16 * j * (K / 4) + 32 * rg + 16 * (G & 1) : kOOB, 0, 0));
                mv[i][j] = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(
                               rm, bv ? 16 * j * (K / 8) + 16 * rg + 8 * (G & 1) : kOOB, 0, 0));
                sv[i][j] = __builtin_amdgcn_raw_buffer_load_b16(rs, bv ? 2 * (16 * j * (K / kGroup) + rg) : kOOB, 0, 0);
            }
        }
        unsigned char* xs = lds + L.xs_off + (wave - 1) * 1024;
        const bool mval = nl < M;
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            if (wave - 1 + kMn * i >= nch) break;
            *reinterpret_cast<h8*>(xs + 16 * lane) = xv[i];
            // B operand of step t: elements 0..7 at chunk k 64 (G / 2) + 16 t +
            // 8 (G & 1), elements 8..15 at 128 more (matching the A blocks).
            h8 x1[4], x2[4];
            const unsigned char* xr = xs + (mval ? nl : 0) * 512 + 2 * (64 * (G >> 1) + 8 * (G & 1));
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                x1[t] = mval ? *reinterpret_cast<const h8*>(xr + 32 * t) : h8{};
                x2[t] = mval ? *reinterpret_cast<const h8*>(xr + 256 + 32 * t) : h8{};
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if (NB > 1 && j >= nbk) break;                       // uniform: the last workgroup
                const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)sv[i][j]);
                const h2 s2 = {s, s};
                acc[j] = smfmac<0>(dequant_word(vv[i][j][0], s2), concat8(x1[0], x2[0]), acc[j], mv[i][j][0]);
                acc[j] = smfmac<1>(dequant_word(vv[i][j][1], s2), concat8(x1[1], x2[1]), acc[j], mv[i][j][0]);
                acc[j] = smfmac<0>(dequant_word(vv[i][j][2], s2), concat8(x1[2], x2[2]), acc[j], mv[i][j][1]);
                acc[j] = smfmac<1>(dequant_word(vv[i][j][3], s2), concat8(x1[3], x2[3]), acc[j], mv[i][j][1]);
            }
        }
    }
    __syncthreads();

    // 5. acc += Rt-slice . T for the 32-column blocks jb = wave, wave + 8, ...
    //    (A: Rt rows from LDS; B: T of token nl, fp16).
    const int nR = r / 32;
    for (int jb = wave; jb < nR; jb += kW) {
        h8 ra[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int q = 16 * j + nl;                               // Rt row in LDS
            if constexpr (QA) {
                // Row q, r-columns 32 jb + 8G .. +8: one codes word, scale of group jb.
                const uint32_t w = *reinterpret_cast<const uint32_t*>(lds + L.rt_off + q * (r / 2) + 16 * jb + 4 * G);
                const _Float16 sc = *reinterpret_cast<const _Float16*>(lds + L.rs_off + 2 * (q * (r / 32) + jb));
                ra[j] = dequant_word(w, h2{sc, sc});
            } else {
                ra[j] = *reinterpret_cast<const h8*>(lds + L.rt_off + q * L.rtp + 2 * (32 * jb + 8 * G));
            }
        }
        h8 tb = {};
        if (nl < M) {
            const f4 lo = *reinterpret_cast<const f4*>(tl + nl * r + 32 * jb + 8 * G);
            const f4 hi = *reinterpret_cast<const f4*>(tl + nl * r + 32 * jb + 8 * G + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                tb[e] = (_Float16)lo[e];
                tb[4 + e] = (_Float16)hi[e];
            }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[j] = mfma16(ra[j], tb, acc[j]);
    }
    if (!tok) {
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[j] = f4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    }

    // 6. Join the partial sums and store fp16 Y (lane: token nl, rows 4G ..
    //    4G+3 of block j; wave j joins block j).
    f4* red = reinterpret_cast<f4*>(lds + L.red_off);
#pragma unroll
    for (int j = 0; j < NB; ++j) red[(j * kW + wave) * 64 + lane] = acc[j];
    __syncthreads();
    if (wave < NB && wave < nbk) {
        const int j = wave;
        f4 sum = red[j * kW * 64 + lane];
#pragma unroll
        for (int w = 1; w < kW; ++w) sum += red[(j * kW + w) * 64 + lane];
        if (nl < M) {
            const h4 out = {(_Float16)sum[0], (_Float16)sum[1], (_Float16)sum[2], (_Float16)sum[3]};
            *reinterpret_cast<h4*>(a.Y + (int64_t)nl * N + n0 + 16 * j + 4 * G) = out;
        }
    }
    if (wave == 0) {
        if (a.M > kGemvMaxM) {                                          // never: M <= 2 here
            unsigned long long z = 0;
#pragma unroll
            for (int q = 0; q < PS; ++q) z ^= ea[q] ^ eb[q];
            reinterpret_cast<unsigned long long*>(a.ws)[lane] = z;
        }
    }
}

// Workgroups of the fused main kernel (CPW chunk slots per wave) that the
// current device holds resident at once; 0 if it cannot be determined.
template <int CPW>
int64_t fused_capacity() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int64_t> cache[kMaxDevices];              // 0: not yet known
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int64_t c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<kDecodeWaves, CPW, true, 1, true>,
                                                     64 * kDecodeWaves, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    c = (int64_t)per_cu * cus;
    cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

int64_t twave_capacity() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int64_t> cache[kMaxDevices];              // 0: not yet known
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int64_t c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
    int per_cu = 0, cus = 0;
    // Every instantiation has the same LDS (one workgroup per CU).
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_twave_kernel<7, 16, false, 1>, kTwThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    c = (int64_t)per_cu * cus;
    cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

template <int CPW>
hipError_t launch_main(const LinearArgs& a, const DecodePlan& p, hipStream_t stream) {
    dim3 grid((unsigned)(a.N / 16), (unsigned)a.batch);
    dim3 block(64 * kDecodeWaves);
    if (a.r == 0)
        hipLaunchKernelGGL((decode_kernel<kDecodeWaves, CPW, false, 1, false>), grid, block, 0, stream, a, p.t_off);
    else if (p.ksplits != 1 && p.ksplits != kMaxKSplits)
        return hipErrorInvalidValue;                   // the plan makes only these two
    else if (p.fused)
        hipLaunchKernelGGL((decode_kernel<kDecodeWaves, CPW, true, 1, true>), grid, block, 0, stream, a, p.t_off);
    else if (p.ksplits == 1)
        hipLaunchKernelGGL((decode_kernel<kDecodeWaves, CPW, true, 1, false>), grid, block, 0, stream, a, p.t_off);
    else
        hipLaunchKernelGGL((decode_kernel<kDecodeWaves, CPW, true, kMaxKSplits, false>), grid, block, 0, stream, a,
                           p.t_off);
    return hipGetLastError();
}

}  // namespace

size_t split_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
bool split_fits(const LinearArgs& a);
hipError_t launch_linear_split(const LinearArgs& a, hipStream_t stream);

size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
    const size_t d = decode_plan(M, N, K, r).total, sp = split_workspace_bytes(M, N, K, r);
    return d > sp ? d : sp;
}

// Row blocks per workgroup of the one-launch T-wave form: 1, or 3 when the
// N / 16 blocks exceed the workgroups the device holds resident; 0 if
// neither fits.
int twave_nb(int64_t N) {
    const int64_t cap = twave_capacity();
    if (N / 16 <= cap) return 1;
    if ((N / 16 + 2) / 3 <= cap) return 3;
    return 0;
}

// The T-wave form with NB blocks per workgroup applies: one or two tokens,
// one problem, one or two rows of Lt per workgroup, the tagged T within one
// poll pass pair, and its LDS layout within one workgroup per CU.
// Threads per workgroup of the T-wave form: 1024 (15 main waves) when the
// 7 main waves of 512 would take more than 3 chunks each in sequence (down:
// 43 chunks, 10.35 -> 9.33 us at one token), for fp16 adapters and one block
// per workgroup; else 512 (q/k/v/o, gate/up: 512 are faster).
int twave_threads(const LinearArgs& a, bool qa, int nb) {
    const int64_t nch = (a.K + 255) / 256;
    return !qa && nb == 1 && nch > 3 * kTwMain ? 1024 : kTwThreads;
}

bool twave_fits(const LinearArgs& a, bool qa, int nb) {
    if (nb < 1) return false;
    const int64_t P = (a.N / 16 + nb - 1) / nb;
    const int64_t nch = (a.K + 255) / 256;
    return a.r > 0 && a.M >= 1 && a.M <= kGemvMaxM && a.batch == 1 && a.r <= 512 && a.M * a.r <= 64 * 16 &&
           a.M * a.r <= kMaxTagged && P <= a.r && a.r <= kFusedTRows * P && nch <= 10 * kTwMain &&
           tw_layout(a.M, a.K, a.r, qa, nb, twave_threads(a, qa, nb)).total <= kTwLds;
}

template <bool QA, int NB>
hipError_t launch_twave(const LinearArgs& a, hipStream_t stream) {
    const int tw = twave_threads(a, QA, NB);
    const TwLayout TL = tw_layout(a.M, a.K, a.r, QA, NB, tw);
    const int nch = (int)((a.K + 255) / 256);
    const dim3 grid((unsigned)((a.N / 16 + NB - 1) / NB)), block(tw);
    const bool one = a.M * a.r <= 64 * 8;          // poll pass of 8 entries per lane, else 16
#define SLIM_TW(C, T)                                                                                  \
    do {                                                                                               \
        if (one) hipLaunchKernelGGL((decode_twave_kernel<C, 8, QA, NB, T>), grid, block, 0, stream, a, TL);  \
        else     hipLaunchKernelGGL((decode_twave_kernel<C, 16, QA, NB, T>), grid, block, 0, stream, a, TL); \
    } while (0)
    if constexpr (!QA && NB == 1) {
        if (tw == 1024) {
            constexpr int m = 1024 / 64 - 1;
            if (nch <= 2 * m)      SLIM_TW(2, 1024);
            else if (nch <= 3 * m) SLIM_TW(3, 1024);
            else                   SLIM_TW(5, 1024);
            return hipGetLastError();
        }
    }
    if (nch <= 2 * kTwMain)      SLIM_TW(2, kTwThreads);
    else if (nch <= 3 * kTwMain) SLIM_TW(3, kTwThreads);
    else if (nch <= 5 * kTwMain) SLIM_TW(5, kTwThreads);
    else if (nch <= 7 * kTwMain) SLIM_TW(7, kTwThreads);
    else                         SLIM_TW(10, kTwThreads);
#undef SLIM_TW
    return hipGetLastError();
}

// Quantised adapters on the one-launch T-wave path.
bool decode_qa_fits(const LinearArgs& a) {
    return twave_fits(a, true, twave_nb(a.N));
}

hipError_t launch_linear_decode_qa(const LinearArgs& a, hipStream_t stream) {
    return twave_nb(a.N) == 1 ? launch_twave<true, 1>(a, stream) : launch_twave<true, 3>(a, stream);
}

// Quantised adapters, one or two tokens, when the one-launch form does not
// fit: T = X deq(L) by the matrix-vector kernel, then the main kernel with
// deq(R) in its epilogue (both read the int4 factors).
bool decode_qa2_fits(const LinearArgs& a) {
    const int64_t nch = (a.K + 255) / 256;
    return a.r > 0 && a.M >= 1 && a.M <= kGemvMaxM && a.batch == 1 && a.r % kGemvCols == 0 &&
           nch <= (int64_t)kDecodeWaves * kDecodeMaxCPW;
}

hipError_t launch_linear_decode_qa2(const LinearArgs& a, hipStream_t stream) {
    const DecodePlan p = decode_plan(a.M, a.N, a.K, a.r);
    if (p.ksplits != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(adapter_down_gemv_kernel<true>, dim3((unsigned)(a.r / kGemvCols), 1u), dim3(kGemvThreads), 0,
                       stream, a, p.t_off);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int cpw = (int)(((a.K + 255) / 256 + kDecodeWaves - 1) / kDecodeWaves);
    const dim3 grid((unsigned)(a.N / 16), 1u), block(64 * kDecodeWaves);
    switch (cpw) {
        case 1: hipLaunchKernelGGL((decode_kernel<kDecodeWaves, 1, true, 1, false, true>), grid, block, 0, stream, a, p.t_off); break;
        case 2: hipLaunchKernelGGL((decode_kernel<kDecodeWaves, 2, true, 1, false, true>), grid, block, 0, stream, a, p.t_off); break;
        case 3: hipLaunchKernelGGL((decode_kernel<kDecodeWaves, 3, true, 1, false, true>), grid, block, 0, stream, a, p.t_off); break;
        default: hipLaunchKernelGGL((decode_kernel<kDecodeWaves, 4, true, 1, false, true>), grid, block, 0, stream, a, p.t_off); break;
    }
    return hipGetLastError();
}

// Hybrid dense / 2:4 tiles at 1 to 16 tokens: the adapter-down launch, then
// decode_kernel with the second pair of codes of dense tiles.
bool decode_hybrid_fits(const LinearArgs& a) {
    const int64_t nch = (a.K + 255) / 256;
    return a.M >= 1 && a.M <= kDecodeMaxM && nch <= (int64_t)kDecodeWaves * kDecodeMaxCPW;
}

hipError_t launch_linear_decode_hybrid(const LinearArgs& a, hipStream_t stream) {
    const DecodePlan p = decode_plan(a.M, a.N, a.K, a.r);
    if (a.r > 0) {
        if (a.M <= kGemvMaxM)
            hipLaunchKernelGGL(adapter_down_gemv_kernel<false>, dim3((unsigned)(a.r / kGemvCols), (unsigned)a.batch),
                               dim3(kGemvThreads), 0, stream, a, p.t_off);
        else
            hipLaunchKernelGGL(adapter_down_kernel, dim3((unsigned)((a.r / 16) * p.ksplits), (unsigned)a.batch),
                               dim3(64 * kDownWaves), 0, stream, a, p.ksplits, p.t_off);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int cpw = (int)(((a.K + 255) / 256 + kDecodeWaves - 1) / kDecodeWaves);
    const dim3 grid((unsigned)(a.N / 16), (unsigned)a.batch), block(64 * kDecodeWaves);
#define SLIM_HYB(C)                                                                                               \
    do {                                                                                                          \
        if (a.r == 0)                                                                                             \
            hipLaunchKernelGGL((decode_kernel<kDecodeWaves, C, false, 1, false, false, true>), grid, block, 0,    \
                               stream, a, p.t_off);                                                               \
        else if (p.ksplits == 1)                                                                                  \
            hipLaunchKernelGGL((decode_kernel<kDecodeWaves, C, true, 1, false, false, true>), grid, block, 0,     \
                               stream, a, p.t_off);                                                               \
        else                                                                                                      \
            hipLaunchKernelGGL((decode_kernel<kDecodeWaves, C, true, kMaxKSplits, false, false, true>), grid,     \
                               block, 0, stream, a, p.t_off);                                                     \
    } while (0)
    if (a.r > 0 && p.ksplits != 1 && p.ksplits != kMaxKSplits) return hipErrorInvalidValue;
    switch (cpw) {
        case 1: SLIM_HYB(1); break;
        case 2: SLIM_HYB(2); break;
        case 3: SLIM_HYB(3); break;
        default: SLIM_HYB(4); break;
    }
#undef SLIM_HYB
    return hipGetLastError();
}

bool decode_fits(const LinearArgs& a) {
    const int64_t nch = (a.K + 255) / 256;
    return a.M >= 1 && a.M <= kDecodeMaxM && nch <= (int64_t)kDecodeWaves * kDecodeMaxCPW;
}

hipError_t launch_linear_decode(const LinearArgs& a, hipStream_t stream) {
    // Three or more tokens: K split over workgroups (linear_split.hip).
    if (a.M > kGemvMaxM && split_fits(a)) return launch_linear_split(a, stream);
    // One launch with three 16-row blocks per workgroup when the blocks
    // exceed the resident workgroups (gate/up: 688 blocks).
    if (twave_nb(a.N) == 3 && twave_fits(a, false, 3)) return launch_twave<false, 3>(a, stream);
    DecodePlan p = decode_plan(a.M, a.N, a.K, a.r);
    const int cpw = (int)(((a.K + 255) / 256 + kDecodeWaves - 1) / kDecodeWaves);
    // One launch (one problem) when its workgroups can all be resident (they
    // wait for each other's rows of T), each owns at least one and at most
    // kFusedTRows rows of Lt (kFusedPieces pieces per thread), and the tagged
    // T fits in the reserved workspace bytes.
    if (a.r > 0 && a.M <= kGemvMaxM && a.batch == 1 && a.M * a.r <= kMaxTagged && a.N / 16 <= a.r &&
        a.r <= kFusedTRows * (a.N / 16) &&
        kFusedTRows * (a.K / 8) <= (int64_t)64 * kDecodeWaves * kFusedPieces) {
        const int64_t cap = cpw == 1 ? fused_capacity<1>() : cpw == 2 ? fused_capacity<2>()
                          : cpw == 3 ? fused_capacity<3>() : fused_capacity<4>();
        p.fused = (a.N / 16) * a.batch <= cap;
        // The T-wave form when its LDS layout fits (one workgroup per CU).
        const int nch = (int)((a.K + 255) / 256);
        const TwLayout TL = tw_layout(a.M, a.K, a.r, false, 1, twave_threads(a, false, 1));
        if (p.fused && TL.total <= kTwLds && a.r <= 512 && a.M * a.r <= 64 * 16 && nch <= 10 * kTwMain &&
            a.N / 16 <= twave_capacity()) {
            return launch_twave<false, 1>(a, stream);
        }
    }
    if (a.r > 0 && !p.fused) {
        if (a.M <= kGemvMaxM) {
            dim3 grid((unsigned)(a.r / kGemvCols), (unsigned)a.batch);
            hipLaunchKernelGGL(adapter_down_gemv_kernel<false>, grid, dim3(kGemvThreads), 0, stream, a, p.t_off);
        } else {
            dim3 grid((unsigned)((a.r / 16) * p.ksplits), (unsigned)a.batch);
            hipLaunchKernelGGL(adapter_down_kernel, grid, dim3(64 * kDownWaves), 0, stream, a, p.ksplits, p.t_off);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    switch (cpw) {
        case 1: return launch_main<1>(a, p, stream);
        case 2: return launch_main<2>(a, p, stream);
        case 3: return launch_main<3>(a, p, stream);
        default: return launch_main<4>(a, p, stream);
    }
}

}  // namespace slim
