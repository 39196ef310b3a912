// slim_linear for decode-shaped problems (M <= 16 tokens): HBM-bound.
//
//   T = X . L                                   (adapter down, dense MFMA)
//   Y = X . deq(W_c)^T + T . R                  (2:4 sparse MFMA + dense MFMA)
//
// Layer: Compression Trinity thesis §2.1 (Y = X W^T) with the sparse weight
// and the low-rank adapter as parallel paths (Ch. 4 introduction).  Decode is
// the memory-bound regime (§2.5.2): the whole call is ONE kernel launch that
// reads every HBM byte once with wide loads, because on this GPU a launch
// alone costs about as much as streaming the whole layer.
//
// decode_kernel<NW, CPW, ADAPTER>: one workgroup of NW waves per 16 rows of W
// (XCD-aware order), for every problem of a batch.
//  * Main term: the waves split K into 256-wide chunks (wave w owns chunks
//    w, w+NW, ...).  Per chunk and lane: 16 B of packed values, 8 B of
//    metadata and one scale of its row, and 2 x 4 x 16 B of X.  Each 64-k step
//    dequantises one values word in registers and issues one
//    v_smfmac_f32_16x16x64_f16 (W rows are the sparse A side, tokens the B
//    side, zero-padded to 16).
//  * Adapter down (ADAPTER): T = X L is cut into pieces (a 32-column chunk of
//    r times one K split).  Every workgroup claims a piece with an atomic
//    ticket when it starts, computes it with dense MFMA next to its main
//    loop and stores an fp32 partial.  The last piece of a chunk to finish
//    (atomic count) adds the partials in a fixed order (deterministic),
//    stores T in fp16 and publishes it.
//  * Epilogue: the workgroup waits until all chunks of T are published.
//    While it waits it claims and computes any piece no running workgroup has
//    claimed, so the wait cannot depend on a workgroup that is not running
//    (no deadlock whatever the residency), and the spin is bounded.  Then it
//    adds T . R with dense MFMA into the same accumulators (one 32-wide slice
//    of r per wave; R was loaded at the start), reduces the waves in LDS and
//    stores fp16 Y.
//  * The last workgroup to finish resets the tickets: the workspace's counter
//    region is zero before and after every call.
// All data loads are unconditional (clamped addresses, values masked after the
// load) so that every wave has its share of HBM traffic in flight before it
// first waits.
#include "internal.hpp"
#include "mfma_util.hpp"

namespace slim {
namespace {

constexpr int kDecodeMaxM = 16;
constexpr int kDecodeWaves = 16;
constexpr int kDecodeMaxCPW = 4;
constexpr int kMaxSplits = 32;
constexpr int kPieceSteps = 1;        // 32-row MFMA steps per wave per piece

// Counter region (u32 index) of each problem's workspace.
constexpr int kCtrClaim = 0;          // problem 0 only: next unclaimed piece
constexpr int kCtrFinished = 1;       // problem 0 only: finished workgroups
constexpr int kCtrReady = 8;          // chunks of T published
constexpr int kCtrChunk = 16;         // [nR]: pieces of chunk c finished

struct DecodePlan {
    size_t t_off, p_off, total;
    int splits;                       // K splits per chunk of r
    int pieces;                       // pieces per problem
};

DecodePlan decode_plan(int64_t N, int64_t K, int64_t r) {
    DecodePlan p;
    const int64_t nR = r / 32, nsteps = K / 32, C = N / 16;
    int64_t S = nR > 0 ? C / nR : 1;
    if (S > kMaxSplits) S = kMaxSplits;
    if (S > nsteps) S = nsteps;
    const int64_t smin = (nsteps + kDecodeWaves * kPieceSteps - 1) / (kDecodeWaves * kPieceSteps);
    if (S < smin) S = smin;
    if (S < 1) S = 1;
    p.splits = (int)S;
    p.pieces = (int)(nR * S);
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    p.t_off = kCounterRegion;
    p.p_off = p.t_off + al((size_t)kDecodeMaxM * (size_t)r * 2);
    p.total = p.p_off + al((size_t)S * kDecodeMaxM * (size_t)r * sizeof(float));
    return p;
}

struct FusedArgs {
    size_t t_off, p_off;
    int splits, pieces, total_pieces;
};

// Cross-workgroup hand-off without L2 write-back/invalidate fences (which
// serialise across the whole GPU): shared data is written with agent-coherent
// (write-through) stores and read with agent-coherent loads; a writer waits
// for its stores to complete before it bumps a counter with an atomic.
__device__ __forceinline__ void st_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coherent(const uint32_t* p) {
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ unsigned int* counters(const LinearArgs& a, int b) {
    return reinterpret_cast<unsigned int*>(a.ws + (size_t)b * a.ws_per_problem);
}

// Operands of one adapter piece held by one lane between load and compute.
struct PieceRegs {
    h8 x[kPieceSteps], l0[kPieceSteps], l1[kPieceSteps];
};

struct PieceId {
    int b, c, s, st0, st1;
};

__device__ __forceinline__ PieceId piece_id(const LinearArgs& a, const FusedArgs& f, int pid) {
    PieceId p;
    const int nR = (int)(a.r / 32);
    p.b = pid / f.pieces;
    const int local = pid % f.pieces;
    p.c = local % nR;
    p.s = local / nR;
    const int nsteps = (int)(a.K / 32);
    p.st0 = (int)((int64_t)p.s * nsteps / f.splits);
    p.st1 = (int)((int64_t)(p.s + 1) * nsteps / f.splits);
    return p;
}

template <int NW>
__device__ __forceinline__ void piece_load(const LinearArgs& a, const PieceId& p, PieceRegs& pr, int wave,
                                           int lane) {
    const int jl = lane & 15, G = lane >> 4;
    const int m = jl < a.M ? jl : 0;
    const int64_t K = a.K, r = a.r;
    const uint16_t* X = a.X + p.b * a.sX + (int64_t)m * K;
    const uint16_t* L = a.L + p.b * a.sL + 32 * p.c + jl;
#pragma unroll
    for (int u = 0; u < kPieceSteps; ++u) {
        const int st = p.st0 + wave + NW * u;
        const int sc = st < p.st1 ? st : p.st0;             // clamp: always a valid row
        const int64_t k0 = (int64_t)sc * 32 + 8 * G;
        pr.x[u] = load_h8(X + k0);
        const uint16_t* lp = L + k0 * r;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pr.l0[u][e] = __builtin_bit_cast(_Float16, lp[e * r]);
            pr.l1[u][e] = __builtin_bit_cast(_Float16, lp[e * r + 16]);
        }
    }
}

// Compute a loaded piece, store its partial, and if it is the last piece of
// its chunk, reduce the chunk into T and publish it.  Called by the whole
// workgroup (uses LDS and barriers).
template <int NW>
__device__ void piece_finish(const LinearArgs& a, const FusedArgs& f, const PieceId& p, const PieceRegs& pr,
                             f4* lds, int* flag, int wave, int lane) {
    const int jl = lane & 15;
    const bool mval = jl < a.M;
    f4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < kPieceSteps; ++u) {
        const bool live = mval && (p.st0 + wave + NW * u < p.st1);
        const h8 xv = live ? pr.x[u] : h8{};
        acc0 = mfma16(pr.l0[u], xv, acc0);                  // rows j = 4G+v, col m
        acc1 = mfma16(pr.l1[u], xv, acc1);                  // rows j = 16+4G+v
    }
    __syncthreads();                                         // lds free
    lds[(wave * 2 + 0) * 64 + lane] = acc0;
    lds[(wave * 2 + 1) * 64 + lane] = acc1;
    __syncthreads();
    const int64_t r = a.r;
    unsigned char* wsb = a.ws + (size_t)p.b * a.ws_per_problem;
    float* P = reinterpret_cast<float*>(wsb + f.p_off);      // [S][16][r]
    const int t = threadIdx.x;
    if (t < 256) {
        const int half = t >> 7, ln = (t >> 1) & 63, v0 = (t & 1) * 2;
        f4 sum = lds[half * 64 + ln];
#pragma unroll
        for (int w = 1; w < NW; ++w) sum += lds[(w * 2 + half) * 64 + ln];
        const int mm = ln & 15;
        const int j = 32 * p.c + 16 * half + 4 * (ln >> 4) + v0;
        if (mm < a.M) {
            float* dst = P + ((size_t)p.s * kDecodeMaxM + mm) * r + j;
            st_coherent(dst, sum[v0]);
            st_coherent(dst + 1, sum[v0 + 1]);
        }
    }
    wait_stores();                                           // partial is at the coherence point
    __syncthreads();
    unsigned int* ctr = counters(a, p.b);
    if (t == 0) *flag = (atomicAdd(ctr + kCtrChunk + p.c, 1u) == (unsigned)(f.splits - 1));
    __syncthreads();
    if (!*flag) return;
    // Last piece of chunk c: T[m][32c + j] = sum over splits, in split order.
    if (t < kDecodeMaxM * 16) {
        const int mm = t >> 4, j = 32 * p.c + 2 * (t & 15);
        if (mm < a.M) {
            float s0 = 0.0f, s1 = 0.0f;
            for (int q0 = 0; q0 < f.splits; q0 += 8) {        // 8 pairs of loads in flight
                float v0[8], v1[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int qq = q0 + q < f.splits ? q0 + q : 0;
                    const float* src = P + ((size_t)qq * kDecodeMaxM + mm) * r + j;
                    v0[q] = ld_coherent(src);
                    v1[q] = ld_coherent(src + 1);
                }
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    s0 += q0 + q < f.splits ? v0[q] : 0.0f;
                    s1 += q0 + q < f.splits ? v1[q] : 0.0f;
                }
            }
            const h2 pair = {(_Float16)s0, (_Float16)s1};
            st_coherent(reinterpret_cast<uint32_t*>(wsb + f.t_off) + (mm * r + j) / 2,
                        __builtin_bit_cast(uint32_t, pair));
        }
    }
    wait_stores();                                           // T chunk is at the coherence point
    __syncthreads();
    if (t == 0) {
        atomicExch(ctr + kCtrChunk + p.c, 0u);
        atomicAdd(ctr + kCtrReady, 1u);
    }
}

template <int NW, int CPW, bool ADAPTER>
__global__ __launch_bounds__(64 * NW) void decode_kernel(LinearArgs a, FusedArgs f) {
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

    __shared__ f4 lds[NW * 2 * 64];
    __shared__ int sh_piece, sh_flag, sh_state;

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

    // 1. All packed-W loads of this wave (the HBM stream).
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

    // 2. R slice of this wave (one 32-wide block of r), and a piece claim.
    const int nR = (int)(a.r / 32);
    h8 ra = {};
    PieceRegs pr;
    PieceId pid = {};
    int piece = 0;
    if constexpr (ADAPTER) {
        const int jb = wave < nR ? wave : nR - 1;
        const uint16_t* rp = a.R + b * a.sR + (int64_t)(32 * jb + 8 * G) * N + n0 + nl;
#pragma unroll
        for (int e = 0; e < 8; ++e) ra[e] = __builtin_bit_cast(_Float16, rp[e * N]);
        if (threadIdx.x == 0) sh_piece = (int)atomicAdd(counters(a, 0) + kCtrClaim, 1u);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load above is issued before the first wait
    if constexpr (ADAPTER) {
        __syncthreads();
        piece = sh_piece;
        if (piece < f.total_pieces) {
            pid = piece_id(a, f, piece);
            piece_load<NW>(a, pid, pr, wave, lane);
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

    if constexpr (ADAPTER) {
        // 4. The claimed adapter piece.
        if (piece < f.total_pieces) piece_finish<NW>(a, f, pid, pr, lds, &sh_flag, wave, lane);

        // 5. Wait for all of T for this problem; help with unclaimed pieces.
        unsigned int* ctr0 = counters(a, 0);
        unsigned int* ctrb = counters(a, b);
        int spins = 0;
        while (true) {
            if (threadIdx.x == 0) {
                int st = 2;
                if (__hip_atomic_load(ctrb + kCtrReady, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
                    (unsigned)nR) {
                    st = 0;
                } else if (__hip_atomic_load(ctr0 + kCtrClaim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                           (unsigned)f.total_pieces) {
                    const int p2 = (int)atomicAdd(ctr0 + kCtrClaim, 1u);
                    if (p2 < f.total_pieces) {
                        st = 1;
                        sh_piece = p2;
                    }
                }
                sh_state = st;
            }
            __syncthreads();
            const int st = sh_state;
            if (st == 0) break;
            if (st == 1) {
                const PieceId p2 = piece_id(a, f, sh_piece);
                PieceRegs pr2;
                piece_load<NW>(a, p2, pr2, wave, lane);
                piece_finish<NW>(a, f, p2, pr2, lds, &sh_flag, wave, lane);
            } else {
                __builtin_amdgcn_s_sleep(4);
                if (++spins > (1 << 20)) break;          // bounded: never hang the device
            }
            __syncthreads();
        }
        // 6. Epilogue: acc[n][m] += sum_j R[j][n] T[m][j]  (T read coherently).
        const uint32_t* Tb = reinterpret_cast<const uint32_t*>(a.ws + b * a.ws_per_problem + f.t_off);
        auto load_t = [&](int jb) {
            const uint32_t* tp = Tb + ((int64_t)(mval ? m : 0) * a.r + 32 * jb + 8 * G) / 2;
            u4 w = {ld_coherent(tp), ld_coherent(tp + 1), ld_coherent(tp + 2), ld_coherent(tp + 3)};
            return __builtin_bit_cast(h8, w);
        };
        {
            const int jb = wave < nR ? wave : nR - 1;
            const h8 tb = load_t(jb);
            acc = mfma16(wave < nR ? ra : h8{}, mval ? tb : h8{}, acc);
        }
        for (int jb = wave + NW; jb < nR; jb += NW) {      // only when r > 32*NW
            h8 r2;
            const uint16_t* rp = a.R + b * a.sR + (int64_t)(32 * jb + 8 * G) * N + n0 + nl;
#pragma unroll
            for (int e = 0; e < 8; ++e) r2[e] = __builtin_bit_cast(_Float16, rp[e * N]);
            const h8 t2 = load_t(jb);
            acc = mfma16(r2, mval ? t2 : h8{}, acc);
        }
        __syncthreads();                                  // lds free
    }

    // 7. Reduce the waves' partial sums and store fp16 Y.
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

    // 8. The last workgroup to finish leaves the counters at zero.
    if constexpr (ADAPTER) {
        if (threadIdx.x == 0) {
            const unsigned total = gridDim.x * gridDim.y;
            unsigned int* ctr0 = counters(a, 0);
            if (atomicAdd(ctr0 + kCtrFinished, 1u) == total - 1) {
                for (int q = 0; q < (int)a.batch; ++q) atomicExch(counters(a, q) + kCtrReady, 0u);
                atomicExch(ctr0 + kCtrClaim, 0u);
                atomicExch(ctr0 + kCtrFinished, 0u);
            }
        }
    }
}

template <int CPW>
hipError_t launch_decode(const LinearArgs& a, const FusedArgs& f, hipStream_t stream) {
    dim3 grid((unsigned)(a.N / 16), (unsigned)a.batch);
    dim3 block(64 * kDecodeWaves);
    if (a.r > 0)
        hipLaunchKernelGGL((decode_kernel<kDecodeWaves, CPW, true>), grid, block, 0, stream, a, f);
    else
        hipLaunchKernelGGL((decode_kernel<kDecodeWaves, CPW, false>), grid, block, 0, stream, a, f);
    return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int64_t N, int64_t K, int64_t r) { return decode_plan(N, K, r).total; }

bool decode_fits(const LinearArgs& a) {
    const int64_t nch = (a.K + 255) / 256;
    return a.M >= 1 && a.M <= kDecodeMaxM && nch <= (int64_t)kDecodeWaves * kDecodeMaxCPW &&
           a.r / 32 <= 128 && (a.batch * a.N / 16) < (1LL << 31);
}

hipError_t launch_linear_decode(const LinearArgs& a, hipStream_t stream) {
    const DecodePlan p = decode_plan(a.N, a.K, a.r);
    FusedArgs f;
    f.t_off = p.t_off;
    f.p_off = p.p_off;
    f.splits = p.splits;
    f.pieces = p.pieces;
    f.total_pieces = (int)(a.batch * p.pieces);
    const int cpw = (int)(((a.K + 255) / 256 + kDecodeWaves - 1) / kDecodeWaves);
    switch (cpw) {
        case 1: return launch_decode<1>(a, f, stream);
        case 2: return launch_decode<2>(a, f, stream);
        case 3: return launch_decode<3>(a, f, stream);
        default: return launch_decode<4>(a, f, stream);
    }
}

}  // namespace slim
