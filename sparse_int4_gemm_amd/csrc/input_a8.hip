// The layer with an 8-bit input: 4-bit 2:4 weights, int8 activations with
// one fp16 scale per token (Compression Trinity thesis, Appendix E.2 "Input
// Quantization" and the captions of Tables E.2 and E.5: 4-bit weights with
// 8-bit input; §1.2.2: INT8 for activations).
//
//   Y = deq(X) . deq(W_c)^T + (deq(X) . L) . R,   deq(X) = q_x * s_x
//
// quantize_input_kernel: one 256-thread workgroup per token: the row's
//   absmax (exact in fp32), s = fp16(absmax / 127), q = clamp(rint(x / s)),
//   the division IEEE fp32 (bit-exact with the definition).
// prefill_a8_kernel: the prefill tile of 256 rows of W x 128 tokens with the
//   int8 sparse matrix core: v_smfmac_i32_16x16x128_i8 covers exactly one
//   128-k scale group of W, so each instruction yields the group's exact
//   int32 dot products, which are converted to fp32 and scaled by the row's
//   group scale; the token's scale multiplies the finished sums.  The W
//   codes become int8 in registers (sign extension of the nibbles, two byte
//   permutes); X stays int8 from HBM to the matrix core (half the bytes of
//   fp16 X).  It serves layers without an adapter: with one, the dequantised
//   input on the one-pass fp16 prefill (T = X . L first, then the sparse and
//   the dense T . R chunks in one kernel) is faster than this tile followed
//   by a separate T . R pass.
// dequantize_input_kernel: q * s rounded once to fp16, for the shapes that
//   run the fp16 kernels on the dequantised input (decode, where the input
//   is a negligible part of the bytes, prefill with an adapter, and the
//   shapes the prefill tile does not fill).
#include "internal.hpp"
#include "mfma_util.hpp"

namespace slim {

size_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);
bool prefill_fits(const LinearArgs& a);

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kQThreads = 256;
constexpr float kQMaxInput = 127.0f;

// ---------------------------------------------------- per-token quantiser
// PPT: 16-byte pieces of the row per thread held in registers between the
// absmax and the quantisation (0: the row is read twice, for long rows).
template <int PPT>
__global__ __launch_bounds__(kQThreads) void quantize_input_kernel(const uint16_t* X, int64_t K, int8_t* q,
                                                                   uint16_t* s) {
    const int64_t m = blockIdx.x;
    const h8* row = reinterpret_cast<const h8*>(X + m * K);
    const int npc = (int)(K / 8);
    float a = 0.0f;
    h8 held[PPT > 0 ? PPT : 1];
    if constexpr (PPT > 0) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = threadIdx.x + kQThreads * i;
            held[i] = p < npc ? row[p] : h8{};
        }
#pragma unroll
        for (int i = 0; i < PPT; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf((float)held[i][e]));
    } else {
        for (int p = threadIdx.x; p < npc; p += kQThreads) {
            const h8 v = row[p];
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf((float)v[e]));
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    __shared__ float red[kQThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kQThreads / 64; ++w) a = fmaxf(a, red[w]);
    const _Float16 s16 = (_Float16)(a / kQMaxInput);          // IEEE fp32 division, then RNE
    const float sf = (float)s16;
    auto quant8 = [&](const h8& v, int p) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float t = sf > 0.0f ? __builtin_rintf((float)v[e] / sf) : 0.0f;
            t = fminf(fmaxf(t, -kQMaxInput), kQMaxInput);
            const uint32_t byte = (uint32_t)(int)t & 0xFFu;
            if (e < 4) lo |= byte << (8 * e);
            else       hi |= byte << (8 * (e - 4));
        }
        *reinterpret_cast<u2*>(q + m * K + 8 * p) = u2{lo, hi};
    };
    if constexpr (PPT > 0) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = threadIdx.x + kQThreads * i;
            if (p < npc) quant8(held[i], p);
        }
    } else {
        for (int p = threadIdx.x; p < npc; p += kQThreads) quant8(row[p], p);
    }
    if (threadIdx.x == 0) s[m] = __builtin_bit_cast(uint16_t, s16);
}

// ------------------------------------------------- q * s -> fp16 (decode)
__global__ __launch_bounds__(256) void dequantize_input_kernel(const int8_t* q, const uint16_t* s, int64_t M,
                                                               int64_t K, uint16_t* X) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;          // piece of 8
    if (i >= M * K / 8) return;
    const int64_t m = i / (K / 8);
    const float sf = (float)__builtin_bit_cast(_Float16, s[m]);
    const u2 w = *reinterpret_cast<const u2*>(q + 8 * i);
    h8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int8_t b = (int8_t)((e < 4 ? w[0] : w[1]) >> (8 * (e & 3)));
        out[e] = (_Float16)((float)b * sf);                      // exact product, one rounding
    }
    *reinterpret_cast<h8*>(X + 8 * i) = out;
}

// ---------------------------------------------------------- prefill, int8
// Sign extension of packed 4-bit two's complement bytes (each byte 0..15):
// ((x ^ 8) + 120) ^ 128, no carry between bytes.
__device__ __forceinline__ uint32_t sext_nibble_bytes(uint32_t x) {
    return ((x ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
}

// One packed values word (8 kept int4 codes of 4 groups: bits [4j, 4j+4) the
// lower-index value of group j, [16+4j, ..) the higher) -> two dwords of
// int8 in smfmac A order (lo0 hi0 lo1 hi1 | lo2 hi2 lo3 hi3).
__device__ __forceinline__ void int4_word_to_int8(uint32_t w, uint32_t& d0, uint32_t& d1) {
    const uint32_t e = sext_nibble_bytes(w & 0x0F0F0F0Fu);          // lo0 lo2 hi0 hi2
    const uint32_t o = sext_nibble_bytes((w >> 4) & 0x0F0F0F0Fu);   // lo1 lo3 hi1 hi3
    d0 = __builtin_amdgcn_perm(o, e, 0x06040200u);
    d1 = __builtin_amdgcn_perm(o, e, 0x07050301u);
}


constexpr int kAN = 256;                 // W rows per workgroup
constexpr int kAM = 128;                 // tokens per workgroup
constexpr int kAK = 128;                 // k per chunk: one scale group, one int8 smfmac
constexpr int kAThreads = 512;           // 8 waves: wave w rows 64 (w & 3), tokens 64 (w >> 2)
constexpr int kAGroupM = 4;              // m-blocks per XCD group of tiles
// LDS of one stage: X int8 rows [128][128 B] (16-byte unit u of row p at slot
// u ^ (p & 7)); values [16 blocks][512 B] (row i's halves at slots 2i + (h ^
// ((i / 4) & 1))); metadata [16][256 B]; scales [16][32 B] in a 1 KB area.
constexpr int kAX = 0;
constexpr int kAV = kAX + kAM * kAK;
constexpr int kAMeta = kAV + kAN * 32;
constexpr int kAS = kAMeta + kAN * 16;
constexpr int kAStage = kAS + 1024;
constexpr int kAStages = 3;
constexpr int kAOps = 4;                 // per wave and chunk: 2 X, 1 values, 1 metadata or scales
static_assert(kAStages * kAStage <= 160 * 1024, "stages must fit in LDS");
static_assert(kAM * kAK / 1024 == 2 * (kAThreads / 64), "two 1 KB X loads per wave and chunk");

// One problem without an adapter: the input is qx [M][K] int8 with scales sx
// [M] fp16 (a.X unused); Y = deq(X) . deq(W_c)^T.
__global__ __launch_bounds__(kAThreads) void prefill_a8_kernel(LinearArgs a, const int8_t* qx, const uint16_t* sx) {
    const int64_t K = a.K, N = a.N, M = a.M;
    const int nNB = (int)((N + kAN - 1) / kAN), nMB = (int)((M + kAM - 1) / kAM);
    // XCD-aware tile order, as the fp16 prefill kernel.
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int gsize = kAGroupM * nNB, gid = L / gsize, fm = gid * kAGroupM;
    const int gm = nMB - fm < kAGroupM ? nMB - fm : kAGroupM;
    const int mb = __builtin_amdgcn_readfirstlane(fm + (L % gsize) % gm);
    const int nb = __builtin_amdgcn_readfirstlane((L % gsize) / gm);
    const int64_t n0 = (int64_t)nb * kAN, m0 = (int64_t)mb * kAM;
    const int nch = (int)(K / kAK);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = wave & 3, mh = wave >> 2;
    const int nl = lane & 15, G = lane >> 4;

    __shared__ __attribute__((aligned(16))) unsigned char lds[kAStages * kAStage];

    const u4 rx = rsrc_words(qx + m0 * K, (M - m0) * K);
    const u4 rv = rsrc_words(a.values + n0 * (K / 4), (N - n0) * (K / 4));
    const u4 rm = rsrc_words(a.meta + n0 * (K / 8), (N - n0) * (K / 8));
    const u4 rs = rsrc_words(a.scales + n0 * (K / kGroup), (N - n0) * (K / kGroup) * 2);

    // Per-lane offsets of the direct loads.  X load j of wave w: rows
    // 16w + 8j + l / 8, slot l % 8 (global unit (l % 8) ^ row).  Values:
    // blocks 2w, 2w + 1.  Metadata (waves 0-3): blocks 4w .. 4w + 3; scales
    // (waves 4-7, the same bytes): lanes 0-31.
    int dxo[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int p = 16 * wave + 8 * j + (lane >> 3);
        dxo[j] = (int)(p * K + 16 * ((lane & 7) ^ (p & 7)));
    }
    const int vs = lane & 31, vrow = vs >> 1, vhalf = (vs & 1) ^ ((vrow >> 2) & 1);
    const int dvo = (int)((2 * wave + (lane >> 5)) * 16 * (K / 4) + 32 * vrow + 16 * vhalf);
    const bool aux_meta = wave < 4;
    const int dao = aux_meta  ? (int)((4 * wave + (lane >> 4)) * 16 * (K / 8) + 16 * (lane & 15))
                  : lane < 32 ? (int)((lane >> 1) * 16 * (K / kGroup) * 2 + 16 * (lane & 1))
                              : kOOB;
    auto issue = [&](int ch) __attribute__((always_inline)) {
        unsigned char* st = lds + (ch % kAStages) * kAStage;
        ch = ch < nch ? ch : nch - 1;                      // past the end: a repeat of the last chunk
#pragma unroll
        for (int j = 0; j < 2; ++j) lds_load16(rx, st + kAX + (16 * wave + 8 * j) * 128, dxo[j], ch * kAK);
        lds_load16(rv, st + kAV + wave * 1024, dvo, ch * 512);
        if (aux_meta) lds_load16(rm, st + kAMeta + wave * 1024, dao, ch * 256);
        else          lds_load16(rs, st + kAS, dao, ch * 32);
    };

    f4 acc[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[f][g] = f4{0, 0, 0, 0};

    auto compute = [&](const unsigned char* st) __attribute__((always_inline)) {
        // A: lane row nl of fragment f, dense k 32G .. 32G + 32 (16-k blocks
        // 2G, 2G + 1: the values words 2G, 2G + 1 and their metadata halves).
        v4i A[4];
        uint32_t mw[4];
        f4 sw[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int blk = 4 * rg + f;
            const u2 vw = *reinterpret_cast<const u2*>(st + kAV + 512 * blk +
                                                        16 * (2 * nl + ((G >> 1) ^ ((nl >> 2) & 1))) + 8 * (G & 1));
            uint32_t d0, d1, d2, d3;
            int4_word_to_int8(vw[0], d0, d1);
            int4_word_to_int8(vw[1], d2, d3);
            A[f] = v4i{(int)d0, (int)d1, (int)d2, (int)d3};
            mw[f] = *reinterpret_cast<const uint32_t*>(st + kAMeta + 256 * blk + 16 * nl + 4 * G);
            // scales of the D rows 4G .. 4G + 3 of this fragment
            const h4 s4 = *reinterpret_cast<const h4*>(st + kAS + 32 * blk + 8 * G);
            sw[f] = f4{(float)s4[0], (float)s4[1], (float)s4[2], (float)s4[3]};
        }
        // All 16 products first, each into registers of its own, then the
        // conversions: one shared destination would make every product wait
        // for the conversion of the one before it.
        v4i d[4][4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int p = 64 * mh + 16 * g + nl;
            const unsigned char* xr = st + kAX + p * 128;
            const u4 x0 = *reinterpret_cast<const u4*>(xr + 16 * (G ^ (p & 7)));
            const u4 x1 = *reinterpret_cast<const u4*>(xr + 16 * ((4 + G) ^ (p & 7)));
            const v8i B = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
#pragma unroll
            for (int f = 0; f < 4; ++f)
                d[f][g] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(A[f], B, v4i{0, 0, 0, 0}, (int)mw[f], 0, 0);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[f][g][v] = fmaf((float)d[f][g][v], sw[f][v], acc[f][g][v]);
    };

    // Pipeline: chunks 0 .. S-2 in flight; iteration ch waits for this wave's
    // loads of chunk ch, one barrier (all of chunk ch in LDS, stage (ch-1) % S
    // no longer read), issues chunk ch + S - 1 into that stage, computes ch.
#pragma unroll
    for (int i = 0; i < kAStages - 1; ++i) issue(i);
    for (int ch = 0; ch < nch; ++ch) {
        wait_vmem_below<kAOps * (kAStages - 2)>();
        __syncthreads();
        issue(ch + kAStages - 1);
        compute(lds + (ch % kAStages) * kAStage);
    }
    wait_vmem_below<0>();
    __syncthreads();

    // The token's scale: lane holds token 64 mh + 16 g + nl (rows 4G + v).
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int64_t m = m0 + 64 * mh + 16 * g + nl;
        if (m >= M) continue;
        const float s = (float)__builtin_bit_cast(_Float16, sx[m]);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int64_t n = n0 + 64 * rg + 16 * f + 4 * G;
            if (n >= N) continue;
            const h4 out = {(_Float16)(acc[f][g][0] * s), (_Float16)(acc[f][g][1] * s), (_Float16)(acc[f][g][2] * s),
                            (_Float16)(acc[f][g][3] * s)};
            *reinterpret_cast<h4*>(a.Y + m * N + n) = out;
        }
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The int8 prefill tile applies without an adapter when there are enough
// tiles to fill the GPU unsplit (at least 128 of them); 32-bit offsets within
// each buffer a workgroup addresses.
bool prefill_a8_fits(const LinearArgs& a) {
    const int64_t tiles = ((a.N + kAN - 1) / kAN) * ((a.M + kAM - 1) / kAM);
    const int64_t lim = 0x7FFFFFF0;
    return a.r == 0 && a.M > 16 && tiles >= 128 && prefill_fits(a) && a.M * a.K < lim && a.N * (a.K / 4) < lim;
}

}  // namespace

size_t linear_a8_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
    return align256(linear_workspace_bytes(M, N, K, r)) + align256((size_t)M * K * 2);
}

hipError_t launch_quantize_input(const uint16_t* X, int64_t M, int64_t K, int8_t* q, uint16_t* s,
                                 hipStream_t stream) {
    const int64_t ppt = (K / 8 + kQThreads - 1) / kQThreads;
    const dim3 grid((unsigned)M), block(kQThreads);
    if (ppt <= 2)      hipLaunchKernelGGL(quantize_input_kernel<2>, grid, block, 0, stream, X, K, q, s);
    else if (ppt <= 4) hipLaunchKernelGGL(quantize_input_kernel<4>, grid, block, 0, stream, X, K, q, s);
    else if (ppt <= 8) hipLaunchKernelGGL(quantize_input_kernel<8>, grid, block, 0, stream, X, K, q, s);
    else               hipLaunchKernelGGL(quantize_input_kernel<0>, grid, block, 0, stream, X, K, q, s);
    return hipGetLastError();
}

// One problem (batch 1): a.X is unused; the input is qx [M][K] int8 and sx [M] fp16.
// The int8 core serves prefill shapes without an adapter.  With one, the
// fp16 one-pass prefill on the dequantised input (its T . R chunks continue
// the main accumulators) is faster than this kernel followed by the T . R
// pass: down at 2048 tokens 164.2 against 185.8 us, gate/up 178.8 against
// 235.2 us, q_proj 88.1 against 94.9 us (graph-timed, one box); without one
// the two take the same time (down: 121.6 and 119.0 us).
hipError_t launch_linear_a8(const LinearArgs& a, const int8_t* qx, const uint16_t* sx, hipStream_t stream) {
    if (prefill_a8_fits(a)) {
        const unsigned tiles = (unsigned)(((a.N + kAN - 1) / kAN) * ((a.M + kAM - 1) / kAM));
        hipLaunchKernelGGL(prefill_a8_kernel, dim3(tiles, 1u), dim3(kAThreads), 0, stream, a, qx, sx);
        return hipGetLastError();
    }
    // The fp16 kernels on q * s (one rounding), the dequantised input in the
    // workspace after the fp16 path's own region.
    uint16_t* xd = reinterpret_cast<uint16_t*>(a.ws + align256(linear_workspace_bytes(a.M, a.N, a.K, a.r)));
    const int64_t pieces = a.M * a.K / 8;
    hipLaunchKernelGGL(dequantize_input_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream, qx, sx,
                       a.M, a.K, xd);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    LinearArgs b = a;
    b.X = xd;
    return launch_linear(b, stream);
}

}  // namespace slim
