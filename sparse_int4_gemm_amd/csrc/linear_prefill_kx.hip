// slim_linear for prefill-shaped problems (M > 16 tokens): MFMA-bound.
//
//   Y = X . deq(W_c)^T + T . R,   T = X . L
//     = [X | T] . [deq(W_c)^T ; R]
//
// Layer: Compression Trinity thesis §2.1 (Y = X W^T) with the sparse weight
// and the low-rank adapter as parallel paths (Ch. 4 introduction); prefill is
// the compute-bound regime (§2.5.1), so the work goes to the matrix cores: 2:4
// sparse MFMA for the main term (§2.2.3: only the kept half of W is
// multiplied) and dense MFMA for the adapter.  The adapter's second product
// continues the main product along the reduction axis (the second line
// above): one set of fp32 accumulators takes the K/128 sparse chunks of
// X . deq(W_c)^T and then the r/64 dense chunks of T . R, and Y is written
// once, in fp16.
//
// kx_t_kernel: T = X . L with dense v_mfma_f32_16x16x32_f16, 256 adapter
//   columns x 128 tokens per workgroup, K split over workgroups so that the
//   GPU is full; fp32 partials that kx_t_reduce_kernel sums into fp16 T.
// kx_main_kernel: one 8-wave workgroup per 256 rows of W x 128 tokens.  Wave
//   (rg, t) owns rows 64 rg .. +64 (4 fragments) for all 128 tokens (8
//   fragments) and half t of every chunk's reduction; the two waves of a row
//   group run on one SIMD and add their halves at the end.  So every W
//   fragment is dequantised once per workgroup, each wave's dequantisation of
//   chunk c + 1 runs between its matrix instructions of chunk c, and the
//   other wave on the SIMD keeps the matrix core busy meanwhile.  This path
//   takes problems with enough 256 x 128 tiles to fill the GPU (M = 2048 at
//   the LLaMA-2-7B widths); fewer tiles go to the K-split prefill kernels.
//
// Every operand goes from HBM straight into LDS (buffer loads with the LDS
// destination: no registers, no LDS store instructions), three stages deep;
// the loads are written as asm (no register outputs) and ordered with
// explicit vmcnt waits, since the compiler cannot see which LDS bytes such a
// load writes.
#include "internal.hpp"
#include "mfma_util.hpp"

namespace slim {
namespace {

constexpr int kTN = 256;            // W rows (or adapter rows) per tile
constexpr int kTM = 128;            // tokens per tile
constexpr int kCK = 128;            // k per sparse chunk: one scale group
constexpr int kDC = 64;             // reduction columns per dense chunk
constexpr int kThreads = 512;       // 8 waves, two per SIMD
constexpr int kGroupM = 4;          // m-blocks per group of tiles
constexpr int kMaxTSplit = 16;      // workgroups sharing one T tile
constexpr int kOps = 6;             // direct loads per wave and chunk, both phases

// LDS, sparse phase: three W stages (values [16 blocks][16 rows x 32 B],
// metadata [16][16 x 16 B] and scales [16][16 x 2 B] in a 1 KB area, in the
// packed format's block order), then three X stages [128 rows][256 B]
// (16-byte unit u of row rho at slot u ^ (rho & 15)).  W first: its reads
// then fit the 16-bit offset field of the LDS instructions.
constexpr int kXRow = kCK * 2;
constexpr int kXStage = kTM * kXRow;                          // 32 KB
constexpr int kWV = 0, kWM = kTN * 32, kWS = kWM + kTN * 16;
constexpr int kWStage = kWS + 1024;                           // 13 KB
constexpr int kWBase = 0, kXBase = 3 * kWStage;
// LDS, dense phase: three stages of B rows [128][128 B] then A rows
// [256][128 B] (16-byte unit u of row rho at slot u ^ (rho & 7)).
constexpr int kDRow = kDC * 2;
constexpr int kDB = 0, kDA = kTM * kDRow;
constexpr int kDStage = kDA + kTN * kDRow;                    // 48 KB
// LDS, final exchange of the two reduction halves: [4 row groups][2][4
// token fragments][4 row fragments][64 lanes] f4.
constexpr int kXchBytes = 4 * 2 * 4 * 4 * 64 * 16;           // 128 KB
constexpr int kSparseLds = kXBase + 3 * kXStage;
constexpr int kMax2(int x, int y) { return x > y ? x : y; }
constexpr int kLdsBytes = kMax2(kMax2(3 * kDStage, kSparseLds), kXchBytes);
static_assert(kLdsBytes <= 160 * 1024, "stages must fit in LDS");
static_assert(kXStage / 1024 == 4 * (kThreads / 64) && kTN * 32 / 1024 == kThreads / 64 &&
                  kTN * 16 / 1024 == kThreads / 128,
              "sparse chunk, per wave: 4 X loads, 1 values load and 1 metadata-or-scale load of 1 KB");
static_assert(kTM * kDRow / 1024 == 2 * (kThreads / 64) && kTN * kDRow / 1024 == 4 * (kThreads / 64),
              "dense chunk, per wave: 2 B-row and 4 A-row loads of 1 KB");

// Workspace of one problem: T fp16 [M][r] at t_off; fp32 partials of T at
// tp_off when K is split for T, tile-major: [tsplit][T tile mb * nJB +
// jb][wave][f][g - 4 t][64 lanes] f4 (each wave's 16 fragments after the
// halves are added: 16 KB of contiguous memory, whole-line 1 KB stores).
struct KxPlan {
    int tsplit;
    size_t t_off, tp_off, total;
};

KxPlan kx_plan(int64_t M, int64_t K, int64_t r) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    KxPlan p;
    const int64_t nMB = (M + kTM - 1) / kTM;
    // T tiles (256 adapter columns x 128 tokens) are few: split K so that
    // the workgroups fill one round of the 256 CUs (one per CU: the stages
    // take most of the LDS).
    int64_t St = 1;
    const int64_t ttiles = ((r + kTN - 1) / kTN) * nMB;
    if (ttiles > 0) {
        St = 256 / ttiles;
        if (St > kMaxTSplit) St = kMaxTSplit;
        if (St > K / kDC) St = K / kDC;
        if (St < 1) St = 1;
    }
    p.tsplit = (int)St;
    p.t_off = kCounterRegion;
    p.tp_off = p.t_off + al((size_t)M * (size_t)r * 2);
    p.total = p.tp_off + (St > 1 ? al((size_t)St * ttiles * kTN * kTM * 4) : 0);
    return p;
}

__device__ __forceinline__ int rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }

// ------------------------------------------------------------ dense phase
// acc[f][g] += sum over the reduction columns of chunks [d0, d0 + nd) (64
// each) that fall in half t (32-column step t of each chunk) of
// A[64 rg + 16 f + i][c] . B[16 g + j][c] (i, j: the lane's row of the
// fragment), for A and B fp16 row-major with leading dimension ld from the
// buffer descriptors ra, rb (rows past each buffer read zero) and columns at
// or past len reading zero.  Direct loads of chunk c, per wave w: B load i
// (0, 1) fills B rows 8 (2w + i) .. +8, A load i (0..3) A rows 8 (4w + i) ..
// +8; lane l: row base + l / 8, slot l % 8, i.e. global unit (l % 8) ^ row.
// Uses the whole LDS; returns with every load landed and the LDS free.
__device__ __forceinline__ void dense_phase(u4 ra, u4 rb, int64_t ld, int64_t len, int d0, int nd,
                                            unsigned char* lds, f4 (&acc)[4][8], int wave, int rg, int t,
                                            int lane) {
    const int nl = lane & 15, G = lane >> 4;
    const int drow = lane >> 3, dslot = lane & 7;
    const uint32_t L = lds_u32(lds);
    auto dma = [&](int st, int ch, int i) __attribute__((always_inline)) {
        ch = d0 + (ch < nd ? ch : nd - 1);                   // past the end: a repeat of the last chunk
        const int row = (i < 2 ? 8 * (2 * wave + i) : 8 * (4 * wave + i - 2)) + drow;
        const int u = dslot ^ (row & 7);
        const bool ok = (int64_t)ch * kDC + 8 * u < len;
        const int voff = ok ? (int)((row * ld + 8 * u) * 2) : kOOB;
        if (i < 2) lds_load16_at(rb, L + st + kDB + (2 * wave + i) * 1024, voff, ch * kDRow);
        else       lds_load16_at(ra, L + st + kDA + (4 * wave + i - 2) * 1024, voff, ch * kDRow);
    };
    const int slot = 16 * ((4 * t + G) ^ (nl & 7));
    const uint32_t aa = L + kDA + (64 * rg + nl) * kDRow + slot, ba = L + kDB + nl * kDRow + slot;
    h8 A[4], B[8];
    auto read_ops = [&](int st, h8 (&a)[4], h8 (&bb)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < 4; ++f) a[f] = lds_ld<h8>(aa + st + 16 * f * kDRow);
#pragma unroll
        for (int g = 0; g < 8; ++g) bb[g] = lds_ld<h8>(ba + st + 16 * g * kDRow);
    };
    constexpr int st0 = 0, st1 = kDStage, st2 = 2 * kDStage;
#pragma unroll
    for (int i = 0; i < kOps; ++i) dma(st0, 0, i);
#pragma unroll
    for (int i = 0; i < kOps; ++i) dma(st1, 1, i);
    wait_vmem_below<kOps>();
    __syncthreads();
    read_ops(st0, A, B);
    // Iteration ch starts with the operands of chunk ch read; steps 0-5
    // issue chunk ch + 2's loads into the stage read in iteration ch - 1.
    // The barrier comes after step 5: past it chunk ch + 1 is complete in
    // LDS and its operands are read while steps 6 and 7 run.
    auto step = [&](int next, int next2, int ch) __attribute__((always_inline)) {
        h8 An[4], Bn[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            if (g == 6) {
                wait_vmem_below<kOps>();
                __syncthreads();
                read_ops(next, An, Bn);
            }
#pragma unroll
            for (int f = 0; f < 4; ++f) acc[f][g] = mfma16(A[f], B[g], acc[f][g]);
            if (g < kOps) dma(next2, ch + 2, g);
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) A[f] = An[f];
#pragma unroll
        for (int g = 0; g < 8; ++g) B[g] = Bn[g];
    };
    int ch = 0;
    for (; ch + 3 <= nd; ch += 3) {
        step(st1, st2, ch);
        step(st2, st0, ch + 1);
        step(st0, st1, ch + 2);
    }
    if (ch < nd) step(st1, st2, ch);
    if (ch + 1 < nd) step(st2, st0, ch + 1);
    wait_vmem_below<0>();
    __syncthreads();
}

// ------------------------------------------------------------ sparse phase
// acc[f][g] += the main product over half t of sparse chunks [c0, c0 + n)
// of the tile at rows n0, tokens m0: X rows m0 + 16 g + j (the lane's
// token), W rows n0 + 64 rg + 16 f + i.  Half t of a chunk is the 16-k
// blocks 2G + t (G = 0..3) of its eight: one values word and one 16-bit
// metadata field per lane and row fragment, the smfmac B operand from the
// matching X columns.
//
// Iteration c computes chunk c with the A fragments dequantised in iteration
// c - 1, and meanwhile reads and dequantises the W of chunk c + 1; so W runs
// one chunk ahead of X.  Loads issued in iteration c: X of chunk c + 2 (4 per
// wave) and W of chunk c + 3 (2 per wave); iteration c waits for X of c and W
// of c + 1, issued in iteration c - 2, i.e. for all but the last kOps.  X and
// W stages rotate with period 3: X of c + 2 goes into the X stage read in
// iteration c - 1, W of c + 3 into the W stage of chunk c, read in iteration
// c - 1.
//
// Direct loads per wave w and chunk: X load j (0..3) fills X rows 4 (4w + j)
// .. +4 (lane l: row base + l / 16, slot l % 16, i.e. global unit
// (l % 16) ^ row); the values load fills blocks 2w, 2w + 1 (lane l: block
// 2w + l / 32, slot s = l % 32 holding row s / 2 and half
// (s % 2) ^ ((row / 4) % 2)); the last load is metadata blocks 4w .. +4
// (waves 0-3; lane l: block 4w + l / 16, row l % 16) or the 16 blocks'
// scales (waves 4-7 all load the same bytes to the same place: lanes 0-31,
// the others read zero into the second half of the 1 KB area).  Rows past M
// or N read zero.
template <int t>
__device__ __forceinline__ void sparse_phase(const LinearArgs& a, int b, int64_t n0, int64_t m0, int c0, int n,
                                             unsigned char* lds, f4 (&acc)[4][8], int wave, int rg, int lane) {
    const int64_t K = a.K, N = a.N, M = a.M;
    const int nl = lane & 15, G = lane >> 4;
    const u4 rx = rsrc_words(a.X + b * a.sX + m0 * K, (M - m0) * K * 2);
    const u4 rv = rsrc_words(a.values + b * a.sV + n0 * (K / 4), (N - n0) * (K / 4));
    const u4 rm = rsrc_words(a.meta + b * a.sMeta + n0 * (K / 8), (N - n0) * (K / 8));
    const u4 rs = rsrc_words(a.scales + b * a.sS + n0 * (K / kGroup), (N - n0) * (K / kGroup) * 2);

    const int drow = lane >> 4, dslot = lane & 15;
    int dxo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 4 * (4 * wave + j) + drow;
        dxo[j] = (int)(row * K * 2 + 16 * (dslot ^ (row & 15)));
    }
    const int vs = lane & 31, vrow = vs >> 1, vhalf = (vs & 1) ^ ((vrow >> 2) & 1);
    const int dvo = (int)((2 * wave + (lane >> 5)) * 16 * (K / 4) + 32 * vrow + 16 * vhalf);
    const bool aux_meta = wave < 4;
    const int dao = aux_meta  ? (int)((4 * wave + (lane >> 4)) * 16 * (K / 8) + 16 * (lane & 15))
                  : lane < 32 ? (int)((lane >> 1) * 16 * (K / kGroup) * 2 + 16 * (lane & 1))
                              : kOOB;
    // The metadata-or-scale load as uniform selects, not a branch: the loop
    // body stays one basic block for the scheduler.
    const u4 raux = aux_meta ? rm : rs;
    const int aux_dst = aux_meta ? kWM + wave * 1024 : kWS, aux_step = aux_meta ? 256 : 32;

    const uint32_t L = lds_u32(lds);
    auto xdma = [&](int s, int ch, int j) __attribute__((always_inline)) {
        ch = c0 + (ch < n ? ch : n - 1);                    // past the end: a repeat of the last chunk
        lds_load16_at(rx, L + kXBase + s * kXStage + (4 * wave + j) * 1024, dxo[j], ch * kXRow);
    };
    auto wdma = [&](int s, int ch, int i) __attribute__((always_inline)) {
        ch = c0 + (ch < n ? ch : n - 1);
        const uint32_t st = L + kWBase + s * kWStage;
        if (i == 0) lds_load16_at(rv, st + kWV + wave * 1024, dvo, ch * 512);
        else        lds_load16_at(raux, st + aux_dst, dao, ch * aux_step);
    };
    // This lane's W rows 64 rg + 16 f + nl (block 4 rg + f, row nl): the
    // values word of 16-k block 2G + t, the metadata word (both halves; the
    // smfmac takes half t) and the dword holding the scale.  Fragments f and
    // f + 1 are 512, 256 and 32 bytes apart: one two-address LDS read each.
    const uint32_t wva = L + kWBase + kWV + 2048 * rg + 16 * (2 * nl + ((G >> 1) ^ ((nl >> 2) & 1))) + 8 * (G & 1) + 4 * t;
    const uint32_t wma = L + kWBase + kWM + 1024 * rg + 16 * nl + 4 * G;
    const uint32_t wsa = L + kWBase + kWS + 128 * rg + 4 * (nl >> 1);
    const uint32_t ssel = (nl & 1) ? 0x07060706u : 0x05040504u;   // the lane's scale in both halves
    auto read_w2 = [&](int s, int f, uint32_t (&vw)[2], uint32_t (&mw)[2], uint32_t (&sw)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            vw[i] = lds_ld<uint32_t>(wva + s * kWStage + 512 * (f + i));
            mw[i] = lds_ld<uint32_t>(wma + s * kWStage + 256 * (f + i));
            sw[i] = lds_ld<uint32_t>(wsa + s * kWStage + 32 * (f + i));
        }
    };
    auto scale2 = [&](uint32_t sw) __attribute__((always_inline)) {
        return __builtin_bit_cast(h2, __builtin_amdgcn_perm(sw, sw, ssel));
    };

    // Prologue: W of chunk 0, X of 0, W of 1 | X of 1, W of 2; then the
    // first A fragments from W of chunk 0.
#pragma unroll
    for (int i = 0; i < 2; ++i) wdma(0, 0, i);
#pragma unroll
    for (int j = 0; j < 4; ++j) xdma(0, 0, j);
#pragma unroll
    for (int i = 0; i < 2; ++i) wdma(1, 1, i);
#pragma unroll
    for (int j = 0; j < 4; ++j) xdma(1, 1, j);
#pragma unroll
    for (int i = 0; i < 2; ++i) wdma(2, 2, i);
    wait_vmem_below<kOps + 6>();
    __syncthreads();
    h8 A[4];
    uint32_t mw[4];
#pragma unroll
    for (int f = 0; f < 4; f += 2) {
        uint32_t vw[2], mw2[2], sw[2];
        read_w2(0, f, vw, mw2, sw);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            mw[f + i] = mw2[i];
            dequant_word_fast(vw[i], scale2(sw[i]), A[f + i]);
        }
    }

    const int gA1 = G >> 1, gA2 = 2 + (G >> 1), hl = G & 1;
    auto slot = [&](int u) { return 16 * (u ^ nl); };    // unit u of a row congruent to nl mod 16
    const int ua = slot(2 * (2 * gA1 + t) + hl), ub = slot(2 * (2 * gA2 + t) + hl);
    const uint32_t xa = L + kXBase + nl * kXRow + ua, xb = L + kXBase + nl * kXRow + ub;
    auto readB = [&](int xs, int g) __attribute__((always_inline)) {
        const uint32_t o = xs * kXStage + 16 * g * kXRow;
        return concat8(lds_ld<h8>(xa + o), lds_ld<h8>(xb + o));
    };
    // X of chunk 0 and W of chunk 1 visible (all but the last kOps loads),
    // then the first two B operands.
    wait_vmem_below<kOps>();
    __syncthreads();
    h16 Bq[3];
    Bq[0] = readB(0, 0);
    Bq[1] = readB(0, 1);

    // Iteration ch (X of ch in stage xs, W of ch + 1 in stage wn; X of ch + 2
    // goes to stage xs2, W of ch + 3 to stage wn2) starts with A, mw and the
    // first two B operands of chunk ch in registers.  Its barrier comes
    // after step 6, when every LDS read of X of ch and W of ch + 1 has been
    // issued: past it X of ch + 1 and W of ch + 2 are visible, the first B
    // operands of chunk ch + 1 are read, and step 7's matrix instructions
    // (operands in registers) cover their latency.  The direct loads of
    // steps 0-5 go into the stages whose reads ended before the previous
    // barrier.
    auto step = [&](int xs, int wn, int xs2, int wn2, int ch) __attribute__((always_inline)) {
        h8 An[4];
        uint32_t mwn[4], vwn[4], swn[4];
        h16 Bn0, Bn1;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            if (g + 2 < 8) Bq[(g + 2) % 3] = readB(xs, g + 2);
            if (g == 0 || g == 2) {
                uint32_t v2[2], m2[2], s2[2];
                read_w2(wn, g, v2, m2, s2);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    vwn[g + i] = v2[i];
                    mwn[g + i] = m2[i];
                    swn[g + i] = s2[i];
                }
            }
            if (g == 7) {
                wait_vmem_below<kOps>();
                __syncthreads();
                Bn0 = readB(wn, 0);                  // X of chunk ch + 1: stage (ch + 1) % 3 = wn
                Bn1 = readB(wn, 1);
            }
            const h16 B = Bq[g % 3];
#pragma unroll
            for (int f = 0; f < 4; ++f) acc[f][g] = smfmac<t>(A[f], B, acc[f][g], mw[f]);
            if (g >= 1 && g <= 4) {
                dequant_word_fast(vwn[g - 1], scale2(swn[g - 1]), An[g - 1]);
                asm volatile("" : "+v"(An[g - 1]));       // computed here, not at its first use
            }
            if (g < 4)       xdma(xs2, ch + 2, g);
            else if (g < 6)  wdma(wn2, ch + 3, g - 4);
            // Keep each step's dequantisation among its matrix instructions
            // (left alone, the compiler gathers it at the next iteration's
            // start, where nothing hides it).
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            A[f] = An[f];
            mw[f] = mwn[f];
        }
        Bq[0] = Bn0;
        Bq[1] = Bn1;
    };
    int ch = 0;
    for (; ch + 3 <= n; ch += 3) {
        step(0, 1, 2, 0, ch);
        step(1, 2, 0, 1, ch + 1);
        step(2, 0, 1, 2, ch + 2);
    }
    if (ch < n) step(0, 1, 2, 0, ch);
    if (ch + 1 < n) step(1, 2, 0, 1, ch + 1);
    wait_vmem_below<0>();
    __syncthreads();
}

// The two waves of row group rg hold the reduction halves t = 0, 1 of the
// same outputs: each gives the other the token fragments it does not own
// (through LDS; the stages are free), then adds the half it receives to its
// own fragments g = 4t .. 4t + 3.  (T is a template argument so that every
// register index is a constant.)
template <int T>
__device__ __forceinline__ void combine_halves_t(unsigned char* lds, f4 (&acc)[4][8], int rg, int lane) {
    f4* x = reinterpret_cast<f4*>(lds);
#pragma unroll
    for (int gl = 0; gl < 4; ++gl)
#pragma unroll
        for (int f = 0; f < 4; ++f) x[(((rg * 2 + T) * 4 + gl) * 4 + f) * 64 + lane] = acc[f][4 * (1 - T) + gl];
    __syncthreads();
#pragma unroll
    for (int gl = 0; gl < 4; ++gl)
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[f][4 * T + gl] += x[(((rg * 2 + (1 - T)) * 4 + gl) * 4 + f) * 64 + lane];
}

__device__ __forceinline__ void combine_halves(unsigned char* lds, f4 (&acc)[4][8], int rg, int t, int lane) {
    if (t == 0) combine_halves_t<0>(lds, acc, rg, lane);
    else        combine_halves_t<1>(lds, acc, rg, lane);
}

// Stores this wave's fragments g = 4T .. 4T + 3: out(f, g, acc[f][g]) for
// the rows n0 + 64 rg + 16 f + 4 G .. +4 and token m0 + 16 g + nl that lie
// in [0, nmax) x [0, M).
template <int T, class Out>
__device__ __forceinline__ void store_half_t(const f4 (&acc)[4][8], int64_t n0, int64_t m0, int64_t nmax, int64_t M,
                                             int rg, int lane, Out&& out) {
    const int nl = lane & 15, G = lane >> 4;
#pragma unroll
    for (int gl = 0; gl < 4; ++gl) {
        const int64_t m = m0 + 16 * (4 * T + gl) + nl;
        if (m >= M) continue;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int64_t n = n0 + 64 * rg + 16 * f + 4 * G;
            if (n < nmax) out(m, n, acc[f][4 * T + gl]);
        }
    }
}

template <class Out>
__device__ __forceinline__ void store_half(const f4 (&acc)[4][8], int64_t n0, int64_t m0, int64_t nmax, int64_t M,
                                           int rg, int t, int lane, Out&& out) {
    if (t == 0) store_half_t<0>(acc, n0, m0, nmax, M, rg, lane, out);
    else        store_half_t<1>(acc, n0, m0, nmax, M, rg, lane, out);
}

__device__ __forceinline__ h4 to_h4(f4 v) { return h4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]}; }

// K-split T partials, tile-major: fragment (f, g = 4 T + gl) of this wave at
// out[(4 f + gl) * 64] (out already points at the wave's block and lane);
// fragments of rows at or past jmax and lanes of tokens past M are not stored.
template <int T>
__device__ __forceinline__ void store_part_t(const f4 (&acc)[4][8], int64_t jw, int64_t m0, int64_t jmax, int64_t M,
                                             int lane, f4* out) {
    const int nl = lane & 15;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int gl = 0; gl < 4; ++gl)
            if (jw + 16 * f < jmax && m0 + 16 * (4 * T + gl) + nl < M) out[(4 * f + gl) * 64] = acc[f][4 * T + gl];
}

// ------------------------------------------------------------ main kernel
__global__ __launch_bounds__(kThreads) void kx_main_kernel(LinearArgs a, KxPlan plan) {
    const int b = blockIdx.y;
    const int64_t K = a.K, N = a.N, M = a.M, r = a.r;
    const int nNB = (int)((N + kTN - 1) / kTN), nMB = (int)((M + kTM - 1) / kTM);
    // XCD-aware tile order: each XCD runs a contiguous range of logical tiles,
    // grouped kGroupM m-blocks at a time so that X and W tiles are shared in
    // L2.  The tile is uniform; readfirstlane keeps it in scalar registers.
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int gsize = kGroupM * nNB, gid = L / gsize, fm = gid * kGroupM;
    const int gm = nMB - fm < kGroupM ? nMB - fm : kGroupM;
    const int mb = rfl(fm + (L % gsize) % gm);
    const int nb = rfl((L % gsize) / gm);
    const int64_t n0 = (int64_t)nb * kTN, m0 = (int64_t)mb * kTM;
    // The K / 128 sparse chunks, then the r / 64 dense ones.
    const int nK = (int)(K / kCK), nR = (int)((r + kDC - 1) / kDC);
    const int lane = threadIdx.x & 63, wave = rfl(threadIdx.x >> 6);
    const int rg = wave & 3, t = wave >> 2;

    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
    f4 acc[4][8];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 8; ++g) acc[f][g] = f4{0, 0, 0, 0};

    if (t == 0) sparse_phase<0>(a, b, n0, m0, 0, nK, lds, acc, wave, rg, lane);
    else        sparse_phase<1>(a, b, n0, m0, 0, nK, lds, acc, wave, rg, lane);
    if (nR > 0) {
        // + T . R: A = rows of Rt [N][r], B = rows of T [M][r].
        const uint16_t* T = reinterpret_cast<const uint16_t*>(a.ws + b * a.ws_per_problem + plan.t_off);
        const u4 rb = rsrc_words(T + m0 * r, (M - m0) * r * 2);
        const u4 ra = rsrc_words(a.Rt + b * a.sRt + n0 * r, (N - n0) * r * 2);
        dense_phase(ra, rb, r, r, 0, nR, lds, acc, wave, rg, t, lane);
    }
    combine_halves(lds, acc, rg, t, lane);

    _Float16* Y = reinterpret_cast<_Float16*>(a.Y + b * a.sY);
    store_half(acc, n0, m0, N, M, rg, t, lane,
               [&](int64_t m, int64_t n, f4 v) { *reinterpret_cast<h4*>(Y + m * N + n) = to_h4(v); });
}

// ------------------------------------------------------------ T = X . L
// Tile: adapter columns j0 .. +256 (rows of Lt) x tokens m0 .. +128, over
// this workgroup's part of K; after the halves are added, lane holds columns
// j = j0 + 64 rg + 16 f + 4 G + v of token m0 + 16 g + nl, g = 4t .. 4t + 3.
__global__ __launch_bounds__(kThreads) void kx_t_kernel(LinearArgs a, KxPlan plan) {
    const int b = blockIdx.y;
    const int64_t K = a.K, M = a.M, r = a.r;
    const int nJB = (int)((r + kTN - 1) / kTN), nMB = (int)((M + kTM - 1) / kTM);
    const int ntiles = nJB * nMB;
    const int LL = xcd_remap(blockIdx.x, gridDim.x);
    const int split = LL / ntiles, L = LL % ntiles;
    const int mb = rfl(L / nJB), jb = rfl(L % nJB);       // neighbours share the X tile
    const int64_t j0 = (int64_t)jb * kTN, m0 = (int64_t)mb * kTM;
    const int nD = (int)(K / kDC), S = plan.tsplit;
    const int d0 = rfl((int)((int64_t)split * nD / S)), d1 = rfl((int)((int64_t)(split + 1) * nD / S));
    const int lane = threadIdx.x & 63, wave = rfl(threadIdx.x >> 6);
    const int rg = wave & 3, t = wave >> 2;

    __shared__ __attribute__((aligned(16))) unsigned char lds[kMax2(3 * kDStage, kXchBytes)];
    f4 acc[4][8];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 8; ++g) acc[f][g] = f4{0, 0, 0, 0};
    const u4 ra = rsrc_words(a.Lt + b * a.sLt + j0 * K, (r - j0) * K * 2);
    const u4 rb = rsrc_words(a.X + b * a.sX + m0 * K, (M - m0) * K * 2);
    if (d1 > d0) dense_phase(ra, rb, K, K, d0, d1 - d0, lds, acc, wave, rg, t, lane);
    combine_halves(lds, acc, rg, t, lane);

    unsigned char* base = a.ws + b * a.ws_per_problem;
    if (S > 1) {
        f4* Tp = reinterpret_cast<f4*>(base + plan.tp_off) + (((size_t)split * ntiles + L) * 8 + wave) * 16 * 64 + lane;
        if (t == 0) store_part_t<0>(acc, j0 + 64 * rg, m0, r, M, lane, Tp);
        else        store_part_t<1>(acc, j0 + 64 * rg, m0, r, M, lane, Tp);
    } else {
        _Float16* T = reinterpret_cast<_Float16*>(base + plan.t_off);
        store_half(acc, j0, m0, r, M, rg, t, lane,
                   [&](int64_t m, int64_t j, f4 v) { *reinterpret_cast<h4*>(T + m * r + j) = to_h4(v); });
    }
}

// T = sum of the S = tsplit partials, to fp16.  Thread q takes the f4 at
// position q of every partial (tile-major, as kx_t_kernel stores them): all S
// loads in flight at once, 1 KB per wave and partial; it holds the four
// columns j .. j + 3 of one token.
template <int S>
__global__ __launch_bounds__(256) void kx_t_reduce_kernel(LinearArgs a, KxPlan plan) {
    const int b = blockIdx.y;
    const int64_t M = a.M, r = a.r;
    const int nJB = (int)((r + kTN - 1) / kTN);
    const int64_t per = (int64_t)nJB * ((M + kTM - 1) / kTM) * 8 * 16 * 64;   // f4 per partial
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= per) return;
    const int lane = (int)(q & 63), fg = (int)((q >> 6) & 15), wave = (int)((q >> 10) & 7);
    const int64_t L = q >> 13;
    const int f = fg >> 2, gl = fg & 3, rg = wave & 3, t = wave >> 2;
    const int64_t m = (L / nJB) * kTM + 16 * (4 * t + gl) + (lane & 15);
    const int64_t j = (L % nJB) * kTN + 64 * rg + 16 * f + 4 * (lane >> 4);
    if (m >= M || j >= r) return;
    const f4* Tp = reinterpret_cast<const f4*>(a.ws + b * a.ws_per_problem + plan.tp_off);
    f4 v[S];
#pragma unroll
    for (int s = 0; s < S; ++s) v[s] = Tp[(size_t)s * per + q];
    f4 sum = v[0];
#pragma unroll
    for (int s = 1; s < S; ++s) sum += v[s];
    const h4 out = {(_Float16)sum[0], (_Float16)sum[1], (_Float16)sum[2], (_Float16)sum[3]};
    *reinterpret_cast<h4*>(reinterpret_cast<_Float16*>(a.ws + b * a.ws_per_problem + plan.t_off) + m * r + j) = out;
}

}  // namespace

size_t prefill_kx_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
    (void)N;
    return kx_plan(M, K, r).total;
}

bool prefill_kx_fits(const LinearArgs& a) {
    // More tiles than the K-split form would split (129 and up: it splits
    // only when two splits' workgroups fit one round of the 256 CUs; fewer
    // tiles go to the K-split prefill kernels), and every offset a workgroup
    // adds to a buffer descriptor below 2 GiB: 128 rows of X or 256 rows of
    // Lt (K halves each), 16 row blocks of W.  Measured (graph-timed, one
    // box): gate/up at 512 tokens (172 tiles) 65.1 us here against 74.6 us
    // unsplit in the K-split form, q_proj at 1280 tokens (160 tiles) 66.1
    // against 68.2; with 128 or 96 tiles the K-split form is faster (q_proj
    // at 1024 tokens 58.2 against 62.2, down at 768 tokens 84.8 against 101.3).
    const int64_t lim = 0x7FFFFFF0;
    const int64_t tiles = ((a.N + kTN - 1) / kTN) * ((a.M + kTM - 1) / kTM);
    return a.M > 16 && tiles > 128 && (int64_t)kTN * a.K * 2 < lim && (int64_t)kTN * a.r * 2 < lim &&
           a.M < (1LL << 31) / kTM && a.N < (1LL << 31) / kTN;
}

namespace {
template <int S>
hipError_t launch_t_reduce_s(const LinearArgs& a, const KxPlan& p, hipStream_t stream) {
    const int64_t ttiles = ((a.r + kTN - 1) / kTN) * ((a.M + kTM - 1) / kTM);
    const unsigned gt = (unsigned)(ttiles * 8 * 16 * 64 / 256);
    hipLaunchKernelGGL(kx_t_reduce_kernel<S>, dim3(gt, (unsigned)a.batch), dim3(256), 0, stream, a, p);
    return hipGetLastError();
}

hipError_t launch_t_reduce(const LinearArgs& a, const KxPlan& p, hipStream_t stream) {
    static_assert(kMaxTSplit == 16, "one case per split count");
    switch (p.tsplit) {
        case 2: return launch_t_reduce_s<2>(a, p, stream);
        case 3: return launch_t_reduce_s<3>(a, p, stream);
        case 4: return launch_t_reduce_s<4>(a, p, stream);
        case 5: return launch_t_reduce_s<5>(a, p, stream);
        case 6: return launch_t_reduce_s<6>(a, p, stream);
        case 7: return launch_t_reduce_s<7>(a, p, stream);
        case 8: return launch_t_reduce_s<8>(a, p, stream);
        case 9: return launch_t_reduce_s<9>(a, p, stream);
        case 10: return launch_t_reduce_s<10>(a, p, stream);
        case 11: return launch_t_reduce_s<11>(a, p, stream);
        case 12: return launch_t_reduce_s<12>(a, p, stream);
        case 13: return launch_t_reduce_s<13>(a, p, stream);
        case 14: return launch_t_reduce_s<14>(a, p, stream);
        case 15: return launch_t_reduce_s<15>(a, p, stream);
        case 16: return launch_t_reduce_s<16>(a, p, stream);
        default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_linear_prefill_kx(const LinearArgs& a, hipStream_t stream) {
    const KxPlan p = kx_plan(a.M, a.K, a.r);
    const unsigned nMB = (unsigned)((a.M + kTM - 1) / kTM);
    hipError_t e;
    if (a.r > 0) {
        const unsigned tt = (unsigned)((a.r + kTN - 1) / kTN) * nMB;
        hipLaunchKernelGGL(kx_t_kernel, dim3(tt * (unsigned)p.tsplit, (unsigned)a.batch), dim3(kThreads), 0, stream,
                           a, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (p.tsplit > 1 && (e = launch_t_reduce(a, p, stream)) != hipSuccess) return e;
    }
    const unsigned tiles = (unsigned)((a.N + kTN - 1) / kTN) * nMB;
    hipLaunchKernelGGL(kx_main_kernel, dim3(tiles, (unsigned)a.batch), dim3(kThreads), 0, stream, a, p);
    return hipGetLastError();
}

}  // namespace slim
