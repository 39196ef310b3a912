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
//   go from HBM straight into LDS (buffer loads with the LDS destination),
//   three stages deep.  Each wave dequantises its W fragments in registers
//   and issues v_smfmac_f32_16x16x64_f16 with 4 row fragments x 4 token
//   fragments.
//   Workgroups of the first r/32 column blocks also compute a 128 x 32 block
//   of T = X . L from the same LDS tile with dense v_mfma_f32_16x16x32_f16
//   (Lt rows are the A operand).  Stores Y_main (fp16) and T (fp16); with K
//   split over workgroups (few tiles), fp32 partials that
//   prefill_t_reduce_kernel and prefill_split_finish_kernel sum.
// prefill_adapter_up_kernel: Y += T . R with dense MFMA, one 8-wave
//   workgroup per 256 rows x 128 tokens; T and Rt stream straight into LDS in
//   three 64-column stages; Y is read during the pipeline and written back
//   through an fp32 LDS tile with 16-byte stores.
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

// Packed-W LDS rows (bytes): values rows 40 B (8-byte reads of 16 rows hit
// distinct bank pairs), metadata rows 24 B (4-byte reads of 16 rows x 2
// columns: distinct banks).
constexpr int kVPitch = 40, kMPitch = 24;

constexpr int kMaxSplits = 8;                  // K splits of one tile (small M)

// Workspace of one problem: T in fp16 [M][r] at t_off; with K split over
// `splits` workgroups per tile (small M: too few tiles to fill the GPU), also
// fp32 partials of T [splits][M][r] at tp_off and of Y at yp_off, tile-major:
// [splits][tile mb * nNB + nb][wave 2 rg + mh][f][g][64 lanes] f4, i.e. each
// wave's 64 x 64 block of one split is 16 KB of contiguous memory (every
// store and load instruction moves 1 KB of whole cache lines).
struct PrefillPlan {
    int splits;
    size_t t_off, tp_off, yp_off, total;
};

PrefillPlan prefill_plan(int64_t M, int64_t N, int64_t K, int64_t r) {
    PrefillPlan p;
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const int64_t tiles = ((N + kPN - 1) / kPN) * ((M + kPM - 1) / kPM);
    const int64_t nch = K / kPK;
    int64_t S = 1;
    // At most the split that keeps S tiles' workgroups within one round of
    // the 256 CUs: partials cost more than the idle CUs of a short round
    // (gate/up at 256 tokens, 86 tiles: S = 2 runs 64.6 us, S = 3 74.1 us).
    // Within that, about six chunks per split, at least two splits: each
    // split adds a partial of Y and a workgroup whose first loads are all
    // latency (q_proj N = 4096 at 256 tokens, graph-timed on one box: K =
    // 1024 best at S = 2 or 3, K = 2048 at S = 3, K = 4096 at S = 5, K =
    // 11008 at S = 8; S = 8 throughout took 32.9, 33.4, 34.6 and 41.0 us,
    // these 25.3, 29.1, 32.4 and 41.0 us).
    if (tiles > 0 && tiles < 192) S = 256 / tiles;
    if (S > kMaxSplits) S = kMaxSplits;
    const int64_t want = (nch + 3) / 6 > 2 ? (nch + 3) / 6 : 2;
    if (S > want) S = want;
    if (S > nch) S = nch;
    if (S < 1) S = 1;
    p.splits = (int)S;
    p.t_off = kCounterRegion;
    p.tp_off = p.t_off + al((size_t)M * (size_t)r * 2);
    p.yp_off = p.tp_off + (S > 1 ? al((size_t)S * M * r * 4) : 0);
    p.total = p.yp_off + (S > 1 ? al((size_t)S * tiles * kPN * kPM * 4) : 0);
    return p;
}

// ------------------------------------------------------------ main kernel
// 8 waves, two per SIMD, so that one wave's matrix instructions run while the
// other waits.  Wave w: W rows 64 (w & 3) .. +64 (4 fragments), tokens
// 64 (w >> 2) .. +64 (4 fragments); each W fragment is dequantised by the two
// waves of its token halves.
//
// Every operand goes global -> LDS directly (buffer loads with the LDS
// destination: no registers, no LDS store instructions), three stages deep:
// iteration ch computes chunk ch while the loads of chunk ch + 2 are in
// flight.  Such a load writes the 16 bytes of lane l at base + 16 l (1 KB per
// wave instruction).  X and Lt: a row of 128 k is 256 contiguous bytes and
// the 16-byte unit u of row r sits in slot u ^ (r & 15), which keeps the
// operand reads (16 rows, one 16-byte unit each) on distinct banks.  Packed
// W: the format keeps a 16-row block's data of one 128-k group contiguous
// (512 B values, 256 B metadata, 32 B scales), so each wave instruction
// carries two value blocks or four metadata blocks or all 16 scale blocks.
// Rows past M or N (and the Lt tile of a workgroup without a T block) read
// zero.
constexpr int kMThreads = 512;
constexpr int kXLRow = kPK * 2;                                // bytes per X or Lt row of one chunk
constexpr int kSXOff = 0;                                      // X rows [128][256 B], swizzled
constexpr int kSLOff = kSXOff + kPM * kXLRow;                  // Lt rows [32][256 B], swizzled
constexpr int kSVOff = kSLOff + kLRows * kXLRow;               // values [16 blocks][16 rows x 32 B]
constexpr int kSMOff = kSVOff + kPN * 32;                      // metadata [16 blocks][16 rows x 16 B]
constexpr int kSSOff = kSMOff + kPN * 16;                      // scales [16 blocks][16 rows x 2 B], 1 KB
constexpr int kStage = kSSOff + 1024;
constexpr int kStages = 3;
static_assert(kStages * kStage <= 160 * 1024, "stages must fit in LDS");
static_assert(kPM * kXLRow / 1024 == 4 * (kMThreads / 64) && kLRows * kXLRow / 1024 == kMThreads / 64 &&
                  kPN * 32 / 1024 == kMThreads / 64 && kPN * 16 / 1024 == 4,
              "per wave and chunk: four X, one Lt, one values and one metadata-or-scale load of 1 KB");
constexpr int kOpsPerChunk = 7;          // vector-memory ops per wave and chunk

// HYB: hybrid dense / 2:4 tiles (a.dvalues, a.dflags int32 [N/16][K/128]):
// the second pair of codes of each wave's four row blocks (8 bytes per lane)
// is loaded into registers one chunk ahead, from zero-range offsets for 2:4
// tiles (no memory access), and a dense tile's fragments get a second smfmac
// per step with the implied positions 2, 3 (a scalar branch on the tile
// flag, read with scalar loads).
template <bool HYB>
__global__ __launch_bounds__(kMThreads) void prefill_main_kernel(LinearArgs a, PrefillPlan plan) {
    const int b = blockIdx.y;
    const int64_t K = a.K, N = a.N, M = a.M;
    const int nNB = (int)((N + kPN - 1) / kPN), nMB = (int)((M + kPM - 1) / kPM);
    // XCD-aware tile order: each XCD runs a contiguous range of logical tiles
    // (split-major), grouped kGroupM m-blocks at a time so that X and W tiles
    // are shared in L2.
    const int LL = xcd_remap(blockIdx.x, gridDim.x);
    const int ntiles = nNB * nMB;
    const int split = LL / ntiles, L = LL % ntiles;
    const int gsize = kGroupM * nNB, gid = L / gsize, fm = gid * kGroupM;
    const int gm = nMB - fm < kGroupM ? nMB - fm : kGroupM;
    // Tile and K range are uniform; readfirstlane keeps them in scalar
    // registers (the buffer descriptors and offsets built from them must be).
    const int mb = __builtin_amdgcn_readfirstlane(fm + (L % gsize) % gm);
    const int nb = __builtin_amdgcn_readfirstlane((L % gsize) / gm);
    const int64_t n0 = (int64_t)nb * kPN, m0 = (int64_t)mb * kPM;
    // This workgroup's K range: chunks [c0, c0 + nchunks) of the K / 128.
    const int ktot = (int)(K / kPK), S = plan.splits;
    const int c0 = __builtin_amdgcn_readfirstlane((int)((int64_t)split * ktot / S));
    const int nchunks = __builtin_amdgcn_readfirstlane((int)((int64_t)(split + 1) * ktot / S) - c0);
    // wave is uniform by construction; readfirstlane makes the compiler see it, so
    // branches on it are scalar (an MFMA under a lane mask would still execute).
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = wave & 3, mh = wave >> 2;
    const int nl = lane & 15, G = lane >> 4;
    const int nR = (int)(a.r / kLRows);
    const bool do_t = nb < nR;

    // Three stage arrays (not one array indexed at run time): every stage
    // index below is a compile-time constant, so the compiler sees which
    // stage an LDS read touches and waits only for the direct loads into it.
    __shared__ __attribute__((aligned(16))) unsigned char stage0[kStage], stage1[kStage], stage2[kStage];

    const u4 rx = rsrc_words(a.X + b * a.sX + m0 * K, (M - m0) * K * 2);
    const u4 rl = rsrc_words(do_t ? a.Lt + b * a.sLt + (int64_t)kLRows * nb * K : a.X, do_t ? (int64_t)kLRows * K * 2 : 0);
    // Packed W: this tile's 16 row blocks start at block n0 / 16 (N is a
    // multiple of 16, so every block is full); blocks past N read zero.
    const u4 rv = rsrc_words(a.values + b * a.sV + n0 * (K / 4), (N - n0) * (K / 4));
    const u4 rm = rsrc_words(a.meta + b * a.sMeta + n0 * (K / 8), (N - n0) * (K / 8));
    const u4 rs = rsrc_words(a.scales + b * a.sS + n0 * (K / kGroup), (N - n0) * (K / kGroup) * 2);

    // Direct-to-LDS loads, per wave and chunk: X load j (0..3) fills X rows
    // 4 (4w + j) .. +4 and the Lt load Lt rows 4w .. +4 (lane l: row base +
    // l / 16, slot l % 16, i.e. global unit (l % 16) ^ row); the values load
    // fills blocks 2w, 2w + 1 (lane l: block 2w + l / 32, slot l % 32 holding
    // row s / 2 and half (s % 2) ^ ((row / 4) % 2), s = l % 32); the last
    // load is metadata blocks 4w .. +4 (waves 0-3; lane l: block 4w + l / 16,
    // row l % 16) or the 16 scale blocks (waves 4-7 all load them, the same
    // bytes to the same place: lanes 0-31, the others read zero into the
    // second half of the 1 KB scale area), so that every wave issues
    // kOpsPerChunk loads per chunk.
    const int drow = lane >> 4, dslot = lane & 15;
    int dxo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * (4 * wave + j) + drow;
        dxo[j] = (int)(r * K * 2 + 16 * (dslot ^ (r & 15)));
    }
    const int dlr = 4 * wave + drow;
    const int dlo = (int)(dlr * K * 2 + 16 * (dslot ^ (dlr & 15)));
    const int vs = lane & 31, vrow = vs >> 1, vhalf = (vs & 1) ^ ((vrow >> 2) & 1);
    const int dvo = (int)((2 * wave + (lane >> 5)) * 16 * (K / 4) + 32 * vrow + 16 * vhalf);
    const bool aux_meta = wave < 4;
    const int dao = aux_meta  ? (int)((4 * wave + (lane >> 4)) * 16 * (K / 8) + 16 * (lane & 15))
                  : lane < 32 ? (int)((lane >> 1) * 16 * (K / kGroup) * 2 + 16 * (lane & 1))
                              : kOOB;
    // (The lambdas below are forced inline: every load index and stage must be
    // a compile-time constant where it is used.)
    auto dma = [&](unsigned char* st, int ch, int i) __attribute__((always_inline)) {   // load i of chunk ch into st
        ch = c0 + (ch < nchunks ? ch : nchunks - 1);       // past the end: a repeat of the last chunk
        if (i < 4)         lds_load16(rx, st + kSXOff + (4 * wave + i) * 1024, dxo[i], ch * kXLRow);
        else if (i == 4)   lds_load16(rl, st + kSLOff + wave * 1024, dlo, ch * kXLRow);
        else if (i == 5)   lds_load16(rv, st + kSVOff + wave * 1024, dvo, ch * 512);
        else if (aux_meta) lds_load16(rm, st + kSMOff + wave * 1024, dao, ch * 256);
        else               lds_load16(rs, st + kSSOff, dao, ch * 32);
    };

    f4 acc[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[f][g] = f4{0, 0, 0, 0};
    f4 acct[4];                                    // T^T partial: 16 columns x this wave's 4 token fragments
#pragma unroll
    for (int g = 0; g < 4; ++g) acct[g] = f4{0, 0, 0, 0};

    const int gA1 = G >> 1, gA2 = 2 + (G >> 1), hl = G & 1;
    // T block: the X operand is the smfmac B fragment already in registers
    // (its 16 values per lane are two 8-k slices), so the Lt operand is read
    // with the same k permutation.  Wave w owns adapter columns 16 (rg & 1) ..
    // +16 for its token half and the steps of k-half tw = rg >> 1: two MFMA per
    // such step, partial over half of k (the halves meet at the end).
    const int jf = rg & 1, tw = rg >> 1;
    // Slot of 16-byte unit u in a row whose index is congruent to nl mod 16.
    auto slot = [&](int u) { return 16 * (u ^ nl); };
    // compute(ch, mover): chunk ch from its stages; mover(q) runs after the
    // matrix instructions of step q.
    // Hybrid tiles: flags and second-pair words of the wave's blocks 4 rg + f.
    const int nG = (int)(K / kGroup);
    const int64_t fbase = (n0 / 16 + 4 * rg) * nG;
    u2 dvc[4] = {}, dvn[4] = {};
    uint32_t dmask = 0, dmask_next = 0;                 // bit f: block 4 rg + f dense (uniform)
    const __amdgpu_buffer_rsrc_t rdv =
        make_rsrc(HYB ? a.dvalues + b * a.sV + n0 * (K / 4) : a.values, HYB ? (N - n0) * (K / 4) : 0);
    auto tile_flags = [&](int ch) __attribute__((always_inline)) {   // scalar loads
        ch = c0 + (ch < nchunks ? ch : nchunks - 1);
        const __attribute__((address_space(4))) uint32_t* fl =
            (const __attribute__((address_space(4))) uint32_t*)(a.dflags);
        uint32_t m = 0;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int64_t blk = n0 / 16 + 4 * rg + f;
            const uint32_t v = blk < (N + 15) / 16 ? fl[__builtin_amdgcn_readfirstlane((int)(fbase + f * nG + ch))] : 0u;
            m |= (v != 0u ? 1u : 0u) << f;
        }
        return __builtin_amdgcn_readfirstlane(m);
    };
    auto load_dv = [&](int ch, uint32_t m) __attribute__((always_inline)) {  // 4 loads, always issued
        ch = c0 + (ch < nchunks ? ch : nchunks - 1);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int off = (int)((4 * rg + f) * 16 * (K / 4) + 32 * (16 * ch + nl) + 8 * G);
            dvn[f] = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rdv, ((m >> f) & 1u) ? off : kOOB, 0, 0));
        }
    };
    auto compute = [&](const unsigned char* xl, auto&& mover) __attribute__((always_inline)) {
        // This lane's W rows 64 rg + 16f + nl (row block 4 rg + f, row nl),
        // 16-k blocks 2G (t = 0) and 2G+1 (t = 1) of the chunk.
        h8 A[4][2];
        h8 A2[HYB ? 4 : 1][2];
        uint32_t mw[4];
        h8 TL[2];
        if (do_t) {
            const unsigned char* lt = xl + kSLOff + (16 * jf + nl) * kXLRow;
            TL[0] = *reinterpret_cast<const h8*>(lt + slot(2 * (2 * gA1 + tw) + hl));
            TL[1] = *reinterpret_cast<const h8*>(lt + slot(2 * (2 * gA2 + tw) + hl));
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int blk = 4 * rg + f;
            const u2 vw = *reinterpret_cast<const u2*>(xl + kSVOff + 512 * blk +
                                                        16 * (2 * nl + ((G >> 1) ^ ((nl >> 2) & 1))) + 8 * (G & 1));
            mw[f] = *reinterpret_cast<const uint32_t*>(xl + kSMOff + 256 * blk + 16 * nl + 4 * G);
            const _Float16 sv = *reinterpret_cast<const _Float16*>(xl + kSSOff + 32 * blk + 2 * nl);
            const h2 s2 = {sv, sv};
            dequant_word_fast(vw[0], s2, A[f][0]);
            dequant_word_fast(vw[1], s2, A[f][1]);
            if constexpr (HYB) {
                if ((dmask >> f) & 1u) {
                    dequant_word_fast(dvc[f][0], s2, A2[f][0]);
                    dequant_word_fast(dvc[f][1], s2, A2[f][1]);
                }
            }
        }
        // 8 steps q = 4t + g (t: k-half, g: token fragment of this wave's
        // half); the B operand of step q + 2 is read from LDS while step q's
        // four smfmac run.
        auto readB = [&](int q) {
            const int t = q >> 2, g = q & 3;
            const unsigned char* xrow = xl + kSXOff + (64 * mh + 16 * g + nl) * kXLRow;
            return concat8(*reinterpret_cast<const h8*>(xrow + slot(2 * (2 * gA1 + t) + hl)),
                           *reinterpret_cast<const h8*>(xrow + slot(2 * (2 * gA2 + t) + hl)));
        };
        h16 Bq[3];
        Bq[0] = readB(0);
        Bq[1] = readB(1);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (q + 2 < 8) Bq[(q + 2) % 3] = readB(q + 2);
            const h16 B = Bq[q % 3];
            const int g = q & 3;
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                if (q < 4) acc[f][g] = smfmac<0>(A[f][0], B, acc[f][g], mw[f]);
                else       acc[f][g] = smfmac<1>(A[f][1], B, acc[f][g], mw[f]);
                if constexpr (HYB) {
                    if ((dmask >> f) & 1u) {                   // uniform: a scalar branch
                        if (q < 4) acc[f][g] = smfmac<0>(A2[f][0], B, acc[f][g], 0xEEEEEEEEu);
                        else       acc[f][g] = smfmac<1>(A2[f][1], B, acc[f][g], 0xEEEEEEEEu);
                    }
                }
            }
            if (do_t && (q >> 2) == tw) {                  // uniform: a scalar branch
                acct[g] = mfma16(TL[0], __builtin_shufflevector(B, B, 0, 1, 2, 3, 4, 5, 6, 7), acct[g]);
                acct[g] = mfma16(TL[1], __builtin_shufflevector(B, B, 8, 9, 10, 11, 12, 13, 14, 15), acct[g]);
            }
            mover(q);
        }
    };

    // Prologue: chunks 0 and 1 in flight (stages 0, 1); hybrid tiles: the
    // second pairs of chunk 0 between them, so that the first wait covers them.
#pragma unroll
    for (int i = 0; i < kOpsPerChunk; ++i) dma(stage0, 0, i);
    if constexpr (HYB) {
        dmask_next = tile_flags(0);
        load_dv(0, dmask_next);
    }
#pragma unroll
    for (int i = 0; i < kOpsPerChunk; ++i) dma(stage1, 1, i);
    // Iteration ch (stage ch % 3): each wave waits for its own loads of chunk
    // ch (all but the kOpsPerChunk loads of the last iteration), then one
    // barrier, after which chunk ch is complete in LDS; compute chunk ch;
    // steps 0..6 each issue one load of chunk ch + 2 into stage (ch + 2) % 3,
    // last read in iteration ch - 1.
    // Hybrid tiles: after the barrier the second pairs of chunk ch + 1 go out
    // (older than chunk ch + 2's loads, so the next wait covers them).
    auto step = [&](const unsigned char* cur, unsigned char* next2, int ch) __attribute__((always_inline)) {
        wait_vmem_below<kOpsPerChunk>();
        __syncthreads();
        if constexpr (HYB) {
#pragma unroll
            for (int f = 0; f < 4; ++f) dvc[f] = dvn[f];
            dmask = dmask_next;
            dmask_next = tile_flags(ch + 1);
            load_dv(ch + 1, dmask_next);
        }
        compute(cur, [&](int q) __attribute__((always_inline)) {
            if (q < kOpsPerChunk) dma(next2, ch + 2, q);
        });
    };
    int ch = 0;
    for (; ch + 3 <= nchunks; ch += 3) {
        step(stage0, stage2, ch);
        step(stage1, stage0, ch + 1);
        step(stage2, stage1, ch + 2);
    }
    if (ch < nchunks) step(stage0, stage2, ch);
    if (ch + 1 < nchunks) step(stage1, stage0, ch + 1);
    // Every direct load has landed before the stages are reused below.
    wait_vmem_below<0>();
    __syncthreads();

    // T block: waves with rg = 2, 3 hold the second k-half of the columns of
    // rg = 0, 1 (same token half); they add it through LDS (the stage buffers
    // are free after the barrier above).  Waves rg < 2 then own T.
    if (do_t) {
        f4* tsum = reinterpret_cast<f4*>(stage0);     // [2 token halves][2 column blocks][4 fragments][64 lanes]
        if (rg >= 2) {
#pragma unroll
            for (int g = 0; g < 4; ++g) tsum[((mh * 2 + jf) * 4 + g) * 64 + lane] = acct[g];
        }
        __syncthreads();
        if (rg < 2) {
#pragma unroll
            for (int g = 0; g < 4; ++g) acct[g] += tsum[((mh * 2 + jf) * 4 + g) * 64 + lane];
        }
    }
    if (S > 1) {
        // K split: fp32 partials of Y (tile-major; lanes of tokens past M and
        // fragments of rows past N are not stored, and the finishing kernel
        // does not use them) and of this workgroup's T block.
        f4* Yp = reinterpret_cast<f4*>(a.ws + b * a.ws_per_problem + plan.yp_off) +
                 (((size_t)split * ntiles + (size_t)mb * nNB + nb) * 8 + 2 * rg + mh) * 16 * 64 + lane;
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                if (n0 + 64 * rg + 16 * f < N && m0 + 64 * mh + 16 * g + nl < M) Yp[(4 * f + g) * 64] = acc[f][g];
        if (do_t && rg < 2) {
            float* Tp = reinterpret_cast<float*>(a.ws + b * a.ws_per_problem + plan.tp_off) + (size_t)split * M * a.r;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t m = m0 + 64 * mh + 16 * g + nl;
                if (m < M) *reinterpret_cast<f4*>(Tp + m * a.r + (int64_t)kLRows * nb + 16 * jf + 4 * G) = acct[g];
            }
        }
        return;
    }
    // Y_main: lane holds rows n = 4G+v of fragment f, token 64 mh + 16g + nl.
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int64_t m = m0 + 64 * mh + 16 * g + nl;
        if (m >= M) continue;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int64_t n = n0 + 64 * rg + 16 * f + 4 * G;
            if (n >= N) continue;
            const h4 out = {(_Float16)acc[f][g][0], (_Float16)acc[f][g][1], (_Float16)acc[f][g][2],
                            (_Float16)acc[f][g][3]};
            *reinterpret_cast<h4*>(a.Y + b * a.sY + m * N + n) = out;
        }
    }
    if (do_t && rg < 2) {
        _Float16* T = reinterpret_cast<_Float16*>(a.ws + b * a.ws_per_problem + plan.t_off);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int64_t m = m0 + 64 * mh + 16 * g + nl;
            if (m >= M) continue;
            const int64_t j = (int64_t)kLRows * nb + 16 * jf + 4 * G;
            const h4 out = {(_Float16)acct[g][0], (_Float16)acct[g][1], (_Float16)acct[g][2], (_Float16)acct[g][3]};
            *reinterpret_cast<h4*>(T + m * a.r + j) = out;
        }
    }
}

// ------------------------------------------------------- Y += T . R
// prefill_adapter_up_kernel: a 256 (rows of Rt) x 128 (tokens) output tile
// per workgroup of 8 waves, two per SIMD (wave w: Rt rows 64 (w & 3) .. +64,
// tokens 64 (w >> 2) .. +64: 4 x 4 fragments of v_mfma_f32_16x16x32_f16).  T
// [M][r] (fp16, from the main kernel) and Rt [N][r] stream into LDS with
// direct-to-LDS loads, 64 columns of r per chunk, three stages deep; a row of
// a chunk is 128 contiguous bytes whose 16-byte unit u sits in slot
// u ^ (row & 7).  Columns past r read zero.  The Y tile (this thread's 8 x 16
// B of one token row) is fetched at the start, so its latency overlaps the
// product; the fp32 product goes through LDS once (the stages are free by
// then) so that each thread adds and stores contiguous 16-byte pieces.
constexpr int kUThreads = 512;
constexpr int kUCols = 64;                        // columns of r per chunk
constexpr int kURow = kUCols * 2;                 // bytes per T or Rt row of one chunk
constexpr int kUTOff = 0, kUROff = kPM * kURow;   // T rows [128][128 B], Rt rows [256][128 B]
constexpr int kUStage = kUROff + kPN * kURow;     // 48 KB
constexpr int kUStages = 3;
constexpr int kUOutPitch = kPN + 4;               // floats per token row of the LDS output tile
static_assert(kPM * kUOutPitch * 4 <= kUStages * kUStage, "output tile reuses the stage buffers");
static_assert(kPM * kURow / 1024 == 2 * (kUThreads / 64) && kPN * kURow / 1024 == 4 * (kUThreads / 64),
              "per wave and chunk: two T and four Rt loads of 1 KB");
constexpr int kUOpsPerChunk = 6;

__global__ __launch_bounds__(kUThreads) void prefill_adapter_up_kernel(LinearArgs a, size_t t_off) {
    const int b = blockIdx.y;
    const int64_t N = a.N, M = a.M, r = a.r;
    const int nNB = (int)((N + kPN - 1) / kPN), nMB = (int)((M + kPM - 1) / kPM);
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int gsize = kGroupM * nNB, gid = L / gsize, fm = gid * kGroupM;
    const int gm = nMB - fm < kGroupM ? nMB - fm : kGroupM;
    const int mb = __builtin_amdgcn_readfirstlane(fm + (L % gsize) % gm);
    const int nb = __builtin_amdgcn_readfirstlane((L % gsize) / gm);
    const int64_t n0 = (int64_t)nb * kPN, m0 = (int64_t)mb * kPM;
    // wave is uniform by construction; readfirstlane makes the compiler see it, so
    // branches on it are scalar (an MFMA under a lane mask would still execute).
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = wave & 3, mh = wave >> 2;
    const int nl = lane & 15, G = lane >> 4;
    const int nch = (int)((r + kUCols - 1) / kUCols);

    __shared__ __attribute__((aligned(16))) unsigned char ust[kUStages * kUStage];
    unsigned char* const ust0 = ust;
    unsigned char* const ust1 = ust + kUStage;
    unsigned char* const ust2 = ust + 2 * kUStage;

    const uint16_t* Tg = reinterpret_cast<const uint16_t*>(a.ws + b * a.ws_per_problem + t_off);
    const u4 rt = rsrc_words(Tg + m0 * r, (M - m0) * r * 2);
    const u4 rr = rsrc_words(a.Rt + b * a.sRt + n0 * r, (N - n0) * r * 2);
    // Direct loads of chunk ch, per wave: T load j (0, 1) fills T rows
    // 8 (2w + j) .. +8, Rt load j (0..3) fills Rt rows 8 (4w + j) .. +8; lane
    // l: row base + l / 8, slot l % 8, i.e. global unit (l % 8) ^ row.  A
    // unit past column r is read at an offset past the buffer: zero.
    const int drow = lane >> 3, dslot = lane & 7;
    auto dma = [&](unsigned char* st, int ch, int i) __attribute__((always_inline)) {
        ch = ch < nch ? ch : nch - 1;                    // past the end: a repeat of the last chunk
        const int row = (i < 2 ? 8 * (2 * wave + i) : 8 * (4 * wave + i - 2)) + drow;
        const int u = dslot ^ (row & 7);
        const bool ok = ch * kUCols + 8 * u < r;
        const int voff = ok ? (int)((row * r + 8 * u) * 2) : kOOB;
        if (i < 2) lds_load16(rt, st + kUTOff + (2 * wave + i) * 1024, voff, ch * kURow);
        else       lds_load16(rr, st + kUROff + (4 * wave + i - 2) * 1024, voff, ch * kURow);
    };

    f4 acc[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[f][g] = f4{0, 0, 0, 0};
    auto compute = [&](const unsigned char* st, auto&& mover) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < kUCols / 32; ++s) {
            const int slot = 16 * ((4 * s + G) ^ (nl & 7));
            h8 A[4], B[4];
#pragma unroll
            for (int f = 0; f < 4; ++f)
                A[f] = *reinterpret_cast<const h8*>(st + kUROff + (64 * rg + 16 * f + nl) * kURow + slot);
#pragma unroll
            for (int g = 0; g < 4; ++g)
                B[g] = *reinterpret_cast<const h8*>(st + kUTOff + (64 * mh + 16 * g + nl) * kURow + slot);
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int f = 0; f < 4; ++f) acc[f][g] = mfma16(A[f], B[g], acc[f][g]);
#pragma unroll
            for (int q = 0; q < 3; ++q) mover(3 * s + q);
        }
    };

#pragma unroll
    for (int i = 0; i < kUOpsPerChunk; ++i) dma(ust0, 0, i);
#pragma unroll
    for (int i = 0; i < kUOpsPerChunk; ++i) dma(ust1, 1, i);
    // The Y tile: thread t holds token row t / 4 of the tile, 64 consecutive
    // columns from 64 (t % 4), as 8 x 16 B (tokens past M or columns past N
    // read zero and are not stored), issued after chunks 0 and 1 so that the
    // first steps do not wait for it.
    const int orow = tid >> 2, ocol = 64 * (tid & 3);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.Y + b * a.sY + m0 * N, (M - m0) * N * 2);
    h8 yv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int64_t n = n0 + ocol + 8 * q;
        yv[q] = buffer_load_h8(ry, n < N ? (int)((orow * N + n) * 2) : kOOB);
    }
    // Iteration ch: this wave's loads of chunk ch are done, one barrier,
    // compute chunk ch, issue chunk ch + 2 into stage (ch + 2) % 3 (last read
    // in iteration ch - 1).  Loads younger than chunk ch's: in iterations 0
    // and 1 the 8 Y loads and the 6 of the next chunk, later the 6 of the
    // next chunk (the Y loads are then older than chunk ch's).
    auto step = [&](const unsigned char* cur, unsigned char* next2, int ch) __attribute__((always_inline)) {
        if (ch < 2) wait_vmem_below<kUOpsPerChunk + 8>();
        else        wait_vmem_below<kUOpsPerChunk>();
        __syncthreads();
        compute(cur, [&](int q) __attribute__((always_inline)) { dma(next2, ch + 2, q); });
    };
    int ch = 0;
    for (; ch + 3 <= nch; ch += 3) {
        step(ust0, ust2, ch);
        step(ust1, ust0, ch + 1);
        step(ust2, ust1, ch + 2);
    }
    if (ch < nch) step(ust0, ust2, ch);
    if (ch + 1 < nch) step(ust1, ust0, ch + 1);
    wait_vmem_below<0>();
    __syncthreads();

    // Output: the accumulators (token 64 mh + 16g + nl, rows 64 rg + 16f +
    // 4G + v) go to an fp32 LDS tile over the stage buffers, then each thread
    // adds its 64 contiguous columns of one token row to Y and stores them.
    float* ot = reinterpret_cast<float*>(ust);
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int f = 0; f < 4; ++f)
            *reinterpret_cast<f4*>(ot + (64 * mh + 16 * g + nl) * kUOutPitch + 64 * rg + 16 * f + 4 * G) = acc[f][g];
    __syncthreads();
    const int64_t m = m0 + orow;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int64_t n = n0 + ocol + 8 * q;
        const f4 lo = *reinterpret_cast<const f4*>(ot + orow * kUOutPitch + ocol + 8 * q);
        const f4 hi = *reinterpret_cast<const f4*>(ot + orow * kUOutPitch + ocol + 8 * q + 4);
        const h8 y = yv[q];
        h8 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            out[e] = (_Float16)((float)y[e] + lo[e]);
            out[4 + e] = (_Float16)((float)y[4 + e] + hi[e]);
        }
        if (m < M && n < N) *reinterpret_cast<h8*>(a.Y + b * a.sY + m * N + n) = out;
    }
}

// ------------------------------------------- K-split: T = sum of partials
// S = plan.splits (2 .. kMaxSplits): every partial's load in flight at once.
template <int S>
__global__ __launch_bounds__(256) void prefill_t_reduce_kernel(LinearArgs a, PrefillPlan plan) {
    const int b = blockIdx.y;
    const int64_t n = a.M * a.r;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float* Tp = reinterpret_cast<const float*>(a.ws + b * a.ws_per_problem + plan.tp_off);
    float v[S];
#pragma unroll
    for (int s = 0; s < S; ++s) v[s] = Tp[(size_t)s * n + i];
    float sum = v[0];
#pragma unroll
    for (int s = 1; s < S; ++s) sum += v[s];
    reinterpret_cast<_Float16*>(a.ws + b * a.ws_per_problem + plan.t_off)[i] = (_Float16)sum;
}

// ------------------------ K-split: Y = sum of partials + T . R
// One 64 (rows of W) x 64 (tokens) tile per 4-wave workgroup (small tiles:
// this path runs when M is small).  Wave w: rows n0 + 16w .. +16, tokens
// m0 + 16g + nl for g < 4; T . R with v_mfma_f32_16x16x32_f16 on operands
// read straight from L2 (rows of Rt and of T), four 32-column steps in flight.
constexpr int kFN = 64, kFM = 64, kFSteps = 4;

template <int S>
__global__ __launch_bounds__(256) void prefill_split_finish_kernel(LinearArgs a, PrefillPlan plan) {
    const int b = blockIdx.y;
    const int64_t N = a.N, M = a.M, r = a.r;
    const int nNB = (int)((N + kFN - 1) / kFN);
    const int64_t n0 = (int64_t)(blockIdx.x % nNB) * kFN, m0 = (int64_t)(blockIdx.x / nNB) * kFM;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nl = lane & 15, G = lane >> 4;
    const int64_t n = n0 + 16 * wave + 4 * G;                 // this lane's 4 output rows n .. n+3
    const bool nok = n < N;

    // The partial sums of this lane's outputs go out first (HBM), all S
    // splits at once.
    // This tile is the 64 x 64 block of main-kernel wave (rg, mh) = ((n0 / 64)
    // % 4, (m0 / 64) % 2) of tile (m0 / 128, n0 / 256); its lane (nl, G) of
    // wave w holds that wave's acc[f = w][g] (same lane).  Fragments wholly
    // past M or N were not stored: their loads re-read a stored fragment of
    // the same tile (an L2 hit); no output uses them, nor the lanes of
    // tokens past M.
    const int64_t ptile = (int64_t)((N + kPN - 1) / kPN) * ((M + kPM - 1) / kPM) * 8 * 16;
    const f4* Yp = reinterpret_cast<const f4*>(a.ws + b * a.ws_per_problem + plan.yp_off) +
                   ((((m0 / kPM) * ((N + kPN - 1) / kPN) + n0 / kPN) * 8 + 2 * ((n0 / 64) % 4) + (m0 / 64) % 2) * 16) * 64 +
                   lane;
    f4 part[S][4];
    const int wv = n0 + 16 * wave < N ? wave : 0;
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            part[s][g] = Yp[((size_t)s * ptile + 4 * wv + (m0 + 16 * g < M ? g : 0)) * 64];

    f4 acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
    if (r > 0) {
        const uint16_t* T = reinterpret_cast<const uint16_t*>(a.ws + b * a.ws_per_problem + plan.t_off);
        const int64_t ra = n0 + 16 * wave + nl;                // A: row of Rt
        const uint16_t* Ap = a.Rt + b * a.sRt + (ra < N ? ra : N - 1) * r + 8 * G;
        const uint16_t* Bp[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int64_t m = m0 + 16 * g + nl;                // B: row of T
            Bp[g] = T + (m < M ? m : M - 1) * r + 8 * G;
        }
        const int nj = (int)(r / 32);
        for (int j0 = 0; j0 < nj; j0 += kFSteps) {
            h8 A[kFSteps], B[kFSteps][4];
#pragma unroll
            for (int u = 0; u < kFSteps; ++u) {
                const int j = j0 + u < nj ? j0 + u : nj - 1;   // clamped: always in bounds
                A[u] = load_h8(Ap + 32 * j);
#pragma unroll
                for (int g = 0; g < 4; ++g) B[u][g] = load_h8(Bp[g] + 32 * j);
            }
#pragma unroll
            for (int u = 0; u < kFSteps; ++u) {
                const h8 Au = j0 + u < nj ? A[u] : h8{};
#pragma unroll
                for (int g = 0; g < 4; ++g) acc[g] = mfma16(Au, B[u][g], acc[g]);
            }
        }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int64_t m = m0 + 16 * g + nl;
        if (!nok || m >= M) continue;
        f4 y = acc[g] + part[0][g];
#pragma unroll
        for (int s = 1; s < S; ++s) y += part[s][g];
        const h4 out = {(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
        *reinterpret_cast<h4*>(a.Y + b * a.sY + m * N + n) = out;
    }
}

// The same with the T and Rt tiles staged in LDS: the workgroup's 64 rows
// of T and of Rt go straight into LDS (one instruction per row), the
// partials of Y are loaded meanwhile, and the T . R steps read their
// operands from LDS, so only one memory latency is exposed.  Same operands,
// same accumulation order as prefill_split_finish_kernel.
constexpr int kF2MaxR = 608;                      // two 64-row tiles of pitch 2r + 16 fit in LDS

template <int S>
__global__ __launch_bounds__(256) void prefill_split_finish_lds_kernel(LinearArgs a, PrefillPlan plan) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * kFM * (2 * kF2MaxR + 16)];
    const int b = blockIdx.y;
    const int64_t N = a.N, M = a.M;
    const int r = (int)a.r;
    const int nNB = (int)((N + kFN - 1) / kFN);
    const int64_t n0 = (int64_t)(blockIdx.x % nNB) * kFN, m0 = (int64_t)(blockIdx.x / nNB) * kFM;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nl = lane & 15, G = lane >> 4;
    const int64_t n = n0 + 16 * wave + 4 * G;                 // this lane's 4 output rows n .. n+3
    const bool nok = n < N;
    const int rp = 2 * r + 16;                                // LDS row pitch (bytes)
    unsigned char* tt = lds;                                  // T rows m0 .. m0 + 63
    unsigned char* rt = lds + kFM * rp;                       // Rt rows n0 .. n0 + 63

    // 1. Wave w copies rows 16w .. 16w + 15 of both tiles (rows past M or N
    //    read zero), then loads the partial sums of this lane's outputs.
    if (r > 0) {
        const uint16_t* T = reinterpret_cast<const uint16_t*>(a.ws + b * a.ws_per_problem + plan.t_off);
        const u4 rtt = rsrc_words(T + m0 * r, (M - m0) * r * 2);
        const u4 rrr = rsrc_words(a.Rt + b * a.sRt + n0 * r, (N - n0) * r * 2);
        for (int q = 16 * wave; q < 16 * wave + 16; ++q)
            for (int i = 0; 1024 * i < 2 * r; ++i)
                if (16 * lane + 1024 * i < 2 * r) {
                    lds_load16(rtt, tt + q * rp + 1024 * i, q * 2 * r + 16 * lane, 1024 * i);
                    lds_load16(rrr, rt + q * rp + 1024 * i, q * 2 * r + 16 * lane, 1024 * i);
                }
    }
    // This tile is the 64 x 64 block of main-kernel wave (rg, mh) = ((n0 / 64)
    // % 4, (m0 / 64) % 2) of tile (m0 / 128, n0 / 256); its lane (nl, G) of
    // wave w holds that wave's acc[f = w][g] (same lane).  Fragments wholly
    // past M or N were not stored: their loads re-read a stored fragment of
    // the same tile (an L2 hit); no output uses them, nor the lanes of
    // tokens past M.
    const int64_t ptile = (int64_t)((N + kPN - 1) / kPN) * ((M + kPM - 1) / kPM) * 8 * 16;
    const f4* Yp = reinterpret_cast<const f4*>(a.ws + b * a.ws_per_problem + plan.yp_off) +
                   ((((m0 / kPM) * ((N + kPN - 1) / kPN) + n0 / kPN) * 8 + 2 * ((n0 / 64) % 4) + (m0 / 64) % 2) * 16) * 64 +
                   lane;
    f4 part[S][4];
    const int wv = n0 + 16 * wave < N ? wave : 0;
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            part[s][g] = Yp[((size_t)s * ptile + 4 * wv + (m0 + 16 * g < M ? g : 0)) * 64];
    // The tile copies are older than the S * 4 partial loads.
    wait_vmem_below<S * 4>();
    __syncthreads();

    // 2. acc[g] += Rt rows 16w + nl . T rows 16g + nl, 32 columns of r per step.
    f4 acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
    for (int jb = 0; jb < r / 32; ++jb) {
        const h8 A = *reinterpret_cast<const h8*>(rt + (16 * wave + nl) * rp + 2 * (32 * jb + 8 * G));
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const h8 B = *reinterpret_cast<const h8*>(tt + (16 * g + nl) * rp + 2 * (32 * jb + 8 * G));
            acc[g] = mfma16(A, B, acc[g]);
        }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int64_t m = m0 + 16 * g + nl;
        if (!nok || m >= M) continue;
        f4 y = acc[g] + part[0][g];
#pragma unroll
        for (int s = 1; s < S; ++s) y += part[s][g];
        const h4 out = {(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
        *reinterpret_cast<h4*>(a.Y + b * a.sY + m * N + n) = out;
    }
}

}  // namespace

size_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) { return prefill_plan(M, N, K, r).total; }

bool prefill_fits(const LinearArgs& a) {
    // The T blocks are produced by the first r/32 column blocks of W; every
    // buffer that a workgroup addresses with 32-bit offsets stays below 2 GiB.
    const int64_t lim = 0x7FFFFFF0;
    return a.M > 16 && (a.r / kLRows) <= (a.N + kPN - 1) / kPN && a.M * a.K * 2 < lim &&
           (int64_t)kLRows * a.K * 2 < lim && a.N * (a.K / 4) < lim && a.M < (1LL << 31) / kPM;
}

// Y += T . R on the 256 x 128 prefill tiles: T fp16 [M][r] at t_off of each
// problem's workspace, Y fp16 read and written.
hipError_t launch_prefill_adapter_up(const LinearArgs& a, size_t t_off, hipStream_t stream) {
    const unsigned tiles = (unsigned)(((a.N + kPN - 1) / kPN) * ((a.M + kPM - 1) / kPM));
    hipLaunchKernelGGL(prefill_adapter_up_kernel, dim3(tiles, (unsigned)a.batch), dim3(kUThreads), 0, stream, a, t_off);
    return hipGetLastError();
}

namespace {
// The kernels after a K-split main kernel: T reduction (with an adapter),
// then Y = sum of the S partials + T . R.
template <int S>
hipError_t launch_split_tail(const LinearArgs& a, const PrefillPlan& p, hipStream_t stream) {
    static_assert(S >= 2 && S <= kMaxSplits, "split count");
    if (a.r > 0) {
        const unsigned gt = (unsigned)((a.M * a.r + 255) / 256);
        hipLaunchKernelGGL(prefill_t_reduce_kernel<S>, dim3(gt, (unsigned)a.batch), dim3(256), 0, stream, a, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const unsigned gf = (unsigned)(((a.N + kFN - 1) / kFN) * ((a.M + kFM - 1) / kFM));
    if (a.r <= kF2MaxR)
        hipLaunchKernelGGL(prefill_split_finish_lds_kernel<S>, dim3(gf, (unsigned)a.batch), dim3(256), 0, stream, a, p);
    else
        hipLaunchKernelGGL(prefill_split_finish_kernel<S>, dim3(gf, (unsigned)a.batch), dim3(256), 0, stream, a, p);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_linear_prefill(const LinearArgs& a, hipStream_t stream) {
    const PrefillPlan p = prefill_plan(a.M, a.N, a.K, a.r);
    const unsigned tiles = (unsigned)(((a.N + kPN - 1) / kPN) * ((a.M + kPM - 1) / kPM));
    if (a.dvalues)
        hipLaunchKernelGGL(prefill_main_kernel<true>, dim3(tiles * (unsigned)p.splits, (unsigned)a.batch),
                           dim3(kMThreads), 0, stream, a, p);
    else
        hipLaunchKernelGGL(prefill_main_kernel<false>, dim3(tiles * (unsigned)p.splits, (unsigned)a.batch),
                           dim3(kMThreads), 0, stream, a, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.splits == 1) {
        if (a.r == 0) return hipSuccess;
        hipLaunchKernelGGL(prefill_adapter_up_kernel, dim3(tiles, (unsigned)a.batch), dim3(kUThreads), 0, stream, a,
                           p.t_off);
        return hipGetLastError();
    }
    switch (p.splits) {
        case 2: return launch_split_tail<2>(a, p, stream);
        case 3: return launch_split_tail<3>(a, p, stream);
        case 4: return launch_split_tail<4>(a, p, stream);
        case 5: return launch_split_tail<5>(a, p, stream);
        case 6: return launch_split_tail<6>(a, p, stream);
        case 7: return launch_split_tail<7>(a, p, stream);
        case 8: return launch_split_tail<8>(a, p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace slim
