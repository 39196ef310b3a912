// Double-pruned transpose of the packed weight (SLoPe: Compression Trinity
// thesis, Ch. 4 list of contributions -- the forward N:M-pruned weight is
// transposed and pruned N:M again, so that the backward product dX = dY W,
// whose reduction runs over the output dimension n, also runs on 2:4 sparse
// matrix cores).  The pages give no procedure for SLiM's quantised weight;
// the operation built here:
//   D = deq(W_c) in fp16 (q * s16 rounded once, as the forward kernels form
//       it), transposed to [K][N];
//   in every 4 consecutive n of a row k the 2 largest |D| are kept, ties to
//       the lower index (the forward prune's rule);
//   per row k, per 16 consecutive n: 8 fp16 kept values (group j: the lower
//       index, then the higher) and one uint16 of 2-bit indices, bits
//       [4j, 4j+2) the lower and [4j+2, 4j+4) the higher -- the forward
//       metadata's bit order, so a 16-n block is one lane's sparse MFMA
//       A operand.  tvalues fp16 [K][N/2], tmeta uint16 [K][N/16].
//
// Work layout: a workgroup takes one 128-k group and 8 row blocks (128 n).
// Their packed words, metadata and scales (8 x 800 B, contiguous per block in
// the packed arrangement) are staged in LDS transposed to [block][k16][row],
// so that the 16 rows a lane needs for one 16-k block sit in 64 + 32
// contiguous bytes.  Lane (b, kb, j) -- b = tid % 8 -- produces the 4 output
// rows k = 16 kb + 4 j + p (p = 0..3) of the 16 n of block b: lanes 8 apart
// in b write one 128-byte line of tvalues per store.
//
// Per row i of the block: the two kept codes of its 4-group j are turned into
// fp16 together (nibble + 8 placed under the exponent of 1024, minus 1032,
// times the scale: exact operations and one rounding of q * s16).  A 16-entry
// LDS table, indexed by the group's 4 metadata bits, gives for each slot p the
// byte selector that places the lower- or higher-index value (the higher one
// winning if both indices are p, as in a plain unpack) or zero, so that one
// byte permute plus one rotate forms the sort key of slot p:
//   key = |d| << 17 | t << 15 | sign(d),   t = 3 - (i mod 4)
// Keys are distinct inside a 4-group of rows and order by magnitude, then
// lower row first; the two largest of four come from a min/max network.
// Rotating a key back gives t << 30 | d, so one max/min orders the two kept
// values by row and the metadata nibble is their two top bit pairs.
//
// A persistent grid walks the tiles; each workgroup loads the next tile's
// packed bytes into registers while it computes and stores the current one.
// About 9 vector instructions per weight, against HBM traffic of 25/64 B read
// and 9/8 B written per weight.  At 4096 x 4096 the grid holds every tile at
// once, so loads, arithmetic and stores run in step across the chip and the
// vector units are busy about half of the time.
#include "internal.hpp"
#include "mfma_util.hpp"

namespace slim {
namespace {

constexpr int kTpBlocks = 8;     // row blocks (16 n each) per tile
constexpr int kTpThreads = 256;
constexpr int kTpGrid = 256 * 4;  // persistent workgroups: 4 per CU of MI355X (1, 2: slower; 6: same)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t rotr(uint32_t x, int s) { return __builtin_amdgcn_alignbit(x, x, s); }

// The packed bytes of one tile, as this thread loads them: one 16-byte piece
// of values (every thread), of metadata (threads 0..127) or of scales
// (threads 128..143).
struct TilePieces {
    u32x4 v, x;
};

__device__ inline void load_tile(const uint8_t* __restrict__ values, const uint8_t* __restrict__ meta,
                                 const uint16_t* __restrict__ scales, int64_t K, int64_t b0, int64_t g, int nb,
                                 int tid, TilePieces& t) {
    const int bv = tid / 32;
    if (bv < nb) t.v = *reinterpret_cast<const u32x4*>(values + (b0 + bv) * 16 * (K / 4) + g * 512 + (tid % 32) * 16);
    if (tid < 16 * kTpBlocks) {
        const int b = tid / 16;
        if (b < nb) t.x = *reinterpret_cast<const u32x4*>(meta + (b0 + b) * 16 * (K / 8) + g * 256 + (tid % 16) * 16);
    } else if (tid < 16 * kTpBlocks + 2 * kTpBlocks) {
        const int q = tid - 16 * kTpBlocks, b = q / 2;
        if (b < nb) t.x = *reinterpret_cast<const u32x4*>(scales + (b0 + b) * 16 * (K / 128) + g * 16 + (q % 2) * 8);
    }
}

__global__ __launch_bounds__(kTpThreads) void pack_transposed_kernel(
    const uint8_t* __restrict__ values, const uint8_t* __restrict__ meta, const uint16_t* __restrict__ scales,
    int64_t N, int64_t K, uint16_t* __restrict__ tvalues, uint16_t* __restrict__ tmeta) {
    // [block][k16 within the group][row], each block padded by 16 bytes so
    // that the 8 lanes reading one k16 of the 8 blocks hit distinct banks.
    __shared__ __align__(16) uint32_t s_w[kTpBlocks][8 * 16 + 4];
    __shared__ __align__(16) uint16_t s_m[kTpBlocks][8 * 16 + 8];
    __shared__ __align__(16) uint16_t s_s[kTpBlocks][16];
    __shared__ __align__(16) uint32_t s_sel[16][4];              // [metadata nibble][slot]

    const int tid = threadIdx.x;
    const int64_t nblk = N / 16;
    const int nbx = (int)((nblk + kTpBlocks - 1) / kTpBlocks);
    const int ntiles = nbx * (int)(K / 128);
    // Tiles are taken in rounds of gridDim.x (a multiple of 8).  XCD-aware
    // order, n tiles fastest: in each round an XCD runs a contiguous range of
    // tiles, so the 8 tiles that share a 128-byte line of tmeta (and the 4
    // sharing a line of scales) meet in its L2 instead of leaving partial
    // lines in several.
    auto tile_of = [&](int L, int64_t& b0, int64_t& g, int& nb) {
        const int t = xcd_remap(L, ntiles);
        b0 = (int64_t)(t % nbx) * kTpBlocks;
        g = t / nbx;
        nb = (int)min<int64_t>(kTpBlocks, nblk - b0);
    };

    if (tid >= kTpThreads - 64) {
        // Slot selectors.  Permute operands: (T, P) with P = lower-index value
        // | higher-index value << 16 and T holding the tie-break bits in its
        // top byte.  Output bytes 0-1: the chosen value or zero; byte 2: zero;
        // byte 3: T's top byte.
        const int t = tid - (kTpThreads - 64), n4 = t / 4, p = t % 4;
        const int lo = n4 & 3, hi = n4 >> 2;
        s_sel[n4][p] = 0x070C0000u | (hi == p ? 0x0302u : lo == p ? 0x0100u : 0x0C0Cu);
    }

    int L = blockIdx.x;
    if (L >= ntiles) return;                         // uniform: before any barrier
    int64_t b0, g;
    int nb;
    tile_of(L, b0, g, nb);
    TilePieces cur;
    load_tile(values, meta, scales, K, b0, g, nb, tid, cur);

    const int b = tid % kTpBlocks;
    const int c = tid / kTpBlocks, kb = c / 4, j = c % 4;
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const u32x4* sel_tab = reinterpret_cast<const u32x4*>(&s_sel[0][0]);

#pragma unroll 1
    for (;;) {
        // Stage the tile: values with every nibble offset by 8 (two's
        // complement -> q + 8), all transposed to [block][k16][row].
        {
            const int bv = tid / 32, pv = tid % 32, i = pv / 2, h = pv % 2;
            if (bv < nb) {
                s_w[bv][(4 * h + 0) * 16 + i] = cur.v.x ^ 0x88888888u;
                s_w[bv][(4 * h + 1) * 16 + i] = cur.v.y ^ 0x88888888u;
                s_w[bv][(4 * h + 2) * 16 + i] = cur.v.z ^ 0x88888888u;
                s_w[bv][(4 * h + 3) * 16 + i] = cur.v.w ^ 0x88888888u;
            }
            if (tid < 16 * kTpBlocks) {
                const int bm = tid / 16, im = tid % 16;
                if (bm < nb) {
                    const uint32_t x[4] = {cur.x.x, cur.x.y, cur.x.z, cur.x.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        s_m[bm][(2 * e) * 16 + im] = (uint16_t)(x[e] & 0xFFFFu);
                        s_m[bm][(2 * e + 1) * 16 + im] = (uint16_t)(x[e] >> 16);
                    }
                }
            } else if (tid < 16 * kTpBlocks + 2 * kTpBlocks) {
                const int q = tid - 16 * kTpBlocks, bs = q / 2;
                if (bs < nb) *reinterpret_cast<u32x4*>(&s_s[bs][8 * (q % 2)]) = cur.x;
            }
        }
        __syncthreads();
        uint32_t w[16], m[8], s[8];
        if (b < nb) {
            const u32x4* wp = reinterpret_cast<const u32x4*>(&s_w[b][kb * 16]);
            const u32x4* mp = reinterpret_cast<const u32x4*>(&s_m[b][kb * 16]);
            const u32x4* sp = reinterpret_cast<const u32x4*>(&s_s[b][0]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 v = wp[q];
                w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const u32x4 v = mp[q], u = sp[q];
                m[4 * q] = v.x; m[4 * q + 1] = v.y; m[4 * q + 2] = v.z; m[4 * q + 3] = v.w;
                s[4 * q] = u.x; s[4 * q + 1] = u.y; s[4 * q + 2] = u.z; s[4 * q + 3] = u.w;
            }
        }
        __syncthreads();                             // the staging buffers are free again

        // Next tile's loads fly while this one is computed and stored.
        const int64_t cb0 = b0, cg = g;
        const int cnb = nb;
        L += gridDim.x;
        const bool more = L < ntiles;
        if (more) {
            tile_of(L, b0, g, nb);
            load_tile(values, meta, scales, K, b0, g, nb, tid, cur);
        }

        if (b < cnb) {
            const int64_t n16 = cb0 + b;             // output 16-n block
            uint32_t outw[4][4], acc[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {         // 4-group of rows along n
                uint32_t key[4][4];                  // [row in the group][slot p]
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * jj + e;
                    const uint32_t x = ((w[i] >> (4 * j)) & 0x000F000Fu) | 0x64006400u;   // 1024 + q + 8, two halves
                    const h2 q = __builtin_bit_cast(h2, x) + bias;
                    const h2 sc = __builtin_bit_cast(h2, __builtin_amdgcn_perm(s[i / 2], s[i / 2],
                                                                               (i % 2) ? 0x03020302u : 0x01000100u));
                    const uint32_t P = __builtin_bit_cast(uint32_t, q * sc);
                    const uint32_t n4 = (m[i / 2] >> (16 * (i % 2) + 4 * j)) & 15u;
                    const u32x4 sel = sel_tab[n4];
                    const uint32_t T = (uint32_t)(3 - e) << 30;
                    key[e][0] = rotr(__builtin_amdgcn_perm(T, P, sel.x), 15);
                    key[e][1] = rotr(__builtin_amdgcn_perm(T, P, sel.y), 15);
                    key[e][2] = rotr(__builtin_amdgcn_perm(T, P, sel.z), 15);
                    key[e][3] = rotr(__builtin_amdgcn_perm(T, P, sel.w), 15);
                }
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const uint32_t k0 = key[0][p], k1 = key[1][p], k2 = key[2][p], k3 = key[3][p];
                    const uint32_t hi01 = max(k0, k1), lo01 = min(k0, k1), hi23 = max(k2, k3), lo23 = min(k2, k3);
                    const uint32_t first = max(hi01, hi23);
                    const uint32_t second = max(min(hi01, hi23), max(lo01, lo23));
                    const uint32_t rf = rotr(first, 17), rs = rotr(second, 17);   // t << 30 | fp16 bits
                    const uint32_t lower = max(rf, rs), higher = min(rf, rs);      // lower row first
                    outw[p][jj] = __builtin_amdgcn_perm(higher, lower, 0x05040100u);
                    acc[p] |= __builtin_amdgcn_alignbit(higher >> 30, lower, 30) << (4 * jj);
                }
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int64_t k = cg * 128 + kb * 16 + 4 * j + p;
                const u32x4 o = {outw[p][0], outw[p][1], outw[p][2], outw[p][3]};
                *reinterpret_cast<u32x4*>(tvalues + k * (N / 2) + n16 * 8) = o;
                tmeta[k * (N / 16) + n16] = (uint16_t)(acc[p] ^ 0xFFFFu);  // t = 3 - index
            }
        }
        if (!more) break;                            // uniform
    }
}

}  // namespace

hipError_t launch_pack_transposed(const uint8_t* values, const uint8_t* meta, const uint16_t* scales, int64_t N,
                                  int64_t K, uint16_t* tvalues, uint16_t* tmeta, hipStream_t stream) {
    const int64_t tiles = (N / 16 + kTpBlocks - 1) / kTpBlocks * (K / 128);
    const unsigned grid = (unsigned)(tiles < kTpGrid ? (tiles + 7) / 8 * 8 : kTpGrid);
    hipLaunchKernelGGL(pack_transposed_kernel, grid, dim3(kTpThreads), 0, stream, values, meta, scales, N, K,
                       tvalues, tmeta);
    return hipGetLastError();
}

}  // namespace slim
