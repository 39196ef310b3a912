"""CPU oracle for the SLiM compressed linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
never calls it, and it shares no code with the GPU path: every step below is
written out from the method's description in plain NumPy, in float64 for the
floating-point products.

Sources (the pages describing the method):
  [CT]  "Compression Trinity: Exploring Sparsity, Quantization, and Low-Rank
        Approximations for LLM Compression", thesis full text
        (paperz.arrangedbits.com "Paper deep dive" page).
  [DL]  developinglight.com study summary of the same thesis.

What the layer computes:
  * Linear layer Y = X W^T, W in R^{d_out x d_in}, X in R^{b x d_in}
    ([CT] §2.1 "The Transformer Bottleneck").
  * SLiM compression pipeline ([CT] Fig. 7.1 caption): (1) symmetric
    quantisation of W, (2) sparsification of the *quantised* weights,
    (3) a low-rank adapter L, R that compensates the error.
  * Quantisation is applied per group to cope with outliers ([CT] §1.2.2
    "Quantization"); SLiM uses 4-bit weight-only quantisation with group size
    128 ([DL], setup paragraph).
  * 2:4 sparsity: in every contiguous block of 4 elements along the reduction
    dimension at least 2 are zero; the non-zeros are stored packed, next to
    small metadata indices that record their original positions
    ([CT] §2.2.3 "Sparse Tensor Core Acceleration"; §1.2.1 "Sparsity").
  * Sparse weights and the dense low-rank adapter are parallel paths, never
    merged into one dense matrix ([CT] Ch. 4 introduction, "Lazy Low-Rank
    Adapters").

Readings taken where the pages are silent (each is a plain choice that the
rest of the text supports):
  R1 int4 range is the symmetric [-7, 7]; scale s = absmax / 7.
  R2 the per-group scale is stored in fp16 (round to nearest even) and the
     quantiser divides by that stored fp16 value, so q * s16 is exactly the
     dequantised weight.
  R3 w / s16 is an IEEE float32 correctly rounded division; rounding to an
     integer is round-half-to-even; then clamp to [-7, 7].
  R4 an all-zero group has s16 = 0 and q = 0.
  R5 the pruning score is |q| inside each group of 4 (the scale is common to
     the group); the 2 largest are kept, ties go to the lower index.
  R6 no re-scaling after pruning: scales come from the unpruned group.
  R7 groups of 128 and groups of 4 both run along K = d_in inside a row.
  R8 packed layout (the pages fix only "packed values + position indices"):
     per row, per block of 16 consecutive k (4 groups of 4):
       values: one little-endian uint32; bits [4j, 4j+4) hold the kept value
               with the lower index of group j, bits [16+4j, 16+4j+4) the one
               with the higher index (4-bit two's complement);
       meta:   one little-endian uint16; bits [4j, 4j+2) hold the lower kept
               index of group j, bits [4j+2, 4j+4) the higher one.
     Row sizes: values K/4 bytes, meta K/8 bytes, scales K/128 fp16.
  R8b arrangement in memory (a storage convention; the pages fix none): rows
     in blocks of 16 (the last block holds N mod 16 rows if that is not 0);
     inside a block the 128-k groups in order, inside a group the rows in
     order; per (group, row) 32 bytes of values, 16 bytes of metadata and one
     fp16 scale.  So one row block's data for one group is contiguous
     (512 + 256 + 32 bytes for a full block), and the array sizes are those
     of the row order above.
  R9 adapter orientation follows Y = X deq(W)^T + (X L) R with
     L [K, r] and R [r, N], both row-major.

Quantised adapters ("Quantized SLiM": [CT] captions of Tables E.13 and E.14
state only that the low-rank adapters are quantised as well):
  QA1 each factor is quantised with the quantiser of W (R1-R4), without
      pruning.
  QA2 groups run along the reduction dimension of the product the factor
      feeds, on the factor stored output-major: Lt = L^T [r, K] in groups of
      128 along K (as W); Rt = R^T [N, r] in groups of 32 along r (every legal
      r is a multiple of 32, not of 128).
  QA3 codes are packed two per byte: per row, per 8 consecutive elements one
      little-endian uint32 in which element e sits in nibble NIB_POS[e] (4-bit
      two's complement); scales are fp16 [rows, cols / group], row-major.

SLoPe's double-pruned transpose ([CT] Ch. 4 list of contributions: the
forward N:M-pruned weight is transposed and pruned N:M again for the
backward pass dX = dY W, whose reduction dimension is d_out = N).  For
SLiM's compressed weight the pages give no procedure; the plain reading:
  T1 the operand is deq(W_c) formed in fp16 (q * s16 rounded once to fp16,
     as the forward kernels form it), so no second quantisation is needed;
  T2 it is transposed to [K, N] and, in every 4 consecutive n of a row k,
     the 2 largest |value| are kept, ties to the lower index (R5's rule);
  T3 per row k, per 16 consecutive n: the 8 kept fp16 values (group j: the
     lower-index one, then the higher) and one uint16 of 2-bit indices in
     R8's bit order; rows in order (tvalues fp16 [K, N/2], tmeta uint16
     [K, N/16]).

4-bit weights with 8-bit input ([CT] Appendix E.2 "Input Quantization", a
table-of-contents entry, and the captions of Tables E.2 and E.5: the same
compressed weights evaluated with the layer input quantised to 8 bits; §1.2.2
names INT8 as a target for activations too).  The pages give no input
quantiser; the plain reading:
  A1 the input is quantised per token (per row of X), symmetrically to
     int8 in [-127, 127], with W's quantiser otherwise: scale
     s = fp16(absmax / 127) (fp32 division, round to nearest even), q =
     clamp(rint(x / s), -127, 127) with an fp32 correctly rounded division and
     half-to-even rounding; a row of zeros has s = 0 and q = 0;
  A2 both products of the layer take the dequantised input q * s:
     Y = deq(X) deq(W_c)^T + (deq(X) L) R;
  A3 q is int8 [M, K] row-major, s is fp16 [M].

Hybrid dense / 2:4 tiles (PATCH, [CT] Ch. 6; Ch. 1 list of contributions:
weight matrices are split into tiles, each either dense or 2:4 sparse, for
an effective sparsity between 0% and 50%, composable with SLiM's joint
quantisation and low-rank adapter; Fig. 6.1 caption: a per-tile mask assigns
each tile to stay dense or follow the 2:4 pattern).  The pages learn the mask
and give neither the tile size nor a storage format; the plain reading:
  P1 a tile is 16 consecutive rows by one 128-k scale group (the unit of the
     packed arrangement R8b); the per-tile choice is an input (dense[b, g],
     b = row block, g = group); learning it is out of scope;
  P2 every tile is quantised as R1-R4 (same scales); dense tiles are not
     pruned, 2:4 tiles are pruned as R5;
  P3 storage: values, meta and scales in the format of R8/R8b, where a dense
     tile's values hold the codes at positions 0 and 1 of each group of 4
     (metadata: positions 0, 1), and a second array dvalues of the same size
     and arrangement holds its codes at positions 2 and 3 (zero in 2:4 tiles);
     the dense flags are uint8 [ceil(N/16), K/128];
  P4 the layer is the plain one on the hybrid weight:
     Y = X deq(W_h)^T + (X L) R.
"""
from __future__ import annotations

import numpy as np

GROUP = 128
QMAX = 7


# ---------------------------------------------------------------- a1: scales
def group_scales(W: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Per-row, per-group fp16 scale s16 = fp16(absmax / 7)   (R1, R2).

    [CT] §1.2.2 (per-group quantisation), Fig. 7.1 (symmetric quantiser),
    [DL] (group size 128).  Returns float16 [N, K/group].
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    absmax = np.max(np.abs(W.reshape(N, K // group, group)), axis=2)  # exact in fp32
    s32 = absmax / np.float32(QMAX)                                    # fp32 division
    return s32.astype(np.float16)                                      # round to nearest even


# -------------------------------------------------------------- a2: quantise
def quantize(W: np.ndarray, s16: np.ndarray, group: int = GROUP) -> np.ndarray:
    """q = clamp(rint(w / s16), -7, 7) in float32, q = 0 where s16 == 0 (R1-R4).

    [CT] Fig. 7.1 caption, step (1).  Returns int8 [N, K].
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    s = s16.astype(np.float32)[:, :, None]          # exact widening of fp16
    Wg = W.reshape(N, K // group, group)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = Wg / s                                  # float32, correctly rounded
    q = np.clip(np.rint(t), -QMAX, QMAX)            # rint: half to even
    q = np.where(s > 0, q, 0.0)
    return q.reshape(N, K).astype(np.int8)


# ----------------------------------------------------------------- a3: prune
def prune_2of4(q: np.ndarray):
    """Keep the 2 largest |q| of every 4 consecutive k; ties to the lower index.

    [CT] §2.2.3 (2:4 along the reduction dimension), Fig. 7.1 step (2): the
    quantised weights are the ones that get sparsified (R5, R6).
    Returns (q_pruned int8 [N, K], keep uint8 [N, K/4, 2] with keep[...,0] <
    keep[...,1], kept int8 [N, K/4, 2]).
    """
    N, K = q.shape
    g = q.reshape(N, K // 4, 4)
    score = -np.abs(g.astype(np.int16))
    order = np.argsort(score, axis=2, kind="stable")   # stable: equal |q| keep index order
    keep = np.sort(order[:, :, :2], axis=2)
    kept = np.take_along_axis(g, keep, axis=2)
    out = np.zeros_like(g)
    np.put_along_axis(out, keep, kept, axis=2)
    return out.reshape(N, K), keep.astype(np.uint8), kept.astype(np.int8)


# ---------------------------------------------------------------- a4: encode
def encode(keep: np.ndarray, kept: np.ndarray):
    """Packed values and 2-bit index metadata in the layout of R8.

    [CT] §2.2.3: only the retained values are stored, with metadata indices
    recording their original positions.  Returns (values uint8 [N, K/4],
    meta uint8 [N, K/8]).
    """
    N, G4, _ = keep.shape
    if G4 % 4:
        raise ValueError("K must be a multiple of 16")
    nib = (kept.astype(np.int32) & 0xF).astype(np.uint32).reshape(N, G4 // 4, 4, 2)
    idx = keep.astype(np.uint32).reshape(N, G4 // 4, 4, 2)
    word = np.zeros((N, G4 // 4), dtype=np.uint32)
    half = np.zeros((N, G4 // 4), dtype=np.uint32)
    for j in range(4):
        word |= nib[:, :, j, 0] << np.uint32(4 * j)
        word |= nib[:, :, j, 1] << np.uint32(16 + 4 * j)
        half |= idx[:, :, j, 0] << np.uint32(4 * j)
        half |= idx[:, :, j, 1] << np.uint32(4 * j + 2)
    values = np.ascontiguousarray(word.astype("<u4")).view(np.uint8).reshape(N, G4)
    meta = np.ascontiguousarray(half.astype("<u2")).view(np.uint8).reshape(N, G4 // 2)
    return values, meta


# ------------------------------------------------------------ a4b: arrange
def arrange(rows: np.ndarray, K: int, per_group: int) -> np.ndarray:
    """Row-ordered per-row data [N, (K/128) * per_group] -> the memory order
    of R8b (blocks of 16 rows; inside a block group by group, row by row).
    Returns a flat array of the same dtype."""
    rows = np.asarray(rows)
    N, C = rows.shape[0], K // GROUP
    parts = []
    for b0 in range(0, N, 16):
        blk = rows[b0:b0 + 16].reshape(-1, C, per_group)     # [rows of the block, group, item]
        parts.append(blk.transpose(1, 0, 2).reshape(-1))     # group-major, then row
    return np.concatenate(parts) if parts else rows.reshape(-1)


def rows_of(flat: np.ndarray, N: int, K: int, per_group: int) -> np.ndarray:
    """Inverse of ``arrange``: [N, (K/128) * per_group] in row order."""
    flat = np.asarray(flat).reshape(-1)
    C = K // GROUP
    out = np.empty((N, C * per_group), dtype=flat.dtype)
    pos = 0
    for b0 in range(0, N, 16):
        nb = min(16, N - b0)
        blk = flat[pos:pos + nb * C * per_group].reshape(C, nb, per_group)
        out[b0:b0 + nb] = blk.transpose(1, 0, 2).reshape(nb, C * per_group)
        pos += nb * C * per_group
    return out


def pack_rows(W: np.ndarray, group: int = GROUP):
    """quantise -> 2:4 prune -> encode, in row order: (values [N, K/4],
    meta [N, K/8], scales fp16 [N, K/128])."""
    s16 = group_scales(W, group)
    q = quantize(W, s16, group)
    _, keep, kept = prune_2of4(q)
    values, meta = encode(keep, kept)
    return values, meta, s16


def pack(W: np.ndarray, group: int = GROUP):
    """slim_pack: ``pack_rows`` in the memory order of R8b.  Returns flat
    (values uint8 [N K / 4], meta uint8 [N K / 8], scales fp16 [N K / 128])."""
    K = np.asarray(W).shape[1]
    values, meta, s16 = pack_rows(W, group)
    return arrange(values, K, 32), arrange(meta, K, 16), arrange(s16, K, 1)


# ------------------------------------------------------------------ decoding
def unpack(values: np.ndarray, meta: np.ndarray, K: int) -> np.ndarray:
    """Inverse of ``pack`` for the codes: int8 [N, K] with zeros at the
    pruned positions (values and meta in the memory order of R8b)."""
    values = np.asarray(values, dtype=np.uint8).reshape(-1)
    N = values.size * 4 // K
    values = np.ascontiguousarray(rows_of(values, N, K, 32))
    meta = np.ascontiguousarray(rows_of(np.asarray(meta, dtype=np.uint8), N, K, 16))
    word = values.reshape(N, K // 16, 4).copy().view("<u4")[:, :, 0].astype(np.uint32)
    half = meta.reshape(N, K // 16, 2).copy().view("<u2")[:, :, 0].astype(np.uint32)
    q = np.zeros((N, K // 16, 16), dtype=np.int8)
    rows = np.arange(N)[:, None]
    blocks = np.arange(K // 16)[None, :]
    for j in range(4):
        for h in range(2):
            nib = (word >> np.uint32(16 * h + 4 * j)) & np.uint32(0xF)
            val = nib.astype(np.int16) - 16 * (nib >= 8)          # 4-bit two's complement
            pos = (half >> np.uint32(4 * j + 2 * h)) & np.uint32(0x3)
            q[rows, blocks, 4 * j + pos.astype(np.int64)] = val.astype(np.int8)
    return q.reshape(N, K)


def dequantize(q: np.ndarray, s16: np.ndarray, group: int = GROUP) -> np.ndarray:
    """deq(W_c) = q * s16 in float64 ([CT] Fig. 7.1: W_C is the compressed weight).
    s16: [N, K/group] in row order, or flat in the memory order of R8b."""
    if np.asarray(s16).ndim == 1:
        s16 = rows_of(s16, q.shape[0], q.shape[1], 1)
    s = np.repeat(s16.astype(np.float64), group, axis=1)
    return q.astype(np.float64) * s


# ------------------------------------------------------------- a5..a7: linear
def linear(X, values, meta, scales, L=None, R=None, group: int = GROUP, rows=None):
    """Y = X deq(W_c)^T + (X L) R in float64.

    [CT] §2.1 (Y = X W^T), Ch. 4 introduction (sparse weights and the dense
    adapter as parallel paths), §1.2.3 (the rank-r factor pair).  ``rows``
    selects a subset of the token rows of X (Y's rows are independent).
    Returns float64 [M or len(rows), N].
    """
    X = np.asarray(X)
    if rows is not None:
        X = X[np.asarray(rows)]
    K = X.shape[1]
    D = dequantize(unpack(values, meta, K), scales, group)
    X64 = X.astype(np.float64)
    Y = X64 @ D.T
    if L is not None and R is not None and L.shape[1] > 0:
        T = X64 @ np.asarray(L).astype(np.float64)
        Y = Y + T @ np.asarray(R).astype(np.float64)
    return Y


def linear_batched(Xs, packs, Ls, Rs, group: int = GROUP):
    """slim_linear_batched: independent problems, one ``linear`` each."""
    return [linear(X, v, m, s, L, R, group) for X, (v, m, s), L, R in zip(Xs, packs, Ls, Rs)]


# ------------------------------------------- quantised adapters (QA1-QA3)
ADAPTER_GROUP_L = 128
ADAPTER_GROUP_R = 32
NIB_POS = (0, 4, 1, 5, 2, 6, 3, 7)    # element e of a run of 8 -> nibble of its uint32 (QA3)


def quantize_adapter(At: np.ndarray, group: int):
    """Codes and fp16 group scales of an adapter factor stored output-major
    (rows: outputs of its product, columns: its reduction dimension), with the
    quantiser of W and no pruning (QA1, QA2).  Returns (q int8 [rows, cols],
    s16 float16 [rows, cols / group])."""
    s16 = group_scales(At, group)
    return quantize(At, s16, group), s16


def pack_adapter(q: np.ndarray) -> np.ndarray:
    """QA3 packing: uint8 [rows, cols / 2]."""
    q = np.asarray(q)
    rows, cols = q.shape
    if cols % 8:
        raise ValueError("adapter columns must be a multiple of 8")
    nib = (q.astype(np.int32) & 0xF).astype(np.uint32).reshape(rows, cols // 8, 8)
    word = np.zeros((rows, cols // 8), dtype=np.uint32)
    for e in range(8):
        word |= nib[:, :, e] << np.uint32(4 * NIB_POS[e])
    return word.astype("<u4").view(np.uint8).reshape(rows, cols // 2)


def unpack_adapter(packed: np.ndarray, cols: int) -> np.ndarray:
    """Inverse of ``pack_adapter``: int8 codes [rows, cols]."""
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1, cols // 2)
    rows = packed.shape[0]
    word = packed.reshape(rows, cols // 8, 4).copy().view("<u4")[:, :, 0].astype(np.uint32)
    q = np.zeros((rows, cols // 8, 8), dtype=np.int8)
    for e in range(8):
        nib = (word >> np.uint32(4 * NIB_POS[e])) & np.uint32(0xF)
        q[:, :, e] = (nib.astype(np.int16) - 16 * (nib >= 8)).astype(np.int8)
    return q.reshape(rows, cols)


def pack_adapters(L: np.ndarray, R: np.ndarray):
    """slim_pack_adapter on Lt = L^T (groups of 128) and Rt = R^T (groups of
    32).  Returns (lq uint8 [r, K/2], ls fp16 [r, K/128], rq uint8 [N, r/2],
    rs fp16 [N, r/32])."""
    Lt = np.ascontiguousarray(np.asarray(L, dtype=np.float32).T)
    Rt = np.ascontiguousarray(np.asarray(R, dtype=np.float32).T)
    lq, ls = quantize_adapter(Lt, ADAPTER_GROUP_L)
    rq, rs = quantize_adapter(Rt, ADAPTER_GROUP_R)
    return pack_adapter(lq), ls, pack_adapter(rq), rs


def dequantized_adapters(lq, ls, rq, rs, K: int, r: int):
    """deq(L) [K, r] and deq(R) [r, N] in float64 from the packed factors."""
    Lt = dequantize(unpack_adapter(lq, K), np.asarray(ls).reshape(-1, K // ADAPTER_GROUP_L), ADAPTER_GROUP_L)
    Rt = dequantize(unpack_adapter(rq, r), np.asarray(rs).reshape(-1, r // ADAPTER_GROUP_R), ADAPTER_GROUP_R)
    return Lt.T, Rt.T


def linear_qa(X, values, meta, scales, lq, ls, rq, rs, r: int, group: int = GROUP, rows=None):
    """Y = X deq(W_c)^T + (X deq(L)) deq(R) in float64 (quantised adapters)."""
    K = np.asarray(X).shape[1]
    Ld, Rd = dequantized_adapters(lq, ls, rq, rs, K, r)
    return linear(X, values, meta, scales, Ld, Rd, group, rows)


# ------------------------------------------ SLoPe double-pruned transpose
def pack_transposed(values, meta, scales, N: int, K: int, group: int = GROUP):
    """Double-pruned transpose of the packed W_c (T1-T3).  Returns (tvalues
    float16 [K, N/2], tmeta uint16 [K, N/16])."""
    if N % 16:
        raise ValueError("N must be a multiple of 16")
    q = unpack(values, meta, K)
    s16 = rows_of(scales, N, K, 1)
    # T1: q * s16 is exact in float32 (a 3-bit integer times an 11-bit
    # significand); the cast is the one rounding to fp16.
    D = (q.astype(np.float32) * np.repeat(s16.astype(np.float32), group, axis=1)).astype(np.float16)
    Dt = np.ascontiguousarray(D.T)                                    # [K, N]
    g = Dt.reshape(K, N // 4, 4)
    order = np.argsort(-np.abs(g.astype(np.float32)), axis=2, kind="stable")
    keep = np.sort(order[:, :, :2], axis=2)                           # T2
    kept = np.take_along_axis(g, keep, axis=2)
    tvalues = kept.reshape(K, N // 2)                                 # T3
    idx = keep.astype(np.uint32).reshape(K, N // 16, 4, 2)
    half = np.zeros((K, N // 16), dtype=np.uint32)
    for j in range(4):
        half |= idx[:, :, j, 0] << np.uint32(4 * j)
        half |= idx[:, :, j, 1] << np.uint32(4 * j + 2)
    return tvalues, half.astype(np.uint16)


def unpack_transposed(tvalues, tmeta, N: int) -> np.ndarray:
    """Inverse of the T3 packing: float16 [K, N] with zeros where pruned."""
    tvalues = np.asarray(tvalues, dtype=np.float16)
    K = tvalues.shape[0]
    out = np.zeros((K, N // 4, 4), dtype=np.float16)
    v = tvalues.reshape(K, N // 16, 4, 2)
    m = np.asarray(tmeta, dtype=np.uint32).reshape(K, N // 16)
    rows = np.arange(K)[:, None]
    for b in range(N // 16):
        for j in range(4):
            for h in range(2):
                pos = (m[:, b] >> np.uint32(4 * j + 2 * h)) & np.uint32(3)
                out[rows[:, 0], 4 * b + j, pos.astype(np.int64)] = v[:, b, j, h]
    return out.reshape(K, N)


# ------------------------------------------------ 8-bit input (A1-A3)
QMAX_INPUT = 127


def quantize_input(X: np.ndarray):
    """Per-token symmetric int8 quantisation of the layer input (A1).

    [CT] Appendix E.2 (input quantisation), captions of Tables E.2 / E.5
    (4-bit weights with 8-bit input).  Returns (q int8 [M, K], s float16 [M]).
    """
    Xf = np.asarray(X).astype(np.float32)          # fp16 -> fp32 is exact
    M, K = Xf.shape
    if M == 0:
        return np.zeros((0, K), dtype=np.int8), np.zeros((0,), dtype=np.float16)
    absmax = np.max(np.abs(Xf), axis=1)            # exact in fp32
    s16 = (absmax / np.float32(QMAX_INPUT)).astype(np.float16)
    s = s16.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = Xf / s                                 # float32, correctly rounded
    q = np.clip(np.rint(t), -QMAX_INPUT, QMAX_INPUT)
    q = np.where(s > 0, q, 0.0)
    return q.astype(np.int8), s16


def dequantize_input(q: np.ndarray, s16: np.ndarray) -> np.ndarray:
    """deq(X) = q * s in float64 (A2)."""
    return np.asarray(q).astype(np.float64) * np.asarray(s16).astype(np.float64)[:, None]


def linear_a8(qx, sx, values, meta, scales, L=None, R=None, group: int = GROUP, rows=None):
    """Y = deq(X) deq(W_c)^T + (deq(X) L) R in float64, the layer with an
    8-bit input (A2).  ``rows`` selects token rows as in ``linear``."""
    return linear(dequantize_input(qx, sx), values, meta, scales, L, R, group, rows)


# ------------------------------------------ hybrid dense / 2:4 tiles (P1-P4)
TILE_ROWS = 16


def expand_tile_flags(dense: np.ndarray, N: int, K: int, group: int = GROUP) -> np.ndarray:
    """Per-tile flags [ceil(N/16), K/group] -> per-element booleans [N, K] (P1)."""
    d = np.asarray(dense).astype(bool)
    return np.repeat(np.repeat(d, TILE_ROWS, axis=0)[:N], group, axis=1)


def pack_hybrid(W: np.ndarray, dense: np.ndarray, group: int = GROUP):
    """PATCH-style hybrid pack (P1-P3).  Returns flat (values, meta, scales,
    dvalues) in the memory order of R8b."""
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    s16 = group_scales(W, group)
    q = quantize(W, s16, group)
    _, keep, kept = prune_2of4(q)
    g = q.reshape(N, K // 4, 4)
    dense_g = expand_tile_flags(dense, N, K, group)[:, ::4]            # [N, K/4]
    first, second = np.array([0, 1], dtype=np.uint8), np.array([2, 3], dtype=np.uint8)
    keep_p = np.where(dense_g[..., None], first, keep).astype(np.uint8)
    kept_p = np.where(dense_g[..., None], g[:, :, 0:2], kept).astype(np.int8)
    values, meta = encode(keep_p, kept_p)
    kept_s = np.where(dense_g[..., None], g[:, :, 2:4], 0).astype(np.int8)
    dvalues, _ = encode(np.broadcast_to(second, keep.shape).astype(np.uint8), kept_s)
    return arrange(values, K, 32), arrange(meta, K, 16), arrange(s16, K, 1), arrange(dvalues, K, 32)


def unpack_hybrid(values, meta, dvalues, K: int) -> np.ndarray:
    """int8 codes [N, K] of the hybrid weight: the 2:4 part plus the second
    pair of every dense tile (positions 2 and 3)."""
    q1 = unpack(values, meta, K)
    fixed = np.full(np.asarray(meta).size, 0xEE, dtype=np.uint8)       # positions (2, 3) in every group
    q2 = unpack(dvalues, fixed, K)
    return (q1.astype(np.int16) + q2.astype(np.int16)).astype(np.int8)


def linear_hybrid(X, values, meta, scales, dvalues, L=None, R=None, group: int = GROUP, rows=None):
    """Y = X deq(W_h)^T + (X L) R in float64 (P4)."""
    X = np.asarray(X)
    if rows is not None:
        X = X[np.asarray(rows)]
    K = X.shape[1]
    D = dequantize(unpack_hybrid(values, meta, dvalues, K), scales, group)
    X64 = X.astype(np.float64)
    Y = X64 @ D.T
    if L is not None and R is not None and L.shape[1] > 0:
        Y = Y + (X64 @ np.asarray(L).astype(np.float64)) @ np.asarray(R).astype(np.float64)
    return Y
