"""Pins for the CPU oracle: facts the method's pages and plain mathematics fix.

None of these tests retypes the oracle's formulas: each compares the oracle
with an independently derived expectation (hand-derived bytes, exhaustive
enumeration, closed forms, exact special cases, a pure-Python brute force
that decodes the bit layout on its own).
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
import workloads as wl


# ----------------------------------------------------------------- helpers
def _read_golden(path):
    sections = {}
    cur = None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = line.strip("[]")
                sections[cur] = []
                continue
            sections[cur].append(line.split())
    return sections


def _decode_bits_pure_python(values_row, meta_row, K):
    """Independent decoder: one k at a time, from the byte-level description
    (per 16 k: uint32 values word, uint16 metadata half-word)."""
    q = [0] * K
    for b in range(K // 16):
        word = int.from_bytes(bytes(int(x) for x in values_row[4 * b:4 * b + 4]), "little")
        half = int.from_bytes(bytes(int(x) for x in meta_row[2 * b:2 * b + 2]), "little")
        for j in range(4):
            for h in range(2):
                nib = (word >> (16 * h + 4 * j)) & 0xF
                v = nib - 16 if nib & 0x8 else nib
                pos = (half >> (4 * j + 2 * h)) & 0x3
                q[16 * b + 4 * j + pos] = v
    return q


# ------------------------------------------------------------ worked example
def test_golden_worked_example(golden_dir):
    g = _read_golden(os.path.join(golden_dir, "pack_worked_example.txt"))
    W = np.zeros((2, 128), dtype=np.float32)
    for n, k, v in g["W"]:
        W[int(n), int(k)] = np.float32(float(v))
    values_r, meta_r, scales_r = oracle.pack_rows(W)
    for row in g["values"]:
        assert [f"{b:02x}" for b in values_r[int(row[0])]] == row[1:]
    for row in g["meta"]:
        assert [f"{b:02x}" for b in meta_r[int(row[0])]] == row[1:]
    for n, hexs in g["scales"]:
        assert scales_r.view(np.uint16)[int(n), 0] == int(hexs, 16)
    # Two rows and one group of 128: the memory order is the row order.
    values, meta, scales = oracle.pack(W)
    assert np.array_equal(values, values_r.reshape(-1)) and np.array_equal(meta, meta_r.reshape(-1))
    assert np.array_equal(scales.view(np.uint16), scales_r.view(np.uint16).reshape(-1))
    X = np.zeros((1, 128), dtype=np.float16)
    X[0, :16] = np.arange(1, 17)
    Y = oracle.linear(X, values, meta, scales)
    for n, v in g["linear"]:
        assert Y[0, int(n)] == float(v)


# ------------------------------------------------------------------- scales
def test_scale_values_and_rounding():
    # absmax 7 -> exactly 1.0
    W = np.zeros((1, 128), np.float32)
    W[0, 5] = -7.0
    assert float(oracle.group_scales(W)[0, 0]) == 1.0
    # 7*(1+2^-11)/7 = 1+2^-11 lies half-way between fp16 1.0 and 1+2^-10: even -> 1.0
    W[0, 5] = np.float32(7.0 * (1 + 2.0 ** -11))
    assert float(oracle.group_scales(W)[0, 0]) == 1.0
    # 1+3*2^-11 lies half-way between 1+2^-10 (odd) and 1+2^-9 (even) -> 1+2^-9
    W[0, 5] = np.float32(7.0 * (1 + 3 * 2.0 ** -11))
    assert float(oracle.group_scales(W)[0, 0]) == 1 + 2.0 ** -9
    # absmax 0.7: fp32(0.7)/7 rounds to fp16 0x2E66
    W[0, 5] = np.float32(0.7)
    assert oracle.group_scales(W).view(np.uint16)[0, 0] == 0x2E66
    # all-zero group -> scale 0 and q = 0
    W[:] = 0
    s = oracle.group_scales(W)
    assert float(s[0, 0]) == 0.0
    assert not oracle.quantize(W, s).any()


def test_quantizer_divides_by_the_stored_fp16_scale():
    # absmax 0.7: s32 = fp32(0.7)/7 ~ 0.1 but the stored s16 = 0.0999755859375.
    # w = 0.24997 gives w/s16 = 2.5003 -> 3, whereas w/s32 = 2.4997 would give 2.
    W = np.zeros((1, 128), np.float32)
    W[0, 0] = np.float32(0.7)
    W[0, 1] = np.float32(0.24997)
    s = oracle.group_scales(W)
    q = oracle.quantize(W, s)
    assert int(q[0, 0]) == 7 and int(q[0, 1]) == 3


def test_scale_is_per_group_of_128_along_k():
    rng = np.random.default_rng(1)
    W = wl.random_weights(rng, 3, 512)
    s = oracle.group_scales(W)
    assert s.shape == (3, 4)
    for n in range(3):
        for j in range(4):
            a = max(abs(float(x)) for x in W[n, 128 * j:128 * j + 128])
            assert float(s[n, j]) == float(np.float16(np.float32(a) / np.float32(7)))


# --------------------------------------------------------------- quantiser
def test_quantizer_closed_form():
    rng = np.random.default_rng(2)
    W = wl.random_weights(rng, 64, 1024)
    W[:, 7] *= 20                                           # an outlier column
    s = oracle.group_scales(W)
    q = oracle.quantize(W, s)
    assert np.abs(q).max() <= 7
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    w = W.astype(np.float64)
    # reconstruction error at most half a step (plus the fp16 scale rounding)
    assert np.all(np.abs(w - q * sf) <= sf / 2 * (1 + 2.0 ** -10))
    # the group's absmax element lands on +-7
    g = np.abs(W).reshape(64, 8, 128)
    amax_pos = g.argmax(axis=2)
    qg = q.reshape(64, 8, 128)
    assert np.all(np.abs(np.take_along_axis(qg, amax_pos[..., None], 2)) == 7)
    # brute force over all 15 codes: q is the nearest code (exact halves may go either way)
    cands = np.arange(-7, 8, dtype=np.float64)
    err = np.abs(w[..., None] - cands * sf[..., None])
    best = err.min(axis=-1)
    mine = np.abs(w - q * sf)
    assert np.all(mine <= best + 1e-12 * sf)


def test_sign_symmetry():
    rng = np.random.default_rng(3)
    W = wl.random_weights(rng, 32, 512)
    v1, m1, s1 = oracle.pack(W)
    v2, m2, s2 = oracle.pack(-W)
    assert np.array_equal(m1, m2)
    assert np.array_equal(s1.view(np.uint16), s2.view(np.uint16))
    q1 = oracle.unpack(v1, m1, 512)
    q2 = oracle.unpack(v2, m2, 512)
    assert np.array_equal(q1, -q2)


# ----------------------------------------------------------------- pruning
def test_prune_rule_exhaustive():
    """All 15^4 int4 groups: stable top-2 equals 'best pair by |a|+|b|, ties to
    the lexicographically smallest pair' (an independent formulation)."""
    vals = np.array(list(itertools.product(range(-7, 8), repeat=4)), dtype=np.int8)
    q = vals.reshape(1, -1)
    _, keep, kept = oracle.prune_2of4(q)
    keep = keep.reshape(-1, 2)
    pairs = list(itertools.combinations(range(4), 2))
    mags = np.abs(vals.astype(np.int16))
    sums = np.stack([mags[:, a] + mags[:, b] for a, b in pairs], axis=1)
    best = np.argmax(sums, axis=1)          # argmax returns the first maximum = lexicographic
    expect = np.array(pairs)[best]
    assert np.array_equal(keep, expect)
    assert np.array_equal(kept.reshape(-1, 2), np.take_along_axis(vals, expect.astype(np.int64), 1))


def test_at_most_two_nonzeros_per_four_small_configs():
    for case in (wl.TINY, wl.QPROJ):
        W = wl.make_inputs(case).W
        v, m, s = oracle.pack(W)
        q = oracle.unpack(v, m, case.K)
        assert (np.count_nonzero(q.reshape(case.N, -1, 4), axis=2) <= 2).all()


@pytest.mark.slow
def test_at_most_two_nonzeros_large_configs():
    for case in (wl.GATEUP, wl.DOWN):
        W = wl.make_inputs(case).W
        v, m, s = oracle.pack(W)
        q = oracle.unpack(v, m, case.K)
        assert (np.count_nonzero(q.reshape(case.N, -1, 4), axis=2) <= 2).all()


def test_round_trip_independent_decoder():
    rng = np.random.default_rng(4)
    W = wl.random_weights(rng, 6, 256)
    W[:, :4] = 0                                  # a group that is all ties
    s = oracle.group_scales(W)
    q_pruned, _, _ = oracle.prune_2of4(oracle.quantize(W, s))
    v, m, _ = oracle.pack_rows(W)
    for n in range(6):
        assert _decode_bits_pure_python(v[n], m[n], 256) == [int(x) for x in q_pruned[n]]
    v, m, _ = oracle.pack(W)
    assert np.array_equal(oracle.unpack(v, m, 256), q_pruned)


def test_idempotent_repack():
    rng = np.random.default_rng(5)
    W = wl.random_weights(rng, 48, 1024)
    W[:, 100] *= 20
    v, m, s = oracle.pack(W)
    Wd = oracle.dequantize(oracle.unpack(v, m, 1024), s).astype(np.float32)  # exact in fp32
    v2, m2, s2 = oracle.pack(Wd)
    assert np.array_equal(v, v2) and np.array_equal(m, m2)
    assert np.array_equal(s.view(np.uint16), s2.view(np.uint16))


def test_memory_order_of_packed_blocks():
    """R8b: rows in blocks of 16 (a short last block), group-major inside a
    block.  Each row's bytes sit where the convention puts them, the order is
    a permutation (round trip), and one block's group is contiguous."""
    rng = np.random.default_rng(12)
    N, K = 37, 384                                  # blocks of 16, 16, 5; three groups
    W = wl.random_weights(rng, N, K)
    vr, mr, sr = oracle.pack_rows(W)
    v, m, s = oracle.pack(W)
    assert v.size == vr.size and m.size == mr.size and s.size == sr.size
    for n in range(N):
        b, i = divmod(n, 16)
        nb = min(16, N - 16 * b)
        for c in range(K // 128):
            assert np.array_equal(v[16 * b * K // 4 + (c * nb + i) * 32:][:32], vr[n, 32 * c:32 * c + 32])
            assert np.array_equal(m[16 * b * K // 8 + (c * nb + i) * 16:][:16], mr[n, 16 * c:16 * c + 16])
            assert s.view(np.uint16)[16 * b * K // 128 + c * nb + i] == sr.view(np.uint16)[n, c]
    assert np.array_equal(oracle.rows_of(v, N, K, 32), vr)
    assert np.array_equal(oracle.rows_of(m, N, K, 16), mr)
    assert np.array_equal(oracle.rows_of(s, N, K, 1).view(np.uint16), sr.view(np.uint16))


def test_packed_sizes_match_the_compression_ratios():
    # 4-bit values at 2:4 = 1/8 of fp16 bytes; 2-bit indices = K/8 bytes per row
    rng = np.random.default_rng(6)
    W = wl.random_weights(rng, 16, 1024)
    v, m, s = oracle.pack(W)
    assert v.nbytes * 8 == W.size * 2
    assert m.nbytes * 8 == W.size
    assert s.nbytes == W.size // 64


# ------------------------------------------------------------------ linear
def _exact_grid_weights(rng, N, K, scale_exp):
    """W already 2:4-sparse with integer codes times a power-of-two scale and a
    +-7 in every group of 128: the pack is lossless on it."""
    q = np.zeros((N, K // 4, 4), np.int64)
    for n in range(N):
        for gidx in range(K // 4):
            a, b = sorted(rng.choice(4, 2, replace=False))
            q[n, gidx, a] = rng.integers(-7, 8)
            q[n, gidx, b] = rng.integers(-7, 8)
    q = q.reshape(N, K)
    for n in range(N):
        for j in range(K // 128):
            blk = q[n, 128 * j:128 * j + 128].reshape(32, 4)
            # force one kept slot of the first group to 7 with the right sign
            nz = np.flatnonzero(blk[0]) if np.count_nonzero(blk[0]) else np.array([0])
            blk[0, nz[0]] = 7 if rng.random() < 0.5 else -7
            q[n, 128 * j:128 * j + 128] = blk.reshape(-1)
    return (q * 2.0 ** scale_exp).astype(np.float32)


def test_linear_lossless_grid_reduces_to_plain_gemm():
    rng = np.random.default_rng(7)
    W = _exact_grid_weights(rng, 24, 256, -6)
    X = wl.random_fp16(rng, (5, 256))
    v, m, s = oracle.pack(W)
    assert np.array_equal(oracle.dequantize(oracle.unpack(v, m, 256), s), W.astype(np.float64))
    Y = oracle.linear(X, v, m, s)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.allclose(Y, ref, rtol=1e-13, atol=1e-13)


def test_linear_zero_weight_is_pure_adapter():
    rng = np.random.default_rng(8)
    W = np.zeros((40, 256), np.float32)
    X = wl.random_fp16(rng, (3, 256))
    L = wl.random_fp16(rng, (256, 32), 0.02)
    R = wl.random_fp16(rng, (32, 40), 0.02)
    v, m, s = oracle.pack(W)
    Y = oracle.linear(X, v, m, s, L, R)
    x, l, r = (a.astype(np.float64) for a in (X, L, R))
    ref = np.einsum("mk,kj,jn->mn", x, l, r)
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-15)


def test_linear_identity_input_recovers_matrices():
    rng = np.random.default_rng(9)
    K = 128
    W = wl.random_weights(rng, 16, K)
    L = wl.random_fp16(rng, (K, 32), 0.02)
    R = wl.random_fp16(rng, (32, 16), 0.02)
    X = np.eye(K, dtype=np.float16)
    v, m, s = oracle.pack(W)
    Y = oracle.linear(X, v, m, s, L, R)
    deq = oracle.dequantize(oracle.unpack(v, m, K), s)
    LR = L.astype(np.float64) @ R.astype(np.float64)
    assert np.allclose(Y, deq.T + LR, rtol=1e-13, atol=1e-15)


def _brute_force_linear(X, v, m, s, L, R, rows):
    M, K = X.shape
    N = s.size // (K // 128)
    r = L.shape[1]
    v, m, s = oracle.rows_of(v, N, K, 32), oracle.rows_of(m, N, K, 16), oracle.rows_of(s, N, K, 1)
    Wd = []
    for n in range(N):
        q = _decode_bits_pure_python(v[n], m[n], K)
        Wd.append([q[k] * float(s[n, k // 128]) for k in range(K)])
    out = []
    for mm in rows:
        x = [float(a) for a in X[mm]]
        t = [math.fsum(x[k] * float(L[k, j]) for k in range(K)) for j in range(r)]
        row = []
        for n in range(N):
            main = math.fsum(x[k] * Wd[n][k] for k in range(K))
            ad = math.fsum(t[j] * float(R[j, n]) for j in range(r))
            row.append(main + ad)
        out.append(row)
    return np.array(out)


def test_brute_force_tiny():
    rng = np.random.default_rng(10)
    X = wl.random_fp16(rng, (3, 128))
    W = wl.random_weights(rng, 5, 128)
    L = wl.random_fp16(rng, (128, 4), 0.02)
    R = wl.random_fp16(rng, (4, 5), 0.02)
    v, m, s = oracle.pack(W)
    Y = oracle.linear(X, v, m, s, L, R)
    B = _brute_force_linear(X, v, m, s, L, R, range(3))
    assert np.allclose(Y, B, rtol=1e-12, atol=1e-12)


def test_brute_force_tiny_config_rows():
    inp = wl.make_inputs(wl.TINY)
    v, m, s = oracle.pack(inp.W)
    rows = [0, 11]
    Y = oracle.linear(inp.X, v, m, s, inp.L, inp.R, rows=rows)
    B = _brute_force_linear(inp.X, v, m, s, inp.L, inp.R, rows)
    assert np.allclose(Y, B, rtol=1e-12, atol=1e-12)


def test_brute_force_batched():
    """linear_batched: each problem equals its own brute force (problems with
    different weights, adapters and inputs; one problem without an adapter)."""
    rng = np.random.default_rng(11)
    Xs, packs, Ls, Rs = [], [], [], []
    for i in range(3):
        Xs.append(wl.random_fp16(rng, (2, 128)))
        packs.append(oracle.pack(wl.random_weights(rng, 4, 128)))
        Ls.append(wl.random_fp16(rng, (128, 4), 0.02) if i != 1 else None)
        Rs.append(wl.random_fp16(rng, (4, 4), 0.02) if i != 1 else None)
    Ys = oracle.linear_batched(Xs, packs, Ls, Rs)
    assert len(Ys) == 3
    for X, (v, m, s), L, R, Y in zip(Xs, packs, Ls, Rs, Ys):
        if L is None:
            L, R = np.zeros((128, 1), np.float16), np.zeros((1, 4), np.float16)
        B = _brute_force_linear(X, v, m, s, L, R, range(2))
        assert np.allclose(Y, B, rtol=1e-12, atol=1e-12)


def test_linear_rows_subset_matches_full():
    inp = wl.make_inputs(wl.TINY)
    v, m, s = oracle.pack(inp.W)
    full = oracle.linear(inp.X, v, m, s, inp.L, inp.R)
    sub = oracle.linear(inp.X, v, m, s, inp.L, inp.R, rows=[3, 7, 15])
    assert np.array_equal(sub, full[[3, 7, 15]])


# ------------------------------------------------------------------ inputs
def test_workload_recipe_is_seeded_and_shaped():
    a = wl.make_inputs(wl.TINY)
    b = wl.make_inputs(wl.TINY)
    assert np.array_equal(a.W, b.W) and np.array_equal(a.X, b.X)
    assert a.X.shape == (16, 512) and a.X.dtype == np.float16
    assert a.W.shape == (512, 512) and a.W.dtype == np.float32
    assert a.L.shape == (512, 32) and a.R.shape == (32, 512)
    assert abs(float(a.W.std()) - 0.02) < 1e-3
    g = wl.make_inputs(wl.Case("g", M=1, N=64, K=4096, r=32, outlier_frac=0.01))
    assert len(g.outlier_cols) == 41


# ------------------------------------------------ quantised adapters (QA1-QA3)
def _read_fixture(path):
    out = {}
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        out[k.strip()] = v.split()
    return out


def test_adapter_pack_worked_example(golden_dir):
    fx = _read_fixture(os.path.join(golden_dir, "adapter_pack_worked_example.txt"))
    codes = np.array([[int(c) for c in fx["codes"]]], dtype=np.int8)
    want = bytes(int(b, 16) for b in fx["bytes"])
    assert oracle.pack_adapter(codes).tobytes() == want
    assert np.array_equal(oracle.unpack_adapter(np.frombuffer(want, dtype=np.uint8), 8), codes)


def test_adapter_pack_against_byte_level_decoder():
    # An independent decoder: element c of a row lives in byte 4 (c // 8) +
    # NIB_POS[c % 8] // 2 of the row, low nibble for an even position.
    rng = np.random.default_rng(5)
    q = rng.integers(-7, 8, size=(3, 48)).astype(np.int8)
    packed = oracle.pack_adapter(q)
    for i in range(3):
        row = packed[i].tobytes()
        for c in range(48):
            pos = oracle.NIB_POS[c % 8]
            byte = row[4 * (c // 8) + pos // 2]
            nib = (byte >> 4) if pos % 2 else (byte & 0xF)
            val = nib - 16 if nib >= 8 else nib
            assert val == q[i, c]


def test_adapter_scales_run_along_the_reduction_dimension():
    # Lt [r, K]: one scale per 128 k of a row; Rt [N, r]: one per 32 of a row.
    r, K, N = 3, 256, 5
    Lt = np.zeros((r, K), dtype=np.float32)
    Rt = np.zeros((N, 64), dtype=np.float32)
    for i in range(r):
        for g in range(2):
            Lt[i, 128 * g + (7 * i + g) % 128] = 0.5 + i + 2 * g      # one peak per group
    for n in range(N):
        for g in range(2):
            Rt[n, 32 * g + (5 * n + g) % 32] = -(0.25 + n + 3 * g)
    L, R = Lt.T, Rt.T
    lq, ls, rq, rs = oracle.pack_adapters(L, R)
    for i in range(r):
        for g in range(2):
            assert ls[i, g] == np.float16(np.float32(0.5 + i + 2 * g) / np.float32(7))
    for n in range(N):
        for g in range(2):
            assert rs[n, g] == np.float16(np.float32(0.25 + n + 3 * g) / np.float32(7))
    # The peak of every group quantises to +-7 exactly.
    ql = oracle.unpack_adapter(lq, K)
    assert sorted(set(np.abs(ql[ql != 0]).tolist())) == [7]


def test_linear_qa_brute_force_tiny():
    rng = np.random.default_rng(11)
    M, N, K, r = 2, 16, 128, 32
    X = rng.standard_normal((M, K)).astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    L = (rng.standard_normal((K, r)) * 0.05).astype(np.float32)
    R = (rng.standard_normal((r, N)) * 0.05).astype(np.float32)
    v, m, s = oracle.pack(W)
    lq, ls, rq, rs = oracle.pack_adapters(L, R)
    Y = oracle.linear_qa(X, v, m, s, lq, ls, rq, rs, r)
    # Brute force from the codes and scales, element by element.
    Wd = oracle.dequantize(oracle.unpack(v, m, K), s)
    qL = oracle.unpack_adapter(lq, K)
    qR = oracle.unpack_adapter(rq, r)
    Ld = [[float(qL[j, k]) * float(ls[j, k // 128]) for j in range(r)] for k in range(K)]
    Rd = [[float(qR[n, j]) * float(rs[n, j // 32]) for n in range(N)] for j in range(r)]
    for i in range(M):
        x = [float(t) for t in X[i]]
        T = [math.fsum(x[k] * Ld[k][j] for k in range(K)) for j in range(r)]
        for n in range(N):
            want = math.fsum(x[k] * Wd[n, k] for k in range(K)) + math.fsum(T[j] * Rd[j][n] for j in range(r))
            assert abs(Y[i, n] - want) <= 1e-12 * (1 + abs(want))


def test_quantized_adapters_on_their_own_grid_are_lossless():
    # Factors that are already q * s (s a power of two, |q| <= 7, each group
    # holding a +-7) come back exactly, so linear_qa equals linear.
    rng = np.random.default_rng(3)
    M, N, K, r = 3, 32, 256, 64
    Lq = rng.integers(-7, 8, size=(r, K))
    Lq[:, ::128] = 7
    Rq = rng.integers(-7, 8, size=(N, r))
    Rq[:, ::32] = -7
    L = (Lq * 2.0 ** -6).T.astype(np.float32)
    R = (Rq * 2.0 ** -5).T.astype(np.float32)
    lq, ls, rq, rs = oracle.pack_adapters(L, R)
    Ld, Rd = oracle.dequantized_adapters(lq, ls, rq, rs, K, r)
    assert np.array_equal(Ld, L.astype(np.float64)) and np.array_equal(Rd, R.astype(np.float64))
    X = rng.standard_normal((M, K)).astype(np.float16)
    v, m, s = oracle.pack((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    assert np.array_equal(oracle.linear_qa(X, v, m, s, lq, ls, rq, rs, r), oracle.linear(X, v, m, s, L, R))


def test_quantized_adapter_bytes():
    # q_proj factors: 2 x 4096 x 416 fp16 = 6.82 MB; int4 codes + fp16 scales.
    K = N = 4096
    r = 416
    L = np.zeros((K, r), dtype=np.float32)
    R = np.zeros((r, N), dtype=np.float32)
    lq, ls, rq, rs = oracle.pack_adapters(L, R)
    assert lq.nbytes == r * K // 2 and ls.size == r * K // 128
    assert rq.nbytes == N * r // 2 and rs.size == N * r // 32
    total = lq.nbytes + 2 * ls.size + rq.nbytes + 2 * rs.size
    assert total == 1837056 and total / (2 * 2 * K * r) < 0.27


# ------------------------------------------------ double-pruned transpose
def _worked_transpose_W():
    W = np.zeros((16, 128), dtype=np.float32)
    W[:4, :4] = [[5, -3, 1, 0], [2, 6, -4, 1], [-7, 1, 3, 3], [4, 4, 0, -2]]
    W[:4, 64] = 7
    return W


def test_transposed_pack_worked_example(golden_dir):
    """Hand-derived case (tests/golden/transposed_pack_worked_example.txt)."""
    W = _worked_transpose_W()
    tv, tm = oracle.pack_transposed(*oracle.pack(W), 16, 128)
    rows = np.loadtxt(os.path.join(golden_dir, "transposed_pack_worked_example.txt"), dtype=np.int64, ndmin=2)
    for k, lo, hi, vlo, vhi in rows:
        half = int(tm[k, 0])
        assert half & 3 == lo and (half >> 2) & 3 == hi, (k, half)
        assert float(tv[k, 0]) == vlo and float(tv[k, 1]) == vhi, (k, tv[k, :2])
    # Every other n-group of these rows is all zero: indices (0, 1), values 0.
    assert np.all(tv[:, 2:] == 0)
    assert np.all((tm[:, 1:] == 0x4444)) and np.all(tm[:, 0] >> 4 == 0x444)


def _pair_rule(g):
    """Independent statement of the 2:4 rule on one group of 4 magnitudes:
    the pair (a < b) with the largest |g_a| + |g_b|, the lexicographically
    smallest among equal sums."""
    best = None
    for a in range(4):
        for b in range(a + 1, 4):
            key = (-(abs(float(g[a])) + abs(float(g[b]))), a, b)
            best = key if best is None or key < best else best
    return best[1], best[2]


@pytest.mark.parametrize("seed,grid", [(1, False), (2, True), (3, True)])
def test_transposed_pack_against_pair_rule(seed, grid):
    """The second prune, checked group by group against the pair rule;
    grid=True draws small integers so that equal magnitudes are common."""
    rng = np.random.default_rng(seed)
    N, K = 32, 256
    if grid:
        W = rng.integers(-3, 4, size=(N, K)).astype(np.float32)
        W[:, ::128] = 7                                   # s16 = 1 in every group
    else:
        W = rng.standard_normal((N, K)).astype(np.float32) * 0.02
    v, m, s = oracle.pack(W)
    tv, tm = oracle.pack_transposed(v, m, s, N, K)
    D = oracle.dequantize(oracle.unpack(v, m, K), s).astype(np.float16).T     # [K, N]
    for k in range(K):
        for j in range(N // 4):
            lo, hi = _pair_rule(D[k, 4 * j:4 * j + 4])
            half = int(tm[k, j // 4]) >> (4 * (j % 4))
            assert (half & 3, (half >> 2) & 3) == (lo, hi), (k, j)
            assert tv[k, 2 * j] == D[k, 4 * j + lo] and tv[k, 2 * j + 1] == D[k, 4 * j + hi]


def test_transposed_pack_keeps_a_transposable_pattern():
    """A weight whose non-zeros form a 2:4 pattern along both dimensions
    (diagonal 2 x 2 blocks of every 4 x 4 tile) loses nothing in either
    prune: the double-pruned transpose is deq(W_c)^T exactly."""
    rng = np.random.default_rng(4)
    N, K = 48, 384
    mask = np.zeros((4, 4), dtype=bool)
    mask[:2, :2] = mask[2:, 2:] = True
    W = rng.standard_normal((N, K)).astype(np.float32) * np.tile(mask, (N // 4, K // 4))
    v, m, s = oracle.pack(W)
    tv, tm = oracle.pack_transposed(v, m, s, N, K)
    D = oracle.dequantize(oracle.unpack(v, m, K), s).astype(np.float16)
    assert np.array_equal(oracle.unpack_transposed(tv, tm, N), D.T)


def test_transposed_pack_invariants():
    rng = np.random.default_rng(5)
    N, K = 64, 512
    W = rng.standard_normal((N, K)).astype(np.float32) * 0.02
    v, m, s = oracle.pack(W)
    tv, tm = oracle.pack_transposed(v, m, s, N, K)
    B = oracle.unpack_transposed(tv, tm, N)                  # [K, N]
    D = oracle.dequantize(oracle.unpack(v, m, K), s).astype(np.float16).T
    assert ((B != 0).reshape(K, N // 4, 4).sum(-1) <= 2).all()
    kept = B != 0
    assert np.array_equal(B[kept], D[kept])                  # kept values are entries of deq(W_c)^T
    # Each group keeps its two largest magnitudes: none dropped is larger.
    bg, dg = np.abs(B.astype(np.float32)).reshape(K, N // 4, 4), np.abs(D.astype(np.float32)).reshape(K, N // 4, 4)
    dropped = np.where(bg == 0, dg, 0).max(-1)
    kept_min = np.where(bg != 0, bg, np.inf).min(-1)
    assert (dropped <= np.where(np.isinf(kept_min), np.inf, kept_min)).all()


# ------------------------------------------------ 8-bit input (A1-A3)
def test_input_quant_worked_example(golden_dir):
    g = _read_golden(os.path.join(golden_dir, "input_quant_worked_example.txt"))
    X = np.array([[float(v) for v in row] for row in g["X"]], dtype=np.float16)
    q_expect = np.array([[int(v) for v in row] for row in g["q"]], dtype=np.int8)
    s_expect = np.array([int(h, 16) for h in g["s_hex"][0]], dtype=np.uint16)
    q, s = oracle.quantize_input(X)
    assert np.array_equal(q, q_expect)
    assert np.array_equal(s.view(np.uint16), s_expect)


def test_input_quantizer_closed_form():
    """|q| <= 127, each row's absmax lands on +-127, q is the nearest of the
    255 codes (exact halves either way), reconstruction within half a step."""
    rng = np.random.default_rng(41)
    X = wl.random_fp16(rng, (24, 640))
    X[:, 13] *= np.float16(30)                     # an outlier channel
    X[5] *= np.float16(0.001)                      # small values: subnormal-range scales
    q, s = oracle.quantize_input(X)
    assert np.abs(q.astype(np.int32)).max() <= 127
    x = X.astype(np.float64)
    sf = s.astype(np.float64)[:, None]
    amax = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(24), amax].astype(np.int32)) == 127)
    cands = np.arange(-127, 128, dtype=np.float64)
    best = np.min(np.abs(x[..., None] - cands * sf[..., None]), axis=-1)
    mine = np.abs(x - q * sf)
    assert np.all(mine <= best + 1e-12 * sf)
    assert np.all(mine <= sf / 2 * (1 + 2.0 ** -9))


def test_input_quantizer_sign_zero_and_per_token():
    rng = np.random.default_rng(42)
    X = wl.random_fp16(rng, (6, 256))
    X[2] = 0
    q, s = oracle.quantize_input(X)
    qn, sn = oracle.quantize_input(-X)
    assert np.array_equal(qn, -q) and np.array_equal(sn.view(np.uint16), s.view(np.uint16))
    assert s[2] == 0 and not q[2].any()
    X2 = X.copy()
    X2[4] *= np.float16(8)                          # another token changes: this row's codes do not
    q2, s2 = oracle.quantize_input(X2)
    keep = [0, 1, 2, 3, 5]
    assert np.array_equal(q2[keep], q[keep]) and np.array_equal(s2[keep], s[keep])
    assert oracle.quantize_input(np.zeros((0, 64), np.float16))[0].shape == (0, 64)


def test_linear_a8_on_the_int8_grid_equals_the_fp16_layer():
    """Inputs already on the grid q * 2^-4 with a +-127 in every row quantise
    losslessly, so the 8-bit-input layer equals the plain layer on X."""
    rng = np.random.default_rng(43)
    q = rng.integers(-127, 128, size=(5, 256))
    q[:, 3] = 127 * np.where(rng.random(5) < 0.5, -1, 1)
    X = (q * 2.0 ** -4).astype(np.float16)
    assert np.array_equal(X.astype(np.float64), q * 2.0 ** -4)
    W = wl.random_weights(rng, 48, 256)
    L = wl.random_fp16(rng, (256, 32), 0.02)
    R = wl.random_fp16(rng, (32, 48), 0.02)
    v, m, s = oracle.pack(W)
    qx, sx = oracle.quantize_input(X)
    assert np.array_equal(qx.astype(np.int64), q) and np.all(sx == np.float16(2.0 ** -4))
    assert np.array_equal(oracle.linear_a8(qx, sx, v, m, s, L, R), oracle.linear(X, v, m, s, L, R))


def test_linear_a8_brute_force_tiny():
    """fsum brute force with the input dequantised element by element."""
    rng = np.random.default_rng(44)
    X = wl.random_fp16(rng, (3, 128))
    W = wl.random_weights(rng, 6, 128)
    L = wl.random_fp16(rng, (128, 4), 0.02)
    R = wl.random_fp16(rng, (4, 6), 0.02)
    v, m, s = oracle.pack(W)
    qx, sx = oracle.quantize_input(X)
    Xd = np.array([[int(qx[i, k]) * float(sx[i]) for k in range(128)] for i in range(3)])
    B = _brute_force_linear(Xd, v, m, s, L, R, range(3))
    Y = oracle.linear_a8(qx, sx, v, m, s, L, R)
    assert np.allclose(Y, B, rtol=1e-12, atol=1e-12)
    # and the input quantisation changed something (the test is not vacuous)
    assert not np.array_equal(Xd, X.astype(np.float64))


# ------------------------------------ hybrid dense / 2:4 tiles (P1-P4)
def test_hybrid_pack_worked_example(golden_dir):
    g = _read_golden(os.path.join(golden_dir, "hybrid_pack_worked_example.txt"))
    W = np.zeros((16, 256), np.float32)
    for k, v in g["w_row0"]:
        W[0, int(k)] = float(v)
    flags = np.array([[int(x) for x in g["flags"][0]]], dtype=np.uint8)
    v, m, s, d = oracle.pack_hybrid(W, flags)
    for name, arr in (("values", v), ("meta", m), ("dvalues", d)):
        for row in g[name]:
            off, expect = int(row[0]), bytes(int(x, 16) for x in row[1:])
            assert arr[off:off + len(expect)].tobytes() == expect, (name, off)
    for off, h in g["scales_hex"]:
        assert s.view(np.uint16)[int(off)] == int(h, 16)


def _tiles(rng, N, K, p):
    return (rng.random(((N + 15) // 16, K // 128)) < p).astype(np.uint8)


def test_hybrid_all_sparse_is_the_plain_pack():
    rng = np.random.default_rng(60)
    W = wl.random_weights(rng, 40, 512)
    v, m, s, d = oracle.pack_hybrid(W, np.zeros((3, 4), np.uint8))
    v0, m0, s0 = oracle.pack(W)
    assert np.array_equal(v, v0) and np.array_equal(m, m0) and np.array_equal(s.view(np.uint16), s0.view(np.uint16))
    assert not d.any()


def test_hybrid_tiles_are_dense_or_two_of_four():
    """Dense tiles keep every quantised code; 2:4 tiles equal the pruned
    codes; the scales are the plain ones.  Random tile masks, a short last
    row block (N = 37)."""
    rng = np.random.default_rng(61)
    N, K = 37, 640
    W = wl.random_weights(rng, N, K)
    flags = _tiles(rng, N, K, 0.4)
    v, m, s, d = oracle.pack_hybrid(W, flags)
    q = oracle.unpack_hybrid(v, m, d, K)
    s16 = oracle.group_scales(W)
    qd = oracle.quantize(W, s16)
    qp, _, _ = oracle.prune_2of4(qd)
    dense = oracle.expand_tile_flags(flags, N, K)
    assert np.array_equal(q[dense], qd[dense])
    assert np.array_equal(q[~dense], qp[~dense])
    assert np.array_equal(oracle.rows_of(s, N, K, 1).view(np.uint16), s16.view(np.uint16))
    # all dense: the whole quantised matrix, no pruning
    v, m, s, d = oracle.pack_hybrid(W, np.ones_like(flags))
    assert np.array_equal(oracle.unpack_hybrid(v, m, d, K), qd)


def test_hybrid_against_independent_decoder():
    """Byte-level decode of both arrays (second pair at fixed positions 2, 3)."""
    rng = np.random.default_rng(62)
    N, K = 18, 256
    W = wl.random_weights(rng, N, K)
    flags = _tiles(rng, N, K, 0.5)
    v, m, s, d = oracle.pack_hybrid(W, flags)
    q = oracle.unpack_hybrid(v, m, d, K)
    vr, mr, dr = oracle.rows_of(v, N, K, 32), oracle.rows_of(m, N, K, 16), oracle.rows_of(d, N, K, 32)
    for n in range(N):
        q1 = _decode_bits_pure_python(vr[n], mr[n], K)
        q2 = _decode_bits_pure_python(dr[n], [0xEE] * (K // 8), K)
        assert [a + b for a, b in zip(q1, q2)] == list(q[n])


def test_linear_hybrid_lossless_dense_grid_is_plain_gemm():
    """All tiles dense, W on the int4 grid with a +-7 in every group:
    nothing is lost, so the layer is the plain product."""
    rng = np.random.default_rng(63)
    N, K = 32, 256
    q = rng.integers(-7, 8, size=(N, K)).astype(np.float64)
    q[:, ::128] = 7
    scale = 2.0 ** rng.integers(-8, -3, size=(N, K // 128))
    W = (q * np.repeat(scale, 128, axis=1)).astype(np.float32)
    X = wl.random_fp16(rng, (5, K))
    v, m, s, d = oracle.pack_hybrid(W, np.ones((2, 2), np.uint8))
    Y = oracle.linear_hybrid(X, v, m, s, d)
    assert np.allclose(Y, X.astype(np.float64) @ W.astype(np.float64).T, rtol=1e-12, atol=1e-12)


def test_linear_hybrid_brute_force_tiny():
    rng = np.random.default_rng(64)
    X = wl.random_fp16(rng, (3, 256))
    W = wl.random_weights(rng, 20, 256)
    L = wl.random_fp16(rng, (256, 4), 0.02)
    R = wl.random_fp16(rng, (4, 20), 0.02)
    flags = np.array([[1, 0], [0, 1]], np.uint8)
    v, m, s, d = oracle.pack_hybrid(W, flags)
    N, K = 20, 256
    vr, mr, dr = oracle.rows_of(v, N, K, 32), oracle.rows_of(m, N, K, 16), oracle.rows_of(d, N, K, 32)
    sr = oracle.rows_of(s, N, K, 1)
    Wd = []
    for n in range(N):
        q1 = _decode_bits_pure_python(vr[n], mr[n], K)
        q2 = _decode_bits_pure_python(dr[n], [0xEE] * (K // 8), K)
        Wd.append([(q1[k] + q2[k]) * float(sr[n, k // 128]) for k in range(K)])
    Y = oracle.linear_hybrid(X, v, m, s, d, L, R)
    for i in range(3):
        x = [float(a) for a in X[i]]
        t = [math.fsum(x[k] * float(L[k, j]) for k in range(K)) for j in range(4)]
        for n in range(N):
            ref = math.fsum(x[k] * Wd[n][k] for k in range(K)) + math.fsum(t[j] * float(R[j, n]) for j in range(4))
            assert abs(Y[i, n] - ref) <= 1e-12 * max(1.0, abs(ref))
