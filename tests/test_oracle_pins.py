"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test checks an oracle function against one of: hand-built blocks with
hand-packed bytes (tests/golden/), the IEEE binary16 definition via numpy's
independent float16 type, exact integer arithmetic (numpy int64 products,
brute force), closed forms (softmax via scipy, SiLU via scipy's expit),
invariants, or compositions with already-pinned functions. A plausible slip
in the oracle (a swapped nibble, a wrong scale index, a dropped min term, a
transposed operand, a half-even instead of half-away rounding) fails one of
these.
"""
import itertools

import numpy as np
import pytest
import scipy.special

import oracle
import synth
from conftest import hexbytes, read_fixture


def _q4k_fixture():
    f = read_fixture("q4k_block.txt")
    blk = hexbytes(f["d"]) + hexbytes(f["dmin"]) + hexbytes(f["scales"]) + hexbytes(f["qs"])
    assert len(blk) == 144
    sc = [int(v) for v in f["sc"]]
    m = [int(v) for v in f["m"]]
    q = [[((32 * j + l) * 97 % 251) % 16 for l in range(32)] for j in range(8)]
    expect = np.array([1.0 * sc[j] * q[j][l] - 0.5 * m[j] for j in range(8) for l in range(32)])
    return np.frombuffer(blk, dtype=np.uint8), sc, m, q, expect


def _q6k_fixture():
    f = read_fixture("q6k_block.txt")
    blk = hexbytes(f["ql"]) + hexbytes(f["qh"]) + hexbytes(f["scales"]) + hexbytes(f["d"])
    assert len(blk) == 210
    sc = [int(v) for v in f["sc"]]
    q = [((97 * i) % 251) % 64 for i in range(256)]
    expect = np.array([0.5 * sc[i // 16] * (q[i] - 32) for i in range(256)])
    return np.frombuffer(blk, dtype=np.uint8), sc, q, expect


def _q8_0_fixture():
    f = read_fixture("q8_0_block.txt")
    q = [int(v) for v in f["q"]]
    blk = hexbytes(f["d"]) + bytes((v & 0xFF) for v in q)
    return np.frombuffer(blk, dtype=np.uint8), np.array(q, dtype=np.float64)


# ---------------------------------------------------------------------------
# O1: binary16 decode, exhaustive against numpy's float16
# ---------------------------------------------------------------------------
def test_half_exhaustive_vs_numpy_float16():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_half_subnormal_and_extremes_closed_form():
    assert oracle.half(0x0001) == 2.0 ** -24
    assert oracle.half(0x03FF) == 1023 * 2.0 ** -24
    assert oracle.half(0x0400) == 2.0 ** -14
    assert oracle.half(0x7BFF) == 65504.0
    assert oracle.half(0x8001) == -(2.0 ** -24)
    assert oracle.half(0x3C00) == 1.0 and oracle.half(0xC000) == -2.0


# ---------------------------------------------------------------------------
# O2: block decoders on hand-built blocks
# ---------------------------------------------------------------------------
def test_q4k_hand_block():
    blk, _, _, _, expect = _q4k_fixture()
    got = oracle.dequant("q4k", blk)
    assert np.array_equal(got, expect)


def test_q4k_hand_block_one_hot_columns():
    blk, _, _, _, expect = _q4k_fixture()
    for c in range(256):
        x = np.zeros(256, dtype=np.float32)
        x[c] = 1.0
        y = oracle.matvec("q4k", blk, x, 1, 256)
        assert y[0] == expect[c]


def test_q4k_subnormal_scales():
    blk, sc, m, q, _ = _q4k_fixture()
    b = blk.copy()
    b[0:2] = [0x01, 0x00]      # d = 2^-24
    b[2:4] = [0xFF, 0x03]      # dmin = 1023 * 2^-24
    expect = np.array([2.0 ** -24 * sc[j] * q[j][l] - 1023 * 2.0 ** -24 * m[j]
                       for j in range(8) for l in range(32)])
    assert np.array_equal(oracle.dequant("q4k", b), expect)


def test_q4k_packer_matches_hand_bytes():
    """The input encoder's scale packer agrees with the hand-packed bytes."""
    f = read_fixture("q4k_block.txt")
    got = synth.pack_q4k_scales([int(v) for v in f["sc"]], [int(v) for v in f["m"]])
    assert bytes(got) == hexbytes(f["scales"])


def test_q6k_hand_block():
    blk, _, _, expect = _q6k_fixture()
    assert np.array_equal(oracle.dequant("q6k", blk), expect)


def test_q6k_hand_block_one_hot_columns():
    blk, _, _, expect = _q6k_fixture()
    for c in range(256):
        x = np.zeros(256, dtype=np.float32)
        x[c] = 1.0
        assert oracle.matvec("q6k", blk, x, 1, 256)[0] == expect[c]


def test_q6k_subnormal_scale():
    blk, sc, q, _ = _q6k_fixture()
    b = blk.copy()
    b[208:210] = [0x07, 0x00]  # d = 7 * 2^-24
    expect = np.array([7 * 2.0 ** -24 * sc[i // 16] * (q[i] - 32) for i in range(256)])
    assert np.array_equal(oracle.dequant("q6k", b), expect)


def test_q6k_packer_matches_hand_bytes():
    f = read_fixture("q6k_block.txt")
    ql, qh = synth.pack_q6k_codes([((97 * i) % 251) % 64 for i in range(256)])
    assert bytes(ql) == hexbytes(f["ql"]) and bytes(qh) == hexbytes(f["qh"])


def _q4_0_fixture():
    f = read_fixture("q4_0_block.txt")
    blk = hexbytes(f["d"]) + hexbytes(f["qs"])
    assert len(blk) == 18
    q = [(5 * j + 3 * (j // 16)) % 16 for j in range(32)]
    return np.frombuffer(blk, dtype=np.uint8), np.array([0.5 * (v - 8) for v in q])


def _q5k_fixture():
    f = read_fixture("q5k_block.txt")
    blk = hexbytes(f["d"]) + hexbytes(f["dmin"]) + hexbytes(f["scales"]) + hexbytes(f["qh"]) + hexbytes(f["qs"])
    assert len(blk) == 176
    sc = [int(v) for v in f["sc"]]
    m = [int(v) for v in f["m"]]
    q = [((97 * i) % 251) % 32 for i in range(256)]
    expect = np.array([1.0 * sc[i // 32] * q[i] - 0.5 * m[i // 32] for i in range(256)])
    return np.frombuffer(blk, dtype=np.uint8), sc, m, q, expect


def test_q4_0_hand_block_and_one_hot_columns():
    blk, expect = _q4_0_fixture()
    assert np.array_equal(oracle.dequant("q4_0", blk), expect)
    for c in range(32):  # nibble order: weight j low nibble, j + 16 high nibble of byte j
        x = np.zeros(32, dtype=np.float32)
        x[c] = 1.0
        assert oracle.matvec("q4_0", blk, x, 1, 32)[0] == expect[c]


def test_q4_0_subnormal_scale_and_zero_code_offset():
    blk, expect = _q4_0_fixture()
    b = blk.copy()
    b[0:2] = [0x03, 0x80]  # d = -3 * 2^-24
    assert np.array_equal(oracle.dequant("q4_0", b), expect / 0.5 * (-3 * 2.0 ** -24))
    b[2:] = 0x88           # every code 8: every weight exactly 0
    assert np.all(oracle.dequant("q4_0", b) == 0.0)


def test_q5k_hand_block_and_one_hot_columns():
    blk, _, _, _, expect = _q5k_fixture()
    assert np.array_equal(oracle.dequant("q5k", blk), expect)
    for c in range(0, 256, 3):
        x = np.zeros(256, dtype=np.float32)
        x[c] = 1.0
        assert oracle.matvec("q5k", blk, x, 1, 256)[0] == expect[c]


def test_q5k_high_bit_and_subnormal_scales():
    blk, sc, m, q, _ = _q5k_fixture()
    b = blk.copy()
    b[16:48] = 0           # clear every bit 4: codes reduce to their low nibbles
    expect = np.array([1.0 * sc[i // 32] * (q[i] & 15) - 0.5 * m[i // 32] for i in range(256)])
    assert np.array_equal(oracle.dequant("q5k", b), expect)
    b = blk.copy()
    b[0:2] = [0x01, 0x00]  # d = 2^-24
    b[2:4] = [0xFF, 0x03]  # dmin = 1023 * 2^-24
    expect = np.array([2.0 ** -24 * sc[i // 32] * q[i] - 1023 * 2.0 ** -24 * m[i // 32] for i in range(256)])
    assert np.array_equal(oracle.dequant("q5k", b), expect)


def test_q4_0_q5k_encoder_roundtrip_bound():
    n, k = 32, 1024
    wf = synth.weight_matrix_f32(8, n, k).astype(np.float64)
    # Q4_0: 16 levels d*(q-8) with d = -(largest weight)/8 -- the step is
    # about 1/8 and the far end of the range is one step short (codes -8..7),
    # so the max error is about one step; Q5_K: 32 levels over a sub-block's
    # range, half a step of about 2/31 plus the 6-bit scale rounding.
    for fmt, f, lim in (("q4_0", synth.FMT_Q4_0, 0.13), ("q5k", synth.FMT_Q5K, 0.05)):
        wd = oracle.dequant(fmt, synth.weights(f, 8, n, k)).reshape(n, k)
        err = np.abs(wd - wf)
        assert err.max() < lim, (fmt, err.max())
        rel = np.sqrt((err ** 2).mean() / (wf ** 2).mean())
        assert rel < (0.07 if fmt == "q4_0" else 0.035), (fmt, rel)


def test_q8_0_hand_block():
    blk, q = _q8_0_fixture()
    assert np.array_equal(oracle.dequant("q8_0", blk), q)
    b = blk.copy()
    b[0:2] = [0x00, 0xB8]      # d = -0.5
    assert np.array_equal(oracle.dequant("q8_0", b), -0.5 * q)


def test_block_order_within_rows():
    """Block b of row r sits at byte (r*nb + b)*size: decode of a 2x2-block matrix."""
    b0, _, _, _, e0 = _q4k_fixture()
    b1 = b0.copy()
    b1[0:2] = [0x00, 0x40]     # d = 2.0 -> scale part doubles
    e1 = e0 + np.array([1.0 * [1, 2, 33, 63, 40, 17, 5, 50][j] * (((32 * j + l) * 97 % 251) % 16)
                        for j in range(8) for l in range(32)])
    w = np.concatenate([b0, b1, b1, b0])
    x = np.arange(512, dtype=np.float32) % 7 - 3
    y = oracle.matvec("q4k", w, x, 2, 512)
    xd = x.astype(np.float64)
    assert y[0] == np.dot(np.concatenate([e0, e1]), xd)
    assert y[1] == np.dot(np.concatenate([e1, e0]), xd)


# ---------------------------------------------------------------------------
# O3: matvec, exact integer closed form and independent numpy products
# ---------------------------------------------------------------------------
def test_matvec_q8_0_integer_exact():
    rng = np.random.default_rng(5)
    n, k = 37, 96
    q = rng.integers(-127, 128, size=(n, k))
    blocks = np.zeros((n, k // 32, 34), dtype=np.uint8)
    blocks[:, :, 0:2] = [0x00, 0x3C]
    blocks[:, :, 2:] = (q.reshape(n, k // 32, 32) & 0xFF).astype(np.uint8)
    x = rng.integers(-20, 21, size=k)
    y = oracle.matvec("q8_0", blocks, x.astype(np.float32), n, k)
    assert np.array_equal(y, (q @ x).astype(np.float64))


@pytest.mark.parametrize("fmt", ["q8_0", "q4k", "q6k", "q4_0", "q5k"])
def test_matvec_vs_numpy_f64_on_random_blocks(fmt):
    f = synth.FMT_NAMES[fmt]
    n, k = 19, 512
    w = synth.random_blocks(f, 77, n * k // synth.BLOCK_WEIGHTS[f], subnormal_every=5)
    x = synth.normal(78, k)
    wd = oracle.dequant(fmt, w).reshape(n, k)
    ref = wd @ x.astype(np.float64)
    got = oracle.matvec(fmt, w, x, n, k)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    rows = np.array([18, 0, 7])
    np.testing.assert_array_equal(oracle.matvec(fmt, w, x, n, k, rows=rows), got[rows])


# ---------------------------------------------------------------------------
# O4: activation quantizer
# ---------------------------------------------------------------------------
def test_quantize_act_half_away_rounding_and_exact_scale():
    # amax = 127 -> inv = 1.0 exactly, xs = 1.0; x*inv == x, so the code is
    # round-half-away-from-zero of x itself.
    x = np.zeros(32, dtype=np.float32)
    x[:10] = [127, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 3.49, -3.51, 126.5]
    xq, xs, xsum = oracle.quantize_act_q8(x, 1, 32)
    assert list(xq[0, :10]) == [127, 3, -3, 1, -1, 2, -2, 3, -4, 127]
    assert xs[0, 0] == 1.0
    assert xsum[0, 0] == float(xq.astype(np.int64).sum())


# Blocks whose codes depend on taking x*inv as ONE f32 product (the reading
# of the quantizer: inv = 127/amax correctly rounded to f32, then the
# product rounded to f32, then rounded half away from zero). In each case
# below the exact product of the two f32 numbers lies just below k + 1/2
# while its f32 rounding is exactly k + 1/2, so the f32 reading gives k + 1
# and an exact (or f64) product gives k. The amax = 0.3 block also tells the
# f32 product from the real quotient 127*x/amax, and the amax = 0.7 block from
# dividing by the scale, x/xs, whose f32 result falls below the half.
_O4_F32_PRODUCT_BLOCKS = [
    # amax = 3.0: inv = f32(127/amax) = 0x42295555 (42.33333206176758), xs = 0x3cc18306
    #   x = 0x3d71e3c8: exact x*inv = 21990232506669/8796093022208 = 2.4999999944462843, f32 product = 2.5 -> 3
    #   x = 0x3dd9b367: exact x*inv = 158329671828531/35184372088832 = 4.499999926921731, f32 product = 4.5 -> 5
    #   x = 0x3e1d3a75: exact x*inv = 114349206815193/17592186044416 = 6.499999859397178, f32 product = 6.5 -> 7
    #   x = 0x3e356ad6: exact x*inv = 65970697520007/8796093022208 = 7.499999983338853, f32 product = 7.5 -> 8
    #   x = 0xbd71e3c8, 0xbdd9b367, 0xbe1d3a75: the negatives of the first three -> -3, -5, -7
    ([0x40400000, 0x3d71e3c8, 0x3dd9b367, 0x3e1d3a75, 0x3e356ad6, 0xbd71e3c8, 0xbdd9b367, 0xbe1d3a75],
     [127, 3, 5, 7, 8, -3, -5, -7], 0x3cc18306),
    # amax = 0.3 (0x3e99999a): inv = 0x43d3aaaa (423.33331298828125), xs = 0x3b1acf38
    #   x = 0x3c2e291f: exact x*inv = 79164833100363/17592186044416 = 4.499999766969893, f32 product = 4.5 -> 5
    #   x = 0x3ca47c2c: exact x*inv = 18691697571239/2199023255552 = 8.49999995409189, f32 product = 8.5 -> 9
    #   x = 0x3cb7d613: exact x*inv = 83562882851663/8796093022208 = 9.499999902307422, f32 product = 9.5 -> 10
    #   x = 0x3ccb2ffa: exact x*inv = 46179487709185/4398046511104 = 10.499999850522954, f32 product = 10.5 -> 11
    #   x = 0xbc2e291f, 0xbca47c2c, 0xbcb7d613: the negatives of the first three -> -5, -9, -10
    ([0x3e99999a, 0x3c2e291f, 0x3ca47c2c, 0x3cb7d613, 0x3ccb2ffa, 0xbc2e291f, 0xbca47c2c, 0xbcb7d613],
     [127, 5, 9, 10, 11, -5, -9, -10], 0x3b1acf38),
    # amax = 0.7 (0x3f333333): inv = 0x43356db7 (181.42857360839844), xs = 0x3bb49c6c
    #   x = 0x3d3fe632: exact x*inv = 74766786849759/8796093022208 = 8.499999563555207, f32 product = 8.5 -> 9
    #                   (x/xs in f32 = 8.499999046325684 -> 8)
    #   x = 0x3d6d0d4d: exact x*inv = 184717946080011/17592186044416 = 10.499999580134215, f32 product = 10.5 -> 11
    #   x = 0xbd3fe632: the negative of the first -> -9
    ([0x3f333333, 0x3d3fe632, 0x3d6d0d4d, 0xbd3fe632], [127, 9, 11, -9], 0x3bb49c6c),
]


def test_quantize_act_single_f32_product_at_half_way_points():
    x = np.zeros((1, 32 * len(_O4_F32_PRODUCT_BLOCKS)), dtype=np.float32)
    want = np.zeros(x.shape, dtype=np.int8)
    for b, (xbits, codes, _) in enumerate(_O4_F32_PRODUCT_BLOCKS):
        x[0, 32 * b:32 * b + len(xbits)] = np.array(xbits, dtype=np.uint32).view(np.float32)
        want[0, 32 * b:32 * b + len(codes)] = codes
    xq, xs, xsum = oracle.quantize_act_q8(x, 1, x.shape[1])
    np.testing.assert_array_equal(xq, want)
    assert [int(v) for v in xs.reshape(-1).view(np.uint32)] == [c[2] for c in _O4_F32_PRODUCT_BLOCKS]
    sums = want.reshape(-1, 32).astype(np.int64).sum(axis=1)
    np.testing.assert_array_equal(xsum.reshape(-1), xs.reshape(-1) * sums.astype(np.float32))


def test_quantize_act_zero_block_and_invariants():
    x = synth.normal(9, 4 * 256).reshape(4, 256)
    x[1, 32:64] = 0.0
    xq, xs, xsum = oracle.quantize_act_q8(x, 4, 256)
    assert xs[1, 1] == 1.0 and xsum[1, 1] == 0.0 and not xq[1, 32:64].any()
    assert np.abs(xq.astype(np.int32)).max() <= 127
    xb = x.reshape(-1, 32)
    qb = xq.reshape(-1, 32).astype(np.int64)
    sb = xs.reshape(-1)
    for b in range(xb.shape[0]):
        amax = np.float32(np.abs(xb[b]).max())
        if amax == 0:
            continue
        # scale is the correctly rounded f32 quotient amax/127
        assert sb[b] == np.float32(amax) / np.float32(127.0)
        # the extreme element maps to +-127
        i = int(np.abs(xb[b]).argmax())
        assert qb[b, i] == (127 if xb[b, i] > 0 else -127)
        # dequantization error within half a step (plus f32 slack)
        err = np.abs(xb[b].astype(np.float64) - sb[b] * qb[b])
        assert err.max() <= 0.5 * sb[b] * (1 + 1e-5)
    # dequantized block sum is xs times the integer code sum, one f32 multiply
    np.testing.assert_array_equal(xsum.reshape(-1),
                                  (sb * qb.sum(axis=1).astype(np.float32)).astype(np.float32))


# ---------------------------------------------------------------------------
# O5 / O6: integer block sums and the q8-activation matvec
# ---------------------------------------------------------------------------
def test_blocksums_brute_force_on_hand_block():
    blk, sc, m, q, _ = _q4k_fixture()
    rng = np.random.default_rng(11)
    xq = rng.integers(-127, 128, size=256).astype(np.int8)
    S = oracle.blocksums_q4k_q8(blk, xq, 1, 256)
    want = [sum(q[j][l] * int(xq[32 * j + l]) for l in range(32)) for j in range(8)]
    assert list(S[0]) == want
    for c in (0, 31, 32, 100, 255):
        one = np.zeros(256, dtype=np.int8)
        one[c] = 1
        assert oracle.blocksums_q4k_q8(blk, one, 1, 256)[0, c // 32] == q[c // 32][c % 32]


def test_q8act_matvec_equals_blocksum_algebra():
    """sum_b (d*sc*xs*S_b - dmin*m*xs*X_b) == W_deq . x_deq on the hand block."""
    blk, sc, m, q, _ = _q4k_fixture()
    x = synth.normal(12, 256)
    xq, xs, _ = oracle.quantize_act_q8(x, 1, 256)
    S = oracle.blocksums_q4k_q8(blk, xq, 1, 256)[0]
    X = xq.reshape(8, 32).astype(np.int64).sum(axis=1)
    alg = sum(1.0 * sc[j] * float(xs[0, j]) * S[j] - 0.5 * m[j] * float(xs[0, j]) * X[j]
              for j in range(8))
    y = oracle.matvec_q8act("q4k", blk, xq, xs, 1, 256)[0]
    assert abs(y - alg) <= 1e-12 * max(1.0, abs(alg))


def test_q8act_matvec_with_unit_scale_is_integer_matvec():
    # amax = 127 in every block -> xs = 1 and x_deq = xq exactly
    n, k = 9, 512
    w = synth.random_blocks(synth.FMT_Q6K, 3, n * k // 256)
    x = np.round(synth.uniform(4, k) * 100).astype(np.float32)
    x[::32] = 127.0
    xq, xs, _ = oracle.quantize_act_q8(x, 1, k)
    assert np.all(xs == 1.0) and np.array_equal(xq[0].astype(np.float32), x)
    np.testing.assert_array_equal(oracle.matvec_q8act("q6k", w, xq, xs, n, k),
                                  oracle.matvec("q6k", w, x, n, k))


# ---------------------------------------------------------------------------
# O7: router
# ---------------------------------------------------------------------------
def test_route_brute_force_tiny():
    rng = np.random.default_rng(3)
    E, topk = 8, 2
    for _ in range(50):
        lg = rng.integers(-3, 4, size=E).astype(np.float32)  # many ties
        ids, w = oracle.moe_route(lg, 1, E, topk)
        # brute force over ordered pairs: the best pair is the lexicographic
        # maximum of ((l_a, -a), (l_b, -b)) with a ranked before b
        best = max(itertools.permutations(range(E), topk),
                   key=lambda p: [(float(lg[i]), -i) for i in p])
        assert tuple(ids[0]) == best
        p = np.exp(lg[list(best)].astype(np.float64) - lg[best[0]])
        np.testing.assert_allclose(w[0], p / p.sum(), rtol=1e-15)


def test_route_full_topk_is_softmax_and_invariants():
    T, E = 6, 128
    lg = synth.normal(3, T * E).reshape(T, E)
    ids, w = oracle.moe_route(lg, T, E, E)
    for t in range(T):
        sm = scipy.special.softmax(lg[t].astype(np.float64))
        np.testing.assert_allclose(w[t], sm[ids[t]], rtol=1e-13)
    ids8, w8 = oracle.moe_route(lg, T, E, 8)
    import torch
    tv, ti = torch.topk(torch.from_numpy(lg), 8, dim=1)
    assert np.array_equal(ids8, ti.numpy().astype(np.int32))  # tie-free data
    np.testing.assert_allclose(w8.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(np.diff(w8, axis=1) <= 0)
    assert all(len(set(r)) == 8 for r in ids8)


def test_route_ties_and_nan():
    E = 16
    lg = np.zeros(E, dtype=np.float32)
    ids, w = oracle.moe_route(lg, 1, E, 4)
    assert list(ids[0]) == [0, 1, 2, 3] and np.allclose(w, 0.25)
    lg = np.full(E, np.nan, dtype=np.float32)
    lg[9] = -1.0
    lg[3] = 2.0
    ids, w = oracle.moe_route(lg, 1, E, 3)
    assert list(ids[0]) == [3, 9, 0]          # NaN ranks as -inf, ties by index
    assert w[0, 2] == 0.0 and abs(w[0].sum() - 1) < 1e-15


# ---------------------------------------------------------------------------
# Router gate GEMV (logits = Wr . x per token) and gate + route
# ---------------------------------------------------------------------------
def test_gemv_integer_exact_non_square():
    # small integers: every product and partial sum is exact in f64, so the
    # oracle must equal the int64 matrix product exactly; E != hidden != T
    # makes a transposed operand or a swapped index fail
    rng = np.random.default_rng(41)
    T, E, hidden = 3, 5, 12
    W = rng.integers(-7, 8, size=(E, hidden))
    X = rng.integers(-9, 10, size=(T, hidden))
    lg = oracle.gemv(W.astype(np.float32), X.astype(np.float32), T, E, hidden)
    assert lg.shape == (T, E)
    assert np.array_equal(lg, (X @ W.T).astype(np.float64))


def test_gemv_random_vs_numpy_f64():
    T, E, hidden = 4, 128, 2048
    W = synth.uniform(51, E * hidden).reshape(E, hidden)
    X = synth.normal(52, T * hidden).reshape(T, hidden)
    lg = oracle.gemv(W, X, T, E, hidden)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    np.testing.assert_allclose(lg, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_gate_route_one_hot_rows_select_inputs():
    # row e of Wr picks coordinate perm[e] of x, so logits[t, e] = x[t, perm[e]]
    # exactly and the route must rank those values (brute force over pairs)
    rng = np.random.default_rng(43)
    T, E, hidden, topk = 4, 9, 16, 3
    perm = rng.permutation(hidden)[:E]
    W = np.zeros((E, hidden), dtype=np.float32)
    W[np.arange(E), perm] = 1.0
    X = rng.standard_normal((T, hidden)).astype(np.float32)
    lg, ids, w = oracle.gate_route(W, X, T, E, hidden, topk)
    assert np.array_equal(lg, X[:, perm].astype(np.float64))
    for t in range(T):
        best = max(itertools.permutations(range(E), topk),
                   key=lambda p: [(float(X[t, perm[i]]), -i) for i in p])
        assert tuple(ids[t]) == best
        p = np.exp(X[t, perm[list(best)]].astype(np.float64) - X[t, perm[best[0]]])
        np.testing.assert_allclose(w[t], p / p.sum(), rtol=1e-15)


# ---------------------------------------------------------------------------
# MoE gather matvec and the FFN layer
# ---------------------------------------------------------------------------
def test_moe_qmv_is_per_slot_matvec():
    E, n, k = 5, 7, 512
    bank = synth.weights(synth.FMT_Q4K, 21, E * n, k)
    x = synth.normal(22, 3 * k).reshape(3, k)
    ids = np.array([4, 0, 4, 2, -1, 5], dtype=np.int32)   # last two invalid
    y = oracle.moe_qmv("q4k", bank, x, 2, ids, 6, n, k, E)
    rb = synth.row_bytes(synth.FMT_Q4K, k)
    for s in range(4):
        e = ids[s]
        ref = oracle.matvec("q4k", bank[e * n:(e + 1) * n], x[s // 2], n, k)
        np.testing.assert_array_equal(y[s], ref)
    assert not y[4:].any()
    assert bank.shape[1] == rb


def test_moe_ffn_single_expert_is_dense_swiglu():
    hidden, inter = 512, 256
    gate = synth.weights(synth.FMT_Q4K, 31, inter, hidden)
    up = synth.weights(synth.FMT_Q4K, 32, inter, hidden)
    down = synth.weights(synth.FMT_Q6K, 33, hidden, inter)
    x = synth.normal(34, 2 * hidden).reshape(2, hidden)
    ids = np.zeros((2, 1), dtype=np.int32)
    wts = np.ones((2, 1), dtype=np.float32)
    y, h, d = oracle.moe_ffn(gate, up, down, x, ids, wts, 2, 1, hidden, inter, 1)
    G = oracle.dequant("q4k", gate).reshape(inter, hidden)
    U = oracle.dequant("q4k", up).reshape(inter, hidden)
    D = oracle.dequant("q6k", down).reshape(hidden, inter)
    xd = x.astype(np.float64)
    g = xd @ G.T
    hh = g * scipy.special.expit(g) * (xd @ U.T)
    np.testing.assert_allclose(h, hh, rtol=1e-12, atol=1e-12 * np.abs(hh).max())
    np.testing.assert_allclose(y, hh @ D.T, rtol=1e-11, atol=1e-12 * np.abs(y).max())


def test_moe_ffn_weighted_combine():
    E, hidden, inter, T, topk = 6, 256, 256, 3, 2
    gate = synth.weights(synth.FMT_Q4K, 41, E * inter, hidden)
    up = synth.weights(synth.FMT_Q4K, 42, E * inter, hidden)
    down = synth.weights(synth.FMT_Q6K, 43, E * hidden, inter)
    x = synth.normal(44, T * hidden).reshape(T, hidden)
    ids = np.array([[5, 0], [2, 5], [1, 3]], dtype=np.int32)
    wts = np.array([[0.75, 0.25], [0.5, 0.5], [0.9, 0.1]], dtype=np.float32)
    y, h, d = oracle.moe_ffn(gate, up, down, x, ids, wts, T, topk, hidden, inter, E)
    g = oracle.moe_qmv("q4k", gate, x, topk, ids.reshape(-1), T * topk, inter, hidden, E)
    u = oracle.moe_qmv("q4k", up, x, topk, ids.reshape(-1), T * topk, inter, hidden, E)
    np.testing.assert_allclose(h, g * scipy.special.expit(g) * u, rtol=1e-12,
                               atol=1e-13 * np.abs(h).max())
    for t in range(T):
        ref = sum(float(wts[t, j]) * d[t * topk + j] for j in range(topk))
        np.testing.assert_allclose(y[t], ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())


# ---------------------------------------------------------------------------
# a11 prefill GEMM
# ---------------------------------------------------------------------------
def test_qmm_rows_equal_q8act_matvec_and_numpy():
    m, n, k = 5, 12, 512
    w = synth.weights(synth.FMT_Q4K, 51, n, k)
    x = synth.normal(52, m * k).reshape(m, k)
    xq, xs, _ = oracle.quantize_act_q8(x, m, k)
    Y = oracle.qmm("q4k", w, xq, xs, m, n, k)
    for i in range(m):
        np.testing.assert_array_equal(Y[i], oracle.matvec_q8act("q4k", w, xq[i], xs[i], n, k))
    Wd = oracle.dequant("q4k", w).reshape(n, k)
    Xd = np.repeat(xs, 32, axis=1).astype(np.float64) * xq
    ref = Xd @ Wd.T
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    np.testing.assert_array_equal(oracle.qmm("q4k", w, xq, xs, m, n, k, mrows=[4, 1]), Y[[4, 1]])


def test_moe_qmm_single_expert_is_qmm():
    m, n, k = 6, 10, 512
    w = synth.weights(synth.FMT_Q4K, 53, n, k)
    x = synth.normal(54, m * k).reshape(m, k)
    xq, xs, _ = oracle.quantize_act_q8(x, m, k)
    ids = np.zeros(m, dtype=np.int32)
    np.testing.assert_array_equal(oracle.moe_qmm("q4k", w, xq, xs, 1, ids, m, n, k, 1),
                                  oracle.qmm("q4k", w, xq, xs, m, n, k))


@pytest.mark.parametrize("fmt,sfmt", [("q4k", synth.FMT_Q4K), ("q6k", synth.FMT_Q6K)])
def test_moe_qmm_slots_pick_expert_and_activation_row(fmt, sfmt):
    # slot s multiplies expert ids[s]'s slice of the bank by activation row
    # s // x_div; experts outside [0, E) give zero rows; E, n, k, T all differ
    E, n, k, T, x_div = 4, 9, 512, 3, 2
    bank = synth.weights(sfmt, 55, E * n, k)
    x = synth.normal(56, T * k).reshape(T, k)
    xq, xs, _ = oracle.quantize_act_q8(x, T, k)
    ids = np.array([3, 0, -1, 2, 3, 4], dtype=np.int32)
    Y = oracle.moe_qmm(fmt, bank, xq, xs, x_div, ids, ids.size, n, k, E)
    Wd = oracle.dequant(fmt, bank).reshape(E, n, k)
    Xd = np.repeat(xs, 32, axis=1).astype(np.float64) * xq
    for s_, e in enumerate(ids):
        if 0 <= e < E:
            ref = Wd[e] @ Xd[s_ // x_div]
            np.testing.assert_allclose(Y[s_], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
        else:
            assert np.all(Y[s_] == 0.0)
    np.testing.assert_array_equal(oracle.moe_qmm(fmt, bank, xq, xs, x_div, ids, ids.size, n, k, E,
                                                 slots=[4, 0]), Y[[4, 0]])


def test_moe_ffn_q8x_equals_f32_layer_on_exact_dequantized_x():
    # with power-of-two scales xs * xq is exact in f32, so the q8 layer must
    # equal the f32 layer (pinned above) on x = xs * xq, token by token
    E, hidden, inter, T, topk = 5, 512, 256, 4, 3
    gate = synth.weights(synth.FMT_Q4K, 61, E * inter, hidden)
    up = synth.weights(synth.FMT_Q4K, 62, E * inter, hidden)
    down = synth.weights(synth.FMT_Q6K, 63, E * hidden, inter)
    rng = np.random.default_rng(64)
    xq = rng.integers(-127, 128, size=(T, hidden)).astype(np.int8)
    xs = (2.0 ** rng.integers(-9, -4, size=(T, hidden // 32))).astype(np.float32)
    x = (np.repeat(xs, 32, axis=1) * xq).astype(np.float32)
    ids = np.array([[4, 0, 2], [1, -1, 3], [2, 2, 0], [0, 5, 4]], dtype=np.int32)  # repeats, out of range
    wts = rng.random((T, topk)).astype(np.float32)
    y = oracle.moe_ffn_q8x(gate, up, down, xq, xs, ids, wts, T, topk, hidden, inter, E)
    ref, _, _ = oracle.moe_ffn(gate, up, down, x, ids, wts, T, topk, hidden, inter, E)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    np.testing.assert_array_equal(oracle.moe_ffn_q8x(gate, up, down, xq, xs, ids, wts, T, topk, hidden, inter,
                                                     E, toks=[3, 1]), y[[3, 1]])


def test_moe_ffn_q8_is_quantized_swiglu_per_slot():
    # each slot: h from numpy on the decoded expert slices, quantized by the
    # pinned quantizer, then the decoded down slice times the dequantized h;
    # repeats and out-of-range experts included
    E, hidden, inter, T, topk = 4, 512, 256, 3, 3
    gate = synth.weights(synth.FMT_Q4K, 65, E * inter, hidden)
    up = synth.weights(synth.FMT_Q4K, 66, E * inter, hidden)
    down = synth.weights(synth.FMT_Q6K, 67, E * hidden, inter)
    x = synth.normal(68, T * hidden).reshape(T, hidden)
    xq, xs, _ = oracle.quantize_act_q8(x, T, hidden)
    ids = np.array([[3, 0, 3], [1, -1, 2], [0, 4, 2]], dtype=np.int32)
    wts = np.array([[0.5, 0.3, 0.2], [0.6, 0.1, 0.3], [0.25, 0.25, 0.5]], dtype=np.float32)
    y, h, hq, hs = oracle.moe_ffn_q8(gate, up, down, xq, xs, ids, wts, T, topk, hidden, inter, E)
    G = oracle.dequant("q4k", gate).reshape(E, inter, hidden)
    U = oracle.dequant("q4k", up).reshape(E, inter, hidden)
    D = oracle.dequant("q6k", down).reshape(E, hidden, inter)
    Xd = np.repeat(xs, 32, axis=1).astype(np.float64) * xq
    for t in range(T):
        ref = np.zeros(hidden)
        for j in range(topk):
            s_, e = t * topk + j, ids[t, j]
            if not 0 <= e < E:
                assert np.all(h[s_] == 0) and np.all(hq[s_] == 0)
                continue
            g = G[e] @ Xd[t]
            hh = g * scipy.special.expit(g) * (U[e] @ Xd[t])
            np.testing.assert_allclose(h[s_], hh, rtol=1e-12, atol=1e-12 * np.abs(hh).max())
            q, sc, _ = oracle.quantize_act_q8(hh.astype(np.float32), 1, inter)
            assert np.array_equal(hq[s_], q[0]) and np.array_equal(hs[s_], sc[0])
            ref += float(wts[t, j]) * (D[e] @ (np.repeat(sc[0], 32).astype(np.float64) * q[0]))
        np.testing.assert_allclose(y[t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


# ---------------------------------------------------------------------------
# input encoders: round-trip bounds through the pinned decoders
# ---------------------------------------------------------------------------
def test_q8_0_encoder_roundtrip_bound():
    n, k = 64, 1024
    wf = synth.weight_matrix_f32(1, n, k).astype(np.float64)
    wd = oracle.dequant("q8_0", synth.weights(synth.FMT_Q8_0, 1, n, k)).reshape(n, k)
    amax = np.abs(wf.reshape(n, -1, 32)).max(axis=2, keepdims=True)
    d = np.abs(wd.reshape(n, -1, 32)).max(axis=2, keepdims=True) / 127
    err = np.abs(wf.reshape(n, -1, 32) - wd.reshape(n, -1, 32))
    bound = amax / 254 + 127 * np.abs(amax / 127 - d) + 1e-6 * amax
    assert np.all(err <= bound)


def test_q4k_q6k_encoder_roundtrip_bound():
    n, k = 32, 1024
    wf = synth.weight_matrix_f32(7, n, k).astype(np.float64)
    for fmt, f in (("q4k", synth.FMT_Q4K), ("q6k", synth.FMT_Q6K)):
        wd = oracle.dequant(fmt, synth.weights(f, 7, n, k)).reshape(n, k)
        err = np.abs(wd - wf)
        # uniform[-1,1) weights: the code step is about 2/15 (Q4_K, 16 levels
        # over a sub-block's range) or 2/62 (Q6_K), so the max error is half a
        # step plus the 6-bit (Q4_K) / 8-bit (Q6_K) scale rounding, and the RMS
        # error is step/sqrt(12), i.e. 0.0667 / 0.0161 of rms(w) = 1/sqrt(3).
        lim = 0.1 if fmt == "q4k" else 0.03
        assert err.max() < lim, (fmt, err.max())
        rel = np.sqrt((err ** 2).mean() / (wf ** 2).mean())
        assert rel < (0.0667 if fmt == "q4k" else 0.0161) * 1.1, (fmt, rel)
