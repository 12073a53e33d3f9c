"""Pins for the CPU oracle (no GPU).  Each test fixes the oracle to something
other than its own formula: hand-packed bytes with hand-derived values, exact
integer arithmetic, library decoders over every bit pattern, round trips,
closed forms, invariants and planted maxima.  A plausible slip in the oracle
(nibble order, group or sub-block index, a dropped bias/min term, a swapped
scale/min field, gate/up order, softmax over the wrong set, tie order) makes
at least one of them fail.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from bit_quantized_decode_group_amd import synth
from tests import packers

# --------------------------------------------------------------- decoders --


def test_bf16_decoder_matches_torch_on_every_pattern():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f64(int(p)) for p in pats])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(ref[~np.isnan(ref)]))


def test_f16_decoder_matches_numpy_on_every_pattern():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(p)) for p in pats])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    # a few hand values: min subnormal, max subnormal, min normal, max finite
    assert oracle.f16_to_f64(0x0001) == 2.0 ** -24
    assert oracle.f16_to_f64(0x03FF) == 1023 * 2.0 ** -24
    assert oracle.f16_to_f64(0x0400) == 2.0 ** -14
    assert oracle.f16_to_f64(0x7BFF) == 65504.0
    assert oracle.f16_to_f64(0xC000) == -2.0


def test_bf16_rne_encoder_matches_torch():
    g = np.random.default_rng(7)
    vals = np.concatenate([
        g.standard_normal(20000) * 10.0 ** g.integers(-30, 30, 20000),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38, 1e-40, -1e-42, 9.2e-41]),
    ]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f64_to_bf16_rne(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert oracle.f64_to_bf16_rne(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.f64_to_bf16_rne(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.f64_to_bf16_rne(float("inf")) == 0x7F80


# ------------------------------------------------- affine-4 (hand-packed) --

# K = 128 (two groups of 64), two rows.
# Row 0: code of weight k is k % 16  -> words 0x76543210 (k%16 = 0..7), 0xFEDCBA98 (8..15)
#        group 0: scale 0.5 (bf16 0x3F00), bias -2.0 (0xC000)
#        group 1: scale 0.25 (0x3E80),   bias  1.0 (0x3F80)
# Row 1: code of weight k is 15 - k % 16 -> words 0x89ABCDEF, 0x01234567
#        group 0: scale 2.0 (0x4000), bias 0.0 (0x0000)
#        group 1: scale 0.125 (0x3E00), bias -0.5 (0xBF00)
HAND_CODES = np.array([[0x76543210, 0xFEDCBA98] * 8, [0x89ABCDEF, 0x01234567] * 8], dtype=np.uint32)
HAND_SCALES = np.array([[0x3F00, 0x3E80], [0x4000, 0x3E00]], dtype=np.uint16)
HAND_BIASES = np.array([[0xC000, 0x3F80], [0x0000, 0xBF00]], dtype=np.uint16)
# (row, k) -> value worked out by hand from the table above
HAND_VALUES = {
    (0, 0): -2.0, (0, 1): -1.5, (0, 15): 5.5, (0, 16): -2.0, (0, 63): 5.5,
    (0, 64): 1.0, (0, 79): 4.75, (0, 127): 4.75, (0, 70): 2.5,
    (1, 0): 30.0, (1, 7): 16.0, (1, 8): 14.0, (1, 63): 0.0,
    (1, 64): 1.375, (1, 100): 0.875, (1, 127): -0.5,
}


def test_affine4_hand_packed_dequant():
    w = oracle.dequant_affine4(HAND_CODES, HAND_SCALES, HAND_BIASES)
    assert w.shape == (2, 128)
    for (n, k), v in HAND_VALUES.items():
        assert w[n, k] == v, (n, k, w[n, k], v)
    # whole rows from the construction
    k = np.arange(128)
    row0 = np.where(k < 64, 0.5 * (k % 16) - 2.0, 0.25 * (k % 16) + 1.0)
    row1 = np.where(k < 64, 2.0 * (15 - k % 16), 0.125 * (15 - k % 16) - 0.5)
    assert np.array_equal(w[0], row0) and np.array_equal(w[1], row1)
    # row subset
    assert np.array_equal(oracle.dequant_affine4(HAND_CODES, HAND_SCALES, HAND_BIASES, rows=(1, 1))[0], row1)


def test_affine4_one_hot_reads_single_weights():
    ks = [0, 7, 8, 63, 64, 100, 127, 1]
    x = np.zeros((8, 128), dtype=np.uint16)
    for m, k in enumerate(ks):
        x[m, k] = 0x3F80  # 1.0
    y = oracle.qgemv_affine4(x, HAND_CODES, HAND_SCALES, HAND_BIASES)
    assert y.shape == (8, 2)
    for m, k in enumerate(ks):
        for n in range(2):
            exp = HAND_VALUES.get((n, k))
            if exp is not None:
                assert y[m, n] == exp
    # a two-hot row sums two weights: 2*w[.,0] + w[.,64]
    x2 = np.zeros((1, 128), dtype=np.uint16)
    x2[0, 0] = 0x4000
    x2[0, 64] = 0x3F80
    y2 = oracle.qgemv_affine4(x2, HAND_CODES, HAND_SCALES, HAND_BIASES)
    assert y2[0, 0] == 2 * -2.0 + 1.0 and y2[0, 1] == 2 * 30.0 + 1.375


# ---------------------------------------------------- Q4_K (hand-packed) --
# One block: d = 1.0 (fp16 0x3C00), dmin = 0.5 (0x3800)
#   sc = [1, 2, 3, 4, 17, 33, 49, 63], m = [5, 6, 7, 8, 20, 40, 60, 10]
#   scale bytes, derived by hand:
#     s[0..3]  = sc_j | (sc_{j+4} >> 4) << 6 = 0x41 0x82 0xC3 0xC4
#     s[4..7]  = m_j  | (m_{j+4}  >> 4) << 6 = 0x45 0x86 0xC7 0x08
#     s[8..11] = (sc_{j+4} & 15) | (m_{j+4} & 15) << 4 = 0x41 0x81 0xC1 0xAF
#   code byte 32c + l = (l % 16) | (15 - l % 16) << 4 for c = 0..3, l = 0..31
Q4K_HAND = np.zeros(144, dtype=np.uint8)
Q4K_HAND[0:4] = [0x00, 0x3C, 0x00, 0x38]
Q4K_HAND[4:16] = [0x41, 0x82, 0xC3, 0xC4, 0x45, 0x86, 0xC7, 0x08, 0x41, 0x81, 0xC1, 0xAF]
for _c in range(4):
    for _l in range(32):
        Q4K_HAND[16 + 32 * _c + _l] = (_l % 16) | ((15 - _l % 16) << 4)
# weight o -> value, worked out by hand (w = d*sc_j*q - dmin*m_j, j = o // 32)
Q4K_HAND_VALUES = {
    0: -2.5,      # j0, low nibble of byte 0: q 0 -> 0 - 0.5*5
    1: -1.5,      # j0, q 1
    31: 12.5,     # j0, q 15
    32: 27.0,     # j1, high nibble of byte 0: q 15 -> 2*15 - 0.5*6
    33: 25.0,     # j1, q 14
    63: -3.0,     # j1, high nibble of byte 31: q 0
    64: -3.5,     # j2, q 0 -> -0.5*7
    100: 40.0,    # j3, high nibble of byte 32+4: q 11 -> 4*11 - 0.5*8
    130: 24.0,    # j4, q 2 -> 17*2 - 0.5*20
    170: 145.0,   # j5, high nibble of byte 64+10: q 5 -> 33*5 - 0.5*40
    200: 362.0,   # j6, q 8 -> 49*8 - 0.5*60
    240: 940.0,   # j7, high nibble of byte 96+16: q 15 -> 63*15 - 0.5*10
    255: -5.0,    # j7, q 0
}


def test_q4k_hand_packed_dequant():
    w = oracle.dequant_q4k(Q4K_HAND.reshape(1, 1, 144))
    assert w.shape == (1, 256)
    for o, v in Q4K_HAND_VALUES.items():
        assert w[0, o] == v, (o, w[0, o], v)


def test_q4k_hand_block_matches_test_packer():
    # the test-side packer reproduces the hand-written bytes (pins the packer too)
    q = np.zeros(256, dtype=np.int64)
    for c in range(4):
        for l in range(32):
            q[64 * c + l] = l % 16
            q[64 * c + 32 + l] = 15 - l % 16
    blk = packers.q4k_block(np.uint16(0x3C00), np.uint16(0x3800),
                            [1, 2, 3, 4, 17, 33, 49, 63], [5, 6, 7, 8, 20, 40, 60, 10], q)
    assert np.array_equal(blk, Q4K_HAND)


def test_q4k_one_hot_through_qgemv():
    ks = [0, 32, 100, 130, 170, 200, 240, 255]
    x = np.zeros((8, 256), dtype=np.uint16)
    for m, k in enumerate(ks):
        x[m, k] = 0x3F80
    y = oracle.qgemv_q4k(x, Q4K_HAND.reshape(1, 1, 144))
    for m, k in enumerate(ks):
        assert y[m, 0] == Q4K_HAND_VALUES[k]


def test_q4k_six_bit_fields_exhaustive():
    """All 64 values in all 8 scale slots and all 8 min slots decode back."""
    rows = 64
    r = np.arange(rows)[:, None]
    j = np.arange(8)[None, :]
    sc = (r + 11 * j) % 64
    m = (5 * r + 3 * j + 1) % 64
    q = np.ones((rows, 256), dtype=np.int64)
    # d = 1, dmin = 0 -> w = sc_j ; d = 0, dmin = 1 -> w = -m_j
    b1 = packers.q4k_block(np.full(rows, 0x3C00, np.uint16), np.zeros(rows, np.uint16), sc, m, q)
    b2 = packers.q4k_block(np.zeros(rows, np.uint16), np.full(rows, 0x3C00, np.uint16), sc, m, q)
    w1 = oracle.dequant_q4k(b1.reshape(rows, 1, 144))
    w2 = oracle.dequant_q4k(b2.reshape(rows, 1, 144))
    for jj in range(8):
        assert np.array_equal(w1[:, 32 * jj: 32 * jj + 32], np.repeat(sc[:, jj:jj + 1], 32, 1).astype(float))
        assert np.array_equal(w2[:, 32 * jj: 32 * jj + 32], -np.repeat(m[:, jj:jj + 1], 32, 1).astype(float))
    for jj in range(8):
        assert sorted(set(sc[:, jj])) == list(range(64)) and sorted(set(m[:, jj])) == list(range(64))


def test_q4k_fp16_super_scales_subnormal_and_negative():
    q = np.full(256, 3)
    blk = packers.q4k_block(np.uint16(0x0001), np.uint16(0xC000), [1] * 8, [2] * 8, q)  # d = 2^-24, dmin = -2
    w = oracle.dequant_q4k(blk.reshape(1, 1, 144))
    assert np.all(w == 2.0 ** -24 * 3 + 4.0)


# ------------------------------------------------------- exact integers --


def _bf16_of_small_ints(a):
    out = np.array([oracle.f64_to_bf16_rne(float(v)) for v in np.asarray(a).reshape(-1)], dtype=np.uint16)
    return out.reshape(np.shape(a))


@pytest.mark.parametrize("M,N,K", [(1, 5, 256), (8, 7, 1024), (3, 16, 4096)])
def test_affine4_exact_integer_arithmetic(M, N, K):
    g = np.random.default_rng(100 + M)
    q = g.integers(0, 16, (N, K))
    s_int = g.choice([1, 2, 4], size=(N, K // 64))
    b_int = g.integers(-8, 9, (N, K // 64))
    x_int = g.integers(-64, 65, (M, K))
    codes = packers.pack_affine4_codes(q)
    y = oracle.qgemv_affine4(_bf16_of_small_ints(x_int), codes, _bf16_of_small_ints(s_int), _bf16_of_small_ints(b_int))
    w_int = s_int.repeat(64, axis=1) * q + b_int.repeat(64, axis=1)
    exact = x_int.astype(np.int64) @ w_int.astype(np.int64).T
    assert np.array_equal(y, exact.astype(np.float64))


def test_q4k_exact_integer_arithmetic():
    g = np.random.default_rng(5)
    N, nb, M = 6, 3, 4
    sc = g.integers(0, 64, (N, nb, 8))
    mn = g.integers(0, 64, (N, nb, 8))
    q = g.integers(0, 16, (N, nb, 256))
    blocks = packers.q4k_block(np.full((N, nb), 0x4000, np.uint16), np.full((N, nb), 0x3C00, np.uint16), sc, mn, q)
    x_int = g.integers(-32, 33, (M, nb * 256))
    y = oracle.qgemv_q4k(_bf16_of_small_ints(x_int), blocks)
    w_int = (2 * sc.repeat(32, axis=2) * q - mn.repeat(32, axis=2)).reshape(N, nb * 256)
    exact = x_int.astype(np.int64) @ w_int.astype(np.int64).T
    assert np.array_equal(y, exact.astype(np.float64))


# ----------------------------------------------------------- round trips --


def test_affine4_requant_recovers_codes():
    g = np.random.default_rng(11)
    N, K = 9, 512
    q = g.integers(0, 16, (N, K))
    sc = synth.uniform_bf16(g, 0.005, 0.02, (N, K // 64))
    bi = synth.uniform_bf16(g, -0.1, 0.1, (N, K // 64))
    w = oracle.dequant_affine4(packers.pack_affine4_codes(q), sc, bi)
    s = np.array([oracle.bf16_to_f64(v) for v in sc.reshape(-1)]).reshape(sc.shape).repeat(64, axis=1)
    b = np.array([oracle.bf16_to_f64(v) for v in bi.reshape(-1)]).reshape(bi.shape).repeat(64, axis=1)
    assert np.array_equal(np.rint((w - b) / s).astype(np.int64), q)


def test_affine4_minmax_requant_is_exact():
    g = np.random.default_rng(12)
    N, K = 4, 256
    q = g.integers(0, 16, (N, K))
    q[:, ::64] = 0
    q[:, 1::64] = 15  # every group holds both extreme codes
    sc = synth.uniform_bf16(g, 0.005, 0.02, (N, K // 64))
    bi = synth.uniform_bf16(g, -0.1, 0.1, (N, K // 64))
    w = oracle.dequant_affine4(packers.pack_affine4_codes(q), sc, bi).reshape(N, K // 64, 64)
    lo, hi = w.min(axis=2), w.max(axis=2)
    s_rt, b_rt = (hi - lo) / 15.0, lo
    s = np.array([oracle.bf16_to_f64(v) for v in sc.reshape(-1)]).reshape(sc.shape)
    b = np.array([oracle.bf16_to_f64(v) for v in bi.reshape(-1)]).reshape(bi.shape)
    assert np.array_equal(s_rt, s) and np.array_equal(b_rt, b)


def test_q4k_requant_recovers_codes():
    g = np.random.default_rng(13)
    N, nb = 5, 2
    sc = g.integers(1, 64, (N, nb, 8))
    mn = g.integers(0, 64, (N, nb, 8))
    q = g.integers(0, 16, (N, nb, 256))
    d = synth.to_f16_bits(g.uniform(1e-3, 1e-2, (N, nb)))
    dm = synth.to_f16_bits(g.uniform(1e-3, 1e-2, (N, nb)))
    w = oracle.dequant_q4k(packers.q4k_block(d, dm, sc, mn, q)).reshape(N, nb, 256)
    dd = np.array([oracle.f16_to_f64(v) for v in d.reshape(-1)]).reshape(N, nb, 1)
    ddm = np.array([oracle.f16_to_f64(v) for v in dm.reshape(-1)]).reshape(N, nb, 1)
    rq = np.rint((w + ddm * mn.repeat(32, axis=2)) / (dd * sc.repeat(32, axis=2))).astype(np.int64)
    assert np.array_equal(rq, q)


def test_affine4_packed_words_round_trip_through_oracle():
    g = np.random.default_rng(14)
    words = g.integers(0, 2**32, (3, 16), dtype=np.uint64).astype(np.uint32)
    ones = np.full((3, 2), 0x3F80, np.uint16)
    zeros = np.zeros((3, 2), np.uint16)
    q = oracle.dequant_affine4(words, ones, zeros).astype(np.int64)
    assert np.array_equal(packers.pack_affine4_codes(q), words)


# ------------------------------------------------- brute force (small) --


def _bf16_bits_to_f64(a):
    return (np.asarray(a, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("N", [1, 2, 15, 16])
def test_affine4_brute_force_small(M, N):
    d = synth.single_projection(M=M, N=N, K=64, seed=2000 + 17 * M + N)
    y = oracle.qgemv_affine4(d["x"], d["codes"], d["scales"], d["biases"])
    q = (d["codes"].astype(np.uint64)[:, :, None] >> (4 * np.arange(8, dtype=np.uint64))) & np.uint64(15)
    q = q.reshape(N, 64).astype(np.float64)
    w = q * _bf16_bits_to_f64(d["scales"]) + _bf16_bits_to_f64(d["biases"])
    x = _bf16_bits_to_f64(d["x"])
    ref = np.zeros((M, N))
    for k in reversed(range(64)):  # reverse order summation, independent loop
        ref += np.outer(x[:, k], w[:, k])
    rms = math.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(y - ref)) <= 1e-12 * rms


# ---------------------------------------------------- RMSNorm / SwiGLU --


def test_rmsnorm_closed_forms():
    K = 256
    g = np.random.default_rng(3)
    gamma = synth.uniform_bf16(g, 0.8, 1.2, (K,))
    gam = _bf16_bits_to_f64(gamma)
    c = 3.0
    x = np.full((1, K), oracle.f64_to_bf16_rne(c), np.uint16)
    xn = oracle.rmsnorm(x, gamma, 1e-6)
    assert np.allclose(xn[0], gam * c / math.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)
    # one-hot a * e_j
    a, j = -5.0, 17
    x = np.zeros((1, K), np.uint16)
    x[0, j] = oracle.f64_to_bf16_rne(a)
    xn = oracle.rmsnorm(x, gamma, 1e-6)
    assert np.count_nonzero(xn) == 1
    assert math.isclose(xn[0, j], gam[j] * a / math.sqrt(a * a / K + 1e-6), rel_tol=1e-15)
    # scale invariance for |alpha| >> sqrt(eps): x and 4x
    xr = synth.normal_bf16(g, (2, K))
    x4 = np.array([[oracle.f64_to_bf16_rne(4 * oracle.bf16_to_f64(v)) for v in row] for row in xr], np.uint16)
    assert np.allclose(oracle.rmsnorm(xr, gamma, 1e-6), oracle.rmsnorm(x4, gamma, 1e-6), rtol=1e-6, atol=0)
    # eps matters for tiny inputs: x = 2^-20 everywhere -> c / sqrt(c^2 + eps)
    t = 2.0 ** -20
    x = np.full((1, K), oracle.f64_to_bf16_rne(t), np.uint16)
    assert np.allclose(oracle.rmsnorm(x, gamma, 1e-6)[0], gam * t / math.sqrt(t * t + 1e-6), rtol=1e-15)


def test_silu_identities():
    assert oracle.silu(0.0) == 0.0
    for gv in [0.1, 0.5, 1.0, 2.0, 7.5, 30.0]:
        assert math.isclose(oracle.silu(gv) - oracle.silu(-gv), gv, rel_tol=1e-15)
        assert math.isclose(oracle.silu(gv), gv / (1 + math.e ** -gv), rel_tol=1e-15)
    assert abs(oracle.silu(40.0) - 40.0) < 1e-15 * 40
    assert abs(oracle.silu(-40.0)) < 1e-15
    assert math.isclose(oracle.silu(1.0), 0.7310585786300049, rel_tol=1e-15)


def test_gateup_order_and_swiglu():
    """Gate rows first, then up; h = silu(gate) * up (not silu(up) * gate)."""
    K, I = 64, 2
    gamma = np.full(K, 0x3F80, np.uint16)
    x = np.zeros((1, K), np.uint16)
    x[0, 5] = 0x3F80  # one-hot 1.0 -> xn = 1/sqrt(1/K + eps) at k = 5
    r = 1.0 / math.sqrt(1.0 / K + 1e-6)
    codes = np.zeros((2 * I, K // 8), np.uint32)
    scales = np.full((2 * I, 1), 0x3F80, np.uint16)
    # constant rows via the bias: gate rows 2.0 and -1.0, up rows 0.5 and 3.0
    biases = np.array([[0x4000], [0xBF80], [0x3F00], [0x4040]], np.uint16)
    h = oracle.rmsnorm_gateup_swiglu(x, gamma, 1e-6, codes, scales, biases)
    gate = np.array([2.0, -1.0]) * r
    up = np.array([0.5, 3.0]) * r
    exp = gate / (1 + np.exp(-gate)) * up
    assert np.allclose(h[0], exp, rtol=1e-14)
    swapped = up / (1 + np.exp(-up)) * gate
    assert not np.allclose(h[0], swapped, rtol=1e-3)


def test_mlp_block_identity_down_reads_h_back():
    """Down rows that are one-hot in h return h itself."""
    D, I = 64, 64
    g = np.random.default_rng(21)
    x = synth.normal_bf16(g, (2, D))
    gamma = synth.uniform_bf16(g, 0.8, 1.2, (D,))
    gu = synth.affine4_matrix(g, 2 * I, D)
    h = oracle.rmsnorm_gateup_swiglu(x, gamma, 1e-6, gu["codes"], gu["scales"], gu["biases"])
    # down row n: code 1 at k = n, 0 elsewhere; scale 1, bias 0 -> y[n] = h[n]
    q = np.eye(D, I, dtype=np.int64)
    codes_d = packers.pack_affine4_codes(q)
    y = oracle.mlp_block(x, gamma, 1e-6, gu["codes"], gu["scales"], gu["biases"], codes_d,
                         np.full((D, I // 64), 0x3F80, np.uint16), np.zeros((D, I // 64), np.uint16))
    assert np.array_equal(y, h)


# ----------------------------------------------------------------- MoE --


def _moe_small(E=8, D=256, I=256, seed=31, n_logit_sets=1):
    return synth.moe_token(E=E, D=D, I=I, top_k=min(8, E), seed=seed, n_logit_sets=n_logit_sets)


def test_moe_top1_equals_dense_mlp_of_argmax_expert():
    d = _moe_small()
    E, D, I = d["E"], d["D"], d["I"]
    logits = d["logits"][0]
    y, ids, p = oracle.moe(d["x"], logits, 1, d["w_gu"], d["w_down"], E, D, I)
    e = int(np.argmax(logits))
    assert ids[0] == e and p[0] == 1.0
    gu = oracle.qgemv_q4k(d["x"], d["w_gu"][e])[0]
    h = np.array([oracle.silu(gv) for gv in gu[:I]]) * gu[I:]
    yd = oracle.qgemv_q4k(np.zeros((1, I), np.uint16), d["w_down"][e])  # shape check only
    assert yd.shape == (1, D)
    wd = oracle.dequant_q4k(d["w_down"][e])
    ref = np.array([sum(h[k] * wd[n, k] for k in range(I)) for n in range(D)])
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_moe_selection_weights_and_permutation_invariance():
    d = _moe_small(E=16, seed=32)
    E, D, I = 16, d["D"], d["I"]
    logits = d["logits"][0]
    y, ids, p = oracle.moe(d["x"], logits, 8, d["w_gu"], d["w_down"], E, D, I)
    order = sorted(range(E), key=lambda e: (-float(logits[e]), e))[:8]
    assert list(ids) == order
    sel = logits[order].astype(np.float64)
    ref_p = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
    assert np.allclose(p, ref_p, rtol=1e-14) and math.isclose(p.sum(), 1.0, rel_tol=1e-14)
    full = np.exp(logits.astype(np.float64) - logits.max()) / np.exp(logits.astype(np.float64) - logits.max()).sum()
    assert not np.allclose(p, full[order])  # not the softmax over all experts
    perm = np.random.default_rng(1).permutation(E)
    y2, ids2, p2 = oracle.moe(d["x"], logits[perm], 8, d["w_gu"][perm], d["w_down"][perm], E, D, I)
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-12 * np.abs(y).max())
    assert list(perm[ids2]) == list(ids)


def test_moe_all_experts_and_tie_order():
    d = _moe_small(E=8, seed=33)
    E, D, I = 8, d["D"], d["I"]
    logits = np.array([0.5, 2.0, 2.0, -1.0, 0.0, 2.0, 1.0, 3.0], np.float32)
    y, ids, p = oracle.moe(d["x"], logits, 3, d["w_gu"], d["w_down"], E, D, I)
    assert list(ids) == [7, 1, 2]  # three-way tie at 2.0 -> lower indices first
    y8, ids8, p8 = oracle.moe(d["x"], logits, 8, d["w_gu"], d["w_down"], E, D, I)
    assert sorted(ids8) == list(range(8)) and math.isclose(p8.sum(), 1.0, rel_tol=1e-14)


def _dense_swiglu_expert(x64, w_gu_e, w_down_e, I):
    """One expert's MLP written out with numpy on the oracle's dequantised
    weights (pinned by the hand-packed Q4_K tests): down . (silu(gate.x) * up.x)."""
    wgu = oracle.dequant_q4k(w_gu_e)
    wd = oracle.dequant_q4k(w_down_e)
    g = wgu[:I] @ x64
    u = wgu[I:] @ x64
    return wd @ (g / (1.0 + np.exp(-g)) * u)


@pytest.mark.parametrize("top_k", [2, 8])
def test_moe_weighted_sum_of_dense_experts(top_k):
    """y = sum over the selected experts of p_e times that expert's dense SwiGLU
    MLP, with p = softmax over the selected logits only (uzu page, section
    "내부 동작 1", mlp row: MixtureOfExperts with a routing function; the
    softmax-weighted top-k sum).  Selection, weights and the per-expert MLPs
    are recomputed here with numpy; an unweighted sum and a full-softmax
    weighting are controls that must fail the same comparison."""
    d = _moe_small(E=16, D=256, I=256, seed=36 + top_k)
    E, D, I = 16, d["D"], d["I"]
    logits = d["logits"][0]
    y, ids, p = oracle.moe(d["x"], logits, top_k, d["w_gu"], d["w_down"], E, D, I)
    lg = logits.astype(np.float64)
    order = sorted(range(E), key=lambda e: (-lg[e], e))[:top_k]
    pe = np.exp(lg[order] - lg[order].max())
    pe /= pe.sum()
    x64 = oracle.bf16_array_to_f64(d["x"]).reshape(-1)
    ye = np.stack([_dense_swiglu_expert(x64, d["w_gu"][e], d["w_down"][e], I) for e in order])
    want = (pe[:, None] * ye).sum(axis=0)
    tol = 1e-12 * np.abs(want).max()

    def agrees(v):
        return float(np.abs(np.asarray(v) - want).max()) <= tol

    assert list(ids) == order
    assert agrees(y), float(np.abs(y - want).max())
    # controls: plausible slips in the weighted sum must not pass this comparison
    assert not agrees(ye.sum(axis=0)), "unweighted sum passed"
    full = np.exp(lg - lg.max())
    full /= full.sum()
    assert not agrees((full[order][:, None] * ye).sum(axis=0)), "full-softmax weights passed"
    assert not agrees((pe[::-1][:, None] * ye).sum(axis=0)), "weights in reverse order passed"


def test_moe_rejects_bad_args():
    d = _moe_small(E=8, seed=34)
    with pytest.raises(ValueError):
        oracle.moe(d["x"], d["logits"][0], 9, d["w_gu"], d["w_down"], 8, d["D"], d["I"])
    with pytest.raises(ValueError):
        oracle.moe(d["x"], d["logits"][0], 0, d["w_gu"], d["w_down"], 8, d["D"], d["I"])


# -------------------------------------------------------- LM head / argmax --


def _lm_bias_rows(V, K, bias_bits):
    codes = np.zeros((V, K // 8), np.uint32)
    scales = np.full((V, K // 64), 0x3F80, np.uint16)
    biases = np.repeat(np.asarray(bias_bits, np.uint16).reshape(V, 1), K // 64, axis=1)
    return codes, scales, biases


def test_lmhead_planted_max_ties_and_nan():
    V, K = 64, 64
    bias = np.full(V, 0x3F00, np.uint16)  # 0.5
    bias[40] = 0x3F80  # 1.0 : unique max
    codes, scales, biases = _lm_bias_rows(V, K, bias)
    x = np.full((1, K), 0x3F80, np.uint16)
    logits, ids, gap, _ = oracle.lmhead(x, codes, scales, biases)
    assert ids[0] == 40 and logits[0, 40] == 64.0 and gap[0] == 32.0
    bias[10] = 0x3F80  # duplicate of the max at a lower index
    codes, scales, biases = _lm_bias_rows(V, K, bias)
    _, ids, gap, _ = oracle.lmhead(x, codes, scales, biases)
    assert ids[0] == 10 and gap[0] == 0.0
    bias[50] = 0x7FC0  # NaN bias -> NaN logit; first NaN wins
    bias[55] = 0x7FC0
    codes, scales, biases = _lm_bias_rows(V, K, bias)
    _, ids, _, _ = oracle.lmhead(x, codes, scales, biases)
    assert ids[0] == 50
    # a negative-row input flips the argmax to the smallest bias
    xn = np.full((1, K), 0xBF80, np.uint16)
    bias2 = np.full(V, 0x3F00, np.uint16)
    bias2[7] = 0x3E80  # 0.25 is the smallest
    codes, scales, biases = _lm_bias_rows(V, K, bias2)
    _, ids, _, _ = oracle.lmhead(xn, codes, scales, biases)
    assert ids[0] == 7


def test_lmhead_accepted_prefix():
    d = synth.lm_head(M=8, V=200, K=128, seed=77)
    _, ids, _, acc = oracle.lmhead(d["x"], d["codes"], d["scales"], d["biases"], draft=None)
    assert acc == 0
    for k in range(0, 9):
        draft = ids.copy()
        if k < 8:
            draft[k] = (ids[k] + 1) % 200
        _, _, _, acc = oracle.lmhead(d["x"], d["codes"], d["scales"], d["biases"], draft=draft)
        assert acc == k
    # logits agree with the plain projection
    logits, _, _, _ = oracle.lmhead(d["x"], d["codes"], d["scales"], d["biases"])
    assert np.array_equal(logits, oracle.qgemv_affine4(d["x"], d["codes"], d["scales"], d["biases"]))


def test_lmhead_topk_planted_order_ties_nan_and_signed_zero():
    V, K = 64, 64
    x = np.full((1, K), 0x3F80, np.uint16)  # ones: logit = 64 * bias
    bias = np.full(V, 0x3F00, np.uint16)  # 0.5
    bias[40] = bias[10] = 0x3F80  # 1.0, tied
    bias[3] = bias[60] = 0x3F40  # 0.75, tied
    bias[20] = 0x3F20  # 0.625
    ids, vals = oracle.lmhead_topk(x, *_lm_bias_rows(V, K, bias), k=6)
    assert ids[0].tolist() == [10, 40, 3, 60, 20, 0]
    assert vals[0].tolist() == [64.0, 64.0, 48.0, 48.0, 40.0, 32.0]
    bias[55] = bias[50] = 0x7FC0  # NaN logits come first, by index
    ids, _ = oracle.lmhead_topk(x, *_lm_bias_rows(V, K, bias), k=3)
    assert ids[0].tolist() == [50, 55, 10]
    neg = np.full(V, 0xBF00, np.uint16)  # -0.5 everywhere ...
    neg[5] = 0x8000  # ... except -0 at 5 and +0 at 2: equal logits, lower index first
    neg[2] = 0x0000
    ids, vals = oracle.lmhead_topk(x, *_lm_bias_rows(V, K, neg), k=3)
    assert ids[0].tolist() == [2, 5, 0] and vals[0, 0] == 0.0 and vals[0, 2] == -32.0


def test_lmhead_topk_matches_a_full_sort():
    d = synth.lm_head(M=3, V=300, K=128, seed=91)
    w = oracle.dequant_affine4(d["codes"], d["scales"], d["biases"])
    xf = torch.from_numpy(d["x"].astype(np.int16)).view(torch.bfloat16).double().numpy()
    logits = xf @ w.T  # numpy's product, not the oracle's ascending-k sum
    for k in (1, 7, 300):
        ids, vals = oracle.lmhead_topk(d["x"], d["codes"], d["scales"], d["biases"], k=k)
        for m in range(3):
            order = np.lexsort((np.arange(300), -logits[m]))[:k]  # larger first, then lower index
            assert ids[m].tolist() == order.tolist()
            np.testing.assert_allclose(vals[m], logits[m, order], rtol=1e-12, atol=1e-12)
    _, am, _, _ = oracle.lmhead(d["x"], d["codes"], d["scales"], d["biases"])
    ids1, _ = oracle.lmhead_topk(d["x"], d["codes"], d["scales"], d["biases"], k=1)
    assert np.array_equal(ids1[:, 0], am)


def test_oracle_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.dequant_affine4(np.zeros((2, 3), np.uint32), np.zeros((2, 1), np.uint16), np.zeros((2, 1), np.uint16))


# ------------------------------------------------------------- O10 / O11 --
# Pins of the input randomised Hadamard transform: scipy's Hadamard matrix
# (an independent construction of the Sylvester matrix), the textbook 2-point
# case, orthonormality (H H^T = n I), the involution without signs, sign
# handling, Parseval, and the projection against the plain O3 on the
# transformed rows.

def _ones_signs(K):
    return np.ones(K, np.int8)


def test_rht_matches_scipy_hadamard_blocks():
    from scipy.linalg import hadamard
    g = np.random.default_rng(501)
    for had, K in ((2, 8), (4, 64), (64, 192), (256, 512)):
        x = synth.normal_bf16(synth.rng(500 + had), (3, K))
        s = g.choice(np.array([-1, 1], np.int8), size=K)
        xr = oracle.rht(x, s, had)
        xf = oracle.bf16_array_to_f64(x.reshape(-1)).reshape(x.shape)
        H = hadamard(had).astype(np.float64) / np.sqrt(had)
        want = np.concatenate([(xf[:, b * had:(b + 1) * had] * s[b * had:(b + 1) * had]) @ H.T
                               for b in range(K // had)], axis=1)
        np.testing.assert_allclose(xr, want, rtol=1e-12, atol=1e-12)


def test_rht_two_point_closed_form_and_unit_vectors():
    x = np.array([[0x4040, 0x3F80]], np.uint16)  # 3.0, 1.0
    xr = oracle.rht(x, np.ones(2, np.int8), 2)
    np.testing.assert_allclose(xr[0], [4.0 / np.sqrt(2), 2.0 / np.sqrt(2)], rtol=0, atol=1e-15)
    had = 16
    eye = np.zeros((had, had), np.uint16)
    eye[np.arange(had), np.arange(had)] = 0x3F80
    cols = oracle.rht(eye, _ones_signs(had), had)  # row i = transform of e_i
    np.testing.assert_allclose(cols @ cols.T, np.eye(had), atol=1e-12)  # orthonormal
    assert set(np.unique(np.round(cols * 4, 12))) == {-1.0, 1.0}  # entries +-1/sqrt(16)


def test_rht_involution_signs_and_parseval():
    K, had = 256, 64
    x = synth.normal_bf16(synth.rng(502), (2, K))
    xf = oracle.bf16_array_to_f64(x.reshape(-1)).reshape(x.shape)
    once = oracle.rht(x, _ones_signs(K), had)
    # the transform of the transform is the identity (H/sqrt(n) is symmetric and orthogonal);
    # apply it to the exact fp64 result via the Sylvester matrix built independently here
    n = had
    H = np.array([[(-1.0) ** bin(i & j).count("1") for j in range(n)] for i in range(n)]) / np.sqrt(n)
    twice = np.concatenate([once[:, b * n:(b + 1) * n] @ H.T for b in range(K // n)], axis=1)
    np.testing.assert_allclose(twice, xf, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(once, axis=1), np.linalg.norm(xf, axis=1), rtol=1e-13)
    s = _ones_signs(K)
    s[[3, 70, 200]] = -1
    neg = x.copy()
    neg[:, [3, 70, 200]] ^= 0x8000  # negating the inputs equals flipping their signs
    np.testing.assert_allclose(oracle.rht(x, s, had), oracle.rht(neg, _ones_signs(K), had), atol=0)


def test_rht_projection_is_plain_projection_of_transformed_rows():
    d = synth.single_projection(M=3, N=20, K=256, seed=503)
    s = np.random.default_rng(504).choice(np.array([-1, 1], np.int8), size=256)
    y = oracle.qgemv_affine4_rht(d["x"], s, 128, d["codes"], d["scales"], d["biases"])
    w = oracle.dequant_affine4(d["codes"], d["scales"], d["biases"])
    np.testing.assert_allclose(y, oracle.rht(d["x"], s, 128) @ w.T, rtol=1e-12, atol=1e-10)
    with pytest.raises(ValueError):
        oracle.rht(d["x"], s, 96)  # not a power of two
    with pytest.raises(ValueError):
        oracle.rht(d["x"], s, 512)  # does not divide K


# ------------------------------------------------- affine-8 (hand-packed) --
# K = 128 (two groups of 64), two rows, codes one byte each, least significant
# byte of a word first.
# Row 0: code of weight k is 2k           -> words 0x06040200, 0x0E0C0A08, ...
#        group 0: scale 0.5, bias -2.0;  group 1: scale 0.25, bias 1.0
# Row 1: code of weight k is 255 - k      -> words 0xFCFDFEFF, 0xF8F9FAFB, ...
#        group 0: scale 2.0, bias 0.0;   group 1: scale 0.125, bias -0.5
HAND8_WORDS = {(0, 0): 0x06040200, (0, 1): 0x0E0C0A08, (0, 31): 0xFEFCFAF8,
               (1, 0): 0xFCFDFEFF, (1, 1): 0xF8F9FAFB, (1, 31): 0x80818283}
HAND8_SCALES = np.array([[0x3F00, 0x3E80], [0x4000, 0x3E00]], dtype=np.uint16)
HAND8_BIASES = np.array([[0xC000, 0x3F80], [0x0000, 0xBF00]], dtype=np.uint16)
HAND8_VALUES = {
    (0, 0): -2.0, (0, 3): 1.0, (0, 63): 61.0, (0, 64): 33.0, (0, 127): 64.5,
    (1, 0): 510.0, (1, 5): 500.0, (1, 63): 384.0, (1, 64): 23.375, (1, 127): 15.5,
}


def _hand8_codes():
    k = np.arange(128)
    return packers.pack_affine8_codes(np.stack([2 * k, 255 - k]))


def test_affine8_hand_packed_words_and_dequant():
    codes = _hand8_codes()
    for (n, j), word in HAND8_WORDS.items():
        assert int(codes[n, j]) == word, (n, j, hex(int(codes[n, j])))
    w = oracle.dequant_affine8(codes, HAND8_SCALES, HAND8_BIASES)
    for (n, k), v in HAND8_VALUES.items():
        assert w[n, k] == v, (n, k, w[n, k], v)
    k = np.arange(128)
    assert np.array_equal(w[0], np.where(k < 64, k - 2.0, k / 2.0 + 1.0))
    assert np.array_equal(w[1], np.where(k < 64, 2.0 * (255 - k), 0.125 * (255 - k) - 0.5))


def test_affine8_one_hot_reads_single_weights():
    ks = [0, 3, 63, 64, 127, 5]
    x = np.zeros((len(ks), 128), dtype=np.uint16)
    for m, k in enumerate(ks):
        x[m, k] = 0x3F80
    y = oracle.qgemv_affine8(x, _hand8_codes(), HAND8_SCALES, HAND8_BIASES)
    for m, k in enumerate(ks):
        for n in range(2):
            if (n, k) in HAND8_VALUES:
                assert y[m, n] == HAND8_VALUES[(n, k)]


def test_affine8_small_codes_equal_affine4():
    """Codes below 16 are the same weights in either format: the two oracles,
    with their own unpackers, must agree exactly."""
    g = np.random.default_rng(21)
    N, K, M = 7, 512, 3
    q = g.integers(0, 16, (N, K))
    sc = synth.uniform_bf16(g, 0.005, 0.02, (N, K // 64))
    bi = synth.uniform_bf16(g, -0.1, 0.1, (N, K // 64))
    x = synth.normal_bf16(g, (M, K))
    y8 = oracle.qgemv_affine8(x, packers.pack_affine8_codes(q), sc, bi)
    y4 = oracle.qgemv_affine4(x, packers.pack_affine4_codes(q), sc, bi)
    assert np.array_equal(y8, y4)


@pytest.mark.parametrize("M,N,K", [(1, 5, 256), (8, 7, 1024)])
def test_affine8_exact_integer_arithmetic(M, N, K):
    g = np.random.default_rng(200 + M)
    q = g.integers(0, 256, (N, K))
    s_int = g.choice([1, 2], size=(N, K // 64))
    b_int = g.integers(-8, 9, (N, K // 64))
    x_int = g.integers(-16, 17, (M, K))  # |partial sums| stay far below 2^53
    y = oracle.qgemv_affine8(_bf16_of_small_ints(x_int), packers.pack_affine8_codes(q), _bf16_of_small_ints(s_int),
                             _bf16_of_small_ints(b_int))
    w_int = s_int.repeat(64, axis=1) * q + b_int.repeat(64, axis=1)
    exact = x_int.astype(np.int64) @ w_int.astype(np.int64).T
    assert np.array_equal(y, exact.astype(np.float64))


def test_affine8_requant_recovers_every_code():
    g = np.random.default_rng(22)
    N, K = 4, 512
    q = np.stack([g.permutation(512) % 256 for _ in range(N)])  # every code 0..255 in every row
    sc = synth.uniform_bf16(g, 0.0003, 0.0012, (N, K // 64))
    bi = synth.uniform_bf16(g, -0.1, 0.1, (N, K // 64))
    w = oracle.dequant_affine8(packers.pack_affine8_codes(q), sc, bi)
    s = _bf16_bits_to_f64(sc).repeat(64, axis=1)
    b = _bf16_bits_to_f64(bi).repeat(64, axis=1)
    assert np.array_equal(np.rint((w - b) / s).astype(np.int64), q)


def test_affine8_packed_words_round_trip_through_oracle():
    g = np.random.default_rng(23)
    words = g.integers(0, 2**32, (3, 32), dtype=np.uint64).astype(np.uint32)
    ones = np.full((3, 2), 0x3F80, np.uint16)
    zeros = np.zeros((3, 2), np.uint16)
    q = oracle.dequant_affine8(words, ones, zeros).astype(np.int64)
    assert q.min() >= 0 and q.max() <= 255
    assert np.array_equal(packers.pack_affine8_codes(q), words)


@pytest.mark.parametrize("M", [1, 8])
@pytest.mark.parametrize("N", [1, 16])
def test_affine8_brute_force_small(M, N):
    d = synth.single_projection8(M=M, N=N, K=64, seed=2100 + M + N)
    y = oracle.qgemv_affine8(d["x"], d["codes"], d["scales"], d["biases"])
    q = d["codes"].view("<u1").reshape(N, 64).astype(np.float64)  # bytes in memory order
    w = q * _bf16_bits_to_f64(d["scales"]) + _bf16_bits_to_f64(d["biases"])
    x = _bf16_bits_to_f64(d["x"])
    ref = np.zeros((M, N))
    for k in reversed(range(64)):
        ref += np.outer(x[:, k], w[:, k])
    assert np.max(np.abs(y - ref)) <= 1e-12 * math.sqrt(np.mean(ref ** 2))


def test_affine8_rejects_bad_shapes():
    codes = np.zeros((2, 16), np.uint32)
    sc = np.zeros((2, 1), np.uint16)
    with pytest.raises(Exception):
        oracle.qgemv_affine8(np.zeros((1, 60), np.uint16), np.zeros((2, 15), np.uint32), sc, sc)
    assert oracle.qgemv_affine8(np.zeros((1, 64), np.uint16), codes, sc, sc).shape == (1, 2)


# ----------------------------------------------------- Q6_K (hand-packed) --
# One block: d = 0.5 (fp16 0x3800); scales (int8) per 16 weights:
#   [1, -1, 2, -2, 3, -3, 4, -4, 127, -128, 5, -5, 6, -6, 7, -7];
# weight o has q = (o % 64) - 32, i.e. stored 6-bit value u = o % 64.
# Bytes worked out by hand from the layout (ql low nibble: quarters 0, 1;
# high nibble: quarters 2, 3; qh bits 2j..2j+1):
#   ql[0] = 0x00, ql[1] = 0x11, ql[33] = 0x11, ql[47] = 0xFF, ql[64] = 0x00
#   qh[0] = 0x88 (u = 0, 32, 0, 32 -> high bits 0, 2, 0, 2), qh[16] = 0xDD, qh[32] = 0x88
Q6K_SCALES = [1, -1, 2, -2, 3, -3, 4, -4, 127, -128, 5, -5, 6, -6, 7, -7]
Q6K_BYTES = {0: 0x00, 1: 0x11, 33: 0x11, 47: 0xFF, 64: 0x00, 128: 0x88, 144: 0xDD, 160: 0x88,
             192: 0x01, 193: 0xFF, 200: 0x7F, 201: 0x80, 208: 0x00, 209: 0x38}
Q6K_VALUES = {0: -16.0, 17: 7.5, 63: -31.0, 130: -1905.0, 150: 640.0, 255: -108.5}


def _q6k_hand():
    o = np.arange(256)
    return packers.q6k_block(np.array([0x3800], np.uint16), np.array([Q6K_SCALES]), (o % 64 - 32)[None])


def test_q6k_hand_packed_bytes_and_values():
    blk = _q6k_hand()
    for i, v in Q6K_BYTES.items():
        assert int(blk[0, i]) == v, (i, hex(int(blk[0, i])), hex(v))
    w = oracle.dequant_q6k(blk.reshape(1, 1, 210))[0]
    for o, v in Q6K_VALUES.items():
        assert w[o] == v, (o, w[o], v)
    o = np.arange(256)
    assert np.array_equal(w, 0.5 * np.array(Q6K_SCALES).repeat(16) * (o % 64 - 32))


def test_q6k_one_hot_through_qgemv():
    blk = _q6k_hand().reshape(1, 1, 210)
    ks = list(Q6K_VALUES)
    x = np.zeros((len(ks), 256), np.uint16)
    for r, k in enumerate(ks):
        x[r, k] = 0x3F80
    y = oracle.qgemv_q6k(x, blk)
    assert [y[r, 0] for r in range(len(ks))] == [Q6K_VALUES[k] for k in ks]


def _q6k_unpack_numpy(blocks):
    """The Q6_K reading restated with numpy over (h, j, l), for comparison with the C oracle."""
    b = blocks.astype(np.int64)
    ql = b[..., 0:128].reshape(b.shape[:-1] + (2, 2, 32))
    qh = b[..., 128:192].reshape(b.shape[:-1] + (2, 32))
    sc = blocks[..., 192:208].view(np.int8).astype(np.float64)
    d = (blocks[..., 208].astype(np.uint16) | (blocks[..., 209].astype(np.uint16) << 8)).view(np.float16)
    u = np.empty(b.shape[:-1] + (2, 4, 32), np.int64)
    for j in range(4):
        nib = (ql[..., j % 2, :] >> (4 * (j // 2))) & 15
        u[..., j, :] = nib | (((qh >> (2 * j)) & 3) << 4)
    q = (u - 32).reshape(b.shape[:-1] + (256,))
    return d.astype(np.float64)[..., None] * sc.repeat(16, axis=-1) * q


def test_q6k_random_blocks_match_numpy_restatement():
    g = np.random.default_rng(31)
    blocks = g.integers(0, 256, (5, 3, 210), dtype=np.uint8)
    d = synth.to_f16_bits(g.uniform(1e-3, 1e-2, (5, 3)))
    blocks[..., 208] = d & 0xFF
    blocks[..., 209] = d >> 8
    assert np.array_equal(oracle.dequant_q6k(blocks), _q6k_unpack_numpy(blocks).reshape(5, 768))


def test_q6k_pack_round_trip_every_code():
    g = np.random.default_rng(32)
    N, nb = 4, 2
    q = np.stack([np.stack([g.permutation(256) % 64 - 32 for _ in range(nb)]) for _ in range(N)])
    sc = g.integers(1, 128, (N, nb, 16)) * g.choice([-1, 1], (N, nb, 16))
    blocks = packers.q6k_block(np.full((N, nb), 0x3C00, np.uint16), sc, q)  # d = 1
    w = oracle.dequant_q6k(blocks).reshape(N, nb, 256)
    assert np.array_equal(np.rint(w / sc.repeat(16, axis=-1)).astype(np.int64), q)


def test_q6k_exact_integer_arithmetic():
    g = np.random.default_rng(33)
    N, nb, M = 5, 2, 3
    q = g.integers(-32, 32, (N, nb, 256))
    sc = g.integers(-8, 9, (N, nb, 16))
    blocks = packers.q6k_block(np.full((N, nb), 0x4000, np.uint16), sc, q)  # d = 2
    x_int = g.integers(-16, 17, (M, nb * 256))
    y = oracle.qgemv_q6k(_bf16_of_small_ints(x_int), blocks)
    w_int = (2 * sc.repeat(16, axis=-1) * q).reshape(N, nb * 256)
    assert np.array_equal(y, (x_int.astype(np.int64) @ w_int.astype(np.int64).T).astype(np.float64))


@pytest.mark.parametrize("M,N", [(1, 1), (8, 5)])
def test_q6k_brute_force_small(M, N):
    g = np.random.default_rng(34 + M + N)
    blocks = g.integers(0, 256, (N, 1, 210), dtype=np.uint8)
    d = synth.to_f16_bits(g.uniform(1e-3, 1e-2, (N, 1)))
    blocks[..., 208] = d & 0xFF
    blocks[..., 209] = d >> 8
    x = synth.normal_bf16(g, (M, 256))
    y = oracle.qgemv_q6k(x, blocks)
    w = _q6k_unpack_numpy(blocks).reshape(N, 256)
    xf = _bf16_bits_to_f64(x)
    ref = np.zeros((M, N))
    for k in reversed(range(256)):
        ref += np.outer(xf[:, k], w[:, k])
    assert np.max(np.abs(y - ref)) <= 1e-12 * math.sqrt(np.mean(ref ** 2))
