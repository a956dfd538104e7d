"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``check_*`` function raises AssertionError on a mismatch.  They are
collected by ``test_oracle_pins.py`` and re-run against copies of the oracle
with planted mistakes by ``test_oracle_mutants.py`` (every planted mistake
must make at least one of them fail).

What the pins rest on (the pages print no worked example, no test vector and
no bit layout; the layout is this library's format definition -- code k of a
row occupies stream bits [k*b, k*b+b), stream bit i is bit i%32 of word i/32,
w = scale*q + min per group of K):
  * numpy's own float16 -> float64 conversion (library routine);
  * numpy ``unpackbits`` / ``packbits`` with little bit order (library bit
    reader / writer) for the bitstream;
  * hand-worked bit-order vectors derived from the layout on paper;
  * numpy float64 matmul of dequantized weights (library routine);
  * closed forms: constant codes, one-hot activations;
  * exact integer arithmetic (numpy int64);
  * exact invariants: power-of-two scaling, sign symmetry.
"""
from __future__ import annotations

import numpy as np

import oracle
from gemm_qmm_gemv_amd import inputs

BITS_ALL = (2, 3, 4, 5, 6, 7, 8)


# ---- independent helpers built on numpy library routines --------------------

def np_unpack(words: np.ndarray, n: int, k: int, bits: int) -> np.ndarray:
    """Codes via numpy's little-bit-order unpackbits over little-endian bytes."""
    b = np.ascontiguousarray(words, dtype="<u4").reshape(n, -1).view(np.uint8)
    stream = np.unpackbits(b, axis=1, bitorder="little")[:, : k * bits]
    fields = stream.reshape(n, k, bits).astype(np.int64)
    return (fields << np.arange(bits, dtype=np.int64)).sum(axis=2)


def np_pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """Packed words via numpy's little-bit-order packbits."""
    codes = np.asarray(codes, dtype=np.int64)
    n, k = codes.shape
    fields = ((codes[:, :, None] >> np.arange(bits)) & 1).astype(np.uint8)
    by = np.packbits(fields.reshape(n, k * bits), axis=1, bitorder="little")
    return np.ascontiguousarray(by).view("<u4").astype(np.uint32).reshape(n, k * bits // 32)


def np_dequant(codes, scales, mins, group):
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    m = np.asarray(mins, dtype=np.float16).astype(np.float64)
    s_full = np.repeat(s, group, axis=1)
    m_full = np.repeat(m, group, axis=1)
    return s_full * codes + m_full


def _rand_problem(n, k, bits, group, m, seed):
    q = inputs.quantized_matrix(n, k, bits, group, key=(99, seed, bits))
    x = inputs.activation_rows(m, k, key=(99, seed, bits))
    return q, x


# ---- fp16 decoder ------------------------------------------------------------

def check_fp16_exhaustive():
    h = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.fp16_to_double(h)
    ref = h.view(np.float16).astype(np.float64)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), "fp16 decode differs at %d patterns" % int((~same).sum())
    # Signed zeros keep their sign.
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


# ---- bit layout ----------------------------------------------------------------

# (bits, K, {code index: value}, expected words) -- worked by hand from the layout.
HAND_VECTORS = [
    # Q4: codes 1..8 in one word, nibble i = code i -> 0x87654321.
    (4, 8, {i: i + 1 for i in range(8)}, [0x87654321]),
    # Q2: codes 0,1,2,3 then zeros -> 0b11_10_01_00 = 0xE4.
    (2, 16, {0: 0, 1: 1, 2: 2, 3: 3}, [0x000000E4]),
    # Q8: bytes in order -> 0x04030201.
    (8, 4, {0: 1, 1: 2, 2: 3, 3: 4}, [0x04030201]),
    # Q3: code 10 = 0b111 sits on stream bits 30..32: word0 bits 30,31 and word1 bit 0.
    (3, 32, {10: 7}, [0xC0000000, 0x00000001, 0x00000000]),
    # Q3: code 0 = 0b101 -> word0 = 5; code 31 = 0b100 -> stream bit 95 = word2 bit 31.
    (3, 32, {0: 5, 31: 4}, [0x00000005, 0x00000000, 0x80000000]),
    # Q6: code 5 = 0b111111 on stream bits 30..35.
    (6, 16, {5: 63}, [0xC0000000, 0x0000000F, 0x00000000]),
    # Q6: code 15 = 0b100001 on stream bits 90..95: word2 bits 26 and 31.
    (6, 16, {15: 33}, [0x00000000, 0x00000000, 0x84000000]),
    # Q5: code 6 = 0b10011 on stream bits 30..34: bits 30,31 (0b11) and 34 (0b1).
    (5, 32, {6: 19}, [0xC0000000, 0x00000004, 0, 0, 0]),
    # Q7: code 4 = 0b1000001 on stream bits 28..34: bit 28 and bit 34.
    (7, 32, {4: 65}, [0x10000000, 0x00000004, 0, 0, 0, 0, 0]),
]


def check_hand_vectors():
    for bits, k, codes_set, words in HAND_VECTORS:
        codes = np.zeros((1, k), dtype=np.uint8)
        for i, v in codes_set.items():
            codes[0, i] = v
        exp = np.array(words, dtype=np.uint32).reshape(1, -1)
        got_w = oracle.pack(codes, bits)
        assert np.array_equal(got_w, exp), (bits, [hex(v) for v in got_w.ravel()])
        got_c = oracle.unpack(exp, 1, k, bits)
        assert np.array_equal(got_c, codes), (bits, got_c)


def check_unpack_library_reader():
    for bits in BITS_ALL:
        for n, k in ((1, 32), (3, 64), (17, 192), (5, 1024)):
            rng = inputs.rng_for(7, bits, n, k)
            w = inputs.packed_words(rng, n, k, bits)
            got = oracle.unpack(w, n, k, bits)
            assert np.array_equal(got.astype(np.int64), np_unpack(w, n, k, bits)), (bits, n, k)


def check_pack_library_writer_and_roundtrips():
    for bits in BITS_ALL:
        for n, k in ((2, 32), (9, 320)):
            rng = inputs.rng_for(8, bits, n, k)
            codes = rng.integers(0, 1 << bits, size=(n, k)).astype(np.uint8)
            w = oracle.pack(codes, bits)
            assert np.array_equal(w, np_pack(codes, bits)), bits
            assert np.array_equal(oracle.unpack(w, n, k, bits), codes), bits
            words = inputs.packed_words(rng, n, k, bits)
            again = oracle.pack(oracle.unpack(words, n, k, bits), bits)
            assert np.array_equal(again, words), bits


# ---- dequantization and products ----------------------------------------------

def check_dequant_library():
    for bits in BITS_ALL:
        for group in (32, 64):
            n, k = 7, 256
            q, _ = _rand_problem(n, k, bits, group, 1, 1)
            codes = np_unpack(q["w"], n, k, bits)
            ref = np_dequant(codes, q["scales"], q["mins"], group)
            got = oracle.dequant(q["w"], q["scales"], q["mins"], n, k, bits, group)
            assert np.array_equal(got, ref), (bits, group)


def check_qmm_library_matmul():
    for bits in BITS_ALL:
        for (n, k, m, group) in ((17, 192, 1, 64), (9, 256, 3, 32), (33, 128, 5, 128)):
            q, x = _rand_problem(n, k, bits, group, m, 2)
            codes = np_unpack(q["w"], n, k, bits)
            wd = np_dequant(codes, q["scales"], q["mins"], group)
            xd = x.astype(np.float64)
            y_ref = xd @ wd.T
            a_ref = np.abs(xd) @ np.abs(wd).T
            y, a = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, group)
            scale = a_ref + 1e-300
            assert np.all(np.abs(y - y_ref) <= 1e-12 * scale), (bits, n, k, m)
            assert np.allclose(a, a_ref, rtol=1e-12, atol=0), (bits, n, k, m)
            # The GEMV form (x given as a vector) is row 0 of the GEMM.
            y0, a0 = oracle.qmm(q["w"], q["scales"], q["mins"], x[0], n, k, bits, group)
            assert np.array_equal(y0, y[0]) and np.array_equal(a0, a[0])


def check_constant_codes_closed_form():
    # q == c everywhere: y[n] = sum_g (c * s[n,g] + m[n,g]) * sum_{k in g} x[k].
    for bits in (2, 3, 4, 5, 6, 8):
        n, k, group = 11, 320, 64
        rng = inputs.rng_for(9, bits)
        s, mn = inputs.scales_mins(rng, n, k, group)
        x = inputs.activations(rng, 2, k)
        for c in (0, 1, (1 << bits) - 1, (1 << bits) // 2 + 1):
            w = np_pack(np.full((n, k), c), bits)
            y, _ = oracle.qmm(w, s, mn, x, n, k, bits, group)
            xs = x.astype(np.float64).reshape(2, k // group, group).sum(axis=2)
            coef = c * s.astype(np.float64) + mn.astype(np.float64)
            y_cf = xs @ coef.T
            assert np.allclose(y, y_cf, rtol=1e-12, atol=1e-12), (bits, c)


def check_one_hot():
    # x = e_j: y[n] = s[n, j/g] * q[n, j] + m[n, j/g], exactly.
    for bits in (2, 3, 4, 5, 6, 8):
        n, k, group = 13, 192, 64
        q, _ = _rand_problem(n, k, bits, group, 1, 3)
        codes = np_unpack(q["w"], n, k, bits)
        s = q["scales"].astype(np.float64)
        mn = q["mins"].astype(np.float64)
        for j in (0, 1, 31, 32, 63, 64, 100, k - 1):
            x = np.zeros(k, dtype=np.float16)
            x[j] = 1.0
            y, _ = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, group)
            exp = s[:, j // group] * codes[:, j] + mn[:, j // group]
            assert np.array_equal(y, exp), (bits, j)


def check_exact_integer():
    # scale 1, min 0, integer x in [-2, 2]: y is an exact integer sum.
    for bits in (2, 3, 4, 5, 6, 8):
        n, k, m, group = 9, 512, 3, 64
        rng = inputs.rng_for(10, bits)
        w = inputs.packed_words(rng, n, k, bits)
        s = np.ones((n, k // group), dtype=np.float16)
        mn = np.zeros((n, k // group), dtype=np.float16)
        xi = rng.integers(-2, 3, size=(m, k))
        y, _ = oracle.qmm(w, s, mn, xi.astype(np.float16), n, k, bits, group)
        exp = xi @ np_unpack(w, n, k, bits).T
        assert np.array_equal(y, exp.astype(np.float64)), bits


def check_exact_invariants():
    for bits in (3, 4, 8):
        n, k, m, group = 10, 256, 2, 64
        q, x = _rand_problem(n, k, bits, group, m, 4)
        y, a = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, group)
        s2 = (q["scales"].astype(np.float32) * 2).astype(np.float16)
        m2 = (q["mins"].astype(np.float32) * 2).astype(np.float16)
        y2, a2 = oracle.qmm(q["w"], s2, m2, x, n, k, bits, group)
        assert np.array_equal(y2, 2 * y) and np.array_equal(a2, 2 * a), bits
        yn, an = oracle.qmm(q["w"], q["scales"], q["mins"], -x, n, k, bits, group)
        assert np.array_equal(yn, -y) and np.array_equal(an, a), bits


def check_sample_matches_full():
    n, k, m, bits, group = 40, 256, 3, 4, 64
    q, x = _rand_problem(n, k, bits, group, m, 5)
    y, a = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, group)
    rm = np.array([0, 2, 1, 2, 0], dtype=np.int64)
    rn = np.array([0, 39, 17, 5, 38], dtype=np.int64)
    ys, as_ = oracle.qmm_sample(q["w"], q["scales"], q["mins"], x, k, bits, group, rm, rn)
    assert np.array_equal(ys, y[rm, rn]) and np.array_equal(as_, a[rm, rn])


def check_moe_per_expert():
    e, n, k, bits, group, t, top = 6, 24, 128, 4, 64, 5, 2
    st = inputs.stacked_experts(e, n, k, bits, group, key=(98,))
    r = inputs.routing(t, e, top, key=(98,))
    x = inputs.activation_rows(t, k, key=(98,))
    off = r["offsets"]
    y, a = oracle.moe(st["w"], st["scales"], st["mins"], x, r["pair_token"], off, e, n, k, bits, group)
    p = int(off[-1])
    assert p == t * top
    for pi in range(p):
        ex = int(r["pair_expert"][pi])
        assert off[ex] <= pi < off[ex + 1]
        codes = np_unpack(st["w"][ex], n, k, bits)
        wd = np_dequant(codes, st["scales"][ex], st["mins"][ex], group)
        xv = x[r["pair_token"][pi]].astype(np.float64)
        assert np.allclose(y[pi], wd @ xv, rtol=1e-12, atol=1e-12), pi
        assert np.allclose(a[pi], np.abs(wd) @ np.abs(xv), rtol=1e-12, atol=0), pi
    # Without a row index, row p of x feeds pair p.
    xp = x[r["pair_token"]]
    y2, _ = oracle.moe(st["w"], st["scales"], st["mins"], xp, None, off, e, n, k, bits, group)
    assert np.array_equal(y2, y)


def check_moe_combine():
    # Token-major brute force: token t's output is the sum over its chosen
    # experts (slot order) of weight * (dequantized expert matrix @ x[t]),
    # built from the per-token routing table, not from the expert-sorted
    # pairs the oracle walks.
    e, n, k, bits, group, t, top = 7, 20, 128, 3, 64, 6, 3
    st = inputs.stacked_experts(e, n, k, bits, group, key=(99,))
    r = inputs.routing(t, e, top, key=(99,))
    x = inputs.activation_rows(t, k, key=(99,))
    y0 = inputs.activation_rows(t, n, key=(99, 1)).astype(np.float64)
    yp, ap = oracle.moe(st["w"], st["scales"], st["mins"], x, r["pair_token"], r["offsets"], e, n, k,
                        bits, group)
    y, a = oracle.moe_combine(yp, ap, r["pair_token"], r["pair_weight"], t, y0)
    for ti in range(t):
        want, scale = y0[ti].copy(), np.zeros(n)
        for j in range(top):
            ex = int(r["experts"][ti, j])
            wgt = float(np.float32(r["weights"][ti, j]))
            wd = np_dequant(np_unpack(st["w"][ex], n, k, bits), st["scales"][ex], st["mins"][ex], group)
            xv = x[ti].astype(np.float64)
            want += wgt * (wd @ xv)
            scale += abs(wgt) * (np.abs(wd) @ np.abs(xv))
        assert np.allclose(y[ti], want, rtol=1e-12, atol=1e-12), ti
        assert np.allclose(a[ti], scale, rtol=1e-12, atol=0), ti
    # Top-1 routing with unit weights and no y0 only permutes the rows.
    r1 = inputs.routing(t, e, 1, key=(99, 2))
    yp1, ap1 = oracle.moe(st["w"], st["scales"], st["mins"], x, r1["pair_token"], r1["offsets"], e, n,
                          k, bits, group)
    y1, _ = oracle.moe_combine(yp1, ap1, r1["pair_token"], np.ones(t, np.float32), t)
    assert np.array_equal(y1[r1["pair_token"]], yp1)
    # A pair whose token is out of range adds nothing.
    tok = r1["pair_token"].copy()
    tok[0] = t
    y2, _ = oracle.moe_combine(yp1, ap1, tok, np.ones(t, np.float32), t)
    assert not np.any(y2[r1["pair_token"][0]]) and np.array_equal(y2[tok[1:]], yp1[1:])


# ---- fp16 weights (bits 16) -------------------------------------------------------

def _f16_words(h):
    """uint16 [n][k] fp16 patterns -> the library's words: k = 2j in the low
    half of word j, k = 2j + 1 in the high half (written out bit by bit)."""
    h = np.asarray(h, dtype=np.uint32)
    return (h[:, 0::2] | (h[:, 1::2] << 16)).astype(np.uint32)


def check_f16_matches_q8_path():
    # Q8 codes with scale 1 and min 0 are integers 0..255, exact in fp16: the
    # fp16-weight product must equal the quantized path's product.
    n, k, m = 9, 256, 3
    rng = inputs.rng_for(11)
    codes = rng.integers(0, 256, size=(n, k))
    x = inputs.activations(rng, m, k)
    w8 = np_pack(codes, 8)
    s = np.ones((n, k // 64), dtype=np.float16)
    mn = np.zeros((n, k // 64), dtype=np.float16)
    y8, a8 = oracle.qmm(w8, s, mn, x, n, k, 8, 64)
    h = codes.astype(np.float16).view(np.uint16)
    y16, a16 = oracle.qmm(_f16_words(h), None, None, x, n, k, 16, 64)
    assert np.allclose(y16, y8, rtol=0, atol=1e-12 * np.abs(a8).max())
    assert np.allclose(a16, a8, rtol=1e-12, atol=0)


def check_f16_one_hot_and_layout():
    # x = e_j picks weight (n, j) exactly; a row with distinct values in every
    # half-word shows which half holds which k.
    n, k = 5, 64
    rng = inputs.rng_for(12)
    h = (0.1 * rng.standard_normal((n, k))).astype(np.float16)
    words = _f16_words(h.view(np.uint16))
    for j in (0, 1, 2, 31, 62, 63):
        x = np.zeros(k, dtype=np.float16)
        x[j] = 1.0
        y, _ = oracle.qmm(words, None, None, x, n, k, 16, 64)
        assert np.array_equal(y, h[:, j].astype(np.float64)), j
    # Weight 1.0 (0x3C00) only in the high half of word 0: it is k = 1.
    w = np.zeros((1, k // 2), dtype=np.uint32)
    w[0, 0] = 0x3C000000
    x = np.arange(k).astype(np.float16)
    y, _ = oracle.qmm(w, None, None, x, 1, k, 16, 64)
    assert y[0] == 1.0


def check_f16_exact_integer():
    # Integer weights in [-8, 8] and activations in [-2, 2]: exact sums.
    n, k, m = 7, 512, 4
    rng = inputs.rng_for(13)
    wi = rng.integers(-8, 9, size=(n, k))
    xi = rng.integers(-2, 3, size=(m, k))
    words = _f16_words(wi.astype(np.float16).view(np.uint16))
    y, a = oracle.qmm(words, None, None, xi.astype(np.float16), n, k, 16, 64)
    assert np.array_equal(y, (xi @ wi.T).astype(np.float64))
    assert np.array_equal(a, (np.abs(xi) @ np.abs(wi).T).astype(np.float64))
    ys, _ = oracle.qmm_sample(words, None, None, xi.astype(np.float16), k, 16, 64,
                              [0, 3, 2], [6, 0, 1])
    assert np.array_equal(ys, y[[0, 3, 2], [6, 0, 1]])


def check_f16_moe_per_expert():
    e, n, k = 3, 6, 128
    rng = inputs.rng_for(14)
    wi = rng.integers(-8, 9, size=(e, n, k))
    words = np.stack([_f16_words(wi[i].astype(np.float16).view(np.uint16)) for i in range(e)])
    x = rng.integers(-2, 3, size=(5, k)).astype(np.float16)
    x_rows = np.array([4, 0, 2, 2, 1, 3], dtype=np.int32)
    off = np.array([0, 2, 2, 6], dtype=np.int32)
    y, _ = oracle.moe(words, None, None, x, x_rows, off, e, n, k, 16, 64)
    xd = x.astype(np.float64)
    for p, ex in enumerate([0, 0, 2, 2, 2, 2]):
        assert np.array_equal(y[p], wi[ex] @ xd[x_rows[p]]), p


def check_silu():
    # sigmoid(1) = 1 / (1 + 1/e) = 0.7310585786300049 (and 1 - that at -1).
    v = oracle.silu(np.array([1.0, -1.0, 0.0, 40.0, -40.0, 2.5]))
    assert abs(v[0] - 0.7310585786300049) < 1e-15
    assert abs(v[1] + 0.2689414213699951) < 1e-15
    assert v[2] == 0.0
    assert abs(v[3] - 40.0) < 1e-12 and abs(v[4]) < 1e-15
    # v * sigmoid(v) - (-v) * sigmoid(-v) = v (sigmoid(v) + sigmoid(-v) = 1).
    z = np.linspace(-12, 12, 97)
    assert np.allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=0, atol=1e-13)


ALL_CHECKS = [
    check_fp16_exhaustive,
    check_hand_vectors,
    check_unpack_library_reader,
    check_pack_library_writer_and_roundtrips,
    check_dequant_library,
    check_qmm_library_matmul,
    check_constant_codes_closed_form,
    check_one_hot,
    check_exact_integer,
    check_exact_invariants,
    check_sample_matches_full,
    check_moe_per_expert,
    check_f16_matches_q8_path,
    check_f16_one_hot_and_layout,
    check_f16_exact_integer,
    check_f16_moe_per_expert,
    check_silu,
    check_moe_combine,
]
