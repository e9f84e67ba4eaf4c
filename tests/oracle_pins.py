"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError if the oracle
disagrees with a fact that does not come from the oracle itself:

* hand-derived packed words for the order maps (tests/golden/awq_pack_words.txt);
* hand-derived worked examples of the activation quantiser
  (tests/golden/quant_act_examples.txt);
* closed forms: exact special cases of the matmul, exhaustive dequantisation;
* brute force: per-element sums computed in Python integers / fractions on tiny
  inputs directly from packed words;
* library routines: numpy's fp16 cast and fp64 matmul, torch's bf16 decode;
* invariants: linearity, scale doubling, symmetric == zero point 8, thread
  count independence, exact integer bounds.

The same pins are run against deliberately broken copies of the oracle
(tests/test_oracle_mutants.py); every planted mistake must trip at least one.
"""
from __future__ import annotations

import os
import math
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Order maps as stated by the pages / chosen for the W4A8 layout.  Used only to
# build brute-force expectations; the golden words pin them independently.
AWQ_MAP = [0, 2, 4, 6, 1, 3, 5, 7]
K8_MAP = [0, 4, 1, 5, 2, 6, 3, 7]


def _golden_words():
    rows = []
    with open(os.path.join(GOLDEN, "awq_pack_words.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, vals, word = line.split()
            words = [int(w, 16) for w in word.split(",")]
            rows.append((kind, [int(v) for v in vals.split(",")], words if kind == "v2" else words[0]))
    return rows


def _golden_quant(name="quant_act_examples.txt"):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("->")
            xs = [float(v) for v in lhs.split(",")]
            s1, a8 = rhs.split()
            rows.append((xs, float(s1), [int(v) for v in a8.split(",")]))
    return rows


def _u32(a):
    return np.asarray(a).astype(np.int64) & 0xFFFFFFFF


def _f16_bits(vals):
    return np.asarray(vals, dtype=np.float16).view(np.uint16)


# ----------------------------------------------------------------------------- packing

def pin_golden_words(orc):
    for kind, vals, word in _golden_words():
        if kind == "v2":
            packed, bad = orc.pack_v2(np.array([vals], np.uint8))
            assert bad == 0
            assert _u32(packed)[0].tolist() == word, (vals, [hex(int(w)) for w in _u32(packed)[0]])
            back = orc.unpack_v2(np.array([word], np.uint32).view(np.int32), len(vals))
            assert back[0].tolist() == vals
        elif kind == "n8":
            packed, bad = orc.pack_n8(np.array([vals], np.uint8))
            assert bad == 0
            assert int(_u32(packed)[0, 0]) == word, (vals, hex(int(_u32(packed)[0, 0])), hex(word))
            back = orc.unpack_n8(np.array([[word]], np.uint32).view(np.int32))
            assert back[0].tolist() == vals
        else:
            packed, bad = orc.pack_k8(np.array(vals, np.int8)[:, None])
            assert bad == 0
            assert int(_u32(packed)[0, 0]) == word, (vals, hex(int(_u32(packed)[0, 0])), hex(word))
            back = orc.unpack_k8(np.array([[word]], np.uint32).view(np.int32))
            assert back[:, 0].tolist() == vals


def pin_pair_extraction(orc):
    """Property of the order map: (w >> 4t) & 0x000F000F holds columns 2t and 2t+1."""
    rng = np.random.default_rng(1)
    words = rng.integers(0, 2 ** 32, size=(64, 4), dtype=np.uint64).astype(np.uint32)
    vals = orc.unpack_n8(words.view(np.int32))
    w = words.astype(np.int64)
    for t in range(4):
        pair = (w >> (4 * t)) & 0x000F000F
        lo = pair & 0xF
        hi = pair >> 16
        assert np.array_equal(lo, vals[:, 2 * t::8].astype(np.int64))
        assert np.array_equal(hi, vals[:, 2 * t + 1::8].astype(np.int64))


def pin_k8_masks(orc):
    """Property of the K8 layout: lo/hi nibble masks give 16*q for k 0..3 / 4..7."""
    rng = np.random.default_rng(2)
    words = rng.integers(0, 2 ** 32, size=(5, 32), dtype=np.uint64).astype(np.uint32)
    q = orc.unpack_k8(words.view(np.int32)).astype(np.int64)  # [40, 32]
    w = words.astype(np.int64)
    lo = (w << 4) & 0xF0F0F0F0
    hi = w & 0xF0F0F0F0
    for b in range(4):
        lob = ((lo >> (8 * b)) & 0xFF).astype(np.int64)
        hib = ((hi >> (8 * b)) & 0xFF).astype(np.int64)
        lob = np.where(lob >= 128, lob - 256, lob)
        hib = np.where(hib >= 128, hib - 256, hib)
        assert np.array_equal(lob, 16 * q[b::8])
        assert np.array_equal(hib, 16 * q[4 + b::8])


def pin_roundtrip(orc):
    rng = np.random.default_rng(3)
    v = rng.integers(0, 16, size=(7, 48), dtype=np.uint8)
    p, bad = orc.pack_n8(v)
    assert bad == 0 and np.array_equal(orc.unpack_n8(p), v)
    edges = np.array([[0, 0x80000000, 0xFFFFFFFF, 0x7FFFFFFF, 0x12345678, 0x88888888]], np.uint32)
    assert np.array_equal(_u32(orc.pack_n8(orc.unpack_n8(edges.view(np.int32)))[0]), _u32(edges))
    w = rng.integers(0, 2 ** 32, size=(9, 40), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(_u32(orc.pack_n8(orc.unpack_n8(w.view(np.int32)))[0]), _u32(w))
    s = rng.integers(-8, 8, size=(48, 5), dtype=np.int8)
    p, bad = orc.pack_k8(s)
    assert bad == 0 and np.array_equal(orc.unpack_k8(p), s)
    assert np.array_equal(_u32(orc.pack_k8(orc.unpack_k8(w.view(np.int32)))[0]), _u32(w))


def pin_pack_clamp(orc):
    v = np.array([[16, 200, 3, 15, 0, 255, 7, 8]], np.uint8)
    p, bad = orc.pack_n8(v)
    assert bad == 3
    assert orc.unpack_n8(p)[0].tolist() == [15, 15, 3, 15, 0, 15, 7, 8]
    s = np.array([-9, 8, -128, 127, 0, -8, 7, 1], np.int8)[:, None]
    p, bad = orc.pack_k8(s)
    assert bad == 4
    assert orc.unpack_k8(p)[:, 0].tolist() == [-8, 7, -8, 7, 0, -8, 7, 1]


# ----------------------------------------------------------------------------- formats

def pin_f16_codec(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(b)) for b in bits])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # encoder vs numpy's correctly rounded cast: finite patterns, midpoints
    # (ties), random doubles, overflow and underflow edges
    fin = ref[ok & np.isfinite(ref)]
    srt = np.unique(fin)
    mids = (srt[:-1] + srt[1:]) / 2
    rng = np.random.default_rng(4)
    rnd = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 5, 3000),
                          [65504.0, 65519.99, 65520.0, 7e4, 2.0 ** -25, 2.0 ** -25 * 1.0001,
                           3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, -0.0, 1e-30]])
    for arr in (fin, mids, rnd):
        with np.errstate(over="ignore"):
            exp = arr.astype(np.float16).view(np.uint16)
        enc = np.array([orc.f64_to_f16(float(v)) for v in arr], np.uint16)
        assert np.array_equal(enc, exp), np.flatnonzero(enc != exp)[:5]


def _rne_bf16_fraction(fr: Fraction) -> float:
    """Exact round-to-nearest-even of a non-negative rational to bfloat16 (8-bit
    significand, binary32 exponent range); inf above the largest finite value."""
    if fr == 0:
        return 0.0
    # exponent e with 2^e <= fr < 2^(e+1): frexp of the nearest double, then
    # corrected by exact comparisons
    e = math.frexp(float(fr))[1] - 1
    while Fraction(2) ** e > fr:
        e -= 1
    while Fraction(2) ** (e + 1) <= fr:
        e += 1
    quantum = Fraction(2) ** (e - 7) if e >= -126 else Fraction(2) ** -133
    n = fr / quantum
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    v = lo * quantum
    return float("inf") if v >= Fraction(2) ** 128 else float(v)


def _bf16_bits(vals):
    return torch.tensor(np.asarray(vals, np.float64), dtype=torch.float64).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def pin_bf16_encode(orc):
    """The bf16 encoder against exact rational rounding: every finite pattern
    round-trips, midpoints between neighbours go to the even one, random
    doubles, and the overflow / subnormal edges."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(vals)
    for b, v in zip(bits[fin], vals[fin]):
        assert orc.f64_to_bf16(float(v)) == int(b) or (v == 0 and orc.f64_to_bf16(float(v)) in (0, 0x8000))
    pos = np.unique(vals[fin & (vals > 0)])
    mids = (pos[:-1] + pos[1:]) / 2  # exact in double (both neighbours have 8-bit significands)
    rng = np.random.default_rng(21)
    rnd = np.concatenate([np.abs(rng.standard_normal(2000)) * 10.0 ** rng.integers(-40, 38, 2000),
                          [2.0 ** -133, 1.5 * 2.0 ** -133, 2.5 * 2.0 ** -133, 2.0 ** -134, 2.0 ** -135,
                           2.0 ** -126, 2.0 ** -126 - 2.0 ** -134, (2 - 2.0 ** -7) * 2.0 ** 127,
                           (2 - 2.0 ** -8) * 2.0 ** 127, (2 - 2.0 ** -8) * 2.0 ** 127 * (1 - 2.0 ** -40)]])
    for v in np.concatenate([mids[::7], rnd]):
        exp = _rne_bf16_fraction(Fraction(float(v)))
        got = orc.bf16_to_f64(orc.f64_to_bf16(float(v)))
        assert got == exp, (v, got, exp)
        assert orc.f64_to_bf16(-float(v)) == orc.f64_to_bf16(float(v)) | 0x8000


def pin_bf16_decode(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.bf16_to_f64(int(b)) for b in bits])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


# ----------------------------------------------------------------------------- W4A16

def _scales_bits(vals, dtype):
    t = torch.tensor(vals, dtype=torch.float64).to(torch.float16 if dtype == 0 else torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def pin_dequant_exhaustive(orc):
    """w = (q - z) * s for every (q, z) pair, per column scales, two groups."""
    for dtype in (0, 1):
        G = 32
        N = 256
        K = 2 * G
        n = np.arange(N)
        q = np.empty((K, N), np.uint8)
        q[:G] = (n % 16)[None, :]
        q[G:] = ((n * 7 + 3) % 16)[None, :]
        z = np.stack([n // 16, (n * 5 + 11) % 16]).astype(np.uint8)
        s_vals = np.stack([0.002 + 0.0001 * n, 0.019 - 0.00005 * n])
        s_bits = _scales_bits(s_vals, dtype)
        s_dec = torch.from_numpy(s_bits.view(np.int16)).view(
            torch.float16 if dtype == 0 else torch.bfloat16).to(torch.float64).numpy()
        qw, _ = orc.pack_n8(q)
        qz, _ = orc.pack_n8(z)
        W = orc.dequant(qw, s_bits, qz, G, dtype)
        for k in range(K):
            g = k // G
            exp = (q[k].astype(np.float64) - z[g].astype(np.float64)) * s_dec[g]
            assert np.array_equal(W[k], exp), (dtype, k)


def pin_w4a16_exact_special(orc):
    """z = 0, s = 2^-3, x in {-1, 0, 1}: every partial sum is an exact dyadic,
    so Y equals the integer product X.Q divided by 8 exactly."""
    rng = np.random.default_rng(5)
    for (M, K, N, G) in ((4, 128, 64, 128), (3, 256, 32, 64)):
        X = rng.integers(-1, 2, size=(M, K)).astype(np.int64)
        Q = rng.integers(0, 16, size=(K, N)).astype(np.int64)
        qw, _ = orc.pack_n8(Q.astype(np.uint8))
        qz, _ = orc.pack_n8(np.zeros((K // G, N), np.uint8))
        s = np.full((K // G, N), 0x3000, np.uint16)  # fp16 0.125
        y = orc.w4a16(_f16_bits(X), qw, s, qz, G)
        exact = (X @ Q).astype(np.float64) / 8.0
        assert np.array_equal(y, exact)


def _brute_w4a16(x, qweight, scales_f, qzeros, G):
    """Per-element sum straight from the packed words, with exact fractions."""
    M, K = x.shape
    N = qweight.shape[1] * 8
    inv = [AWQ_MAP.index(c) for c in range(8)]  # nibble index of column c within a word
    y = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            j, c = divmod(n, 8)
            acc = Fraction(0)
            for k in range(K):
                qv = (int(qweight[k, j]) & 0xFFFFFFFF) >> (4 * inv[c]) & 0xF
                zv = 8 if qzeros is None else (int(qzeros[k // G, j]) & 0xFFFFFFFF) >> (4 * inv[c]) & 0xF
                acc += Fraction(float(x[m, k])) * (qv - zv) * Fraction(float(scales_f[k // G, n]))
            y[m, n] = float(acc)
    return y


def pin_w4a16_bruteforce(orc):
    rng = np.random.default_rng(6)
    for G in (32, 64, 128):
        for sym in (False, True):
            M, K, N = 3, G, 16
            x = rng.standard_normal((M, K)).astype(np.float16)
            qw = rng.integers(0, 2 ** 32, size=(K, N // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
            qz = None if sym else rng.integers(0, 2 ** 32, size=(K // G, N // 8),
                                                dtype=np.uint64).astype(np.uint32).view(np.int32)
            s = (0.002 + 0.018 * rng.random((K // G, N))).astype(np.float16)
            y = orc.w4a16(x.view(np.uint16), qw, s.view(np.uint16), qz, G)
            ref = _brute_w4a16(x.astype(np.float64), qw, s.astype(np.float64), qz, G)
            assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max()), (G, sym)


def _bf16_values(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def pin_w4a16_bf16(orc):
    """bf16 activations and scales (the dtype branch of the W4A16 oracle):
    a brute force straight from the packed words with exact fractions of the
    bf16 values, and the exact special case z = 0, s = 2^-3, x in {-1, 0, 1}
    written as bf16 bit patterns.  Values are chosen so that reading a bf16
    pattern as fp16 (or the reverse) changes the result."""
    rng = np.random.default_rng(24)
    for G in (32, 128):
        for sym in (False, True):
            M, K, N = 2, G, 16
            xb = _bf16_bits(rng.standard_normal((M, K)) * 3.0)
            qw = rng.integers(0, 2 ** 32, size=(K, N // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
            qz = None if sym else rng.integers(0, 2 ** 32, size=(K // G, N // 8),
                                                dtype=np.uint64).astype(np.uint32).view(np.int32)
            sb = _bf16_bits(0.002 + 0.018 * rng.random((K // G, N)))
            y = orc.w4a16(xb, qw, sb, qz, G, dtype=1)
            ref = _brute_w4a16(_bf16_values(xb), qw, _bf16_values(sb), qz, G)
            assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max()), (G, sym)
    M, K, N, G = 3, 128, 32, 128
    X = rng.integers(-1, 2, size=(M, K)).astype(np.int64)
    Q = rng.integers(0, 16, size=(K, N)).astype(np.int64)
    qw, _ = orc.pack_n8(Q.astype(np.uint8))
    qz, _ = orc.pack_n8(np.zeros((K // G, N), np.uint8))
    s = np.full((K // G, N), 0x3E00, np.uint16)  # bf16 0.125
    y = orc.w4a16(_bf16_bits(X.astype(np.float64)), qw, s, qz, G, dtype=1)
    assert np.array_equal(y, (X @ Q).astype(np.float64) / 8.0)


def pin_w4a16_numpy(orc):
    """fp64 matmul by numpy on the oracle's dequantised W agrees with the oracle."""
    rng = np.random.default_rng(7)
    M, K, N, G = 5, 512, 96, 128
    x = rng.standard_normal((M, K)).astype(np.float16)
    qw = rng.integers(0, 2 ** 32, size=(K, N // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
    qz = rng.integers(0, 2 ** 32, size=(K // G, N // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
    s = (0.002 + 0.018 * rng.random((K // G, N))).astype(np.float16)
    W = orc.dequant(qw, s.view(np.uint16), qz, G)
    y = orc.w4a16(x.view(np.uint16), qw, s.view(np.uint16), qz, G, nthreads=3)
    ref = x.astype(np.float64) @ W
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def pin_w4a16_invariants(orc):
    rng = np.random.default_rng(8)
    M, K, N, G = 4, 256, 64, 64
    x = rng.standard_normal((M, K)).astype(np.float16)
    qw = rng.integers(0, 2 ** 32, size=(K, N // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
    qz = rng.integers(0, 2 ** 32, size=(K // G, N // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
    s = (0.002 + 0.018 * rng.random((K // G, N))).astype(np.float16)
    y = orc.w4a16(x.view(np.uint16), qw, s.view(np.uint16), qz, G)
    # doubling X (exact in fp16) doubles Y exactly
    y2 = orc.w4a16((x * np.float16(2)).view(np.uint16), qw, s.view(np.uint16), qz, G)
    assert np.array_equal(y2, 2 * y)
    # doubling the scales doubles Y exactly
    y3 = orc.w4a16(x.view(np.uint16), qw, (s * np.float16(2)).view(np.uint16), qz, G)
    assert np.array_equal(y3, 2 * y)
    # symmetric (no qzeros) == zero points all 8
    z8 = np.full((K // G, N // 8), 0x88888888, np.uint32).view(np.int32)
    assert np.array_equal(orc.w4a16(x.view(np.uint16), qw, s.view(np.uint16), None, G),
                          orc.w4a16(x.view(np.uint16), qw, s.view(np.uint16), z8, G))
    # the thread split does not change any bit
    assert np.array_equal(y, orc.w4a16(x.view(np.uint16), qw, s.view(np.uint16), qz, G, nthreads=5))
    # Y is linear in X: Y(e_k) rows pick out rows of W
    e = np.zeros((2, K), np.float16)
    e[0, 3] = 1
    e[1, K - 1] = 1
    W = orc.dequant(qw, s.view(np.uint16), qz, G)
    ye = orc.w4a16(e.view(np.uint16), qw, s.view(np.uint16), qz, G)
    assert np.array_equal(ye[0], W[3]) and np.array_equal(ye[1], W[K - 1])


# ----------------------------------------------------------------------------- W4A8

def _rne_f16_fraction(fr: Fraction) -> float:
    """Exact round-to-nearest-even of a positive rational to binary16 (brute force)."""
    if fr == 0:
        return 0.0
    # candidates: all finite positive fp16 values; pick nearest, ties to even mantissa
    e = 15
    while e > -14 and Fraction(2) ** e > fr:
        e -= 1
    quantum = Fraction(2) ** (e - 10) if e >= -14 else Fraction(2) ** -24
    if fr < Fraction(2) ** -14:
        quantum = Fraction(2) ** -24
    n = fr / quantum
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return float(lo * quantum)


def pin_quant_examples(orc):
    for xs, s1, a8 in _golden_quant():
        xb = _f16_bits([xs])
        got_a8, got_s1 = orc.quant_act(xb)
        assert float(got_s1[0]) == s1, (xs, got_s1[0], s1)
        assert got_a8[0].tolist() == a8, (xs, got_a8[0].tolist(), a8)


def pin_quant_s1_exhaustive(orc):
    """s1 = fp16(amax/127) for every positive finite fp16 amax equals the exact
    rational quotient rounded once to fp16; the row extremes map to +-127."""
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    x = np.stack([bits, bits | 0x8000], axis=1)  # rows [a, -a]
    a8, s1 = orc.quant_act(x)
    amax = bits.view(np.float16).astype(np.float64)
    for i in range(0, len(bits), 1):
        exp = _rne_f16_fraction(Fraction(float(amax[i])) / 127)
        assert float(s1[i]) == exp, (hex(bits[i]), s1[i], exp)
    normal = s1 >= 2.0 ** -14
    assert np.all(a8[normal, 0] == 127) and np.all(a8[normal, 1] == -127)


def pin_quant_random(orc):
    """Random rows: a8 equals numpy's fp32 divide + rint + clamp with the pinned s1."""
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((6, 1000)) * np.array([[1], [0.01], [30], [1e-3], [1], [5]])).astype(np.float16)
    x[4, :] = 0
    a8, s1 = orc.quant_act(x.view(np.uint16))
    for m in range(x.shape[0]):
        amax = np.abs(x[m].astype(np.float64)).max()
        exp_s1 = _rne_f16_fraction(Fraction(float(amax)) / 127)
        assert float(s1[m]) == exp_s1
        if exp_s1 == 0:
            assert np.all(a8[m] == 0)
            continue
        q = np.rint(x[m].astype(np.float32) / np.float32(exp_s1))
        assert np.array_equal(a8[m], np.clip(q, -128, 127).astype(np.int8))


def pin_quant_bf16_examples(orc):
    for xs, s1, a8 in _golden_quant("quant_act_examples_bf16.txt"):
        got_a8, got_s1 = orc.quant_act(_bf16_bits([xs]), dtype=1)
        assert float(got_s1[0]) == s1, (xs, got_s1[0], s1)
        assert got_a8[0].tolist() == a8, (xs, got_a8[0].tolist(), a8)


def pin_quant_bf16_s1_exhaustive(orc):
    """bf16 activations: s1 = bf16(amax/127) for every positive finite bf16 amax
    equals the exact rational quotient rounded once to bf16; with a normal s1 the
    row extremes map to +-127."""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    x = np.stack([bits, bits | 0x8000], axis=1)
    a8, s1 = orc.quant_act(x, dtype=1)
    amax = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for i in range(len(bits)):
        exp = _rne_bf16_fraction(Fraction(float(amax[i])) / 127)
        assert float(s1[i]) == exp, (hex(bits[i]), s1[i], exp)
    normal = s1 >= 2.0 ** -126
    assert np.all(a8[normal, 0] == 127) and np.all(a8[normal, 1] == -127)


def pin_quant_bf16_random(orc):
    """Random bf16 rows: a8 equals numpy's fp32 divide + rint + clamp with the pinned s1."""
    rng = np.random.default_rng(22)
    xd = rng.standard_normal((5, 700)) * np.array([[1], [0.01], [300], [1e-30], [1]])
    xd[4, :] = 0
    xb = _bf16_bits(xd)
    xv = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    a8, s1 = orc.quant_act(xb, dtype=1)
    for m in range(xd.shape[0]):
        exp_s1 = _rne_bf16_fraction(Fraction(float(np.abs(xv[m]).max())) / 127)
        assert float(s1[m]) == exp_s1
        if exp_s1 == 0:
            assert np.all(a8[m] == 0)
            continue
        q = np.rint(xv[m].astype(np.float32) / np.float32(exp_s1))
        assert np.array_equal(a8[m], np.clip(q, -128, 127).astype(np.int8))


def pin_w4a8_bf16_scales(orc):
    """bf16 s2 / s3: the same exact accumulators as fp16 scales of equal value,
    and Y64 = acc * s1 * s2 with s2 read as bf16 (brute force in rationals)."""
    rng = np.random.default_rng(23)
    for G in (-1, 64):
        M, K, N = 2, 128, 16
        a8 = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        q = rng.integers(-8, 8, size=(K, N)).astype(np.int8)
        b, _ = orc.pack_k8(q)
        s1 = (rng.random(M) * 0.05 + 0.001).astype(np.float32)
        s2d = 0.002 + 0.018 * rng.random(N)
        s2b = _bf16_bits(s2d)
        s3d = None if G < 0 else rng.integers(1, 17, size=(K // G, N)).astype(np.float64)
        s3b = None if s3d is None else _bf16_bits(s3d)
        acc, y = orc.w4a8(a8, b, s1, s2b, s3b, G, dtype=1)
        acc16, _ = orc.w4a8(a8, b, s1, _f16_bits(s2d), None if s3d is None else _f16_bits(s3d), G)
        assert np.array_equal(acc, acc16)
        s2v = torch.from_numpy(s2b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
        for m in range(M):
            for n in range(N):
                ref = sum(int(a8[m, k]) * int(q[k, n]) * (1 if s3d is None else int(s3d[k // G, n]))
                          for k in range(K))
                assert acc[m, n] == ref
                exp_y = Fraction(ref) * Fraction(float(s1[m])) * Fraction(float(s2v[n]))
                assert abs(y[m, n] - float(exp_y)) <= 1e-15 * max(1.0, abs(float(exp_y)))


def pin_w4a8_bruteforce(orc):
    rng = np.random.default_rng(10)
    for G in (-1, 32, 64):
        M, K, N = 3, 128, 8
        a8 = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        q = rng.integers(-8, 8, size=(K, N)).astype(np.int8)
        b, _ = orc.pack_k8(q)
        s1 = (rng.random(M) * 0.05 + 0.001).astype(np.float32)
        s2 = (0.002 + 0.018 * rng.random(N)).astype(np.float16)
        s3 = None if G < 0 else rng.integers(1, 17, size=(K // G, N)).astype(np.float16)
        acc, y = orc.w4a8(a8, b, s1, s2.view(np.uint16), None if s3 is None else s3.view(np.uint16), G)
        for m in range(M):
            for n in range(N):
                ref = 0
                for k in range(K):
                    w = int(q[k, n]) * (1 if s3 is None else int(s3[k // G, n]))
                    ref += int(a8[m, k]) * w
                assert acc[m, n] == ref
                exp_y = Fraction(ref) * Fraction(float(s1[m])) * Fraction(float(s2[n]))
                assert abs(y[m, n] - float(exp_y)) <= 1e-15 * max(1.0, abs(float(exp_y)))


def pin_w4a8_group16_is_channel(orc):
    """Per-group with every s3 = 16 and s2/16 reproduces per-channel exactly."""
    rng = np.random.default_rng(11)
    M, K, N, G = 4, 256, 24, 128
    a8 = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    b = rng.integers(0, 2 ** 32, size=(K // 8, N), dtype=np.uint64).astype(np.uint32).view(np.int32)
    s1 = (rng.random(M) * 0.05 + 0.001).astype(np.float32)
    s2 = (0.002 + 0.018 * rng.random(N)).astype(np.float16)
    acc_c, y_c = orc.w4a8(a8, b, s1, s2.view(np.uint16))
    s3 = np.full((K // G, N), 16, np.float16)
    acc_g, y_g = orc.w4a8(a8, b, s1, (s2 / np.float16(16)).view(np.uint16), s3.view(np.uint16), G)
    assert np.array_equal(acc_g, 16 * acc_c)
    assert np.array_equal(y_g, y_c)
    # the largest possible |acc| over K = 21760 fits in int32
    assert 128 * 128 * 21760 < 2 ** 31


# ----------------------------------------------------------------------------- second AWQ packing

def pin_v2_roundtrip(orc):
    """Identity-order packing round-trips, ragged rows included, and leaves the
    nibbles past the last value zero (skipped)."""
    rng = np.random.default_rng(41)
    for cols in (8, 3, 11, 32, 43):
        v = rng.integers(0, 16, size=(5, cols), dtype=np.uint8)
        p, bad = orc.pack_v2(v)
        assert bad == 0 and np.array_equal(orc.unpack_v2(p, cols), v)
        used = cols % 8
        if used:
            assert np.all((_u32(p[:, -1]) >> (4 * used)) == 0)
        # element c sits in word c // 8 at nibble c % 8
        c = cols - 1
        assert np.array_equal((_u32(p[:, c // 8]) >> (4 * (c % 8))) & 0xF, v[:, c].astype(np.int64))


def _brute_w4a16_v2(x, qweight, scales_f, qzeros, G):
    M, K = x.shape
    N = qweight.shape[1] * 8
    y = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // G
                qv = (int(qweight[k, n // 8]) & 0xFFFFFFFF) >> (4 * (n % 8)) & 0xF
                zv = 8 if qzeros is None else (int(qzeros[n, g // 8]) & 0xFFFFFFFF) >> (4 * (g % 8)) & 0xF
                acc += Fraction(float(x[m, k])) * (qv - zv) * Fraction(float(scales_f[g, n]))
            y[m, n] = float(acc)
    return y


def pin_w4a16_v2_bruteforce(orc):
    rng = np.random.default_rng(42)
    for G, K in ((32, 96), (64, 640)):   # 3 and 10 groups: ragged zero words
        for sym in (False, True):
            M, N = 2, 16
            x = rng.standard_normal((M, K)).astype(np.float16)
            qw = rng.integers(0, 2 ** 32, size=(K, N // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
            zw = (K // G + 7) // 8
            qz = None if sym else orc.pack_v2(rng.integers(0, 16, size=(N, K // G), dtype=np.uint8))[0]
            s = (0.002 + 0.018 * rng.random((K // G, N))).astype(np.float16)
            y = orc.w4a16_v2(x.view(np.uint16), qw, s.view(np.uint16), qz, G)
            ref = _brute_w4a16_v2(x.astype(np.float64), qw, s.astype(np.float64), qz, G)
            assert qz is None or qz.shape == (N, zw)
            assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max()), (G, sym)


def pin_w4a16_v2_matches_first_packing(orc):
    """The same logical weights in either packing give the same Y, bit for
    bit (the first packing's words built from the values by its own packer)."""
    rng = np.random.default_rng(43)
    M, K, N, G = 3, 384, 24, 128
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    z = rng.integers(0, 16, size=(K // G, N), dtype=np.uint8)
    s = (0.002 + 0.018 * rng.random((K // G, N))).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    y1 = orc.w4a16(x.view(np.uint16), orc.pack_n8(q)[0], s.view(np.uint16), orc.pack_n8(z)[0], G)
    y2 = orc.w4a16_v2(x.view(np.uint16), orc.pack_v2(q)[0], s.view(np.uint16), orc.pack_v2(z.T.copy())[0], G)
    assert np.array_equal(y1, y2)
    assert np.array_equal(orc.w4a16_v2(x.view(np.uint16), orc.pack_v2(q)[0], s.view(np.uint16), None, G),
                          orc.w4a16(x.view(np.uint16), orc.pack_n8(q)[0], s.view(np.uint16), None, G))


# ----------------------------------------------------------------------------- INT4-FP8 W4A8

def _e4m3_torch(codes):
    """Library decode of E4M3 codes (torch's float8_e4m3fn)."""
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _e4m3_exact(fr: Fraction) -> int:
    """Round-to-nearest-even of a rational to E4M3, saturating at 448: the
    candidate grid written out from the format (quantum 2^-9 below 2^-6, else
    2^(e-3) in [2^e, 2^(e+1)))."""
    neg = fr < 0
    a = -fr if neg else fr
    if a >= 448:
        return (0x80 if neg else 0) | 0x7E
    if a < Fraction(1, 64):
        quantum, e = Fraction(1, 512), None
    else:
        e = 0
        while Fraction(2) ** (e + 1) <= a:
            e += 1
        while Fraction(2) ** e > a:
            e -= 1
        quantum = Fraction(2) ** (e - 3)
    n = a / quantum
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    v = lo * quantum
    if v == 0:
        return 0x80 if neg else 0
    # encode the (exactly representable) value v
    if v < Fraction(1, 64):
        code = int(v * 512)
    else:
        e = 0
        while Fraction(2) ** (e + 1) <= v:
            e += 1
        while Fraction(2) ** e > v:
            e -= 1
        code = ((e + 7) << 3) | int(v / Fraction(2) ** (e - 3) - 8)
    return (0x80 if neg else 0) | code


def pin_e4m3_decode(orc):
    """Every E4M3 code decodes as torch's float8_e4m3fn does (NaN at 0x7f and 0xff)."""
    ref = _e4m3_torch(np.arange(256))
    got = np.array([orc.e4m3_to_f64(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.flatnonzero(np.isnan(ref)).tolist() == [0x7F, 0xFF]


def pin_e4m3_encode(orc):
    """The encoder: every finite code round-trips, every midpoint goes to the
    even neighbour (exact rationals), random values match exact rounding and
    torch's float32 -> float8_e4m3fn cast, and values beyond 448 saturate."""
    vals = _e4m3_torch(np.arange(256))
    for c in range(256):
        if not np.isnan(vals[c]):
            assert orc.f64_to_e4m3(float(vals[c])) == c, hex(c)
    pos = np.unique(vals[(vals > 0) & ~np.isnan(vals)])
    mids = np.concatenate([[pos[0] / 2], (pos[:-1] + pos[1:]) / 2])
    for v in mids:
        exp = _e4m3_exact(Fraction(float(v)))
        assert orc.f64_to_e4m3(float(v)) == exp and orc.f64_to_e4m3(-float(v)) == exp | 0x80, v
    rng = np.random.default_rng(31)
    rnd = (rng.standard_normal(3000) * 10.0 ** rng.integers(-4, 3, 3000)).astype(np.float32)
    rnd = rnd[np.abs(rnd) <= 448]
    tor = torch.from_numpy(rnd).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for v, t in zip(rnd, tor):
        exp = _e4m3_exact(Fraction(float(v)))
        got = orc.f64_to_e4m3(float(v))
        assert got == exp and (got == int(t) or float(v) == 0), (float(v), hex(got), hex(exp), hex(int(t)))
    for v, c in ((448.0, 0x7E), (463.9, 0x7E), (464.0, 0x7E), (1e30, 0x7E), (-1e30, 0xFE), (-448.0, 0xFE)):
        assert orc.f64_to_e4m3(v) == c, v
    assert orc.f64_to_e4m3(float("nan")) == 0x7F


def _golden_fp8():
    rows = []
    with open(os.path.join(GOLDEN, "quant_act_fp8_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("->")
            dt, xs = lhs.split()
            s1, codes, asum = rhs.split()
            rows.append((0 if dt == "f16" else 1, [float(v) for v in xs.split(",")], float(s1),
                         [int(c, 16) for c in codes.split(",")], float(asum)))
    return rows


def pin_quant_fp8_examples(orc):
    for dt, xs, s1, codes, asum in _golden_fp8():
        xb = _f16_bits([xs]) if dt == 0 else _bf16_bits([xs])
        a, got_s1, got_sum = orc.quant_act_fp8(xb, dtype=dt)
        assert float(got_s1[0]) == s1, (xs, got_s1[0], s1)
        assert a[0].tolist() == codes, (xs, [hex(c) for c in a[0]], [hex(c) for c in codes])
        assert float(got_sum[0]) == asum, (xs, got_sum[0], asum)


def pin_quant_fp8_s1_exhaustive(orc):
    """s1 = fp16(amax/448) for every positive finite fp16 amax equals the exact
    quotient rounded once; with a normal s1 the row extremes map to +-448."""
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    x = np.stack([bits, bits | 0x8000], axis=1)
    a, s1, asum = orc.quant_act_fp8(x)
    amax = bits.view(np.float16).astype(np.float64)
    for i in range(len(bits)):
        assert float(s1[i]) == _rne_f16_fraction(Fraction(float(amax[i])) / 448), hex(bits[i])
    normal = s1 >= 2.0 ** -14
    assert np.all(a[normal, 0] == 0x7E) and np.all(a[normal, 1] == 0xFE)
    assert np.all(asum[normal] == 0)


def pin_quant_fp8_random(orc):
    """Random fp16 and bf16 rows: codes equal torch's cast of the clamped fp32
    quotient, and asum is the exact sum of the codes' values rounded once."""
    rng = np.random.default_rng(32)
    for dt in (0, 1):
        xd = rng.standard_normal((5, 600)) * np.array([[1], [0.01], [30], [1e-3], [1]])
        xd[4, :] = 0
        xb = _f16_bits(xd) if dt == 0 else _bf16_bits(xd)
        xv = xb.view(np.float16).astype(np.float64) if dt == 0 else \
            torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
        a, s1, asum = orc.quant_act_fp8(xb, dtype=dt)
        for m in range(xd.shape[0]):
            amax = Fraction(float(np.abs(xv[m]).max())) / 448
            exp_s1 = _rne_f16_fraction(amax) if dt == 0 else _rne_bf16_fraction(amax)
            assert float(s1[m]) == exp_s1
            if exp_s1 == 0:
                assert np.all(a[m] == 0) and asum[m] == 0
                continue
            q = np.clip(xv[m].astype(np.float32) / np.float32(exp_s1), -448, 448).astype(np.float32)
            tor = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(a[m], tor), m
            exact = sum(Fraction(float(v)) for v in _e4m3_torch(a[m]))
            assert float(asum[m]) == float(np.float32(float(exact)))


def pin_w4a8_fp8_bruteforce(orc):
    """acc and Y64 straight from packed words and codes, in exact rationals."""
    rng = np.random.default_rng(33)
    M, K, N = 3, 64, 8
    a = rng.integers(0, 256, size=(M, K)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38  # no NaN codes
    q = rng.integers(-8, 8, size=(K, N)).astype(np.int8)
    b, _ = orc.pack_k8(q)
    s1 = (rng.random(M) * 0.05 + 0.001).astype(np.float32)
    s2 = (0.002 + 0.018 * rng.random(N)).astype(np.float16)
    acc, y = orc.w4a8_fp8(a, b, s1, s2.view(np.uint16))
    av = _e4m3_torch(a)
    for m in range(M):
        for n in range(N):
            ref = sum(Fraction(float(av[m, k])) * int(q[k, n]) for k in range(K))
            assert acc[m, n] == float(ref)
            exp_y = ref * Fraction(float(s1[m])) * Fraction(float(s2[n]))
            assert abs(y[m, n] - float(exp_y)) <= 1e-15 * max(1.0, abs(float(exp_y)))


def pin_w4a8_fp8_integer_codes(orc):
    """Codes of the integers -16..16 (all exact in E4M3) give the same
    accumulators as the int8 W4A8 oracle on those integers: the two routines
    agree where both are defined."""
    rng = np.random.default_rng(34)
    M, K, N = 4, 256, 24
    ints = rng.integers(-16, 17, size=(M, K))
    codes = np.array([[orc.f64_to_e4m3(float(v)) for v in row] for row in ints], np.uint8)
    b = rng.integers(0, 2 ** 32, size=(K // 8, N), dtype=np.uint64).astype(np.uint32).view(np.int32)
    s1 = np.ones(M, np.float32)
    s2 = np.full(N, 0.5, np.float16)
    acc8, _ = orc.w4a8(ints.astype(np.int8), b, s1, s2.view(np.uint16))
    acc, y = orc.w4a8_fp8(codes, b, s1, s2.view(np.uint16))
    assert np.array_equal(acc, acc8.astype(np.float64))
    assert np.array_equal(y, acc8 * 0.5)


ALL_PINS = [
    pin_golden_words, pin_pair_extraction, pin_k8_masks, pin_roundtrip, pin_pack_clamp,
    pin_dequant_exhaustive, pin_w4a16_exact_special, pin_w4a16_numpy, pin_w4a16_invariants,
    pin_quant_examples, pin_quant_bf16_examples, pin_quant_random, pin_quant_bf16_random,
    pin_w4a8_bruteforce, pin_w4a8_group16_is_channel, pin_w4a8_bf16_scales, pin_bf16_decode,
    pin_w4a16_bruteforce, pin_w4a16_bf16, pin_f16_codec, pin_bf16_encode, pin_quant_s1_exhaustive,
    pin_quant_bf16_s1_exhaustive, pin_e4m3_decode, pin_e4m3_encode, pin_quant_fp8_examples,
    pin_w4a8_fp8_bruteforce, pin_w4a8_fp8_integer_codes, pin_quant_fp8_random, pin_quant_fp8_s1_exhaustive,
    pin_v2_roundtrip, pin_w4a16_v2_bruteforce, pin_w4a16_v2_matches_first_packing,
]
