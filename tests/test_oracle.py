"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:
  * hand-computed products (tests/golden/hand_products.txt);
  * the IEEE-754 definitions of the 16-bit formats (tests/golden/*.txt) and the
    library conversions of numpy (float16) and torch-CPU (bfloat16), exhaustively
    over all 65536 bit patterns for decoding; the OCP 8-bit formats against
    torch-CPU float8_e4m3fn / float8_e5m2 over all 256 codes, and their special
    values;
  * exact rational brute force (fractions.Fraction) on tiny shapes, within the
    fp64 summation bound, and equal on integer inputs;
  * closed forms: identity, all-ones, zero and permutation operands;
  * a library routine: numpy float64 matmul on independently decoded inputs.
The exact int8 path is pinned by its own hand-computed products
(tests/golden/int8_products.txt), Python-integer brute force over the whole
int8 range, numpy int64 matmul, and closed forms at the range ends.
A mistake planted in a copy of the oracle's result (transposed operand, dropped
last term, wrong sign) must fail these pins.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import tolerance
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U64 = 2.0 ** -53


def gamma(k):
    return k * U64 / (1 - k * U64)


def parse_products():
    cases = []
    lines = [l.strip() for l in open(os.path.join(GOLDEN, "hand_products.txt"))]
    lines = [l for l in lines if l and not l.startswith("#")]
    i = 0
    while i < len(lines):
        tag, name, M, N, K = lines[i].split()
        assert tag == "case"
        M, N, K = int(M), int(N), int(K)
        rows = [[float(v) for v in l.split()] for l in lines[i + 1:i + 1 + M + N + M]]
        A = np.array(rows[:M])
        B = np.array(rows[M:M + N])
        C = np.array(rows[M + N:])
        assert A.shape == (M, K) and B.shape == (N, K) and C.shape == (M, N)
        cases.append((name, A, B, C))
        i += 1 + M + N + M
    return cases


FP8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def indep_decode(bits, in_dtype):
    """Library decode (numpy float16 / torch bfloat16 / torch float8), independent of the oracle's C decoders."""
    if in_dtype in FP8:
        b8 = np.ascontiguousarray(bits).astype(np.uint8)
        return torch.from_numpy(b8.copy()).view(FP8[in_dtype]).to(torch.float64).numpy()
    b = np.ascontiguousarray(bits).view(np.uint16)
    if in_dtype == "f16":
        return b.view(np.float16).astype(np.float64)
    t = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------- golden fixtures

@pytest.mark.parametrize("in_dtype", ["bf16", "f16", "e4m3"])  # the fixture's inputs are not all exact in e5m2
def test_hand_products(in_dtype):
    for name, A, B, C in parse_products():
        a = synth.round_bits(A, in_dtype)
        b = synth.round_bits(B, in_dtype)
        assert np.array_equal(indep_decode(a, in_dtype), A), name  # inputs exact in the format
        c, nA, nB = oracle.gemm_bt_ref(a, b, in_dtype)
        assert np.array_equal(c, C), (name, c, C)
        assert np.allclose(nA, np.sqrt((A * A).sum(1)), rtol=1e-15)
        assert np.allclose(nB, np.sqrt((B * B).sum(1)), rtol=1e-15)
        for out in ("f32", "bf16", "f16"):
            got = oracle.round_to(c, out)
            back = indep_decode(got, out) if out != "f32" else got.view(np.float32).astype(np.float64)
            assert np.array_equal(back, C), (name, out)


def test_golden_bit_patterns():
    n = 0
    for line in open(os.path.join(GOLDEN, "ieee_16bit_patterns.txt")):
        if line.startswith("#") or not line.strip():
            continue
        d, h, v = line.split()
        bits = np.array([int(h, 16)], dtype=np.uint16)
        got = oracle.decode(bits, d)[0]
        want = float(v)
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (d, h, got, want)
        n += 1
    assert n >= 20


def test_golden_rne_cases():
    n = 0
    for line in open(os.path.join(GOLDEN, "rne_cases.txt")):
        if line.startswith("#") or not line.strip():
            continue
        d, v, h = line.split()
        got = int(oracle.round_to(np.array([float(v)]), d)[0])
        assert got == int(h, 16), (d, v, hex(got), h)
        n += 1
    assert n >= 25


# ---------------------------------------------------------------- decoders / encoders vs libraries

def test_decode_exhaustive_vs_libraries():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    for d, bits in (("bf16", allbits), ("f16", allbits), ("e4m3", codes), ("e5m2", codes)):
        got = oracle.decode(bits, d)
        want = indep_decode(bits, d)
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), d
        assert np.array_equal(got[~nan], want[~nan]), d
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), d


def test_fp8_special_values():
    # OCP 8-bit formats: E4M3 has no infinity, S.1111.111 is NaN and 448 is the
    # largest finite value; E5M2 follows IEEE (infinity at exponent 31,
    # fraction 0).  Smallest subnormals 2^-9 and 2^-16, smallest normals
    # 2^-6 and 2^-14.
    e4 = {0x00: 0.0, 0x80: -0.0, 0x01: 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5, 0x7E: 448.0,
          0xFE: -448.0, 0x7F: math.nan, 0xFF: math.nan, 0x77: 240.0, 0x48: 4.0}
    e5 = {0x00: 0.0, 0x01: 2.0 ** -16, 0x04: 2.0 ** -14, 0x3C: 1.0, 0x3E: 1.5, 0x7B: 57344.0,
          0x7C: math.inf, 0xFC: -math.inf, 0x7D: math.nan, 0x7F: math.nan, 0x44: 4.0}
    for d, table in (("e4m3", e4), ("e5m2", e5)):
        codes = np.array(list(table), dtype=np.uint8)
        got = oracle.decode(codes, d)
        for c, g in zip(table, got):
            want = table[c]
            if math.isnan(want):
                assert math.isnan(g), (d, hex(c))
            else:
                assert g == want and math.copysign(1, g) == math.copysign(1, want), (d, hex(c), g, want)


def test_round_f16_vs_numpy():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 6, 200000),
        rng.uniform(-70000, 70000, 20000),
        (rng.integers(-4096, 4096, 20000) + 0.5) * 2.0 ** rng.integers(-30, 5, 20000),  # many ties
    ])
    got = oracle.round_to(x, "f16")
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_round_bf16_vs_torch_on_fp32_values():
    rng = np.random.default_rng(12)
    x32 = np.concatenate([
        (rng.standard_normal(200000) * 10.0 ** rng.integers(-40, 38, 200000)).astype(np.float32),
        ((rng.integers(-65536, 65536, 20000) + 0.5) * 2.0 ** rng.integers(-140, 100, 20000)).astype(np.float32),
    ])
    x32 = x32[np.isfinite(x32)]
    got = oracle.round_to(x32.astype(np.float64), "bf16")
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_round_f32_vs_numpy():
    rng = np.random.default_rng(13)
    x = rng.standard_normal(100000) * 10.0 ** rng.integers(-40, 38, 100000)
    got = oracle.round_to(x, "f32")
    want = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, want)


def _rne_exact(x, p, emin, maxfin):
    """Nearest-even rounding by exact rational arithmetic (brute force, tiny inputs)."""
    if x == 0:
        return 0.0
    a = abs(Fraction(x))
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, emin) - p)
    n = a / q
    fl = n.numerator // n.denominator
    fr = n - fl
    if fr > Fraction(1, 2) or (fr == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * q
    r = math.inf if r > maxfin else float(r)
    return math.copysign(r, x)


def test_round_vs_exact_rationals():
    rng = np.random.default_rng(14)
    xs = rng.standard_normal(3000) * 10.0 ** rng.integers(-8, 5, 3000)
    for d, p, emin, mx in (("bf16", 7, -126, (2 - Fraction(1, 128)) * Fraction(2) ** 127),
                           ("f16", 10, -14, Fraction(65504))):
        got = oracle.decode(oracle.round_to(xs, d), d)
        for x, g in zip(xs, got):
            assert g == _rne_exact(float(x), p, emin, mx), (d, x, g)


# ---------------------------------------------------------------- brute force on tiny shapes

def _exact_products(a_val, b_val):
    M, K = a_val.shape
    N = b_val.shape[0]
    C = [[sum((Fraction(float(a_val[i, k])) * Fraction(float(b_val[j, k])) for k in range(K)), Fraction(0))
          for j in range(N)] for i in range(M)]
    S = np.abs(a_val) @ np.abs(b_val).T
    return C, S


@pytest.mark.parametrize("in_dtype", ["bf16", "f16", "e4m3", "e5m2"])
def test_brute_force_random_tiny(in_dtype):
    rng = np.random.default_rng(21)
    for trial in range(25):
        M, N, K = (int(v) for v in rng.integers(1, 9, 3))
        a, b = synth.make(M, N, K, in_dtype, "normal", seed=1000 + trial)
        c, _, _ = oracle.gemm_bt_ref(a, b, in_dtype)
        av, bv = indep_decode(a, in_dtype), indep_decode(b, in_dtype)
        C, S = _exact_products(av, bv)
        for i in range(M):
            for j in range(N):
                assert abs(Fraction(c[i, j]) - C[i][j]) <= Fraction(gamma(K) * S[i, j]), (trial, i, j)


@pytest.mark.parametrize("in_dtype", ["bf16", "f16", "e4m3", "e5m2"])
def test_brute_force_integer_exact(in_dtype):
    for trial in range(10):
        M, N, K = 3 + trial % 4, 2 + trial % 5, 1 + 3 * trial
        a, b = synth.make(M, N, K, in_dtype, "int", seed=2000 + trial)
        c, _, _ = oracle.gemm_bt_ref(a, b, in_dtype)
        av, bv = indep_decode(a, in_dtype), indep_decode(b, in_dtype)
        C, _ = _exact_products(av, bv)
        assert all(c[i, j] == C[i][j] for i in range(M) for j in range(N))


def test_brute_force_cancellation():
    # rows whose terms cancel to a small remainder: fp64 keeps it exactly at this size
    A = np.array([[256.0, 1.0, -256.0, 0.0078125], [1024.0, -1024.0, 3.0, -3.0]])
    B = np.array([[1.0, 1.0, 1.0, 1.0], [0.5, 0.5, 0.5, 0.5]])
    a, b = synth.round_bits(A, "bf16"), synth.round_bits(B, "bf16")
    c, _, _ = oracle.gemm_bt_ref(a, b, "bf16")
    assert np.array_equal(c, np.array([[1.0078125, 0.50390625], [0.0, 0.0]]))


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("in_dtype", ["bf16", "f16", "e4m3", "e5m2"])
def test_identity_B(in_dtype):
    M, K = 37, 45
    a, _ = synth.make(M, 1, K, in_dtype, "normal", seed=5)
    for N in (K, 20, 60):  # N = K, N < K, N > K
        B = np.eye(N, K)
        b = synth.round_bits(B, in_dtype)
        c, _, _ = oracle.gemm_bt_ref(a, b, in_dtype)
        av = indep_decode(a, in_dtype)
        want = np.zeros((M, N))
        want[:, :min(N, K)] = av[:, :min(N, K)]
        assert np.array_equal(c, want)


@pytest.mark.parametrize("K", [1, 7, 64, 2050, 4096])
def test_all_ones(K):
    M, N = 3, 5
    ones = np.ones((max(M, N), K))
    for d in ("bf16", "f16"):
        a = synth.round_bits(ones[:M], d)
        b = synth.round_bits(ones[:N], d)
        c, nA, nB = oracle.gemm_bt_ref(a, b, d)
        assert np.all(c == K)
        assert np.allclose(nA, math.sqrt(K)) and np.allclose(nB, math.sqrt(K))
    # the downcast of K: e.g. 2050 -> 2048 in bf16 (spacing 16 there)
    if K == 2050:
        assert oracle.decode(oracle.round_to(np.array([2050.0]), "bf16"), "bf16")[0] == 2048.0
        assert oracle.decode(oracle.round_to(np.array([2050.0]), "f16"), "f16")[0] == 2050.0


def test_zero_operand():
    a, b = synth.make(9, 11, 13, "bf16", "normal", seed=6)
    z = np.zeros_like(b)
    c, _, nB = oracle.gemm_bt_ref(a, z, "bf16")
    assert np.all(c == 0) and np.all(nB == 0)
    c, nA, _ = oracle.gemm_bt_ref(np.zeros_like(a), b, "bf16")
    assert np.all(c == 0) and np.all(nA == 0)


def test_permutation_B():
    M, K = 10, 12
    a, _ = synth.make(M, 1, K, "f16", "normal", seed=7)
    perm = np.random.default_rng(3).permutation(K)
    P = np.zeros((K, K))
    P[np.arange(K), perm] = 1.0  # row j of stored B picks column perm[j] of A
    c, _, _ = oracle.gemm_bt_ref(a, synth.round_bits(P, "f16"), "f16")
    assert np.array_equal(c, indep_decode(a, "f16")[:, perm])


def test_empty_shapes():
    a = np.zeros((0, 5), np.uint16)
    b = np.zeros((3, 5), np.uint16)
    c, nA, nB = oracle.gemm_bt_ref(a, b, "bf16")
    assert c.shape == (0, 3)
    a = np.zeros((4, 0), np.uint16)
    b = np.zeros((3, 0), np.uint16)
    c, nA, nB = oracle.gemm_bt_ref(a, b, "bf16")
    assert c.shape == (4, 3) and np.all(c == 0)  # empty sum


# ---------------------------------------------------------------- library cross-check

@pytest.mark.parametrize("in_dtype,shape", [("bf16", (64, 80, 96)), ("f16", (33, 65, 127)),
                                            ("bf16", (512, 512, 512)), ("e4m3", (70, 90, 160)),
                                            ("e5m2", (65, 33, 256))])
def test_vs_numpy_matmul(in_dtype, shape):
    M, N, K = shape
    a, b = synth.make(M, N, K, in_dtype, "normal", seed=8)
    c, nA, nB = oracle.gemm_bt_ref(a, b, in_dtype)
    av, bv = indep_decode(a, in_dtype), indep_decode(b, in_dtype)
    ref = av @ bv.T
    S = np.abs(av) @ np.abs(bv).T
    # both sides carry fp64 summation error
    assert np.all(np.abs(c - ref) <= 2 * gamma(K) * S + 1e-300)
    assert np.allclose(nA, np.linalg.norm(av, axis=1), rtol=1e-13)
    assert np.allclose(nB, np.linalg.norm(bv, axis=1), rtol=1e-13)


def test_entries_and_norms_match_full():
    a, b = synth.make(70, 90, 130, "bf16", "uniform", seed=9)
    c, nA, nB = oracle.gemm_bt_ref(a, b, "bf16")
    rng = np.random.default_rng(0)
    I = rng.integers(0, 70, 500)
    J = rng.integers(0, 90, 500)
    e = oracle.gemm_bt_entries(a, b, "bf16", I, J)
    assert np.array_equal(e, c[I, J])
    assert np.array_equal(oracle.row_norms(a, "bf16"), nA)
    assert np.array_equal(oracle.row_norms(b, "bf16"), nB)
    with pytest.raises(ValueError):
        oracle.gemm_bt_entries(a, b, "bf16", np.array([70]), np.array([0]))


# ---------------------------------------------------------------- planted mistakes

def test_planted_mistakes_fail_the_pins():
    """A plausible oracle bug must be caught: compare each corrupted variant to the exact result."""
    M = N = K = 7  # square, so a transposed operand still has the right shape
    a, b = synth.make(M, N, K, "bf16", "normal", seed=31)
    av, bv = indep_decode(a, "bf16"), indep_decode(b, "bf16")
    C, S = _exact_products(av, bv)
    good, _, _ = oracle.gemm_bt_ref(a, b, "bf16")
    variants = {
        "transposed result": good.T,
        "B read as K x N": av @ bv,
        "A read as K x M": av.T @ bv.T,
        "dropped last term": av[:, :-1] @ bv[:, :-1].T,
        "sign of one term": good - 2 * np.outer(av[:, 3], bv[:, 3]),
        "off-by-one k": av[:, 1:] @ bv[:, :-1].T,
    }

    def pins_ok(c):
        return all(abs(Fraction(float(c[i, j])) - C[i][j]) <= Fraction(gamma(K) * S[i, j])
                   for i in range(M) for j in range(N))

    assert pins_ok(good)
    for name, bad in variants.items():
        assert not pins_ok(bad), name


# ---------------------------------------------------------------- tolerance checker

def test_tolerance_rules():
    rng = np.random.default_rng(41)
    cref = rng.standard_normal((50, 60)) * 10
    d = np.full_like(cref, 1e-6)  # tiny D: the ulp term dominates for 16-bit outputs
    for out in ("bf16", "f16"):
        u = tolerance.ulp(cref, out)
        assert tolerance.check(cref + 0.9 * u, cref, d, out)
        assert not tolerance.check(cref + 3 * u, cref, d, out)
    D = np.abs(rng.standard_normal((50, 60))) + 1
    for out in ("f32", "bf16", "f16"):
        lim = tolerance.bound(cref, D, out)
        assert tolerance.check(cref + 0.99 * lim, cref, D, out)
        assert not tolerance.check(cref - 1.5 * lim, cref, D, out)
    # zero D requires an exact zero
    z = np.zeros((2, 2))
    assert tolerance.check(z, z, z, "bf16")
    assert not tolerance.check(z + 1e-30, z, z, "bf16")
    # non-finite handling
    inf = np.array([[np.inf, 1.0]])
    assert tolerance.check(inf, inf, np.ones_like(inf), "f16")
    assert not tolerance.check(np.array([[np.nan, 1.0]]), inf, np.ones_like(inf), "f16")
    assert not tolerance.check(np.array([[1.0, np.inf]]), np.array([[1.0, 1.0]]), np.ones((1, 2)), "f32")


def test_ulp_values():
    assert tolerance.ulp(np.array([1.0]), "bf16")[0] == 2.0 ** -7
    assert tolerance.ulp(np.array([1.5]), "f16")[0] == 2.0 ** -10
    assert tolerance.ulp(np.array([4096.0]), "bf16")[0] == 32.0
    assert tolerance.ulp(np.array([0.0]), "f16")[0] == 2.0 ** -24
    assert tolerance.ulp(np.array([0.0]), "bf16")[0] == 2.0 ** -133
    assert tolerance.ulp(np.array([1e-40]), "bf16")[0] == 2.0 ** -133


def test_bit_exact_helper():
    r = np.array([0x3F80, 0x8000, 0x4000], np.uint16)
    g = np.array([0x3F80, 0x0000, 0x4000], np.uint16)
    assert tolerance.bit_exact(g, r, "bf16")
    g[2] = 0x4001
    assert not tolerance.bit_exact(g, r, "bf16")


# ---------------------------------------------------------------- input recipe

def test_synth_recipe():
    w = synth.WORKLOADS["sq512_bf16_f32"]
    a1, b1 = synth.make_workload(w)
    a2, b2 = synth.make_workload(w)
    assert a1.dtype == np.uint16 and a1.shape == (512, 512) and b1.shape == (512, 512)
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2)
    av = indep_decode(a1, "bf16")
    assert abs(av.mean()) < 0.02 and abs(av.std() - 1) < 0.02
    ai, bi = synth.make_workload(w.integer_twin())
    vi = indep_decode(ai, "bf16")
    assert set(np.unique(vi)) <= set(range(-4, 5)) and len(np.unique(vi)) == 9
    ws = synth.WORKLOADS["skinny_m16_n8192_k8192_bf16_bf16"]
    a, _ = synth.make(ws.M, 4, ws.K, "bf16", ws.dist, ws.seed)
    assert abs(indep_decode(a, "bf16").std() - 1 / math.sqrt(ws.K)) < 0.001
    wu = synth.WORKLOADS["ragged_m1000_n3000_k2050_bf16_f32"]
    a, _ = synth.make(50, 4, wu.K, "bf16", wu.dist, wu.seed)
    v = indep_decode(a, "bf16")
    assert v.min() >= -1 and v.max() <= 1 and abs(v.std() - 1 / math.sqrt(3)) < 0.01
    assert [x.seed for x in synth.WORKLOADS.values()] == list(range(12))
    w8 = synth.WORKLOADS["sq4096_e4m3_bf16"]
    a8, _ = synth.make(64, 4, w8.K, w8.in_dtype, w8.dist, w8.seed)
    assert a8.dtype == np.uint8 and w8.compulsory_bytes == 2 * 4096 * 4096 + 4096 * 4096 * 2
    v8 = indep_decode(a8, "e4m3")
    assert abs(v8.std() - 1) < 0.02  # N(0,1) rounded to 3 fraction bits


# ---------------------------------------------------------------- 8-bit integer inputs

def parse_int_products():
    cases = []
    lines = [l.strip() for l in open(os.path.join(GOLDEN, "int8_products.txt"))]
    lines = [l for l in lines if l and not l.startswith("#")]
    i = 0
    while i < len(lines):
        tag, name, M, N, K = lines[i].split()
        assert tag == "case"
        M, N, K = int(M), int(N), int(K)
        rows = [[int(v) for v in l.split()] for l in lines[i + 1:i + 1 + M + N + M]]
        A = np.array(rows[:M], dtype=np.int64)
        B = np.array(rows[M:M + N], dtype=np.int64)
        C = np.array(rows[M + N:], dtype=np.int64)
        assert A.shape == (M, K) and B.shape == (N, K) and C.shape == (M, N)
        cases.append((name, A, B, C))
        i += 1 + M + N + M
    assert len(cases) == 3
    return cases


def test_i8_hand_products():
    for name, A, B, C in parse_int_products():
        a = synth.round_bits(A.astype(np.float64), "i8")
        b = synth.round_bits(B.astype(np.float64), "i8")
        assert a.dtype == np.uint8 and np.array_equal(a.view(np.int8), A)  # two's-complement bytes
        assert np.array_equal(oracle.gemm_bt_i8(a, b), C), name


def test_i8_brute_force_full_range():
    rng = np.random.default_rng(61)
    for M, N, K in [(1, 1, 1), (3, 5, 7), (4, 4, 16), (6, 3, 33)]:
        a = rng.integers(-128, 128, (M, K)).astype(np.int8)
        b = rng.integers(-128, 128, (N, K)).astype(np.int8)
        c = oracle.gemm_bt_i8(a, b)
        for i in range(M):
            for j in range(N):
                assert int(c[i, j]) == sum(int(a[i, k]) * int(b[j, k]) for k in range(K))


def test_i8_vs_numpy_int64():
    for (M, N, K), seed in [((70, 90, 160), 62), ((33, 65, 4096), 63), ((128, 1, 1000), 64)]:
        a, b = synth.make(M, N, K, "i8", "int8", seed)
        ref = a.view(np.int8).astype(np.int64) @ b.view(np.int8).astype(np.int64).T
        assert np.array_equal(oracle.gemm_bt_i8(a, b), ref)


def test_i8_closed_forms():
    K = 131071  # the largest K whose every sum fits int32
    lo = np.full((1, K), -128, np.int8)
    hi = np.full((1, K), 127, np.int8)
    c = oracle.gemm_bt_i8(lo, np.concatenate([lo, hi]))
    assert c[0, 0] == 16384 * K and c[0, 1] == -16256 * K
    assert c[0, 0] < 2 ** 31 and 16384 * (K + 1) == 2 ** 31
    rng = np.random.default_rng(65)
    a = rng.integers(-128, 128, (9, 12)).astype(np.int8)
    eye = np.eye(12, dtype=np.int8)
    assert np.array_equal(oracle.gemm_bt_i8(a, eye), a.astype(np.int64))  # identity B
    perm = rng.permutation(12)
    assert np.array_equal(oracle.gemm_bt_i8(a, eye[perm]), a[:, perm].astype(np.int64))  # permutation B
    assert np.all(oracle.gemm_bt_i8(a, np.zeros((5, 12), np.int8)) == 0)
    assert oracle.gemm_bt_i8(np.zeros((4, 0), np.int8), np.zeros((3, 0), np.int8)).tolist() == [[0] * 3] * 4


def test_i8_entries_match_full_and_planted_mistakes():
    a, b = synth.make(40, 50, 96, "i8", "int8", 66)
    c = oracle.gemm_bt_i8(a, b)
    rng = np.random.default_rng(67)
    I = rng.integers(0, 40, 300)
    J = rng.integers(0, 50, 300)
    assert np.array_equal(oracle.gemm_bt_i8_entries(a, b, I, J), c[I, J])
    with pytest.raises(ValueError):
        oracle.gemm_bt_i8_entries(a, b, np.array([40]), np.array([0]))
    # each plausible slip gives a different product
    av, bv = a.view(np.int8).astype(np.int64), b.view(np.int8).astype(np.int64)
    bad = {"unsigned bytes": a.astype(np.int64) @ b.astype(np.int64).T,
           "dropped last term": av[:, :-1] @ bv[:, :-1].T,
           "off-by-one k": av[:, 1:] @ bv[:, :-1].T,
           "int8 wrap of each product": (((av[:, None, :] * bv[None, :, :] + 128) % 256) - 128).sum(-1)}
    for name, v in bad.items():
        assert not np.array_equal(v, c), name


def test_i8_recipe():
    w = synth.WORKLOADS["sq4096_i8_i32"]
    a, b = synth.make(64, 8, w.K, w.in_dtype, w.dist, w.seed)
    v = a.view(np.int8)
    assert a.dtype == np.uint8 and v.min() == -128 and v.max() == 127
    assert abs(v.astype(np.float64).mean() + 0.5) < 0.2  # uniform on [-128, 127]
    assert w.compulsory_bytes == 2 * 4096 * 4096 + 4 * 4096 * 4096
    with pytest.raises(ValueError):
        synth.round_bits(np.array([0.5]), "i8")
    with pytest.raises(ValueError):
        synth.round_bits(np.array([128.0]), "i8")


# ---------------------------------------------------------------- batched products

def test_batched_items_brute_force():
    """Each item of a batch is its own product: exact rationals per item, no item mixed with another."""
    Z, M, N, K = 3, 3, 4, 5
    a, b = synth.make_batched(Z, M, N, K, "bf16", "normal", 71)
    c, nA, nB = oracle.gemm_bt_batched_ref(a, b, "bf16")
    assert c.shape == (Z, M, N) and nA.shape == (Z, M) and nB.shape == (Z, N)
    for z in range(Z):
        av, bv = indep_decode(a[z], "bf16"), indep_decode(b[z], "bf16")
        C, S = _exact_products(av, bv)
        for i in range(M):
            for j in range(N):
                assert abs(Fraction(float(c[z, i, j])) - C[i][j]) <= Fraction(gamma(K) * S[i, j])
    # the items differ, so a swapped or repeated item would show
    assert not np.array_equal(c[0], c[1]) and not np.array_equal(c[1], c[2])


def test_batched_shared_operand_closed_forms():
    """A shared B: stacking the A items gives one product of (Z·M)×K with B.  A shared A with
    identity-then-permutation B items gives A and its column permutation."""
    Z, M, N, K = 4, 5, 6, 7
    a, b = synth.make_batched(Z, M, N, K, "f16", "normal", 72)
    c, _, _ = oracle.gemm_bt_batched_ref(a, b[0], "f16")
    av, bv = indep_decode(a.reshape(Z * M, K), "f16"), indep_decode(b[0], "f16")
    ref = av @ bv.T
    S = np.abs(av) @ np.abs(bv).T
    assert np.all(np.abs(c.reshape(Z * M, N) - ref) <= 2 * gamma(K) * S)
    a2, _ = synth.make(M, 1, K, "bf16", "normal", 73)
    eye = np.eye(K)
    perm = np.random.default_rng(74).permutation(K)
    bi = np.stack([synth.round_bits(eye, "bf16"), synth.round_bits(eye[perm], "bf16")])
    c2, _, _ = oracle.gemm_bt_batched_ref(a2, bi, "bf16")
    A2 = indep_decode(a2, "bf16")
    assert np.array_equal(c2[0], A2) and np.array_equal(c2[1], A2[:, perm])


def test_batched_int8_and_recipe():
    a, b = synth.make_batched(3, 4, 5, 32, "i8", "int8", 75)
    c, _, _ = oracle.gemm_bt_batched_ref(a, b, "i8")
    ref = np.einsum("zmk,znk->zmn", a.view(np.int8).astype(np.int64), b.view(np.int8).astype(np.int64))
    assert c.dtype == np.int64 and np.array_equal(c, ref)
    w = synth.WORKLOADS["batch64_sq512_bf16_bf16"]
    assert w.batch == 64 and w.flops == 64 * 2 * 512 ** 3 and w.compulsory_bytes == 64 * 3 * 512 * 512 * 2
    wa, wb = synth.make_batched(2, 3, 4, 8, "bf16", "normal", 9)
    fa, fb = synth.make(6, 8, 8, "bf16", "normal", 9)  # the same draws: all of A, then all of B
    assert np.array_equal(wa.reshape(6, 8), fa) and np.array_equal(wb.reshape(8, 8), fb)
