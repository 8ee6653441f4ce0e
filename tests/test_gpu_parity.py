"""GPU parity: the HIP kernels, called through the C-ABI, against the CPU oracle.

Every case prints its name, shape and seed before it touches the GPU.  Outputs
are poisoned with NaN before each call so a missed store cannot pass.  The
rules (oracle.tolerance): fp32 out |err| <= 1e-3·‖A_i‖‖B_j‖; 16-bit out adds one
ulp of the oracle value; integer-valued inputs must match bit for bit, and so
must every int32 result of int8 inputs (against the oracle's exact int64 sums).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import tolerance

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32,
            "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2, "i8": torch.int8, "i32": torch.int32}
# int32 poison: no sum of K <= 131071 products of int8 values reaches -2^31
I32_POISON = -2 ** 31


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(bits, in_dtype):
    raw = np.uint8 if in_dtype in ("e4m3", "e5m2", "i8") else np.int16
    t = torch.from_numpy(np.ascontiguousarray(bits).view(raw))
    return t.to("cuda").view(TORCH_DT[in_dtype])


def run_gpu(gb, a_bits, b_bits, in_dtype, out_dtype, split_k=False):
    """C through gemm_bt (split_k=False) or through mm_bt's default path, gemm_bt_ws where the plan splits K."""
    a = to_dev(a_bits, in_dtype)
    b = to_dev(b_bits, in_dtype)
    M, N = a.shape[0], b.shape[0]
    poison = I32_POISON if out_dtype == "i32" else float("nan")
    c = torch.full((M, N), poison, dtype=TORCH_DT[out_dtype], device="cuda")
    gb.mm_bt(a, b, out_dtype=TORCH_DT[out_dtype], out=c, split_k=split_k)
    torch.cuda.synchronize()
    return c.cpu()


def check_i8(c, a_bits, b_bits, what, I=None, J=None):
    """int32 results of int8 inputs: equal to the oracle's exact sums, entry for entry."""
    got = c.numpy().astype(np.int64)
    if I is None:
        ref = oracle.gemm_bt_i8(a_bits, b_bits)
    else:
        ref = oracle.gemm_bt_i8_entries(a_bits, b_bits, I, J)
        got = got[I, J]
    bad = np.argwhere(got != ref)
    assert bad.size == 0, (what, len(bad), [(tuple(x), int(got[tuple(x)]), int(ref[tuple(x)])) for x in bad[:5]])


def f64(c):
    return c.to(torch.float64).numpy()


def out_bits(c):
    if c.dtype == torch.float32:
        return c.view(torch.int32).numpy().view(np.uint32)
    return c.view(torch.int16).numpy().view(np.uint16)


def check_full(c, a_bits, b_bits, in_dtype, out_dtype, what):
    cref, nA, nB = oracle.gemm_bt_ref(a_bits, b_bits, in_dtype)
    rep = tolerance.check(f64(c), cref, np.outer(nA, nB), out_dtype)
    assert rep.ok, (what, rep)
    return cref


def check_bits_full(c, a_bits, b_bits, in_dtype, out_dtype, what):
    cref, _, _ = oracle.gemm_bt_ref(a_bits, b_bits, in_dtype)
    rep = tolerance.bit_exact(out_bits(c), oracle.round_to(cref, out_dtype), out_dtype)
    assert rep.ok, (what, rep)


SHAPES = [
    (1, 1, 1), (1, 7, 3), (2, 3, 8), (16, 16, 16), (17, 33, 65), (31, 63, 127), (64, 64, 64),
    (65, 129, 200), (127, 255, 64), (128, 128, 128), (130, 260, 72), (200, 100, 300),
    (257, 513, 129), (300, 700, 1000), (129, 1031, 64), (513, 257, 520),
    # 16-byte rows of C with ragged tile edges (whole-row epilogue), long K
    (130, 264, 72), (520, 1032, 264), (256, 256, 4096),
    # 4-byte rows whose K is not a whole number of 8-element chunks (K tail), and K < 8
    (130, 264, 74), (96, 200, 36), (300, 520, 1006), (64, 64, 6), (257, 300, 2050),
    # shapes that select the 64x64, 128x128 and 256x256 tiles (most above take 32x64)
    (1024, 1024, 200), (1030, 1030, 202), (2048, 1536, 200), (1540, 2050, 136), (4096, 4096, 72),
    (64, 4104, 200), (100, 2050, 134),
    # 256x256 tiles (five-slot ring): one K step, a K tail, ragged edges with three steps, a wrapped ring
    (4096, 4096, 8), (4096, 4096, 130), (4900, 4100, 136), (4096, 4096, 200),
    # just above one wave of 256x256 tiles (289 of them): the 128x256 tier, ragged edges
    (4100, 4100, 136),
    # 128x256 tiles (one wave of them): whole tiles, ragged edges, a K tail, C rows of 8-byte and 2-byte alignment
    # (K a multiple of 64: rows that are 16-byte but not 128-byte aligned take the line ring's 128x128 tiles
    # instead, as the first, second and fourth do)
    (2048, 4096, 136), (2000, 4000, 200), (2048, 4096, 130), (2048, 4004, 72), (2048, 3999, 64),
    (2048, 4096, 128), (2000, 4000, 192), (2048, 4004, 64),
    # fewer 256x256 tiles than CUs where 128-row tiles of either width need more than one wave: 192 tiles (rows
    # that take the line ring elsewhere, and 512-byte rows), 156, 136, 144 with odd K, 160 with line-ring rows;
    # then one wave of 128x256 tiles where 128x128 ones would need two
    (3072, 4096, 72), (3072, 4096, 256), (2880, 3200, 64), (2048, 4352, 128), (3000, 3000, 73), (2560, 3900, 72),
    (2560, 2560, 64), (3072, 1536, 64),
    # 304 tiles of 256x256 (1.19 waves, the edge of the band that takes smaller tiles)
    (4864, 4096, 136),
    # 96x128 tiles (at most one wave of them, more than 128x128 tiles would use): one exact wave, partial tile
    # rows and columns with a K tail, odd K
    (768, 4096, 136), (700, 3200, 130), (3000, 1000, 72), (760, 4000, 137),
    # 128x96 tiles (output rows of 12 or 24 16-byte chunks through the whole-row epilogue; C rows that are not
    # whole chunks store directly): one exact wave with ragged edges, a K tail, odd N
    (1000, 3000, 136), (2048, 1536, 72), (1024, 3072, 130), (1000, 2999, 72),
    # odd K: rows only 2-byte aligned (every other row starts mid-dword), K tails of 1 to 7 elements, on
    # every tile tier and with no whole chunk at all
    (130, 264, 73), (300, 520, 1007), (64, 64, 7), (1000, 3000, 2051), (4096, 4096, 131), (2048, 4096, 135),
    (4100, 4100, 137), (96, 200, 35),
    # the line ring on 64x64 tiles (more of them than CUs; rows 16-byte but not 128-byte aligned), ragged edges
    (700, 2000, 200), (1000, 1500, 136), (1030, 1500, 72),
    # several waves of line-ring 128x96 or 96x128 tiles in place of 128x128 ones (rows 16-byte but not 128-byte
    # aligned, 256x256 tiles under 0.6 of the CUs), ragged edges
    (3000, 3000, 72), (2048, 4352, 136), (1700, 3500, 72),
]
SKINNY = [(1, 100, 512), (16, 1000, 520), (5, 33, 35), (16, 8192, 64), (3, 4099, 2050), (16, 64, 8200),
          # K tails of 7 and 1 element, odd K with no whole chunk, 2-byte aligned rows
          (16, 8192, 8191), (11, 300, 1001), (16, 1000, 7)]


@pytest.mark.parametrize("in_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
def test_shape_sweep(gpu, in_dtype, out_dtype):
    for i, (M, N, K) in enumerate(SHAPES + SKINNY):
        seed = 500 + i
        say("sweep", in_dtype, out_dtype, M, N, K, "seed", seed)
        a, b = synth.make(M, N, K, in_dtype, "normal", seed)
        c = run_gpu(gpu, a, b, in_dtype, out_dtype)
        check_full(c, a, b, in_dtype, out_dtype, (M, N, K))


@pytest.mark.parametrize("in_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
def test_integer_bit_exact_sweep(gpu, in_dtype, out_dtype):
    for i, (M, N, K) in enumerate(SHAPES + SKINNY):
        seed = 700 + i
        say("int sweep", in_dtype, out_dtype, M, N, K, "seed", seed)
        a, b = synth.make(M, N, K, in_dtype, "int", seed)
        c = run_gpu(gpu, a, b, in_dtype, out_dtype)
        check_bits_full(c, a, b, in_dtype, out_dtype, (M, N, K))


# 8-bit float inputs (K a multiple of 16): one K step of 128, a partial last
# step, the 64x64, 128x128 and 256x256 tiles (the last with ragged edges and
# several steps of its five-slot ring; 4350 x 4090, 272 256x256 tiles just
# above one wave, takes 128x128 ones), and M <= 16 (no streaming kernel for
# 8-bit inputs: the 64x64 tiles take it).
FP8_SHAPES = [(1, 1, 16), (16, 16, 16), (17, 33, 64), (8, 1000, 64), (64, 64, 128), (130, 260, 160),
              (257, 513, 144), (300, 700, 1024), (1024, 1024, 256), (4096, 4096, 128), (4900, 4100, 272),
              (4096, 4096, 400), (4350, 4090, 272),
              # fewer 256x256 tiles than CUs (144, 132 and 136, ragged edges) where 128x128 ones need more than a wave
              (3072, 3072, 64), (2600, 3000, 160), (2000, 4100, 272)]


@pytest.mark.parametrize("in_dtype", ["e4m3", "e5m2"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
def test_fp8_sweep(gpu, in_dtype, out_dtype):
    for i, (M, N, K) in enumerate(FP8_SHAPES):
        seed = 900 + i
        say("fp8 sweep", in_dtype, out_dtype, M, N, K, "seed", seed)
        a, b = synth.make(M, N, K, in_dtype, "normal", seed)
        c = run_gpu(gpu, a, b, in_dtype, out_dtype)
        check_full(c, a, b, in_dtype, out_dtype, (M, N, K))


@pytest.mark.parametrize("in_dtype", ["e4m3", "e5m2"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
def test_fp8_integer_bit_exact(gpu, in_dtype, out_dtype):
    for i, (M, N, K) in enumerate(FP8_SHAPES):
        seed = 950 + i
        say("fp8 int sweep", in_dtype, out_dtype, M, N, K, "seed", seed)
        a, b = synth.make(M, N, K, in_dtype, "int", seed)
        c = run_gpu(gpu, a, b, in_dtype, out_dtype)
        check_bits_full(c, a, b, in_dtype, out_dtype, (M, N, K))


def test_fp8_unsupported_layouts(gpu):
    """8-bit inputs need K % 16 == 0 and 16-byte aligned A and B; anything else is refused before any launch."""
    s = torch.cuda.current_stream().cuda_stream
    a = torch.zeros(64 * 48 + 64, dtype=torch.uint8, device="cuda")
    b = torch.zeros(64 * 48 + 64, dtype=torch.uint8, device="cuda")
    c = torch.full((64, 64), float("nan"), dtype=torch.float32, device="cuda")
    for code in (gpu.FP8_E4M3, gpu.FP8_E5M2):
        say("fp8 unsupported", code)
        assert gpu.gemm_bt(a.data_ptr(), b.data_ptr(), c.data_ptr(), 64, 64, 40, code, gpu.F32, s) == gpu.ERR_UNSUPPORTED
        assert gpu.gemm_bt(a.data_ptr() + 8, b.data_ptr(), c.data_ptr(), 64, 64, 48, code, gpu.F32, s) == \
            gpu.ERR_UNSUPPORTED
        assert gpu.gemm_bt(a.data_ptr(), b.data_ptr(), c.data_ptr(), 64, 64, 48, code, code, s) == gpu.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(c).all()


# 8-bit integer inputs: the same shapes over the whole int8 range, the range
# ends at the largest K whose sums all fit int32, and the refused layouts.
@pytest.mark.parametrize("dist", ["int8", "int"])
def test_i8_sweep(gpu, dist):
    for i, (M, N, K) in enumerate(FP8_SHAPES):
        seed = (1100 if dist == "int8" else 1150) + i
        say("i8 sweep", dist, M, N, K, "seed", seed)
        a, b = synth.make(M, N, K, "i8", dist, seed)
        c = run_gpu(gpu, a, b, "i8", "i32")
        check_i8(c, a, b, (M, N, K))


def test_i8_range_ends(gpu):
    """Rows of all -128 or all 127 at K = 131056: the sums 16384·K, -16256·K and 16129·K, next to 2^31."""
    M, N, K = 64, 96, 131056
    say("i8 range ends", M, N, K)
    ra = np.where(np.arange(M)[:, None] % 2 == 0, -128, 127) * np.ones((1, K))
    rb = np.where(np.arange(N)[:, None] % 3 == 0, -128, 127) * np.ones((1, K))
    a, b = synth.round_bits(ra, "i8"), synth.round_bits(rb, "i8")
    c = run_gpu(gpu, a, b, "i8", "i32")
    want = ra[:, :1] * rb[:, :1].T * K
    assert np.array_equal(c.numpy().astype(np.int64), want.astype(np.int64))
    assert int(c.max()) == 16384 * K and int(c.min()) == -16256 * K
    check_i8(c, a, b, "range ends")


def test_i8_unsupported(gpu):
    """int8 needs int32 out (and the reverse), K % 16 == 0, 16-byte aligned A and B, K <= 131071."""
    s = torch.cuda.current_stream().cuda_stream
    a = torch.zeros(64 * 131072 + 64, dtype=torch.int8, device="cuda")
    b = torch.zeros(64 * 131072 + 64, dtype=torch.int8, device="cuda")
    c = torch.full((64, 64), I32_POISON, dtype=torch.int32, device="cuda")
    A, B, C = a.data_ptr(), b.data_ptr(), c.data_ptr()
    I8, I32 = gpu.INT8, gpu.INT32
    cases = [(A, B, 48, I8, gpu.F32), (A, B, 48, I8, gpu.BF16), (A, B, 48, gpu.BF16, I32), (A, B, 48, gpu.FP8_E4M3, I32),
             (A, B, 40, I8, I32), (A + 8, B, 48, I8, I32), (A, B + 4, 48, I8, I32), (A, B, 131072, I8, I32)]
    for A_, B_, K, ind, outd in cases:
        say("i8 unsupported", K, ind, outd, A_ - A, B_ - B)
        assert gpu.gemm_bt(A_, B_, C, 64, 64, K, ind, outd, s) == gpu.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (c == I32_POISON).all()
    say("i8 K = 0")
    assert gpu.gemm_bt(A, B, C, 64, 64, 0, I8, I32, s) == gpu.OK  # the empty sum
    torch.cuda.synchronize()
    assert (c == 0).all()


def sample_entries(M, N, rng, tile=256):
    """Rows and columns at every tile edge plus random ones; returns (I, J)."""
    edge_r = sorted({0, M - 1} | {min(M - 1, t + d) for t in range(0, M, tile) for d in (-1, 0)} - {-1})
    edge_c = sorted({0, N - 1} | {min(N - 1, t + d) for t in range(0, N, tile) for d in (-1, 0)} - {-1})
    rows = np.unique(np.concatenate([edge_r[:64], rng.integers(0, M, 24)]))
    cols = np.unique(np.concatenate([edge_c[:64], rng.integers(0, N, 24)]))
    I1, J1 = np.meshgrid(rows, np.arange(N), indexing="ij")
    I2, J2 = np.meshgrid(np.arange(M), cols, indexing="ij")
    I3 = rng.integers(0, M, 20000)
    J3 = rng.integers(0, N, 20000)
    I = np.concatenate([I1.ravel(), I2.ravel(), I3])
    J = np.concatenate([J1.ravel(), J2.ravel(), J3])
    return I, J


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_full_size(gpu, name):
    """Each measured workload at its full size, in the launch configuration the benchmark times."""
    w = synth.WORKLOADS[name]
    say("workload", name, w.M, w.N, w.K, w.in_dtype, w.out_dtype, "seed", w.seed)
    a, b = synth.make_workload(w)
    if w.batch > 1:
        c = gpu.mm_bt(to_dev(a, w.in_dtype), to_dev(b, w.in_dtype), out_dtype=TORCH_DT[w.out_dtype])
        torch.cuda.synchronize()
        cref, nA, nB = oracle.gemm_bt_batched_ref(a, b, w.in_dtype)
        for z in range(w.batch):
            rep = tolerance.check(f64(c[z].cpu()), cref[z], np.outer(nA[z], nB[z]), w.out_dtype)
            assert rep.ok, (name, z, rep)
        return
    if w.b_layout:
        c = run_layout(gpu, a, b, 0, w.b_layout, w.in_dtype, w.out_dtype)
    else:
        c = run_gpu(gpu, a, b, w.in_dtype, w.out_dtype, split_k=True)  # the entry point the benchmark times
    if w.in_dtype == "i8":
        I, J = sample_entries(w.M, w.N, np.random.default_rng(w.seed))
        check_i8(c, a, b, name, I, J)
        return
    cf = f64(c)
    assert np.isfinite(cf).all(), name
    if w.M * w.N * w.K <= 8e9:
        check_full(c, a, b, w.in_dtype, w.out_dtype, name)
    else:
        rng = np.random.default_rng(w.seed)
        I, J = sample_entries(w.M, w.N, rng)
        ref = oracle.gemm_bt_entries(a, b, w.in_dtype, I, J)
        nA = oracle.row_norms(a, w.in_dtype)
        nB = oracle.row_norms(b, w.in_dtype)
        rep = tolerance.check(cf[I, J], ref, nA[I] * nB[J], w.out_dtype)
        assert rep.ok, (name, rep)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_integer_twin_bit_exact(gpu, name):
    w = synth.WORKLOADS[name].integer_twin()
    say("workload int twin", w.name, w.M, w.N, w.K, "seed", w.seed)
    a, b = synth.make_workload(w)
    if w.batch > 1:
        c = gpu.mm_bt(to_dev(a, w.in_dtype), to_dev(b, w.in_dtype), out_dtype=TORCH_DT[w.out_dtype])
        torch.cuda.synchronize()
        cref, _, _ = oracle.gemm_bt_batched_ref(a, b, w.in_dtype)
        for z in range(w.batch):
            rep = tolerance.bit_exact(out_bits(c[z].cpu()), oracle.round_to(cref[z], w.out_dtype), w.out_dtype)
            assert rep.ok, (w.name, z, rep)
        return
    if w.b_layout:
        c = run_layout(gpu, a, b, 0, w.b_layout, w.in_dtype, w.out_dtype)
    else:
        c = run_gpu(gpu, a, b, w.in_dtype, w.out_dtype, split_k=True)  # the entry point the benchmark times
    if w.in_dtype == "i8":
        I, J = sample_entries(w.M, w.N, np.random.default_rng(w.seed))
        check_i8(c, a, b, w.name, I, J)
    elif w.M * w.N * w.K <= 8e9:
        check_bits_full(c, a, b, w.in_dtype, w.out_dtype, w.name)
    else:
        rng = np.random.default_rng(w.seed)
        I, J = sample_entries(w.M, w.N, rng)
        ref = oracle.gemm_bt_entries(a, b, w.in_dtype, I, J)
        rep = tolerance.bit_exact(out_bits(c)[I, J], oracle.round_to(ref, w.out_dtype), w.out_dtype)
        assert rep.ok, (w.name, rep)


@pytest.mark.parametrize("in_dtype", ["bf16", "f16"])
def test_closed_forms(gpu, in_dtype):
    M, K = 300, 264
    a, _ = synth.make(M, 1, K, in_dtype, "normal", 41)
    av = oracle.decode(a, in_dtype)
    for N in (K, 100, 400):
        say("identity B", in_dtype, M, N, K)
        eye = synth.round_bits(np.eye(N, K), in_dtype)
        for out in ("f32", in_dtype):
            c = run_gpu(gpu, a, eye, in_dtype, out)
            want = np.zeros((M, N))
            want[:, :min(N, K)] = av[:, :min(N, K)]
            assert np.array_equal(f64(c), want), (N, out)
    for K in (1, 63, 2050, 4096):
        say("all ones", in_dtype, K)
        ones_a = synth.round_bits(np.ones((70, K)), in_dtype)
        ones_b = synth.round_bits(np.ones((90, K)), in_dtype)
        for out in ("f32", "bf16", "f16"):
            c = run_gpu(gpu, ones_a, ones_b, in_dtype, out)
            want = oracle.decode(oracle.round_to(np.array([float(K)]), out), out)[0] if out != "f32" else float(K)
            assert np.all(f64(c) == want), (K, out)
    say("zero operand", in_dtype)
    a, b = synth.make(129, 257, 96, in_dtype, "normal", 42)
    c = run_gpu(gpu, a, np.zeros_like(b), in_dtype, "f32")
    assert np.all(f64(c) == 0)
    say("permutation B", in_dtype)
    perm = np.random.default_rng(5).permutation(K := 192)
    P = np.zeros((K, K))
    P[np.arange(K), perm] = 1.0
    a, _ = synth.make(77, 1, K, in_dtype, "normal", 43)
    c = run_gpu(gpu, a, synth.round_bits(P, in_dtype), in_dtype, "f32")
    assert np.array_equal(f64(c), oracle.decode(a, in_dtype)[:, perm])


def test_k_zero_and_empty(gpu):
    for out in ("f32", "bf16", "f16"):
        say("K=0", out)
        a = torch.empty((33, 0), dtype=torch.bfloat16, device="cuda")
        b = torch.empty((65, 0), dtype=torch.bfloat16, device="cuda")
        c = torch.full((33, 65), float("nan"), dtype=TORCH_DT[out], device="cuda")
        gpu.mm_bt(a, b, out_dtype=TORCH_DT[out], out=c)
        torch.cuda.synchronize()
        assert torch.all(c == 0).item()
    say("M=0")
    a = torch.empty((0, 16), dtype=torch.bfloat16, device="cuda")
    b = torch.ones((8, 16), dtype=torch.bfloat16, device="cuda")
    c = gpu.mm_bt(a, b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert c.shape == (0, 8)


def test_buffer_end_is_never_read(gpu):
    """A and B sit at the very start of allocations whose remainder is NaN: any
    read past an operand's last element would poison the result."""
    for (M, N, K) in [(65, 130, 70), (300, 200, 66), (16, 300, 130), (257, 257, 257)]:
        say("tail poison", M, N, K)
        a_bits, b_bits = synth.make(M, N, K, "bf16", "uniform", 77)
        big_a = torch.full((M * K + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
        big_b = torch.full((N * K + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
        big_a[:M * K] = to_dev(a_bits, "bf16").reshape(-1)
        big_b[:N * K] = to_dev(b_bits, "bf16").reshape(-1)
        c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        st = gpu.gemm_bt(big_a.data_ptr(), big_b.data_ptr(), c.data_ptr(), M, N, K, gpu.BF16, gpu.F32,
                         torch.cuda.current_stream().cuda_stream)
        assert st == gpu.OK
        torch.cuda.synchronize()
        check_full(c.cpu(), a_bits, b_bits, "bf16", "f32", (M, N, K))


def test_unaligned_pointers_and_odd_k(gpu):
    """Operands starting 2 or 4 bytes past an aligned address, and odd K, select the narrow loaders."""
    for (M, N, K, off) in [(70, 90, 64, 1), (70, 90, 64, 2), (40, 300, 33, 0), (130, 66, 130, 1), (9, 77, 101, 1),
                           (130, 66, 130, 2), (70, 90, 66, 2)]:
        say("unaligned", M, N, K, "offset elems", off)
        a_bits, b_bits = synth.make(M, N, K, "f16", "normal", 88)
        ba = torch.zeros(M * K + 8, dtype=torch.float16, device="cuda")
        bb = torch.zeros(N * K + 8, dtype=torch.float16, device="cuda")
        ba[off:off + M * K] = to_dev(a_bits, "f16").reshape(-1)
        bb[off:off + N * K] = to_dev(b_bits, "f16").reshape(-1)
        bc = torch.full((M * N + 8,), float("nan"), dtype=torch.float16, device="cuda")
        st = gpu.gemm_bt(ba.data_ptr() + 2 * off, bb.data_ptr() + 2 * off, bc.data_ptr() + 2 * off, M, N, K,
                         gpu.F16, gpu.F16, torch.cuda.current_stream().cuda_stream)
        assert st == gpu.OK
        torch.cuda.synchronize()
        c = bc[off:off + M * N].reshape(M, N).cpu()
        check_full(c, a_bits, b_bits, "f16", "f16", (M, N, K, off))
        # neighbours of C untouched
        assert torch.isnan(bc[:off].cpu()).all() and torch.isnan(bc[off + M * N:].cpu()).all()


def test_line_ring_shifted_bases(gpu):
    """The line ring with operands that start 16, 48 or 112 bytes past a 128-byte line: every row's phase in its
    line moves with the base, on the 128x128, 128x96 and 64x64 ring tiles, against the oracle in full."""
    for (M, N, K, off) in [(1540, 2050, 136, 8), (1000, 3000, 72, 24), (1000, 1500, 136, 56), (1540, 2050, 200, 56)]:
        a_bits, b_bits = synth.make(M, N, K, "bf16", "normal", 89)
        plan = gpu.gemm_bt_plan(M, N, K, gpu.BF16, gpu.F32, 16, 16, 16)
        say("ring shifted", M, N, K, "offset elems", off, "variant", plan.variant)
        assert plan.variant in (12, 13, 14, 15), "the case must take the line ring"
        ba = torch.zeros(M * K + off, dtype=torch.bfloat16, device="cuda")
        bb = torch.zeros(N * K + off, dtype=torch.bfloat16, device="cuda")
        ba[off:] = to_dev(a_bits, "bf16").reshape(-1)
        bb[off:] = to_dev(b_bits, "bf16").reshape(-1)
        c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        st = gpu.gemm_bt(ba.data_ptr() + 2 * off, bb.data_ptr() + 2 * off, c.data_ptr(), M, N, K, gpu.BF16, gpu.F32,
                         torch.cuda.current_stream().cuda_stream)
        assert st == gpu.OK
        torch.cuda.synchronize()
        check_full(c.cpu(), a_bits, b_bits, "bf16", "f32", (M, N, K, off))


def test_deterministic_and_stream(gpu):
    w = synth.WORKLOADS["ragged_m1000_n3000_k2050_bf16_f32"]
    say("determinism", w.name)
    a_bits, b_bits = synth.make_workload(w)
    a, b = to_dev(a_bits, "bf16"), to_dev(b_bits, "bf16")
    c1 = gpu.mm_bt(a, b, out_dtype=torch.float32)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c2 = gpu.mm_bt(a, b, out_dtype=torch.float32)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))


# ---------------------------------------------------------------- batched products

RAW = {"bf16": torch.int16, "f16": torch.int16, "e4m3": torch.uint8, "e5m2": torch.uint8, "i8": torch.uint8}


def _flat_items(items, rows, K, pad, in_dtype):
    """Device buffer holding the items (z, rows, K) at a stride of rows*K + pad elements."""
    stride = rows * K + pad
    raw = RAW[in_dtype]
    nbytes_el = 1 if raw == torch.uint8 else 2
    buf = torch.zeros((items.shape[0] - 1) * stride + rows * K + 64, dtype=raw, device="cuda")
    for z in range(items.shape[0]):
        src = torch.from_numpy(np.ascontiguousarray(items[z]).view(np.uint8 if nbytes_el == 1 else np.int16))
        buf[z * stride:z * stride + rows * K] = src.reshape(-1).to("cuda")
    return buf, stride


def run_batched(gb, Z, M, N, K, in_dtype, out_dtype, share=None, pad=(0, 0, 0), dist="normal", seed=0):
    """One gemm_bt_batched call; returns (C items (Z,M,N) on the CPU, a_bits, b_bits) after checking
    that the padding between items of C was not written."""
    a3, b3 = synth.make_batched(Z, M, N, K, in_dtype, dist, seed)
    a_bits = a3[0] if share == "a" else a3
    b_bits = b3[0] if share == "b" else b3
    abuf, sa = _flat_items(a_bits[None] if share == "a" else a_bits, M, K, pad[0], in_dtype)
    bbuf, sb = _flat_items(b_bits[None] if share == "b" else b_bits, N, K, pad[1], in_dtype)
    sc = M * N + pad[2]
    poison = I32_POISON if out_dtype == "i32" else float("nan")
    cbuf = torch.full(((Z - 1) * sc + M * N,), poison, dtype=TORCH_DT[out_dtype], device="cuda")
    st = gb.gemm_bt_batched(abuf.data_ptr(), bbuf.data_ptr(), cbuf.data_ptr(), Z, M, N, K,
                            0 if share == "a" else sa, 0 if share == "b" else sb, sc,
                            getattr(gb, {"bf16": "BF16", "f16": "F16", "e4m3": "FP8_E4M3", "e5m2": "FP8_E5M2",
                                         "i8": "INT8"}[in_dtype]),
                            getattr(gb, {"f32": "F32", "bf16": "BF16", "f16": "F16", "i32": "INT32"}[out_dtype]),
                            torch.cuda.current_stream().cuda_stream)
    assert st == gb.OK, gb.status_string(st)
    torch.cuda.synchronize()
    c = cbuf.cpu()
    items = torch.stack([c[z * sc:z * sc + M * N].reshape(M, N) for z in range(Z)])
    for z in range(Z - 1):
        gap = c[z * sc + M * N:(z + 1) * sc]
        assert (gap == I32_POISON).all() if out_dtype == "i32" else torch.isnan(gap).all(), ("pad written", z)
    return items, a_bits, b_bits


# (Z, M, N, K, in, out, shared operand, element padding of A, B, C items): the 64x64, 128x128 and
# 256x256 tiers, 2-byte aligned rows (odd K, or an odd item stride), both streaming kernels,
# 8-bit inputs, shared A and shared B
BATCHED = [
    (3, 130, 260, 72, "bf16", "f32", None, (0, 0, 0)),
    (5, 300, 200, 520, "f16", "f16", "b", (8, 0, 40)),
    (4, 257, 513, 129, "bf16", "bf16", "a", (0, 8, 16)),
    (2, 1024, 1024, 200, "bf16", "f32", None, (0, 0, 0)),
    (2, 4096, 4096, 136, "bf16", "bf16", None, (0, 0, 8)),
    (3, 16, 1000, 520, "bf16", "bf16", None, (0, 0, 0)),
    (2, 5, 33, 35, "f16", "f32", "b", (0, 0, 3)),
    (3, 100, 130, 200, "bf16", "f32", None, (1, 0, 0)),
    (3, 130, 260, 160, "e4m3", "bf16", None, (16, 32, 0)),
    (3, 300, 200, 256, "i8", "i32", "b", (0, 0, 5)),
    (7, 64, 96, 48, "e5m2", "f32", "a", (0, 0, 0)),
    # items stacked into 128x256 tiles: 68 items of 512x512 (272 tiles of 256x256, just above one wave) and
    # 16 items of 512x1024 (one wave of 128x256 tiles)
    (68, 512, 512, 128, "bf16", "bf16", None, (0, 0, 0)),
    (16, 512, 1024, 192, "f16", "f32", None, (0, 0, 0)),
    # the line ring (128x128 tiles, rows 16-byte but not 128-byte aligned) on items whose bases sit at a
    # different phase of the cache line each (an item stride of 139280 bytes), and with A shared
    (9, 512, 512, 136, "bf16", "bf16", None, (8, 0, 0)),
    (9, 512, 512, 136, "f16", "f32", "a", (0, 8, 0)),
    # fewer stacked 256x256 tiles than CUs against more than one wave of 128-row tiles (144 of them, the second
    # with 4-byte rows, ragged edges and B shared), and one wave of 128x256 tiles where 128x128 ones need two
    (9, 1024, 1024, 64, "bf16", "bf16", None, (0, 0, 0)),
    (6, 1000, 1500, 130, "f16", "f32", "b", (0, 0, 8)),
    (4, 1000, 1500, 64, "bf16", "bf16", None, (0, 0, 0)),
    # just past one wave of 256x256 tiles: the first items as one wave, then the rest in a second launch (16 + 1
    # items with B shared and C rows padded, 4 + 1 with A shared and 144-byte rows; 64 + 4 above)
    (17, 256, 4096, 64, "f16", "f32", "b", (0, 0, 8)),
    (5, 1024, 4096, 72, "bf16", "bf16", "a", (0, 16, 0)),
    (33, 256, 2048, 64, "bf16", "bf16", None, (0, 0, 0)),  # 32 items as one wave, then 1
]


@pytest.mark.parametrize("case", range(len(BATCHED)))
def test_batched(gpu, case):
    Z, M, N, K, ind, outd, share, pad = BATCHED[case]
    seed = 1200 + case
    say("batched", Z, M, N, K, ind, outd, "share", share, "pad", pad, "seed", seed)
    items, a_bits, b_bits = run_batched(gpu, Z, M, N, K, ind, outd, share, pad, seed=seed if ind != "i8" else seed,
                                        dist="int8" if ind == "i8" else "normal")
    cref, nA, nB = oracle.gemm_bt_batched_ref(a_bits, b_bits, ind)
    for z in range(Z):
        if ind == "i8":
            assert np.array_equal(items[z].numpy().astype(np.int64), cref[z]), z
        else:
            rep = tolerance.check(f64(items[z]), cref[z], np.outer(nA[z], nB[z]), outd)
            assert rep.ok, (z, rep)


LINE_RING = [(1024, 4096, 4104, "f16", "f16"), (768, 4096, 4104, "bf16", "bf16"), (1000, 3000, 3000, "bf16", "f32"),
             (1540, 2050, 1000, "bf16", "bf16"), (2048, 4096, 1000, "f16", "f16"), (1000, 1500, 3000, "f16", "f16")]


def sampled_large(gpu, M, N, K, ind, outd, seed, variants, what):
    """Tile edges plus 20000 random entries against the oracle, and the integer twin bit for bit on the same
    entries, after checking that the plan takes one of `variants`."""
    plan = gpu.gemm_bt_plan(M, N, K, gpu._torch_code(TORCH_DT[ind]), gpu._torch_code(TORCH_DT[outd]))
    say(what, M, N, K, ind, outd, "variant", plan.variant, "tile", plan.bm, plan.bn)
    assert variants is None or plan.variant in variants, (what, plan.variant)
    rng = np.random.default_rng(seed)
    I, J = sample_entries(M, N, rng)
    a, b = synth.make(M, N, K, ind, "normal", seed)
    c = f64(run_gpu(gpu, a, b, ind, outd))
    ref = oracle.gemm_bt_entries(a, b, ind, I, J)
    rep = tolerance.check(c[I, J], ref, oracle.row_norms(a, ind)[I] * oracle.row_norms(b, ind)[J], outd)
    assert rep.ok, rep
    ai, bi = synth.make(M, N, K, ind, "int", seed + 50)
    ci = run_gpu(gpu, ai, bi, ind, outd)
    refi = oracle.round_to(oracle.gemm_bt_entries(ai, bi, ind, I, J), outd)
    rep = tolerance.bit_exact(out_bits(ci)[I, J], refi, outd)
    assert rep.ok, rep


@pytest.mark.parametrize("case", range(len(LINE_RING)))
def test_line_ring_large(gpu, case):
    """Large products whose rows are 16-byte but not 128-byte aligned: the line ring on the 128x128, 96x128,
    128x96 and 64x64 tiers, up to 129 K steps."""
    sampled_large(gpu, *LINE_RING[case], 1700 + case, (12, 13, 14, 15), "line ring")


# fewer 256x256 tiles than CUs against more than one wave of 128-row tiles (odd K, line-ring rows, 4-byte rows),
# one wave of 128x256 tiles where 128x128 ones would need two, and the row split of 1.27 waves of 256x256 tiles
# (14 tile rows of 256x256, then 1024 rows on 128x96 tiles), at full K
PARTIAL_WAVE = [((3000, 3000, 3001, "bf16", "f32"), (0,)), ((2000, 7000, 3000, "f16", "f16"), (0,)),
                ((5000, 2000, 2002, "bf16", "bf16"), (0,)), ((2560, 2560, 4096, "bf16", "bf16"), (7,)),
                ((4608, 4608, 4096, "bf16", "bf16"), (0,)), ((8448, 4100, 2048, "f16", "f16"), (0,))]


@pytest.mark.parametrize("case", range(len(PARTIAL_WAVE)))
def test_partial_wave_tiers_large(gpu, case):
    shape, variants = PARTIAL_WAVE[case]
    sampled_large(gpu, *shape, 1800 + case, variants, "partial wave")


# rows of C that are not 16-byte aligned (N * output size not a multiple of 16): the whole-row epilogue writes
# aligned chunks of C, each from two parked chunks, and the chunks a tile row shares with its neighbours element by
# element; 2-, 4- and 8-byte aligned rows on the 128x256, 128x128 (line ring), 128x96 and 256x256 tiers
UNALIGNED_C = [(4096, 4097, 4096, "bf16", "bf16"), (1234, 5678, 3000, "f16", "f16"),
               (1000, 2999, 2048, "bf16", "f32"), (4500, 4500, 1000, "bf16", "bf16")]


@pytest.mark.parametrize("case", range(len(UNALIGNED_C)))
def test_unaligned_c_rows_large(gpu, case):
    sampled_large(gpu, *UNALIGNED_C[case], 1900 + case, None, "unaligned C rows")


def test_batched_integer_bit_exact(gpu):
    Z, M, N, K = 4, 257, 300, 136
    say("batched int", Z, M, N, K)
    items, a_bits, b_bits = run_batched(gpu, Z, M, N, K, "bf16", "bf16", None, (0, 8, 4), dist="int", seed=1250)
    cref, _, _ = oracle.gemm_bt_batched_ref(a_bits, b_bits, "bf16")
    for z in range(Z):
        rep = tolerance.bit_exact(out_bits(items[z]), oracle.round_to(cref[z], "bf16"), "bf16")
        assert rep.ok, (z, rep)


def test_batched_k_zero_and_refused_strides(gpu):
    s = torch.cuda.current_stream().cuda_stream
    c = torch.full((3 * 40 + 8,), float("nan"), dtype=torch.float32, device="cuda")
    a = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    say("batched K = 0")
    assert gpu.gemm_bt_batched(a.data_ptr(), a.data_ptr(), c.data_ptr(), 3, 4, 8, 0, 0, 0, 40, gpu.BF16, gpu.F32, s) == gpu.OK
    torch.cuda.synchronize()
    cc = c.cpu()
    for z in range(3):
        assert (cc[z * 40:z * 40 + 32] == 0).all() and torch.isnan(cc[z * 40 + 32:z * 40 + 40]).all()
    say("batched refused")
    # 8-bit items 8 bytes apart are not 16-byte aligned; C items overlapping
    assert gpu.gemm_bt_batched(a.data_ptr(), a.data_ptr(), c.data_ptr(), 2, 4, 4, 16, 72, 0, 16, gpu.FP8_E4M3, gpu.F32,
                               s) == gpu.ERR_UNSUPPORTED
    assert gpu.gemm_bt_batched(a.data_ptr(), a.data_ptr(), c.data_ptr(), 2, 4, 4, 16, 64, 0, 15, gpu.FP8_E4M3, gpu.F32,
                               s) == gpu.ERR_INVALID_VALUE
    torch.cuda.synchronize()


def test_mm_bt_batched_wrapper(gpu):
    """The torch wrapper: 3-D operands, a 2-D (shared) operand, an expanded one, int8."""
    say("mm_bt batched")
    a3, b3 = synth.make_batched(3, 70, 90, 64, "bf16", "normal", 1260)
    A, B = to_dev(a3, "bf16"), to_dev(b3, "bf16")
    cref, nA, nB = oracle.gemm_bt_batched_ref(a3, b3, "bf16")
    for got, bb in ((gpu.mm_bt(A, B, out_dtype=torch.float32), b3), (gpu.mm_bt(A, B[0], out_dtype=torch.float32), b3[0]),
                    (gpu.mm_bt(A, B[0].expand(3, 90, 64), out_dtype=torch.float32), b3[0])):
        torch.cuda.synchronize()
        ref, nA2, nB2 = oracle.gemm_bt_batched_ref(a3, bb, "bf16")
        for z in range(3):
            assert tolerance.check(f64(got[z].cpu()), ref[z], np.outer(nA2[z], nB2[z]), "f32").ok
    a8, b8 = synth.make_batched(2, 33, 17, 48, "i8", "int8", 1261)
    got = gpu.mm_bt(to_dev(a8, "i8"), to_dev(b8, "i8"))
    torch.cuda.synchronize()
    assert got.dtype == torch.int32 and got.shape == (2, 33, 17)
    assert np.array_equal(got.cpu().numpy().astype(np.int64), oracle.gemm_bt_batched_ref(a8, b8, "i8")[0])


# ---------------------------------------------------------------- operands stored K-outer

def run_layout(gb, a_bits, b_bits, a_layout, b_layout, in_dtype, out_dtype):
    """Upload A (M,K) and B (N,K) bits in the requested storage (K-outer = transposed) and call gemm_bt_layout."""
    KO = gb.K_OUTER
    a_st = np.ascontiguousarray(a_bits.T) if a_layout == KO else a_bits
    b_st = np.ascontiguousarray(b_bits.T) if b_layout == KO else b_bits
    a, b = to_dev(a_st, in_dtype), to_dev(b_st, in_dtype)
    M, N = a_bits.shape[0], b_bits.shape[0]
    c = torch.full((M, N), float("nan"), dtype=TORCH_DT[out_dtype], device="cuda")
    out = gb.mm_layout(a, b, a_layout, b_layout, out_dtype=TORCH_DT[out_dtype], out=c)
    torch.cuda.synchronize()
    return out.cpu()


# (M, N, K, A K-outer, B K-outer, in, out): one tile, ragged tiles, K tails of one step, odd K with both
# operands K-outer, the plain product A·B at several sizes, and 16-bit edges of M and N
LAYOUTS = [
    (16, 16, 16, 1, 1, "bf16", "f32"), (64, 64, 64, 0, 1, "bf16", "bf16"), (136, 264, 72, 1, 0, "f16", "f32"),
    (136, 256, 200, 0, 1, "bf16", "f32"), (200, 104, 301, 1, 1, "f16", "f16"), (1000, 3000, 2048, 0, 1, "bf16", "f32"),
    (520, 1032, 264, 1, 1, "bf16", "bf16"), (257, 512, 136, 0, 1, "f16", "f16"), (512, 264, 136, 1, 0, "bf16", "bf16"),
    (4096, 4096, 200, 0, 1, "bf16", "bf16"), (64, 4104, 64, 1, 1, "bf16", "f32"), (8, 8, 5, 1, 1, "bf16", "f32"),
    # the 256 x 256 tier: each layout, ragged edges, a K tail
    (6152, 4096, 136, 1, 1, "bf16", "bf16"), (4096, 6152, 72, 1, 0, "f16", "f32"), (4096, 4096, 100, 1, 1, "bf16", "f16"),
    # just above one wave of 256 x 256 tiles (272 of them): 128 x 128 tiles, ragged edges
    (4104, 4096, 136, 1, 1, "bf16", "bf16"), (4096, 4104, 72, 1, 0, "f16", "f32"),
    # fewer 256 x 256 tiles than CUs (144, 153, 192) where 128 x 128 ones need more than one wave, ragged edges
    (3000, 3000, 72, 1, 0, "bf16", "bf16"), (2056, 4352, 136, 0, 1, "f16", "f32"), (3072, 4096, 64, 1, 1, "bf16", "f16"),
    # rows of C 2- and 4-byte aligned (A stored K-outer, B K-inner with any N): the shifted whole-row epilogue
    (1000, 1001, 136, 1, 0, "bf16", "bf16"), (512, 1003, 200, 1, 0, "f16", "f32"),
]


@pytest.mark.parametrize("case", range(len(LAYOUTS)))
def test_layouts(gpu, case):
    M, N, K, la, lb, ind, outd = LAYOUTS[case]
    seed = 1300 + case
    say("layout", M, N, K, "A K-outer" if la else "A K-inner", "B K-outer" if lb else "B K-inner", ind, outd, "seed", seed)
    a, b = synth.make(M, N, K, ind, "normal", seed)
    c = run_layout(gpu, a, b, la, lb, ind, outd)
    check_full(c, a, b, ind, outd, LAYOUTS[case])


@pytest.mark.parametrize("case", [0, 3, 4, 6, 9])
def test_layouts_integer_bit_exact(gpu, case):
    M, N, K, la, lb, ind, outd = LAYOUTS[case]
    seed = 1350 + case
    say("layout int", M, N, K, la, lb, ind, outd, "seed", seed)
    a, b = synth.make(M, N, K, ind, "int", seed)
    c = run_layout(gpu, a, b, la, lb, ind, outd)
    check_bits_full(c, a, b, ind, outd, LAYOUTS[case])


def test_layouts_refused_and_inner_equals_gemm_bt(gpu):
    s = torch.cuda.current_stream().cuda_stream
    buf = torch.zeros(1 << 16, dtype=torch.int16, device="cuda")
    c = torch.full((100, 64), float("nan"), dtype=torch.float32, device="cuda")
    p = buf.data_ptr()
    say("layout refused")
    assert gpu.gemm_bt_layout(p, p, c.data_ptr(), 100, 64, 64, 1, 0, gpu.BF16, gpu.F32, s) == gpu.ERR_UNSUPPORTED
    assert gpu.gemm_bt_layout(p + 8, p, c.data_ptr(), 64, 64, 64, 1, 0, gpu.BF16, gpu.F32, s) == gpu.ERR_UNSUPPORTED
    assert gpu.gemm_bt_layout(p, p, c.data_ptr(), 64, 64, 64, 1, 7, gpu.BF16, gpu.F32, s) == gpu.ERR_INVALID_VALUE
    torch.cuda.synchronize()
    assert torch.isnan(c).all()
    say("layout K-inner = gemm_bt")
    a, b = synth.make(300, 200, 136, "bf16", "normal", 1399)
    c1 = run_layout(gpu, a, b, 0, 0, "bf16", "bf16")
    c2 = run_gpu(gpu, a, b, "bf16", "bf16")
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_mm_wrapper_is_a_times_b(gpu):
    say("mm wrapper")
    a, bt = synth.make(96, 80, 64, "bf16", "normal", 1398)  # bt is B^T (N x K)
    A = to_dev(a, "bf16")
    Bkn = to_dev(np.ascontiguousarray(bt.T), "bf16")  # B stored K x N
    got = gpu.mm(A, Bkn, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_full(got.cpu(), a, bt, "bf16", "f32", "mm")


# ---------------------------------------------------------------- graph capture

def test_graph_capture_replays_match_eager(gpu):
    """Calls captured into a HIP graph (plain, batched, K-outer, int8, K = 0, split K through a workspace)
    replay bit for bit like eager calls, several times, with eager work and synchronisation between the
    replays.  The library allocates nothing and clears memory with a kernel, never a memset node; the split
    kernel leaves its counters zero for the next replay."""
    say("graph capture")
    a, b = synth.make(300, 520, 136, "bf16", "normal", 1400)
    ask, bsk = synth.make(1024, 1024, 8192, "bf16", "normal", 1403)
    Ask, Bsk = to_dev(ask, "bf16"), to_dev(bsk, "bf16")
    need = gpu.gemm_bt_workspace_size(1024, 1024, 8192, gpu.BF16, gpu.F32)
    assert need > 0, "the split plan must be taken"
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    a3, b3 = synth.make_batched(3, 64, 96, 64, "f16", "normal", 1401)
    a8, b8 = synth.make(130, 260, 160, "i8", "int8", 1402)
    A, B = to_dev(a, "bf16"), to_dev(b, "bf16")
    Bko = to_dev(np.ascontiguousarray(b.T), "bf16")
    A3, B3 = to_dev(a3, "f16"), to_dev(b3, "f16")
    A8, B8 = to_dev(a8, "i8"), to_dev(b8, "i8")
    outs = [torch.empty(300, 520, dtype=torch.bfloat16, device="cuda"),
            torch.empty(300, 520, dtype=torch.float32, device="cuda"),
            torch.empty(3, 64, 96, dtype=torch.float16, device="cuda"),
            torch.empty(130, 260, dtype=torch.int32, device="cuda"),
            torch.full((40, 24), float("nan"), dtype=torch.float32, device="cuda"),
            torch.empty(1024, 1024, dtype=torch.float32, device="cuda")]

    def work(stream):
        s = stream.cuda_stream
        assert gpu.gemm_bt(A.data_ptr(), B.data_ptr(), outs[0].data_ptr(), 300, 520, 136, gpu.BF16, gpu.BF16, s) == 0
        assert gpu.gemm_bt_layout(A.data_ptr(), Bko.data_ptr(), outs[1].data_ptr(), 300, 520, 136, gpu.K_INNER,
                                  gpu.K_OUTER, gpu.BF16, gpu.F32, s) == 0
        assert gpu.gemm_bt_batched(A3.data_ptr(), B3.data_ptr(), outs[2].data_ptr(), 3, 64, 96, 64, 64 * 64, 96 * 64,
                                   64 * 96, gpu.F16, gpu.F16, s) == 0
        assert gpu.gemm_bt(A8.data_ptr(), B8.data_ptr(), outs[3].data_ptr(), 130, 260, 160, gpu.INT8, gpu.INT32, s) == 0
        assert gpu.gemm_bt(A.data_ptr(), B.data_ptr(), outs[4].data_ptr(), 40, 24, 0, gpu.BF16, gpu.F32, s) == 0
        assert gpu.gemm_bt_ws(Ask.data_ptr(), Bsk.data_ptr(), outs[5].data_ptr(), 1024, 1024, 8192, gpu.BF16,
                              gpu.F32, ws.data_ptr(), need, s) == 0

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        work(side)
    side.synchronize()
    eager = [o.clone() for o in outs]
    bits = lambda t: t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        work(side)
    for rep in range(3):
        for o in outs:
            o.fill_(7)  # eager work between replays; the replay must overwrite all of it
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(bits(o), bits(e)), ("replay", rep, "output", i)
    # and the eager results are right
    check_full(eager[0].cpu(), a, b, "bf16", "bf16", "graph plain")
    check_full(eager[1].cpu(), a, b, "bf16", "f32", "graph K-outer")
    assert np.array_equal(eager[3].cpu().numpy().astype(np.int64), oracle.gemm_bt_i8(a8, b8))
    assert (eager[4] == 0).all()
    assert int(ws[:gpu.SK_COUNTER_BYTES].count_nonzero()) == 0
    I, J = sample_entries(1024, 1024, np.random.default_rng(1404), tile=128)
    ref = oracle.gemm_bt_entries(ask, bsk, "bf16", I, J)
    norms = oracle.row_norms(ask, "bf16")[I] * oracle.row_norms(bsk, "bf16")[J]
    rep = tolerance.check(f64(eager[5].cpu())[I, J], ref, norms, "f32")
    assert rep.ok, ("graph split-K", rep)


# ---------------------------------------------------------------- the largest supported K

@pytest.mark.parametrize("M,N,K,ind,outd", [
    (32, 40, 4194296, "bf16", "f32"),    # tiled kernel: 256 rows of K at the 32-bit panel limit (K % 8 == 0)
    (33, 24, 4194298, "f16", "f16"),     # tiled kernel with a K tail of 2
    (40, 33, 4194303, "bf16", "f32"),    # the largest K: odd, rows 2-byte aligned, a K tail of 7
    (16, 24, 4194296, "bf16", "bf16"),   # streaming kernel (M <= 16)
    (32, 32, 8388592, "e4m3", "bf16"),   # 8-bit inputs: the largest K % 16 == 0 below the limit
])
def test_largest_k(gpu, M, N, K, ind, outd):
    """The largest K that the 32-bit buffer offsets allow (256 * K * element size < 2^31), and the first refused."""
    say("largest K", M, N, K, ind, outd)
    a, b = synth.make(M, N, K, ind, "normal_scaled", 1450)
    c = run_gpu(gpu, a, b, ind, outd)
    check_full(c, a, b, ind, outd, (M, N, K))
    isz = 1 if ind == "e4m3" else 2
    code = {"bf16": gpu.BF16, "f16": gpu.F16, "e4m3": gpu.FP8_E4M3}[ind]
    too_big = (0x7FFFFFFF // (256 * isz)) + 16
    with pytest.raises(gpu.GemmBtError) as ei:
        gpu.gemm_bt_plan(M, N, too_big, code, gpu.F32)
    assert ei.value.status == gpu.ERR_UNSUPPORTED


# ---------------------------------------------------------------- batched products with operands stored K-outer

BATCHED_LAYOUTS = [  # (Z, M, N, K, A K-outer, B K-outer, shared operand)
    (3, 136, 264, 72, 1, 0, None), (4, 200, 104, 301, 1, 1, "b"), (64, 512, 512, 512, 0, 1, None),
    (2, 520, 1032, 264, 1, 1, "a"),
]


@pytest.mark.parametrize("case", range(len(BATCHED_LAYOUTS)))
def test_batched_layouts(gpu, case):
    Z, M, N, K, la, lb, share = BATCHED_LAYOUTS[case]
    seed = 1500 + case
    say("batched layout", Z, M, N, K, la, lb, "share", share, "seed", seed)
    a3, b3 = synth.make_batched(Z, M, N, K, "bf16", "normal", seed)
    a_bits = a3[0] if share == "a" else a3
    b_bits = b3[0] if share == "b" else b3
    tr = lambda x, lay: np.ascontiguousarray(np.swapaxes(x, -1, -2)) if lay else x
    A = to_dev(tr(a_bits, la), "bf16")
    B = to_dev(tr(b_bits, lb), "bf16")
    c = gpu.mm_layout(A, B, la, lb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    cref, nA, nB = oracle.gemm_bt_batched_ref(a_bits, b_bits, "bf16")
    for z in range(Z):
        rep = tolerance.check(f64(c[z].cpu()), cref[z], np.outer(nA[z], nB[z]), "f32")
        assert rep.ok, (z, rep)


# ---------------------------------------------------------------- non-finite inputs and output overflow

@pytest.mark.parametrize("M,N,K", [(100, 130, 72), (16, 600, 256)])  # tiled and streaming kernels
def test_non_finite_inputs(gpu, M, N, K):
    """Inf and NaN inputs give the IEEE classes the fp64 oracle gives, entry for entry: ±Inf where one infinite
    product dominates, NaN for Inf·0, NaN inputs, or +Inf and -Inf in one sum; finite entries stay within the rule."""
    say("non-finite", M, N, K)
    a = np.random.default_rng(1700).standard_normal((M, K))
    b = np.random.default_rng(1701).standard_normal((N, K))
    a[3, 5] = np.inf            # row 3: ±Inf against columns with b[:, 5] != 0
    b[:, 5][::7] = 0.0          # ... and NaN where b[j, 5] == 0 (Inf * 0)
    a[7, 9] = np.nan            # row 7: NaN everywhere
    b[11, 20] = -np.inf         # column 11: ±Inf ...
    a[2, 21] = np.inf           # ... and +Inf + -Inf = NaN at (2, 11) with b[11, 21] < 0
    b[11, 21] = -1.0
    a[2, 20] = 1.0
    a_bits, b_bits = synth.round_bits(a, "bf16"), synth.round_bits(b, "bf16")
    for out in ("f32", "bf16"):
        c = run_gpu(gpu, a_bits, b_bits, "bf16", out)
        cref, nA, nB = oracle.gemm_bt_ref(a_bits, b_bits, "bf16")
        assert np.isnan(cref).any() and np.isinf(cref).any() and np.isfinite(cref).any()
        got = f64(c)
        assert np.array_equal(np.isnan(got), np.isnan(cref)), out
        assert np.array_equal(np.isinf(got), np.isinf(cref)), out
        inf = np.isinf(cref)
        assert np.array_equal(np.sign(got[inf]), np.sign(cref[inf])), out
        fin = np.isfinite(cref) & np.isfinite(nA)[:, None] & np.isfinite(nB)[None, :]
        rep = tolerance.check(got[fin], cref[fin], np.outer(nA, nB)[fin], out)
        assert rep.ok, (out, rep)


def test_f16_overflow_boundary(gpu):
    """All-4 operands: every entry is 16 K exactly.  K = 4094 gives 65504, the largest finite f16; K = 4095 gives
    65520, the midpoint to 65536, which rounds to nearest even into +Inf; bit-exact against the oracle's rounding."""
    for K in (4094, 4095):
        say("f16 overflow", K)
        a = synth.round_bits(np.full((40, K), 4.0), "f16")
        b = synth.round_bits(np.full((72, K), 4.0), "f16")
        c = run_gpu(gpu, a, b, "f16", "f16")
        want = 65504.0 if K == 4094 else np.inf
        assert (f64(c) == want).all(), (K, f64(c)[0, 0])
        check_bits_full(c, a, b, "f16", "f16", ("overflow", K))


@pytest.mark.parametrize("fmt", ["e5m2", "e4m3"])
def test_non_finite_8bit_inputs(gpu, fmt):
    """8-bit float codes for Inf (E5M2 only) and NaN (both formats) give the oracle's IEEE classes entry for entry."""
    M, N, K = 100, 130, 128
    say("non-finite 8-bit", fmt, M, N, K)
    a_bits = synth.round_bits(np.random.default_rng(1710).standard_normal((M, K)), fmt)
    b_bits = synth.round_bits(np.random.default_rng(1711).standard_normal((N, K)), fmt)
    one, neg = synth.round_bits(np.array([1.0, -1.0]), fmt)
    if fmt == "e5m2":
        a_bits[3, 5] = 0x7C                       # +Inf
        b_bits[::7, 5] = 0                        # Inf * 0 = NaN in row 3
        b_bits[11, 20] = 0xFC                     # -Inf
        a_bits[2, 21], b_bits[11, 21], a_bits[2, 20] = 0x7C, neg, one  # +Inf + -Inf = NaN at (2, 11)
        a_bits[7, 9] = 0x7F                       # NaN
    else:
        a_bits[7, 9], b_bits[13, 2] = 0x7F, 0xFF  # NaN codes (S.1111.111); E4M3 has no infinity
    c = run_gpu(gpu, a_bits, b_bits, fmt, "f32")
    cref, nA, nB = oracle.gemm_bt_ref(a_bits, b_bits, fmt)
    got = f64(c)
    assert np.isnan(cref).any()
    assert np.array_equal(np.isnan(got), np.isnan(cref)) and np.array_equal(np.isinf(got), np.isinf(cref))
    inf = np.isinf(cref)
    assert np.array_equal(np.sign(got[inf]), np.sign(cref[inf]))
    fin = np.isfinite(cref) & np.isfinite(nA)[:, None] & np.isfinite(nB)[None, :]
    rep = tolerance.check(got[fin], cref[fin], np.outer(nA, nB)[fin], "f32")
    assert rep.ok, rep



def test_c_program_through_the_header(gpu):
    """A C++ program that uses only include/gemm_bt.h and hipMalloc (no Python, no PyTorch) gets the closed-form
    results: all-ones operands give K in every entry (plain and batched with a shared B), an identity B gives A."""
    import os
    import subprocess

    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_check")
    if not os.path.exists(exe):
        pytest.skip("tests/c_abi_check is not built (run the build entry point)")
    say("C program", exe)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("c_abi_check ok"), (r.returncode, r.stdout, r.stderr)


# ---------------------------------------------------------------- stream-K (gemm_bt_ws)
# Shapes the split plan takes on 256 CUs (at most 128 tiles of 128x128, each
# split along K into S = 256 // tiles pieces of at least 32 K steps): 4-way
# (1024x1024), 8-way with f16 out, 4-way with ragged tile edges and a partial
# last K step, 14-way with a K tail (the last to arrive usually reads its own
# piece back), C rows of 8-byte (direct 8-byte stores) and 2-byte alignment
# (element stores), one tile row (M = 64), and 2-way.
SK_CASES = [  # (M, N, K, in, out)
    (1024, 1024, 16384, "bf16", "bf16"), (512, 1024, 32768, "f16", "f16"), (1000, 1000, 8200, "bf16", "f32"),
    (300, 700, 30002, "bf16", "f32"), (130, 4100, 8192, "f16", "f16"), (200, 1999, 17000, "bf16", "f32"),
    (64, 4096, 16384, "bf16", "bf16"), (1024, 2048, 8192, "f16", "f32"), (1024, 1024, 16383, "bf16", "f32"),
    # thin products: 64x64 and 32x64 tiles, ragged M, N and K, fewer pieces for short K, 16 pieces
    (64, 8192, 8192, "bf16", "bf16"), (17, 4100, 4099, "f16", "f32"), (40, 6000, 8195, "bf16", "f32"),
    (33, 3000, 8192, "f16", "f16"), (64, 1024, 65536, "bf16", "bf16"),
    # the line ring's split form (rows 16-byte but not 128-byte aligned)
    (512, 1024, 16392, "f16", "f16"), (300, 700, 30008, "bf16", "bf16"),
]


def run_ws(gb, a_bits, b_bits, in_dtype, out_dtype, ws=None):
    """C through gemm_bt_ws with a zeroed workspace (or `ws`); returns (C on the host, workspace)."""
    a = to_dev(a_bits, in_dtype)
    b = to_dev(b_bits, in_dtype)
    M, K = a.shape
    N = b.shape[0]
    ic, oc = gb._torch_code(a.dtype), gb._torch_code(TORCH_DT[out_dtype])
    nbytes = gb.gemm_bt_workspace_size(M, N, K, ic, oc)
    if ws is None:
        ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    c = torch.full((M, N), float("nan"), dtype=TORCH_DT[out_dtype], device="cuda")
    st = gb.gemm_bt_ws(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, ic, oc, ws.data_ptr(), ws.numel(),
                       torch.cuda.current_stream().cuda_stream)
    assert st == gb.OK, gb.status_string(st)
    torch.cuda.synchronize()
    return c.cpu(), ws


@pytest.mark.parametrize("case", range(len(SK_CASES)))
def test_stream_k(gpu, case):
    M, N, K, ind, outd = SK_CASES[case]
    plan = gpu.gemm_bt_plan_ws(M, N, K, gpu._torch_code(TORCH_DT[ind]), gpu._torch_code(TORCH_DT[outd]))
    say("split-K", M, N, K, ind, outd, "grid", plan.grid, "split tiles", plan.split_tiles)
    assert plan.split_tiles > 0, "the case must take the split plan"
    a, b = synth.make(M, N, K, ind, "normal", 1500 + case)
    c, ws = run_ws(gpu, a, b, ind, outd)
    check_full(c, a, b, ind, outd, ("split-K", M, N, K))
    # the counters are back to zero, and a second call through the same
    # workspace gives the same bits (fixed summation order, any arrival order)
    assert int(ws[:gpu.SK_COUNTER_BYTES].count_nonzero()) == 0
    c2, _ = run_ws(gpu, a, b, ind, outd, ws)
    assert torch.equal(out_bits_t(c), out_bits_t(c2)), "split result differs between runs"
    ai, bi = synth.make(M, N, K, ind, "int", 1600 + case)
    ci, _ = run_ws(gpu, ai, bi, ind, outd, ws)
    check_bits_full(ci, ai, bi, ind, outd, ("split-K int", M, N, K))


def out_bits_t(c):
    return c.view(torch.int32) if c.dtype == torch.float32 else c.view(torch.int16)


# row split: one wave of 256x256 tiles over the first rows, then the remaining rows (64 of them through the thin
# split, 512 through the 128x128 split, 256 on the plain grid) through gemm_bt_ws, at full size
ROW_SPLIT_WS = [(4160, 4096, 4096, "bf16", "bf16"), (4608, 4096, 4096, "f16", "f32"), (4352, 4096, 4104, "bf16", "bf16")]


@pytest.mark.parametrize("case", range(len(ROW_SPLIT_WS)))
def test_row_split_ws_large(gpu, case):
    M, N, K, ind, outd = ROW_SPLIT_WS[case]
    plan = gpu.gemm_bt_plan_ws(M, N, K, gpu._torch_code(TORCH_DT[ind]), gpu._torch_code(TORCH_DT[outd]))
    say("row split ws", M, N, K, ind, outd, "split rows", plan.split_rows, "workspace", plan.workspace_bytes)
    assert plan.split_rows == 4096
    seed = 2000 + case
    rng = np.random.default_rng(seed)
    I, J = sample_entries(M, N, rng)
    a, b = synth.make(M, N, K, ind, "normal", seed)
    c, ws = run_ws(gpu, a, b, ind, outd)
    c = f64(c)
    ref = oracle.gemm_bt_entries(a, b, ind, I, J)
    rep = tolerance.check(c[I, J], ref, oracle.row_norms(a, ind)[I] * oracle.row_norms(b, ind)[J], outd)
    assert rep.ok, rep
    ai, bi = synth.make(M, N, K, ind, "int", seed + 50)
    ci, _ = run_ws(gpu, ai, bi, ind, outd, ws)
    refi = oracle.round_to(oracle.gemm_bt_entries(ai, bi, ind, I, J), outd)
    rep = tolerance.bit_exact(out_bits(ci)[I, J], refi, outd)
    assert rep.ok, rep


def test_stream_k_fallback_and_refusals(gpu):
    """Shapes the plan does not split run gemm_bt exactly; a short workspace is refused before any launch."""
    for (M, N, K) in [(4096, 4096, 256), (300, 260, 200), (16, 1000, 520), (1000, 3000, 2050), (1024, 1024, 4096)]:
        say("ws fallback", M, N, K)
        a, b = synth.make(M, N, K, "bf16", "normal", 77)
        assert gpu.gemm_bt_workspace_size(M, N, K, gpu.BF16, gpu.BF16) == 0
        c_ws, _ = run_ws(gpu, a, b, "bf16", "bf16")
        c = run_gpu(gpu, a, b, "bf16", "bf16")
        assert torch.equal(out_bits_t(c_ws), out_bits_t(c))
    M, N, K = 1024, 1024, 16384
    need = gpu.gemm_bt_workspace_size(M, N, K, gpu.BF16, gpu.F32)
    assert need > 0
    a = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    c = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert gpu.gemm_bt_ws(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, gpu.BF16, gpu.F32, ws.data_ptr(),
                          need - 1, s) == gpu.ERR_INVALID_VALUE
    assert gpu.gemm_bt_ws(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, gpu.BF16, gpu.F32, ws.data_ptr() + 4,
                          need - 4, s) == gpu.ERR_INVALID_VALUE
    torch.cuda.synchronize()
    assert bool((c == 7.0).all()), "a refused call wrote C"
    # a NULL workspace is gemm_bt
    assert gpu.gemm_bt_ws(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, gpu.BF16, gpu.F32, 0, 0, s) == gpu.OK
    torch.cuda.synchronize()
    assert bool((c == 0).all())


def test_mm_bt_split_k_default(gpu):
    """mm_bt takes the split path by default (per-stream workspace) and matches the oracle."""
    M, N, K = 512, 1024, 32768
    assert gpu.gemm_bt_workspace_size(M, N, K, gpu.BF16, gpu.F32) > 0
    a_bits, b_bits = synth.make(M, N, K, "bf16", "normal", 3)
    a, b = to_dev(a_bits, "bf16"), to_dev(b_bits, "bf16")
    c = gpu.mm_bt(a, b, out_dtype=torch.float32)
    c_plain = gpu.mm_bt(a, b, out_dtype=torch.float32, split_k=False)
    torch.cuda.synchronize()
    check_full(c.cpu(), a_bits, b_bits, "bf16", "f32", "mm_bt split")
    check_full(c_plain.cpu(), a_bits, b_bits, "bf16", "f32", "mm_bt plain")
    ws = gpu.workspace_for(a.device, torch.cuda.current_stream().cuda_stream, 0)
    assert int(ws[:gpu.SK_COUNTER_BYTES].count_nonzero()) == 0
