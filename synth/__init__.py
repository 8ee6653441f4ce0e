"""Seeded synthetic inputs for C = A·Bᵀ, shared by the oracle side and the GPU side.

This module draws random numbers and rounds them to the input format.
It holds none of the product's arithmetic: no dot products, no accumulation,
no output rounding.  Each generator returns raw bit patterns (uint16 arrays for
the 16-bit formats, uint8 for the 8-bit ones, two's-complement bytes for int8),
so the very same bits feed the GPU kernel and the CPU oracle.

Recipe (also stated in the design notes):
  * ``numpy.random.default_rng(seed)`` (PCG64); A is drawn first (M×K, row-major
    order), then B (N×K, row-major order — B is stored transposed).  A batch of
    Z products draws all of A (Z×M×K) and then all of B (Z×N×K), row-major.
  * distributions: ``normal`` N(0, 1); ``normal_scaled`` N(0, σ=1/√K);
    ``uniform`` U[-1, 1) via ``rng.uniform(-1, 1)``; ``int`` uniform integers in
    [-4, 4] (exact in every input format, so fp32 accumulation is exact);
    ``int8`` uniform integers over the whole int8 range [-128, 127].
  * rounding: bf16 values go float64 → float32 (numpy, round-to-nearest-even)
    → bfloat16 (torch CPU conversion, round-to-nearest-even); f16 values go
    float64 → float16 directly (numpy, round-to-nearest-even); e4m3 / e5m2
    values go float64 → float32 → torch ``float8_e4m3fn`` / ``float8_e5m2``
    (torch CPU conversion, round-to-nearest-even; the distributions used stay
    far inside both formats' range); i8 takes integer draws only (anything
    else is an error) and stores them as two's-complement bytes.

The workloads are the matrix products the pages measure: 4096³ square
("Optimizing Blackwell matrix multiplication in Mojo (part 2)", section
"Starting from the 4-line kernel") and M=1024, K=N=4096 f16 with normally
distributed data ("Collective matrix multiplication", the single-device
timing in its introduction), plus a small square case, a ragged case and a
skinny memory-bound case.
"""
from __future__ import annotations

import dataclasses

import numpy as np

IN_DTYPES = ("bf16", "f16", "e4m3", "e5m2", "i8")
OUT_DTYPES = ("f32", "f16", "bf16", "i32")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    in_dtype: str
    out_dtype: str
    dist: str
    seed: int
    batch: int = 1
    b_layout: int = 0  # 1: B is stored K x N (the plain product A·B), read through gemm_bt_layout

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.M * self.N * self.K

    @property
    def compulsory_bytes(self) -> int:
        osz = 4 if self.out_dtype in ("f32", "i32") else 2
        isz = 1 if self.in_dtype in ("e4m3", "e5m2", "i8") else 2
        return self.batch * ((self.M * self.K + self.N * self.K) * isz + self.M * self.N * osz)

    def integer_twin(self) -> "Workload":
        return dataclasses.replace(self, name=self.name + "_int", dist="int", seed=self.seed + 100)


# The five measured shapes, seeds 0..4 in this order, the 4096³ product
# with 8-bit E4M3 inputs (seed 5) and with int8 inputs and int32 output (seed 6),
# a batch of 64 products of 512³ (seed 7), 4096³ with B stored K×N (seed 8),
# 1024×1024×16384, whose 64 tiles the split plan divides along K (seed 9),
# the ragged shape with an odd K (rows only 2-byte aligned, a K tail of 1; seed 10),
# and the thin product 64×8192×8192 (64 × 64 tiles split along K; seed 11).
WORKLOADS = {
    "sq512_bf16_f32": Workload("sq512_bf16_f32", 512, 512, 512, "bf16", "f32", "normal", 0),
    "m1024_n4096_k4096_f16_f16": Workload("m1024_n4096_k4096_f16_f16", 1024, 4096, 4096, "f16", "f16",
                                          "normal", 1),
    "sq4096_bf16_bf16": Workload("sq4096_bf16_bf16", 4096, 4096, 4096, "bf16", "bf16", "normal", 2),
    "ragged_m1000_n3000_k2050_bf16_f32": Workload("ragged_m1000_n3000_k2050_bf16_f32", 1000, 3000, 2050,
                                                  "bf16", "f32", "uniform", 3),
    "skinny_m16_n8192_k8192_bf16_bf16": Workload("skinny_m16_n8192_k8192_bf16_bf16", 16, 8192, 8192,
                                                 "bf16", "bf16", "normal_scaled", 4),
    "sq4096_e4m3_bf16": Workload("sq4096_e4m3_bf16", 4096, 4096, 4096, "e4m3", "bf16", "normal", 5),
    "sq4096_i8_i32": Workload("sq4096_i8_i32", 4096, 4096, 4096, "i8", "i32", "int8", 6),
    "batch64_sq512_bf16_bf16": Workload("batch64_sq512_bf16_bf16", 512, 512, 512, "bf16", "bf16", "normal", 7, 64),
    "sq4096_nn_bf16_bf16": Workload("sq4096_nn_bf16_bf16", 4096, 4096, 4096, "bf16", "bf16", "normal", 8, 1, 1),
    "splitk_m1024_n1024_k16384_bf16_bf16": Workload("splitk_m1024_n1024_k16384_bf16_bf16", 1024, 1024, 16384,
                                                    "bf16", "bf16", "normal", 9),
    "oddk_m1000_n3000_k2049_bf16_f32": Workload("oddk_m1000_n3000_k2049_bf16_f32", 1000, 3000, 2049,
                                                "bf16", "f32", "uniform", 10),
    "thin_m64_n8192_k8192_bf16_bf16": Workload("thin_m64_n8192_k8192_bf16_bf16", 64, 8192, 8192,
                                               "bf16", "bf16", "normal", 11),
}


def _to_bf16_bits(x64: np.ndarray) -> np.ndarray:
    import torch  # CPU conversion only

    f32 = np.ascontiguousarray(x64, dtype=np.float32)
    t = torch.from_numpy(f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _to_f16_bits(x64: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x64).astype(np.float16).view(np.uint16)


def _to_fp8_bits(x64: np.ndarray, in_dtype: str) -> np.ndarray:
    import torch  # CPU conversion only

    f32 = np.ascontiguousarray(x64, dtype=np.float32)
    t = torch.from_numpy(f32).to(torch.float8_e4m3fn if in_dtype == "e4m3" else torch.float8_e5m2)
    return t.view(torch.uint8).numpy().copy()


def _to_i8_bits(x64: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x64, dtype=np.float64)
    if x.size and (not np.all(x == np.rint(x)) or x.min() < -128 or x.max() > 127):
        raise ValueError("int8 inputs must be integers in [-128, 127]")
    return x.astype(np.int8).view(np.uint8)


def round_bits(x64: np.ndarray, in_dtype: str) -> np.ndarray:
    """Round float64 values to the input format, returning raw bits."""
    if in_dtype == "bf16":
        return _to_bf16_bits(x64)
    if in_dtype == "f16":
        return _to_f16_bits(x64)
    if in_dtype in ("e4m3", "e5m2"):
        return _to_fp8_bits(x64, in_dtype)
    if in_dtype == "i8":
        return _to_i8_bits(x64)
    raise ValueError("in_dtype must be bf16, f16, e4m3, e5m2 or i8")


def _draw(rng: np.random.Generator, shape, dist: str, K: int) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(shape)
    if dist == "normal_scaled":
        return rng.normal(0.0, 1.0 / np.sqrt(K), shape)
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, shape)
    if dist == "int":
        return rng.integers(-4, 5, shape).astype(np.float64)
    if dist == "int8":
        return rng.integers(-128, 128, shape).astype(np.float64)
    raise ValueError("unknown distribution %r" % dist)


def make(M: int, N: int, K: int, in_dtype: str, dist: str, seed: int):
    """Return (a_bits (M,K), b_bits (N,K)): uint16 for 16-bit inputs, uint8 for 8-bit ones."""
    rng = np.random.default_rng(seed)
    a = _draw(rng, (M, K), dist, K)
    b = _draw(rng, (N, K), dist, K)
    return round_bits(a, in_dtype), round_bits(b, in_dtype)


def make_batched(Z: int, M: int, N: int, K: int, in_dtype: str, dist: str, seed: int):
    """Return (a_bits (Z,M,K), b_bits (Z,N,K)): all of A drawn first, then all of B."""
    a, b = make(Z * M, Z * N, K, in_dtype, dist, seed)
    return a.reshape(Z, M, K), b.reshape(Z, N, K)


def make_workload(w: Workload):
    """(a_bits, b_bits) of a workload: 2-D for one product, 3-D (Z, rows, K) for a batch."""
    if w.batch > 1:
        return make_batched(w.batch, w.M, w.N, w.K, w.in_dtype, w.dist, w.seed)
    return make(w.M, w.N, w.K, w.in_dtype, w.dist, w.seed)
