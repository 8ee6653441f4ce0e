"""Acceptance rules for a GPU result against the fp64 oracle (TEST INFRASTRUCTURE).

Rules, applied elementwise with E = |C_gpu - C_ref| and D = ‖A_i‖₂·‖B_j‖₂
(row i of A, row j of stored B, both in fp64 over all K):

* f32 output:       E <= 1e-3·D
* bf16 output:      E <= ulp_bf16(C_ref) + 1e-3·D
* f16 output:       E <= ulp_f16(C_ref) + 1e-3·D
* D == 0:           E == 0 (a zero row or column gives an exact zero)
* non-finite:       a non-finite C_ref must be matched exactly (same infinity);
                    a finite C_ref must give a finite result.
* integer-valued inputs: bit-exact against the oracle's RNE of C_ref, with
                    +0 and -0 treated as equal (``bit_exact``).

The 1e-3·D term holds for any fp32 summation order: the rounding error of a
K-term fp32 sum is at most γ_K·Σ|a_k b_k| <= γ_K·D (Cauchy–Schwarz), and
γ_K = K·2⁻²⁴/(1-K·2⁻²⁴) is below 1e-3 for K <= 16000.  "Chapter 7: Writing
custom kernels with Pallas", section 4.1', keeps the accumulator in fp32 and
rounds once at the end, which the ulp term of the 16-bit rules accounts for.

ulp is taken at the oracle value: ulp_bf16(x) = 2^(max(floor(log2|x|), -126) - 7),
ulp_f16(x) = 2^(max(floor(log2|x|), -14) - 10); at x = 0 the subnormal spacing.
"""
from __future__ import annotations

import numpy as np

from . import F16, BF16, F32, dtype_code

REL = 1e-3


def ulp(x: np.ndarray, out_dtype) -> np.ndarray:
    """Spacing of the output format at |x| (float64 array)."""
    code = dtype_code(out_dtype)
    x = np.abs(np.asarray(x, dtype=np.float64))
    if code == BF16:
        p, emin = 7, -126
    elif code == F16:
        p, emin = 10, -14
    elif code == F32:
        p, emin = 23, -126
    else:
        raise ValueError("unknown dtype")
    with np.errstate(divide="ignore", invalid="ignore"):
        _, e = np.frexp(x)            # x = m·2^e, m in [0.5, 1)
    ex = np.maximum(e.astype(np.int64) - 1, emin)
    ex = np.where(x == 0, emin, ex)
    return np.ldexp(1.0, (ex - p).astype(np.int32))


def bound(cref: np.ndarray, dnorm: np.ndarray, out_dtype) -> np.ndarray:
    """Allowed |C_gpu - C_ref| for each entry."""
    code = dtype_code(out_dtype)
    b = REL * dnorm
    if code in (BF16, F16):
        b = b + ulp(cref, code)
    return b


class Report:
    def __init__(self, ok, n, n_bad, worst_ratio, worst_index, detail=""):
        self.ok = ok
        self.n = n
        self.n_bad = n_bad
        self.worst_ratio = worst_ratio
        self.worst_index = worst_index
        self.detail = detail

    def __bool__(self):
        return bool(self.ok)

    def __repr__(self):
        return ("Report(ok=%s, n=%d, n_bad=%d, worst_err/bound=%.3g at %s%s)"
                % (self.ok, self.n, self.n_bad, self.worst_ratio, self.worst_index,
                   (", " + self.detail) if self.detail else ""))


def check(c_gpu: np.ndarray, cref: np.ndarray, dnorm: np.ndarray, out_dtype) -> Report:
    """Compare GPU values (as float64) with the oracle under the rules above.

    ``dnorm`` is ‖A_i‖·‖B_j‖ broadcast to ``cref``'s shape (or a matching array).
    """
    c = np.asarray(c_gpu, dtype=np.float64)
    r = np.asarray(cref, dtype=np.float64)
    d = np.broadcast_to(np.asarray(dnorm, dtype=np.float64), r.shape)
    if c.shape != r.shape:
        raise ValueError("shape mismatch %s vs %s" % (c.shape, r.shape))
    n = r.size
    if n == 0:
        return Report(True, 0, 0, 0.0, None)
    fin_r = np.isfinite(r)
    fin_c = np.isfinite(c)
    # non-finite reference: must match exactly (same infinity); NaN never passes
    bad_nf = (~fin_r) & ~((c == r) & ~np.isnan(r))
    # finite reference but non-finite result
    bad_nf |= fin_r & ~fin_c
    with np.errstate(invalid="ignore"):
        err = np.where(fin_r & fin_c, np.abs(c - r), 0.0)
    lim = np.where(fin_r, bound(np.where(fin_r, r, 0.0), d, out_dtype), 0.0)
    zero_d = fin_r & (d == 0)
    bad_zero = zero_d & (err != 0)
    bad_tol = fin_r & fin_c & ~zero_d & (err > lim)
    bad = bad_nf | bad_zero | bad_tol
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(lim > 0, err / lim, np.where(err > 0, np.inf, 0.0))
    ratio = np.where(bad_nf, np.inf, ratio)
    k = int(np.argmax(ratio))
    worst_idx = np.unravel_index(k, r.shape)
    n_bad = int(bad.sum())
    detail = ""
    if n_bad:
        detail = "gpu=%r ref=%r bound=%r" % (float(c.flat[k]), float(r.flat[k]), float(lim.flat[k]))
    return Report(n_bad == 0, n, n_bad, float(ratio.flat[k]), tuple(int(i) for i in worst_idx),
                  detail)


def bit_exact(gpu_bits: np.ndarray, ref_bits: np.ndarray, out_dtype) -> Report:
    """Bit equality, +0 == -0."""
    g = np.asarray(gpu_bits)
    r = np.asarray(ref_bits)
    if g.shape != r.shape:
        raise ValueError("shape mismatch")
    code = dtype_code(out_dtype)
    if code == F32:
        g = g.view(np.uint32) if g.dtype != np.uint32 else g
        r = r.view(np.uint32) if r.dtype != np.uint32 else r
        mag = np.uint32(0x7FFFFFFF)
    else:
        g = g.view(np.uint16) if g.dtype != np.uint16 else g
        r = r.view(np.uint16) if r.dtype != np.uint16 else r
        mag = np.uint16(0x7FFF)
    both_zero = ((g & mag) == 0) & ((r & mag) == 0)
    bad = (g != r) & ~both_zero
    n_bad = int(bad.sum())
    idx = None
    detail = ""
    if n_bad:
        k = int(np.argmax(bad))
        idx = tuple(int(i) for i in np.unravel_index(k, r.shape))
        detail = "gpu=0x%x ref=0x%x" % (int(g.flat[k]), int(r.flat[k]))
    return Report(n_bad == 0, r.size, n_bad, float(n_bad), idx, detail)
