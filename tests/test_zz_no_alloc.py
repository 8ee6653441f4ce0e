"""gemm_bt_noalloc (the split plan with the library's own device scratch) against gemm_bt_ws, through the C-ABI.

Two calls in a row, the second smaller, each compared bit for bit with gemm_bt_ws on a zeroed workspace of its
own (same plan, same kernels) and checked against the oracle; then a shape that is not split (gemm_bt's plan).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import tolerance

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _dev(bits, in_dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(DT[in_dtype])


def _bits(c):
    return c.view(torch.int32) if c.dtype == torch.float32 else c.view(torch.int16)


def _both(gb, M, N, K, ind, outd, seed):
    a_bits, b_bits = synth.make(M, N, K, ind, "normal", seed)
    a, b = _dev(a_bits, ind), _dev(b_bits, ind)
    ic, oc = gb._torch_code(DT[ind]), gb._torch_code(DT[outd])
    s = torch.cuda.current_stream().cuda_stream
    c_na = torch.full((M, N), float("nan"), dtype=DT[outd], device="cuda")
    print("[case] noalloc", M, N, K, ind, outd, "seed", seed, flush=True)
    assert gb.gemm_bt_noalloc(a.data_ptr(), b.data_ptr(), c_na.data_ptr(), M, N, K, ic, oc, s) == gb.OK
    need = gb.gemm_bt_workspace_size(M, N, K, ic, oc)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
    c_ws = torch.full((M, N), float("nan"), dtype=DT[outd], device="cuda")
    assert gb.gemm_bt_ws(a.data_ptr(), b.data_ptr(), c_ws.data_ptr(), M, N, K, ic, oc, ws.data_ptr(), ws.numel(),
                         s) == gb.OK
    torch.cuda.synchronize()
    assert torch.equal(_bits(c_na), _bits(c_ws)), ("noalloc differs from gemm_bt_ws", M, N, K)
    cref, nA, nB = oracle.gemm_bt_ref(a_bits, b_bits, ind)
    rep = tolerance.check(c_na.cpu().to(torch.float64).numpy(), cref, np.outer(nA, nB), outd)
    assert rep.ok, rep
    return need


def test_noalloc_matches_gemm_bt_ws(gpu):
    # split twice in a row, the second product smaller (fewer tiles, more pieces each)
    assert _both(gpu, 1024, 1024, 16384, "bf16", "bf16", 31) > 0
    assert _both(gpu, 300, 700, 30002, "bf16", "f32", 32) > 0
    # a thin product: 64x64 tiles in pieces; rows 16-byte but not 128-byte aligned: the line ring in pieces
    assert _both(gpu, 64, 8192, 8192, "bf16", "bf16", 34) > 0
    assert _both(gpu, 1000, 1000, 8200, "bf16", "f32", 35) > 0
    # not split: the plain plan through the same entry point
    assert _both(gpu, 1000, 3000, 2050, "f16", "f16", 33) == 0
