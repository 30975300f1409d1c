"""conv2d_bwd_filter_noalloc: backward-filter with its split-K partial sums in the library's
static device scratch array instead of a caller workspace (for callers that cannot allocate).

Called through the C ABI (ctypes) and compared with conv2d_bwd_filter given a workspace of the
scratch capacity: the same plan, so bitwise the same dW, and within the bf16 / fp32 tolerance
of the oracle.  Calls run back to back on one device, the second with a smaller problem, so the
array holds the first call's partial sums when the second starts.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, ConvShape, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCRATCH = 128 << 20
TOL = {"f32": 1e-5, "bf16": 1e-2}


@pytest.fixture(scope="module")
def mc():
    import convolution_implicit_gemm_nchw_amd as m
    L = m.lib()
    L.conv2d_bwd_filter_noalloc.argtypes = [ctypes.c_int] * 14 + [ctypes.c_void_p] * 4
    L.conv2d_bwd_filter_noalloc.restype = ctypes.c_int
    return m


def _noalloc(mc, s, d, code, dw, stream):
    return mc.lib().conv2d_bwd_filter_noalloc(*s.args13(), code, d["x"].data_ptr(), d["dy"].data_ptr(),
                                              dw.data_ptr(), stream.cuda_stream)


def _rel(got, ref):
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


# (workload whose distributions are used, dtype, shape), each planned with split-K so the
# scratch array is used: the first needs 75.5 MB of partial sums (8 splits of 512 x 4608 fp32,
# the LDS-patch kernel), the second 0.9 MB (6 splits), the last two run the implicit-GEMM
# kernel in fp32 with 4 and 16 splits.
CASES = [
    ("deep3x3", "bf16", ConvShape(40, 512, 14, 14, 512, 3, 3, (1, 1), (1, 1), 14, 14)),
    ("resnet3x3", "bf16", ConvShape(6, 64, 20, 20, 64, 3, 3, (1, 1), (1, 1), 20, 20)),
    ("proj1x1", "f32", ConvShape(16, 256, 23, 23, 192, 1, 1, (0, 0), (2, 2), 12, 12)),
    ("stem7x7", "f32", ConvShape(8, 3, 64, 64, 64, 7, 7, (3, 3), (2, 2), 32, 32)),
]


def test_noalloc_matches_workspace_entry_point(mc):
    stream = torch.cuda.current_stream()
    for name, dt, s in CASES:
        t = inputs(WORKLOADS[name], dt, shape=s, seed_offset=41)
        d = {k: v.to(DEV) for k, v in t.items()}
        code = mc.dtype_code(d["x"])
        desc = mc.plan_describe(mc.BWD_FILTER, code, s.args13(), SCRATCH)
        print(f"[noalloc] {name} {dt} {s} :: {desc}", flush=True)
        need = mc.workspace_size(mc.BWD_FILTER, code, s.args13(), SCRATCH)
        assert 0 < need <= SCRATCH
        ws = torch.empty(SCRATCH, dtype=torch.uint8, device=DEV)
        ref = torch.full(s.w_shape, float("nan"), device=DEV)
        mc.conv2d_bwd_filter(d["x"], d["dy"], (s.R, s.S), s.pad, s.stride, dw=ref, workspace=ws)
        outs = []
        for _ in range(2):   # twice in a row on the shared array
            dw = torch.full(s.w_shape, float("nan"), device=DEV)
            assert _noalloc(mc, s, d, code, dw, stream) == 0
            outs.append(dw)
        torch.cuda.synchronize()
        for dw in outs:
            assert torch.equal(dw, ref)
        o = oracle.conv2d_bwd_filter(t["x"].float().numpy(), t["dy"].float().numpy(), (s.R, s.S), s.pad, s.stride)
        err = _rel(outs[0].cpu().double().numpy(), o)
        print(f"    rel err vs oracle {err:.3e}", flush=True)
        assert err <= TOL[dt]


def test_noalloc_second_call_smaller(mc):
    """A large call, then a smaller one with no synchronisation in between, on one stream:
    the second must not see the first one's partial sums."""
    stream = torch.cuda.current_stream()
    big_name, big_dt, big = CASES[0]
    small_name, small_dt, small = CASES[1]
    tb = {k: v.to(DEV) for k, v in inputs(WORKLOADS[big_name], big_dt, shape=big, seed_offset=43).items()}
    ts_host = inputs(WORKLOADS[small_name], small_dt, shape=small, seed_offset=44)
    ts = {k: v.to(DEV) for k, v in ts_host.items()}
    dw_big = torch.full(big.w_shape, float("nan"), device=DEV)
    dw_small = torch.full(small.w_shape, float("nan"), device=DEV)
    assert _noalloc(mc, big, tb, mc.BF16, dw_big, stream) == 0
    assert _noalloc(mc, small, ts, mc.BF16, dw_small, stream) == 0
    torch.cuda.synchronize()
    ws = torch.empty(SCRATCH, dtype=torch.uint8, device=DEV)
    ref_small = mc.conv2d_bwd_filter(ts["x"], ts["dy"], (small.R, small.S), small.pad, small.stride, workspace=ws)
    ref_big = mc.conv2d_bwd_filter(tb["x"], tb["dy"], (big.R, big.S), big.pad, big.stride, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(dw_small, ref_small)
    assert torch.equal(dw_big, ref_big)
    o = oracle.conv2d_bwd_filter(ts_host["x"].float().numpy(), ts_host["dy"].float().numpy(), (small.R, small.S),
                                 small.pad, small.stride)
    assert _rel(dw_small.cpu().double().numpy(), o) <= TOL["bf16"]


def test_noalloc_rejects_invalid_arguments(mc):
    """Validation happens before anything is enqueued, as for the workspace entry point."""
    L = mc.lib()
    x = torch.zeros(16, device=DEV)
    bad = (1, 1, 4, 4, 1, 3, 3, 0, 0, 1, 1, 3, 3)   # P, Q should be 2, 2
    assert L.conv2d_bwd_filter_noalloc(*bad, 0, x.data_ptr(), x.data_ptr(), x.data_ptr(), None) == 3
    ok = (1, 1, 4, 4, 1, 3, 3, 0, 0, 1, 1, 2, 2)
    assert L.conv2d_bwd_filter_noalloc(*ok, 0, None, x.data_ptr(), x.data_ptr(), None) == 1
