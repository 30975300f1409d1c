"""GPU parity of every candidate plan the autotuner can install, and the plan search itself.

The plan search (miconv_find_plan) may install any candidate of the enumeration, so each
candidate of each pass of every workload (reduced shapes, both dtypes) is installed in turn
with miconv_plan_select and compared element by element with the oracle; integer-valued
inputs make every partial sum exact, so there the candidates must match bit for bit.  The
search is then run on several shapes: its results are ordered by time, every candidate
succeeds, the fastest is the plan later calls run, and those calls match the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, ConvShape, inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}
DEV = "cuda:0"

REDUCED = {
    "tiny": ConvShape(2, 3, 8, 8, 4, 3, 3, (1, 1), (1, 1), 8, 8),
    "resnet3x3": ConvShape(2, 64, 19, 19, 64, 3, 3, (1, 1), (1, 1), 19, 19),
    "proj1x1": ConvShape(2, 256, 24, 24, 192, 1, 1, (0, 0), (2, 2), 12, 12),
    "stem7x7": ConvShape(2, 3, 37, 37, 64, 7, 7, (3, 3), (2, 2), 19, 19),
    "deconv4x4": ConvShape(2, 96, 14, 14, 256, 4, 4, (1, 1), (2, 2), 7, 7),
    "deep3x3": ConvShape(3, 160, 14, 14, 160, 3, 3, (1, 1), (1, 1), 14, 14),
}

# public pass id of each pass name (deconvolution passes read the sizes in deconv order)
_PID = {"fwd": 0, "bwd_data": 1, "bwd_filter": 2, "deconv_fwd": 3, "deconv_bwd_data": 4, "deconv_bwd_filter": 5}


@pytest.fixture(scope="module")
def mc():
    import convolution_implicit_gemm_nchw_amd as m
    yield m
    m.plan_cache_clear()


def _say(*a):
    print(*a, flush=True)


def rel_err(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    d = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return d / m if m > 0 else d


def _sizes(pass_id, s):
    """The 13 sizes in the reading of the public pass."""
    if pass_id.startswith("deconv"):
        return (s.N, s.K, s.P, s.Q, s.C, s.R, s.S, s.pad[0], s.pad[1], s.stride[0], s.stride[1], s.H, s.W)
    return s.args13()


def _buffers(pass_id, s, d):
    """(in0, in1, out) in the reading of the pass's compute entry point; out NaN-filled."""
    if pass_id == "fwd":
        return d["x"], d["w"], torch.full(s.y_shape, float("nan"), device=DEV)
    if pass_id == "bwd_data":
        return d["dy"], d["w"], torch.full(s.x_shape, float("nan"), device=DEV)
    if pass_id == "bwd_filter":
        return d["x"], d["dy"], torch.full(s.w_shape, float("nan"), device=DEV)
    if pass_id == "deconv_fwd":
        return d["x_in"], d["w"], torch.full(s.x_shape, float("nan"), device=DEV)
    if pass_id == "deconv_bwd_data":
        return d["dout"], d["w"], torch.full(s.y_shape, float("nan"), device=DEV)
    return d["x_in"], d["dout"], torch.full(s.w_shape, float("nan"), device=DEV)


def _compute(mc, pass_id, s, d):
    a, b, out = _buffers(pass_id, s, d)
    if pass_id == "fwd":
        mc.conv2d_fwd(a, b, s.pad, s.stride, y=out)
    elif pass_id == "bwd_data":
        mc.conv2d_bwd_data(a, b, (s.H, s.W), s.pad, s.stride, dx=out)
    elif pass_id == "bwd_filter":
        mc.conv2d_bwd_filter(a, b, (s.R, s.S), s.pad, s.stride, dw=out)
    elif pass_id == "deconv_fwd":
        mc.deconv2d_fwd(a, b, (s.H, s.W), s.pad, s.stride, y=out)
    elif pass_id == "deconv_bwd_data":
        mc.deconv2d_bwd_data(a, b, (s.P, s.Q), s.pad, s.stride, dx=out)
    else:
        mc.deconv2d_bwd_filter(a, b, (s.R, s.S), s.pad, s.stride, dw=out)
    torch.cuda.synchronize()
    return out


def _oracle(pass_id, s, t):
    f = {k: v.float().numpy() for k, v in t.items()}
    if pass_id == "fwd":
        return oracle.conv2d_fwd(f["x"], f["w"], s.pad, s.stride)
    if pass_id == "bwd_data":
        return oracle.conv2d_bwd_data(f["dy"], f["w"], (s.H, s.W), s.pad, s.stride)
    if pass_id == "bwd_filter":
        return oracle.conv2d_bwd_filter(f["x"], f["dy"], (s.R, s.S), s.pad, s.stride)
    if pass_id == "deconv_fwd":
        return oracle.deconv2d_fwd(f["x_in"], f["w"], (s.H, s.W), s.pad, s.stride)
    if pass_id == "deconv_bwd_data":
        return oracle.deconv2d_bwd_data(f["dout"], f["w"], (s.P, s.Q), s.pad, s.stride)
    return oracle.deconv2d_bwd_filter(f["x_in"], f["dout"], (s.R, s.S), s.pad, s.stride)


CANDIDATE_CASES = [(n, dt, p) for n, wl in WORKLOADS.items() for dt in ("f32", "bf16") for p in wl.passes]


@pytest.mark.parametrize("name,dt,pass_id", CANDIDATE_CASES)
def test_every_candidate_plan_matches_oracle(mc, name, dt, pass_id):
    wl, s = WORKLOADS[name], REDUCED[name]
    code = mc.F32 if dt == "f32" else mc.BF16
    pid, sizes = _PID[pass_id], _sizes(pass_id, s)
    n, _ = mc.plan_candidates(pid, code, sizes)
    t = inputs(wl, dt, shape=s, seed_offset=71)
    ti = inputs(wl, dt, shape=s, integer=True, seed_offset=72)
    ref, refi = _oracle(pass_id, s, t), _oracle(pass_id, s, ti)
    d, di = {k: v.to(DEV) for k, v in t.items()}, {k: v.to(DEV) for k, v in ti.items()}
    try:
        for i in range(n):
            mc.plan_select(pid, code, sizes, i)
            desc = mc.plan_describe(pid, code, sizes)
            _say(f"[candidate {i}/{n}] {name} {dt} {pass_id} :: {desc}")
            got = _compute(mc, pass_id, s, d).cpu().numpy()
            assert not np.isnan(got).any(), "output elements left unwritten"
            err = rel_err(got, ref)
            _say(f"    rel err {err:.3e}")
            assert err <= TOL[dt]
            goti = _compute(mc, pass_id, s, di).cpu().numpy()
            assert np.array_equal(goti.astype(np.float64), refi)
    finally:
        mc.plan_select(pid, code, sizes, -1)


FIND_CASES = [("deep3x3", "bf16", "bwd_filter"), ("resnet3x3", "bf16", "fwd"), ("proj1x1", "bf16", "bwd_data"),
              ("deconv4x4", "f32", "deconv_fwd"), ("stem7x7", "f32", "bwd_filter")]


@pytest.mark.parametrize("name,dt,pass_id", FIND_CASES)
def test_find_plan_installs_the_fastest(mc, name, dt, pass_id):
    wl, s = WORKLOADS[name], REDUCED[name]
    code = mc.F32 if dt == "f32" else mc.BF16
    pid, sizes = _PID[pass_id], _sizes(pass_id, s)
    n, _ = mc.plan_candidates(pid, code, sizes)
    t = inputs(wl, dt, shape=s, seed_offset=73)
    d = {k: v.to(DEV) for k, v in t.items()}
    a, b, out = _buffers(pass_id, s, d)
    try:
        res = mc.find_plan(pid, a, b, out, sizes)
        for r in res:
            _say(f"[find] {name} {dt} {pass_id} #{r['index']} {r['time_ms']:.4f} ms status={r['status']} :: {r['plan']}")
        assert len(res) == n
        assert sorted(r["index"] for r in res) == list(range(n))
        assert all(r["status"] == 0 and r["time_ms"] > 0 for r in res)
        times = [r["time_ms"] for r in res]
        assert times == sorted(times)
        assert mc.plan_describe(pid, code, sizes) == res[0]["plan"]
        assert mc.plan_cache_entries()[0] >= 1
        err = rel_err(_compute(mc, pass_id, s, d).cpu().numpy(), _oracle(pass_id, s, t))
        _say(f"    after the search: rel err {err:.3e}")
        assert err <= TOL[dt]
        # the inputs are untouched by the search
        for k, v in t.items():
            assert torch.equal(d[k].cpu(), v)
    finally:
        mc.plan_select(pid, code, sizes, -1)
