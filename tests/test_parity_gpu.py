"""GPU parity: the HIP library against the CPU oracle, through the C ABI binding.

Tolerance (fixed by the target): err = max|gpu - oracle| / max|oracle| must be
<= 1e-5 for fp32 inputs and <= 1e-2 for bf16 inputs (the oracle is fed the
same bf16-rounded values the GPU sees).

- Reduced shapes of every workload (same C, K, R, S, pad, stride; smaller N, H,
  W so the GEMMs span several tiles with ragged tails) are compared element by
  element with the full oracle, in both dtypes, for every pass.
- Full workload shapes, launched exactly as the benchmark launches them, are
  compared on sampled outputs (random positions plus borders and corners)
  that the oracle evaluates one by one; integer-valued inputs make every
  partial sum exact, so those samples must match bit for bit; every output
  element must be written (NaN pre-fill), and the adjoint identity must hold
  over the whole tensors.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, ConvShape, Dist, as_dtype, draw, inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}
DEV = "cuda:0"


@pytest.fixture(scope="module")
def mc():
    import convolution_implicit_gemm_nchw_amd as m
    return m


def _say(*a):
    print(*a, flush=True)


def rel_err(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    d = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return d / m if m > 0 else d


def _np(t):
    return t.detach().float().cpu().numpy()


def _run_conv(mc, pass_id, s: ConvShape, t, ws=None):
    """One pass on the GPU; outputs are pre-filled with NaN so unwritten elements show."""
    if pass_id == "fwd":
        out = torch.full(s.y_shape, float("nan"), device=DEV)
        mc.conv2d_fwd(t["x"], t["w"], s.pad, s.stride, y=out, workspace=ws)
    elif pass_id == "bwd_data":
        out = torch.full(s.x_shape, float("nan"), device=DEV)
        mc.conv2d_bwd_data(t["dy"], t["w"], (s.H, s.W), s.pad, s.stride, dx=out, workspace=ws)
    elif pass_id == "bwd_filter":
        out = torch.full(s.w_shape, float("nan"), device=DEV)
        mc.conv2d_bwd_filter(t["x"], t["dy"], (s.R, s.S), s.pad, s.stride, dw=out, workspace=ws)
    elif pass_id == "deconv_fwd":  # deconvolution: x_in [N, K, P, Q], w [K, C, R, S] -> [N, C, H, W]
        out = torch.full(s.x_shape, float("nan"), device=DEV)
        mc.deconv2d_fwd(t["x_in"], t["w"], (s.H, s.W), s.pad, s.stride, y=out, workspace=ws)
    elif pass_id == "deconv_bwd_data":  # dout [N, C, H, W], w -> din [N, K, P, Q]
        out = torch.full(s.y_shape, float("nan"), device=DEV)
        mc.deconv2d_bwd_data(t["dout"], t["w"], (s.P, s.Q), s.pad, s.stride, dx=out, workspace=ws)
    else:  # deconv_bwd_filter: x_in [N, K, P, Q], dout [N, C, H, W] -> dw [K, C, R, S]
        out = torch.full(s.w_shape, float("nan"), device=DEV)
        mc.deconv2d_bwd_filter(t["x_in"], t["dout"], (s.R, s.S), s.pad, s.stride, dw=out, workspace=ws)
    torch.cuda.synchronize()
    return out


def _oracle_full(pass_id, s, t):
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


def _oracle_points(pass_id, s, t, idx):
    f = {k: v.float().numpy() for k, v in t.items()}
    if pass_id == "fwd":
        return oracle.conv2d_fwd_points(f["x"], f["w"], idx, s.pad, s.stride)
    if pass_id == "bwd_data":
        return oracle.conv2d_bwd_data_points(f["dy"], f["w"], (s.H, s.W), idx, s.pad, s.stride)
    if pass_id == "bwd_filter":
        return oracle.conv2d_bwd_filter_points(f["x"], f["dy"], (s.R, s.S), idx, s.pad, s.stride)
    if pass_id == "deconv_fwd":
        return oracle.conv2d_bwd_data_points(f["x_in"], f["w"], (s.H, s.W), idx, s.pad, s.stride)
    if pass_id == "deconv_bwd_data":
        return oracle.deconv2d_bwd_data_points(f["dout"], f["w"], (s.P, s.Q), idx, s.pad, s.stride)
    return oracle.deconv2d_bwd_filter_points(f["x_in"], f["dout"], (s.R, s.S), idx, s.pad, s.stride)


def _dev(t):
    return {k: v.to(DEV) for k, v in t.items()}


# ----------------------------------------------------------------------------- reduced shapes

REDUCED = {
    "tiny": ConvShape(2, 3, 8, 8, 4, 3, 3, (1, 1), (1, 1), 8, 8),
    "resnet3x3": ConvShape(2, 64, 19, 19, 64, 3, 3, (1, 1), (1, 1), 19, 19),
    "proj1x1": ConvShape(2, 256, 23, 23, 192, 1, 1, (0, 0), (2, 2), 12, 12),
    "stem7x7": ConvShape(2, 3, 37, 37, 64, 7, 7, (3, 3), (2, 2), 19, 19),
    "deconv4x4": ConvShape(2, 96, 14, 14, 256, 4, 4, (1, 1), (2, 2), 7, 7),
    "deep3x3": ConvShape(3, 160, 14, 14, 160, 3, 3, (1, 1), (1, 1), 14, 14),
}

REDUCED_CASES = [(n, dt, p) for n, wl in WORKLOADS.items() for dt in ("f32", "bf16")
                 for p in wl.passes]


@pytest.mark.parametrize("name,dt,pass_id", REDUCED_CASES)
def test_reduced_shapes_full_compare(mc, name, dt, pass_id):
    wl, s = WORKLOADS[name], REDUCED[name]
    t = inputs(wl, dt, shape=s)
    _say(f"[reduced] {name} {dt} {pass_id} {s}")
    got = _np(_run_conv(mc, pass_id, s, _dev(t)))
    ref = _oracle_full(pass_id, s, t)
    assert not np.isnan(got).any(), "output elements left unwritten"
    err = rel_err(got, ref)
    _say(f"    rel err {err:.3e}")
    assert err <= TOL[dt]


@pytest.mark.parametrize("name,dt,pass_id", [c for c in REDUCED_CASES if c[1] == "f32"])
def test_reduced_shapes_no_workspace(mc, name, dt, pass_id):
    """A zero workspace budget (filter read in place, no split-K) gives the same results."""
    wl, s = WORKLOADS[name], REDUCED[name]
    t = inputs(wl, dt, shape=s, seed_offset=7)
    empty = torch.empty(0, dtype=torch.uint8, device=DEV)
    _say(f"[no-ws] {name} {dt} {pass_id}")
    got = _np(_run_conv(mc, pass_id, s, _dev(t), ws=empty))
    err = rel_err(got, _oracle_full(pass_id, s, t))
    _say(f"    rel err {err:.3e}")
    assert err <= TOL[dt]


@pytest.mark.parametrize("name,dt,pass_id", [c for c in REDUCED_CASES if c[1] == "bf16"])
def test_reduced_shapes_integer_exact(mc, name, dt, pass_id):
    """Integer inputs in [-4, 4]: every product and partial sum is exact in fp32."""
    wl, s = WORKLOADS[name], REDUCED[name]
    t = inputs(wl, dt, shape=s, integer=True)
    _say(f"[int-exact] {name} {dt} {pass_id}")
    got = _np(_run_conv(mc, pass_id, s, _dev(t)))
    assert np.array_equal(got.astype(np.float64), _oracle_full(pass_id, s, t))


# ----------------------------------------------------------------------------- full workloads

def _sample_indices(shape, n, seed):
    total = int(np.prod(shape))
    g = np.random.Generator(np.random.PCG64(seed))
    idx = set(g.integers(0, total, n).tolist())
    # borders and corners of every spatial plane of the first and last images/filters
    A, B, H, W = shape
    for a in (0, A - 1):
        for b in (0, B - 1):
            for h in (0, H // 2, H - 1):
                for w in (0, 1, W // 2, W - 2, W - 1):
                    if 0 <= w < W:
                        idx.add(((a * B + b) * H + h) * W + w)
    return np.array(sorted(idx), dtype=np.int64)


FULL_CASES = [(n, dt, p) for n, wl in WORKLOADS.items() for dt in wl.dtypes for p in wl.passes]

# Full-size oracle results, computed once per (workload, dtype, pass, integer) and shared by the
# tests of this module (the whole deep3x3 step takes the oracle about 12 s on 16 host threads).
_ORACLE_CACHE = {}


def _oracle_full_cached(name, dt, pass_id, t, integer=False):
    key = (name, dt, pass_id, integer)
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE[key] = _oracle_full(pass_id, WORKLOADS[name].shape, t)
    return _ORACLE_CACHE[key]


@pytest.mark.parametrize("name,dt,pass_id", FULL_CASES)
def test_full_workload_full_compare(mc, name, dt, pass_id):
    """Every output element of every pass at the workload's full size, launched as the benchmark
    launches it (default workspace), against the full oracle."""
    wl = WORKLOADS[name]
    s = wl.shape
    t = inputs(wl, dt)
    pid = {"fwd": mc.FWD, "bwd_data": mc.BWD_DATA, "bwd_filter": mc.BWD_FILTER, "deconv_fwd": mc.DECONV_FWD,
           "deconv_bwd_data": mc.DECONV_BWD_DATA, "deconv_bwd_filter": mc.DECONV_BWD_FILTER}[pass_id]
    a = s.args13() if not wl.deconv else (s.N, s.K, s.P, s.Q, s.C, s.R, s.S, s.pad[0], s.pad[1], s.stride[0],
                                          s.stride[1], s.H, s.W)
    _say(f"[full] {name} {dt} {pass_id} :: {mc.plan_describe(pid, mc.dtype_code(t[next(iter(t))]), a)}")
    out = _run_conv(mc, pass_id, s, _dev(t))
    got = _np(out)
    del out
    assert not np.isnan(got).any(), "output elements left unwritten"
    ref = _oracle_full_cached(name, dt, pass_id, t)
    err = rel_err(got, ref)
    _say(f"    rel err {err:.3e} over {got.size} elements")
    assert err <= TOL[dt]


@pytest.mark.parametrize("name,dt,pass_id", [(n, WORKLOADS[n].dtypes[-1], p)
                                             for n in WORKLOADS for p in WORKLOADS[n].passes])
def test_full_workload_integer_exact(mc, name, dt, pass_id):
    """Integer inputs in [-4, 4] at full size: every partial sum is an exact integer below 2^24,
    so every element must equal the oracle bit for bit, whatever the summation order."""
    wl = WORKLOADS[name]
    s = wl.shape
    t = inputs(wl, dt, integer=True)
    _say(f"[full int-exact] {name} {dt} {pass_id}")
    out = _np(_run_conv(mc, pass_id, s, _dev(t)))
    ref = _oracle_full_cached(name, dt, pass_id, t, integer=True)
    assert np.array_equal(out.astype(np.float64), ref)


def _run_shape(pass_id, s):
    return {"fwd": s.y_shape, "bwd_data": s.x_shape, "bwd_filter": s.w_shape,
            "deconv_fwd": s.x_shape, "deconv_bwd_data": s.y_shape, "deconv_bwd_filter": s.w_shape}[pass_id]


@pytest.mark.parametrize("name,dt", [(n, dt) for n, wl in WORKLOADS.items() for dt in wl.dtypes
                                     if not wl.deconv])
def test_full_workload_adjoint_identity(mc, name, dt):
    """<dy, fwd(x,W)> = <bwd_data(dy,W), x> = <bwd_filter(x,dy), W>, over whole tensors."""
    wl = WORKLOADS[name]
    s = wl.shape
    t = inputs(wl, dt)
    d = _dev(t)
    _say(f"[adjoint] {name} {dt}")
    y = _run_conv(mc, "fwd", s, d).double()
    dx = _run_conv(mc, "bwd_data", s, d).double()
    dw = _run_conv(mc, "bwd_filter", s, d).double()
    x, w, dy = (d[k].double() for k in ("x", "w", "dy"))
    a = float((dy * y).sum())
    b = float((dx * x).sum())
    c = float((dw * w).sum())
    # each output is within TOL * max|output| of exact, so each inner product is
    # within TOL * max|out| * sum|other operand| of the exact (common) value
    bound = 2 * TOL[dt] * (float(y.abs().max()) * float(dy.abs().sum()) +
                           float(dx.abs().max()) * float(x.abs().sum()) +
                           float(dw.abs().max()) * float(w.abs().sum()))
    _say(f"    {a:.6e} {b:.6e} {c:.6e} bound {bound:.3e}")
    assert abs(a - b) <= bound and abs(a - c) <= bound


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_full_deconv_adjoint_identity(mc, dt):
    """<dout, deconv(x_in, w)> = <deconv_bwd_data(dout, w), x_in> = <deconv_bwd_filter(x_in, dout), w>."""
    wl = WORKLOADS["deconv4x4"]
    s = wl.shape
    d = _dev(inputs(wl, dt))
    _say(f"[deconv adjoint] {dt}")
    y = _run_conv(mc, "deconv_fwd", s, d).double()
    din = _run_conv(mc, "deconv_bwd_data", s, d).double()
    dw = _run_conv(mc, "deconv_bwd_filter", s, d).double()
    x, w, z = (d[k].double() for k in ("x_in", "w", "dout"))
    a, b, c = float((z * y).sum()), float((din * x).sum()), float((dw * w).sum())
    bound = 2 * TOL[dt] * (float(y.abs().max()) * float(z.abs().sum()) +
                           float(din.abs().max()) * float(x.abs().sum()) +
                           float(dw.abs().max()) * float(w.abs().sum()))
    _say(f"    {a:.6e} {b:.6e} {c:.6e} bound {bound:.3e}")
    assert abs(a - b) <= bound and abs(a - c) <= bound


# ----------------------------------------------------------------------------- fused forward epilogue

EPI_CASES = [
    dict(alpha=1.0, beta=0.0, bias=True, relu=True),
    dict(alpha=0.5, beta=1.0, bias=False, relu=False),
    dict(alpha=-1.5, beta=-0.25, bias=True, relu=True),
]


def _epi_args(t, s, case, seed, integer=False):
    K = s.K
    dist = Dist("int", -4, 4) if integer else Dist("uniform", -1, 1)
    bias = draw((K,), dist, seed) if case["bias"] else None
    y0 = draw(s.y_shape, dist, seed + 1)
    return bias, y0


def _run_fwd_ex(mc, s, t, case, bias, y0):
    y = y0.clone().to(DEV) if case["beta"] != 0.0 else torch.full(s.y_shape, float("nan"), device=DEV)
    mc.conv2d_fwd_ex(t["x"], t["w"], s.pad, s.stride, bias=None if bias is None else bias.to(DEV),
                     alpha=case["alpha"], beta=case["beta"], relu=case["relu"], y=y)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("case", range(len(EPI_CASES)))
@pytest.mark.parametrize("name,dt", [(n, dt) for n, wl in WORKLOADS.items() if not wl.deconv
                                     for dt in ("f32", "bf16")])
def test_fused_forward_reduced(mc, name, dt, case):
    """act(alpha*conv + beta*y + bias) against the oracle; with beta = 0 the NaN-filled y is not read."""
    wl, s, c = WORKLOADS[name], REDUCED[name], EPI_CASES[case]
    t = inputs(wl, dt, shape=s, seed_offset=31)
    bias, y0 = _epi_args(t, s, c, 91)
    _say(f"[fused fwd] {name} {dt} {c} :: {mc.plan_describe(mc.FWD, mc.dtype_code(t['x']), s.args13())}")
    got = _np(_run_fwd_ex(mc, s, _dev(t), c, bias, y0))
    ref = oracle.conv2d_fwd_ex(t["x"].float().numpy(), t["w"].float().numpy(), s.pad, s.stride,
                               bias=None if bias is None else bias.numpy(), alpha=c["alpha"], beta=c["beta"],
                               y_prev=y0.numpy(), relu=c["relu"])
    assert not np.isnan(got).any()
    err = rel_err(got, ref)
    _say(f"    rel err {err:.3e}")
    assert err <= TOL[dt]


@pytest.mark.parametrize("sh", [REDUCED["resnet3x3"], REDUCED["deep3x3"], REDUCED["stem7x7"],
                                ConvShape(1, 32, 9, 14, 64, 5, 3, (2, 0), (1, 1), 9, 12),
                                ConvShape(2, 40, 18, 22, 64, 4, 4, (2, 2), (2, 2), 10, 12)])
def test_fused_forward_integer_exact(mc, sh):
    """Integer inputs, bias and previous output, alpha 2, beta -1: every value is an exact integer."""
    c = dict(alpha=2.0, beta=-1.0, bias=True, relu=True)
    t = inputs(WORKLOADS["deep3x3"], "bf16", shape=sh, integer=True, seed_offset=32)
    bias, y0 = _epi_args(t, sh, c, 93, integer=True)
    _say(f"[fused fwd int] {sh}")
    got = _np(_run_fwd_ex(mc, sh, _dev(t), c, bias, y0))
    ref = oracle.conv2d_fwd_ex(t["x"].float().numpy(), t["w"].float().numpy(), sh.pad, sh.stride,
                               bias=bias.numpy(), alpha=2.0, beta=-1.0, y_prev=y0.numpy(), relu=True)
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("name,dt", [("resnet3x3", "bf16"), ("proj1x1", "f32"), ("deep3x3", "bf16")])
def test_fused_forward_full_sampled(mc, name, dt):
    wl, s, c = WORKLOADS[name], WORKLOADS[name].shape, EPI_CASES[2]
    t = inputs(wl, dt)
    bias, y0 = _epi_args(t, s, c, 95)
    _say(f"[fused fwd full] {name} {dt}")
    y = _run_fwd_ex(mc, s, _dev(t), c, bias, y0)
    got = _np(y).ravel()
    idx = _sample_indices(s.y_shape, 1024, 29)
    ref = oracle.conv2d_fwd_ex_points(t["x"].float().numpy(), t["w"].float().numpy(), idx, s.pad, s.stride,
                                      bias=bias.numpy(), alpha=c["alpha"], beta=c["beta"], y_prev=y0.numpy(),
                                      relu=c["relu"])
    err = rel_err(got[idx], ref)
    _say(f"    sampled rel err {err:.3e}")
    assert err <= TOL[dt]


@pytest.mark.parametrize("case", [0, 1])
@pytest.mark.parametrize("name,dt", [("resnet3x3", "bf16"), ("deep3x3", "bf16"), ("proj1x1", "f32"),
                                     ("stem7x7", "bf16"), ("stem7x7", "f32"), ("patch64", "bf16")])
def test_fused_forward_bf16_output(mc, name, dt, case):
    """bf16 y is the fp32-output result rounded to nearest even, bit for bit (the same fp32
    accumulation, one rounding at the store), and within the bf16 tolerance of the oracle."""
    if name == "patch64":   # 64 filter rows on the patch kernel, ragged row tiles
        wl, s = WORKLOADS["resnet3x3"], ConvShape(2, 64, 20, 24, 64, 3, 3, (1, 1), (1, 1), 20, 24)
    else:
        wl, s = WORKLOADS[name], REDUCED[name]
    c = [dict(alpha=1.0, beta=0.0, bias=True, relu=True), dict(alpha=0.5, beta=1.0, bias=True, relu=False)][case]
    t = inputs(wl, dt, shape=s, seed_offset=33)
    bias, y0 = _epi_args(t, s, c, 97)
    d = _dev(t)
    b = bias.to(DEV)
    _say(f"[fused fwd bf16 out] {name} {dt} {c} :: {mc.plan_describe(mc.FWD, mc.dtype_code(t['x']), s.args13())}")
    y0b = y0.to(torch.bfloat16)
    yb = y0b.clone().to(DEV) if c["beta"] else torch.full(s.y_shape, float("nan"), device=DEV).to(torch.bfloat16)
    mc.conv2d_fwd_ex(d["x"], d["w"], s.pad, s.stride, bias=b, alpha=c["alpha"], beta=c["beta"], relu=c["relu"], y=yb)
    yf = y0b.float().to(DEV) if c["beta"] else torch.full(s.y_shape, float("nan"), device=DEV)
    mc.conv2d_fwd_ex(d["x"], d["w"], s.pad, s.stride, bias=b, alpha=c["alpha"], beta=c["beta"], relu=c["relu"], y=yf)
    torch.cuda.synchronize()
    assert torch.equal(yb.view(torch.int16), yf.to(torch.bfloat16).view(torch.int16))
    ref = oracle.conv2d_fwd_ex(t["x"].float().numpy(), t["w"].float().numpy(), s.pad, s.stride, bias=bias.numpy(),
                               alpha=c["alpha"], beta=c["beta"], y_prev=y0b.float().numpy(), relu=c["relu"])
    err = rel_err(yb.float().cpu().numpy(), ref)
    _say(f"    rel err {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("name,dt", [("resnet3x3", "bf16"), ("stem7x7", "f32"), ("deep3x3", "bf16")])
def test_concurrent_backward_passes_match_serial(mc, name, dt):
    """Backward-data and backward-filter on two streams with separate workspaces (the bench's
    schedule) give exactly the results of running them in order on one stream."""
    wl = WORKLOADS[name]
    s = wl.shape
    d = _dev(inputs(wl, dt))
    _say(f"[two streams] {name} {dt}")
    dx1 = _run_conv(mc, "bwd_data", s, d)
    dw1 = _run_conv(mc, "bwd_filter", s, d)
    need = max(mc.workspace_size(mc.BWD_DATA, mc.dtype_code(d["x"]), s.args13()),
               mc.workspace_size(mc.BWD_FILTER, mc.dtype_code(d["x"]), s.args13()), 1)
    ws_a = torch.empty(need, dtype=torch.uint8, device=DEV)
    ws_b = torch.empty(need, dtype=torch.uint8, device=DEV)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream(device=DEV)
    dx2 = torch.full(s.x_shape, float("nan"), device=DEV)
    dw2 = torch.full(s.w_shape, float("nan"), device=DEV)
    ready = torch.cuda.Event()
    ready.record(main)
    side.wait_event(ready)
    for _ in range(3):   # repeated, so the two streams overlap
        mc.conv2d_bwd_filter(d["x"], d["dy"], (s.R, s.S), s.pad, s.stride, dw=dw2, workspace=ws_b, stream=side)
        mc.conv2d_bwd_data(d["dy"], d["w"], (s.H, s.W), s.pad, s.stride, dx=dx2, workspace=ws_a, stream=main)
    done = torch.cuda.Event()
    done.record(side)
    main.wait_event(done)
    torch.cuda.synchronize()
    assert torch.equal(dx1, dx2) and torch.equal(dw1, dw2)


_OUT_SHAPE = {"fwd": "y_shape", "bwd_data": "x_shape", "bwd_filter": "w_shape", "deconv_fwd": "x_shape",
              "deconv_bwd_data": "y_shape", "deconv_bwd_filter": "w_shape"}


def _issue(mc, pass_id, s: ConvShape, t, out, ws):
    """Enqueue one pass on the current stream into a preallocated output (no allocation, no sync)."""
    if pass_id == "fwd":
        mc.conv2d_fwd(t["x"], t["w"], s.pad, s.stride, y=out, workspace=ws)
    elif pass_id == "bwd_data":
        mc.conv2d_bwd_data(t["dy"], t["w"], (s.H, s.W), s.pad, s.stride, dx=out, workspace=ws)
    elif pass_id == "bwd_filter":
        mc.conv2d_bwd_filter(t["x"], t["dy"], (s.R, s.S), s.pad, s.stride, dw=out, workspace=ws)
    elif pass_id == "deconv_fwd":
        mc.deconv2d_fwd(t["x_in"], t["w"], (s.H, s.W), s.pad, s.stride, y=out, workspace=ws)
    elif pass_id == "deconv_bwd_data":
        mc.deconv2d_bwd_data(t["dout"], t["w"], (s.P, s.Q), s.pad, s.stride, dx=out, workspace=ws)
    else:
        mc.deconv2d_bwd_filter(t["x_in"], t["dout"], (s.R, s.S), s.pad, s.stride, dw=out, workspace=ws)


@pytest.mark.parametrize("name,dt", [("resnet3x3", "bf16"), ("stem7x7", "f32"), ("deconv4x4", "bf16")])
def test_graph_replays_match_eager(mc, name, dt):
    """Every pass of a workload, sharing one workspace, captured into one HIP graph: each of
    several replays (with eager work and synchronisations between them, and the outputs poisoned
    before each) gives bitwise the eager results.  The library issues only kernel launches on the
    caller's stream, so a step can be recorded once and replayed."""
    wl = WORKLOADS[name]
    s = wl.shape
    d = _dev(inputs(wl, dt))
    eager = {p: _run_conv(mc, p, s, d) for p in wl.passes}
    code = mc.dtype_code(next(iter(d.values())))
    a13 = s.args13()
    d13 = (s.N, s.K, s.P, s.Q, s.C, s.R, s.S, s.pad[0], s.pad[1], s.stride[0], s.stride[1], s.H, s.W)
    pid = {"fwd": mc.FWD, "bwd_data": mc.BWD_DATA, "bwd_filter": mc.BWD_FILTER, "deconv_fwd": mc.DECONV_FWD,
           "deconv_bwd_data": mc.DECONV_BWD_DATA, "deconv_bwd_filter": mc.DECONV_BWD_FILTER}
    need = max(max(mc.workspace_size(pid[p], code, d13 if p.startswith("deconv") else a13) for p in wl.passes), 1)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    outs = {p: torch.empty(getattr(s, _OUT_SHAPE[p]), dtype=torch.float32, device=DEV) for p in wl.passes}
    _say(f"[graph] {name} {dt} passes {wl.passes} ws {need}")
    side = torch.cuda.Stream(device=DEV)   # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # one eager run on the capture stream first
        for p in wl.passes:
            _issue(mc, p, s, d, outs[p], ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for p in wl.passes:
            _issue(mc, p, s, d, outs[p], ws)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs.values():
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for p in wl.passes:
            assert torch.equal(outs[p], eager[p]), f"replay {rep}, {p}"
        _run_conv(mc, wl.passes[0], s, d)   # eager work between replays
    del g


def test_largest_accepted_tensors(mc):
    """The size limit: every tensor, and its fp32 counterpart, must stay under 2 GiB.  With N=127,
    C=K=64, 256x256 images and a 3x3 filter (pad 1), x and dy are 1.07 GB in bf16 and y and dx
    2.13 GB in fp32, just under the limit (N=128 is rejected).  All three passes, sampled outputs
    against the oracle's point evaluations, corners of the first and last image included."""
    s = ConvShape(127, 64, 256, 256, 64, 3, 3, (1, 1), (1, 1), 256, 256)
    big = ConvShape(128, 64, 256, 256, 64, 3, 3, (1, 1), (1, 1), 256, 256)
    with pytest.raises(ValueError, match="status 10"):
        mc.workspace_size(mc.FWD, 1, big.args13())
    assert 4 * s.N * s.C * s.H * s.W < 2 ** 31
    _say(f"[largest] drawing inputs {s}")
    t = {"x": as_dtype(draw(s.x_shape, Dist("relu_normal"), 911), "bf16"),
         "w": as_dtype(draw(s.w_shape, Dist("normal", float(np.sqrt(2.0 / (64 * 9)))), 912), "bf16"),
         "dy": as_dtype(draw(s.y_shape, Dist("normal", 0.01), 913), "bf16")}
    d = _dev(t)
    for pass_id, npts in (("fwd", 1024), ("bwd_data", 1024), ("bwd_filter", 256)):
        _say(f"[largest] {pass_id}")
        out = _run_conv(mc, pass_id, s, d)
        assert not torch.isnan(out).any().item(), "output elements left unwritten"
        idx = _sample_indices(out.shape, npts, 23)
        got = out.view(-1)[torch.from_numpy(idx).to(DEV)].cpu().double().numpy()
        del out
        ref = _oracle_points(pass_id, s, t, idx)
        err = rel_err(got, ref)
        _say(f"    sampled rel err {err:.3e} over {idx.size} points")
        assert err <= TOL["bf16"]


# ----------------------------------------------------------------------------- exact special cases

@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("sh", [
    ConvShape(2, 16, 11, 9, 16, 3, 2, (1, 0), (1, 1), 11, 8),
    ConvShape(1, 8, 15, 15, 8, 7, 7, (3, 3), (2, 2), 8, 8),
    ConvShape(2, 64, 12, 12, 64, 3, 3, (1, 1), (1, 1), 12, 12),
])
def test_delta_filter_is_exact_shift(mc, dt, sh):
    x = as_dtype(draw(sh.x_shape, Dist("uniform", -1, 1), 61), dt)
    for r0, s0 in ((0, sh.S - 1), (sh.R - 1, 0), (sh.R // 2, sh.S // 2)):
        w = torch.zeros(sh.w_shape)
        for c in range(sh.C):
            w[c, c, r0, s0] = 1.0
        _say(f"[delta] {dt} {sh} tap ({r0},{s0})")
        y = _np(mc.conv2d_fwd(x.to(DEV), as_dtype(w, dt).to(DEV), sh.pad, sh.stride))
        ref = oracle.conv2d_fwd(x.float().numpy(), w.numpy(), sh.pad, sh.stride)
        assert np.array_equal(y.astype(np.float64), ref)


def test_bwd_filter_is_deterministic(mc):
    for name, dt in (("deep3x3", "bf16"), ("resnet3x3", "bf16"), ("resnet3x3", "f32"), ("stem7x7", "f32")):
        wl = WORKLOADS[name]
        s = wl.shape
        d = _dev(inputs(wl, dt))
        _say(f"[determinism] {name} {dt}")
        a = _run_conv(mc, "bwd_filter", s, d)
        b = _run_conv(mc, "bwd_filter", s, d)
        assert torch.equal(a, b)


# ----------------------------------------------------------------------------- edge shapes

EDGE = [
    ConvShape(1, 1, 1, 1, 1, 1, 1, (0, 0), (1, 1), 1, 1),
    ConvShape(1, 2, 3, 3, 2, 3, 3, (4, 4), (3, 3), 3, 3),          # pad larger than the filter
    ConvShape(1, 1, 5, 7, 2, 5, 7, (0, 0), (1, 1), 1, 1),          # H == R and W == S
    ConvShape(1, 3, 11, 10, 5, 5, 3, (2, 1), (3, 2), 4, 5),        # stride 3 x 2, R != S, floor cases
    ConvShape(2, 5, 9, 8, 7, 3, 3, (1, 0), (2, 2), 5, 3),
    ConvShape(3, 9, 6, 6, 33, 1, 1, (0, 0), (2, 2), 3, 3),          # 1x1 stride 2, ragged C/K
    ConvShape(1, 40, 4, 12, 70, 4, 3, (0, 2), (1, 1), 1, 14),
]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("sh", EDGE)
def test_edge_shapes(mc, dt, sh):
    wl = WORKLOADS["tiny"]
    t = inputs(wl, dt, shape=sh, seed_offset=3)
    for pass_id in ("fwd", "bwd_data", "bwd_filter"):
        _say(f"[edge] {dt} {pass_id} {sh}")
        got = _np(_run_conv(mc, pass_id, sh, _dev(t)))
        err = rel_err(got, _oracle_full(pass_id, sh, t))
        assert not np.isnan(got).any()
        assert err <= TOL[dt], (pass_id, err)


def _random_shapes(count, seed, family):
    """Seeded shapes.  generic: any sizes, pads and strides 1-3; fewc: 1-4 input channels,
    strides 1-2 (the vector-ALU backward-data); patch: stride 1, 32-multiple channels, even
    widths, pads below the filter size (the bf16 LDS-patch kernels)."""
    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    while len(out) < count:
        N = int(g.integers(1, 4))
        H, W = int(g.integers(1, 22)), int(g.integers(1, 22))
        R, S = int(g.integers(1, 6)), int(g.integers(1, 6))
        if family == "patch":
            C, K = 32 * int(g.integers(1, 4)), 32 * int(g.integers(1, 5)) - int(g.integers(0, 2)) * 7
            W += W % 2
            ph, pw, sh, sw = int(g.integers(0, R)), int(g.integers(0, S)), 1, 1
        else:
            C = int(g.integers(1, 5)) if family == "fewc" else int(g.integers(1, 72))
            K = int(g.integers(1, 72))
            ph, pw = int(g.integers(0, R + 1)), int(g.integers(0, S + 1))
            smax = 3 if family == "fewc" else 4
            sh, sw = int(g.integers(1, smax)), int(g.integers(1, smax))
        P, Q = (H + 2 * ph - R) // sh + 1, (W + 2 * pw - S) // sw + 1
        if P >= 1 and Q >= 1:
            out.append(ConvShape(N, C, H, W, K, R, S, (ph, pw), (sh, sw), P, Q))
    return out


RANDOM_SHAPES = (_random_shapes(16, 2024, "generic") + _random_shapes(8, 2025, "fewc") +
                 _random_shapes(12, 2026, "patch"))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("sh", RANDOM_SHAPES)
def test_random_small_shapes(mc, sh, dt):
    """Seeded random sizes, pads and strides (1-3): every pass against the full oracle."""
    t = inputs(WORKLOADS["tiny"], dt, shape=sh, seed_offset=5)
    for pass_id in ("fwd", "bwd_data", "bwd_filter"):
        desc = mc.plan_describe({"fwd": mc.FWD, "bwd_data": mc.BWD_DATA, "bwd_filter": mc.BWD_FILTER}[pass_id],
                                mc.dtype_code(t["x"]), sh.args13())
        _say(f"[random] {dt} {pass_id} {sh} :: {desc.split(' gemm')[0]}")
        got = _np(_run_conv(mc, pass_id, sh, _dev(t)))
        assert not np.isnan(got).any()
        err = rel_err(got, _oracle_full(pass_id, sh, t))
        assert err <= TOL[dt], (pass_id, err)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("i", range(0, len(RANDOM_SHAPES), 3))
def test_random_fused_forward(mc, i, dt):
    """The fused forward on the random shapes with seeded alpha, beta, bias, ReLU and output type."""
    sh = RANDOM_SHAPES[i]
    g = np.random.Generator(np.random.PCG64(3000 + i))
    c = dict(alpha=float(g.uniform(-2, 2)), beta=float(g.choice([0.0, 1.0, -0.5])), bias=bool(g.integers(0, 2)),
             relu=bool(g.integers(0, 2)))
    out_bf16 = bool(g.integers(0, 2))
    t = inputs(WORKLOADS["tiny"], dt, shape=sh, seed_offset=6)
    bias, y0 = _epi_args(t, sh, c, 3100 + i)
    if out_bf16:
        y0 = y0.to(torch.bfloat16)
    _say(f"[random fused] {dt} {sh} {c} bf16_out={out_bf16}")
    y = y0.clone().to(DEV) if c["beta"] else torch.full(sh.y_shape, float("nan"), device=DEV).to(y0.dtype)
    d = _dev(t)
    mc.conv2d_fwd_ex(d["x"], d["w"], sh.pad, sh.stride, bias=None if bias is None else bias.to(DEV), alpha=c["alpha"],
                     beta=c["beta"], relu=c["relu"], y=y)
    torch.cuda.synchronize()
    ref = oracle.conv2d_fwd_ex(t["x"].float().numpy(), t["w"].float().numpy(), sh.pad, sh.stride,
                               bias=None if bias is None else bias.numpy(), alpha=c["alpha"], beta=c["beta"],
                               y_prev=y0.float().numpy(), relu=c["relu"])
    got = y.float().cpu().numpy()
    assert not np.isnan(got).any()
    assert rel_err(got, ref) <= (TOL["bf16"] if out_bf16 else TOL[dt])


def test_sentence_cnn_shape(mc):
    """The conv1d-like shape the SystemDS page special-cases (W == S), 10% dense input."""
    s = ConvShape(1, 1, 2060, 300, 500, 5, 300, (0, 0), (1, 1), 2056, 1)
    g = np.random.Generator(np.random.PCG64(71))
    x = torch.from_numpy((g.uniform(-1, 1, s.x_shape) * (g.random(s.x_shape) < 0.1)).astype(np.float32))
    t = {"x": x, "w": draw(s.w_shape, Dist("uniform", -1, 1), 72),
         "dy": draw(s.y_shape, Dist("uniform", -1, 1), 73)}
    for pass_id in ("fwd", "bwd_data", "bwd_filter"):
        _say(f"[sentence-cnn] {pass_id}")
        out = _run_conv(mc, pass_id, s, _dev(t))
        got = _np(out).ravel()
        idx = np.unique(np.random.Generator(np.random.PCG64(74)).integers(0, got.size, 400))
        err = rel_err(got[idx], _oracle_points(pass_id, s, t, idx))
        _say(f"    sampled rel err {err:.3e}")
        assert err <= 1e-5


def test_binding_rejects_bad_arguments(mc):
    x = torch.zeros((1, 2, 4, 4), device=DEV)
    w = torch.zeros((3, 2, 3, 3), device=DEV, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mc.conv2d_fwd(x, w)                      # mixed dtypes
    with pytest.raises(ValueError):
        mc.conv2d_fwd(x.half(), w.half())        # unsupported dtype
    w = torch.zeros((3, 2, 3, 3), device=DEV)
    y = torch.zeros((1, 3, 2, 2), device=DEV)
    with pytest.raises(ValueError):
        mc.conv2d_fwd(x, w, y=x.view(-1)[:12].view(1, 3, 2, 2))   # output aliases the input
    mc.conv2d_fwd(x, w, y=y)
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------- stride-1 patch path

PATCH_SHAPES = [
    ConvShape(2, 64, 20, 24, 96, 3, 3, (1, 1), (1, 1), 20, 24),    # 16-byte row loads, ragged row tiles
    ConvShape(1, 32, 9, 14, 64, 5, 3, (2, 0), (1, 1), 9, 12),      # R != S, 4-byte row loads
    ConvShape(2, 96, 7, 12, 288, 1, 3, (0, 1), (1, 1), 7, 12),     # 1x3, 8-byte loads, ragged 128-row tile
    ConvShape(1, 64, 30, 64, 64, 3, 3, (1, 1), (1, 1), 30, 64),    # 64-row tile, 7 output rows per tile
    ConvShape(3, 32, 6, 6, 32, 3, 3, (0, 0), (1, 1), 4, 4),        # no padding, 2-byte-aligned rows
    ConvShape(2, 128, 14, 14, 160, 3, 3, (1, 1), (1, 1), 14, 14),  # whole-image tiles, ragged rows
    # more tiles than resident work-groups: each work-group runs several tiles
    ConvShape(600, 32, 8, 8, 96, 3, 3, (1, 1), (1, 1), 8, 8),
    ConvShape(300, 32, 8, 8, 160, 3, 3, (1, 1), (1, 1), 8, 8),     # two filter-row tiles, the second ragged
    ConvShape(2, 256, 8, 8, 256, 3, 3, (1, 1), (1, 1), 8, 8),      # large filter: tiled fragment copy
    # 5x5 with 128-row tiles: 8-byte fill loads, one output row per tile to keep the fill items
    # within 512
    ConvShape(1, 32, 12, 96, 160, 5, 5, (2, 2), (1, 1), 12, 96),
]


@pytest.mark.parametrize("pass_id", ["fwd", "bwd_data"])
@pytest.mark.parametrize("sh", PATCH_SHAPES)
def test_patch_path_full_compare(mc, sh, pass_id):
    pid = mc.FWD if pass_id == "fwd" else mc.BWD_DATA
    desc = mc.plan_describe(pid, mc.BF16, sh.args13())
    assert "algo=patch" in desc, desc
    wl = WORKLOADS["deep3x3"]
    t = inputs(wl, "bf16", shape=sh, seed_offset=11)
    _say(f"[patch] {pass_id} {sh} :: {desc}")
    got = _np(_run_conv(mc, pass_id, sh, _dev(t)))
    assert not np.isnan(got).any()
    err = rel_err(got, _oracle_full(pass_id, sh, t))
    _say(f"    rel err {err:.3e}")
    assert err <= TOL["bf16"]
    ti = inputs(wl, "bf16", shape=sh, integer=True, seed_offset=12)
    got = _np(_run_conv(mc, pass_id, sh, _dev(ti)))
    assert np.array_equal(got.astype(np.float64), _oracle_full(pass_id, sh, ti))


# The tail form: 128 filter rows, 3x3, tiles of 193..208 pixels computed as six 32-pixel
# blocks and one 16-pixel block on 16x16x32 MFMAs.  (shape, passes whose plan takes it)
TAIL_SHAPES = [
    (ConvShape(2, 96, 14, 14, 160, 3, 3, (1, 1), (1, 1), 14, 14), ("fwd", "bwd_data")),   # 196 pixels, ragged rows
    (ConvShape(1, 128, 20, 10, 160, 3, 3, (1, 1), (1, 1), 20, 10), ("fwd", "bwd_data")),  # 200 pixels
    (ConvShape(2, 64, 9, 22, 136, 3, 3, (1, 1), (1, 1), 9, 22), ("fwd",)),                # 198 pixels, ragged rows
    (ConvShape(2, 160, 11, 18, 96, 3, 3, (1, 1), (1, 1), 11, 18), ("bwd_data",)),         # 198 pixels
    (ConvShape(3, 96, 16, 14, 160, 3, 3, (0, 1), (1, 1), 14, 14), ("fwd",)),              # unequal pads
    # more tiles than resident work-groups (each work-group runs two tiles)
    (ConvShape(300, 128, 14, 14, 160, 3, 3, (1, 1), (1, 1), 14, 14), ("fwd",)),
]


@pytest.mark.parametrize("case", range(len(TAIL_SHAPES)))
def test_patch_tail_form(mc, case):
    sh, passes = TAIL_SHAPES[case]
    wl = WORKLOADS["deep3x3"]
    for pass_id in passes:
        pid = mc.FWD if pass_id == "fwd" else mc.BWD_DATA
        desc = mc.plan_describe(pid, mc.BF16, sh.args13())
        assert "algo=patch" in desc and "form=tail16" in desc, desc
        t = inputs(wl, "bf16", shape=sh, seed_offset=41)
        _say(f"[patch tail] {pass_id} {sh} :: {desc}")
        got = _np(_run_conv(mc, pass_id, sh, _dev(t)))
        assert not np.isnan(got).any()
        err = rel_err(got, _oracle_full(pass_id, sh, t))
        _say(f"    rel err {err:.3e}")
        assert err <= TOL["bf16"]
        ti = inputs(wl, "bf16", shape=sh, integer=True, seed_offset=42)
        got = _np(_run_conv(mc, pass_id, sh, _dev(ti)))
        assert np.array_equal(got.astype(np.float64), _oracle_full(pass_id, sh, ti))


BWDF_PATCH_SHAPES = [PATCH_SHAPES[0], ConvShape(2, 96, 7, 12, 288, 1, 1, (0, 0), (1, 1), 7, 12),
                     PATCH_SHAPES[2], PATCH_SHAPES[3], PATCH_SHAPES[5],
                     ConvShape(3, 64, 10, 10, 64, 3, 3, (1, 1), (1, 1), 10, 10),
                     ConvShape(2, 64, 9, 8, 200, 2, 3, (0, 1), (1, 1), 8, 8)]


@pytest.mark.parametrize("budget", ["plan", "none"])
@pytest.mark.parametrize("sh", BWDF_PATCH_SHAPES)
def test_patch_bwd_filter_full_compare(mc, sh, budget):
    ws = torch.empty(0, dtype=torch.uint8, device=DEV) if budget == "none" else None
    desc = mc.plan_describe(mc.BWD_FILTER, mc.BF16, sh.args13(), 0 if budget == "none" else 10 ** 9)
    assert "algo=patch" in desc, desc
    wl = WORKLOADS["deep3x3"]
    t = inputs(wl, "bf16", shape=sh, seed_offset=13)
    _say(f"[patch bwd_filter] {sh} :: {desc}")
    got = _np(_run_conv(mc, "bwd_filter", sh, _dev(t), ws=ws))
    assert not np.isnan(got).any()
    err = rel_err(got, _oracle_full("bwd_filter", sh, t))
    _say(f"    rel err {err:.3e}")
    assert err <= TOL["bf16"]
    ti = inputs(wl, "bf16", shape=sh, integer=True, seed_offset=14)
    got = _np(_run_conv(mc, "bwd_filter", sh, _dev(ti), ws=ws))
    assert np.array_equal(got.astype(np.float64), _oracle_full("bwd_filter", sh, ti))


def _bwdf_full_compare(mc, sh, wl, seed, want):
    desc = mc.plan_describe(mc.BWD_FILTER, mc.BF16, sh.args13())
    for w in want:
        assert w in desc, (w, desc)
    for integer in (False, True):
        t = inputs(wl, "bf16", shape=sh, integer=integer, seed_offset=seed)
        _say(f"[bwd_filter form] {sh} integer={integer} :: {desc}")
        got = _np(_run_conv(mc, "bwd_filter", sh, _dev(t)))
        ref = _oracle_full("bwd_filter", sh, t)
        assert not np.isnan(got).any()
        if integer:
            assert np.array_equal(got.astype(np.float64), ref)
        else:
            err = rel_err(got, ref)
            _say(f"    rel err {err:.3e}")
            assert err <= TOL["bf16"]


@pytest.mark.parametrize("n", [257, 300])
def test_bwd_filter_k16_64_filter_rows(mc, n):
    """64 filter rows, 3x3 on 16x16 images: the 16x16x32 kernel's stream form with two whole
    images per split (64-row tiles); N = 257 leaves a last split of one image.  Every dW element
    against the full oracle; integer inputs bit for bit."""
    sh = ConvShape(n, 64, 16, 16, 64, 3, 3, (1, 1), (1, 1), 16, 16)
    _bwdf_full_compare(mc, sh, WORKLOADS["resnet3x3"], 15,
                       ["algo=patch", "tile=64x", "form=stream", "mma=16x16x32"])


def test_bwd_filter_k16_64_filter_rows_bands(mc):
    """64 filter rows, 3x3 on 20x20 images (whole-image patches too large for the stream
    form): the 16x16x32 kernel's bands form, bands of 11 and 9 output rows.  Every dW element."""
    sh = ConvShape(37, 64, 20, 20, 64, 3, 3, (1, 1), (1, 1), 20, 20)
    _bwdf_full_compare(mc, sh, WORKLOADS["resnet3x3"], 20,
                       ["algo=patch", "tile=64x", "form=bands", "mma=16x16x32"])


def test_bwd_filter_k16_many_filter_rows(mc):
    """512 filter rows in 128-row tiles, 3x3, five 14x14 images per split, 8 splits: the form the
    deep3x3 backward-filter runs (the split's pixels taken 32 per step across image boundaries,
    dy staged through three LDS slots, each image's patch filled while the previous one is in
    use).  Every dW element; integer inputs bit for bit."""
    sh = ConvShape(40, 512, 14, 14, 512, 3, 3, (1, 1), (1, 1), 14, 14)
    _bwdf_full_compare(mc, sh, WORKLOADS["deep3x3"], 16,
                       ["algo=patch", "tile=128x", "chunk=5 ", "form=stream", "mma=16x16x32"])


@pytest.mark.parametrize("sh,want", [
    # one image per split (the patch of a second image is filled but never read)
    (ConvShape(3, 512, 14, 14, 512, 3, 3, (1, 1), (1, 1), 14, 14), ["tile=128x", "chunk=1 "]),
    # ragged filter rows (200 = 128 + 72) and five channel tiles
    (ConvShape(41, 160, 14, 14, 200, 3, 3, (1, 1), (1, 1), 14, 14), ["tile=128x"]),
    # 64 rows, 12x12 images (144 pixels: 4.5 steps per image), 8-byte fill loads
    (ConvShape(9, 64, 12, 12, 64, 3, 3, (1, 1), (1, 1), 12, 12), ["tile=64x"]),
])
def test_bwd_filter_stream_edges(mc, sh, want):
    """Edge cases of the stream form.  Every dW element; integer inputs bit for bit."""
    _bwdf_full_compare(mc, sh, WORKLOADS["deep3x3"], 21,
                       ["algo=patch", "form=stream", "mma=16x16x32"] + want)


def test_bwd_filter_stream_one_split(mc):
    """No workspace: the stream form in one split of 70 images (dW written directly), so the
    32-pixel steps straddle image boundaries at every offset the 14x14 images produce.  Every
    dW element; integer inputs bit for bit."""
    sh = ConvShape(70, 64, 14, 14, 64, 3, 3, (1, 1), (1, 1), 14, 14)
    desc = mc.plan_describe(mc.BWD_FILTER, mc.BF16, sh.args13(), 0)
    for w in ("algo=patch", "splits=1 ", "chunk=70 ", "form=stream"):
        assert w in desc, (w, desc)
    ws = torch.empty(0, dtype=torch.uint8, device=DEV)
    wl = WORKLOADS["deep3x3"]
    for integer in (False, True):
        t = inputs(wl, "bf16", shape=sh, integer=integer, seed_offset=22)
        _say(f"[bwd_filter stream, one split] integer={integer} :: {desc}")
        got = _np(_run_conv(mc, "bwd_filter", sh, _dev(t), ws=ws))
        ref = _oracle_full("bwd_filter", sh, t)
        assert not np.isnan(got).any()
        if integer:
            assert np.array_equal(got.astype(np.float64), ref)
        else:
            err = rel_err(got, ref)
            _say(f"    rel err {err:.3e}")
            assert err <= TOL["bf16"]


def test_bwd_filter_k16_many_filter_rows_wide(mc):
    """128-row tiles on 28x28 images (8 output rows per band, 16-byte fill loads capped to
    8 bytes), ragged K: every dW element against the full oracle."""
    sh = ConvShape(6, 96, 28, 28, 200, 3, 3, (1, 1), (1, 1), 28, 28)
    _bwdf_full_compare(mc, sh, WORKLOADS["deep3x3"], 19,
                       ["algo=patch", "tile=128x", "form=bands", "mma=16x16x32"])


@pytest.mark.parametrize("n", [257, 300])
def test_bwd_filter_pair_form(mc, n):
    """The 32x32x16 kernel's pair form (64 filter rows, 3x3, two bands per split, both patches
    filled first, one per wave pair), which 3x3 shapes whose P*Q is not a multiple of 4 take
    (13x14 images here); N = 257 leaves a last split with a single band.  Every dW element."""
    sh = ConvShape(n, 64, 13, 14, 64, 3, 3, (1, 1), (1, 1), 13, 14)
    _bwdf_full_compare(mc, sh, WORKLOADS["resnet3x3"], 17,
                       ["algo=patch", "tile=64x", "chunk=2 ", "form=pair", "mma=32x32x16"])


def test_bwd_filter_32x32_bands_form(mc):
    """The 32x32x16 kernel's bands form with 128-row tiles and several bands per split (13x14
    images, 512 filter rows).  Every dW element; integer inputs bit for bit."""
    sh = ConvShape(20, 512, 13, 14, 512, 3, 3, (1, 1), (1, 1), 13, 14)
    _bwdf_full_compare(mc, sh, WORKLOADS["deep3x3"], 18,
                       ["algo=patch", "tile=128x", "chunk=3 ", "form=bands", "mma=32x32x16"])


def test_implicit_workspace_on_side_stream(mc):
    """workspace=None with stream= a side stream: the binding allocates the workspace from that
    stream's pool, so main-stream allocations made while the side-stream kernels run cannot
    take its block.  Results equal the serial ones bit for bit."""
    wl = WORKLOADS["resnet3x3"]
    s = wl.shape
    d = _dev(inputs(wl, "bf16"))
    ref_dw = _run_conv(mc, "bwd_filter", s, d)
    ref_y = _run_conv(mc, "fwd", s, d)
    side = torch.cuda.Stream(device=DEV)   # default priority
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        dw = torch.full(s.w_shape, float("nan"), device=DEV)
        y = torch.full(s.y_shape, float("nan"), device=DEV)
        side.wait_stream(torch.cuda.current_stream())
        mc.conv2d_bwd_filter(d["x"], d["dy"], (s.R, s.S), s.pad, s.stride, dw=dw, stream=side)
        mc.conv2d_fwd(d["x"], d["w"], s.pad, s.stride, y=y, stream=side)
        # main-stream allocations of the same sizes while the side stream still runs
        junk = [torch.full((mc.workspace_size(mc.BWD_FILTER, mc.BF16, s.args13()),), 7, dtype=torch.uint8,
                           device=DEV) for _ in range(3)]
        outs.append((dw, y, junk))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for dw, y, _ in outs:
        assert torch.equal(dw, ref_dw) and torch.equal(y, ref_y)


# ----------------------------------------------------------------------------- few input channels

TINYC_SHAPES = [
    ConvShape(2, 3, 37, 70, 16, 7, 7, (3, 3), (2, 2), 19, 35),     # stem-like, ragged tiles both ways
    ConvShape(3, 1, 20, 66, 8, 3, 3, (1, 1), (1, 1), 20, 66),      # C = 1, stride 1
    ConvShape(2, 2, 17, 33, 12, 5, 3, (2, 0), (2, 1), 9, 31),      # C = 2, strides (2, 1), R != S
    ConvShape(2, 4, 18, 20, 24, 1, 1, (0, 0), (2, 2), 9, 10),      # C = 4, 1x1 stride 2: phases without taps
]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("sh", TINYC_SHAPES)
def test_few_channel_backward_data(mc, sh, dt):
    desc = mc.plan_describe(mc.BWD_DATA, mc.F32 if dt == "f32" else mc.BF16, sh.args13())
    assert "algo=tinyc" in desc, desc
    wl = WORKLOADS["stem7x7"]
    t = inputs(wl, dt, shape=sh, seed_offset=21)
    _say(f"[tinyc] {dt} {sh} :: {desc}")
    got = _np(_run_conv(mc, "bwd_data", sh, _dev(t)))
    assert not np.isnan(got).any()
    err = rel_err(got, _oracle_full("bwd_data", sh, t))
    _say(f"    rel err {err:.3e}")
    assert err <= TOL[dt]
    ti = inputs(wl, dt, shape=sh, integer=True, seed_offset=22)
    got = _np(_run_conv(mc, "bwd_data", sh, _dev(ti)))
    assert np.array_equal(got.astype(np.float64), _oracle_full("bwd_data", sh, ti))


TINYC_MFMA_SHAPES = [
    ConvShape(2, 3, 37, 70, 64, 7, 7, (3, 3), (2, 2), 19, 35),      # odd pad: odd dx rows read one row further
    ConvShape(3, 3, 40, 226, 32, 7, 7, (2, 2), (2, 2), 19, 112),    # even pad, K = 32 (one lane half absent)
    ConvShape(2, 4, 30, 254, 64, 7, 7, (3, 3), (2, 2), 15, 127),    # C * S = 28 columns, Q = 127
    ConvShape(2, 1, 16, 16, 64, 7, 3, (3, 1), (2, 2), 8, 8),        # 7 x 3 filter, one channel
    ConvShape(2, 3, 224, 224, 64, 7, 7, (3, 3), (2, 2), 112, 112),  # the stem's image size: several bands
    ConvShape(5, 2, 9, 12, 64, 7, 7, (0, 3), (2, 2), 2, 6),         # pad 0 rows, dy rows past the image
]


@pytest.mark.parametrize("sh", TINYC_MFMA_SHAPES)
def test_few_channel_backward_data_mfma(mc, sh):
    """fp32, stride 2, 7 filter rows: the MFMA form (filter-row sums per dx row, then the
    column taps), compared element by element."""
    desc = mc.plan_describe(mc.BWD_DATA, mc.F32, sh.args13())
    assert "algo=tinyc" in desc and "form=mfma" in desc, desc
    wl = WORKLOADS["stem7x7"]
    t = inputs(wl, "f32", shape=sh, seed_offset=23)
    _say(f"[tinyc mfma] {sh} :: {desc}")
    got = _np(_run_conv(mc, "bwd_data", sh, _dev(t)))
    assert not np.isnan(got).any()
    err = rel_err(got, _oracle_full("bwd_data", sh, t))
    _say(f"    rel err {err:.3e}")
    assert err <= TOL["f32"]
    ti = inputs(wl, "f32", shape=sh, integer=True, seed_offset=24)
    got = _np(_run_conv(mc, "bwd_data", sh, _dev(ti)))
    assert np.array_equal(got.astype(np.float64), _oracle_full("bwd_data", sh, ti))


TINYC_BWDF_SHAPES = [
    ConvShape(2, 3, 37, 71, 64, 7, 7, (3, 3), (2, 2), 19, 36),      # odd rows and pad, Q = 36 of 112
    ConvShape(3, 3, 40, 226, 64, 7, 7, (2, 2), (2, 2), 19, 112),    # even pad, full 112-pixel rows
    ConvShape(2, 3, 224, 224, 64, 7, 7, (3, 3), (2, 2), 112, 112),  # the stem's image size
    ConvShape(2, 1, 16, 16, 64, 7, 3, (3, 1), (2, 2), 8, 8),        # 7 x 3 filter, one channel
    ConvShape(2, 4, 30, 32, 64, 7, 5, (3, 2), (1, 2), 30, 16),      # row stride 1, 140 filter values
    ConvShape(1, 3, 12, 23, 64, 7, 7, (3, 3), (2, 2), 6, 12),       # 6 output rows: 6 splits of one row
    ConvShape(1, 3, 7, 23, 64, 7, 7, (0, 3), (2, 2), 1, 12),        # one output row: dW written directly
]


@pytest.mark.parametrize("sh", TINYC_BWDF_SHAPES)
def test_few_channel_backward_filter_mfma(mc, sh):
    """fp32 backward-filter with C <= 4, 7 filter rows, column stride 2: the few-channel MFMA
    kernel, in every candidate plan that uses it (split counts, one split), compared element
    by element."""
    sizes = sh.args13()
    n, _ = mc.plan_candidates(mc.BWD_FILTER, mc.F32, sizes)
    wl = WORKLOADS["stem7x7"]
    t, ti = inputs(wl, "f32", shape=sh, seed_offset=25), inputs(wl, "f32", shape=sh, integer=True, seed_offset=26)
    ref, refi = _oracle_full("bwd_filter", sh, t), _oracle_full("bwd_filter", sh, ti)
    d, di = _dev(t), _dev(ti)
    seen = 0
    try:
        for i in range(n):
            mc.plan_select(mc.BWD_FILTER, mc.F32, sizes, i)
            desc = mc.plan_describe(mc.BWD_FILTER, mc.F32, sizes)
            if "algo=tinyc" not in desc:
                continue
            assert "form=mfma" in desc, desc
            seen += 1
            _say(f"[tinyc bwd-filter] {sh} :: {desc}")
            got = _np(_run_conv(mc, "bwd_filter", sh, d))
            assert not np.isnan(got).any()
            err = rel_err(got, ref)
            _say(f"    rel err {err:.3e}")
            assert err <= TOL["f32"]
            goti = _np(_run_conv(mc, "bwd_filter", sh, di))
            assert np.array_equal(goti.astype(np.float64), refi)
    finally:
        mc.plan_select(mc.BWD_FILTER, mc.F32, sizes, -1)
    assert seen >= 1
    assert "algo=tinyc" in mc.plan_describe(mc.BWD_FILTER, mc.F32, sizes)


TINYC_FWD_SHAPES = [
    ConvShape(2, 3, 37, 70, 64, 7, 7, (3, 3), (2, 2), 19, 35),      # Q = 35: a ragged pixel tile
    ConvShape(3, 3, 40, 226, 64, 7, 7, (2, 2), (2, 2), 19, 112),    # even pad, seven full pixel tiles
    ConvShape(2, 3, 224, 224, 64, 7, 7, (3, 3), (2, 2), 112, 112),  # the stem's image size
    ConvShape(2, 4, 30, 32, 64, 7, 5, (3, 2), (1, 2), 30, 16),      # row stride 1, 140 filter values
    ConvShape(1, 2, 9, 20, 64, 7, 4, (0, 1), (2, 2), 2, 10),        # pad 0 rows, S = 4
]


@pytest.mark.parametrize("sh", TINYC_FWD_SHAPES)
def test_few_channel_forward_mfma(mc, sh):
    """fp32 forward with C <= 4, 7 filter rows, column stride 2: the few-channel MFMA kernel,
    compared element by element."""
    desc = mc.plan_describe(mc.FWD, mc.F32, sh.args13())
    assert "algo=tinyc" in desc and "form=mfma" in desc, desc
    wl = WORKLOADS["stem7x7"]
    t = inputs(wl, "f32", shape=sh, seed_offset=27)
    _say(f"[tinyc fwd] {sh} :: {desc}")
    got = _np(_run_conv(mc, "fwd", sh, _dev(t)))
    assert not np.isnan(got).any()
    err = rel_err(got, _oracle_full("fwd", sh, t))
    _say(f"    rel err {err:.3e}")
    assert err <= TOL["f32"]
    ti = inputs(wl, "f32", shape=sh, integer=True, seed_offset=28)
    got = _np(_run_conv(mc, "fwd", sh, _dev(ti)))
    assert np.array_equal(got.astype(np.float64), _oracle_full("fwd", sh, ti))
    # the fused epilogue at the kernel's store: bias, alpha, beta, ReLU
    c = EPI_CASES[-1]
    bias, y0 = _epi_args(t, sh, c, 95)
    got = _np(_run_fwd_ex(mc, sh, _dev(t), c, bias, y0))
    ref = oracle.conv2d_fwd_ex(t["x"].float().numpy(), t["w"].float().numpy(), sh.pad, sh.stride,
                               bias=bias.numpy(), alpha=c["alpha"], beta=c["beta"], y_prev=y0.numpy(),
                               relu=c["relu"])
    err = rel_err(got, ref)
    _say(f"    epilogue rel err {err:.3e}")
    assert err <= TOL["f32"]


# ----------------------------------------------------------------------------- stride-phase patch path

PHASE_SHAPES = [
    ConvShape(2, 96, 28, 28, 256, 4, 4, (1, 1), (2, 2), 14, 14),     # 128-row tile, 96 rows used
    ConvShape(3, 64, 20, 24, 96, 4, 4, (1, 1), (2, 2), 10, 12),      # 64-row tile, H != W
    ConvShape(2, 160, 18, 22, 64, 4, 4, (2, 2), (2, 2), 10, 12),     # pad 2: equal phase pads; 2 row tiles
    ConvShape(2, 64, 64, 64, 64, 4, 4, (1, 1), (2, 2), 32, 32),      # four row tiles per phase image
    ConvShape(40, 128, 32, 32, 256, 4, 4, (1, 1), (2, 2), 16, 16),   # several tiles per work-group
]


@pytest.mark.parametrize("sh", PHASE_SHAPES)
def test_phase_patch_backward_data(mc, sh):
    """bf16 backward-data at stride 2 with a 4x4 filter (the transposed-convolution case): every
    stride phase a stride-1 2x2 correlation on the patch kernel (plan asserted), every dx element
    against the oracle, integer inputs bit for bit, no element left unwritten."""
    desc = mc.plan_describe(mc.BWD_DATA, mc.BF16, sh.args13())
    assert "form=phase-patch" in desc, desc
    wl = WORKLOADS["deconv4x4"]
    t = inputs(wl, "bf16", shape=sh, seed_offset=81)
    _say(f"[phase patch] {sh} :: {desc}")
    got = _np(_run_conv(mc, "deconv_fwd", sh, _dev(t)))
    assert not np.isnan(got).any()
    err = rel_err(got, _oracle_full("deconv_fwd", sh, t))
    _say(f"    rel err {err:.3e}")
    assert err <= TOL["bf16"]
    ti = inputs(wl, "bf16", shape=sh, integer=True, seed_offset=82)
    got = _np(_run_conv(mc, "deconv_fwd", sh, _dev(ti)))
    assert np.array_equal(got.astype(np.float64), _oracle_full("deconv_fwd", sh, ti))


S2D_SHAPES = [
    ConvShape(2, 96, 28, 28, 256, 4, 4, (1, 1), (2, 2), 14, 14),     # ragged z pitch (15 -> 16)
    ConvShape(3, 64, 20, 24, 96, 4, 4, (1, 1), (2, 2), 10, 12),      # H != W, ragged K (96 = 64 + 32)
    ConvShape(2, 40, 18, 22, 64, 4, 4, (2, 2), (2, 2), 10, 12),      # pad 2, 160 z channels
    ConvShape(2, 32, 15, 17, 72, 4, 4, (0, 3), (2, 2), 6, 10),       # odd sizes, pad 0 / 3
    ConvShape(2, 64, 64, 64, 64, 4, 4, (1, 1), (2, 2), 32, 32),      # 8 output rows per tile
    ConvShape(40, 128, 32, 32, 256, 4, 4, (1, 1), (2, 2), 16, 16),   # the deconvolution's input gradient
]


@pytest.mark.parametrize("sh", [ConvShape(2, 64, 17, 20, 64, 2, 2, (1, 0), (1, 1), 18, 19),     # 64 rows
                                ConvShape(2, 96, 30, 30, 128, 2, 2, (0, 0), (1, 1), 29, 29)])   # 128 rows
def test_patch_2x2_forward(mc, sh):
    """Stride-1 bf16 forward with a 2x2 filter on the patch kernels: the 64-row form runs the
    compile-time-tap kernel's 4-tap schedule (three patch buffers), the 128-row form the
    runtime-tap kernel.  Every output element; integer inputs bit for bit."""
    desc = mc.plan_describe(mc.FWD, mc.BF16, sh.args13())
    assert "algo=patch" in desc, desc
    wl = WORKLOADS["deep3x3"]
    _say(f"[patch 2x2] {sh} :: {desc}")
    t = inputs(wl, "bf16", shape=sh, seed_offset=85)
    got = _np(_run_conv(mc, "fwd", sh, _dev(t)))
    assert not np.isnan(got).any()
    err = rel_err(got, _oracle_full("fwd", sh, t))
    _say(f"    rel err {err:.3e}")
    assert err <= TOL["bf16"]
    ti = inputs(wl, "bf16", shape=sh, integer=True, seed_offset=86)
    got = _np(_run_conv(mc, "fwd", sh, _dev(ti)))
    assert np.array_equal(got.astype(np.float64), _oracle_full("fwd", sh, ti))


@pytest.mark.parametrize("sh", S2D_SHAPES)
def test_space_to_depth_forward(mc, sh):
    """bf16 forward at stride 2 with a 4x4 filter (the transposed convolution's input
    gradient): x regrouped by stride phase into channels, then a stride-1 2x2 correlation on the
    patch kernel (plan asserted); every output element against the oracle, through the
    convolution forward and the deconvolution's backward-data entry points, integer inputs bit
    for bit, no element left unwritten."""
    desc = mc.plan_describe(mc.FWD, mc.BF16, sh.args13())
    assert "form=space-to-depth" in desc, desc
    _say(f"[space-to-depth] {sh} :: {desc}")
    for pass_id, wl in (("fwd", WORKLOADS["deep3x3"]), ("deconv_bwd_data", WORKLOADS["deconv4x4"])):
        t = inputs(wl, "bf16", shape=sh, seed_offset=83)
        got = _np(_run_conv(mc, pass_id, sh, _dev(t)))
        assert not np.isnan(got).any()
        err = rel_err(got, _oracle_full(pass_id, sh, t))
        _say(f"    {pass_id} rel err {err:.3e}")
        assert err <= TOL["bf16"]
        ti = inputs(wl, "bf16", shape=sh, integer=True, seed_offset=84)
        got = _np(_run_conv(mc, pass_id, sh, _dev(ti)))
        assert np.array_equal(got.astype(np.float64), _oracle_full(pass_id, sh, ti))


# ----------------------------------------------------------------------------- 1x1 pointwise path

POINTWISE_SHAPES = [
    (ConvShape(2, 64, 16, 16, 128, 1, 1, (0, 0), (2, 2), 8, 8), ("fwd", "bwd_data")),
    (ConvShape(3, 192, 40, 40, 64, 1, 1, (0, 0), (2, 2), 20, 20), ("fwd", "bwd_data")),   # ragged rows and C
    (ConvShape(2, 128, 12, 12, 200, 1, 1, (0, 0), (1, 1), 12, 12), ("fwd",)),             # stride 1, ragged K
    (ConvShape(2, 96, 8, 8, 128, 1, 1, (0, 0), (1, 1), 8, 8), ("bwd_data",)),             # stride 1, ragged C
    (ConvShape(2, 256, 56, 56, 512, 1, 1, (0, 0), (2, 2), 28, 28), ("fwd", "bwd_data")),  # N reduced proj1x1
]


@pytest.mark.parametrize("case", range(len(POINTWISE_SHAPES)))
def test_pointwise_path_full_compare(mc, case):
    """1x1 bf16, pad 0, stride 1 or 2: the pointwise GEMM kernel (plan asserted), every output
    element against the oracle, and integer inputs bit for bit (dx's uncovered positions too)."""
    sh, passes = POINTWISE_SHAPES[case]
    wl = WORKLOADS["proj1x1"]
    for pass_id in passes:
        pid = mc.FWD if pass_id == "fwd" else mc.BWD_DATA
        desc = mc.plan_describe(pid, mc.BF16, sh.args13())
        assert "algo=pointwise" in desc, desc
        t = inputs(wl, "bf16", shape=sh, seed_offset=51)
        _say(f"[pointwise] {pass_id} {sh} :: {desc}")
        got = _np(_run_conv(mc, pass_id, sh, _dev(t)))
        assert not np.isnan(got).any()
        err = rel_err(got, _oracle_full(pass_id, sh, t))
        _say(f"    rel err {err:.3e}")
        assert err <= TOL["bf16"]
        ti = inputs(wl, "bf16", shape=sh, integer=True, seed_offset=52)
        got = _np(_run_conv(mc, pass_id, sh, _dev(ti)))
        assert np.array_equal(got.astype(np.float64), _oracle_full(pass_id, sh, ti))


# 1x1 bf16 backward-filter, pad 0, stride 1 or 2: the pointwise GEMM over the flat pixel index
POINTWISE_BWDF_SHAPES = [
    ConvShape(2, 64, 16, 16, 128, 1, 1, (0, 0), (2, 2), 8, 8),
    ConvShape(3, 192, 40, 40, 64, 1, 1, (0, 0), (2, 2), 20, 20),    # ragged C tile, ragged last step
    ConvShape(4, 256, 56, 56, 512, 1, 1, (0, 0), (2, 2), 28, 28),   # N reduced proj1x1
    ConvShape(64, 32, 16, 16, 40, 1, 1, (0, 0), (2, 2), 8, 8),      # one step per split, 64 splits
    ConvShape(2, 96, 8, 8, 200, 1, 1, (0, 0), (1, 1), 8, 8),        # stride 1 (a plan candidate), ragged K
]


def _select_pointwise(mc, sh):
    """Installs the pointwise candidate for this backward-filter problem (the default plan when it
    is pointwise); returns its description."""
    args = sh.args13()
    if "algo=pointwise" in mc.plan_describe(mc.BWD_FILTER, mc.BF16, args):
        return mc.plan_describe(mc.BWD_FILTER, mc.BF16, args)
    n, _ = mc.plan_candidates(mc.BWD_FILTER, mc.BF16, args)
    for i in range(n):
        mc.plan_select(mc.BWD_FILTER, mc.BF16, args, i)
        d = mc.plan_describe(mc.BWD_FILTER, mc.BF16, args)
        if "algo=pointwise" in d:
            return d
    raise AssertionError("no pointwise candidate")


@pytest.mark.parametrize("budget", ["plan", "none"])
@pytest.mark.parametrize("case", range(len(POINTWISE_BWDF_SHAPES)))
def test_pointwise_bwd_filter(mc, case, budget):
    """The pointwise backward-filter (plan asserted; split-K and, with no workspace, one split
    written directly): every dW element against the oracle, integer inputs bit for bit."""
    sh = POINTWISE_BWDF_SHAPES[case]
    ws = torch.empty(0, dtype=torch.uint8, device=DEV) if budget == "none" else None
    try:
        if budget == "none":
            desc = mc.plan_describe(mc.BWD_FILTER, mc.BF16, sh.args13(), 0)
            if sh.stride[0] == 1:
                pytest.skip("stride 1 reaches the pointwise kernel as a candidate under a workspace budget")
        else:
            desc = _select_pointwise(mc, sh)
        assert "algo=pointwise" in desc, desc
        if budget == "none":
            assert "splits=1" in desc, desc
        wl = WORKLOADS["proj1x1"]
        _say(f"[pointwise bwd_filter] {sh} budget={budget} :: {desc}")
        t = inputs(wl, "bf16", shape=sh, seed_offset=55)
        got = _np(_run_conv(mc, "bwd_filter", sh, _dev(t), ws=ws))
        assert not np.isnan(got).any()
        err = rel_err(got, _oracle_full("bwd_filter", sh, t))
        _say(f"    rel err {err:.3e}")
        assert err <= TOL["bf16"]
        ti = inputs(wl, "bf16", shape=sh, integer=True, seed_offset=56)
        got = _np(_run_conv(mc, "bwd_filter", sh, _dev(ti), ws=ws))
        assert np.array_equal(got.astype(np.float64), _oracle_full("bwd_filter", sh, ti))
    finally:
        mc.plan_select(mc.BWD_FILTER, mc.BF16, sh.args13(), -1)


@pytest.mark.parametrize("form", ["algo=pointwise", "form=space-to-depth"])
@pytest.mark.parametrize("case", [0, 1])
def test_pointwise_fused_forward(mc, case, form):
    """The fused forward epilogue (bias, ReLU, alpha, beta; fp32 and bf16 y) on the pointwise
    kernel and on the space-to-depth form, against the oracle; the bf16 y equals the fp32 y
    rounded once, bit for bit."""
    sh = POINTWISE_SHAPES[1][0] if form == "algo=pointwise" else S2D_SHAPES[1]
    c = [dict(alpha=1.0, beta=0.0, bias=True, relu=True), dict(alpha=-0.75, beta=0.5, bias=True, relu=False)][case]
    assert form in mc.plan_describe(mc.FWD, mc.BF16, sh.args13())
    t = inputs(WORKLOADS["proj1x1"], "bf16", shape=sh, seed_offset=53)
    bias, y0 = _epi_args(t, sh, c, 98)
    d = _dev(t)
    b = bias.to(DEV)
    y0b = y0.to(torch.bfloat16)
    yb = y0b.clone().to(DEV) if c["beta"] else torch.full(sh.y_shape, float("nan"), device=DEV).to(torch.bfloat16)
    mc.conv2d_fwd_ex(d["x"], d["w"], sh.pad, sh.stride, bias=b, alpha=c["alpha"], beta=c["beta"], relu=c["relu"],
                     y=yb)
    yf = y0b.float().to(DEV) if c["beta"] else torch.full(sh.y_shape, float("nan"), device=DEV)
    mc.conv2d_fwd_ex(d["x"], d["w"], sh.pad, sh.stride, bias=b, alpha=c["alpha"], beta=c["beta"], relu=c["relu"],
                     y=yf)
    torch.cuda.synchronize()
    assert torch.equal(yb.view(torch.int16), yf.to(torch.bfloat16).view(torch.int16))
    ref = oracle.conv2d_fwd_ex(t["x"].float().numpy(), t["w"].float().numpy(), sh.pad, sh.stride, bias=bias.numpy(),
                               alpha=c["alpha"], beta=c["beta"], y_prev=y0b.float().numpy(), relu=c["relu"])
    err = rel_err(yf.cpu().numpy(), ref)
    _say(f"[{form} fused] {c} rel err {err:.3e}")
    assert err <= TOL["bf16"]
