"""GPU parity of the output epilogues: backward-data, backward-filter and the three
deconvolution passes with out = act(alpha * result + beta * out_prev + bias), fp32 or bf16
output, and the bias gradient, through the C ABI binding against the oracle.

- Every output element is compared with the oracle's epilogue (fp64) at the input
  dtype's tolerance (fp32: 1e-5, bf16: 1e-2); a bf16 output adds one rounding to nearest
  even (8 significant bits: at most 2^-8 of the value), so its bound is the input dtype's
  plus 2^-8.
- A bf16 output must equal the fp32 output of the same call (same previous values)
  rounded to nearest even, bit for bit: one fp32 accumulation, one rounding at the store.
- With beta = 0 the output is pre-filled with NaN: it must not be read, and every
  element must be written (including dx positions no filter window reaches).
- Each kernel family that writes dx or dW is reached with its plan asserted: the
  generic implicit GEMM (with and without phases that have no taps), the few-channel
  kernel, the pointwise kernel, the stride-1 patch kernel, and every backward-filter
  form with one split (the kernel applies the epilogue) and with several (the split-K
  reduce applies it).
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, ConvShape, Dist, draw, inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}
DEV = "cuda:0"
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}

REDUCED = {
    "tiny": ConvShape(2, 3, 8, 8, 4, 3, 3, (1, 1), (1, 1), 8, 8),
    "resnet3x3": ConvShape(2, 64, 19, 19, 64, 3, 3, (1, 1), (1, 1), 19, 19),
    "proj1x1": ConvShape(2, 256, 24, 24, 192, 1, 1, (0, 0), (2, 2), 12, 12),
    "stem7x7": ConvShape(2, 3, 37, 37, 64, 7, 7, (3, 3), (2, 2), 19, 19),
    "deconv4x4": ConvShape(2, 96, 14, 14, 256, 4, 4, (1, 1), (2, 2), 7, 7),
    "deep3x3": ConvShape(3, 160, 14, 14, 160, 3, 3, (1, 1), (1, 1), 14, 14),
}

CASES = [
    dict(alpha=0.5, beta=1.0, out="f32"),
    dict(alpha=-1.5, beta=-0.25, out="bf16"),
    dict(alpha=2.0, beta=0.0, out="bf16"),
]

# convolution pass that runs each call, for plan_describe on the convolution view of the shape
_PID = {"bwd_data": 1, "bwd_filter": 2, "deconv_fwd": 1, "deconv_bwd_data": 0, "deconv_bwd_filter": 2}


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


def _out_shape(pass_id, s):
    return {"bwd_data": s.x_shape, "bwd_filter": s.w_shape, "deconv_fwd": s.x_shape,
            "deconv_bwd_data": s.y_shape, "deconv_bwd_filter": s.w_shape}[pass_id]


def _gpu(mc, pass_id, s, d, alpha, beta, out, ws=None, bias=None, relu=False):
    """One epilogue call; `out` holds the previous values (or NaN when beta == 0)."""
    if pass_id == "bwd_data":
        mc.conv2d_bwd_data_ex(d["dy"], d["w"], (s.H, s.W), s.pad, s.stride, alpha, beta, dx=out, workspace=ws)
    elif pass_id == "bwd_filter":
        mc.conv2d_bwd_filter_ex(d["x"], d["dy"], (s.R, s.S), s.pad, s.stride, alpha, beta, dw=out, workspace=ws)
    elif pass_id == "deconv_fwd":
        mc.deconv2d_fwd_ex(d["x_in"], d["w"], (s.H, s.W), s.pad, s.stride, bias=bias, alpha=alpha, beta=beta,
                           relu=relu, y=out, workspace=ws)
    elif pass_id == "deconv_bwd_data":
        mc.deconv2d_bwd_data_ex(d["dout"], d["w"], (s.P, s.Q), s.pad, s.stride, alpha, beta, dx=out, workspace=ws)
    else:
        mc.deconv2d_bwd_filter_ex(d["x_in"], d["dout"], (s.R, s.S), s.pad, s.stride, alpha, beta, dw=out,
                                  workspace=ws)
    torch.cuda.synchronize()
    return out


def _oracle(pass_id, s, t, alpha, beta, prev, bias=None, relu=False):
    f = {k: v.float().numpy() for k, v in t.items()}
    if pass_id == "bwd_data":
        return oracle.conv2d_bwd_data_ex(f["dy"], f["w"], (s.H, s.W), s.pad, s.stride, alpha, beta, prev)
    if pass_id == "bwd_filter":
        return oracle.conv2d_bwd_filter_ex(f["x"], f["dy"], (s.R, s.S), s.pad, s.stride, alpha, beta, prev)
    if pass_id == "deconv_fwd":
        return oracle.deconv2d_fwd_ex(f["x_in"], f["w"], (s.H, s.W), s.pad, s.stride, bias, alpha, beta, prev, relu)
    if pass_id == "deconv_bwd_data":
        return oracle.deconv2d_bwd_data_ex(f["dout"], f["w"], (s.P, s.Q), s.pad, s.stride, alpha, beta, prev)
    return oracle.deconv2d_bwd_filter_ex(f["x_in"], f["dout"], (s.R, s.S), s.pad, s.stride, alpha, beta, prev)


def check_epilogue(mc, pass_id, s, t, dt, c, seed, ws=None, bias=None, relu=False, want=()):
    """Runs case c of the epilogue on pass_id and checks it against the oracle (and, for a bf16
    output, bit for bit against the fp32 output rounded once)."""
    code = mc.F32 if dt == "f32" else mc.BF16
    desc = mc.plan_describe(_PID[pass_id], code, s.args13(), 0 if ws is not None else 10 ** 9)
    for w in want:
        assert w in desc, (w, desc)
    _say(f"[epilogue] {pass_id} {dt} {c} bias={bias is not None} relu={relu} {s} :: {desc}")
    shape = _out_shape(pass_id, s)
    prev = draw(shape, Dist("uniform", -1, 1), seed).to(TDT[c["out"]])   # exact in the output dtype
    d = {k: v.to(DEV) for k, v in t.items()}
    b = None if bias is None else bias.to(DEV)

    def run(odt):
        out = prev.to(DEV, odt) if c["beta"] != 0.0 else torch.full(shape, float("nan"), device=DEV, dtype=odt)
        return _gpu(mc, pass_id, s, d, c["alpha"], c["beta"], out, ws, b, relu)

    got = run(TDT[c["out"]])
    assert not torch.isnan(got).any(), "output elements left unwritten (or a NaN previous value was read)"
    if c["out"] == "bf16":
        g32 = run(torch.float32)
        assert torch.equal(got.view(torch.int16), g32.to(torch.bfloat16).view(torch.int16))
    ref = _oracle(pass_id, s, t, c["alpha"], c["beta"], prev.double().numpy(),
                  None if bias is None else bias.numpy(), relu)
    err = rel_err(got.double().cpu().numpy(), ref)
    tol = TOL[dt] + (2.0 ** -8 if c["out"] == "bf16" else 0.0)
    _say(f"    rel err {err:.3e} (bound {tol:.3e})")
    assert err <= tol


# ----------------------------------------------------------------------------- every workload, reduced

EPI_REDUCED = [(n, dt, p) for n, wl in WORKLOADS.items() for dt in ("f32", "bf16") for p in wl.passes
               if p != "fwd"]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("name,dt,pass_id", EPI_REDUCED)
def test_epilogue_reduced_workloads(mc, name, dt, pass_id, case):
    wl, s = WORKLOADS[name], REDUCED[name]
    t = inputs(wl, dt, shape=s, seed_offset=61)
    check_epilogue(mc, pass_id, s, t, dt, CASES[case], 611 + case)


@pytest.mark.parametrize("name,dt,pass_id", [c for c in EPI_REDUCED if c[2].endswith("bwd_filter")])
def test_epilogue_backward_filter_without_workspace(mc, name, dt, pass_id):
    """Budget 0: one split, so the backward-filter kernel itself applies the epilogue."""
    wl, s = WORKLOADS[name], REDUCED[name]
    t = inputs(wl, dt, shape=s, seed_offset=62)
    empty = torch.empty(0, dtype=torch.uint8, device=DEV)
    check_epilogue(mc, pass_id, s, t, dt, CASES[1], 621, ws=empty, want=("splits=1",))


def test_epilogue_identity_is_the_plain_call(mc):
    """alpha 1, beta 0, fp32 output runs the plain kernels: bitwise the plain result."""
    s = REDUCED["resnet3x3"]
    t = {k: v.to(DEV) for k, v in inputs(WORKLOADS["resnet3x3"], "bf16", shape=s, seed_offset=63).items()}
    a = mc.conv2d_bwd_data(t["dy"], t["w"], (s.H, s.W), s.pad, s.stride)
    b = mc.conv2d_bwd_data_ex(t["dy"], t["w"], (s.H, s.W), s.pad, s.stride, 1.0, 0.0)
    assert torch.equal(a, b)
    a = mc.conv2d_bwd_filter(t["x"], t["dy"], (s.R, s.S), s.pad, s.stride)
    b = mc.conv2d_bwd_filter_ex(t["x"], t["dy"], (s.R, s.S), s.pad, s.stride, 1.0, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ----------------------------------------------------------------------------- each kernel family

FAMILY = [
    # (shape, dtype, pass, plan words)
    (ConvShape(2, 3, 37, 70, 16, 7, 7, (3, 3), (2, 2), 19, 35), "bf16", "bwd_data", ("algo=tinyc",)),
    (ConvShape(2, 4, 18, 20, 24, 1, 1, (0, 0), (2, 2), 9, 10), "f32", "bwd_data", ("algo=tinyc",)),
    (ConvShape(2, 3, 37, 70, 64, 7, 7, (3, 3), (2, 2), 19, 35), "f32", "bwd_data", ("algo=tinyc", "form=mfma")),
    (ConvShape(3, 192, 40, 40, 64, 1, 1, (0, 0), (2, 2), 20, 20), "bf16", "bwd_data", ("algo=pointwise",)),
    (ConvShape(2, 96, 8, 8, 128, 1, 1, (0, 0), (1, 1), 8, 8), "bf16", "bwd_data", ("algo=pointwise",)),
    (ConvShape(2, 64, 20, 24, 96, 3, 3, (1, 1), (1, 1), 20, 24), "bf16", "bwd_data", ("algo=patch",)),
    (ConvShape(1, 32, 9, 14, 64, 5, 3, (2, 0), (1, 1), 9, 12), "bf16", "bwd_data", ("algo=patch",)),
    (ConvShape(2, 40, 18, 18, 48, 1, 1, (0, 0), (3, 3), 6, 6), "f32", "bwd_data", ("algo=igemm",)),   # dead phases
    (ConvShape(2, 40, 20, 20, 48, 1, 1, (0, 0), (5, 5), 4, 4), "f32", "bwd_data", ("algo=igemm",)),   # 25 phases
    (ConvShape(257, 64, 16, 16, 64, 3, 3, (1, 1), (1, 1), 16, 16), "bf16", "bwd_filter", ("mma=16x16x32",)),
    (ConvShape(6, 96, 28, 28, 200, 3, 3, (1, 1), (1, 1), 28, 28), "bf16", "bwd_filter", ("tile=128x", "mma=16x16x32")),
    (ConvShape(257, 64, 13, 14, 64, 3, 3, (1, 1), (1, 1), 13, 14), "bf16", "bwd_filter", ("form=pair",)),
    (ConvShape(20, 512, 13, 14, 512, 3, 3, (1, 1), (1, 1), 13, 14), "bf16", "bwd_filter",
     ("tile=128x", "mma=32x32x16")),
    (ConvShape(2, 64, 9, 8, 200, 2, 3, (0, 1), (1, 1), 8, 8), "bf16", "bwd_filter", ("algo=patch",)),
    (ConvShape(2, 48, 17, 15, 40, 3, 3, (1, 1), (2, 2), 9, 8), "f32", "bwd_filter", ("algo=igemm",)),
    (ConvShape(3, 192, 40, 40, 64, 1, 1, (0, 0), (2, 2), 20, 20), "bf16", "bwd_filter", ("algo=pointwise",)),
    (ConvShape(2, 3, 37, 71, 64, 7, 7, (3, 3), (2, 2), 19, 36), "f32", "bwd_filter", ("algo=tinyc", "form=mfma")),
    (ConvShape(1, 3, 7, 23, 64, 7, 7, (0, 3), (2, 2), 1, 12), "f32", "bwd_filter", ("algo=tinyc", "splits=1")),
]


@pytest.mark.parametrize("budget", ["plan", "none"])
@pytest.mark.parametrize("i", range(len(FAMILY)))
def test_epilogue_kernel_families(mc, i, budget):
    s, dt, pass_id, want = FAMILY[i]
    if budget == "none" and pass_id != "bwd_filter":
        pytest.skip("the budget changes only the backward-filter split count")
    ws = torch.empty(0, dtype=torch.uint8, device=DEV) if budget == "none" else None
    t = inputs(WORKLOADS["deep3x3"], dt, shape=s, seed_offset=64)
    for j, c in enumerate(CASES[:2]):
        check_epilogue(mc, pass_id, s, t, dt, c, 641 + j, ws=ws, want=want if ws is None else ("splits=1",))


# ----------------------------------------------------------------------------- deconvolution bias

DECONV_BIAS = [
    ConvShape(2, 96, 14, 14, 256, 4, 4, (1, 1), (2, 2), 7, 7),      # deconv4x4 reduced
    ConvShape(2, 8, 12, 12, 16, 1, 1, (0, 0), (2, 2), 6, 6),        # 1x1 stride 2: positions with no tap
    ConvShape(1, 24, 15, 15, 32, 1, 1, (0, 0), (3, 3), 5, 5),       # stride 3: 8 of 9 phases without taps
    ConvShape(2, 96, 16, 16, 128, 1, 1, (0, 0), (2, 2), 8, 8),      # bf16: the pointwise kernel
    ConvShape(2, 3, 20, 20, 16, 4, 4, (1, 1), (2, 2), 10, 10),      # 3 output channels: few-channel kernel
    ConvShape(2, 64, 12, 12, 64, 3, 3, (1, 1), (1, 1), 12, 12),     # stride 1, bf16: the patch kernel
    ConvShape(2, 96, 28, 28, 256, 4, 4, (1, 1), (2, 2), 14, 14),    # bf16: the patch kernel by stride phases
]


@pytest.mark.parametrize("relu", [False, True])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("i", range(len(DECONV_BIAS)))
def test_deconv_forward_bias(mc, i, dt, relu):
    """act(alpha * deconv + beta * y + bias[c_out]); positions that no tap reaches get
    act(beta * y + bias)."""
    s = DECONV_BIAS[i]
    t = inputs(WORKLOADS["deconv4x4"], dt, shape=s, seed_offset=65)
    bias = draw((s.C,), Dist("uniform", -1, 1), 651)
    for j, c in enumerate(CASES):
        check_epilogue(mc, "deconv_fwd", s, t, dt, c, 652 + j, bias=bias, relu=relu)


# ----------------------------------------------------------------------------- bias gradient

BIAS_SHAPES = [(2, 4, 8, 8), (64, 64, 56, 56), (64, 512, 28, 28), (32, 64, 112, 112), (256, 512, 14, 14),
               (3, 7, 13, 13), (5, 33, 1, 1), (1, 1, 3, 5)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", BIAS_SHAPES)
def test_bias_gradient(mc, shape, dt):
    """db = alpha * sum_{n,p,q} dy + beta * db against the oracle, the workloads' dy shapes and
    ragged ones (P*Q not a multiple of 4); repeated calls are bitwise identical."""
    dy = draw(shape, Dist("normal", 0.01), 661).to(TDT[dt])
    prev = draw((shape[1],), Dist("uniform", -1, 1), 662)
    _say(f"[bias grad] {shape} {dt}")
    d = dy.to(DEV)
    got = mc.conv2d_bwd_bias(d, 0.75, -0.5, db=prev.to(DEV))
    again = mc.conv2d_bwd_bias(d, 0.75, -0.5, db=prev.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(got, again)
    ref = oracle.conv2d_bwd_bias(dy.float().numpy(), 0.75, -0.5, prev.numpy())
    err = rel_err(got.cpu().numpy(), ref)
    _say(f"    rel err {err:.3e}")
    assert err <= TOL["f32"]   # fp64 sums: only the final rounding to fp32
    plain = mc.conv2d_bwd_bias(d)
    torch.cuda.synchronize()
    assert rel_err(plain.cpu().numpy(), oracle.conv2d_bwd_bias(dy.float().numpy())) <= TOL["f32"]
