"""GPU parity of the generalised convolution (convnd_*): 1 to 3 spatial dimensions, groups,
dilation, asymmetric and "same" padding, every stride, fp32 and bf16 inputs, all three passes,
against the generalised oracle element by element, and bit for bit on integer-valued inputs
(every partial sum exact).  Outputs are pre-filled with NaN, so an unwritten element fails.
Problems that are plain 2-D or 1-D convolutions must run the specialised 2-D kernels; the rest
the generic kernel (plan asserted).  Shapes span several 64 x 64 tiles with ragged tails and
reductions longer than several steps.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import Dist, draw

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}
DEV = "cuda:0"
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


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


# (N, C, K, groups, in, filt, pad_lo, pad_hi, stride, dilation, generic)
ND_CASES = [
    # 1-D
    (3, 40, 72, 1, (131,), (5,), (2,), (2,), (1,), (1,), False),        # plain: the 2-D kernels (H = 1)
    (2, 48, 80, 1, (150,), (3,), (4,), (1,), (2,), (3,), True),         # dilated, strided, asymmetric
    (2, 64, 64, 8, (97,), (7,), (3,), (3,), (1,), (1,), True),          # grouped
    # 2-D
    (2, 32, 96, 4, (17, 19), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1), True),      # 4 groups
    (2, 48, 48, 48, (21, 20), (3, 3), (1, 1), (1, 1), (2, 2), (1, 1), True),     # depthwise, stride 2
    (2, 40, 72, 1, (23, 18), (3, 3), (2, 2), (2, 2), (1, 1), (2, 2), True),      # dilation 2
    (2, 24, 80, 2, (19, 22), (3, 2), (0, 2), (2, 1), (2, 1), (1, 3), True),      # asym pads, mixed
    (3, 36, 68, 1, (15, 16), (5, 3), (3, 0), (1, 2), (1, 1), (1, 1), True),      # asymmetric only
    # 3-D
    (2, 16, 40, 1, (6, 10, 12), (3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), (1, 1, 1), True),
    (2, 24, 24, 3, (7, 9, 8), (3, 3, 2), (1, 0, 1), (1, 1, 0), (2, 1, 2), (1, 2, 1), True),
    (1, 20, 36, 1, (5, 11, 13), (1, 3, 3), (0, 2, 1), (0, 2, 1), (1, 2, 1), (1, 2, 1), True),
    (2, 32, 16, 2, (8, 8, 8), (1, 1, 1), (0, 0, 0), (0, 0, 0), (2, 2, 2), (1, 1, 1), True),
    (1, 8, 12, 1, (1, 9, 10), (1, 3, 3), (0, 1, 1), (0, 1, 1), (1, 1, 1), (1, 1, 1), False),   # depth 1
]


def _case(i):
    N, C, K, G, ins, filt, lo, hi, st, dil, generic = ND_CASES[i]
    outs = oracle.nd_out_size(ins, filt, lo, hi, st, dil)
    return N, C, K, G, ins, filt, lo, hi, st, dil, outs, generic


def _inputs(i, dt, integer, seed):
    N, C, K, G, ins, filt, lo, hi, st, dil, outs, _ = _case(i)
    dist = Dist("int", -4, 4) if integer else Dist("uniform", -1, 1)
    t = {"x": draw((N, C) + ins, dist, seed), "w": draw((K, C // G) + filt, dist, seed + 1),
         "dy": draw((N, K) + outs, dist, seed + 2)}
    return {k: v.to(TDT[dt]) for k, v in t.items()}


def _run(mc, pass_id, i, t, ws=None):
    N, C, K, G, ins, filt, lo, hi, st, dil, outs, _ = _case(i)
    d = {k: v.to(DEV) for k, v in t.items()}
    kw = dict(groups=G, pad_lo=lo, pad_hi=hi, stride=st, dilation=dil, workspace=ws)
    if pass_id == "fwd":
        out = torch.full((N, K) + outs, float("nan"), device=DEV)
        mc.convnd_fwd(d["x"], d["w"], y=out, **kw)
    elif pass_id == "bwd_data":
        out = torch.full((N, C) + ins, float("nan"), device=DEV)
        mc.convnd_bwd_data(d["dy"], d["w"], ins, dx=out, **kw)
    else:
        out = torch.full((K, C // G) + filt, float("nan"), device=DEV)
        mc.convnd_bwd_filter(d["x"], d["dy"], filt, dw=out, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle(pass_id, i, t):
    N, C, K, G, ins, filt, lo, hi, st, dil, outs, _ = _case(i)
    f = {k: v.float().numpy() for k, v in t.items()}
    if pass_id == "fwd":
        return oracle.convnd_fwd(f["x"], f["w"], G, lo, hi, st, dil)
    if pass_id == "bwd_data":
        return oracle.convnd_bwd_data(f["dy"], f["w"], ins, G, lo, hi, st, dil)
    return oracle.convnd_bwd_filter(f["x"], f["dy"], filt, G, lo, hi, st, dil)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("pass_id", ["fwd", "bwd_data", "bwd_filter"])
@pytest.mark.parametrize("i", range(len(ND_CASES)))
def test_convnd_matches_oracle(mc, i, pass_id, dt):
    N, C, K, G, ins, filt, lo, hi, st, dil, outs, generic = _case(i)
    d = mc.nd_desc(N, C, K, ins, filt, G, lo, hi, st, dil)
    assert mc.nd_out(d) == outs
    pid = {"fwd": mc.FWD, "bwd_data": mc.BWD_DATA, "bwd_filter": mc.BWD_FILTER}[pass_id]
    desc = mc.convnd_describe(pid, d, mc.F32 if dt == "f32" else mc.BF16)
    assert ("algo=generic" in desc) == generic, desc
    _say(f"[convnd] case {i} {pass_id} {dt} {ND_CASES[i][:10]} :: {desc}")
    t = _inputs(i, dt, False, 700 + 10 * i)
    got = _run(mc, pass_id, i, t)
    assert not np.isnan(got).any(), "output elements left unwritten"
    err = rel_err(got, _oracle(pass_id, i, t))
    _say(f"    rel err {err:.3e}")
    assert err <= TOL[dt]
    ti = _inputs(i, dt, True, 900 + 10 * i)
    got = _run(mc, pass_id, i, ti)
    assert np.array_equal(got.astype(np.float64), _oracle(pass_id, i, ti))


@pytest.mark.parametrize("i", [i for i, c in enumerate(ND_CASES) if c[-1]])
def test_convnd_backward_filter_without_workspace(mc, i):
    """Budget 0: one split, dW written directly (bitwise equal on integer inputs)."""
    N, C, K, G, ins, filt, lo, hi, st, dil, outs, _ = _case(i)
    d = mc.nd_desc(N, C, K, ins, filt, G, lo, hi, st, dil)
    assert "splits=1 " in mc.convnd_describe(mc.BWD_FILTER, d, mc.BF16, 0)
    ti = _inputs(i, "bf16", True, 950 + i)
    got = _run(mc, "bwd_filter", i, ti, ws=torch.empty(0, dtype=torch.uint8, device=DEV))
    assert np.array_equal(got.astype(np.float64), _oracle("bwd_filter", i, ti))


@pytest.mark.parametrize("dims", [1, 2, 3])
def test_convnd_same_padding(mc, dims):
    """"same" padding: output ceil(in / stride), the library's pads equal the oracle's reading."""
    ins = (13, 11, 9)[:dims]
    filt, st, dil = (4, 3, 5)[:dims], (2, 1, 3)[:dims], (1, 2, 1)[:dims]
    d = mc.nd_desc(2, 12, 20, ins, filt, 2, stride=st, dilation=dil, padding="same")
    lo, hi = oracle.padding_for("same", ins, filt, st, dil)
    assert tuple(d.pad_lo[:dims]) == lo and tuple(d.pad_hi[:dims]) == hi
    assert mc.nd_out(d) == tuple(-(-i // s) for i, s in zip(ins, st))
    x = draw((2, 12) + ins, Dist("uniform", -1, 1), 960).to(DEV)
    w = draw((20, 6) + filt, Dist("uniform", -1, 1), 961).to(DEV)
    y = mc.convnd_fwd(x, w, groups=2, stride=st, dilation=dil, padding="same")
    torch.cuda.synchronize()
    ref = oracle.convnd_fwd(x.cpu().numpy(), w.cpu().numpy(), 2, lo, hi, st, dil)
    assert rel_err(y.cpu().numpy(), ref) <= TOL["f32"]


def test_sentence_cnn_as_1d(mc):
    """The sentence-classification shape as a 1-D convolution: 300-dimensional embeddings as
    channels, 2060 positions, 500 filters of width 5 (plain 1-D: the 2-D kernels)."""
    N, C, K, L, S = 1, 300, 500, 2060, 5
    x = draw((N, C, L), Dist("uniform", -1, 1), 970).to(torch.bfloat16)
    w = draw((K, C, S), Dist("uniform", -1, 1), 971).to(torch.bfloat16)
    d = mc.nd_desc(N, C, K, (L,), (S,))
    assert "algo=generic" not in mc.convnd_describe(mc.FWD, d, mc.BF16)
    y = mc.convnd_fwd(x.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.convnd_fwd(x.float().numpy(), w.float().numpy())
    err = rel_err(y.cpu().numpy(), ref)
    _say(f"[sentence 1-D] rel err {err:.3e}")
    assert err <= TOL["bf16"]
