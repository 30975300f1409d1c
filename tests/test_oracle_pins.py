"""Pins for the CPU oracle: checks it against things other than itself.

Each pin ties the oracle to something the pages or the mathematics fix
independently of the oracle's own loops:

- 2-D cross-correlation of scipy.signal.correlate2d (a library routine) for the
  forward pass, with stride as subsampling and padding as explicit zeros;
- the 1x1, stride-1, pad-0 forward pass is a plain matrix product;
- a delta filter reproduces the shifted (zero-padded) input exactly;
- all-ones input and filter give the count of in-bounds taps, exactly;
- the adjoint identities <y, fwd(x,W)> = <bwd_data(y,W), x> = <bwd_filter(x,y), W>;
- the dense operator built column by column from the forward pass: its
  transpose is backward-data and its filter responses give backward-filter;
- backward-data equals a full (flipped-kernel) convolution of the zero-upsampled
  gradient, the textbook transposed-convolution identity;
- torch's CPU float64 conv2d / conv2d_input / conv2d_weight / conv_transpose2d
  (a library implementation of the same operators);
- the deconvolution role swap (MXNet "mkldnn_deconvolution.cc",
  MKLDNNDeconvFwd::Execute) against torch's conv_transpose2d, whose weight is
  (in, out, kh, kw) like the page's.

A last test plants plausible mistakes (flipped filter, swapped R/S, padding off
by one, a dropped channel, swapped K/C, a sign error) in copies of the oracle
and checks that the pins reject every one of them.
"""
import json
import os

import numpy as np
import pytest
import scipy.signal
import torch
import torch.nn.functional as F

import oracle
from workloads import Dist, draw

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# (N, C, H, W, K, R, S, pad_h, pad_w, stride_h, stride_w)
SHAPES = [
    (2, 3, 8, 8, 4, 3, 3, 1, 1, 1, 1),      # the tiny workload's shape
    (1, 2, 7, 9, 3, 3, 2, 0, 1, 1, 1),      # R != S, H != W, mixed pads
    (2, 2, 9, 8, 3, 3, 3, 1, 0, 2, 2),      # stride 2, floor case on W
    (1, 3, 11, 10, 2, 5, 3, 2, 1, 3, 2),    # stride 3 / 2, floor cases
    (2, 2, 6, 6, 2, 1, 1, 0, 0, 2, 2),      # 1x1 stride 2 (uncovered dx positions)
    (1, 1, 5, 7, 2, 5, 7, 0, 0, 1, 1),      # H == R and W == S: 1x1 output
    (1, 2, 4, 12, 3, 4, 3, 0, 2, 1, 1),     # H == R only (conv1d-like)
    (1, 2, 7, 7, 2, 7, 7, 3, 3, 2, 2),      # 7x7 stride 2 stem-like
    (2, 2, 6, 5, 3, 4, 4, 3, 3, 2, 2),      # pad == R - 1, 4x4 stride 2
    (1, 2, 3, 3, 2, 3, 3, 4, 4, 3, 3),      # pad larger than the filter
]


def _dims(sh):
    N, C, H, W, K, R, S, ph, pw, sh_, sw = sh
    P, Q = oracle.out_size(H, W, R, S, (ph, pw), (sh_, sw))
    return N, C, H, W, K, R, S, (ph, pw), (sh_, sw), P, Q


def _rand(shape, seed):
    return draw(shape, Dist("uniform", -1.0, 1.0), seed).numpy().astype(np.float64)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ----------------------------------------------------------------------------- pins
# Each pin takes the implementation under test as arguments so that the same
# pin can be run against planted mistakes (see test_pins_reject_planted_mistakes).

def pin_fwd_scipy(fwd, sh, seed=1):
    """Forward = sum over c of scipy.signal.correlate2d(padded x, W, 'valid'), subsampled."""
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(sh)
    x, w = _rand((N, C, H, W), seed), _rand((K, C, R, S), seed + 1)
    xp = np.pad(x, ((0, 0), (0, 0), (pad[0], pad[0]), (pad[1], pad[1])))
    ref = np.zeros((N, K, P, Q))
    for n in range(N):
        for k in range(K):
            acc = sum(scipy.signal.correlate2d(xp[n, c], w[k, c], mode="valid") for c in range(C))
            ref[n, k] = acc[::st[0], ::st[1]][:P, :Q]
    return _rel(fwd(x, w, pad, st), ref) < 1e-12


def pin_fwd_gemm(fwd, seed=2):
    """1x1, stride 1, pad 0: y[n] = W[:, :, 0, 0] @ x[n] reshaped to (C, H*W)."""
    N, C, H, W, K = 2, 5, 4, 6, 3
    x, w = _rand((N, C, H, W), seed), _rand((K, C, 1, 1), seed + 1)
    ref = np.stack([(w[:, :, 0, 0] @ x[n].reshape(C, H * W)).reshape(K, H, W) for n in range(N)])
    return _rel(fwd(x, w, (0, 0), (1, 1)), ref) < 1e-13


def pin_fwd_delta(fwd, sh, r0, s0, seed=3):
    """W[k,c,r,s] = [k == c][r == r0][s == s0] reproduces the shifted input exactly."""
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(sh)
    K = C
    x = _rand((N, C, H, W), seed)
    w = np.zeros((K, C, R, S))
    for c in range(C):
        w[c, c, r0, s0] = 1.0
    ref = np.zeros((N, K, P, Q))
    for p in range(P):
        for q in range(Q):
            i, j = p * st[0] - pad[0] + r0, q * st[1] - pad[1] + s0
            if 0 <= i < H and 0 <= j < W:
                ref[:, :, p, q] = x[:, :, i, j]
    return np.array_equal(fwd(x, w, pad, st), ref)


def pin_fwd_ones(fwd, sh):
    """x = 1, W = 1: y[n,k,p,q] = C * #valid r * #valid s, exactly."""
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(sh)
    x, w = np.ones((N, C, H, W)), np.ones((K, C, R, S))
    vr = np.array([sum(0 <= p * st[0] - pad[0] + r < H for r in range(R)) for p in range(P)])
    vs = np.array([sum(0 <= q * st[1] - pad[1] + s < W for s in range(S)) for q in range(Q)])
    ref = np.broadcast_to(C * vr[:, None] * vs[None, :], (N, K, P, Q))
    return np.array_equal(fwd(x, w, pad, st), ref)


def pin_adjoint(fwd, bwd_data, bwd_filter, sh, seed=4):
    """<y, fwd(x,W)> = <bwd_data(y,W), x> = <bwd_filter(x,y), W>."""
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(sh)
    x, w, y = _rand((N, C, H, W), seed), _rand((K, C, R, S), seed + 1), _rand((N, K, P, Q), seed + 2)
    a = float(np.sum(y * fwd(x, w, pad, st)))
    b = float(np.sum(bwd_data(y, w, (H, W), pad, st) * x))
    c = float(np.sum(bwd_filter(x, y, (R, S), pad, st) * w))
    scale = float(np.sum(np.abs(y)) * np.sum(np.abs(w)) * np.max(np.abs(x)))
    return abs(a - b) <= 1e-12 * scale and abs(a - c) <= 1e-12 * scale


def pin_operator(fwd, bwd_data, bwd_filter, sh, seed=5):
    """Dense operator T built from fwd on basis inputs: bwd_data = T^T dy entrywise;
    bwd_filter[kcrs] = <dy, fwd(x, e_kcrs)> entrywise."""
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(sh)
    w, x, dy = _rand((K, C, R, S), seed), _rand((N, C, H, W), seed + 1), _rand((N, K, P, Q), seed + 2)
    nx = N * C * H * W
    T = np.zeros((N * K * P * Q, nx))
    for j in range(nx):
        e = np.zeros(nx)
        e[j] = 1.0
        T[:, j] = fwd(e.reshape(N, C, H, W), w, pad, st).ravel()
    ok_d = _rel(bwd_data(dy, w, (H, W), pad, st).ravel(), T.T @ dy.ravel()) < 1e-12
    nw = K * C * R * S
    ref = np.zeros(nw)
    for j in range(nw):
        e = np.zeros(nw)
        e[j] = 1.0
        ref[j] = np.sum(dy * fwd(x, e.reshape(K, C, R, S), pad, st))
    ok_f = _rel(bwd_filter(x, dy, (R, S), pad, st).ravel(), ref) < 1e-12
    return ok_d and ok_f


def pin_zero_insertion(bwd_data, sh, seed=6):
    """bwd_data = crop(full 2-D convolution of the zero-upsampled dy with W[k,c])."""
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(sh)
    w, dy = _rand((K, C, R, S), seed), _rand((N, K, P, Q), seed + 1)
    up = np.zeros((N, K, (P - 1) * st[0] + 1, (Q - 1) * st[1] + 1))
    up[:, :, ::st[0], ::st[1]] = dy
    ref = np.zeros((N, C, H, W))
    for n in range(N):
        for c in range(C):
            full = sum(scipy.signal.convolve2d(up[n, k], w[k, c], mode="full") for k in range(K))
            big = np.zeros((H + pad[0] + full.shape[0], W + pad[1] + full.shape[1]))
            big[:full.shape[0], :full.shape[1]] = full
            ref[n, c] = big[pad[0]:pad[0] + H, pad[1]:pad[1] + W]
    return _rel(bwd_data(dy, w, (H, W), pad, st), ref) < 1e-12


def pin_torch(fwd, bwd_data, bwd_filter, sh, seed=7):
    """torch CPU float64 conv2d and its input / weight gradients."""
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(sh)
    x, w, dy = _rand((N, C, H, W), seed), _rand((K, C, R, S), seed + 1), _rand((N, K, P, Q), seed + 2)
    tx, tw, tdy = (torch.from_numpy(a) for a in (x, w, dy))
    y_ref = F.conv2d(tx, tw, stride=st, padding=pad).numpy()
    dx_ref = torch.nn.grad.conv2d_input(tx.shape, tw, tdy, stride=st, padding=pad).numpy()
    dw_ref = torch.nn.grad.conv2d_weight(tx, tw.shape, tdy, stride=st, padding=pad).numpy()
    return (_rel(fwd(x, w, pad, st), y_ref) < 1e-12 and
            _rel(bwd_data(dy, w, (H, W), pad, st), dx_ref) < 1e-12 and
            _rel(bwd_filter(x, dy, (R, S), pad, st), dw_ref) < 1e-12)


ORACLE = (oracle.conv2d_fwd, oracle.conv2d_bwd_data, oracle.conv2d_bwd_filter)


# ----------------------------------------------------------------------------- tests

@pytest.mark.parametrize("sh", SHAPES)
def test_fwd_matches_library_correlation(sh):
    assert pin_fwd_scipy(oracle.conv2d_fwd, sh)


def test_fwd_1x1_is_gemm():
    assert pin_fwd_gemm(oracle.conv2d_fwd)


@pytest.mark.parametrize("sh", [SHAPES[1], SHAPES[3], SHAPES[7], SHAPES[8]])
def test_fwd_delta_filter_is_exact_shift(sh):
    R, S = sh[5], sh[6]
    # r0 != s0 and corner taps, so a swapped R/S or a flipped filter shows
    for r0, s0 in {(0, S - 1), (R - 1, 0), (R // 2, 0), (R - 1, S - 1)}:
        assert pin_fwd_delta(oracle.conv2d_fwd, sh, r0, s0)


@pytest.mark.parametrize("sh", SHAPES)
def test_fwd_all_ones_counts_taps(sh):
    assert pin_fwd_ones(oracle.conv2d_fwd, sh)


def test_fwd_all_ones_resnet_border_counts():
    # 3x3, pad 1, stride 1 on 6x6 with C = 64: interior 576, edges 384, corners 256
    y = oracle.conv2d_fwd(np.ones((1, 64, 6, 6)), np.ones((1, 64, 3, 3)), (1, 1), (1, 1))[0, 0]
    assert y[2, 2] == 576 and y[0, 2] == 384 and y[2, 5] == 384 and y[0, 0] == 256 and y[5, 5] == 256


@pytest.mark.parametrize("sh", SHAPES)
def test_adjoint_identities(sh):
    assert pin_adjoint(*ORACLE, sh)


@pytest.mark.parametrize("sh", [SHAPES[0], SHAPES[2], SHAPES[3], SHAPES[4], SHAPES[8]])
def test_bruteforce_operator(sh):
    sh = (1,) + sh[1:]  # one image keeps the dense operator small
    assert pin_operator(*ORACLE, sh)


@pytest.mark.parametrize("sh", SHAPES)
def test_bwd_data_zero_insertion_identity(sh):
    assert pin_zero_insertion(oracle.conv2d_bwd_data, sh)


@pytest.mark.parametrize("sh", SHAPES)
def test_library_conv_and_gradients(sh):
    assert pin_torch(*ORACLE, sh)


def test_fwd_scaling_and_linearity():
    sh = SHAPES[3]
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(sh)
    x1, x2, w = _rand((N, C, H, W), 11), _rand((N, C, H, W), 12), _rand((K, C, R, S), 13)
    y1 = oracle.conv2d_fwd(x1, w, pad, st)
    assert np.array_equal(oracle.conv2d_fwd(8.0 * x1, w, pad, st), 8.0 * y1)
    y12 = oracle.conv2d_fwd(0.5 * x1 - 3.0 * x2, w, pad, st)
    assert _rel(y12, 0.5 * y1 - 3.0 * oracle.conv2d_fwd(x2, w, pad, st)) < 1e-13


@pytest.mark.parametrize("shape", [
    # (N, Cin, Hin, Win, Cout, R, S, pad, stride, Hout, Wout)
    (2, 4, 5, 5, 3, 4, 4, 1, 2, 10, 10),
    (1, 3, 4, 6, 2, 3, 3, 1, 2, 8, 12),     # Hout one above the minimum (floor reading)
    (2, 2, 3, 3, 5, 3, 3, 0, 1, 5, 5),
])
def test_deconv_role_swap_matches_conv_transpose(shape):
    N, Cin, Hin, Win, Cout, R, S, p, s, Hout, Wout = shape
    x_in, w = _rand((N, Cin, Hin, Win), 21), _rand((Cin, Cout, R, S), 22)
    out = oracle.deconv2d_fwd(x_in, w, (Hout, Wout), (p, p), (s, s))
    # role swap: identical to backward-data with the weight used as KCRS, K = Cin
    assert np.array_equal(out, oracle.conv2d_bwd_data(x_in, w, (Hout, Wout), (p, p), (s, s)))
    # torch's conv_transpose2d takes weights (in, out, kh, kw) like the page
    Hmin, Wmin = (Hin - 1) * s - 2 * p + R, (Win - 1) * s - 2 * p + S
    ref = F.conv_transpose2d(torch.from_numpy(x_in), torch.from_numpy(w), stride=s, padding=p,
                             output_padding=(Hout - Hmin, Wout - Wmin)).numpy()
    assert _rel(out, ref) < 1e-12
    # adjoint: <deconv(x_in, w), z> = <x_in, conv2d_fwd(z, w as KCRS)>
    z = _rand((N, Cout, Hout, Wout), 23)
    a = np.sum(out * z)
    b = np.sum(x_in * oracle.conv2d_fwd(z, w, (p, p), (s, s)))
    assert abs(a - b) <= 1e-12 * np.sum(np.abs(out)) * np.max(np.abs(z))


DECONV_SHAPES = [
    # (N, Cin, Hin, Win, Cout, R, S, pad, stride, Hout, Wout)
    (2, 4, 5, 5, 3, 4, 4, 1, 2, 10, 10),
    (1, 3, 4, 6, 2, 3, 3, 1, 2, 8, 12),     # Hout one above the minimum (floor reading)
    (2, 2, 3, 3, 5, 3, 3, 0, 1, 5, 5),
    (1, 2, 3, 4, 3, 2, 3, 0, 3, 9, 13),     # stride 3, R != S, output one above the minimum
]


@pytest.mark.parametrize("shape", DECONV_SHAPES)
def test_deconv_backward_matches_autograd(shape):
    """Both deconvolution gradients against torch autograd of conv_transpose2d in fp64."""
    N, Cin, Hin, Win, Cout, R, S, p, s, Hout, Wout = shape
    x_in, w, z = _rand((N, Cin, Hin, Win), 41), _rand((Cin, Cout, R, S), 42), _rand((N, Cout, Hout, Wout), 43)
    Hmin, Wmin = (Hin - 1) * s - 2 * p + R, (Win - 1) * s - 2 * p + S
    xt = torch.from_numpy(x_in).requires_grad_(True)
    wt = torch.from_numpy(w).requires_grad_(True)
    out = F.conv_transpose2d(xt, wt, stride=s, padding=p, output_padding=(Hout - Hmin, Wout - Wmin))
    out.backward(torch.from_numpy(z))
    din = oracle.deconv2d_bwd_data(z, w, (Hin, Win), (p, p), (s, s))
    dw = oracle.deconv2d_bwd_filter(x_in, z, (R, S), (p, p), (s, s))
    assert din.shape == x_in.shape and dw.shape == w.shape
    assert _rel(din, xt.grad.numpy()) < 1e-12
    assert _rel(dw, wt.grad.numpy()) < 1e-12


@pytest.mark.parametrize("shape", DECONV_SHAPES)
def test_deconv_backward_adjoint_and_brute_force(shape):
    """<deconv(x, w), z> = <x, deconv_bwd_data(z, w)> = <w, deconv_bwd_filter(x, z)>, and on
    the smallest shapes each gradient entry equals the response to one basis vector."""
    N, Cin, Hin, Win, Cout, R, S, p, s, Hout, Wout = shape
    pad, st = (p, p), (s, s)
    x_in, w, z = _rand((N, Cin, Hin, Win), 44), _rand((Cin, Cout, R, S), 45), _rand((N, Cout, Hout, Wout), 46)
    a = np.sum(oracle.deconv2d_fwd(x_in, w, (Hout, Wout), pad, st) * z)
    din = oracle.deconv2d_bwd_data(z, w, (Hin, Win), pad, st)
    dw = oracle.deconv2d_bwd_filter(x_in, z, (R, S), pad, st)
    assert abs(a - np.sum(x_in * din)) <= 1e-12 * max(1.0, abs(a)) * 100
    assert abs(a - np.sum(w * dw)) <= 1e-12 * max(1.0, abs(a)) * 100
    if x_in.size > 200:
        return
    for j in range(x_in.size):
        e = np.zeros(x_in.size)
        e[j] = 1.0
        col = oracle.deconv2d_fwd(e.reshape(x_in.shape), w, (Hout, Wout), pad, st)
        assert abs(din.ravel()[j] - np.sum(col * z)) < 1e-12 * np.sum(np.abs(z)) * np.max(np.abs(w))
    for j in range(w.size):
        e = np.zeros(w.size)
        e[j] = 1.0
        resp = oracle.deconv2d_fwd(x_in, e.reshape(w.shape), (Hout, Wout), pad, st)
        assert abs(dw.ravel()[j] - np.sum(resp * z)) < 1e-12 * np.sum(np.abs(z)) * np.max(np.abs(x_in))


@pytest.mark.parametrize("shape", DECONV_SHAPES[:2])
def test_deconv_backward_point_evaluators(shape):
    N, Cin, Hin, Win, Cout, R, S, p, s, Hout, Wout = shape
    pad, st = (p, p), (s, s)
    x_in, w, z = _rand((N, Cin, Hin, Win), 47), _rand((Cin, Cout, R, S), 48), _rand((N, Cout, Hout, Wout), 49)
    din = oracle.deconv2d_bwd_data(z, w, (Hin, Win), pad, st)
    dw = oracle.deconv2d_bwd_filter(x_in, z, (R, S), pad, st)
    i = np.arange(din.size)
    assert np.allclose(oracle.deconv2d_bwd_data_points(z, w, (Hin, Win), i, pad, st), din.ravel(),
                       rtol=0, atol=1e-13)
    i = np.arange(dw.size)
    assert np.allclose(oracle.deconv2d_bwd_filter_points(x_in, z, (R, S), i, pad, st), dw.ravel(),
                       rtol=0, atol=1e-13)


@pytest.mark.parametrize("case", [
    dict(alpha=1.0, beta=0.0, bias=False, relu=False),
    dict(alpha=0.5, beta=0.0, bias=True, relu=True),
    dict(alpha=-2.0, beta=1.0, bias=False, relu=False),
    dict(alpha=1.0, beta=-0.75, bias=True, relu=True),
])
def test_fused_forward_epilogue_matches_torch(case):
    """act(alpha * conv + beta * y_prev + bias) against torch fp64 (conv2d, broadcast add, relu)."""
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(SHAPES[3])
    x, w = _rand((N, C, H, W), 51), _rand((K, C, R, S), 52)
    bias = _rand((K,), 53) if case["bias"] else None
    y0 = _rand((N, K, P, Q), 54)
    got = oracle.conv2d_fwd_ex(x, w, pad, st, bias=bias, alpha=case["alpha"], beta=case["beta"],
                               y_prev=y0, relu=case["relu"])
    ref = case["alpha"] * F.conv2d(torch.from_numpy(x), torch.from_numpy(w), stride=st, padding=pad)
    ref = ref + case["beta"] * torch.from_numpy(y0)
    if bias is not None:
        ref = ref + torch.from_numpy(bias).view(1, K, 1, 1)
    if case["relu"]:
        ref = F.relu(ref)
    assert _rel(got, ref.numpy()) < 1e-12
    if case["relu"]:
        assert (got >= 0).all() and (got == 0).any()
    idx = np.random.Generator(np.random.PCG64(55)).integers(0, got.size, 40)
    pts = oracle.conv2d_fwd_ex_points(x, w, idx, pad, st, bias=bias, alpha=case["alpha"],
                                      beta=case["beta"], y_prev=y0, relu=case["relu"])
    assert np.allclose(pts, got.ravel()[idx], rtol=0, atol=1e-12)


def test_fused_forward_identity_and_unread_output():
    """alpha 1, beta 0, no bias, no relu is the plain forward bit for bit, and with beta 0 the
    previous output is never read (NaN there does not leak)."""
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(SHAPES[0])
    x, w = _rand((N, C, H, W), 56), _rand((K, C, R, S), 57)
    nan = np.full((N, K, P, Q), np.nan)
    assert np.array_equal(oracle.conv2d_fwd_ex(x, w, pad, st, y_prev=nan), oracle.conv2d_fwd(x, w, pad, st))


def _torch_grads(x, w, dy, pad, st, bias=None):
    """torch CPU float64 autograd of conv2d (+ bias): (dx, dw, db)."""
    xt = torch.from_numpy(x).requires_grad_(True)
    wt = torch.from_numpy(w).requires_grad_(True)
    bt = None if bias is None else torch.from_numpy(bias).requires_grad_(True)
    F.conv2d(xt, wt, bt, stride=st, padding=pad).backward(torch.from_numpy(dy))
    return xt.grad.numpy(), wt.grad.numpy(), None if bt is None else bt.grad.numpy()


EPI_CASES = [(1.0, 0.0), (0.5, 0.0), (-2.0, 1.0), (1.0, -0.75)]


@pytest.mark.parametrize("alpha,beta", EPI_CASES)
@pytest.mark.parametrize("sh", [SHAPES[1], SHAPES[3], SHAPES[4]])
def test_backward_epilogues_match_torch_autograd(sh, alpha, beta):
    """alpha * gradient + beta * previous, for both convolution gradients and both
    deconvolution gradients, against torch fp64 autograd scaled and added in torch."""
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(sh)
    x, w, dy = _rand((N, C, H, W), 61), _rand((K, C, R, S), 62), _rand((N, K, P, Q), 63)
    dx_prev, dw_prev = _rand((N, C, H, W), 64), _rand((K, C, R, S), 65)
    gx, gw, _ = _torch_grads(x, w, dy, pad, st)
    got = oracle.conv2d_bwd_data_ex(dy, w, (H, W), pad, st, alpha, beta, dx_prev)
    assert _rel(got, alpha * gx + beta * dx_prev) < 1e-12
    got = oracle.conv2d_bwd_filter_ex(x, dy, (R, S), pad, st, alpha, beta, dw_prev)
    assert _rel(got, alpha * gw + beta * dw_prev) < 1e-12
    # deconvolution view of the same operator: x_in = dy (C_in = K), out = [N, C, H, W]
    got = oracle.deconv2d_bwd_data_ex(x, w, (P, Q), pad, st, alpha, beta, dy)
    ref = alpha * F.conv2d(torch.from_numpy(x), torch.from_numpy(w), stride=st, padding=pad).numpy() + beta * dy
    assert _rel(got, ref) < 1e-12
    got = oracle.deconv2d_bwd_filter_ex(dy, x, (R, S), pad, st, alpha, beta, dw_prev)
    assert _rel(got, alpha * gw + beta * dw_prev) < 1e-12


@pytest.mark.parametrize("shape", DECONV_SHAPES)
@pytest.mark.parametrize("relu", [False, True])
def test_deconv_forward_epilogue_matches_conv_transpose(shape, relu):
    """act(alpha * deconv + beta * y_prev + bias[c_out]) against torch's conv_transpose2d with
    its bias argument (fp64), scaled and added in torch."""
    N, Cin, Hin, Win, Cout, R, S, p, s, Hout, Wout = shape
    x_in, w = _rand((N, Cin, Hin, Win), 66), _rand((Cin, Cout, R, S), 67)
    bias, y0 = _rand((Cout,), 68), _rand((N, Cout, Hout, Wout), 69)
    Hmin, Wmin = (Hin - 1) * s - 2 * p + R, (Win - 1) * s - 2 * p + S
    for alpha, beta in EPI_CASES:
        got = oracle.deconv2d_fwd_ex(x_in, w, (Hout, Wout), (p, p), (s, s), bias, alpha, beta, y0, relu)
        # alpha * (deconv + bias / alpha) = alpha * deconv + bias
        ref = alpha * F.conv_transpose2d(torch.from_numpy(x_in), torch.from_numpy(w), torch.from_numpy(bias / alpha),
                                         stride=s, padding=p, output_padding=(Hout - Hmin, Wout - Wmin))
        ref = ref + beta * torch.from_numpy(y0)
        if relu:
            ref = F.relu(ref)
        assert _rel(got, ref.numpy()) < 1e-12


@pytest.mark.parametrize("sh", [SHAPES[0], SHAPES[2], SHAPES[7]])
def test_bias_gradient_pins(sh):
    """db against (i) torch fp64 autograd of conv2d with a bias, (ii) backward-filter of a
    1x1 filter over an all-ones input (dW[k, 0, 0, 0] = sum of dy over channel k), and
    (iii) the adjoint of adding a bias: <dy, fwd_ex(bias = b) - fwd_ex(bias = 0)> = <db, b>."""
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(sh)
    x, w, dy, b = _rand((N, C, H, W), 71), _rand((K, C, R, S), 72), _rand((N, K, P, Q), 73), _rand((K,), 74)
    db = oracle.conv2d_bwd_bias(dy)
    assert db.shape == (K,)
    assert _rel(db, _torch_grads(x, w, dy, pad, st, bias=b)[2]) < 1e-12
    ones = np.ones((N, 1, P, Q))
    assert _rel(db, oracle.conv2d_bwd_filter(ones, dy, (1, 1))[:, 0, 0, 0]) < 1e-12
    d_out = oracle.conv2d_fwd_ex(x, w, pad, st, bias=b) - oracle.conv2d_fwd_ex(x, w, pad, st)
    assert abs(np.sum(dy * d_out) - np.sum(db * b)) < 1e-12 * np.sum(np.abs(dy)) * np.max(np.abs(b))
    prev = _rand((K,), 75)
    assert _rel(oracle.conv2d_bwd_bias(dy, -0.5, 2.0, prev), -0.5 * db + 2.0 * prev) < 1e-15


def test_backward_epilogue_identity_and_unread_output():
    """alpha 1, beta 0 is the plain gradient bit for bit, and with beta 0 the previous output
    is never read (NaN there does not leak)."""
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(SHAPES[2])
    x, w, dy = _rand((N, C, H, W), 76), _rand((K, C, R, S), 77), _rand((N, K, P, Q), 78)
    assert np.array_equal(oracle.conv2d_bwd_data_ex(dy, w, (H, W), pad, st, dx_prev=np.full((N, C, H, W), np.nan)),
                          oracle.conv2d_bwd_data(dy, w, (H, W), pad, st))
    assert np.array_equal(oracle.conv2d_bwd_filter_ex(x, dy, (R, S), pad, st, dw_prev=np.full(w.shape, np.nan)),
                          oracle.conv2d_bwd_filter(x, dy, (R, S), pad, st))
    assert np.array_equal(oracle.conv2d_bwd_bias(dy, db_prev=np.full(K, np.nan)), oracle.conv2d_bwd_bias(dy))


def _bias_grad_mutants():
    """Plausible mistakes in the bias gradient: the wrong axes summed, one image dropped,
    the mean instead of the sum, the previous value added with alpha's weight."""
    ref = oracle.conv2d_bwd_bias
    return {
        "sum over channels' spatial mean": lambda dy, a=1.0, b=0.0, p=None: a * np.asarray(dy).mean(axis=(0, 2, 3)),
        "last image dropped": lambda dy, a=1.0, b=0.0, p=None: ref(np.asarray(dy)[:-1], a, b, p),
        "width axis skipped": lambda dy, a=1.0, b=0.0, p=None: a * np.asarray(dy).sum(axis=(0, 2))[:, 0],
        "beta uses alpha": lambda dy, a=1.0, b=0.0, p=None: a * np.asarray(dy).sum(axis=(0, 2, 3)) + a * (
            0 if p is None else np.asarray(p)),
    }


@pytest.mark.parametrize("name", sorted(_bias_grad_mutants()))
def test_bias_gradient_pins_reject_planted_mistakes(name):
    mut = _bias_grad_mutants()[name]
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(SHAPES[2])
    x, w, dy, b = _rand((N, C, H, W), 81), _rand((K, C, R, S), 82), _rand((N, K, P, Q), 83), _rand((K,), 84)
    prev = _rand((K,), 85)
    ref = _torch_grads(x, w, dy, pad, st, bias=b)[2]
    ok_torch = _rel(mut(dy), ref) < 1e-12
    ok_beta = _rel(mut(dy, -0.5, 2.0, prev), -0.5 * ref + 2.0 * prev) < 1e-12
    assert not (ok_torch and ok_beta), f"planted mistake '{name}' passed the bias-gradient pins"


def test_deconv_workload_output_size():
    # input 16x16, 4x4 weights, stride 2, pad 1 -> 32x32 output; its conv view gives back 16x16
    assert oracle.out_size(32, 32, 4, 4, (1, 1), (2, 2)) == (16, 16)
    assert (16 - 1) * 2 - 2 * 1 + 4 == 32


@pytest.mark.parametrize("sh", [SHAPES[0], SHAPES[3], SHAPES[4], SHAPES[7]])
def test_point_evaluators_match_full(sh):
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(sh)
    x, w, dy = _rand((N, C, H, W), 31), _rand((K, C, R, S), 32), _rand((N, K, P, Q), 33)
    g = np.random.Generator(np.random.PCG64(34))
    y = oracle.conv2d_fwd(x, w, pad, st)
    i = g.integers(0, y.size, 50)
    assert np.allclose(oracle.conv2d_fwd_points(x, w, i, pad, st), y.ravel()[i], rtol=0, atol=1e-13)
    dx = oracle.conv2d_bwd_data(dy, w, (H, W), pad, st)
    i = g.integers(0, dx.size, 50)
    assert np.allclose(oracle.conv2d_bwd_data_points(dy, w, (H, W), i, pad, st), dx.ravel()[i],
                       rtol=0, atol=1e-13)
    dw = oracle.conv2d_bwd_filter(x, dy, (R, S), pad, st)
    i = g.integers(0, dw.size, 50)
    assert np.allclose(oracle.conv2d_bwd_filter_points(x, dy, (R, S), i, pad, st), dw.ravel()[i],
                       rtol=0, atol=1e-13)


def test_thread_count_does_not_change_results():
    # each thread owns whole output slices, so results are bitwise independent of threads
    sh = SHAPES[3]
    N, C, H, W, K, R, S, pad, st, P, Q = _dims(sh)
    x, w = _rand((N, C, H, W), 41), _rand((K, C, R, S), 42)
    y = oracle.conv2d_fwd(x, w, pad, st)
    y2 = oracle.conv2d_fwd(np.copy(x), np.copy(w), pad, st)
    assert np.array_equal(y, y2)


def test_golden_page_shapes():
    """Shapes and limits the pages state, with their output sizes (tests/golden)."""
    with open(os.path.join(GOLDEN, "page_shapes.json")) as f:
        g = json.load(f)
    sc = g["sentence_cnn"]
    P, Q = oracle.out_size(sc["H"], sc["W"], sc["R"], sc["S"], (0, 0), (1, 1))
    assert (P, Q) == (sc["expect_P"], sc["expect_Q"])
    assert g["workspace_cap_bytes"]["value"] == 1_000_000_000


def test_sentence_cnn_shape_reduced_filters():
    """The conv1d-like sentence-CNN shape (W == S) with 10% dense input, fewer filters:
    forward vs the library correlation, and the adjoint identity."""
    g = np.random.Generator(np.random.PCG64(51))
    H, W, R, S, K = 2060, 300, 5, 300, 3
    x = g.uniform(-1, 1, (1, 1, H, W)) * (g.random((1, 1, H, W)) < 0.1)
    w = g.uniform(-1, 1, (K, 1, R, S))
    y = oracle.conv2d_fwd(x, w)
    assert y.shape == (1, K, H - R + 1, 1)
    for k in range(K):
        ref = scipy.signal.correlate2d(x[0, 0], w[k, 0], mode="valid")
        assert _rel(y[0, k], ref) < 1e-12
    dy = g.uniform(-1, 1, y.shape)
    a = np.sum(dy * y)
    b = np.sum(oracle.conv2d_bwd_data(dy, w, (H, W)) * x)
    c = np.sum(oracle.conv2d_bwd_filter(x, dy, (R, S)) * w)
    assert abs(a - b) < 1e-9 and abs(a - c) < 1e-9


# ----------------------------------------------------------------------------- planted mistakes

def _mut_flip(w):
    return np.ascontiguousarray(w[:, :, ::-1, ::-1])


def _mut_rs_swap(w):
    K, C, R, S = w.shape
    return np.ascontiguousarray(w.reshape(K, C, S, R).swapaxes(2, 3))


def _mutant_set():
    f, d, b = ORACLE

    def fwd_flip(x, w, pad, st):
        return f(x, _mut_flip(w), pad, st)

    def fwd_rs(x, w, pad, st):
        return f(x, _mut_rs_swap(w), pad, st)

    def fwd_pad_off(x, w, pad, st):
        y = f(x, w, (pad[0] + 1, pad[1]), st)
        P = (x.shape[2] + 2 * pad[0] - w.shape[2]) // st[0] + 1
        return y[:, :, :P]

    def fwd_drop_c(x, w, pad, st):
        w2 = np.copy(w)
        w2[:, -1] = 0.0
        return f(x, w2, pad, st)

    def fwd_sign(x, w, pad, st):
        y = f(x, w, pad, st)
        y[..., -1] *= -1.0
        return y

    def bwd_data_flip(dy, w, hw, pad, st):
        return d(dy, _mut_flip(w), hw, pad, st)

    def bwd_data_kc(dy, w, hw, pad, st):
        K, C, R, S = w.shape
        w2 = np.ascontiguousarray(w.reshape(C, K, R, S).swapaxes(0, 1))
        return d(dy, w2, hw, pad, st)

    def bwd_data_no_stride(dy, w, hw, pad, st):
        out = d(dy, w, hw, pad, st)
        if st == (1, 1):
            out[..., 0, 0] += 1e-3
        else:
            out[..., 1::st[0], :] = 0.0
        return out

    def bwd_filter_rs(x, dy, RS, pad, st):
        return _mut_rs_swap(b(x, dy, RS, pad, st))

    def bwd_filter_flip(x, dy, RS, pad, st):
        return _mut_flip(b(x, dy, RS, pad, st))

    def bwd_filter_last_image(x, dy, RS, pad, st):
        return b(x[:-1] if x.shape[0] > 1 else 0.5 * x, dy[:-1] if x.shape[0] > 1 else dy, RS, pad, st)

    return {
        "fwd: convolution (flipped filter)": (fwd_flip, d, b),
        "fwd: swapped R/S strides": (fwd_rs, d, b),
        "fwd: padding off by one": (fwd_pad_off, d, b),
        "fwd: last channel dropped": (fwd_drop_c, d, b),
        "fwd: sign error in last column": (fwd_sign, d, b),
        "bwd_data: flipped filter": (f, bwd_data_flip, b),
        "bwd_data: K/C transposed": (f, bwd_data_kc, b),
        "bwd_data: wrong stride phase": (f, bwd_data_no_stride, b),
        "bwd_filter: R/S swapped": (f, d, bwd_filter_rs),
        "bwd_filter: flipped": (f, d, bwd_filter_flip),
        "bwd_filter: last image dropped": (f, d, bwd_filter_last_image),
    }


MUTANT_SHAPES = [SHAPES[1], SHAPES[3], SHAPES[8], (2, 3, 6, 6, 3, 3, 3, 1, 1, 2, 2)]


@pytest.mark.parametrize("name", sorted(_mutant_set()))
def test_pins_reject_planted_mistakes(name):
    f, d, b = _mutant_set()[name]
    caught = []
    for sh in MUTANT_SHAPES:
        caught.append(not pin_adjoint(f, d, b, sh))
        caught.append(not pin_torch(f, d, b, sh))
        caught.append(not pin_fwd_scipy(f, sh))
        caught.append(not pin_fwd_ones(f, sh))
        caught.append(not pin_zero_insertion(d, sh))
    assert any(caught), f"planted mistake '{name}' passed every pin"


def test_golden_tiny_oracle_outputs():
    """The oracle and the seeded generators still give the stored tiny-workload outputs."""
    from workloads import WORKLOADS, inputs
    with open(os.path.join(GOLDEN, "tiny_oracle.json")) as f:
        g = json.load(f)
    wl = WORKLOADS["tiny"]
    s = wl.shape
    assert list(s.args13()) == g["shape"]
    t = inputs(wl, "f32")
    x, w, dy = (t[k].numpy() for k in ("x", "w", "dy"))
    assert np.array_equal(oracle.conv2d_fwd(x, w, s.pad, s.stride).ravel(), np.array(g["y"]))
    assert np.array_equal(oracle.conv2d_bwd_data(dy, w, (s.H, s.W), s.pad, s.stride).ravel(),
                          np.array(g["dx"]))
    assert np.array_equal(oracle.conv2d_bwd_filter(x, dy, (s.R, s.S), s.pad, s.stride).ravel(),
                          np.array(g["dw"]))


# ----------------------------------------------------------------------------- compiled source mutants
# Each entry: (function the mistake is planted in, exact source text, replacement).  The text
# must occur inside that function of conv_oracle.c; the mutated copy is compiled with the
# oracle's own gcc flags and loaded in place of the real library, and at least one pin must
# reject it.  Every mutant keeps all memory accesses inside the arrays (indices stay bounded).
SOURCE_MUTANTS = {
    "fwd: filter rows flipped (convolution, not correlation)":
        ("oracle_conv2d_fwd", "int i = p * stride_h - pad_h + r;", "int i = p * stride_h - pad_h + (R - 1 - r);"),
    "fwd: padding off by one":
        ("oracle_conv2d_fwd", "int i = p * stride_h - pad_h + r;", "int i = p * stride_h - pad_h + r + 1;"),
    "fwd: last channel dropped":
        ("oracle_conv2d_fwd", "for (int c = 0; c < C; ++c) {", "for (int c = 0; c < C - 1; ++c) {"),
    "fwd: column uses the row stride":
        ("oracle_conv2d_fwd", "int j = q * stride_w - pad_w + s;", "int j = q * stride_h - pad_w + s;"),
    "fwd: output written transposed in p/q":
        ("oracle_conv2d_fwd", "y[(((size_t)n * K + k) * P + p) * Q + q] = acc;",
         "y[(((size_t)n * K + k) * P + (p * Q + q) % P) * Q + (p * Q + q) / P] = acc;"),
    "bwd_data: K and C of the filter exchanged":
        ("oracle_conv2d_bwd_data", "out[(size_t)i * W + j] += w[(((size_t)k * C + c) * R + r) * S + s] * g;",
         "out[(size_t)i * W + j] += w[(((size_t)c * K + k) * R + r) * S + s] * g;"),
    "bwd_data: filter rotated":
        ("oracle_conv2d_bwd_data", "out[(size_t)i * W + j] += w[(((size_t)k * C + c) * R + r) * S + s] * g;",
         "out[(size_t)i * W + j] += w[(((size_t)k * C + c) * R + (R - 1 - r)) * S + (S - 1 - s)] * g;"),
    "bwd_data: stride ignored":
        ("oracle_conv2d_bwd_data", "int i = p * stride_h - pad_h + r;", "int i = p - pad_h + r;"),
    "bwd_filter: last image dropped":
        ("oracle_conv2d_bwd_filter", "for (int n = 0; n < N; ++n) {", "for (int n = 0; n < N - (N > 1); ++n) {"),
    "bwd_filter: result stored with R flipped":
        ("oracle_conv2d_bwd_filter", "dw[(((size_t)k * C + c) * R + r) * S + s] = acc;",
         "dw[(((size_t)k * C + c) * R + (R - 1 - r)) * S + s] = acc;"),
    "bwd_filter: sign error on the last output column":
        ("oracle_conv2d_bwd_filter", "acc += dy[", "acc += (q == Q - 1 ? -1.0 : 1.0) * dy["),
    "bwd_filter: padding applied on the wrong side":
        ("oracle_conv2d_bwd_filter", "int j = q * stride_w - pad_w + s;", "int j = q * stride_w + pad_w + s;"),
}


def _mutated_source(func, old, new):
    with open(os.path.join(os.path.dirname(oracle.__file__), "conv_oracle.c")) as f:
        src = f.read()
    start = src.index("void " + func + "(")
    end = src.find("\nvoid ", start + 1)
    end = len(src) if end < 0 else end
    body = src[start:end]
    assert body.count(old) >= 1, (func, old)
    return src[:start] + body.replace(old, new, 1) + src[end:]


@pytest.mark.parametrize("name", sorted(SOURCE_MUTANTS))
def test_pins_reject_compiled_source_mutants(name, tmp_path):
    import subprocess
    func, old, new = SOURCE_MUTANTS[name]
    src = tmp_path / "mutant.c"
    src.write_text(_mutated_source(func, old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", str(src), "-o", str(lib)],
                   check=True)
    f, d, b = oracle.conv2d_fwd, oracle.conv2d_bwd_data, oracle.conv2d_bwd_filter
    caught = []
    with oracle.use_library(str(lib)):
        for sh in MUTANT_SHAPES:
            caught.append(not pin_adjoint(f, d, b, sh))
            caught.append(not pin_torch(f, d, b, sh))
            caught.append(not pin_fwd_scipy(f, sh))
            caught.append(not pin_fwd_ones(f, sh))
            caught.append(not pin_zero_insertion(d, sh))
    assert any(caught), f"planted mistake '{name}' passed every pin"
    # the real oracle is back in place and passes the same pins
    assert pin_adjoint(f, d, b, MUTANT_SHAPES[0]) and pin_torch(f, d, b, MUTANT_SHAPES[0])
