"""CPU oracle for 2-D NCHW/KCRS convolution: forward, backward-data,
backward-filter, and deconvolution forward and its two backward passes, in fp64.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library and
its Python binding never import it, and this package imports nothing from
them.

The arithmetic lives in ``conv_oracle.c`` (plain direct loops in double
precision, one function per pass); this module only marshals numpy arrays to
it.  The definitions follow:

- cross-correlation, dilation 1, symmetric zero padding, per-dimension stride:
  SystemDS "LibMatrixCuDNNConvolutionAlgorithm.java", allocateConvolutionDescriptor;
- NCHW input, NKPQ output, KCRS filter: same page, private constructor and the
  descriptor helpers; P and Q are caller-supplied sizes there;
- forward / backward-filter / backward-data with overwrite semantics: same
  page's three factory methods, and the FilterDescriptor.SetFilter4dDescriptor
  examples page (Conv2D, Conv2DKernelsGradient: alpha 1, beta 0);
- deconvolution forward = backward-data with the weight read as
  (in, out, h, w), and deconvolution backward-data = forward with the same
  reading: MXNet "mkldnn_deconvolution.cc", MKLDNNDeconvFwd::Execute;
  deconvolution backward-weights (MKLDNNDeconvBwd::ScheduleBwdWeights) is the
  adjoint in w, i.e. backward-filter with the two activations' roles swapped;
- the fused forward epilogue y = act(alpha * conv(x, W) + beta * y_prev + bias[k]):
  the alpha/beta scaling of the cuDNN calls on the SystemDS and C# pages, the
  per-output-channel bias tensor (1 x K x 1 x 1) and ReLU activation of the C#
  page's ConvolutionalLayer, the optional bias of the MXNet deconvolution;
- the same output epilogue on the backward passes (alpha/beta of the C# page's
  ConvolutionBackwardData / ConvolutionBackwardFilter calls; beta 0 or 1 is the
  write or add-to request that MXNet's MKLDNNDeconvBwd::ScheduleBwdData /
  ScheduleBwdWeights honour) and on the deconvolution forward with its bias;
- the bias gradient db[k] = sum over n, p, q of dy[n, k, p, q]: the derivative of
  sum(y * dy) in a bias added to every output of channel k (MXNet
  ScheduleBwdWeights, diff_bias).  Written in numpy as that sum;
- the generalised convolution (``convnd_*``, arithmetic in ``convnd_oracle.c``):
  1 to 3 spatial dimensions (MXNet SupportMKLDNNDeconv admits 1-3), groups
  (MXNet num_group), dilation (MXNet DeconvDescCreator's dilates) and separate
  low / high zero padding per dimension; "same" and "valid" padding modes (the
  C# page's Tensor.GetPaddingParams / PaddingType, whose definition the page
  does not give) are read as: valid = no padding; same = output size
  ceil(in / stride), total padding max((out - 1) * stride + dil * (f - 1) + 1 - in, 0)
  split with the smaller half low.

Inputs of any float dtype are widened to float64 exactly (fp32 and bf16 values
are exactly representable), so the oracle sees the same values as the GPU.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libconv_oracle.so")
_ND_LIB_PATH = os.path.join(_HERE, "libconvnd_oracle.so")
_lib = None
_nd_lib = None

_I = ctypes.c_int
_DP = ctypes.POINTER(ctypes.c_double)
_LP = ctypes.POINTER(ctypes.c_int64)


def _configure(lib):
    """Declares the C signatures on a loaded copy of the oracle library."""
    for name in ("oracle_conv2d_fwd", "oracle_conv2d_bwd_data", "oracle_conv2d_bwd_filter"):
        fn = getattr(lib, name)
        fn.argtypes = [_DP, _DP, _DP] + [_I] * 13
        fn.restype = None
    for name in ("oracle_deconv2d_fwd", "oracle_deconv2d_bwd_data", "oracle_deconv2d_bwd_filter"):
        fn = getattr(lib, name)
        fn.argtypes = [_DP, _DP, _DP] + [_I] * 13
        fn.restype = None
    for name in ("oracle_conv2d_fwd_points", "oracle_conv2d_bwd_data_points",
                 "oracle_conv2d_bwd_filter_points"):
        fn = getattr(lib, name)
        fn.argtypes = [_DP, _DP, _LP, _I, _DP] + [_I] * 13
        fn.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = _I
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build_oracle
        build_oracle.build()
    _lib = _configure(ctypes.CDLL(_LIB_PATH))
    return _lib


class use_library:
    """Context manager: the module's functions call the oracle built at ``path`` (a copy of
    ``conv_oracle.c`` with a planted mistake, in the pin tests) instead of the real one."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = _configure(ctypes.CDLL(self.path))
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def num_threads() -> int:
    """Threads the oracle's OpenMP regions use."""
    return int(_load().oracle_num_threads())


def out_size(H, W, R, S, pad, stride):
    """P = floor((H + 2 pad_h - R) / stride_h) + 1, Q likewise (floor reading)."""
    ph, pw = pad
    sh, sw = stride
    return (H + 2 * ph - R) // sh + 1, (W + 2 * pw - S) // sw + 1


def _f64(a):
    a = np.asarray(a)
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(_DP)


def _dims(N, C, H, W, K, R, S, pad, stride):
    P, Q = out_size(H, W, R, S, pad, stride)
    if P < 1 or Q < 1:
        raise ValueError("filter larger than the padded input")
    return (N, C, H, W, K, R, S, pad[0], pad[1], stride[0], stride[1], P, Q)


def conv2d_fwd(x, w, pad=(0, 0), stride=(1, 1)):
    """y = conv2d(x, w): x [N,C,H,W], w [K,C,R,S] -> y [N,K,P,Q] (float64)."""
    x, w = _f64(x), _f64(w)
    N, C, H, W = x.shape
    K, C2, R, S = w.shape
    assert C2 == C
    d = _dims(N, C, H, W, K, R, S, pad, stride)
    y = np.empty((N, K, d[11], d[12]), np.float64)
    _load().oracle_conv2d_fwd(_ptr(x), _ptr(w), _ptr(y), *d)
    return y


def conv2d_bwd_data(dy, w, in_hw, pad=(0, 0), stride=(1, 1)):
    """dx = adjoint of conv2d_fwd in x: dy [N,K,P,Q], w [K,C,R,S] -> dx [N,C,H,W]."""
    dy, w = _f64(dy), _f64(w)
    N, K, P, Q = dy.shape
    K2, C, R, S = w.shape
    assert K2 == K
    H, W = in_hw
    d = _dims(N, C, H, W, K, R, S, pad, stride)
    if (d[11], d[12]) != (P, Q):
        raise ValueError("dy spatial size does not match the forward output size")
    dx = np.empty((N, C, H, W), np.float64)
    _load().oracle_conv2d_bwd_data(_ptr(dy), _ptr(w), _ptr(dx), *d)
    return dx


def conv2d_bwd_filter(x, dy, RS, pad=(0, 0), stride=(1, 1)):
    """dW = adjoint of conv2d_fwd in w: x [N,C,H,W], dy [N,K,P,Q] -> dW [K,C,R,S]."""
    x, dy = _f64(x), _f64(dy)
    N, C, H, W = x.shape
    N2, K, P, Q = dy.shape
    assert N2 == N
    R, S = RS
    d = _dims(N, C, H, W, K, R, S, pad, stride)
    if (d[11], d[12]) != (P, Q):
        raise ValueError("dy spatial size does not match the forward output size")
    dw = np.empty((K, C, R, S), np.float64)
    _load().oracle_conv2d_bwd_filter(_ptr(x), _ptr(dy), _ptr(dw), *d)
    return dw


def deconv2d_fwd(x_in, w, out_hw, pad=(0, 0), stride=(1, 1)):
    """Transposed convolution: x_in [N,Cin,Hin,Win], w [Cin,Cout,R,S] -> [N,Cout,Hout,Wout]."""
    x_in, w = _f64(x_in), _f64(w)
    N, Cin, Hin, Win = x_in.shape
    Cin2, Cout, R, S = w.shape
    assert Cin2 == Cin
    Hout, Wout = out_hw
    P, Q = out_size(Hout, Wout, R, S, pad, stride)
    if (P, Q) != (Hin, Win):
        raise ValueError("output size inconsistent with the input size, pad and stride")
    out = np.empty((N, Cout, Hout, Wout), np.float64)
    _load().oracle_deconv2d_fwd(_ptr(x_in), _ptr(w), _ptr(out), N, Cin, Hin, Win, Cout, R, S,
                                pad[0], pad[1], stride[0], stride[1], Hout, Wout)
    return out


def _deconv_dims(x_in_shape, w_shape, out_hw, pad, stride):
    N, Cin, Hin, Win = x_in_shape
    Cin2, Cout, R, S = w_shape
    assert Cin2 == Cin
    Hout, Wout = out_hw
    if out_size(Hout, Wout, R, S, pad, stride) != (Hin, Win):
        raise ValueError("output size inconsistent with the input size, pad and stride")
    return (N, Cin, Hin, Win, Cout, R, S, pad[0], pad[1], stride[0], stride[1], Hout, Wout)


def deconv2d_bwd_data(dout, w, in_hw, pad=(0, 0), stride=(1, 1)):
    """Adjoint of deconv2d_fwd in its input: dout [N,Cout,Hout,Wout], w [Cin,Cout,R,S]
    -> din [N,Cin,Hin,Win]."""
    dout, w = _f64(dout), _f64(w)
    N, Cout, Hout, Wout = dout.shape
    Hin, Win = in_hw
    d = _deconv_dims((N, w.shape[0], Hin, Win), w.shape, (Hout, Wout), pad, stride)
    assert d[4] == Cout
    din = np.empty((N, d[1], Hin, Win), np.float64)
    _load().oracle_deconv2d_bwd_data(_ptr(dout), _ptr(w), _ptr(din), *d)
    return din


def deconv2d_bwd_filter(x_in, dout, RS, pad=(0, 0), stride=(1, 1)):
    """Adjoint of deconv2d_fwd in w: x_in [N,Cin,Hin,Win], dout [N,Cout,Hout,Wout]
    -> dw [Cin,Cout,R,S]."""
    x_in, dout = _f64(x_in), _f64(dout)
    N, Cin, Hin, Win = x_in.shape
    N2, Cout, Hout, Wout = dout.shape
    assert N2 == N
    d = _deconv_dims(x_in.shape, (Cin, Cout) + tuple(RS), (Hout, Wout), pad, stride)
    dw = np.empty((Cin, Cout) + tuple(RS), np.float64)
    _load().oracle_deconv2d_bwd_filter(_ptr(x_in), _ptr(dout), _ptr(dw), *d)
    return dw


def _points(fname, a, b, idx, d):
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int64))
    out = np.empty(idx.shape[0], np.float64)
    getattr(_load(), fname)(_ptr(a), _ptr(b), idx.ctypes.data_as(_LP), int(idx.shape[0]),
                            _ptr(out), *d)
    return out


def conv2d_fwd_points(x, w, idx, pad=(0, 0), stride=(1, 1)):
    """Forward output at flat indices ``idx`` into y [N,K,P,Q]."""
    x, w = _f64(x), _f64(w)
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    return _points("oracle_conv2d_fwd_points", x, w, idx, _dims(N, C, H, W, K, R, S, pad, stride))


def conv2d_bwd_data_points(dy, w, in_hw, idx, pad=(0, 0), stride=(1, 1)):
    """Backward-data output at flat indices ``idx`` into dx [N,C,H,W] (gather form)."""
    dy, w = _f64(dy), _f64(w)
    N, K, P, Q = dy.shape
    _, C, R, S = w.shape
    H, W = in_hw
    d = _dims(N, C, H, W, K, R, S, pad, stride)
    assert (d[11], d[12]) == (P, Q)
    return _points("oracle_conv2d_bwd_data_points", dy, w, idx, d)


def conv2d_bwd_filter_points(x, dy, RS, idx, pad=(0, 0), stride=(1, 1)):
    """Backward-filter output at flat indices ``idx`` into dW [K,C,R,S]."""
    x, dy = _f64(x), _f64(dy)
    N, C, H, W = x.shape
    _, K, P, Q = dy.shape
    R, S = RS
    d = _dims(N, C, H, W, K, R, S, pad, stride)
    assert (d[11], d[12]) == (P, Q)
    return _points("oracle_conv2d_bwd_filter_points", x, dy, idx, d)


def deconv2d_bwd_data_points(dout, w, in_hw, idx, pad=(0, 0), stride=(1, 1)):
    """deconv2d_bwd_data at flat indices ``idx`` into din [N,Cin,Hin,Win] (the forward
    convolution of dout with w read as KCRS, K = Cin)."""
    dout, w = _f64(dout), _f64(w)
    assert out_size(dout.shape[2], dout.shape[3], w.shape[2], w.shape[3], pad, stride) == tuple(in_hw)
    return conv2d_fwd_points(dout, w, idx, pad, stride)


def deconv2d_bwd_filter_points(x_in, dout, RS, idx, pad=(0, 0), stride=(1, 1)):
    """deconv2d_bwd_filter at flat indices ``idx`` into dw [Cin,Cout,R,S] (backward-filter
    with x := dout and dy := x_in)."""
    return conv2d_bwd_filter_points(dout, x_in, RS, idx, pad, stride)


def _epilogue(conv, k_index, bias, alpha, beta, y_prev, relu):
    """act(alpha * conv + beta * y_prev + bias[k]) elementwise in float64; y_prev is not
    read when beta == 0 (it may hold anything, NaN included)."""
    v = float(alpha) * conv
    if beta != 0.0:
        v = v + float(beta) * _f64(y_prev)
    if bias is not None:
        v = v + _f64(bias)[k_index]
    if relu:
        v = np.maximum(v, 0.0)
    return v


def conv2d_fwd_ex(x, w, pad=(0, 0), stride=(1, 1), bias=None, alpha=1.0, beta=0.0, y_prev=None,
                  relu=False):
    """Forward with the fused epilogue: y = act(alpha * conv2d(x, w) + beta * y_prev + bias[k]),
    act = max(0, .) when relu.  bias [K] or None; y_prev [N,K,P,Q] (read only if beta != 0)."""
    conv = conv2d_fwd(x, w, pad, stride)
    k = np.arange(conv.shape[1]).reshape(1, -1, 1, 1)
    return _epilogue(conv, k, bias, alpha, beta, y_prev, relu)


def conv2d_fwd_ex_points(x, w, idx, pad=(0, 0), stride=(1, 1), bias=None, alpha=1.0, beta=0.0,
                         y_prev=None, relu=False):
    """conv2d_fwd_ex at flat indices ``idx`` into y [N,K,P,Q]."""
    idx = np.asarray(idx, dtype=np.int64)
    conv = conv2d_fwd_points(x, w, idx, pad, stride)
    K = np.asarray(w).shape[0]
    N, C, H, W = np.asarray(x).shape
    P, Q = out_size(H, W, w.shape[2], w.shape[3], pad, stride)
    k = (idx // (P * Q)) % K
    yp = None if beta == 0.0 else _f64(y_prev).ravel()[idx]
    return _epilogue(conv, k, bias, alpha, beta, yp, relu)


def _channel_index(shape):
    return np.arange(shape[1]).reshape(1, -1, 1, 1)


def conv2d_bwd_data_ex(dy, w, in_hw, pad=(0, 0), stride=(1, 1), alpha=1.0, beta=0.0, dx_prev=None):
    """alpha * conv2d_bwd_data(dy, w) + beta * dx_prev (dx_prev read only if beta != 0)."""
    r = conv2d_bwd_data(dy, w, in_hw, pad, stride)
    return _epilogue(r, _channel_index(r.shape), None, alpha, beta, dx_prev, False)


def conv2d_bwd_filter_ex(x, dy, RS, pad=(0, 0), stride=(1, 1), alpha=1.0, beta=0.0, dw_prev=None):
    """alpha * conv2d_bwd_filter(x, dy) + beta * dw_prev (dw_prev read only if beta != 0)."""
    r = conv2d_bwd_filter(x, dy, RS, pad, stride)
    return _epilogue(r, 0, None, alpha, beta, dw_prev, False)


def deconv2d_fwd_ex(x_in, w, out_hw, pad=(0, 0), stride=(1, 1), bias=None, alpha=1.0, beta=0.0, y_prev=None,
                    relu=False):
    """act(alpha * deconv2d_fwd(x_in, w) + beta * y_prev + bias[c_out]); bias [C_out] or None."""
    r = deconv2d_fwd(x_in, w, out_hw, pad, stride)
    return _epilogue(r, _channel_index(r.shape), bias, alpha, beta, y_prev, relu)


def deconv2d_bwd_data_ex(dout, w, in_hw, pad=(0, 0), stride=(1, 1), alpha=1.0, beta=0.0, dx_prev=None):
    """alpha * deconv2d_bwd_data(dout, w) + beta * dx_prev."""
    r = deconv2d_bwd_data(dout, w, in_hw, pad, stride)
    return _epilogue(r, 0, None, alpha, beta, dx_prev, False)


def deconv2d_bwd_filter_ex(x_in, dout, RS, pad=(0, 0), stride=(1, 1), alpha=1.0, beta=0.0, dw_prev=None):
    """alpha * deconv2d_bwd_filter(x_in, dout) + beta * dw_prev."""
    r = deconv2d_bwd_filter(x_in, dout, RS, pad, stride)
    return _epilogue(r, 0, None, alpha, beta, dw_prev, False)


def conv2d_bwd_bias(dy, alpha=1.0, beta=0.0, db_prev=None):
    """db[k] = alpha * sum_{n,p,q} dy[n,k,p,q] + beta * db_prev[k] in float64 (db_prev read only
    if beta != 0).  For a deconvolution bias, dy is the deconvolution's output gradient."""
    r = _f64(dy).sum(axis=(0, 2, 3))
    return _epilogue(r, 0, None, alpha, beta, db_prev, False)


# ----------------------------------------------------------------------------- generalised (N-D)

def _load_nd():
    global _nd_lib
    if _nd_lib is not None:
        return _nd_lib
    if not os.path.exists(_ND_LIB_PATH):
        from . import build_oracle
        build_oracle.build()
    _nd_lib = _configure_nd(ctypes.CDLL(_ND_LIB_PATH))
    return _nd_lib


def _configure_nd(lib):
    for name in ("oracle_convnd_fwd", "oracle_convnd_bwd_data", "oracle_convnd_bwd_filter"):
        fn = getattr(lib, name)
        fn.argtypes = [_DP, _DP, _DP, ctypes.POINTER(_I)]
        fn.restype = None
    return lib


class use_nd_library:
    """Context manager: the convnd_* functions call the N-D oracle built at ``path`` (a copy of
    ``convnd_oracle.c`` with a planted mistake, in the pin tests) instead of the real one."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _nd_lib
        self.saved = _load_nd()
        _nd_lib = _configure_nd(ctypes.CDLL(self.path))
        return _nd_lib

    def __exit__(self, *exc):
        global _nd_lib
        _nd_lib = self.saved


def nd_out_size(in_sizes, filt, pad_lo, pad_hi, stride, dilation):
    """floor((in + lo + hi - dil * (f - 1) - 1) / stride) + 1 per dimension."""
    return tuple((i + lo + hi - d * (f - 1) - 1) // s + 1
                 for i, f, lo, hi, s, d in zip(in_sizes, filt, pad_lo, pad_hi, stride, dilation))


def padding_for(mode, in_sizes, filt, stride, dilation):
    """(pad_lo, pad_hi) of a padding mode: "valid" pads nothing; "same" gives output size
    ceil(in / stride) with total padding max((out - 1) * stride + dil * (f - 1) + 1 - in, 0),
    the smaller half low."""
    n = len(in_sizes)
    if mode == "valid":
        return (0,) * n, (0,) * n
    if mode != "same":
        raise ValueError(mode)
    lo, hi = [], []
    for i, f, s, d in zip(in_sizes, filt, stride, dilation):
        out = -(-i // s)
        tot = max((out - 1) * s + d * (f - 1) + 1 - i, 0)
        lo.append(tot // 2)
        hi.append(tot - tot // 2)
    return tuple(lo), tuple(hi)


def _nd_vec(N, C, K, groups, in_sizes, filt, out_sizes, pad_lo, stride, dilation):
    """The oracle's 22-int size vector, the problem lifted to three spatial dimensions."""
    nd = len(in_sizes)
    assert 1 <= nd <= 3 and len(filt) == nd and len(out_sizes) == nd
    lift = lambda v, one: (one,) * (3 - nd) + tuple(v)
    z = [N, C, K, groups] + list(lift(in_sizes, 1)) + list(lift(filt, 1)) + list(lift(out_sizes, 1)) + \
        list(lift(pad_lo, 0)) + list(lift(stride, 1)) + list(lift(dilation, 1))
    return (_I * 22)(*z)


def _nd_args(nd, groups, pad_lo, pad_hi, stride, dilation):
    pad_lo = tuple(pad_lo) if pad_lo is not None else (0,) * nd
    pad_hi = tuple(pad_hi) if pad_hi is not None else pad_lo
    stride = tuple(stride) if stride is not None else (1,) * nd
    dilation = tuple(dilation) if dilation is not None else (1,) * nd
    assert groups >= 1 and all(len(v) == nd for v in (pad_lo, pad_hi, stride, dilation))
    return pad_lo, pad_hi, stride, dilation


def convnd_fwd(x, w, groups=1, pad_lo=None, pad_hi=None, stride=None, dilation=None):
    """y[n,k,o] = sum_{c < C/G, taps} w[k,c,taps] * x~(n, g*C/G + c, o*stride - pad_lo + tap*dil),
    g = k // (K/G); x [N, C, *in], w [K, C/G, *filt] -> y [N, K, *out] (1 to 3 dims)."""
    x, w = _f64(x), _f64(w)
    N, C, *ins = x.shape
    K, Cg, *filt = w.shape
    nd = len(ins)
    pad_lo, pad_hi, stride, dilation = _nd_args(nd, groups, pad_lo, pad_hi, stride, dilation)
    assert C % groups == 0 and K % groups == 0 and Cg == C // groups
    outs = nd_out_size(ins, filt, pad_lo, pad_hi, stride, dilation)
    assert all(o >= 1 for o in outs)
    y = np.empty((N, K) + outs)
    _load_nd().oracle_convnd_fwd(_ptr(x), _ptr(w), _ptr(y),
                                 _nd_vec(N, C, K, groups, ins, filt, outs, pad_lo, stride, dilation))
    return y


def convnd_bwd_data(dy, w, in_sizes, groups=1, pad_lo=None, pad_hi=None, stride=None, dilation=None):
    """Adjoint of convnd_fwd in x applied to dy [N, K, *out] -> dx [N, C, *in]."""
    dy, w = _f64(dy), _f64(w)
    N, K, *outs = dy.shape
    _, Cg, *filt = w.shape
    nd = len(outs)
    pad_lo, pad_hi, stride, dilation = _nd_args(nd, groups, pad_lo, pad_hi, stride, dilation)
    C = Cg * groups
    assert tuple(outs) == nd_out_size(in_sizes, filt, pad_lo, pad_hi, stride, dilation)
    dx = np.empty((N, C) + tuple(in_sizes))
    _load_nd().oracle_convnd_bwd_data(_ptr(dy), _ptr(w), _ptr(dx),
                                      _nd_vec(N, C, K, groups, in_sizes, filt, outs, pad_lo, stride, dilation))
    return dx


def convnd_bwd_filter(x, dy, filt, groups=1, pad_lo=None, pad_hi=None, stride=None, dilation=None):
    """Adjoint of convnd_fwd in w applied to dy: x [N, C, *in], dy [N, K, *out] -> dw [K, C/G, *filt]."""
    x, dy = _f64(x), _f64(dy)
    N, C, *ins = x.shape
    _, K, *outs = dy.shape
    nd = len(ins)
    pad_lo, pad_hi, stride, dilation = _nd_args(nd, groups, pad_lo, pad_hi, stride, dilation)
    assert tuple(outs) == nd_out_size(ins, filt, pad_lo, pad_hi, stride, dilation)
    dw = np.empty((K, C // groups) + tuple(filt))
    _load_nd().oracle_convnd_bwd_filter(_ptr(x), _ptr(dy), _ptr(dw),
                                        _nd_vec(N, C, K, groups, ins, filt, outs, pad_lo, stride, dilation))
    return dw


def deconvnd_fwd(x_in, w, out_sizes, groups=1, pad_lo=None, pad_hi=None, stride=None, dilation=None):
    """Generalised deconvolution forward: convnd_bwd_data with the weight [C_in, C_out/G, *filt]
    read as the convolution filter (K = C_in), x_in [N, C_in, *in] -> [N, C_out, *out_sizes]."""
    return convnd_bwd_data(x_in, w, out_sizes, groups, pad_lo, pad_hi, stride, dilation)

