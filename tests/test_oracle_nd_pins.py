"""Pins for the generalised (N-D) oracle: 1 to 3 spatial dimensions, groups, dilation, separate
low / high padding.  Each pin ties it to something other than itself:

- torch's CPU float64 conv1d / conv2d / conv3d (groups, dilation, stride, symmetric padding) and
  their autograd gradients, a library implementation of the same operators; asymmetric padding
  through explicit zeros (torch.nn.functional.pad, then no padding);
- the 2-D oracle (a separate C implementation) on 2-D problems with one group, dilation 1 and
  symmetric padding;
- a grouped convolution equals the per-group convolutions of the channel slices, concatenated,
  each evaluated by the 2-D oracle;
- a dilated filter equals the filter with dilation - 1 zeros inserted between its taps, used
  with dilation 1 (the textbook identity);
- the adjoint identities <y, fwd(x, w)> = <bwd_data(y, w), x> = <bwd_filter(x, y), w>;
- the padding modes' closed forms.

Compiled copies of convnd_oracle.c with planted mistakes must each fail at least one pin.
"""
import os
import subprocess

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).uniform(-1.0, 1.0, shape)


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    m = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / m) if m > 0 else float(np.max(np.abs(a - b)))


# (N, C, K, groups, in, filt, pad_lo, pad_hi, stride, dilation)
ND_SHAPES = [
    (2, 3, 4, 1, (17,), (3,), (1,), (1,), (1,), (1,)),                          # 1-D
    (2, 4, 6, 2, (19,), (5,), (3,), (1,), (2,), (2,)),                          # 1-D grouped, dilated, asym
    (1, 6, 6, 6, (9, 10), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1)),              # depthwise
    (2, 4, 6, 2, (11, 9), (3, 2), (2, 0), (1, 1), (2, 1), (2, 3)),              # groups, dilation, asym
    (1, 3, 4, 1, (10, 12), (3, 3), (0, 2), (2, 0), (1, 2), (1, 1)),             # asym only
    (2, 2, 3, 1, (5, 6, 7), (3, 2, 3), (1, 0, 1), (1, 1, 1), (1, 2, 1), (1, 1, 2)),   # 3-D
    (1, 4, 4, 2, (6, 7, 5), (2, 3, 3), (0, 1, 2), (1, 1, 0), (2, 1, 1), (2, 1, 1)),   # 3-D grouped
    (1, 2, 2, 1, (4, 4, 4), (1, 1, 1), (0, 0, 0), (0, 0, 0), (2, 2, 2), (1, 1, 1)),   # 3-D 1x1x1 stride 2
]


def _unpack(sh):
    N, C, K, G, ins, filt, lo, hi, st, dil = sh
    outs = oracle.nd_out_size(ins, filt, lo, hi, st, dil)
    return N, C, K, G, ins, filt, lo, hi, st, dil, outs


_TORCH_CONV = {1: F.conv1d, 2: F.conv2d, 3: F.conv3d}


def pin_torch(fwd, bwd_data, bwd_filter, sh, seed=1):
    """Forward and both gradients against torch fp64 autograd; asymmetric padding as explicit
    zeros (F.pad, which takes the last dimension first), then no padding."""
    N, C, K, G, ins, filt, lo, hi, st, dil, outs = _unpack(sh)
    x, w, dy = _rand((N, C) + ins, seed), _rand((K, C // G) + filt, seed + 1), _rand((N, K) + outs, seed + 2)
    xt = torch.from_numpy(x).requires_grad_(True)
    wt = torch.from_numpy(w).requires_grad_(True)
    nd = len(ins)
    if tuple(lo) == tuple(hi):
        yt = _TORCH_CONV[nd](xt, wt, stride=st, padding=lo, dilation=dil, groups=G)
    else:
        padspec = []
        for d in reversed(range(nd)):
            padspec += [lo[d], hi[d]]
        yt = _TORCH_CONV[nd](F.pad(xt, padspec), wt, stride=st, padding=0, dilation=dil, groups=G)
    yt.backward(torch.from_numpy(dy))
    ok = _rel(fwd(x, w, G, lo, hi, st, dil), yt.detach().numpy()) < 1e-12
    ok &= _rel(bwd_data(dy, w, ins, G, lo, hi, st, dil), xt.grad.numpy()) < 1e-12
    ok &= _rel(bwd_filter(x, dy, filt, G, lo, hi, st, dil), wt.grad.numpy()) < 1e-12
    return bool(ok)


def pin_adjoint(fwd, bwd_data, bwd_filter, sh, seed=11):
    N, C, K, G, ins, filt, lo, hi, st, dil, outs = _unpack(sh)
    x, w, dy = _rand((N, C) + ins, seed), _rand((K, C // G) + filt, seed + 1), _rand((N, K) + outs, seed + 2)
    a = np.sum(dy * fwd(x, w, G, lo, hi, st, dil))
    b = np.sum(bwd_data(dy, w, ins, G, lo, hi, st, dil) * x)
    c = np.sum(bwd_filter(x, dy, filt, G, lo, hi, st, dil) * w)
    scale = max(1.0, abs(a))
    return abs(a - b) < 1e-11 * scale and abs(a - c) < 1e-11 * scale


def pin_dilation(fwd, sh, seed=21):
    """fwd with dilation == fwd of the zero-inserted filter with dilation 1."""
    N, C, K, G, ins, filt, lo, hi, st, dil, outs = _unpack(sh)
    x, w = _rand((N, C) + ins, seed), _rand((K, C // G) + filt, seed + 1)
    big = tuple(d * (f - 1) + 1 for f, d in zip(filt, dil))
    wd = np.zeros((K, C // G) + big)
    wd[(slice(None), slice(None)) + tuple(slice(None, None, d) for d in dil)] = w
    ones = (1,) * len(ins)
    return _rel(fwd(x, w, G, lo, hi, st, dil), fwd(x, wd, G, lo, hi, st, ones)) < 1e-13


def pin_groups_and_2d(fwd, bwd_data, bwd_filter, sh, seed=31):
    """2-D problems with dilation 1 and symmetric padding: each group's slice against the 2-D
    oracle, concatenated."""
    N, C, K, G, ins, filt, lo, hi, st, dil, outs = _unpack(sh)
    if len(ins) != 2 or tuple(lo) != tuple(hi) or any(d != 1 for d in dil):
        return True
    x, w, dy = _rand((N, C) + ins, seed), _rand((K, C // G) + filt, seed + 1), _rand((N, K) + outs, seed + 2)
    Cg, Kg = C // G, K // G
    y = fwd(x, w, G, lo, hi, st, dil)
    dx = bwd_data(dy, w, ins, G, lo, hi, st, dil)
    dw = bwd_filter(x, dy, filt, G, lo, hi, st, dil)
    ok = True
    for g in range(G):
        xs, ws, dys = x[:, g * Cg:(g + 1) * Cg], w[g * Kg:(g + 1) * Kg], dy[:, g * Kg:(g + 1) * Kg]
        ok &= _rel(y[:, g * Kg:(g + 1) * Kg], oracle.conv2d_fwd(xs, ws, tuple(lo), tuple(st))) < 1e-13
        ok &= _rel(dx[:, g * Cg:(g + 1) * Cg], oracle.conv2d_bwd_data(dys, ws, ins, tuple(lo), tuple(st))) < 1e-13
        ok &= _rel(dw[g * Kg:(g + 1) * Kg], oracle.conv2d_bwd_filter(xs, dys, filt, tuple(lo), tuple(st))) < 1e-13
    return bool(ok)


def _oracle_fns():
    f = lambda x, w, G, lo, hi, st, dil: oracle.convnd_fwd(x, w, G, lo, hi, st, dil)
    d = lambda dy, w, ins, G, lo, hi, st, dil: oracle.convnd_bwd_data(dy, w, ins, G, lo, hi, st, dil)
    b = lambda x, dy, filt, G, lo, hi, st, dil: oracle.convnd_bwd_filter(x, dy, filt, G, lo, hi, st, dil)
    return f, d, b


@pytest.mark.parametrize("sh", ND_SHAPES)
def test_nd_oracle_matches_torch(sh):
    assert pin_torch(*_oracle_fns(), sh)


@pytest.mark.parametrize("sh", ND_SHAPES)
def test_nd_adjoint_identities(sh):
    assert pin_adjoint(*_oracle_fns(), sh)


@pytest.mark.parametrize("sh", ND_SHAPES)
def test_nd_dilation_is_zero_inserted_filter(sh):
    assert pin_dilation(_oracle_fns()[0], sh)


@pytest.mark.parametrize("sh", [s for s in ND_SHAPES if len(s[4]) == 2] +
                         [(2, 6, 4, 2, (8, 9), (3, 3), (1, 1), (1, 1), (2, 1), (1, 1)),
                          (1, 4, 8, 4, (7, 7), (1, 3), (0, 1), (0, 1), (1, 1), (1, 1))])
def test_nd_groups_against_2d_oracle(sh):
    assert pin_groups_and_2d(*_oracle_fns(), sh)


def test_nd_plain_2d_equals_2d_oracle():
    x, w, dy = _rand((2, 3, 9, 8), 41), _rand((5, 3, 3, 3), 42), _rand((2, 5, 5, 4), 43)
    assert _rel(oracle.convnd_fwd(x, w, 1, (1, 1), (1, 1), (2, 2)), oracle.conv2d_fwd(x, w, (1, 1), (2, 2))) < 1e-14
    assert _rel(oracle.convnd_bwd_data(dy, w, (9, 8), 1, (1, 1), (1, 1), (2, 2)),
                oracle.conv2d_bwd_data(dy, w, (9, 8), (1, 1), (2, 2))) < 1e-14
    assert _rel(oracle.convnd_bwd_filter(x, dy, (3, 3), 1, (1, 1), (1, 1), (2, 2)),
                oracle.conv2d_bwd_filter(x, dy, (3, 3), (1, 1), (2, 2))) < 1e-14


def test_padding_modes():
    """valid: no padding.  same: output ceil(in / stride); stride 1 and an odd dilated filter
    extent pad equally on both sides; the high side never gets less than the low side."""
    assert oracle.padding_for("valid", (10, 7), (3, 3), (1, 2), (1, 1)) == ((0, 0), (0, 0))
    for i in range(1, 20):
        for f in range(1, 8):
            for s in (1, 2, 3):
                for d in (1, 2):
                    lo, hi = oracle.padding_for("same", (i,), (f,), (s,), (d,))
                    assert oracle.nd_out_size((i,), (f,), lo, hi, (s,), (d,)) == (-(-i // s),)
                    assert 0 <= lo[0] <= hi[0] <= lo[0] + 1
                    if s == 1 and (d * (f - 1)) % 2 == 0:
                        assert lo[0] == hi[0] == d * (f - 1) // 2
    with pytest.raises(ValueError):
        oracle.padding_for("full", (4,), (3,), (1,), (1,))


# ----------------------------------------------------------------------------- compiled source mutants
# (function, exact source text inside it, replacement); every mutant keeps its accesses in bounds.
ND_MUTANTS = {
    "fwd: width dilation ignored":
        ("oracle_convnd_fwd", "int l = ow * z[ZSW] - z[ZPW] + s * z[ZDW];", "int l = ow * z[ZSW] - z[ZPW] + s;"),
    "fwd: dilation used as the stride":
        ("oracle_convnd_fwd", "int j = oh * z[ZSH] - z[ZPH] + r * z[ZDH];", "int j = oh * z[ZDH] - z[ZPH] + r * z[ZSH];"),
    "fwd: group channel offset dropped":
        ("oracle_convnd_fwd", "x[((((size_t)n * C + g * Cg + c) * D + i)", "x[((((size_t)n * C + c) * D + i)"),
    "fwd: depth padding ignored":
        ("oracle_convnd_fwd", "int i = od * z[ZSD] - z[ZPD] + t * z[ZDD];", "int i = od * z[ZSD] + t * z[ZDD];"),
    "fwd: height and width taps exchanged in the filter":
        ("oracle_convnd_fwd", "w[((((size_t)k * Cg + c) * T + t) * R + r) * S + s] *",
         "w[((((size_t)k * Cg + c) * T + t) * R + (r * S + s) % R) * S + (r * S + s) / R] *"),
    "bwd_data: wrong group of filters":
        ("oracle_convnd_bwd_data", "for (int k = g * Kg; k < (g + 1) * Kg; ++k)", "for (int k = 0; k < Kg; ++k)"),
    "bwd_data: dilation ignored in height":
        ("oracle_convnd_bwd_data", "int j = oh * z[ZSH] - z[ZPH] + r * z[ZDH];", "int j = oh * z[ZSH] - z[ZPH] + r;"),
    "bwd_data: filter flipped in width":
        ("oracle_convnd_bwd_data", "w[((((size_t)k * Cg + c) * T + t) * R + r) * S + s] * gr;",
         "w[((((size_t)k * Cg + c) * T + t) * R + r) * S + (S - 1 - s)] * gr;"),
    "bwd_filter: group channel offset dropped":
        ("oracle_convnd_bwd_filter", "x[((((size_t)n * C + g * Cg + c) * D + i)", "x[((((size_t)n * C + c) * D + i)"),
    "bwd_filter: depth stride ignored":
        ("oracle_convnd_bwd_filter", "int i = od * z[ZSD] - z[ZPD] + t * z[ZDD];", "int i = od - z[ZPD] + t * z[ZDD];"),
    "bwd_filter: last image dropped":
        ("oracle_convnd_bwd_filter", "for (int n = 0; n < N; ++n)", "for (int n = 0; n < N - (N > 1); ++n)"),
}

MUTANT_SHAPES = [ND_SHAPES[1], ND_SHAPES[3], ND_SHAPES[5], ND_SHAPES[6],
                 (2, 4, 4, 2, (7, 8), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1))]


def _mutated_source(func, old, new):
    with open(os.path.join(os.path.dirname(oracle.__file__), "convnd_oracle.c")) as f:
        src = f.read()
    start = src.index("void " + func + "(")
    end = src.find("\nvoid ", start + 1)
    end = len(src) if end < 0 else end
    body = src[start:end]
    assert body.count(old) >= 1, (func, old)
    return src[:start] + body.replace(old, new, 1) + src[end:]


@pytest.mark.parametrize("name", sorted(ND_MUTANTS))
def test_nd_pins_reject_compiled_source_mutants(name, tmp_path):
    func, old, new = ND_MUTANTS[name]
    src = tmp_path / "mutant.c"
    src.write_text(_mutated_source(func, old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", str(src), "-o", str(lib)], check=True)
    f, d, b = _oracle_fns()
    caught = []
    with oracle.use_nd_library(str(lib)):
        for sh in MUTANT_SHAPES:
            caught.append(not pin_torch(f, d, b, sh))
            caught.append(not pin_adjoint(f, d, b, sh))
            caught.append(not pin_dilation(f, sh))
            caught.append(not pin_groups_and_2d(f, d, b, sh))
    assert any(caught), f"planted mistake '{name}' passed every pin"
    assert pin_torch(f, d, b, MUTANT_SHAPES[0]) and pin_adjoint(f, d, b, MUTANT_SHAPES[0])
