"""CPU tests of the C-ABI boundary (no GPU needed, no compute calls).

- the shared library loads and exports every function include/miconv.h declares;
- every validation error is returned before anything is enqueued (the calls use
  fake device addresses that are never dereferenced);
- workspace sizing and plan selection respect the caller's budget and the 1e9 cap;
- the host index helpers and plan invariants, built with g++ and sanitizers.
"""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "miconv.h")
LIB = os.path.join(ROOT, "convolution_implicit_gemm_nchw_amd", "libmiconv.so")
CSRC = os.path.join(ROOT, "convolution_implicit_gemm_nchw_amd", "csrc")

OK, E_NULL, E_DIM, E_OUT, E_DT, E_ALIAS, E_ALIGN, E_WS, E_HIP, E_PASS, E_BIG, E_INDEX = range(12)


def _ensure_lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()


@pytest.fixture(scope="module")
def lib():
    _ensure_lib()
    L = ctypes.CDLL(LIB)
    I, SZ, VP = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    for n in ("conv2d_fwd", "conv2d_bwd_data", "conv2d_bwd_filter", "deconv2d_fwd", "deconv2d_bwd_data",
              "deconv2d_bwd_filter"):
        getattr(L, n).argtypes = [I] * 14 + [VP, VP, VP, VP, SZ, VP]
        getattr(L, n).restype = I
    L.conv2d_fwd_ex.argtypes = [I] * 14 + [VP, VP, VP, ctypes.c_float, ctypes.c_float, I, I, VP, VP, SZ, VP]
    L.conv2d_fwd_ex.restype = I
    L.miconv_workspace_size.argtypes = [I] * 15 + [SZ, ctypes.POINTER(SZ)]
    L.miconv_plan_describe.argtypes = [I] * 15 + [SZ, ctypes.c_char_p, SZ]
    L.miconv_status_string.restype = ctypes.c_char_p
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^(?:const\s+char\s*\*|int)\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_passes():
    names = declared_functions()
    for n in ("conv2d_fwd", "conv2d_bwd_data", "conv2d_bwd_filter", "deconv2d_fwd",
              "deconv2d_bwd_data", "deconv2d_bwd_filter", "miconv_workspace_size", "miconv_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    for s in range(12):
        assert lib.miconv_status_string(s)
    assert lib.miconv_status_string(999) == b"unknown status"


# fake, 16-byte aligned, non-overlapping device addresses (never dereferenced)
X, WP, Y, WS = 0x10000000, 0x20000000, 0x30000000, 0x40000000
TINY = [2, 3, 8, 8, 4, 3, 3, 1, 1, 1, 1, 8, 8]


def _fwd(lib, dims=TINY, dtype=0, x=X, w=WP, y=Y, ws=None, wsb=0):
    return lib.conv2d_fwd(*dims, dtype, x, w, y, ws, wsb, None)


def test_validation_errors_forward(lib):
    assert _fwd(lib, dims=[0] + TINY[1:]) == E_DIM
    assert _fwd(lib, dims=TINY[:7] + [-1] + TINY[8:]) == E_DIM
    assert _fwd(lib, dims=TINY[:9] + [0] + TINY[10:]) == E_DIM
    assert _fwd(lib, dims=TINY[:5] + [20, 3] + TINY[7:]) == E_DIM          # filter > padded input
    assert _fwd(lib, dims=TINY[:11] + [7, 8]) == E_OUT                     # wrong P
    assert _fwd(lib, dims=TINY[:11] + [8, 9]) == E_OUT                     # wrong Q
    assert _fwd(lib, dtype=2) == E_DT
    assert _fwd(lib, x=None) == E_NULL
    assert _fwd(lib, y=None) == E_NULL
    assert _fwd(lib, ws=None, wsb=1024) == E_NULL
    assert _fwd(lib, x=X + 8) == E_ALIGN
    assert _fwd(lib, ws=WS + 4, wsb=1024) == E_ALIGN
    assert _fwd(lib, y=X) == E_ALIAS                                       # output on the input
    assert _fwd(lib, y=WP + 64) == E_ALIAS                                 # output over the filter
    assert _fwd(lib, y=WS, ws=WS, wsb=1 << 20) == E_ALIAS                  # output on the workspace
    big = [4096, 512, 1024, 1024, 4, 3, 3, 1, 1, 1, 1, 1024, 1024]
    assert _fwd(lib, dims=big) == E_BIG


def test_validation_errors_other_passes(lib):
    a = TINY
    assert lib.conv2d_bwd_data(*a, 0, X, WP, X, None, 0, None) == E_ALIAS   # dx on dy
    assert lib.conv2d_bwd_data(*a[:11], 9, 8, 0, X, WP, Y, None, 0, None) == E_OUT
    assert lib.conv2d_bwd_filter(*a, 1, X, WP, WP, None, 0, None) == E_ALIAS  # dW on dy
    assert lib.conv2d_bwd_filter(*a, 1, None, WP, Y, None, 0, None) == E_NULL
    # deconvolution: (N, C_in, H_in, W_in, C_out, R, S, pads, strides, H_out, W_out)
    d = [32, 256, 16, 16, 128, 4, 4, 1, 1, 2, 2, 32, 32]
    assert lib.deconv2d_fwd(*d[:11], 31, 32, 0, X, WP, Y, None, 0, None) == E_OUT
    assert lib.deconv2d_fwd(*d[:11], 30, 32, 0, X, WP, Y, None, 0, None) == E_OUT
    assert lib.deconv2d_fwd(*d, 0, X, WP, X, None, 0, None) == E_ALIAS
    for fn in (lib.deconv2d_bwd_data, lib.deconv2d_bwd_filter):
        assert fn(*d[:11], 31, 32, 0, X, WP, Y, None, 0, None) == E_OUT
        assert fn(*d, 0, X, WP, WP, None, 0, None) == E_ALIAS
        assert fn(*d, 0, None, WP, Y, None, 0, None) == E_NULL
        assert fn(*d, 2, X, WP, Y, None, 0, None) == E_DT
        assert fn(*d, 0, X + 8, WP, Y, None, 0, None) == E_ALIGN


def test_validation_errors_fused_forward(lib):
    ex = lib.conv2d_fwd_ex
    B = 0x50000000   # fake bias address
    assert ex(*TINY, 0, X, WP, B + 2, 1.0, 0.0, 0, 0, Y, None, 0, None) == E_ALIGN      # bias not 4-byte aligned
    assert ex(*TINY, 0, X, WP, Y + 16, 1.0, 0.0, 1, 0, Y, None, 0, None) == E_ALIAS     # bias inside y
    assert ex(*TINY, 0, None, WP, B, 0.5, 1.0, 1, 0, Y, None, 0, None) == E_NULL
    assert ex(*TINY[:11], 9, 8, 0, X, WP, B, 0.5, 1.0, 1, 0, Y, None, 0, None) == E_OUT
    assert ex(*TINY, 3, X, WP, B, 0.5, 1.0, 1, 0, Y, None, 0, None) == E_DT
    assert ex(*TINY, 0, X, WP, B, 0.5, 1.0, 1, 2, Y, None, 0, None) == E_DT             # output dtype
    assert ex(*TINY, 0, X, WP, B, 0.5, 1.0, 1, 0, X, None, 0, None) == E_ALIAS          # y on x


def test_validation_errors_backward_epilogues(lib):
    I, F, VP, SZ = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    for n in ("conv2d_bwd_data_ex", "conv2d_bwd_filter_ex", "deconv2d_bwd_data_ex", "deconv2d_bwd_filter_ex"):
        getattr(lib, n).argtypes = [I] * 14 + [VP, VP, F, F, I, VP, VP, SZ, VP]
    lib.deconv2d_fwd_ex.argtypes = [I] * 14 + [VP, VP, VP, F, F, I, I, VP, VP, SZ, VP]
    lib.conv2d_bwd_bias.argtypes = [I] * 5 + [VP, F, F, VP, VP]
    a = TINY
    bd, bf = lib.conv2d_bwd_data_ex, lib.conv2d_bwd_filter_ex
    assert bd(*a, 0, X, WP, 1.0, 1.0, 2, Y, None, 0, None) == E_DT               # output dtype
    assert bd(*a, 0, X, WP, 1.0, 1.0, 1, X, None, 0, None) == E_ALIAS            # dx on dy
    assert bd(*a[:11], 9, 8, 0, X, WP, 1.0, 1.0, 0, Y, None, 0, None) == E_OUT
    assert bd(*a, 0, X, WP, 1.0, 1.0, 0, None, None, 0, None) == E_NULL
    # dW [4][3][3][3] is 432 bytes in fp32 and 216 in bf16: both run into dy here
    assert bf(*a, 0, X, WP, 0.5, 0.0, 0, WP - 416, None, 0, None) == E_ALIAS
    assert bf(*a, 0, X, WP, 0.5, 0.0, 1, WP - 208, None, 0, None) == E_ALIAS
    assert bf(*a, 0, X + 8, WP, 0.5, 0.0, 1, Y, None, 0, None) == E_ALIGN
    d = [32, 256, 16, 16, 128, 4, 4, 1, 1, 2, 2, 32, 32]
    B = 0x50000000
    ex = lib.deconv2d_fwd_ex
    assert ex(*d, 0, X, WP, B + 2, 1.0, 0.0, 0, 0, Y, None, 0, None) == E_ALIGN          # bias alignment
    assert ex(*d, 0, X, WP, Y + 16, 1.0, 0.0, 0, 0, Y, None, 0, None) == E_ALIAS         # bias inside y
    assert ex(*d[:11], 31, 32, 0, X, WP, B, 1.0, 0.0, 0, 0, Y, None, 0, None) == E_OUT
    assert ex(*d, 0, X, WP, B, 1.0, 0.0, 0, 3, Y, None, 0, None) == E_DT
    for fn in (lib.deconv2d_bwd_data_ex, lib.deconv2d_bwd_filter_ex):
        assert fn(*d[:11], 31, 32, 0, X, WP, 1.0, 0.0, 0, Y, None, 0, None) == E_OUT
        assert fn(*d, 0, X, WP, 1.0, 0.0, 0, WP, None, 0, None) == E_ALIAS
        assert fn(*d, 0, X, WP, 1.0, 0.0, 5, Y, None, 0, None) == E_DT
    bb = lib.conv2d_bwd_bias
    assert bb(2, 4, 8, 8, 0, None, 1.0, 0.0, Y, None) == E_NULL
    assert bb(2, 4, 8, 8, 0, X, 1.0, 0.0, None, None) == E_NULL
    assert bb(0, 4, 8, 8, 0, X, 1.0, 0.0, Y, None) == E_DIM
    assert bb(2, 4, 8, -1, 0, X, 1.0, 0.0, Y, None) == E_DIM
    assert bb(2, 4, 8, 8, 2, X, 1.0, 0.0, Y, None) == E_DT
    assert bb(2, 4, 8, 8, 0, X + 4, 1.0, 0.0, Y, None) == E_ALIGN
    assert bb(2, 4, 8, 8, 0, X, 1.0, 0.0, Y + 2, None) == E_ALIGN
    assert bb(2, 4, 8, 8, 0, X, 1.0, 0.0, X + 64, None) == E_ALIAS
    assert bb(1 << 16, 1 << 10, 64, 64, 1, X, 1.0, 0.0, Y, None) == E_BIG


def test_build_rejects_kernels_with_scratch():
    """The build's resource-report reader flags any kernel with a nonzero scratch size."""
    from convolution_implicit_gemm_nchw_amd.build import scratch_kernels
    lines = [
        "a.hip:1:1: remark: Function Name: _Z3foov [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs: 40 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: _Z3barv [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 24 [-Rpass-analysis=kernel-resource-usage]",
        "warning: something else",
    ]
    assert scratch_kernels(lines) == [("_Z3barv", 24)]
    assert scratch_kernels(lines[:3]) == []


def test_deconv_passes_map_to_the_convolution_passes(lib):
    """Deconvolution forward / backward-data / backward-weights plan exactly as convolution
    backward-data / forward / backward-filter with K = C_in, C = C_out, H = H_out, P = H_in."""
    d = [32, 256, 16, 16, 128, 4, 4, 1, 1, 2, 2, 32, 32]
    conv = [32, 128, 32, 32, 256, 4, 4, 1, 1, 2, 2, 16, 16]
    for dtype in (0, 1):
        for dpass, cpass in ((3, 1), (4, 0), (5, 2)):
            a, b = ctypes.create_string_buffer(512), ctypes.create_string_buffer(512)
            assert lib.miconv_plan_describe(dpass, dtype, *d, 10 ** 9, a, 512) == OK
            assert lib.miconv_plan_describe(cpass, dtype, *conv, 10 ** 9, b, 512) == OK
            assert a.value == b.value


WORKLOAD_DIMS = {
    "resnet3x3": [64, 64, 56, 56, 64, 3, 3, 1, 1, 1, 1, 56, 56],
    "proj1x1": [64, 256, 56, 56, 512, 1, 1, 0, 0, 2, 2, 28, 28],
    "stem7x7": [32, 3, 224, 224, 64, 7, 7, 3, 3, 2, 2, 112, 112],
    "deep3x3": [256, 512, 14, 14, 512, 3, 3, 1, 1, 1, 1, 14, 14],
    "sentence": [1, 1, 2060, 300, 500, 5, 300, 0, 0, 1, 1, 2056, 1],
}


@pytest.mark.parametrize("name", sorted(WORKLOAD_DIMS))
@pytest.mark.parametrize("pass_id", [0, 1, 2])
@pytest.mark.parametrize("dtype", [0, 1])
def test_workspace_respects_budget(lib, name, pass_id, dtype):
    dims = WORKLOAD_DIMS[name]
    out = ctypes.c_size_t(0)
    for limit in (0, 4096, 1 << 20, 1 << 26, 10 ** 9, 1 << 40):
        assert lib.miconv_workspace_size(pass_id, dtype, *dims, limit, ctypes.byref(out)) == OK
        assert out.value <= min(limit, 10 ** 9)
    buf = ctypes.create_string_buffer(512)
    assert lib.miconv_plan_describe(pass_id, dtype, *dims, 0, buf, 512) == OK
    desc = buf.value.decode()
    assert "splits=1 " in desc and "ws=0" in desc
    if pass_id != 2 and not (pass_id == 0 and dims[5] * dims[6] == 1):
        assert "wt=0" in desc    # no budget: the filter is read in place


def test_tail_form_plans(lib):
    """bf16 stride-1 3x3 forward / backward-data with 128-row tiles of 193..208 pixels and 2-column
    fill loads take the 16-pixel tail form; 224-pixel tiles, 64-row tiles, fp32 and other filters
    do not."""
    def describe(pass_id, dtype, dims):
        buf = ctypes.create_string_buffer(512)
        assert lib.miconv_plan_describe(pass_id, dtype, *dims, 10 ** 9, buf, 512) == OK
        return buf.value.decode()

    deep = (256, 512, 14, 14, 512, 3, 3, 1, 1, 1, 1, 14, 14)
    for pass_id in (0, 1):
        assert "form=tail16" in describe(pass_id, 1, deep)
        assert "form=tail16" not in describe(pass_id, 0, deep)            # fp32: the generic kernel
    assert "form=tail16" in describe(0, 1, (1, 128, 20, 10, 160, 3, 3, 1, 1, 1, 1, 20, 10))    # 200 pixels
    assert "form=tail16" in describe(0, 1, (2, 64, 9, 22, 136, 3, 3, 1, 1, 1, 1, 9, 22))      # 198 pixels
    assert "form=tail16" in describe(1, 1, (2, 160, 11, 18, 96, 3, 3, 1, 1, 1, 1, 11, 18))    # 198 pixels
    assert "form=tail16" not in describe(0, 1, (2, 64, 56, 56, 128, 3, 3, 1, 1, 1, 1, 56, 56))  # 224 pixels
    assert "form=tail16" not in describe(0, 1, (2, 64, 14, 14, 64, 3, 3, 1, 1, 1, 1, 14, 14))   # 64 rows
    assert "form=tail16" not in describe(1, 1, (2, 64, 14, 14, 160, 3, 3, 1, 1, 1, 1, 14, 14))  # 64 rows
    assert "form=tail16" not in describe(0, 1, (2, 64, 14, 16, 160, 3, 3, 1, 1, 1, 1, 14, 16))  # 224 pixels
    assert "form=tail16" not in describe(0, 1, (2, 64, 14, 14, 160, 5, 5, 2, 2, 1, 1, 14, 14))  # 5x5


def test_few_channel_mfma_form_plans(lib):
    """fp32 backward-data with C <= 4, stride 2, 7 filter rows, C*S <= 32, Q <= 128 and K of 32 or 64
    takes the MFMA form of the few-channel kernel; the 7x7 stem (112 dx row pairs, 32 images) runs
    7 pairs per work-group, 512 work-groups (two per CU).  bf16, other K, strides or filters keep
    the vector form."""
    def describe(dtype, dims):
        buf = ctypes.create_string_buffer(512)
        assert lib.miconv_plan_describe(1, dtype, *dims, 10 ** 9, buf, 512) == OK
        return buf.value.decode()

    stem = (32, 3, 224, 224, 64, 7, 7, 3, 3, 2, 2, 112, 112)
    assert "algo=tinyc" in describe(0, stem) and "form=mfma pairs=7" in describe(0, stem)
    assert "algo=tinyc" in describe(1, stem) and "form=mfma" not in describe(1, stem)       # bf16
    assert "form=mfma" in describe(0, (2, 3, 40, 226, 32, 7, 7, 2, 2, 2, 2, 19, 112))        # K = 32
    assert "form=mfma" not in describe(0, (2, 3, 37, 70, 16, 7, 7, 3, 3, 2, 2, 19, 35))     # K = 16
    assert "form=mfma" not in describe(0, (2, 3, 37, 70, 48, 7, 7, 3, 3, 2, 2, 19, 35))     # K = 48
    assert "form=mfma" not in describe(0, (2, 3, 20, 20, 64, 5, 5, 2, 2, 2, 2, 10, 10))     # 5 rows
    assert "form=mfma" not in describe(0, (2, 3, 20, 20, 64, 7, 7, 3, 3, 1, 1, 20, 20))     # stride 1
    assert "form=mfma" not in describe(0, (2, 3, 20, 270, 64, 7, 7, 3, 3, 2, 2, 10, 135))   # Q > 128
    assert "form=mfma" not in describe(0, (2, 4, 20, 20, 64, 7, 9, 3, 4, 2, 2, 10, 10))     # C*S = 36


def test_few_channel_bwd_filter_plans(lib):
    """fp32 backward-filter with K = 64, C <= 4, 7 filter rows, column stride 2, C*R*S <= 160 and Q a
    multiple of 4 up to 112 takes the few-channel MFMA kernel: for the stem 3584 output rows, 7 per
    work-group (512 splits); with no workspace, or for bf16 and other shapes, it does not."""
    def describe(dtype, dims, budget=10 ** 9):
        buf = ctypes.create_string_buffer(512)
        assert lib.miconv_plan_describe(2, dtype, *dims, budget, buf, 512) == OK
        return buf.value.decode()

    stem = (32, 3, 224, 224, 64, 7, 7, 3, 3, 2, 2, 112, 112)
    d = describe(0, stem)
    assert "algo=tinyc" in d and "form=mfma rows=7" in d and "splits=512" in d, d
    assert "algo=tinyc" not in describe(0, stem, 0)                                          # no workspace
    assert "algo=tinyc" not in describe(1, stem)                                             # bf16
    assert "algo=tinyc" in describe(0, (1, 3, 7, 23, 64, 7, 7, 0, 3, 2, 2, 1, 12), 0)        # one row: direct
    assert "algo=tinyc" not in describe(0, (2, 3, 37, 70, 64, 7, 7, 3, 3, 2, 2, 19, 35))     # Q % 4 != 0
    assert "algo=tinyc" not in describe(0, (2, 3, 37, 71, 32, 7, 7, 3, 3, 2, 2, 19, 36))     # K = 32
    assert "algo=tinyc" not in describe(0, (2, 3, 40, 240, 64, 7, 7, 3, 3, 2, 2, 20, 120))   # Q > 112
    assert "algo=tinyc" not in describe(0, (2, 4, 30, 32, 64, 7, 7, 3, 3, 2, 2, 15, 16))     # 196 values


def test_few_channel_forward_plans(lib):
    """fp32 forward with K = 64, C <= 4, 7 filter rows (S >= 4), column stride 2, C*R*S <= 148 and
    Q <= 112 takes the few-channel MFMA kernel (the stem: 3584 output rows, 7 per work-group);
    bf16 and other shapes do not."""
    def describe(dtype, dims):
        buf = ctypes.create_string_buffer(512)
        assert lib.miconv_plan_describe(0, dtype, *dims, 10 ** 9, buf, 512) == OK
        return buf.value.decode()

    stem = (32, 3, 224, 224, 64, 7, 7, 3, 3, 2, 2, 112, 112)
    d = describe(0, stem)
    assert "algo=tinyc" in d and "form=mfma rows=7" in d, d
    assert "algo=tinyc" not in describe(1, stem)                                              # bf16
    assert "algo=tinyc" in describe(0, (2, 3, 37, 70, 64, 7, 7, 3, 3, 2, 2, 19, 35))          # Q = 35
    assert "algo=tinyc" not in describe(0, (2, 3, 37, 70, 32, 7, 7, 3, 3, 2, 2, 19, 35))      # K = 32
    assert "algo=tinyc" not in describe(0, (2, 1, 16, 16, 64, 7, 3, 3, 1, 2, 2, 8, 8))        # S = 3
    assert "algo=tinyc" not in describe(0, (2, 3, 40, 240, 64, 7, 7, 3, 3, 2, 2, 20, 120))    # Q > 112


def test_pointwise_bwd_filter_plans(lib):
    """bf16 1x1 backward-filter, pad 0, stride 2 (x of exactly 2 x the output size): the pointwise
    kernel, split-K to about one work-group per CU (8 tiles of 128 x 128 for 512 x 256), one split
    with no workspace; stride 1 keeps the patch kernel; fp32 and padded problems the generic one."""
    def describe(pass_id, dtype, dims, budget=10 ** 9):
        buf = ctypes.create_string_buffer(512)
        assert lib.miconv_plan_describe(pass_id, dtype, *dims, budget, buf, 512) == OK
        return buf.value.decode()

    proj = (64, 256, 56, 56, 512, 1, 1, 0, 0, 2, 2, 28, 28)
    d = describe(2, 1, proj)
    assert "algo=pointwise" in d and "grid=4x2x32" in d and "splits=32" in d, d
    assert "algo=pointwise" in describe(2, 1, proj, 0) and "splits=1" in describe(2, 1, proj, 0)
    assert "algo=pointwise" not in describe(2, 0, proj)                                          # fp32
    assert "algo=patch" in describe(2, 1, (2, 96, 8, 8, 200, 1, 1, 0, 0, 1, 1, 8, 8))           # stride 1
    assert "algo=pointwise" not in describe(2, 1, (2, 64, 14, 14, 128, 1, 1, 0, 0, 2, 2, 7, 7))   # Q % 4
    assert "algo=pointwise" not in describe(2, 1, (2, 64, 18, 18, 128, 1, 1, 1, 1, 2, 2, 10, 10)) # padding


def test_plan_candidates_select_and_cache(lib):
    """Candidate enumeration, installing a candidate (plan_describe and workspace_size then
    report it), the index range, removal and clearing.  Pure host calls."""
    I, SZ = ctypes.c_int, ctypes.c_size_t
    lib.miconv_plan_candidates.argtypes = [I] * 15 + [SZ, ctypes.POINTER(I), ctypes.POINTER(SZ)]
    lib.miconv_plan_select.argtypes = [I] * 15 + [SZ, I]
    lib.miconv_plan_cache_entries.argtypes = [ctypes.POINTER(I), ctypes.POINTER(I)]
    lib.miconv_plan_cache_clear()

    def describe(pass_id, dtype, dims, budget=10 ** 9):
        buf = ctypes.create_string_buffer(512)
        assert lib.miconv_plan_describe(pass_id, dtype, *dims, budget, buf, 512) == OK
        return buf.value.decode()

    n, mx = I(0), SZ(0)
    for name, dims in sorted(WORKLOAD_DIMS.items()):
        for pass_id in (0, 1, 2):
            for dtype in (0, 1):
                assert lib.miconv_plan_candidates(pass_id, dtype, *dims, 10 ** 9, ctypes.byref(n), ctypes.byref(mx)) == OK
                assert 1 <= n.value <= 16 and mx.value <= 10 ** 9
                default = describe(pass_id, dtype, dims)
                seen = set()
                for i in range(n.value):
                    assert lib.miconv_plan_select(pass_id, dtype, *dims, 10 ** 9, i) == OK
                    d = describe(pass_id, dtype, dims)
                    seen.add(d)
                    ws = ctypes.c_size_t(0)
                    assert lib.miconv_workspace_size(pass_id, dtype, *dims, 10 ** 9, ctypes.byref(ws)) == OK
                    assert d.endswith("ws=%d" % ws.value) and ws.value <= mx.value
                    if i == 0:
                        assert d == default
                    # a budget the installed plan does not fit falls back to the default for it
                    assert describe(pass_id, dtype, dims, 0).endswith("ws=0")
                assert len(seen) >= min(n.value, 2)
                assert lib.miconv_plan_select(pass_id, dtype, *dims, 10 ** 9, n.value) == E_INDEX
                assert lib.miconv_plan_select(pass_id, dtype, *dims, 10 ** 9, -1) == OK
                assert describe(pass_id, dtype, dims) == default
    tuned, total = I(-1), I(-1)
    assert lib.miconv_plan_cache_entries(ctypes.byref(tuned), ctypes.byref(total)) == OK
    assert tuned.value == 0 and total.value > 0
    assert lib.miconv_plan_cache_clear() == OK
    assert lib.miconv_plan_cache_entries(ctypes.byref(tuned), ctypes.byref(total)) == OK
    assert tuned.value == 0 and total.value == 0
    assert lib.miconv_plan_candidates(0, 0, *TINY, 0, None, None) == E_NULL
    assert lib.miconv_plan_select(0, 0, *TINY[:11], 7, 8, 0, 0) == E_OUT
    assert lib.miconv_status_string(11) == b"plan candidate index out of range"


class _NdDesc(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int), ("N", ctypes.c_int), ("C", ctypes.c_int), ("K", ctypes.c_int),
                ("groups", ctypes.c_int), ("in_", ctypes.c_int * 3), ("filter", ctypes.c_int * 3),
                ("out", ctypes.c_int * 3), ("pad_lo", ctypes.c_int * 3), ("pad_hi", ctypes.c_int * 3),
                ("stride", ctypes.c_int * 3), ("dilation", ctypes.c_int * 3)]


def _nd(ndim, N, C, K, G, ins, filt, lo, hi, st, dil):
    d = _NdDesc()
    d.ndim, d.N, d.C, d.K, d.groups = ndim, N, C, K, G
    for i in range(ndim):
        d.in_[i], d.filter[i], d.pad_lo[i], d.pad_hi[i] = ins[i], filt[i], lo[i], hi[i]
        d.stride[i], d.dilation[i] = st[i], dil[i]
        d.out[i] = (ins[i] + lo[i] + hi[i] - dil[i] * (filt[i] - 1) - 1) // st[i] + 1
    return d


def test_convnd_validation_and_routing(lib):
    """Generalised entry points: argument errors before any launch, plain 2-D / 1-D problems on
    the 2-D plans, the rest on the generic kernel, and the padding modes.  Pure host calls."""
    P = ctypes.POINTER(_NdDesc)
    for n in ("convnd_fwd", "convnd_bwd_data", "convnd_bwd_filter"):
        getattr(lib, n).argtypes = [P, ctypes.c_int] + [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p]
    lib.convnd_describe.argtypes = [ctypes.c_int, P, ctypes.c_int, ctypes.c_size_t, ctypes.c_char_p, ctypes.c_size_t]
    lib.convnd_workspace_size.argtypes = [ctypes.c_int, P, ctypes.c_int, ctypes.c_size_t,
                                          ctypes.POINTER(ctypes.c_size_t)]
    lib.miconv_nd_padding.argtypes = [P, ctypes.c_int]

    def describe(pass_id, d, ws=10 ** 9):
        buf = ctypes.create_string_buffer(512)
        assert lib.convnd_describe(pass_id, ctypes.byref(d), 1, ws, buf, 512) == OK
        return buf.value.decode()

    g = _nd(2, 2, 8, 12, 4, (9, 10), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1))
    for fn in (lib.convnd_fwd, lib.convnd_bwd_data, lib.convnd_bwd_filter):
        assert fn(None, 0, X, WP, Y, None, 0, None) == E_NULL
        assert fn(ctypes.byref(g), 2, X, WP, Y, None, 0, None) == E_DT
        assert fn(ctypes.byref(g), 0, None, WP, Y, None, 0, None) == E_NULL
        assert fn(ctypes.byref(g), 0, X + 4, WP, Y, None, 0, None) == E_ALIGN
        assert fn(ctypes.byref(g), 0, X, WP, X, None, 0, None) == E_ALIAS
    bad = _nd(2, 2, 8, 12, 3, (9, 10), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1))    # 8 % 3 != 0
    assert lib.convnd_fwd(ctypes.byref(bad), 0, X, WP, Y, None, 0, None) == E_DIM
    bad = _nd(2, 2, 8, 12, 4, (9, 10), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1))
    bad.out[1] += 1
    assert lib.convnd_fwd(ctypes.byref(bad), 0, X, WP, Y, None, 0, None) == E_OUT
    bad = _nd(2, 2, 8, 12, 4, (9, 10), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1))
    bad.ndim = 4
    assert lib.convnd_fwd(ctypes.byref(bad), 0, X, WP, Y, None, 0, None) == E_DIM
    bad = _nd(1, 2, 8, 12, 1, (9,), (3,), (1,), (1,), (1,), (0,))
    assert lib.convnd_fwd(ctypes.byref(bad), 0, X, WP, Y, None, 0, None) == E_DIM
    # routing: groups, dilation, asymmetric padding or depth -> generic; plain 2-D and 1-D -> 2-D plans
    assert "algo=generic groups=4" in describe(0, g)
    assert "algo=generic" in describe(1, _nd(2, 2, 8, 12, 1, (9, 10), (3, 3), (1, 1), (1, 1), (1, 1), (2, 1)))
    assert "algo=generic" in describe(2, _nd(2, 2, 8, 12, 1, (9, 10), (3, 3), (1, 0), (1, 1), (1, 1), (1, 1)))
    assert "algo=generic" in describe(0, _nd(3, 2, 8, 12, 1, (3, 9, 10), (2, 3, 3), (0, 1, 1), (0, 1, 1),
                                             (1, 1, 1), (1, 1, 1)))
    plain = _nd(2, 2, 64, 64, 1, (14, 14), (3, 3), (1, 1), (1, 1), (1, 1), (1, 1))
    buf = ctypes.create_string_buffer(512)
    assert lib.miconv_plan_describe(0, 1, 2, 64, 14, 14, 64, 3, 3, 1, 1, 1, 1, 14, 14, 10 ** 9, buf, 512) == OK
    assert describe(0, plain) == buf.value.decode()
    one = _nd(1, 1, 300, 500, 1, (2060,), (5,), (0,), (0,), (1,), (1,))
    assert lib.miconv_plan_describe(0, 1, 1, 300, 1, 2060, 500, 1, 5, 0, 0, 1, 1, 1, 2056, 10 ** 9, buf, 512) == OK
    assert describe(0, one) == buf.value.decode()
    ws = ctypes.c_size_t(0)
    assert lib.convnd_workspace_size(2, ctypes.byref(g), 1, 0, ctypes.byref(ws)) == OK and ws.value == 0
    assert lib.convnd_workspace_size(2, ctypes.byref(g), 1, 10 ** 9, ctypes.byref(ws)) == OK
    assert lib.convnd_workspace_size(7, ctypes.byref(g), 1, 0, ctypes.byref(ws)) == E_PASS
    # padding modes
    d = _nd(3, 1, 4, 4, 1, (13, 11, 9), (4, 3, 5), (0, 0, 0), (0, 0, 0), (2, 1, 3), (1, 2, 1))
    assert lib.miconv_nd_padding(ctypes.byref(d), 1) == OK
    assert list(d.out) == [7, 11, 3]
    for i, (n, f, s, dl) in enumerate(zip((13, 11, 9), (4, 3, 5), (2, 1, 3), (1, 2, 1))):
        tot = max((d.out[i] - 1) * s + dl * (f - 1) + 1 - n, 0)
        assert d.pad_lo[i] == tot // 2 and d.pad_hi[i] == tot - tot // 2
    assert lib.miconv_nd_padding(ctypes.byref(d), 0) == OK and list(d.pad_lo) == [0, 0, 0]
    assert list(d.out) == [5, 7, 2]
    assert lib.miconv_nd_padding(ctypes.byref(d), 5) == E_DIM


def test_workspace_size_errors(lib):
    out = ctypes.c_size_t(0)
    assert lib.miconv_workspace_size(7, 0, *TINY, 0, ctypes.byref(out)) == E_PASS
    assert lib.miconv_workspace_size(0, 0, *TINY, 0, None) == E_NULL
    assert lib.miconv_workspace_size(0, 0, *TINY[:11], 1, 1, 0, ctypes.byref(out)) == E_OUT
    deconv = [32, 256, 16, 16, 128, 4, 4, 1, 1, 2, 2, 32, 32]
    assert lib.miconv_workspace_size(3, 1, *deconv, 1 << 30, ctypes.byref(out)) == OK
    assert out.value == 256 * 128 * 16 * 2      # the tap-major bf16 filter copy


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_logic_with_sanitizers(tmp_path):
    exe = str(tmp_path / "host_logic")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-pthread", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(ROOT, "tests", "host", "test_host_logic.cpp"),
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "ndplan.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "OK (0 failures)" in r.stdout
