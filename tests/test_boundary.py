"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects every bad argument on the host before any HIP call."""

import math
import os
import re

import pytest

import io_aware_tiled_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, NULL, SHAPE, DTYPE, BAD_D, SCALE, ALIGN, LARGE, HIP = range(9)
P = 0x10000  # a 16-byte aligned fake address (never dereferenced: validation only)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = fa.load()
    names = _declared_functions()
    assert set(names) >= {"fa_fwd", "fa_check_args", "fa_bwd", "fa_bwd_check_args",
                          "fa_fwd_splitkv", "fa_splitkv_workspace_bytes", "fa_splitkv_check_args",
                          "fa_status_string", "fa_abi_version", "fa_fwd_splitkv_noalloc"}
    for n in names:
        assert hasattr(lib, n), n
    assert fa.fa_abi_version() == 6


def test_status_strings():
    for code, name in fa.STATUS.items():
        assert fa.fa_status_string(code).startswith(name)
    assert "unknown" in fa.fa_status_string(99)


FWD_ORDER = ("q", "k", "v", "o", "lse", "B", "H", "M", "N", "D", "scale", "causal", "dtype")
BWD_ORDER = ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta", "B", "H", "M", "N",
             "D", "scale", "causal", "dtype")
SPLIT_ORDER = FWD_ORDER + ("splits", "ws", "wsb")


def fwd_args(kw):
    """fa_check_args' arguments for one table row, in call order."""
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=3, M=100, N=70, D=64, scale=0.125, causal=0,
             dtype=fa.DTYPE_BF16)
    a.update(kw)
    return tuple(a[n] for n in FWD_ORDER)


def _chk(**kw):
    return fa.fa_check_args(*fwd_args(kw))


FWD_CHECK_CASES = [
    ({}, OK),
    ({"dtype": 3}, DTYPE), ({"dtype": -1}, DTYPE),
    ({"B": -1}, SHAPE), ({"H": -2}, SHAPE), ({"M": -1}, SHAPE), ({"N": -5}, SHAPE),
    ({"causal": 2}, SHAPE),
    ({"D": 0}, BAD_D), ({"D": 129}, BAD_D), ({"D": -3}, BAD_D), ({"D": 1}, OK), ({"D": 128}, OK),
    ({"scale": 0.0}, OK), ({"scale": -0.1}, OK), ({"scale": -1e30}, OK), ({"scale": 1e-45}, OK),
    ({"scale": 2.3e38}, OK), ({"scale": -2.3e38}, OK),   # scale*log2(e) still finite in fp32
    ({"scale": 3e38}, SCALE), ({"scale": -3e38}, SCALE),  # scale*log2(e) overflows fp32
    ({"scale": math.inf}, SCALE), ({"scale": -math.inf}, SCALE), ({"scale": math.nan}, SCALE),
    ({"q": 0}, NULL), ({"o": 0}, NULL), ({"lse": 0}, NULL), ({"k": 0}, NULL), ({"v": 0}, NULL),
    ({"q": P + 8}, ALIGN), ({"k": P + 2}, ALIGN), ({"o": P + 4}, ALIGN), ({"lse": P + 2}, ALIGN),
    ({"lse": P + 4}, OK),
    ({"B": 0, "q": 0, "k": 0, "v": 0, "o": 0, "lse": 0}, OK),   # empty: nothing to do
    ({"M": 0, "q": 0, "o": 0, "lse": 0}, OK),
    ({"N": 0, "k": 0, "v": 0}, OK),                             # no keys: every row empty
    ({"M": 1 << 25, "D": 64}, LARGE), ({"N": 1 << 25, "D": 64}, LARGE),
    ({"B": 1 << 20, "H": 1 << 12, "M": 128}, LARGE),
    # int64 edges: M * D, N * D, M + 127, B * H would overflow if formed
    ({"M": (1 << 63) - 1, "D": 128}, LARGE), ({"N": (1 << 63) - 1, "D": 128}, LARGE),
    ({"M": (1 << 57), "D": 64}, LARGE), ({"B": (1 << 62), "H": 4}, LARGE),
    ({"B": (1 << 63) - 1, "H": (1 << 63) - 1, "M": 1}, LARGE),
    ({"M": (1 << 31) // 64 - 1, "N": (1 << 31) // 64 - 1, "D": 64, "B": 1, "H": 1}, OK),
    ({"M": (1 << 31) // 64, "D": 64, "B": 1, "H": 1}, LARGE),
]


@pytest.mark.parametrize("kw,code", FWD_CHECK_CASES)
def test_check_args(kw, code):
    assert _chk(**kw) == code


@pytest.mark.parametrize("kw,code", [
    ({"dtype": 7}, DTYPE), ({"D": 200}, BAD_D), ({"scale": math.nan}, SCALE), ({"q": 0}, NULL),
    ({"q": P + 8}, ALIGN), ({"B": 0}, OK), ({"M": 0}, OK),
])
def test_fa_fwd_rejects_before_any_hip_call(kw, code):
    # Every case here returns from host validation (or is an empty problem) and
    # never reaches the HIP runtime, so it runs without a GPU.
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=3, M=100, N=70, D=64, scale=0.125, causal=1,
             dtype=fa.DTYPE_F16)
    a.update(kw)
    st = fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["M"], a["N"],
                   a["D"], a["scale"], a["causal"], a["dtype"], None)
    assert st == code


def bwd_args(kw):
    """fa_bwd_check_args' arguments for one table row, in call order."""
    a = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, delta=P, B=2, H=3, M=100, N=70,
             D=64, scale=0.125, causal=0, dtype=fa.DTYPE_BF16)
    a.update(kw)
    return tuple(a[n] for n in BWD_ORDER)


def _bchk(**kw):
    return fa.fa_bwd_check_args(*bwd_args(kw))


BWD_CHECK_CASES = [
    ({}, OK), ({"dtype": fa.DTYPE_F16}, OK), ({"dtype": fa.DTYPE_F32}, OK),
    ({"dtype": 3}, DTYPE),
    ({"B": -1}, SHAPE), ({"N": -1}, SHAPE), ({"causal": 2}, SHAPE),
    ({"D": 0}, BAD_D), ({"D": 129}, BAD_D), ({"scale": 0.0}, OK), ({"scale": -0.5}, OK),
    ({"scale": math.nan}, SCALE), ({"scale": 3e38}, SCALE),
    ({"q": 0}, NULL), ({"o": 0}, NULL), ({"lse": 0}, NULL), ({"dout": 0}, NULL), ({"dq": 0}, NULL),
    ({"delta": 0}, NULL), ({"k": 0}, NULL), ({"v": 0}, NULL), ({"dk": 0}, NULL), ({"dv": 0}, NULL),
    ({"dout": P + 8}, ALIGN), ({"dq": P + 2}, ALIGN), ({"dk": P + 4}, ALIGN), ({"dv": P + 8}, ALIGN),
    ({"delta": P + 2}, ALIGN), ({"delta": P + 4}, OK),
    ({"B": 0, "q": 0, "k": 0, "v": 0, "o": 0, "lse": 0, "dout": 0, "dq": 0, "dk": 0, "dv": 0,
      "delta": 0}, OK),
    ({"M": 0, "N": 0, "q": 0, "k": 0, "v": 0, "o": 0, "lse": 0, "dout": 0, "dq": 0, "dk": 0,
      "dv": 0, "delta": 0}, OK),
    # no queries: only dk, dv (zeros) and the K, V they come from are needed
    ({"M": 0, "q": 0, "o": 0, "lse": 0, "dout": 0, "dq": 0, "delta": 0}, OK),
    # no keys: only dq (zeros) and the query-side inputs are needed
    ({"N": 0, "k": 0, "v": 0, "dk": 0, "dv": 0}, OK),
    ({"M": 1 << 25, "D": 64}, LARGE), ({"N": 1 << 25, "D": 64}, LARGE),
    ({"B": 1 << 20, "H": 1 << 12, "M": 128, "N": 128}, LARGE),
    ({"M": (1 << 63) - 1, "D": 128}, LARGE), ({"N": (1 << 63) - 1, "D": 96}, LARGE),
    ({"B": (1 << 63) - 1, "H": (1 << 63) - 1}, LARGE),
]


@pytest.mark.parametrize("kw,code", BWD_CHECK_CASES)
def test_bwd_check_args(kw, code):
    assert _bchk(**kw) == code


@pytest.mark.parametrize("kw,code", [
    ({"dtype": 5}, DTYPE), ({"D": 200}, BAD_D), ({"dq": 0}, NULL),
    ({"dk": P + 8}, ALIGN), ({"B": 0}, OK), ({"M": 0, "N": 0}, OK),
])
def test_fa_bwd_rejects_before_any_hip_call(kw, code):
    a = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, delta=P, B=2, H=3, M=100, N=70,
             D=64, scale=0.125, causal=1, dtype=fa.DTYPE_F16)
    a.update(kw)
    st = fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"],
                   a["delta"], a["B"], a["H"], a["M"], a["N"], a["D"], a["scale"], a["causal"],
                   a["dtype"], None)
    assert st == code


WS = 1 << 20  # a fake 16-byte aligned workspace address


def split_args(kw):
    """fa_splitkv_check_args' arguments for one table row, in call order."""
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=3, M=100, N=70, D=64, scale=0.125, causal=0,
             dtype=fa.DTYPE_BF16, splits=4, ws=WS, wsb=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = fa.fa_splitkv_workspace_bytes(a["B"], a["H"], a["M"], a["D"], a["splits"])
    return tuple(a[n] for n in SPLIT_ORDER)


def _schk(**kw):
    return fa.fa_splitkv_check_args(*split_args(kw))


WORKSPACE = 9


SPLIT_CHECK_CASES = [
    ({}, OK), ({"dtype": fa.DTYPE_F32}, OK), ({"splits": 1}, OK), ({"splits": 64}, OK),
    ({"splits": 0}, SHAPE), ({"splits": 65}, SHAPE), ({"splits": -3}, SHAPE),
    ({"ws": 0}, WORKSPACE), ({"ws": WS + 8}, WORKSPACE), ({"wsb": 1000}, WORKSPACE),
    ({"D": 0}, BAD_D), ({"q": 0}, NULL), ({"scale": math.inf}, SCALE),  # fa_fwd's checks come first
    ({"N": 0, "k": 0, "v": 0, "ws": 0, "wsb": 0}, OK),  # no keys: no chunk, no workspace needed
    ({"M": 0, "q": 0, "o": 0, "lse": 0, "ws": 0, "wsb": 0}, OK),
]


@pytest.mark.parametrize("kw,code", SPLIT_CHECK_CASES)
def test_splitkv_check_args(kw, code):
    assert _schk(**kw) == code


def test_splitkv_workspace_bytes():
    assert fa.fa_splitkv_workspace_bytes(2, 3, 100, 64, 4) == 4 * 2 * 3 * 100 * 65 * 4
    assert fa.fa_splitkv_workspace_bytes(1, 1, 1, 1, 1) == 8
    assert fa.fa_splitkv_workspace_bytes(1, 1, 1, 0, 1) == -1
    assert fa.fa_splitkv_workspace_bytes(1, 1, 1, 8, 0) == -1
    assert fa.fa_splitkv_workspace_bytes(1, 1, 1, 129, 1) == -1
    assert fa.fa_splitkv_workspace_bytes(1 << 40, 1 << 20, 1 << 10, 128, 64) == -1  # beyond int64


def test_noalloc_rejects_before_any_hip_call():
    """The allocation-free entry point validates like fa_fwd_splitkv and refuses
    problems whose partials exceed its static scratch, all on the host."""
    lim = fa.NOALLOC_MAX_BYTES
    assert lim == 64 << 20
    # 2*3*100 rows * 65 * 4 B * 64 splits = 9.98 MB fits; 1024 heads of 512 rows do not
    assert fa.fa_splitkv_workspace_bytes(2, 3, 100, 64, 64) <= lim
    big = (1, 1024, 512, 64, 4)
    assert fa.fa_splitkv_workspace_bytes(*big) > lim
    assert fa.fa_fwd_splitkv_noalloc(P, P, P, P, P, 1, 1024, 512, 700, 64, 0.125, 1,
                                     fa.DTYPE_F16, 4, None) == 10
    assert fa.fa_status_string(10).startswith("FA_ERR_SCRATCH_LIMIT")
    assert fa.fa_fwd_splitkv_noalloc(P, P, P, P, P, 2, 3, 100, 70, 64, 0.125, 1, fa.DTYPE_F16,
                                     0, None) == SHAPE
    assert fa.fa_fwd_splitkv_noalloc(0, P, P, P, P, 2, 3, 100, 70, 64, 0.125, 1, fa.DTYPE_F16,
                                     4, None) == NULL
    assert fa.fa_fwd_splitkv_noalloc(P, P, P, P, P, 0, 3, 100, 70, 64, 0.125, 1, fa.DTYPE_F16,
                                     4, None) == OK


def test_fa_fwd_splitkv_rejects_before_any_hip_call():
    wsb = fa.fa_splitkv_workspace_bytes(2, 3, 100, 64, 4)
    assert fa.fa_fwd_splitkv(P, P, P, P, P, 2, 3, 100, 70, 64, 0.125, 1, fa.DTYPE_F16, 4, 0, wsb,
                             None) == WORKSPACE
    assert fa.fa_fwd_splitkv(P, P, P, P, P, 2, 3, 100, 70, 64, 0.125, 1, fa.DTYPE_F16, 99, WS, wsb,
                             None) == SHAPE
    assert fa.fa_fwd_splitkv(P, P, P, P, P, 0, 3, 100, 70, 64, 0.125, 1, fa.DTYPE_F16, 4, 0, 0,
                             None) == OK


def test_python_wrapper_validates_before_the_library(monkeypatch):
    import torch

    q = torch.zeros(1, 1, 4, 8)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q)  # CPU tensors are refused
    with pytest.raises(ValueError):
        fa.fwd(q[0], q[0], q[0])
    with pytest.raises(TypeError):
        fa._dtype_code(torch.zeros(1, dtype=torch.int32))
    lse = torch.zeros(1, 1, 4)
    with pytest.raises(ValueError):
        fa.bwd(q, q, q, q, lse, q)  # CPU tensors are refused
    with pytest.raises(ValueError):
        fa.bwd(q, q, q, q, lse.double(), q)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_LIB", None)
    monkeypatch.setattr(fa, "lib_path", lambda: str(tmp_path / "nope.so"))
    with pytest.raises(ImportError):
        fa.load()
    with pytest.raises(ImportError):
        fa.fa_fwd(P, P, P, P, P, 1, 1, 1, 1, 8, 1.0, 0, 0, None)


def test_binding_checks_caller_supplied_buffers():
    """Output and workspace tensors handed to the binding must match what the
    kernels write through their pointers; anything else is refused before a
    launch (shape, dtype, device, layout)."""
    import torch

    from io_aware_tiled_fa_amd import _check_given

    dev = torch.device("cpu")
    good = torch.empty(2, 3, 5, 8, dtype=torch.float16)
    _check_given(good, "out", (2, 3, 5, 8), torch.float16, dev)
    with pytest.raises(ValueError, match="shape"):
        _check_given(good, "out", (2, 3, 5, 9), torch.float16, dev)
    with pytest.raises(TypeError, match="float32"):
        _check_given(good, "out", (2, 3, 5, 8), torch.float32, dev)
    with pytest.raises(ValueError, match="on cuda"):
        _check_given(good, "out", (2, 3, 5, 8), torch.float16, torch.device("cuda:0"))
    with pytest.raises(ValueError, match="contiguous"):
        _check_given(good.transpose(2, 3).contiguous().transpose(2, 3), "out", (2, 3, 5, 8),
                     torch.float16, dev)
