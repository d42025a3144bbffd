"""The C ABI without a GPU: the library loads, exports every declared symbol, and
rejects every invalid argument with its status code before any launch.

Only validation failures are exercised here (they return before the first HIP
call), plus the pure host function attn_bwd_workspace_bytes.  The fake device
pointers are never dereferenced.
"""

import ctypes
import os
import re

import pytest
import torch

import online_softmax_attn_amd as osa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "osattn.h")

P = 0x10000  # a 16-byte aligned fake address, never dereferenced
S = osa.STATUS


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\*?\s+\**((?:attn|rowsoftmax|rowxent)_[a-z0-9_]+)\s*\(",
                                 text, flags=re.M)))


def header_enum(name_prefix):
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"(ATTN_[A-Z0-9_]+)\s*=\s*(-?\d+)", text)
            if m.group(1).startswith(name_prefix)}


def test_library_exports_every_header_symbol():
    lib = osa.library()
    names = header_functions()
    assert set(names) == set(osa.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_status_codes_match_header():
    enum = header_enum("ATTN_ERR")
    enum["ATTN_OK"] = header_enum("ATTN_OK")["ATTN_OK"]
    assert enum == S
    for name, code in S.items():
        assert osa.status_string(code) and osa.status_string(code) != "unknown status"
    assert osa.status_string(-99) == "unknown status"


def fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Hkv=1, N=8, d=64, scale=0.125, causal=0,
             dtype=2, stream=None)
    a.update(kw)
    return osa.library().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                  a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"],
                                  a["stream"])


def bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=2, Hkv=1, N=8, d=64,
             scale=0.125, causal=0, dtype=2, ws=P, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return osa.library().attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                                  a["dk"], a["dv"], a["B"], a["H"], a["Hkv"], a["N"], a["d"],
                                  a["scale"], a["causal"], a["dtype"], a["ws"], a["ws_bytes"],
                                  a["stream"])


INVALID = [
    ({"q": None}, "ATTN_ERR_NULL"),
    ({"lse": None}, "ATTN_ERR_NULL"),
    ({"B": 0}, "ATTN_ERR_SHAPE"),
    ({"H": 0}, "ATTN_ERR_SHAPE"),
    ({"Hkv": 0}, "ATTN_ERR_SHAPE"),
    ({"N": 0}, "ATTN_ERR_SHAPE"),
    ({"N": -5}, "ATTN_ERR_SHAPE"),
    ({"B": 1 << 16, "H": 1 << 10, "Hkv": 1 << 10, "N": 1 << 10}, "ATTN_ERR_SHAPE"),
    ({"causal": 2}, "ATTN_ERR_SHAPE"),
    ({"d": 32}, "ATTN_ERR_HEAD_DIM"),
    ({"d": 256}, "ATTN_ERR_HEAD_DIM"),
    ({"d": 96}, "ATTN_ERR_HEAD_DIM"),
    ({"H": 3, "Hkv": 2}, "ATTN_ERR_GQA"),
    ({"dtype": 3}, "ATTN_ERR_DTYPE"),
    ({"dtype": -1}, "ATTN_ERR_DTYPE"),
    ({"scale": 0.0}, "ATTN_ERR_SCALE"),
    ({"scale": -1.0}, "ATTN_ERR_SCALE"),
    ({"scale": float("inf")}, "ATTN_ERR_SCALE"),
    ({"scale": float("nan")}, "ATTN_ERR_SCALE"),
    ({"q": P + 8}, "ATTN_ERR_ALIGN"),
    ({"lse": P + 4}, "ATTN_ERR_ALIGN"),
]


@pytest.mark.parametrize("kw,code", INVALID, ids=[f"{k}->{c}" for k, c in INVALID])
def test_fwd_rejects(kw, code):
    assert fwd(**kw) == S[code]


@pytest.mark.parametrize("kw,code", INVALID + [
    ({"do": None}, "ATTN_ERR_NULL"),
    ({"dv": None}, "ATTN_ERR_NULL"),
    ({"ws": None}, "ATTN_ERR_WORKSPACE"),
    ({"ws_bytes": 16}, "ATTN_ERR_WORKSPACE"),
    ({"dk": P + 2}, "ATTN_ERR_ALIGN"),
    ({"ws": P + 8}, "ATTN_ERR_ALIGN"),
], ids=lambda x: str(x))
def test_bwd_rejects(kw, code):
    assert bwd(**kw) == S[code]


def bwd_noalloc(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=2, Hkv=1, N=8, d=64,
             scale=0.125, causal=0, dtype=2, stream=None)
    a.update(kw)
    return osa.library().attn_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"],
                                          a["dq"], a["dk"], a["dv"], a["B"], a["H"], a["Hkv"],
                                          a["N"], a["d"], a["scale"], a["causal"], a["dtype"],
                                          a["stream"])


@pytest.mark.parametrize("kw,code", [
    ({"q": None}, "ATTN_ERR_NULL"),
    ({"dv": None}, "ATTN_ERR_NULL"),
    ({"N": 0}, "ATTN_ERR_SHAPE"),
    ({"causal": 2}, "ATTN_ERR_SHAPE"),
    ({"d": 96}, "ATTN_ERR_HEAD_DIM"),
    ({"H": 3, "Hkv": 2}, "ATTN_ERR_GQA"),
    ({"dtype": 7}, "ATTN_ERR_DTYPE"),
    ({"scale": float("nan")}, "ATTN_ERR_SCALE"),
    ({"scale": 0.0}, "ATTN_ERR_SCALE"),
    ({"dk": P + 8}, "ATTN_ERR_ALIGN"),
    # one query row over the 4194304 the fixed scratch holds (two float32 per row)
    ({"B": 1, "H": 1, "Hkv": 1, "N": 4194305}, "ATTN_ERR_SCRATCH"),
    ({"B": 2, "H": 64, "Hkv": 8, "N": 32769}, "ATTN_ERR_SCRATCH"),
])
def test_bwd_noalloc_rejects(kw, code):
    """Every invalid argument, and any problem larger than the fixed scratch, is
    refused before the device is asked for anything."""
    assert bwd_noalloc(**kw) == S[code]


def test_noalloc_scratch_limit_matches_workspace_formula():
    f = osa.library().attn_bwd_workspace_bytes
    assert f(1, 1, 1, 4194304, 64, 2) == 32 << 20      # the largest problem it takes
    assert f(1, 1, 1, 4194305, 64, 2) > 32 << 20


def pre(**kw):
    a = dict(o=P, lse=P, do=P, B=1, H=2, Hkv=1, N=8, d=64, dtype=2, ws=P, ws_bytes=1 << 20,
             stream=None)
    a.update(kw)
    return osa.library().attn_bwd_preprocess(a["o"], a["lse"], a["do"], a["B"], a["H"], a["Hkv"],
                                             a["N"], a["d"], a["dtype"], a["ws"], a["ws_bytes"],
                                             a["stream"])


def stage(fn, **kw):
    a = dict(q=P, k=P, v=P, lse=P, do=P, out1=P, out2=P, B=1, H=2, Hkv=1, N=8, d=64,
             scale=0.125, causal=0, dtype=2, ws=P, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    lib = osa.library()
    tail = (a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"],
            a["ws"], a["ws_bytes"], a["stream"])
    if fn == "dkdv":
        return lib.attn_bwd_dkdv(a["q"], a["k"], a["v"], a["lse"], a["do"], a["out1"], a["out2"],
                                 *tail)
    return lib.attn_bwd_dq(a["q"], a["k"], a["v"], a["lse"], a["do"], a["out1"], *tail)


STAGE_INVALID = [kw for kw in INVALID if "o" not in kw[0]] + [
    ({"do": None}, "ATTN_ERR_NULL"),
    ({"out1": None}, "ATTN_ERR_NULL"),
    ({"ws": None}, "ATTN_ERR_WORKSPACE"),
    ({"ws_bytes": 16}, "ATTN_ERR_WORKSPACE"),
    ({"out1": P + 2}, "ATTN_ERR_ALIGN"),
    ({"ws": P + 8}, "ATTN_ERR_ALIGN"),
]


@pytest.mark.parametrize("fn", ["dkdv", "dq"])
@pytest.mark.parametrize("kw,code", STAGE_INVALID, ids=lambda x: str(x))
def test_bwd_stage_rejects(fn, kw, code):
    assert stage(fn, **kw) == S[code]


def test_bwd_stage_dkdv_checks_second_output():
    assert stage("dkdv", out2=None) == S["ATTN_ERR_NULL"]
    assert stage("dkdv", out2=P + 4) == S["ATTN_ERR_ALIGN"]


@pytest.mark.parametrize("kw,code", [
    ({"o": None}, "ATTN_ERR_NULL"),
    ({"lse": None}, "ATTN_ERR_NULL"),
    ({"do": None}, "ATTN_ERR_NULL"),
    ({"N": 0}, "ATTN_ERR_SHAPE"),
    ({"d": 96}, "ATTN_ERR_HEAD_DIM"),
    ({"H": 3, "Hkv": 2}, "ATTN_ERR_GQA"),
    ({"dtype": 7}, "ATTN_ERR_DTYPE"),
    ({"ws": None}, "ATTN_ERR_WORKSPACE"),
    ({"ws_bytes": 100}, "ATTN_ERR_WORKSPACE"),
    ({"o": P + 8}, "ATTN_ERR_ALIGN"),
    ({"ws": P + 4}, "ATTN_ERR_ALIGN"),
], ids=lambda x: str(x))
def test_bwd_preprocess_rejects(kw, code):
    assert pre(**kw) == S[code]


def test_workspace_bytes():
    f = osa.library().attn_bwd_workspace_bytes
    assert f(1, 1, 1, 1, 64, 0) == 2 * 256
    n = 4 * 16 * 8192
    assert f(4, 16, 16, 8192, 128, 2) == 2 * n * 4
    assert f(1, 32, 8, 16384, 128, 2) == 2 * 32 * 16384 * 4
    assert f(1, 3, 3, 5, 64, 1) == 2 * 256
    assert f(1, 3, 2, 8, 64, 2) == 0          # H not a multiple of Hkv
    assert f(1, 1, 1, 8, 80, 2) == 0          # unsupported d
    assert f(0, 1, 1, 8, 64, 2) == 0


def test_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        osa.attn_fwd(q, q, q)


def split(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=4, Hkv=2, Nq=3, Nk=100, d=128, scale=0.125,
             causal=1, dtype=2, n_splits=0, ws=P, ws_bytes=1 << 24, stream=None)
    a.update(kw)
    return osa.library().attn_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                          a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"],
                                          a["causal"], a["dtype"], a["n_splits"], a["ws"],
                                          a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    ({"q": None}, "ATTN_ERR_NULL"),
    ({"lse": None}, "ATTN_ERR_NULL"),
    ({"Nq": 0}, "ATTN_ERR_SHAPE"),
    ({"Nk": 0}, "ATTN_ERR_SHAPE"),
    ({"B": 0}, "ATTN_ERR_SHAPE"),
    ({"n_splits": -1}, "ATTN_ERR_SHAPE"),
    ({"causal": 2}, "ATTN_ERR_SHAPE"),
    ({"causal": 1, "Nq": 101}, "ATTN_ERR_SHAPE"),
    ({"d": 96}, "ATTN_ERR_HEAD_DIM"),
    ({"H": 3}, "ATTN_ERR_GQA"),
    ({"dtype": 0}, "ATTN_ERR_DTYPE"),
    ({"dtype": 5}, "ATTN_ERR_DTYPE"),
    ({"scale": 0.0}, "ATTN_ERR_SCALE"),
    ({"ws": None}, "ATTN_ERR_WORKSPACE"),
    ({"ws_bytes": 64}, "ATTN_ERR_WORKSPACE"),
    ({"o": P + 8}, "ATTN_ERR_ALIGN"),
    ({"ws": P + 4}, "ATTN_ERR_ALIGN"),
    # Over 2^26 query rows: the merge's one wave per row would count 2^32 work-items.
    ({"B": 9, "H": 1, "Hkv": 1, "Nq": (1 << 23) - 1, "Nk": 1000, "d": 64, "causal": 0,
      "n_splits": 1, "ws_bytes": 1 << 62}, "ATTN_ERR_SHAPE"),
], ids=lambda x: str(x))
def test_splitkv_rejects(kw, code):
    assert split(**kw) == S[code]


def test_splitkv_workspace_bytes():
    f = osa.library().attn_fwd_splitkv_workspace_bytes
    r256 = lambda x: (x + 255) // 256 * 256
    # One query of 4 heads, 100 keys = 4 tiles, auto: at most one chunk per 4 tiles.
    assert f(1, 4, 2, 1, 100, 128, 1, 2, 0) == r256(1 * 4 * 1 * 128 * 4) + r256(4 * 4)
    # Explicit chunk counts: 3 chunks of 2 tiles (64 keys) leave 2 non-empty chunks.
    assert f(1, 4, 2, 1, 100, 128, 0, 2, 3) == r256(2 * 4 * 128 * 4) + r256(2 * 4 * 4)
    # Requests above one chunk per 32 keys are capped at 4 chunks here.
    assert f(1, 4, 2, 1, 100, 64, 0, 1, 99) == r256(4 * 4 * 64 * 4) + r256(4 * 4 * 4)
    # Invalid arguments give 0.
    assert f(1, 4, 2, 1, 100, 128, 1, 0, 0) == 0       # fp32 has no split-KV kernel
    assert f(1, 4, 2, 200, 100, 128, 1, 2, 0) == 0     # causal with Nq > Nk
    assert f(1, 4, 2, 1, 100, 128, 0, 2, -2) == 0
    # The largest row count whose merge grid fits, and the first that does not.
    assert f(8, 1, 1, (1 << 23) - 1, 1000, 64, 0, 2, 1) > 0
    assert f(9, 1, 1, (1 << 23) - 1, 1000, 64, 0, 2, 1) == 0


def masked(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=4, Hkv=2, Nq=3, Nk=100, d=128, scale=0.125,
             lo=P, hi=P, dtype=2, stream=None)
    a.update(kw)
    return osa.library().attn_fwd_masked(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                         a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["lo"],
                                         a["hi"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    ({"q": None}, "ATTN_ERR_NULL"),
    ({"lo": None}, "ATTN_ERR_NULL"),
    ({"hi": None}, "ATTN_ERR_NULL"),
    ({"Nq": 0}, "ATTN_ERR_SHAPE"),
    ({"Nk": 0}, "ATTN_ERR_SHAPE"),
    ({"d": 32}, "ATTN_ERR_HEAD_DIM"),
    ({"H": 3}, "ATTN_ERR_GQA"),
    ({"dtype": 9}, "ATTN_ERR_DTYPE"),
    ({"scale": -2.0}, "ATTN_ERR_SCALE"),
    ({"o": P + 8}, "ATTN_ERR_ALIGN"),
    ({"lo": P + 2}, "ATTN_ERR_ALIGN"),
], ids=lambda x: str(x))
def test_masked_fwd_rejects(kw, code):
    assert masked(**kw) == S[code]


def masked_bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=4, Hkv=2, Nq=3, Nk=100,
             d=128, scale=0.125, lo=P, hi=P, dtype=2, ws=P, ws_bytes=1 << 24, stream=None)
    a.update(kw)
    return osa.library().attn_bwd_masked(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"],
                                         a["dq"], a["dk"], a["dv"], a["B"], a["H"], a["Hkv"],
                                         a["Nq"], a["Nk"], a["d"], a["scale"], a["lo"], a["hi"],
                                         a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    ({"do": None}, "ATTN_ERR_NULL"),
    ({"hi": None}, "ATTN_ERR_NULL"),
    ({"Nk": 0}, "ATTN_ERR_SHAPE"),
    ({"d": 80}, "ATTN_ERR_HEAD_DIM"),
    ({"H": 5}, "ATTN_ERR_GQA"),
    ({"dtype": 4}, "ATTN_ERR_DTYPE"),
    ({"scale": float("inf")}, "ATTN_ERR_SCALE"),
    ({"ws": None}, "ATTN_ERR_WORKSPACE"),
    ({"ws_bytes": 512}, "ATTN_ERR_WORKSPACE"),
    ({"dv": P + 2}, "ATTN_ERR_ALIGN"),
    ({"lo": P + 1}, "ATTN_ERR_ALIGN"),
], ids=lambda x: str(x))
def test_masked_bwd_rejects(kw, code):
    assert masked_bwd(**kw) == S[code]


def test_masked_bwd_workspace_bytes():
    f = osa.library().attn_bwd_masked_workspace_bytes
    r256 = lambda x: (x + 255) // 256 * 256
    assert f(2, 4, 2, 100, 300, 128, 2) == 2 * r256(2 * 4 * 100 * 4) + r256(2 * 2 * 16)
    assert f(1, 1, 1, 1, 1, 64, 0) == 2 * 256 + 256
    assert f(1, 4, 2, 100, 0, 128, 2) == 0


# ---- row softmax / log-softmax / cross-entropy --------------------------------------
def row_call(fn, **kw):
    lib = osa.library()
    a = dict(x=P, y=P, dy=P, dx=P, t=P, loss=P, lse=P, dloss=P, rows=4, cols=64, log=0, dtype=2,
             stream=None)
    a.update(kw)
    if fn == "rowsoftmax_fwd":
        return lib.rowsoftmax_fwd(a["x"], a["y"], a["rows"], a["cols"], a["log"], a["dtype"],
                                  a["stream"])
    if fn == "rowsoftmax_bwd":
        return lib.rowsoftmax_bwd(a["y"], a["dy"], a["dx"], a["rows"], a["cols"], a["log"],
                                  a["dtype"], a["stream"])
    if fn == "rowxent_fwd":
        return lib.rowxent_fwd(a["x"], a["t"], a["loss"], a["lse"], a["rows"], a["cols"],
                               a["dtype"], a["stream"])
    return lib.rowxent_bwd(a["x"], a["t"], a["lse"], a["dloss"], a["dx"], a["rows"], a["cols"],
                           a["dtype"], a["stream"])


ROW_FNS = ("rowsoftmax_fwd", "rowsoftmax_bwd", "rowxent_fwd", "rowxent_bwd")
ROW_INVALID = [
    ({"rows": 0}, "ATTN_ERR_SHAPE"),
    ({"rows": -1}, "ATTN_ERR_SHAPE"),
    ({"rows": 1 << 31}, "ATTN_ERR_SHAPE"),
    ({"cols": 0}, "ATTN_ERR_SHAPE"),
    ({"cols": -3}, "ATTN_ERR_SHAPE"),
    ({"cols": (1 << 30) + 1}, "ATTN_ERR_SHAPE"),
    ({"dtype": 3}, "ATTN_ERR_DTYPE"),
    ({"dtype": -1}, "ATTN_ERR_DTYPE"),
]
ROW_NULLS = {
    "rowsoftmax_fwd": ("x", "y"),
    "rowsoftmax_bwd": ("y", "dy", "dx"),
    "rowxent_fwd": ("x", "t", "loss", "lse"),
    "rowxent_bwd": ("x", "t", "lse", "dloss", "dx"),
}
ROW_ALIGN = {
    "rowsoftmax_fwd": {"x": P + 8, "y": P + 2},
    "rowsoftmax_bwd": {"y": P + 4, "dy": P + 8, "dx": P + 2},
    "rowxent_fwd": {"x": P + 8, "t": P + 2, "loss": P + 1, "lse": P + 3},
    "rowxent_bwd": {"x": P + 8, "dx": P + 4, "t": P + 2, "lse": P + 1, "dloss": P + 3},
}


@pytest.mark.parametrize("fn", ROW_FNS)
@pytest.mark.parametrize("kw,code", ROW_INVALID)
def test_row_rejects_sizes(fn, kw, code):
    assert row_call(fn, **kw) == S[code]


@pytest.mark.parametrize("fn", ROW_FNS)
def test_row_rejects_null_and_misalignment(fn):
    for name in ROW_NULLS[fn]:
        assert row_call(fn, **{name: None}) == S["ATTN_ERR_NULL"], name
    for name, addr in ROW_ALIGN[fn].items():
        assert row_call(fn, **{name: addr}) == S["ATTN_ERR_ALIGN"], name


@pytest.mark.parametrize("fn", ("rowsoftmax_fwd", "rowsoftmax_bwd"))
def test_row_rejects_bad_log_flag(fn):
    assert row_call(fn, log=2) == S["ATTN_ERR_SHAPE"]
    assert row_call(fn, log=-1) == S["ATTN_ERR_SHAPE"]


def test_row_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 8)
    t = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        osa.rowsoftmax_fwd(x)
    with pytest.raises(ValueError):
        osa.rowsoftmax_bwd(x, x)
    with pytest.raises(ValueError):
        osa.rowxent_fwd(x, t)
    with pytest.raises(ValueError):
        osa.rowxent_bwd(x, t, t.float(), t.float())


# ---- fp8 forward ----------------------------------------------------------------------
def fp8(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Hkv=1, N=100, d=128, scale=0.125, dq=0.01,
             dk=0.01, dv=0.01, causal=0, ws=P, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return osa.library().attn_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                      a["Hkv"], a["N"], a["d"], a["scale"], a["dq"], a["dk"],
                                      a["dv"], a["causal"], a["ws"], a["ws_bytes"], a["stream"])


FP8_INVALID = [
    ({"q": None}, "ATTN_ERR_NULL"),
    ({"ws": None}, "ATTN_ERR_NULL"),
    ({"N": 0}, "ATTN_ERR_SHAPE"),
    ({"B": 0}, "ATTN_ERR_SHAPE"),
    ({"d": 96}, "ATTN_ERR_HEAD_DIM"),
    ({"d": 32}, "ATTN_ERR_HEAD_DIM"),
    ({"H": 3, "Hkv": 2}, "ATTN_ERR_GQA"),
    ({"causal": 2}, "ATTN_ERR_SHAPE"),
    ({"scale": 0.0}, "ATTN_ERR_SCALE"),
    ({"dq": float("nan")}, "ATTN_ERR_SCALE"),
    ({"dk": -1.0}, "ATTN_ERR_SCALE"),
    ({"dv": float("inf")}, "ATTN_ERR_SCALE"),
    ({"k": P + 8}, "ATTN_ERR_ALIGN"),
    ({"ws": P + 4}, "ATTN_ERR_ALIGN"),
    ({"ws_bytes": 100}, "ATTN_ERR_WORKSPACE"),
]


@pytest.mark.parametrize("kw,code", FP8_INVALID)
def test_fp8_rejects(kw, code):
    assert fp8(**kw) == S[code]


def test_fp8_workspace_bytes():
    lib = osa.library()
    # V transposed: B * Hkv * d dims * N rounded up to 128 keys, rounded to 256 bytes.
    assert lib.attn_fwd_fp8_workspace_bytes(2, 3, 100, 128) == 2 * 3 * 128 * 128
    assert lib.attn_fwd_fp8_workspace_bytes(1, 1, 129, 128) == 128 * 256
    assert lib.attn_fwd_fp8_workspace_bytes(1, 1, 100, 64) == 64 * 128
    assert lib.attn_fwd_fp8_workspace_bytes(1, 1, 100, 96) == 0
    assert lib.attn_fwd_fp8_workspace_bytes(0, 1, 100, 128) == 0
    assert osa.attn_fwd_fp8_workspace_bytes(4, 16, 8192) == 4 * 16 * 128 * 8192


def test_tensors_on_two_devices_are_refused():
    """The binding runs each call on its tensors' device and refuses a mix of devices
    before anything is enqueued (stand-ins with a device attribute; no GPU here)."""
    from types import SimpleNamespace as NS
    dev = lambda s: NS(device=torch.device(s))
    assert osa._common_device([dev("cuda:1"), dev("cuda:1"), dev("cpu")]) == torch.device("cuda:1")
    assert osa._common_device([dev("cpu")]) is None
    assert osa._common_device([]) is None
    with pytest.raises(ValueError, match="more than one device"):
        osa._common_device([dev("cuda:0"), dev("cuda:1")])


def test_public_calls_carry_the_device_guard():
    for name in osa.__all__:
        fn = getattr(osa, name)
        if name.endswith("_bytes") or not callable(fn) or name in ("library", "status_string",
                                                                   "AttnError", "library_path"):
            continue
        assert getattr(fn, "__wrapped__", None) is not None, name
