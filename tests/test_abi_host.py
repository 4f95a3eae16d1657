"""Host tests of the C ABI: every declared symbol is exported, and argument
errors are reported before any HIP call (so these run without a GPU; the
fake pointers below are never dereferenced)."""

import ctypes
import os
import re

import pytest

from gated_deltanet_recurrent_delta_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

P = ctypes.c_void_p(0x10000)        # fake, 16-byte aligned, never touched
MIS = ctypes.c_void_p(0x10004)      # fake, misaligned
NULL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(bd.SIGNATURES)


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(bd.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    assert bd.status_str(0) == "GDN_OK"
    for s in range(1, 5):
        assert bd.status_str(s).startswith("GDN_E")
    assert bd.status_str(99) == "GDN_UNKNOWN_STATUS"
    assert re.fullmatch(r"\d+\.\d+\.\d+", bd.version())


def test_workspace_bytes():
    ws = bd.prefill_workspace_bytes
    chunk = 33792                                # per head per 64-token chunk
    assert ws(1, 64, 1, 128, 128) == chunk
    assert ws(1, 65, 1, 128, 128) == 2 * chunk
    # many heads: no segmentation, only the chunk tiles
    assert ws(8, 4096, 16, 128, 128) == 8 * 16 * 64 * chunk
    # few heads, long sequence: chunk tiles plus segment buffers
    big = ws(1, 16384, 16, 128, 128)
    assert big > 16 * 256 * chunk
    assert big >= 16 * 256 * chunk + 16 * 16384 * 128 * 2
    assert ws(1, 0, 16, 128, 128) == 0
    assert ws(0, 10, 16, 128, 128) == 0
    assert ws(1, 64, 1, 96, 128) == 0


def test_prefill_segments_plan():
    seg = bd.prefill_segments
    assert seg(8, 4096, 16, 128, 128) == (1, 64)          # enough heads
    n, sc = seg(1, 16384, 16, 128, 128)                   # few heads, long
    assert n > 1 and sc >= 8 and n * sc >= 256 and (n - 1) * sc < 256
    import torch
    assert seg(1, 16384, 16, 128, 128, torch.float32, torch.float32) == (1, 256)
    assert seg(1, 100, 1, 128, 128) == (1, 2)             # too short
    with pytest.raises(ValueError):
        seg(1, 100, 1, 96, 128)


def prefill(**kw):
    a = dict(q=P, k=P, v=P, alpha=P, beta=P, S0=NULL, o=P, ST=P, B=1, T=100,
             H=2, dk=128, dv=128, in_dtype=1, out_dtype=1, ws=P,
             ws_bytes=10 ** 9, stream=NULL)
    a.update(kw)
    return bd.lib.gdn_prefill(a["q"], a["k"], a["v"], a["alpha"], a["beta"],
                              a["S0"], a["o"], a["ST"], a["B"], a["T"],
                              a["H"], a["dk"], a["dv"], a["in_dtype"],
                              a["out_dtype"], a["ws"], a["ws_bytes"],
                              a["stream"])


def decode(**kw):
    a = dict(q=P, k=P, v=P, alpha=P, beta=P, S_in=P, S_out=P, o=P, B=4, H=2,
             dk=128, dv=128, in_dtype=1, out_dtype=1, stream=NULL)
    a.update(kw)
    return bd.lib.gdn_decode_step(a["q"], a["k"], a["v"], a["alpha"],
                                  a["beta"], a["S_in"], a["S_out"], a["o"],
                                  a["B"], a["H"], a["dk"], a["dv"],
                                  a["in_dtype"], a["out_dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), bd.GDN_EINVAL),
    (dict(H=-1), bd.GDN_EINVAL),
    (dict(T=-5), bd.GDN_EINVAL),
    (dict(B=70000), bd.GDN_EINVAL),
    (dict(dk=96), bd.GDN_ESHAPE),
    (dict(dk=256), bd.GDN_ESHAPE),
    (dict(dv=32), bd.GDN_ESHAPE),
    (dict(in_dtype=2), bd.GDN_ESHAPE),
    (dict(out_dtype=-1), bd.GDN_ESHAPE),
    (dict(q=NULL), bd.GDN_EINVAL),
    (dict(v=NULL), bd.GDN_EINVAL),
    (dict(alpha=NULL), bd.GDN_EINVAL),
    (dict(o=NULL), bd.GDN_EINVAL),
    (dict(q=MIS), bd.GDN_EINVAL),
    (dict(o=MIS), bd.GDN_EINVAL),
    (dict(S0=MIS), bd.GDN_EINVAL),
    (dict(ws=NULL), bd.GDN_EWORKSPACE),
    (dict(ws_bytes=33792), bd.GDN_EWORKSPACE),          # needs 2 chunks x 2 heads
    (dict(S0=ctypes.c_void_p(0x10000), ST=ctypes.c_void_p(0x10100)),
     bd.GDN_EINVAL),                                     # partial overlap
])
def test_prefill_argument_errors(kw, status):
    assert prefill(**kw) == status


def test_prefill_empty_sequence_without_state_is_a_noop():
    # T == 0 and no ST: nothing to launch, nothing touched
    assert prefill(T=0, ST=NULL, q=NULL, k=NULL, v=NULL, o=NULL,
                   ws=NULL, ws_bytes=0) == bd.GDN_OK


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), bd.GDN_EINVAL),
    (dict(H=0), bd.GDN_EINVAL),
    (dict(dk=32), bd.GDN_ESHAPE),
    (dict(dv=256), bd.GDN_ESHAPE),
    (dict(in_dtype=5), bd.GDN_ESHAPE),
    (dict(S_in=NULL), bd.GDN_EINVAL),
    (dict(o=NULL), bd.GDN_EINVAL),
    (dict(k=MIS), bd.GDN_EINVAL),
    (dict(S_in=ctypes.c_void_p(0x100000), S_out=ctypes.c_void_p(0x100010)),
     bd.GDN_EINVAL),                                     # partial overlap
])
def test_decode_argument_errors(kw, status):
    assert decode(**kw) == status


def test_prepare_and_scan_argument_errors():
    lib = bd.lib
    assert lib.gdn_prefill_prepare(P, P, P, P, 1, 64, 1, 128, 128, 1, 1, NULL,
                                   0, NULL) == bd.GDN_EWORKSPACE
    assert lib.gdn_prefill_prepare(P, P, P, P, 1, 64, 1, 100, 128, 1, 1, P,
                                   10 ** 6, NULL) == bd.GDN_ESHAPE
    assert lib.gdn_prefill_prepare(P, P, P, P, 1, 64, 1, 128, 128, 1, 7, P,
                                   10 ** 6, NULL) == bd.GDN_ESHAPE
    assert lib.gdn_prefill_scan(P, P, P, NULL, P, P, 1, 64, 1, 128, 128, 1,
                                1, P, 100, NULL) == bd.GDN_EWORKSPACE
    assert lib.gdn_prefill_scan(NULL, P, P, NULL, P, P, 1, 64, 1, 128, 128, 1,
                                1, P, 10 ** 6, NULL) == bd.GDN_EINVAL


def test_python_wrappers_reject_host_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 64)
    with pytest.raises(ValueError):
        bd.prefill(x, x, x, torch.ones(1, 4, 2), torch.ones(1, 4, 2))


def test_truncate_workspace_bytes():
    ws = bd.truncate_workspace_bytes
    assert ws(16, 128, 128) == 16 * 128 * 128 * 8
    assert ws(16, 128, 64) == 16 * 64 * 128 * 8
    assert ws(16, 64, 128) == 16 * 64 * 64 * 8
    assert ws(0, 128, 128) == 0
    assert ws(4, 96, 128) == 0


def truncate(**kw):
    a = dict(S=P, BH=16, dv=128, dk=128, r=4, er=P, ws=P, ws_bytes=10 ** 9,
             stream=NULL)
    a.update(kw)
    return bd.lib.gdn_truncate_rank(a["S"], a["BH"], a["dv"], a["dk"],
                                    a["r"], a["er"], a["ws"], a["ws_bytes"],
                                    a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(BH=0), bd.GDN_EINVAL),
    (dict(BH=70000), bd.GDN_EINVAL),
    (dict(r=0), bd.GDN_EINVAL),
    (dict(r=-3), bd.GDN_EINVAL),
    (dict(S=NULL), bd.GDN_EINVAL),
    (dict(S=MIS), bd.GDN_EINVAL),
    (dict(dk=32), bd.GDN_ESHAPE),
    (dict(dv=256), bd.GDN_ESHAPE),
    (dict(ws=NULL), bd.GDN_EWORKSPACE),
    (dict(ws_bytes=16 * 128 * 128 * 4 - 1), bd.GDN_EWORKSPACE),
    (dict(dk=64, ws_bytes=16 * 64 * 128 * 4 - 4), bd.GDN_EWORKSPACE),
])
def test_truncate_argument_errors(kw, status):
    assert truncate(**kw) == status


def test_truncate_full_rank_needs_no_workspace_or_launch():
    # r >= min(dv, dk) with no stable rank requested: nothing to do, and no
    # workspace is needed (the fake S is never touched)
    assert truncate(r=128, er=NULL, ws=NULL, ws_bytes=0) == bd.GDN_OK
    assert truncate(dk=64, r=64, er=NULL, ws=NULL, ws_bytes=0) == bd.GDN_OK


# --- the input path (gdn_prefill_qk / gdn_decode_step_qk) -----------------

def test_prefill_qk_workspace_bytes():
    ws = bd.lib.gdn_prefill_qk_workspace_bytes
    chunk = 33792
    assert ws(1, 64, 1, 128, 128, 1, 0) == chunk                 # no gather: gdn_prefill's
    assert ws(1, 64, 1, 128, 128, 1, 1) == chunk + 2 * 64 * 128 * 2
    assert ws(1, 64, 1, 64, 128, 0, 1) == chunk + 2 * 64 * 64 * 4
    assert ws(2, 100, 3, 64, 64, 1, 1) == (
        2 * 3 * 2 * chunk + 2 * 2 * 100 * 3 * 64 * 2)
    assert ws(1, 0, 1, 128, 128, 1, 1) == 0
    assert ws(1, 64, 1, 96, 128, 1, 1) == 0
    assert ws(1, 64, 1, 128, 128, 3, 1) == 0


def prefill_qk(**kw):
    a = dict(q=P, k=P, v=P, alpha=P, beta=P, S0=NULL, o=P, ST=P, B=1, T=100,
             H=2, dk=64, dv=128, dk_in=128, ch=P, l2norm=1, scale=1.0,
             in_dtype=1, out_dtype=1, ws=P, ws_bytes=10 ** 9, stream=NULL)
    a.update(kw)
    return bd.lib.gdn_prefill_qk(a["q"], a["k"], a["v"], a["alpha"], a["beta"],
                                 a["S0"], a["o"], a["ST"], a["B"], a["T"],
                                 a["H"], a["dk"], a["dv"], a["dk_in"], a["ch"],
                                 a["l2norm"], a["scale"], a["in_dtype"],
                                 a["out_dtype"], a["ws"], a["ws_bytes"],
                                 a["stream"])


def decode_qk(**kw):
    a = dict(q=P, k=P, v=P, alpha=P, beta=P, S_in=P, S_out=P, o=P, B=4, H=2,
             dk=64, dv=128, dk_in=128, ch=P, l2norm=1, scale=1.0, in_dtype=1,
             out_dtype=1, stream=NULL)
    a.update(kw)
    return bd.lib.gdn_decode_step_qk(a["q"], a["k"], a["v"], a["alpha"],
                                     a["beta"], a["S_in"], a["S_out"], a["o"],
                                     a["B"], a["H"], a["dk"], a["dv"],
                                     a["dk_in"], a["ch"], a["l2norm"],
                                     a["scale"], a["in_dtype"],
                                     a["out_dtype"], a["stream"])


QK_ERRORS = [
    (dict(ch=NULL), bd.GDN_ESHAPE),                    # no subset: dk_in must be dk
    (dict(ch=NULL, dk_in=64, dk=128), bd.GDN_ESHAPE),
    (dict(dk_in=0), bd.GDN_ESHAPE),
    (dict(dk_in=(1 << 20) + 1), bd.GDN_ESHAPE),
    (dict(l2norm=2), bd.GDN_EINVAL),
    (dict(ch=MIS), bd.GDN_EINVAL),                      # index table not 16-byte aligned
    (dict(q=ctypes.c_void_p(0x10001)), bd.GDN_EINVAL),  # bf16 element misaligned
    (dict(q=ctypes.c_void_p(0x10002), in_dtype=0), bd.GDN_EINVAL),   # fp32 element misaligned
    (dict(ch=NULL, dk_in=64, q=ctypes.c_void_p(0x10008)), bd.GDN_EINVAL),  # whole rows: 16 B
    (dict(dk=96), bd.GDN_ESHAPE),
    (dict(B=0), bd.GDN_EINVAL),
    (dict(k=NULL), bd.GDN_EINVAL),
    (dict(S_in=NULL), bd.GDN_EINVAL),
]


@pytest.mark.parametrize("kw,status", QK_ERRORS + [
    (dict(ws=NULL), bd.GDN_EWORKSPACE),
    # gdn_prefill's workspace is not enough once the gathered copy is needed
    (dict(ws_bytes=2 * 2 * 33792), bd.GDN_EWORKSPACE),
    (dict(alpha=NULL), bd.GDN_EINVAL),
    (dict(o=MIS), bd.GDN_EINVAL),
    (dict(S0=ctypes.c_void_p(0x10000), ST=ctypes.c_void_p(0x10100)), bd.GDN_EINVAL),
])
def test_prefill_qk_argument_errors(kw, status):
    kw = {("S0" if k == "S_in" else k): v for k, v in kw.items()}
    if "S0" in kw and kw["S0"] is NULL and "ST" not in kw:
        kw["v"] = NULL                                   # no S_in in prefill: test v
    assert prefill_qk(**kw) == status


@pytest.mark.parametrize("kw,status", QK_ERRORS + [
    (dict(S_in=ctypes.c_void_p(0x100000), S_out=ctypes.c_void_p(0x100010)),
     bd.GDN_EINVAL),
])
def test_decode_step_qk_argument_errors(kw, status):
    assert decode_qk(**kw) == status


# --- generalised gates (gdn_gated_recurrent) --------------------------------

def gated(**kw):
    a = dict(q=P, k=P, v=P, alpha=P, b=P, w=P, S0=NULL, o=P, ST=P, B=1, T=10, H=2,
             dk=128, dv=128, in_dtype=1, out_dtype=1, stream=NULL)
    a.update(kw)
    return bd.lib.gdn_gated_recurrent(a["q"], a["k"], a["v"], a["alpha"], a["b"], a["w"],
                                      a["S0"], a["o"], a["ST"], a["B"], a["T"], a["H"],
                                      a["dk"], a["dv"], a["in_dtype"], a["out_dtype"],
                                      a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), bd.GDN_EINVAL),
    (dict(T=-1), bd.GDN_EINVAL),
    (dict(dk=96), bd.GDN_ESHAPE),
    (dict(dv=32), bd.GDN_ESHAPE),
    (dict(in_dtype=3), bd.GDN_ESHAPE),
    (dict(q=NULL), bd.GDN_EINVAL),
    (dict(alpha=NULL), bd.GDN_EINVAL),
    (dict(b=NULL), bd.GDN_EINVAL),
    (dict(w=NULL), bd.GDN_EINVAL),
    (dict(o=NULL), bd.GDN_EINVAL),
    (dict(k=MIS), bd.GDN_EINVAL),
    (dict(alpha=MIS), bd.GDN_EINVAL),
    (dict(w=ctypes.c_void_p(0x10002)), bd.GDN_EINVAL),
    (dict(S0=MIS), bd.GDN_EINVAL),
    (dict(S0=ctypes.c_void_p(0x10000), ST=ctypes.c_void_p(0x10100)), bd.GDN_EINVAL),
])
def test_gated_argument_errors(kw, status):
    assert gated(**kw) == status


# --- backward pass (gdn_backward) -------------------------------------------

def test_backward_workspace_bytes():
    f = bd.lib.gdn_backward_workspace_bytes
    # fp32 inputs, recurrent form: checkpoints every 8 tokens ([B H,
    # ceil(T/8), dv, dk], rounded up to 64 floats) + per-workgroup partials
    # ([B H, T, dv / 32, 2 dk + 2])
    assert f(1, 8, 1, 128, 128, 0) == 4 * (128 * 128 + 8 * 4 * 258)
    ck = 2 * 3 * 2 * 64 * 128                  # B=2, H=3, T=9 -> 2 checkpoints, dv=64, dk=128
    assert f(2, 9, 3, 128, 64, 0) == 4 * (ck + 6 * 9 * 2 * 258)
    ck = 2 * 3 * 64 * 64
    assert f(1, 17, 2, 64, 64, 0) == 4 * (ck + 2 * 17 * 2 * 130)
    # bf16 inputs, chunked form: per head and 64-token chunk the prepare
    # tiles (33,792 B), T itself (16,384 B) and two dv x dk fp32 states
    assert f(1, 64, 1, 128, 128, 1) == 33792 + 16384 + 2 * 128 * 128 * 4
    assert f(2, 65, 3, 64, 128, 1) == 6 * 2 * (33792 + 16384 + 2 * 128 * 64 * 4)
    assert f(8, 4096, 16, 128, 128, 1) == 8 * 16 * 64 * 181248
    for dt in (0, 1):
        assert f(1, 0, 2, 64, 64, dt) == 0
        assert f(1, 8, 1, 96, 128, dt) == 0 and f(0, 8, 1, 128, 128, dt) == 0
    assert f(1, 8, 1, 128, 128, 7) == 0


def backward(**kw):
    a = dict(q=P, k=P, v=P, alpha=P, beta=P, S0=NULL, d_o=P, dST=NULL, dq=P, dk_=P, dv_=P,
             dalpha=P, dbeta=P, dS0=P, B=1, T=10, H=2, dk=128, dv=128, in_dtype=1,
             ws=P, ws_bytes=1 << 40, stream=NULL)
    a.update(kw)
    return bd.lib.gdn_backward(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S0"],
                               a["d_o"], a["dST"], a["dq"], a["dk_"], a["dv_"], a["dalpha"],
                               a["dbeta"], a["dS0"], a["B"], a["T"], a["H"], a["dk"], a["dv"],
                               a["in_dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), bd.GDN_EINVAL),
    (dict(T=-1), bd.GDN_EINVAL),
    (dict(dk=96), bd.GDN_ESHAPE),
    (dict(dv=32), bd.GDN_ESHAPE),
    (dict(in_dtype=2), bd.GDN_ESHAPE),
    (dict(q=NULL), bd.GDN_EINVAL),
    (dict(d_o=NULL), bd.GDN_EINVAL),
    (dict(dalpha=NULL), bd.GDN_EINVAL),
    (dict(dk_=NULL), bd.GDN_EINVAL),
    (dict(k=MIS), bd.GDN_EINVAL),
    (dict(v=ctypes.c_void_p(0x10001)), bd.GDN_EINVAL),
    (dict(d_o=ctypes.c_void_p(0x10008)), bd.GDN_EINVAL),       # bf16 d_o: 16-byte units
    (dict(S0=MIS), bd.GDN_EINVAL),
    (dict(dS0=MIS), bd.GDN_EINVAL),
    (dict(dST=ctypes.c_void_p(0x10000), dS0=ctypes.c_void_p(0x10100)), bd.GDN_EINVAL),
    (dict(ws=NULL), bd.GDN_EWORKSPACE),
    (dict(ws=MIS), bd.GDN_EWORKSPACE),
    (dict(ws_bytes=1024), bd.GDN_EWORKSPACE),
])
def test_backward_argument_errors(kw, status):
    assert backward(**kw) == status


def test_backward_empty_sequence_without_dS0_is_a_noop():
    assert backward(T=0, dS0=NULL, q=NULL, ws=NULL, ws_bytes=0) == bd.GDN_OK


def prefill_noalloc(**kw):
    a = dict(q=P, k=P, v=P, alpha=P, beta=P, S0=NULL, o=P, ST=P, B=1, T=100,
             H=2, dk=128, dv=128, in_dtype=1, out_dtype=1, stream=NULL)
    a.update(kw)
    return bd.lib.gdn_prefill_noalloc(a["q"], a["k"], a["v"], a["alpha"], a["beta"],
                                      a["S0"], a["o"], a["ST"], a["B"], a["T"],
                                      a["H"], a["dk"], a["dv"], a["in_dtype"],
                                      a["out_dtype"], a["stream"])


def test_noalloc_scratch_size_matches_header():
    m = re.search(r"#define GDN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                  open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == bd.NOALLOC_SCRATCH_BYTES
    # the 16-head, 16K-token layer fits; the batched B=8 T=4096 H=16 does not
    assert bd.prefill_workspace_bytes(1, 16384, 16, 128, 128) <= bd.NOALLOC_SCRATCH_BYTES
    assert bd.prefill_workspace_bytes(8, 4096, 16, 128, 128) > bd.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), bd.GDN_EINVAL),
    (dict(T=-1), bd.GDN_EINVAL),
    (dict(dk=96), bd.GDN_ESHAPE),
    (dict(out_dtype=3), bd.GDN_ESHAPE),
    (dict(q=NULL), bd.GDN_EINVAL),
    (dict(beta=NULL), bd.GDN_EINVAL),
    (dict(v=MIS), bd.GDN_EINVAL),
    (dict(ST=MIS), bd.GDN_EINVAL),
    (dict(S0=ctypes.c_void_p(0x10000), ST=ctypes.c_void_p(0x10100)), bd.GDN_EINVAL),
    # more scratch than the static array holds: rejected before any HIP call
    (dict(B=8, T=4096, H=16), bd.GDN_EWORKSPACE),
    (dict(B=1, T=40000, H=16), bd.GDN_EWORKSPACE),
])
def test_prefill_noalloc_argument_errors(kw, status):
    assert prefill_noalloc(**kw) == status


def test_prefill_noalloc_empty_sequence_without_state_is_a_noop():
    assert prefill_noalloc(T=0, ST=NULL, q=NULL, k=NULL, v=NULL, o=NULL) == bd.GDN_OK


def test_gated_prefill_workspace_bytes():
    f = bd.lib.gdn_gated_prefill_workspace_bytes
    # per head and 64-token chunk: T/P tiles 32,768 B, six [64][dk] bf16
    # weighted-key matrices and e^{G_C} (dk fp32)
    assert f(1, 64, 1, 128, 128, 1) == 32768 + 6 * 64 * 128 * 2 + 128 * 4
    assert f(2, 65, 3, 64, 128, 1) == 6 * 2 * (32768 + 6 * 64 * 64 * 2 + 64 * 4)
    assert f(2, 65, 3, 64, 128, 0) == 0              # fp32 inputs: recurrent form
    assert f(1, 0, 1, 128, 128, 1) == 0 and f(1, 8, 1, 96, 128, 1) == 0


def gated_prefill(**kw):
    a = dict(q=P, k=P, v=P, alpha=P, b=P, w=P, S0=NULL, o=P, ST=P, B=1, T=100, H=2,
             dk=128, dv=128, in_dtype=1, out_dtype=1, ws=P, ws_bytes=1 << 40, stream=NULL)
    a.update(kw)
    return bd.lib.gdn_gated_prefill(a["q"], a["k"], a["v"], a["alpha"], a["b"], a["w"],
                                    a["S0"], a["o"], a["ST"], a["B"], a["T"], a["H"],
                                    a["dk"], a["dv"], a["in_dtype"], a["out_dtype"],
                                    a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), bd.GDN_EINVAL),
    (dict(dk=96), bd.GDN_ESHAPE),
    (dict(out_dtype=5), bd.GDN_ESHAPE),
    (dict(q=NULL), bd.GDN_EINVAL),
    (dict(w=NULL), bd.GDN_EINVAL),
    (dict(alpha=ctypes.c_void_p(0x10002)), bd.GDN_EINVAL),
    # gates and keys are read four channels at a time (16-byte units)
    (dict(alpha=ctypes.c_void_p(0x10008)), bd.GDN_EINVAL),
    (dict(b=ctypes.c_void_p(0x10004)), bd.GDN_EINVAL),
    (dict(k=ctypes.c_void_p(0x10008)), bd.GDN_EINVAL),
    (dict(S0=MIS), bd.GDN_EINVAL),
    (dict(ws=NULL), bd.GDN_EWORKSPACE),
    (dict(ws_bytes=4096), bd.GDN_EWORKSPACE),
])
def test_gated_prefill_argument_errors(kw, status):
    assert gated_prefill(**kw) == status
