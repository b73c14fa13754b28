"""C-ABI boundary tests that need no GPU.

The library loads, exports every function include/moe_route.h declares, and
rejects invalid arguments with the documented status before any HIP call.
Every call below carries at least one argument the host-side checks reject
(or T == 0), so nothing is ever enqueued.  The module is skipped where a GPU
is visible, so that fake pointers can never reach a kernel.
"""
import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_route.h")

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-only checks with fake pointers; run without a GPU")

from combine_topk_route_amd import _lib  # noqa: E402

OK, INVALID, ALIGN, CAP, WS, HIP = (_lib.MOE_OK, _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_ALIGNMENT,
                                    _lib.MOE_ERR_CAPACITY, _lib.MOE_ERR_WORKSPACE, _lib.MOE_ERR_HIP)
P16 = 0x10000  # a fake, 16-byte aligned address; never dereferenced
P4 = 0x10004   # 4-byte but not 16-byte aligned
S = None       # null stream


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_and_binding_declare_the_same_functions():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    assert set(declared_functions()) <= exported


def test_version_and_strerror(lib):
    assert lib.moe_abi_version() == 1
    for code in (OK, INVALID, ALIGN, CAP, WS, HIP, 12345):
        s = lib.moe_strerror(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.moe_strerror(12345) == b"unknown status"


def test_route_rejects_bad_arguments(lib):
    f = lib.moe_route_topk
    assert f(P16, -1, 8, 2, P16, P16, S) == INVALID           # T < 0
    assert f(P16, 4, 0, 1, P16, P16, S) == INVALID            # E < 1
    assert f(P16, 4, 1025, 2, P16, P16, S) == INVALID         # E > 1024
    assert f(P16, 4, 8, 0, P16, P16, S) == INVALID            # k < 1
    assert f(P16, 4, 8, 9, P16, P16, S) == INVALID            # k > E
    assert f(P16, 4, 64, 33, P16, P16, S) == INVALID          # k > 32
    assert f(None, 4, 8, 2, P16, P16, S) == INVALID           # null logits
    assert f(P16, 4, 8, 2, None, P16, S) == INVALID
    assert f(P16, 4, 8, 2, P16, None, S) == INVALID
    assert f(P16, 2**30, 8, 2, P16, P16, S) == INVALID        # T*k >= 2^31
    assert f(P16 + 1, 4, 8, 2, P16, P16, S) == ALIGN          # misaligned fp32
    assert f(None, 0, 8, 2, None, None, S) == OK              # T == 0 is a no-op


def test_workspace_size_function(lib):
    f = lib.moe_dispatch_workspace_bytes
    assert f(0, 8, 2) == 0
    assert f(16, 8, 2) == 0            # small inputs run fused in one block
    assert f(128, 256, 8) == 0
    ws = f(8192, 256, 8)
    assert ws > 0 and ws % 256 == 0
    assert f(8192, 0, 8) == 0          # rejected shapes report 0
    assert f(-1, 8, 2) == 0


def test_dispatch_send_rejects_bad_arguments(lib):
    f = lib.moe_dispatch_send
    ok_ws = lib.moe_dispatch_workspace_bytes(8192, 256, 8)
    args = lambda **kw: [kw.get("idx", P16), kw.get("T", 8192), kw.get("E", 256), kw.get("k", 8),
                         kw.get("R", 32), kw.get("counts", P16), kw.get("offsets", P16),
                         kw.get("pair_row", P16), kw.get("row_token", P16), kw.get("rank", None),
                         kw.get("ws", P16), kw.get("wsb", ok_ws), S]
    assert f(*args(R=3)) == INVALID                 # E % R != 0
    assert f(*args(R=0)) == INVALID
    assert f(*args(R=512)) == INVALID               # R > E
    assert f(*args(k=0)) == INVALID
    assert f(*args(idx=None)) == INVALID
    assert f(*args(counts=None)) == INVALID
    assert f(*args(offsets=None)) == INVALID
    assert f(*args(pair_row=None)) == INVALID
    assert f(*args(row_token=None)) == INVALID
    assert f(*args(pair_row=P16 + 2)) == ALIGN
    assert f(*args(ws=None)) == WS                  # workspace needed but missing
    assert f(*args(wsb=ok_ws - 1)) == WS            # workspace too small
    assert f(*args(T=0, idx=None, counts=None, offsets=None, pair_row=None, row_token=None,
                   ws=None, wsb=0)) == OK


def test_dispatch_recv_and_combine_reject_bad_arguments(lib):
    r = lib.moe_dispatch_recv
    assert r(P16, P16, 16, 256, 2, P16, 31, S) == CAP          # capacity < T*k
    assert r(P16, P16, 16, 255, 2, P16, 32, S) == ALIGN        # H % 8 != 0
    assert r(P16, P16, 16, 0, 2, P16, 32, S) == INVALID        # H < 8
    assert r(P4, P16, 16, 256, 2, P16, 32, S) == ALIGN         # x not 16-byte aligned
    assert r(P16, P16, 16, 256, 2, P4, 32, S) == ALIGN         # buf not 16-byte aligned
    assert r(None, P16, 16, 256, 2, P16, 32, S) == INVALID
    assert r(P16, None, 16, 256, 2, P16, 32, S) == INVALID
    assert r(P16, P16, 16, 256, 0, P16, 32, S) == INVALID      # k < 1
    assert r(P16, P16, -1, 256, 2, P16, 32, S) == INVALID
    assert r(None, None, 0, 256, 2, None, 0, S) == OK

    c = lib.moe_combine
    assert c(P16, P16, P16, 16, 256, 2, 31, P16, S) == CAP
    assert c(P16, P16, P16, 16, 12, 2, 32, P16, S) == ALIGN
    assert c(P4, P16, P16, 16, 256, 2, 32, P16, S) == ALIGN
    assert c(P16, P16, P16, 16, 256, 2, 32, P4, S) == ALIGN
    assert c(P16, None, P16, 16, 256, 2, 32, P16, S) == INVALID
    assert c(P16, P16, None, 16, 256, 2, 32, P16, S) == INVALID
    assert c(None, P16, P16, 16, 256, 2, 32, P16, S) == INVALID
    assert c(P16, P16, P16, 16, 256, 33, 32 * 16, P16, S) == INVALID  # k > 32
    assert c(None, None, None, 0, 256, 2, 0, None, S) == OK


def test_dispatch_checks_both_halves_before_enqueueing(lib):
    f = lib.moe_dispatch
    ws = lib.moe_dispatch_workspace_bytes(8192, 256, 8)
    base = [P16, P16, 8192, 256, 8, 7168, 32, P16, P16, P16, P16, None, P16, 8192 * 8, P16, ws, S]
    bad_cap = list(base)
    bad_cap[13] = 8192 * 8 - 1
    assert f(*bad_cap) == CAP                      # recv half rejected, send never enqueued
    bad_r = list(base)
    bad_r[6] = 5
    assert f(*bad_r) == INVALID
    bad_ws = list(base)
    bad_ws[15] = 0
    assert f(*bad_ws) == WS
    bad_h = list(base)
    bad_h[5] = 7170
    assert f(*bad_h) == ALIGN


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()


def test_fp8_dispatch_rejects_bad_arguments(lib):
    r = lib.moe_dispatch_recv_fp8
    assert r(P16, P16, 16, 256, 2, P16, P16, 31, S) == CAP
    assert r(P16, P16, 16, 264, 2, P16, P16, 32, S) == ALIGN      # H % 128 != 0 (but % 8 == 0)
    assert r(P16, P16, 16, 256, 2, P4, P16, 32, S) == ALIGN       # codes not 16-byte aligned
    assert r(P16, P16, 16, 256, 2, P16, P16 + 2, 32, S) == ALIGN  # scales not 4-byte aligned
    assert r(P16, P16, 16, 256, 2, P16, None, 32, S) == INVALID
    assert r(P16, None, 16, 256, 2, P16, P16, 32, S) == INVALID
    assert r(None, None, 0, 256, 2, None, None, 0, S) == OK
    f = lib.moe_dispatch_fp8
    ws = lib.moe_dispatch_workspace_bytes(8192, 256, 8)
    base = [P16, P16, 8192, 256, 8, 7168, 32, P16, P16, P16, P16, None, P16, P16, 8192 * 8, P16,
            ws, S]
    bad = list(base)
    bad[5] = 7176                    # H % 128 != 0
    assert f(*bad) == ALIGN
    bad = list(base)
    bad[13] = None                   # no scale buffer
    assert f(*bad) == INVALID
    bad = list(base)
    bad[6] = 7                       # E % R != 0
    assert f(*bad) == INVALID


def test_grouped_route_rejects_bad_arguments(lib):
    f = lib.moe_route_topk_grouped
    assert f(P16, 4, 256, 8, 3, 1, P16, P16, S) == INVALID     # E % n_group != 0
    assert f(P16, 4, 256, 8, 0, 1, P16, P16, S) == INVALID     # n_group < 1
    assert f(P16, 4, 256, 8, 128, 2, P16, P16, S) == INVALID   # n_group > 64
    assert f(P16, 4, 256, 8, 8, 0, P16, P16, S) == INVALID     # topk_group < 1
    assert f(P16, 4, 256, 8, 8, 9, P16, P16, S) == INVALID     # topk_group > n_group
    assert f(P16, 4, 256, 8, 64, 1, P16, P16, S) == INVALID    # 1 group of 4 < k = 8
    assert f(None, 4, 256, 8, 8, 4, P16, P16, S) == INVALID
    assert f(None, 0, 256, 8, 8, 4, None, None, S) == OK


def test_route_dispatch_checks_every_part_before_enqueueing(lib):
    f = lib.moe_route_dispatch
    wsf = lib.moe_route_dispatch_workspace_bytes
    assert wsf(128, 256, 8) == 256                 # the arrival counter block only
    assert wsf(8192, 256, 8) == 256 + lib.moe_dispatch_workspace_bytes(8192, 256, 8)
    assert wsf(8192, 0, 8) == 0
    ws = wsf(8192, 256, 8)
    # logits, x, T, E, k, n_group, topk_group, H, R, idx, w, counts, offsets, pair_row,
    # row_token, rank, buf, cap, ws, wsb
    base = [P16, P16, 8192, 256, 8, 1, 1, 7168, 32, P16, P16, P16, P16, P16, P16, None, P16,
            8192 * 8, P16, ws, S]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a4=33) == INVALID                  # k > 32 (routing)
    assert call(a5=3) == INVALID                   # E % n_group != 0
    assert call(a5=8, a6=9) == INVALID             # topk_group > n_group
    assert call(a5=64, a6=1) == INVALID            # one group of 4 experts < k
    assert call(a0=None) == INVALID                # null logits
    assert call(a10=None) == INVALID               # null weights
    assert call(a0=P16 + 2) == ALIGN               # misaligned logits
    assert call(a8=5) == INVALID                   # E % R != 0 (send)
    assert call(a17=8192 * 8 - 1) == CAP           # capacity < T*k (recv)
    assert call(a7=7170) == ALIGN                  # H % 8 != 0
    assert call(a18=None) == WS                    # no workspace
    assert call(a19=ws - 1) == WS                  # short: the send part does not fit
    assert call(a2=128, a17=1024, a19=255) == WS   # short: no room for the counter
    assert call(a2=128, a17=1024, a19=256, a18=P16 + 2) == ALIGN
    assert call(a2=0, a0=None, a1=None, a9=None, a10=None, a11=None, a12=None, a13=None,
                a14=None, a16=None, a17=0, a18=None, a19=0) == OK


def test_route_dispatch_fp8_checks_every_part_before_enqueueing(lib):
    f = lib.moe_route_dispatch_fp8
    ws = lib.moe_route_dispatch_workspace_bytes(8192, 256, 8)
    # logits, x, T, E, k, n_group, topk_group, H, R, idx, w, counts, offsets, pair_row,
    # row_token, rank, buf_q, buf_scale, cap, ws, wsb
    base = [P16, P16, 8192, 256, 8, 1, 1, 7168, 32, P16, P16, P16, P16, P16, P16, None, P16, P16,
            8192 * 8, P16, ws, S]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a4=33) == INVALID                  # k > 32 (routing)
    assert call(a5=3) == INVALID                   # E % n_group != 0
    assert call(a0=None) == INVALID                # null logits
    assert call(a8=5) == INVALID                   # E % R != 0 (send)
    assert call(a18=8192 * 8 - 1) == CAP           # capacity < T*k (recv)
    assert call(a7=7176) == ALIGN                  # H % 128 != 0 (fp8 blocks)
    assert call(a7=7170) == ALIGN                  # H % 8 != 0
    assert call(a17=None) == INVALID               # null scales
    assert call(a16=P16 + 8) == ALIGN              # codes not 16-byte aligned
    assert call(a19=None) == WS                    # no workspace
    assert call(a20=ws - 1) == WS                  # short workspace
    assert call(a2=0, a0=None, a1=None, a9=None, a10=None, a11=None, a12=None, a13=None,
                a14=None, a16=None, a17=None, a18=0, a19=None, a20=0) == OK


def test_noalloc_dispatch_checks_every_argument_before_the_device(lib):
    """moe_dispatch_noalloc validates every argument before it looks up the
    device's scratch array, so each bad call fails with its own status (here,
    with no GPU, a call that passed the checks would fail with MOE_ERR_HIP)."""
    f = lib.moe_dispatch_noalloc
    base = [P16, P16, 8192, 256, 8, 7168, 32, P16, P16, P16, P16, None, P16, 8192 * 8, S]
    cases = [(0, 0, INVALID), (1, 0, INVALID), (13, 8192 * 8 - 1, CAP), (6, 5, INVALID), (5, 7170, ALIGN), (3, 0, INVALID),
             (4, 33, INVALID), (7, 0, INVALID), (12, 0, INVALID), (12, P4, ALIGN), (2, -1, INVALID)]
    for i, v, want in cases:
        args = list(base)
        args[i] = v
        assert f(*args) == want, (i, v)
    zero = list(base)
    zero[2] = 0
    assert f(*zero) == OK                          # T == 0: nothing to do, no device needed
    small = list(base)
    small[2], small[13] = 16, 16 * 8               # T*k <= 4096 needs no scratch
    small[5] = 7170
    assert f(*small) == ALIGN
    assert f(*base) == HIP                         # valid arguments, but no device here
