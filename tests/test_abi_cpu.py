"""The C ABI on the CPU: the library loads (no GPU needed), exports every
function include/spec_verify.h declares, and its host-side validation returns
the documented status codes.  No compute call is made here."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s+\**(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def sv():
    import lossless_token_verification_amd as m
    if not os.path.exists(m.LIB_PATH):
        # a fresh checkout: build the library (hipcc cross-compiles without a GPU)
        from lossless_token_verification_amd import build
        build.build()
    m.library()
    return m


def test_every_declared_symbol_is_exported(sv):
    names = declared_functions()
    assert len(names) == 17, names
    assert set(names) == set(sv.EXPORTED)
    lib = ctypes.CDLL(sv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(sv):
    lib = sv.library()
    assert sv.abi_version() == 4
    for code, name in ((0, b"SV_OK"), (1, b"SV_ERR_INVALID_ARG"), (2, b"SV_ERR_UNSUPPORTED"),
                       (3, b"SV_ERR_MISALIGNED"), (4, b"SV_ERR_WORKSPACE"), (5, b"SV_ERR_DEVICE"),
                       (99, b"SV_ERR_UNKNOWN")):
        assert lib.spec_verify_status_string(code) == name


def test_workspace_size_formula(sv):
    # 256 B of flags + 12 B per sequence + 2 draw-tile sums per (sequence, tile)
    # (each area padded to 256 B) + one 16-byte partial per (row, 64 KiB chunk)
    def pad(n):
        return (n + 255) // 256 * 256

    def tiles(V, per):
        return -(-V // per)
    def parts(rows, nc, B, k):
        # chunk partials (16 B), entropy partials (8 B), outcome-export partials (72 B)
        return pad(rows * nc * 16) + pad(rows * nc * 8) + B * 2 * (k + 1) * nc * 72

    assert sv.workspace_bytes(256, 8, 128256, 1, 3) == \
        256 + pad((256 * 29 + 1) * 4) + pad(256 * 2 * tiles(128256, 512) * 4) + parts(256 * 26, 4, 256, 8)
    assert sv.workspace_bytes(64, 4, 32000, 1, 2) == \
        256 + pad((64 * 17 + 1) * 4) + pad(64 * 2 * tiles(32000, 512) * 4) + parts(64 * 9, 1, 64, 4)
    assert sv.workspace_bytes(32, 5, 151936, 0, 2) == \
        256 + pad((32 * 20 + 1) * 4) + pad(32 * 2 * tiles(151936, 256) * 4) + parts(32 * 11, 10, 32, 5)
    assert sv.workspace_bytes(0, 4, 10, 0, 2) == 256
    assert sv.workspace_bytes(1, 64, 10, 0, 2) == 0        # invalid descriptor -> 0


def _status(sv, **kw):
    base = dict(batch=4, num_draft=3, vocab=100, dtype_code=0, row_stride=0)
    base.update({k: v for k, v in kw.items() if k in base})
    d = sv.make_desc(**base)
    if "reserved" in kw:
        d.reserved = kw["reserved"]
    return sv.validate(d, kw.get("exits", 2), kw.get("window", 4), kw.get("ws", 1 << 30))


def test_validation_codes(sv):
    assert _status(sv) == sv.SV_OK
    assert _status(sv, exits=3) == sv.SV_OK
    assert _status(sv, batch=0) == sv.SV_OK
    assert _status(sv, num_draft=0) == sv.SV_OK
    assert _status(sv, num_draft=63) == sv.SV_OK
    assert _status(sv, batch=-1) == sv.SV_ERR_INVALID_ARG
    assert _status(sv, num_draft=-1) == sv.SV_ERR_INVALID_ARG
    assert _status(sv, num_draft=64) == sv.SV_ERR_UNSUPPORTED
    assert _status(sv, vocab=0) == sv.SV_ERR_INVALID_ARG
    assert _status(sv, vocab=(1 << 20) + 1) == sv.SV_ERR_UNSUPPORTED
    assert _status(sv, dtype_code=2) == sv.SV_ERR_UNSUPPORTED
    assert _status(sv, row_stride=99) == sv.SV_ERR_INVALID_ARG
    assert _status(sv, row_stride=128) == sv.SV_OK
    assert _status(sv, exits=3, window=0) == sv.SV_ERR_INVALID_ARG
    assert _status(sv, exits=4) == sv.SV_ERR_INVALID_ARG
    assert _status(sv, ws=10) == sv.SV_ERR_WORKSPACE
    assert _status(sv, reserved=1) == sv.SV_ERR_INVALID_ARG
    lib = sv.library()
    assert lib.spec_verify_validate(None, 2, 1, 1 << 20) == sv.SV_ERR_INVALID_ARG
    assert b"desc is NULL" in lib.spec_verify_last_error()


def test_kv_truncate_host_checks(sv):
    lib = sv.library()
    assert lib.kv_blocktable_truncate(-1, 4, 16, None, None, None, None, 1, None, None) == 1
    assert lib.kv_blocktable_truncate(2, 4, 0, None, None, None, None, 1, None, None) == 1
    assert lib.kv_blocktable_truncate(2, 4, 16, None, None, None, None, 1, None, None) == 1
    assert lib.kv_blocktable_truncate(0, 4, 16, None, None, None, None, 1, None, None) == 0


def test_verify_host_checks_without_gpu(sv):
    """Failing validation returns before any HIP call, so it runs without a GPU."""
    lib = sv.library()
    d = sv.make_desc(2, 3, 100, 0)
    args = [None] * 11 + [0, None, None]
    assert lib.spec_verify_single(ctypes.byref(d), *args) == sv.SV_ERR_INVALID_ARG
    assert b"NULL" in lib.spec_verify_last_error()
    d0 = sv.make_desc(0, 3, 100, 0)
    ws = ctypes.create_string_buffer(1024)
    # B = 0 with a workspace: nothing to launch, SV_OK
    a = (ctypes.c_char * 1024).from_buffer(ws)
    addr = (ctypes.addressof(a) + 255) // 256 * 256
    if addr + 256 <= ctypes.addressof(a) + 1024:
        assert lib.spec_verify_single(ctypes.byref(d0), *([None] * 10), ctypes.c_void_p(addr),
                                      256, None, None) == sv.SV_OK
    # misaligned logits pointer
    args = [ctypes.c_void_p(0x1002), ctypes.c_void_p(0x1000)] + [ctypes.c_void_p(0x1000)] * 8
    assert lib.spec_verify_single(ctypes.byref(d), *args, ctypes.c_void_p(0x10000), 1 << 20,
                                  None, None) == sv.SV_ERR_MISALIGNED


def test_lmhead_workspace_formula_and_checks(sv):
    """LM-head plan: flags + 8 B per sequence + draw-tile sums of fp32 rows +
    one 16-byte partial per (GEMM row, 384-entry vocabulary tile of the
    statistics GEMM) + merged partials + gathered logits + stopped-row ids +
    two fp32 rows per sequence."""
    def pad(n):
        return (n + 255) // 256 * 256
    B, k, V, d = 128, 4, 128256, 4096
    M = B * (2 * k + 1)
    nt = -(-V // 256)
    want = (256 + pad(B * 8) + pad(B * 2 * nt * 4) + pad(M * (-(-V // 384)) * 16) +
            pad(M * 16) + pad(M * 4) + pad(2 * B * 4) + 2 * B * V * 4)
    assert sv.lmhead_workspace_bytes(B, k, V, d) == want
    assert sv.lmhead_workspace_bytes(3, 2, 1001, 64) > 0
    assert sv.lmhead_workspace_bytes(3, 2, 1001, 96) == 0          # hidden % 64 != 0
    assert sv.lmhead_workspace_bytes(3, 2, 1001, 0) == 0
    assert sv.lmhead_workspace_bytes(3, 2, 1001, 64, row_stride=68) == 0   # stride % 8
    assert sv.lmhead_workspace_bytes(3, 2, 1001, 64, row_stride=72) > 0
    lib = sv.library()
    d32 = sv.make_desc(2, 3, 100, 0)          # fp32 is not an LM-head type
    args = [None] * 12 + [0, None, None]
    assert lib.spec_verify_lmhead_single(ctypes.byref(d32), 64, *args) == sv.SV_ERR_UNSUPPORTED
    db = sv.make_desc(2, 3, 100, 1)
    assert lib.spec_verify_lmhead_single(ctypes.byref(db), 64, *args) == sv.SV_ERR_INVALID_ARG
    assert b"NULL" in lib.spec_verify_last_error()
    ptrs = [ctypes.c_void_p(0x1008), ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1000)]
    rest = [ctypes.c_void_p(0x1000)] * 8
    assert lib.spec_verify_lmhead_single(ctypes.byref(db), 64, *ptrs, *rest,
                                         ctypes.c_void_p(0x10000), 1 << 30, None,
                                         None) == sv.SV_ERR_MISALIGNED


def test_byproduct_host_checks_without_gpu(sv):
    """By-product requests are validated before any launch: top_m range, output
    alignment, and the calls that cannot produce them (lazy final exit, LM head)."""
    lib = sv.library()
    d = sv.make_desc(2, 3, 100, 0)
    p = ctypes.c_void_p(0x1000)
    single = [p] * 10 + [ctypes.c_void_p(0x10000), 1 << 30]

    dg = sv.Diag()
    dg.residual_tokens = 0x2000
    dg.top_m = 0
    assert lib.spec_verify_single(ctypes.byref(d), *single, ctypes.byref(dg), None) == \
        sv.SV_ERR_INVALID_ARG
    assert b"top_m" in lib.spec_verify_last_error()
    dg.top_m = sv.MAX_TOP_M + 1
    assert lib.spec_verify_single(ctypes.byref(d), *single, ctypes.byref(dg), None) == \
        sv.SV_ERR_INVALID_ARG

    dg = sv.Diag()
    dg.entropy = 0x2002
    assert lib.spec_verify_single(ctypes.byref(d), *single, ctypes.byref(dg), None) == \
        sv.SV_ERR_MISALIGNED

    dg = sv.Diag()
    dg.entropy = 0x2000
    hier = [p] * 10 + [4, 16, p, p, p, 1, p, ctypes.c_void_p(0x10000), 1 << 30]
    assert lib.spec_verify_hier_rollback_lazy(ctypes.byref(d), 4, *hier, ctypes.byref(dg),
                                              None) == sv.SV_ERR_UNSUPPORTED
    assert b"lazy" in lib.spec_verify_last_error()
    dg = sv.Diag()
    dg.accept_mass = 0x2000
    db = sv.make_desc(2, 3, 100, 1)
    lm = [ctypes.c_void_p(0x1000)] * 11 + [ctypes.c_void_p(0x10000), 1 << 30]
    assert lib.spec_verify_lmhead_single(ctypes.byref(db), 64, *lm, ctypes.byref(dg), None) == \
        sv.SV_ERR_UNSUPPORTED
    # row statistics: 8-byte aligned, and only where every row is streamed
    dg = sv.Diag()
    dg.row_log2z = 0x2004
    assert lib.spec_verify_single(ctypes.byref(d), *single, ctypes.byref(dg), None) == \
        sv.SV_ERR_MISALIGNED
    assert b"row_log2z" in lib.spec_verify_last_error()
    dg = sv.Diag()
    dg.row_argmax = 0x2000
    assert lib.spec_verify_hier_rollback_lazy(ctypes.byref(d), 4, *hier, ctypes.byref(dg),
                                              None) == sv.SV_ERR_UNSUPPORTED
    assert lib.spec_verify_lmhead_single(ctypes.byref(db), 64, *lm, ctypes.byref(dg), None) == \
        sv.SV_ERR_UNSUPPORTED


def test_tentative_host_checks_without_gpu(sv):
    """Workspace sizing and the failures the tentative calls report before any
    launch: capacity outside [1, 63], a missing pending state, a short
    workspace."""
    lib = sv.library()
    B, k, V = 4, 3, 1000
    d = sv.make_desc(B, k, V, 0)

    def pad(n):
        return (n + 255) // 256 * 256

    cap = 10
    rnd = sv.workspace_bytes(B, k, V, 0, 2)
    fl = sv.workspace_bytes(B, cap, V, 0, 2)
    want = max(pad(rnd) + pad(B * (k + 1) * 4) + pad(B * 4),
               pad(fl) + pad(B * 4) + pad((2 * B * cap + 1) * 4))
    assert sv.tentative_workspace_bytes(B, k, V, 0, cap) == want
    assert sv.tentative_workspace_bytes(B, k, V, 0, 0) == 0
    assert sv.tentative_workspace_bytes(B, k, V, 0, 64) == 0
    p = ctypes.c_void_p(0x1000)
    pend = sv.Pending(0x2000, 0x3000, 0x4000, 64)
    args = [p] * 5
    assert lib.spec_verify_tentative_round(ctypes.byref(d), *args, ctypes.byref(pend), p, p,
                                           ctypes.c_void_p(0x10000), 1 << 30, None) == \
        sv.SV_ERR_UNSUPPORTED
    assert lib.spec_verify_tentative_round(ctypes.byref(d), *args, None, p, p,
                                           ctypes.c_void_p(0x10000), 1 << 30, None) == \
        sv.SV_ERR_INVALID_ARG
    pend = sv.Pending(0x2000, 0x3000, 0x4000, cap)
    assert lib.spec_verify_tentative_round(ctypes.byref(d), *args, ctypes.byref(pend), p, p,
                                           ctypes.c_void_p(0x10000), 16, None) == \
        sv.SV_ERR_WORKSPACE
    assert lib.spec_verify_tentative_flush(ctypes.byref(d), p, None, -1, ctypes.byref(pend), p,
                                           p, p, p, ctypes.c_void_p(0x10000), 1 << 30, None) == \
        sv.SV_ERR_INVALID_ARG
    pend = sv.Pending(0x2000, 0x3000, 0x4002, cap)
    assert lib.spec_verify_tentative_flush(ctypes.byref(d), p, None, 4, ctypes.byref(pend), p,
                                           p, p, p, ctypes.c_void_p(0x10000), 1 << 30, None) == \
        sv.SV_ERR_MISALIGNED


def test_noalloc_rejects_oversized_calls_on_the_host(sv):
    """spec_verify_hier_rollback_noalloc refuses a call whose workspace exceeds
    its static scratch before any HIP call (so it works here, without a GPU),
    and reports the sizes."""
    lib = sv.library()
    # V = 2^20 bf16, k = 63: the workspace runs far past 16 MiB
    d = sv.make_desc(256, 63, 1 << 20, sv.SV_DTYPE_BF16)
    assert sv.workspace_bytes(256, 63, 1 << 20, sv.SV_DTYPE_BF16, 3) > sv.NOALLOC_SCRATCH_BYTES
    z = ctypes.c_void_p(16)
    st = lib.spec_verify_hier_rollback_noalloc(ctypes.byref(d), 4, z, z, z, z, None, z, z, z, z,
                                               None, 8, 16, z, z, z, 1, z, None, None)
    assert st == sv.SV_ERR_WORKSPACE
    msg = lib.spec_verify_last_error().decode()
    assert "scratch" in msg and str(sv.NOALLOC_SCRATCH_BYTES) in msg
    # an invalid descriptor is reported as such, not as a size problem
    bad = sv.make_desc(4, 3, 0, sv.SV_DTYPE_BF16)
    assert lib.spec_verify_hier_rollback_noalloc(ctypes.byref(bad), 4, z, z, z, z, None, z, z, z,
                                                 z, None, 8, 16, z, z, z, 1, z, None,
                                                 None) == sv.SV_ERR_INVALID_ARG
