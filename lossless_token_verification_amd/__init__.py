"""Python binding of libspecverify.so (the MI355X batched lossless token
verification library).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, and their data pointers and torch's current HIP stream are handed
to the C ABI declared in ``include/spec_verify.h``.  Every step of the
verification runs in the library's HIP kernels; there is no fallback path.  If
the library has not been built, every call raises ``RuntimeError``.

Functions mirror the C entry points:

* ``spec_verify_single``  -- standard rule, draft vs target (+ bonus token);
* ``spec_verify_hier``    -- HiSpec two-stage L_d -> L_i -> L_f verification;
* ``kv_blocktable_truncate`` -- paged-KV rollback of rejected drafted slots;
* ``spec_verify_hier_rollback`` -- the two above in the same launches;
* ``spec_verify_tentative_round`` / ``spec_verify_tentative_flush`` -- the
  hierarchy across calls: intermediate rounds append to a pending state
  (``make_pending``), a flush verifies it against the final exit;
* ``workspace_bytes``, ``validate``, ``device_status``, ``abi_version``.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SPEC_VERIFY_LIB names another build of the same library (the host-sanitizer
# build of the tests); by default the one built next to this file.
LIB_PATH = os.environ.get("SPEC_VERIFY_LIB") or os.path.join(_HERE, "libspecverify.so")

SV_OK = 0
SV_ERR_INVALID_ARG = 1
SV_ERR_UNSUPPORTED = 2
SV_ERR_MISALIGNED = 3
SV_ERR_WORKSPACE = 4
SV_ERR_DEVICE = 5
SV_DTYPE_F32 = 0
SV_DTYPE_BF16 = 1
SV_FLAG_TOKEN_RANGE = 1
SV_FLAG_TEMPERATURE = 2
SV_FLAG_PENDING_FULL = 4
MAX_DRAFT = 63
MAX_VOCAB = 1 << 20
MAX_HIDDEN = 1 << 16
MAX_TOP_M = 8

# Every symbol include/spec_verify.h declares.
EXPORTED = (
    "spec_verify_abi_version", "spec_verify_status_string", "spec_verify_last_error",
    "spec_verify_workspace_bytes", "spec_verify_validate", "spec_verify_single",
    "spec_verify_hier", "kv_blocktable_truncate", "spec_verify_hier_rollback",
    "spec_verify_device_status", "spec_verify_lmhead_workspace_bytes",
    "spec_verify_lmhead_single", "spec_verify_hier_rollback_lazy",
    "spec_verify_tentative_workspace_bytes", "spec_verify_tentative_round",
    "spec_verify_tentative_flush", "spec_verify_hier_rollback_noalloc",
)
# bytes of the static scratch of spec_verify_hier_rollback_noalloc (SV_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 16 << 20


class Desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_draft", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("row_stride", ctypes.c_int64), ("seed", ctypes.c_uint64),
                ("offset", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class Diag(ctypes.Structure):
    _fields_ = [("uniforms", ctypes.c_void_p), ("probs", ctypes.c_void_p),
                ("draws", ctypes.c_void_p), ("stats_begin", ctypes.c_void_p),
                ("stats_end", ctypes.c_void_p), ("entropy", ctypes.c_void_p),
                ("accept_mass", ctypes.c_void_p), ("residual_tokens", ctypes.c_void_p),
                ("residual_mass", ctypes.c_void_p), ("top_m", ctypes.c_int32),
                ("row_log2z", ctypes.c_void_p), ("row_argmax", ctypes.c_void_p)]


class Pending(ctypes.Structure):
    _fields_ = [("count", ctypes.c_void_p), ("tokens", ctypes.c_void_p),
                ("rows", ctypes.c_void_p), ("capacity", ctypes.c_int32)]


class SpecVerifyError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def library():
    """The loaded ctypes library; raises RuntimeError when it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    _lib = load_library(LIB_PATH)
    return _lib


def load_library(path):
    """A ctypes handle of a build of the library at ``path`` with the entry
    points' signatures set (the bindings use ``library()``; a test that
    compares two builds swaps ``_lib``)."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, u32, sz = ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    lib.spec_verify_abi_version.restype = i32
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    lib.spec_verify_status_string.argtypes = [i32]
    lib.spec_verify_last_error.restype = ctypes.c_char_p
    lib.spec_verify_workspace_bytes.restype = sz
    lib.spec_verify_workspace_bytes.argtypes = [ctypes.POINTER(Desc), i32]
    lib.spec_verify_validate.restype = i32
    lib.spec_verify_validate.argtypes = [ctypes.POINTER(Desc), i32, i32, sz]
    lib.spec_verify_single.restype = i32
    lib.spec_verify_single.argtypes = [ctypes.POINTER(Desc), P, P, P, P, P, P, P, P, P, P, P, sz,
                                       ctypes.POINTER(Diag), P]
    lib.spec_verify_hier.restype = i32
    lib.spec_verify_hier.argtypes = [ctypes.POINTER(Desc), i32, P, P, P, P, P, P, P, P, P, P, P,
                                     P, P, sz, ctypes.POINTER(Diag), P]
    lib.spec_verify_hier_rollback.restype = i32
    lib.spec_verify_hier_rollback.argtypes = [ctypes.POINTER(Desc), i32, P, P, P, P, P, P, P, P,
                                              P, P, i32, i32, P, P, P, i32, P, P, sz,
                                              ctypes.POINTER(Diag), P]
    lib.spec_verify_hier_rollback_lazy.restype = i32
    lib.spec_verify_hier_rollback_lazy.argtypes = lib.spec_verify_hier_rollback.argtypes
    lib.spec_verify_hier_rollback_noalloc.restype = i32
    lib.spec_verify_hier_rollback_noalloc.argtypes = [ctypes.POINTER(Desc), i32, P, P, P, P, P, P,
                                                      P, P, P, P, i32, i32, P, P, P, i32, P,
                                                      ctypes.POINTER(Diag), P]
    lib.kv_blocktable_truncate.restype = i32
    lib.kv_blocktable_truncate.argtypes = [i32, i32, i32, P, P, P, P, i32, P, P]
    lib.spec_verify_device_status.restype = i32
    lib.spec_verify_device_status.argtypes = [P, ctypes.POINTER(u32), P]
    lib.spec_verify_lmhead_workspace_bytes.restype = sz
    lib.spec_verify_lmhead_workspace_bytes.argtypes = [ctypes.POINTER(Desc), i32]
    lib.spec_verify_lmhead_single.restype = i32
    lib.spec_verify_lmhead_single.argtypes = [ctypes.POINTER(Desc), i32, P, P, P, P, P, P, P, P,
                                              P, P, P, P, sz, ctypes.POINTER(Diag), P]
    lib.spec_verify_tentative_workspace_bytes.restype = sz
    lib.spec_verify_tentative_workspace_bytes.argtypes = [ctypes.POINTER(Desc), i32]
    lib.spec_verify_tentative_round.restype = i32
    lib.spec_verify_tentative_round.argtypes = [ctypes.POINTER(Desc), P, P, P, P, P,
                                                ctypes.POINTER(Pending), P, P, P, sz, P]
    lib.spec_verify_tentative_flush.restype = i32
    lib.spec_verify_tentative_flush.argtypes = [ctypes.POINTER(Desc), P, P, i32,
                                                ctypes.POINTER(Pending), P, P, P, P, P, sz, P]
    return lib


def _check(status):
    if status != SV_OK:
        lib = library()
        raise SpecVerifyError(status, lib.spec_verify_status_string(status).decode() + ": " +
                              lib.spec_verify_last_error().decode())


def abi_version():
    return int(library().spec_verify_abi_version())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return SV_DTYPE_BF16
    if t.dtype == torch.float32:
        return SV_DTYPE_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def make_desc(batch, num_draft, vocab, dtype_code, row_stride=0, seed=0, offset=0):
    return Desc(batch, num_draft, vocab, dtype_code, row_stride, seed & (2 ** 64 - 1),
                offset & 0xFFFFFFFF, 0)


def workspace_bytes(batch, num_draft, vocab, dtype, num_exits, row_stride=0):
    """Workspace bytes for a call (dtype: torch dtype or SV_DTYPE_* code)."""
    code = dtype if isinstance(dtype, int) else (SV_DTYPE_BF16 if dtype == torch.bfloat16
                                                 else SV_DTYPE_F32)
    d = make_desc(batch, num_draft, vocab, code, row_stride)
    return int(library().spec_verify_workspace_bytes(ctypes.byref(d), num_exits))


def validate(desc, num_exits, window, ws_bytes):
    """Host-side validation status (SV_*) of a descriptor, without a GPU."""
    return int(library().spec_verify_validate(ctypes.byref(desc), num_exits, window, ws_bytes))


def alloc_workspace(nbytes, device):
    """A 256-byte aligned device buffer of at least ``nbytes`` (uint8 tensor)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _logits(t, name, B, P, dtype):
    """Checks one exit tensor [B, P, V]; returns its row stride in elements, or
    None when a single row leaves it undetermined."""
    if t.dim() != 3 or t.shape[0] != B or t.shape[1] != P:
        raise ValueError(f"{name} must have shape [{B}, {P}, V], got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.shape[2] > 1 and t.stride(2) != 1:
        raise ValueError(f"{name} must be contiguous along the vocabulary")
    ld = None
    if P > 1:
        ld = t.stride(1)
        if B > 1 and t.stride(0) != P * ld:
            raise ValueError(f"{name} rows must be evenly strided")
    elif P == 1 and B > 1:
        ld = t.stride(0)
    return ld


def _common_stride(strides, V):
    known = {s for s in strides if s is not None}
    if len(known) > 1:
        raise ValueError("all exits must share one row stride")
    return known.pop() if known else V


def _int_out(shape, device):
    return torch.empty(shape, dtype=torch.int32, device=device)


def _diag_buffers(B, k, device):
    return dict(uniforms=torch.empty((B, 2, k + 1, 2), dtype=torch.float32, device=device),
                probs=torch.empty((B, 2, k + 1, 2), dtype=torch.float64, device=device),
                draws=torch.empty((B, 2, 4), dtype=torch.float64, device=device))


def _make_diag(diag, events, B, k, dev, out, rows=0, entropy=False, outcome=False, top_m=0,
               row_stats=False):
    """Diag struct: export buffers when ``diag``; ``events`` = (begin, end)
    hipEvent_t handles (ints) that take the row-statistics kernel's start and
    end times; by-product outputs when ``entropy`` (out["entropy"], one float
    per row of every exit) or ``outcome`` (out["accept_mass"] [B, 2, k+1] and,
    for top_m > 0, out["residual_tokens"] / out["residual_mass"]
    [B, 2, k+1, top_m]); every row's merged statistics when ``row_stats``
    (out["row_log2z"] float64 and out["row_argmax"] int32, one per row)."""
    if not diag and events is None and not entropy and not outcome and not row_stats:
        return None
    dg = Diag()
    if diag:
        bufs = _diag_buffers(B, k, dev)
        out.update({"diag_" + n: v for n, v in bufs.items()})
        dg.uniforms, dg.probs, dg.draws = (bufs["uniforms"].data_ptr(), bufs["probs"].data_ptr(),
                                           bufs["draws"].data_ptr())
    if events is not None:
        dg.stats_begin, dg.stats_end = events
    if entropy:
        out["entropy"] = torch.empty((max(1, rows),), dtype=torch.float32, device=dev)
        dg.entropy = out["entropy"].data_ptr()
    if outcome:
        out["accept_mass"] = torch.empty((B, 2, k + 1), dtype=torch.float32, device=dev)
        dg.accept_mass = out["accept_mass"].data_ptr()
        if top_m:
            out["residual_tokens"] = torch.empty((B, 2, k + 1, top_m), dtype=torch.int32,
                                                 device=dev)
            out["residual_mass"] = torch.empty((B, 2, k + 1, top_m), dtype=torch.float32,
                                               device=dev)
            dg.residual_tokens = out["residual_tokens"].data_ptr()
            dg.residual_mass = out["residual_mass"].data_ptr()
            dg.top_m = int(top_m)
    if row_stats:
        out["row_log2z"] = torch.empty((max(1, rows),), dtype=torch.float64, device=dev)
        out["row_argmax"] = torch.empty((max(1, rows),), dtype=torch.int32, device=dev)
        dg.row_log2z = out["row_log2z"].data_ptr()
        dg.row_argmax = out["row_argmax"].data_ptr()
    return dg


def _prep_common(draft_tokens, temperature, B, k, device):
    if draft_tokens.dtype != torch.int32 or draft_tokens.shape != (B, k) or \
            not draft_tokens.is_contiguous() or draft_tokens.device != device:
        raise ValueError("draft_tokens must be a contiguous int32 [B, k] tensor on the logits' device")
    if temperature is not None:
        if temperature.dtype != torch.float32 or temperature.shape != (B,) or \
                not temperature.is_contiguous() or temperature.device != device:
            raise ValueError("temperature must be a contiguous float32 [B] tensor on the logits' device")


def spec_verify_single(draft_logits, target_logits, draft_tokens, temperature=None, *, seed=0,
                       offset=0, packed=False, diag=False, workspace=None, events=None,
                       entropy=False, outcome=False, top_m=0, row_stats=False):
    """Single-stage verify (standard rule).  Returns a dict of device tensors:
    accept_len, out_tokens [B, k+1] (-1 padded), num_emitted, num_drop, and
    packed_tokens / cu_offsets, diag buffers and by-products (``entropy``,
    ``outcome`` with ``top_m``, see ``_make_diag``) when asked.  Asynchronous."""
    lib = library()
    B, k, V = draft_logits.shape
    dev = draft_logits.device
    code = _dtype_code(draft_logits)
    ld_q = _logits(draft_logits, "draft_logits", B, k, draft_logits.dtype)
    ld_p = _logits(target_logits, "target_logits", B, k + 1, draft_logits.dtype)
    if target_logits.shape[2] != V:
        raise ValueError("draft and target vocabularies differ")
    _prep_common(draft_tokens, temperature, B, k, dev)
    desc = make_desc(B, k, V, code, _common_stride([ld_q, ld_p], V), seed, offset)
    need = lib.spec_verify_workspace_bytes(ctypes.byref(desc), 2)
    ws = workspace if workspace is not None else alloc_workspace(need, dev)
    out = dict(accept_len=_int_out((B,), dev), out_tokens=_int_out((B, k + 1), dev),
               num_emitted=_int_out((B,), dev), num_drop=_int_out((B,), dev), workspace=ws)
    if packed:
        out["packed_tokens"] = _int_out((max(1, B * (k + 1)),), dev)
        out["cu_offsets"] = _int_out((B + 1,), dev)
    dg = _make_diag(diag, events, B, k, dev, out, B * (2 * k + 1), entropy, outcome, top_m,
                    row_stats)
    _check(lib.spec_verify_single(
        ctypes.byref(desc), _ptr(draft_logits), _ptr(target_logits), _ptr(draft_tokens),
        _ptr(temperature), _ptr(out["accept_len"]), _ptr(out["out_tokens"]),
        _ptr(out["num_emitted"]), _ptr(out["num_drop"]), _ptr(out.get("packed_tokens")),
        _ptr(out.get("cu_offsets")), _ptr(ws), ws.numel(),
        ctypes.byref(dg) if dg is not None else None, _stream(dev)))
    return out


def lmhead_workspace_bytes(batch, num_draft, vocab, hidden, row_stride=0):
    desc = make_desc(batch, num_draft, vocab, SV_DTYPE_BF16, row_stride)
    return library().spec_verify_lmhead_workspace_bytes(ctypes.byref(desc), hidden)


def _bf16_rows(t, name, shape, device):
    if t.dtype != torch.bfloat16 or tuple(t.shape) != shape or not t.is_contiguous() or \
            t.device != device:
        raise ValueError(f"{name} must be a contiguous bf16 {list(shape)} tensor on one device")


def spec_verify_lmhead_single(h_draft, h_target, w_vocab, draft_tokens, temperature=None, *,
                              seed=0, offset=0, packed=False, diag=False, workspace=None,
                              events=None, out=None, entropy=False, outcome=False, top_m=0,
                              row_stats=False):
    """Single-stage verify through a linear LM head W [V, d] (one d-vector per
    vocabulary entry): q from h_draft [B, k, d], p from h_target [B, k+1, d].
    Returns the same dict as spec_verify_single.  ``out`` reuses the output
    tensors of an earlier call with the same shapes.  Asynchronous."""
    lib = library()
    B, k1, d = h_target.shape
    k = k1 - 1
    V = w_vocab.shape[0]
    dev = h_target.device
    _bf16_rows(h_target, "h_target", (B, k + 1, d), dev)
    _bf16_rows(h_draft, "h_draft", (B, k, d), dev)
    if w_vocab.dim() != 2 or w_vocab.shape[1] != d or w_vocab.dtype != torch.bfloat16 or \
            w_vocab.stride(1) != 1 or w_vocab.device != dev:
        raise ValueError("w_vocab must be a bf16 [V, d] tensor, contiguous along d")
    _prep_common(draft_tokens, temperature, B, k, dev)
    desc = make_desc(B, k, V, SV_DTYPE_BF16, w_vocab.stride(0) if V > 1 else d, seed, offset)
    need = lib.spec_verify_lmhead_workspace_bytes(ctypes.byref(desc), d)
    if need == 0:
        raise SpecVerifyError(SV_ERR_UNSUPPORTED, "unsupported LM-head shape")
    ws = workspace if workspace is not None else alloc_workspace(need, dev)
    if out is None:
        out = dict(accept_len=_int_out((B,), dev), out_tokens=_int_out((B, k + 1), dev),
                   num_emitted=_int_out((B,), dev), num_drop=_int_out((B,), dev))
        if packed:
            out["packed_tokens"] = _int_out((max(1, B * (k + 1)),), dev)
            out["cu_offsets"] = _int_out((B + 1,), dev)
    out["workspace"] = ws
    dg = _make_diag(diag, events, B, k, dev, out, B * (2 * k + 1), entropy, outcome, top_m,
                    row_stats)
    _check(lib.spec_verify_lmhead_single(
        ctypes.byref(desc), d, _ptr(h_draft), _ptr(h_target), _ptr(w_vocab),
        _ptr(draft_tokens), _ptr(temperature), _ptr(out["accept_len"]), _ptr(out["out_tokens"]),
        _ptr(out["num_emitted"]), _ptr(out["num_drop"]), _ptr(out.get("packed_tokens")),
        _ptr(out.get("cu_offsets")), _ptr(ws), ws.numel(),
        ctypes.byref(dg) if dg is not None else None, _stream(dev)))
    return out


def spec_verify_hier(ld_logits, li_logits, lf_logits, draft_tokens, temperature=None, *,
                     window=4, seed=0, offset=0, packed=False, diag=False, workspace=None,
                     events=None, entropy=False, outcome=False, top_m=0, row_stats=False):
    """HiSpec two-stage verify L_d -> L_i -> L_f.  Returns a dict of device
    tensors: accept_len_inter (a1), accept_len_final (a2), out_tokens,
    num_emitted, num_drop (+ packed / diag on request).  Asynchronous."""
    lib = library()
    B, k, V = ld_logits.shape
    dev = ld_logits.device
    code = _dtype_code(ld_logits)
    s0 = _logits(ld_logits, "ld_logits", B, k, ld_logits.dtype)
    s1 = _logits(li_logits, "li_logits", B, k + 1, ld_logits.dtype)
    s2 = _logits(lf_logits, "lf_logits", B, k + 1, ld_logits.dtype)
    if li_logits.shape[2] != V or lf_logits.shape[2] != V:
        raise ValueError("exit vocabularies differ")
    _prep_common(draft_tokens, temperature, B, k, dev)
    desc = make_desc(B, k, V, code, _common_stride([s0, s1, s2], V), seed, offset)
    need = lib.spec_verify_workspace_bytes(ctypes.byref(desc), 3)
    ws = workspace if workspace is not None else alloc_workspace(need, dev)
    out = dict(accept_len_inter=_int_out((B,), dev), accept_len_final=_int_out((B,), dev),
               out_tokens=_int_out((B, k + 1), dev), num_emitted=_int_out((B,), dev),
               num_drop=_int_out((B,), dev), workspace=ws)
    if packed:
        out["packed_tokens"] = _int_out((max(1, B * (k + 1)),), dev)
        out["cu_offsets"] = _int_out((B + 1,), dev)
    dg = _make_diag(diag, events, B, k, dev, out, B * (3 * k + 2), entropy, outcome, top_m,
                    row_stats)
    _check(lib.spec_verify_hier(
        ctypes.byref(desc), int(window), _ptr(ld_logits), _ptr(li_logits), _ptr(lf_logits),
        _ptr(draft_tokens), _ptr(temperature), _ptr(out["accept_len_inter"]),
        _ptr(out["accept_len_final"]), _ptr(out["out_tokens"]), _ptr(out["num_emitted"]),
        _ptr(out["num_drop"]), _ptr(out.get("packed_tokens")), _ptr(out.get("cu_offsets")),
        _ptr(ws), ws.numel(), ctypes.byref(dg) if dg is not None else None, _stream(dev)))
    return out


def spec_verify_hier_rollback(ld_logits, li_logits, lf_logits, draft_tokens, temperature,
                              block_table, seq_lens, *, block_size, max_freed, window=4,
                              seed=0, offset=0, diag=False, workspace=None, events=None,
                              out=None, entropy=False, outcome=False, top_m=0, row_stats=False,
                              _lazy=False, _noalloc=False):
    """spec_verify_hier plus the paged-KV rollback of block_table / seq_lens
    (in place) in the same launches.  Returns the spec_verify_hier dict plus
    freed_blocks [B, max_freed] and num_freed [B].  ``out``: a dict returned
    by an earlier call of the same shape, whose buffers are reused.
    Asynchronous."""
    lib = library()
    B, k, V = ld_logits.shape
    dev = ld_logits.device
    code = _dtype_code(ld_logits)
    s0 = _logits(ld_logits, "ld_logits", B, k, ld_logits.dtype)
    s1 = _logits(li_logits, "li_logits", B, k + 1, ld_logits.dtype)
    s2 = _logits(lf_logits, "lf_logits", B, k + 1, ld_logits.dtype)
    if li_logits.shape[2] != V or lf_logits.shape[2] != V:
        raise ValueError("exit vocabularies differ")
    _prep_common(draft_tokens, temperature, B, k, dev)
    max_blocks = block_table.shape[1]
    for name, t, shape in (("block_table", block_table, (B, max_blocks)),
                           ("seq_lens", seq_lens, (B,))):
        if t.dtype != torch.int32 or tuple(t.shape) != shape or not t.is_contiguous() or \
                t.device != dev:
            raise ValueError(f"{name} must be a contiguous int32 {shape} device tensor")
    desc = make_desc(B, k, V, code, _common_stride([s0, s1, s2], V), seed, offset)
    need = lib.spec_verify_workspace_bytes(ctypes.byref(desc), 3)
    if out is None:
        ws = None if _noalloc else (workspace if workspace is not None
                                    else alloc_workspace(need, dev))
        out = dict(accept_len_inter=_int_out((B,), dev), accept_len_final=_int_out((B,), dev),
                   out_tokens=_int_out((B, k + 1), dev), num_emitted=_int_out((B,), dev),
                   num_drop=_int_out((B,), dev), freed_blocks=_int_out((B, max_freed), dev),
                   num_freed=_int_out((B,), dev), workspace=ws)
    else:
        ws = out.get("workspace")
        if tuple(out["out_tokens"].shape) != (B, k + 1) or \
                tuple(out["freed_blocks"].shape) != (B, max_freed):
            raise ValueError("out buffers do not match this call's shapes")
    dg = _make_diag(diag, events, B, k, dev, out, B * (3 * k + 2), entropy, outcome, top_m,
                    row_stats)
    if _noalloc:
        _check(lib.spec_verify_hier_rollback_noalloc(
            ctypes.byref(desc), int(window), _ptr(ld_logits), _ptr(li_logits), _ptr(lf_logits),
            _ptr(draft_tokens), _ptr(temperature), _ptr(out["accept_len_inter"]),
            _ptr(out["accept_len_final"]), _ptr(out["out_tokens"]), _ptr(out["num_emitted"]),
            _ptr(out["num_drop"]), int(max_blocks), int(block_size), _ptr(block_table),
            _ptr(seq_lens), _ptr(out["freed_blocks"]) if max_freed > 0 else None,
            int(max_freed), _ptr(out["num_freed"]),
            ctypes.byref(dg) if dg is not None else None, _stream(dev)))
        return out
    fn = lib.spec_verify_hier_rollback_lazy if _lazy else lib.spec_verify_hier_rollback
    _check(fn(
        ctypes.byref(desc), int(window), _ptr(ld_logits), _ptr(li_logits), _ptr(lf_logits),
        _ptr(draft_tokens), _ptr(temperature), _ptr(out["accept_len_inter"]),
        _ptr(out["accept_len_final"]), _ptr(out["out_tokens"]), _ptr(out["num_emitted"]),
        _ptr(out["num_drop"]), int(max_blocks), int(block_size), _ptr(block_table),
        _ptr(seq_lens), _ptr(out["freed_blocks"]) if max_freed > 0 else None, int(max_freed),
        _ptr(out["num_freed"]), _ptr(ws), ws.numel(),
        ctypes.byref(dg) if dg is not None else None, _stream(dev)))
    return out


def spec_verify_hier_rollback_lazy(ld_logits, li_logits, lf_logits, draft_tokens, temperature,
                                   block_table, seq_lens, **kw):
    """spec_verify_hier_rollback reading only the L_f rows stage 2 can reach
    (rows 0..a1 of each sequence); bit-identical results."""
    return spec_verify_hier_rollback(ld_logits, li_logits, lf_logits, draft_tokens, temperature,
                                     block_table, seq_lens, _lazy=True, **kw)


def spec_verify_hier_rollback_noalloc(ld_logits, li_logits, lf_logits, draft_tokens,
                                      temperature, block_table, seq_lens, **kw):
    """spec_verify_hier_rollback whose workspace is the library's static
    per-GPU scratch (the C call allocates nothing; calls that overlap on one
    GPU race).  Takes no ``workspace``; the returned dict has workspace None."""
    if kw.get("workspace") is not None:
        raise ValueError("the no-allocation call takes no workspace")
    kw.pop("workspace", None)
    return spec_verify_hier_rollback(ld_logits, li_logits, lf_logits, draft_tokens, temperature,
                                     block_table, seq_lens, _noalloc=True, **kw)


def kv_blocktable_truncate(block_table, seq_lens, num_drop, block_size, max_freed):
    """Roll back paged-KV state in place (block_table, seq_lens) and return
    (freed_blocks [B, max_freed], num_freed [B]).  Asynchronous."""
    lib = library()
    B, max_blocks = block_table.shape
    dev = block_table.device
    for name, t, shape in (("block_table", block_table, (B, max_blocks)),
                           ("seq_lens", seq_lens, (B,)), ("num_drop", num_drop, (B,))):
        if t.dtype != torch.int32 or tuple(t.shape) != shape or not t.is_contiguous() or \
                t.device != dev:
            raise ValueError(f"{name} must be a contiguous int32 {shape} device tensor")
    freed = _int_out((B, max_freed), dev)
    num_freed = _int_out((B,), dev)
    _check(lib.kv_blocktable_truncate(B, max_blocks, int(block_size), _ptr(block_table),
                                      _ptr(seq_lens), _ptr(num_drop),
                                      _ptr(freed) if max_freed > 0 else None, int(max_freed),
                                      _ptr(num_freed), _stream(dev)))
    return freed, num_freed


def device_status(workspace):
    """Synchronises and returns the SV_FLAG_* bits of the last call on ``workspace``."""
    lib = library()
    flags = ctypes.c_uint32(0)
    _check(lib.spec_verify_device_status(_ptr(workspace), ctypes.byref(flags),
                                         _stream(workspace.device)))
    return int(flags.value)


# --- cross-call tentative buffering ------------------------------------------

def tentative_workspace_bytes(batch, num_draft, vocab, dtype, capacity, row_stride=0):
    """Workspace bytes of the tentative round and flush calls."""
    code = dtype if isinstance(dtype, int) else (SV_DTYPE_BF16 if dtype == torch.bfloat16
                                                 else SV_DTYPE_F32)
    d = make_desc(batch, num_draft, vocab, code, row_stride)
    return int(library().spec_verify_tentative_workspace_bytes(ctypes.byref(d), int(capacity)))


def make_pending(batch, capacity, vocab, dtype, device, row_stride=None):
    """A zeroed pending state: count [B], tokens [B, capacity] int32 and the
    pending L_i rows [B, capacity, row_stride] of ``dtype``."""
    ld = vocab if row_stride is None else row_stride
    return dict(count=torch.zeros((batch,), dtype=torch.int32, device=device),
                tokens=torch.full((batch, capacity), -1, dtype=torch.int32, device=device),
                rows=torch.zeros((batch, capacity, ld), dtype=dtype, device=device),
                capacity=int(capacity))


def _pending_struct(pending, B):
    for name in ("count", "tokens", "rows"):
        t = pending[name]
        if not t.is_contiguous() or t.shape[0] != B:
            raise ValueError(f"pending[{name!r}] must be contiguous with {B} sequences")
    return Pending(pending["count"].data_ptr(), pending["tokens"].data_ptr(),
                   pending["rows"].data_ptr(), int(pending["capacity"]))


def spec_verify_tentative_round(ld_logits, li_logits, draft_tokens, temperature, pending, *,
                                active=None, seed=0, offset=0, workspace=None):
    """One intermediate verification round (stage 1, L_d -> L_i); every active
    sequence's output and L_i rows are appended to ``pending`` (in place).
    Returns dict(accept_len [B], num_drop [B], workspace).  Asynchronous."""
    lib = library()
    B, k, V = ld_logits.shape
    dev = ld_logits.device
    code = _dtype_code(ld_logits)
    s0 = _logits(ld_logits, "ld_logits", B, k, ld_logits.dtype)
    s1 = _logits(li_logits, "li_logits", B, k + 1, ld_logits.dtype)
    if li_logits.shape[2] != V:
        raise ValueError("exit vocabularies differ")
    _prep_common(draft_tokens, temperature, B, k, dev)
    rows = pending["rows"]
    if rows.dtype != ld_logits.dtype or rows.dim() != 3 or rows.shape[1] != pending["capacity"]:
        raise ValueError("pending rows must be [B, capacity, row_stride] of the logits' dtype")
    ld = _common_stride([s0, s1, rows.shape[2]], V)
    if active is not None and (active.dtype != torch.int32 or tuple(active.shape) != (B,)):
        raise ValueError("active must be an int32 [B] device tensor")
    desc = make_desc(B, k, V, code, ld, seed, offset)
    need = lib.spec_verify_tentative_workspace_bytes(ctypes.byref(desc), int(pending["capacity"]))
    ws = workspace if workspace is not None else alloc_workspace(need, dev)
    out = dict(accept_len=_int_out((B,), dev), num_drop=_int_out((B,), dev), workspace=ws)
    pd = _pending_struct(pending, B)
    _check(lib.spec_verify_tentative_round(
        ctypes.byref(desc), _ptr(ld_logits), _ptr(li_logits), _ptr(draft_tokens),
        _ptr(temperature), _ptr(active), ctypes.byref(pd), _ptr(out["accept_len"]),
        _ptr(out["num_drop"]), _ptr(ws), ws.numel(), _stream(dev)))
    return out


def spec_verify_tentative_flush(lf_logits, temperature, pending, *, min_pending, seed=0,
                                offset=0, workspace=None):
    """Verify the pending tokens of every sequence holding at least
    max(1, min_pending) of them against the final exit (lf_logits
    [B, capacity+1, V]); the flushed sequences' counts become 0.  Returns
    dict(accept_len (a2, -1 if not flushed), out_tokens [B, capacity+1],
    num_emitted, num_drop, workspace).  Asynchronous."""
    lib = library()
    cap = int(pending["capacity"])
    B, P, V = lf_logits.shape
    dev = lf_logits.device
    code = _dtype_code(lf_logits)
    s = _logits(lf_logits, "lf_logits", B, cap + 1, lf_logits.dtype)
    rows = pending["rows"]
    if rows.dtype != lf_logits.dtype:
        raise ValueError("pending rows and lf_logits differ in dtype")
    if temperature is not None and (temperature.dtype != torch.float32 or
                                    tuple(temperature.shape) != (B,) or
                                    not temperature.is_contiguous() or temperature.device != dev):
        raise ValueError("temperature must be a contiguous float32 [B] tensor on the logits' device")
    ld = _common_stride([s, rows.shape[2]], V)
    desc = make_desc(B, 1, V, code, ld, seed, offset)
    need = lib.spec_verify_tentative_workspace_bytes(ctypes.byref(desc), cap)
    ws = workspace if workspace is not None else alloc_workspace(need, dev)
    out = dict(accept_len=_int_out((B,), dev), out_tokens=_int_out((B, cap + 1), dev),
               num_emitted=_int_out((B,), dev), num_drop=_int_out((B,), dev), workspace=ws)
    pd = _pending_struct(pending, B)
    _check(lib.spec_verify_tentative_flush(
        ctypes.byref(desc), _ptr(lf_logits), _ptr(temperature), int(min_pending),
        ctypes.byref(pd), _ptr(out["accept_len"]), _ptr(out["out_tokens"]),
        _ptr(out["num_emitted"]), _ptr(out["num_drop"]), _ptr(ws), ws.numel(), _stream(dev)))
    return out
