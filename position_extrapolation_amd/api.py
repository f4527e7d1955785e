"""Thin Python binding of libdca (include/dca.h): argument marshalling only.

Every function named dca_* calls the C entry point of the same name through
ctypes; torch is used for device memory and the current HIP stream. The
library must be built (python -m position_extrapolation_amd.build); there is
no fallback path -- a missing library raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# DCA_LIBRARY names another build of the same library (the host-only
# sanitizer build the CPU tests make); the default is the in-tree libdca.so
LIB_PATH = os.environ.get("DCA_LIBRARY") or os.path.join(_PKG, "libdca.so")

DCA_OK, DCA_E_INVALID, DCA_E_UNSUPPORTED, DCA_E_WORKSPACE, DCA_E_DEVICE = range(5)
DCA_F32, DCA_BF16 = 0, 1

EXPORTS = [
    "dca_status_str", "dca_last_error", "dca_remap_positions", "dca_workspace_size",
    "dca_prefill", "dca_remap", "dca_vs_index", "dca_attention",
    "dca_chunk_workspace_size", "dca_prefill_chunk", "dca_decode", "dca_decode_static", "dca_fused_workspace_size",
    "dca_prefill_fused", "dca_vs_estimate_workspace_size", "dca_vs_estimate",
    "dca_debug_positions", "dca_debug_tile_regions", "dca_debug_unpack", "dca_debug_vs_lists",
    "dca_debug_vs_tiles",
]


class DcaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class dca_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class dca_vs_mask(ctypes.Structure):
    _fields_ = [("vertical", ctypes.c_void_p), ("slash", ctypes.c_void_p),
                ("n_vertical", ctypes.c_int32), ("n_slash", ctypes.c_int32)]


_lib = None

_I64, _I32P, _VP = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p
_SIGS = {
    "dca_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "dca_last_error": (ctypes.c_char_p, []),
    "dca_remap_positions": (ctypes.c_int, [_I64, _I64, _I64, _VP, _VP, _VP, _VP]),
    "dca_workspace_size": (ctypes.c_int, [_I64, _I64, _I64, _VP, _VP, ctypes.POINTER(ctypes.c_size_t)]),
    "dca_prefill": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, ctypes.c_double,
                                   ctypes.c_float, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    "dca_remap": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I64, _I64, ctypes.c_double, ctypes.c_float, _VP, _VP,
                                 ctypes.c_size_t, _VP]),
    "dca_vs_index": (ctypes.c_int, [_I64, _I64, _I64, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    "dca_chunk_workspace_size": (ctypes.c_int, [_I64, _I64, _I64, _I64, _VP, _VP, ctypes.POINTER(ctypes.c_size_t)]),
    "dca_prefill_chunk": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, _I64, ctypes.c_double,
                                         ctypes.c_float, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    "dca_fused_workspace_size": (ctypes.c_int, [_I64, _I64, _I64, _VP, _VP, ctypes.POINTER(ctypes.c_size_t)]),
    "dca_prefill_fused": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, ctypes.c_double,
                                         ctypes.c_float, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    "dca_vs_estimate_workspace_size": (ctypes.c_int, [_I64, _VP, ctypes.POINTER(ctypes.c_size_t)]),
    "dca_vs_estimate": (ctypes.c_int, [_VP, _VP, _I64, ctypes.c_int32, ctypes.c_double, ctypes.c_float,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP,
                                       _VP, ctypes.c_size_t, _VP]),
    "dca_decode": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, ctypes.c_double, ctypes.c_float,
                                  _VP, _VP, ctypes.c_size_t, _VP]),
    "dca_decode_static": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _I64, ctypes.c_double,
                                         ctypes.c_float, _VP, _VP, ctypes.c_size_t, _VP]),
    "dca_attention": (ctypes.c_int, [_VP, _VP, _I64, _I64, _I64, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    "dca_debug_positions": (ctypes.c_int, [_I64, _I64, _I64, _VP, _VP, _VP, _VP, _VP]),
    "dca_debug_tile_regions": (ctypes.c_int, [_I64, _I64, _VP, _VP]),
    "dca_debug_unpack": (ctypes.c_int, [_VP, ctypes.c_size_t, ctypes.c_int, _I64, _I64, _I64, _VP, _VP, _VP]),
    "dca_debug_vs_lists": (ctypes.c_int, [_VP, ctypes.c_size_t, _I64, _I64, _I64, _VP, _VP, _VP, _VP,
                                          _VP, _VP, _VP]),
    "dca_debug_vs_tiles": (ctypes.c_int, [_VP, ctypes.c_size_t, _I64, _I64, _I64, _VP, _VP, ctypes.c_int32,
                                          _I64, ctypes.c_int32, _VP, _VP, ctypes.c_int32, _VP, _VP]),
}


def lib():
    """Load libdca.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m position_extrapolation_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def dca_status_str(status: int) -> str:
    return lib().dca_status_str(status).decode()


def dca_last_error() -> str:
    return lib().dca_last_error().decode()


def _check(status: int, where: str):
    if status != DCA_OK:
        raise DcaError(status, where, f"{dca_status_str(status)}: {dca_last_error()}")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def make_shape(batch, n_q_heads, n_kv_heads, head_dim, dtype, softmax_scale=0.0) -> dca_shape:
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: DCA_F32, torch.bfloat16: DCA_BF16}[dtype]
    return dca_shape(batch, n_q_heads, n_kv_heads, head_dim, dtype, softmax_scale)


def shape_of(q: torch.Tensor, k: torch.Tensor, softmax_scale: float = 0.0) -> dca_shape:
    return make_shape(q.shape[0], q.shape[1], k.shape[1], q.shape[3], q.dtype, softmax_scale)


def _check_list(t: torch.Tensor, name: str, n_q_heads: int | None):
    """The library reads n_q_heads x n entries of a mask list from device
    memory at h * n + e: anything but a contiguous 2-D int32 device tensor of
    that many rows would be read wrongly or past its end."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32 (got {t.dtype})")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dim() != 2 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [n_q_heads, n] tensor (got shape {tuple(t.shape)})")
    if n_q_heads is not None and t.shape[0] != n_q_heads:
        raise ValueError(f"{name} has {t.shape[0]} rows, the queries have {n_q_heads} heads")


def make_mask(vertical: torch.Tensor | None, slash: torch.Tensor | None,
              n_q_heads: int | None = None) -> dca_vs_mask | None:
    """vertical [Hq, nv], slash [Hq, ns]: contiguous device int32 tensors (kept
    alive by the caller); n_q_heads, when given, must equal their row count."""
    if vertical is None and slash is None:
        return None
    if vertical is not None:
        _check_list(vertical, "vertical", n_q_heads)
    if slash is not None:
        _check_list(slash, "slash", n_q_heads)
    if vertical is not None and slash is not None and vertical.device != slash.device:
        raise ValueError("vertical and slash must be on one device")
    nv = 0 if vertical is None else vertical.shape[1]
    ns = 0 if slash is None else slash.shape[1]
    return dca_vs_mask(_ptr(vertical), _ptr(slash), nv, ns)


def _ref(x):
    return None if x is None else ctypes.byref(x)


# ---- entry points, same names as include/dca.h ---------------------------

def dca_remap_positions(seq: int, C: int, W: int):
    """Host position map -> (pq_intra, pq_succ, pq_inter, pk) as int32 tensors."""
    pqi = torch.empty(seq, dtype=torch.int32)
    pqs = torch.empty(seq, dtype=torch.int32)
    pk = torch.empty(seq, dtype=torch.int32)
    pinter = torch.empty(1, dtype=torch.int32)
    _check(lib().dca_remap_positions(seq, C, W, _ptr(pqi), _ptr(pqs), _ptr(pinter), _ptr(pk)),
           "dca_remap_positions")
    return pqi, pqs, int(pinter[0]), pk


def dca_workspace_size(seq: int, C: int, W: int, shape: dca_shape, mask: dca_vs_mask | None = None) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dca_workspace_size(seq, C, W, ctypes.byref(shape), _ref(mask), ctypes.byref(n)),
           "dca_workspace_size")
    return n.value


def dca_prefill(q, k, v, out, lse, seq, C, W, rope_base, yarn_scale, mask, shape, workspace,
                workspace_bytes, stream=None):
    _check(lib().dca_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), seq, C, W, rope_base,
                             yarn_scale, _ref(mask), ctypes.byref(shape), _ptr(workspace), workspace_bytes,
                             _stream(stream)), "dca_prefill")


def dca_remap(q, k, v, seq, C, W, rope_base, yarn_scale, shape, workspace, workspace_bytes, stream=None):
    _check(lib().dca_remap(_ptr(q), _ptr(k), _ptr(v), seq, C, W, rope_base, yarn_scale, ctypes.byref(shape),
                           _ptr(workspace), workspace_bytes, _stream(stream)), "dca_remap")


def dca_vs_index(seq, C, W, mask, shape, workspace, workspace_bytes, stream=None):
    _check(lib().dca_vs_index(seq, C, W, _ref(mask), ctypes.byref(shape), _ptr(workspace), workspace_bytes,
                              _stream(stream)), "dca_vs_index")


def dca_attention(out, lse, seq, C, W, mask, shape, workspace, workspace_bytes, stream=None):
    _check(lib().dca_attention(_ptr(out), _ptr(lse), seq, C, W, _ref(mask), ctypes.byref(shape),
                               _ptr(workspace), workspace_bytes, _stream(stream)), "dca_attention")


def dca_chunk_workspace_size(seq: int, max_rows: int, C: int, W: int, shape: dca_shape,
                             mask: dca_vs_mask | None = None) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dca_chunk_workspace_size(seq, max_rows, C, W, ctypes.byref(shape), _ref(mask), ctypes.byref(n)),
           "dca_chunk_workspace_size")
    return n.value


def dca_prefill_chunk(q, k, v, out, lse, q_offset, n_rows, seq, C, W, rope_base, yarn_scale, mask, shape,
                      workspace, workspace_bytes, stream=None):
    _check(lib().dca_prefill_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), q_offset, n_rows, seq, C, W,
                                   rope_base, yarn_scale, _ref(mask), ctypes.byref(shape), _ptr(workspace),
                                   workspace_bytes, _stream(stream)), "dca_prefill_chunk")


def dca_fused_workspace_size(seq: int, C: int, W: int, shape: dca_shape, mask: dca_vs_mask | None = None) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dca_fused_workspace_size(seq, C, W, ctypes.byref(shape), _ref(mask), ctypes.byref(n)),
           "dca_fused_workspace_size")
    return n.value


def dca_prefill_fused(q, k, v, out, lse, seq, C, W, rope_base, yarn_scale, mask, shape, workspace,
                      workspace_bytes, stream=None):
    _check(lib().dca_prefill_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), seq, C, W, rope_base,
                                   yarn_scale, _ref(mask), ctypes.byref(shape), _ptr(workspace), workspace_bytes,
                                   _stream(stream)), "dca_prefill_fused")


def dca_vs_estimate_workspace_size(seq: int, shape: dca_shape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dca_vs_estimate_workspace_size(seq, ctypes.byref(shape), ctypes.byref(n)),
           "dca_vs_estimate_workspace_size")
    return n.value


def dca_vs_estimate(q, k, seq, n_last, rope_base, yarn_scale, n_vertical, n_slash, n_forced, shape, vertical, slash,
                    vertical_score, slash_score, workspace, workspace_bytes, stream=None):
    _check(lib().dca_vs_estimate(_ptr(q), _ptr(k), seq, n_last, rope_base, yarn_scale, n_vertical, n_slash, n_forced,
                                 ctypes.byref(shape), _ptr(vertical), _ptr(slash), _ptr(vertical_score),
                                 _ptr(slash_score), _ptr(workspace), workspace_bytes, _stream(stream)),
           "dca_vs_estimate")


def dca_decode(q, k, v, out, lse, pos, seq, C, W, rope_base, yarn_scale, shape, workspace, workspace_bytes,
               stream=None):
    _check(lib().dca_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), pos, seq, C, W, rope_base, yarn_scale,
                            ctypes.byref(shape), _ptr(workspace), workspace_bytes, _stream(stream)), "dca_decode")


def dca_decode_static(q, k, v, out, lse, pos, seq, C, W, rope_base, yarn_scale, shape, workspace, workspace_bytes,
                      stream=None):
    _check(lib().dca_decode_static(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), pos, seq, C, W, rope_base,
                                   yarn_scale, ctypes.byref(shape), _ptr(workspace), workspace_bytes,
                                   _stream(stream)), "dca_decode_static")


def dca_debug_positions(seq, C, W, pq_intra, pq_succ, pq_inter, pk, stream=None):
    _check(lib().dca_debug_positions(seq, C, W, _ptr(pq_intra), _ptr(pq_succ), _ptr(pq_inter), _ptr(pk),
                                     _stream(stream)), "dca_debug_positions")


def dca_debug_tile_regions(seq, C, out, stream=None):
    _check(lib().dca_debug_tile_regions(seq, C, _ptr(out), _stream(stream)), "dca_debug_tile_regions")


def dca_debug_unpack(workspace, workspace_bytes, which, seq, C, W, shape, dst, stream=None):
    _check(lib().dca_debug_unpack(_ptr(workspace), workspace_bytes, which, seq, C, W, ctypes.byref(shape),
                                  _ptr(dst), _stream(stream)), "dca_debug_unpack")


def dca_debug_vs_lists(workspace, workspace_bytes, seq, C, W, mask, shape, vt, vt_count, dl, dl_count,
                       stream=None):
    _check(lib().dca_debug_vs_lists(_ptr(workspace), workspace_bytes, seq, C, W, _ref(mask), ctypes.byref(shape),
                                    _ptr(vt), _ptr(vt_count), _ptr(dl), _ptr(dl_count), _stream(stream)),
           "dca_debug_vs_lists")


def dca_debug_vs_tiles(workspace, workspace_bytes, seq, C, W, mask, shape, head, q_tile, group, kt_out,
                       mask_out, n_out, stream=None):
    """kt_out / mask_out: int32 tensors of the same length (the cap); n_out: one int32."""
    assert kt_out.numel() == mask_out.numel()
    _check(lib().dca_debug_vs_tiles(_ptr(workspace), workspace_bytes, seq, C, W, _ref(mask), ctypes.byref(shape),
                                    head, q_tile, group, _ptr(kt_out), _ptr(mask_out), kt_out.numel(),
                                    _ptr(n_out), _stream(stream)),
           "dca_debug_vs_tiles")


# ---- convenience --------------------------------------------------------------

def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """A 256-byte aligned device byte buffer of at least nbytes."""
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + nbytes]


def prefill(q, k, v, C: int, W: int, rope_base: float = 1e7, yarn_scale: float = 1.0,
            vertical=None, slash=None, return_lse: bool = False, softmax_scale: float = 0.0,
            workspace: torch.Tensor | None = None, fused: bool = False):
    """DCA prefill on torch device tensors q [B, Hq, S, d], k and v [B, Hkv, S, d]
    (contiguous, one dtype); optional vertical [Hq, nv] / slash [Hq, ns] int32
    device tensors. Returns out (and lse) allocated with torch; the call is
    enqueued on the current stream. fused=True rotates the queries inside the
    attention kernel (dca_prefill_fused; smaller workspace, same results)."""
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k and v must be contiguous")
    seq = q.shape[2]
    shape = shape_of(q, k, softmax_scale)
    mask = make_mask(vertical, slash, q.shape[1])
    size = dca_fused_workspace_size if fused else dca_workspace_size
    nbytes = size(seq, C, W, shape, mask)
    if workspace is None or workspace.numel() < nbytes:
        workspace = alloc_workspace(nbytes, q.device)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    run = dca_prefill_fused if fused else dca_prefill
    run(q, k, v, out, lse, seq, C, W, rope_base, yarn_scale, mask, shape, workspace, workspace.numel())
    return (out, lse) if return_lse else out


def prefill_chunked(q, k, v, C: int, W: int, chunk: int, rope_base: float = 1e7, yarn_scale: float = 1.0,
                    vertical=None, slash=None, return_lse: bool = False, softmax_scale: float = 0.0):
    """Chunked DCA prefill: the same result as prefill(), computed by
    dca_prefill_chunk over blocks of `chunk` rows (a multiple of 64) on one
    workspace sized for the whole sequence's keys and one block's queries."""
    if chunk < 64 or chunk % 64 != 0:
        raise ValueError("chunk must be a positive multiple of 64")
    seq = q.shape[2]
    shape = shape_of(q, k, softmax_scale)
    mask = make_mask(vertical, slash, q.shape[1])
    nbytes = dca_chunk_workspace_size(seq, min(chunk, seq), C, W, shape, mask)
    workspace = alloc_workspace(nbytes, q.device)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    for q0 in range(0, seq, chunk):
        n = min(chunk, seq - q0)
        qc = q[:, :, q0:q0 + n].contiguous()
        kc = k[:, :, q0:q0 + n].contiguous()
        vc = v[:, :, q0:q0 + n].contiguous()
        oc = torch.empty_like(qc)
        lc = torch.empty(qc.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
        dca_prefill_chunk(qc, kc, vc, oc, lc, q0, n, seq, C, W, rope_base, yarn_scale, mask, shape, workspace,
                          workspace.numel())
        out[:, :, q0:q0 + n] = oc
        if return_lse:
            lse[:, :, q0:q0 + n] = lc
    return (out, lse) if return_lse else out


def vs_estimate(q, k, n_vertical: int, n_slash: int, n_forced: int = 64, n_last: int = 64, rope_base: float = 1e7,
                yarn_scale: float = 1.0, softmax_scale: float = 0.0, return_scores: bool = False):
    """Per-head vertical columns [Hq, n_vertical] and slash offsets [Hq, n_slash]
    (int32, ascending, device) from the last n_last query rows under
    continuous positions (dca_vs_estimate); batch 1."""
    seq = q.shape[2]
    shape = shape_of(q, k, softmax_scale)
    nbytes = dca_vs_estimate_workspace_size(seq, shape)
    ws = alloc_workspace(nbytes, q.device)
    hq = q.shape[1]
    vert = torch.empty((hq, n_vertical), dtype=torch.int32, device=q.device)
    slash = torch.empty((hq, n_slash), dtype=torch.int32, device=q.device)
    vs = torch.empty((hq, seq), dtype=torch.float32, device=q.device) if return_scores else None
    ss = torch.empty((hq, seq), dtype=torch.float32, device=q.device) if return_scores else None
    dca_vs_estimate(q, k, seq, n_last, rope_base, yarn_scale, n_vertical, n_slash, n_forced, shape, vert, slash, vs,
                    ss, ws, nbytes)
    return (vert, slash, vs, ss) if return_scores else (vert, slash)
