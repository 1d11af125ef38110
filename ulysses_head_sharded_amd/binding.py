"""Thin Python binding of libulysses.so (ctypes; argument marshalling only).

The ``ulys_*`` functions mirror the C ABI of ``include/ulysses.h`` one to one
(plain integers for pointers and sizes).  The tensor helpers below them only
allocate outputs with torch, read ``data_ptr()`` and the current stream, and
raise on a non-zero status: every step of the path runs in the HIP kernels.
There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libulysses.so")

ULYS_F32, ULYS_BF16 = 0, 1
ULYS_OK = 0
ULYS_ERR_NULL, ULYS_ERR_DIM, ULYS_ERR_DIVISIBILITY = -1, -2, -3
ULYS_ERR_UNSUPPORTED, ULYS_ERR_ALIGNMENT, ULYS_ERR_ALIAS, ULYS_ERR_HIP = -4, -5, -6, -7

# every symbol include/ulysses.h declares
EXPORTED = ("ulys_pack_seq2head", "ulys_unpack_head2seq", "ulys_pack_seq2head_kv",
            "ulys_unpack_head2seq_kv", "ulys_pack_seq2head_qkv", "ulys_attn_fwd", "ulys_attn_fwd_ws",
            "ulys_attn_fwd_workspace_size", "ulys_attn_bwd", "ulys_attn_bwd_workspace_size",
            "ulys_attn_merge", "ulys_seq2head_push", "ulys_head2seq_push", "ulys_attn_fwd_push",
            "ulys_attn_bwd_push", "ulys_attn_fwd_noalloc",
            "ulys_status_string", "ulys_abi_version")

_lib = None


class UlyssesError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {ulys_status_string(status)} (status {status})")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950); there is no fallback path")
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lay = [vp, vp, i64, i64, i64, i64, i32, i32, vp]
    lib.ulys_pack_seq2head.argtypes = lay
    lib.ulys_pack_seq2head.restype = ctypes.c_int
    lib.ulys_unpack_head2seq.argtypes = lay
    lib.ulys_unpack_head2seq.restype = ctypes.c_int
    lib.ulys_pack_seq2head_kv.argtypes = lay
    lib.ulys_pack_seq2head_kv.restype = ctypes.c_int
    lib.ulys_unpack_head2seq_kv.argtypes = lay
    lib.ulys_unpack_head2seq_kv.restype = ctypes.c_int
    lib.ulys_pack_seq2head_qkv.argtypes = [vp] * 6 + [i64] * 5 + [i32, i32, vp]
    lib.ulys_pack_seq2head_qkv.restype = ctypes.c_int
    lib.ulys_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, i32, vp]
    lib.ulys_attn_fwd.restype = ctypes.c_int
    lib.ulys_attn_fwd_ws.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, i32,
                                     vp, i64, vp]
    lib.ulys_attn_fwd_ws.restype = ctypes.c_int
    lib.ulys_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32,
                                          i32, vp]
    lib.ulys_attn_fwd_noalloc.restype = ctypes.c_int
    lib.ulys_attn_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, i32, i32]
    lib.ulys_attn_fwd_workspace_size.restype = ctypes.c_int64
    lib.ulys_attn_bwd.argtypes = [vp] * 9 + [i64] * 5 + [i32] * 3 + [vp, i64, vp]
    lib.ulys_attn_bwd.restype = ctypes.c_int
    lib.ulys_attn_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, i32, i32]
    lib.ulys_attn_bwd_workspace_size.restype = ctypes.c_int64
    push = [vp, ctypes.POINTER(vp), i32, i64, i64, i64, i64, i32, i32, vp]
    lib.ulys_seq2head_push.argtypes = push
    lib.ulys_seq2head_push.restype = ctypes.c_int
    lib.ulys_head2seq_push.argtypes = push
    lib.ulys_head2seq_push.restype = ctypes.c_int
    lib.ulys_attn_fwd_push.argtypes = [vp, vp, vp, ctypes.POINTER(vp), i32, vp] + [i64] * 5 + \
        [i32, i32, i32, vp, i64, vp]
    lib.ulys_attn_fwd_push.restype = ctypes.c_int
    pp = ctypes.POINTER(vp)
    lib.ulys_attn_bwd_push.argtypes = [vp] * 6 + [pp, pp, pp, i32] + [i64] * 5 + \
        [i32, i32, i32, vp, i64, vp]
    lib.ulys_attn_bwd_push.restype = ctypes.c_int
    lib.ulys_attn_merge.argtypes = [vp] * 6 + [i64] * 4 + [i32, vp]
    lib.ulys_attn_merge.restype = ctypes.c_int
    lib.ulys_status_string.argtypes = [ctypes.c_int]
    lib.ulys_status_string.restype = ctypes.c_char_p
    lib.ulys_abi_version.argtypes = []
    lib.ulys_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


# ------------------------------------------------------------------ raw C-ABI mirrors
def ulys_pack_seq2head(x, y, s, b, h, d_h, P, dtype, stream=None) -> int:
    return load().ulys_pack_seq2head(x, y, s, b, h, d_h, P, dtype, stream)


def ulys_unpack_head2seq(y, x, s, b, h, d_h, P, dtype, stream=None) -> int:
    return load().ulys_unpack_head2seq(y, x, s, b, h, d_h, P, dtype, stream)


def ulys_pack_seq2head_kv(x, y, s, b, h_kv, d_h, P, dtype, stream=None) -> int:
    return load().ulys_pack_seq2head_kv(x, y, s, b, h_kv, d_h, P, dtype, stream)


def ulys_unpack_head2seq_kv(y, x, s, b, h_kv, d_h, P, dtype, stream=None) -> int:
    return load().ulys_unpack_head2seq_kv(y, x, s, b, h_kv, d_h, P, dtype, stream)


def ulys_pack_seq2head_qkv(xq, xk, xv, yq, yk, yv, s, b, h, h_kv, d_h, P, dtype,
                           stream=None) -> int:
    return load().ulys_pack_seq2head_qkv(xq, xk, xv, yq, yk, yv, s, b, h, h_kv, d_h, P, dtype,
                                         stream)


def ulys_attn_fwd(q, k, v, o, lse, s, b, h, h_kv, d_h, P, causal, dtype, stream=None) -> int:
    return load().ulys_attn_fwd(q, k, v, o, lse, s, b, h, h_kv, d_h, P, causal, dtype, stream)


def ulys_attn_fwd_ws(q, k, v, o, lse, s, b, h, h_kv, d_h, P, causal, dtype, workspace,
                     workspace_bytes, stream=None) -> int:
    return load().ulys_attn_fwd_ws(q, k, v, o, lse, s, b, h, h_kv, d_h, P, causal, dtype,
                                   workspace, workspace_bytes, stream)


def ulys_attn_fwd_noalloc(q, k, v, o, lse, s, b, h, h_kv, d_h, P, causal, dtype,
                          stream=None) -> int:
    return load().ulys_attn_fwd_noalloc(q, k, v, o, lse, s, b, h, h_kv, d_h, P, causal, dtype,
                                        stream)


def ulys_attn_fwd_workspace_size(s, b, h, h_kv, d_h, P, causal, dtype) -> int:
    return load().ulys_attn_fwd_workspace_size(s, b, h, h_kv, d_h, P, causal, dtype)


def ulys_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, s, b, h, h_kv, d_h, P, causal, dtype,
                  workspace, workspace_bytes, stream=None) -> int:
    return load().ulys_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, s, b, h, h_kv, d_h, P, causal,
                                dtype, workspace, workspace_bytes, stream)


def ulys_attn_bwd_workspace_size(s, b, h, h_kv, d_h, P, causal, dtype) -> int:
    return load().ulys_attn_bwd_workspace_size(s, b, h, h_kv, d_h, P, causal, dtype)


def ulys_attn_merge(o_a, lse_a, o_b, lse_b, o, lse, s, b, hp, d_h, dtype, stream=None) -> int:
    return load().ulys_attn_merge(o_a, lse_a, o_b, lse_b, o, lse, s, b, hp, d_h, dtype, stream)


def _ptr_table(ptrs):
    vp = ctypes.c_void_p
    return (vp * len(ptrs))(*[vp(p) if p else None for p in ptrs])


def ulys_seq2head_push(x, y_ranks, rank, s, b, h, d_h, P, dtype, stream=None) -> int:
    """y_ranks: sequence of P device addresses (ints)."""
    return load().ulys_seq2head_push(x, _ptr_table(y_ranks), rank, s, b, h, d_h, P, dtype, stream)


def ulys_head2seq_push(o, x_ranks, rank, s, b, h, d_h, P, dtype, stream=None) -> int:
    """x_ranks: sequence of P device addresses (ints)."""
    return load().ulys_head2seq_push(o, _ptr_table(x_ranks), rank, s, b, h, d_h, P, dtype, stream)


def ulys_attn_fwd_push(q, k, v, x_ranks, rank, lse, s, b, h, h_kv, d_h, P, causal, dtype,
                       workspace, workspace_bytes, stream=None) -> int:
    """x_ranks: sequence of P device addresses (ints)."""
    return load().ulys_attn_fwd_push(q, k, v, _ptr_table(x_ranks), rank, lse, s, b, h, h_kv, d_h,
                                     P, causal, dtype, workspace, workspace_bytes, stream)


def ulys_attn_bwd_push(q, k, v, o, dout, lse, dq_ranks, dk_ranks, dv_ranks, rank, s, b, h, h_kv,
                       d_h, P, causal, dtype, workspace, workspace_bytes, stream=None) -> int:
    """dq_ranks, dk_ranks, dv_ranks: sequences of P device addresses (ints)."""
    return load().ulys_attn_bwd_push(q, k, v, o, dout, lse, _ptr_table(dq_ranks),
                                     _ptr_table(dk_ranks), _ptr_table(dv_ranks), rank, s, b, h,
                                     h_kv, d_h, P, causal, dtype, workspace, workspace_bytes,
                                     stream)


def ulys_status_string(status: int) -> str:
    return load().ulys_status_string(status).decode()


def ulys_abi_version() -> int:
    return load().ulys_abi_version()


# ------------------------------------------------------------------ tensor helpers
def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return ULYS_F32
    if t.dtype == torch.bfloat16:
        return ULYS_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _stream(stream):
    if stream is not None:
        return stream
    return _torch().cuda.current_stream().cuda_stream


def _hold(stream, *tensors) -> None:
    """Tensors allocated here on torch's current stream but used by kernels
    enqueued on another stream: tell the caching allocator, so that it does not
    hand their memory to a new allocation before that stream's work is done
    (a workspace dropped on return would otherwise be reusable while the
    kernels still read and write it)."""
    if stream is None:
        return
    torch = _torch()
    live = [t for t in tensors if t is not None]
    if not live:
        return
    handle = int(stream)
    if handle == torch.cuda.current_stream(live[0].device).cuda_stream:
        return
    other = (torch.cuda.default_stream(live[0].device) if handle == 0 else
             torch.cuda.ExternalStream(handle, device=live[0].device))
    for t in live:
        t.record_stream(other)


def _check(rc: int, what: str) -> None:
    if rc != ULYS_OK:
        raise UlyssesError(rc, what)


def pack_seq2head(x, P: int, out=None, stream=None):
    """x [s/P, b, h, d] (CUDA tensor) -> send buffer [P, s/P, b, h/P, d]."""
    sl, b, h, d = x.shape
    if h % P:
        raise ValueError(f"P={P} must divide h={h}")
    if out is None:
        out = _torch().empty((P, sl, b, h // P, d), dtype=x.dtype, device=x.device)
    _check(ulys_pack_seq2head(x.data_ptr(), out.data_ptr(), sl * P, b, h, d, P,
                              dtype_code(x), _stream(stream)), "ulys_pack_seq2head")
    _hold(stream, out)
    return out


def unpack_head2seq(y, out=None, stream=None):
    """y [P, s/P, b, h/P, d] (received blocks) -> [s/P, b, h, d]."""
    P, sl, b, hp, d = y.shape
    if out is None:
        out = _torch().empty((sl, b, hp * P, d), dtype=y.dtype, device=y.device)
    _check(ulys_unpack_head2seq(y.data_ptr(), out.data_ptr(), sl * P, b, hp * P, d, P,
                                dtype_code(y), _stream(stream)), "ulys_unpack_head2seq")
    _hold(stream, out)
    return out


def kv_heads_per_rank(h_kv: int, P: int) -> int:
    """KV heads of one rank's share: h_kv/P, or 1 when h_kv < P (replicated)."""
    return h_kv // P if h_kv % P == 0 else 1


def pack_seq2head_kv(x, P: int, out=None, stream=None):
    """K or V shard x [s/P, b, h_kv, d] -> send buffer [P, s/P, b, max(1, h_kv/P), d];
    with h_kv < P block r is KV head floor(r*h_kv/P)."""
    sl, b, h_kv, d = x.shape
    if out is None:
        out = _torch().empty((P, sl, b, kv_heads_per_rank(h_kv, P), d), dtype=x.dtype,
                             device=x.device)
    _check(ulys_pack_seq2head_kv(x.data_ptr(), out.data_ptr(), sl * P, b, h_kv, d, P,
                                 dtype_code(x), _stream(stream)), "ulys_pack_seq2head_kv")
    _hold(stream, out)
    return out


def unpack_head2seq_kv(y, h_kv: int, out=None, stream=None):
    """Received K/V gradient blocks y [P, s/P, b, max(1, h_kv/P), d] -> [s/P, b, h_kv, d];
    with h_kv < P the copies of each KV head are summed."""
    P, sl, b, _, d = y.shape
    if out is None:
        out = _torch().empty((sl, b, h_kv, d), dtype=y.dtype, device=y.device)
    _check(ulys_unpack_head2seq_kv(y.data_ptr(), out.data_ptr(), sl * P, b, h_kv, d, P,
                                   dtype_code(y), _stream(stream)), "ulys_unpack_head2seq_kv")
    _hold(stream, out)
    return out


def attn_fwd(q, k, v, P: int = 1, causal: bool = False, out=None, lse=False, stream=None):
    """One rank's share: q [s, b, h/P, d], k/v [s, b, h_kv/P, d] -> o [s, b, h/P, d].

    ``lse`` may be False (skip), True (allocate [b, h/P, s] float32) or a tensor.
    Allocates (with torch) the workspace ulys_attn_fwd_ws asks for, if any.
    Returns (o, lse or None)."""
    torch = _torch()
    s, b, hp, d = q.shape
    hkvp = k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    lse_t = None
    if lse is True:
        lse_t = torch.empty((b, hp, s), dtype=torch.float32, device=q.device)
    elif lse is not False and lse is not None:
        lse_t = lse
    h, h_kv, code = hp * P, hkvp * P, dtype_code(q)
    ws_bytes = ulys_attn_fwd_workspace_size(s, b, h, h_kv, d, P, int(bool(causal)), code)
    if ws_bytes < 0:
        raise UlyssesError(int(ws_bytes), "ulys_attn_fwd_workspace_size")
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes > 0 else None
    rc = ulys_attn_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse_t.data_ptr() if lse_t is not None else None,
                          s, b, h, h_kv, d, P, int(bool(causal)), code,
                          ws.data_ptr() if ws is not None else None, ws_bytes, _stream(stream))
    _check(rc, "ulys_attn_fwd_ws")
    _hold(stream, ws, out, lse_t)
    return out, lse_t


def attn_bwd(q, k, v, o, dout, lse, P: int = 1, causal: bool = False, stream=None):
    """Gradients of one rank's share: q, o, dout [s, b, h/P, d], k/v [s, b, h_kv/P, d],
    lse [b, h/P, s] float32 (ulys_attn_fwd's outputs for the same q, k, v).
    Allocates (with torch) the outputs and the workspace; returns (dq, dk, dv)."""
    torch = _torch()
    s, b, hp, d = q.shape
    hkvp = k.shape[2]
    h, h_kv, code = hp * P, hkvp * P, dtype_code(q)
    ws_bytes = ulys_attn_bwd_workspace_size(s, b, h, h_kv, d, P, int(bool(causal)), code)
    if ws_bytes < 0:
        raise UlyssesError(int(ws_bytes), "ulys_attn_bwd_workspace_size")
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    rc = ulys_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                       lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), s, b, h, h_kv,
                       d, P, int(bool(causal)), code, ws.data_ptr(), ws_bytes, _stream(stream))
    _check(rc, "ulys_attn_bwd")
    _hold(stream, ws, dq, dk, dv)
    return dq, dk, dv


def attn_merge(o_a, lse_a, o_b, lse_b, out=None, lse_out=None, stream=None):
    """Merge two partial attention results of one share: o_* [s, b, hp, d],
    lse_* [b, hp, s] float32.  out/lse_out may be o_a/lse_a (in place); by
    default new tensors.  Returns (o, lse)."""
    torch = _torch()
    s, b, hp, d = o_a.shape
    if out is None:
        out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    _check(ulys_attn_merge(o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(), lse_b.data_ptr(),
                           out.data_ptr(), lse_out.data_ptr(), s, b, hp, d, dtype_code(o_a),
                           _stream(stream)), "ulys_attn_merge")
    _hold(stream, out, lse_out)
    return out, lse_out
