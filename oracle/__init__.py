"""CPU oracle for the Ulysses per-rank hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, loads or calls it, and the two share no
code: this wrapper only marshals numpy arrays into ``ulys_oracle.c``.

Every function follows a passage of the pages cited in ``ulys_oracle.c``:
  * ``pack`` / ``unpack``        -- the local halves of the two all-to-alls
    ("02 · DeepSpeed-Ulysses", §2 "all-to-all 的转置与重分布");
  * ``seq2head`` / ``head2seq``  -- the whole exchange across P emulated ranks
    (same section; "5. AllToAll（全交换）" of the collectives tutorial);
  * ``pack_kv`` / ``unpack_kv_sum`` -- K/V send side when there are fewer KV heads
    than ranks (each head replicated to the ranks whose queries use it) and its
    backward (the copies' gradients summed) ("Ulysses vs Ring Attention", §三;
    "长上下文训练中的 SP 与 CP", Ulysses section);
  * ``attn_merge``               -- two partial attention results over disjoint
    key sets combined through their log-sum-exp ("长上下文训练中的 SP 与 CP",
    Ring section's online-softmax state; the USP and hierarchical schemes);
  * ``attn`` / ``attn_rows``     -- softmax(Q K^T / sqrt(d_h)) V per head, dense
    or causal (j <= t), GQA by contiguous groups ("DeepSpeed-Ulysses 深度解析",
    core design step 4), in fp64.
All are pinned by the CPU tests; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ulys_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libulys_oracle.so")
_lib = None

F32, BF16 = 0, 1
_c_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with the host compiler (plain C, no HIP headers)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if needed) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if (not os.path.exists(_LIB_PATH)
                or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    lay = [_vp, _vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64]
    for name in ("orc_pack", "orc_unpack", "orc_seq2head", "orc_head2seq", "orc_pack_kv"):
        fn = getattr(lib, name)
        fn.argtypes = lay
        fn.restype = ctypes.c_int
    lib.orc_unpack_kv_sum.argtypes = [_vp, _vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                      ctypes.c_int]
    lib.orc_attn_merge.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64,
                                   _c_i64]
    lib.orc_attn_merge.restype = ctypes.c_int
    lib.orc_unpack_kv_sum.restype = ctypes.c_int
    lib.orc_attn.argtypes = [_vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i64,
                             _c_i64, _c_i64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.orc_attn.restype = ctypes.c_int
    lib.orc_attn_rows.argtypes = [_vp, _vp, _vp, _vp, _c_i64, _vp, _vp, _c_i64, _c_i64,
                                  _c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int]
    lib.orc_attn_rows.restype = ctypes.c_int
    lib.orc_attn_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64,
                                 _c_i64, _c_i64, _c_i64, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int]
    lib.orc_attn_bwd.restype = ctypes.c_int
    lib.orc_attn_bwd_rows.argtypes = [_vp, _vp, _vp, _vp, _vp, _c_i64, _vp, _c_i64, _vp, _vp,
                                      _vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.orc_attn_bwd_rows.restype = ctypes.c_int
    return lib


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def _contig(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # raw bf16 bit patterns
        return BF16
    raise TypeError(f"oracle attention takes float32 or uint16 (bf16 bits), got {a.dtype}")


# ----------------------------------------------------------------------------- layout
def pack(x: np.ndarray, s: int, b: int, h: int, d: int, P: int, lib=None) -> np.ndarray:
    """[s/P,b,h,d] -> send buffer [P,s/P,b,h/P,d]; any fixed-size dtype, bit moves only."""
    lib = lib or load()
    x = _contig(x)
    y = np.empty(x.size, dtype=x.dtype)
    _check(lib.orc_pack(_ptr(x), _ptr(y), s, b, h, d, P, x.itemsize), "pack")
    return y.reshape(P, s // P, b, h // P, d)


def unpack(y: np.ndarray, s: int, b: int, h: int, d: int, P: int, lib=None) -> np.ndarray:
    """received blocks [P,s/P,b,h/P,d] -> [s/P,b,h,d]."""
    lib = lib or load()
    y = _contig(y)
    x = np.empty(y.size, dtype=y.dtype)
    _check(lib.orc_unpack(_ptr(y), _ptr(x), s, b, h, d, P, y.itemsize), "unpack")
    return x.reshape(s // P, b, h, d)


def seq2head(x_all: np.ndarray, s: int, b: int, h: int, d: int, P: int, lib=None) -> np.ndarray:
    """All P shards [P,s/P,b,h,d] -> all P shares [P,s,b,h/P,d]."""
    lib = lib or load()
    x_all = _contig(x_all)
    y = np.empty(x_all.size, dtype=x_all.dtype)
    _check(lib.orc_seq2head(_ptr(x_all), _ptr(y), s, b, h, d, P, x_all.itemsize), "seq2head")
    return y.reshape(P, s, b, h // P, d)


def head2seq(y_all: np.ndarray, s: int, b: int, h: int, d: int, P: int, lib=None) -> np.ndarray:
    """All P shares [P,s,b,h/P,d] -> all P shards [P,s/P,b,h,d]."""
    lib = lib or load()
    y_all = _contig(y_all)
    x = np.empty(y_all.size, dtype=y_all.dtype)
    _check(lib.orc_head2seq(_ptr(y_all), _ptr(x), s, b, h, d, P, y_all.itemsize), "head2seq")
    return x.reshape(P, s // P, b, h, d)


def kv_heads_per_rank(h_kv: int, P: int) -> int:
    """KV heads in one rank's share: h_kv/P, or 1 when each head is replicated."""
    return h_kv // P if h_kv % P == 0 else 1


def pack_kv(x: np.ndarray, s: int, b: int, h_kv: int, d: int, P: int, lib=None) -> np.ndarray:
    """K or V shard [s/P,b,h_kv,d] -> send buffer [P,s/P,b,max(1,h_kv/P),d]; with
    h_kv < P rank r's block is KV head floor(r*h_kv/P) (replication)."""
    lib = lib or load()
    x = _contig(x)
    hk = kv_heads_per_rank(h_kv, P)
    y = np.empty(P * (s // P) * b * hk * d, dtype=x.dtype)
    _check(lib.orc_pack_kv(_ptr(x), _ptr(y), s, b, h_kv, d, P, x.itemsize), "pack_kv")
    return y.reshape(P, s // P, b, hk, d)


def unpack_kv_sum(y: np.ndarray, s: int, b: int, h_kv: int, d: int, P: int,
                  lib=None) -> np.ndarray:
    """Gradient blocks [P,s/P,b,max(1,h_kv/P),d] (float32 or bf16 bits) -> [s/P,b,h_kv,d];
    with h_kv < P the blocks of the ranks sharing a KV head are summed (exactly,
    rounded once)."""
    lib = lib or load()
    y = _contig(y)
    x = np.empty((s // P) * b * h_kv * d, dtype=y.dtype)
    _check(lib.orc_unpack_kv_sum(_ptr(y), _ptr(x), s, b, h_kv, d, P, _dtype_code(y)),
           "unpack_kv_sum")
    return x.reshape(s // P, b, h_kv, d)


# ----------------------------------------------------------------------------- attention
def attn(q, k, v, s, b, h, h_kv, d, P, causal, nthreads=None, lib=None):
    """One rank's share: q [s,b,h/P,d], k/v [s,b,h_kv/P,d] (float32 or bf16 bits as uint16).

    Returns (o [s,b,h/P,d] float64, lse [b,h/P,s] float64)."""
    lib = lib or load()
    q, k, v = _contig(q), _contig(k), _contig(v)
    dt = _dtype_code(q)
    assert _dtype_code(k) == dt and _dtype_code(v) == dt
    hp = h // P
    o = np.empty((s, b, hp, d), dtype=np.float64)
    lse = np.empty((b, hp, s), dtype=np.float64)
    rc = lib.orc_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), s, b, h, h_kv, d, P,
                      int(bool(causal)), dt, nthreads or default_threads())
    _check(rc, "attn")
    return o, lse


def attn_rows(q, k, v, rows, s, b, h, h_kv, d, P, causal, nthreads=None, lib=None):
    """Attention on listed rows only; rows is int64 [n,3] of (beta, local head, t).

    Returns (o [n,d] float64, lse [n] float64)."""
    lib = lib or load()
    q, k, v = _contig(q), _contig(k), _contig(v)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    dt = _dtype_code(q)
    assert _dtype_code(k) == dt and _dtype_code(v) == dt
    n = rows.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib.orc_attn_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(rows), n, _ptr(o), _ptr(lse),
                           s, b, h, h_kv, d, P, int(bool(causal)), dt,
                           nthreads or default_threads())
    _check(rc, "attn_rows")
    return o, lse



def attn_merge(o_a, lse_a, o_b, lse_b, lib=None):
    """Merge two partial attention results of one share over disjoint key sets
    (float64): o_* [s, b, hp, d], lse_* [b, hp, s] (the attention's layouts).
    Returns (o, lse) float64."""
    lib = lib or load()
    o_a, o_b = (np.ascontiguousarray(x, dtype=np.float64) for x in (o_a, o_b))
    lse_a, lse_b = (np.ascontiguousarray(x, dtype=np.float64) for x in (lse_a, lse_b))
    s, b, hp, d = o_a.shape
    assert o_b.shape == o_a.shape and lse_a.shape == (b, hp, s) and lse_b.shape == (b, hp, s)
    o = np.empty_like(o_a)
    lse = np.empty_like(lse_a)
    _check(lib.orc_attn_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o),
                              _ptr(lse), s, b, hp, d), "attn_merge")
    return o, lse


# ----------------------------------------------------------------------------- backward
def attn_bwd(q, k, v, dout, s, b, h, h_kv, d, P, causal, nthreads=None, lib=None):
    """Gradients of one rank's share: q, dout [s,b,h/P,d], k/v [s,b,h_kv/P,d] (float32 or
    bf16 bits as uint16).  Returns (dq [s,b,h/P,d], dk, dv [s,b,h_kv/P,d]) float64."""
    lib = lib or load()
    q, k, v, dout = _contig(q), _contig(k), _contig(v), _contig(dout)
    dt = _dtype_code(q)
    assert _dtype_code(k) == dt and _dtype_code(v) == dt and _dtype_code(dout) == dt
    hp, hkvp = h // P, h_kv // P
    dq = np.empty((s, b, hp, d), dtype=np.float64)
    dk = np.empty((s, b, hkvp, d), dtype=np.float64)
    dv = np.empty((s, b, hkvp, d), dtype=np.float64)
    rc = lib.orc_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                          s, b, h, h_kv, d, P, int(bool(causal)), dt,
                          nthreads or default_threads())
    _check(rc, "attn_bwd")
    return dq, dk, dv


def attn_bwd_rows(q, k, v, dout, qrows, krows, s, b, h, h_kv, d, P, causal, nthreads=None,
                  lib=None):
    """Gradients at listed places only: qrows int64 [n,3] of (beta, local head, t) -> dq [n,d];
    krows int64 [m,3] of (beta, local KV head, j) -> dk, dv [m,d].  float64."""
    lib = lib or load()
    q, k, v, dout = _contig(q), _contig(k), _contig(v), _contig(dout)
    qrows = np.ascontiguousarray(qrows, dtype=np.int64).reshape(-1, 3)
    krows = np.ascontiguousarray(krows, dtype=np.int64).reshape(-1, 3)
    dt = _dtype_code(q)
    assert _dtype_code(k) == dt and _dtype_code(v) == dt and _dtype_code(dout) == dt
    n, m = qrows.shape[0], krows.shape[0]
    dq = np.empty((max(n, 1), d), dtype=np.float64)
    dk = np.empty((max(m, 1), d), dtype=np.float64)
    dv = np.empty((max(m, 1), d), dtype=np.float64)
    rc = lib.orc_attn_bwd_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(qrows), n,
                               _ptr(krows), m, _ptr(dq), _ptr(dk), _ptr(dv), s, b, h, h_kv, d,
                               P, int(bool(causal)), dt, nthreads or default_threads())
    _check(rc, "attn_bwd_rows")
    return dq[:n], dk[:m], dv[:m]
