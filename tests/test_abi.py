"""The C-ABI library: it loads, exports every symbol the header declares, and
rejects bad arguments on the host before any HIP call (no GPU needed: every
call here returns from validation without launching)."""
import os
import re

import pytest

from ulysses_head_sharded_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ulysses.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from ulysses_head_sharded_amd import build
        build.build()
    return B.load()


def declared_symbols():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ulys_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_symbols() == sorted(B.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_version(lib):
    assert B.ulys_abi_version() == (1 << 16) | 12


def test_status_strings(lib):
    codes = [B.ULYS_OK, B.ULYS_ERR_NULL, B.ULYS_ERR_DIM, B.ULYS_ERR_DIVISIBILITY,
             B.ULYS_ERR_UNSUPPORTED, B.ULYS_ERR_ALIGNMENT, B.ULYS_ERR_ALIAS, B.ULYS_ERR_HIP]
    texts = [B.ulys_status_string(c) for c in codes]
    assert len(set(texts)) == len(texts)
    assert B.ulys_status_string(12345) == "unknown status"


# fake, never-dereferenced device addresses: validation rejects every call below
X, Y = 0x7F0000000000, 0x7F0100000000


@pytest.mark.parametrize("fn", [B.ulys_pack_seq2head, B.ulys_unpack_head2seq])
@pytest.mark.parametrize("args,expect", [
    ((None, Y, 16, 1, 8, 64, 4, B.ULYS_BF16), B.ULYS_ERR_NULL),
    ((X, None, 16, 1, 8, 64, 4, B.ULYS_BF16), B.ULYS_ERR_NULL),
    ((X, Y, 0, 1, 8, 64, 4, B.ULYS_BF16), B.ULYS_ERR_DIM),
    ((X, Y, 16, -1, 8, 64, 4, B.ULYS_BF16), B.ULYS_ERR_DIM),
    ((X, Y, 16, 1, 8, 64, 0, B.ULYS_BF16), B.ULYS_ERR_DIM),
    ((X, Y, 18, 1, 8, 64, 4, B.ULYS_BF16), B.ULYS_ERR_DIVISIBILITY),
    ((X, Y, 16, 1, 6, 64, 4, B.ULYS_BF16), B.ULYS_ERR_DIVISIBILITY),
    ((X, Y, 16, 1, 8, 64, 4, 7), B.ULYS_ERR_UNSUPPORTED),
    ((X + 8, Y, 16, 1, 8, 64, 4, B.ULYS_F32), B.ULYS_ERR_ALIGNMENT),
    ((X, Y + 2, 16, 1, 8, 64, 4, B.ULYS_F32), B.ULYS_ERR_ALIGNMENT),
    ((X, X + 4096, 16, 1, 8, 64, 4, B.ULYS_F32), B.ULYS_ERR_ALIAS),   # 8 KiB each
    ((X + 4096, X, 16, 1, 8, 64, 4, B.ULYS_F32), B.ULYS_ERR_ALIAS),
    ((X, Y, 1 << 41, 1, 8, 64, 1, B.ULYS_F32), B.ULYS_ERR_DIM),
])
def test_layout_rejects(lib, fn, args, expect):
    assert fn(*args) == expect


Q, K, V, O, L = (0x7F0000000000 + i * (1 << 32) for i in range(5))


ATTN_REJECTS = [
    ((None, K, V, O, L, 64, 1, 8, 8, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_NULL),
    ((Q, K, V, None, L, 64, 1, 8, 8, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_NULL),
    ((Q, K, V, O, L, 0, 1, 8, 8, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_DIM),
    ((Q, K, V, O, L, 64, 1, 8, 0, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_DIM),
    ((Q, K, V, O, L, 66, 1, 8, 8, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_DIVISIBILITY),
    ((Q, K, V, O, L, 64, 1, 12, 6, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_DIVISIBILITY),  # P, h_kv
    ((Q, K, V, O, L, 64, 1, 12, 8, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_DIVISIBILITY),
    ((Q, K, V, O, L, 64, 1, 8, 8, 96, 4, 1, B.ULYS_BF16), B.ULYS_ERR_UNSUPPORTED),
    ((Q, K, V, O, L, 64, 1, 8, 8, 128, 4, 1, 3), B.ULYS_ERR_UNSUPPORTED),
    ((Q, K + 4, V, O, L, 64, 1, 8, 8, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_ALIGNMENT),
    ((Q, K, V, O, L + 4, 64, 1, 8, 8, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_ALIGNMENT),
    ((Q, K, V, Q + 256, L, 64, 1, 8, 8, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_ALIAS),
    ((Q, K, V, V, None, 64, 1, 8, 8, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_ALIAS),
    ((Q, K, V, O, O + 64, 64, 1, 8, 8, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_ALIAS),
    ((Q, K, V, O, K, 64, 1, 8, 8, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_ALIAS),
]


@pytest.mark.parametrize("args,expect", ATTN_REJECTS)
def test_attn_rejects(lib, args, expect):
    assert B.ulys_attn_fwd(*args) == expect


@pytest.mark.parametrize("args,expect", ATTN_REJECTS)
def test_attn_noalloc_rejects(lib, args, expect):
    """The allocation-free forward validates its arguments as ulys_attn_fwd
    does, before it resolves its scratch or launches anything."""
    assert B.ulys_attn_fwd_noalloc(*args) == expect


def test_tensor_helper_raises_status(lib):
    err = B.UlyssesError(B.ULYS_ERR_DIVISIBILITY, "ulys_pack_seq2head")
    assert "divide" in str(err) and err.status == B.ULYS_ERR_DIVISIBILITY


def test_product_path_does_not_reach_the_oracle():
    """The package sources never import or load the CPU oracle."""
    pkg = os.path.join(ROOT, "ulysses_head_sharded_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "ulys_oracle" not in text, f
                assert "from oracle" not in text, f


W = 0x7F0000000000 + 5 * (1 << 32)


@pytest.mark.parametrize("ws,nbytes,expect", [
    (W + 8, 1 << 20, B.ULYS_ERR_ALIGNMENT),
    (W, -1, B.ULYS_ERR_DIM),
    (Q + 4096, 1 << 20, B.ULYS_ERR_ALIAS),      # overlaps q
    (O - 64, 1 << 20, B.ULYS_ERR_ALIAS),        # overlaps o
    (L, 64, B.ULYS_ERR_ALIAS),                  # overlaps lse
])
def test_attn_ws_rejects(lib, ws, nbytes, expect):
    args = (Q, K, V, O, L, 64, 1, 8, 8, 128, 4, 1, B.ULYS_BF16, ws, nbytes)
    assert B.ulys_attn_fwd_ws(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((0, 1, 8, 8, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_DIM),
    ((66, 1, 8, 8, 128, 4, 1, B.ULYS_BF16), B.ULYS_ERR_DIVISIBILITY),
    ((64, 1, 8, 8, 96, 4, 1, B.ULYS_BF16), B.ULYS_ERR_UNSUPPORTED),
    ((64, 1, 8, 8, 128, 4, 1, 9), B.ULYS_ERR_UNSUPPORTED),
])
def test_workspace_size_rejects(lib, args, expect):
    assert B.ulys_attn_fwd_workspace_size(*args) == expect


def test_bf16_offset_bound(lib):
    """The bf16 kernels form 32-bit byte offsets up to one 256-row block past a
    tensor's end: s = 1048312 with 8 local heads of 128 is the largest share of
    that head layout the ABI admits, and the next multiple of P is refused
    (fp32 inputs, which the kernels address with 64-bit offsets, are not)."""
    ok = (1048312, 1, 64, 64, 128, 8, 1, B.ULYS_BF16)
    assert B.ulys_attn_fwd_workspace_size(*ok) >= 0
    assert B.ulys_attn_bwd_workspace_size(*ok) > 0
    over = (1048320, 1, 64, 64, 128, 8, 1, B.ULYS_BF16)
    assert B.ulys_attn_fwd_workspace_size(*over) == B.ULYS_ERR_DIM
    assert B.ulys_attn_bwd_workspace_size(*over) == B.ULYS_ERR_DIM
    assert B.ulys_attn_fwd_workspace_size(1048320, 1, 64, 64, 128, 8, 1, B.ULYS_F32) == 0


def test_workspace_size_fp32_is_zero(lib):
    assert B.ulys_attn_fwd_workspace_size(16, 1, 8, 8, 64, 4, 0, B.ULYS_F32) == 0


# ---------------------------------------------------------------------- backward
DO, DQ, DK, DV, WS = (0x7F0000000000 + i * (1 << 32) for i in range(6, 11))
BWD_OK = (Q, K, V, O, DO, L, DQ, DK, DV, 64, 1, 8, 8, 128, 4, 1, B.ULYS_BF16, WS, 1 << 20)


def bwd_args(**kw):
    names = ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "s", "b", "h", "h_kv", "d",
             "P", "causal", "dtype", "ws", "nbytes")
    a = dict(zip(names, BWD_OK))
    a.update(kw)
    return tuple(a[n] for n in names)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), B.ULYS_ERR_NULL),
    (dict(lse=None), B.ULYS_ERR_NULL),
    (dict(dv=None), B.ULYS_ERR_NULL),
    (dict(ws=None), B.ULYS_ERR_NULL),
    (dict(s=0), B.ULYS_ERR_DIM),
    (dict(s=66), B.ULYS_ERR_DIVISIBILITY),
    (dict(h=12, h_kv=6), B.ULYS_ERR_DIVISIBILITY),
    (dict(h_kv=3), B.ULYS_ERR_DIVISIBILITY),
    (dict(d=96), B.ULYS_ERR_UNSUPPORTED),
    (dict(dtype=9), B.ULYS_ERR_UNSUPPORTED),
    (dict(dtype=B.ULYS_F32, b=16384, h=32, h_kv=32), B.ULYS_ERR_DIM),  # b*h/P past the grid
    (dict(dtype=B.ULYS_F32, nbytes=256), B.ULYS_ERR_DIM),  # fp32 needs b*hp*s floats
    (dict(nbytes=16), B.ULYS_ERR_DIM),
    (dict(dk=DK + 4), B.ULYS_ERR_ALIGNMENT),
    (dict(dq=Q + 256), B.ULYS_ERR_ALIAS),
    (dict(dv=DK + 64), B.ULYS_ERR_ALIAS),
    (dict(ws=DO), B.ULYS_ERR_ALIAS),
    (dict(dq=L), B.ULYS_ERR_ALIAS),
])
def test_attn_bwd_rejects(lib, kw, expect):
    assert B.ulys_attn_bwd(*bwd_args(**kw)) == expect


def test_attn_bwd_workspace_size(lib):
    # D and lse * log2(e) per query row, rows padded to 4 queries
    assert B.ulys_attn_bwd_workspace_size(64, 1, 8, 8, 128, 4, 1, B.ULYS_BF16) == 2 * 2 * 64 * 4
    assert B.ulys_attn_bwd_workspace_size(66, 1, 8, 8, 128, 2, 1, B.ULYS_BF16) == 2 * 4 * 68 * 4
    assert B.ulys_attn_bwd_workspace_size(64, 1, 8, 8, 64, 4, 1, B.ULYS_BF16) == 2 * 2 * 64 * 4
    assert B.ulys_attn_bwd_workspace_size(64, 1, 8, 8, 96, 4, 1, B.ULYS_BF16) == B.ULYS_ERR_UNSUPPORTED
    # fp32: D = rowsum(dout * o) per query row, rounded up to 256 bytes
    assert B.ulys_attn_bwd_workspace_size(64, 1, 8, 8, 128, 4, 1, B.ULYS_F32) == 512
    assert B.ulys_attn_bwd_workspace_size(100, 1, 8, 8, 64, 4, 0, B.ULYS_F32) == 1024
    assert B.ulys_attn_bwd_workspace_size(64, 1, 8, 8, 128, 4, 1, 9) == B.ULYS_ERR_UNSUPPORTED
    assert B.ulys_attn_bwd_workspace_size(0, 1, 8, 8, 128, 4, 1, B.ULYS_BF16) == B.ULYS_ERR_DIM


# ---------------------------------------------------------------------- fewer KV heads than ranks
@pytest.mark.parametrize("fn", [B.ulys_pack_seq2head_kv, B.ulys_unpack_head2seq_kv])
@pytest.mark.parametrize("args,expect", [
    ((None, Y, 16, 1, 2, 64, 4, B.ULYS_BF16), B.ULYS_ERR_NULL),
    ((X, None, 16, 1, 2, 64, 4, B.ULYS_BF16), B.ULYS_ERR_NULL),
    ((X, Y, 0, 1, 2, 64, 4, B.ULYS_BF16), B.ULYS_ERR_DIM),
    ((X, Y, 16, 1, 0, 64, 4, B.ULYS_BF16), B.ULYS_ERR_DIM),
    ((X, Y, 18, 1, 2, 64, 4, B.ULYS_BF16), B.ULYS_ERR_DIVISIBILITY),
    ((X, Y, 16, 1, 3, 64, 4, B.ULYS_BF16), B.ULYS_ERR_DIVISIBILITY),   # neither divides
    ((X, Y, 16, 1, 6, 64, 4, B.ULYS_BF16), B.ULYS_ERR_DIVISIBILITY),
    ((X, Y, 16, 1, 2, 64, 4, 5), B.ULYS_ERR_UNSUPPORTED),
    ((X + 8, Y, 16, 1, 2, 64, 4, B.ULYS_F32), B.ULYS_ERR_ALIGNMENT),
    ((X, Y + 4, 16, 1, 2, 64, 4, B.ULYS_F32), B.ULYS_ERR_ALIGNMENT),
    # replicated: shard 4*1*2*64*4 = 2 KiB, blocks 4*4*1*1*64*4 = 4 KiB
    ((X, X + 1024, 16, 1, 2, 64, 4, B.ULYS_F32), B.ULYS_ERR_ALIAS),
    ((X + 1024, X, 16, 1, 2, 64, 4, B.ULYS_F32), B.ULYS_ERR_ALIAS),
])
def test_layout_kv_rejects(lib, fn, args, expect):
    assert fn(*args) == expect


def test_attention_accepts_fewer_kv_heads_than_ranks(lib):
    """h_kv < P with h_kv | P is a valid share (one replicated KV head); neither
    dividing the other is not."""
    assert B.ulys_attn_fwd_workspace_size(64, 1, 8, 2, 128, 4, 1, B.ULYS_BF16) >= 0
    assert B.ulys_attn_fwd_workspace_size(64, 1, 8, 1, 128, 8, 0, B.ULYS_BF16) >= 0
    assert B.ulys_attn_fwd_workspace_size(64, 1, 12, 6, 128, 4, 1, B.ULYS_BF16) == \
        B.ULYS_ERR_DIVISIBILITY
    # the backward's statistics are per query head: b * hp * s_pad * 2 floats
    assert B.ulys_attn_bwd_workspace_size(64, 1, 8, 2, 128, 4, 1, B.ULYS_BF16) == 2 * 2 * 64 * 4


# ---------------------------------------------------------------------- merge of partial results
OA, LA, OB, LB, OO, LO = (0x7F0000000000 + i * (1 << 32) for i in range(11, 17))
MERGE_OK = (OA, LA, OB, LB, OO, LO, 64, 1, 2, 128, B.ULYS_BF16)


def merge_args(**kw):
    names = ("o_a", "lse_a", "o_b", "lse_b", "o", "lse", "s", "b", "hp", "d", "dtype")
    a = dict(zip(names, MERGE_OK))
    a.update(kw)
    return tuple(a[n] for n in names)


@pytest.mark.parametrize("kw,expect", [
    (dict(o_a=None), B.ULYS_ERR_NULL),
    (dict(lse=None), B.ULYS_ERR_NULL),
    (dict(s=0), B.ULYS_ERR_DIM),
    (dict(hp=-1), B.ULYS_ERR_DIM),
    (dict(d=96), B.ULYS_ERR_UNSUPPORTED),
    (dict(dtype=7), B.ULYS_ERR_UNSUPPORTED),
    (dict(o_b=OB + 8), B.ULYS_ERR_ALIGNMENT),
    (dict(lse=LO + 4), B.ULYS_ERR_ALIGNMENT),
    (dict(o=OB), B.ULYS_ERR_ALIAS),              # output on the second input
    (dict(o=OA + 256), B.ULYS_ERR_ALIAS),        # partial overlap with the first
    (dict(lse=LB), B.ULYS_ERR_ALIAS),
    (dict(lse=OO + 512), B.ULYS_ERR_ALIAS),      # lse inside o
    (dict(o=LA), B.ULYS_ERR_ALIAS),              # o over lse_a
])
def test_attn_merge_rejects(lib, kw, expect):
    assert B.ulys_attn_merge(*merge_args(**kw)) == expect


# ---------------------------------------------------------------------- fused Q/K/V pack
XQ, XK, XV, YQ, YK, YV = (0x7F0000000000 + i * (1 << 32) for i in range(20, 26))
QKV_OK = (XQ, XK, XV, YQ, YK, YV, 64, 1, 8, 2, 128, 4, B.ULYS_BF16)


def qkv_args(**kw):
    names = ("xq", "xk", "xv", "yq", "yk", "yv", "s", "b", "h", "h_kv", "d", "P", "dtype")
    a = dict(zip(names, QKV_OK))
    a.update(kw)
    return tuple(a[n] for n in names)


@pytest.mark.parametrize("kw,expect", [
    (dict(xv=None), B.ULYS_ERR_NULL),
    (dict(yk=None), B.ULYS_ERR_NULL),
    (dict(s=0), B.ULYS_ERR_DIM),
    (dict(s=66), B.ULYS_ERR_DIVISIBILITY),
    (dict(h=6), B.ULYS_ERR_DIVISIBILITY),
    (dict(h_kv=3), B.ULYS_ERR_DIVISIBILITY),
    (dict(dtype=9), B.ULYS_ERR_UNSUPPORTED),
    (dict(yv=YV + 8), B.ULYS_ERR_ALIGNMENT),
    (dict(yq=XK), B.ULYS_ERR_ALIAS),            # an output over another tensor's input
    (dict(yv=YK + 1024), B.ULYS_ERR_ALIAS),     # two outputs overlapping
    (dict(yk=XK + 16), B.ULYS_ERR_ALIAS),
])
def test_pack_qkv_rejects(lib, kw, expect):
    assert B.ulys_pack_seq2head_qkv(*qkv_args(**kw)) == expect


# ---------------------------------------------------------------------- exchange as pushes
PX = 0x7F0000000000 + 30 * (1 << 32)
PY = [0x7F0000000000 + (31 + r) * (1 << 32) for r in range(4)]


@pytest.mark.parametrize("fn", [B.ulys_seq2head_push, B.ulys_head2seq_push])
@pytest.mark.parametrize("kw,expect", [
    (dict(x=None), B.ULYS_ERR_NULL),
    (dict(dst=[PY[0], None, PY[2], PY[3]]), B.ULYS_ERR_NULL),
    (dict(rank=4), B.ULYS_ERR_DIM),
    (dict(rank=-1), B.ULYS_ERR_DIM),
    (dict(P=65, dst=PY * 17, s=65 * 16, h=65), B.ULYS_ERR_DIM),
    (dict(s=18), B.ULYS_ERR_DIVISIBILITY),
    (dict(h=6), B.ULYS_ERR_DIVISIBILITY),
    (dict(dtype=3), B.ULYS_ERR_UNSUPPORTED),
    (dict(x=PX + 8), B.ULYS_ERR_ALIGNMENT),
    (dict(dst=[PY[0], PY[1] + 4, PY[2], PY[3]]), B.ULYS_ERR_ALIGNMENT),
    (dict(dst=[PY[0], PY[0], PY[2], PY[3]]), B.ULYS_ERR_ALIAS),      # two ranks, one buffer
    (dict(dst=[PX, PY[1], PY[2], PY[3]]), B.ULYS_ERR_ALIAS),         # over the local tensor
])
def test_push_rejects(lib, fn, kw, expect):
    a = dict(x=PX, dst=PY, rank=1, s=16, b=1, h=8, d=64, P=4, dtype=B.ULYS_BF16)
    a.update(kw)
    assert fn(a["x"], a["dst"], a["rank"], a["s"], a["b"], a["h"], a["d"], a["P"],
              a["dtype"]) == expect


# ------------------------------------------------------ attention with a pushing epilogue
AQ, AK, AV = (0x7F0000000000 + (40 + i) * (1 << 32) for i in range(3))
AD = [0x7F0000000000 + (50 + r) * (1 << 32) for r in range(4)]
AL, AW = 0x7F0000000000 + 60 * (1 << 32), 0x7F0000000000 + 61 * (1 << 32)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), B.ULYS_ERR_NULL),
    (dict(dst=None), B.ULYS_ERR_NULL),
    (dict(dst=[AD[0], None, AD[2], AD[3]]), B.ULYS_ERR_NULL),
    (dict(rank=4), B.ULYS_ERR_DIM),
    (dict(rank=-1), B.ULYS_ERR_DIM),
    (dict(s=18), B.ULYS_ERR_DIVISIBILITY),
    (dict(h_kv=3), B.ULYS_ERR_DIVISIBILITY),
    (dict(dtype=B.ULYS_F32), B.ULYS_ERR_UNSUPPORTED),  # fp32 has no pushing epilogue
    (dict(d=96), B.ULYS_ERR_UNSUPPORTED),
    (dict(q=AQ + 8), B.ULYS_ERR_ALIGNMENT),
    (dict(dst=[AD[0], AD[1], AD[2] + 4, AD[3]]), B.ULYS_ERR_ALIGNMENT),
    (dict(lse=AL + 4), B.ULYS_ERR_ALIGNMENT),
    (dict(dst=[AD[0], AD[0], AD[2], AD[3]]), B.ULYS_ERR_ALIAS),     # two ranks, one buffer
    (dict(dst=[AD[0], AQ, AD[2], AD[3]]), B.ULYS_ERR_ALIAS),        # over q
    # rank 1 writes from byte hp*d*2 = 512 of each destination on: over lse
    (dict(dst=[AD[0], AD[1], AD[2], AL - 512]), B.ULYS_ERR_ALIAS),
    (dict(dst=[AW, AD[1], AD[2], AD[3]], ws=AW, wsb=1 << 20), B.ULYS_ERR_ALIAS),
    (dict(lse=AK), B.ULYS_ERR_ALIAS),
])
def test_attn_push_rejects(lib, kw, expect):
    a = dict(q=AQ, k=AK, v=AV, dst=AD, rank=1, lse=AL, s=64, b=1, h=8, h_kv=4, d=128, P=4,
             causal=1, dtype=B.ULYS_BF16, ws=None, wsb=0)
    a.update(kw)
    if a["dst"] is None:
        rc = B.load().ulys_attn_fwd_push(a["q"], a["k"], a["v"], None, a["rank"], a["lse"], a["s"],
                                         a["b"], a["h"], a["h_kv"], a["d"], a["P"], a["causal"],
                                         a["dtype"], a["ws"], a["wsb"], None)
    else:
        rc = B.ulys_attn_fwd_push(a["q"], a["k"], a["v"], a["dst"], a["rank"], a["lse"], a["s"],
                                  a["b"], a["h"], a["h_kv"], a["d"], a["P"], a["causal"],
                                  a["dtype"], a["ws"], a["wsb"])
    assert rc == expect


# ------------------------------------------------ attention backward with pushing epilogues
BQ, BK, BV, BO, BG = (0x7F0000000000 + (70 + i) * (1 << 32) for i in range(5))
BL, BW = 0x7F0000000000 + 76 * (1 << 32), 0x7F0000000000 + 77 * (1 << 32)
BDQ = [0x7F0000000000 + (80 + r) * (1 << 32) for r in range(4)]
BDK = [0x7F0000000000 + (90 + r) * (1 << 32) for r in range(4)]
BDV = [0x7F0000000000 + (100 + r) * (1 << 32) for r in range(4)]


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), B.ULYS_ERR_NULL),
    (dict(ws=None), B.ULYS_ERR_NULL),
    (dict(dk=[BDK[0], None, BDK[2], BDK[3]]), B.ULYS_ERR_NULL),
    (dict(wsb=16), B.ULYS_ERR_DIM),                 # smaller than the workspace it needs
    (dict(rank=4), B.ULYS_ERR_DIM),
    (dict(s=18), B.ULYS_ERR_DIVISIBILITY),
    (dict(h_kv=2), B.ULYS_ERR_UNSUPPORTED),         # replicated KV heads
    (dict(dtype=B.ULYS_F32), B.ULYS_ERR_UNSUPPORTED),
    (dict(dv=[BDV[0], BDV[1] + 8, BDV[2], BDV[3]]), B.ULYS_ERR_ALIGNMENT),
    (dict(dq=[BDQ[0], BDQ[1], BDK[2], BDQ[3]]), B.ULYS_ERR_ALIAS),   # a dQ shard over a dK one
    (dict(dv=[BDV[0], BDV[0], BDV[2], BDV[3]]), B.ULYS_ERR_ALIAS),   # two ranks, one buffer
    (dict(dq=[BO, BDQ[1], BDQ[2], BDQ[3]]), B.ULYS_ERR_ALIAS),       # over o
    (dict(dk=[BDK[0], BDK[1], BW, BDK[3]]), B.ULYS_ERR_ALIAS),       # over the workspace
])
def test_attn_bwd_push_rejects(lib, kw, expect):
    a = dict(q=BQ, k=BK, v=BV, o=BO, g=BG, lse=BL, dq=BDQ, dk=BDK, dv=BDV, rank=1, s=64, b=1,
             h=8, h_kv=4, d=128, P=4, causal=1, dtype=B.ULYS_BF16, ws=BW, wsb=1 << 24)
    a.update(kw)
    rc = B.ulys_attn_bwd_push(a["q"], a["k"], a["v"], a["o"], a["g"], a["lse"], a["dq"], a["dk"],
                              a["dv"], a["rank"], a["s"], a["b"], a["h"], a["h_kv"], a["d"],
                              a["P"], a["causal"], a["dtype"], a["ws"], a["wsb"])
    assert rc == expect
