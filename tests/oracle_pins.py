"""Pins for the CPU oracle: each pin checks the oracle against something other
than itself -- the pages' worked examples, closed forms, invariants, or an
independent library evaluation (numpy reshapes, torch's float64 attention).

Each pin takes the oracle library handle so the mutant tests can run the same
pins against deliberately broken builds of the oracle.  A pin raises
AssertionError on a mismatch.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

import oracle
from ulysses_head_sharded_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------- helpers
def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


def np_pack(x, s, b, h, d, P):
    """Pack by numpy reshapes: [s/P,b,(P,hp),d] -> [P,s/P,b,hp,d]."""
    return x.reshape(s // P, b, P, h // P, d).transpose(2, 0, 1, 3, 4).copy()


def np_seq2head(x_all, s, b, h, d, P):
    """Exchange by numpy reshapes: [j,t,b,(r,hp),d] -> [r,(j,t),b,hp,d]."""
    v = x_all.reshape(P, s // P, b, P, h // P, d).transpose(3, 0, 1, 2, 4, 5)
    return v.reshape(P, s, b, h // P, d).copy()


def torch_attention(q, k, v, causal):
    """Independent reference: torch's float64 scaled_dot_product_attention.

    q [s,b,nq,d], k/v [s,b,nkv,d] float64 numpy; KV heads are repeated by
    contiguous groups.  Returns (o [s,b,nq,d], lse [b,nq,s])."""
    s, b, nq, d = q.shape
    nkv = k.shape[2]
    G = nq // nkv
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 2, 0, 3)))  # [b,nq,s,d]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 2, 0, 3))).repeat_interleave(G, 1)
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 2, 0, 3))).repeat_interleave(G, 1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=bool(causal))
    sc = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) / math.sqrt(d)
    if causal:
        mask = torch.ones(s, s, dtype=torch.bool).tril()
        sc = sc.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(sc, dim=-1)
    return o.numpy().transpose(2, 0, 1, 3), lse.numpy()


def widen(a):
    return synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else \
        a.astype(np.float64)


# ---------------------------------------------------------------------------- layout pins
def pin_alltoall_worked_example(lib):
    """The two-rank AllToAll example of the collectives tutorial."""
    rows = _read_golden("alltoall_2rank.txt")
    code = {"A0": 0xA0, "A1": 0xA1, "B0": 0xB0, "B1": 0xB1}
    before = {}
    after = {}
    for r in rows:
        rank, rest = r.split(":")
        lhs, rhs = rest.split("->")
        before[int(rank)] = [code[t] for t in lhs.split()]
        after[int(rank)] = [code[t] for t in rhs.split()]
    P, s, b, h, d = 2, 2, 1, 2, 1
    x_all = np.array([before[0], before[1]], dtype=np.uint16).reshape(P, 1, b, h, d)
    y_all = oracle.seq2head(x_all, s, b, h, d, P, lib=lib)
    for r in range(P):
        assert y_all[r].reshape(-1).tolist() == after[r], (r, y_all[r].reshape(-1))
    # one token per rank: pack alone is the identity, the routing does the work
    for j in range(P):
        y = oracle.pack(x_all[j], s, b, h, d, P, lib=lib)
        assert y.reshape(-1).tolist() == before[j]
    back = oracle.head2seq(y_all, s, b, h, d, P, lib=lib)
    assert np.array_equal(back, x_all)


def pin_two_card_blocks(lib):
    """Two-card X_{i,j} example: keep X00, send X01, receive X10."""
    rows = _read_golden("two_card_blocks.txt")
    P, s, b, h, d = 2, 4, 1, 4, 3
    sl, hp = s // P, h // P
    # element value = 1000*i + 100*j + position inside the block
    x_all = np.empty((P, sl, b, h, d), dtype=np.int32)
    for i in range(P):
        for t in range(sl):
            for hh in range(h):
                for e in range(d):
                    j, k = divmod(hh, hp)
                    x_all[i, t, 0, hh, e] = 1000 * i + 100 * j + (t * hp + k) * d + e

    def block_label(arr):
        vals = np.unique(arr // 100)
        assert vals.size == 1, vals
        i, j = divmod(int(vals[0]), 10)
        return f"X{i}{j}"

    y_all = oracle.seq2head(x_all, s, b, h, d, P, lib=lib)
    for r_line in rows:
        rank, keeps, sends, receives, after = r_line.split()
        rank = int(rank)
        send = oracle.pack(x_all[rank], s, b, h, d, P, lib=lib)
        assert block_label(send[rank]) == keeps
        assert block_label(send[1 - rank]) == sends
        other = oracle.pack(x_all[1 - rank], s, b, h, d, P, lib=lib)
        assert block_label(other[rank]) == receives
        seq_blocks = [block_label(y_all[rank][c * sl:(c + 1) * sl]) for c in range(P)]
        assert ",".join(seq_blocks) == after
        # inside each block the order of tokens and heads is kept
        for c in range(P):
            blk = y_all[rank][c * sl:(c + 1) * sl] % 100
            assert np.array_equal(blk.reshape(-1), np.arange(sl * hp * d))


def pin_conservation_4card(lib):
    """4 cards, 16 tokens, 8 heads: 32*d_h elements per card before and after."""
    g = dict(line.split(None, 1) for line in _read_golden("shapes_4card_16tok_8head.txt"))
    P, s, h = int(g["P"]), int(g["s"]), int(g["h"])
    per = int(g["elements_per_card_over_d_h"])
    bsh = tuple(int(v) for v in g["before_shape"].split())
    ash = tuple(int(v) for v in g["after_shape"].split())
    for d in (1, 4, 64):
        b = 1
        x_all = np.arange(P * (s // P) * b * h * d, dtype=np.int64).reshape(P, s // P, b, h, d)
        y_all = oracle.seq2head(x_all, s, b, h, d, P, lib=lib)
        for r in range(P):
            assert x_all[r].shape[0] * x_all[r].shape[2] == bsh[0] * bsh[1]
            assert (y_all[r].shape[0], y_all[r].shape[2]) == ash
            assert x_all[r].size == per * d and y_all[r].size == per * d
        # nothing duplicated, nothing lost: the exchange is a permutation
        assert np.array_equal(np.sort(y_all.reshape(-1)), np.arange(x_all.size))


def pin_inverse_random_bits(lib):
    """unpack(pack(x)) = x and head2seq(seq2head(X)) = X on raw bit patterns."""
    cases = [(16, 1, 8, 64, 4, 4), (12, 2, 6, 5, 3, 2), (8, 2, 4, 3, 2, 8), (32, 1, 16, 7, 8, 2)]
    for n, (s, b, h, d, P, elt) in enumerate(cases):
        dt = {2: np.uint16, 4: np.uint32, 8: np.uint64}[elt]
        nbytes = (s // P) * b * h * d * elt
        x = synth.random_bits(109 + n, nbytes).view(dt).reshape(s // P, b, h, d)
        y = oracle.pack(x, s, b, h, d, P, lib=lib)
        assert np.array_equal(oracle.unpack(y, s, b, h, d, P, lib=lib), x)
        x_all = synth.random_bits(209 + n, nbytes * P).view(dt).reshape(P, s // P, b, h, d)
        y_all = oracle.seq2head(x_all, s, b, h, d, P, lib=lib)
        assert np.array_equal(oracle.head2seq(y_all, s, b, h, d, P, lib=lib), x_all)
    # float payloads survive untouched (NaN with payload, -0, subnormal, inf)
    special = np.array([0x7FC01234, 0x80000000, 0x00000001, 0x7F800000, 0xFFBFFFFF,
                        0x3F800000, 0x7FA00000, 0x807FFFFF], dtype=np.uint32)
    xs = special.view(np.float32).reshape(2, 1, 4, 1)
    ys = oracle.pack(xs, 4, 1, 4, 1, 2, lib=lib)
    assert np.array_equal(ys.view(np.uint32).reshape(-1),
                          np_pack(special.reshape(2, 1, 4, 1), 4, 1, 4, 1, 2).reshape(-1))


def pin_brute_force_tiny(lib):
    """Every P | s, P | h with s, h <= 12, b <= 2, d <= 3: index-valued inputs
    against numpy reshapes/transposes."""
    for s in range(1, 13):
        for h in range(1, 13):
            for P in range(1, min(s, h) + 1):
                if s % P or h % P:
                    continue
                for b in (1, 2):
                    for d in (1, 3):
                        n = (s // P) * b * h * d
                        x = np.arange(n, dtype=np.int32).reshape(s // P, b, h, d)
                        y = oracle.pack(x, s, b, h, d, P, lib=lib)
                        assert np.array_equal(y, np_pack(x, s, b, h, d, P)), (s, h, P, b, d)
                        assert np.array_equal(oracle.unpack(y, s, b, h, d, P, lib=lib), x)
                        if s <= 8 and h <= 8:
                            x_all = np.arange(n * P, dtype=np.int32).reshape(P, s // P, b, h, d)
                            y_all = oracle.seq2head(x_all, s, b, h, d, P, lib=lib)
                            assert np.array_equal(y_all, np_seq2head(x_all, s, b, h, d, P))


def pin_pack_then_route_is_seq2head(lib):
    """Pack on every rank, then route block r of every rank j to rank r in source
    order: the result is the whole exchange (the receive side is a view)."""
    for (s, b, h, d, P) in [(16, 1, 8, 4, 4), (12, 2, 6, 2, 3), (8, 2, 8, 1, 8)]:
        x_all = np.arange(s * b * h * d, dtype=np.int32).reshape(P, s // P, b, h, d)
        send = np.stack([oracle.pack(x_all[j], s, b, h, d, P, lib=lib) for j in range(P)])
        recv = np.stack([np.concatenate([send[j, r] for j in range(P)], axis=0)
                         for r in range(P)])
        assert np.array_equal(recv, oracle.seq2head(x_all, s, b, h, d, P, lib=lib))


# ---------------------------------------------------------------------------- attention pins
def _rand_share(seed, s, b, nq, nkv, d, dtype):
    q = synth.tensor(seed + 1, (s, b, nq, d), dtype)
    k = synth.tensor(seed + 2, (s, b, nkv, d), dtype)
    v = synth.tensor(seed + 3, (s, b, nkv, d), dtype)
    return q, k, v


def pin_attn_vs_torch(lib):
    """Random tiny shares, dense and causal, MHA and GQA, fp32 and bf16 inputs,
    against torch's float64 attention: max error 1e-12."""
    cases = [  # s, b, h, h_kv, P, d, dtype
        (1, 1, 2, 2, 1, 4, "f32"), (7, 1, 2, 2, 1, 8, "f32"), (16, 1, 8, 8, 4, 64, "f32"),
        (33, 2, 4, 2, 2, 8, "bf16"), (24, 1, 8, 2, 2, 16, "bf16"), (40, 2, 6, 3, 3, 4, "f32"),
        (19, 1, 4, 1, 1, 128, "bf16"),
    ]
    for n, (s, b, h, h_kv, P, d, dtype) in enumerate(cases):
        q, k, v = _rand_share(900 + 10 * n, s, b, h // P, h_kv // P, d, dtype)
        for causal in (False, True):
            o, lse = oracle.attn(q, k, v, s, b, h, h_kv, d, P, causal, lib=lib)
            o_t, lse_t = torch_attention(widen(q), widen(k), widen(v), causal)
            assert np.max(np.abs(o - o_t)) < 1e-12, (n, causal, np.max(np.abs(o - o_t)))
            assert np.max(np.abs(lse - lse_t)) < 1e-12, (n, causal)


def pin_attn_large_scores(lib):
    """Scores of size ~100 (Q scaled by 60): the max subtraction keeps exp finite."""
    s, b, nq, d = 24, 1, 2, 8
    q, k, v = _rand_share(950, s, b, nq, nq, d, "f32")
    q = (q * 60.0).astype(np.float32)
    for causal in (False, True):
        o, lse = oracle.attn(q, k, v, s, b, nq, nq, d, 1, causal, lib=lib)
        o_t, lse_t = torch_attention(widen(q), widen(k), widen(v), causal)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        assert np.max(np.abs(o - o_t)) < 1e-10 and np.max(np.abs(lse - lse_t)) < 1e-10


def pin_attn_closed_forms(lib):
    """Q = 0 gives uniform weights; V = c gives O = c; causal row 0 gives V_0
    exactly; s = 1 gives O = V."""
    s, b, nq, nkv, d = 13, 2, 4, 2, 8
    _, k, v = _rand_share(960, s, b, nq, nkv, d, "f32")
    q0 = np.zeros((s, b, nq, d), dtype=np.float32)
    vd = v.astype(np.float64)
    G = nq // nkv
    o, lse = oracle.attn(q0, k, v, s, b, nq, nkv, d, 1, True, lib=lib)
    csum = np.cumsum(vd, axis=0) / np.arange(1, s + 1)[:, None, None, None]
    for i in range(nq):
        assert np.max(np.abs(o[:, :, i] - csum[:, :, i // G])) < 1e-12
        assert np.max(np.abs(lse[:, i] - np.log(np.arange(1, s + 1))[None, :])) < 1e-12
    o, lse = oracle.attn(q0, k, v, s, b, nq, nkv, d, 1, False, lib=lib)
    mean = vd.mean(axis=0)
    for i in range(nq):
        assert np.max(np.abs(o[:, :, i] - mean[None, :, i // G])) < 1e-12
        assert np.max(np.abs(lse[:, i] - math.log(s))) < 1e-12
    # V = c
    q, k, _ = _rand_share(970, s, b, nq, nkv, d, "f32")
    vc = np.full((s, b, nkv, d), 0.375, dtype=np.float32)
    for causal in (False, True):
        o, _ = oracle.attn(q, k, vc, s, b, nq, nkv, d, 1, causal, lib=lib)
        assert np.max(np.abs(o - 0.375)) < 1e-12
    # causal row 0 sees only key 0: weight exactly 1
    o, lse = oracle.attn(q, k, v, s, b, nq, nkv, d, 1, True, lib=lib)
    for i in range(nq):
        assert np.array_equal(o[0, :, i], vd[0, :, i // G])
        sc0 = (q[0, :, i].astype(np.float64) * k[0, :, i // G].astype(np.float64)).sum(-1)
        assert np.max(np.abs(lse[:, i, 0] - sc0 / math.sqrt(d))) < 1e-12
    # s = 1
    q1, k1, v1 = _rand_share(980, 1, b, nq, nkv, d, "bf16")
    for causal in (False, True):
        o, _ = oracle.attn(q1, k1, v1, 1, b, nq, nkv, d, 1, causal, lib=lib)
        for i in range(nq):
            assert np.array_equal(o[0, :, i], widen(v1)[0, :, i // G])


def pin_attn_rows_sum_to_one(lib):
    """sum_j exp(S_j - LSE) = 1 with S from numpy, and V = 1 gives O = 1."""
    s, b, nq, d = 21, 1, 3, 16
    q, k, v = _rand_share(990, s, b, nq, nq, d, "bf16")
    qd, kd = widen(q), widen(k)
    for causal in (False, True):
        _, lse = oracle.attn(q, k, v, s, b, nq, nq, d, 1, causal, lib=lib)
        for i in range(nq):
            S = (qd[:, 0, i, :] @ kd[:, 0, i, :].T) / math.sqrt(d)
            if causal:
                S = np.where(np.tri(s, dtype=bool), S, -np.inf)
            tot = np.exp(S - lse[0, i][:, None]).sum(axis=1)
            assert np.max(np.abs(tot - 1.0)) < 1e-12
        ones = np.full(v.shape, 0x3F80, dtype=np.uint16)  # bf16 1.0
        o, _ = oracle.attn(q, k, ones, s, b, nq, nq, d, 1, causal, lib=lib)
        assert np.max(np.abs(o - 1.0)) < 1e-12


def pin_attn_equivariance(lib):
    """Dense: permuting K and V rows together leaves O unchanged; permuting Q
    rows permutes O rows."""
    s, b, nq, nkv, d = 17, 2, 4, 2, 8
    q, k, v = _rand_share(1000, s, b, nq, nkv, d, "f32")
    perm = np.argsort(synth.uniform01(1007, s))
    o, _ = oracle.attn(q, k, v, s, b, nq, nkv, d, 1, False, lib=lib)
    o2, _ = oracle.attn(q, k[perm], v[perm], s, b, nq, nkv, d, 1, False, lib=lib)
    assert np.max(np.abs(o - o2)) < 1e-12
    o3, _ = oracle.attn(q[perm], k, v, s, b, nq, nkv, d, 1, False, lib=lib)
    assert np.max(np.abs(o3 - o[perm])) < 1e-12


def pin_head_independence(lib):
    """Unsharded attention over all heads of the global tensors, sliced to rank
    r's heads, equals rank r's attention on its exchanged share (bit-exact)."""
    s, b, h, h_kv, d, P = 16, 2, 8, 4, 8, 2
    qg = synth.tensor(1101, (s, b, h, d), "bf16")
    kg = synth.tensor(1102, (s, b, h_kv, d), "bf16")
    vg = synth.tensor(1103, (s, b, h_kv, d), "bf16")
    for causal in (False, True):
        o_full, lse_full = oracle.attn(qg, kg, vg, s, b, h, h_kv, d, 1, causal, lib=lib)
        shards = lambda g, hh: g.reshape(P, s // P, b, hh, d)  # noqa: E731 - seq split
        qs = oracle.seq2head(shards(qg, h), s, b, h, d, P, lib=lib)
        ks = oracle.seq2head(shards(kg, h_kv), s, b, h_kv, d, P, lib=lib)
        vs = oracle.seq2head(shards(vg, h_kv), s, b, h_kv, d, P, lib=lib)
        hp = h // P
        for r in range(P):
            o_r, lse_r = oracle.attn(qs[r], ks[r], vs[r], s, b, h, h_kv, d, P, causal, lib=lib)
            assert np.array_equal(o_r, o_full[:, :, r * hp:(r + 1) * hp])
            assert np.array_equal(lse_r, lse_full[:, r * hp:(r + 1) * hp])


def pin_rows_match_full(lib):
    """attn_rows on a row sample equals the full evaluation at those rows."""
    s, b, nq, nkv, d = 50, 2, 4, 1, 16
    q, k, v = _rand_share(1200, s, b, nq, nkv, d, "bf16")
    rows = synth.row_sample(1207, s, b, nq, n_random=8, edge=3, tile_bounds=(16,))
    for causal in (False, True):
        o, lse = oracle.attn(q, k, v, s, b, nq, nkv, d, 1, causal, lib=lib)
        orows, lrows = oracle.attn_rows(q, k, v, rows, s, b, nq, nkv, d, 1, causal, lib=lib)
        assert np.array_equal(orows, o[rows[:, 2], rows[:, 0], rows[:, 1]])
        assert np.array_equal(lrows, lse[rows[:, 0], rows[:, 1], rows[:, 2]])


# ---------------------------------------------------------------------------- backward pins
def torch_attention_grads(q, k, v, dout, causal):
    """Independent reference for the backward: torch float64 autograd through
    scaled_dot_product_attention.  Shapes as torch_attention; returns
    (dq [s,b,nq,d], dk, dv [s,b,nkv,d]) with KV gradients summed over each
    contiguous GQA group."""
    s, b, nq, d = q.shape
    nkv = k.shape[2]
    G = nq // nkv
    to_t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 2, 0, 3)))  # noqa: E731
    qt = to_t(q).requires_grad_(True)
    kt = to_t(k).requires_grad_(True)
    vt = to_t(v).requires_grad_(True)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(G, 1), vt.repeat_interleave(G, 1), is_causal=bool(causal))
    o.backward(to_t(dout))
    back = lambda t: t.grad.numpy().transpose(2, 0, 1, 3)  # noqa: E731
    return back(qt), back(kt), back(vt)


def _rand_bwd(seed, s, b, nq, nkv, d, dtype):
    q, k, v = _rand_share(seed, s, b, nq, nkv, d, dtype)
    dout = synth.tensor(seed + 4, (s, b, nq, d), dtype)
    return q, k, v, dout


def pin_bwd_finite_differences(lib):
    """Every gradient element against a central difference of
    L = sum(dout * attn(q, k, v)) evaluated with the (pinned) forward oracle:
    the derivative of the definition, computed without the backward formulas.
    fp32 inputs; the step is taken between fp32 neighbours, so the forward sees
    the exact perturbed values."""
    for (s, b, nq, nkv, d, causal) in ((5, 1, 2, 1, 4, True), (4, 2, 2, 2, 3, False)):
        q, k, v, dout = _rand_bwd(1300 + s, s, b, nq, nkv, d, "f32")
        dq, dk, dv = oracle.attn_bwd(q, k, v, dout, s, b, nq, nkv, d, 1, causal, lib=lib)
        dd = dout.astype(np.float64)

        def loss(q_, k_, v_):
            o, _ = oracle.attn(q_, k_, v_, s, b, nq, nkv, d, 1, causal, lib=lib)
            return float((o * dd).sum())

        for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for idx in np.ndindex(arr.shape):
                hi, lo = arr.copy(), arr.copy()
                x = np.float64(arr[idx])
                hi[idx] = np.float32(x + 1e-3)
                lo[idx] = np.float32(x - 1e-3)
                args_hi = {"q": (hi, k, v), "k": (q, hi, v), "v": (q, k, hi)}[name]
                args_lo = {"q": (lo, k, v), "k": (q, lo, v), "v": (q, k, lo)}[name]
                fd = (loss(*args_hi) - loss(*args_lo)) / (np.float64(hi[idx]) - np.float64(lo[idx]))
                assert abs(fd - grad[idx]) < 1e-5 * (1.0 + abs(fd)), (name, idx, fd, grad[idx])


def pin_bwd_vs_torch(lib):
    """Random tiny shares, dense and causal, MHA and GQA, fp32 and bf16 inputs,
    against torch's float64 autograd: max error 1e-12."""
    cases = [  # s, b, nq, nkv, d, dtype
        (1, 1, 2, 2, 4, "f32"), (9, 1, 2, 2, 8, "f32"), (17, 2, 4, 2, 8, "bf16"),
        (12, 1, 8, 1, 16, "bf16"), (20, 2, 6, 3, 4, "f32"), (11, 1, 2, 1, 128, "bf16"),
    ]
    for n, (s, b, nq, nkv, d, dtype) in enumerate(cases):
        q, k, v, dout = _rand_bwd(1400 + 10 * n, s, b, nq, nkv, d, dtype)
        for causal in (False, True):
            got = oracle.attn_bwd(q, k, v, dout, s, b, nq, nkv, d, 1, causal, lib=lib)
            ref = torch_attention_grads(widen(q), widen(k), widen(v), widen(dout), causal)
            for name, g, r in zip(("dq", "dk", "dv"), got, ref):
                err = np.max(np.abs(g - r))
                assert err < 1e-12, (n, causal, name, err)


def pin_bwd_closed_forms(lib):
    """dout = 0 gives zero gradients; s = 1 gives dq = dk = 0 and dv = the
    group's summed dout; Q = 0 (uniform causal weights) gives
    dv_j = sum_{t >= j} dout_t / (t + 1); and the keys' dk always sum to zero
    (each softmax row's dS sums to zero)."""
    s, b, nq, nkv, d = 9, 2, 4, 2, 8
    G = nq // nkv
    q, k, v, dout = _rand_bwd(1500, s, b, nq, nkv, d, "f32")
    zero = np.zeros_like(dout)
    for causal in (False, True):
        for g in oracle.attn_bwd(q, k, v, zero, s, b, nq, nkv, d, 1, causal, lib=lib):
            assert np.max(np.abs(g)) == 0.0
        dq, dk, dv = oracle.attn_bwd(q, k, v, dout, s, b, nq, nkv, d, 1, causal, lib=lib)
        assert np.max(np.abs(dk.sum(axis=0))) < 1e-12
    q1, k1, v1, d1 = _rand_bwd(1510, 1, b, nq, nkv, d, "bf16")
    dq, dk, dv = oracle.attn_bwd(q1, k1, v1, d1, 1, b, nq, nkv, d, 1, True, lib=lib)
    assert np.max(np.abs(dq)) < 1e-15 and np.max(np.abs(dk)) < 1e-15
    dw = widen(d1)
    for g in range(nkv):
        assert np.max(np.abs(dv[0, :, g] - dw[0, :, g * G:(g + 1) * G].sum(axis=1))) < 1e-12
    q0 = np.zeros_like(q)
    _, _, dv = oracle.attn_bwd(q0, k, v, dout, s, b, nq, nkv, d, 1, True, lib=lib)
    dd = dout.astype(np.float64) / np.arange(1, s + 1)[:, None, None, None]
    tail = np.cumsum(dd[::-1], axis=0)[::-1]  # sum over t >= j
    for g in range(nkv):
        ref = tail[:, :, g * G:(g + 1) * G].sum(axis=2)
        assert np.max(np.abs(dv[:, :, g] - ref)) < 1e-12


def pin_bwd_rows_match_full(lib):
    """attn_bwd_rows at sampled query rows and keys equals the full evaluation."""
    s, b, nq, nkv, d = 30, 2, 4, 2, 8
    q, k, v, dout = _rand_bwd(1600, s, b, nq, nkv, d, "bf16")
    qrows = synth.row_sample(1607, s, b, nq, n_random=6, edge=2, tile_bounds=(16,))
    krows = synth.row_sample(1608, s, b, nkv, n_random=6, edge=2, tile_bounds=(16,))
    for causal in (False, True):
        dq, dk, dv = oracle.attn_bwd(q, k, v, dout, s, b, nq, nkv, d, 1, causal, lib=lib)
        rq, rk, rv = oracle.attn_bwd_rows(q, k, v, dout, qrows, krows, s, b, nq, nkv, d, 1,
                                          causal, lib=lib)
        assert np.array_equal(rq, dq[qrows[:, 2], qrows[:, 0], qrows[:, 1]])
        assert np.array_equal(rk, dk[krows[:, 2], krows[:, 0], krows[:, 1]])
        assert np.array_equal(rv, dv[krows[:, 2], krows[:, 0], krows[:, 1]])


def pin_bwd_sharded_chain(lib):
    """The backward of the whole Ulysses layer: the gradients of unsharded
    attention over all heads equal, per rank, the share's gradients computed
    after the seq->head exchange of q, k, v and dout and returned with the
    head->seq exchange (the backward exchanges are the forward ones with their
    axes swapped), bit-exact."""
    s, b, h, h_kv, d, P = 12, 2, 8, 4, 8, 2
    qg, kg, vg, dg = (synth.tensor(1700 + n, (s, b, hh, d), "bf16")
                      for n, hh in enumerate((h, h_kv, h_kv, h)))
    sh = lambda g, hh: g.reshape(P, s // P, b, hh, d)  # noqa: E731 - contiguous token chunks
    for causal in (False, True):
        dq_f, dk_f, dv_f = oracle.attn_bwd(qg, kg, vg, dg, s, b, h, h_kv, d, 1, causal, lib=lib)
        qs = oracle.seq2head(sh(qg, h), s, b, h, d, P, lib=lib)
        ks = oracle.seq2head(sh(kg, h_kv), s, b, h_kv, d, P, lib=lib)
        vs = oracle.seq2head(sh(vg, h_kv), s, b, h_kv, d, P, lib=lib)
        ds = oracle.seq2head(sh(dg, h), s, b, h, d, P, lib=lib)
        grads = [oracle.attn_bwd(qs[r], ks[r], vs[r], ds[r], s, b, h, h_kv, d, P, causal, lib=lib)
                 for r in range(P)]
        for n, (full, hh) in enumerate(((dq_f, h), (dk_f, h_kv), (dv_f, h_kv))):
            back = oracle.head2seq(np.stack([g[n] for g in grads]), s, b, hh, d, P, lib=lib)
            assert np.array_equal(back.reshape(s, b, hh, d), full), (n, causal)


LAYOUT_PINS = [pin_alltoall_worked_example, pin_two_card_blocks, pin_conservation_4card,
               pin_inverse_random_bits, pin_brute_force_tiny, pin_pack_then_route_is_seq2head]
ATTN_PINS = [pin_attn_vs_torch, pin_attn_large_scores, pin_attn_closed_forms,
             pin_attn_rows_sum_to_one, pin_attn_equivariance, pin_head_independence,
             pin_rows_match_full]
BWD_PINS = [pin_bwd_finite_differences, pin_bwd_vs_torch, pin_bwd_closed_forms,
            pin_bwd_rows_match_full, pin_bwd_sharded_chain]
# ---------------------------------------------------------------------------- KV replication pins
def _route(blocks_per_rank, P):
    """The exchange's routing: rank r receives block r of every sender j, in
    source order, concatenated along the sequence."""
    return [np.concatenate([blocks_per_rank[j][r] for j in range(P)], axis=0) for r in range(P)]


def pin_kv_replication_example(lib):
    """One KV head on four ranks: the plain head split leaves ranks 1-3 with no
    KV head; with replication every rank holds the head's whole sequence."""
    rows = _read_golden("kv_replication_1head_4rank.txt")
    P, s, b, h_kv, d = 4, 4, 1, 1, 1
    heads = [int(t) for t in rows[0].split(":")[1].split()]
    # the plain split of the head axis into P parts (the first parts take the
    # remainder) -- what the page shows -- and the basic method rejects it
    assert heads == [len(part) for part in np.array_split(np.arange(h_kv), P)]
    with np.testing.assert_raises(ValueError):
        oracle.pack(np.zeros(1, np.uint16), s, b, h_kv, d, P, lib=lib)
    code = {f"K{j}": 0x100 + j for j in range(P)}
    shards, expect = {}, {}
    for r in rows[1:]:
        rank, rest = r.split(":")
        lhs, rhs = rest.split("->")
        shards[int(rank)] = np.array([code[t] for t in lhs.split()], dtype=np.uint16)
        expect[int(rank)] = [code[t] for t in rhs.split()]
    sent = [oracle.pack_kv(shards[j].reshape(1, 1, 1, 1), s, b, h_kv, d, P, lib=lib)
            for j in range(P)]
    got = _route(sent, P)
    for r in range(P):
        assert got[r].reshape(-1).tolist() == expect[r], (r, got[r].reshape(-1))


def pin_pack_kv_brute_force(lib):
    """Every tiny shape with h_kv < P, P | h_kv * k, values equal to their flat
    index: rank r's block is KV head r*h_kv//P (numpy indexing); with P | h_kv
    the replicated pack is the plain one."""
    for P in (2, 3, 4, 6, 8):
        for h_kv in range(1, 2 * P + 1):
            if not (h_kv % P == 0 or P % h_kv == 0):
                continue
            for b in (1, 2):
                s, d = 2 * P, 3
                x = np.arange((s // P) * b * h_kv * d, dtype=np.int32).reshape(s // P, b, h_kv, d)
                y = oracle.pack_kv(x, s, b, h_kv, d, P, lib=lib)
                if h_kv % P == 0:
                    ref = np_pack(x, s, b, h_kv, d, P)
                else:
                    ref = np.stack([x[:, :, r * h_kv // P][:, :, None] for r in range(P)])
                assert y.shape == ref.shape and np.array_equal(y, ref), (P, h_kv, b)


def _bf16_rne_bits(f32):
    """float32 -> bf16 bits, nearest-even, by the usual integer trick."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def pin_unpack_kv_sum(lib):
    """Backward of the replication.  Replicate-then-sum multiplies by R = P/h_kv
    exactly (R a power of two); with P | h_kv it is the plain unpack; and a sum
    of R = 2 bf16 blocks (exact in float32 when the exponents are close) rounds
    like the independent integer nearest-even conversion."""
    for P, h_kv in ((4, 1), (8, 2), (8, 4), (16, 4)):
        s, b, d = 2 * P, 2, 8
        R = P // h_kv
        for dt in ("f32", "bf16"):
            x = synth.tensor(1700 + P + h_kv, (s // P, b, h_kv, d), dt)
            y = oracle.pack_kv(x, s, b, h_kv, d, P, lib=lib)
            z = oracle.unpack_kv_sum(y, s, b, h_kv, d, P, lib=lib)
            assert np.array_equal(widen(z), R * widen(x)), (P, h_kv, dt)
    s, b, d, P, h_kv = 8, 1, 4, 4, 4
    x = synth.tensor(1710, (s // P, b, h_kv, d), "bf16")
    y = oracle.pack_kv(x, s, b, h_kv, d, P, lib=lib)
    assert np.array_equal(oracle.unpack_kv_sum(y, s, b, h_kv, d, P, lib=lib), x)
    # rounding: blocks with magnitudes in [1, 2) so that pair sums are exact in float32
    P, h_kv, s, b, d = 4, 2, 4, 1, 64
    mags = 1.0 + synth.uniform01(1720, P * d).astype(np.float32)
    signs = np.where(synth.uniform01(1721, P * d) < 0.5, -1.0, 1.0).astype(np.float32)
    y = _bf16_rne_bits(mags * signs).reshape(P, 1, b, 1, d)
    got = oracle.unpack_kv_sum(y, s, b, h_kv, d, P, lib=lib)
    yf = widen(y).astype(np.float32).reshape(P, d)
    for g in range(h_kv):
        ref = _bf16_rne_bits(yf[2 * g] + yf[2 * g + 1])
        assert np.array_equal(got[0, 0, g], ref), g


def _gqa_case(seed, s, b, h, h_kv, d, dt):
    q = synth.tensor(seed, (s, b, h, d), dt)
    k = synth.tensor(seed + 1, (s, b, h_kv, d), dt)
    v = synth.tensor(seed + 2, (s, b, h_kv, d), dt)
    return q, k, v


def pin_kv_replication_head_independence(lib):
    """Unsharded GQA attention with fewer KV heads than ranks, sliced to rank
    r's query heads, equals rank r's attention on its exchanged share, whose
    single KV head arrived by replication (bit for bit in the oracle)."""
    for (s, b, h, h_kv, P, causal) in ((16, 1, 8, 2, 4, True), (12, 2, 8, 1, 4, False),
                                       (16, 1, 16, 2, 8, True)):
        d = 8
        q, k, v = _gqa_case(1730 + h_kv, s, b, h, h_kv, d, "bf16")
        o_full, lse_full = oracle.attn(q, k, v, s, b, h, h_kv, d, 1, causal, lib=lib)
        sl, hp = s // P, h // P
        qs = _route([oracle.pack(q[j * sl:(j + 1) * sl], s, b, h, d, P, lib=lib)
                     for j in range(P)], P)
        ks = _route([oracle.pack_kv(k[j * sl:(j + 1) * sl], s, b, h_kv, d, P, lib=lib)
                     for j in range(P)], P)
        vs = _route([oracle.pack_kv(v[j * sl:(j + 1) * sl], s, b, h_kv, d, P, lib=lib)
                     for j in range(P)], P)
        for r in range(P):
            # one KV head per share: the attention of the share has h_kv_eff = P
            o, lse = oracle.attn(qs[r], ks[r], vs[r], s, b, h, P, d, P, causal, lib=lib)
            assert np.array_equal(o, o_full[:, :, r * hp:(r + 1) * hp]), (r, s, h_kv)
            assert np.array_equal(lse, lse_full[:, r * hp:(r + 1) * hp]), (r, s, h_kv)


def pin_kv_replication_backward_chain(lib):
    """The backward with replicated KV heads: each rank's dK, dV (fp64, rounded
    to float32) go back through the head->seq exchange and the copies of a KV
    head are summed (unpack_kv_sum); the result equals the unsharded
    gradients to float32 rounding."""
    s, b, h, h_kv, P, d = 16, 1, 8, 2, 4, 8
    sl = s // P
    for causal in (False, True):
        q, k, v = _gqa_case(1740, s, b, h, h_kv, d, "f32")
        dout = synth.tensor(1743, (s, b, h, d), "f32")
        _, dk_f, dv_f = oracle.attn_bwd(q, k, v, dout, s, b, h, h_kv, d, 1, causal, lib=lib)
        share = lambda t, kv: _route([(oracle.pack_kv if kv else oracle.pack)(  # noqa: E731
            t[j * sl:(j + 1) * sl], s, b, h_kv if kv else h, d, P, lib=lib) for j in range(P)], P)
        qs, ks, vs, gs = share(q, False), share(k, True), share(v, True), share(dout, False)
        dks, dvs = [], []
        for r in range(P):
            _, dk, dv = oracle.attn_bwd(qs[r], ks[r], vs[r], gs[r], s, b, h, P, d, P, causal,
                                        lib=lib)
            dks.append(dk.astype(np.float32))
            dvs.append(dv.astype(np.float32))
        for grads, full in ((dks, dk_f), (dvs, dv_f)):
            for j in range(P):  # rank j gets sequence segment j of every rank's gradient
                recv = np.stack([grads[r][j * sl:(j + 1) * sl] for r in range(P)])
                got = oracle.unpack_kv_sum(recv, s, b, h_kv, d, P, lib=lib).astype(np.float64)
                ref = full[j * sl:(j + 1) * sl]
                assert np.max(np.abs(got - ref)) <= 4e-7 * max(1.0, np.max(np.abs(ref))), \
                    (causal, j)


# ---------------------------------------------------------------------------- merge pins
def _chunk_attn(q, k, v, i, j, c, b, nq, nkv, d, causal, lib):
    """Attention of query chunk i against key chunk j (c tokens each): with a
    causal mask, causal inside the diagonal block and dense for an earlier key
    chunk; without one, dense."""
    qi, kj, vj = q[i * c:(i + 1) * c], k[j * c:(j + 1) * c], v[j * c:(j + 1) * c]
    return oracle.attn(qi, kj, vj, c, b, nq, nkv, d, 1, causal and i == j, lib=lib)


def _merge_all(parts, lib):
    o, lse = parts[0]
    for o2, lse2 in parts[1:]:
        o, lse = oracle.attn_merge(o, lse, o2, lse2, lib=lib)
    return o, lse


def pin_merge_recovers_full_attention(lib):
    """Attention over all keys equals the merge of attention over disjoint key
    chunks: dense over two chunks, and causal over four chunks merged in the
    order a four-rank ring delivers them to rank 3 (KV_3, KV_2, KV_1, KV_0),
    to 1e-12."""
    for dt, (c, b, nq, nkv, d) in (("f32", (6, 2, 4, 2, 8)), ("bf16", (5, 1, 2, 1, 16))):
        for causal, n in ((False, 2), (True, 4)):
            s = n * c
            q = synth.tensor(1800 + s, (s, b, nq, d), dt)
            k = synth.tensor(1801 + s, (s, b, nkv, d), dt)
            v = synth.tensor(1802 + s, (s, b, nkv, d), dt)
            o_full, lse_full = oracle.attn(q, k, v, s, b, nq, nkv, d, 1, causal, lib=lib)
            for i in range(n):
                keys = range(i, -1, -1) if causal else range(n)  # later chunks are skipped
                o, lse = _merge_all([_chunk_attn(q, k, v, i, j, c, b, nq, nkv, d, causal, lib)
                                     for j in keys], lib)
                ref_o = o_full[i * c:(i + 1) * c]
                ref_l = lse_full[:, :, i * c:(i + 1) * c]
                assert np.max(np.abs(o - ref_o)) < 1e-12, (dt, causal, i)
                assert np.max(np.abs(lse - ref_l)) < 1e-12, (dt, causal, i)


def pin_merge_special_cases(lib):
    """An empty partial (lse = -inf) leaves the other exactly; two empties give
    O = 0 and lse = -inf; the merge is symmetric bit for bit; merging a result
    with itself keeps O and adds ln 2 to lse."""
    s, b, hp, d = 7, 2, 3, 5
    rows = s * b * hp
    o_a = synth.normal_f32(1810, rows * d).astype(np.float64).reshape(s, b, hp, d)
    o_b = synth.normal_f32(1811, rows * d).astype(np.float64).reshape(s, b, hp, d)
    l_a = 3.0 * synth.normal_f32(1812, rows).astype(np.float64).reshape(b, hp, s)
    l_b = 3.0 * synth.normal_f32(1813, rows).astype(np.float64).reshape(b, hp, s)
    empty = np.full((b, hp, s), -np.inf)
    o, lse = oracle.attn_merge(o_a, l_a, o_b, empty, lib=lib)
    assert np.array_equal(o, o_a) and np.array_equal(lse, l_a)
    o, lse = oracle.attn_merge(o_a, empty, o_b, empty, lib=lib)
    assert np.array_equal(o, np.zeros_like(o)) and np.all(lse == -np.inf)
    o1, l1 = oracle.attn_merge(o_a, l_a, o_b, l_b, lib=lib)
    o2, l2 = oracle.attn_merge(o_b, l_b, o_a, l_a, lib=lib)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o, lse = oracle.attn_merge(o_a, l_a, o_a, l_a, lib=lib)
    assert np.max(np.abs(o - o_a)) < 1e-15 * (1 + np.max(np.abs(o_a)))
    assert np.max(np.abs(lse - (l_a + math.log(2.0)))) < 1e-14 * (1 + np.max(np.abs(l_a)))
    # weights by hand: lse_a = ln 3, lse_b = ln 1 -> O = (3 O_a + O_b) / 4, lse = ln 4
    o, lse = oracle.attn_merge(o_a, np.full((b, hp, s), math.log(3.0)), o_b,
                               np.zeros((b, hp, s)), lib=lib)
    assert np.max(np.abs(o - (3 * o_a + o_b) / 4)) < 4e-15 * (1 + np.max(np.abs(o_a)))
    assert np.max(np.abs(lse - math.log(4.0))) < 1e-15
    # the row map: lse [b, hp, s] pairs with o [s, b, hp, :] -- one row at a time
    la, lb = l_a.copy(), l_b.copy()
    la[1, 2, 4], lb[1, 2, 4] = 0.0, -np.inf
    o, lse = oracle.attn_merge(o_a, la, o_b, lb, lib=lib)
    assert np.array_equal(o[4, 1, 2], o_a[4, 1, 2]) and lse[1, 2, 4] == 0.0


def pin_usp_four_by_two(lib):
    """The USP arrangement of the SP/CP page at small scale: eight cards, a
    Ulysses degree of 4 and a ring degree of 2.  Each card starts with s/8
    tokens; inside each group of four the Ulysses exchange gives every card
    its group's s/2 tokens for h/4 heads; the two cards holding the same heads
    in the two groups then exchange K and V, and each merges attention over
    its own half (causal) with attention over the other group's half (dense
    when that half comes first, skipped when it comes after).  The head->seq
    exchange inside each group then returns outputs equal to unsharded causal
    attention, to 1e-12."""
    U, Rg = 4, 2
    s, b, h, h_kv, d = 16, 1, 8, 4, 4
    half, hp, hkvp = s // Rg, h // U, h_kv // U
    q = synth.tensor(1820, (s, b, h, d), "bf16")
    k = synth.tensor(1821, (s, b, h_kv, d), "bf16")
    v = synth.tensor(1822, (s, b, h_kv, d), "bf16")
    o_full, _ = oracle.attn(q, k, v, s, b, h, h_kv, d, 1, True, lib=lib)
    # group g holds tokens [g*half, (g+1)*half); card u of group g holds s/8 of them
    shares = {}
    for g in range(Rg):
        grp = slice(g * half, (g + 1) * half)
        xq = q[grp].reshape(U, half // U, b, h, d)  # the four cards' shards, in order
        xk = k[grp].reshape(U, half // U, b, h_kv, d)
        xv = v[grp].reshape(U, half // U, b, h_kv, d)
        sq = oracle.seq2head(xq, half, b, h, d, U, lib=lib)      # [U, half, b, hp, d]
        sk = oracle.seq2head(xk, half, b, h_kv, d, U, lib=lib)
        sv = oracle.seq2head(xv, half, b, h_kv, d, U, lib=lib)
        for u in range(U):
            shares[g, u] = (sq[u], sk[u], sv[u])
    for g in range(Rg):
        outs = []
        for u in range(U):
            qs, ks, vs = shares[g, u]
            parts = [oracle.attn(qs, ks, vs, half, b, hp, hkvp, d, 1, True, lib=lib)]
            for g2 in range(g):  # the other group's K/V, received around the ring
                _, k2, v2 = shares[g2, u]
                parts.append(oracle.attn(qs, k2, v2, half, b, hp, hkvp, d, 1, False, lib=lib))
            outs.append(_merge_all(parts, lib)[0])
        back = oracle.head2seq(np.stack(outs), half, b, h, d, U, lib=lib)  # [U, half/U, b, h, d]
        got = back.reshape(half, b, h, d)
        assert np.max(np.abs(got - o_full[g * half:(g + 1) * half])) < 1e-12, g


MERGE_PINS = [pin_merge_recovers_full_attention, pin_merge_special_cases, pin_usp_four_by_two]

KV_PINS = [pin_kv_replication_example, pin_pack_kv_brute_force, pin_unpack_kv_sum,
           pin_kv_replication_head_independence, pin_kv_replication_backward_chain]

ALL_PINS = LAYOUT_PINS + ATTN_PINS + BWD_PINS + KV_PINS + MERGE_PINS
