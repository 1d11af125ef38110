"""GPU parity of the attention backward (ulys_attn_bwd) against the fp64 CPU
oracle (orc_attn_bwd), through the C ABI.

The oracle recomputes everything from q, k, v and dout.  The GPU kernels take
the forward's o and lse as inputs; the small cases feed them the oracle's own
forward result (o rounded to bf16 once, lse to fp32), so they test the
backward alone, and the chain cases feed them the GPU forward's outputs.

Tolerance: max |g_gpu - g_ref| <= 2e-2 * max(1, max |g_ref|) per gradient
tensor.  The GPU rounds P and dS to bf16 before the products that consume
them (relative 2^-9 per term), uses the bf16-rounded o in D = rowsum(dout * o)
and rounds each gradient once to bf16 (relative 2^-9); 2e-2 of the tensor's
scale is the forward's bf16 bound carried over to gradients whose magnitude
exceeds 1."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import Guarded, as_f64, dev, from_dev, share_inputs, to_dev
from ulysses_head_sharded_amd import binding, synth
from ulysses_head_sharded_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

REL = 2e-2


def check(name, got, ref, rel=REL):
    err = np.max(np.abs(as_f64(got) - ref)) if ref.size else 0.0
    bound = rel * max(1.0, float(np.max(np.abs(ref))) if ref.size else 1.0)
    print(f"  {name}: max err {err:.3e} (bound {bound:.3e})", flush=True)
    assert err <= bound, (name, err, bound)


def oracle_fwd_inputs(q, k, v, s, b, h, h_kv, d, P, causal):
    """The oracle's forward: o rounded once to bf16 bits, lse to fp32."""
    o, lse = oracle.attn(q, k, v, s, b, h, h_kv, d, P, causal)
    return synth.f32_to_bf16_bits(o.astype(np.float32)), lse.astype(np.float32)


def gpu_bwd(q, k, v, o, lse, dout, s, b, h, h_kv, d, P, causal):
    """ulys_attn_bwd with guarded outputs and workspace; host arrays in and out
    (bf16 bit patterns or float32, which selects the kernels)."""
    dev()
    hp, hkvp = h // P, h_kv // P
    f32 = q.dtype == np.float32
    tdt, code = (torch.float32, binding.ULYS_F32) if f32 else (torch.bfloat16, binding.ULYS_BF16)
    qd, kd, vd, od, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(o), to_dev(dout)
    ld = to_dev(np.ascontiguousarray(lse, dtype=np.float32))
    dq = Guarded((s, b, hp, d), tdt)
    dk = Guarded((s, b, hkvp, d), tdt)
    dv = Guarded((s, b, hkvp, d), tdt)
    nbytes = binding.ulys_attn_bwd_workspace_size(s, b, h, h_kv, d, P, int(causal), code)
    assert nbytes > 0, binding.ulys_status_string(int(nbytes))
    ws = Guarded((nbytes,), torch.uint8)
    rc = binding.ulys_attn_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), od.data_ptr(),
                               gd.data_ptr(), ld.data_ptr(), dq.tensor.data_ptr(),
                               dk.tensor.data_ptr(), dv.tensor.data_ptr(), s, b, h, h_kv, d, P,
                               int(causal), code, ws.tensor.data_ptr(), nbytes,
                               torch.cuda.current_stream().cuda_stream)
    assert rc == 0, binding.ulys_status_string(rc)
    torch.cuda.synchronize()
    for g in (dq, dk, dv, ws):
        assert g.guards_intact()
    return from_dev(dq.tensor), from_dev(dk.tensor), from_dev(dv.tensor)


def gpu_fwd(q, k, v, s, b, h, h_kv, d, P, causal):
    """The GPU forward through the workspace entry point (o and lse)."""
    dev()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o, lse = binding.attn_fwd(qd, kd, vd, P=P, causal=causal, lse=True)
    torch.cuda.synchronize()
    return from_dev(o), from_dev(lse)


# s spans several 32-query and 64-key tiles with ragged tails; heads cover MHA,
# GQA 4:1 and 8:1 (two subgroups per KV head in the dq kernel) and MQA; both
# head sizes (d_h = 64 on a subset of the lengths)
SMALL = []
for (s, b) in [(1, 1), (5, 2), (32, 1), (33, 1), (64, 1), (100, 2), (200, 1), (321, 1), (640, 1)]:
    for (h, h_kv, P) in [(2, 2, 1), (8, 2, 2), (16, 2, 1), (8, 8, 4), (4, 1, 1)]:
        if s % P:
            continue
        for causal in (False, True):
            SMALL.append((s, b, h, h_kv, 128, P, causal))
            if s in (1, 33, 100, 321, 640):
                SMALL.append((s, b, h, h_kv, 64, P, causal))


@pytest.mark.parametrize("s,b,h,h_kv,d,P,causal", SMALL)
def test_bwd_small_parity(s, b, h, h_kv, d, P, causal):
    print(f"case bwd s={s} b={b} h={h} h_kv={h_kv} d={d} P={P} causal={causal}", flush=True)
    q, k, v = share_inputs(7, s, b, h // P, h_kv // P, d, "bf16")
    dout = synth.tensor(704, (s, b, h // P, d), "bf16")
    o, lse = oracle_fwd_inputs(q, k, v, s, b, h, h_kv, d, P, causal)
    dq, dk, dv = gpu_bwd(q, k, v, o, lse, dout, s, b, h, h_kv, d, P, causal)
    rq, rk, rv = oracle.attn_bwd(q, k, v, dout, s, b, h, h_kv, d, P, causal)
    check("dq", dq, rq)
    check("dk", dk, rk)
    check("dv", dv, rv)


# The fp32 kernels on the same shapes up to s = 321.  The oracle's forward o
# and lse enter as float32; everything on the GPU is fp32, so the bound is the
# fp32 forward's 1e-4 (of each gradient's scale past 1).
REL_F32 = 1e-4
SMALL_F32 = [c for c in SMALL if c[0] <= 321]


@pytest.mark.parametrize("s,b,h,h_kv,d,P,causal", SMALL_F32)
def test_bwd_small_parity_f32(s, b, h, h_kv, d, P, causal):
    print(f"case bwd f32 s={s} b={b} h={h} h_kv={h_kv} d={d} P={P} causal={causal}", flush=True)
    q, k, v = share_inputs(7, s, b, h // P, h_kv // P, d, "f32")
    dout = synth.tensor(704, (s, b, h // P, d), "f32")
    o, lse = oracle.attn(q, k, v, s, b, h, h_kv, d, P, causal)
    dq, dk, dv = gpu_bwd(q, k, v, o.astype(np.float32), lse.astype(np.float32), dout, s, b, h,
                         h_kv, d, P, causal)
    rq, rk, rv = oracle.attn_bwd(q, k, v, dout, s, b, h, h_kv, d, P, causal)
    check("dq", dq, rq, REL_F32)
    check("dk", dk, rk, REL_F32)
    check("dv", dv, rv, REL_F32)


@pytest.mark.parametrize("s,b,h,h_kv,d,P,causal", [
    (300, 2, 8, 2, 128, 2, True), (257, 1, 4, 4, 64, 1, False), (16, 1, 8, 8, 64, 4, False)])
def test_bwd_chain_after_gpu_forward_f32(s, b, h, h_kv, d, P, causal):
    """The fp32 backward fed by the fp32 GPU forward's o and lse (the last
    case is the tiny workload's share)."""
    print(f"case chain f32 s={s} b={b} h={h} h_kv={h_kv} d={d} P={P} causal={causal}",
          flush=True)
    q, k, v = share_inputs(8, s, b, h // P, h_kv // P, d, "f32")
    dout = synth.tensor(804, (s, b, h // P, d), "f32")
    o, lse = gpu_fwd(q, k, v, s, b, h, h_kv, d, P, causal)
    dq, dk, dv = gpu_bwd(q, k, v, o, lse, dout, s, b, h, h_kv, d, P, causal)
    rq, rk, rv = oracle.attn_bwd(q, k, v, dout, s, b, h, h_kv, d, P, causal)
    check("dq", dq, rq, REL_F32)
    check("dk", dk, rk, REL_F32)
    check("dv", dv, rv, REL_F32)


@pytest.mark.parametrize("s,b,h,h_kv,d,P,causal", [
    (300, 2, 8, 2, 128, 2, True), (257, 1, 4, 4, 128, 1, False), (1024, 1, 2, 2, 128, 1, True),
    (1024, 1, 2, 2, 128, 1, False), (2048, 1, 8, 2, 128, 1, True), (2048, 1, 8, 2, 64, 1, True),
    (1000, 2, 4, 4, 64, 2, False)])
def test_bwd_chain_after_gpu_forward(s, b, h, h_kv, d, P, causal):
    """The backward fed by the GPU forward's o and lse (as a training step)."""
    print(f"case chain s={s} b={b} h={h} h_kv={h_kv} d={d} P={P} causal={causal}", flush=True)
    q, k, v = share_inputs(8, s, b, h // P, h_kv // P, d, "bf16")
    dout = synth.tensor(804, (s, b, h // P, d), "bf16")
    o, lse = gpu_fwd(q, k, v, s, b, h, h_kv, d, P, causal)
    dq, dk, dv = gpu_bwd(q, k, v, o, lse, dout, s, b, h, h_kv, d, P, causal)
    rq, rk, rv = oracle.attn_bwd(q, k, v, dout, s, b, h, h_kv, d, P, causal)
    check("dq", dq, rq)
    check("dk", dk, rk)
    check("dv", dv, rv)


def test_bwd_layer_chain_with_exchanges():
    """The whole layer's backward on one GPU: every rank's seq-sharded output
    gradient is packed (ulys_pack_seq2head), routed as the exchange would,
    differentiated on its share (ulys_attn_bwd after ulys_attn_fwd), routed
    back and unpacked (ulys_unpack_head2seq); the result equals the oracle's
    gradients of unsharded attention over all heads, sharded by sequence."""
    s, b, h, h_kv, d, P, causal = 128, 2, 8, 4, 128, 2, True
    sl, hp, hkvp = s // P, h // P, h_kv // P
    qg, kg, vg, gg = (synth.tensor(1900 + n, (s, b, hh, d), "bf16")
                      for n, hh in enumerate((h, h_kv, h_kv, h)))
    dev()

    def exchange(shards, hh):
        """seq->head exchange on the GPU: pack every rank's shard, route block r
        of every sender to rank r (source order)."""
        packed = [binding.pack_seq2head(to_dev(x), P) for x in shards]
        return [torch.cat([packed[j][r] for j in range(P)], dim=0).reshape(s, b, hh // P, d)
                for r in range(P)]

    def back(shares, hh):
        """head->seq exchange on the GPU: block j of every rank to rank j, unpack."""
        out = []
        for j in range(P):
            recv = torch.stack([sh.reshape(P, sl, b, hh // P, d)[j] for sh in shares])
            out.append(from_dev(binding.unpack_head2seq(recv.contiguous())))
        return np.concatenate(out, axis=0)

    seq = lambda g: [g[j * sl:(j + 1) * sl] for j in range(P)]  # noqa: E731
    qs, ks, vs, gs = (exchange(seq(t), hh) for t, hh in ((qg, h), (kg, h_kv), (vg, h_kv), (gg, h)))
    grads = []
    for r in range(P):
        o, lse = binding.attn_fwd(qs[r], ks[r], vs[r], P=P, causal=causal, lse=True)
        grads.append(binding.attn_bwd(qs[r], ks[r], vs[r], o, gs[r], lse, P=P, causal=causal))
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(qg, kg, vg, gg, s, b, h, h_kv, d, 1, causal)
    check("dq", back([g[0] for g in grads], h), rq)
    check("dk", back([g[1] for g in grads], h_kv), rk)
    check("dv", back([g[2] for g in grads], h_kv), rv)


def test_bwd_deterministic():
    s, b, h, h_kv, d, P = 322, 1, 8, 2, 128, 2
    q, k, v = share_inputs(9, s, b, h // P, h_kv // P, d, "bf16")
    dout = synth.tensor(904, (s, b, h // P, d), "bf16")
    o, lse = oracle_fwd_inputs(q, k, v, s, b, h, h_kv, d, P, True)
    a = gpu_bwd(q, k, v, o, lse, dout, s, b, h, h_kv, d, P, True)
    c = gpu_bwd(q, k, v, o, lse, dout, s, b, h, h_kv, d, P, True)
    for x, y in zip(a, c):
        assert np.array_equal(x, y)


# full-size shares: the GPU forward then backward; the oracle computes sampled
# query rows (dq) and late keys (dk, dv: a causal key j is seen only by rows
# t >= j, so keys near the end are cheap to evaluate one by one)
FULL = {"gpt1.2b-32k": (96, 24, 16), "mha-128k": (24, 8, 6)}


@pytest.mark.parametrize("name", list(FULL))
def test_bwd_full_size_sampled(name):
    w = WORKLOADS[name]
    n_random, edge, n_keys = FULL[name]
    print(f"case bwd {name}: s={w.s} b={w.b} hp={w.hp} hkvp={w.hkvp}", flush=True)
    q, k, v = share_inputs(w.c, w.s, w.b, w.hp, w.hkvp, w.d, w.dtype)
    dout = synth.tensor(100 * w.c + 4, (w.s, w.b, w.hp, w.d), w.dtype)
    o, lse = gpu_fwd(q, k, v, w.s, w.b, w.h, w.h_kv, w.d, w.P, w.causal)
    dq, dk, dv = gpu_bwd(q, k, v, o, lse, dout, w.s, w.b, w.h, w.h_kv, w.d, w.P, w.causal)
    qrows = synth.row_sample(100 * w.c + 7, w.s, w.b, w.hp, n_random=n_random, edge=edge,
                             tile_bounds=(32, 64))
    js = w.s - 1 - np.arange(n_keys) * 3
    krows = np.stack([np.arange(n_keys) % w.b, np.arange(n_keys) % w.hkvp, js], axis=1)
    rq, rk, rv = oracle.attn_bwd_rows(q, k, v, dout, qrows, krows, w.s, w.b, w.h, w.h_kv, w.d,
                                      w.P, w.causal)
    check("dq rows", dq[qrows[:, 2], qrows[:, 0], qrows[:, 1]], rq)
    check("dk keys", dk[krows[:, 2], krows[:, 0], krows[:, 1]], rk)
    check("dv keys", dv[krows[:, 2], krows[:, 0], krows[:, 1]], rv)
    # every softmax row's dS sums to zero, so the keys' dk sum to zero (up to
    # rounding) for each (batch, KV head); and every gradient is finite
    dkf = as_f64(dk)
    for g in (dq, dk, dv):
        assert np.all(np.isfinite(as_f64(g)))
    tot = np.abs(dkf.sum(axis=0)).max()
    scale = np.abs(dkf).sum(axis=0).max()
    print(f"  |sum_j dk_j| = {tot:.3e} against sum_j |dk_j| = {scale:.3e}", flush=True)
    assert tot <= 1e-2 * scale
    # every softmax row sums to one, so sum_j dv_j = sum over the group's query
    # heads and all rows of dout, for each (batch, KV head): a check of dv at
    # every key, early ones included
    G = w.hp // w.hkvp
    dvs = as_f64(dv).sum(axis=0)                                   # [b, hkvp, d]
    gs = as_f64(dout).sum(axis=0).reshape(w.b, w.hkvp, G, w.d).sum(axis=2)
    err = np.abs(dvs - gs).max()
    scale = np.abs(as_f64(dv)).sum(axis=0).max()
    print(f"  |sum_j dv_j - sum_t dout_t| = {err:.3e} against sum_j |dv_j| = {scale:.3e}",
          flush=True)
    assert err <= 1e-2 * scale


# causal shares whose split dQ and dK/dV units fill part of one round of
# workgroups or two rounds (8192 x 2 GQA: 512 dQ units), so the first-round
# reordering of units is exercised with whole runs, tails and a second round
@pytest.mark.parametrize("s,b,h,h_kv,P", [(4096, 1, 16, 16, 8), (8192, 2, 32, 8, 8)])
def test_bwd_split_unit_rounds(s, b, h, h_kv, P):
    """At s = 4096 (the 32K share's heads and split, one eighth of its length)
    every element of dq, dk and dv is compared with the oracle.  At s = 8192
    (GQA 4:1, b = 2) sampled query rows, late keys and early and middle keys
    (j = 0, s/4, s/2, 3s/4 - 1: keys that every later query row sees, so
    their gradients sum the longest runs of query tiles and both split
    halves)."""
    d, hp, hkvp = 128, h // P, h_kv // P
    print(f"case bwd split rounds s={s} b={b} h={h} h_kv={h_kv} P={P}", flush=True)
    q, k, v = share_inputs(23, s, b, hp, hkvp, d, "bf16")
    dout = synth.tensor(2304, (s, b, hp, d), "bf16")
    o, lse = gpu_fwd(q, k, v, s, b, h, h_kv, d, P, True)
    dq, dk, dv = gpu_bwd(q, k, v, o, lse, dout, s, b, h, h_kv, d, P, True)
    for g in (dq, dk, dv):
        assert np.all(np.isfinite(as_f64(g)))
    if s <= 4096:
        rq, rk, rv = oracle.attn_bwd(q, k, v, dout, s, b, h, h_kv, d, P, True)
        check("dq", dq, rq)
        check("dk", dk, rk)
        check("dv", dv, rv)
        return
    qrows = synth.row_sample(2307, s, b, hp, n_random=48, edge=8, tile_bounds=(32, 64))
    n_keys = 12
    js = s - 1 - np.arange(n_keys) * 5
    late = np.stack([np.arange(n_keys) % b, np.arange(n_keys) % hkvp, js], axis=1)
    early = np.array([(0, 0, 0), (b - 1, hkvp - 1, 0), (0, 0, s // 4),
                      (b - 1, hkvp - 1, s // 2), (0, 0, 3 * s // 4 - 1)], dtype=np.int64)
    krows = np.concatenate([early, late], axis=0)
    rq, rk, rv = oracle.attn_bwd_rows(q, k, v, dout, qrows, krows, s, b, h, h_kv, d, P, True)
    check("dq rows", dq[qrows[:, 2], qrows[:, 0], qrows[:, 1]], rq)
    check("dk keys", dk[krows[:, 2], krows[:, 0], krows[:, 1]], rk)
    check("dv keys", dv[krows[:, 2], krows[:, 0], krows[:, 1]], rv)


def test_bwd_counter_shape_repeats():
    """A share whose dQ work is four or more rounds of workgroups (2048 items)
    takes its dQ units from a counter that the prep kernel clears: two calls
    in a row give the same bits, and sampled rows match the oracle."""
    s, b, h, h_kv, d, P = 16384, 4, 64, 16, 128, 8
    hp, hkvp = h // P, h_kv // P
    q, k, v = share_inputs(24, s, b, hp, hkvp, d, "bf16")
    dout = synth.tensor(2404, (s, b, hp, d), "bf16")
    o, lse = gpu_fwd(q, k, v, s, b, h, h_kv, d, P, True)
    first = gpu_bwd(q, k, v, o, lse, dout, s, b, h, h_kv, d, P, True)
    second = gpu_bwd(q, k, v, o, lse, dout, s, b, h, h_kv, d, P, True)
    for x, y in zip(first, second):
        assert np.array_equal(x, y)
    qrows = synth.row_sample(2407, s, b, hp, n_random=8, edge=2, tile_bounds=(64,))
    krows = np.array([[0, 0, s - 1], [3, 1, s - 7]])
    rq, rk, rv = oracle.attn_bwd_rows(q, k, v, dout, qrows, krows, s, b, h, h_kv, d, P, True)
    dq, dk, dv = first
    check("dq rows", dq[qrows[:, 2], qrows[:, 0], qrows[:, 1]], rq)
    check("dk keys", dk[krows[:, 2], krows[:, 0], krows[:, 1]], rk)
    check("dv keys", dv[krows[:, 2], krows[:, 0], krows[:, 1]], rv)


def test_bwd_counter_matches_batch_slices():
    """The dQ counter path against calls without it: a b = 4 share whose dQ
    work is 2048 items (units from the counter) and the same share cut into
    four b = 1 calls (512 items each: no counter, no split).  Every dQ unit
    is computed by the same code whichever workgroup takes it, so dq must be
    equal bit for bit in every element -- a unit skipped or run twice would
    show.  dk and dv of the b = 1 calls run their key blocks as split halves
    (too few items to fill the GPU twice), a different summation order, so
    they are compared to a bf16 ulp of their scale.  Every gradient finite."""
    s, b, h, h_kv, d, P = 16384, 4, 64, 16, 128, 8
    hp, hkvp = h // P, h_kv // P
    q, k, v = share_inputs(25, s, b, hp, hkvp, d, "bf16")
    dout = synth.tensor(2504, (s, b, hp, d), "bf16")
    o, lse = gpu_fwd(q, k, v, s, b, h, h_kv, d, P, True)
    dq, dk, dv = gpu_bwd(q, k, v, o, lse, dout, s, b, h, h_kv, d, P, True)
    for g in (dq, dk, dv):
        assert np.all(np.isfinite(as_f64(g)))
    for be in range(b):
        sl = slice(be, be + 1)
        one = gpu_bwd(*(np.ascontiguousarray(x[:, sl]) for x in (q, k, v, o)),
                      np.ascontiguousarray(lse[sl]), np.ascontiguousarray(dout[:, sl]),
                      s, 1, h, h_kv, d, P, True)
        assert np.array_equal(dq[:, sl], one[0]), f"dq of batch entry {be}"
        for name, full, part in (("dk", dk, one[1]), ("dv", dv, one[2])):
            a, c = as_f64(full[:, sl]), as_f64(part)
            err = np.max(np.abs(a - c))
            assert err <= 2 ** -7 * max(1.0, np.max(np.abs(c))), (name, be, err)
