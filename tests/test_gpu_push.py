"""GPU parity of the exchange as pushes (ulys_seq2head_push, ulys_head2seq_push):
every emulated rank pushes its blocks straight into the P destination
buffers (here P regions of one GPU's memory, as peer-mapped receive buffers
would be on a node), and the P destinations together equal the oracle's
whole exchange (orc_seq2head, orc_head2seq) bit for bit; and a whole layer
built on pushes -- Q, K, V in, attention on each share, O back -- equals the
oracle's unsharded attention within the attention tolerance."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import Guarded, as_f64, dev, from_dev, to_dev
from ulysses_head_sharded_amd import binding, synth

pytestmark = pytest.mark.gpu

TORCH_DT = {2: torch.bfloat16, 4: torch.float32}
NP_DT = {2: np.uint16, 4: np.float32}
CODE = {2: binding.ULYS_BF16, 4: binding.ULYS_F32}


def stream():
    return torch.cuda.current_stream().cuda_stream


def bits(seed, shape, elt):
    raw = synth.random_bits(seed, int(np.prod(shape)) * elt)
    return raw.view(NP_DT[elt]).reshape(shape)


# (s, b, h, d, P, elt): runs of 16-byte vectors, of 4-byte words (d = 2,
# fp32 hp = 1) and of 2-byte elements (d = 3 bf16), up to P = 16
CASES = [(16, 1, 8, 64, 4, 2), (24, 2, 8, 128, 8, 2), (12, 2, 6, 3, 3, 2), (40, 1, 16, 2, 8, 4),
         (64, 2, 32, 128, 16, 2), (8, 1, 4, 64, 2, 4)]


@pytest.mark.parametrize("s,b,h,d,P,elt", CASES)
def test_seq2head_push_equals_exchange(s, b, h, d, P, elt):
    print(f"case seq2head_push s={s} b={b} h={h} d={d} P={P} elt={elt}", flush=True)
    sl, hp = s // P, h // P
    x_all = bits(4000 + s + d, (P, sl, b, h, d), elt)
    dev()
    shares = [Guarded((s, b, hp, d), TORCH_DT[elt]) for _ in range(P)]
    ptrs = [g.tensor.data_ptr() for g in shares]
    for j in range(P):
        xj = to_dev(np.ascontiguousarray(x_all[j]))
        rc = binding.ulys_seq2head_push(xj.data_ptr(), ptrs, j, s, b, h, d, P, CODE[elt], stream())
        assert rc == 0, binding.ulys_status_string(rc)
    torch.cuda.synchronize()
    assert all(g.guards_intact() for g in shares)
    ref = oracle.seq2head(x_all, s, b, h, d, P)
    for r in range(P):
        got = from_dev(shares[r].tensor)
        assert np.array_equal(got.view(np.uint8), ref[r].view(np.uint8)), r


@pytest.mark.parametrize("s,b,h,d,P,elt", CASES)
def test_head2seq_push_equals_exchange(s, b, h, d, P, elt):
    print(f"case head2seq_push s={s} b={b} h={h} d={d} P={P} elt={elt}", flush=True)
    sl, hp = s // P, h // P
    y_all = bits(4100 + s + d, (P, s, b, hp, d), elt)
    dev()
    shards = [Guarded((sl, b, h, d), TORCH_DT[elt]) for _ in range(P)]
    ptrs = [g.tensor.data_ptr() for g in shards]
    for r in range(P):
        yr = to_dev(np.ascontiguousarray(y_all[r]))
        rc = binding.ulys_head2seq_push(yr.data_ptr(), ptrs, r, s, b, h, d, P, CODE[elt], stream())
        assert rc == 0, binding.ulys_status_string(rc)
    torch.cuda.synchronize()
    assert all(g.guards_intact() for g in shards)
    ref = oracle.head2seq(y_all, s, b, h, d, P)
    for j in range(P):
        got = from_dev(shards[j].tensor)
        assert np.array_equal(got.view(np.uint8), ref[j].view(np.uint8)), j


@pytest.mark.parametrize("causal", [True, False])
def test_layer_on_pushes(causal):
    """Q, K, V pushed from every rank's shard into every rank's share, attention
    on each share, O pushed back into every rank's shard: equals the oracle's
    unsharded attention over all heads."""
    s, b, h, h_kv, d, P = 256, 2, 8, 4, 128, 4
    sl = s // P
    qg, kg, vg = (synth.tensor(4200 + n, (s, b, hh, d), "bf16")
                  for n, hh in enumerate((h, h_kv, h_kv)))
    dev()

    def push_in(t, hh):
        shares = [torch.empty((s, b, hh // P, d), dtype=torch.bfloat16, device="cuda")
                  for _ in range(P)]
        ptrs = [x.data_ptr() for x in shares]
        for j in range(P):
            xj = to_dev(np.ascontiguousarray(t[j * sl:(j + 1) * sl]))
            assert binding.ulys_seq2head_push(xj.data_ptr(), ptrs, j, s, b, hh, d, P,
                                              binding.ULYS_BF16, stream()) == 0
            torch.cuda.synchronize()  # xj is freed after this iteration
        return shares

    qs, ks, vs = push_in(qg, h), push_in(kg, h_kv), push_in(vg, h_kv)
    outs = [torch.empty((sl, b, h, d), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    optrs = [x.data_ptr() for x in outs]
    for r in range(P):
        o, _ = binding.attn_fwd(qs[r], ks[r], vs[r], P=P, causal=causal)
        assert binding.ulys_head2seq_push(o.data_ptr(), optrs, r, s, b, h, d, P,
                                          binding.ULYS_BF16, stream()) == 0
        torch.cuda.synchronize()
    got = np.concatenate([from_dev(x) for x in outs], axis=0)
    ref, _ = oracle.attn(qg, kg, vg, s, b, h, h_kv, d, 1, causal)
    err = np.max(np.abs(as_f64(got) - ref))
    print(f"  o: max err {err:.3e}", flush=True)
    assert err <= 2e-2


# (s, b, h, h_kv, d, P, rank, causal): a wave's 32 rows inside one sequence
# segment (sl = 64) and across segment boundaries (sl = 25, 40, 125), GQA,
# d = 64, the 32K share, whose workspace path splits every item, and a share
# of 2048 items, whose workspace path hands out units from a counter
ATTN_PUSH = [(256, 1, 8, 4, 128, 4, 1, True), (100, 2, 8, 8, 128, 4, 3, False),
             (320, 1, 16, 2, 64, 8, 5, True), (1000, 1, 8, 2, 128, 8, 0, True),
             (1000, 2, 8, 8, 128, 8, 7, False), (32768, 1, 16, 16, 128, 8, 3, True),
             (16384, 4, 64, 16, 128, 8, 5, True)]


@pytest.mark.parametrize("ws", [False, True], ids=["plain", "ws"])
@pytest.mark.parametrize("s,b,h,h_kv,d,P,rank,causal", ATTN_PUSH)
def test_attn_push_equals_attn_then_push(s, b, h, h_kv, d, P, rank, causal, ws):
    """ulys_attn_fwd_push writes, bit for bit, what ulys_attn_fwd_ws followed by
    ulys_head2seq_push writes: this rank's head columns of every destination
    shard (the rest, and the guard bands, untouched), and the same lse."""
    print(f"case attn_push s={s} b={b} h={h} h_kv={h_kv} d={d} P={P} rank={rank} "
          f"causal={causal} ws={ws}", flush=True)
    sl, hp, hkvp = s // P, h // P, binding.kv_heads_per_rank(h_kv, P)
    from gpu_util import share_inputs
    q, k, v = share_inputs(40 + P, s, b, hp, hkvp, d, "bf16")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    code = binding.ULYS_BF16
    nbytes = binding.ulys_attn_fwd_workspace_size(s, b, h, h_kv, d, P, int(causal), code) if ws else 0
    assert nbytes >= 0
    wsbuf = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    wsp = wsbuf.data_ptr() if nbytes > 0 else None
    o = torch.empty((s, b, hp, d), dtype=torch.bfloat16, device="cuda")
    lse_ref = torch.empty((b, hp, s), dtype=torch.float32, device="cuda")
    rc = binding.ulys_attn_fwd_ws(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(),
                                  lse_ref.data_ptr(), s, b, h, h_kv, d, P, int(causal), code, wsp,
                                  nbytes, stream())
    assert rc == 0, binding.ulys_status_string(rc)
    ref = [Guarded((sl, b, h, d), torch.bfloat16) for _ in range(P)]
    rc = binding.ulys_head2seq_push(o.data_ptr(), [g.tensor.data_ptr() for g in ref], rank, s, b,
                                    h, d, P, code, stream())
    assert rc == 0, binding.ulys_status_string(rc)
    got = [Guarded((sl, b, h, d), torch.bfloat16) for _ in range(P)]
    lse = Guarded((b, hp, s), torch.float32)
    rc = binding.ulys_attn_fwd_push(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                                    [g.tensor.data_ptr() for g in got], rank, lse.tensor.data_ptr(),
                                    s, b, h, h_kv, d, P, int(causal), code, wsp, nbytes, stream())
    assert rc == 0, binding.ulys_status_string(rc)
    torch.cuda.synchronize()
    for j in range(P):
        assert torch.equal(got[j].raw, ref[j].raw), j
    assert lse.guards_intact()
    assert torch.equal(lse.tensor, lse_ref)


# (s, b, h, h_kv, d, P, rank, causal): segments of 64, 25 and 125 rows, GQA,
# both head sizes, and the 32K share, whose backward splits both its dQ and
# dK/dV items
BWD_PUSH = [(256, 1, 8, 4, 128, 4, 1, True), (100, 2, 8, 8, 128, 4, 3, False),
            (1000, 1, 16, 8, 128, 8, 0, True), (32768, 1, 16, 16, 128, 8, 6, True),
            (1000, 1, 16, 8, 64, 8, 5, True)]


@pytest.mark.parametrize("s,b,h,h_kv,d,P,rank,causal", BWD_PUSH)
def test_attn_bwd_push_equals_bwd_then_push(s, b, h, h_kv, d, P, rank, causal):
    """ulys_attn_bwd_push writes, bit for bit, what ulys_attn_bwd followed by
    ulys_head2seq_push of dQ, dK and dV writes (the rest of every destination
    shard, and its guard bands, untouched)."""
    print(f"case attn_bwd_push s={s} b={b} h={h} h_kv={h_kv} d={d} P={P} rank={rank} "
          f"causal={causal}", flush=True)
    sl, hp, hkvp = s // P, h // P, h_kv // P
    from gpu_util import share_inputs
    q, k, v = share_inputs(60 + P, s, b, hp, hkvp, d, "bf16")
    g = synth.tensor(6000 + s, (s, b, hp, d), "bf16")
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    o, lse = binding.attn_fwd(qd, kd, vd, P=P, causal=causal, lse=True)
    dq, dk, dv = binding.attn_bwd(qd, kd, vd, o, gd, lse, P=P, causal=causal)
    code = binding.ULYS_BF16
    ref = {}
    for name, t, heads in (("dq", dq, h), ("dk", dk, h_kv), ("dv", dv, h_kv)):
        ref[name] = [Guarded((sl, b, heads, d), torch.bfloat16) for _ in range(P)]
        rc = binding.ulys_head2seq_push(t.data_ptr(), [x.tensor.data_ptr() for x in ref[name]],
                                        rank, s, b, heads, d, P, code, stream())
        assert rc == 0, binding.ulys_status_string(rc)
    got = {"dq": [Guarded((sl, b, h, d), torch.bfloat16) for _ in range(P)],
           "dk": [Guarded((sl, b, h_kv, d), torch.bfloat16) for _ in range(P)],
           "dv": [Guarded((sl, b, h_kv, d), torch.bfloat16) for _ in range(P)]}
    nbytes = binding.ulys_attn_bwd_workspace_size(s, b, h, h_kv, d, P, int(causal), code)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    rc = binding.ulys_attn_bwd_push(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(),
                                    gd.data_ptr(), lse.data_ptr(),
                                    *[[x.tensor.data_ptr() for x in got[n]]
                                      for n in ("dq", "dk", "dv")],
                                    rank, s, b, h, h_kv, d, P, int(causal), code, ws.data_ptr(),
                                    nbytes, stream())
    assert rc == 0, binding.ulys_status_string(rc)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv"):
        for j in range(P):
            assert torch.equal(got[name][j].raw, ref[name][j].raw), (name, j)
