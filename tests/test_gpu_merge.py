"""GPU parity of ulys_attn_merge (two partial attention results of one share
over disjoint key sets combined through their log-sum-exp) against the
oracle's orc_attn_merge, and of the schemes built on it: a causal ring over
sequence chunks, and the USP arrangement of Ulysses groups whose same-head
ranks exchange K and V (Ulysses degree 4 x ring degree 2), against the
oracle's unsharded attention.

Tolerances.  The merge computes in fp32 (exp2/log2 within a few ulp) and
rounds O once: |O - O_ref| <= ulp(O_ref) + 1e-5 (|O_a| + |O_b|) for bf16 and
1e-5 (|O_a| + |O_b|) for fp32; |lse - lse_ref| <= 1e-5 (1 + |lse_ref|).  The
chains end in attention outputs and use the attention bounds (2e-2 bf16;
lse 1e-3)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import as_f64, dev, from_dev, to_dev
from ulysses_head_sharded_amd import binding, synth

pytestmark = pytest.mark.gpu


def partials(seed, s, b, hp, d, dt):
    """Two seeded partial results with some empty rows (lse = -inf): one side
    empty, and both."""
    o_a = synth.tensor(seed, (s, b, hp, d), dt)
    o_b = synth.tensor(seed + 1, (s, b, hp, d), dt)
    la = (3.0 * synth.normal_f32(seed + 2, b * hp * s)).reshape(b, hp, s)
    lb = (3.0 * synth.normal_f32(seed + 3, b * hp * s)).reshape(b, hp, s)
    la[:, :, ::7] = -np.inf
    lb[:, :, ::5] = -np.inf
    return o_a, la.astype(np.float32), o_b, lb.astype(np.float32)


def ulp(a, dt):
    mant = 7 if dt == "bf16" else 23
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(a), 1e-30))) - mant)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("s,b,hp,d", [(37, 2, 3, 64), (128, 1, 2, 128), (5, 1, 8, 128),
                                      (300, 2, 1, 64)])
def test_merge_vs_oracle(s, b, hp, d, dt):
    print(f"case merge s={s} b={b} hp={hp} d={d} {dt}", flush=True)
    o_a, la, o_b, lb = partials(2500 + s, s, b, hp, d, dt)
    dev()
    o, lse = binding.attn_merge(to_dev(o_a), to_dev(la), to_dev(o_b), to_dev(lb))
    torch.cuda.synchronize()
    o, lse = as_f64(from_dev(o)), from_dev(lse).astype(np.float64)
    o_ref, lse_ref = oracle.attn_merge(as_f64(o_a), la, as_f64(o_b), lb)
    scale = np.abs(as_f64(o_a)) + np.abs(as_f64(o_b))
    bound = 1e-5 * scale + (ulp(o_ref, dt) if dt == "bf16" else 0.0)
    assert np.all(np.abs(o - o_ref) <= bound)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin) and np.all(lse[~fin] == -np.inf)
    assert np.all(np.abs(lse[fin] - lse_ref[fin]) <= 1e-5 * (1 + np.abs(lse_ref[fin])))
    # rows with both partials empty: O = 0
    both = ~fin.transpose(2, 0, 1)  # [s, b, hp]
    assert np.all(o[both] == 0.0)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_merge_in_place(dt):
    """o = o_a, lse = lse_a accumulates in place with the same bits as out of place."""
    s, b, hp, d = 200, 2, 2, 128
    o_a, la, o_b, lb = partials(2600, s, b, hp, d, dt)
    dev()
    oa, lad, ob, lbd = to_dev(o_a), to_dev(la), to_dev(o_b), to_dev(lb)
    o1, l1 = binding.attn_merge(oa, lad, ob, lbd)
    o2, l2 = binding.attn_merge(oa, lad, ob, lbd, out=oa, lse_out=lad)
    torch.cuda.synchronize()
    assert o2.data_ptr() == oa.data_ptr()
    assert torch.equal(o1.view(torch.uint8), oa.view(torch.uint8))
    assert torch.equal(l1, lad)


def chunk_attn(q, k, v, causal):
    o, lse = binding.attn_fwd(q, k, v, P=1, causal=causal, lse=True)
    return o, lse


@pytest.mark.parametrize("n_chunks,c", [(4, 96), (3, 200)])
def test_ring_causal_chain(n_chunks, c):
    """Causal attention over n_chunks * c tokens, computed chunk by chunk as a
    ring delivers the key blocks to the rank holding query chunk i: its own
    block (causal), then the earlier ones (dense), merged in that order."""
    s, b, hp, d = n_chunks * c, 1, 2, 128
    print(f"case ring n={n_chunks} c={c}", flush=True)
    q = synth.tensor(2700, (s, b, hp, d), "bf16")
    k = synth.tensor(2701, (s, b, hp, d), "bf16")
    v = synth.tensor(2702, (s, b, hp, d), "bf16")
    dev()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o_ref, lse_ref = oracle.attn(q, k, v, s, b, hp, hp, d, 1, True)
    for i in range(n_chunks):
        blk = lambda t, j: t[j * c:(j + 1) * c].contiguous()  # noqa: E731
        o, lse = chunk_attn(blk(qd, i), blk(kd, i), blk(vd, i), True)
        for j in range(i - 1, -1, -1):
            o2, lse2 = chunk_attn(blk(qd, i), blk(kd, j), blk(vd, j), False)
            o, lse = binding.attn_merge(o, lse, o2, lse2, out=o, lse_out=lse)
        torch.cuda.synchronize()
        err = np.max(np.abs(as_f64(from_dev(o)) - o_ref[i * c:(i + 1) * c]))
        lerr = np.max(np.abs(from_dev(lse) - lse_ref[:, :, i * c:(i + 1) * c]))
        print(f"  chunk {i}: o err {err:.3e} lse err {lerr:.3e}", flush=True)
        assert err <= 2e-2 and lerr <= 1e-3


def test_usp_four_by_two():
    """The SP/CP page's USP arrangement on one GPU: 8 emulated cards, Ulysses
    degree 4 inside each of 2 groups (pack, route, unpack through the C ABI),
    ring degree 2 across the groups (the same-head card of the other group
    supplies K/V; attention with lse on the GPU; ulys_attn_merge), against the
    oracle's unsharded causal attention over all heads."""
    U, Rg = 4, 2
    s, b, h, h_kv, d = 512, 1, 8, 4, 128
    half = s // Rg
    qg, kg, vg = (synth.tensor(2800 + n, (s, b, hh, d), "bf16")
                  for n, hh in enumerate((h, h_kv, h_kv)))
    dev()

    def group_exchange(t, g, hh):
        """Ulysses exchange inside group g: shares of the group's half sequence."""
        shards = t[g * half:(g + 1) * half].reshape(U, half // U, b, hh, d)
        packed = [binding.pack_seq2head(to_dev(np.ascontiguousarray(x)), U) for x in shards]
        return [torch.cat([packed[j][r] for j in range(U)], dim=0).contiguous()
                for r in range(U)]

    shares = {}
    for g in range(Rg):
        qs, ks, vs = (group_exchange(t, g, hh) for t, hh in ((qg, h), (kg, h_kv), (vg, h_kv)))
        for u in range(U):
            shares[g, u] = (qs[u], ks[u], vs[u])
    o_ref, _ = oracle.attn(qg, kg, vg, s, b, h, h_kv, d, 1, True)
    for g in range(Rg):
        outs = []
        for u in range(U):
            q, k, v = shares[g, u]
            o, lse = binding.attn_fwd(q, k, v, P=U, causal=True, lse=True)
            for g2 in range(g):  # the earlier group's K/V around the ring
                _, k2, v2 = shares[g2, u]
                o2, lse2 = binding.attn_fwd(q, k2, v2, P=U, causal=False, lse=True)
                o, lse = binding.attn_merge(o, lse, o2, lse2, out=o, lse_out=lse)
            outs.append(o)
        res = []
        for j in range(U):  # head->seq inside the group: card j gets segment j
            recv = torch.stack([o.reshape(U, half // U, b, h // U, d)[j] for o in outs])
            res.append(from_dev(binding.unpack_head2seq(recv.contiguous())))
        got = np.concatenate(res, axis=0)
        err = np.max(np.abs(as_f64(got) - o_ref[g * half:(g + 1) * half]))
        print(f"  group {g}: o err {err:.3e}", flush=True)
        assert err <= 2e-2
