"""GPU parity of the KV-head replication (fewer KV heads than ranks) through
the C ABI: ulys_pack_seq2head_kv bit-exact against the oracle's orc_pack_kv,
ulys_unpack_head2seq_kv (the copies' gradients summed) against
orc_unpack_kv_sum, and the whole emulated layer -- forward and backward --
with a GQA model whose KV heads are fewer than the ranks, against the
oracle's unsharded attention and gradients.

Tolerances.  The pack is a bit move: bit-exact.  The sum accumulates R = P/h_kv
copies in fp32 in ascending order and rounds once; the oracle sums exactly and
rounds once, so the two differ by at most the fp32 accumulation error,
(R-1) 2^-24 sum|y|, plus one unit in the last place of the output (half from
the oracle's rounding, half from the GPU's): |gpu - ref| <= ulp(|ref|) +
R 2^-24 sum|y|.  Attention and gradients use the bounds of the other GPU
tests (2e-2, and 2e-2 max(1, max|ref|) per gradient tensor)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import Guarded, as_f64, dev, from_dev, share_inputs, to_dev
from ulysses_head_sharded_amd import binding, synth
from ulysses_head_sharded_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
CODE = {"bf16": binding.ULYS_BF16, "f32": binding.ULYS_F32}


def stream():
    return torch.cuda.current_stream().cuda_stream


def gpu_pack_kv(x, s, b, h_kv, d, P, dt):
    dev()
    hk = binding.kv_heads_per_rank(h_kv, P)
    xd = to_dev(x)
    y = Guarded((P, s // P, b, hk, d), TORCH_DT[dt])
    rc = binding.ulys_pack_seq2head_kv(xd.data_ptr(), y.tensor.data_ptr(), s, b, h_kv, d, P,
                                       CODE[dt], stream())
    assert rc == 0, binding.ulys_status_string(rc)
    torch.cuda.synchronize()
    assert y.guards_intact()
    return from_dev(y.tensor)


def gpu_unpack_kv(y, s, b, h_kv, d, P, dt):
    dev()
    yd = to_dev(y)
    x = Guarded((s // P, b, h_kv, d), TORCH_DT[dt])
    rc = binding.ulys_unpack_head2seq_kv(yd.data_ptr(), x.tensor.data_ptr(), s, b, h_kv, d, P,
                                         CODE[dt], stream())
    assert rc == 0, binding.ulys_status_string(rc)
    torch.cuda.synchronize()
    assert x.guards_intact()
    return from_dev(x.tensor)


def ulp(a, dt):
    """Spacing of the output format at |a| (normal range)."""
    mant = 7 if dt == "bf16" else 23
    e = np.floor(np.log2(np.maximum(np.abs(a), 1e-30)))
    return np.exp2(e - mant)


# (s, b, h_kv, d, P): replication factors 2, 4, 8 and 16, ragged sequence
# blocks, runs of 16-byte vectors (d = 64, 128) and of single elements (d = 3)
SHAPES = [(8, 1, 1, 3, 4), (20, 2, 2, 64, 4), (24, 1, 2, 128, 8), (48, 2, 8, 128, 16),
          (64, 1, 1, 128, 16), (36, 2, 4, 8, 12), (16, 1, 8, 128, 8)]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("s,b,h_kv,d,P", SHAPES)
def test_pack_kv_bit_exact(s, b, h_kv, d, P, dt):
    print(f"case pack_kv s={s} b={b} h_kv={h_kv} d={d} P={P} {dt}", flush=True)
    x = synth.tensor(2000 + s + d, (s // P, b, h_kv, d), dt)
    got = gpu_pack_kv(x, s, b, h_kv, d, P, dt)
    ref = oracle.pack_kv(x, s, b, h_kv, d, P)
    assert got.shape == ref.shape and np.array_equal(got.view(np.uint8), ref.view(np.uint8))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("s,b,h_kv,d,P", SHAPES)
def test_unpack_kv_sum(s, b, h_kv, d, P, dt):
    print(f"case unpack_kv s={s} b={b} h_kv={h_kv} d={d} P={P} {dt}", flush=True)
    hk = binding.kv_heads_per_rank(h_kv, P)
    y = synth.tensor(2100 + s + d, (P, s // P, b, hk, d), dt)
    got = as_f64(gpu_unpack_kv(y, s, b, h_kv, d, P, dt))
    ref = as_f64(oracle.unpack_kv_sum(y, s, b, h_kv, d, P))
    if h_kv % P == 0:
        assert np.array_equal(got, ref)
        return
    R = P // h_kv
    yabs = np.abs(as_f64(y)).reshape(h_kv, R, s // P, b, d).sum(axis=1).transpose(1, 2, 0, 3)
    bound = ulp(ref, dt) + R * 2.0 ** -24 * yabs
    assert np.all(np.abs(got - ref) <= bound)
    # replicate-then-sum multiplies by R (a power of two here); exact on the GPU
    # too when the fp32 running sums of R copies need no rounding: bf16 inputs
    # (8 significant bits + log2 R <= 24), or R = 2 for fp32 (3x may already
    # need a 25th bit)
    if R & (R - 1) == 0 and (dt == "bf16" or R == 2):
        x = synth.tensor(2200 + s, (s // P, b, h_kv, d), dt)
        back = gpu_unpack_kv(gpu_pack_kv(x, s, b, h_kv, d, P, dt), s, b, h_kv, d, P, dt)
        assert np.array_equal(as_f64(back), R * as_f64(x))


def exchange(shards, P, fn):
    """Pack every rank's shard on the GPU and route block r of every sender to
    rank r in source order: rank r's received share [s, b, heads, d]."""
    packed = [fn(to_dev(x), P) for x in shards]
    return [torch.cat([packed[j][r] for j in range(P)], dim=0) for r in range(P)]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("s,b,h,h_kv,P", [(256, 2, 8, 2, 4), (192, 1, 16, 1, 8),
                                          (128, 1, 16, 4, 16)])
def test_layer_with_replicated_kv(s, b, h, h_kv, P, causal):
    """Forward and backward of the whole Ulysses layer on one GPU, KV heads
    fewer than ranks: Q and dO by ulys_pack_seq2head, K and V by
    ulys_pack_seq2head_kv, attention and its backward on each share with the
    model's h_kv, O and dQ back by ulys_unpack_head2seq, dK and dV by
    ulys_unpack_head2seq_kv -- against the oracle's unsharded GQA attention and
    gradients over all heads."""
    d, sl = 128, s // P
    print(f"case layer s={s} b={b} h={h} h_kv={h_kv} P={P} causal={causal}", flush=True)
    qg, kg, vg, gg = (synth.tensor(2300 + n, (s, b, hh, d), "bf16")
                      for n, hh in enumerate((h, h_kv, h_kv, h)))
    dev()
    seq = lambda t: [t[j * sl:(j + 1) * sl] for j in range(P)]  # noqa: E731
    qs = exchange(seq(qg), P, binding.pack_seq2head)
    ks = exchange(seq(kg), P, binding.pack_seq2head_kv)
    vs = exchange(seq(vg), P, binding.pack_seq2head_kv)
    gs = exchange(seq(gg), P, binding.pack_seq2head)
    outs, grads = [], []
    for r in range(P):
        q, k, v = (t.reshape(s, b, -1, d).contiguous() for t in (qs[r], ks[r], vs[r]))
        g = gs[r].reshape(s, b, -1, d).contiguous()
        assert k.shape[2] == 1  # one replicated KV head per share
        o, lse = binding.attn_fwd(q, k, v, P=P, causal=causal, lse=True)
        outs.append(o)
        grads.append(binding.attn_bwd(q, k, v, o, g, lse, P=P, causal=causal))
    torch.cuda.synchronize()

    def back(shares, unpack):
        res = []
        for j in range(P):
            recv = torch.stack([sh.reshape(P, sl, b, -1, d)[j] for sh in shares]).contiguous()
            res.append(from_dev(unpack(recv)))
        return np.concatenate(res, axis=0)

    o_ref, _ = oracle.attn(qg, kg, vg, s, b, h, h_kv, d, 1, causal)
    o_got = back(outs, binding.unpack_head2seq)
    err = np.max(np.abs(as_f64(o_got) - o_ref))
    print(f"  o: max err {err:.3e}", flush=True)
    assert err <= 2e-2
    rq, rk, rv = oracle.attn_bwd(qg, kg, vg, gg, s, b, h, h_kv, d, 1, causal)
    for name, got, ref in (
            ("dq", back([g[0] for g in grads], binding.unpack_head2seq), rq),
            ("dk", back([g[1] for g in grads], lambda y: binding.unpack_head2seq_kv(y, h_kv)), rk),
            ("dv", back([g[2] for g in grads], lambda y: binding.unpack_head2seq_kv(y, h_kv)), rv)):
        err = np.max(np.abs(as_f64(got) - ref))
        bound = 2e-2 * max(1.0, float(np.max(np.abs(ref))))
        print(f"  {name}: max err {err:.3e} (bound {bound:.3e})", flush=True)
        assert err <= bound, (name, err, bound)


def test_full_size_replicated_gqa_share():
    """The 64K GQA share at P = 16 (8 KV heads, so each KV head goes to two
    ranks): the K and V packs bit-exact against the oracle, and the share's
    attention on sampled rows against the oracle."""
    w = WORKLOADS["gqa-64k-p16"]
    sl = w.s // w.P
    print(f"case {w.name}: P={w.P} s={w.s} b={w.b} h={w.h} h_kv={w.h_kv}", flush=True)
    for n in (2, 3):
        x = synth.tensor(100 * w.c + n, (sl, w.b, w.h_kv, w.d), w.dtype)
        got = gpu_pack_kv(x, w.s, w.b, w.h_kv, w.d, w.P, w.dtype)
        ref = oracle.pack_kv(x, w.s, w.b, w.h_kv, w.d, w.P)
        assert np.array_equal(got, ref)
    q, k, v = share_inputs(w.c, w.s, w.b, w.hp, w.hkvp, w.d, w.dtype)
    dev()
    o, lse = binding.attn_fwd(to_dev(q), to_dev(k), to_dev(v), P=w.P, causal=w.causal, lse=True)
    torch.cuda.synchronize()
    o, lse = from_dev(o), from_dev(lse)
    rows = synth.row_sample(100 * w.c + 7, w.s, w.b, w.hp, n_random=48, edge=16)
    # the share holds one KV head: the oracle's share attention with h_kv_eff = P
    o_ref, lse_ref = oracle.attn_rows(q, k, v, rows, w.s, w.b, w.h, w.P, w.d, w.P, w.causal)
    got = as_f64(o[rows[:, 2], rows[:, 0], rows[:, 1]])
    err = np.max(np.abs(got - o_ref))
    print(f"  o rows: max err {err:.3e}", flush=True)
    assert err <= 2e-2
    assert np.max(np.abs(lse[rows[:, 0], rows[:, 1], rows[:, 2]] - lse_ref)) <= 1e-3
