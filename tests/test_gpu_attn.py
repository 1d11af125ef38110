"""GPU parity of the head-sharded attention against the fp64 CPU oracle.

Tolerances: max |O_gpu - O_ref| <= 2e-2 for bf16 inputs, <= 1e-4 for fp32
inputs (the oracle runs in fp64 on the same rounded inputs).  LSE is checked to
1e-3 (bf16) / 1e-5 (fp32) absolute."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import Guarded, as_f64, dev, from_dev, share_inputs, to_dev
from ulysses_head_sharded_amd import binding, synth
from ulysses_head_sharded_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
LSE_TOL = {"bf16": 1e-3, "f32": 1e-5}
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def gpu_attn(q, k, v, s, b, h, h_kv, d, P, causal, dtype, want_lse=True, ws=False):
    """Attention through the C ABI: ulys_attn_fwd, or with ws=True
    ulys_attn_fwd_ws with the workspace it asks for (guarded too)."""
    dev()
    hp = h // P
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o = Guarded((s, b, hp, d), TORCH_DT[dtype])
    lse = Guarded((b, hp, s), torch.float32) if want_lse else None
    code = binding.ULYS_BF16 if dtype == "bf16" else binding.ULYS_F32
    stream = torch.cuda.current_stream().cuda_stream
    wsbuf = None
    if ws:
        nbytes = binding.ulys_attn_fwd_workspace_size(s, b, h, h_kv, d, P, int(causal), code)
        assert nbytes >= 0
        wsbuf = Guarded((max(nbytes, 16),), torch.uint8)
        rc = binding.ulys_attn_fwd_ws(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                                      o.tensor.data_ptr(), lse.tensor.data_ptr() if lse else None,
                                      s, b, h, h_kv, d, P, int(causal), code,
                                      wsbuf.tensor.data_ptr(), nbytes, stream)
    else:
        rc = binding.ulys_attn_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                                   o.tensor.data_ptr(), lse.tensor.data_ptr() if lse else None,
                                   s, b, h, h_kv, d, P, int(causal), code, stream)
    assert rc == 0, binding.ulys_status_string(rc)
    torch.cuda.synchronize()
    assert o.guards_intact()
    if lse:
        assert lse.guards_intact()
    if wsbuf is not None:
        assert wsbuf.guards_intact()
    return from_dev(o.tensor), (from_dev(lse.tensor) if lse else None)


# s spans several 64-key tiles with ragged tails; (h, h_kv, P) covers MHA,
# GQA 4:1 and 8:1 (two head subgroups per KV head) and MQA
SMALL = []
for dtype, d in [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)]:
    for (s, b) in [(1, 1), (5, 2), (64, 1), (65, 1), (200, 2), (321, 1), (1000, 1)]:
        for (h, h_kv, P) in [(2, 2, 1), (8, 2, 2), (16, 2, 1), (8, 8, 4), (4, 1, 1)]:
            if dtype == "f32" and s > 321:
                continue
            if s % P:
                continue  # the ABI rejects P !| s (covered by the CPU error-path tests)
            for causal in (False, True):
                SMALL.append((dtype, d, s, b, h, h_kv, P, causal))


@pytest.mark.parametrize("ws", [False, True], ids=["plain", "ws"])
@pytest.mark.parametrize("dtype,d,s,b,h,h_kv,P,causal", SMALL)
def test_small_full_parity(dtype, d, s, b, h, h_kv, P, causal, ws):
    print(f"case {dtype} d={d} s={s} b={b} h={h} h_kv={h_kv} P={P} causal={causal} ws={ws}",
          flush=True)
    q, k, v = share_inputs(7, s, b, h // P, h_kv // P, d, dtype)
    o, lse = gpu_attn(q, k, v, s, b, h, h_kv, d, P, causal, dtype, ws=ws)
    o_ref, lse_ref = oracle.attn(q, k, v, s, b, h, h_kv, d, P, causal)
    err = np.max(np.abs(as_f64(o) - o_ref))
    assert err <= TOL[dtype], err
    assert np.max(np.abs(lse.astype(np.float64) - lse_ref)) <= LSE_TOL[dtype]


def test_tiny_workload_parity():
    w = WORKLOADS["tiny"]
    q, k, v = share_inputs(w.c, w.s, w.b, w.hp, w.hkvp, w.d, w.dtype)
    o, lse = gpu_attn(q, k, v, w.s, w.b, w.h, w.h_kv, w.d, w.P, w.causal, w.dtype)
    o_ref, lse_ref = oracle.attn(q, k, v, w.s, w.b, w.h, w.h_kv, w.d, w.P, w.causal)
    assert np.max(np.abs(as_f64(o) - o_ref)) <= TOL[w.dtype]
    assert np.max(np.abs(lse - lse_ref)) <= LSE_TOL[w.dtype]


# full-size workloads: sampled rows (the oracle computes them one by one) plus,
# where the oracle can afford it, every row of whole work units: the first, a
# middle and the last query block of the listed local query heads (a work unit
# is 8 waves x 32 queries spread over the query heads of one KV group, so the
# GQA share lists all four heads of its group)
FULL = {
    "gpt1.2b-32k": dict(n_random=256, edge=32, unit_heads=(0, 1)),
    "mha-128k": dict(n_random=48, edge=16, unit_heads=(0, 3)),
    "gqa-64k": dict(n_random=64, edge=16, unit_heads=(0, 1, 2, 3)),
    "mtok-1m": dict(n_random=12, edge=6, unit_heads=()),
    "dit-256k": dict(n_random=6, edge=4, unit_heads=()),
}


def full_rows(name):
    """The sampled rows of a full-size share and the rows of its whole units."""
    w = WORKLOADS[name]
    spec = dict(FULL[name])
    heads = spec.pop("unit_heads")
    rows = synth.row_sample(100 * w.c + 7, w.s, w.b, w.hp, tile_bounds=(64, 128), **spec)
    if heads:
        G = w.hp // w.hkvp
        qh = 8 if G % 8 == 0 else 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1
        qb = 32 * (8 // qh)
        nblk = (w.s + qb - 1) // qb
        ts = np.concatenate([np.arange(k * qb, min(w.s, (k + 1) * qb))
                             for k in sorted({0, nblk // 2, nblk - 1})])
        units = np.array([(be, i, t) for be in range(w.b) for i in heads for t in ts],
                         dtype=np.int64)
        rows = np.unique(np.concatenate([rows, units], axis=0), axis=0)
    return rows


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled_parity(name):
    w = WORKLOADS[name]
    print(f"case {name}: s={w.s} b={w.b} hp={w.hp} hkvp={w.hkvp} causal={w.causal}", flush=True)
    q, k, v = share_inputs(w.c, w.s, w.b, w.hp, w.hkvp, w.d, w.dtype)
    # the workspace entry point, as the bench calls it (it splits only where
    # the causal work would otherwise be unbalanced, e.g. the 32K share)
    o, lse = gpu_attn(q, k, v, w.s, w.b, w.h, w.h_kv, w.d, w.P, w.causal, w.dtype, ws=True)
    rows = full_rows(name)
    o_ref, lse_ref = oracle.attn_rows(q, k, v, rows, w.s, w.b, w.h, w.h_kv, w.d, w.P,
                                      w.causal)
    got = as_f64(o[rows[:, 2], rows[:, 0], rows[:, 1]])
    err = np.max(np.abs(got - o_ref))
    print(f"  {rows.shape[0]} rows, max err {err:.3e}", flush=True)
    assert err <= TOL[w.dtype]
    lse_got = lse[rows[:, 0], rows[:, 1], rows[:, 2]].astype(np.float64)
    assert np.max(np.abs(lse_got - lse_ref)) <= LSE_TOL[w.dtype]
    # properties over every row: finite, and |O| bounded by max |V| (convex combination)
    of = as_f64(o)
    assert np.all(np.isfinite(of)) and np.all(np.isfinite(lse))
    assert np.max(np.abs(of)) <= np.max(np.abs(as_f64(v))) + TOL[w.dtype]


@pytest.mark.parametrize("name", [n for n in FULL if WORKLOADS[n].dtype == "bf16"])
def test_full_size_sampled_parity_push(name):
    """The bench step's attention: ulys_attn_fwd_push (rank P-1 writing its
    head columns into P destination shards, with the workspace) at the full
    share, the sampled rows read back from the shards they landed in."""
    w = WORKLOADS[name]
    print(f"case push {name}: s={w.s} b={w.b} hp={w.hp} hkvp={w.hkvp} causal={w.causal}",
          flush=True)
    q, k, v = share_inputs(w.c, w.s, w.b, w.hp, w.hkvp, w.d, w.dtype)
    dev()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    sl, rank, code = w.s // w.P, w.P - 1, binding.ULYS_BF16
    shards = [torch.empty((sl, w.b, w.h, w.d), dtype=torch.bfloat16, device="cuda")
              for _ in range(w.P)]
    lse = torch.empty((w.b, w.hp, w.s), dtype=torch.float32, device="cuda")
    nbytes = binding.ulys_attn_fwd_workspace_size(w.s, w.b, w.h, w.h_kv, w.d, w.P,
                                                  int(w.causal), code)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    rc = binding.ulys_attn_fwd_push(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                                    [t.data_ptr() for t in shards], rank, lse.data_ptr(), w.s, w.b,
                                    w.h, w.h_kv, w.d, w.P, int(w.causal), code,
                                    ws.data_ptr() if nbytes > 0 else None, nbytes,
                                    torch.cuda.current_stream().cuda_stream)
    assert rc == 0, binding.ulys_status_string(rc)
    torch.cuda.synchronize()
    rows = full_rows(name)
    o_ref, lse_ref = oracle.attn_rows(q, k, v, rows, w.s, w.b, w.h, w.h_kv, w.d, w.P,
                                      w.causal)
    # row (be, i, t) of the share sits in shard t // sl, token t % sl, head rank*hp + i
    got = np.stack([from_dev(shards[int(t) // sl][int(t) % sl, int(be), rank * w.hp + int(i)])
                    for be, i, t in rows])
    err = np.max(np.abs(as_f64(got) - o_ref))
    print(f"  {rows.shape[0]} rows, max err {err:.3e}", flush=True)
    assert err <= TOL[w.dtype]
    lse_h = from_dev(lse)
    assert np.max(np.abs(lse_h[rows[:, 0], rows[:, 1], rows[:, 2]] - lse_ref)) <= LSE_TOL[w.dtype]


@pytest.mark.parametrize("causal", [False, True])
def test_value_ones_gives_ones(causal):
    s, b, h, h_kv, d, P = 777, 1, 4, 2, 128, 1
    q, k, _ = share_inputs(11, s, b, h, h_kv, d, "bf16")
    ones = np.full((s, b, h_kv, d), 0x3F80, dtype=np.uint16)
    o, _ = gpu_attn(q, k, ones, s, b, h, h_kv, d, P, causal, "bf16", want_lse=False)
    assert np.max(np.abs(as_f64(o) - 1.0)) <= TOL["bf16"]


def test_causal_row0_is_v0_and_q_zero_is_mean():
    s, b, h, d = 300, 2, 2, 128
    q, k, v = share_inputs(12, s, b, h, h, d, "bf16")
    o, _ = gpu_attn(q, k, v, s, b, h, h, d, 1, True, "bf16")
    assert np.array_equal(o[0], v[0])  # weight exactly 1 on key 0, exact bf16 round trip
    qz = np.zeros_like(q)
    o, lse = gpu_attn(qz, k, v, s, b, h, h, d, 1, True, "bf16")
    mean = np.cumsum(as_f64(v), axis=0) / np.arange(1, s + 1)[:, None, None, None]
    assert np.max(np.abs(as_f64(o) - mean)) <= TOL["bf16"]
    assert np.max(np.abs(lse - np.log(np.arange(1, s + 1))[None, None, :])) <= 1e-4


def test_large_scores_stay_finite():
    s, b, h, d = 500, 1, 2, 128
    q, k, v = share_inputs(13, s, b, h, h, d, "f32")
    q8 = synth.f32_to_bf16_bits(q * 8.0)
    kb, vb = synth.f32_to_bf16_bits(k), synth.f32_to_bf16_bits(v)
    for causal in (False, True):
        o, lse = gpu_attn(q8, kb, vb, s, b, h, h, d, 1, causal, "bf16")
        o_ref, lse_ref = oracle.attn(q8, kb, vb, s, b, h, h, d, 1, causal)
        assert np.all(np.isfinite(as_f64(o)))
        assert np.max(np.abs(as_f64(o) - o_ref)) <= TOL["bf16"]


def rising_scores_inputs(seed, s, b, h, d, log2_jump_per_tile):
    """Q near a common direction u and keys along u with a magnitude that grows
    with the key index, so a row's scores rise from tile to tile by about
    `log2_jump_per_tile` (log2 units, i.e. scaled by log2(e)/sqrt(d)): every
    64-key tile passes the row's earlier max by that much."""
    q, k, v = share_inputs(seed, s, b, h, h, d, "f32")
    u = np.ones(d)
    raw_per_key = log2_jump_per_tile * np.sqrt(d) / np.log2(np.e) / 64.0
    a = raw_per_key / d * np.arange(s)  # score of key j against u: d * a_j
    qd = u[None, None, None, :] + 0.05 * q
    kd = a[:, None, None, None] * u[None, None, None, :] + 0.05 * k
    return (synth.f32_to_bf16_bits(qd.astype(np.float32)),
            synth.f32_to_bf16_bits(kd.astype(np.float32)), synth.f32_to_bf16_bits(v))


@pytest.mark.parametrize("ws", [False, True], ids=["plain", "ws"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("jump", [15.0, 100.0], ids=["rescale", "overflow-retry"])
def test_rising_scores(jump, causal, ws):
    """Scores that keep rising along the keys.  A jump of 15 log2 units per
    tile makes the fast steps' probability sums pass 2^8, so the reference
    max moves after the PV product; 100 per tile would overflow them, so the
    unit is redone with the row max on every tile.  Both must match the
    oracle."""
    s, b, h, d = 1024, 1, 2, 128
    q, k, v = rising_scores_inputs(15, s, b, h, d, jump)
    o, lse = gpu_attn(q, k, v, s, b, h, h, d, 1, causal, "bf16", ws=ws)
    o_ref, lse_ref = oracle.attn(q, k, v, s, b, h, h, d, 1, causal)
    assert np.all(np.isfinite(as_f64(o))) and np.all(np.isfinite(lse))
    assert np.max(np.abs(as_f64(o) - o_ref)) <= TOL["bf16"]
    # lse is in the thousands here; bf16 inputs make fp32 scores exact to ~1e-7 relative
    assert np.max(np.abs(lse - lse_ref) / np.maximum(1.0, np.abs(lse_ref))) <= 1e-5


def test_deterministic():
    s, b, h, h_kv, d = 2048, 2, 8, 2, 128
    q, k, v = share_inputs(14, s, b, h, h_kv, d, "bf16")
    o1, l1 = gpu_attn(q, k, v, s, b, h, h_kv, d, 1, True, "bf16")
    o2, l2 = gpu_attn(q, k, v, s, b, h, h_kv, d, 1, True, "bf16")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_head_independence_chain():
    """Emulated exchange of all P ranks, then per-rank attention, then the
    reverse exchange, equals unsharded attention over all heads (GQA, causal)."""
    P, s, b, h, h_kv, d = 4, 512, 2, 8, 4, 128
    qg = synth.tensor(1501, (s, b, h, d), "bf16")
    kg = synth.tensor(1502, (s, b, h_kv, d), "bf16")
    vg = synth.tensor(1503, (s, b, h_kv, d), "bf16")
    sl = s // P

    def exchange(glob, heads):
        sends = [binding.pack_seq2head(to_dev(glob.reshape(P, sl, b, heads, d)[j]), P)
                 for j in range(P)]
        return [torch.cat([sends[j][r] for j in range(P)], dim=0) for r in range(P)]

    qs, ks, vs = exchange(qg, h), exchange(kg, h_kv), exchange(vg, h_kv)
    outs = [binding.attn_fwd(qs[r], ks[r], vs[r], P=P, causal=True)[0] for r in range(P)]
    back = [binding.unpack_head2seq(torch.stack([outs[r][j * sl:(j + 1) * sl]
                                                 for r in range(P)])) for j in range(P)]
    torch.cuda.synchronize()
    got = np.concatenate([from_dev(x) for x in back], axis=0)
    o_ref, _ = oracle.attn(qg, kg, vg, s, b, h, h_kv, d, 1, True)
    assert np.max(np.abs(as_f64(got) - o_ref)) <= TOL["bf16"]


def test_workspace_split_matches_plain_32k():
    """At the 32K share the workspace path splits every q-block's keys in two;
    it must agree with the unsplit kernel to bf16 rounding."""
    w = WORKLOADS["gpt1.2b-32k"]
    code = binding.ULYS_BF16
    assert binding.ulys_attn_fwd_workspace_size(w.s, w.b, w.h, w.h_kv, w.d, w.P, 1, code) > 0
    q, k, v = share_inputs(w.c, w.s, w.b, w.hp, w.hkvp, w.d, w.dtype)
    o1, l1 = gpu_attn(q, k, v, w.s, w.b, w.h, w.h_kv, w.d, w.P, True, w.dtype, ws=False)
    o2, l2 = gpu_attn(q, k, v, w.s, w.b, w.h, w.h_kv, w.d, w.P, True, w.dtype, ws=True)
    assert np.max(np.abs(as_f64(o1) - as_f64(o2))) <= 2 ** -7  # one bf16 ulp at |O| < 1
    assert np.max(np.abs(l1.astype(np.float64) - l2)) <= 1e-4
    o3, l3 = gpu_attn(q, k, v, w.s, w.b, w.h, w.h_kv, w.d, w.P, True, w.dtype, ws=True)
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3)  # deterministic


# causal shares whose split units (two per item) fill part of one round of
# workgroups (64, 144 units) or two rounds (512 units, GQA), so that the
# first-round reordering of units covers whole runs, a partial tail and a
# second round
@pytest.mark.parametrize("s,b,h,h_kv,P", [(4096, 1, 16, 16, 8), (6144, 1, 24, 24, 8),
                                          (8192, 2, 32, 8, 8)])
def test_split_unit_rounds(s, b, h, h_kv, P):
    d, hp, hkvp = 128, h // P, h_kv // P
    print(f"case split rounds s={s} b={b} h={h} h_kv={h_kv} P={P}", flush=True)
    q, k, v = share_inputs(21, s, b, hp, hkvp, d, "bf16")
    o, lse = gpu_attn(q, k, v, s, b, h, h_kv, d, P, True, "bf16", ws=True)
    rows = synth.row_sample(2107, s, b, hp, n_random=96, edge=16, tile_bounds=(64, 256))
    o_ref, lse_ref = oracle.attn_rows(q, k, v, rows, s, b, h, h_kv, d, P, True)
    err = np.max(np.abs(as_f64(o[rows[:, 2], rows[:, 0], rows[:, 1]]) - o_ref))
    print(f"  {rows.shape[0]} rows, max err {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    lse_got = lse[rows[:, 0], rows[:, 1], rows[:, 2]].astype(np.float64)
    assert np.max(np.abs(lse_got - lse_ref)) <= LSE_TOL["bf16"]
    assert np.all(np.isfinite(as_f64(o))) and np.all(np.isfinite(lse))


# shares of four or more rounds of workgroups (1024 and 2048 work items):
# with a workspace every workgroup takes its unit from a counter, and the
# result must be the plain call's, bit for bit (every unit computed once)
@pytest.mark.parametrize("s,b,h,h_kv,d,P,causal", [(32768, 1, 64, 64, 128, 8, True),
                                                   (32768, 1, 64, 64, 128, 8, False),
                                                   (16384, 4, 64, 16, 128, 8, True),
                                                   (32768, 1, 64, 64, 64, 8, True)])
def test_workspace_counter_matches_plain(s, b, h, h_kv, d, P, causal):
    code = binding.ULYS_BF16
    print(f"case counter s={s} b={b} h={h} h_kv={h_kv} d={d} P={P} causal={causal}", flush=True)
    assert binding.ulys_attn_fwd_workspace_size(s, b, h, h_kv, d, P, int(causal), code) == 256
    q, k, v = share_inputs(31, s, b, h // P, h_kv // P, d, "bf16")
    o1, l1 = gpu_attn(q, k, v, s, b, h, h_kv, d, P, causal, "bf16", ws=False)
    for _ in range(2):  # the counter is cleared by every call
        o2, l2 = gpu_attn(q, k, v, s, b, h, h_kv, d, P, causal, "bf16", ws=True)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_workspace_counter_two_streams():
    """Two long-share calls in flight at once on two streams, each with its own
    workspace (and so its own unit counter), give the plain calls' results."""
    s, b, h, h_kv, d, P = 32768, 1, 64, 64, 128, 8
    hp, hkvp, code = h // P, h_kv // P, binding.ULYS_BF16
    nbytes = binding.ulys_attn_fwd_workspace_size(s, b, h, h_kv, d, P, 1, code)
    assert nbytes == 256
    dev()
    ins = [tuple(to_dev(x) for x in share_inputs(41 + i, s, b, hp, hkvp, d, "bf16"))
           for i in range(2)]
    # the reference: ulys_attn_fwd, no workspace and so no counter
    plain = [torch.empty_like(q) for q, _, _ in ins]
    for (q, k, v), o in zip(ins, plain):
        rc = binding.ulys_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), None,
                                   s, b, h, h_kv, d, P, 1, code,
                                   torch.cuda.current_stream().cuda_stream)
        assert rc == 0, binding.ulys_status_string(rc)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = [torch.empty_like(ins[i][0]) for i in range(2)]
    wss = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    for _ in range(3):
        for i in range(2):
            q, k, v = ins[i]
            rc = binding.ulys_attn_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          outs[i].data_ptr(), None, s, b, h, h_kv, d, P, 1, code,
                                          wss[i].data_ptr(), nbytes, streams[i].cuda_stream)
            assert rc == 0, binding.ulys_status_string(rc)
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], plain[i])


def test_helper_on_a_side_stream():
    """The binding's tensor helpers run on the stream they are given; the
    workspace and outputs they allocate stay reserved for that stream, and the
    results equal the ones on torch's current stream (a long share, so the
    forward's workspace holds the unit counter and the backward's the dQ
    counter)."""
    s, b, h, h_kv, d, P = 32768, 1, 64, 64, 128, 8
    dev()
    q, k, v = (to_dev(x) for x in share_inputs(51, s, b, h // P, h_kv // P, d, "bf16"))
    g = to_dev(synth.tensor(5104, (s, b, h // P, d), "bf16"))
    o_ref, l_ref = binding.attn_fwd(q, k, v, P=P, causal=True, lse=True)
    grads_ref = binding.attn_bwd(q, k, v, o_ref, g, l_ref, P=P, causal=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(2):
        o, lse = binding.attn_fwd(q, k, v, P=P, causal=True, lse=True, stream=side.cuda_stream)
        grads = binding.attn_bwd(q, k, v, o, g, lse, P=P, causal=True, stream=side.cuda_stream)
        # allocations on the current stream meanwhile must not take the
        # side stream's workspace
        junk = [torch.full((1 << 20,), 7, dtype=torch.uint8, device="cuda") for _ in range(8)]
        side.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        for x, y in zip(grads, grads_ref):
            assert torch.equal(x, y)
        del junk
