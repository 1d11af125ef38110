"""The whole layer at a full workload size on one GPU, every emulated rank
resident, against the oracle's attention over the global (unsharded)
tensors ("02 · DeepSpeed-Ulysses" §2: the two all-to-alls are a transpose
and its inverse; "DeepSpeed-Ulysses 深度解析", core design steps 3-5: exchange
Q, K and V, attend per head group over the whole sequence, exchange the
output back).

Each rank's Q, K and V shards are packed in one call
(ulys_pack_seq2head_qkv), block r of every sender is routed to rank r in
source order (the one-GPU stand-in for the all-to-all: the P received blocks
are the rank's [s, b, h/P, d] share), and every rank runs the bench step's
attention, ulys_attn_fwd_push with the workspace it asks for, whose epilogue
writes each output row into the P ranks' output shards.  The shards,
concatenated along the sequence, are the layer's output [s, b, h, d].

Compared, every element: whole work units of the attention kernel -- the
first, a middle and the last query block of the listed query heads (256
queries of one head at the 32K and 128K shares, 64 queries of each of the
four heads of a KV group at the GQA share; with the workspace the 32K share's
blocks run their keys as two halves merged afterwards, so both halves of
every block are covered) -- and their log-sum-exp.  At the 32K share every
head is listed; at the 128K and GQA shares the heads of the first, a middle
and the last rank (the oracle's cost grows with s^2), whose inputs are drawn
on the device (synth.device_normal_bf16) and copied back for the oracle.
Bound: max |O - O_ref| <= 2e-2 (bf16 inputs, fp64 oracle on the same bits);
LSE to 1e-3.  Every element of the layer's output is finite and inside the
range of V.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import as_f64, dev, from_dev, to_dev
from ulysses_head_sharded_amd import binding, synth
from ulysses_head_sharded_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

TOL, LSE_TOL = 2e-2, 1e-3


def query_block(w) -> int:
    """Queries per head of one work unit of the forward kernel: 8 waves of 32
    queries spread over the query heads that share a KV head (up to 8)."""
    G = w.hp // w.hkvp
    qh = 8 if G % 8 == 0 else 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1
    return 32 * (8 // qh)


# workload -> (query heads whose units are compared, inputs drawn on the device)
CASES = {
    "gpt1.2b-32k": (None, False),
    "mha-128k": ((0, 1, 12, 13, 14, 15, 30, 31), True),
    "gqa-64k": ((0, 1, 2, 3, 12, 13, 14, 15, 28, 29, 30, 31), True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_chain_full_size(name):
    w = WORKLOADS[name]
    heads_listed, on_device = CASES[name]
    P, s, b, h, h_kv, d = w.P, w.s, w.b, w.h, w.h_kv, w.d
    sl, hp, hkvp = s // P, w.hp, w.hkvp
    print(f"case chain {name}: P={P} s={s} b={b} h={h} h_kv={h_kv}", flush=True)
    dev()
    # the global tensors; rank j's shard is rows [j*sl, (j+1)*sl) (contiguous
    # chunks), so rank 0's shard is the bench's rank-local input
    if on_device:
        xq = synth.device_normal_bf16(100 * w.c + 11, (s, b, h, d))
        xk = synth.device_normal_bf16(100 * w.c + 12, (s, b, h_kv, d))
        xv = synth.device_normal_bf16(100 * w.c + 13, (s, b, h_kv, d))
        qg, kg, vg = from_dev(xq), from_dev(xk), from_dev(xv)
    else:
        qg = synth.tensor(100 * w.c + 1, (s, b, h, d), w.dtype)
        kg = synth.tensor(100 * w.c + 2, (s, b, h_kv, d), w.dtype)
        vg = synth.tensor(100 * w.c + 3, (s, b, h_kv, d), w.dtype)
        xq, xk, xv = to_dev(qg), to_dev(kg), to_dev(vg)
    print("  inputs drawn", flush=True)
    vmax = float(xv.abs().max())
    code = binding.ULYS_BF16
    stream = torch.cuda.current_stream().cuda_stream
    bf = torch.bfloat16
    yq = torch.empty((P, P, sl, b, hp, d), dtype=bf, device="cuda")  # [sender][block]
    yk = torch.empty((P, P, sl, b, hkvp, d), dtype=bf, device="cuda")
    yv = torch.empty_like(yk)
    for j in range(P):
        rc = binding.ulys_pack_seq2head_qkv(xq[j * sl:(j + 1) * sl].data_ptr(),
                                            xk[j * sl:(j + 1) * sl].data_ptr(),
                                            xv[j * sl:(j + 1) * sl].data_ptr(),
                                            yq[j].data_ptr(), yk[j].data_ptr(), yv[j].data_ptr(),
                                            s, b, h, h_kv, d, P, code, stream)
        assert rc == 0, binding.ulys_status_string(rc)
    del xq, xk, xv
    # rank r receives block r of every sender j, in source order: its share
    shares = [tuple(y[:, r].contiguous().view(s, b, heads, d)
                    for y, heads in ((yq, hp), (yk, hkvp), (yv, hkvp))) for r in range(P)]
    del yq, yk, yv
    out = [torch.empty((sl, b, h, d), dtype=bf, device="cuda") for _ in range(P)]
    lse = torch.empty((P, b, hp, s), dtype=torch.float32, device="cuda")
    ws_bytes = binding.ulys_attn_fwd_workspace_size(s, b, h, h_kv, d, P, int(w.causal), code)
    assert ws_bytes >= 0
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    for r in range(P):
        q, k, v = shares[r]
        rc = binding.ulys_attn_fwd_push(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        [t.data_ptr() for t in out], r, lse[r].data_ptr(), s, b,
                                        h, h_kv, d, P, int(w.causal), code,
                                        ws.data_ptr() if ws_bytes > 0 else None, ws_bytes,
                                        stream)
        assert rc == 0, binding.ulys_status_string(rc)
    torch.cuda.synchronize()
    del shares
    # every element of the layer's output is finite and inside the range of V
    for t in out:
        assert bool(torch.isfinite(t).all())
        assert float(t.abs().max()) <= vmax + TOL
    assert bool(torch.isfinite(lse).all())
    got = np.concatenate([from_dev(t) for t in out], axis=0)  # [s, b, h, d]
    lse_h = from_dev(lse)                                      # [P, b, hp, s]
    del out, lse
    torch.cuda.empty_cache()
    print("  chain done on the GPU", flush=True)

    # whole work units: first, middle and last query block of the listed heads
    qb = query_block(w)
    nblk = (s + qb - 1) // qb
    ts = np.concatenate([np.arange(blk * qb, min(s, (blk + 1) * qb))
                         for blk in sorted({0, nblk // 2, nblk - 1})])
    heads = range(h) if heads_listed is None else heads_listed
    rows = np.array([(be, head, t) for be in range(b) for head in heads for t in ts],
                    dtype=np.int64)
    o_ref, lse_ref = oracle.attn_rows(qg, kg, vg, rows, s, b, h, h_kv, d, 1, w.causal)
    g = as_f64(got[rows[:, 2], rows[:, 0], rows[:, 1]])
    err = np.max(np.abs(g - o_ref))
    rank, i = rows[:, 1] // hp, rows[:, 1] % hp
    lerr = np.max(np.abs(lse_h[rank, rows[:, 0], i, rows[:, 2]].astype(np.float64) - lse_ref))
    print(f"  {rows.shape[0]} rows ({len(ts)} per head), max err {err:.3e}, lse {lerr:.3e}",
          flush=True)
    assert err <= TOL
    assert lerr <= LSE_TOL
