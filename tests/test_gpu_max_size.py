"""GPU parity at the largest sizes the C ABI accepts.

* Layout: tensors past 4 GiB, so byte offsets need more than 32 bits (the
  kernels index 16-byte vectors with 32-bit integers below 2^32 vectors):
  once through the output-order walk (2560-byte runs over 8 ranks) and once
  through the LDS-tiled pack (256-byte runs over 64 ranks).
* Attention, forward and backward: the bf16 kernels address every tensor
  with 32-bit byte offsets, and the ABI admits a share while
  bytes + one 256-row block stay below 2^31.  s = 1048312 with 8 local heads
  of 128 sits 16 KiB under that bound (s + 8 is refused), and its last query
  block is ragged (248 rows), so the largest offsets the kernels form, the
  ragged tail's included, are exercised.

The inputs are drawn on the device (``synth.device_normal_bf16``: torch's
seeded Philox generator; the host draws gigabytes too slowly for a test) and
copied back for the oracle, which computes sampled rows and keys one by one
(the first, the last and the ragged block, block boundaries and random rows,
for the first, a middle and the last local head); every output is also
checked finite and, for attention, inside the convex hull bound |O| <= max |V|.
Tolerances as in the other parity tests: 2e-2 absolute on O, 1e-3 on LSE, 2e-2
of each gradient's scale."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import as_f64, dev, from_dev
from ulysses_head_sharded_amd import binding, synth

pytestmark = pytest.mark.gpu

S, B, H, D, P = 1048312, 1, 64, 128, 8   # hp = 8 local heads, MHA
HP = H // P
TOL, LSE_TOL, REL = 2e-2, 1e-3, 2e-2


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def at(t, idx):
    """Rows of a device tensor at host index arrays, copied to the host."""
    return from_dev(t[tuple(torch.from_numpy(np.ascontiguousarray(i)).to(t.device)
                            for i in idx)])


@pytest.mark.parametrize("sl,h,Pr", [(262144, 80, 8), (327680, 64, 64)],
                         ids=["walk-2560B-runs", "lds-tile-256B-runs"])
def test_layout_past_4gib(sl, h, Pr):
    dev()
    hp = h // Pr
    nbytes = sl * B * h * D * 2
    assert nbytes > (1 << 32)
    print(f"case layout sl={sl} h={h} P={Pr}: {nbytes / 2**30:.2f} GiB", flush=True)
    x = synth.device_bits(4101, (sl, B, h, D)).view(torch.bfloat16)
    y = binding.pack_seq2head(x, Pr)
    torch.cuda.synchronize()
    # the pack is row-local: the oracle's pack of a few rows equals those rows
    # of every block
    xh = x.view(torch.int16)
    yh = y.view(torch.int16)
    for t0 in (0, sl // 2 + 3, sl - 8):
        part = from_dev(xh[t0:t0 + 8].contiguous().view(torch.bfloat16))
        ref = oracle.pack(part, 8 * Pr, B, h, D, Pr)
        got = from_dev(yh[:, t0:t0 + 8].contiguous().view(torch.bfloat16))
        assert np.array_equal(got, ref), t0
    # block r is head group r of every row (the defining slice), for the first,
    # a middle and the last rank
    xv = xh.view(sl, B, Pr, hp, D)
    for r in sorted({0, Pr // 2, Pr - 1}):
        assert torch.equal(yh[r], xv[:, :, r]), r
    del xv
    back = binding.unpack_head2seq(y)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), xh)
    del x, y, back, xh, yh
    free()


def rows_to_check(s, seed):
    ts = {0, 1, 63, 64, 255, 256, s // 2 - 1, s // 2, (1 << 19) + 7}
    last_blk = (s - 1) // 256 * 256
    ts.update({last_blk - 1, last_blk, last_blk + 1, s - 2, s - 1})
    u = synth.uniform01(seed, 6)
    ts.update(int(x) for x in np.minimum((u * s).astype(np.int64), s - 1))
    return np.array([(0, i, t) for i in (0, HP // 2, HP - 1) for t in sorted(ts)],
                    dtype=np.int64)


def test_attention_at_the_offset_limit():
    dev()
    code = binding.ULYS_BF16
    assert binding.ulys_attn_fwd_workspace_size(S, B, H, H, D, P, 1, code) >= 0
    assert binding.ulys_attn_fwd_workspace_size(S + P, B, H, H, D, P, 1, code) == \
        binding.ULYS_ERR_DIM
    print(f"case attention s={S} b={B} hp={HP} d={D} causal", flush=True)
    q = synth.device_normal_bf16(4111, (S, B, HP, D))
    k = synth.device_normal_bf16(4112, (S, B, HP, D))
    v = synth.device_normal_bf16(4113, (S, B, HP, D))
    o, lse = binding.attn_fwd(q, k, v, P=P, causal=True, lse=True)
    torch.cuda.synchronize()
    print("  forward done", flush=True)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    assert float(o.abs().max()) <= float(v.abs().max()) + TOL
    rows = rows_to_check(S, 4117)
    qh, kh, vh = from_dev(q), from_dev(k), from_dev(v)
    o_ref, lse_ref = oracle.attn_rows(qh, kh, vh, rows, S, B, H, H, D, P, True)
    oh = at(o, (rows[:, 2], rows[:, 0], rows[:, 1]))
    lh = from_dev(lse)[rows[:, 0], rows[:, 1], rows[:, 2]].astype(np.float64)
    err = np.max(np.abs(as_f64(oh) - o_ref))
    lerr = np.max(np.abs(lh - lse_ref))
    print(f"  {rows.shape[0]} rows: max err {err:.3e}, lse {lerr:.3e}", flush=True)
    assert err <= TOL and lerr <= LSE_TOL
    del q, k, v, o, lse
    free()


def check(name, got, ref):
    err = np.max(np.abs(as_f64(got) - ref))
    bound = REL * max(1.0, float(np.max(np.abs(ref))))
    print(f"  {name}: max err {err:.3e} (bound {bound:.3e})", flush=True)
    assert err <= bound, (name, err, bound)


def test_backward_at_the_offset_limit():
    dev()
    code = binding.ULYS_BF16
    need = binding.ulys_attn_bwd_workspace_size(S, B, H, H, D, P, 1, code)
    assert need > 0, binding.ulys_status_string(int(need))
    print(f"case backward s={S} b={B} hp={HP} d={D} causal, workspace {need} bytes", flush=True)
    q = synth.device_normal_bf16(4121, (S, B, HP, D))
    k = synth.device_normal_bf16(4122, (S, B, HP, D))
    v = synth.device_normal_bf16(4123, (S, B, HP, D))
    dout = synth.device_normal_bf16(4124, (S, B, HP, D))
    o, lse = binding.attn_fwd(q, k, v, P=P, causal=True, lse=True)
    dq, dk, dv = binding.attn_bwd(q, k, v, o, dout, lse, P=P, causal=True)
    torch.cuda.synchronize()
    print("  backward done", flush=True)
    for g in (dq, dk, dv):
        assert bool(torch.isfinite(g).all())
    del o, lse
    # dq at sampled rows; dk, dv at late keys (a causal key j is seen only by
    # the rows t >= j, so the oracle evaluates them one by one)
    qrows = rows_to_check(S, 4127)[::2]
    js = np.array([S - 1, S - 2, S - 5, S - 16], dtype=np.int64)
    krows = np.array([(0, i, j) for i in (0, HP - 1) for j in js], dtype=np.int64)
    qh, kh, vh, gh = from_dev(q), from_dev(k), from_dev(v), from_dev(dout)
    rq, rk, rv = oracle.attn_bwd_rows(qh, kh, vh, gh, qrows, krows, S, B, H, H, D, P, True)
    check("dq rows", at(dq, (qrows[:, 2], qrows[:, 0], qrows[:, 1])), rq)
    check("dk keys", at(dk, (krows[:, 2], krows[:, 0], krows[:, 1])), rk)
    check("dv keys", at(dv, (krows[:, 2], krows[:, 0], krows[:, 1])), rv)
    del q, k, v, dout, dq, dk, dv
    free()
