"""ulys_attn_fwd_noalloc, the forward for callers that cannot allocate: its
workspace is the library's fixed device scratch instead of caller memory.

Checked through the C ABI against ulys_attn_fwd_ws with a caller-owned
workspace of the size it asks for: the same kernels on the same inputs, so
O and LSE must agree bit for bit (stricter than the 2e-2 bound the attention
is held to against the oracle).  The calls run in a row on one stream, each
on a smaller input than the one before where the scratch use allows: the
unit counter of a long share, the split partial states of the 32K share,
a smaller split share, a shorter counter share, and a share that needs no
workspace -- so every call finds the previous call's leftovers in the
scratch.  A share whose split states would not fit is rejected before any
launch.
"""
import numpy as np
import pytest
import torch

from gpu_util import dev, share_inputs, to_dev
from ulysses_head_sharded_amd import binding

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 96 << 20

# (s, b, h, h_kv, d, P, causal), in the order they run
SEQUENCE = [
    (32768, 1, 64, 64, 128, 8, True),   # 1024 items: the unit counter
    (32768, 1, 16, 16, 128, 8, True),   # 256 items: split halves, ~69 MB of partial states
    (4096, 1, 16, 16, 128, 8, True),    # 32 items: split halves, smaller
    (16384, 2, 64, 16, 128, 8, True),   # 1024 GQA items: the counter again
    (1000, 2, 8, 2, 64, 2, False),      # dense: no workspace at all
]


def run_ws(q, k, v, s, b, h, h_kv, d, P, causal, nbytes):
    hp = h // P
    o = torch.empty((s, b, hp, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, hp, s), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    rc = binding.ulys_attn_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), s, b, h, h_kv, d, P, int(causal),
                                  binding.ULYS_BF16, ws.data_ptr() if nbytes > 0 else None,
                                  nbytes, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, binding.ulys_status_string(rc)
    return o, lse


def run_noalloc(q, k, v, s, b, h, h_kv, d, P, causal):
    hp = h // P
    o = torch.empty((s, b, hp, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, hp, s), dtype=torch.float32, device="cuda")
    rc = binding.ulys_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       lse.data_ptr(), s, b, h, h_kv, d, P, int(causal),
                                       binding.ULYS_BF16, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, binding.ulys_status_string(rc)
    return o, lse


def test_noalloc_matches_workspace_calls_in_a_row():
    dev()
    for n, (s, b, h, h_kv, d, P, causal) in enumerate(SEQUENCE):
        print(f"case noalloc #{n}: s={s} b={b} h={h} h_kv={h_kv} d={d} P={P} causal={causal}",
              flush=True)
        nbytes = binding.ulys_attn_fwd_workspace_size(s, b, h, h_kv, d, P, int(causal),
                                                      binding.ULYS_BF16)
        assert 0 <= nbytes <= SCRATCH_BYTES
        q, k, v = (to_dev(x) for x in share_inputs(60 + n, s, b, h // P, h_kv // P, d, "bf16"))
        o_ref, l_ref = run_ws(q, k, v, s, b, h, h_kv, d, P, causal, nbytes)
        torch.cuda.synchronize()
        for _ in range(2):
            o, lse = run_noalloc(q, k, v, s, b, h, h_kv, d, P, causal)
            torch.cuda.synchronize()
            assert torch.equal(o, o_ref), f"O differs, case #{n}"
            assert torch.equal(lse, l_ref), f"LSE differs, case #{n}"
            assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_noalloc_rejects_beyond_the_scratch():
    """s = 51200 with two heads of 128 per share: 400 causal items, split in
    halves, whose partial states (~108 MB) exceed the 96 MiB scratch."""
    dev()
    s, b, h, h_kv, d, P = 51200, 1, 16, 16, 128, 8
    nbytes = binding.ulys_attn_fwd_workspace_size(s, b, h, h_kv, d, P, 1, binding.ULYS_BF16)
    assert nbytes > SCRATCH_BYTES
    hp = h // P
    q = torch.zeros((s, b, hp, d), dtype=torch.bfloat16, device="cuda")
    k, v = torch.zeros_like(q), torch.zeros_like(q)
    o = torch.full_like(q, 3.0)
    rc = binding.ulys_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       None, s, b, h, h_kv, d, P, 1, binding.ULYS_BF16,
                                       torch.cuda.current_stream().cuda_stream)
    assert rc == binding.ULYS_ERR_DIM
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())  # nothing was launched
    # the shares that fit still run after the rejection
    s2 = 4096
    q2, k2, v2 = (to_dev(x) for x in share_inputs(70, s2, b, hp, hp, d, "bf16"))
    n2 = binding.ulys_attn_fwd_workspace_size(s2, b, h, h_kv, d, P, 1, binding.ULYS_BF16)
    o_ref, l_ref = run_ws(q2, k2, v2, s2, b, h, h_kv, d, P, True, n2)
    o2, l2 = run_noalloc(q2, k2, v2, s2, b, h, h_kv, d, P, True)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref) and torch.equal(l2, l_ref)
    assert np.isfinite(l2.cpu().numpy()).all()
