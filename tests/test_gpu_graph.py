"""The allocation-free forward inside a captured HIP graph, the use it exists
for: ulys_attn_fwd_noalloc is captured once (torch.cuda.graph, on torch's
capture stream) and the graph is replayed several times, with eager work of
the program's own and synchronisations between the replays; every replay's
O and LSE must equal the eager ulys_attn_fwd_ws result bit for bit (the same
kernels on the same inputs).  Nothing the call enqueues is a memset: the unit
counter is cleared by a one-wave kernel, and the split path's partial states
are written before they are read.

Shares: a long one (the unit counter), the 32K share's shape with fewer heads
(split halves and their merge) and a dense one (no workspace).  The
allocation-free entry point is called once eagerly first, so that the scratch
array's device address is resolved before the capture starts.
"""
import pytest
import torch

from gpu_util import dev, share_inputs, to_dev
from ulysses_head_sharded_amd import binding

pytestmark = pytest.mark.gpu


def call_noalloc(q, k, v, o, lse, s, b, h, h_kv, d, P, causal):
    rc = binding.ulys_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       lse.data_ptr(), s, b, h, h_kv, d, P, int(causal),
                                       binding.ULYS_BF16, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, binding.ulys_status_string(rc)


@pytest.mark.parametrize("s,b,h,h_kv,d,P,causal", [
    (32768, 1, 64, 64, 128, 8, True),    # 1024 items, four rounds: the unit counter
    (8192, 1, 16, 16, 128, 8, True),     # 64 items: split halves and their merge
    (1000, 2, 8, 2, 64, 2, False),       # dense: no workspace
], ids=["counter", "split", "dense"])
def test_noalloc_in_a_captured_graph(s, b, h, h_kv, d, P, causal):
    dev()
    print(f"case graph s={s} b={b} h={h} h_kv={h_kv} d={d} P={P} causal={causal}", flush=True)
    hp = h // P
    q, k, v = (to_dev(x) for x in share_inputs(80, s, b, hp, h_kv // P, d, "bf16"))
    # the eager reference through the workspace entry point
    nbytes = binding.ulys_attn_fwd_workspace_size(s, b, h, h_kv, d, P, int(causal),
                                                  binding.ULYS_BF16)
    assert nbytes >= 0
    o_ref = torch.empty((s, b, hp, d), dtype=torch.bfloat16, device="cuda")
    l_ref = torch.empty((b, hp, s), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    rc = binding.ulys_attn_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_ref.data_ptr(),
                                  l_ref.data_ptr(), s, b, h, h_kv, d, P, int(causal),
                                  binding.ULYS_BF16, ws.data_ptr() if nbytes > 0 else None,
                                  nbytes, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, binding.ulys_status_string(rc)
    # static outputs of the graph; one eager call resolves the scratch address
    o = torch.empty_like(o_ref)
    lse = torch.empty_like(l_ref)
    call_noalloc(q, k, v, o, lse, s, b, h, h_kv, d, P, causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):   # captures on torch's own side stream
        call_noalloc(q, k, v, o, lse, s, b, h, h_kv, d, P, causal)
    torch.cuda.synchronize()
    junk = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for rep in range(4):
        # eager work of the program's own between the replays: scribble over
        # the outputs (and other memory) so each replay must rewrite them
        o.fill_(7.0)
        lse.fill_(-3.0)
        junk.normal_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"O differs on replay {rep}"
        assert torch.equal(lse, l_ref), f"LSE differs on replay {rep}"
    del graph
