"""GPU parity of pack (seq->head send side) and unpack (head->seq receive side):
bit-exact against the CPU oracle, guard bands intact, on random bit patterns."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import Guarded, dev, from_dev, to_dev
from ulysses_head_sharded_amd import binding, synth
from ulysses_head_sharded_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

NP_DT = {2: np.uint16, 4: np.float32}
TORCH_DT = {2: torch.bfloat16, 4: torch.float32}
CODE = {2: binding.ULYS_BF16, 4: binding.ULYS_F32}


def run_pack_unpack(x_host, s, b, h, d, P, elt):
    """pack then unpack through the C ABI into guarded buffers."""
    dev()
    x = to_dev(x_host)
    y = Guarded((P, s // P, b, h // P, d), TORCH_DT[elt])
    rc = binding.ulys_pack_seq2head(x.data_ptr(), y.tensor.data_ptr(), s, b, h, d, P, CODE[elt],
                                    torch.cuda.current_stream().cuda_stream)
    assert rc == 0, binding.ulys_status_string(rc)
    z = Guarded((s // P, b, h, d), TORCH_DT[elt])
    rc = binding.ulys_unpack_head2seq(y.tensor.data_ptr(), z.tensor.data_ptr(), s, b, h, d, P,
                                      CODE[elt], torch.cuda.current_stream().cuda_stream)
    assert rc == 0, binding.ulys_status_string(rc)
    torch.cuda.synchronize()
    assert y.guards_intact() and z.guards_intact()
    return from_dev(y.tensor), from_dev(z.tensor)


def bits(seed, shape, elt):
    n = int(np.prod(shape))
    raw = synth.random_bits(seed, n * elt)
    return raw.view(NP_DT[elt]).reshape(shape)


def same_bits(a, b):
    return np.array_equal(a.view(np.uint8), b.view(np.uint8))


# K/V of a share with fewer KV heads than ranks go through the replicating
# entry points instead (tests/test_gpu_kv_replication.py)
PLAIN = [(n, kv) for n in WORKLOADS for kv in (False, True)
         if not (kv and WORKLOADS[n].h_kv % WORKLOADS[n].P)]


@pytest.mark.parametrize("name,kv", PLAIN, ids=[f"{n}-{'kv' if kv else 'q'}" for n, kv in PLAIN])
def test_workload_pack_unpack_bit_exact(name, kv):
    w = WORKLOADS[name]
    h = w.h_kv if kv else w.h
    shape = (w.s // w.P, w.b, h, w.d)
    print(f"case {name} kv={kv} shape={shape}", flush=True)
    x = bits(100 * w.c + 9 + int(kv), shape, w.elt)
    y, z = run_pack_unpack(x, w.s, w.b, h, w.d, w.P, w.elt)
    y_ref = oracle.pack(x, w.s, w.b, h, w.d, w.P)
    assert same_bits(y, y_ref)
    assert same_bits(z, x)          # unpack(pack(x)) = x
    assert same_bits(oracle.unpack(y_ref, w.s, w.b, h, w.d, w.P), x)


SMALL = [(s, b, h, d, P, elt)
         for (s, h, P) in [(1, 1, 1), (2, 2, 2), (6, 6, 3), (12, 8, 4), (16, 16, 16),
                           (40, 8, 8), (7, 3, 1), (64, 4, 2)]
         for b in (1, 2) for d in (1, 3, 8, 64) for elt in (2, 4)]


@pytest.mark.parametrize("s,b,h,d,P,elt", SMALL)
def test_small_shapes_bit_exact(s, b, h, d, P, elt):
    x = bits(9000 + s * 7 + h * 3 + d + b + elt, (s // P, b, h, d), elt)
    y, z = run_pack_unpack(x, s, b, h, d, P, elt)
    assert same_bits(y, oracle.pack(x, s, b, h, d, P))
    assert same_bits(z, x)


# shapes whose pack takes the LDS-staged tile transpose (runs of at most 256
# bytes, input rows of at least 8 KiB, at least as many token rows as ranks):
# 256-byte runs over 32 and 64 ranks, 128-byte runs over 64 ranks; the unpack
# of the same shapes takes the output-order walk
LDS_TILE = [(1024, 1, 32, 128, 32, 2), (2048, 2, 64, 64, 64, 4), (4096, 1, 64, 64, 64, 2),
            (8192, 3, 64, 128, 64, 2)]


@pytest.mark.parametrize("s,b,h,d,P,elt", LDS_TILE)
def test_lds_tile_shapes_bit_exact(s, b, h, d, P, elt):
    print(f"case lds tile s={s} b={b} h={h} d={d} P={P} elt={elt}", flush=True)
    x = bits(9500 + s + h + d + b + elt, (s // P, b, h, d), elt)
    y, z = run_pack_unpack(x, s, b, h, d, P, elt)
    assert same_bits(y, oracle.pack(x, s, b, h, d, P))
    assert same_bits(z, x)


def test_unpack_alone_matches_oracle():
    s, b, h, d, P, elt = 48, 2, 12, 16, 4, 2
    y_host = bits(4242, (P, s // P, b, h // P, d), elt)
    dev()
    y = to_dev(y_host)
    out = Guarded((s // P, b, h, d), torch.bfloat16)
    binding.unpack_head2seq(y, out=out.tensor)
    torch.cuda.synchronize()
    assert out.guards_intact()
    assert same_bits(from_dev(out.tensor), oracle.unpack(y_host, s, b, h, d, P))


def test_exchange_chain_identity_tiny():
    """All 4 ranks of the tiny workload: pack -> route -> (route back) -> unpack
    returns every rank's shard bit for bit, and the routed shares equal the
    oracle's whole exchange."""
    w = WORKLOADS["tiny"]
    s, b, h, d, P = w.s, w.b, w.h, w.d, w.P
    x_all = bits(109, (P, s // P, b, h, d), 4)
    shards = [to_dev(x_all[j]) for j in range(P)]
    sends = [binding.pack_seq2head(x, P) for x in shards]
    shares = [torch.cat([sends[j][r] for j in range(P)], dim=0) for r in range(P)]
    sl = s // P
    back = [binding.unpack_head2seq(torch.stack([shares[r][j * sl:(j + 1) * sl]
                                                 for r in range(P)])) for j in range(P)]
    torch.cuda.synchronize()
    y_ref = oracle.seq2head(x_all, s, b, h, d, P)
    for r in range(P):
        assert same_bits(from_dev(shares[r]), y_ref[r])
    for j in range(P):
        assert same_bits(from_dev(back[j]), x_all[j])


def test_deterministic_and_stream_ordered():
    s, b, h, d, P = 4096, 2, 16, 128, 8
    x = to_dev(bits(77, (s // P, b, h, d), 2))
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        y1 = binding.pack_seq2head(x, P)
        y2 = binding.pack_seq2head(x, P)
    st.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def run_pack_qkv(xq, xk, xv, s, b, h, h_kv, d, P, elt):
    """ulys_pack_seq2head_qkv into guarded buffers."""
    dev()
    hk = h_kv // P if h_kv % P == 0 else 1
    ins = [to_dev(x) for x in (xq, xk, xv)]
    outs = [Guarded((P, s // P, b, hh, d), TORCH_DT[elt]) for hh in (h // P, hk, hk)]
    rc = binding.ulys_pack_seq2head_qkv(*(t.data_ptr() for t in ins),
                                        *(g.tensor.data_ptr() for g in outs), s, b, h, h_kv, d, P,
                                        CODE[elt], torch.cuda.current_stream().cuda_stream)
    assert rc == 0, binding.ulys_status_string(rc)
    torch.cuda.synchronize()
    assert all(g.guards_intact() for g in outs)
    return [from_dev(g.tensor) for g in outs]


QKV_CASES = [(w.s, w.b, w.h, w.h_kv, w.d, w.P, w.elt, n) for n, w in WORKLOADS.items()] + [
    (40, 2, 8, 2, 64, 8, 2, "replicated"), (24, 1, 12, 3, 128, 6, 4, "replicated-f32"),
    (12, 2, 8, 8, 3, 4, 2, "vectorless"), (16, 1, 4, 1, 8, 4, 4, "mqa")]


@pytest.mark.parametrize("s,b,h,h_kv,d,P,elt,name", QKV_CASES, ids=[c[-1] for c in QKV_CASES])
def test_pack_qkv_bit_exact(s, b, h, h_kv, d, P, elt, name):
    """One call packs Q (plain) and K, V (plain, or replicated when h_kv < P)
    exactly as the oracle's three separate packs."""
    print(f"case pack_qkv {name} s={s} b={b} h={h} h_kv={h_kv} d={d} P={P} elt={elt}", flush=True)
    xq = bits(3000 + s, (s // P, b, h, d), elt)
    xk = bits(3001 + s, (s // P, b, h_kv, d), elt)
    xv = bits(3002 + s, (s // P, b, h_kv, d), elt)
    yq, yk, yv = run_pack_qkv(xq, xk, xv, s, b, h, h_kv, d, P, elt)
    assert same_bits(yq, oracle.pack(xq, s, b, h, d, P))
    assert same_bits(yk, oracle.pack_kv(xk, s, b, h_kv, d, P))
    assert same_bits(yv, oracle.pack_kv(xv, s, b, h_kv, d, P))
