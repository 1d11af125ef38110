"""bench.py's command-line contract, on the CPU: more than one GPU is refused
with a message before anything touches a GPU, and the workload table holds
every shape the bench line can name with its algorithmic work."""
import os
import subprocess
import sys

from ulysses_head_sharded_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "ONE GPU" in r.stderr and r.stdout == ""


def test_workload_flops_and_bytes():
    w = WORKLOADS["gpt1.2b-32k"]
    # 4 d_h b hp s(s+1)/2 = 5.4977e11 for this share
    assert w.attn_flops() == 4 * 128 * 1 * 2 * (32768 * 32769 // 2)
    assert abs(w.attn_flops() - 5.4977e11) / 5.4977e11 < 1e-4
    assert w.attn_bwd_flops() == 2.5 * w.attn_flops()
    # pack Q, K, V + unpack O, read + write: 4 tensors x 2 x 16 MiB
    assert w.layout_bytes() == 8 * 16 * 2 ** 20
    g = WORKLOADS["gqa-64k-p16"]
    assert g.hkvp == 1 and g.hp == 2
    # a replicated K block set is P/h_kv = 2 times the K shard
    assert g.kv_blocks_bytes() == 2 * g.shard_bytes(kv=True)
    for w in WORKLOADS.values():
        assert w.s % w.P == 0 and w.h % w.P == 0 and w.h % w.h_kv == 0


def test_settle_waits_for_the_step_time_to_stop_moving():
    """bench.settle keeps running untimed steps until the time per step has
    stopped moving (two consecutive runs within 1%) and at least min_s has
    passed: a simulated board whose step time rises from 1.0 to 1.3 ms over
    the first 0.6 s (the clock falling under load) is timed at its final
    rate, and a steady one returns soon after min_s."""
    import time as _time
    import types

    sys.path.insert(0, ROOT)
    import bench

    fake_torch = types.SimpleNamespace(cuda=types.SimpleNamespace(synchronize=lambda: None))

    def board(rise_s, lo_ms, hi_ms):
        t_start = _time.perf_counter()

        def run(n):
            t = _time.perf_counter() - t_start
            ms = hi_ms if t >= rise_s else lo_ms + (hi_ms - lo_ms) * t / rise_s
            _time.sleep(n * ms / 1e3)
        return run

    spent, steps, ms = bench.settle(fake_torch, board(0.6, 1.0, 1.3), 0.3, 5.0)
    assert spent >= 0.6 and spent < 5.0
    assert abs(ms - 1.3) <= 0.03 * 1.3, ms
    spent, steps, ms = bench.settle(fake_torch, board(1e-9, 1.0, 1.0), 0.3, 5.0)
    assert 0.3 <= spent < 1.5 and abs(ms - 1.0) <= 0.03
