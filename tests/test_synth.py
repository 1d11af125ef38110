"""The seeded input generator (no GPU)."""
import numpy as np
import torch

from ulysses_head_sharded_amd import synth


def test_splitmix64_known_answers():
    # first three outputs of SplitMix64 started from state 0 (published test values)
    got = [int(x) for x in synth.splitmix64(0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_offsets():
    a = synth.splitmix64(77, 100)
    assert np.array_equal(a[40:60], synth.splitmix64(77, 20, start=40))
    big = synth.normal_f32(5, (1 << 22) + 3)          # spans several threaded chunks
    assert np.array_equal(big[:1001], synth.normal_f32(5, 1001))


def test_normal_moments():
    x = synth.normal_f32(123, 1 << 20).astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    assert abs(np.mean(x ** 3)) < 2e-2 and abs(np.mean(x ** 4) - 3.0) < 3e-2


def test_bf16_rounding_matches_torch():
    f = np.concatenate([synth.normal_f32(9, 4096) * 1e3,
                        np.array([1.0, -0.0, 3.0e38, 1e-40, 1.00390625, 1.01171875],
                                 dtype=np.float32)]).astype(np.float32)
    ours = synth.f32_to_bf16_bits(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(f).to(torch.bfloat16).float().numpy())


def test_row_sample_covers_edges():
    rows = synth.row_sample(507, 4096, 2, 3, n_random=16, edge=4)
    t = set(rows[rows[:, 0] == 1][:, 2].tolist())
    assert {0, 1, 2, 3, 4092, 4093, 4094, 4095} <= t
    assert rows[:, 1].max() == 2 and rows[:, 0].max() == 1
    assert rows[:, 2].max() < 4096
