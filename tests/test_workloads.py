"""The seeded workload description: lengths, layouts and bf16 rounding."""
import numpy as np
import torch

import workloads as W


def test_lengths_fill_sequence_and_respect_bounds():
    for fn, lo, hi in ((W.ring_rank, 128, 8192), (W.zigzag_rank, 256, 32768), (W.training, 1, 16384)):
        w = fn()
        assert sum(w.lengths) == w.total
        assert all(lo <= L <= hi for L in w.lengths[:-1])
        assert 1 <= w.lengths[-1] <= hi
        assert fn().lengths == w.lengths          # deterministic
    u = W.ulysses()
    assert u.lengths[:2] == [262144, 131072] and sum(u.lengths) == 524288
    assert all(64 <= L <= 2048 for L in u.lengths[2:-1])
    g = W.by_name("ulysses_gqa")
    assert (g.hq, g.hkv) == (4, 1) and g.lengths == u.lengths and g.name != u.name


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000, dtype=np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.0e38]   # ties and a large value
    ours = W.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_layouts():
    z = W.zigzag_rank(3)
    assert z.tq == 16384
    assert z.q_segs == [(24576, 32768, 0), (98304, 106496, 8192)]
    assert [s.chunks for s in z.steps][:3] == [[3, 12], [2, 13], [1, 14]]
    r = W.ring_rank(3)
    assert [s.chunks[0] for s in r.steps] == [3, 2, 1, 0, 7, 6, 5, 4]
    g = r.q_global_rows()
    assert g[0] == 12288 and g[-1] == 16383
