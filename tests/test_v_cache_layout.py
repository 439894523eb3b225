"""The test-side converters of the blocked decode V cache against its
definition in include/gdr.h (CPU only): position 32 b + i of dim d of
(sequence n, kv head h) is element [n][h][b][d][8 ((i mod 16) / 4) +
4 (i / 16) + i mod 4]."""
import numpy as np
import torch

from helpers import VC_KEY, VC_POS, v_cache_blocked, v_cache_natural


def test_positions_are_a_permutation():
    assert sorted(VC_POS) == list(range(32))
    assert all(VC_POS[VC_KEY[p]] == p for p in range(32))
    # lane group g of the decode's value product reads positions 8 g .. 8 g + 7:
    # keys 4 g .. 4 g + 3, then 16 + 4 g .. 16 + 4 g + 3
    for g in range(4):
        assert VC_KEY[8 * g:8 * g + 8] == [4 * g, 4 * g + 1, 4 * g + 2, 4 * g + 3,
                                           16 + 4 * g, 17 + 4 * g, 18 + 4 * g, 19 + 4 * g]


def test_blocked_matches_definition_elementwise():
    rng = np.random.default_rng(3)
    N, L, Hk, D = 2, 64, 3, 5
    nat = rng.standard_normal((N, L, Hk, D))
    blk = v_cache_blocked(nat)
    assert blk.shape == (N, Hk, L // 32, D, 32)
    for n in range(N):
        for h in range(Hk):
            for pos in range(L):
                b, i = divmod(pos, 32)
                slot = 8 * ((i % 16) // 4) + 4 * (i // 16) + i % 4
                for d in range(D):
                    assert blk[n, h, b, d, slot] == nat[n, pos, h, d]
    assert np.array_equal(v_cache_natural(blk), nat)


def test_torch_and_numpy_agree():
    x = torch.arange(2 * 96 * 2 * 4, dtype=torch.float32).reshape(2, 96, 2, 4)
    assert np.array_equal(v_cache_blocked(x).numpy(), v_cache_blocked(x.numpy()))
    assert torch.equal(v_cache_natural(v_cache_blocked(x)), x)
