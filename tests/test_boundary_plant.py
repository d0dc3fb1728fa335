"""CPU check of the boundary-planting helper used by the GPU selection test:
the planted candidates must sit on the intended ladder around the selection
boundary, with no other candidate closer to the boundary than the ladder's
spacing."""
import numpy as np

import synth
from oracle import locks_oracle as O
from tests import locks_harness as Hh


def test_plant_boundary_ladder():
    b = synth.make_decode_batch([1500 * 16 - 5], 2, 4, [40], seed=200, needles_per_head=1)
    summ = Hh.oracle_summaries(b.k_pool, b.block_table, b.seq_lens, b.H, 8, b.num_blocks)
    L = int(b.seq_lens[0])
    P = (L + 15) // 16
    for h, gap in ((0, 2e-5), (1, 3e-4)):
        key, top = Hh.plant_boundary(summ, b.block_table, b.q, L, 40, h, b.G, 8, gap)
        ora = Hh.oracle_head(b.q, b.k_pool, b.v_pool, b.block_table, b.seq_lens, b.budgets, summ,
                             0, h, b.G, 8)
        np.testing.assert_allclose(ora["key"], key, atol=1e-12)
        cand = sorted(range(1, P - 1), key=lambda j: (-float(key[j]), j))
        k2 = 38
        # the boundary pair and its neighbours are the planted pages, `gap` apart
        ladder = cand[k2 - 3:k2 + 3]
        assert set(ladder) == set(top), (ladder, top)
        gaps = -np.diff([key[j] for j in ladder])
        np.testing.assert_allclose(gaps, gap, rtol=0.15)
        # nothing else within the ladder's span (+ one gap) of the boundary
        lo, hi = key[ladder[-1]] - gap, key[ladder[0]] + gap
        others = [j for j in cand if lo < key[j] < hi and j not in top]
        assert not others
        # the oracle's selection cuts the ladder in the middle
        assert set(ladder[:3]) <= set(ora["sel"]) and not (set(ladder[3:]) & set(ora["sel"]))
