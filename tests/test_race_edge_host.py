"""The race-edge rows sit where they are meant to (CPU only).

The rows of tests/race_edge_rows.py plant a winner that beats every other
token by 2e-5 to 7e-5 relative, with noise for which the race screen's bound
on 1 - u is tight.  Here the oracle confirms the planted winner wins outside
the 1e-6 tie band, and the screen's float32 test, emulated on the host, shows
that a margin on the unsafe side (R lowered by 2e-3) would screen that winner
out against its lane's running best while the safe side (R raised by 2e-3)
lets it through ("What do temperature, top-k and top-p each do ...", "A
strong answer", last paragraph: the race must draw exactly from p).
"""
import numpy as np

import race_edge_rows


def test_planted_winners_win_and_sit_at_the_screen_edge(oracle_lib):
    o = oracle_lib.default()
    B, V = 8, 32768
    L, T, S, W = race_edge_rows.build(o, B, V, base_seed=777)
    P = np.ones(B, np.float32)
    rows, _ = oracle_lib.sample(L, T, P, np.zeros(B, np.int32), np.zeros(B, np.float32), seed=0, seeds=S)
    assert np.array_equal(rows["token"], W)
    assert np.all(rows["race_margin"] > 1e-5)
    for b in range(B):
        word = o.noise_word(int(S[b]), 0, b, int(W[b]))
        runner_up = rows["race_s2"][b]
        for sstar in (runner_up, runner_up * (1 - 4e-5)):
            assert race_edge_rows.screen_rejects(L[b, W[b]], 0.0, T[b], sstar, word, -2e-3), (b, sstar)
            assert not race_edge_rows.screen_rejects(L[b, W[b]], 0.0, T[b], sstar, word, 2e-3), (b, sstar)
