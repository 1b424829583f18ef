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


def test_rejection_rows_take_the_planted_second_proposal(oracle_lib):
    """The rejection rows of tests/race_edge_rows.py: the oracle's rejection
    sampler accepts W2 in round 2 and its sampler draws W2 too, away from
    every band; without W2 the decoy D would be the best listed token above
    the pivot; and the kernel's list screen against 1/64 of the best keeps W2
    only with its margin on the safe side."""
    o = oracle_lib.default()
    B, V = 4, 65536
    L, P, S, W1, W2, D = race_edge_rows.build_rejection(o, B, V, base_seed=4242)
    T = np.ones(B, np.float32)
    K = np.zeros(B, np.int32)
    MP = np.zeros(B, np.float32)
    rj = oracle_lib.sample_rejection(L, T, P, MP, seed=0, seeds=S)
    assert np.array_equal(rj["token"], W2)
    assert np.all(rj["rounds"] == 2)
    assert np.all(rj["band"] > 1e-5) and np.all(rj["race_margin"] > 1e-6)
    rows, _ = oracle_lib.sample(L, T, P, K, MP, seed=0, seeds=S)
    assert np.array_equal(rows["token"], W2)
    for b in range(B):
        words = o.noise_words(int(S[b]), 0, b, V)
        E = -np.log((words.astype(np.float64) + 0.5) * 2.0 ** -32)
        e = np.exp(L[b].astype(np.float64))
        score = e / E
        s1 = score[W1[b]]
        assert s1 == score.max()                       # round 1's winner
        above = e > e[W1[b]]
        rest = above.copy()
        rest[W2[b]] = False
        assert int(np.argmax(np.where(rest, score, -1.0))) == D[b]
        assert score[D[b]] >= s1 / 64.0                # listed
        assert score[W2[b]] > score[D[b]] * (1.0 + 5e-6)
        thr = s1 / 64.0
        assert race_edge_rows.screen_rejects(L[b, W2[b]], 0.0, 1.0, thr, int(words[W2[b]]), -2e-3)
        assert not race_edge_rows.screen_rejects(L[b, W2[b]], 0.0, 1.0, thr, int(words[W2[b]]), 2e-3)
