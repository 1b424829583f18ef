"""Race winners that beat the running best by a hair, on every path.

Rows from tests/race_edge_rows.py: every token but one scores within 5e-5
below the max token's score, and the planted winner scores 2e-5 above it with
noise for which the race screen's bound is tight.  Every path of the sampler
must return the oracle's token (the planted winner) on every row ("What do
temperature, top-k and top-p each do ...", "A strong answer", last
paragraph: the race draws exactly from p).
"""
import numpy as np
import pytest

import race_edge_rows
from gpu_util import say

pytestmark = pytest.mark.gpu

PATHS = [None, "single", "split", "rows"]


@pytest.mark.parametrize("path", PATHS)
def test_race_edge_rows(path, oracle_lib):
    import torch

    import nucleus_sampling_amd as ns

    o = oracle_lib.default()
    B, V = 16, 32768
    L, T, S, W = race_edge_rows.build(o, B, V, base_seed=901)
    P = np.ones(B, np.float32)
    K = np.zeros(B, np.int32)
    MP = np.zeros(B, np.float32)
    rows, _ = oracle_lib.sample(L, T, P, K, MP, seed=0, seeds=S)
    assert np.array_equal(rows["token"], W)
    say(f"race edge rows B={B} V={V} path={path}")
    lg = torch.from_numpy(L).to("cuda:0")
    res = ns.sample(lg, T, P, K, MP, seed=0, step=0, seeds=S, single_workgroup=path == "single",
                    split_rows=path == "split", row_race=path == "rows")
    torch.cuda.synchronize()
    tok = res.token.cpu().numpy()
    cnt = res.keep_count.cpu().numpy()
    say(f"path={path}: tokens {tok.tolist()}")
    assert np.array_equal(tok, W), (tok, W)
    assert np.array_equal(cnt, rows["keep_count"])


def test_rejection_second_proposal_from_the_list(oracle_lib):
    """nucleus_sample_rejection on rows where round 1's winner lies outside
    the nucleus and round 2's proposal W2 scores 2e-5 above 1/64 of the best,
    with noise for which the list screen's bound is tight; a decoy 1e-5
    above 1/64 would be proposed (and accepted) if the list lost W2.  The
    kernel must accept W2 in round 2, as the oracle does; nucleus_sample on
    every path draws W2 too ("Top-p (Nucleus) Sampling, in depth",
    "Sort-free top-p by rejection sampling")."""
    import torch

    import nucleus_sampling_amd as ns

    o = oracle_lib.default()
    B, V = 8, 65536
    L, P, S, W1, W2, D = race_edge_rows.build_rejection(o, B, V, base_seed=9191)
    T = np.ones(B, np.float32)
    MP = np.zeros(B, np.float32)
    rj = oracle_lib.sample_rejection(L, T, P, MP, seed=0, seeds=S)
    assert np.array_equal(rj["token"], W2) and np.all(rj["rounds"] == 2)
    say(f"rejection race edge rows B={B} V={V}")
    lg = torch.from_numpy(L).to("cuda:0")
    r = ns.sample_rejection(lg, T, P, MP, seed=0, step=0, seeds=S)
    torch.cuda.synchronize()
    tok, rounds = r.token.cpu().numpy(), r.rounds.cpu().numpy()
    say(f"rejection: tokens {tok.tolist()} rounds {rounds.tolist()}")
    assert np.array_equal(tok, W2), (tok, W2, D)
    assert np.all(rounds == 2)
    for path in PATHS:
        res = ns.sample(lg, T, P, np.zeros(B, np.int32), MP, seed=0, step=0, seeds=S,
                        single_workgroup=path == "single", split_rows=path == "split", row_race=path == "rows")
        torch.cuda.synchronize()
        assert np.array_equal(res.token.cpu().numpy(), W2), path
