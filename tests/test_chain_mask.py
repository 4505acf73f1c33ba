"""The chain-rule verification mask (jaehun.me review, "Flash-Verify": the
verification mask is causal so that the mask view scores the block's true
joint, Appx. C; "How It Works", Step 1 Verification: the two views of a
position cannot see each other).  Checks of the oracle-side definition
against the structure the pages fix, and of the workload generator against
the oracle-side definition."""
import random

import torch

from io_aware_kv_amd.workloads import make_workload
from oracle.decode import chain_visibility, verify_rows, view_visibility


def _random_sets(rng, n_t=5, n_d=3, n_s=6, n=200):
    pos = rng.sample(range(n), n_t + n_d + n_s)
    return sorted(pos[:n_t]), sorted(pos[n_t:n_t + n_d]), sorted(pos[n_t + n_d:])


def test_every_row_sees_each_exploratory_position_in_exactly_one_view():
    rng = random.Random(7)
    for _ in range(20):
        T_v, D, S = _random_sets(rng)
        rows = verify_rows(T_v, D, S)
        vis = chain_visibility(rows)
        for i in range(len(rows)):
            for p in S:
                views = [j for j, (g, q) in enumerate(rows) if q == p and g in ("draft", "mask")]
                assert sum(vis[i][j] for j in views) == 1


def test_mask_row_commits_exactly_the_earlier_positions():
    rng = random.Random(11)
    for _ in range(20):
        T_v, D, S = _random_sets(rng)
        rows = verify_rows(T_v, D, S)
        vis = chain_visibility(rows)
        for i, (g, p) in enumerate(rows):
            committed = sorted(q for j, (h, q) in enumerate(rows) if h == "draft" and vis[i][j])
            if g == "mask":
                assert committed == [q for q in S if q < p]      # the chain rule's conditioning set
                assert vis[i][i] == 1
            else:
                assert committed == S                            # context and draft rows: the whole draft


def test_views_of_one_position_never_see_each_other_and_context_is_shared():
    rng = random.Random(3)
    T_v, D, S = _random_sets(rng)
    rows = verify_rows(T_v, D, S)
    vis = chain_visibility(rows)
    for i, (gi, pi) in enumerate(rows):
        for j, (gj, pj) in enumerate(rows):
            if pi == pj and {gi, gj} == {"draft", "mask"}:
                assert vis[i][j] == 0
            if gj in ("track", "confident"):
                assert vis[i][j] == 1


def test_single_exploratory_position_matches_the_worked_example_pattern():
    # worked example: [track, D=2, S draft=3, S mask=3]; the two views of
    # position 3 are mutually invisible, as in the block mask
    rows = verify_rows([], [2], [3])
    chain, block = chain_visibility(rows), view_visibility(rows)
    for i, (gi, _) in enumerate(rows):
        for j, (gj, _) in enumerate(rows):
            if gi in ("draft", "mask") and gj in ("draft", "mask"):
                assert chain[i][j] == block[i][j]


def test_generator_chain_mask_matches_oracle_definition():
    wl = make_workload(7)
    for b in range(wl.shape.B):
        groups = wl.meta["groups"][b]
        pos = wl.pos_ids[b].tolist()
        T_v = [p for g, p in zip(groups, pos) if g == "track"]
        D = [p for g, p in zip(groups, pos) if g == "confident"]
        S = [p for g, p in zip(groups, pos) if g == "draft"]
        rows = verify_rows(T_v, D, S)
        assert [g for g, _ in rows] == groups and [p for _, p in rows] == pos
        ref = torch.tensor(chain_visibility(rows), dtype=torch.uint8)
        assert torch.equal(wl.vis[b], ref)
