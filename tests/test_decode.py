"""Decision logic of the draft/verify passes against the pages' worked example.

Fixture: tests/golden/worked_example.json, the mini example of the jaehun.me
review ("How It Works: A Concrete Example", Step 1: Draft and Step 1:
Verification) with vocabulary {A, B, [MASK]}, N=4, beta_m=2, beta_t=1,
eps=0.9, gamma=0.8.  The TV statements come from the same page's
"Flash-Verify" section (Appx. C of the paper).
"""
import json
import os
import random

import pytest

from oracle import decode

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def ex():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        return json.load(f)


def _probs(d):
    return {int(k): v for k, v in d.items()}


def test_query_set_is_tracked_plus_front_masks(ex):
    assert decode.front_masks(ex["masked"], ex["beta_m"]) == ex["expected_front_masks"]
    assert decode.query_set(ex["tracked"], ex["masked"], ex["beta_m"]) == ex["expected_Q"]


def test_draft_split_by_confidence(ex):
    D, S, pred, conf = decode.draft_split(ex["expected_Q"], _probs(ex["draft_probs"]), ex["eps"],
                                          ex["mask_id"])
    assert D == ex["expected_D"] and S == ex["expected_S"]
    for p, c in ex["expected_confidence"].items():
        assert conf[int(p)] == pytest.approx(c)
    for p, tok in ex["expected_draft_pred"].items():
        assert ex["vocab"][pred[int(p)]] == tok


def test_verification_accepts_agreeing_confident_token(ex):
    D, S, x_hat, _ = decode.draft_split(ex["expected_Q"], _probs(ex["draft_probs"]), ex["eps"],
                                        ex["mask_id"])
    x_t, c_t = {}, {}
    for p, probs in _probs(ex["verify_mask_view_probs"]).items():
        x_t[p], c_t[p] = decode.confidence(probs, ex["mask_id"])
        assert ex["vocab"][x_t[p]] == ex["expected_mask_view_pred"][str(p)]
        assert c_t[p] == pytest.approx(ex["expected_mask_view_conf"][str(p)])
    acc = decode.accept(S, x_hat, x_t, c_t, ex["gamma"])
    assert acc == ex["expected_accepted"]
    tv = decode.block_tv([c_t[p] for p in acc])
    assert tv == pytest.approx(ex["expected_block_tv"])
    b1, b2 = decode.tv_bounds(len(acc), ex["gamma"])
    assert [b1, b2] == pytest.approx(ex["expected_tv_bounds"])
    assert tv <= b1 + 1e-12 <= b2 + 2e-12


def test_flipped_variants_of_the_example_reject(ex):
    S = ex["expected_S"]
    x_hat = {3: 0}
    # confidence just under gamma
    assert decode.accept(S, x_hat, {3: 0}, {3: 0.79}, ex["gamma"]) == []
    # mask view disagrees with the draft
    assert decode.accept(S, x_hat, {3: 1}, {3: 0.95}, ex["gamma"]) == []
    # threshold is inclusive
    assert decode.accept(S, x_hat, {3: 0}, {3: 0.8}, ex["gamma"]) == [3]
    # two exploratory tokens: a rejected first one stops the walk
    assert decode.accept([3, 4], {3: 0, 4: 1}, {3: 1, 4: 1}, {3: 0.9, 4: 0.99}, 0.8) == []
    assert decode.accept([3, 4], {3: 0, 4: 1}, {3: 0, 4: 0}, {3: 0.9, 4: 0.99}, 0.8) == [3]


def test_verification_layout_and_view_mask(ex):
    rows = decode.verify_rows([7], ex["expected_D"], ex["expected_S"])
    assert rows == [("track", 7), ("confident", 2), ("draft", 3), ("mask", 3)]
    assert len(rows) == 1 + len(ex["expected_D"]) + 2 * len(ex["expected_S"])
    vis = decode.view_visibility(rows)
    assert vis[2][3] == 0 and vis[3][2] == 0            # views cannot see each other
    assert vis[2][2] == 1 and vis[3][3] == 1            # each view sees itself
    assert all(vis[0][j] == 1 for j in range(4))       # context rows see both views
    # the row count grows with 2|S|, not with the sequence length
    for s in range(0, 6):
        S = list(range(10, 10 + s))
        assert len(decode.verify_rows([1, 2], [5], S)) == 3 + 2 * s


def test_confidence_excludes_mask_and_breaks_ties_low():
    assert decode.confidence([0.2, 0.2, 0.6], mask_id=2) == (0, 0.2)
    assert decode.confidence([0.1, 0.5, 0.4], mask_id=None) == (1, 0.5)


def test_tv_bound_chain_holds_for_random_accepted_blocks():
    rnd = random.Random(5)
    for _ in range(2000):
        gamma = rnd.uniform(0.5, 0.99)
        m = rnd.randint(1, 12)
        cs = [rnd.uniform(gamma, 1.0) for _ in range(m)]
        tv = decode.block_tv(cs)
        b1, b2 = decode.tv_bounds(m, gamma)
        assert 0.0 <= tv <= b1 + 1e-12 and b1 <= b2 + 1e-12


# --------------------------------------------------------------------------
# confidences from logits (the form the device decision kernel takes)
# --------------------------------------------------------------------------

def test_confidences_from_log_probs_reproduce_the_example(ex):
    """Logits = log of the example's probabilities: the softmax gives them
    back, so prediction, confidence and the eps split are the page's."""
    import numpy as np
    rows = [ex["draft_probs"]["2"], ex["draft_probs"]["3"], ex["verify_mask_view_probs"]["3"]]
    pred, conf = decode.confidences(np.log(np.array(rows)), ex["mask_id"])
    assert [ex["vocab"][i] for i in pred] == ["A", "A", "A"]
    assert conf == pytest.approx([0.92, 0.70, 0.85])
    assert [c >= ex["eps"] for c in conf[:2]] == [True, False]
    assert conf[2] >= ex["gamma"]


def test_confidences_equal_the_row_loop_and_are_shift_invariant():
    import numpy as np
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, 37)) * 3
    x[3, [4, 9]] = x[3].max() + 1.0          # a tie at the top: the lower id wins
    x[5, 0] = x[5].max() + 5.0               # the [MASK] id on top: excluded
    pred, conf = decode.confidences(x, 0)
    p = decode.softmax_fp64(x)
    for r in range(40):
        t, c = decode.confidence(list(p[r]), 0)
        assert pred[r] == t and conf[r] == pytest.approx(c, rel=1e-15)
    assert pred[3] == 4 and pred[5] != 0
    pred2, conf2 = decode.confidences(x + 123.0, 0)
    assert (pred2 == pred).all() and np.allclose(conf2, conf, rtol=1e-12)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)
