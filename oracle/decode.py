"""Decision logic around the fused step, written from the pages (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding ..." as
reviewed on jaehun.me, sections "Flash-Verify: Cache-Based Draft-Verification
Parallel Decoding" and "How It Works: A Concrete Example" (which cite the
paper's section 2.3, Alg. 2, Fig. 2 and Appx. C).

Notation follows the pages: T_t tracked set, M_t masked positions,
M_t^{beta_m} the first beta_m masks, Q_t = T_t u M_t^{beta_m}, c_i the draft
confidence, D_t = {c_i >= eps} (confident), S_t = {c_i < eps} (exploratory),
x_hat the draft prediction, x_tilde / c_tilde the [MASK]-view prediction and
confidence in the verification pass, gamma the acceptance threshold.

Readings where the pages are silent:
  - Q order is [T_t ascending | M_t^{beta_m} ascending]; verification rows are
    [T_v | D_t | S_t draft view | S_t mask view].
  - c_i >= eps and c_tilde >= gamma are inclusive (the pages write ">=").
  - the argmax excludes the [MASK] token and breaks ties to the lowest id.
  - "decoding order" for the sequential acceptance is ascending position.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np


def front_masks(masked: Sequence[int], beta_m: int) -> List[int]:
    """M_t^{beta_m}: the first beta_m still-masked positions (ascending)."""
    return sorted(masked)[:beta_m]


def query_set(tracked: Sequence[int], masked: Sequence[int], beta_m: int) -> List[int]:
    """Q_t = T_t u M_t^{beta_m}, ordered [T_t | M_t^{beta_m}], both ascending."""
    fm = front_masks(masked, beta_m)
    t = sorted(p for p in set(tracked) if p not in fm)
    return t + fm


def confidence(probs: Sequence[float], mask_id: int | None) -> Tuple[int, float]:
    """(prediction, confidence): argmax and max over the non-[MASK] tokens."""
    best, best_p = -1, float("-inf")
    for tok, p in enumerate(probs):
        if tok == mask_id:
            continue
        if p > best_p:  # strict: ties keep the lowest token id
            best, best_p = tok, p
    return best, best_p


def draft_split(positions: Sequence[int], probs: Dict[int, Sequence[float]], eps: float,
                mask_id: int | None):
    """Split the masked query positions by draft confidence into D_t and S_t.

    Returns (D, S, pred, conf) where D and S are ascending position lists and
    pred / conf map each position to x_hat_i / c_i.
    """
    pred, conf = {}, {}
    D, S = [], []
    for p in sorted(positions):
        x, c = confidence(probs[p], mask_id)
        pred[p], conf[p] = x, c
        (D if c >= eps else S).append(p)
    return D, S, pred, conf


def verify_rows(T_v: Sequence[int], D: Sequence[int], S: Sequence[int]):
    """Row layout of the verification query: [(group, position), ...].

    Groups are 'track', 'confident', 'draft' and 'mask'; the draft and mask
    views of S share positions.  Its length is |T_v| + |D| + 2|S|, so the
    extra cost grows with 2 beta_m, not with the sequence length.
    """
    return ([("track", p) for p in T_v] + [("confident", p) for p in D] +
            [("draft", p) for p in S] + [("mask", p) for p in S])


def view_visibility(rows) -> List[List[int]]:
    """Visibility over the rows of ``verify_rows``: 1 = row i may see row j.

    The draft view and the [MASK] view of S cannot see each other; every other
    pair is visible (bidirectional attention).
    """
    n = len(rows)
    vis = [[1] * n for _ in range(n)]
    for i, (gi, _) in enumerate(rows):
        for j, (gj, _) in enumerate(rows):
            if {gi, gj} == {"draft", "mask"}:
                vis[i][j] = 0
    return vis


def chain_visibility(rows) -> List[List[int]]:
    """Chain-rule visibility over the rows of ``verify_rows`` (jaehun.me review,
    "Flash-Verify": the verification mask is causal so that the mask view
    scores the block's true joint, Appx. C).  Reading: the mask-view row of
    the k-th exploratory position in decoding (ascending position) order sees
    the draft view of the positions before it and the mask view of itself and
    the positions after it; draft-view and context rows see the context and
    the draft view only.  1 = row i may see row j."""
    n = len(rows)
    s_pos = sorted({p for g, p in rows if g == "draft"})
    rank = {p: k for k, p in enumerate(s_pos)}
    vis = [[0] * n for _ in range(n)]
    for i, (gi, pi) in enumerate(rows):
        for j, (gj, pj) in enumerate(rows):
            if gi != "mask":
                vis[i][j] = 0 if gj == "mask" else 1
            elif gj == "draft":
                vis[i][j] = 1 if rank[pj] < rank[pi] else 0
            elif gj == "mask":
                vis[i][j] = 1 if rank[pj] >= rank[pi] else 0
            else:
                vis[i][j] = 1
    return vis


def accept(S_order: Sequence[int], x_hat: Dict[int, int], x_tilde: Dict[int, int],
           c_tilde: Dict[int, float], gamma: float) -> List[int]:
    """Sequential acceptance: walk S_t in decoding order and accept position i
    while the mask-view prediction agrees with the draft (x_tilde_i == x_hat_i)
    and its confidence c_tilde_i >= gamma; stop at the first failure."""
    out = []
    for i in S_order:
        if x_tilde[i] == x_hat[i] and c_tilde[i] >= gamma:
            out.append(i)
        else:
            break
    return out


def block_tv(c_tilde_accepted: Sequence[float]) -> float:
    """TV distance between the committed point mass and the mask-view joint over
    an accepted block A: 1 - prod_k c_tilde_{i_k} (Appx. C)."""
    prod = 1.0
    for c in c_tilde_accepted:
        prod *= c
    return 1.0 - prod


def tv_bounds(m: int, gamma: float) -> Tuple[float, float]:
    """The two upper bounds of the block TV distance: (1 - gamma^m, m (1 - gamma))."""
    return 1.0 - gamma ** m, m * (1.0 - gamma)


def softmax_fp64(logits) -> np.ndarray:
    """Softmax over the last axis in fp64 (the distribution behind a row of logits)."""
    x = np.asarray(logits, dtype=np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def confidences(logits, mask_id: int | None):
    """(pred, conf) for every row of logits [..., V]: the softmax over all ids
    in fp64, then, over the non-[MASK] ids, the first largest probability (the
    lowest id among equal ones) and its value -- ``confidence`` applied to each
    row, with numpy doing the per-row work."""
    p = softmax_fp64(logits)
    if mask_id is not None and 0 <= mask_id < p.shape[-1]:
        p = p.copy()
        p[..., mask_id] = -np.inf
    pred = np.argmax(p, axis=-1)          # first occurrence: lowest id on ties
    conf = np.take_along_axis(p, pred[..., None], axis=-1)[..., 0]
    return pred.astype(np.int64), conf
