"""GPU parity of the Flash-Verify decision kernels (per-row prediction and
confidence, the eps / gamma threshold flags, sequential acceptance) through
the C ABI against the oracle (oracle.decode), on the review's worked example
("How It Works: A Concrete Example", Step 1: Draft / Verification) and on
seeded logits over a synthetic vocabulary.

Bar: predictions and acceptance counts are integers decided from the same
input values on both sides and must match exactly; the confidence is an fp32
softmax probability (relative error <= 1e-5 against fp64); a threshold flag
must equal (gpu conf >= thr) and the oracle's decision wherever the oracle's
confidence is more than 1e-5 (relative) away from the threshold.
"""
import json
import os

import numpy as np
import pytest
import torch

from io_aware_kv_amd import binding
from io_aware_kv_amd.workloads import decision_logits
from oracle import decode
from parity_util import log

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def gpu_confidence(logits, mask_id, thr):
    dev = torch.device("cuda")
    x = logits.to(dev).contiguous()
    rows = x.numel() // x.shape[-1]
    pred = torch.full((rows,), -7, dtype=torch.int32, device=dev)
    conf = torch.full((rows,), float("nan"), dtype=torch.float32, device=dev)
    over = torch.full((rows,), 7, dtype=torch.uint8, device=dev)
    binding.confidence(x, mask_id, thr, pred, conf, over)
    torch.cuda.synchronize()
    return pred.cpu().numpy(), conf.cpu().numpy(), over.cpu().numpy()


def test_worked_example_on_the_device():
    log("case: worked example on the device")
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        ex = json.load(f)
    rows = [ex["draft_probs"]["2"], ex["draft_probs"]["3"]]
    logits = torch.tensor(np.log(np.array(rows)), dtype=torch.float32)
    pred, conf, over = gpu_confidence(logits, ex["mask_id"], ex["eps"])
    assert [ex["vocab"][i] for i in pred] == ["A", "A"]
    assert conf == pytest.approx([0.92, 0.70], rel=1e-6)
    D = [p for p, o in zip(ex["expected_Q"], over) if o]
    S = [p for p, o in zip(ex["expected_Q"], over) if not o]
    assert D == ex["expected_D"] and S == ex["expected_S"]
    mv = torch.tensor(np.log(np.array([ex["verify_mask_view_probs"]["3"]])), dtype=torch.float32)
    xt, ct, ot = gpu_confidence(mv, ex["mask_id"], ex["gamma"])
    assert ct == pytest.approx([0.85], rel=1e-6) and ot.tolist() == [1]
    dev = torch.device("cuda")
    n = torch.full((1,), -7, dtype=torch.int32, device=dev)
    binding.accept(torch.tensor([[pred[1]]], dtype=torch.int32, device=dev),
                   torch.tensor([[xt[0]]], dtype=torch.int32, device=dev),
                   torch.tensor([[ct[0]]], dtype=torch.float32, device=dev), ex["gamma"], n)
    torch.cuda.synchronize()
    assert S[:int(n.item())] == ex["expected_accepted"]


@pytest.mark.parametrize("rows,V,dtype,mask_id", [
    (512, 131072, torch.bfloat16, 126),     # the synthetic vocabulary, vector loads
    (64, 1001, torch.float32, 1000),        # ragged vocabulary, scalar loads
    (33, 4096, torch.float32, -1),          # no [MASK] id excluded
])
def test_confidence_matches_oracle(rows, V, dtype, mask_id):
    log("case: confidence rows=%d V=%d %s" % (rows, V, dtype))
    x = decision_logits(rows, V, seed=rows + V, dtype=dtype)
    if dtype == torch.float32:
        # exact ties at the top of some rows: the lower id wins on both sides
        x[0, 10] = x[0].max() + 1.0
        x[0, 20] = x[0, 10]
    thr = 0.5
    pred, conf, over = gpu_confidence(x, mask_id, thr)
    rp, rc = decode.confidences(x.double().numpy(), mask_id if mask_id >= 0 else None)
    assert np.array_equal(pred, rp), "predictions differ"
    rel = np.abs(conf - rc) / np.maximum(rc, 1e-30)
    log("conf max rel err %.2e, %d of %d rows over %.2f" % (rel.max(), int(over.sum()), rows, thr))
    assert rel.max() <= 1e-5
    assert np.array_equal(over.astype(bool), conf >= thr)
    decided = np.abs(rc - thr) > 1e-5 * thr
    assert np.array_equal(over.astype(bool)[decided], (rc >= thr)[decided])
    if dtype == torch.float32:
        assert pred[0] == 10


@pytest.mark.parametrize("dtype,V", [(torch.float32, 32768), (torch.bfloat16, 65536)])
def test_confidence_argmax_corner_rows(dtype, V):
    """Rows built to hit each step of the argmax: equal maxima in one lane's
    consecutive rounds and in one round's different loads (a lane reads 16 B
    at ids v, v + 1024 * e, ... with e elements per 16 B, four loads per
    round), the [MASK] id holding the row's maximum, all but two logits -inf,
    the maximum at the last id, and a row of equal logits."""
    log("case: confidence argmax corner rows %s V=%d" % (dtype, V))
    e = 16 // (4 if dtype == torch.float32 else 2)       # elements per 16-byte load
    load, rnd = 1024 * e, 4 * 1024 * e                    # id stride of a load and of a round
    mask_id = 126
    x = decision_logits(6, V, seed=V + 5, dtype=torch.float32)
    top = float(x.max()) + 1.0
    x[0, 5] = top
    x[0, 5 + rnd] = top                                   # same lane, next round: id 5 wins
    x[1, 9] = top
    x[1, 9 + 2 * load] = top                              # same lane and round, third load: id 9 wins
    x[2, mask_id] = top + 4.0                             # the [MASK] id is the row's maximum
    x[2, 3000] = top
    x[3, :] = float("-inf")
    x[3, 7] = 0.0
    x[3, V - 3] = -1.0
    x[4, V - 1] = top                                     # maximum at the last id
    x[5, :] = 0.25
    x = x.to(dtype)
    pred, conf, over = gpu_confidence(x, mask_id, 0.5)
    rp, rc = decode.confidences(x.double().numpy(), mask_id)
    assert pred.tolist() == [5, 9, 3000, 7, V - 1, 0]
    assert np.array_equal(pred, rp)
    rel = np.abs(conf - rc) / np.maximum(rc, 1e-30)
    assert rel.max() <= 1e-5


def row_ranges(rows, V, esz):
    """The launch rule for rows of esz-byte logits: with fewer than 256 rows
    a row is cut into up to eight ranges of whole rounds (512 threads x four
    16-byte loads), while rows x ranges stays within two workgroups per CU."""
    rid = 512 * 4 * (16 // esz)
    rounds = -(-V // rid)
    ns = 1
    if rows < 256:
        while ns < 8 and rows * ns * 2 <= 512 and ns * 2 <= rounds:
            ns *= 2
    return ns, (-(-rounds // ns)) * rid


SPLIT_CASES = [
    # (label, rows, V, dtype)
    ("bf16-8-ranges", 5, 131072, torch.bfloat16),
    ("bf16-128-rows-4-ranges", 128, 131072, torch.bfloat16),
    ("bf16-200-rows-2-ranges", 200, 131072, torch.bfloat16),
    ("f32-8-ranges", 3, 131072, torch.float32),
    ("f32-ragged", 2, 131072 - 4, torch.float32),      # last range short
    ("bf16-ragged-scalar", 4, 70001, torch.bfloat16),  # V not a multiple of 8: element loads; last range empty
]


@pytest.mark.parametrize("label,rows,V,dtype", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_confidence_rows_split_over_workgroups(label, rows, V, dtype):
    """Fewer rows than CUs: each row's ids are cut into ranges on separate
    workgroups and the last range to finish merges them.  Corner rows put
    equal maxima in different ranges (the lowest id wins), the maximum on both
    sides of a range boundary, the [MASK] id holding the maximum in a later
    range, and a row whose only finite logit sits in the last range.  Three
    calls in a row (the meeting slots must be back at zero) give the same
    bits."""
    log("case: confidence split rows %s" % label)
    ns, rlen = row_ranges(rows, V, 4 if dtype == torch.float32 else 2)
    assert ns > 1
    x = decision_logits(rows, V, seed=V + rows, dtype=torch.float32)
    top = float(x.max()) + 1.0
    mask_id = min(2 * rlen + 77, V - 1)
    first = rlen + rlen // 2 + 9
    x[0, first] = top                                     # equal maxima in two ranges: the lower id wins
    x[0, V - 5] = top
    if rows > 1:
        x[1, rlen - 1] = top                              # last id of a range ...
        x[1, rlen] = top                                  # ... and the first of the next: rlen - 1 wins
    if rows > 2:
        x[2, mask_id] = top + 3.0                         # [MASK] holds the maximum
        x[2, 11] = top
    if rows > 3:
        x[3, :] = float("-inf")
        x[3, V - 2] = -2.0                                # only finite logit in the last range
    x = x.to(dtype)
    runs = [gpu_confidence(x, mask_id, 0.5) for _ in range(3)]
    pred, conf, over = runs[0]
    for p2, c2, o2 in runs[1:]:
        assert np.array_equal(p2, pred) and np.array_equal(c2.view(np.int32), conf.view(np.int32))
        assert np.array_equal(o2, over)
    rp, rc = decode.confidences(x.double().numpy(), mask_id)
    assert np.array_equal(pred, rp), "predictions differ"
    assert pred[0] == first
    if rows > 1:
        assert pred[1] == rlen - 1
    if rows > 2:
        assert pred[2] == 11
    if rows > 3:
        assert pred[3] == V - 2 and conf[3] == pytest.approx(1.0, rel=1e-6)
    rel = np.abs(conf - rc) / np.maximum(rc, 1e-30)
    log("%d ranges of %d ids, conf max rel err %.2e" % (ns, rlen, rel.max()))
    assert rel.max() <= 1e-5
    assert np.array_equal(over.astype(bool), conf >= 0.5)


def test_confidence_split_calls_on_two_streams():
    """Split-row calls in flight together on two streams meet in separate
    slots of the library's table: interleaved calls on two streams, with no
    ordering between them, give the bits of the same calls made one by one."""
    log("case: confidence split rows on two streams")
    dev = torch.device("cuda")
    xs = [decision_logits(24, 131072, seed=900 + i).to(dev) for i in range(4)]
    want = [gpu_confidence(x, 126, 0.5) for x in xs]
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    outs = []
    torch.cuda.synchronize()
    for rep in range(3):
        for i, x in enumerate(xs):
            st = streams[i % 2]
            pred = torch.full((24,), -7, dtype=torch.int32, device=dev)
            conf = torch.full((24,), float("nan"), dtype=torch.float32, device=dev)
            over = torch.full((24,), 7, dtype=torch.uint8, device=dev)
            # the output fills were made on the current stream: order them
            st.wait_stream(torch.cuda.current_stream())
            binding.confidence(x, 126, 0.5, pred, conf, over, stream=st)
            outs.append((i, pred, conf, over))
    torch.cuda.synchronize()
    for i, pred, conf, over in outs:
        wp, wc, wo = want[i]
        assert np.array_equal(pred.cpu().numpy(), wp)
        assert np.array_equal(conf.cpu().numpy().view(np.int32), wc.view(np.int32))
        assert np.array_equal(over.cpu().numpy(), wo)


def test_accept_matches_oracle():
    log("case: sequential acceptance")
    rng = np.random.default_rng(11)
    B, S = 200, 32
    x_hat = rng.integers(0, 5, size=(B, S)).astype(np.int32)
    x_tilde = np.where(rng.random((B, S)) < 0.9, x_hat, (x_hat + 1) % 5).astype(np.int32)
    c_tilde = rng.random((B, S)).astype(np.float32) * 0.4 + 0.6
    gamma = float(np.float32(0.7))   # the threshold both sides compare against
    dev = torch.device("cuda")
    n = torch.full((B,), -7, dtype=torch.int32, device=dev)
    binding.accept(torch.from_numpy(x_hat).to(dev), torch.from_numpy(x_tilde).to(dev),
                   torch.from_numpy(c_tilde).to(dev), gamma, n)
    torch.cuda.synchronize()
    got = n.cpu().numpy()
    for b in range(B):
        acc = decode.accept(list(range(S)), dict(enumerate(x_hat[b].tolist())),
                            dict(enumerate(x_tilde[b].tolist())), dict(enumerate(c_tilde[b].tolist())), gamma)
        assert got[b] == len(acc)
    assert 0 < got.mean() < S
