"""Pins of the fp64 oracle against things other than itself.

Each test ties a part of the oracle to a library routine (torch linear,
scaled-dot-product attention, logsumexp, the Hugging Face rotary helper, the
bf16 cast), to a closed form, or to an invariant the pages state, chosen so
that a dropped term, a wrong sign or index, or a transposed operand fails at
least one of them.  Sources: the Flash-dLLM pages (jaehun.me review sections
"Flash-Verify" and "How It Works: A Concrete Example"; alanhou.org "Core
Mechanism").
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import ROUND_BF16, ROUND_EXACT, ROUND_FP32, Shape
from io_aware_kv_amd.workloads import LayerShape, make_random_case, make_workload


def _shape(ls: LayerShape) -> Shape:
    return Shape(ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, ls.rope_base)


def _rot_complex(x, pos, base):
    """Rotary embedding written as complex multiplication: the pair
    (x_i, x_{i+dh/2}) is z = x_i + i x_{i+dh/2}, rotated by exp(i pos theta_i),
    theta_i = base^(-2i/dh)."""
    dh = x.shape[-1]
    half = dh // 2
    theta = base ** (-2.0 * np.arange(half) / dh)
    phase = np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * theta)
    z = (x[..., :half] + 1j * x[..., half:]) * phase
    return np.concatenate([z.real, z.imag], axis=-1)


def _proj_reference(ls, X, Q, P, W):
    """q, k, v via torch.nn.functional.linear in fp64 + complex rotation."""
    X64 = X.double()
    B, nq = Q.shape
    rows = torch.stack([X64[b, Q[b].long()] for b in range(B)])  # [B,nq,d]
    y = F.linear(rows, W.double()).numpy()                        # [B,nq,cols]
    H, Hkv, dh = ls.H, ls.Hkv, ls.dh
    q = y[..., : H * dh].reshape(B, nq, H, dh)
    k = y[..., H * dh:(H + Hkv) * dh].reshape(B, nq, Hkv, dh)
    v = y[..., (H + Hkv) * dh:].reshape(B, nq, Hkv, dh)
    pos = P.numpy()[:, :, None]
    return _rot_complex(q, pos, ls.rope_base), _rot_complex(k, pos, ls.rope_base), v


def _attn_reference(ls, q, k, v, P, vis, Kc_old, Vc_old):
    """Attention of each query row over its key set, via torch SDPA (fp64) and
    logsumexp: keys = old cache positions not written this step, then the new
    rows j visible under vis[b,i,j].  Heads map to kv head h * Hkv // H."""
    B, nq = P.shape
    H, Hkv, dh, N = ls.H, ls.Hkv, ls.dh, ls.N
    O = np.zeros((B, nq, H, dh))
    L = np.zeros((B, nq, H))
    for b in range(B):
        written = set(int(p) for p in P[b].tolist())
        keep = [p for p in range(N) if p not in written]
        for h in range(H):
            g = h * Hkv // H
            keys = np.concatenate([Kc_old[b, g, keep], k[b, :, g]], axis=0)
            vals = np.concatenate([Vc_old[b, g, keep], v[b, :, g]], axis=0)
            mask = np.ones((nq, len(keep) + nq), dtype=bool)
            if vis is not None:
                mask[:, len(keep):] = vis[b].numpy().astype(bool)
            qt = torch.from_numpy(np.ascontiguousarray(q[b, :, h]))[None, None]
            kt = torch.from_numpy(np.ascontiguousarray(keys))[None, None]
            vt = torch.from_numpy(np.ascontiguousarray(vals))[None, None]
            mt = torch.from_numpy(mask)[None, None]
            o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt)[0, 0].numpy()
            s = (qt[0, 0] @ kt[0, 0].T) / math.sqrt(dh)
            s = s.masked_fill(~mt[0, 0], float("-inf"))
            lse = torch.logsumexp(s, dim=-1).numpy()
            empty = ~mask.any(axis=1)
            o[empty] = 0.0
            O[b, :, h] = o
            L[b, :, h] = lse
    return O, L


# --------------------------------------------------------------------------
# rounding helper
# --------------------------------------------------------------------------

def test_round_bf16_matches_torch_cast():
    g = torch.Generator().manual_seed(1)
    x = torch.cat([torch.randn(20000, generator=g, dtype=torch.float64) * (10.0 ** e)
                   for e in (-40, -39, -38, -5, 0, 5, 30, 38)])
    # exact ties between two bf16 neighbours (ties-to-even must pick the even one)
    base = torch.randn(2000, generator=g).to(torch.bfloat16).double()
    ulp = torch.tensor([math.ldexp(1.0, math.frexp(float(t))[1] - 8) for t in base], dtype=torch.float64)
    x = torch.cat([x, base + ulp / 2, base - ulp / 2, torch.tensor([0.0, -0.0, 3.4e38, -3.4e38])])
    # torch rounds fp32 -> bf16 to nearest even; go through fp32 only where that is exact
    x32 = x.float().double()
    ref = x32.float().to(torch.bfloat16).double().numpy()
    got = oracle.round_store(x32.numpy(), ROUND_BF16)
    np.testing.assert_array_equal(got, ref)


def test_round_fp32_matches_numpy_cast():
    x = np.random.default_rng(2).standard_normal(10000) * 1e3
    np.testing.assert_array_equal(oracle.round_store(x, ROUND_FP32), x.astype(np.float32).astype(np.float64))
    np.testing.assert_array_equal(oracle.round_store(x, ROUND_EXACT), x)


# --------------------------------------------------------------------------
# a1-a3: gather, projection, rotary
# --------------------------------------------------------------------------

def test_projection_matches_linear_and_complex_rotation():
    ls = LayerShape(B=2, N=40, d_model=24, H=4, Hkv=2, dh=8, dtype=torch.float32)
    wl = make_random_case(ls, nq=7, seed=3, n_extra_rows=3, dup_frac=0.3)
    q, k, v = oracle.project(_shape(ls), wl.X, wl.Q_idx, wl.pos_ids, wl.W, ROUND_EXACT)
    rq, rk, rv = _proj_reference(ls, wl.X, wl.Q_idx, wl.pos_ids, wl.W)
    np.testing.assert_allclose(q, rq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(k, rk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(v, rv, rtol=0, atol=1e-12)


def test_rotation_matches_huggingface_rotate_half():
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb
    dh, H = 32, 4
    cfg = LlamaConfig(hidden_size=H * dh, num_attention_heads=H, num_key_value_heads=H,
                      head_dim=dh, rope_theta=10000.0, max_position_embeddings=4096)
    rot = LlamaRotaryEmbedding(cfg)
    ls = LayerShape(B=1, N=300, d_model=H * dh, H=H, Hkv=H, dh=dh, dtype=torch.float32)
    pos = [[0, 1, 7, 123, 299]]
    wl = make_random_case(ls, nq=5, seed=4, positions=pos)
    q, k, _ = oracle.project(_shape(ls), wl.X, wl.Q_idx, wl.pos_ids, wl.W, ROUND_EXACT)
    # unrotated projections: position 0 for every row is the identity rotation
    zero = torch.zeros_like(wl.pos_ids)
    q0, k0, _ = oracle.project(_shape(ls), wl.X, wl.Q_idx, zero, wl.W, ROUND_EXACT)
    cos, sin = rot(torch.zeros(1, 5, dh), wl.pos_ids.long())
    tq = torch.from_numpy(q0).permute(0, 2, 1, 3).float()  # [B,H,nq,dh]
    tk = torch.from_numpy(k0).permute(0, 2, 1, 3).float()
    rq, rk = apply_rotary_pos_emb(tq, tk, cos, sin)
    # the library builds its phases in fp32: agreement to fp32 phase accuracy
    np.testing.assert_allclose(q, rq.permute(0, 2, 1, 3).double().numpy(), atol=2e-4, rtol=0)
    np.testing.assert_allclose(k, rk.permute(0, 2, 1, 3).double().numpy(), atol=2e-4, rtol=0)


def test_rotation_identity_norm_and_relative_position():
    ls = LayerShape(B=1, N=5000, d_model=16, H=2, Hkv=1, dh=16, dtype=torch.float32)
    wl = make_random_case(ls, nq=4, seed=5, positions=[[0, 10, 999, 4321]])
    sh = _shape(ls)
    q, k, v = oracle.project(sh, wl.X, wl.Q_idx, wl.pos_ids, wl.W, ROUND_EXACT)
    z = torch.zeros_like(wl.pos_ids)
    q0, k0, v0 = oracle.project(sh, wl.X, wl.Q_idx, z, wl.W, ROUND_EXACT)
    # position 0 is the identity; v is never rotated
    np.testing.assert_array_equal(q[:, 0], q0[:, 0])
    np.testing.assert_array_equal(v, v0)
    # each (i, i+dh/2) pair keeps its norm
    half = ls.dh // 2
    n1 = q[..., :half] ** 2 + q[..., half:] ** 2
    n0 = q0[..., :half] ** 2 + q0[..., half:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12, atol=1e-14)
    # q(p) . k(p') depends only on p - p': shift every position by s
    shifted = wl.pos_ids + 17
    q2, k2, _ = oracle.project(sh, wl.X, wl.Q_idx, shifted, wl.W, ROUND_EXACT)
    s1 = np.einsum("bihd,bjd->bijh", q, k[:, :, 0])
    s2 = np.einsum("bihd,bjd->bijh", q2, k2[:, :, 0])
    np.testing.assert_allclose(s1, s2, rtol=1e-9, atol=1e-9)


def test_identity_block_weight_copies_rows():
    # W = [I; I; I] per head (d_model = dh, one head each): q = k = v = rotated x
    dh = 8
    ls = LayerShape(B=1, N=10, d_model=dh, H=1, Hkv=1, dh=dh, dtype=torch.float32)
    wl = make_random_case(ls, nq=3, seed=6)
    W = torch.cat([torch.eye(dh)] * 3)
    q, k, v = oracle.project(_shape(ls), wl.X, wl.Q_idx, wl.pos_ids, W, ROUND_EXACT)
    rows = wl.X[0, wl.Q_idx[0].long()].double().numpy()
    np.testing.assert_array_equal(v[0, :, 0], rows)
    np.testing.assert_allclose(q[0, :, 0], _rot_complex(rows, wl.pos_ids[0].numpy(), 10000.0),
                               atol=1e-13)
    np.testing.assert_array_equal(q, k)


# --------------------------------------------------------------------------
# a4: write-back
# --------------------------------------------------------------------------

def test_write_back_touches_only_query_positions_first_occurrence_wins():
    ls = LayerShape(B=2, N=30, d_model=16, H=2, Hkv=2, dh=8, dtype=torch.float32)
    wl = make_random_case(ls, nq=9, seed=7, n_extra_rows=4, dup_frac=0.4, masked_vis=True)
    sh = _shape(ls)
    sentinel = 1234.5
    Kc = np.full((ls.B, ls.Hkv, ls.N, ls.dh), sentinel)
    Vc = np.full_like(Kc, -sentinel)
    r = oracle.step(sh, wl.X, wl.Q_idx, wl.pos_ids, wl.vis, wl.W, Kc, Vc, ROUND_EXACT)
    P = wl.pos_ids.numpy()
    assert any(len(set(P[b])) < P.shape[1] for b in range(ls.B)), "case needs duplicates"
    for b in range(ls.B):
        first = {}
        for j, p in enumerate(P[b]):
            first.setdefault(int(p), j)
        for p in range(ls.N):
            if p in first:
                np.testing.assert_array_equal(r["Kc"][b, :, p], r["k"][b, first[p]])
                np.testing.assert_array_equal(r["Vc"][b, :, p], r["v"][b, first[p]])
            else:
                assert (r["Kc"][b, :, p] == sentinel).all() and (r["Vc"][b, :, p] == -sentinel).all()


# --------------------------------------------------------------------------
# a5-a7: attention
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dup,masked", [(0.0, False), (0.3, False), (0.3, True), (0.0, True)])
def test_attention_matches_sdpa_over_explicit_key_set(dup, masked):
    ls = LayerShape(B=2, N=48, d_model=20, H=6, Hkv=2, dh=8, dtype=torch.float32)
    wl = make_random_case(ls, nq=11, seed=8 + int(dup * 10) + masked, n_extra_rows=5,
                          dup_frac=dup, masked_vis=masked, w_std=0.5)
    sh = _shape(ls)
    g = np.random.default_rng(9)
    Kc = g.standard_normal((ls.B, ls.Hkv, ls.N, ls.dh))
    Vc = g.standard_normal((ls.B, ls.Hkv, ls.N, ls.dh))
    r = oracle.step(sh, wl.X, wl.Q_idx, wl.pos_ids, wl.vis, wl.W, Kc, Vc, ROUND_EXACT)
    q, k, v = _proj_reference(ls, wl.X, wl.Q_idx, wl.pos_ids, wl.W)
    O, L = _attn_reference(ls, q, k, v, wl.pos_ids, wl.vis, Kc, Vc)
    np.testing.assert_allclose(r["O"], O, atol=1e-11, rtol=0)
    np.testing.assert_allclose(r["LSE"], L, atol=1e-11, rtol=0)


def test_consistent_cache_equals_full_bidirectional_attention():
    """Cache built from the same hidden states, distinct positions, all visible:
    the step equals full bidirectional MHA over the sequence, taken at Q."""
    ls = LayerShape(B=2, N=32, d_model=16, H=4, Hkv=4, dh=8, dtype=torch.float32)
    wl = make_random_case(ls, nq=6, seed=10, w_std=0.4)
    sh = _shape(ls)
    Kc, Vc = oracle.prefill(sh, wl.X, wl.W, ROUND_EXACT)
    r = oracle.step(sh, wl.X, wl.Q_idx, wl.pos_ids, None, wl.W, Kc, Vc, ROUND_EXACT)
    allpos = torch.arange(ls.N, dtype=torch.int32).repeat(ls.B, 1)
    q, k, v = _proj_reference(ls, wl.X, allpos, allpos, wl.W)
    for b in range(ls.B):
        qt = torch.from_numpy(q[b]).permute(1, 0, 2)   # [H,N,dh]
        kt = torch.from_numpy(k[b]).permute(1, 0, 2)
        vt = torch.from_numpy(v[b]).permute(1, 0, 2)
        o = F.scaled_dot_product_attention(qt, kt, vt).permute(1, 0, 2).numpy()
        lse = torch.logsumexp((qt @ kt.transpose(1, 2)) / math.sqrt(ls.dh), -1).T.numpy()
        rows = wl.pos_ids[b].long().numpy()
        np.testing.assert_allclose(r["O"][b], o[rows], atol=1e-11)
        np.testing.assert_allclose(r["LSE"][b], lse[rows], atol=1e-11)


def test_single_visible_key_and_identical_keys_closed_forms():
    ls = LayerShape(B=1, N=2, d_model=8, H=1, Hkv=1, dh=8, dtype=torch.float32)
    wl = make_random_case(ls, nq=2, seed=11, positions=[[0, 1]])
    sh = _shape(ls)
    vis = torch.tensor([[[1, 0], [1, 0]]], dtype=torch.uint8)   # both rows see only row 0
    Kc = np.zeros((1, 1, 2, 8))
    r = oracle.step(sh, wl.X, wl.Q_idx, wl.pos_ids, vis, wl.W, Kc, Kc, ROUND_EXACT)
    for i in range(2):
        np.testing.assert_allclose(r["O"][0, i, 0], r["v"][0, 0, 0], atol=1e-14)
        s = float(r["q"][0, i, 0] @ r["k"][0, 0, 0]) / math.sqrt(8)
        assert abs(r["LSE"][0, i, 0] - s) < 1e-13

    # n identical old keys (the query cannot see its own new row): O = v, LSE = s + ln n
    ls = LayerShape(B=1, N=9, d_model=8, H=1, Hkv=1, dh=8, dtype=torch.float32)
    wl = make_random_case(ls, nq=1, seed=12, positions=[[4]])
    sh = _shape(ls)
    kr = np.random.default_rng(13).standard_normal(8)
    vr = np.random.default_rng(14).standard_normal(8)
    Kc = np.tile(kr, (1, 1, 9, 1))
    Vc = np.tile(vr, (1, 1, 9, 1))
    r = oracle.step(sh, wl.X, wl.Q_idx, wl.pos_ids, torch.zeros((1, 1, 1), dtype=torch.uint8),
                    wl.W, Kc, Vc, ROUND_EXACT)
    np.testing.assert_allclose(r["O"][0, 0, 0], vr, atol=1e-13)
    s = float(r["q"][0, 0, 0] @ kr) / math.sqrt(8)
    assert abs(r["LSE"][0, 0, 0] - (s + math.log(8))) < 1e-12


def test_empty_key_set_gives_zero_output_and_minus_inf_lse():
    ls = LayerShape(B=1, N=3, d_model=8, H=2, Hkv=1, dh=4, dtype=torch.float32)
    wl = make_random_case(ls, nq=3, seed=15, positions=[[2, 0, 1]])
    vis = torch.zeros((1, 3, 3), dtype=torch.uint8)
    vis[0, 1, 1] = 1
    Kc = np.ones((1, 1, 3, 4))
    r = oracle.step(_shape(ls), wl.X, wl.Q_idx, wl.pos_ids, vis, wl.W, Kc, Kc, ROUND_EXACT)
    assert np.all(r["O"][0, [0, 2]] == 0) and np.all(np.isneginf(r["LSE"][0, [0, 2]]))
    assert np.isfinite(r["LSE"][0, 1]).all()


def test_gqa_equals_mha_with_replicated_kv_heads():
    H, Hkv, dh, d = 6, 2, 8, 16
    G = H // Hkv
    ls = LayerShape(B=2, N=20, d_model=d, H=H, Hkv=Hkv, dh=dh, dtype=torch.float32)
    wl = make_random_case(ls, nq=5, seed=16, n_extra_rows=2, dup_frac=0.3, masked_vis=True, w_std=0.4)
    g = np.random.default_rng(17)
    Kc = g.standard_normal((2, Hkv, 20, dh))
    Vc = g.standard_normal((2, Hkv, 20, dh))
    r = oracle.step(_shape(ls), wl.X, wl.Q_idx, wl.pos_ids, wl.vis, wl.W, Kc, Vc, ROUND_EXACT)
    Wq = wl.W[: H * dh]
    Wk = wl.W[H * dh:(H + Hkv) * dh].reshape(Hkv, dh, d)
    Wv = wl.W[(H + Hkv) * dh:].reshape(Hkv, dh, d)
    rep = torch.arange(H) // G
    W2 = torch.cat([Wq, Wk[rep].reshape(H * dh, d), Wv[rep].reshape(H * dh, d)])
    ls2 = LayerShape(B=2, N=20, d_model=d, H=H, Hkv=H, dh=dh, dtype=torch.float32)
    r2 = oracle.step(_shape(ls2), wl.X, wl.Q_idx, wl.pos_ids, wl.vis, W2,
                     Kc[:, rep.numpy()], Vc[:, rep.numpy()], ROUND_EXACT)
    np.testing.assert_allclose(r["O"], r2["O"], atol=1e-13)
    np.testing.assert_allclose(r["LSE"], r2["LSE"], atol=1e-13)


def test_views_are_mutually_invisible():
    """Perturbing the draft view's hidden states leaves the mask view's outputs
    bit-identical, and vice versa (the views cannot see each other)."""
    ls = LayerShape(B=1, N=64, d_model=32, H=4, Hkv=2, dh=8, dtype=torch.float32)
    # a small verification layout: 2 tracked, 2 confident, 3 exploratory x 2 views
    tv, D, S = [3, 9], [40, 43], [41, 42, 44]
    pos = tv + D + S + S
    idx = tv + D + S + [64, 65, 66]
    groups = [["track"] * 2 + ["confident"] * 2 + ["draft"] * 3 + ["mask"] * 3]
    from io_aware_kv_amd.workloads import view_block_mask
    vis = view_block_mask(groups)
    g = torch.Generator().manual_seed(18)
    X = torch.randn((1, 67, 32), generator=g)
    W = torch.randn((ls.cols, 32), generator=g) * 0.3
    Kc = np.random.default_rng(19).standard_normal((1, 2, 64, 8))
    Vc = np.random.default_rng(20).standard_normal((1, 2, 64, 8))
    Q = torch.tensor([idx], dtype=torch.int32)
    P = torch.tensor([pos], dtype=torch.int32)
    sh = _shape(ls)
    base = oracle.step(sh, X, Q, P, vis, W, Kc, Vc, ROUND_BF16)
    draft_rows = [i for i in range(len(pos)) if groups[0][i] == "draft"]
    mask_rows = [i for i in range(len(pos)) if groups[0][i] == "mask"]
    X2 = X.clone()
    X2[0, [idx[i] for i in draft_rows]] += 3.0
    pert = oracle.step(sh, X2, Q, P, vis, W, Kc, Vc, ROUND_BF16)
    np.testing.assert_array_equal(pert["O"][0, mask_rows], base["O"][0, mask_rows])
    np.testing.assert_array_equal(pert["LSE"][0, mask_rows], base["LSE"][0, mask_rows])
    assert not np.array_equal(pert["O"][0, draft_rows], base["O"][0, draft_rows])
    X3 = X.clone()
    X3[0, [idx[i] for i in mask_rows]] -= 2.0
    pert = oracle.step(sh, X3, Q, P, vis, W, Kc, Vc, ROUND_BF16)
    np.testing.assert_array_equal(pert["O"][0, draft_rows], base["O"][0, draft_rows])
    np.testing.assert_array_equal(pert["LSE"][0, draft_rows], base["LSE"][0, draft_rows])


def test_rounding_points_change_results_only_slightly_and_deterministically():
    ls = LayerShape(B=1, N=40, d_model=32, H=4, Hkv=2, dh=16)
    wl = make_random_case(ls, nq=6, seed=21)
    sh = _shape(ls)
    Kc = torch.randn((1, 2, 40, 16), generator=torch.Generator().manual_seed(22)).to(torch.bfloat16)
    a = oracle.step(sh, wl.X, wl.Q_idx, wl.pos_ids, None, wl.W, Kc, Kc, ROUND_BF16)
    b = oracle.step(sh, wl.X, wl.Q_idx, wl.pos_ids, None, wl.W, Kc, Kc, ROUND_BF16)
    e = oracle.step(sh, wl.X, wl.Q_idx, wl.pos_ids, None, wl.W, Kc, Kc, ROUND_EXACT)
    np.testing.assert_array_equal(a["O"], b["O"])
    # stored values (O, k, v) are bf16 values; q is the unrounded on-chip value
    np.testing.assert_array_equal(oracle.round_store(a["O"], ROUND_BF16), a["O"])
    np.testing.assert_array_equal(oracle.round_store(a["k"], ROUND_BF16), a["k"])
    np.testing.assert_array_equal(oracle.round_store(a["v"], ROUND_BF16), a["v"])
    np.testing.assert_array_equal(a["q"], e["q"])
    assert not np.array_equal(oracle.round_store(a["q"], ROUND_BF16), a["q"])
    assert np.abs(a["O"] - e["O"]).max() < 2e-2 * np.abs(e["O"]).max()
    assert np.abs(a["LSE"] - e["LSE"]).max() < 5e-3


def test_empty_query_set_is_a_no_op():
    ls = LayerShape(B=1, N=8, d_model=8, H=2, Hkv=1, dh=4, dtype=torch.float32)
    X = torch.randn(1, 8, 8)
    W = torch.randn(16, 8)
    Kc = np.random.default_rng(23).standard_normal((1, 1, 8, 4))
    r = oracle.step(_shape(ls), X, torch.zeros((1, 0), dtype=torch.int32),
                    torch.zeros((1, 0), dtype=torch.int32), None, W, Kc, Kc, ROUND_EXACT)
    assert r["O"].shape == (1, 0, 2, 4)
    np.testing.assert_array_equal(r["Kc"], Kc)


def test_prefill_equals_step_over_every_position():
    ls = LayerShape(B=2, N=12, d_model=16, H=2, Hkv=2, dh=8, dtype=torch.float32)
    wl = make_random_case(ls, nq=3, seed=24)
    sh = _shape(ls)
    Kc, Vc = oracle.prefill(sh, wl.X, wl.W, ROUND_FP32)
    allpos = torch.arange(12, dtype=torch.int32).repeat(2, 1)
    _, k, v = oracle.project(sh, wl.X, allpos, allpos, wl.W, ROUND_FP32)
    np.testing.assert_array_equal(Kc, k.transpose(0, 2, 1, 3))
    np.testing.assert_array_equal(Vc, v.transpose(0, 2, 1, 3))


def test_tiny_fp32_layer_end_to_end_against_library_composition():
    """The tiny fp32 layer (B=1, N=64, d=128, H=Hkv=4, dh=32, queries 33..36),
    cache prefilled from the full sequence, against the SDPA composition."""
    wl = make_workload(1)
    ls = wl.shape
    sh = _shape(ls)
    Kc, Vc = oracle.prefill(sh, wl.X_pre, wl.W, ROUND_EXACT)
    r = oracle.step(sh, wl.X, wl.Q_idx, wl.pos_ids, None, wl.W, Kc, Vc, ROUND_EXACT)
    q, k, v = _proj_reference(ls, wl.X, wl.Q_idx, wl.pos_ids, wl.W)
    O, L = _attn_reference(ls, q, k, v, wl.pos_ids, None, Kc, Vc)
    np.testing.assert_allclose(r["O"], O, atol=1e-11)
    np.testing.assert_allclose(r["LSE"], L, atol=1e-11)


# --------------------------------------------------------------------------
# tracked-set scores (next step after the path): attention mass per position
# --------------------------------------------------------------------------

def _mass_reference(ls, q, k, P, vis, sel, Kc_old):
    """Per cache position, the summed softmax probability that the selected
    rows give it, from torch.softmax over each row's explicit key set (old
    positions not written this step, then the new rows j visible to i); a new
    row counts toward its position only if it is the first row there."""
    B, nq = P.shape
    H, Hkv, dh, N = ls.H, ls.Hkv, ls.dh, ls.N
    out = np.zeros((B, N))
    for b in range(B):
        pos = [int(p) for p in P[b].tolist()]
        written = set(pos)
        keep = [p for p in range(N) if p not in written]
        first = [pos.index(pos[j]) == j for j in range(nq)]
        for h in range(H):
            g = h * Hkv // H
            keys = torch.from_numpy(np.concatenate([Kc_old[b, g, keep], k[b, :, g]], axis=0))
            for i in range(nq):
                if not sel[b, i]:
                    continue
                s = keys @ torch.from_numpy(np.ascontiguousarray(q[b, i, h])) / math.sqrt(dh)
                m = torch.ones(len(keep) + nq, dtype=torch.bool)
                if vis is not None:
                    m[len(keep):] = torch.from_numpy(vis[b, i].numpy().astype(bool))
                if not m.any():
                    continue
                pr = torch.softmax(s.masked_fill(~m, float("-inf")), dim=0).numpy()
                out[b, keep] += pr[:len(keep)]
                for j in range(nq):
                    if first[j]:
                        out[b, pos[j]] += pr[len(keep) + j]
    return out


@pytest.mark.parametrize("dup,masked", [(0.0, False), (0.3, True), (0.3, False), (0.0, True)])
def test_key_scores_match_softmax_columns(dup, masked):
    ls = LayerShape(B=2, N=40, d_model=20, H=6, Hkv=2, dh=8, dtype=torch.float32)
    wl = make_random_case(ls, nq=10, seed=21 + int(dup * 10) + masked, n_extra_rows=4,
                          dup_frac=dup, masked_vis=masked, w_std=0.5)
    sh = _shape(ls)
    g = np.random.default_rng(22)
    Kc = g.standard_normal((ls.B, ls.Hkv, ls.N, ls.dh))
    Vc = g.standard_normal((ls.B, ls.Hkv, ls.N, ls.dh))
    r = oracle.step(sh, wl.X, wl.Q_idx, wl.pos_ids, wl.vis, wl.W, Kc, Vc, ROUND_EXACT)
    sel = (g.random((ls.B, 10)) < 0.6).astype(np.uint8)
    a = oracle.key_scores(sh, r["q"], r["Kc"], r["LSE"], wl.pos_ids, wl.vis, sel)
    q, k, _ = _proj_reference(ls, wl.X, wl.Q_idx, wl.pos_ids, wl.W)
    ref = _mass_reference(ls, q, k, wl.pos_ids, wl.vis, sel, Kc)
    np.testing.assert_allclose(a, ref, atol=1e-11, rtol=0)


def test_key_scores_closed_forms():
    """All rows selected, distinct positions, no mask: every row-head
    distribution sums to one over the cache, so the scores sum to nq * H.
    A mask hiding every new row leaves the written positions at zero."""
    ls = LayerShape(B=2, N=30, d_model=16, H=4, Hkv=2, dh=8, dtype=torch.float32)
    wl = make_random_case(ls, nq=6, seed=23, w_std=0.5)
    sh = _shape(ls)
    g = np.random.default_rng(24)
    Kc = g.standard_normal((ls.B, ls.Hkv, ls.N, ls.dh))
    Vc = g.standard_normal((ls.B, ls.Hkv, ls.N, ls.dh))
    r = oracle.step(sh, wl.X, wl.Q_idx, wl.pos_ids, None, wl.W, Kc, Vc, ROUND_EXACT)
    sel = np.ones((ls.B, 6), dtype=np.uint8)
    a = oracle.key_scores(sh, r["q"], r["Kc"], r["LSE"], wl.pos_ids, None, sel)
    np.testing.assert_allclose(a.sum(axis=1), 6 * ls.H, rtol=1e-12)
    assert (a > 0).all()
    hide = torch.zeros((ls.B, 6, 6), dtype=torch.uint8)
    r2 = oracle.step(sh, wl.X, wl.Q_idx, wl.pos_ids, hide, wl.W, Kc, Vc, ROUND_EXACT)
    a2 = oracle.key_scores(sh, r2["q"], r2["Kc"], r2["LSE"], wl.pos_ids, hide, sel)
    for b in range(ls.B):
        written = wl.pos_ids[b].numpy()
        assert np.all(a2[b, written] == 0.0)
        np.testing.assert_allclose(a2[b].sum(), 6 * ls.H, rtol=1e-12)
    # one selected row: its scores are its own softmax, summed over heads
    sel1 = np.zeros_like(sel)
    sel1[0, 2] = 1
    a1 = oracle.key_scores(sh, r["q"], r["Kc"], r["LSE"], wl.pos_ids, None, sel1)
    assert np.all(a1[1] == 0.0)
    np.testing.assert_allclose(a1[0].sum(), ls.H, rtol=1e-12)


def test_select_top_by_hand():
    sc = np.array([[0.5, 0.9, 0.9, 0.1, 0.7],
                   [0.0, 0.0, 0.3, 0.0, 0.0]], dtype=np.float32)
    cand = np.array([[1, 1, 1, 1, 1], [1, 1, 0, 1, 0]], dtype=np.uint8)
    assert oracle.select_top(sc, cand, 3).tolist() == [[1, 2, 4], [0, 1, 3]]
    cand2 = np.array([[1, 0, 1, 0, 0], [0, 0, 0, 0, 0]], dtype=np.uint8)
    assert oracle.select_top(sc, cand2, 3).tolist() == [[2, 0, -1], [-1, -1, -1]]
    assert oracle.select_top(sc, cand, 0).shape == (2, 0)


# --------------------------------------------------------------------------
# paged cache and ragged sequences (serving variant)
# --------------------------------------------------------------------------

def test_paged_step_equals_flat_step_and_moves_rows_with_the_table():
    """Full lengths and row counts: the paged step is the flat step with the
    cache rows found through the table; the pool rows it writes are the flat
    step's rows at their blocks, every other pool row is untouched."""
    from io_aware_kv_amd.workloads import initial_cache, paged_layout
    ls = LayerShape(B=2, N=40, d_model=16, H=4, Hkv=2, dh=8, dtype=torch.float32)
    wl = make_random_case(ls, nq=6, seed=51, n_extra_rows=2, dup_frac=0.3, masked_vis=True, w_std=0.5)
    sh = _shape(ls)
    table, Kp, Vp, L, nb = paged_layout(wl, block_size=16, ragged=False)
    K0, V0 = initial_cache(wl)
    flat = oracle.step(sh, wl.X, wl.Q_idx, wl.pos_ids, wl.vis, wl.W, K0, V0, ROUND_FP32)
    pg = oracle.step_paged(sh, wl.X, wl.Q_idx, wl.pos_ids, nb, wl.vis, wl.W, Kp, Vp, table, 16, L, ROUND_FP32)
    np.testing.assert_array_equal(pg["O"], flat["O"])
    np.testing.assert_array_equal(pg["LSE"], flat["LSE"])
    Kp0 = Kp.double().numpy()
    used = np.zeros(Kp0.shape[0], dtype=bool)
    for b in range(ls.B):
        for p in range(ls.N):
            blk, row = int(table[b, p // 16]), p % 16
            used[blk] = True
            np.testing.assert_array_equal(pg["Kpool"][blk, :, row], flat["Kc"][b, :, p])
    np.testing.assert_array_equal(pg["Kpool"][~used], Kp0[~used])


def test_ragged_rows_are_padding_and_short_sequences_see_only_their_keys():
    """A sequence with fewer rows and a shorter length is the same step run
    on its live rows over its first seq_len positions; padding rows give
    zero output and -inf LSE."""
    from io_aware_kv_amd.workloads import initial_cache
    ls = LayerShape(B=2, N=40, d_model=16, H=4, Hkv=2, dh=8, dtype=torch.float32)
    wl = make_random_case(ls, nq=6, seed=52, w_std=0.5, positions=[[3, 9, 1, 30, 31, 39], [5, 6, 7, 8, 0, 2]])
    sh = _shape(ls)
    K0, V0 = initial_cache(wl)
    table = torch.arange(2 * 3, dtype=torch.int32).reshape(2, 3)
    Kp = torch.zeros((6, 2, 16, 8))
    Vp = torch.zeros((6, 2, 16, 8))
    for b in range(2):
        for k in range(3):
            n = min(16, 40 - 16 * k)
            Kp[3 * b + k, :, :n] = K0[b, :, 16 * k:16 * k + n]
            Vp[3 * b + k, :, :n] = V0[b, :, 16 * k:16 * k + n]
    L = torch.tensor([40, 12], dtype=torch.int32)
    nb = torch.tensor([6, 4], dtype=torch.int32)
    pg = oracle.step_paged(sh, wl.X, wl.Q_idx, wl.pos_ids, nb, None, wl.W, Kp, Vp, table, 16, L, ROUND_EXACT)
    # sequence 1 alone: 4 rows over 12 positions
    sh1 = Shape(1, 12, ls.d_model, ls.H, ls.Hkv, ls.dh, ls.rope_base)
    r1 = oracle.step(sh1, wl.X[1:2], wl.Q_idx[1:2, :4], wl.pos_ids[1:2, :4], None, wl.W, K0[1:2, :, :12],
                     V0[1:2, :, :12], ROUND_EXACT)
    np.testing.assert_allclose(pg["O"][1, :4], r1["O"][0], rtol=0, atol=0)
    assert np.all(pg["O"][1, 4:] == 0) and np.all(np.isneginf(pg["LSE"][1, 4:]))
    # the short sequence's keys stop at 12: positions 12.. of its cache are unused
    q, k, v = _proj_reference(ls, wl.X[1:2], wl.Q_idx[1:2, :4], wl.pos_ids[1:2, :4], wl.W)
    O, Lr = _attn_reference(LayerShape(B=1, N=12, d_model=16, H=4, Hkv=2, dh=8, dtype=torch.float32), q, k, v,
                            wl.pos_ids[1:2, :4], None, K0[1:2, :, :12].double().numpy(),
                            V0[1:2, :, :12].double().numpy())
    np.testing.assert_allclose(pg["LSE"][1, :4], Lr[0], atol=1e-11, rtol=0)
