"""Pins for the CPU oracle, checked against things other than the oracle.

* the dense limit (tau = -inf) against a brute-force softmax and against
  torch's scaled_dot_product_attention in float64;
* key blocks with constant rows, where the centroid term is exact, so any
  routing must reproduce dense attention (pins the per-row centroid logit,
  the log-mass bias log(n_c) and the ragged tail);
* an independent full-matrix brute force at N <= 256 that routes from
  token-level scores and applies one masked softmax over N + n_b columns;
* hand-derived routing results (tests/golden/route_hand.json) and a
  closed-form centroid case;
* invariants: tau monotonicity, top-K counts, convex hull of V, the Jensen
  bound on centroid mass, prefix rows equal dense rows, and block-permutation
  equivariance.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import sol_oracle as O
from block_sparse_video_fp32_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(bits):
    return inputs.bf16_bits_to_f32(bits).astype(np.float64)


def _rand(B, N, H, D, seed):
    q, k, v = inputs.iid(B, N, H, D, seed)
    return _f64(q), _f64(k), _f64(v)


def dense_reference(q, k, v, scale=None):
    """softmax(q k^T * scale) v per (b, h), written out directly."""
    B, N, H, D = q.shape
    s = (1.0 / math.sqrt(D)) if scale is None else scale
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            L = q[b, :, h] @ k[b, :, h].T * s
            W = np.exp(L - L.max(axis=1, keepdims=True))
            out[b, :, h] = (W / W.sum(axis=1, keepdims=True)) @ v[b, :, h]
    return out


def brute_force(q, k, v, *, tau=1.0, topk_ratio=None, prefix_len=0, prefix_rows=True, centroid=True, logmass=True):
    """Independent small-N implementation: token-level scores, one masked
    softmax over [N exact keys | n_b centroids] per query row."""
    B, N, H, D = q.shape
    nb = (N + 63) // 64
    blk = np.arange(N) // 64
    sizes = np.bincount(blk, minlength=nb).astype(np.float64)
    ind = np.zeros((N, nb))
    ind[np.arange(N), blk] = 1.0  # token -> block indicator
    pb = (prefix_len + 63) // 64
    scale = 1.0 / math.sqrt(D)
    out = np.empty_like(q)
    sels = np.zeros((B, H, nb, nb), dtype=bool)
    for b in range(B):
        for h in range(H):
            Q, K, V = q[b, :, h], k[b, :, h], v[b, :, h]
            T = Q @ K.T  # token scores
            # block score = mean over the block pair of token scores
            S = (ind.T @ T @ ind) / np.outer(sizes, sizes)
            sel = np.zeros((nb, nb), dtype=bool)
            for a in range(nb):
                row = S[a]
                if topk_ratio is not None:
                    kk = O.topk_count(topk_ratio, nb)
                    order = np.lexsort((np.arange(nb), -row))
                    sel[a, order[:kk]] = True
                elif tau == -math.inf:
                    sel[a] = True
                elif tau == math.inf:
                    pass
                else:
                    sel[a] = row >= row.mean() + tau * np.std(row)
            sel[:, :pb] = True
            if prefix_rows:
                sel[:pb, :] = True
            sels[b, h] = sel
            tok = sel[blk][:, blk]  # [N, N] token-level mask
            Kc = (ind.T @ K) / sizes[:, None]
            Vc = (ind.T @ V) / sizes[:, None]
            Lx = np.where(tok, T * scale, -np.inf)
            Ly = Q @ Kc.T * scale + (np.log(sizes)[None, :] if logmass else 0.0)
            Ly = np.where(sel[blk] | (not centroid), -np.inf, Ly)
            L = np.concatenate([Lx, Ly], axis=1)
            empty = np.isneginf(L).all(axis=1)  # no term at all: output 0
            L[empty] = 0.0
            W = np.exp(L - L.max(axis=1, keepdims=True))
            W[empty] = 0.0
            den = np.where(empty, 1.0, W.sum(axis=1))
            out[b, :, h] = (W @ np.concatenate([V, Vc])) / den[:, None]
    return out, sels


# ---------------------------------------------------------------- dense limit


@pytest.mark.parametrize("B,N,H,D", [(1, 200, 2, 64), (2, 256, 3, 128), (1, 130, 1, 64)])
def test_dense_limit_matches_softmax_and_sdpa(B, N, H, D):
    q, k, v = _rand(B, N, H, D, seed=11 + N)
    out, info = O.forward(q, k, v, tau=-math.inf)
    assert info["sel"].all()
    ref = dense_reference(q, k, v)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    import torch

    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)  # BTHD -> BHTD
    sdpa = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))
    np.testing.assert_allclose(out, sdpa.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)


def test_dense_limit_custom_scale():
    q, k, v = _rand(1, 192, 2, 64, seed=5)
    out, _ = O.forward(q, k, v, tau=-math.inf, sm_scale=0.37)
    np.testing.assert_allclose(out, dense_reference(q, k, v, scale=0.37), atol=1e-12)


# ------------------------------------------------- centroid exact on constant K


def _constant_key_blocks(q, k, seed):
    rng = np.random.default_rng(seed)
    B, N, H, D = k.shape
    k = k.copy()
    for c in range(0, N, 64):
        k[:, c : c + 64] = rng.standard_normal((B, 1, H, D))
    return k


@pytest.mark.parametrize(
    "route",
    [
        dict(tau=1.0),
        dict(tau=0.0),
        dict(tau=2.5),
        dict(tau=math.inf),
        dict(topk_ratio=0.25),
        dict(tau=1.0, prefix_len=70),
        dict(topk_ratio=0.1, prefix_len=64),
    ],
)
@pytest.mark.parametrize("N", [256, 200, 333])
def test_constant_key_blocks_reproduce_dense(route, N):
    q, k, v = _rand(1, N, 2, 64, seed=3 + N)
    k = _constant_key_blocks(q, k, seed=N)
    out, info = O.forward(q, k, v, **route)
    if route.get("tau") != math.inf:
        assert not info["sel"].all(), "routing left nothing to approximate"
    np.testing.assert_allclose(out, dense_reference(q, k, v), rtol=0, atol=1e-12)


def test_constant_key_blocks_need_the_log_mass_bias():
    q, k, v = _rand(1, 200, 2, 64, seed=9)
    k = _constant_key_blocks(q, k, seed=1)
    out, _ = O.forward(q, k, v, tau=1.0, logmass=False)
    assert np.abs(out - dense_reference(q, k, v)).max() > 1e-3


# ----------------------------------------------------------- brute force N<=256


@pytest.mark.parametrize(
    "N,H,D,kw",
    [
        (256, 2, 64, dict(tau=1.0)),
        (256, 2, 64, dict(tau=0.3)),
        (200, 2, 64, dict(tau=1.0)),
        (255, 1, 128, dict(topk_ratio=0.5)),
        (256, 2, 64, dict(topk_ratio=0.25, prefix_len=64)),
        (250, 2, 64, dict(tau=0.5, prefix_len=100)),
        (256, 2, 64, dict(tau=1.0, centroid=False)),
        (256, 2, 64, dict(tau=1.0, logmass=False)),
        (64, 1, 64, dict(tau=1.0)),
        (1, 1, 64, dict(tau=1.0)),
        (100, 3, 64, dict(tau=math.inf, prefix_len=10)),
        (256, 2, 64, dict(tau=1.0, prefix_len=100, prefix_rows=False)),
        (250, 2, 64, dict(topk_ratio=0.25, prefix_len=64, prefix_rows=False)),
        (100, 3, 64, dict(tau=math.inf, prefix_len=10, prefix_rows=False)),
    ],
)
def test_brute_force_small(N, H, D, kw):
    q, k, v = _rand(2, N, H, D, seed=N * 7 + H)
    # clustered-ish content so that routing is not trivial
    q = q + 1.5 * np.sin(np.arange(N) / 20.0)[None, :, None, None]
    k = q.copy() * 0.5 + k * 0.5
    out, info = O.forward(q, k, v, **kw)
    ref, sel = brute_force(q, k, v, **kw)
    np.testing.assert_array_equal(info["sel"], sel)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_brute_force_clustered_generator():
    q, k, v = inputs.clustered(1, 256, 2, 64, seed=4)
    q, k, v = _f64(q), _f64(k), _f64(v)
    out, info = O.forward(q, k, v, tau=1.0)
    ref, sel = brute_force(q, k, v, tau=1.0)
    np.testing.assert_array_equal(info["sel"], sel)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------- hand-derived routes


def _golden_cases():
    with open(os.path.join(GOLDEN, "route_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_route_hand_examples(case):
    if "S" in case:
        S = np.array(case["S"], dtype=np.float64)
    elif case["name"] == "topk_many_ties_low_index":
        S = (np.arange(640) % 5).astype(np.float64)[None, :]
    else:  # rule-built row
        S = -np.arange(640, dtype=np.float64)[None, :]
    nb = S.shape[1]
    full = np.zeros((nb, nb))
    full[: S.shape[0]] = S
    tau = case.get("tau")
    if isinstance(tau, str):
        tau = float(tau)
    r = O.route(full[None, None], tau=tau if tau is not None else 1.0,
                topk_ratio=case.get("topk_ratio"), prefix_len=case.get("prefix_len", 0),
                prefix_rows=case.get("prefix_rows", True))
    sel = r["sel"][0, 0]
    if "expect" in case:
        for a, want in enumerate(case["expect"]):
            assert list(np.nonzero(sel[a])[0]) == want, (case["name"], a)
    elif case["name"] == "topk_many_ties_low_index":
        assert list(np.nonzero(sel[0])[0]) == [5 * j + 4 for j in range(64)]
    else:
        assert sel[0].sum() == case["expect_count"]


def test_closed_form_centroid_case():
    """Two blocks, D = 4, all content in dimension 0 (scale = 1/2).

    Query rows alternate x in {0.5, 1.5} (block mean 1).  Block-0 keys
    alternate {1, 3} (mean 2) with v = e_0; block-1 keys alternate {0, 1}
    (mean 0.5) with v = 0.  Scores are 2 and 0.5: mean 1.25, std 0.75,
    tau = 1 gives thr = 2, so block 0 is exact and block 1 goes through its
    centroid.  Output dim 0 for a row with query x is E0 / (E0 + C1) with
    E0 = 32 e^{x/2} + 32 e^{3x/2} and C1 = 64 e^{x/4} (log-mass log 64)."""
    N, D = 128, 4
    q = np.zeros((1, N, 1, D))
    k = np.zeros((1, N, 1, D))
    v = np.zeros((1, N, 1, D))
    xs = np.where(np.arange(N) % 2 == 0, 0.5, 1.5)
    q[0, :, 0, 0] = xs
    k[0, :64, 0, 0] = np.where(np.arange(64) % 2 == 0, 1.0, 3.0)
    k[0, 64:, 0, 0] = np.where(np.arange(64) % 2 == 0, 0.0, 1.0)
    v[0, :64, 0, 0] = 1.0
    out, info = O.forward(q, k, v, tau=1.0)
    assert info["sel"][0, 0].tolist() == [[True, False], [True, False]]
    E0 = 32 * np.exp(xs / 2) + 32 * np.exp(1.5 * xs)
    C1 = 64 * np.exp(xs / 4)
    np.testing.assert_allclose(out[0, :, 0, 0], E0 / (E0 + C1), rtol=1e-14, atol=0)
    assert np.all(out[0, :, 0, 1:] == 0)


# ------------------------------------------------------------------- invariants


def test_tau_monotone_nesting():
    q, k, v = inputs.clustered(1, 1024, 3, 64, seed=2)
    qb, kb = O.pool(_f64(q)), O.pool(_f64(k))
    S = O.block_scores(qb, kb)
    prev = None
    for tau in [-1.0, 0.0, 0.5, 1.0, 1.5, 3.0]:
        sel = O.route(S, tau=tau)["sel"]
        if prev is not None:
            assert not (sel & ~prev).any()
        prev = sel


def test_topk_counts_with_sink():
    q, k, v = _rand(1, 1000, 2, 64, seed=4)
    S = O.block_scores(O.pool(q), O.pool(k))
    nb = S.shape[-1]
    r = O.route(S, topk_ratio=0.2, prefix_len=130)
    kk = O.topk_count(0.2, nb)
    pb = 3
    sel = r["sel"]
    assert sel[:, :, :pb].all()
    for a in range(pb, nb):
        cnt = sel[0, :, a].sum(axis=-1)
        topk_only = O.route(S, topk_ratio=0.2)["sel"][0, :, a]
        extra = (~topk_only[:, :pb]).sum(axis=-1)
        np.testing.assert_array_equal(cnt, kk + extra)


def test_output_inside_value_hull_and_prefix_rows_dense():
    q, k, v = _rand(1, 300, 2, 64, seed=8)
    out, _ = O.forward(q, k, v, tau=1.0, prefix_len=100)
    lo = v.min(axis=1, keepdims=True)
    hi = v.max(axis=1, keepdims=True)
    assert (out >= lo - 1e-12).all() and (out <= hi + 1e-12).all()
    dense = dense_reference(q, k, v)
    np.testing.assert_allclose(out[:, :128], dense[:, :128], atol=1e-12)
    assert np.abs(out[:, 128:] - dense[:, 128:]).max() > 1e-6


def test_centroid_never_overcounts_block_mass():
    """Jensen: n_c exp(q . kbar_c s) <= sum_j exp(q . k_j s).  With V = the
    indicator of block c, output dim 0 is block c's share of the softmax mass,
    which must not grow when c moves from the exact to the centroid path."""
    q, k, v = _rand(1, 256, 1, 64, seed=12)
    c = 2
    v = np.zeros_like(v)
    v[:, c * 64 : (c + 1) * 64, :, 0] = 1.0
    nb = 4
    exact = np.ones((1, 1, nb, nb), dtype=bool)
    approx = exact.copy()
    approx[..., c] = False
    o_exact, _ = O.forward(q, k, v, mask=exact)
    o_approx, _ = O.forward(q, k, v, mask=approx)
    assert (o_approx[..., 0] <= o_exact[..., 0] + 1e-15).all()
    assert (o_approx[..., 0] < o_exact[..., 0]).mean() > 0.99


def test_block_permutation_equivariance():
    q, k, v = inputs.clustered(1, 512, 2, 64, seed=6)
    q, k, v = _f64(q), _f64(k), _f64(v)
    out, info = O.forward(q, k, v, tau=1.0)
    perm = np.array([3, 0, 7, 5, 1, 6, 2, 4])
    rows = (perm[:, None] * 64 + np.arange(64)[None]).reshape(-1)
    k2, v2 = k[:, rows], v[:, rows]
    out2, info2 = O.forward(q, k2, v2, tau=1.0)
    np.testing.assert_array_equal(info2["sel"], info["sel"][..., perm])
    np.testing.assert_allclose(out2, out, atol=1e-12)


def test_selection_lists_are_ascending():
    q, k, v = _rand(1, 640, 2, 64, seed=1)
    _, info = O.forward(q, k, v, tau=0.8)
    lists, counts = O.selection_lists(info["sel"])
    for h in range(2):
        for a in range(10):
            idx = lists[0, h, a, : counts[0, h, a]]
            assert (np.diff(idx) > 0).all()
            assert (lists[0, h, a, counts[0, h, a]:] == -1).all()


def test_tiny_iid_density_is_about_one_sigma_tail():
    """For i.i.d. inputs the scores of a row are roughly normal, so tau = 1
    keeps about P(Z >= 1) = 0.159 of the blocks (a sanity range, not a pin)."""
    w = inputs.make_workload("tiny")
    q, k = _f64(w.q), _f64(w.k)
    S = O.block_scores(O.pool(q), O.pool(k))
    d = O.route(S, tau=1.0)["sel"].mean()
    assert 0.10 < d < 0.22


# ----------------------------------------------------------------- generators


def test_bf16_rounding_matches_torch():
    import torch

    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37
    x[:4] = [1.0 + 2**-8, 1.0 + 3 * 2**-8, -(1.0 + 2**-8), 0.0]  # ties
    mine = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)


def test_generators_are_seeded_and_shaped():
    a = inputs.make_workload("tiny")
    b = inputs.make_workload("tiny")
    assert a.q.shape == (1, 1024, 2, 64) and a.q.dtype == np.uint16
    np.testing.assert_array_equal(a.q, b.q)
    c = inputs.clustered(1, 512, 2, 64, seed=1)
    assert c[0] is c[1]  # Q = K
    h = inputs.h3_joint(1, 1100, 2, 64, prefix_len=64, seed=4)
    assert h[0].shape == (1, 1100, 2, 64)
    assert not np.array_equal(h[0][:, :64], h[1][:, :64])  # independent prefix
    np.testing.assert_array_equal(h[0][:, 64:], h[1][:, 64:])  # Q = K on video rows


def test_exact_kv_mode_changes_only_prefix_rows():
    """exact_kv (prefix_rows=False) differs from exact_kv_and_rows only on
    query blocks that hold prefix rows; there the list is the rows' own
    routing plus the sink, and with no prefix the two modes coincide."""
    rng = np.random.default_rng(11)
    S = rng.standard_normal((2, 3, 12, 12))
    for kw in (dict(tau=1.0), dict(topk_ratio=0.25)):
        a = O.route(S, prefix_len=130, **kw)["sel"]
        b = O.route(S, prefix_len=130, prefix_rows=False, **kw)["sel"]
        plain = O.route(S, **kw)["sel"]
        pb = 3
        np.testing.assert_array_equal(a[:, :, pb:], b[:, :, pb:])
        assert a[:, :, :pb].all()
        want = plain[:, :, :pb].copy()
        want[..., :pb] = True
        np.testing.assert_array_equal(b[:, :, :pb], want)
        np.testing.assert_array_equal(O.route(S, prefix_rows=False, **kw)["sel"], plain)


# ------------------------------------------------------------- Spark-Reweight


def test_reweight_equal_keys_reduce_to_log_mass():
    """A block whose keys are all equal has uniform anchor weights: the
    weighted summaries are the means and the bias is log(n_c), so reweight
    mode gives exactly the default (mean pooling + log-mass) output."""
    rng = np.random.default_rng(21)
    B, N, H, D = 1, 200, 2, 64
    q = rng.standard_normal((B, N, H, D))
    kb = rng.standard_normal((B, (N + 63) // 64, H, D))
    k = np.repeat(kb, 64, axis=1)[:, :N]
    v = rng.standard_normal((B, N, H, D))
    for kw in (dict(tau=1.0), dict(topk_ratio=0.5, prefix_len=30)):
        a, _ = O.forward(q, k, v, **kw)
        b, info = O.forward(q, k, v, reweight=True, **kw)
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)
        want = np.broadcast_to(np.log(O.block_sizes(N)), info["cbias"].shape)
        np.testing.assert_allclose(info["cbias"], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("prefix_len", [0, 70])
def test_reweight_is_exact_for_the_anchor_query(prefix_len):
    """For the anchor query itself (the mean of the rows >= prefix_len), the
    reweighted centroid of a block carries that block's exact mass and
    exact attention-weighted value, so dropping blocks to their centroids
    leaves the anchor row's output unchanged.  The prefix rows are placed far
    from the anchor so that an anchor taken over all rows would fail."""
    rng = np.random.default_rng(22)
    B, N, H, D = 1, 300, 1, 64
    t_star = 150
    a = rng.standard_normal(D) * 0.8
    delta = rng.standard_normal((N, D))
    delta[:prefix_len] += 6.0  # prefix rows: not part of the anchor
    video = [t for t in range(prefix_len, N) if t != t_star]
    delta[video] -= delta[video].mean(axis=0)
    delta[t_star] = 0.0
    q = (a[None, :] + delta)[None, :, None, :]
    k = rng.standard_normal((B, N, H, D))
    v = rng.standard_normal((B, N, H, D))
    nb = (N + 63) // 64
    full = np.ones((B, H, nb, nb), dtype=bool)
    part = full.copy()
    part[..., 1::2] = False  # half of the key blocks only through centroids
    ref, _ = O.forward(q, k, v, mask=full, reweight=True, prefix_len=prefix_len)
    got, info = O.forward(q, k, v, mask=part, reweight=True, prefix_len=prefix_len)
    np.testing.assert_allclose(info["anchor"][0, 0], a, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[0, t_star, 0], ref[0, t_star, 0], rtol=0, atol=1e-10)
    # other rows do change: the centroid is exact for the anchor only
    assert np.abs(got[0, 0, 0] - ref[0, 0, 0]).max() > 1e-6


def test_reweight_bias_is_the_weight_entropy():
    """bias = logsumexp(x) - sum_j w_j x_j with w = softmax(x) is the entropy
    of w: between 0 and log(n_c)."""
    q, k, v = _rand(1, 300, 2, 64, seed=23)
    _, kt, vt, cb = O.reweight_summaries(q * 2.0, k, v, prefix_len=10)
    n = O.block_sizes(300)
    assert (cb >= -1e-12).all()
    assert (cb <= np.log(n)[None, None, :] + 1e-12).all()
    assert np.isfinite(kt).all() and np.isfinite(vt).all()


# ------------------------------------------------------------- INT8 QK^T


def test_int8_equal_keys_are_exact():
    """Blocks of identical (bf16) keys have a zero residual: every code and
    block scale is 0 and the bf16 mean is the key itself, so the INT8 logits
    equal the exact ones and the forward output does not change."""
    rng = np.random.default_rng(31)
    B, N, H, D = 1, 200, 2, 64
    q, _, v = _rand(B, N, H, D, seed=31)
    kb = _f64(inputs.f32_to_bf16_bits(rng.standard_normal((B, 4, H, D)).astype(np.float32)))
    k = np.repeat(kb, 64, axis=1)[:, :N]
    codes = O.int8_qk_codes(q, k)
    assert (codes["kcode"] == 0).all() and (codes["kscale"] == 0).all()
    np.testing.assert_array_equal(codes["kbase"], kb.transpose(0, 2, 1, 3))
    for kw in (dict(tau=1.0), dict(tau=-math.inf)):
        a, _ = O.forward(q, k, v, **kw)
        b, _ = O.forward(q, k, v, int8_qk=True, **kw)
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)


def test_int8_codes_round_to_nearest():
    """Codes times scale reconstruct the residual (and q) to half a step;
    the largest code of every block (and of every query row) is 127; the
    base is the fp64 block mean to within one bf16 rounding; rows past N
    carry no code."""
    q, k, _ = _rand(1, 200, 3, 64, seed=32)
    c = O.int8_qk_codes(q, k)
    nb, sizes = O.num_blocks(200), O.block_sizes(200)
    mean = O.pool(k)  # [B, H, nb, D]
    assert (np.abs(c["kbase"] - mean) <= 2.0**-8 * np.abs(mean) + 1e-6).all()
    for b in range(1):
        for h in range(3):
            for j in range(nb):
                rows = slice(64 * j, 64 * j + sizes[j])
                r = k[b, rows, h] - c["kbase"][b, h, j]
                s = float(c["kscale"][b, h, j])
                code = c["kcode"][b, rows, h].astype(np.float64)
                assert s > 0 and np.abs(code).max() == 127
                assert (np.abs(code * s - r) <= 0.5 * s * (1 + 1e-5)).all()
                np.testing.assert_allclose(np.abs(r).max(), 127 * s, rtol=1e-6)
    qs = c["qscale"][..., None].astype(np.float64)
    assert (np.abs(c["qcode"] * qs - q) <= 0.5 * qs * (1 + 1e-5)).all()
    assert (np.abs(c["qcode"]).max(axis=3) == 127).all()


def test_int8_logit_error_bound():
    """q.k = q.base + q.r exactly, so the INT8 logit differs from the exact
    one only by the rounding of q and r:
    |err| <= |q|_1 s_c / 2 + |r|_1 s_q / 2 + D s_q s_c / 4.  The error is
    not zero (the quantisation is really applied)."""
    q, k, _ = _rand(1, 256, 2, 64, seed=33)
    c = O.int8_qk_codes(q, k)
    worst = 0.0
    for h in range(2):
        hd = {key: (c[key][0, :, h] if key in ("qcode", "qscale", "kcode") else c[key][0, h]) for key in c}
        keys = np.arange(256)
        rows = slice(0, 64)
        got = O.int8_logits(q[0, rows, h], keys, dict(hd, qcode=hd["qcode"][rows], qscale=hd["qscale"][rows]))
        exact = q[0, rows, h] @ k[0, :, h].T
        blk = keys // 64
        r = k[0, :, h] - c["kbase"][0, h][blk]
        sq = c["qscale"][0, rows, h].astype(np.float64)[:, None]
        sk = c["kscale"][0, h].astype(np.float64)[blk][None, :]
        bound = (np.abs(q[0, rows, h]).sum(1)[:, None] * sk / 2 + np.abs(r).sum(1)[None, :] * sq / 2
                 + 64 * sq * sk / 4)
        err = np.abs(got - exact)
        assert (err <= bound * (1 + 1e-9) + 1e-12).all()
        worst = max(worst, float(err.max()))
    assert worst > 1e-4


def test_int8_residual_beats_full_key_quantisation():
    """The pages compare the residual design with quantising whole keys and
    find it several times closer to the exact path.  On clustered video-like
    inputs the oracle's residual variant must be closer to the exact output
    than the whole-key variant, and within a few percent of it."""
    q, k, v = (_f64(x) for x in inputs.clustered(1, 1024, 2, 64, seed=34))
    ref, info = O.forward(q, k, v, tau=1.0)
    base = {key: info[key] for key in ("qbar", "kbar", "vbar", "sel")}
    res, _ = O.forward(q, k, v, tau=1.0, int8_qk=True, info=dict(base))
    full, _ = O.forward(q, k, v, tau=1.0, int8_qk=True, info=dict(base, int8=O.int8_qk_codes(q, k, residual=False)))

    def rel(x):
        return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))

    print(f"relative L2: residual {rel(res):.4f}, whole keys {rel(full):.4f}")
    assert 0 < rel(res) < 0.03
    assert rel(res) < rel(full)


# ------------------------------------------------------------- Spark-Reblock


def test_reblock_metric_is_score_pattern_cosine():
    """u_i^T M u_j with M = K^T K is the cosine of the score patterns K q_i
    and K q_j, computed here directly over all keys."""
    rng = np.random.default_rng(41)
    x = rng.standard_normal((20, 16))
    other = rng.standard_normal((300, 16))
    u, M = O.mahalanobis_units(x, other)
    S = x @ other.T  # score patterns
    cos = (S @ S.T) / np.outer(np.linalg.norm(S, axis=1), np.linalg.norm(S, axis=1))
    np.testing.assert_allclose(u @ M @ u.T, cos, rtol=0, atol=1e-12)


def test_pivot_split_hand_example():
    """Four unit rows with M = I, leaning towards (1, 0): the row least
    similar to the mean direction is (0, 1); the row least similar to it is
    (1, 0); ranking by u . ((1, 0) - (0, 1)) puts the two rows nearer (0, 1)
    in the left child."""
    c1, c3 = 1 / math.sqrt(0.82), 1 / math.sqrt(0.68)
    u = np.array([[1.0, 0.0], [0.9 * c1, 0.1 * c1], [0.0, 1.0], [0.2 * c3, 0.8 * c3]])
    a, b, p, left = O.pivot_split(u, np.eye(2), 2)
    assert (a, b) == (2, 0)
    np.testing.assert_allclose(p, [1.0, 0.8 * c1, -1.0, -0.6 * c3], atol=1e-12)
    assert left.tolist() == [False, False, True, True]
    # a metric that stretches the second axis changes the similarities
    a2, b2, _, _ = O.pivot_split(u, np.diag([1.0, 9.0]), 2)
    assert (a2, b2) != (a, b) or not np.allclose(O.pivot_split(u, np.diag([1.0, 9.0]), 2)[2], p)


def test_reblock_recovers_planted_clusters():
    """Queries drawn tightly around four directions (two blocks each) in
    shuffled positions, keys around four other directions with the same
    labels by position: in the shared layout (q_reuse_k) every block holds
    one cluster of queries and, since the keys reuse the query partition,
    one cluster of keys; the prefix rows stay in place.  In the separate
    layout the keys, labelled independently, get pure blocks of their own."""
    rng = np.random.default_rng(42)
    B, N, H, D, pre = 1, 64 + 512, 1, 32, 64
    cq, ck = rng.standard_normal((4, D)), rng.standard_normal((4, D))
    lab = np.repeat(np.arange(4), 128)
    rng.shuffle(lab)
    q = rng.standard_normal((B, N, H, D))
    q[0, pre:, 0] = cq[lab] + 0.02 * rng.standard_normal((512, D))
    k = rng.standard_normal((B, N, H, D))
    k[0, pre:, 0] = ck[lab] + 0.02 * rng.standard_normal((512, D))
    pq, pk = O.reblock_orders(q, k, prefix_len=pre)
    assert (pk == pq).all()
    assert (pq[0, 0, :pre] == np.arange(pre)).all()
    assert sorted(pq[0, 0].tolist()) == list(range(N))
    for blk in (pq[0, 0, pre:] - pre).reshape(8, 64):
        assert len(set(lab[blk].tolist())) == 1
    labk = lab.copy()
    rng.shuffle(labk)
    k[0, pre:, 0] = ck[labk] + 0.02 * rng.standard_normal((512, D))
    pq2, pk2 = O.reblock_orders(q, k, prefix_len=pre, layout="separate")
    assert (pk2[0, 0, :pre] == np.arange(pre)).all()
    for perm, lb in ((pq2, lab), (pk2, labk)):
        assert sorted(perm[0, 0].tolist()) == list(range(N))
        for blk in (perm[0, 0, pre:] - pre).reshape(8, 64):
            assert len(set(lb[blk].tolist())) == 1


def test_reblock_q_reuse_k_shares_the_query_partition():
    """reblock_layout=q_reuse_k (Spark-H3 news, 워크플로 section): the keys and
    values take the partition made for the queries (in M = K^T K), which is
    also the separate layout's query partition; the separate layout's own key
    partition (in M = Q^T Q) differs on generic inputs."""
    q, k, v = _rand(2, 64 + 700, 2, 32, seed=46)
    pq, pk = O.reblock_orders(q, k, prefix_len=64)
    sq, sk = O.reblock_orders(q, k, prefix_len=64, layout="separate")
    assert (pk == pq).all() and (sq == pq).all()
    assert not (sk == pq).all()
    a, info = O.forward(q, k, v, tau=1.0, prefix_len=64, reblock=True)
    assert (info["perm_k"] == info["perm_q"]).all()
    with pytest.raises(ValueError):
        O.reblock_orders(q, k, layout="k_reuse_q")


def test_reblock_leaves_do_not_depend_on_row_order():
    """Shuffling the rows after the prefix permutes the input but leaves the
    partition (as sets of rows) unchanged: the split of a group depends only
    on its set of rows (continuous data, no ties)."""
    q, k, _ = _rand(1, 64 + 640, 2, 32, seed=43)
    pre = 64
    pq, pk = O.reblock_orders(q, k, prefix_len=pre)
    rng = np.random.default_rng(44)
    sh = np.concatenate([np.arange(pre), pre + rng.permutation(640)])
    pq2, pk2 = O.reblock_orders(q[:, sh], k[:, sh], prefix_len=pre)
    for p1, p2 in ((pq, pq2), (pk, pk2)):
        for h in range(2):
            a = {frozenset(bl) for bl in p1[0, h, pre:].reshape(10, 64).tolist()}
            bset = {frozenset(sh[bl].tolist()) for bl in p2[0, h, pre:].reshape(10, 64)}
            assert a == bset


def test_reblock_keeps_dense_attention_and_changes_routed():
    """Dense attention does not depend on the row order, so reblocking leaves
    it unchanged; routed attention with centroids does change."""
    q, k, v = _rand(1, 300, 2, 32, seed=45)
    a, _ = O.forward(q, k, v, tau=-math.inf)
    b, info = O.forward(q, k, v, tau=-math.inf, reblock=True, prefix_len=70)
    np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)
    assert not (info["perm_q"][0, 0] == np.arange(300)).all()
    c, _ = O.forward(q, k, v, tau=1.0, prefix_len=70)
    d, _ = O.forward(q, k, v, tau=1.0, prefix_len=70, reblock=True)
    assert np.abs(c - d).max() > 1e-3
