"""The seeded input recipes, pinned on the CPU.

The generators are the one module the HIP path and the oracle share, so
what they draw is part of every parity claim.  These tests fix the draw
order and the statistics that the module docstring states for each recipe:
which draws are shared between recipes, the element variances, the
row-to-row correlation of the smooth signal and the per-block structure that
makes routing content-dependent."""

import math

import numpy as np
import pytest

from block_sparse_video_fp32_amd import inputs


def _f64(bits):
    return inputs.bf16_bits_to_f32(bits).astype(np.float64)


def test_h3_prefix_is_the_iid_draws():
    """The prefix rows of Q, K and V are the first three N(0,1) draws of the
    seed, in that order, exactly as the i.i.d. recipe draws them."""
    B, N, H, D, P = 1, 1500, 2, 64, 128
    q, k, v = inputs.h3_joint(B, N, H, D, prefix_len=P, seed=9)
    iq, ik, iv = inputs.iid(B, P, H, D, seed=9)
    np.testing.assert_array_equal(q[:, :P], iq)
    np.testing.assert_array_equal(k[:, :P], ik)
    np.testing.assert_array_equal(v[:, :P], iv)


def test_soft_variants_share_the_signal_and_query_noise():
    """clustered_soft and h3_joint(shared_qk=False) draw the same periods,
    phases and query noise as their shared-key recipes before the key noise,
    so at the default amplitude their queries are bit-identical."""
    q, k, _ = inputs.clustered(1, 1024, 2, 64, seed=5)
    qs, ks, _ = inputs.clustered_soft(1, 1024, 2, 64, seed=5, amp=1.5)
    np.testing.assert_array_equal(qs, q)
    assert not np.array_equal(ks, k)
    h = inputs.h3_joint(1, 1200, 2, 64, prefix_len=64, seed=3)
    hs = inputs.h3_joint(1, 1200, 2, 64, prefix_len=64, seed=3, shared_qk=False)
    np.testing.assert_array_equal(hs[0], h[0])
    np.testing.assert_array_equal(hs[1][:, :64], h[1][:, :64])
    assert not np.array_equal(hs[1][:, 64:], h[1][:, 64:])


def test_iid_moments():
    q, k, v = (_f64(x) for x in inputs.iid(1, 4096, 2, 64, seed=11))
    for x in (q, k, v):
        assert abs(x.mean()) < 0.01
        assert abs(x.var() - 1.0) < 0.02
    assert abs(np.corrcoef(q.ravel(), k.ravel())[0, 1]) < 0.01


def test_clustered_moments_and_smoothness():
    """Q = 1.5 s + N(0,1) with a unit-variance signal: element variance
    1.5^2 + 1 = 3.25.  The signal's periods are at least 256 rows, so
    neighbouring rows share it almost fully: their correlation is close to
    2.25 / 3.25.  V is N(0,1) and carries no signal."""
    q, k, v = (_f64(x) for x in inputs.clustered(1, 8192, 2, 64, seed=12))
    assert abs(q.var() - 3.25) < 0.25
    assert abs(v.var() - 1.0) < 0.02
    a = q[0, :-1].ravel()
    b = q[0, 1:].ravel()
    assert abs(np.corrcoef(a, b)[0, 1] - 2.25 / 3.25) < 0.03
    assert abs(np.corrcoef(v[0, :-1].ravel(), v[0, 1:].ravel())[0, 1]) < 0.01


def test_clustered_block_means_carry_the_signal():
    """64-row block means: noise alone leaves a variance of 1/64 per
    coordinate (the i.i.d. recipe), the smooth signal leaves about 1.5^2 of
    it, so neighbouring blocks differ in content and routing has something
    to select."""
    N, H, D = 8192, 2, 64
    qc = _f64(inputs.clustered(1, N, H, D, seed=13)[0])[0]
    qi = _f64(inputs.iid(1, N, H, D, seed=13)[0])[0]
    mc = qc.reshape(N // 64, 64, H, D).mean(axis=1)
    mi = qi.reshape(N // 64, 64, H, D).mean(axis=1)
    assert abs(mi.var() - 1.0 / 64) < 0.003
    assert mc.var() > 1.5


def test_h3_video_rows_follow_the_grid():
    """Video rows: Q = 1.5 s + N(0,1) with s a unit-variance sum of sines
    over (frame, y, x); element variance about 3.25.  The periods are at
    most 32 grid steps, so rows one frame apart (24 x 42 rows) stay
    correlated while shuffled rows do not."""
    B, H, D, P = 1, 2, 64, 64
    frame = 24 * 42
    N = P + 6 * frame
    q, k, v = inputs.h3_joint(B, N, H, D, prefix_len=P, seed=14)
    qv = _f64(q)[0, P:]
    assert abs(qv.var() - 3.25) < 0.3
    assert abs(_f64(v)[0, P:].var() - 1.0) < 0.03
    x = qv - qv.mean(axis=0)
    noise_only = 1.0 / 3.25
    shuf = np.random.default_rng(0).permutation(len(x))
    r_shuf = np.corrcoef(x.ravel(), x[shuf].ravel())[0, 1]
    assert abs(r_shuf) < 0.02
    # The signal at lag one frame keeps the (y, x) phase and moves f by 1:
    # per channel the lag correlation of s is sum_j cos(2 pi / Pf_j) / 4.
    # With ln Pf uniform on [ln 2, ln 32] the mean of cos(2 pi / Pf) is
    # (1 / ln 16) * integral of cos(2 pi / P) / P dP, taken here by the
    # midpoint rule; Q's correlation is that times 2.25 / 3.25.
    lo, hi = math.log(2.0), math.log(32.0)
    u = lo + (np.arange(100000) + 0.5) * (hi - lo) / 100000
    expect = np.cos(2 * math.pi / np.exp(u)).mean() * 2.25 / 3.25
    r_frame = np.corrcoef(x[:-frame].ravel(), x[frame:].ravel())[0, 1]
    assert abs(r_frame - expect) < 0.08
    assert r_frame < 1.0 - noise_only


@pytest.mark.parametrize("name", ["tiny"])
def test_make_workload_overrides(name):
    w = inputs.make_workload(name, H=1, N=256, tau=float("-inf"))
    assert w.q.shape == (1, 256, 1, 64)
    assert w.params()["tau"] == float("-inf")
    assert w.params()["prefix_len"] == 0
    base = inputs.make_workload(name)
    assert base.tau == 1.0 and base.topk_ratio is None
    with pytest.raises(ValueError):
        inputs.make_workload(name, kind="nope")


def test_named_problem_sizes():
    """The named problems keep the sizes the package is measured on."""
    c = inputs.CONFIGS
    for name in ("n4k", "n16k", "n32k"):
        assert (c[name]["B"], c[name]["H"], c[name]["D"]) == (1, 56, 128)
        assert c[name]["kind"] == "clustered" and c[name]["tau"] == 1.0
    assert [c[n]["N"] for n in ("n4k", "n16k", "n32k")] == [4096, 16384, 32768]
    h = c["h3"]
    assert (h["N"], h["H"], h["D"], h["prefix_len"], h["topk_ratio"]) == (38247, 56, 128, 1024, 0.1)
    assert math.ceil(h["N"] / 64) == 598
