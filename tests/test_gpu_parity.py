"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bars:
* pooled means: fp32 sums of 64 bf16 rows against the fp64 means, within
  the fp32 summation bound (64 * 2^-24 * mean |x| per element, x2 slack);
* selected-block lists: bit-exact against the oracle's routing, except
  blocks within 1e-4 standard deviations of the row's cut (the tau
  threshold, or in top-K mode the midpoint between the k-th and (k+1)-th
  scores), which must be under 0.1% of all blocks of the call;
* output, computed by the oracle on the GPU's own lists: max-abs <= 2e-2,
  mean-abs <= 2e-3, cosine >= 0.9995 (bf16 output vs fp64).

Small problems are compared on every output row; the large workloads
(N = 16384 / 32768 / 38247, H = 56, D = 128) route every row and compare
sampled query blocks (plus the tail and prefix blocks) one by one, in the
launch configuration the benchmark times.
"""

import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_sparse_video_fp32_amd import binding, inputs
from oracle import sol_oracle as O

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, MIN_COS = 2e-2, 2e-3, 0.9995
BAND_SIGMA, BAND_MAX_FRAC = 1e-4, 1e-3


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _f32(bits):
    return inputs.bf16_bits_to_f32(bits)


class GpuRun:
    """One forward through the C ABI; keeps the workspace for inspection."""

    def __init__(self, q, k, v, strides=None, **kw):
        dev = _dev()
        B, N, H, D = q.shape
        self.plan = binding.SparseAttnPlan(B, N, H, D, **kw)
        self.q, self.k, self.v = (inputs.to_torch_bf16(x, dev) for x in (q, k, v))
        self.out = torch.empty_like(self.q)
        self.ws = self.plan.workspace(dev)
        self.plan.forward(self.q, self.k, self.v, out=self.out, ws=self.ws)
        torch.cuda.synchronize()
        print(f"  gpu forward done: B={B} N={N} H={H} D={D} {kw}", flush=True)

    def out_f64(self):
        return self.out.float().cpu().numpy().astype(np.float64)

    def selection(self):
        return selection_from(*self.plan.route_views(self.ws))


def selection_from(counts, lists):
    """bool [B, H, n_b, n_b] from the library's counts and lists (checked:
    counts in range, entries valid, ascending and distinct)."""
    counts = counts.cpu().numpy()
    lists = lists.cpu().numpy()
    B, H, nb = counts.shape
    assert ((counts >= 0) & (counts <= nb)).all()
    valid = np.arange(nb)[None, None, None, :] < counts[..., None]
    ent = np.where(valid, lists, -1)
    assert ((ent[valid] >= 0) & (ent[valid] < nb)).all()
    # ascending and distinct within each list
    d = np.diff(np.where(valid, lists, np.iinfo(np.int32).max), axis=-1)
    vv = valid[..., 1:]
    assert (d[vv] > 0).all()
    sel = np.zeros((B, H, nb, nb), dtype=bool)
    bb, hh, aa, jj = np.nonzero(valid)
    sel[bb, hh, aa, lists[bb, hh, aa, jj]] = True
    return sel


def check_route(sel_gpu, info, dense_rows_from=0):
    """Lists equal the oracle's except blocks within 1e-4 standard
    deviations of their row's cut (|S - cut| <= 1e-4 sigma, the row's
    population std of block scores).  The blocks this excuses (in the band
    and different) must be under 0.1% of all blocks of the call (B H n_b^2)
    where the call has at least 1000 blocks; the band itself must be under
    0.1% where the call has at least 10^4 blocks.  Returns the band's share."""
    ref = info["sel"]
    S, thr, sigma = info.get("S"), info["cut"], info["sigma"]
    diff = sel_gpu != ref
    if S is None:
        assert not diff.any()
        return 0.0
    routed = ~np.isnan(thr) & np.isfinite(thr)
    band = np.abs(S - thr[..., None]) <= (BAND_SIGMA * sigma)[..., None]
    band &= routed[..., None]
    bad = diff & ~band
    frac = band.sum() / S.size
    excused = int((diff & band).sum())
    assert not bad.any(), f"{int(bad.sum())} selection mismatches outside the band, first at {np.argwhere(bad)[:5]}"
    # Below 1000 blocks 0.1% is less than one block (a lone block always
    # sits at its own row's cut in top-K mode).  On continuous scores about
    # 1e-4 of the blocks fall within 1e-4 sigma of a cut by chance, so on
    # calls under 10^4 blocks one or two chance near-ties already exceed a
    # 0.1% bar on the band itself; there the bar bounds what it excuses.
    if S.size >= 1000:
        assert excused < BAND_MAX_FRAC * S.size, f"{excused} in-band mismatches of {S.size} blocks"
    if S.size >= 10000:
        assert frac < BAND_MAX_FRAC, f"band holds {frac:.2e} of all blocks"
    return frac


def metrics(got, ref):
    err = np.abs(got - ref)
    cos = float((got * ref).sum() / math.sqrt((got * got).sum() * (ref * ref).sum()))
    return float(err.max()), float(err.mean()), cos


def check_output(got, ref, label=""):
    mx, mean, cos = metrics(got, ref)
    print(f"  {label} max-abs {mx:.3e} mean-abs {mean:.3e} cos {cos:.7f}", flush=True)
    assert np.isfinite(got).all()
    assert mx <= MAX_ABS and mean <= MEAN_ABS and cos >= MIN_COS, (mx, mean, cos)


def oracle_kw(kw):
    o = {k: kw[k] for k in ("tau", "topk_ratio", "prefix_len", "centroid", "logmass", "reweight", "int8_qk",
                            "sm_scale") if k in kw}
    if kw.get("exact_kv_only"):
        o["prefix_rows"] = False  # exact_kv: the sink without dense prefix rows
    return o


def full_parity(q, k, v, **kw):
    run = GpuRun(q, k, v, **kw)
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    okw = oracle_kw(kw)
    _, info = O.forward_blocks(qf, kf, vf, [], **okw)
    dense = run.plan.dense
    if not dense:
        sel = run.selection()
        check_route(sel, info)
    else:
        sel = info["sel"]
    ref, _ = O.forward(qf, kf, vf, info=dict(info, sel=sel), **okw)
    check_output(run.out_f64(), ref, f"N={q.shape[1]} {kw}")
    return run, info


# ----------------------------------------------------------------- pooling


def _kappa(r):
    return (r & 7) | ((r & 8) << 1) | ((r & 16) >> 1)


def _unpack_k(tile, D):
    """Packed K half tile (32*D,) -> [32, D] per the order in sparse_attn.h:
    element ((m*64 + l)*8 + e) is K[kappa(l % 32)][16 m + 8 (l // 32) + e]."""
    t = tile.reshape(D // 16, 2, 32, 8)  # [m, l // 32, l % 32, e]
    k = np.empty((32, D), dtype=tile.dtype)
    for r in range(32):
        k[_kappa(r)] = t[:, :, r, :].reshape(D)  # d = 16 m + 8 (l // 32) + e
    return k


def _unpack_vt(tile, D):
    """Packed V^T half tile (32*D,) -> V [32 keys, D]: element
    ((m*64 + l)*8 + e), m = 2 dt + j, is
    V[16 (e // 4) + 8 j + 4 (l // 32) + e % 4][32 dt + l % 32]."""
    t = tile.reshape(D // 32, 2, 2, 32, 2, 4)  # [dt, j, l // 32, l % 32, e // 4, e % 4]
    v = np.empty((32, D), dtype=tile.dtype)
    for dt in range(D // 32):
        for j in range(2):
            for hh in range(2):
                for e4 in range(2):
                    for e0 in range(4):
                        v[16 * e4 + 8 * j + 4 * hh + e0, 32 * dt : 32 * dt + 32] = t[dt, j, hh, :, e4, e0]
    return v


@pytest.mark.parametrize("N,D", [(1024, 64), (200, 128), (38247 - 37 * 1024, 128)])
def test_pooled_means_and_packed_tiles(N, D):
    q, k, v = inputs.iid(2, N, 3, D, seed=N)
    run = GpuRun(q, k, v, tau=1.0)
    qb, kb, vb = (t.float().cpu().numpy() for t in run.plan.pooled_views(run.ws))
    for got, x in ((qb, q), (kb, k), (vb, v)):
        xf = _f32(x).astype(np.float64)
        ref = O.pool(xf)
        bound = 2 * 64 * 2.0**-24 * np.abs(xf).max()
        assert np.abs(got - ref).max() <= bound
    kp, vp, kbp, vbp = (t.float().cpu().numpy() for t in run.plan.packed_views(run.ws))
    B, H, nb = qb.shape[:3]
    kf, vf = _f32(k), _f32(v)
    for b in range(B):
        for h in range(H):
            for c in (0, nb // 2, nb - 1):
                for ht in range(2):
                    rows = np.arange(c * 64 + 32 * ht, c * 64 + 32 * ht + 32)
                    want_k = np.where((rows < N)[:, None], kf[b, np.minimum(rows, N - 1), h], 0)
                    want_v = np.where((rows < N)[:, None], vf[b, np.minimum(rows, N - 1), h], 0)
                    np.testing.assert_array_equal(_unpack_k(kp[b, h, c, ht], D), want_k)
                    np.testing.assert_array_equal(_unpack_vt(vp[b, h, c, ht], D), want_v)
            # centroids: fp32 means rounded to nearest even, rows past n_b zero
            ck = np.concatenate([_unpack_k(t, D) for t in kbp[b, h]])
            cv = np.concatenate([_unpack_vt(t, D) for t in vbp[b, h]])
            np.testing.assert_array_equal(ck[:nb], _f32(inputs.f32_to_bf16_bits(kb[b, h])))
            np.testing.assert_array_equal(cv[:nb], _f32(inputs.f32_to_bf16_bits(vb[b, h])))
            assert (ck[nb:] == 0).all() and (cv[nb:] == 0).all()


@pytest.mark.parametrize("N,D,prefix_len", [(1100, 64, 100), (1024, 128, 0), (300, 128, 300), (777, 128, 128)])
def test_reweight_summaries(N, D, prefix_len):
    """Anchor, centroid bias and the packed Ktilde / Vtilde centroids against
    the oracle's fp64 summaries; the fp32 means stay the block means."""
    q, k, v = inputs.clustered(2, N, 2, D, seed=N + D) if N >= 256 else inputs.iid(2, N, 2, D, seed=N)
    run = GpuRun(q, k, v, tau=1.0, prefix_len=prefix_len, reweight=True)
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    anchor, kt, vt, cb = O.reweight_summaries(qf, kf, vf, prefix_len=prefix_len)
    ga, gcb = (t.cpu().numpy().astype(np.float64) for t in run.plan.reweight_views(run.ws))
    nb = O.num_blocks(N)
    # fp32 block sums then a sum over blocks: (64 + n_b) roundings of |q|max
    bound = 2 * (64 + nb) * 2.0**-24 * np.abs(qf).max()
    assert np.abs(ga - anchor).max() <= bound, np.abs(ga - anchor).max()
    # bias: log2 units on the GPU; fp32 dot products of length D
    err = np.abs(gcb[:, :, :nb] * math.log(2.0) - cb)
    print(f"  cbias max err {err.max():.3e}", flush=True)
    assert err.max() <= 1e-3
    assert (gcb[:, :, nb:] == 0).all()
    kb = run.plan.pooled_views(run.ws)[1].float().cpu().numpy()
    assert np.abs(kb - O.pool(kf)).max() <= 2 * 64 * 2.0**-24 * np.abs(kf).max()
    _, _, kbp, vbp = (t.float().cpu().numpy() for t in run.plan.packed_views(run.ws))
    for b in range(2):
        for h in range(2):
            ck = np.concatenate([_unpack_k(t, D) for t in kbp[b, h]])
            cv = np.concatenate([_unpack_vt(t, D) for t in vbp[b, h]])
            for got, ref in ((ck[:nb], kt[b, h]), (cv[:nb], vt[b, h])):
                # one bf16 rounding of an fp32 sum: at most one unit in the
                # last place (2^-7 relative) plus the fp32 summation error
                tol = 2.0**-7 * np.abs(ref) + 1e-4 * np.abs(ref).max()
                assert (np.abs(got - ref) <= tol).all(), np.abs(got - ref).max()
            assert (ck[nb:] == 0).all() and (cv[nb:] == 0).all()


def _unpack_k8(tile, D):
    """Packed INT8 residual half tile (32*D,) -> [32, D] per sparse_attn.h:
    byte ((t*64 + l)*16 + j) is the code of
    K[kappa(l % 32)][32 t + 16 (j // 8) + 8 (l // 32) + j % 8]."""
    t = tile.reshape(D // 32, 2, 32, 2, 8)  # [t, l // 32, l % 32, j // 8, j % 8]
    k = np.empty((32, D), dtype=tile.dtype)
    for r in range(32):
        k[_kappa(r)] = t[:, :, r].transpose(0, 2, 1, 3).reshape(D)
    return k


@pytest.mark.parametrize("N,D", [(1100, 64), (1024, 128), (200, 128)])
def test_int8_codes_match_oracle(N, D):
    """Residual codes, bf16 base rows and block scales are decided in fp32 on
    both sides: they must be bit-identical to the oracle's."""
    q, k, v = inputs.clustered(2, N, 2, D, seed=N + 7) if N >= 256 else inputs.iid(2, N, 2, D, seed=N + 7)
    run = GpuRun(q, k, v, tau=1.0, int8_qk=True)
    want = O.int8_qk_codes(_f32(q), _f32(k))
    codes, base, scale = (t.cpu() for t in run.plan.int8_views(run.ws))
    np.testing.assert_array_equal(base.float().numpy(), want["kbase"])
    np.testing.assert_array_equal(scale.numpy(), want["kscale"])
    codes = codes.numpy()
    nb = O.num_blocks(N)
    kc = np.zeros((2, nb * 64, 2, D), dtype=np.int8)
    kc[:, :N] = want["kcode"]
    for b in range(2):
        for h in range(2):
            for c in range(nb):
                for ht in range(2):
                    rows = slice(64 * c + 32 * ht, 64 * c + 32 * ht + 32)
                    np.testing.assert_array_equal(_unpack_k8(codes[b, h, c, ht], D), kc[b, rows, h])


# ---------------------------------------------------- small, every output row


SMALL = [
    ("tiny_tau1", dict(kind="tiny"), dict(tau=1.0)),
    ("tail_d64", dict(B=2, N=200, H=3, D=64), dict(tau=1.0)),
    ("tail_d128", dict(B=1, N=1000, H=2, D=128), dict(tau=1.0)),
    ("tau0", dict(B=1, N=1024, H=2, D=128), dict(tau=0.0)),
    ("tau_inf_sink", dict(B=1, N=700, H=2, D=64), dict(tau=math.inf, prefix_len=130)),
    ("topk", dict(B=1, N=1500, H=2, D=128), dict(topk_ratio=0.25)),
    ("topk_prefix", dict(B=2, N=1100, H=2, D=64), dict(topk_ratio=0.1, prefix_len=100)),
    ("prefix_tau", dict(B=1, N=1024, H=3, D=128), dict(tau=1.0, prefix_len=64)),
    ("exact_kv_tau", dict(B=1, N=1024, H=2, D=128), dict(tau=1.0, prefix_len=130, exact_kv_only=True)),
    ("exact_kv_topk", dict(B=2, N=1100, H=2, D=64), dict(topk_ratio=0.1, prefix_len=100, exact_kv_only=True)),
    ("reweight_tau", dict(B=1, N=1024, H=2, D=128), dict(tau=1.0, reweight=True)),
    ("reweight_prefix_tail", dict(B=2, N=1100, H=2, D=64), dict(tau=1.0, prefix_len=100, reweight=True)),
    ("reweight_topk", dict(B=1, N=1500, H=2, D=128), dict(topk_ratio=0.25, prefix_len=128, reweight=True)),
    ("reweight_exact_kv", dict(B=1, N=1000, H=3, D=64), dict(tau=0.5, prefix_len=70, exact_kv_only=True,
                                                              reweight=True)),
    ("reweight_dense", dict(B=1, N=777, H=2, D=128), dict(tau=-math.inf, reweight=True)),
    ("int8_tau", dict(B=1, N=1024, H=2, D=128), dict(tau=1.0, int8_qk=True)),
    ("int8_prefix_tail_d64", dict(B=2, N=1100, H=2, D=64), dict(tau=1.0, prefix_len=100, int8_qk=True)),
    ("int8_topk_reweight", dict(B=1, N=1500, H=2, D=128), dict(topk_ratio=0.25, prefix_len=128, reweight=True,
                                                                int8_qk=True)),
    ("int8_exact_kv", dict(B=1, N=1000, H=3, D=64), dict(tau=0.5, prefix_len=70, exact_kv_only=True, int8_qk=True)),
    ("int8_dense_tail", dict(B=1, N=777, H=2, D=128), dict(tau=-math.inf, int8_qk=True)),
    ("no_centroid", dict(B=1, N=1024, H=2, D=128), dict(tau=1.0, centroid=False)),
    ("no_logmass", dict(B=1, N=1024, H=2, D=64), dict(tau=1.0, logmass=False)),
    ("scale", dict(B=1, N=512, H=2, D=64), dict(tau=0.5, sm_scale=0.3)),
    ("dense_tail", dict(B=1, N=777, H=2, D=128), dict(tau=-math.inf)),
    ("dense_d64", dict(B=2, N=256, H=1, D=64), dict(tau=-math.inf)),
    ("one_row", dict(B=1, N=1, H=1, D=64), dict(tau=1.0)),
    ("one_block", dict(B=1, N=64, H=2, D=128), dict(tau=1.0)),
    # every row a prefix row: all query blocks dense through the routed path
    ("prefix_all", dict(B=1, N=300, H=2, D=64), dict(tau=1.0, prefix_len=300)),
    # every block selected by routing (no centroid tiles), not by the dense flag
    ("topk_all", dict(B=1, N=700, H=2, D=128), dict(topk_ratio=1.0)),
    ("tau_neg_huge", dict(B=1, N=777, H=2, D=64), dict(tau=-1e30)),
]


def _small_inputs(shape, seed):
    if shape.get("kind") == "tiny":
        w = inputs.make_workload("tiny")
        return w.q, w.k, w.v
    B, N, H, D = shape["B"], shape["N"], shape["H"], shape["D"]
    if N >= 256:
        return inputs.clustered(B, N, H, D, seed)
    return inputs.iid(B, N, H, D, seed)


@pytest.mark.parametrize("name,shape,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_full_parity(name, shape, kw):
    q, k, v = _small_inputs(shape, seed=len(name))
    full_parity(q, k, v, **kw)


def _spike_inputs(N, H, D, spike_block, seed):
    """Every query row and every key of one block lie along the same +-4
    vector u, so that block's logits (about 16 D * scale) exceed those of the
    first block a query sees by far more than the 2^100 headroom of the fixed
    softmax reference: the kernel must take its exact-maximum recompute."""
    rng = np.random.default_rng(seed)
    u = np.where(rng.random((1, 1, H, D)) < 0.5, -4.0, 4.0)
    q = u + 0.5 * rng.standard_normal((1, N, H, D))
    k = rng.standard_normal((1, N, H, D))
    v = rng.standard_normal((1, N, H, D))
    k[:, spike_block * 64 : (spike_block + 1) * 64] = u
    return tuple(inputs.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("tau,int8_qk", [(1.0, False), (-math.inf, False), (1.0, True)],
                         ids=["tau1", "dense", "tau1_int8"])
def test_logit_spike_recompute(D, tau, int8_qk):
    q, k, v = _spike_inputs(N=650, H=2, D=D, spike_block=5, seed=D)
    full_parity(q, k, v, tau=tau, int8_qk=int8_qk)


# The dense path (tau = -inf) has a kernel of its own at D = 64 and 128 (four
# query blocks per workgroup, 64 rows per wave).  Each of its rows does the
# same arithmetic in the same order as the routed kernel does when every
# key block is selected (top-K ratio 1: ascending exact tiles, no centroid
# tiles), so the two outputs agree bit for bit; the routed kernel is checked
# against the oracle throughout this file.

@pytest.mark.parametrize("shape", [(1, 1, 1, 128), (1, 65, 2, 128), (2, 777, 3, 128), (1, 4133, 2, 128),
                                   (1, 256, 2, 64), (2, 1100, 2, 64), (1, 6000, 1, 128)],
                         ids=lambda t: "B{}_N{}_H{}_D{}".format(*t))
def test_dense_kernel_matches_all_selected(shape):
    B, N, H, D = shape
    q, k, v = inputs.clustered_soft(B, N, H, D, seed=N) if N >= 256 else inputs.iid(B, N, H, D, seed=N)
    dense = GpuRun(q, k, v, tau=-math.inf)
    full = GpuRun(q, k, v, topk_ratio=1.0)
    assert full.selection().all()
    a, b = dense.out.view(torch.int16), full.out.view(torch.int16)
    assert torch.equal(a, b), f"{int((a != b).sum())} of {a.numel()} elements differ"


def test_tiny_matches_oracle_lists_exactly():
    w = inputs.make_workload("tiny")
    run = GpuRun(w.q, w.k, w.v, tau=1.0)
    _, info = O.forward_blocks(_f32(w.q), _f32(w.k), _f32(w.v), [], tau=1.0)
    np.testing.assert_array_equal(run.selection(), info["sel"])


def test_deterministic_reruns():
    q, k, v = inputs.clustered(1, 2048, 4, 128, seed=5)
    a = GpuRun(q, k, v, tau=1.0)
    o1 = a.out.clone()
    a.plan.forward(a.q, a.k, a.v, out=a.out, ws=a.ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), a.out.view(torch.int16))


def test_strided_fused_qkv_views():
    """q, k, v as strided views of one [B, N, 3, H, D] projection output
    (thakicloud accel-stack post, 이 기술은 무엇인가: strided views of the
    fused qkv instead of copies), written into a strided output view: lists
    and every output row against the oracle, the rest of the output buffer
    untouched, and bit-identical to the same call on contiguous copies."""
    dev = _dev()
    B, N, H, D = 2, 1100, 2, 128
    q, k, v = inputs.clustered_soft(B, N, H, D, seed=9)
    fused = np.stack([q, k, v], axis=2)  # [B, N, 3, H, D]
    ft = inputs.to_torch_bf16(fused, dev)
    tq, tk, tv = ft[:, :, 0], ft[:, :, 1], ft[:, :, 2]
    out_big = torch.zeros((B, N, 2, H, D), dtype=torch.bfloat16, device=dev)
    out = out_big[:, :, 1]
    kw = dict(tau=1.0, prefix_len=70)
    _, counts, lists = binding.sparse_attn(tq, tk, tv, out=out, return_route=True, **kw)
    torch.cuda.synchronize()
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    _, info = O.forward_blocks(qf, kf, vf, [], **kw)
    sel = selection_from(counts, lists)
    check_route(sel, info)
    ref, _ = O.forward(qf, kf, vf, info=dict(info, sel=sel), **kw)
    check_output(out.float().cpu().numpy().astype(np.float64), ref, "strided views")
    assert (out_big[:, :, 0] == 0).all()
    ref_run = GpuRun(q, k, v, **kw)
    assert torch.equal(out.contiguous().view(torch.int16), ref_run.out.view(torch.int16))


def test_injected_lists_through_attend():
    """sparse_attn_attend on caller-written lists (random masks, including
    empty lists) against the oracle on the same mask."""
    dev = _dev()
    B, N, H, D = 1, 1000, 2, 128
    q, k, v = inputs.clustered(B, N, H, D, seed=3)
    plan = binding.SparseAttnPlan(B, N, H, D, tau=1.0)
    tq, tk, tv = (inputs.to_torch_bf16(x, dev) for x in (q, k, v))
    ws = plan.workspace(dev)
    plan.pool(tq, tk, tv, ws)
    nb = plan.layout["n_blocks"]
    rng = np.random.default_rng(0)
    sel = rng.random((B, H, nb, nb)) < 0.2
    sel[0, 0, 3] = False  # a query block with nothing exact
    sel[0, 1, 5] = True   # a fully exact query block
    counts, lists = plan.route_views(ws)
    cnt = sel.sum(-1).astype(np.int32)
    lst = np.zeros((B, H, nb, nb), dtype=np.int32)
    for h in range(H):
        for a in range(nb):
            idx = np.nonzero(sel[0, h, a])[0]
            lst[0, h, a, : len(idx)] = idx[::-1] if a % 2 else idx  # order must not matter
    counts.copy_(torch.from_numpy(cnt))
    lists.copy_(torch.from_numpy(lst))
    out = torch.empty_like(tq)
    plan.attend(tq, out, ws)
    torch.cuda.synchronize()
    ref, _ = O.forward(_f32(q), _f32(k), _f32(v), mask=sel)
    check_output(out.float().cpu().numpy().astype(np.float64), ref, "injected")


def test_max_blocks():
    """n_b = 2048 (N = 131072), the largest supported length."""
    B, N, H, D = 1, 131072, 1, 64
    q, k, v = inputs.clustered(B, N, H, D, seed=12)
    run = GpuRun(q, k, v, tau=1.0)
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    _, info = O.forward_blocks(qf, kf, vf, [], tau=1.0)
    sel = run.selection()
    check_route(sel, info)
    blocks = [(0, 0, a) for a in (0, 1, 777, 1500, 2047)]
    parts, _ = O.forward_blocks(qf, kf, vf, blocks, info=dict(info, sel=sel))
    got = run.out_f64()
    for (b, h, a), ref in parts.items():
        check_output(got[b, a * 64 : a * 64 + ref.shape[0], h], ref, f"block {a}")


# -------------------------------------------- the benchmarked workloads


def _sampled_parity(name, n_sample=48, int8_qk=False, **over):
    w = inputs.make_workload(name, **over)
    kw = dict(tau=w.tau, topk_ratio=w.topk_ratio, prefix_len=w.prefix_len)
    if int8_qk:
        kw["int8_qk"] = True
    if w.topk_ratio is not None:
        kw.pop("tau")
    else:
        kw.pop("topk_ratio")
    print(f"  {name}: generated {w.shape}", flush=True)
    run = GpuRun(w.q, w.k, w.v, **kw)
    qf, kf, vf = _f32(w.q), (None if w.k is w.q else _f32(w.k)), _f32(w.v)
    kf = qf if kf is None else kf
    _, info = O.forward_blocks(qf, kf, vf, [], **oracle_kw(kw))
    B, N, H, D = w.shape
    nb = O.num_blocks(N)
    if run.plan.dense:
        sel = info["sel"]
    else:
        sel = run.selection()
        frac = check_route(sel, info)
        print(f"  {name}: density {sel.mean():.4f} oracle {info['sel'].mean():.4f} band {frac:.2e}", flush=True)
    rng = np.random.default_rng(1)
    blocks = {(0, int(rng.integers(H)), int(rng.integers(nb))) for _ in range(n_sample)}
    blocks |= {(0, 0, nb - 1), (0, H - 1, nb - 1), (0, 3, 0)}
    pb = O.prefix_blocks(w.prefix_len)
    if pb:
        blocks |= {(0, 5, pb - 1), (0, 6, pb)}
    parts, _ = O.forward_blocks(qf, kf, vf, sorted(blocks), info=dict(info, sel=sel), **oracle_kw(kw))
    got = run.out_f64()
    g = np.concatenate([got[b, a * 64 : a * 64 + r.shape[0], h] for (b, h, a), r in parts.items()])
    r = np.concatenate(list(parts.values()))
    check_output(g, r, f"{name} ({len(parts)} blocks)")


def test_workload_n4k_full():
    w = inputs.make_workload("n4k")
    full_parity(w.q, w.k, w.v, tau=1.0)


def test_workload_n16k_sampled():
    _sampled_parity("n16k")


def test_workload_n16k_dense_sampled():
    _sampled_parity("n16k", tau=-math.inf)


def test_workload_n32k_sampled():
    _sampled_parity("n32k")


def test_workload_h3_sampled():
    _sampled_parity("h3")


def test_workload_n32k_int8_sampled():
    _sampled_parity("n32k", n_sample=24, int8_qk=True)


# ------------------------------------------------ soft softmax, full n_b
#
# With Q = K the diagonal key takes almost all of each row's softmax weight,
# so the benchmarked workloads barely weigh the centroid terms.  These cases
# draw keys independently of the queries (clustered_soft / the H3 layout with
# its own key noise, amplitude 0.5): the routing still follows the signal,
# but the unselected blocks' centroids carry most of the mass.  Every case
# spans n_b >= 512 (16 to 19 centroid half tiles), and the oracle's own
# centroid share of the sampled rows is asserted, so the output bars
# measure the centroid path.

SOFT = [
    ("n32k_tau1", dict(gen="soft", N=32768, D=128), dict(tau=1.0)),
    ("n32k_tau1_reweight", dict(gen="soft", N=32768, D=128), dict(tau=1.0, reweight=True)),
    ("n32k_tau1_int8", dict(gen="soft", N=32768, D=128), dict(tau=1.0, int8_qk=True)),
    ("n33000_d64_tau05", dict(gen="soft", N=33000, D=64), dict(tau=0.5)),
    ("n33000_d64_topk_reweight", dict(gen="soft", N=33000, D=64), dict(topk_ratio=0.15, reweight=True)),
    ("h3_topk", dict(gen="h3soft", N=38247, D=128), dict(topk_ratio=0.1, prefix_len=1024)),
    ("h3_topk_reweight", dict(gen="h3soft", N=38247, D=128), dict(topk_ratio=0.1, prefix_len=1024, reweight=True)),
    ("h3_topk_exact_kv", dict(gen="h3soft", N=38247, D=128), dict(topk_ratio=0.1, prefix_len=1024,
                                                                  exact_kv_only=True)),
]


def _soft_inputs(gen, N, D, H=2, seed=50):
    if gen == "soft":
        return inputs.clustered_soft(1, N, H, D, seed=seed)
    return inputs.h3_joint(1, N, H, D, prefix_len=1024, seed=seed, amp=0.5, shared_qk=False)


@pytest.mark.parametrize("name,shape,kw", SOFT, ids=[s[0] for s in SOFT])
def test_soft_softmax_full_nb_sampled(name, shape, kw):
    q, k, v = _soft_inputs(shape["gen"], shape["N"], shape["D"], seed=50 + len(name))
    run = GpuRun(q, k, v, **kw)
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    okw = oracle_kw(kw)
    _, info = O.forward_blocks(qf, kf, vf, [], **okw)
    sel = run.selection()
    frac = check_route(sel, info)
    B, N, H, D = q.shape
    nb = O.num_blocks(N)
    nct = -(-nb // 32)
    pb = O.prefix_blocks(kw.get("prefix_len", 0))
    rng = np.random.default_rng(7)
    blocks = {(0, int(rng.integers(H)), int(rng.integers(pb, nb))) for _ in range(40)}
    blocks |= {(0, 0, nb - 1), (0, 1, nb - 2), (0, 1, 0)}
    if pb:
        blocks |= {(0, 0, pb - 1), (0, 1, pb)}
    blocks = sorted(blocks)
    shares = {}
    parts, _ = O.forward_blocks(qf, kf, vf, blocks, info=dict(info, sel=sel), shares=shares, **okw)
    routed = [key for key in blocks if kw.get("exact_kv_only") or key[2] >= pb]
    share = np.concatenate([shares[key] for key in routed])
    # the unselected blocks of the sampled rows reach every centroid half
    # tile, the ragged tail's centroid included
    tiles = set()
    tail_missed = 0
    for b, h, a in routed:
        missed = np.nonzero(~sel[b, h, a])[0]
        tiles |= set((missed // 32).tolist())
        tail_missed += int(not sel[b, h, a, nb - 1])
    print(f"  {name}: density {sel.mean():.4f} band {frac:.2e} centroid share median {np.median(share):.3f} "
          f"p10 {np.percentile(share, 10):.3f}; centroid half tiles reached {len(tiles)}/{nct}; "
          f"tail centroid in {tail_missed} sampled rows", flush=True)
    assert np.median(share) > 0.3, "the centroid terms must carry a material share of the softmax weight"
    assert tiles == set(range(nct)) and tail_missed > 0
    got = run.out_f64()
    g = np.concatenate([got[b, a * 64 : a * 64 + r.shape[0], h] for (b, h, a), r in parts.items()])
    r = np.concatenate(list(parts.values()))
    check_output(g, r, f"{name} ({len(parts)} blocks)")


@pytest.mark.parametrize("N,density", [(8192, 0.5), (32768, 0.35)])
def test_injected_lists_full_nb(N, density):
    """Caller-written random lists at n_b = 128 and 512 on soft inputs: the
    pair unions run past 64 half tiles (the kernel's union table is refilled
    every 64), with empty and full rows; every sampled row against the oracle
    on the same mask."""
    dev = _dev()
    B, H, D = 1, 2, 128
    q, k, v = inputs.clustered_soft(B, N, H, D, seed=N)
    plan = binding.SparseAttnPlan(B, N, H, D, tau=1.0)
    tq, tk, tv = (inputs.to_torch_bf16(x, dev) for x in (q, k, v))
    ws = plan.workspace(dev)
    plan.pool(tq, tk, tv, ws)
    nb = plan.layout["n_blocks"]
    rng = np.random.default_rng(N)
    sel = rng.random((B, H, nb, nb)) < density
    sel[0, 0, 3] = False  # nothing exact
    sel[0, 1, 5] = True   # fully exact
    sel[0, 0, 10] = False
    sel[0, 0, 10, nb - 1] = True  # only the last block exact
    counts, lists = plan.route_views(ws)
    cnt = sel.sum(-1).astype(np.int32)
    lst = np.zeros((B, H, nb, nb), dtype=np.int32)
    for h in range(H):
        for a in range(nb):
            idx = np.nonzero(sel[0, h, a])[0]
            lst[0, h, a, : len(idx)] = idx
    counts.copy_(torch.from_numpy(cnt))
    lists.copy_(torch.from_numpy(lst))
    out = torch.empty_like(tq)
    plan.attend(tq, out, ws)
    torch.cuda.synchronize()
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    blocks = sorted({(0, h, a) for h in range(H) for a in (0, 3, 5, 10, 11, nb - 1)}
                    | {(0, int(rng.integers(H)), int(rng.integers(nb))) for _ in range(24)})
    shares = {}
    parts, _ = O.forward_blocks(qf, kf, vf, blocks, mask=sel, shares=shares)
    share = np.concatenate(list(shares.values()))
    print(f"  injected N={N}: centroid share median {np.median(share):.3f}", flush=True)
    assert np.median(share) > 0.1
    got = out.float().cpu().numpy().astype(np.float64)
    g = np.concatenate([got[b, a * 64 : a * 64 + r.shape[0], h] for (b, h, a), r in parts.items()])
    r = np.concatenate(list(parts.values()))
    check_output(g, r, f"injected N={N} ({len(parts)} blocks)")


# ------------------------------------------------------------- Spark-Reblock


def _group_range(n, level, g):
    """Node g at depth `level` of the split tree of n rows (as in the kernel)."""
    start, size = 0, n
    for t in range(level):
        bit = (g >> (level - 1 - t)) & 1
        if size <= 64:
            if bit:
                return start, 0
            continue
        m = -(-size // 64)
        nl = 64 * (-(-m // 2))
        if bit:
            start, size = start + nl, size - nl
        else:
            size = nl
    return start, size


def _near_min(x, tol):
    return np.nonzero(x <= x.min() + tol * max(1.0, np.abs(x).max()))[0]


def _tree_groups(nv):
    """(level, start, size) of every group of more than 64 rows in the split
    tree of nv rows, as the kernels lay it out."""
    levels = max(0, int(math.ceil(math.log2(max(1, -(-nv // 64))))))
    for level in range(levels):
        for g in range(1 << level):
            start, n = _group_range(nv, level, g)
            if n > 64:
                yield level, start, n


def check_reblock_tree(order, u, M, rel=2.0**-5, exact=False):
    """Every split of the GPU's tree against the oracle's own fp64 values.

    order: the GPU's final order of the n_v moving rows (positions 0..n_v-1);
    u, M: O.mahalanobis_units of the raw inputs.  A group of the tree holds
    the rows at its positions of the final order, its left child the first
    n_L of them; when it was split its rows stood in ascending order (the
    root is the identity and children keep the parent's order, so every leaf
    must list its rows ascending).  The left child must be the n_L rows that
    the oracle's pivot split ranks first, for the oracle's pivots or any
    pivot within the GPU's rounding of the minimum (the pivot rule's ties),
    rows within that rounding of the cut falling on either side, unless
    exact, which requires the left child to be exactly one of those sets.

    The GPU compares rows through bf16 u and M u, so a dot product
    (M u_i) . w carries an error of a few 2^-9 |M u_i| |w|; the tolerance is
    rel * max_i |M u_i| * |w| for each quantity compared (w = the mean
    direction, the pivot u_a, or u_b - u_a).  A fixed tolerance would not
    do: when the group's unit rows nearly cancel, every row's similarity to
    the mean direction lies within a tiny range.  Returns (splits checked,
    rows admitted within tolerance of a cut)."""
    nv = len(order)
    for start in range(0, nv, 64):
        assert (np.diff(order[start : start + 64]) > 0).all(), f"leaf at {start} not in parent order"
    n_split, loose = 0, 0
    for level, start, n in _tree_groups(nv):
        m = -(-n // 64)
        nl = 64 * (-(-m // 2))
        gpu_left_rows = set(order[start : start + nl].tolist())
        rows = np.sort(order[start : start + n])
        gl = np.isin(rows, order[start : start + nl])
        uu = u[rows]
        mu = uu @ M
        scale = rel * np.linalg.norm(mu, axis=1).max()
        ubar = uu.mean(axis=0)
        s = mu @ ubar
        best = None
        for a in np.nonzero(s <= s.min() + scale * np.linalg.norm(ubar))[0]:
            t = mu @ uu[a]
            for b in np.nonzero(t <= t.min() + scale * np.linalg.norm(uu[a]))[0]:
                p = mu @ (uu[b] - uu[a])
                rank = np.lexsort((np.arange(n), p))
                if set(rows[rank[:nl]].tolist()) == gpu_left_rows:
                    best = 0
                    break
                if exact:
                    continue
                ps = p[rank]
                cut = 0.5 * (ps[nl - 1] + ps[nl])
                d = scale * np.linalg.norm(uu[b] - uu[a])
                if (p[gl] <= cut + d).all() and (p[~gl] >= cut - d).all():
                    oracle_left = np.zeros(n, dtype=bool)
                    oracle_left[rank[:nl]] = True
                    k = int((oracle_left != gl).sum())
                    best = k if best is None else min(best, k)
            if best == 0:
                break
        assert best is not None, f"level {level} group at {start} ({n} rows): split differs from the oracle's"
        loose += best
        n_split += 1
    return n_split, loose


def check_reblock_splits(U, M, order, MU=None, tol=1e-5):
    """Secondary check on the GPU's own intermediates: every split of its
    tree, given its unit rows U [n_v, D], rows M u (MU) and metric M, must be
    the oracle's pivot split of the same group to within tol (pivots within
    tol of the minimum accepted as alternatives).  The primary check,
    check_reblock_tree, uses the oracle's values from the raw inputs."""
    nv = len(order)
    n_split = 0
    for level, start, n in _tree_groups(nv):
        m = -(-n // 64)
        nl = 64 * (-(-m // 2))
        rows = order[start : start + n]
        gpu_left = np.zeros(n, dtype=bool)
        gpu_left[:nl] = True
        u = U[rows]
        mu = u @ M if MU is None else MU[rows]
        a0, b0, p0, left0 = O.pivot_split(u, M, nl, mu=mu)
        ok = False
        s = mu @ u.mean(axis=0)
        for a in [a0] + [x for x in _near_min(s, tol) if x != a0]:
            t = mu @ u[a]
            for b in ([b0] if a == a0 else []) + [x for x in _near_min(t, tol) if not (a == a0 and x == b0)]:
                p = mu @ (u[b] - u[a])
                ps = np.sort(p)
                thr = 0.5 * (ps[nl - 1] + ps[nl])
                d = tol * max(1.0, np.abs(p).max())
                if (p[gpu_left] <= thr + d).all() and (p[~gpu_left] >= thr - d).all():
                    ok = True
                    break
            if ok:
                break
        assert ok, f"level {level} group at {start}: split differs from the oracle's ({(left0 != gpu_left).sum()} rows)"
        n_split += 1
    return n_split


def _permute(x, perm):
    out = np.empty_like(x)
    for b in range(x.shape[0]):
        for h in range(x.shape[2]):
            out[b, :, h] = x[b, perm[b, h], h]
    return out


def reblock_parity(q, k, v, check_heads=None, layout="q_reuse_k", **kw):
    run = GpuRun(q, k, v, reblock=True, reblock_layout=layout, **kw)
    M, U, MU, pq, pk = run.plan.reblock_views(run.ws)
    M = M.cpu().numpy().astype(np.float64)
    pq, pk = pq.cpu().numpy(), pk.cpu().numpy()
    B, N, H, D = q.shape
    r0 = min(O.prefix_blocks(kw.get("prefix_len", 0)) * 64, N)
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    heads = [(b, h) for b in range(B) for h in range(H)] if check_heads is None else check_heads
    sides = [(qf, kf, pq)] if layout == "q_reuse_k" else [(qf, kf, pq), (kf, qf, pk)]
    if layout == "q_reuse_k":
        assert (pk == pq).all(), "q_reuse_k: keys and values must take the query partition"
    n_split, n_loose, n_split2 = 0, 0, 0
    for side, (x, other, perm) in enumerate(sides):
        for b in range(B):
            for h in range(H):
                assert sorted(perm[b, h].tolist()) == list(range(N))
                assert (perm[b, h, :r0] == np.arange(r0)).all()
        for b, h in heads:
            u_ref, M_ref = O.mahalanobis_units(x[b, r0:, h], other[b, :, h])
            np.testing.assert_allclose(M[side, b, h], M_ref, rtol=0, atol=1e-4 * np.abs(M_ref).max())
            ug = U[side, b, h].float().cpu().numpy().astype(np.float64)
            assert (np.abs(ug - u_ref) <= 2.0**-7 * np.abs(u_ref) + 2e-2 * np.abs(u_ref).max(axis=1, keepdims=True)).all()
            mug = MU[side, b, h].float().cpu().numpy().astype(np.float64)
            mref = ug @ M[side, b, h]
            assert (np.abs(mug - mref) <= 2.0**-6 * np.abs(mref) + 2e-2 * np.abs(mref).max(axis=1, keepdims=True)).all()
            ns, nl_ = check_reblock_tree(perm[b, h, r0:] - r0, u_ref, M_ref)
            n_split += ns
            n_loose += nl_
            n_split2 += check_reblock_splits(ug, M[side, b, h], perm[b, h, r0:] - r0, MU=mug)
    print(f"  reblock ({layout}): {n_split} splits against the oracle's values ({n_loose} rows within tol of a cut), "
          f"{n_split2} against the GPU's own u, M u", flush=True)
    qp, kp, vp = _permute(qf, pq), _permute(kf, pk), _permute(vf, pk)
    okw = oracle_kw(kw)
    _, info = O.forward_blocks(qp, kp, vp, [], **okw)
    sel = run.selection()
    check_route(sel, info)
    ref_p, _ = O.forward(qp, kp, vp, info=dict(info, sel=sel), **okw)
    ref = np.empty_like(ref_p)
    for b in range(B):
        for h in range(H):
            ref[b, pq[b, h], h] = ref_p[b, :, h]
    check_output(run.out_f64(), ref, f"reblock N={N} {kw}")
    return run, pq, pk


def _hier_clusters(B, N, H, D, pre, seed, ratio=2.5, noise=0.005):
    """Query rows after the prefix blocks in 2^L tight clusters of 64 rows
    (shuffled positions) whose centres form a binary hierarchy: centre j is
    sum_l s_l(j) ratio^(-l/2) e_l over orthonormal e_l, s_l(j) = +-1 the
    bits of j.  Each level's weight outweighs all deeper ones together, so
    the pivot split separates the hierarchy level by level with a wide gap at
    every cut (the two halves of a node are mirror images, so which one goes
    left is a tie of the pivot rule).  Keys and values are i.i.d. N(0, 1)."""
    rng = np.random.default_rng(seed)
    r0 = min(O.prefix_blocks(pre) * 64, N)
    nv = N - r0
    ncl = nv // 64
    L = int(round(math.log2(ncl)))
    assert nv == 64 * ncl and 2**L == ncl
    q = rng.standard_normal((B, N, H, D))
    k = rng.standard_normal((B, N, H, D))
    v = rng.standard_normal((B, N, H, D))
    labels = {}
    for b in range(B):
        for h in range(H):
            E = np.linalg.qr(rng.standard_normal((D, L)))[0]
            signs = np.array([[1.0 if (j >> (L - 1 - l)) & 1 else -1.0 for l in range(L)] for j in range(ncl)])
            cen = (signs * ratio ** (-0.5 * np.arange(L))) @ E.T
            lab = np.repeat(np.arange(ncl), 64)
            rng.shuffle(lab)
            q[b, r0:, h] = cen[lab] + noise * rng.standard_normal((nv, D))
            labels[(b, h)] = lab
    return [inputs.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v)], labels


def _oracle_min_cut_gap(u, M):
    """Smallest gap between the n_L-th and next rank value over every split
    of the oracle's own tree (its pivots)."""
    worst = math.inf

    def rec(idx):
        nonlocal worst
        if len(idx) <= 64:
            return
        m = -(-len(idx) // 64)
        nl = 64 * (-(-m // 2))
        _, _, p, left = O.pivot_split(u[idx], M, nl)
        ps = np.sort(p)
        worst = min(worst, ps[nl] - ps[nl - 1])
        rec(idx[left])
        rec(idx[~left])

    rec(np.arange(len(u)))
    return worst


HIER = [
    ("d64_prefix_8", (1, 64 + 512, 2, 64, 64)),
    ("d128_b2_16", (2, 1024, 1, 128, 0)),
    ("d128_prefix_straddle_16", (1, 128 + 1024, 2, 128, 100)),
]


@pytest.mark.parametrize("name,shape", HIER, ids=[h[0] for h in HIER])
def test_reblock_tree_matches_oracle_on_raw_inputs(name, shape):
    """The GPU's partition against O.reblock_orders-style splits computed by
    the oracle from the raw inputs alone (fp64 u and M, no GPU value), on
    planted hierarchical clusters whose every cut the oracle separates by a
    wide gap: every split must be exactly one the oracle's pivot rule gives
    (mirror-image ties either way), so the leaves are exactly the oracle's
    leaves; the keys reuse the query partition; the output against the
    oracle's own reblocked forward (its orders, not the GPU's)."""
    B, N, H, D, pre = shape
    (q, k, v), labels = _hier_clusters(B, N, H, D, pre, seed=7)
    run = GpuRun(q, k, v, reblock=True, tau=1.0, prefix_len=pre)
    _, _, _, pq, pk = run.plan.reblock_views(run.ws)
    pq, pk = pq.cpu().numpy(), pk.cpu().numpy()
    assert (pk == pq).all()
    r0 = min(O.prefix_blocks(pre) * 64, N)
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    opq, opk = O.reblock_orders(qf, kf, prefix_len=pre)
    n_split = 0
    for b in range(B):
        for h in range(H):
            u, M = O.mahalanobis_units(qf[b, r0:, h], kf[b, :, h])
            # the precondition: every cut of the oracle's own tree is wide
            assert _oracle_min_cut_gap(u, M) > 0.1
            ns, loose = check_reblock_tree(pq[b, h, r0:] - r0, u, M, exact=True)
            assert loose == 0
            n_split += ns
            gpu_leaves = {frozenset(x.tolist()) for x in np.split(pq[b, h, r0:], range(64, N - r0, 64))}
            ora_leaves = {frozenset(x.tolist()) for x in np.split(opq[b, h, r0:], range(64, N - r0, 64))}
            assert gpu_leaves == ora_leaves
            for leaf in ora_leaves:
                assert len(set(labels[(b, h)][np.array(sorted(leaf)) - r0].tolist())) == 1
    print(f"  {name}: {n_split} splits equal to the oracle's", flush=True)
    ref, _ = O.forward(qf, kf, vf, reblock=True, tau=1.0, prefix_len=pre)
    check_output(run.out_f64(), ref, f"reblock {name} vs the oracle's own orders")


REBLOCK = [
    ("tau_prefix_d64", dict(B=1, N=1100, H=2, D=64), dict(tau=1.0, prefix_len=100)),
    ("tau_d128", dict(B=1, N=1024, H=2, D=128), dict(tau=1.0)),
    ("topk_tail_b2", dict(B=2, N=777, H=1, D=128), dict(topk_ratio=0.25, prefix_len=64)),
    ("reweight_int8", dict(B=1, N=700, H=2, D=64), dict(tau=0.5, prefix_len=30, reweight=True, int8_qk=True)),
    ("exact_kv", dict(B=1, N=1000, H=2, D=128), dict(tau=1.0, prefix_len=130, exact_kv_only=True)),
    ("short", dict(B=1, N=100, H=2, D=64), dict(tau=1.0, prefix_len=40)),
    ("separate_tau_prefix_d64", dict(B=1, N=1100, H=2, D=64), dict(tau=1.0, prefix_len=100, layout="separate")),
    ("separate_topk_tail_b2", dict(B=2, N=777, H=1, D=128), dict(topk_ratio=0.25, prefix_len=64, layout="separate")),
    # more than 1024 moving rows on few problems: the first levels run wide
    # (1024-row chunks, the last one ragged), the deepest from registers
    ("wide_d64_b2_prefix", dict(B=2, N=5000, H=3, D=64), dict(tau=1.0, prefix_len=200)),
    ("wide_d128_separate_topk", dict(B=1, N=4500, H=2, D=128), dict(topk_ratio=0.2, prefix_len=64, layout="separate")),
]


@pytest.mark.parametrize("name,shape,kw", REBLOCK, ids=[r[0] for r in REBLOCK])
def test_reblock_parity(name, shape, kw):
    B, N, H, D = shape["B"], shape["N"], shape["H"], shape["D"]
    q, k, v = inputs.clustered_soft(B, N, H, D, seed=len(name) + 100) if N >= 256 else inputs.iid(B, N, H, D, 100)
    reblock_parity(q, k, v, **kw)


def test_reblock_recovers_planted_clusters():
    """Query rows tightly around four directions in shuffled positions: every
    block of the GPU's query order holds one cluster."""
    rng = np.random.default_rng(42)
    B, N, H, D, pre = 1, 64 + 512, 1, 64, 64
    centers = rng.standard_normal((4, D))
    lab = np.repeat(np.arange(4), 128)
    rng.shuffle(lab)
    q = rng.standard_normal((B, N, H, D))
    q[0, pre:, 0] = centers[lab] + 0.02 * rng.standard_normal((512, D))
    k = rng.standard_normal((B, N, H, D))
    v = rng.standard_normal((B, N, H, D))
    bits = [inputs.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v)]
    _, pq, _ = reblock_parity(*bits, tau=1.0, prefix_len=pre)
    for blk in (pq[0, 0, pre:] - pre).reshape(8, 64):
        assert len(set(lab[blk].tolist())) == 1


def test_workload_n16k_reblock_sampled():
    """n16k (H = 56) reordered in the shared layout: metric, unit rows and
    every split of four heads against the oracle's values from the raw
    inputs (and, secondarily, the GPU's own), lists, and sampled output
    blocks."""
    w = inputs.make_workload("n16k")
    kw = dict(tau=w.tau, prefix_len=w.prefix_len)
    run = GpuRun(w.q, w.k, w.v, reblock=True, **kw)
    M, U, MU, pq, pk = run.plan.reblock_views(run.ws)
    M = M.cpu().numpy().astype(np.float64)
    pq, pk = pq.cpu().numpy(), pk.cpu().numpy()
    assert (pk == pq).all()
    B, N, H, D = w.shape
    r0 = min(O.prefix_blocks(w.prefix_len) * 64, N)
    qf, kf, vf = _f32(w.q), _f32(w.k), _f32(w.v)
    n_split, n_loose, n_split2 = 0, 0, 0
    for h in (0, 17, 38, H - 1):
        assert sorted(pq[0, h].tolist()) == list(range(N))
        u_ref, M_ref = O.mahalanobis_units(qf[0, r0:, h], kf[0, :, h])
        np.testing.assert_allclose(M[0, 0, h], M_ref, rtol=0, atol=1e-4 * np.abs(M_ref).max())
        ns, nl_ = check_reblock_tree(pq[0, h, r0:] - r0, u_ref, M_ref)
        n_split += ns
        n_loose += nl_
        ug = U[0, 0, h].float().cpu().numpy().astype(np.float64)
        mug = MU[0, 0, h].float().cpu().numpy().astype(np.float64)
        n_split2 += check_reblock_splits(ug, M[0, 0, h], pq[0, h, r0:] - r0, MU=mug)
    print(f"  n16k reblock: {n_split} splits against the oracle's values ({n_loose} rows within tol of a cut), "
          f"{n_split2} against the GPU's own", flush=True)
    assert n_loose <= 0.02 * 4 * (N - r0)  # rows the oracle's values place within rounding of a cut
    qp, kp, vp = _permute(qf, pq), _permute(kf, pk), _permute(vf, pk)
    _, info = O.forward_blocks(qp, kp, vp, [], **kw)
    sel = run.selection()
    check_route(sel, info)
    nb = O.num_blocks(N)
    rng = np.random.default_rng(3)
    blocks = sorted({(0, int(rng.integers(H)), int(rng.integers(nb))) for _ in range(24)} | {(0, 0, nb - 1)})
    parts, _ = O.forward_blocks(qp, kp, vp, blocks, info=dict(info, sel=sel), **kw)
    got = run.out_f64()
    g, r = [], []
    for (b, h, a), o in parts.items():
        rows = pq[b, h, a * 64 : a * 64 + o.shape[0]]
        g.append(got[b, rows, h])
        r.append(o)
    check_output(np.concatenate(g), np.concatenate(r), f"n16k reblock ({len(parts)} blocks)")


def test_reblock_strided_views_and_reruns():
    """Reblock on strided views of a fused [B, N, 3, H, D] projection, writing
    into a strided output: its orders pass the split check against the
    oracle's values, its output matches the oracle on those orders, it
    equals reblock on contiguous inputs bit for bit, and a rerun on the same
    workspace repeats orders and output exactly."""
    dev = _dev()
    B, N, H, D, pre = 2, 1300, 3, 128, 90
    q, k, v = inputs.clustered_soft(B, N, H, D, seed=19)
    fused = np.stack([q, k, v], axis=2)
    ft = inputs.to_torch_bf16(fused, dev)
    tq, tk, tv = ft[:, :, 0], ft[:, :, 1], ft[:, :, 2]
    out_big = torch.zeros((B, N, 2, H, D), dtype=torch.bfloat16, device=dev)
    out = out_big[:, :, 1]
    plan = binding.SparseAttnPlan(B, N, H, D, tau=1.0, prefix_len=pre, reblock=True,
                                  in_strides=tq.stride()[:3], out_strides=out.stride()[:3])
    ws = plan.workspace(dev)
    plan.forward(tq, tk, tv, out=out, ws=ws)
    torch.cuda.synchronize()
    _, _, _, pq, pk = plan.reblock_views(ws)
    pq, pk = pq.cpu().numpy(), pk.cpu().numpy()
    assert (pk == pq).all()
    r0 = min(O.prefix_blocks(pre) * 64, N)
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    for b in range(B):
        for h in range(H):
            u, M = O.mahalanobis_units(qf[b, r0:, h], kf[b, :, h])
            check_reblock_tree(pq[b, h, r0:] - r0, u, M)
    qp, kp, vp = _permute(qf, pq), _permute(kf, pk), _permute(vf, pk)
    _, info = O.forward_blocks(qp, kp, vp, [], tau=1.0, prefix_len=pre)
    sel = selection_from(*plan.route_views(ws))
    check_route(sel, info)
    ref_p, _ = O.forward(qp, kp, vp, info=dict(info, sel=sel), tau=1.0, prefix_len=pre)
    ref = np.empty_like(ref_p)
    for b in range(B):
        for h in range(H):
            ref[b, pq[b, h], h] = ref_p[b, :, h]
    check_output(out.float().cpu().numpy().astype(np.float64), ref, "reblock strided views")
    assert (out_big[:, :, 0] == 0).all()
    ref_run = GpuRun(q, k, v, tau=1.0, prefix_len=pre, reblock=True)
    assert torch.equal(out.contiguous().view(torch.int16), ref_run.out.view(torch.int16))
    _, _, _, pq1, pk1 = ref_run.plan.reblock_views(ref_run.ws)
    pq1, pk1, o1 = pq1.clone(), pk1.clone(), ref_run.out.clone()
    ref_run.plan.forward(ref_run.q, ref_run.k, ref_run.v, out=ref_run.out, ws=ref_run.ws)
    torch.cuda.synchronize()
    _, _, _, pq2, pk2 = ref_run.plan.reblock_views(ref_run.ws)
    assert torch.equal(pq1, pq2) and torch.equal(pk1, pk2)
    assert torch.equal(o1.view(torch.int16), ref_run.out.view(torch.int16))


def test_reblock_d64_deeper_tree():
    """D = 64, 4160 moving rows (66 blocks, a 7-level tree with ragged
    groups): every split of every head against the oracle."""
    q, k, v = inputs.clustered(1, 4224, 2, 64, seed=23)
    reblock_parity(q, k, v, tau=1.0, prefix_len=64)


def test_route_entry_point_matches_stages():
    """sparse_attn_route leaves the same counts and lists as pool + select."""
    dev = _dev()
    q, k, v = inputs.clustered(1, 1500, 2, 128, seed=31)
    tq, tk, tv = (inputs.to_torch_bf16(x, dev) for x in (q, k, v))
    plan = binding.SparseAttnPlan(1, 1500, 2, 128, topk_ratio=0.2, prefix_len=70)
    ws1 = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    ws2 = torch.empty_like(ws1)
    plan.route(tq, tk, tv, ws1)
    plan.pool(tq, tk, tv, ws2)
    plan.select(ws2)
    torch.cuda.synchronize()
    c1, l1 = plan.route_views(ws1)
    c2, l2 = plan.route_views(ws2)
    assert torch.equal(c1, c2)
    nb = c1.shape[-1]
    valid = torch.arange(nb, device=dev).view(1, 1, 1, nb) < c1.unsqueeze(-1)
    assert torch.equal(torch.where(valid, l1, 0), torch.where(valid, l2, 0))


# ------------------------------------------------------- mode combinations

_COMBOS = []
for _i, (_D, _B, _N, _pre) in enumerate([(64, 2, 333, 0), (128, 1, 700, 70), (64, 1, 1000, 1000), (128, 2, 450, 130)]):
    for _flags in ({}, dict(reweight=True), dict(int8_qk=True), dict(reweight=True, int8_qk=True, exact_kv_only=True),
                   dict(reblock=True), dict(reblock=True, int8_qk=True, reweight=True)):
        _route = dict(tau=0.7) if _i % 2 == 0 else dict(topk_ratio=0.3)
        _COMBOS.append((dict(B=_B, N=_N, H=2, D=_D), dict(prefix_len=_pre, **_route, **_flags)))


@pytest.mark.parametrize("shape,kw", _COMBOS, ids=[f"D{s['D']}_B{s['B']}_N{s['N']}_" + "_".join(
    f"{k}" if v is True else f"{k}{v}" for k, v in kw.items()) for s, kw in _COMBOS])
def test_mode_combinations(shape, kw):
    """Every flag combination against the oracle on every output row: ragged
    tails, B = 2, a prefix straddling a block and one covering all rows."""
    q, k, v = inputs.iid(shape["B"], shape["N"], shape["H"], shape["D"], seed=shape["N"] + len(kw))
    if kw.get("reblock"):
        reblock_parity(q, k, v, **{a: b for a, b in kw.items() if a != "reblock"})
    else:
        full_parity(q, k, v, **kw)


def test_workload_h3_reblock_reweight_int8_sampled():
    """h3 (N = 38247, 1024 prefix rows, top-K 0.1, ragged tail, a 10-level
    tree) with reblock, reweight and INT8 QK^T together: orders valid and
    prefix fixed, every split of two heads against the oracle's values from
    the raw inputs, lists, and sampled output blocks against the oracle on
    the GPU's orders."""
    w = inputs.make_workload("h3")
    kw = dict(topk_ratio=w.topk_ratio, prefix_len=w.prefix_len, reweight=True, int8_qk=True)
    run = GpuRun(w.q, w.k, w.v, reblock=True, **kw)
    M, U, MU, pq, pk = run.plan.reblock_views(run.ws)
    M = M.cpu().numpy().astype(np.float64)
    pq, pk = pq.cpu().numpy(), pk.cpu().numpy()
    assert (pk == pq).all()
    B, N, H, D = w.shape
    r0 = min(O.prefix_blocks(w.prefix_len) * 64, N)
    assert run.plan.layout["reblock_levels"] == 10
    qf, kf, vf = _f32(w.q), _f32(w.k), _f32(w.v)
    for h in range(H):
        assert (pq[0, h, :r0] == np.arange(r0)).all()
        assert np.array_equal(np.sort(pq[0, h]), np.arange(N))
    n_split, n_loose, n_split2 = 0, 0, 0
    for h in (7, 41):
        u_ref, M_ref = O.mahalanobis_units(qf[0, r0:, h], kf[0, :, h])
        ns, nl_ = check_reblock_tree(pq[0, h, r0:] - r0, u_ref, M_ref)
        n_split += ns
        n_loose += nl_
        ug = U[0, 0, h].float().cpu().numpy().astype(np.float64)
        mug = MU[0, 0, h].float().cpu().numpy().astype(np.float64)
        n_split2 += check_reblock_splits(ug, M[0, 0, h], pq[0, h, r0:] - r0, MU=mug)
    print(f"  h3 reblock: {n_split} splits against the oracle's values ({n_loose} rows within tol of a cut), "
          f"{n_split2} against the GPU's own", flush=True)
    assert n_loose <= 0.02 * 2 * (N - r0)  # rows the oracle's values place within rounding of a cut
    qp, kp, vp = _permute(qf, pq), _permute(kf, pk), _permute(vf, pk)
    okw = oracle_kw(kw)
    _, info = O.forward_blocks(qp, kp, vp, [], **okw)
    sel = run.selection()
    check_route(sel, info)
    nb = O.num_blocks(N)
    rng = np.random.default_rng(5)
    blocks = sorted({(0, int(rng.integers(H)), int(rng.integers(nb))) for _ in range(16)}
                    | {(0, 0, nb - 1), (0, 3, 0), (0, 5, 15), (0, 6, 16)})
    parts, _ = O.forward_blocks(qp, kp, vp, blocks, info=dict(info, sel=sel), **okw)
    got = run.out_f64()
    g, r = [], []
    for (b, h, a), o in parts.items():
        g.append(got[b, pq[b, h, a * 64 : a * 64 + o.shape[0]], h])
        r.append(o)
    check_output(np.concatenate(g), np.concatenate(r), f"h3 reblock+reweight+int8 ({len(parts)} blocks)")


# -------------------------------------------------- seeded random configurations
#
# Shapes, routing, prefix, scale and flags drawn from one seed per case
# (N in [1, 64] for a quarter of the cases, else in [65, 2600]; i.i.d. or
# soft clustered inputs), every
# output row against the oracle with the same bars as above.

def _random_config(seed):
    rng = np.random.default_rng(1000 + seed)
    B, H, D = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.choice([64, 128]))
    N = int(rng.integers(1, 65)) if rng.random() < 0.25 else int(rng.integers(65, 2601))
    kw = {}
    if rng.random() < 0.6:
        kw["tau"] = float(rng.choice([-0.5, 0.0, 0.5, 1.0, 2.5]))
    else:
        kw["topk_ratio"] = float(rng.choice([0.03, 0.2, 0.5, 1.0]))
    if rng.random() < 0.5:
        kw["prefix_len"] = int(rng.integers(0, N + 1))
    if rng.random() < 0.2:
        kw["sm_scale"] = float(rng.uniform(0.05, 0.2))
    if rng.random() < 0.2:
        kw["centroid"] = False
    elif rng.random() < 0.3:
        kw["reweight"] = True
    if rng.random() < 0.2:
        kw["logmass"] = False
    if rng.random() < 0.25:
        kw["int8_qk"] = True
    if rng.random() < 0.2:
        kw["exact_kv_only"] = True
    reblock = rng.random() < 0.25
    layout = "separate" if reblock and rng.random() < 0.5 else "q_reuse_k"
    soft = N >= 256 and rng.random() < 0.5
    return dict(B=B, N=N, H=H, D=D, soft=soft, reblock=reblock, layout=layout), kw


@pytest.mark.parametrize("seed", range(32))
def test_random_configurations(seed):
    shape, kw = _random_config(seed)
    B, N, H, D = shape["B"], shape["N"], shape["H"], shape["D"]
    print(f"  seed {seed}: B={B} N={N} H={H} D={D} soft={shape['soft']} reblock={shape['reblock']} "
          f"({shape['layout']}) {kw}", flush=True)
    gen = inputs.clustered_soft if shape["soft"] else inputs.iid
    q, k, v = gen(B, N, H, D, seed=seed + 7)
    if shape["reblock"]:
        reblock_parity(q, k, v, layout=shape["layout"], **kw)
    else:
        full_parity(q, k, v, **kw)


# Seeded random shapes through the dense path (tau = -inf: the dense kernel
# at D = 64 and 128, or the routed kernel with INT8 QK^T), every output row
# against the oracle's softmax over all keys.

def _random_dense_config(seed):
    rng = np.random.default_rng(3000 + seed)
    B, H, D = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.choice([64, 128]))
    N = int(rng.integers(1, 65)) if rng.random() < 0.25 else int(rng.integers(65, 3001))
    kw = dict(tau=-math.inf)
    if rng.random() < 0.25:
        kw["sm_scale"] = float(rng.uniform(0.05, 0.2))
    if seed % 4 == 3:  # a quarter of the cases through the INT8 QK^T kernel
        kw["int8_qk"] = True
    soft = N >= 256 and rng.random() < 0.5
    return dict(B=B, N=N, H=H, D=D, soft=soft), kw


@pytest.mark.parametrize("seed", range(16))
def test_random_dense_configurations(seed):
    shape, kw = _random_dense_config(seed)
    B, N, H, D = shape["B"], shape["N"], shape["H"], shape["D"]
    print(f"  seed {seed}: B={B} N={N} H={H} D={D} soft={shape['soft']} {kw}", flush=True)
    gen = inputs.clustered_soft if shape["soft"] else inputs.iid
    q, k, v = gen(B, N, H, D, seed=seed + 90)
    full_parity(q, k, v, **kw)


# ------------------------------------------------------------ graph capture
#
# The library launches only kernels on the caller's stream (no memset, no
# allocation, no synchronisation), so a forward call can be captured into a
# HIP graph.  Each replay runs after eager work and a synchronisation and
# must equal the eager call bit for bit.

@pytest.mark.parametrize("kw", [dict(tau=1.0, prefix_len=100), dict(topk_ratio=0.2, reweight=True, int8_qk=True),
                                dict(tau=1.0, prefix_len=70, reblock=True), dict(tau=-math.inf)],
                         ids=["tau_prefix", "topk_reweight_int8", "reblock", "dense"])
def test_graph_capture_replays_match_eager(kw):
    dev = _dev()
    B, N, H, D = 1, 3000, 4, 128
    q, k, v = (inputs.to_torch_bf16(x, dev) for x in inputs.clustered_soft(B, N, H, D, seed=5))
    plan = binding.SparseAttnPlan(B, N, H, D, **kw)
    ws = plan.workspace(dev)
    ref = plan.forward(q, k, v, out=torch.empty_like(q), ws=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.forward(q, k, v, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.forward(q, k, v, out=out, ws=ws)
    for i in range(4):
        out.zero_()
        ws.zero_()
        junk = torch.randn(4096, device=dev).sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i} differs ({junk.item():.1f})"


# ------------------------------------------- seeded random large configurations
#
# N from 4000 to 40000 (n_b 63 to 625: long lists, many centroid half tiles,
# union tables refilled), one or two heads, random routing, prefix and
# flags on soft clustered inputs; every list against the oracle, and 16
# sampled query blocks plus the tail and prefix boundary blocks.

def _random_large_config(seed):
    rng = np.random.default_rng(5000 + seed)
    H, D = int(rng.integers(1, 3)), int(rng.choice([64, 128]))
    N = int(rng.integers(4000, 40001))
    kw = {}
    if rng.random() < 0.5:
        kw["tau"] = float(rng.choice([0.0, 0.5, 1.0, 2.0]))
    else:
        kw["topk_ratio"] = float(rng.choice([0.05, 0.1, 0.2]))
    if rng.random() < 0.6:
        kw["prefix_len"] = int(rng.integers(1, 2049))
    if rng.random() < 0.15:
        kw["centroid"] = False
    elif rng.random() < 0.3:
        kw["reweight"] = True
    if rng.random() < 0.15:
        kw["logmass"] = False
    if rng.random() < 0.3:
        kw["int8_qk"] = True
    if "prefix_len" in kw and rng.random() < 0.3:
        kw["exact_kv_only"] = True
    return dict(B=1, N=N, H=H, D=D), kw


@pytest.mark.parametrize("seed", range(12))
def test_random_large_configurations(seed):
    shape, kw = _random_large_config(seed)
    B, N, H, D = shape["B"], shape["N"], shape["H"], shape["D"]
    print(f"  seed {seed}: B={B} N={N} H={H} D={D} {kw}", flush=True)
    q, k, v = inputs.clustered_soft(B, N, H, D, seed=seed + 300)
    run = GpuRun(q, k, v, **kw)
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    okw = oracle_kw(kw)
    _, info = O.forward_blocks(qf, kf, vf, [], **okw)
    sel = run.selection()
    frac = check_route(sel, info)
    nb = O.num_blocks(N)
    rng = np.random.default_rng(seed)
    blocks = {(0, int(rng.integers(H)), int(rng.integers(nb))) for _ in range(16)}
    blocks |= {(0, 0, nb - 1), (0, H - 1, 0)}
    pb = O.prefix_blocks(kw.get("prefix_len", 0))
    if 0 < pb < nb:
        blocks |= {(0, 0, pb - 1), (0, H - 1, pb)}
    parts, _ = O.forward_blocks(qf, kf, vf, sorted(blocks), info=dict(info, sel=sel), **okw)
    got = run.out_f64()
    g = np.concatenate([got[b, a * 64 : a * 64 + r.shape[0], h] for (b, h, a), r in parts.items()])
    r = np.concatenate(list(parts.values()))
    print(f"  density {sel.mean():.4f} band {frac:.2e}", flush=True)
    check_output(g, r, f"seed {seed} ({len(parts)} blocks)")


def test_reblock_max_blocks():
    """Spark-Reblock at n_b = 2048 (N = 131072, the largest supported length),
    one head: an 11-level tree whose first seven levels run over 1024-row
    chunks.  Every split against the oracle's values from the raw inputs,
    the lists against the oracle on the GPU's order, and sampled output
    blocks."""
    B, N, H, D = 1, 131072, 1, 128
    q, k, v = inputs.clustered_soft(B, N, H, D, seed=13)
    run = GpuRun(q, k, v, reblock=True, tau=1.0)
    M, U, MU, pq, pk = run.plan.reblock_views(run.ws)
    pq, pk = pq.cpu().numpy(), pk.cpu().numpy()
    assert (pk == pq).all() and sorted(pq[0, 0].tolist()) == list(range(N))
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    u_ref, M_ref = O.mahalanobis_units(qf[0, :, 0], kf[0, :, 0])
    Mg = M.cpu().numpy().astype(np.float64)[0, 0, 0]
    np.testing.assert_allclose(Mg, M_ref, rtol=0, atol=1e-4 * np.abs(M_ref).max())
    ns, nl_ = check_reblock_tree(pq[0, 0], u_ref, M_ref)
    print(f"  n_b 2048 reblock: {ns} splits against the oracle's values ({nl_} rows within tol of a cut)", flush=True)
    assert nl_ <= 0.02 * N
    qp, kp, vp = _permute(qf, pq), _permute(kf, pk), _permute(vf, pk)
    _, info = O.forward_blocks(qp, kp, vp, [], tau=1.0)
    sel = run.selection()
    check_route(sel, info)
    blocks = [(0, 0, a) for a in (0, 1, 777, 1500, 2047)]
    parts, _ = O.forward_blocks(qp, kp, vp, blocks, info=dict(info, sel=sel), tau=1.0)
    got = run.out_f64()
    for (b, h, a), ref in parts.items():
        rows = pq[b, h, a * 64 : a * 64 + ref.shape[0]]
        check_output(got[b, rows, h], ref, f"reblock block {a}")
