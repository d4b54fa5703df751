"""CPU oracle for Sol-style routed block-sparse attention (NumPy, float64).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: it is used by the tests, by the package's smoke check
and by the benchmark's CPU-baseline leg.  It shares no code with the HIP
library; the only common module is the seeded input generator, which holds
none of this arithmetic.

What is computed, step by step, and where the pages state it:

1. Pool.  The sequence is cut into 64-row blocks; Q, K and V are mean-pooled
   per block (Star7 README "MiniMax H3 Activation Chunk & Attention
   Acceleration", section 工作原理 > Sol: Q64/K64 blocks; comfyui-wiki
   "Spark-H3" news, Spark-Reweight bullet: mean-pooled K/V summaries).
2. Score.  Every query block is scored against every key block with the
   pooled product Qbar_a . Kbar_c (keys-SM121 MiniMax-H3 README, optimisation
   table, Sol-Attn row: each query block goes to its highest-scoring KV blocks).
3. Route.  Either a threshold "tau standard deviations above the mean of the
   block scores" (thakicloud "MiniMax-H3 ComfyUI accel stack", section
   이 기술은 무엇인가; Star7 README, Sol: tau = 1.0), or a top-K ratio
   (Spark-H3 news, 워크플로 section: topk_mode = topk_ratio, 0.1 / 0.2).
   The packed conditioning prefix is kept as an exact KV sink (thakicloud
   post, same section; Star7 README, Sol: audio-range KV sink) and prefix
   query rows get full attention (Star7 README, Sol; aikraft.ru news,
   section "Нововведения версии 2.0": exact_kv_and_rows).  The same news
   item names a lighter mode, exact_kv, that keeps only the sink; with
   prefix_rows=False the prefix query rows are routed like every other row.
4. Combine.  Selected blocks are attended exactly; every unselected block is
   not dropped but contributes once through its K/V centroid, and both kinds
   of term share one softmax (Star7 README, Sol).  Each centroid logit gets a
   log-mass bias so that the centroid stands for the block's mass (Spark-H3
   news, Spark-Reweight bullet and its figure caption: mean pooling gives
   exp(E[x]) where the block's mass is E[exp(x)]).
5. Reweight (optional, reweight=True).  Spark-Reweight (Spark-H3 news, same
   bullet) replaces the mean-pooled K/V summaries by weighted summaries plus
   a log-mass bias, scored against one anchor per head, the mean of the
   video queries.  Reading: anchor a = mean of the query rows >= prefix_len
   (all rows when there are none); per key block, x_j = a . k_j * scale and
   w = softmax(x) over the block's rows; Ktilde = sum w_j k_j,
   Vtilde = sum w_j v_j, bias = logsumexp(x) - a . Ktilde * scale.  For the
   anchor itself the centroid term then equals the block's exact terms in
   mass and value; for a block of equal keys it is the mean-pooled centroid
   with bias log(n_c).
6. INT8 QK^T (optional, int8_qk=True).  The thakicloud post (section
   실제 실험 결과) describes an int8 QK path that quantises only each key
   block's residual about the block mean and keeps the mean term exact in
   bf16 (the Star7 README's 注意力模式 table lists QK-int8 modes with FP32
   softmax).  Reading: base_c = the block's fp32 key mean (rows summed in
   order) rounded to bf16; r = k - base_c; one scale per key block,
   s_c = max |r| / 127 over its valid rows and all dimensions; residual
   codes rint(r / s_c) clipped to [-127, 127]; one scale per query row,
   s_q = max_d |q| / 127, codes rint(q / s_q).  An exact-block logit is
   scale * (q . base_c + s_q * s_c * (q8 . r8)), q unquantised in the first
   term.  Codes are decided in float32, the precision the kernel uses;
   centroid logits are unchanged.
7. Reblock (optional, reblock=True).  Spark-Reblock (Spark-H3 news,
   Spark-Reblock bullet) replaces the fixed 64-row tiles by an input-, layer-
   and head-dependent partition: two queries are alike when their score
   patterns over the keys are alike, measured by the cosine in the metric of
   the keys' second moment (and keys by that of the queries), and a
   hierarchical partitioner splits groups until every leaf has the block
   size, in O(N log N).  The shipped workflows pin the layout q_reuse_k
   (same news, 워크플로 section): read as one partition per (b, h), made
   for the queries, that the keys and values reuse.  Reading: per (b, h),
   M = K^T K over all N keys (the "separate" layout also partitions the
   keys on their own, in M = Q^T Q), u_i = x_i / sqrt(x_i^T M x_i) for the rows after
   the prefix blocks (prefix blocks stay in place), so that
   cos_M(x_i, x_j) = u_i^T M u_j; a group of n > 64 rows with m = ceil(n/64)
   blocks splits into a left child of 64 * ceil(m / 2) rows and the rest.
   The pages do not give the split rule; it is taken as a pivot split that
   uses only the stated similarity: a = the row least similar to the group's
   mean direction (u_i^T M ubar), b = the row least similar to a, and the
   left child is the rows ranked first by u_i^T M (u_b - u_a) (ties by
   position), i.e. those most like a.  Children keep their parent's order,
   left before right; the leaves in order are the new blocks.  Attention then
   runs on Q, K, V permuted that way, and the output rows go back to their
   positions.

Readings where the pages leave a step open (each is argued in the design
notes of this repository):

* score scale: the routing score is the unscaled Qbar . Kbar; mean/std
  thresholds and top-K are invariant under a positive scale;
* std is the population standard deviation over all key blocks of the row,
  computed two-pass; every key block (prefix and ragged tail included)
  enters the mean and std;
* tau = -inf selects every block; tau = +inf selects none (before the sink);
  otherwise block c is selected iff S_ac >= mean + tau * std;
* top-K keeps k = clamp(ceil(r * n_b - 1e-6), 1, n_b) blocks (r is the float32
  ratio; the 1e-6 keeps ratios such as 0.1 * 640 from rounding up), ties
  going to the lower block index;
* the prefix sink (every key block holding a row < prefix_len) is OR-ed in
  after ranking; every query block holding a prefix row is computed densely
  (exact_kv_and_rows, the default), or, in exact_kv mode, routed by the same
  rule as the other rows;
* the centroid logit uses the individual query row: q_i . Kbar_c * scale;
* the log-mass bias is log(n_c), n_c = valid rows of block c (64, or the
  tail count), i.e. the centroid counts as n_c copies of itself;
* softmax scale 1/sqrt(D) unless given; non-causal; rows past N do not exist
  (the tail block has n_c < 64 rows);
* a query row left with no term at all (centroids off and nothing selected)
  outputs 0.

The one-shot softmax below is the definition; an online softmax differs from
it only by rounding.
"""

from __future__ import annotations

import math
from typing import Dict, Iterable, Optional, Tuple

import numpy as np

BLOCK = 64

__all__ = [
    "BLOCK",
    "num_blocks",
    "block_sizes",
    "prefix_blocks",
    "topk_count",
    "pool",
    "block_scores",
    "route",
    "selection_lists",
    "attend_block",
    "forward",
    "reweight_summaries",
    "int8_qk_codes",
    "mahalanobis_units",
    "pivot_split",
    "reblock_orders",
    "forward_blocks",
]


def num_blocks(N: int) -> int:
    """n_b = ceil(N / 64)."""
    return -(-int(N) // BLOCK)


def block_sizes(N: int) -> np.ndarray:
    """Valid row count n_c of every block: 64, except a ragged last block."""
    nb = num_blocks(N)
    n = np.full(nb, BLOCK, dtype=np.int64)
    n[-1] = N - BLOCK * (nb - 1)
    return n


def prefix_blocks(prefix_len: int) -> int:
    """Blocks that hold at least one packed-prefix row: ceil(prefix_len / 64)."""
    return -(-int(prefix_len) // BLOCK)


def topk_count(topk_ratio: float, nb: int) -> int:
    """Blocks kept per query block in top-K mode (float32 ratio, see header)."""
    r = float(np.float32(topk_ratio))
    return int(min(nb, max(1, math.ceil(r * nb - 1e-6))))


def pool(x) -> np.ndarray:
    """Per-block means of the valid rows.

    x: [B, N, H, D] array of bf16-exact values (float32 or float64).
    Returns float64 [B, H, n_b, D].
    """
    B, N, H, D = x.shape
    nb = num_blocks(N)
    out = np.empty((B, H, nb, D), dtype=np.float64)
    for c in range(nb):
        rows = np.asarray(x[:, c * BLOCK : min(N, (c + 1) * BLOCK)], dtype=np.float64)
        out[:, :, c, :] = rows.sum(axis=1) / rows.shape[1]
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """S[b, h, a, c] = Qbar_a . Kbar_c (unscaled)."""
    return np.matmul(qbar, np.swapaxes(kbar, -1, -2))


def route(
    S: np.ndarray,
    *,
    tau: Optional[float] = 1.0,
    topk_ratio: Optional[float] = None,
    prefix_len: int = 0,
    prefix_rows: bool = True,
) -> Dict[str, np.ndarray]:
    """Block selection from the score matrix S [B, H, n_b, n_b].

    prefix_rows: query blocks holding prefix rows attend to every key block
    (exact_kv_and_rows); False keeps only the key sink (exact_kv).

    Returns a dict with ``sel`` (bool [B, H, n_b, n_b]) and, per row, ``mu``,
    ``sigma``, ``thr`` (the tau threshold, or the k-th largest score in
    top-K mode) and ``cut``, the score value that separates kept from dropped
    blocks (thr in tau mode; in top-K mode the midpoint between the k-th and
    (k+1)-th largest scores, -inf when k = n_b).  Both are NaN on dense
    prefix rows.
    """
    B, H, nb, nb2 = S.shape
    assert nb == nb2
    pb = min(nb, prefix_blocks(prefix_len))
    mu = S.mean(axis=-1)
    sigma = np.sqrt(((S - mu[..., None]) ** 2).mean(axis=-1))
    thr = np.full(mu.shape, np.nan)
    if topk_ratio is not None:
        k = topk_count(topk_ratio, nb)
        # Descending score, ties broken towards the lower block index.
        order = np.argsort(-S, axis=-1, kind="stable")
        sel = np.zeros(S.shape, dtype=bool)
        np.put_along_axis(sel, order[..., :k], True, axis=-1)
        thr = np.take_along_axis(S, order[..., k - 1 : k], axis=-1)[..., 0]
        if k < nb:
            nxt = np.take_along_axis(S, order[..., k : k + 1], axis=-1)[..., 0]
            cut = 0.5 * (thr + nxt)
        else:
            cut = np.full(mu.shape, -math.inf)
    else:
        t = float(np.float32(tau))
        if t == -math.inf:
            sel = np.ones(S.shape, dtype=bool)
        elif t == math.inf:
            sel = np.zeros(S.shape, dtype=bool)
            thr = np.full(mu.shape, math.inf)
        else:
            thr = mu + t * sigma
            sel = S >= thr[..., None]
        cut = thr.copy()
    # Exact KV sink: every key block that holds a prefix row.
    sel[..., :pb] = True
    # Prefix query rows see every key exactly (exact_kv_and_rows).
    if prefix_rows and pb:
        sel[:, :, :pb, :] = True
        thr[:, :, :pb] = np.nan
        cut[:, :, :pb] = np.nan
    return dict(sel=sel, mu=mu, sigma=sigma, thr=thr, cut=cut)


def selection_lists(sel: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Ascending index lists [B, H, n_b, n_b] (padded with -1) and counts."""
    counts = sel.sum(axis=-1).astype(np.int32)
    lists = np.full(sel.shape, -1, dtype=np.int32)
    B, H, nb, _ = sel.shape
    for b in range(B):
        for h in range(H):
            for a in range(nb):
                idx = np.nonzero(sel[b, h, a])[0]
                lists[b, h, a, : len(idx)] = idx
    return lists, counts


def attend_block(
    q_rows: np.ndarray,
    k_head: np.ndarray,
    v_head: np.ndarray,
    kbar_head: np.ndarray,
    vbar_head: np.ndarray,
    sel_row: np.ndarray,
    sizes: np.ndarray,
    *,
    scale: float,
    centroid: bool,
    logmass: bool,
    cbias_head: Optional[np.ndarray] = None,
    int8_head: Optional[dict] = None,
    share: Optional[list] = None,
) -> np.ndarray:
    """Output rows of one query block of one head.

    q_rows [n_a, D]; k_head, v_head [N, D]; kbar_head, vbar_head [n_b, D]
    (the centroid summaries); sel_row bool [n_b].  Exact logits for every
    valid key of a selected block, one centroid logit per unselected block,
    one softmax over all of them.  cbias_head [n_b], when given, is the
    centroid bias (reweight mode) in place of log(n_c).  int8_head, when
    given, holds this head's INT8 QK^T quantities (qcode, qscale for these
    rows; kbase, kscale, kcode of the head) and sets the exact logits.
    ``share``, when given, receives per row the centroid terms' share of the
    softmax weight (float64 [n_a]; 0 without centroid terms).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    chosen = np.nonzero(sel_row)[0]
    keys = np.concatenate(
        [np.arange(c * BLOCK, c * BLOCK + sizes[c]) for c in chosen]
    ) if len(chosen) else np.zeros(0, dtype=np.int64)
    kx = np.asarray(k_head[keys], dtype=np.float64)
    vx = np.asarray(v_head[keys], dtype=np.float64)
    if int8_head is None:
        logits = [q_rows @ kx.T * scale]
    else:
        logits = [int8_logits(q_rows, keys, int8_head) * scale]
    values = [vx]
    if centroid:
        missed = np.nonzero(~sel_row)[0]
        y = q_rows @ kbar_head[missed].T * scale
        if cbias_head is not None:
            y = y + cbias_head[missed][None, :]
        elif logmass:
            y = y + np.log(sizes[missed].astype(np.float64))[None, :]
        logits.append(y)
        values.append(vbar_head[missed])
    L = np.concatenate(logits, axis=1)
    Vall = np.concatenate(values, axis=0)
    if L.shape[1] == 0:
        if share is not None:
            share.append(np.zeros(q_rows.shape[0]))
        return np.zeros((q_rows.shape[0], q_rows.shape[1]))
    M = L.max(axis=1, keepdims=True)
    W = np.exp(L - M)
    if share is not None:
        n_exact = logits[0].shape[1]
        share.append(W[:, n_exact:].sum(axis=1) / W.sum(axis=1))
    return (W @ Vall) / W.sum(axis=1, keepdims=True)


def reweight_summaries(q, k, v, prefix_len: int = 0, sm_scale: Optional[float] = None):
    """Spark-Reweight summaries (reading in the module docstring).

    Returns (anchor [B, H, D], ktilde [B, H, n_b, D], vtilde [B, H, n_b, D],
    cbias [B, H, n_b]), all float64.  cbias is in natural-log units.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, N, H, D = q.shape
    scale = (1.0 / math.sqrt(D)) if not sm_scale else float(sm_scale)
    first = int(prefix_len) if 0 <= int(prefix_len) < N else 0
    anchor = q[:, first:].mean(axis=1)  # [B, H, D]
    nb = num_blocks(N)
    sizes = block_sizes(N)
    kt = np.empty((B, H, nb, D))
    vt = np.empty((B, H, nb, D))
    cb = np.empty((B, H, nb))
    for b in range(B):
        for h in range(H):
            a = anchor[b, h]
            for c in range(nb):
                rows = slice(c * BLOCK, c * BLOCK + sizes[c])
                kc, vc = k[b, rows, h], v[b, rows, h]
                x = kc @ a * scale
                m = x.max()
                e = np.exp(x - m)
                w = e / e.sum()
                kt[b, h, c] = w @ kc
                vt[b, h, c] = w @ vc
                cb[b, h, c] = (m + math.log(e.sum())) - float(kt[b, h, c] @ a) * scale
    return anchor, kt, vt, cb


def int8_logits(q_rows, keys, h):
    """Unscaled INT8 QK^T logits q . base_c + s_q s_c (q8 . r8) of the query
    rows against the keys ``keys`` of one head (reading 6)."""
    blk = np.asarray(keys, dtype=np.int64) // BLOCK
    mean_term = np.asarray(q_rows, dtype=np.float64) @ np.asarray(h["kbase"], dtype=np.float64)[blk].T
    dots = h["qcode"].astype(np.int64) @ h["kcode"][keys].astype(np.int64).T  # exact integers
    sq = np.asarray(h["qscale"], dtype=np.float64)[:, None]
    sk = np.asarray(h["kscale"], dtype=np.float64)[blk][None, :]
    return mean_term + sq * sk * dots


def _bf16_round(x):
    """float32 -> nearest bfloat16 value (ties to even), as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def int8_qk_codes(q, k, residual: bool = True):
    """INT8 QK^T quantities (reading 6 in the module docstring), in float32.

    Returns a dict: kbase [B, H, n_b, D] (bf16 block means; zero when
    residual=False, which quantises whole keys instead), kscale [B, H, n_b],
    kcode [B, N, H, D] int8 residual codes, qscale [B, N, H] and
    qcode [B, N, H, D] int8.
    """
    q = np.asarray(q, dtype=np.float32)
    k = np.asarray(k, dtype=np.float32)
    B, N, H, D = k.shape
    nb = num_blocks(N)
    sizes = block_sizes(N)
    kp = np.zeros((B, nb * BLOCK, H, D), dtype=np.float32)
    kp[:, :N] = k
    kb = kp.reshape(B, nb, BLOCK, H, D)
    valid = (np.arange(nb * BLOCK) < N).reshape(nb, BLOCK)
    if residual:
        acc = np.zeros((B, nb, H, D), dtype=np.float32)
        for r in range(BLOCK):  # rows in order; padded rows add +0
            acc = acc + kb[:, :, r]
        mean = acc / sizes.astype(np.float32)[None, :, None, None]
        base = _bf16_round(mean)
    else:
        base = np.zeros((B, nb, H, D), dtype=np.float32)
    res = kb - base[:, :, None]
    res = np.where(valid[None, :, :, None, None], res, np.float32(0))
    amax = np.abs(res).max(axis=(2, 4))  # [B, nb, H]
    ks = amax / np.float32(127)
    safe = np.where(ks > 0, ks, np.float32(1))
    code = np.rint(res / safe[:, :, None, :, None])
    code = np.where(ks[:, :, None, :, None] > 0, np.clip(code, -127, 127), 0)
    kcode = code.reshape(B, nb * BLOCK, H, D)[:, :N].astype(np.int8)
    qs = np.abs(q).max(axis=3) / np.float32(127)  # [B, N, H]
    qsafe = np.where(qs > 0, qs, np.float32(1))
    qcode = np.where(qs[..., None] > 0, np.clip(np.rint(q / qsafe[..., None]), -127, 127), 0).astype(np.int8)
    return dict(
        kbase=base.transpose(0, 2, 1, 3).copy(),
        kscale=ks.transpose(0, 2, 1).copy(),
        kcode=kcode,
        qscale=qs,
        qcode=qcode,
    )


def _prepare(q, k, v, tau, topk_ratio, prefix_len, mask, prefix_rows=True):
    B, N, H, D = q.shape
    qbar, kbar, vbar = pool(q), pool(k), pool(v)
    info = dict(qbar=qbar, kbar=kbar, vbar=vbar)
    if mask is None:
        S = block_scores(qbar, kbar)
        r = route(S, tau=tau, topk_ratio=topk_ratio, prefix_len=prefix_len, prefix_rows=prefix_rows)
        info.update(S=S, **r)
    else:
        info["sel"] = np.asarray(mask, dtype=bool)
    return info


def forward_blocks(
    q,
    k,
    v,
    blocks: Iterable[Tuple[int, int, int]],
    *,
    tau: Optional[float] = 1.0,
    topk_ratio: Optional[float] = None,
    prefix_len: int = 0,
    prefix_rows: bool = True,
    centroid: bool = True,
    logmass: bool = True,
    reweight: bool = False,
    int8_qk: bool = False,
    sm_scale: Optional[float] = None,
    mask: Optional[np.ndarray] = None,
    info: Optional[dict] = None,
    shares: Optional[dict] = None,
):
    """Output of selected (b, h, query block) triples, one by one.

    q, k, v: [B, N, H, D] bf16-exact values.  ``mask`` (bool [B,H,n_b,n_b])
    replaces the routing step when given.  ``info`` lets a caller reuse the
    pooled tensors and routing of an earlier call on the same inputs.
    ``shares``, when given, receives {(b, h, a): per-row centroid share of
    the softmax weight} (see attend_block).
    Returns ({(b, h, a): float64 [n_a, D]}, info).
    """
    B, N, H, D = q.shape
    scale = (1.0 / math.sqrt(D)) if not sm_scale else float(sm_scale)
    if info is None:
        info = _prepare(q, k, v, tau, topk_ratio, prefix_len, mask, prefix_rows)
    if reweight and "cbias" not in info:
        info["anchor"], info["ktilde"], info["vtilde"], info["cbias"] = reweight_summaries(
            q, k, v, prefix_len=prefix_len, sm_scale=sm_scale)
    if int8_qk and "int8" not in info:
        info["int8"] = int8_qk_codes(q, k)
    ksum = info["ktilde"] if reweight else info["kbar"]
    vsum = info["vtilde"] if reweight else info["vbar"]
    sel = info["sel"]
    sizes = block_sizes(N)
    out = {}
    for b, h, a in blocks:
        rows = slice(a * BLOCK, a * BLOCK + sizes[a])
        sh = [] if shares is not None else None
        out[(b, h, a)] = attend_block(
            q[b, rows, h, :],
            k[b, :, h, :],
            v[b, :, h, :],
            ksum[b, h],
            vsum[b, h],
            sel[b, h, a],
            sizes,
            scale=scale,
            centroid=centroid,
            logmass=logmass,
            cbias_head=info["cbias"][b, h] if reweight else None,
            int8_head=_int8_head(info["int8"], b, h, rows) if int8_qk else None,
            share=sh,
        )
        if shares is not None:
            shares[(b, h, a)] = sh[0]
    return out, info


def _int8_head(d, b, h, rows):
    return dict(
        qcode=d["qcode"][b, rows, h],
        qscale=d["qscale"][b, rows, h],
        kbase=d["kbase"][b, h],
        kscale=d["kscale"][b, h],
        kcode=d["kcode"][b, :, h],
    )


def mahalanobis_units(x, other):
    """Rows u_i = x_i / ||x_i||_M of one head, M = other^T other (reading 7),
    so that u_i^T M u_j is the cosine of the score patterns other @ x_i and
    other @ x_j.  A row with ||x_i||_M = 0 maps to 0.  Returns (u, M)."""
    x = np.asarray(x, dtype=np.float64)
    other = np.asarray(other, dtype=np.float64)
    M = other.T @ other
    n2 = np.einsum("id,de,ie->i", x, M, x)
    norm = np.sqrt(np.maximum(n2, 0.0))
    u = np.where(norm[:, None] > 0, x / np.where(norm > 0, norm, 1.0)[:, None], 0.0)
    return u, M


def pivot_split(u, M, n_left, mu=None):
    """One split of a group (rows u [n, D] in group order), reading 7.
    Returns (a, b, p, left): the two pivots (positions in the group, first
    minimum on ties), the rank values p_i = u_i^T M (u_b - u_a) and the bool
    mask of the n_left rows ranked first by (p_i, position).  ``mu`` may
    give the rows M u_i (M is symmetric, so u_i^T M v = (M u_i) . v)."""
    u = np.asarray(u, dtype=np.float64)
    n = u.shape[0]
    mu = u @ M if mu is None else np.asarray(mu, dtype=np.float64)
    s = mu @ u.mean(axis=0)
    a = int(np.argmin(s))
    t = mu @ u[a]
    b = int(np.argmin(t))
    p = mu @ (u[b] - u[a])
    rank = np.lexsort((np.arange(n), p))
    left = np.zeros(n, dtype=bool)
    left[rank[:n_left]] = True
    return a, b, p, left


def _reblock_head(x, other, r0):
    N = x.shape[0]
    u, M = mahalanobis_units(x[r0:], other)

    def rec(idx):
        if len(idx) <= BLOCK:
            return [idx]
        m = -(-len(idx) // BLOCK)
        n_left = BLOCK * (-(-m // 2))
        left = pivot_split(u[idx], M, n_left)[3]
        return rec(idx[left]) + rec(idx[~left])

    leaves = rec(np.arange(N - r0)) if N > r0 else []
    return np.concatenate([np.arange(r0)] + [r0 + leaf for leaf in leaves]).astype(np.int64)


def reblock_orders(q, k, prefix_len: int = 0, layout: str = "q_reuse_k"):
    """Spark-Reblock orders (reading 7): perm_q, perm_k int64 [B, H, N];
    new position i of a head holds original row perm[..., i].  Queries use
    M = K^T K.  layout "q_reuse_k" (the layout the shipped workflows pin,
    Spark-H3 news, 워크플로 section) gives the keys, and with them the
    values, the query partition: perm_k = perm_q.  layout "separate"
    partitions the keys on their own, in M = Q^T Q."""
    if layout not in ("q_reuse_k", "separate"):
        raise ValueError(f"unknown reblock layout {layout!r}")
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, N, H, D = q.shape
    r0 = min(prefix_blocks(prefix_len) * BLOCK, N)
    pq = np.empty((B, H, N), dtype=np.int64)
    pk = np.empty((B, H, N), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            pq[b, h] = _reblock_head(q[b, :, h], k[b, :, h], r0)
            if layout == "q_reuse_k":
                pk[b, h] = pq[b, h]
            else:
                pk[b, h] = _reblock_head(k[b, :, h], q[b, :, h], r0)
    return pq, pk


def _gather_rows(x, perm):
    x = np.asarray(x)
    out = np.empty_like(x)
    for b in range(x.shape[0]):
        for h in range(x.shape[2]):
            out[b, :, h] = x[b, perm[b, h], h]
    return out


def forward(q, k, v, reblock: bool = False, perms=None, reblock_layout: str = "q_reuse_k", **kw):
    """Full output [B, N, H, D] float64 plus the routing info.  With
    reblock=True the attention runs on the Spark-Reblock orders (``perms`` =
    (perm_q, perm_k) to use given ones, else reblock_orders with
    ``reblock_layout``) and the rows are put back."""
    if reblock:
        pq, pk = perms if perms is not None else reblock_orders(q, k, kw.get("prefix_len", 0), reblock_layout)
        kw.pop("info", None)
        out_p, info = forward(_gather_rows(q, pq), _gather_rows(k, pk), _gather_rows(v, pk), **kw)
        out = np.empty_like(out_p)
        for b in range(out.shape[0]):
            for h in range(out.shape[2]):
                out[b, pq[b, h], h] = out_p[b, :, h]
        info["perm_q"], info["perm_k"] = pq, pk
        return out, info
    B, N, H, D = q.shape
    nb = num_blocks(N)
    blocks = [(b, h, a) for b in range(B) for h in range(H) for a in range(nb)]
    parts, info = forward_blocks(q, k, v, blocks, **kw)
    out = np.empty((B, N, H, D), dtype=np.float64)
    for (b, h, a), o in parts.items():
        out[b, a * BLOCK : a * BLOCK + o.shape[0], h, :] = o
    return out, info

