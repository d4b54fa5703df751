"""Benchmark: routed block-sparse attention on one MI355X.

One step = one full pass of the path over one batch of synthetic input:
pool -> select -> attend through the C ABI (the same three launches as
sparse_attn_forward, issued one by one so that HIP events on the launch
stream can time each kernel).  Inputs are resident in HBM before the timed
region starts.

Default workload: B=1, H=56, N=32768, D=128 bf16 BTHD, clustered synthetic
inputs, tau = 1.0 threshold routing, centroid terms with the log-mass bias.
The same inputs are also run through the dense path (tau = -inf) of the same
library for the speedup.

Prints ONE JSON line (rank 0 = the only rank).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def _traffic(workload: str):
    """HBM bytes per attend launch from the committed rocprofv3 counter runs,
    or None when they are missing or were taken on other kernel source."""
    p = os.path.join(ROOT, "profiles", f"attend_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    from block_sparse_video_fp32_amd.profiling import kernel_source_hash

    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d.get("bytes_per_launch")


def _mfma_busy(workload: str):
    """Share of the attend kernel's cycles its MFMA pipes were busy
    (SQ_VALU_MFMA_BUSY_CYCLES) from the committed rocprofv3 counter run, or
    None when it is missing or was taken on other kernel source."""
    p = os.path.join(ROOT, "profiles", f"attend_{workload}_mfma.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    from block_sparse_video_fp32_amd.profiling import kernel_source_hash

    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return {k: round(d[k], 4) for k in ("mfma_busy_frac", "clock_ghz", "executed_mfma_tflop")}


def selected_flops(plan, ws, N, D):
    """4 * D * rows_a * rows_c summed over every selected (b, h, a, c)."""
    import torch

    counts, lists = plan.route_views(ws)
    nb = counts.shape[-1]
    tail = N - 64 * (nb - 1)
    idx = torch.arange(nb, device=counts.device, dtype=torch.int32)
    valid = idx.view(1, 1, 1, nb) < counts.unsqueeze(-1)
    rows_c = torch.where(lists == nb - 1, tail, 64).to(torch.float64)
    per_row = torch.where(valid, rows_c, torch.zeros_like(rows_c)).sum(-1)  # [B,H,nb]
    rows_a = torch.full((nb,), 64.0, dtype=torch.float64, device=counts.device)
    rows_a[-1] = tail
    flops = 4.0 * D * (per_row * rows_a.view(1, 1, nb)).sum().item()
    density = counts.to(torch.float64).sum().item() / (counts.numel() * nb)
    return flops, density


def attend_mfma_count(plan, ws, D, centroid=True):
    """MFMA instructions one launch of the default attend instance executes.

    A query block's two waves each run one 32-key half tile with D/16 k-steps
    for S^T and (D/32 column tiles) x 2 k-steps for PV, i.e. D/8
    v_mfma_f32_32x32x16_bf16.  A block runs both half tiles of every key block
    in its list, and, when it is routed (count < n_b) with centroids on, one
    centroid half tile for each group of 32 key blocks that holds at least one
    unselected block.  Rows are counted from the routing lists, so the figure
    is exact for the launch (no logit overflow recompute assumed)."""
    import torch

    counts, lists = plan.route_views(ws)
    B, H, nb = counts.shape
    idx = torch.arange(nb, device=counts.device, dtype=torch.int32)
    valid = idx.view(1, 1, 1, nb) < counts.unsqueeze(-1)
    col = torch.where(valid, lists.clamp(0, nb - 1), nb).long()
    nct = (nb + 31) // 32
    sel = torch.zeros(B, H, nb, 32 * nct + 1, dtype=torch.bool, device=counts.device)
    sel[..., nb:] = True  # padding past the last block never needs a centroid
    sel.scatter_(-1, col, True)
    half_tiles = 2 * int(counts.to(torch.int64).sum().item())
    if centroid:
        chunk_unsel = (~sel[..., : 32 * nct]).view(B, H, nb, nct, 32).any(-1)
        need = chunk_unsel & (counts < nb).unsqueeze(-1)
        half_tiles += int(need.sum().item())
    return 2 * half_tiles * (D // 8)


def cpu_baseline(w, seconds_target=20.0):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    routing of every query block (pool + scores + selection) plus the output
    of as many query blocks as fit in the time budget.  Reported as
    selected-block TFLOP/s, the unit of the GPU figure."""
    import numpy as np

    from block_sparse_video_fp32_amd import inputs
    from oracle import sol_oracle as O

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    qf = inputs.bf16_bits_to_f32(w.q)
    kf = qf if w.k is w.q else inputs.bf16_bits_to_f32(w.k)
    vf = inputs.bf16_bits_to_f32(w.v)
    kw = dict(tau=w.tau) if w.topk_ratio is None else dict(topk_ratio=w.topk_ratio)
    kw["prefix_len"] = w.prefix_len
    B, N, H, D = w.shape
    nb = O.num_blocks(N)
    sizes = O.block_sizes(N)
    t0 = time.perf_counter()
    _, info = O.forward_blocks(qf, kf, vf, [], **kw)
    t_route = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    order = [(0, int(h), int(a)) for h, a in zip(rng.integers(0, H, 10**6), rng.integers(0, nb, 10**6))]
    flops = 0.0
    done = 0
    t1 = time.perf_counter()
    for blk in order:
        O.forward_blocks(qf, kf, vf, [blk], info=info, **kw)
        b, h, a = blk
        flops += 4.0 * D * sizes[a] * float(sizes[info["sel"][b, h, a]].sum())
        done += 1
        if time.perf_counter() - t1 > seconds_target:
            break
    t_attend = time.perf_counter() - t1
    # scale the sampled attend time to the whole workload, add the full routing
    frac = done / (B * H * nb)
    est_total = t_route + t_attend / frac
    total_flops = flops / frac
    return {
        "value": total_flops / est_total / 1e12,
        "unit": "TFLOP/s (selected-block, effective)",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (
            f"numpy fp64 oracle: routing of all {B * H * nb} query blocks ({t_route:.1f} s) + outputs of "
            f"{done} random query blocks ({t_attend:.1f} s), extrapolated to the full workload: "
            f"{est_total:.0f} s per call"
        ),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="n32k", choices=["tiny", "n4k", "n16k", "n32k", "h3"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--graph", action="store_true", help="also time the call replayed from a HIP graph")
    ap.add_argument("--no-modes", action="store_true", help="skip the reweight, INT8 QK^T, exact_kv (with a prefix), strided fused-QKV and reblock timings")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 256 MiB device copy before the steps (scales rocprofv3 byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(
            "bench.py measures one GPU: the path shards by head with no communication, "
            "so multi-GPU figures are not produced; run with --gpus 1",
            file=sys.stderr,
        )
        sys.exit(2)

    import torch

    from block_sparse_video_fp32_amd import binding, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    w = inputs.make_workload(args.workload)
    B, N, H, D = w.shape
    q, k, v = (inputs.to_torch_bf16(x, dev) for x in (w.q, w.k, w.v))
    out = torch.empty_like(q)
    print(f"# generated {args.workload} {w.shape} in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    rkw = dict(tau=w.tau) if w.topk_ratio is None else dict(topk_ratio=w.topk_ratio)
    plan = binding.SparseAttnPlan(B, N, H, D, prefix_len=w.prefix_len, **rkw)
    ws = plan.workspace(dev)
    stream = torch.cuda.current_stream(dev)

    if args.copy_calibration:
        src = torch.empty(128 * 1024 * 1024, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        plan.pool(q, k, v, ws)
        plan.select(ws)
        plan.attend(q, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(K):
        ev[i][0].record(stream)
        plan.pool(q, k, v, ws)
        ev[i][1].record(stream)
        plan.select(ws)
        ev[i][2].record(stream)
        plan.attend(q, out, ws)
        ev[i][3].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / K
    t_pool = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    t_sel = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    t_att = sum(e[2].elapsed_time(e[3]) for e in ev) / K
    print(f"# sparse: {ms_step:.3f} ms/step (pool {t_pool:.3f}, select {t_sel:.3f}, attend {t_att:.3f})",
          file=sys.stderr, flush=True)

    flops, density = selected_flops(plan, ws, N, D)
    nb = plan.layout["n_blocks"]

    # the same call captured once into a HIP graph and replayed (the library
    # only launches kernels on the caller's stream, so it captures as is)
    graph_ms = None
    if args.graph:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            plan.forward(q, k, v, out=out, ws=ws)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            plan.forward(q, k, v, out=out, ws=ws)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(K):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / K
        print(f"# graph replay: {graph_ms:.3f} ms/call", file=sys.stderr, flush=True)
        del graph

    # dense path of the same library on the same inputs
    dense_ms = None
    if not args.no_dense:
        dplan = binding.SparseAttnPlan(B, N, H, D, tau=-math.inf)
        dws = dplan.workspace(dev)
        for _ in range(2):
            dplan.forward(q, k, v, out=out, ws=dws)
        torch.cuda.synchronize()
        kd = max(3, K // 4)
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(kd):
            dplan.forward(q, k, v, out=out, ws=dws)
        s1.record(stream)
        torch.cuda.synchronize()
        dense_ms = s0.elapsed_time(s1) / kd
        print(f"# dense: {dense_ms:.3f} ms/call", file=sys.stderr, flush=True)

    # optional modes of the same call on the same inputs: Spark-Reweight
    # centroids and INT8 QK^T on the exact blocks (same routing)
    modes = None
    if not args.no_modes:
        modes = {}
        variants = [("reweight", dict(reweight=True)), ("int8_qk", dict(int8_qk=True))]
        if w.prefix_len > 0:  # the sink without the dense prefix query rows
            variants.append(("exact_kv", dict(exact_kv_only=True)))
        for name, extra in variants:
            mplan = binding.SparseAttnPlan(B, N, H, D, prefix_len=w.prefix_len, **rkw, **extra)
            mws = mplan.workspace(dev)
            for _ in range(2):
                mplan.pool(q, k, v, mws)
                mplan.select(mws)
                mplan.attend(q, out, mws)
            torch.cuda.synchronize()
            km = max(3, K // 2)
            me = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(km)]
            for i in range(km):
                me[i][0].record(stream)
                mplan.pool(q, k, v, mws)
                me[i][1].record(stream)
                mplan.select(mws)
                me[i][2].record(stream)
                mplan.attend(q, out, mws)
                me[i][3].record(stream)
            torch.cuda.synchronize()
            m_call = sum(e[0].elapsed_time(e[3]) for e in me) / km
            m_pool = sum(e[0].elapsed_time(e[1]) for e in me) / km
            m_att = sum(e[2].elapsed_time(e[3]) for e in me) / km
            modes[name] = {"ms_per_call": round(m_call, 4), "pool_ms": round(m_pool, 4), "attend_ms": round(m_att, 4),
                           "attend_vs_default": round(t_att / m_att, 3)}
            print(f"# {name}: {m_call:.3f} ms/call (pool {m_pool:.3f}, attend {m_att:.3f})", file=sys.stderr,
                  flush=True)
            del mws, mplan
        # Q, K, V as strided views of one fused [B, N, 3, H, D] projection
        # output (no copies), same routing and output
        fused = torch.stack([q, k, v], dim=2)
        fq, fk, fv = fused[:, :, 0], fused[:, :, 1], fused[:, :, 2]
        mplan = binding.SparseAttnPlan(B, N, H, D, prefix_len=w.prefix_len, in_strides=fq.stride()[:3], **rkw)
        mws = mplan.workspace(dev)
        for _ in range(2):
            mplan.forward(fq, fk, fv, out=out, ws=mws)
        torch.cuda.synchronize()
        km = max(3, K // 2)
        me = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(km)]
        for i in range(km):
            me[i][0].record(stream)
            mplan.pool(fq, fk, fv, mws)
            me[i][1].record(stream)
            mplan.select(mws)
            me[i][2].record(stream)
            mplan.attend(fq, out, mws)
            me[i][3].record(stream)
        torch.cuda.synchronize()
        m_call = sum(e[0].elapsed_time(e[3]) for e in me) / km
        m_pool = sum(e[0].elapsed_time(e[1]) for e in me) / km
        m_att = sum(e[2].elapsed_time(e[3]) for e in me) / km
        modes["strided_qkv"] = {"ms_per_call": round(m_call, 4), "pool_ms": round(m_pool, 4), "attend_ms": round(m_att, 4),
                                "attend_vs_default": round(t_att / m_att, 3)}
        print(f"# strided_qkv: {m_call:.3f} ms/call (pool {m_pool:.3f}, attend {m_att:.3f})", file=sys.stderr,
              flush=True)
        del mws, mplan, fq, fk, fv, fused
        # Spark-Reblock runs through the forward call (the partition, then the
        # path reading Q, K, V rows through the final order and writing each
        # output row at its own position)
        mplan = binding.SparseAttnPlan(B, N, H, D, prefix_len=w.prefix_len, reblock=True, **rkw)
        mws = mplan.workspace(dev)
        for _ in range(2):
            mplan.forward(q, k, v, out=out, ws=mws)
        torch.cuda.synchronize()
        km = max(3, K // 2)
        r0_ev, r1_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0_ev.record(stream)
        for _ in range(km):
            mplan.forward(q, k, v, out=out, ws=mws)
        r1_ev.record(stream)
        torch.cuda.synchronize()
        m_call = r0_ev.elapsed_time(r1_ev) / km
        rb_flops, rb_density = selected_flops(mplan, mws, N, D)
        modes["reblock"] = {"ms_per_call": round(m_call, 4), "density": round(rb_density, 5),
                            "selected_tflop_per_call": round(rb_flops / 1e12, 4)}
        print(f"# reblock: {m_call:.3f} ms/call, density {rb_density:.4f}", file=sys.stderr, flush=True)
        del mws, mplan
        torch.cuda.empty_cache()

    dense_flops = 4.0 * B * H * N * N * D
    # pool = pool_q (reads Q, writes Qbar) + pack_kv (reads K, V; writes Kbar,
    # Vbar, the packed K and V^T tiles and the packed bf16 centroids).  The
    # algorithmic bytes of the step are Q, K, V read and the fp32 means
    # written; the packed tiles the attend kernel copies from are written on
    # top of that.
    nbp = plan.layout["n_blocks_padded"]
    pool_alg_bytes = 3 * B * N * H * D * 2 + 3 * B * H * nb * D * 4
    pool_bytes = pool_alg_bytes + 2 * B * H * nb * 64 * D * 2 + 2 * B * H * nbp * D * 2
    sel_bytes = 2 * B * H * nb * D * 4 + B * H * nb * 4 + density * B * H * nb * nb * 4
    achieved = flops / (t_att * 1e-3) / 1e12
    traffic = _traffic(args.workload)

    result = {
        "metric": "ms/call + effective TFLOP/s, sparse attn N=32768 H=56 D=128 vs own dense",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s (selected-block FLOPs / ms per call)",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded clustered generator), inputs resident in HBM",
        "config": {
            "workload": args.workload,
            "B": B, "N": N, "H": H, "D": D,
            "routing": rkw, "prefix_len": w.prefix_len,
            "centroid": True, "logmass_bias": True,
        },
        "density": round(density, 5),
        "selected_tflop_per_call": round(flops / 1e12, 4),
        "attend_mfma_per_launch": attend_mfma_count(plan, ws, D),
        "graph_ms_per_call": None if graph_ms is None else round(graph_ms, 4),
        "dense_ms_per_call": None if dense_ms is None else round(dense_ms, 3),
        "speedup_vs_own_dense": None if dense_ms is None else round(dense_ms / ms_step, 3),
        "dense_equivalent_tflops": round(dense_flops / (ms_step * 1e-3) / 1e12, 2),
        "own_dense_tflops": None if dense_ms is None else round(dense_flops / (dense_ms * 1e-3) / 1e12, 2),
        "kernels_ms": {"pool": round(t_pool, 4), "select": round(t_sel, 4), "attend": round(t_att, 4)},
        "modes": modes,
        "pool_gbs": round(pool_alg_bytes / (t_pool * 1e-3) / 1e9, 1),
        "pool_gbs_with_packed_writes": round(pool_bytes / (t_pool * 1e-3) / 1e9, 1),
        "select_gbs": round(sel_bytes / (t_sel * 1e-3) / 1e9, 1),
        "roofline": {
            "kernel": "attend_kernel<128, 2, false, false>",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "mfma_counters": _mfma_busy(args.workload),
        },
        "context": "pages' RTX 5090 figures at N=32768, H=56 (density 0.08): SDPA 144.5 ms, Sol-Attn 16.06 ms; other hardware and inputs, not a target",
    }
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a sample ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
