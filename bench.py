"""Benchmark of the HiNM sparse-weight x dense-activation product on one MI355X.

Workload: LLaMA-7B down_proj weight 4096 x 11008 (cout x cin) in bf16, HiNM
packed with tile_rows 64, t_s 0.75, v_s 0.55 (550 dense / 4404 2:4 / 6054
pruned vectors per tile), random per-tile input permutations; X bf16
[11008 x batch].  A step is one product Y = (W (.) M) X at batch 2048 (the
compute-bound point); the batch-16 product (the bandwidth-bound point) and
the one-time pack are timed beside it and reported in the same JSON line.

Inputs are resident in HBM before timing starts; successive steps rotate
through enough copies of the packed weight, X and Y (>= 1 GiB) that the
256 MB last-level cache cannot serve a repeat.  The K timed steps are one
replay of a HIP graph holding K products (captured once, replayed once
untimed first), bracketed by device synchronisation and timed with HIP
events on the replaying stream: the products run back to back as a serving
loop would issue them, without the Python binding's per-call host cost
(about 10 us, which exceeds a batch-16 product).  Eager per-call times are
reported beside.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
ROTATE_BYTES = 1 << 30
WARM_REPLAYS = 10              # untimed graph replays, back to back, before each timed replay


def log(msg: str) -> None:
    """Progress line on stderr (the JSON result is the only stdout line)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=2048)
    ap.add_argument("--decode-batch", type=int, default=16)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense torch.matmul comparator")
    ap.add_argument("--no-stack", action="store_true", help="skip the 32-layer stack batch sweep")
    ap.add_argument("--profile-only", type=int, default=0, metavar="K",
                    help="run K products at each batch plus a 256 MiB calibration copy, print nothing else "
                         "(for rocprofv3 runs)")
    return ap.parse_args()


CALIB_BYTES = 256 << 20        # size of the plain copy used to scale the HBM byte counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_down_proj_4096x11008.md")
KERNEL_SOURCES = ("structured_sparse_gemm_amd/csrc/hinm_spmm.hip", "structured_sparse_gemm_amd/csrc/hinm_plan.cpp")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(batch):
    """HBM bytes per launch from the committed counter summary, if it matches this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, ValueError, IndexError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    ent = rec.get("per_launch", {}).get(str(batch))
    return None if ent is None else ent.get("hbm_bytes")


def algorithmic(p, batch):
    """Algorithmic bytes and flops of one product (padding excluded)."""
    kept = p.cin - p.z
    val = p.cout * kept * 2
    meta = p.cout * p.n_24 // 8
    idx = p.n_tiles * (p.n_dense + p.n_24) * 4
    xb = p.cin * batch * 2
    yb = p.cout * batch * 2
    return {"bytes": val + meta + idx + xb + yb, "useful_flops": 2 * p.cout * kept * batch,
            "dense_equiv_flops": 2 * p.cout * p.cin * batch,
            "executed_flops": 2 * p.cout * (p.n_dense_pad + p.n_24_pad // 2) * batch}


class Rotation:
    """k copies of (packed weight, X, Y) so that k * bytes >= ROTATE_BYTES."""

    def __init__(self, hinm, torch, pk, x, batch):
        per = pk.nbytes() + x.numel() * 2 + pk.plan.cout * batch * 2
        self.k = max(2, -(-ROTATE_BYTES // per))
        self.items = []
        for i in range(self.k):
            pki = pk if i == 0 else hinm.HinmPacked(pk.plan, pk.val_dense.clone(), pk.idx_dense.clone(),
                                                    pk.val_24.clone(), pk.meta_24.clone(), pk.idx_24.clone())
            xi = x if i == 0 else x.clone()
            yi = torch.empty(pk.plan.cout, batch, dtype=torch.bfloat16, device=x.device)
            self.items.append((pki, xi, yi))
        ws_bytes = hinm.spmm_workspace_bytes(pk.plan, batch)
        self.ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)

    def __getitem__(self, i):
        return self.items[i % self.k]


def time_spmm(hinm, torch, rot, steps, warmup):
    """Per-step times from HIP events on the launching stream, plus the whole-loop time."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        pk, x, y = rot[i]
        hinm.spmm(pk, x, out=y, workspace=rot.ws)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        pk, x, y = rot[warmup + i]
        hinm.spmm(pk, x, out=y, workspace=rot.ws)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    total_ms = ev[0].elapsed_time(ev[steps])
    return {"ms_total": total_ms, "ms_mean": total_ms / steps, "ms_median": per[len(per) // 2],
            "ms_p10": per[len(per) // 10], "ms_p90": per[(9 * len(per)) // 10], "wall_s": wall}


def time_spmm_graph(hinm, torch, rot, steps, extra=4, out_rows=None):
    """Time of exactly `steps` products launched from one HIP graph.

    Product i uses rotation copy i % k.  The graph is captured on a side
    stream and replayed WARM_REPLAYS times back to back untimed (the clock
    settles only after tens of milliseconds of continuous work: a traced run
    shows the batch-2048 product falling from 116 to 99 us over its first
    eight passes); the timed region is one replay,
    bracketed by device synchronisation, with HIP events on the replaying
    stream.  A graph launches the products back to back with no host work in
    between, so short products are not bound by the host's per-call cost.
    `extra` further replays give the spread (per-step time of each replay).
    """
    def run():
        for i in range(steps):
            pk, x, y = rot[i]
            hinm.spmm(pk, x, out=y, workspace=rot.ws, out_rows=out_rows)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for _ in range(WARM_REPLAYS):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 + extra)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    g.replay()
    ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(extra):
        g.replay()
        ev[2 + i].record(stream)
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[1])
    per = sorted([total_ms / steps] + [ev[1 + i].elapsed_time(ev[2 + i]) / steps for i in range(extra)])
    return {"ms_total": total_ms, "ms_mean": total_ms / steps, "steps": steps, "wall_s": wall,
            "replay_ms_per_step_min": per[0], "replay_ms_per_step_max": per[-1]}


def time_dense(torch, w, x, steps, warmup):
    """torch.matmul of the unpruned weight, timed like the products: one replay of a graph of `steps` calls."""
    y = torch.empty(w.shape[0], x.shape[1], dtype=torch.bfloat16, device=x.device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(warmup):
            torch.matmul(w, x, out=y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            torch.matmul(w, x, out=y)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


STACK_LAYERS = 32
STACK_BATCHES = (1, 16, 64, 256, 1024, 2048, 4096)


def stack_sweep(hinm, torch, synth, dev, with_dense):
    """The 7B-shaped stack: 32 layers x {q, k, v, o 4096x4096; gate, up 11008x4096;
    down 4096x11008}, HiNM packed once (tile_rows 64, t_s 0.75, v_s 0.55), and
    the sum of all linear-layer products of one forward pass at each batch.

    Weights are drawn on the device (iid N(0, 0.02), importance |W|, random
    per-tile permutations): the product's time depends on the shapes and the
    region counts only.  The 224 products of a forward are captured in one
    HIP graph (X and Y buffers shared by the projections of the same shape),
    replayed untimed, then timed over one replay with HIP events.  The packed
    stack (3.4 GB) is well past the 256 MB last-level cache, so every weight
    comes from HBM.  The dense comparator runs torch.matmul on the unpruned
    bf16 weights (13 GB) the same way.
    """
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    packs, dense = [], []
    t0 = time.perf_counter()
    for _layer in range(STACK_LAYERS):
        for _name, cout, cin in synth.STACK_PROJS:
            w = (torch.randn(cout, cin, device=dev, generator=g) * 0.02).to(torch.bfloat16)
            imp = w.float().abs()
            perm = torch.rand(cout // 64, cin, device=dev, generator=g).argsort(dim=1).to(torch.int32)
            packs.append(hinm.pack(w, imp, 64, 0.75, 0.55, perm))
            del imp, perm
            if with_dense:
                dense.append(w)
            else:
                del w
    pack_s = time.perf_counter() - t0

    def run_graph(fn, replays=3):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        for _ in range(replays):
            graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        del graph
        return ms

    rows = []
    for B in STACK_BATCHES:
        xs = {c: torch.randn(c, B, device=dev, generator=g).to(torch.bfloat16) for c in (4096, 11008)}
        ys = {c: torch.empty(c, B, dtype=torch.bfloat16, device=dev) for c in (4096, 11008)}
        ws_bytes = max(hinm.spmm_workspace_bytes(pk.plan, B) for pk in packs[:7])
        ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        useful = sum(2 * pk.plan.cout * (pk.plan.cin - pk.plan.z) * B for pk in packs)

        def fwd():
            for pk in packs:
                hinm.spmm(pk, xs[pk.plan.cin], out=ys[pk.plan.cout], workspace=ws)
        ms = run_graph(fwd)
        log(f"stack batch {B}: {ms:.3f} ms per forward")
        row = {"batch": B, "ms_per_forward": round(ms, 4), "useful_tflops": round(useful / (ms * 1e-3) / 1e12, 2)}
        if with_dense:
            def fwd_dense():
                for i, wt in enumerate(dense):
                    _n, cout, cin = synth.STACK_PROJS[i % 7]
                    torch.matmul(wt, xs[cin], out=ys[cout])
            dms = run_graph(fwd_dense)
            row["dense_ms_per_forward"] = round(dms, 4)
            row["speedup_vs_dense"] = round(dms / ms, 3)
        rows.append(row)
        del xs, ys, ws
    packed_gb = sum(pk.nbytes() for pk in packs) / 1e9
    del packs, dense
    torch.cuda.empty_cache()
    return {"what": "32-layer 7B-shaped stack (q, k, v, o 4096x4096; gate, up 11008x4096; down 4096x11008), "
                    "tile_rows 64, t_s 0.75, v_s 0.55, packed once; time of all 224 linear-layer products of one "
                    "forward pass, one HIP graph replay after three untimed ones",
            "packed_gb": round(packed_gb, 3), "pack_all_s": round(pack_s, 2), "per_batch": rows}


def cpu_baseline(w, batch):
    """The CPU oracle as it stands: pack, then the float64 product, on this host's cores."""
    import numpy as np

    import oracle.hinm as oh
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    p = oh.plan(w.cout, w.cin, w.tile_rows, w.t_s, w.v_s)
    bits = w.w_bf16.view(__import__("torch").int16).numpy().view(np.uint16)
    t0 = time.perf_counter()
    _, inter = oh.pack(bits, w.importance.numpy(), w.perm.numpy(), p, with_intermediates=True)
    t_pack = time.perf_counter() - t0
    wh = oh.masked_weight(bits, inter["mask"])
    xf = synth.as_f64(w.x_bf16)
    t0 = time.perf_counter()
    oh.spmm(wh, xf)
    t_first = time.perf_counter() - t0
    # repeat the product for about 10 s so that the rate is not one short timing
    reps = max(1, min(200, int(10.0 / max(t_first, 1e-3))))
    t0 = time.perf_counter()
    for _ in range(reps):
        oh.spmm(wh, xf)
    t_prod = (time.perf_counter() - t0) / reps
    useful = 2 * p.cout * (p.cin - p.z) * batch
    return {"value": round(useful / t_prod / 1e12, 4), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"whole workload: oracle pack of the 4096x11008 weight once ({t_pack:.2f} s), then its "
                       f"float64 product at batch {batch} {reps} times ({t_prod:.3f} s each, {t_prod * reps:.1f} s); "
                       f"value = useful flops / mean product time"),
            "pack_s": round(t_pack, 3), "product_s": round(t_prod, 4), "product_reps": reps,
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}



def cpu_baseline_boundary(wb):
    """CPU-baseline leg for the boundary-search row: the oracle's cost of one grid point of the same search
    (retained importance at v_s 0.6, t_s 0.7), the vector scores computed beforehand."""
    import oracle.hinm as oh
    p_b = oh.plan(wb.cout, wb.cin, 64, 0.7, 0.7)
    s_b = oh.vector_scores(wb.importance.numpy(), p_b)
    t0 = time.perf_counter()
    oh.retained_importance(wb.importance.numpy(), wb.perm.numpy(), oh.plan(wb.cout, wb.cin, 64, 0.7, 0.6), s_b)
    return {"oracle_s_per_grid_point": round(time.perf_counter() - t0, 3),
            "oracle_sample": "one grid point (v_s 0.6) of the same search, scores precomputed"}


def cpu_baseline_gyro(w, g_sample, g_init, g_cs, g_it):
    """CPU-baseline leg for the gyro-permutation row: one oracle round on tiles 0 and 1 with the same draws,
    scaled to all tiles."""
    import oracle.gyro as og
    import oracle.hinm as oh
    dd = w.importance.numpy()
    op = oh.plan(w.cout, w.cin, w.tile_rows, w.t_s, w.v_s)
    reg = oh.regions(oh.vector_scores(dd, op), op)
    _, idx_s = oh.index_lists(reg, w.perm.numpy().astype("int64"), op)
    t0 = time.perf_counter()
    for t in range(2):
        og.gyro_round(dd[t * 64:(t + 1) * 64], idx_s[t, :op.n_24].reshape(op.groups, 4).astype("int64"),
                      g_sample[0, t].astype("int64"), g_init[0, t].astype("int64"), g_cs, g_it)
    return {"oracle_s_per_round_all_tiles": round((time.perf_counter() - t0) / 2 * op.n_tiles, 2),
            "oracle_sample": "one round on tiles 0 and 1, scaled to all tiles"}

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the product shards by output tiles with no exchange, see the design notes).", file=sys.stderr)
        sys.exit(2)
    import torch

    import structured_sparse_gemm_amd as hinm
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, Bd = args.batch, args.decode_batch
    w = synth.down_proj(batch=B)
    wd_ = synth.down_proj(batch=Bd)          # same weight and perms (same seed), batch-16 activations
    p = hinm.plan(w.cout, w.cin, w.tile_rows, w.t_s, w.v_s)

    wgpu, igpu, pgpu = w.w_bf16.to(dev), w.importance.to(dev), w.perm.to(dev)
    torch.cuda.synchronize()
    pack_ms = []
    for _ in range(3):
        t0 = time.perf_counter()
        pk = hinm.pack(wgpu, igpu, w.tile_rows, w.t_s, w.v_s, pgpu)
        pack_ms.append((time.perf_counter() - t0) * 1e3)
    x = w.x_bf16.to(dev)
    xd = wd_.x_bf16.to(dev)

    if args.profile_only:
        y = torch.empty(p.cout, B, dtype=torch.bfloat16, device=dev)
        yd = torch.empty(p.cout, Bd, dtype=torch.bfloat16, device=dev)
        for _ in range(args.profile_only):
            hinm.spmm(pk, x, out=y)
            hinm.spmm(pk, xd, out=yd)
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)                      # calibration: reads and writes CALIB_BYTES once
        torch.cuda.synchronize()
        return

    log(f"packed: {[round(v, 2) for v in pack_ms]} ms; timing batch {B}")
    rot = Rotation(hinm, torch, pk, x, B)
    r_eager = time_spmm(hinm, torch, rot, args.steps, args.warmup)
    r = time_spmm_graph(hinm, torch, rot, args.steps)
    alg = algorithmic(p, B)
    ms = r["ms_mean"]
    value = alg["useful_flops"] / (ms * 1e-3) / 1e12

    log(f"batch {B}: {ms * 1e3:.2f} us per product; timing batch {Bd}")
    rotd = Rotation(hinm, torch, pk, xd, Bd)
    rd_eager = time_spmm(hinm, torch, rotd, max(args.steps, 200), args.warmup)
    steps_d = max(args.steps, 200)
    rd = time_spmm_graph(hinm, torch, rotd, steps_d)
    algd = algorithmic(p, Bd)
    gbs_d = algd["bytes"] / (rd["ms_mean"] * 1e-3) / 1e9

    log(f"batch {Bd}: {rd['ms_mean'] * 1e3:.2f} us per product; side rows")
    # NEXT row: output-channel permutation fused into the write-out, and the
    # one-time cross-layer index translation
    out_rows = torch.from_numpy(__import__("numpy").random.default_rng(0).permutation(p.cout).astype("int32")).to(dev)
    r_rows = time_spmm_graph(hinm, torch, rot, args.steps, extra=0, out_rows=out_rows)
    rd_rows = time_spmm_graph(hinm, torch, rotd, steps_d, extra=0, out_rows=out_rows)
    sigma = torch.from_numpy(__import__("numpy").random.default_rng(1).permutation(p.cin).astype("int32")).to(dev)
    pk_t = hinm.HinmPacked(pk.plan, pk.val_dense, pk.idx_dense.clone(), pk.val_24, pk.meta_24, pk.idx_24.clone())
    tr_ms = []
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        hinm.translate_indices(pk_t, sigma)
        tr_ms.append((time.perf_counter() - t0) * 1e3)
    next_rows = {"what": "hinm_spmm_rows (Y row r written to out_rows[r]) next to hinm_spmm, same timing method; "
                         "hinm_translate_indices wall time (synchronous, includes the permutation check)",
                 "spmm_rows_batch_2048_ms": round(r_rows["ms_mean"], 5), "spmm_batch_2048_ms": round(ms, 5),
                 "spmm_rows_batch_16_ms": round(rd_rows["ms_mean"], 5), "spmm_batch_16_ms": round(rd["ms_mean"], 5),
                 "translate_indices_ms": [round(v, 3) for v in tr_ms]}

    # NEXT row: the boundary search for v_s on the device (down_proj sweep workload, t_s 0.7)
    wb_ = synth.down_proj_sweep(0.7)
    imp_b, perm_b = wb_.importance.to(dev), wb_.perm.to(dev)
    hinm.boundary_search(imp_b, perm_b, 64, 0.7)
    torch.cuda.synchronize()
    bs_ms = []
    for _ in range(3):
        t0 = time.perf_counter()
        v_b, tr_b = hinm.boundary_search(imp_b, perm_b, 64, 0.7)
        bs_ms.append((time.perf_counter() - t0) * 1e3)
    next_bs = {"what": "hinm_boundary_search wall time, down_proj 4096x11008 with 5% outlier columns, importance W*W, "
                       "t_s 0.7 (synchronous: checks, scores, ranking, then one device pass and one host read per grid "
                       "point)", "ms": [round(x, 2) for x in bs_ms], "v_s": v_b, "grid_points": len(tr_b)}
    if not args.no_cpu:
        next_bs.update(cpu_baseline_boundary(wb_))

    # NEXT row: per-tile v_s (per-tile boundary search on the same weight and importance, then the
    # per-tile layout), products timed like the uniform ones but without buffer rotation
    t0 = time.perf_counter()
    v_tiles, _ = hinm.boundary_search_tiles(igpu, pgpu, w.tile_rows, w.t_s)
    search_tiles_ms = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    pk_tiles = hinm.pack_tiles(wgpu, igpu, w.tile_rows, w.t_s, v_tiles, pgpu)
    pack_tiles_ms = (time.perf_counter() - t0) * 1e3

    def graph_ms(fn, steps):
        s_ = torch.cuda.Stream()
        s_.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_):
            fn()
        torch.cuda.current_stream().wait_stream(s_)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                fn()
        for _ in range(WARM_REPLAYS):
            g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(5):            # median of five replays: single replays vary by several percent
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            g.replay()
            b_.record()
            torch.cuda.synchronize()
            times.append(a_.elapsed_time(b_) / steps)
        return sorted(times)[2]

    y_t = torch.empty(p.cout, B, dtype=torch.bfloat16, device=dev)
    yd_t = torch.empty(p.cout, Bd, dtype=torch.bfloat16, device=dev)
    ws_t = torch.zeros(max(1, hinm.spmm_tiles_workspace_bytes(pk_tiles.plan, Bd)), dtype=torch.uint8, device=dev)
    costs = [(int(r[1]) + 31) // 32 + 2 * ((int(r[3]) + 63) // 64) for r in pk_tiles.plan.tiles]
    kept_t = sum(int(r[1]) + int(r[3]) // 2 for r in pk_tiles.plan.tiles)       # kept entries per row, summed over tiles
    useful_t = 2 * p.tile_rows * kept_t * B
    next_tiles = {
        "what": "per-tile v_s from hinm_boundary_search_tiles on this weight (importance |W|, t_s 0.75), packed by "
                "hinm_pack_tiles, products by hinm_spmm_tiles; graph-timed (median of five replays) on one resident "
                "copy, beside the uniform product timed the same way; tile cost = dense blocks + 2 x 2:4 blocks "
                "(X rows gathered / 32)",
        "v_s_min": round(min(v_tiles), 5), "v_s_max": round(max(v_tiles), 5),
        "dense_blocks": pk_tiles.plan.dense_blocks, "blocks_24": pk_tiles.plan.blocks_24,
        "uniform_dense_blocks": p.n_tiles * p.n_dense_pad // 32, "uniform_blocks_24": p.n_tiles * p.n_24_pad // 64,
        "search_tiles_ms": round(search_tiles_ms, 2), "pack_tiles_ms": round(pack_tiles_ms, 2),
        "spmm_tiles_batch_2048_ms": round(graph_ms(lambda: hinm.spmm(pk_tiles, x, out=y_t), 20), 5),
        "spmm_uniform_resident_batch_2048_ms": round(graph_ms(lambda: hinm.spmm(pk, x, out=y_t), 20), 5),
        "spmm_tiles_batch_16_ms": round(graph_ms(lambda: hinm.spmm(pk_tiles, xd, out=yd_t, workspace=ws_t), 100), 5),
        "spmm_uniform_resident_batch_16_ms": round(graph_ms(lambda: hinm.spmm(pk, xd, out=yd_t, workspace=ws_t), 100),
                                                   5),
        "tile_cost_min": int(min(costs)), "tile_cost_mean": round(sum(costs) / len(costs), 2),
        "tile_cost_max": int(max(costs)),
        "useful_tflops_batch_2048": None}
    next_tiles["useful_tflops_batch_2048"] = round(useful_t / (next_tiles["spmm_tiles_batch_2048_ms"] * 1e-3) / 1e12, 2)

    # NEXT row: the in-tile input-channel gyro permutation on this weight (importance |W|, the bench's
    # regions), wall time per round; the oracle's round on a sample of tiles beside it
    g_rounds, g_cs, g_it = 2, 32, 5
    n_cl = -(-p.groups // g_cs)
    g_sample, g_init = synth.gyro_draws(11, g_rounds, p.n_tiles, p.groups, n_cl)
    hinm.gyro_permute(igpu, pgpu, p.tile_rows, p.t_s, p.v_s, 0, g_cs, g_it, g_sample[:0], g_init[:0])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_perm, g_trace = hinm.gyro_permute(igpu, pgpu, p.tile_rows, p.t_s, p.v_s, g_rounds, g_cs, g_it, g_sample, g_init)
    torch.cuda.synchronize()
    g_s = time.perf_counter() - t0
    tot24 = float(w.importance.numpy().astype("float64").sum())   # context for the cost: all importance
    next_gyro = {"what": f"hinm_gyro_permute on down_proj 4096x11008, importance |W|, t_s 0.75, v_s 0.55: "
                         f"{p.groups} 2:4 groups per tile, {g_rounds} rounds, clusters of {g_cs} ({n_cl} per tile), "
                         f"{g_it} K-means steps; wall time (synchronous, includes the region lists)",
                 "s_total": round(g_s, 3), "s_per_round": round(g_s / g_rounds, 3),
                 "pruning_cost_before": round(float(g_trace[0].sum()), 3),
                 "pruning_cost_after": round(float(g_trace[-1].sum()), 3),
                 "cost_removed_frac": round(float(1 - g_trace[-1].sum() / g_trace[0].sum()), 5),
                 "total_importance": round(tot24, 3)}
    if not args.no_cpu:
        next_gyro.update(cpu_baseline_gyro(w, g_sample, g_init, g_cs, g_it))

    dense = None
    if not args.no_dense:
        dense_ms = time_dense(torch, wgpu, x, max(10, args.steps // 2), 3)
        dense_ms_d = time_dense(torch, wgpu, xd, 200, 10)
        dense = {"what": "torch.matmul bf16 of the unpruned 4096x11008 weight (hipBLASLt), same shapes, "
                         "timed from one graph replay (no rotation: the dense weight stays in the last-level cache)",
                 "batch_2048_ms": round(dense_ms, 4), "batch_16_ms": round(dense_ms_d, 4),
                 "speedup_batch_2048": round(dense_ms / ms, 3), "speedup_batch_16": round(dense_ms_d / rd["ms_mean"], 3)}

    log("stack sweep")
    stack = None if args.no_stack else stack_sweep(hinm, torch, synth, dev, not args.no_dense)
    log("CPU oracle baseline")

    cpu = None if args.no_cpu else cpu_baseline(w, B)

    line = {
        "metric": "HiNM SpMM effective TFLOP/s + HBM GB/s, 4096x11008 bf16 at batch 16 and 2048",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,0.02) x LogNormal column scales, random per-tile perms)",
        "config": {"workload": "down_proj 4096x11008 HiNM SpMM, tile_rows 64, t_s 0.75, v_s 0.55, batch 2048",
                   "cout": p.cout, "cin": p.cin, "tile_rows": p.tile_rows, "t_s": p.t_s, "v_s": p.v_s,
                   "batch": B, "regions_per_tile": {"dense": p.n_dense, "two_four": p.n_24, "pruned": p.n_pruned}},
        "roofline": {"bound": "mfma", "achieved": round(value, 3), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / MFMA_BF16_PEAK_TFLOPS, 5), "traffic": measured_traffic(B),
                     "kernel": "prefill_kernel<256, false> (one launch per step)",
                     "kernel_source_hash": kernel_source_hash(),
                     "per_launch": {"useful_flops": alg["useful_flops"], "algorithmic_bytes": alg["bytes"],
                                    "ms_mean": round(ms, 5),
                                    "replay_ms_min": round(r["replay_ms_per_step_min"], 5),
                                    "replay_ms_max": round(r["replay_ms_per_step_max"], 5)},
                     "timing": f"one HIP graph replay of {args.steps} products over {rot.k} rotated copies, after "
                               f"{WARM_REPLAYS} untimed replays; "
                               f"eager launches from Python: {r_eager['ms_mean'] * 1e3:.1f} us per step",
                     "eager_ms_mean": round(r_eager["ms_mean"], 5),
                     "rotation_copies": rot.k},
        "decode": {"batch": Bd, "ms_mean": round(rd["ms_mean"], 5),
                   "replay_ms_min": round(rd["replay_ms_per_step_min"], 5),
                   "replay_ms_max": round(rd["replay_ms_per_step_max"], 5),
                   "timing": f"one HIP graph replay of {steps_d} products over {rotd.k} rotated copies, after "
                             f"{WARM_REPLAYS} untimed replays; "
                             f"eager launches from Python: {rd_eager['ms_mean'] * 1e3:.1f} us per call",
                   "eager_ms_mean": round(rd_eager["ms_mean"], 5),
                   "algorithmic_bytes": algd["bytes"], "hbm_gbs": round(gbs_d, 1),
                   "roofline": {"bound": "hbm", "achieved": round(gbs_d, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(gbs_d / HBM_PEAK_GBS, 4), "traffic": measured_traffic(Bd),
                                "kernel": "decode5_kernel<16,24,true,2> (one launch per call)"},
                   "useful_tflops": round(algd["useful_flops"] / (rd["ms_mean"] * 1e-3) / 1e12, 3),
                   "rotation_copies": rotd.k},
        "batch_2048_hbm_gbs": round(alg["bytes"] / (ms * 1e-3) / 1e9, 1),
        "pack_ms": [round(v, 2) for v in pack_ms],
        "next_output_permutation": next_rows,
        "next_boundary_search": next_bs,
        "next_per_tile_v_s": next_tiles,
        "next_gyro_permutation": next_gyro,
        "dense_comparator": dense,
        "stack_sweep": stack,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
