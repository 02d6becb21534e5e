"""Benchmark of the HiNM sparse-weight x dense-activation product on one MI355X.

Headline workload: LLaMA-7B down_proj weight 4096 x 11008 (cout x cin) in
bf16, HiNM packed with tile_rows 64, t_s 0.75, v_s 0.55 (550 dense / 4404 2:4
/ 6054 pruned vectors per tile), random per-tile input permutations; X bf16
[11008 x batch].  A step is one product Y = (W (.) M) X at batch 2048 (the
compute-bound point); the batch-16 product (the bandwidth-bound point) and
the one-time pack are timed beside it and reported in the same JSON line,
with one row per workload and batch of the five configurations (each with
its roofline fractions), the 13-point batch sweep of the 32-layer 7B-shaped
stack, the dense torch.matmul comparator, the GPU's empirical peaks and its
clocks, the side rows (output-row map, boundary search, per-tile v_s, gyro
permutation, block-diagonal perms) and the CPU oracle baseline.

Inputs are resident in HBM before timing starts; successive products rotate
through enough copies of the packed weight, X and Y (>= 1 GiB) that the
256 MB last-level cache cannot serve a repeat, and so does the dense
comparator's weight.  The K timed steps are one replay of a HIP graph
holding K products (captured once, replayed ten times untimed first),
bracketed by device synchronisation and timed with HIP events on the
replaying stream: the products run back to back as a serving loop would
issue them, without the Python binding's per-call host cost (about 10 us,
which exceeds a batch-16 product).  Further replays give the median, p10
and p90.  Eager per-call times are reported beside.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-stack] [--no-configs]
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
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration rows")
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


REPLAYS = 7                    # timed graph replays behind each spread (median, p10, p90)


def graph_replays(torch, run, steps, replays=REPLAYS):
    """Per-product times of `run` (which launches `steps` products) from a HIP graph.

    The graph is captured once on a side stream and replayed WARM_REPLAYS
    times back to back untimed (the clock settles only after tens of
    milliseconds of continuous work: a traced run shows the batch-2048
    product falling from 116 to 99 us over its first eight passes).  Then
    `replays` timed replays, each bracketed by device synchronisation and
    timed with HIP events on the replaying stream.  The first timed replay is
    the step time; the others give the spread.  A graph launches the products
    back to back with no host work in between, so short products are not
    bound by the host's per-call cost.
    """
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
    per = []
    wall = None
    for i in range(replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        if i == 0:
            wall = time.perf_counter() - t0
        per.append(a.elapsed_time(b) / steps)
    srt = sorted(per)
    q = lambda f: srt[min(len(srt) - 1, int(round(f * (len(srt) - 1))))]
    del g
    return {"ms_step": per[0], "ms_median": q(0.5), "ms_p10": q(0.1), "ms_p90": q(0.9), "ms_min": srt[0],
            "ms_max": srt[-1], "replays": replays, "steps": steps, "wall_s": wall}


def time_spmm_graph(hinm, torch, rot, steps, out_rows=None, replays=REPLAYS):
    """Graph-timed products over the rotation copies (product i uses copy i % k)."""
    def run():
        for i in range(steps):
            pk, x, y = rot[i]
            hinm.spmm(pk, x, out=y, workspace=rot.ws, out_rows=out_rows)
    return graph_replays(torch, run, steps, replays)


def spread(r):
    return {"ms_median": round(r["ms_median"], 5), "ms_p10": round(r["ms_p10"], 5), "ms_p90": round(r["ms_p90"], 5)}


def time_dense(torch, w, x, steps, replays=REPLAYS):
    """torch.matmul (hipBLASLt) of the unpruned weight at the same shape, timed like the products: the
    weight rotates over copies of >= 1 GiB in all, so the last-level cache does not serve repeats."""
    k = max(2, -(-ROTATE_BYTES // (w.numel() * 2 + x.numel() * 2 + w.shape[0] * x.shape[1] * 2)))
    ws = [w] + [w.clone() for _ in range(k - 1)]
    xs = [x] + [x.clone() for _ in range(k - 1)]
    ys = [torch.empty(w.shape[0], x.shape[1], dtype=torch.bfloat16, device=x.device) for _ in range(k)]

    def run():
        for i in range(steps):
            torch.matmul(ws[i % k], xs[i % k], out=ys[i % k])
    r = graph_replays(torch, run, steps, replays)
    r["rotation_copies"] = k
    del ws, xs, ys
    return r


def fracs(alg, ms, batch):
    """Throughputs of one product and their fractions of the MI355X peaks; the bound is HBM up to batch
    256, MFMA from batch 1024, both near the ridge (512)."""
    gbs = alg["bytes"] / (ms * 1e-3) / 1e9
    tfl = alg["useful_flops"] / (ms * 1e-3) / 1e12
    bound = "hbm" if batch <= 256 else ("mfma" if batch >= 1024 else "ridge")
    return {"hbm_gbs": round(gbs, 1), "useful_tflops": round(tfl, 3), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "frac_mfma": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4), "bound": bound,
            "frac": round(gbs / HBM_PEAK_GBS if bound == "hbm" else tfl / MFMA_BF16_PEAK_TFLOPS, 4)}


def config_rows(hinm, torch, synth, dev, steps, with_dense):
    """One row per workload and batch of the five configurations that a single product covers (the
    stack is its own sweep): the product graph-timed over >= 1 GiB of rotated copies, its algorithmic
    bytes and useful flops, the roofline fractions, and (for the two orientations of the 4096 x 11008
    headline shape and q_proj) the dense torch.matmul beside it."""
    rows = []
    cases = [("tiny 128x256 (fp32 drawn, bf16 path), tile_rows 32, t_s 0.75, v_s 0.5", synth.tiny(), None, (8,)),
             ("q_proj 4096x4096, t_s 0.5, v_s 0.25", synth.q_proj(batch=16), None, (16,)),
             ("up_proj 11008x4096, t_s 0.75, v_s 0.55", synth.up_proj(batch=16), None, (16, 2048)),
             ("down_proj 4096x11008, t_s 0.75, v_s 0.55", synth.down_proj(batch=16), None, (16, 2048))]
    for t in (0.6, 0.7, 0.8):
        w = synth.down_proj_sweep(t, batch=1)
        # v_s from the boundary search on the device (equal to the oracle's search, tested)
        v, _ = hinm.boundary_search(w.importance.to(dev), w.perm.to(dev), 64, t)
        cases.append((f"down_proj sweep 4096x11008 (5% outlier columns x10, importance W^2), t_s {t}, v_s {v:.4f} "
                      f"(device boundary search)", w, v, (1, 64, 512)))
    dense_for = {"q_proj", "up_proj", "down_proj"}
    for name, w, v_s, batches in cases:
        v = w.v_s if v_s is None else v_s
        pk = hinm.pack(w.w_bf16.to(dev), w.importance.to(dev), w.tile_rows, w.t_s, v, w.perm.to(dev))
        p = pk.plan
        wd = w.w_bf16.to(dev) if with_dense and name.split()[0] in dense_for else None
        for B in batches:
            x = torch.randn(p.cin, B, device=dev, generator=torch.Generator(device=dev).manual_seed(B)).to(
                torch.bfloat16)
            rot = Rotation(hinm, torch, pk, x, B)
            nst = max(steps, 200) if B <= 64 else steps
            r = time_spmm_graph(hinm, torch, rot, nst)
            alg = algorithmic(p, B)
            row = {"workload": name, "batch": B, "ms": round(r["ms_step"], 5), **spread(r),
                   "rotation_copies": rot.k, "algorithmic_bytes": alg["bytes"], "useful_flops": alg["useful_flops"],
                   "regions_per_tile": {"dense": p.n_dense, "two_four": p.n_24, "pruned": p.n_pruned},
                   **fracs(alg, r["ms_step"], B)}
            if wd is not None:
                d = time_dense(torch, wd, x, nst)
                row["dense_ms"] = round(d["ms_step"], 5)
                row["dense_rotation_copies"] = d["rotation_copies"]
                row["speedup_vs_dense"] = round(d["ms_step"] / r["ms_step"], 3)
            log(f"{name.split(',')[0]} batch {B}: {r['ms_step'] * 1e3:.2f} us, frac {row['frac']}")
            rows.append(row)
            del rot, x
        del pk, wd
        torch.cuda.empty_cache()
    return rows


def empirical_peaks(torch, dev):
    """What this GPU reaches on plain work, beside the published peaks: a 1 GiB read (sum of fp32), a 1 GiB
    copy (read + write) and torch.matmul bf16 at 8192^3.  Timed eagerly (each call lasts 100 us or more, so
    the launch cost is noise), with HIP events around ten calls after three warm-up calls; the median of
    five such groups."""
    def eager(fn, n=10, groups=5):
        for _ in range(3):
            fn()
        t = []
        for _ in range(groups):
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                fn()
            b.record()
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b) / n)
        return sorted(t)[len(t) // 2]
    n = (1 << 30) // 4
    src = torch.rand(n, device=dev)
    dst = torch.empty_like(src)
    t_read = eager(lambda: torch.sum(src))
    t_copy = eager(lambda: dst.copy_(src))
    del src, dst
    a = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    c = torch.empty(8192, 8192, dtype=torch.bfloat16, device=dev)
    t_mm = eager(lambda: torch.matmul(a, b, out=c))
    del a, b, c
    torch.cuda.empty_cache()
    gib = float(1 << 30)
    return {"read_1gib_gbs": round(gib / (t_read * 1e-3) / 1e9, 1),
            "copy_1gib_gbs": round(2 * gib / (t_copy * 1e-3) / 1e9, 1),
            "matmul_bf16_8192_tflops": round(2 * 8192 ** 3 / (t_mm * 1e-3) / 1e12, 1),
            "what": "torch.sum over 1 GiB of fp32 (read), copy_ of 1 GiB (read + write, counted twice), "
                    "torch.matmul bf16 8192^3 (hipBLASLt); eager, median of five groups of ten calls"}


def gpu_clocks(busy=None):
    """GPU clocks as amd-smi (else rocm-smi) reports them, read in a child process; with `busy`, that
    function keeps the GPU working until the report is in, so the clocks are those under load.  None where
    neither tool answers."""
    import subprocess
    for cmd in (["amd-smi", "metric", "-c", "--json"], ["rocm-smi", "--showclocks", "--json"]):
        try:
            proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
        except OSError:
            continue
        t0 = time.perf_counter()
        while busy is not None and proc.poll() is None and time.perf_counter() - t0 < 20:
            busy()
        try:
            out, _ = proc.communicate(timeout=20)
        except subprocess.TimeoutExpired:
            proc.kill()
            continue
        if proc.returncode == 0 and out.strip():
            try:
                rep = json.loads(out)
            except ValueError:
                rep = out.strip()[:2000]
            return {"tool": cmd[0], "under_load": busy is not None, "report": rep}
    return None


STACK_LAYERS = 32
STACK_BATCHES = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096)


def stack_sweep(hinm, torch, synth, dev, with_dense):
    """The 7B-shaped stack: 32 layers x {q, k, v, o 4096x4096; gate, up 11008x4096;
    down 4096x11008}, HiNM packed once (tile_rows 64, t_s 0.75, v_s 0.55), and
    the sum of all linear-layer products of one forward pass at each of 13
    batches.

    Weights are drawn on the device (iid N(0, 0.02), importance |W|, random
    per-tile permutations): the product's time depends on the shapes and the
    region counts only.  Every layer has its own activations and outputs
    (three inputs of 4096 rows - attention, o, MLP - and one of 11008), so no
    product reads an X that an earlier one left in a cache.  A forward pass
    is timed two ways, each from one HIP graph: grouped (q, k, v in one
    hinm_spmm_group launch, gate and up in another: they read the same X), and
    one launch per product.  The packed stack (3.8 GB) is well past the 256 MB
    last-level cache, so every weight comes from HBM.  The dense comparator
    runs torch.matmul on the unpruned bf16 weights (13 GB) the same way.
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
    layers = [packs[7 * l:7 * l + 7] for l in range(STACK_LAYERS)]
    groups = [(hinm.Group(ly[0:3]), hinm.Group(ly[4:6])) for ly in layers]
    bytes_w = sum(pk.nbytes() for pk in packs)

    rows = []
    for B in STACK_BATCHES:
        gen = torch.Generator(device=dev)
        gen.manual_seed(B)
        xs = [[torch.randn(c, B, device=dev, generator=gen).to(torch.bfloat16) for c in (4096, 4096, 4096, 11008)]
              for _ in range(STACK_LAYERS)]
        ys = [[torch.empty(pk.plan.cout, B, dtype=torch.bfloat16, device=dev) for pk in ly] for ly in layers]
        need = max([hinm.spmm_workspace_bytes(pk.plan, B) for pk in packs[:7]] +
                   [grp.workspace_bytes(B) for grp in groups[0]])
        ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
        useful = sum(2 * pk.plan.cout * (pk.plan.cin - pk.plan.z) * B for pk in packs)
        nbytes = bytes_w + sum(2 * B * (pk.plan.cin + pk.plan.cout) for pk in packs)
        xin = (0, 0, 0, 1, 2, 2, 3)                # which of a layer's four inputs each product reads

        def fwd_grouped():
            for l, ly in enumerate(layers):
                hinm.spmm_group(groups[l][0], xs[l][0], outs=ys[l][0:3], workspace=ws)
                hinm.spmm(ly[3], xs[l][1], out=ys[l][3], workspace=ws)
                hinm.spmm_group(groups[l][1], xs[l][2], outs=ys[l][4:6], workspace=ws)
                hinm.spmm(ly[6], xs[l][3], out=ys[l][6], workspace=ws)

        def fwd_single():
            for l, ly in enumerate(layers):
                for i, pk in enumerate(ly):
                    hinm.spmm(pk, xs[l][xin[i]], out=ys[l][i], workspace=ws)
        rg = graph_replays(torch, fwd_grouped, 1, 5)
        rs = graph_replays(torch, fwd_single, 1, 3)
        ms = rg["ms_step"]
        gbs, tfl = nbytes / (ms * 1e-3) / 1e9, useful / (ms * 1e-3) / 1e12
        bound = "hbm" if B <= 256 else ("mfma" if B >= 1024 else "ridge")
        row = {"batch": B, "ms_per_forward": round(ms, 4), **spread(rg),
               "ms_per_forward_one_launch_per_product": round(rs["ms_step"], 4),
               "useful_tflops": round(tfl, 2), "hbm_gbs": round(gbs, 1), "algorithmic_bytes": nbytes,
               "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "frac_mfma": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
               "bound": bound,
               "frac": round(gbs / HBM_PEAK_GBS if bound == "hbm" else tfl / MFMA_BF16_PEAK_TFLOPS, 4)}
        if with_dense:
            def fwd_dense():
                for l in range(STACK_LAYERS):
                    for i in range(7):
                        torch.matmul(dense[7 * l + i], xs[l][xin[i]], out=ys[l][i])
            rd = graph_replays(torch, fwd_dense, 1, 3)
            row["dense_ms_per_forward"] = round(rd["ms_step"], 4)
            row["speedup_vs_dense"] = round(rd["ms_step"] / ms, 3)
        log(f"stack batch {B}: {ms:.3f} ms per forward grouped, {rs['ms_step']:.3f} one launch per product")
        rows.append(row)
        del xs, ys, ws
        torch.cuda.empty_cache()
    del packs, dense, layers, groups
    torch.cuda.empty_cache()
    return {"what": "32-layer 7B-shaped stack (q, k, v, o 4096x4096; gate, up 11008x4096; down 4096x11008), "
                    "tile_rows 64, t_s 0.75, v_s 0.55, packed once; time of all 224 linear-layer products of one "
                    "forward pass (q/k/v and gate/up grouped into one launch each: 128 launches; beside it one "
                    "launch per product: 224), every layer with its own activations; one HIP graph replay "
                    "after ten untimed ones; algorithmic bytes = packed weights + X and Y of every product",
            "packed_gb": round(bytes_w / 1e9, 3), "pack_all_s": round(pack_s, 2), "per_batch": rows}


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
    pack_times = []
    for _ in range(4):                       # one warm-up, then the median of three
        t0 = time.perf_counter()
        _, inter = oh.pack(bits, w.importance.numpy(), w.perm.numpy(), p, with_intermediates=True)
        pack_times.append(time.perf_counter() - t0)
    t_pack = sorted(pack_times[1:])[1]
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
            "sample": (f"whole workload: oracle pack of the 4096x11008 weight (median of 3 after one warm-up: "
                       f"{t_pack:.2f} s), then its float64 product at batch {batch} {reps} times ({t_prod:.3f} s each, "
                       f"{t_prod * reps:.1f} s); value = useful flops / mean product time"),
            "pack_s": round(t_pack, 3), "product_s": round(t_prod, 4), "product_reps": reps,
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}



def cpu_baseline_stack(batches=(1, 16, 2048)):
    """CPU-baseline leg for the stack sweep: the oracle packs one layer's seven weights (the stack's layer 0),
    then runs their float64 products at each batch; a forward is 32 such layers."""
    import numpy as np
    import torch

    import oracle.hinm as oh
    import synth
    whs, pack_s = [], 0.0
    for proj in range(len(synth.STACK_PROJS)):
        w = synth.stack_layer(0, proj, batch=1)
        p = oh.plan(w.cout, w.cin, w.tile_rows, w.t_s, w.v_s)
        bits = w.w_bf16.view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        _, inter = oh.pack(bits, w.importance.numpy(), w.perm.numpy(), p, with_intermediates=True)
        pack_s += time.perf_counter() - t0
        whs.append(oh.masked_weight(bits, inter["mask"]))
    per = {}
    for b in batches:
        xs = {cin: synth.as_f64(torch.randn(cin, b, generator=torch.Generator().manual_seed(b)).to(torch.bfloat16))
              for cin in sorted({wh.shape[1] for wh in whs})}
        t0 = time.perf_counter()
        for wh in whs:
            oh.spmm(wh, xs[wh.shape[1]])
        per[str(b)] = round((time.perf_counter() - t0) * 32 * 1e3, 1)
    return {"oracle_ms_per_forward": per, "oracle_pack_s_per_layer": round(pack_s, 2),
            "oracle_sample": ("one layer's seven products (layer 0 of the stack, oracle pack then float64 "
                              "products) timed once per batch, times 32 layers")}


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
    import numpy as np
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
        # the products as the timed runs issue them: each on the next rotation copy
        for bb, xx in ((B, x), (Bd, xd)):
            rot = Rotation(hinm, torch, pk, xx, bb)
            for i in range(args.profile_only):
                pki, xi, yi = rot[i]
                hinm.spmm(pki, xi, out=yi, workspace=rot.ws)
            torch.cuda.synchronize()
            del rot
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)                      # calibration: reads and writes CALIB_BYTES once
        torch.cuda.synchronize()
        return

    clocks_idle = gpu_clocks()
    log(f"packed: {[round(v, 2) for v in pack_ms]} ms; timing batch {B}")
    rot = Rotation(hinm, torch, pk, x, B)
    r_eager = time_spmm(hinm, torch, rot, args.steps, args.warmup)
    r = time_spmm_graph(hinm, torch, rot, args.steps)
    alg = algorithmic(p, B)
    ms = r["ms_step"]
    value = alg["useful_flops"] / (ms * 1e-3) / 1e12

    def busy():                              # about 2 ms of the headline products
        for i in range(20):
            pki, xi, yi = rot[i]
            hinm.spmm(pki, xi, out=yi, workspace=rot.ws)
        torch.cuda.synchronize()
    clocks_load = gpu_clocks(busy)
    log(f"batch {B}: {ms * 1e3:.2f} us per product; timing batch {Bd}")
    rotd = Rotation(hinm, torch, pk, xd, Bd)
    steps_d = max(args.steps, 200)
    rd_eager = time_spmm(hinm, torch, rotd, steps_d, args.warmup)
    rd = time_spmm_graph(hinm, torch, rotd, steps_d)
    algd = algorithmic(p, Bd)
    gbs_d = algd["bytes"] / (rd["ms_step"] * 1e-3) / 1e9

    log(f"batch {Bd}: {rd['ms_step'] * 1e3:.2f} us per product; side rows")
    # NEXT row: output-channel permutation fused into the write-out, and the
    # one-time cross-layer index translation
    out_rows = torch.from_numpy(np.random.default_rng(0).permutation(p.cout).astype("int32")).to(dev)
    r_rows = time_spmm_graph(hinm, torch, rot, args.steps, out_rows=out_rows, replays=3)
    rd_rows = time_spmm_graph(hinm, torch, rotd, steps_d, out_rows=out_rows, replays=3)
    sigma = torch.from_numpy(np.random.default_rng(1).permutation(p.cin).astype("int32")).to(dev)
    pk_t = hinm.HinmPacked(pk.plan, pk.val_dense, pk.idx_dense.clone(), pk.val_24, pk.meta_24, pk.idx_24.clone())
    tr_ms = []
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        hinm.translate_indices(pk_t, sigma)
        tr_ms.append((time.perf_counter() - t0) * 1e3)
    next_rows = {"what": "hinm_spmm_rows (Y row r written to out_rows[r]) next to hinm_spmm, same timing method; "
                         "hinm_translate_indices wall time (synchronous, includes the permutation check)",
                 "spmm_rows_batch_2048_ms": round(r_rows["ms_step"], 5), "spmm_batch_2048_ms": round(ms, 5),
                 "spmm_rows_batch_16_ms": round(rd_rows["ms_step"], 5), "spmm_batch_16_ms": round(rd["ms_step"], 5),
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
                       "point)", "ms": [round(v, 2) for v in bs_ms], "v_s": v_b, "grid_points": len(tr_b)}
    if not args.no_cpu:
        next_bs.update(cpu_baseline_boundary(wb_))

    # NEXT row: per-tile v_s (per-tile boundary search on the same weight and importance, then the
    # per-tile layout), graph-timed on one resident copy beside the uniform product timed the same way
    t0 = time.perf_counter()
    v_tiles, _ = hinm.boundary_search_tiles(igpu, pgpu, w.tile_rows, w.t_s)
    search_tiles_ms = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    pk_tiles = hinm.pack_tiles(wgpu, igpu, w.tile_rows, w.t_s, v_tiles, pgpu)
    pack_tiles_ms = (time.perf_counter() - t0) * 1e3
    y_t = torch.empty(p.cout, B, dtype=torch.bfloat16, device=dev)
    yd_t = torch.empty(p.cout, Bd, dtype=torch.bfloat16, device=dev)
    ws_t = torch.zeros(max(1, hinm.spmm_tiles_workspace_bytes(pk_tiles.plan, Bd),
                           hinm.spmm_workspace_bytes(p, Bd)), dtype=torch.uint8, device=dev)

    def gms(fn, n):
        return graph_replays(torch, lambda: [fn() for _ in range(n)], n, 5)["ms_median"]
    costs = [(int(rr[1]) + 31) // 32 + 2 * ((int(rr[3]) + 63) // 64) for rr in pk_tiles.plan.tiles]
    kept_t = sum(int(rr[1]) + int(rr[3]) // 2 for rr in pk_tiles.plan.tiles)
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
        "spmm_tiles_batch_2048_ms": round(gms(lambda: hinm.spmm(pk_tiles, x, out=y_t), 20), 5),
        "spmm_uniform_resident_batch_2048_ms": round(gms(lambda: hinm.spmm(pk, x, out=y_t), 20), 5),
        "spmm_tiles_batch_16_ms": round(gms(lambda: hinm.spmm(pk_tiles, xd, out=yd_t, workspace=ws_t), 100), 5),
        "spmm_uniform_resident_batch_16_ms": round(gms(lambda: hinm.spmm(pk, xd, out=yd_t, workspace=ws_t), 100), 5),
        "tile_cost_min": int(min(costs)), "tile_cost_mean": round(sum(costs) / len(costs), 2),
        "tile_cost_max": int(max(costs))}
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
    # NEXT row: block-diagonal input permutations (blocks of 64 channels): the pack flags the weight and
    # the product pairs token blocks per tile; beside it the random-perm product above, and the same
    # block-diagonal weight with the plain schedule (one token block per group, every tile's K loop from
    # its first block)
    rngb = np.random.default_rng(5)
    permb = torch.from_numpy(np.stack([np.concatenate([64 * b + rngb.permutation(64) for b in range(p.cin // 64)])
                                       for _ in range(p.n_tiles)]).astype(np.int32)).to(dev)
    pkb = hinm.pack(wgpu, igpu, w.tile_rows, w.t_s, w.v_s, permb)
    rotb, rotbd = Rotation(hinm, torch, pkb, x, B), Rotation(hinm, torch, pkb, xd, Bd)
    rb_ = time_spmm_graph(hinm, torch, rotb, args.steps, replays=3)
    rbd = time_spmm_graph(hinm, torch, rotbd, steps_d, replays=3)
    with hinm.options(prefill_tb_group=1, prefill_stagger=1):
        rb_plain = time_spmm_graph(hinm, torch, rotb, args.steps, replays=3)
    next_block = {"what": "down_proj 4096x11008 packed with a block-diagonal input permutation (blocks of 64 "
                          "channels; the pack sets HINM_PACKED_WINDOWED and the batch > 64 schedule pairs token "
                          "blocks per tile, K loops staggered per tile), graph-timed over rotated copies like the "
                          "headline; beside it the random-perm headline and the block-diagonal weight on the plain "
                          "schedule (one token block per group, every tile from its first K-block)",
                  "flags": int(pkb.flags), "batch_2048_ms": round(rb_["ms_step"], 5),
                  "batch_16_ms": round(rbd["ms_step"], 5), "random_perm_batch_2048_ms": round(ms, 5),
                  "random_perm_batch_16_ms": round(rd["ms_step"], 5),
                  "plain_schedule_batch_2048_ms": round(rb_plain["ms_step"], 5),
                  "useful_tflops_batch_2048": round(alg["useful_flops"] / (rb_["ms_step"] * 1e-3) / 1e12, 2)}
    del rot, rotd, rotb, rotbd, pkb
    torch.cuda.empty_cache()

    dense = None
    if not args.no_dense:
        d2 = time_dense(torch, wgpu, x, args.steps)
        d16 = time_dense(torch, wgpu, xd, steps_d)
        dense = {"what": "torch.matmul bf16 of the unpruned 4096x11008 weight (hipBLASLt), same shapes, graph-timed "
                         "over rotated copies (>= 1 GiB) like the products",
                 "batch_2048_ms": round(d2["ms_step"], 4), "batch_16_ms": round(d16["ms_step"], 4),
                 "batch_2048_spread": spread(d2), "batch_16_spread": spread(d16),
                 "rotation_copies": [d2["rotation_copies"], d16["rotation_copies"]],
                 "speedup_batch_2048": round(d2["ms_step"] / ms, 3),
                 "speedup_batch_16": round(d16["ms_step"] / rd["ms_step"], 3)}

    log("configuration rows")
    configs = None if args.no_configs else config_rows(hinm, torch, synth, dev, args.steps, not args.no_dense)
    log("empirical peaks")
    peaks = empirical_peaks(torch, dev)
    log("stack sweep")
    stack = None if args.no_stack else stack_sweep(hinm, torch, synth, dev, not args.no_dense)
    log("CPU oracle baseline")
    cpu = None if args.no_cpu else cpu_baseline(w, B)
    if cpu is not None and stack is not None:
        stack.update(cpu_baseline_stack())

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
                     "kernel": "prefill_kernel<256, false, false> (one launch per step)",
                     "kernel_source_hash": kernel_source_hash(),
                     "frac_of_measured_matmul_peak": round(value / peaks["matmul_bf16_8192_tflops"], 4),
                     "per_launch": {"useful_flops": alg["useful_flops"], "algorithmic_bytes": alg["bytes"],
                                    "ms": round(ms, 5), **spread(r)},
                     "timing": f"one HIP graph replay of {args.steps} products over {rot_k(p, B)} rotated copies, "
                               f"after {WARM_REPLAYS} untimed replays; spread over {REPLAYS} replays; eager launches "
                               f"from Python: {r_eager['ms_mean'] * 1e3:.1f} us per step",
                     "eager_ms_mean": round(r_eager["ms_mean"], 5)},
        "decode": {"batch": Bd, "ms": round(rd["ms_step"], 5), **spread(rd),
                   "timing": f"one HIP graph replay of {steps_d} products over {rot_k(p, Bd)} rotated copies, after "
                             f"{WARM_REPLAYS} untimed replays; eager launches from Python: "
                             f"{rd_eager['ms_mean'] * 1e3:.1f} us per call",
                   "eager_ms_mean": round(rd_eager["ms_mean"], 5),
                   "algorithmic_bytes": algd["bytes"], "hbm_gbs": round(gbs_d, 1),
                   "roofline": {"bound": "hbm", "achieved": round(gbs_d, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(gbs_d / HBM_PEAK_GBS, 4), "traffic": measured_traffic(Bd),
                                "frac_of_measured_read_peak": round(gbs_d / peaks["read_1gib_gbs"], 4),
                                "kernel": "decode5_kernel<16,24,true,2,false> (one launch per call)"},
                   "useful_tflops": round(algd["useful_flops"] / (rd["ms_step"] * 1e-3) / 1e12, 3)},
        "batch_2048_hbm_gbs": round(alg["bytes"] / (ms * 1e-3) / 1e9, 1),
        "pack_ms": [round(v, 2) for v in pack_ms],
        "configs": configs,
        "empirical_peaks": peaks,
        "gpu_clocks": {"idle": clocks_idle, "under_headline_load": clocks_load},
        "next_output_permutation": next_rows,
        "next_block_diagonal_perm": next_block,
        "next_boundary_search": next_bs,
        "next_per_tile_v_s": next_tiles,
        "next_gyro_permutation": next_gyro,
        "dense_comparator": dense,
        "stack_sweep": stack,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def rot_k(p, batch):
    per = p.packed_bytes + p.cin * batch * 2 + p.cout * batch * 2
    return max(2, -(-ROTATE_BYTES // per))


if __name__ == "__main__":
    main()
