"""Benchmark of the UA hot path on one MI355X.

Headline: the ragged-stress decode layer (1B shape: hidden 2048, 32 query / 8
KV heads, head dim 64; B = 64 sequences with nominal contexts 1k..32k and
per-head compression 2..114x), the largest single-GPU decode workload: one
decode step + eviction + in-place compaction per layer instance per step (one
fused launch), p = 0.05.  A layer's decode working set fits in the 256 MB
Infinity Cache, so a step runs a ring of R independent layer instances
(distinct caches, >= 1 GiB in total), as an R-layer model would, and
throughput is counted per layer: value = B * R / step time.  Inputs are
resident in HBM before timing starts.

The same line carries the other decode workloads (3B-shape long context, 1B
shape, tiny fp32) as objects of their own, each with its roofline and the
oracle's rate on the host cores; the 1B-shape chunked prefill with the final
eviction at p = 0.05 inside its timed region; the prefill variants; and the
attention backward of one training chunk.

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0


KERNEL_FILES = {
    "decode": ["decode.hip", "ua_device.hpp", "ua_kernels.hpp"],
    "prefill": ["prefill.hip", "ua_device.hpp", "ua_kernels.hpp"],
}


def kernel_source_hash(path: str) -> str:
    """Hash of the sources of one path's kernels (counters go stale when it changes)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "kv_cache_pruning_amd", "csrc")
    for f in KERNEL_FILES[path]:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def progress(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def load_traffic(name: str, path: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if current."""
    p = os.path.join(ROOT, "profiles", f"{name}_counters.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("source_hash") != kernel_source_hash(path):
        return None
    return d.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# the oracle on the host cores: one (sequence, KV head) unit per task
# ---------------------------------------------------------------------------
def host_cores() -> int:
    """Cores this process may use (the GPU machine gives one GPU's share: at most 16)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_unit(cfg, w, c, b: int, h: int):
    """The oracle's problem for one (sequence b, KV head h) unit: dims with one
    sequence and one KV head, the parameters' columns of that head, and a cache
    holding its one segment.  Units share nothing (the decay gates, the bias
    and eviction are per KV head), so running them apart is the same work."""
    import oracle as U

    G = cfg.H_q // cfg.H_kv
    cols = [h, cfg.H_kv + h, 2 * cfg.H_kv + h]
    qs = slice(h * G * cfg.d, (h + 1) * G * cfg.d)
    f = lambda a: np.asarray(a, np.float64)
    od = U.Dims(B=1, H_q=G, H_kv=1, d=cfg.d, D=cfg.D, r=cfg.r, terms=U.TERMS_ALL, rope_base=10000.0,
                cache_bf16=cfg.bf16)
    op = U.Params(W_dec=f(w.W_dec)[:, cols], b_dec=f(w.b_dec)[cols], W_dn=f(w.W_dn), W_up=f(w.W_up)[:, qs],
                  b_up=f(w.b_up)[qs])
    s = b * cfg.H_kv + h
    o, n = int(c.seg_off[s]), int(c.seg_len[s])
    oc = U.RefCache(K=[f(c.K[o : o + n])], V=[f(c.V[o : o + n])], lam=[f(c.lam[o : o + n])], lk=[f(c.lk[o : o + n])],
                    next_pos=np.array([int(c.next_pos[b])], np.int64), cap=np.array([int(c.seg_cap[s])], np.int64))
    return od, op, oc


def _oracle_decode_units(job):
    """Worker: ``k`` decode + compaction steps of each unit; returns its compute seconds."""
    name, over, units, k = job
    import oracle as U
    from ua_inputs import config, make_cache, make_step_inputs, make_weights

    cfg = config(name, **over)
    w = make_weights(cfg, 0)
    c = make_cache(cfg, w, 0)
    probs = [oracle_unit(cfg, w, c, b, h) for b, h in units]
    inps = [make_step_inputs(cfg, t, 1, 0) for t in range(k)]
    G = cfg.H_q // cfg.H_kv
    log_p = math.log(cfg.p)
    t0 = time.perf_counter()
    for (b, h), (od, op, oc) in zip(units, probs):
        for inp in inps:
            U.decode_step(od, op, oc, inp.q[b : b + 1, 0, h * G : (h + 1) * G], inp.k[b : b + 1, 0, h : h + 1],
                          inp.v[b : b + 1, 0, h : h + 1], inp.x[b : b + 1, 0], log_p)
            U.compact(oc, log_p)
    return time.perf_counter() - t0


def _oracle_prefill_units(job):
    """Worker: the first ``m`` tokens of call 0 of each unit, token by token."""
    name, over, units, m = job
    import oracle as U
    from ua_inputs import config, make_cache, make_step_inputs, make_weights

    cfg = config(name, **over)
    w = make_weights(cfg, 0)
    c = make_cache(cfg, w, 0)
    probs = [oracle_unit(cfg, w, c, b, h) for b, h in units]
    inp = make_step_inputs(cfg, 0, m, 0)
    G = cfg.H_q // cfg.H_kv
    t0 = time.perf_counter()
    for (b, h), (od, op, oc) in zip(units, probs):
        U.prefill(od, op, oc, inp.q[b : b + 1, :, h * G : (h + 1) * G], inp.k[b : b + 1, :, h : h + 1],
                  inp.v[b : b + 1, :, h : h + 1], inp.x[b : b + 1])
    return time.perf_counter() - t0


def _pool_run(fn, cfg, over, per_unit, budget_s: float, probe_arg, max_arg, granule: int = 1):
    """Run ``fn`` over every unit of ``cfg`` on the host cores.

    A one-unit probe times ``probe_arg`` of work; the amount per unit is then
    chosen so the whole pool takes about ``budget_s`` of wall time.  Returns
    (amount per unit, wall seconds of the slowest worker's compute, cores).
    """
    import concurrent.futures as cf
    import multiprocessing as mp

    units = [(b, h) for b in range(cfg.B) for h in range(cfg.H_kv)]
    cores = min(host_cores(), len(units))
    t1 = fn((cfg.name, over, units[:1], probe_arg)) / probe_arg
    amount = int(budget_s * cores / (len(units) * t1 * per_unit))
    amount = max(granule, min(max_arg, amount // granule * granule))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"  # one BLAS thread per worker process
    jobs = [(cfg.name, over, units[i::cores], amount) for i in range(cores)]
    with cf.ProcessPoolExecutor(max_workers=cores, mp_context=mp.get_context("spawn")) as ex:
        times = list(ex.map(fn, jobs))
    return amount, max(times), cores


def cpu_baseline_decode(cfg, over, budget_s: float):
    """The fp64 oracle, as is, on the first steps of the same workload (instance 0),
    its (sequence, KV head) units spread over the host cores."""
    k, wall, cores = _pool_run(_oracle_decode_units, cfg, over, 1.0, budget_s, 4, cfg.steps)
    return {"value": cfg.B * k / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{cfg.name} instance 0: the first {k} decode + compaction steps of all {cfg.B * cfg.H_kv} "
                      f"(sequence, KV head) units, numpy fp64, {cores} worker processes, one BLAS thread each "
                      f"({wall:.1f} s of the slowest worker's compute)"}


# ---------------------------------------------------------------------------
# decode workloads
# ---------------------------------------------------------------------------
def cache_desc(cfg) -> str:
    """The initial cache of a decode workload, in words."""
    if cfg.len_kind == "empty":
        return "from an empty cache"
    if cfg.len_kind == "ragged":
        return (f"ragged pruned cache, nominal contexts {cfg.nom_lo}..{cfg.nom_hi}, compression "
                f"{cfg.rho_lo:g}..{cfg.rho_hi:g}x per head")
    return f"pruned cache nominal {cfg.nominal} (~{cfg.nominal / cfg.len_mean:.0f}x)"


def bench_decode(args, name: str, over=None, cpu: bool = True):
    """One decode workload: a ring of R layer instances (>= ring-bytes of live
    cache), each step one fused decode + eviction + compaction call per
    instance (a token launch and a tile launch), captured in a HIP graph and
    timed with events around every step.  The same steps are replayed as two
    calls (decode, then ua_compact) from the same state, and once more untimed
    to count live entries and moved rows."""
    import torch

    from kv_cache_pruning_amd.layer import DeviceCache, DeviceWeights, Layer, LayerShape, Workspace
    from ua_inputs import config, make_cache, make_step_inputs, make_weights

    over = dict(over or {})
    cfg = config(name, **over)
    steps = min(args.steps, cfg.steps - args.warmup)
    assert steps > 0, "more warmup steps than the cache has room for"
    log_p = math.log(cfg.p)
    shape = LayerShape(B=cfg.B, H_q=cfg.H_q, H_kv=cfg.H_kv, d=cfg.d, D=cfg.D, r=cfg.r, bf16=cfg.bf16)
    w = make_weights(cfg, 0)
    dw = DeviceWeights(shape, w.W_dec, w.b_dec, w.W_dn, w.W_up, w.b_up)
    elem = 2 if cfg.bf16 else 4
    entry_bytes = 2 * cfg.d * elem + 12  # K + V + logbias read/write + key gate

    t0 = time.time()
    caches, live0 = [], 0
    i = 0
    while True:
        ci = make_cache(cfg, w, seed=i)
        caches.append(DeviceCache(shape, ci.K, ci.V, ci.lam, ci.lk, ci.seg_off, ci.seg_len, ci.seg_cap,
                                  ci.next_pos))
        live0 += int(ci.seg_len.sum()) * entry_bytes
        i += 1
        if (args.ring and i >= args.ring) or (not args.ring and live0 >= args.ring_bytes) or i >= 4096:
            break
    R = len(caches)
    ws = Workspace(shape, max(caches, key=lambda c: c.total_slots), 1)  # calls are serialised on one stream
    insts = [Layer(shape, dw, c, workspace=ws) for c in caches]
    nsteps = args.warmup + steps
    dt = shape.dtype
    toks = []
    for s in range(nsteps):
        inp = make_step_inputs(cfg, s, 1, 0)
        toks.append([torch.from_numpy(np.ascontiguousarray(a[:, 0])).to("cuda", dt) for a in (inp.q, inp.k, inp.v, inp.x)])
    y = torch.empty((cfg.B, cfg.H_q, cfg.d), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    progress(f"{cfg.name}: {R} layer instances ready ({setup_s:.1f} s)")
    static_in = [t.clone() for t in toks[0]]

    def load_inputs(s):
        for dst, src in zip(static_in, toks[s]):
            dst.copy_(src)

    def cap(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    def all_decode():
        for L_ in insts:
            L_.decode_step(*static_in, log_p, y=y)

    def all_compact():
        for L_ in insts:
            L_.compact(log_p)

    def all_step():
        for L_ in insts:
            L_.decode_compact_step(*static_in, log_p, y=y)

    g_step, g_dec, g_cmp = cap(all_step), cap(all_decode), cap(all_compact)
    torch.cuda.synchronize()
    for s in range(args.warmup):
        load_inputs(s)
        g_step.replay()
    torch.cuda.synchronize()
    snap = [(c.K.clone(), c.V.clone(), c.logbias.clone(), c.kgate.clone(), c.seg_len.clone(), c.next_pos.clone())
            for c in caches]

    def restore():
        for c, sn in zip(caches, snap):
            c.K.copy_(sn[0]); c.V.copy_(sn[1]); c.logbias.copy_(sn[2]); c.kgate.copy_(sn[3])
            c.seg_len.copy_(sn[4]); c.next_pos.copy_(sn[5])
        torch.cuda.synchronize()

    # ---- timed region: `steps` steps of the whole hot path.  Events bracket
    # each step's graph (R fused launches back to back on this stream), which
    # gives the launch's average duration as well.
    ev_s = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        load_inputs(args.warmup + s)
        ev_s[s][0].record()
        g_step.replay()
        ev_s[s][1].record()
    torch.cuda.synchronize()
    total_ms = ev_s[0][0].elapsed_time(ev_s[-1][1])
    fused_ms = [e[0].elapsed_time(e[1]) / R for e in ev_s]
    progress(f"{cfg.name}: timed steps done")
    st = int(sum(int(c.status.item()) for c in caches))

    # ---- the same steps as two calls (decode, then compaction), from the same state
    restore()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for s in range(steps):
        load_inputs(args.warmup + s)
        ev[s][0].record()
        g_dec.replay()
        ev[s][1].record()
        g_cmp.replay()
        ev[s][2].record()
    torch.cuda.synchronize()
    dec_ms = [e[0].elapsed_time(e[1]) / R for e in ev]
    cmp_ms = [e[1].elapsed_time(e[2]) / R for e in ev]
    progress(f"{cfg.name}: two-call steps done")

    # ---- untimed replay of the same steps: live entries scanned, rows moved
    restore()
    scanned = moved = moved_fused = cmp_scanned = 0
    for s in range(steps):
        q, k, v, x = toks[args.warmup + s]
        for L_ in insts:
            offs = L_.cache.seg_off.cpu().numpy()
            scanned += int(L_.cache.seg_len.sum().item())
            L_.decode_step(q, k, v, x, log_p, y=y)
            lens = L_.cache.seg_len.cpu().numpy()
            lam = L_.cache.logbias.cpu().numpy()
            for o, n in zip(offs, lens):
                seg = lam[o : o + n]
                dead = np.flatnonzero(seg < log_p)
                cmp_scanned += int(n)
                if dead.size:
                    moved += int(np.count_nonzero(seg[dead[0]:] >= log_p))
                    moved_fused += int(np.count_nonzero(seg[dead[0]:-1] >= log_p))  # the new entry lands in place
            L_.compact(log_p)
    torch.cuda.synchronize()
    del g_step, g_dec, g_cmp, snap

    n_calls = steps * R
    S = cfg.B * cfg.H_kv
    per_step_extra = (S * (2 * cfg.d * elem + 8)  # appends
                      + cfg.B * (cfg.H_q + 2 * cfg.H_kv) * cfg.d * elem + cfg.B * cfg.D * elem  # q, k, v, x
                      + cfg.B * cfg.H_q * cfg.d * 4  # y (fp32)
                      + (cfg.D * (3 * cfg.H_kv + cfg.r) + cfg.r * cfg.H_q * cfg.d) * elem)  # gate weights
    row_bytes = 2 * cfg.d * elem + 8  # K, V, log-bias, key gate of one moved row
    dec_bytes = scanned * entry_bytes + n_calls * per_step_extra
    # compaction: 4 B per entry scanned, plus each moved row read and written
    cmp_bytes = cmp_scanned * 4 + moved * 2 * row_bytes
    fused_bytes = dec_bytes + moved_fused * (row_bytes - 4)  # moved rows: K, V, key gate written
    tile_kernel = (f"decode_tile_mf_kernel<{cfg.d}, {cfg.H_q // cfg.H_kv}, true>" if cfg.bf16
                   else f"decode_tile_kernel<{cfg.d}, {cfg.H_q // cfg.H_kv}, false, true>")
    dec_avg_ms, cmp_avg_ms = float(np.mean(dec_ms)), float(np.mean(cmp_ms))
    fused_avg_ms = float(np.mean(fused_ms))
    achieved = fused_bytes / n_calls / (fused_avg_ms * 1e-3) / 1e9
    ms_per_step = total_ms / steps
    tokens = cfg.B * R  # layer-tokens per step
    cmp_gbs = cmp_bytes / n_calls / (cmp_avg_ms * 1e-3) / 1e9
    res = {
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "steps": steps,
        "ms_per_step": ms_per_step,
        "dtype": "bf16" if cfg.bf16 else "f32",
        "workload": f"{cfg.name}: UA decode layer B={cfg.B} H_q={cfg.H_q} H_kv={cfg.H_kv} d={cfg.d} D={cfg.D}, "
                    f"{cache_desc(cfg)}, p={cfg.p}, decode + eviction + compaction every step (one fused call: "
                    f"token launch + tile launch), "
                    f"ring of {R} layer instances",
        "ring_instances": R,
        "tokens_per_step": tokens,
        "live_entries_per_layer_step": scanned / n_calls,
        "rows_moved_per_layer_step": moved_fused / n_calls,
        "fused_call_us": fused_avg_ms * 1e3,
        "status": st,
        "setup_s": setup_s,
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": load_traffic(f"decode_{cfg.name}", "decode"),
            "kernel": f"ua_decode_compact_step = decode_token_kernel<{cfg.d}, {'true' if cfg.bf16 else 'false'}> + "
                      f"{tile_kernel} (the tile launch is about 85% of the call): one call per layer step, its "
                      "average duration from events around each timed step's R back-to-back calls",
            "launch_us": fused_avg_ms * 1e3,
            "alg_bytes_per_launch": fused_bytes / n_calls,
        },
        "two_calls": {
            "decode_call_us": dec_avg_ms * 1e3,
            "decode_gbs": dec_bytes / n_calls / (dec_avg_ms * 1e-3) / 1e9,
        },
        "compact": {
            "what": "standalone ua_compact after ua_decode_step (the lazy-eviction path), same steps and state",
            "call_us": cmp_avg_ms * 1e3,
            "alg_bytes_per_call": cmp_bytes / n_calls,
            "achieved": cmp_gbs,
            "unit": "GB/s",
            "frac": cmp_gbs / HBM_PEAK_GBS,
        },
    }
    if cpu and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(cfg, over, args.cpu_seconds)
    del insts, caches, ws, toks
    torch.cuda.empty_cache()
    return res


DECODE_WORKLOADS = ["ragged-decode", "3b-decode", "1b-decode", "tiny-decode-f32"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ragged-decode",
                    help="the headline decode workload (the largest single-GPU one by default)")
    ap.add_argument("--only", action="store_true",
                    help="time the headline decode workload only (profiles, sweeps)")
    ap.add_argument("--batch", type=int, default=0,
                    help="override the decode workload's batch (a sweep; the default line uses the workload's own)")
    ap.add_argument("--q-heads", type=int, default=0,
                    help="override the decode workload's query heads (a multiple of its KV heads: the group size)")
    ap.add_argument("--ring", type=int, default=0, help="layer instances (0: enough for --ring-bytes)")
    ap.add_argument("--ring-bytes", type=float, default=1.0 * 2**30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-prefill", action="store_true", help="skip the 1b-prefill figures")
    ap.add_argument("--no-prefill-variants", action="store_true",
                    help="skip the pruned, chunk-boundary and variable-length prefill figures")
    ap.add_argument("--no-backward", action="store_true", help="skip the attention-backward figures")
    ap.add_argument("--only-prefill", action="store_true",
                    help="time the 1b-prefill pass only and print its object (profiles)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="first run three plain device copies of MIB MiB (a known-size reference for the HBM "
                         "byte counters of a rocprofv3 --pmc run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the UA path here runs on "
              f"a single MI355X", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from kv_cache_pruning_amd import load

    load()
    if args.copy_probe > 0:
        src = torch.ones(args.copy_probe << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    over = {}
    if args.batch:
        over["B"] = args.batch
    if args.q_heads:
        over["H_q"] = args.q_heads
    def note(what, t0):
        print(f"[bench] {what} done ({time.time() - t0:.1f} s)", file=sys.stderr, flush=True)

    if args.only_prefill:
        t0 = time.time()
        print(json.dumps({"prefill": bench_prefill(args)}), flush=True)
        note("prefill", t0)
        return

    t0 = time.time()
    head = bench_decode(args, args.workload, over)
    note(f"decode {args.workload}", t0)
    out = {
        "metric": "UA decode tokens/s + achieved HBM GB/s on pruned KV cache; prefill tok/s",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": {k: head[k] for k in ("workload", "ring_instances", "tokens_per_step",
                                         "live_entries_per_layer_step", "rows_moved_per_layer_step",
                                         "fused_call_us", "status", "setup_s", "two_calls", "compact")},
        "roofline": head["roofline"],
    }
    out["config"]["global_batch"] = head["tokens_per_step"] // head["ring_instances"]
    if "cpu_baseline" in head:
        out["cpu_baseline"] = head["cpu_baseline"]
    if not args.only:
        out["decode_configs"] = {}
        for name in DECODE_WORKLOADS:
            if name != args.workload:
                t0 = time.time()
                out["decode_configs"][name] = bench_decode(args, name)
                note(f"decode {name}", t0)
        if not args.no_prefill:
            t0 = time.time()
            out["prefill"] = bench_prefill(args)
            note("prefill", t0)
            if not args.no_prefill_variants:
                t0 = time.time()
                out["prefill_pruned"] = bench_prefill_pruned(args)
                out["prefill_chunked"] = bench_prefill_pruned(args, chunked=True)
                out["prefill_varlen"] = bench_prefill_varlen(args)
                note("prefill variants", t0)
        if not args.no_backward:
            t0 = time.time()
            out["backward"] = bench_backward(args)
            note("backward", t0)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# prefill workload
# ---------------------------------------------------------------------------

def prefill_work(cfg, len0: int, n: int):
    """Algorithmic work of one call: causal (token, key) pairs per KV group,
    MFMA flops (G * 4d for Q.K^T and P.V plus 2d for K.K^T per pair) and
    transcendentals (G softmax exponentials plus 3 for the pair term)."""
    pairs_per_seg = n * len0 + n * (n + 1) // 2
    pairs = pairs_per_seg * cfg.B * cfg.H_kv
    G = cfg.H_q // cfg.H_kv
    return pairs, pairs * (G * 4 * cfg.d + 2 * cfg.d), pairs * (G + 3)


def bench_prefill(args, name: str = "1b-prefill", passes: int = 3, warm: int = 1):
    """The 1B-shape chunked prefill: 16 calls of 1024 tokens from an empty cache,
    then the eviction of the final log-biases at p = 0.05 (one ua_compact), all
    inside the timed region.  Events bracket every call."""
    import torch

    from kv_cache_pruning_amd.layer import layer_from_arrays
    from ua_inputs import config, make_cache, make_step_inputs, make_weights

    cfg = config(name)
    n = cfg.chunk
    calls = cfg.n_total // n
    log_p = math.log(cfg.p)
    w = make_weights(cfg, 0)
    c = make_cache(cfg, w, 0)
    layer = layer_from_arrays(cfg.B, cfg.H_q, cfg.H_kv, cfg.d, cfg.D, cfg.r, cfg.bf16, w, c, max_tokens=n,
                              y_bf16=True)
    dt = torch.bfloat16
    toks = []
    for i in range(calls):
        inp = make_step_inputs(cfg, i, n, 0)
        toks.append([torch.from_numpy(a).to("cuda", dt) for a in (inp.q, inp.k, inp.v, inp.x)])
    y = torch.empty((cfg.B, n, cfg.H_q, cfg.d), dtype=torch.bfloat16, device="cuda")
    seg_len0 = layer.cache.seg_len.clone()
    pos0 = layer.cache.next_pos.clone()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(calls + 2)]
    call_ms = np.zeros(calls + 1)
    for p in range(warm + passes):
        # every pass starts from the empty cache (lengths and positions reset; the
        # slots it writes are rewritten before they are read)
        layer.cache.seg_len.copy_(seg_len0)
        layer.cache.next_pos.copy_(pos0)
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(calls):
            layer.prefill(*toks[i], y=y)
            ev[i + 1].record()
        layer.compact(log_p)
        ev[calls + 1].record()
        torch.cuda.synchronize()
        if p >= warm:
            call_ms += np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(calls + 1)])
    call_ms /= passes
    kept = layer.cache.seg_len.cpu().numpy()
    st = int(layer.cache.status.item())
    total_ms = float(call_ms.sum())
    prefill_ms = float(call_ms[:calls].sum())
    flops = trans = 0.0
    for i in range(calls):
        _, f, t = prefill_work(cfg, i * n, n)
        flops += f
        trans += t
    tflops = flops / (total_ms * 1e-3) / 1e12
    tflops_calls = flops / (prefill_ms * 1e-3) / 1e12
    tts = trans / (prefill_ms * 1e-3) / 1e12
    tokens = cfg.B * calls * n
    return {
        "workload": f"{cfg.name}: UA chunked prefill B={cfg.B} H_q={cfg.H_q} H_kv={cfg.H_kv} d={cfg.d} D={cfg.D}, "
                    f"{calls} calls of {n} tokens from an empty cache (N={cfg.n_total}), then eviction of the final "
                    f"log-biases at p={cfg.p} (ua_compact), bf16 storage, y bf16",
        "value": tokens / (total_ms * 1e-3),
        "unit": "tokens/s",
        "ms_per_pass": total_ms,
        "passes": passes,
        "call_ms": [round(float(x), 4) for x in call_ms[:calls]],
        "eviction_ms": float(call_ms[calls]),
        "kept_entries_per_segment": float(kept.mean()),
        "status": st,
        "roofline": {
            "bound": "mfma",
            "achieved": tflops,
            "peak": MFMA_BF16_PEAK_TFS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFS,
            "traffic": load_traffic(f"prefill_{cfg.name}", "prefill"),
            "kernel": "ua_prefill = prep + token + attention kernels, timed per call with events (the attention "
                      "kernel dominates); the eviction is inside the time",
            "alg_flops": flops,
            "calls_only_frac": tflops_calls / MFMA_BF16_PEAK_TFS,
            "transcendentals_per_s": tts * 1e12,
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_prefill(cfg, args.cpu_seconds),
    }


def bench_prefill_pruned(args, chunked: bool = False, name: str = "1b-prefill", passes: int = 3, warm: int = 1):
    """The 1b-prefill tokens with eviction at the workload's p.

    pruned: 16 calls of ua_prefill_pruned (1024 tokens each, attention masked
    at log p, compaction at the end of each call).  chunked: one call of
    ua_prefill_chunked over all 16384 tokens, dense inside 128-token chunks
    with a compaction after each.  Every pass starts from the empty cache.
    The roofline counts the (token, key) pairs of each call over the cache as
    the call finds it (lengths read in an untimed pass), as for dense prefill.
    """
    import torch

    from kv_cache_pruning_amd.layer import layer_from_arrays
    from ua_inputs import config, make_cache, make_step_inputs, make_weights

    cfg = config(name)
    log_p = math.log(cfg.p)
    n = 128 if chunked else cfg.chunk
    per_call = cfg.n_total if chunked else n
    calls = cfg.n_total // per_call
    w = make_weights(cfg, 0)
    c = make_cache(cfg, w, 0)
    layer = layer_from_arrays(cfg.B, cfg.H_q, cfg.H_kv, cfg.d, cfg.D, cfg.r, cfg.bf16, w, c, max_tokens=n,
                              y_bf16=True)
    dt = torch.bfloat16
    inps = [make_step_inputs(cfg, i, cfg.chunk, 0) for i in range(cfg.n_total // cfg.chunk)]
    full = [np.concatenate([getattr(x, f) for x in inps], axis=1) for f in ("q", "k", "v", "x")]
    toks = [[torch.from_numpy(np.ascontiguousarray(a[:, i * per_call:(i + 1) * per_call])).to("cuda", dt)
             for a in full] for i in range(calls)]
    y = torch.empty((cfg.B, per_call, cfg.H_q, cfg.d), dtype=torch.bfloat16, device="cuda")
    seg_len0 = layer.cache.seg_len.clone()
    pos0 = layer.cache.next_pos.clone()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(calls + 1)]
    call_ms = np.zeros(calls)
    lens = []
    for p in range(warm + passes + 1):
        layer.cache.seg_len.copy_(seg_len0)
        layer.cache.next_pos.copy_(pos0)
        torch.cuda.synchronize()
        if p == warm + passes:
            # untimed: the same work as separate calls, to read the lengths each
            # chunk (or call) finds
            for i in range(calls):
                for c0 in range(0, per_call, n):
                    lens.append(layer.cache.seg_len.cpu().numpy().copy())
                    part = [t[:, c0:c0 + n].contiguous() for t in toks[i]]
                    if chunked:
                        layer.prefill(*part, y=y[:, c0:c0 + n].contiguous())
                        layer.compact(log_p)
                    else:
                        layer.prefill_pruned(*part, log_p, y=y)
            torch.cuda.synchronize()
            break
        ev[0].record()
        for i in range(calls):
            if chunked:
                layer.prefill_chunked(*toks[i], n, log_p, y=y)
            else:
                layer.prefill_pruned(*toks[i], log_p, y=y)
            ev[i + 1].record()
        torch.cuda.synchronize()
        if warm <= p < warm + passes:
            call_ms += np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(calls)])
    call_ms /= passes
    kept = layer.cache.seg_len.cpu().numpy()
    st = int(layer.cache.status.item())
    total_ms = float(call_ms.sum())
    G = cfg.H_q // cfg.H_kv
    pairs = float(sum(sum(n * int(l0) + n * (n + 1) // 2 for l0 in ls) for ls in lens))
    flops, trans = pairs * (G * 4 * cfg.d + 2 * cfg.d), pairs * (G + 3)
    tts = trans / (total_ms * 1e-3) / 1e12
    tflops = flops / (total_ms * 1e-3) / 1e12
    tokens = cfg.B * cfg.n_total
    what = (f"ua_prefill_chunked, dense 128-token chunks with compaction at p={cfg.p} after each" if chunked else
            f"{calls} calls of ua_prefill_pruned ({n} tokens, attention masked at p={cfg.p}, compaction per call)")
    return {
        "workload": f"{cfg.name}: {what}; B={cfg.B} H_q={cfg.H_q} H_kv={cfg.H_kv} d={cfg.d}, N={cfg.n_total} "
                    f"from an empty cache, bf16 storage, y bf16",
        "value": tokens / (total_ms * 1e-3),
        "unit": "tokens/s",
        "ms_per_pass": total_ms,
        "passes": passes,
        "kept_entries_per_segment": float(kept.mean()),
        "call_ms": [round(float(x), 4) for x in call_ms] if not chunked else None,
        "status": st,
        "roofline": {
            "bound": "mfma",
            "achieved": tflops,
            "peak": MFMA_BF16_PEAK_TFS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFS,
            "pairs": pairs,
            "transcendentals_per_s": tts * 1e12,
        },
    }


def bench_prefill_varlen(args, B: int = 8, passes: int = 3, warm: int = 1, seed: int = 7):
    """One ua_prefill_varlen call of B packed sequences with lengths uniform in
    [128, 2048] (seeded), 1B head shape, from an empty cache.  The roofline
    counts each sequence's own causal pairs."""
    import torch

    from kv_cache_pruning_amd.layer import layer_from_arrays
    from ua_inputs import config, make_cache, make_step_inputs, make_weights

    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(128, 2049, B)]
    nmax = max(lens)
    cfg = config("1b-prefill", B=B, n_total=nmax, chunk=nmax)
    w = make_weights(cfg, 0)
    c = make_cache(cfg, w, 0)
    layer = layer_from_arrays(cfg.B, cfg.H_q, cfg.H_kv, cfg.d, cfg.D, cfg.r, cfg.bf16, w, c, max_tokens=nmax,
                              y_bf16=True)
    inp = make_step_inputs(cfg, 0, nmax, 0)
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    pack = lambda a: torch.from_numpy(np.concatenate([a[b, : lens[b]] for b in range(B)], axis=0)).to(
        "cuda", torch.bfloat16)
    toks = [pack(a) for a in (inp.q, inp.k, inp.v, inp.x)]
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    y = torch.empty((T, cfg.H_q, cfg.d), dtype=torch.bfloat16, device="cuda")
    import kv_cache_pruning_amd as K

    _, tok = layer._tokens(*toks)
    seg_len0 = layer.cache.seg_len.clone()
    pos0 = layer.cache.next_pos.clone()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ms = []
    for p in range(warm + passes):
        layer.cache.seg_len.copy_(seg_len0)
        layer.cache.next_pos.copy_(pos0)
        torch.cuda.synchronize()
        ev[0].record()
        K.ua_prefill_varlen(layer.dims, layer.w.params, layer.cache.struct, tok, cu_d, T, nmax, y, layer.ws.ptr,
                            layer.ws.nbytes)
        ev[1].record()
        torch.cuda.synchronize()
        if p >= warm:
            ms.append(ev[0].elapsed_time(ev[1]))
    st = int(layer.cache.status.item())
    t = float(np.mean(ms))
    G = cfg.H_q // cfg.H_kv
    pairs = float(sum(n * (n + 1) // 2 for n in lens) * cfg.H_kv)
    flops, trans = pairs * (G * 4 * cfg.d + 2 * cfg.d), pairs * (G + 3)
    tts = trans / (t * 1e-3) / 1e12
    tflops = flops / (t * 1e-3) / 1e12
    return {
        "workload": f"ua_prefill_varlen: {B} packed sequences of {lens} tokens (1B heads H_q={cfg.H_q} "
                    f"H_kv={cfg.H_kv} d={cfg.d}) from an empty cache, bf16 storage, y bf16",
        "value": T / (t * 1e-3),
        "unit": "tokens/s",
        "ms_per_call": t,
        "passes": passes,
        "status": st,
        "roofline": {
            "bound": "mfma",
            "achieved": tflops,
            "peak": MFMA_BF16_PEAK_TFS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFS,
            "pairs": pairs,
            "transcendentals_per_s": tts * 1e12,
        },
    }


def cpu_baseline_prefill(cfg, budget_s: float):
    """The fp64 oracle's token-by-token prefill on the first tokens of call 0,
    its (sequence, KV head) units spread over the host cores."""
    m, wall, cores = _pool_run(_oracle_prefill_units, cfg, {}, 1.0, budget_s, 32, cfg.chunk, granule=32)
    return {"value": cfg.B * m / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{cfg.name} call 0: the first {m} tokens of each of the {cfg.B * cfg.H_kv} (sequence, KV "
                      f"head) units from an empty cache, numpy fp64, {cores} worker processes ({wall:.1f} s of the "
                      f"slowest worker's compute; later tokens cost more)"}


# ---------------------------------------------------------------------------
# attention backward (one training chunk per sequence)
# ---------------------------------------------------------------------------
FP32_VECTOR_PEAK_TFS = 157.3  # fp32 vector and fp32 matrix-core peak alike


def backward_work(B: int, N: int, H_q: int, H_kv: int, d: int):
    """Algorithmic flops of the backward: per causal (token, key) pair and
    query head, five length-d products (Q.K^T recomputed, dO.V^T, and the
    dV, dQ, dK accumulations: 10d flops); per pair and KV head, the key
    similarity and its two key gradients (6d)."""
    pairs = B * H_kv * (N * (N + 1) // 2)
    G = H_q // H_kv
    return pairs * (G * 10 * d + 6 * d)


def bench_backward(args, B: int = 2, N: int = 4096, H_q: int = 32, H_kv: int = 8, d: int = 64, passes: int = 3,
                   warm: int = 1):
    import torch

    import kv_cache_pruning_amd as K
    from ua_inputs import make_grad_inputs

    g = make_grad_inputs(B, N, H_q, H_kv, d, True, 0)
    dims = K.make_dims(B, H_q, H_kv, d, 2048, bf16=True)
    dev = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", t)
    q, k, v = dev(g.q, torch.bfloat16), dev(g.k, torch.bfloat16), dev(g.v, torch.bfloat16)
    lq, lk, lb, dO = dev(g.lq), dev(g.lk), dev(g.lb), dev(g.dO)
    outs = [torch.empty(a.shape, dtype=torch.float32, device="cuda") for a in (g.q, g.k, g.v, g.lq, g.lk, g.lb)]
    nb = K.ua_backward_workspace_bytes(dims, N)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ms = []
    for p in range(warm + passes):
        torch.cuda.synchronize()
        ev[0].record()
        K.ua_attention_backward(dims, N, q, k, v, lq, lk, lb, dO, *outs, ws, nb)
        ev[1].record()
        torch.cuda.synchronize()
        if p >= warm:
            ms.append(ev[0].elapsed_time(ev[1]))
    t = float(np.mean(ms))
    flops = backward_work(B, N, H_q, H_kv, d)
    tf = flops / (t * 1e-3) / 1e12
    return {
        "workload": f"UA attention backward, one training chunk per sequence: B={B} N={N} H_q={H_q} H_kv={H_kv} "
                    f"d={d}, all three decay terms, bf16 q/k/v, fp32 gates and gradients",
        "value": B * N / (t * 1e-3),
        "unit": "tokens/s",
        "ms_per_call": t,
        "passes": passes,
        "roofline": {
            "bound": "alu",
            "achieved": tf,
            "peak": FP32_VECTOR_PEAK_TFS,
            "unit": "TFLOP/s (fp32)",
            "frac": tf / FP32_VECTOR_PEAK_TFS,
            "traffic": None,
            "kernel": "ua_attention_backward = bias, stats, kv, q, decay column and row kernels (timed per call)",
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_backward(g, args.cpu_seconds / 2),
    }


def cpu_baseline_backward(g, budget_s: float):
    """The fp64 oracle's backward, one (sequence, KV head) group at a time, until the budget is spent."""
    import torch

    import oracle as U

    B, N, H_q, d = g.q.shape
    H_kv = g.k.shape[2]
    G = H_q // H_kv
    t0 = time.time()
    done = 0
    while done < B * H_kv and time.time() - t0 < budget_s:
        b, h = divmod(done, H_kv)
        qs, hs = slice(h * G, (h + 1) * G), slice(h, h + 1)
        U.ua_grad.attention_backward(g.q[b, :, qs].astype(np.float64), g.k[b, :, hs].astype(np.float64),
                                     g.v[b, :, hs].astype(np.float64), g.lq[b, :, hs].astype(np.float64),
                                     g.lk[b, :, hs].astype(np.float64), g.lb[b, :, hs].astype(np.float64),
                                     g.dO[b, :, qs].astype(np.float64), 7, 1.0 / math.sqrt(d))
        done += 1
    dt = time.time() - t0
    return {"value": B * N / (dt * B * H_kv / done), "unit": "tokens/s", "cores": torch.get_num_threads(),
            "kind": "oracle",
            "sample": f"{done} of the {B * H_kv} (sequence, KV head) groups ({dt:.1f} s, torch fp64 autograd on "
                      f"the CPU), scaled to all groups"}


if __name__ == "__main__":
    main()
