#!/usr/bin/env python3
"""Decode throughput of the constant-shape decode step on one MI355X.

Workload (default): the 8B-shaped bf16 decoder (32 layers, d_model 4096, 32 q / 8 kv heads of 128, SwiGLU 14336,
vocab 128256, RoPE theta 5e5), batch 1, contiguous KV of capacity 8192 pre-filled with N(0,1) keys and values up to
position 2048; greedy decode from position 2048 (warm-up steps first, then the timed steps, 512 in total by
default). Weights are seeded N(0, 0.02) draws rounded to bf16; nothing is trained or downloaded.

One step = one HIP-graph replay of every kernel of the step (the slot buffers hold token and position). By default
the greedy token is picked on the device and fed to the next step, and the host waits once per --chain steps
(reading back the ids; fewer when the timed steps would give under five waits, so the wall-time percentiles have
samples); `value` is decode tokens/s over the timed steps (rows x steps / wall time). Beside it,
`step.per_token_readback` times the same engine with one host wait per step, the logits copied back and the greedy
token picked on the host (--chain 0 makes that the headline).

Printed as one JSON line, with:
  roofline      the dominant kernel's achieved HBM bandwidth against MI355X's 8 TB/s: algorithmic bytes per
                launch / mean launch time, where each kernel kind's launches of a step are replayed as a graph of
                their own between HIP events on the engine's stream; `traffic` is the HBM bytes per launch from
                the committed rocprofv3 counter summary of that kernel (null if none, or if the kernel source
                changed since);
  step          whole-step device time (HIP events around the replay) and bytes, kernels per step, host submit
                time for the graph replay and for one-launch-per-kernel;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload on this host (all cores; one core
                too for the tiny and 1B-shaped workloads), with its seconds per step and the algorithmic bytes per
                second of oracle time;
  parity        the timed engine against that oracle run, from the same initial state: teacher-forced (the oracle's
                tokens) max-abs logits error and greedy agreement where the oracle's top-2 margin exceeds 5e-2, and
                the free-running agreement length of the device's own greedy chain.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tokens/s + % HBM roofline, batch 1, 8B-shaped bf16, cap 8192"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_bytes(w) -> float:
    """Bytes one step must move: all weights streamed once (layers, final norm, head), the embedding rows read,
    the whole [cap] K and V sweep of every layer and row, and the K/V write."""
    m = w.model
    wb = 2 if m.weight_dtype == "bf16" else 4
    kvb = 2 if w.kv_dtype == "bf16" else 4
    d, hd, F, L, V, R = m.d_model, m.head_dim, m.ffn_dim, m.n_layers, m.vocab, w.rows
    per_layer = d * (m.n_q_heads + 2 * m.n_kv_heads) * hd + m.n_q_heads * hd * d + 3 * d * F + 2 * d
    return (wb * (L * per_layer + V * d + d) + R * d * wb + L * R * 2 * w.cap * m.n_kv_heads * hd * kvb
            + L * R * 2 * m.n_kv_heads * hd * kvb)


def engine_for(w, ws, exec_mode, kernel_plan="auto", trace="off", prefill_rows=None):
    from decode_step_03_amd import Engine, make_config
    m = w.model
    cfg = make_config(n_layers=m.n_layers, d_model=m.d_model, n_q_heads=m.n_q_heads, n_kv_heads=m.n_kv_heads,
                      head_dim=m.head_dim, ffn_dim=m.ffn_dim, vocab=m.vocab, rms_eps=m.rms_eps,
                      rope_theta=m.rope_theta, rows=w.rows, cap=w.cap, kv_layout=w.kv_layout,
                      page_size=w.page_size, pool_pages=w.pool_pages, weight_dtype=m.weight_dtype,
                      kv_dtype=w.kv_dtype, exec_mode=exec_mode, kernel_plan=kernel_plan, trace=trace,
                      prefill_rows=(64 if w.start == "prefill_tokens" else 0) if prefill_rows is None else prefill_rows)
    eng = Engine(cfg, "cuda:0")
    eng.load_weights(ws.layers, ws.glob)
    return eng


def prefill(eng, w, start_pos):
    """Initial state: the page table (paged layout) and N(0,1) K/V for positions [0, start) of every row; or, for
    a workload that starts from a prompt, the prompt (ds3_prefill in chunks, or one-token steps), and then the
    first decode token of each row (the greedy pick of the prompt's last logits) is returned. None otherwise."""
    from concurrent.futures import ThreadPoolExecutor

    import synth
    if w.kv_layout == "paged":
        eng.set_slot_map(synth.page_table(w))
    if w.start == "prefill_tokens":
        toks = synth.prefill_tokens(w)
        first = np.zeros(w.rows, np.int32)
        if eng.cfg.prefill_rows > 0:   # the prompt in chunks of prefill_rows tokens per launch sequence
            # (a chunk sweeps only the positions up to its own: bit-identical to the full sweep, and a 64-token chunk
            # would otherwise read every row's whole capacity; decode steps sweep the full capacity again)
            eng.set_kv_sweep("visible")
            for r in range(w.rows):   # (untimed: captures the prefill graph; the timed pass rewrites the same K/V)
                eng.prefill(r, toks[r], 0)
            t0 = time.perf_counter()
            for r in range(w.rows):
                lg, _ = eng.prefill(r, toks[r], 0)
                first[r] = int(np.argmax(lg))
            dt = time.perf_counter() - t0
            eng.set_kv_sweep("full")
            prefill.last = {"tokens": int(w.rows * w.prefill_len), "chunk": int(eng.cfg.prefill_rows),
                            "sweep": "visible", "ms": round(1e3 * dt, 3), "tok_s": round(w.rows * w.prefill_len / dt, 1),
                            "gpu_ms": round(eng.stats()["last_prefill_gpu_us"] / 1e3, 3)}
            return first
        for p in range(w.prefill_len):
            lg, _ = eng.step(toks[:, p], np.full(w.rows, p, np.int32))
        return lg.argmax(axis=1).astype(np.int32)   # the first decode token: the prompt's last logits' pick
    jobs = [(li, r, int(start_pos[r])) for r in range(w.rows) for li in range(w.model.n_layers) if start_pos[r] > 0]

    def gen(job):
        li, r, n = job
        return li, r, synth.kv_prefill(w, li, r, "k", n), synth.kv_prefill(w, li, r, "v", n)

    t0 = time.time()
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        for i, (li, r, k, v) in enumerate(ex.map(gen, jobs)):
            eng.write_kv(li, r, 0, k, v)
            if (i + 1) % 64 == 0:
                log(f"K/V prefill {i + 1}/{len(jobs)} (layer, row) pairs, {time.time() - t0:.0f}s")


prefill.last = None


def oracle_start(w, model, start_pos, start_tok, n_extra: int = 64):
    """The oracle's state of row 0 where the workload's decode steps begin, and its first token: N(0,1) K/V up to
    the start position (the same seeded draws the engine gets), or the prompt through a causal forward (its K/V, and
    the first token picked from its last logits); the tiny workload starts empty at position 0."""
    import oracle
    import synth
    cache = oracle.RowCache(model, int(start_pos[0]) + n_extra, w.kv_dtype)
    tok = int(start_tok[0])
    if w.start == "prefill_tokens":
        lg = oracle.causal_forward(model, synth.prefill_tokens(w)[0], w.kv_dtype, cache=cache)
        tok = int(np.argmax(lg[-1]))
    else:
        n = int(start_pos[0])
        for li in range(w.model.n_layers if n > 0 else 0):
            cache.set(li, 0, synth.kv_prefill(w, li, 0, "k", n), synth.kv_prefill(w, li, 0, "v", n))
    return cache, tok


def cpu_baseline(w, ws, start_pos, start_tok, budget_s: float, single_core_s: float = 0.0) -> tuple:
    """The oracle as it is, on this host's cores, over a bounded sample of the workload: whole greedy decode steps
    of row 0 from its start. Returns (the baseline record, the steps' tokens and logits for the parity check).
    With single_core_s > 0 the oracle is timed again on one core (one thread, one BLAS thread)."""
    import oracle
    model = oracle.OracleModel.from_weightset(ws)

    def run(budget, max_steps):
        cache, tok = oracle_start(w, model, start_pos, start_tok)
        p = int(start_pos[0])
        toks, logits = [], []
        t0 = time.time()
        while True:
            lg = oracle.decode_step(model, cache, tok, p)
            toks.append(tok)
            logits.append(lg.astype(np.float32))
            tok, p = int(np.argmax(lg)), p + 1
            if time.time() - t0 >= budget or len(toks) >= max_steps:
                break
        return time.time() - t0, toks, logits

    dt, toks, logits = run(budget_s, 32)
    steps = len(toks)
    nbytes = algorithmic_bytes(w) / w.rows   # one row's share of the step's bytes (the oracle runs one row)
    out = {"value": steps / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
           "sample": f"{steps} greedy decode step(s) of row 0 from position {int(start_pos[0])}, all "
                     f"{w.model.n_layers} layers and the head, float64, weights widened per 256-row block",
           "seconds": round(dt, 2), "s_per_step": round(dt / steps, 4),
           "gbs_of_algorithmic_bytes": round(nbytes * steps / dt / 1e9, 3), "host": host_info()}
    if single_core_s > 0:
        from threadpoolctl import threadpool_limits
        n_threads = oracle.threads()
        oracle.set_threads(1)
        try:
            with threadpool_limits(1):
                dt1, t1, _ = run(single_core_s, 8)
        finally:
            oracle.set_threads(n_threads)
        out["single_core"] = {"value": len(t1) / dt1, "unit": "tokens/s", "cores": 1, "steps": len(t1),
                              "seconds": round(dt1, 2), "s_per_step": round(dt1 / len(t1), 4),
                              "gbs_of_algorithmic_bytes": round(nbytes * len(t1) / dt1 / 1e9, 4)}
    return out, {"tokens": toks, "logits": logits}


def parity_leg(eng, w, start_pos, start_tok, ref) -> dict:
    """The engine against the oracle's run of row 0, from the same initial state (reset, then the workload's
    prefill): teacher-forced by the oracle's tokens, the max-abs logits error and the greedy ids wherever the
    oracle's top-2 margin exceeds 5e-2; then the device's own greedy chain from the same start, and for how many
    steps its picks agree with the oracle's."""
    tol = 1e-4 if w.model.weight_dtype == "f32" else 2e-2
    toks, refl = ref["tokens"], ref["logits"]
    n = len(toks)

    def restart():
        eng.reset_state()
        first = prefill(eng, w, start_pos)
        t = (first if first is not None else start_tok).copy()
        t[0] = toks[0]
        return t

    tok, pos = restart(), start_pos.copy()
    err, checked, agree, inside = 0.0, 0, 0, 0
    for i in range(n):
        lg, flags = eng.step(tok, pos)
        err = max(err, float(np.max(np.abs(lg[0].astype(np.float64) - refl[i]))))
        top2 = np.partition(refl[i], -2)[-2:]
        if top2[1] - top2[0] > 5e-2:
            checked += 1
            agree += int(int(np.argmax(lg[0])) == int(np.argmax(refl[i])))
        else:
            inside += 1
        tok = lg.argmax(axis=1).astype(np.int32)
        if i + 1 < n:
            tok[0] = toks[i + 1]
        pos = pos + 1
    tok, pos = restart(), start_pos.copy()
    ids, _ = eng.step_greedy(tok, pos, n)
    run = 0
    for i in range(n - 1):
        if int(ids[i, 0]) != int(toks[i + 1]):
            break
        run += 1
    return {"rows_checked": 1, "steps": n, "logits_max_abs_err": float(f"{err:.3e}"), "tolerance": tol,
            "within_tolerance": bool(err <= tol), "greedy_checked": checked, "greedy_equal": agree,
            "greedy_inside_margin": inside, "free_running_agreement": run, "free_running_of": n - 1}


CSRC = os.path.join(ROOT, "decode_step_03_amd", "csrc")


def kernel_sources(kind: str) -> list:
    """The source files a kernel kind is compiled from (its own file and the device headers it includes)."""
    main = "ds3_fused.hip" if kind == "decode_step_fused" else "ds3_kernels.hip"
    return [os.path.join(CSRC, f) for f in (main, "ds3_device.h", "ds3_kernels.h")]


def sources_sha256(kind: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for path in kernel_sources(kind):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def pmc_traffic(kind: str, workload: str):
    """HBM bytes per launch of kernel kind `kind` on `workload`, from the committed rocprofv3 counter summary
    profiles/pmc_<kind>_<workload>.md (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the counter
    reads for a plain copy of known size). None when there is no summary, or when the kernel source has changed
    since the counters were taken (the summary records the SHA-256 of its source files)."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kind}_{workload}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    try:
        if sources_sha256(kind) != vals["kernel_source_sha256"]:
            return None
        return (float(vals["fetch_kib_per_launch"]) * float(vals["fetch_scale"])
                + float(vals["write_kib_per_launch"]) * float(vals["write_scale"])) * 1024.0
    except (KeyError, ValueError, OSError):
        return None


def host_info() -> dict:
    """What the oracle's time is measured on: CPU model, logical cores, host RAM, the BLAS behind NumPy and its
    threads."""
    info = {"cpu_model": None, "logical_cpus": os.cpu_count(), "host_ram_gb": None, "blas": None}
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                info["host_ram_gb"] = round(int(line.split()[1]) / 2**20, 1)
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        info["blas"] = [{"api": d.get("internal_api"), "threads": d.get("num_threads")} for d in threadpool_info()
                        if d.get("user_api") == "blas"]
    except Exception:   # (threadpoolctl absent or failing: leave it unrecorded)
        pass
    return info


def achievable_bandwidth(torch) -> dict:
    """What plain streaming reaches on this GPU, beside the roofline's 8 TB/s: the library's streaming-read probe
    (the weight streams' access pattern: 16-byte non-temporal loads, 1 KB per wave instruction) over 4 GiB, and a
    device-to-device copy of 1 GiB (bytes read + written); both are larger than the 256 MB infinity cache. HIP
    events on torch's stream, best of 3 after a warm-up."""
    from decode_step_03_amd import _ds3

    def best(fn, reps=3):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]) * 1e3)
        return min(ts)
    n_read = 4 << 30
    a = torch.ones(n_read // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    us_read = best(lambda: _ds3.ds3_probe_read(a.data_ptr(), n_read, sink.data_ptr(), stream))
    del a, sink
    src = torch.ones((1 << 30) // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    us_copy = best(lambda: dst.copy_(src))
    del src, dst
    torch.cuda.empty_cache()
    return {"read_gbs": round(n_read / us_read / 1e3, 1), "copy_gbs": round(2 * (1 << 30) / us_copy / 1e3, 1),
            "probe": "ds3_probe_read over 4 GiB (read only); copy of 1 GiB (read + write)"}


def copy_calibration(torch, nbytes: int = 1 << 30, reps: int = 5) -> int:
    """A plain copy kernel of known size: each launch reads and writes exactly `nbytes`. A hardware byte counter
    read over these launches gives the factor that turns the counter's units into bytes."""
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda:0").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / reps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": reps,
                      "us_per_launch": round(us, 1), "gbs": round(2 * nbytes / us / 1e3, 1)}), flush=True)
    return 0


def steps_per_host_wait(chain: int, steps: int) -> int:
    """Steps per host wait of the chained greedy run: `chain`, or fewer so that the timed steps give at least five
    wall-time samples (0: no chaining, the host picks every token)."""
    return min(chain, max(1, steps // 5)) if chain > 0 else 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=504)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama8b-bf16-cap8192")
    ap.add_argument("--cap", type=int, default=0,
                    help="run the workload at this K/V capacity instead of its own (reported beside it, not as the "
                         "headline)")
    ap.add_argument("--profile-iters", type=int, default=10)
    ap.add_argument("--eager-steps", type=int, default=16,
                    help="steps of the per-operation kernels, as a graph replay and launched one by one")
    ap.add_argument("--kernel-plan", default="auto", choices=["auto", "fused", "per_op"])
    ap.add_argument("--chain", type=int, default=32,
                    help="steps per host wait, each step's token picked on the device (0: every step returns its "
                         "logits and the host picks)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--visible-steps", type=int, default=64,
                    help="also time this many steps with the visible K/V sweep (0: skip)")
    ap.add_argument("--sample-steps", type=int, default=64,
                    help="also time this many steps with the sampling suffix in place of the greedy pick (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of known size (for scaling HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (the decode step runs on a single MI355X with no sharding); "
              f"asked for --gpus {args.gpus} / WORLD_SIZE {world}", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        return copy_calibration(torch)

    import synth
    w = synth.workload(args.workload)
    if args.cap:
        from dataclasses import replace
        w = replace(w, cap=args.cap, name=f"{w.name}@cap{args.cap}")
    m = w.model
    t0 = time.time()
    ws = synth.make_weights(m)
    log(f"weights drawn in {time.time() - t0:.1f}s ({m.n_params() / 1e9:.2f} B parameters)")
    start_pos = synth.start_positions(w)
    start_tok = synth.start_tokens(w)

    t0 = time.time()
    eng = engine_for(w, ws, "graph", args.kernel_plan)
    first = prefill(eng, w, start_pos)
    if first is not None:   # a prompt workload: decoding starts from the prompt's greedy pick
        start_tok = first
    log(f"engine loaded and K/V pre-filled in {time.time() - t0:.1f}s")

    pos = start_pos.copy()
    tok = start_tok.copy()
    total = args.warmup + args.steps
    if int(pos.max()) + total > w.cap:
        total = w.cap - int(pos.max())
        args.steps = max(1, total - args.warmup)
        total = args.warmup + args.steps
        log(f"steps limited to {args.steps} by the KV capacity")
    wall, gpu_us, submit_us = [], [], []
    chain = steps_per_host_wait(args.chain, args.steps)
    torch.cuda.synchronize()
    if chain > 0:
        # chained greedy steps: the device picks each token; one host wait per `chain` steps
        def run(n_total, timed):
            nonlocal tok, pos
            done = 0
            while done < n_total:
                n = min(chain, n_total - done)
                ts = time.perf_counter()
                ids, flags = eng.step_greedy(tok, pos, n)
                tok, pos, done = ids[-1].copy(), pos + n, done + n
                if timed:
                    wall.append((time.perf_counter() - ts) / n)
                    st = eng.stats()
                    gpu_us.append(st["last_gpu_us"])
                    submit_us.append(st["last_submit_us"] / n)
                if flags.any():
                    log(f"warning: non-finite logits in {int(flags.sum())} of {n} chained steps")
        run(args.warmup, False)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        run(args.steps, True)
    else:
        for i in range(total):
            if i == args.warmup:
                torch.cuda.synchronize()
                t_start = time.perf_counter()
            ts = time.perf_counter()
            logits, flags = eng.step(tok, pos)
            tok = logits.argmax(axis=1).astype(np.int32)
            pos = pos + 1
            if i >= args.warmup:
                wall.append(time.perf_counter() - ts)
                st = eng.stats()
                gpu_us.append(st["last_gpu_us"])
                submit_us.append(st["last_submit_us"])
            if flags:
                log(f"warning: non-finite logits at step {i}")
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    stats = eng.stats()
    tok_s = w.rows * args.steps / elapsed
    step_bytes = algorithmic_bytes(w)
    gpu_ms = float(np.median(gpu_us)) / 1e3
    log(f"{tok_s:.1f} tok/s, wall {1e3 * elapsed / args.steps:.3f} ms/step, GPU {gpu_ms:.3f} ms/step, "
        f"{step_bytes / gpu_ms / 1e6:.0f} GB/s")

    kernels = eng.profile_kernels(args.profile_iters)
    dom = max(kernels, key=lambda k: k["us_per_step"])
    per_launch_bytes = dom["bytes_per_step"] / dom["launches"]
    per_launch_us = dom["us_per_step"] / dom["launches"]
    achieved = per_launch_bytes / per_launch_us / 1e3
    traffic = pmc_traffic(dom["name"], w.name)
    reach = achievable_bandwidth(torch)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": round(traffic) if traffic is not None else None, "kernel": dom["name"],
                "bytes_per_launch": per_launch_bytes, "us_per_launch": round(per_launch_us, 3),
                "achievable": reach, "frac_of_achievable_read": round(achieved / reach["read_gbs"], 4)}

    # beyond the method: the visible K/V sweep (chunks wholly after pos not loaded; outputs bit-identical), timed
    # on the same engine and capture from where the timed steps ended; fewer bytes than the formula's count
    visible = None
    n_vis = min(64, w.cap - int(pos.max()))
    if args.visible_steps > 0 and n_vis >= 8:
        n_vis = min(n_vis, args.visible_steps)
        eng.set_kv_sweep("visible")
        torch.cuda.synchronize()
        tv = time.perf_counter()
        gv = []
        done = 0
        while done < n_vis:
            n = min(32, n_vis - done)
            ids, _ = eng.step_greedy(tok, pos, n)
            tok, pos, done = ids[-1].copy(), pos + n, done + n
            gv.append(eng.stats()["last_gpu_us"])
        torch.cuda.synchronize()
        ev = time.perf_counter() - tv
        eng.set_kv_sweep("full")
        visible = {"tok_s": round(w.rows * n_vis / ev, 2), "gpu_ms": round(float(np.median(gv)) / 1e3, 4),
                   "steps": n_vis, "note": "K/V chunks wholly after pos skipped; not the method's full sweep"}
        log(f"visible sweep: {visible['tok_s']} tok/s, GPU {visible['gpu_ms']} ms/step")

    # the sampling suffix in place of the greedy pick (temperature, top-k, top-p, min-p, repetition penalty, the
    # drawn token's log-probability and the top 5), on the same engine from where the steps above ended
    sampled = None
    n_smp = min(args.sample_steps, w.cap - int(pos.max()))
    if args.sample_steps > 0 and n_smp >= 8:
        params = dict(temperature=0.8, top_k=40, top_p=0.95, min_p=0.02, repetition_penalty=1.1, n_logprobs=5)
        for r in range(w.rows):
            eng.set_sampling(r, seed=1234 + r, **params)
            eng.set_history(r, [int(tok[r])])
        torch.cuda.synchronize()
        ts0 = time.perf_counter()
        gs = []
        done = 0
        while done < n_smp:
            n = min(32, n_smp - done)
            ids, _, _, _ = eng.step_sample(tok, pos, n)
            tok, pos, done = ids[-1].copy(), pos + n, done + n
            gs.append(eng.stats()["last_gpu_us"])
        torch.cuda.synchronize()
        es = time.perf_counter() - ts0
        sampled = {"tok_s": round(w.rows * n_smp / es, 2), "gpu_ms": round(float(np.median(gs)) / 1e3, 4),
                   "steps": n_smp, "params": params}
        log(f"sampling suffix: {sampled['tok_s']} tok/s, GPU {sampled['gpu_ms']} ms/step")
    # the step as the pages count it per token: one host wait per step, the logits copied back, the greedy token
    # picked on the host (same engine, from where the steps above ended)
    readback = None
    n_rb = min(32, w.cap - int(pos.max()))
    if n_rb >= 4:
        wr, gr = [], []
        torch.cuda.synchronize()
        tr = time.perf_counter()
        for _ in range(n_rb):
            ts = time.perf_counter()
            lg, _ = eng.step(tok, pos)
            tok = lg.argmax(axis=1).astype(np.int32)
            pos = pos + 1
            wr.append(time.perf_counter() - ts)
            gr.append(eng.stats()["last_gpu_us"])
        er = time.perf_counter() - tr
        readback = {"tok_s": round(w.rows * n_rb / er, 2), "steps": n_rb,
                    "wall_ms_p10_p50_p90": [round(1e3 * float(np.percentile(wr, q)), 4) for q in (10, 50, 90)],
                    "gpu_ms": round(float(np.median(gr)) / 1e3, 4),
                    "token_pick": "host argmax of the copied logits, one host wait per step"}
        log(f"per-token readback: {readback['tok_s']} tok/s")

    # the oracle on this host's cores (a bounded sample of the same workload), and the engine against it
    cpu = parity = None
    if not args.no_cpu_baseline:
        single = 10.0 if w.name in ("tiny-fp32", "llama1b-bf16") else 0.0
        cpu, ref = cpu_baseline(w, ws, start_pos, start_tok, args.cpu_baseline_seconds, single)
        log(f"cpu oracle {cpu['value']:.4f} tok/s on {cpu['cores']} threads")
        parity = parity_leg(eng, w, start_pos, start_tok, ref)
        log(f"parity: max-abs logits error {parity['logits_max_abs_err']}, greedy {parity['greedy_equal']}/"
            f"{parity['greedy_checked']}, free-running agreement {parity['free_running_agreement']}/"
            f"{parity['free_running_of']}")
    eng.close()
    del eng
    torch.cuda.empty_cache()

    # the per-operation kernels, replayed as one graph and launched one by one: host time per token
    per_op = {}
    if args.eager_steps > 0:
        for mode in ("graph", "eager"):
            e2 = engine_for(w, ws, mode, "per_op")
            prefill(e2, w, start_pos)   # (start_tok already holds a prompt workload's first token)
            sub, wl, gu = [], [], []
            p2, t2 = start_pos.copy(), start_tok.copy()
            for i in range(args.eager_steps + 2):
                ts = time.perf_counter()
                lg, _ = e2.step(t2, p2)
                t2 = lg.argmax(axis=1).astype(np.int32)
                p2 = p2 + 1
                if i >= 2:
                    wl.append(time.perf_counter() - ts)
                    st2 = e2.stats()
                    sub.append(st2["last_submit_us"])
                    gu.append(st2["last_gpu_us"])
            per_op[mode] = {"host_submit_us": round(float(np.median(sub)), 1),
                            "wall_ms": round(1e3 * float(np.median(wl)), 3),
                            "gpu_ms": round(float(np.median(gu)) / 1e3, 4),
                            "kernels_per_step": e2.stats()["kernels_per_step"]}
            e2.close()
            del e2
            torch.cuda.empty_cache()


    metric = METRIC if w.name == "llama8b-bf16-cap8192" else f"decode tokens/s + % HBM roofline, {w.name}"
    out = {
        "metric": metric,
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m.weight_dtype,
        "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) K/V prefill, greedy tokens)",
        "config": {"workload": w.name, "rows": w.rows, "layers": m.n_layers, "d_model": m.d_model,
                   "heads": f"{m.n_q_heads}q/{m.n_kv_heads}kv x {m.head_dim}", "ffn": m.ffn_dim,
                   "vocab": m.vocab, "cap": w.cap, "kv": f"{w.kv_layout} {w.kv_dtype}",
                   "start_pos": int(start_pos[0])},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "step": {"bytes": step_bytes, "gpu_ms": round(gpu_ms, 4),
                 "hbm_gbs": round(step_bytes / gpu_ms / 1e6, 1),
                 "hbm_frac": round(step_bytes / gpu_ms / 1e6 / HBM_PEAK_GBS, 4),
                 "wall_ms_p10_p50_p90": [round(1e3 * float(np.percentile(wall, q)), 4) for q in (10, 50, 90)],
                 "wall_samples": len(wall), "per_token_readback": readback,
                 "kernel_plan": stats["kernel_plan"],
                 "kernels_per_step": stats["kernels_per_step"], "graph_replays_per_step": 1,
                 "steps_per_host_wait": chain if chain > 0 else 1,
                 "token_pick": "device (greedy, chained)" if chain > 0 else "host argmax of copied logits",
                 "host_submit_us_graph": round(float(np.median(submit_us)), 1),
                 "per_op_graph": per_op.get("graph", {}), "eager": per_op.get("eager", {}),
                 "attn_splits": stats["attn_splits"], "visible_sweep": visible, "sampled": sampled, "prompt_prefill": prefill.last},
        "kernels": [{"name": k["name"], "launches": k["launches"], "us_per_step": round(k["us_per_step"], 2),
                     "gbs": round(k["bytes_per_step"] / k["us_per_step"] / 1e3, 1) if k["us_per_step"] else None}
                    for k in kernels],
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
