#!/usr/bin/env python3
"""Benchmark: verified draft positions per second on one MI355X, with the HBM
roofline of the dominant kernel and the CPU oracle timed beside it.

One step = the whole hot path on one batch already resident in HBM:
  sv_allocate_budget (prefix-confidence products + radix select of the top K)
  -> sv_verify_batch (row statistics, acceptance rates, accept scan, draw,
     and the batch's acceptance statistics, the outputs of sv_accept_stats,
     from one extra workgroup of its float64 tile kernel).
Default workload: the 64 x 16 x 151936 bf16 batch at T = 1 with the budget
keeping every position (K = 1024).  Inputs are synthetic (seeded Gaussian
logits shaped like the AngelSpec pages' block-drafting workload).  Four input
copies rotate between steps so that no step finds its logits in the 256 MB
Infinity Cache.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4full]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c4full",
                    choices=["c4full", "c4", "c3", "c3_t0", "c2", "c5"])
    ap.add_argument("--copies", type=int, default=4,
                    help="input copies rotated between steps (beyond the 256 MB Infinity Cache)")
    ap.add_argument("--row-pass", choices=("team", "stream"), default="team",
                    help="team: each row pair read once into registers (k_rowteam); "
                         "stream: streaming pass that reads a row pair twice (k_rowpass)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU work budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the draft-side, decode-loop and sharded figures (profiling runs)")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the plain streaming-read measurement (k_stream_read)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB "
                         "(a reference dispatch for scaling rocprofv3 byte counters)")
    return ap.parse_args()


# Sources each row-pass kernel is built from: a counter summary stays valid
# while their code (comments aside) is unchanged.
KERNEL_SOURCES = {
    "k_rowteam": ["sv_rowteam.hip", "sv_block.hpp", "sv_device.hpp", "sv_internal.hpp"],
    "k_rowpass": ["sv_rowpass.hip", "sv_block.hpp", "sv_device.hpp", "sv_internal.hpp"],
}


def _code_only(text: str) -> str:
    """Source text without comments and blank lines: a comment edit leaves
    the compiled kernel, and so its counters, unchanged."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "lossless_draft_verification_softmax_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, digest: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(f"{kernel}@{workload}")
    if not ent or ent.get("source_digest") != digest:
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_baseline(w, target_packed, depth, tr0, dr0, seconds: float):
    """The oracle, as it stands, on whole requests of the same batch, one
    request per call on a pool of host threads (the oracle's C calls run
    outside the GIL), until the batch is done or about `seconds` have passed:
    verified positions per second of wall time."""
    import concurrent.futures
    import threading
    import numpy as np
    import oracle
    th = target_packed.float().cpu().numpy().reshape(-1, w.V)
    dh = w.draft.float().cpu().numpy().reshape(-1, w.V)
    tok = w.draft_tokens.cpu().numpy()
    temps = w.temperature.cpu().numpy()
    dep = depth.cpu().numpy()
    tr = tr0.cpu().numpy()
    dr = dr0.cpu().numpy()
    oracle.lib()
    t0 = time.perf_counter()
    oracle.allocate_budget(w.conf.numpy(), w.K)
    budget_s = time.perf_counter() - t0
    # the host share of one GPU: at most 16 threads
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    lock = threading.Lock()
    state = {"next": 0, "positions": 0, "done": 0}
    t0 = time.perf_counter()

    def worker():
        while True:
            with lock:
                r = state["next"]
                if r >= w.B or time.perf_counter() - t0 >= seconds:
                    return
                state["next"] = r + 1
            oracle.verify_batch(th, dh, tr[r:r + 1], dr[r:r + 1], tok[r:r + 1], dep[r:r + 1],
                                temps[r:r + 1], request_id=np.array([r], np.uint32), D_max=w.D)
            with lock:
                state["positions"] += int(dep[r])
                state["done"] += 1

    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(worker) for _ in range(workers)]:
            f.result()
    elapsed = time.perf_counter() - t0
    # the same oracle on one core: requests in order, one per call, until the
    # batch is done or a third of the budget has passed
    t1 = time.perf_counter()
    one_pos = one_done = 0
    for r in range(w.B):
        if time.perf_counter() - t1 >= seconds / 3.0:
            break
        oracle.verify_batch(th, dh, tr[r:r + 1], dr[r:r + 1], tok[r:r + 1], dep[r:r + 1],
                            temps[r:r + 1], request_id=np.array([r], np.uint32), D_max=w.D)
        one_pos += int(dep[r])
        one_done += 1
    one_s = time.perf_counter() - t1
    return dict(value=state["positions"] / elapsed, unit="positions/s", cores=workers,
                kind="oracle",
                sample=f"{state['done']} of {w.B} requests ({state['positions']} verified "
                       f"positions) of the {w.name} batch, one request per call on "
                       f"{workers} host threads, {elapsed:.1f} s wall; budget "
                       f"{budget_s * 1e3:.2f} ms single-threaded",
                cpu_model=cpu_model(),
                single_core={"value": one_pos / one_s if one_s > 0 else None,
                             "unit": "positions/s", "cores": 1,
                             "sample": f"requests 0..{one_done - 1} of the {w.name} batch "
                                       f"({one_pos} verified positions) in order on one host "
                                       f"thread, {one_s:.1f} s"})


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo, as lscpu reports it)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def read_ceiling(sv, torch, dev, nbytes: int, reps: int = 10):
    """The chip's plain streaming-read rate (sv_stream_read) over two buffers
    of the row pass's algorithmic size, read alternately so that neither is
    served from the 256 MB Infinity Cache: the best of four launch shapes."""
    n = (nbytes + 15) // 16 * 16
    bufs = [torch.full((n // 4,), 1.0, dtype=torch.float32, device=dev) for _ in range(2)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    best = None
    for per_cu in (1, 2, 4, 8):
        for b in bufs:
            sv.stream_read(b, sink, per_cu)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            sv.stream_read(bufs[i % 2], sink, per_cu)
        e1.record()
        torch.cuda.synchronize()
        gbs = n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, per_cu)
    del bufs
    return {"kernel": "k_stream_read", "bytes": n, "GBps": round(best[0], 1),
            "workgroups_per_cu": best[1], "frac_of_peak": round(best[0] / HBM_PEAK_GBS, 4)}


def draft_side(sv, torch, w, copies, dr0, bud, verifiers, esize):
    """The budget's inputs, timed apart from the verification step: the
    drafter confidence q_k(d_k) of every drafted position (one pass over the
    draft rows, rotating the input copies), and D-cut's keep-ratio choice
    from a cost table profiled here by timing the verification step at each
    ratio's budget."""
    B, D, V = w.B, w.D, w.V
    dc = sv.DraftConfidence(B, D, V, w.dtype, copies[0][1].device)
    drafts = [d.reshape(B * D, V) for _, d in copies]
    for i in range(6):
        dc(drafts[i % len(drafts)], dr0, w.draft_tokens, w.temperature)
    torch.cuda.synchronize()
    n = 40
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        dc(drafts[i % len(drafts)], dr0, w.draft_tokens, w.temperature)
    e1.record()
    torch.cuda.synchronize()
    conf_us = e0.elapsed_time(e1) / n * 1e3
    conf_bytes = B * D * V * esize
    conf = dc.conf.clone()
    # cost table: verification step time at each ratio's K on this batch
    ratios = list(sv.DCUT_RATIOS)
    lat = []
    for rho in ratios:
        K = math.ceil(rho * B * D)
        b = sv.allocate_budget(conf, K)
        for v in verifiers:  # padded target rows: row r (D + 1) + k
            v.prepare(w.target.reshape(-1, V), w.draft, torch.arange(B, device=conf.device) * (D + 1),
                      dr0, w.draft_tokens, b["depth"], w.temperature, seed=0, step=0)
        for i in range(3):
            verifiers[i % len(verifiers)].run()
        torch.cuda.synchronize()
        e0.record()
        for i in range(10):
            verifiers[i % len(verifiers)].run()
        e1.record()
        torch.cuda.synchronize()
        lat.append(e0.elapsed_time(e1) / 10 * 1e3)
    for i in range(3):
        sel = sv.select_budget_ratio(conf, [B], [lat], ratios)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        sel = sv.select_budget_ratio(conf, [B], [lat], ratios)
    e1.record()
    torch.cuda.synchronize()
    sel_us = e0.elapsed_time(e1) / n * 1e3
    ach = conf_bytes / (conf_us * 1e-6) / 1e9
    # utility retained at the chosen K: the global top-K against the
    # fixed-depth baseline (the budget widget's comparison)
    K_sel = int(sel["K"].item())

    def retained_at(c):
        ug = sv.allocate_budget(c, K_sel)["utility"].cpu().tolist()
        uf = sv.allocate_fixed_depth(c, K_sel)["utility"].cpu().tolist()
        return {"global": round(ug[0] / ug[1], 4) if ug[1] else None,
                "fixed": round(uf[0] / uf[1], 4) if uf[1] else None}

    retained = {"K": K_sel, "kernels": "k_budget, k_budget_fixed",
                "drafter_confidence": retained_at(conf)}
    if w.conf is not None:  # the workload's Beta(8, 2) / Beta(3, 3) confidences
        retained["beta_confidence"] = retained_at(w.conf.to(conf.device).contiguous())
    return {
        "draft_confidence": {"kernels": "k_conf_part + k_conf_final", "us": round(conf_us, 2),
                             "algorithmic_bytes": conf_bytes, "achieved_GBps": round(ach, 1),
                             "frac": round(ach / HBM_PEAK_GBS, 4)},
        "ratio_choice": {"kernel": "k_budget_ratio", "us": round(sel_us, 2),
                         "ratios": ratios, "verify_us_at_ratio": [round(x, 1) for x in lat],
                         "projected_tokens_per_us": [round(float(x), 5) for x in sel["projected"].cpu()],
                         "choice": int(sel["choice"].item()), "K": int(sel["K"].item())},
        "utility_retained": retained,
    }


def sharded_figure(sv, torch, w, tgt, dft, bud, dr0, n_shards, rowpass_bytes, step_us):
    """The same verification with the vocabulary split over n_shards buffers
    (a tensor-parallel target's layout, all on this GPU): time per call."""
    B, D, V = w.B, w.D, w.V
    W = -(-V // n_shards)
    W = -(-W // 8) * 8

    def split(rows):
        out = []
        for s in range(0, V, W):
            buf = torch.empty((rows.shape[0], W), dtype=rows.dtype, device=rows.device)
            part = rows[:, s:s + W]
            buf[:, : part.shape[1]] = part
            out.append(buf)
        return out

    ts, ds = split(tgt), split(dft.reshape(B * D, V))
    v = sv.Verifier(B, D, V, tgt.device, alpha=True, diag=True)
    v.prepare_sharded(ts, ds, W, bud["target_row0"], dr0, w.draft_tokens, bud["depth"],
                      w.temperature, seed=0, step=0)
    for _ in range(5):
        v.run()
    torch.cuda.synchronize()
    n = 30
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        v.run()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    del ts, ds
    return {"shards": len(range(0, V, W)), "shard_width": W, "verify_us": round(us, 1),
            "unsharded_verify_us": round(step_us, 1),
            "algorithmic_GBps": round(rowpass_bytes / (us * 1e-6) / 1e9, 1)}


def decode_loop_figure(sv, torch, dev, V=32768, B=64, D=8, steps=30):
    """The multi-step decode loop on a synthetic Markov target (bf16 tables of
    V x V, target P ~ 3 N(0, 1), drafter Q = P + N(0, 1), T = 1): time per
    step (D sampler calls, row gather, verification, statistics), emitted
    tokens per second, MAL and position-wise acceptance."""
    from lossless_draft_verification_softmax_amd.decode_loop import MarkovDecodeLoop
    g = torch.Generator(device=dev)
    g.manual_seed(4000)
    P = (3.0 * torch.randn((V, V), generator=g, device=dev)).to(torch.bfloat16)
    Q = (P.float() + torch.randn((V, V), generator=g, device=dev)).to(torch.bfloat16)
    start = torch.randint(0, V, (B,), generator=g, device=dev, dtype=torch.int64).to(torch.int32)
    loop = MarkovDecodeLoop(P, Q, start, D, torch.ones(B, device=dev), seed=0)
    for _ in range(3):
        loop.step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    emitted = torch.zeros((), dtype=torch.int64, device=dev)
    e0.record()
    for _ in range(steps):
        out = loop.step()
        emitted += out.accepted_len.sum() + B
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    summ = loop.summary()
    del P, Q
    return {"workload": f"Markov target V={V} bf16, B={B}, D={D}, T=1", "us_per_step": round(us, 1),
            "emitted_tokens_per_s": round(float(emitted.item()) / (us * steps * 1e-6), 1),
            "mal": round(summ["mal"], 4), "expected_mal": round(summ["expected_mal"], 4),
            "mean_acceptance": round(summ["mean_acceptance"], 4),
            "position_acceptance_P_tau_ge_k": [round(x, 4) for x in summ["position_acceptance"]]}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(every step of this workload fits one MI355X; the path shards by request or by "
              "vocabulary, but no multi-GPU run is made here)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    sys.path.insert(0, ROOT)
    from lossless_draft_verification_softmax_amd import specverify as sv
    from lossless_draft_verification_softmax_amd import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    sv.load()
    w = synth.make(args.workload, device=dev)
    B, D, V = w.B, w.D, w.V
    esize = 2 if w.dtype == torch.bfloat16 else 4

    conf = (w.conf if w.conf is not None else torch.ones((B, D))).to(dev).contiguous()
    K = w.K if w.K is not None else B * D
    bud = sv.allocate_budget(conf, K)
    torch.cuda.synchronize()
    depth_h = bud["depth"].cpu()
    # Target logits only for the kept positions, packed in the budget's order
    # (what a target forward over the surviving tokens produces); the drafter
    # produced all D positions, so draft rows stay padded.
    idx = torch.cat([torch.arange(int(n) + 1, device=dev) + r * (D + 1)
                     for r, n in enumerate(depth_h.tolist())])
    copies = []
    for c in range(args.copies):
        tgt = w.target.reshape(-1, V).index_select(0, idx).contiguous()
        dft = w.draft.clone() if c else w.draft
        copies.append((tgt, dft))
    dr0 = torch.arange(B, dtype=torch.int64, device=dev) * D
    row_flags = sv.SV_FLAG_STREAMING_ROW_PASS if args.row_pass == "stream" else 0
    row_kernel = "k_rowpass" if args.row_pass == "stream" else "k_rowteam"
    verifiers = []
    for tgt, dft in copies:
        v = sv.Verifier(B, D, V, dev, alpha=True, diag=True, stats=True)
        v.prepare(tgt, dft, bud["target_row0"], dr0, w.draft_tokens, bud["depth"], w.temperature,
                  seed=0, step=0, flags=row_flags)
        verifiers.append(v)
    stats_out = None

    n_pos = int(depth_h.sum())
    n_t0 = int((w.temperature == 0).sum())
    temps_h = w.temperature.cpu()
    draft_rows = int(sum(int(n) for n, t in zip(depth_h.tolist(), temps_h.tolist()) if t > 0))
    target_rows = n_pos + B
    # The row pass needs every logit row once: algorithmic bytes count each
    # row once (the streaming pass's second read of a row pair is traffic,
    # not algorithmic bytes)
    rowpass_bytes = (target_rows + draft_rows) * V * esize
    step_bytes = rowpass_bytes + n_pos * 4  # + draft token ids

    def step(v):
        nonlocal stats_out
        sv.allocate_budget(conf, K, out=bud)
        stats_out = v.run().stats  # the batch statistics come with the verification

    for i in range(args.warmup):
        step(verifiers[i % len(verifiers)])
    torch.cuda.synchronize()

    nev = sv.SV_NUM_STAGE_EVENTS

    def make_events(n, which):
        evs = [[torch.cuda.Event(enable_timing=True) if j in which else None for j in range(nev)]
               for _ in range(n)]
        for row in evs:
            for e in row:
                if e is not None:
                    e.record()
        return evs

    # Timed region: HIP events around the row pass (events [1] and [2] of
    # sv_verify_batch, on the stream the kernels run on) on every fourth
    # step; an event pair costs a few microseconds of idle GPU time.
    events = make_events(args.steps, (1, 2))
    for i in range(args.steps):
        if i % 4:
            events[i] = [None] * nev
    sampled = [evs for evs in events if evs[1] is not None]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        v = verifiers[i % len(verifiers)]
        v.set_stage_events(events[i])
        step(v)
    stop.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    rowpass_ms = sum(evs[1].elapsed_time(evs[2]) for evs in sampled) / len(sampled)

    # Stage breakdown from a separate, untimed loop with all five events.
    n_st = min(args.steps, 20)
    events = make_events(n_st, range(nev))
    torch.cuda.synchronize()
    for i in range(n_st):
        v = verifiers[i % len(verifiers)]
        v.set_stage_events(events[i])
        step(v)
    torch.cuda.synchronize()
    for v in verifiers:
        v.set_stage_events(None)
    stage_ms = [sum(evs[j].elapsed_time(evs[j + 1]) for evs in events) / n_st
                for j in range(nev - 1)]

    # Step-time distribution: one event between consecutive steps (each
    # recorded event leaves a few microseconds of idle GPU, so these spans
    # sit slightly above the timed loop's mean).
    n_ds = max(args.steps, 20)
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(n_ds + 1)]
    torch.cuda.synchronize()
    bounds[0].record()
    for i in range(n_ds):
        step(verifiers[i % len(verifiers)])
        bounds[i + 1].record()
    torch.cuda.synchronize()
    spans = sorted(bounds[i].elapsed_time(bounds[i + 1]) * 1e3 for i in range(n_ds))

    def pct(q):
        return round(spans[min(n_ds - 1, int(round(q * (n_ds - 1))))], 2)

    achieved = rowpass_bytes / (rowpass_ms * 1e-3) / 1e9
    digest = source_digest(row_kernel)
    traffic = measured_traffic(row_kernel, args.workload, digest)
    value = n_pos * args.steps / (total_ms * 1e-3)
    res = {
        "metric": "verified draft positions/sec @ V=151,936 bf16 + % of MI355X HBM roofline",
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if esize == 2 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: B={B} requests x D={D} draft positions, "
                               f"V={V} {'bf16' if esize == 2 else 'fp32'} logits, "
                               f"T={'mixed' if w.temperature.unique().numel() > 1 else float(temps_h[0])}, "
                               f"budget K={K}",
                   "batch": B, "depth": D, "vocab": V, "verified_positions": n_pos,
                   "budget_K": K, "greedy_requests": n_t0},
        "roofline": {"bound": "hbm", "kernel": row_kernel,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": rowpass_bytes,
                     "avg_launch_us": round(rowpass_ms * 1e3, 2)},
        "step_us_distribution": {"p10": pct(0.10), "p50": pct(0.50), "p90": pct(0.90),
                                 "steps": n_ds, "note": "one event per step boundary"},
        "step_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_algorithmic_bytes": step_bytes,
        "stages_us": {"plan": round(stage_ms[0] * 1e3, 2), "rowpass": round(stage_ms[1] * 1e3, 2),
                      "accept": round(stage_ms[2] * 1e3, 2), "draw": round(stage_ms[3] * 1e3, 2)},
        "wall_s": round(wall_s, 3),
        "mean_accepted_length": round(float(stats_out["summary"][0]), 4),
        "expected_mean_accepted_length": round(float(stats_out["summary"][1]), 4),
        "source_digest": digest,
    }
    if not args.no_read_ceiling:
        rc = read_ceiling(sv, torch, dev, rowpass_bytes)
        rc["rowpass_frac_of_ceiling"] = round(achieved / rc["GBps"], 4)
        res["read_ceiling"] = rc
    if D > 0 and draft_rows > 0 and not args.no_extras:
        res["draft_side"] = draft_side(sv, torch, w, copies, dr0, bud, verifiers, esize)
        res["decode_loop"] = decode_loop_figure(sv, torch, dev)
        verify_us = sum(stage_ms) * 1e3  # the stage events cover the whole verification
        res["sharded_tp8"] = sharded_figure(sv, torch, w, copies[0][0], copies[0][1], bud, dr0, 8,
                                            rowpass_bytes, verify_us)
    if args.calib_copy_mb:
        # a plain device copy of known size: scales rocprofv3's byte counters
        # and gives the copy bandwidth for context (read + write bytes / time)
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        res["calib_copy_bytes"] = n * 4
        res["device_copy_GBps"] = round(2 * n * 4 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, copies[0][0], bud["depth"], bud["target_row0"],
                                           dr0, args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
