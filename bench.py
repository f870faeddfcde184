"""Benchmark of one full optimizer step (Muon on every hidden matrix + AdamW
on embedding, LM head and norm vectors) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--coef quintic|cubic]

The default workload is the largest mixed one, ``ragged_500``: 500 ragged
matrices (1.01e10 parameters) flattened into one buffer plus AdamW on a
163840 x 7168 embedding and 128 vectors.

Prints ONE JSON line.  The step is launched through the C ABI stage entry
points (the same launches muon_step makes, in the same order, on torch's
current stream) so that HIP events can bracket each kernel inside the
timed region.  Inputs are seeded synthetic tensors already resident in
HBM; gradients stay fixed across steps (the optimizer work does not
depend on their values).  After the timed region the fp64 oracle checks
sampled matrices and an AdamW slice of the first step and of the last
timed step (their inputs are copied aside on the device before each of
those steps: a few MB).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X fp32 matrix
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def traffic_summary(workload):
    return os.path.join(PROFILES, f"ns_gemm_{workload}_traffic.md")


def mfma_summary(workload):
    return os.path.join(PROFILES, f"ns_gemm_{workload}_mfma.md")
# the NS kernels are compiled from these two files
NS_SOURCES = [os.path.join(ROOT, "muon_newton_schulz_amd", "csrc", f)
              for f in ("ns_gemm.hip", "muon_internal.h")]


def ns_source_sha256():
    """sha256 over the NS kernels' source files, in order."""
    import hashlib
    h = hashlib.sha256()
    for f in NS_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, or None when the summary is missing, is for
    another workload, or was taken on a different kernel source."""
    try:
        text = open(traffic_summary(workload)).read()
        block = text.split("```json", 1)[1].split("```", 1)[0]
        data = json.loads(block)
        sha = ns_source_sha256()
    except (OSError, IndexError, ValueError):
        return None
    if data.get("ns_sources_sha256") != sha or data.get("workload") != workload:
        return None
    return data["fetch_bytes_per_launch"] + data["write_bytes_per_launch"]


def measured_mfma_util(workload):
    """rocprofv3 MfmaUtil (MFMA-busy cycles per SIMD over active cycles, in
    %) of each NS kernel from the committed counter summary, or None when
    it is missing, is for another workload, or was taken on a different
    kernel source."""
    try:
        text = open(mfma_summary(workload)).read()
        data = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        sha = ns_source_sha256()
    except (OSError, IndexError, ValueError):
        return None
    if data.get("ns_sources_sha256") != sha or data.get("workload") != workload:
        return None
    return {k: round(v["mfma_util_pct"], 1) for k, v in data["kernels"].items()}


def run_ceiling(name):
    """One of the stand-alone measurement programs (muon_newton_schulz_amd/
    mfma_ceiling: back-to-back MFMAs from registers on every SIMD, no memory
    traffic; hbm_ceiling: plain read + write, read and write streams over
    2 GiB buffers), or None if it is missing or fails.  Run as a child
    process after the timed region."""
    import subprocess
    exe = os.path.join(ROOT, "muon_newton_schulz_amd", name)
    if not os.path.exists(exe):
        return None
    try:
        res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        return json.loads(res.stdout.strip().splitlines()[-1]) if res.returncode == 0 else None
    except (OSError, ValueError, IndexError, subprocess.TimeoutExpired):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ragged_500")
    ap.add_argument("--coef", default="quintic", choices=["quintic", "cubic"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-flops", type=float, default=5e12,
                    help="fp64 NS flops of the oracle's CPU sample (about 10 s on 16 cores)")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the oracle checks of the first and last step")
    ap.add_argument("--no-fp32-ns", action="store_true",
                    help="skip the timing of the fp32 NS engine on one dense layer")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the MFMA and HBM ceiling programs (profiling runs)")
    ap.add_argument("--adamw-stream", choices=["same", "side"], default="side",
                    help="AdamW on the Muon stream, or on a second stream beside the NS kernels")
    ap.add_argument("--adamw-beside", type=int, choices=[1, 2, 3], default=1,
                    help="with a side stream: the NS phase of the first iteration AdamW starts with")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also launch one plain device copy of this many MiB (counter scale)")
    return ap.parse_args()


def van_der_corput(n):
    """0, 1/2, 1/4, 3/4, 1/8, 5/8, 3/8, 7/8, ...: positions that spread any
    prefix of the sequence evenly over [0, 1)."""
    out = []
    for k in range(n):
        x, f, q = 0.0, 0.5, k
        while q:
            x += f * (q & 1)
            q >>= 1
            f /= 2
        out.append(x)
    return out


def cpu_sample(wl, hp, flop_budget):
    """Deterministic sample of the workload's matrices for the oracle: the
    matrices sorted by NS flops, visited at van der Corput positions (so the
    sample spreads over small and large matrices), each taken while the
    sample's flops stay within the budget.  A workload within the budget is
    taken whole."""
    from muon_newton_schulz_amd import workloads as W
    shapes = wl.shapes
    fl = [W.ns_flops_matrix(r, c, hp.ns_steps, hp.ns_c) for r, c in shapes]
    if sum(fl) <= flop_budget:
        return list(range(len(shapes)))
    order = sorted(range(len(shapes)), key=lambda i: (fl[i], i))
    picked, seen, total = [], set(), 0
    for x in van_der_corput(4 * len(order)):
        j = order[min(len(order) - 1, int(x * len(order)))]
        if j in seen:
            continue
        seen.add(j)
        if total + fl[j] <= flop_budget:
            picked.append(j)
            total += fl[j]
    return sorted(picked)


def cpu_baseline(wl, hp, flop_budget, adam_n):
    """The fp64 oracle, as it stands, on a bounded sample of the same
    workload, timed on the host cores: the full Muon step of the sampled
    matrices (cpu_sample) and AdamW over adam_n elements.  The whole-step
    oracle time is extrapolated linearly (Muon by NS flops, AdamW by
    elements) and reported in the GPU value's unit: NS flops of the whole
    step per second of the whole step."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from muon_newton_schulz_amd import workloads as W
    from oracle import muon_oracle as O

    ohp = O.MuonHP(lr=hp.lr, weight_decay=hp.weight_decay, momentum=hp.momentum,
                   nesterov=hp.nesterov, ns_a=hp.ns_a, ns_b=hp.ns_b, ns_c=hp.ns_c,
                   ns_steps=hp.ns_steps, eps=hp.eps, scale_mode=hp.scale_mode,
                   rms_target=hp.rms_target)
    mats = wl.mats()
    sample = cpu_sample(wl, hp, flop_budget)
    t_muon = 0.0
    for i in sample:   # inputs drawn per matrix (not timed), then its oracle step
        o, r, c = mats[i]
        w = W.normal_tensor(r * c, wl.w_std, wl.param_dtype, W.seed_key(wl.config_id, 0, i, 0))
        g = W.normal_tensor(r * c, wl.g_std, wl.grad_dtype, W.seed_key(wl.config_id, 1, i, 1))
        w, g = w.double().numpy().reshape(r, c), g.double().numpy().reshape(r, c)
        t0 = time.perf_counter()
        O.muon_matrix_math(w, g, np.zeros((r, c)), ohp)
        t_muon += time.perf_counter() - t0
    n_adam_total = wl.adam_numel()
    adam_n = min(adam_n, n_adam_total)
    t_adam = 0.0
    if adam_n:
        grp = wl.adam[0]
        ap = W.normal_tensor(adam_n, max(grp.p_std, 0.02), "fp32", 99).double().numpy()
        ag = W.normal_tensor(adam_n, grp.g_std, grp.grad_dtype, 98).double().numpy()
        ahp = O.AdamWHP(wl.adam_hp.lr, wl.adam_hp.beta1, wl.adam_hp.beta2, wl.adam_hp.eps,
                        wl.adam_hp.weight_decay)
        t0 = time.perf_counter()
        O.adamw_step_stored(O.bf16_round(ap), ap, ag, np.zeros(adam_n), np.zeros(adam_n), ahp,
                            1, "bf16")
        t_adam = time.perf_counter() - t0
    flops_sample = sum(W.ns_flops_matrix(mats[i][1], mats[i][2], hp.ns_steps, hp.ns_c)
                       for i in sample)
    flops_total = W.ns_flops_workload(wl, hp.ns_steps, hp.ns_c)
    full = len(sample) == len(mats) and adam_n == n_adam_total
    t_step = (t_muon * flops_total / flops_sample
              + (t_adam * n_adam_total / adam_n if adam_n else 0.0))
    threads = max((d.get("num_threads", 1) for d in threadpool_info()
                   if d.get("user_api") == "blas"), default=1)
    sample_params = sum(mats[i][1] * mats[i][2] for i in sample)
    return {
        "value": flops_total / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 NumPy oracle, {'whole step' if full else 'extrapolated'}: full Muon "
                   f"step on {len(sample)} of {len(mats)} matrices ({sample_params / wl.muon_numel():.1%}"
                   f" of the Muon params, {flops_sample / 1e12:.2f} of {flops_total / 1e12:.1f} "
                   f"TFLOP of NS; matrices sorted by flops, taken at van der Corput positions "
                   f"within a {flop_budget / 1e12:.3g} TFLOP budget) in {t_muon:.1f} s, plus "
                   f"AdamW on {adam_n} of {n_adam_total} elements in {t_adam:.2f} s; whole "
                   f"step {t_step:.0f} s {'measured' if full else 'extrapolated linearly by NS flops and AdamW elements'}"),
        "extrapolated": not full,
        "sample_matrices": sample,
        "ns_tflops_sample": flops_sample / t_muon / 1e12 if t_muon else None,
        "muon_seconds": t_muon,
        "adamw_seconds": t_adam,
        "step_seconds_extrapolated": t_step,
    }


def parity_matrices(wl):
    """Matrices the oracle checks at the first and last step: the smallest
    whose offset and cols are multiples of 8 and the smallest of the others
    (with bf16 parameters both take the update fused into the last NS phase,
    the second with its rows realigned onto the 8-element grid)."""
    mats = wl.mats()
    size = lambda i: mats[i][1] * mats[i][2]  # noqa: E731
    on8 = [i for i, (o, r, c) in enumerate(mats) if o % 8 == 0 and c % 8 == 0]
    off8 = [i for i, (o, r, c) in enumerate(mats) if not (o % 8 == 0 and c % 8 == 0)]
    return sorted({min(grp, key=size) for grp in (on8, off8) if grp})


def half_ulp(x, dtype):
    """Half an ulp of each stored value (bf16: 8 significant bits, fp32: 24)."""
    import numpy as np
    bits = 8 if dtype == "bf16" else 24
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - bits)


def oracle_check(wl, hp, ahp_w, snap_pre, snap_post, t):
    """fp64 oracle against one step's results: per sampled matrix M (<= 2e-6)
    and the update W implies, O_impl = (decay W0 - W1) / step, against O
    (<= 1e-2 bf16 NS, 1e-4 fp32 NS, plus the storage rounding of W1 over
    step); AdamW master, m, v (<= 2e-6) and the 16-bit parameter equal to
    the cast of the master."""
    import math

    import numpy as np

    from oracle import muon_oracle as O
    ohp = O.MuonHP(lr=hp.lr, weight_decay=hp.weight_decay, momentum=hp.momentum,
                   nesterov=hp.nesterov, ns_a=hp.ns_a, ns_b=hp.ns_b, ns_c=hp.ns_c,
                   ns_steps=hp.ns_steps, eps=hp.eps, scale_mode=hp.scale_mode,
                   rms_target=hp.rms_target)

    def rel(a, b):
        nb = np.linalg.norm(b)
        return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))

    tol_o = 1e-2
    res, ok = {"t": t, "matrices": {}}, True
    for i, (r, c, W0, G, M0) in snap_pre["mats"].items():
        W1, M1 = snap_post["mats"][i][2], snap_post["mats"][i][4]
        _, Mr, Or = O.muon_matrix_math(W0, G, M0, ohp)
        em = rel(M1, O.fp32_round(Mr))
        decay = float(np.float32(1.0) - np.float32(hp.lr) * np.float32(hp.weight_decay))
        step = float(np.float32(hp.lr) * np.float32(
            O.update_scale(r, c, hp.scale_mode, hp.rms_target)))
        eo = rel((decay * W0 - W1) / step, Or)
        slack = float(np.linalg.norm(half_ulp(W1, wl.param_dtype)) / (step * np.linalg.norm(Or)))
        good = em <= 2e-6 and eo <= tol_o + slack
        ok &= good
        res["matrices"][str(i)] = {"shape": [r, c], "M": em, "O_from_W": eo,
                                   "O_tol": tol_o + slack, "ok": good}
    if snap_pre.get("adam") is not None:
        p0, m0, e0, v0, g = snap_pre["adam"]
        p1, m1, e1, v1, _ = snap_post["adam"]
        pdt = wl.adam[0].param_dtype
        pr, mr, er, vr = O.adamw_step_stored(p0, m0, g, e0, v0, ahp_w, t, pdt)
        th1 = m1 if m1 is not None else p1
        thr = mr if mr is not None else pr
        ea = {"theta": rel(th1, thr), "m": rel(e1, er), "v": rel(v1, vr)}
        cast_ok = True if m1 is None else bool(np.array_equal(p1, O.round_to(m1, pdt)))
        good = max(ea.values()) <= 2e-6 and cast_ok
        ok &= good
        res["adamw"] = {**ea, "param_is_cast_of_master": cast_ok, "ok": good}
    res["ok"] = bool(ok)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the optimizer step runs on one GPU only; --gpus must be 1 "
                          "(the path shards by whole matrices across GPUs, not implemented)"}))
        sys.exit(2)

    import torch

    import muon_newton_schulz_amd as M
    from muon_newton_schulz_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M.lib()
    wl = W.workload(args.workload)
    coef = W.QUINTIC if args.coef == "quintic" else W.CUBIC
    hp = wl.muon_hp
    hp.ns_a, hp.ns_b, hp.ns_c = coef
    ahp = wl.adam_hp

    # ---- inputs resident in HBM (seeded, generated on the device)
    inp = W.make_muon_inputs(wl, dev, step=1)
    plan = M.muon_plan_create(wl.mats(), wl.muon_numel(), wl.param_dtype, wl.grad_dtype, "bf16")
    info = plan.info()
    ws = plan.alloc_workspace(dev)
    adam = [W.make_adam_inputs(wl, gi, device=dev, step=1) for gi in range(len(wl.adam))]
    calib = None
    if args.copy_calibration:
        nb = args.copy_calibration << 20
        calib = (torch.empty(nb, dtype=torch.uint8, device=dev),
                 torch.empty(nb, dtype=torch.uint8, device=dev))
        calib[0].fill_(1)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    # AdamW does not depend on the Muon group: optionally on its own stream
    # (default priority), joined back at the end of the step
    side = torch.cuda.Stream() if args.adamw_stream == "side" else None
    n_waves = info.n_waves
    phases = (1, 2, 3) if hp.ns_c != 0.0 else (1, 3)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    t_step = [0]

    def one_step(record):
        """One optimizer step; with ``record`` returns per-kernel event pairs."""
        marks = {"momentum": [], "ns1": [], "ns2": [], "ns3": [], "ns3_apply": [], "adamw": []}

        def timed(key, fn, st=None):
            st = stream if st is None else st
            if record:
                a, b = ev(), ev()
                a.record(st)
                fn()
                b.record(st)
                marks[key].append((a, b))
            else:
                fn()

        def adamw_all():
            for a in adam:
                timed("adamw", lambda: M.adamw_step(a.param, a.master, a.grad, a.exp_avg,
                                                    a.exp_avg_sq, ahp, t_step[0]),
                      side)

        t_step[0] += 1
        for w in range(n_waves):
            timed("momentum", lambda: M.muon_stage_momentum(plan, w, inp.grads, inp.momentum,
                                                            ws, hp))
            # the last phase 3 applies the update (as muon_step does)
            for it in range(hp.ns_steps):
                for ph in phases:
                    if side is not None and w == 0 and it == 0 and ph == args.adamw_beside:
                        # after the (bandwidth-bound) momentum pass, beside
                        # a compute-bound NS kernel
                        side.wait_stream(stream)
                        with torch.cuda.stream(side):
                            adamw_all()
                    if ph == 3 and it == hp.ns_steps - 1:
                        timed("ns3_apply",
                              lambda: M.muon_stage_ns_apply(plan, w, inp.params, ws, hp))
                    else:
                        timed(f"ns{ph}", lambda: M.muon_stage_ns_phase(plan, w, ws, hp, it, ph))
        if side is None:
            adamw_all()
        else:
            stream.wait_stream(side)
        return marks

    # ---- oracle checks of the first step and of the last timed step: the
    # inputs and results of a few sampled matrices and of an AdamW slice are
    # copied aside on the device (device-to-device, on the stream: a few MB)
    do_parity = not args.no_parity
    chk = parity_matrices(wl) if do_parity else []
    mats = wl.mats()
    asl = slice(0, min(4096, wl.adam[0].numel)) if wl.adam else None

    def snap():
        out = {"mats": {}, "adam": None}
        for i in chk:
            o, r, c = mats[i]
            sl = slice(o, o + r * c)
            out["mats"][i] = (r, c, inp.params[sl].clone(), inp.grads[sl].clone(),
                              inp.momentum[sl].clone())
        if asl is not None:
            a = adam[0]
            out["adam"] = (a.param[asl].clone(),
                           a.master[asl].clone() if a.master is not None else None,
                           a.exp_avg[asl].clone(), a.exp_avg_sq[asl].clone(), a.grad[asl].clone())
        return out

    def host(sn):
        f64 = lambda t: None if t is None else t.double().cpu().numpy()  # noqa: E731
        return {"mats": {i: (r, c, f64(w).reshape(r, c), f64(g).reshape(r, c),
                             f64(m).reshape(r, c))
                         for i, (r, c, w, g, m) in sn["mats"].items()},
                "adam": None if sn["adam"] is None else tuple(f64(t) for t in sn["adam"])}

    snaps = {}
    n_done = 0

    def counted_step(record):
        nonlocal n_done
        if do_parity and n_done == 0:
            snaps["first_pre"] = snap()
        marks = one_step(record)
        n_done += 1
        if do_parity and n_done == 1:
            snaps["first_post"] = snap()
        return marks

    for _ in range(args.warmup):
        counted_step(False)
    if calib is not None:
        calib[1].copy_(calib[0])
    torch.cuda.synchronize()

    start, end = ev(), ev()
    step_ev = [ev() for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    all_marks = []
    for j in range(args.steps):
        if do_parity and j == args.steps - 1:
            snaps["last_pre"] = snap()
        step_ev[j].record(stream)
        all_marks.append(counted_step(True))
    step_ev[args.steps].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / args.steps
    step_ms = sorted(step_ev[j].elapsed_time(step_ev[j + 1]) for j in range(args.steps))
    ms_median = (step_ms[(args.steps - 1) // 2] + step_ms[args.steps // 2]) / 2
    parity = None
    if do_parity:
        snaps["last_post"] = snap()
        torch.cuda.synchronize()
        ahp_o = None
        if wl.adam:
            from oracle import muon_oracle as O
            ahp_o = O.AdamWHP(ahp.lr, ahp.beta1, ahp.beta2, ahp.eps, ahp.weight_decay)
        parity = {
            "first_step": oracle_check(wl, hp, ahp_o, host(snaps["first_pre"]),
                                       host(snaps["first_post"]), 1),
            "last_step": oracle_check(wl, hp, ahp_o, host(snaps["last_pre"]),
                                      host(snaps["last_post"]), n_done),
        }
        parity["ok"] = parity["first_step"]["ok"] and parity["last_step"]["ok"]
        del snaps

    def avg_ms(key):
        vals = [a.elapsed_time(b) for mk in all_marks for (a, b) in mk[key]]
        return (sum(vals) / len(vals)) if vals else 0.0, len(vals) // max(1, args.steps)

    k = {key: avg_ms(key) for key in ("momentum", "ns1", "ns2", "ns3", "ns3_apply", "adamw")}

    # practical reference for the elementwise kernels: a plain device copy
    # (read + write) of 1 GiB, outside the timed region
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b_ = ev(), ev()
    a.record(stream)
    for _ in range(5):
        dst.copy_(src)
    b_.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * (1 << 30) / (a.elapsed_time(b_) * 1e-3) / 1e9
    del src, dst

    # ---- the safety net around the step (outside the timed step): the
    # global gradient norm behind clipping and the step guard, over every
    # gradient of the workload, and the statistics of the Muon momentum
    grad_bufs = [inp.grads] + [a.grad for a in adam]
    grad_bytes = sum(g.numel() * g.element_size() for g in grad_bufs)
    clip_ws = torch.empty(max(8, M.grad_norm_clip_workspace_size(len(grad_bufs))),
                          dtype=torch.uint8, device=dev)
    clip_out = torch.zeros(16, dtype=torch.uint8, device=dev)
    stats_ws = torch.empty(M.state_stats_workspace_size(), dtype=torch.uint8, device=dev)
    stats_out = torch.zeros(64, dtype=torch.uint8, device=dev)

    def time_launch(fn, reps=5):
        fn()
        a, b_ = ev(), ev()
        a.record(stream)
        for _ in range(reps):
            fn()
        b_.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b_) / reps

    clip_ms = time_launch(lambda: M.grad_norm_clip(grad_bufs, 1.0, out=clip_out,
                                                   workspace=clip_ws))
    stats_ms = time_launch(lambda: M.state_stats(inp.momentum, out=stats_out,
                                                 workspace=stats_ws))
    guard = {
        "grad_norm_clip": {"ms": clip_ms, "bytes": grad_bytes,
                           "gbps": grad_bytes / (clip_ms * 1e-3) / 1e9},
        "state_stats_momentum": {"ms": stats_ms, "bytes": inp.momentum.numel() * 4,
                                 "gbps": inp.momentum.numel() * 4 / (stats_ms * 1e-3) / 1e9},
    }

    # ---- the separate apply kernel (used with out_update and for matrices
    # whose update is not fused) over every matrix, outside the step
    apply_ms = sum(time_launch(lambda w=w: M.muon_stage_apply(plan, w, inp.params, ws, hp))
                   for w in range(n_waves))
    # AdamW over every group alone (inside the step it may share the GPU
    # with NS phase 1)
    adamw_alone_ms = (time_launch(lambda: [M.adamw_step(a.param, a.master, a.grad, a.exp_avg,
                                                        a.exp_avg_sq, ahp, t_step[0] + 1)
                                           for a in adam]) if adam else 0.0)

    # ---- AdamW with compressed optimizer states (optimizer tutorial 2.4 /
    # 3.3: 16-bit m and v), on the largest AdamW group, fresh zero states
    adamw_states = None
    if adam:
        big = max(range(len(adam)), key=lambda gi: wl.adam[gi].numel)
        ga, grp = adam[big], wl.adam[big]
        states = {}
        for mdt, vdt in (("fp32", "fp32"), ("bf16", "bf16"), ("bf16", "fp16")):
            tdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}
            m_s = torch.zeros(grp.numel, dtype=tdt[mdt], device=dev)
            v_s = torch.zeros(grp.numel, dtype=tdt[vdt], device=dev)
            p_s, mst_s = ga.param.clone(), (ga.master.clone() if ga.master is not None else None)
            ms_ = time_launch(lambda: M.adamw_step(p_s, mst_s, ga.grad, m_s, v_s, ahp, 1))
            nb = grp.numel * W.adamw_bytes_per_param(grp.param_dtype, grp.grad_dtype, grp.master,
                                                     mdt, vdt)
            states[f"m_{mdt}_v_{vdt}"] = {"ms": ms_, "bytes": nb, "gbps": nb / (ms_ * 1e-3) / 1e9,
                                          "bytes_per_param": nb // grp.numel}
            del m_s, v_s, p_s, mst_s
        adamw_states = {"group": grp.name, "params": grp.numel, **states}

    # ---- MuonClip (K2 answer section 4) on every W_q and W_k of the stack
    # (the first two square matrices of each layer of 7), outside the step
    muon_clip = None
    sq = [m for m in wl.mats() if m[1] == m[2]]
    if wl.name == "dense_d2048_l16":
        qk = [sq[4 * l + j] for l in range(len(sq) // 4) for j in (0, 1)]
        n_qk = sum(r * c for _, r, c in qk)
        # in place on the step's parameters: the timed region is over and
        # nothing reads them afterwards (a clone would be the largest device
        # copy of the run, which the traffic calibration must not meet)
        wclip = inp.params
        fplan = M.muon_clip_plan_create([(o, r, c) for o, r, c in qk], wclip.numel(),
                                        wl.param_dtype)
        fws = fplan.alloc_workspace(dev)
        d_head = 128
        heads = [(o + h * d_head * c, d_head, c, c, (i // 2) * (r // d_head) + h)
                 for i, (o, r, c) in enumerate(qk) for h in range(r // d_head)]
        n_groups = len(heads) // 2
        hplan = M.muon_clip_plan_create(heads, wclip.numel(), wl.param_dtype, n_groups)
        norms0 = torch.empty(len(qk), device=dev)
        M.muon_clip(fplan, wclip, "frobenius", 1e30, workspace=fws, norms_out=norms0)
        torch.cuda.synchronize()
        tau0 = 0.5 * float(norms0.min())

        def time_seq(fns):
            fns[0]()
            a, b_ = ev(), ev()
            a.record(stream)
            for f in fns[1:]:
                f()
            b_.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b_) / (len(fns) - 1)

        # each call clips every block (gamma ~ 0.9 against the previous call)
        clipped = time_seq([lambda t=tau0 * 0.9 ** k: M.muon_clip(fplan, wclip, "frobenius", t,
                                                                  workspace=fws)
                            for k in range(6)])
        unclipped = time_launch(lambda: M.muon_clip(fplan, wclip, "frobenius", 1e30,
                                                    workspace=fws))
        logits = torch.full((n_groups,), 400.0, device=dev)   # tau 100: gamma 1/2 everywhere
        per_head = time_launch(lambda: M.muon_clip(hplan, wclip, "max_logit", 100.0,
                                                   max_logits=logits))
        eb = 2 if wl.param_dtype == "bf16" else 4

        def entry(ms_, per_param):
            nb = n_qk * per_param * eb
            return {"ms": ms_, "bytes": nb, "gbps": nb / (ms_ * 1e-3) / 1e9}

        muon_clip = {"params": n_qk, "blocks_frobenius": len(qk), "blocks_per_head": len(heads),
                     "frobenius_all_clipped": entry(clipped, 3),
                     "frobenius_none_clipped": entry(unclipped, 1),
                     "max_logit_per_head_all_clipped": entry(per_head, 2)}
        del fplan, hplan

    # ---- the fp32 NS engine (the 1e-4 tolerance path), timed apart on one
    # dense layer's seven matrices in fp32 (4 x 2048^2, 2 x 2048x5632,
    # 5632x2048; seeded N(0, 0.02^2) weights and gradients): muon_step with
    # fp32 NS, against the fp32 matrix-core peak
    ns_fp32 = None
    if not args.no_fp32_ns:
        f_shapes = [(2048, 2048)] * 4 + [(2048, 5632)] * 2 + [(5632, 2048)]
        f_mats, f_n = [], 0
        for r_, c_ in f_shapes:
            f_mats.append((f_n, r_, c_))
            f_n += r_ * c_
        fg = torch.Generator(device=dev)
        fg.manual_seed(W.seed_key(wl.config_id, 9, 0, 0))
        f_p = torch.randn(f_n, generator=fg, device=dev) * 0.02
        f_g = torch.randn(f_n, generator=fg, device=dev) * 0.02
        f_m = torch.zeros(f_n, device=dev)
        f_plan = M.muon_plan_create(f_mats, f_n, "fp32", "fp32", "fp32")
        f_ws = f_plan.alloc_workspace(dev)
        f_ms = time_launch(lambda: M.muon_step(f_plan, f_p, f_g, f_m, f_ws, hp), reps=3)
        f_fl = sum(W.ns_flops_matrix(r_, c_, hp.ns_steps, hp.ns_c) for r_, c_ in f_shapes)
        ns_fp32 = {"matrices": "4 x 2048x2048, 2 x 2048x5632, 5632x2048 (fp32)",
                   "ns_flops": f_fl, "ms_per_step": f_ms,
                   "tflops": f_fl / (f_ms * 1e-3) / 1e12,
                   "frac_of_fp32_mfma_peak": f_fl / (f_ms * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS}
        del f_plan, f_ws, f_p, f_g, f_m

    ceiling = None if args.no_ceilings else run_ceiling("mfma_ceiling")
    hbm_ceiling = None if args.no_ceilings else run_ceiling("hbm_ceiling")

    # ---- algorithmic work
    shapes = wl.shapes
    mm = [(min(r, c), max(r, c)) for r, c in shapes]
    f1 = sum(m * (m + 1) * n for m, n in mm)           # X X^T, one triangle
    f2 = sum(m * m * (m + 1) for m, n in mm) if hp.ns_c != 0.0 else 0
    f3 = sum(2 * m * m * n for m, n in mm)             # B X
    ns_flops_step = (f1 + f2 + f3) * hp.ns_steps
    # NS kernel time per step; the last phase 3 includes the fused update
    ns_ms_step = (sum(k[f"ns{p}"][0] * k[f"ns{p}"][1] for p in phases)
                  + k["ns3_apply"][0] * k["ns3_apply"][1])
    n_muon = wl.muon_numel()
    mom_bytes = n_muon * W.momentum_bytes_per_param(wl.grad_dtype)
    app_bytes = n_muon * W.apply_bytes_per_param(wl.param_dtype)
    adam_bytes = [g.numel * W.adamw_bytes_per_param(g.param_dtype, g.grad_dtype, g.master)
                  for g in wl.adam]
    adam_ms_total = k["adamw"][0] * k["adamw"][1]

    # the dominant kernel: the plain phase-3 launches (all but the last)
    f3_tflops = f3 / (k["ns3"][0] * 1e-3) / 1e12 if k["ns3"][0] else 0.0
    result = {
        "metric": "Muon NS TFLOP/s (% MFMA peak) + AdamW/momentum HBM GB/s, 1 GPU",
        "value": ns_flops_step / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_median": ms_median,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0, std^2) weights and gradients, generated on the device)",
        "config": {
            "workload": args.workload,
            "muon_matrices": len(shapes),
            "muon_params": n_muon,
            "adamw_params": wl.adam_numel(),
            "ns_steps": hp.ns_steps,
            "ns_coefficients": list(coef),
            "ns_dtype": "bf16",
            "param_dtype": wl.param_dtype,
            "waves": n_waves,
            "adamw_stream": args.adamw_stream,
            "adamw_beside_phase": args.adamw_beside if args.adamw_stream == "side" else None,
            "workspace_GiB": round(plan.workspace_bytes / 2 ** 30, 3),
            # NS phases whose XCD tile rounds the plan holds together (bit p-1)
            "round_sync_phases": info.round_sync_phases,
        },
        "value_definition": "algorithmic NS flops of one step / whole optimizer step time",
        "roofline": {
            "kernel": "k_ns_bf16<3> (X <- a X + B X)",
            "bound": "mfma",
            "achieved": f3_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": f3_tflops / PEAK_BF16_TFLOPS,
            "traffic": measured_traffic(args.workload),
            "traffic_unit": "bytes per launch (HBM fetch + write, rocprofv3 counters scaled "
                            "by a plain-copy calibration)",
            "flops_per_launch": f3,
            "avg_launch_ms": k["ns3"][0],
            # the same GPU's sustained MFMA-only rate (clock under its own
            # power management), measured after the timed region
            "sustained_mfma_ceiling": ceiling,
            "frac_of_sustained_ceiling": (f3_tflops / ceiling["tflops"]) if ceiling else None,
            # rocprofv3 MfmaUtil of each NS kernel (counter summary under
            # profiles/, null once the kernel source has changed)
            "mfma_busy_pct": measured_mfma_util(args.workload),
        },
        "breakdown_ms_per_step": {
            "momentum+norm": k["momentum"][0] * k["momentum"][1],
            "ns_phase1_xxt": k["ns1"][0] * k["ns1"][1],
            "ns_phase2_aa": k["ns2"][0] * k["ns2"][1],
            "ns_phase3_bx": k["ns3"][0] * k["ns3"][1],
            "ns_phase3_bx_last_with_apply": k["ns3_apply"][0] * k["ns3_apply"][1],
            "adamw": adam_ms_total,
        },
        "ns_tflops_kernels_only": ns_flops_step / (ns_ms_step * 1e-3) / 1e12,
        "ns_frac_of_peak": ns_flops_step / (ns_ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "phase_tflops": {
            "xxt": f1 / (k["ns1"][0] * 1e-3) / 1e12,
            "aa": (f2 / (k["ns2"][0] * 1e-3) / 1e12) if f2 else None,
            "bx": f3_tflops,
        },
        "hbm_gbps": {
            "momentum+norm": mom_bytes / (k["momentum"][0] * 1e-3) / 1e9,
            "apply_kernel_alone": app_bytes / (apply_ms * 1e-3) / 1e9,
            "adamw_alone": (sum(adam_bytes) / (adamw_alone_ms * 1e-3) / 1e9
                            if adamw_alone_ms else None),
            "peak": PEAK_HBM_GBPS,
            "plain_copy_1GiB": copy_gbps,
            # best plain copy / read / write streams of this GPU over 2 GiB
            # buffers (hbm_ceiling), measured after the timed region
            "stream_ceiling": hbm_ceiling,
        },
        "wall_s_timed_region": wall1 - wall0,
        # fp64 oracle on sampled matrices and an AdamW slice of the first step
        # and of the last timed step
        "parity": parity,
        # optimizer-tutorial 5.4 safety net, timed separately from the step
        # (algorithmic bytes: every gradient, or the momentum, read once)
        "guard": guard,
        # AdamW over the largest group with fp32 / 16-bit states, timed apart
        "adamw_state_dtypes": adamw_states,
        # MuonClip over the stack's W_q / W_k, timed apart (bytes: read once
        # for the norm, read + write when a block is rescaled)
        "muon_clip": muon_clip,
        # the fp32 NS engine (tolerance path), timed apart on a dense layer
        "ns_fp32_engine": ns_fp32,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, hp, args.cpu_flops, 1 << 23)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
