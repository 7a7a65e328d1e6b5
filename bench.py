#!/usr/bin/env python3
"""Benchmark of the DSpark per-round draft-and-verify hot path on one MI355X.

One step = one decoding round of the high-concurrency workload (R = 256
requests, gamma = 16 block positions, V = 151,936, rank-256 Markov head,
bf16): dspark_draft_step + dspark_verify (all gamma positions verified) +
dspark_schedule on the round's c* (prefix products and the causal scheduler).
For a workload with a confidence head (the full scheduled round: R = 512,
V = 129,280) a step is instead dspark_draft_step + dspark_confidence +
dspark_schedule on the head's confidences + dspark_verify of the scheduled
lengths.  Inputs are seeded synthetic tensors already resident in HBM when
timing starts.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic.json")
METRIC = "draft+verify positions/sec at V=151,936, R=256, γ=16; % HBM roofline"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def build_target(cfg, synth, U, Ub, W1, W2, anchors, tokens):
    """Target logits T = storage(draft logits + noise) from this round's drafted
    tokens (input construction, outside the timed region)."""
    W2f = synth.bf16_bits_to_f32(W2) if cfg.dtype == "bf16" else W2
    W1f = synth.bf16_bits_to_f32(W1) if cfg.dtype == "bf16" else W1
    T = np.empty((cfg.R, cfg.gamma + 1, cfg.V), U.dtype)
    for r in range(cfg.R):
        prev = np.concatenate([[anchors[r]], tokens[r, :-1]])
        Ur = synth.bf16_bits_to_f32(U[r]) if cfg.dtype == "bf16" else U[r]
        base = Ur + W1f[prev] @ W2f
        T[r] = synth.target_rows(cfg, r, base, Ub[r])
    return T


def algorithmic_bytes(name, cfg, n_bonus=0, n_rows=None):
    """HBM bytes a launch of kernel `name` must move at minimum (see design
    notes); n_rows = verified rows (default every position)."""
    R, g, V, e = cfg.R, cfg.gamma, cfg.V, (2 if cfg.dtype == "bf16" else 4)
    rows = R * g if n_rows is None else n_rows
    w2 = 256 * V * e
    w1row = 256 * e
    if name == "draft_bias":      # one position: U_k, gathered W1 rows, W2 once per draft call
        return R * V * e + R * w1row + w2 / g
    if name == "cstar_bias":      # every verified row: U, T, W2, gathered W1 rows
        return 2 * rows * V * e + w2 + rows * w1row
    if name == "target_lse":      # every verified target row
        return rows * V * e
    if name == "confidence":      # backbone states of every position
        return R * g * cfg.confidence_H * 2
    if name == "residual_bias":
        return 2 * R * V * e + w2 + R * w1row
    if name == "bonus":
        return n_bonus * V * e
    return 0.0


def path_bytes(cfg, n_bonus, n_rows=None):
    """Algorithmic HBM bytes of one step: draft (U, W2, W1 rows) + verify (U,
    verified T rows, bonus rows, W2, W1 rows) + per-row outputs, and the
    confidence head's backbone states when the step runs it."""
    R, g, V, e = cfg.R, cfg.gamma, cfg.V, (2 if cfg.dtype == "bf16" else 4)
    rows = R * g if n_rows is None else n_rows
    draft = R * g * V * e + 256 * V * e + R * g * 256 * e
    verify = 2 * rows * V * e + n_bonus * V * e + 256 * V * e + rows * 256 * e
    head = R * g * cfg.confidence_H * 2
    outputs = R * g * (4 + 8 + 8 + 4) + R * 8
    return draft + verify + head + outputs


def source_digest(path):
    """SHA-256 over a kernel source and, in the order first met, every local
    header it includes (#include "..." found beside it), so that a change to
    any code compiled into the kernel changes the digest."""
    h = hashlib.sha256()
    seen, todo = set(), [os.path.normpath(path)]
    while todo:
        p = todo.pop(0)
        if p in seen:
            continue
        seen.add(p)
        with open(os.path.join(HERE, p), "rb") as f:
            data = f.read()
        h.update(p.encode() + b"\0" + data)
        for inc in re.findall(rb'^\s*#include\s+"([^"]+)"', data, flags=re.M):
            q = os.path.normpath(os.path.join(os.path.dirname(p), inc.decode()))
            if os.path.exists(os.path.join(HERE, q)):
                todo.append(q)
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), or None when
    there is none or the kernel's code (its source or a local header it
    includes) changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        ent = t["kernels"][kernel]
        if source_digest(ent["source"]) != ent["sources_sha256"]:
            return None
        return ent["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


# bench kernel name -> (pattern of its demangled name, source file)
KERNELS = {
    "draft_bias": ("k_bias_bf16<0, 2, true, false>", "csrc/bias_pass.hip"),
    "cstar_bias": ("k_bias_bf16<1, 2, true, false>", "csrc/bias_pass.hip"),
    "residual_bias": ("k_bias_bf16<2, 2, true, false>", "csrc/bias_pass.hip"),
    "target_lse": ("k_target_lse<unsigned short>", "csrc/verify_aux.hip"),
    "decide": ("k_decide<unsigned short>", "csrc/verify_aux.hip"),
    "bonus": ("k_bonus<unsigned short>", "csrc/verify_aux.hip"),
    "draft_select": ("k_select<0>", "csrc/select.hip"),
    "final_select": ("k_select_final", "csrc/select.hip"),
    "schedule": ("k_schedule<4, 0>", "csrc/schedule.hip"),
}


def write_traffic(fetch_csv, write_csv, copy_mib, commands):
    """profiles/traffic.json from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch) of `bench.py --calibrate-copy copy_mib`: each
    counter is scaled by what it reads for the three plain copies of copy_mib
    MiB, and each kernel keyed by the digest of its source and local headers
    (stale once any of them changes).  Prints the per-kernel table."""
    import csv
    pkg = "draft_sampling_verification_w1_amd"

    def load(path):
        per = {}
        with open(path) as f:
            rows = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
        for row in rows:
            per.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return per

    fetch, write = load(fetch_csv), load(write_csv)
    # the calibration copies are the process's first three device copies (later
    # copies, e.g. the cold-cache flushes, are not calibrated sizes)
    copy_bytes = 3 * copy_mib * 2 ** 20
    fetch_scale = copy_bytes / (sum(fetch["__amd_rocclr_copyBuffer"][:3]) * 1024)
    write_scale = copy_bytes / (sum(write["__amd_rocclr_copyBuffer"][:3]) * 1024)
    out = {"command_fetch": commands[0], "command_write": commands[1],
           "fetch_scale": fetch_scale, "write_scale": write_scale, "kernels": {}}
    print("| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | "
          "scaled MB read | scaled MB written |")
    print("|---|---|---|---|---|---|")
    for name, (pat, src) in KERNELS.items():
        fk = [k for k in fetch if pat in k]
        wk = [k for k in write if pat in k]
        if not fk or not wk:
            continue
        fv, wv = fetch[fk[0]], write[wk[0]]
        rd = sum(fv) / len(fv) * 1024 * fetch_scale
        wr = sum(wv) / len(wv) * 1024 * write_scale
        path = f"{pkg}/{src}"
        out["kernels"][name] = {"source": path, "sources_sha256": source_digest(path),
                                "bytes_per_launch": int(rd + wr), "read_bytes": int(rd),
                                "write_bytes": int(wr)}
        print(f"| {name} (`{pat}`) | {len(fv)} | {sum(fv) / len(fv):.1f} | {sum(wv) / len(wv):.1f} | "
              f"{rd / 1e6:.2f} | {wr / 1e6:.2f} |")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(f"fetch scale {fetch_scale:.4f}, write scale {write_scale:.4f}; wrote {TRAFFIC_FILE}")


def calibrate_copy(mb):
    """A plain device copy of `mb` MiB (the reference kernel for the traffic counters)."""
    import torch
    n = mb << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 3 copies of {mb} MiB")


def memory_probe(reps=30):
    """Read bandwidth against working-set size: a float32 buffer of S MiB summed
    by torch (one read of every byte) many times in a row; sizes within the
    256 MB Infinity Cache against sizes well beyond it.  One JSON line."""
    import torch
    out = []
    for mib in (32, 64, 128, 192, 256, 384, 1024, 4096):
        buf = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
        for _ in range(3):
            buf.sum()
        times = []
        for _ in range(reps if mib <= 1024 else max(5, reps // 4)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            buf.sum()
            e1.record()
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        med = times[len(times) // 2]
        out.append({"MiB": mib, "median_us": round(med * 1e3, 1),
                    "GB_per_s_median": round((mib << 20) / (med * 1e-3) / 1e9, 1),
                    "GB_per_s_best": round((mib << 20) / (times[0] * 1e-3) / 1e9, 1)})
        log(f"[bench] memory probe {mib} MiB: median {med * 1e3:.1f} us, "
            f"{out[-1]['GB_per_s_median']:.0f} GB/s")
        del buf
    return {"probe": "read bandwidth vs working set (torch.sum of a float32 buffer, repeated)",
            "sizes": out}


def cpu_model():
    """The host CPU's model name (first 'model name' of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, synth, inp, T, n_req, n_req_1t, runs=3):
    """The oracle (fp64 CPU) on the first requests of the same workload: the
    same step as the GPU's (draft, verify of every position, schedule on c*;
    with a confidence head: draft, confidence, schedule, verify of the
    scheduled lengths -- on a sample the scheduler sees the sample's requests
    only).  Median of `runs` runs on all the host's threads over n_req
    requests, and the same at one thread over n_req_1t requests."""
    from threadpoolctl import threadpool_limits
    from oracle import oracle as O
    sps = synth.sps_table(cfg)
    scheduled = cfg.confidence_H > 0
    if scheduled:
        h_all, w = synth.confidence_inputs(cfg, requests=range(max(n_req, n_req_1t)))
        temps = synth.sts_temperatures(cfg)

    def one(n):
        req = list(range(n))
        U, anchors = inp["U"][:n], inp["anchors"][:n]
        t0 = time.perf_counter()
        od = O.draft(U, inp["W1"], inp["W2"], anchors, cfg.seed)
        if scheduled:
            c = O.confidence(h_all[:n], w, temps, inp["W1"], anchors, od["tokens"])
            lengths = O.schedule(O.prefix_products(c), sps)["lengths"]
            O.verify(U, inp["W1"], inp["W2"], anchors, od["tokens"], T[:n], lengths, cfg.seed,
                     requests=req)
        else:
            ov = O.verify(U, inp["W1"], inp["W2"], anchors, od["tokens"], T[:n], None, cfg.seed,
                          requests=req)
            O.schedule(O.prefix_products(np.nan_to_num(ov["cstar"], nan=0.0).astype(np.float32)), sps)
        return time.perf_counter() - t0

    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count())
    out = {}
    for label, n, nt in (("all", n_req, threads), ("one", n_req_1t, 1)):
        O.set_threads(nt)
        with threadpool_limits(limits=nt):
            times = sorted(one(n) for _ in range(runs))
        out[label] = (n, nt, times[len(times) // 2], times)
        log(f"[bench] oracle on {n} requests at {nt} thread(s): " +
            ", ".join(f"{t:.2f}s" for t in times))
    O.set_threads(threads)
    n, nt, med, times = out["all"]
    n1, _, med1, times1 = out["one"]
    steps = ("draft + confidence + schedule + verify(scheduled lengths)" if scheduled
             else "draft + verify + schedule")
    what = "the whole batch" if n == cfg.R else f"the first {n} of {cfg.R} requests"
    return {"value": round(n * cfg.gamma / med, 2), "unit": "positions/s", "cores": nt,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": (f"{what} ({n * cfg.gamma} positions): oracle {steps} in fp64 at {nt} threads, "
                       f"median of {runs} runs ({', '.join(f'{t:.2f}' for t in times)} s)"),
            "single_thread": {"value": round(n1 * cfg.gamma / med1, 2), "unit": "positions/s",
                              "cores": 1,
                              "sample": (f"the first {n1} of {cfg.R} requests ({n1 * cfg.gamma} "
                                         f"positions) at 1 thread, median of {runs} runs "
                                         f"({', '.join(f'{t:.2f}' for t in times1)} s)")}}


def scheduler_variants(cfg, dspark, synth, steps, warmup):
    """Per-call time of the production scheduler (capacity from the round two
    earlier, top-K on the current round), the static threshold, the
    acceptance statistics at the workload's R and gamma, and the STS fit
    (65,536 rollouts, 53 temperatures, 15 bins).  Inputs: seeded
    confidences; the accept mask follows them (position k accepted with
    probability c_k, until the first rejection)."""
    import torch
    R, g = cfg.R, cfg.gamma
    dev = torch.device("cuda:0")
    cs = [synth.survival_inputs(cfg, index=i) for i in range(3)]
    rng = np.random.default_rng(cfg.seed)
    acc = rng.random((R, g)) < cs[2]
    mask = np.full((R, g), 255, np.uint8)
    for r in range(R):
        for k in range(g):
            mask[r, k] = 1 if acc[r, k] else 0
            if not acc[r, k]:
                break
    n_acc = (np.cumprod(acc, axis=1)).sum(axis=1).astype(np.int32)
    dc = [torch.from_numpy(c).to(dev) for c in cs]
    dmask = torch.from_numpy(mask).to(dev)
    dn = torch.from_numpy(n_acc).to(dev)
    thr = torch.linspace(0.0, 1.0, 64, dtype=torch.float64, device=dev)
    sps = torch.from_numpy(synth.sps_table(cfg)).to(dev)

    def one():
        cap = dspark.schedule_capacity(dc[0], sps, with_path=False)   # round t-2
        top = dspark.schedule_topk(dc[2], cap["K"], sps)               # round t
        th = dspark.schedule_threshold(dc[2], 0.5)
        dspark.acceptance_stats(dmask, top["a"], dn, thr)
        return cap, top, th

    # STS calibration on 65,536 held-out rollouts: seeded scores, labels from a
    # model whose acceptance is sigmoid(s / 1.3) at every position
    n_cal = 65536
    s_cal = rng.normal(1.5, 1.5, (n_cal, g))
    y_cal = np.cumprod(rng.random((n_cal, g)) < 1.0 / (1.0 + np.exp(-s_cal / 1.3)), axis=1)
    ds_cal = torch.from_numpy(s_cal).to(dev)
    dy_cal = torch.from_numpy(y_cal.astype(np.uint8)).to(dev)
    grid = torch.from_numpy(np.round(np.linspace(0.4, 3.0, 53), 10)).to(dev)

    for _ in range(warmup):
        one()
        dspark.sts_fit(ds_cal, dy_cal, grid)
    torch.cuda.synchronize()
    dspark.timing_enable(True)
    for _ in range(steps):
        cap, top, th = one()
        sts = dspark.sts_fit(ds_cal, dy_cal, grid)
    torch.cuda.synchronize()
    dspark.timing_enable(False)
    kern = dspark.timing_report()
    return {"metric": "scheduler variants: microseconds per call", "unit": "us",
            "higher_is_better": False, "n_gpus": 1, "steps": steps, "data": "synthetic",
            "config": {"workload": cfg.name, "R": R, "gamma": g, "n_thresholds": 64,
                       "sts": {"rollouts": n_cal, "grid": 53, "bins": 15}},
            "kernels_us": {k: round(ms * 1e3 / n, 2) for k, (n, ms) in kern.items()},
            "capacity_K": int(cap["K"].cpu()[0]),
            "topk_B": float(top["stats"][0].cpu()),
            "threshold_mean_length": float(th["lengths"].float().mean().cpu()),
            "sts_temps": [round(float(t), 3) for t in sts["temps"].cpu()]}


def decode_rounds(cfg, dspark, synth, rounds, warmup):
    """Multi-round decoding at the workload's shape: each round's anchors are
    the previous round's last emitted token (handed over on the device), its
    Philox key carries the round index.  Per round: fresh synthetic backbone
    logits (the workload's recipe, generated on the GPU with torch), the
    draft, synthetic target logits built from the drafted tokens (the
    workload's recipe: draft logits + noise), then verify of every position
    and Algorithm 1 on c*.  T_draft and T_verify are GPU times from HIP
    events recorded on the stream around the library calls, so the target
    logits built between them (input construction) are not counted."""
    import torch
    from draft_sampling_verification_w1_amd.decode import DecodeLoop
    R, g, V = cfg.R, cfg.gamma, cfg.V
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    W1n, W2n = synth.weights(cfg)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    W1, W2 = to_dev(W1n), to_dev(W2n)
    W1f, W2f = W1.float(), W2.float()
    W2p = dspark.pack_w2(W2, V)
    sps = torch.from_numpy(synth.sps_table(cfg)).to(dev)
    loop = DecodeLoop(W1, W2p, to_dev(synth.anchors(cfg)), cfg.seed, g, sps=sps)
    sig = torch.tensor([cfg.noise_sigma(k) for k in range(1, g + 2)], dtype=torch.float32, device=dev)
    gen = torch.Generator(device=dev)
    zrng = np.random.default_rng(cfg.seed)
    state = {}

    def backbone(t):
        gen.manual_seed(cfg.seed * 100003 + t)
        U = torch.randn((R, g + 1, V), generator=gen, device=dev) * cfg.u_sigma
        if cfg.zipf_boost:
            p = np.arange(1, V + 1, dtype=np.float64) ** -1.1
            ids = np.searchsorted(np.cumsum(p) / p.sum(), zrng.random(R * (g + 1)), side="right")
            U.view(-1, V)[torch.arange(R * (g + 1), device=dev),
                          torch.from_numpy(ids.clip(0, V - 1)).to(dev)] += cfg.zipf_boost
        state["Ub"] = U[:, g].to(tdt)
        return U[:, :g].to(tdt).contiguous()

    def target(t, tok):
        U = state["U"].float()
        if cfg.target_from_draft:
            prev = torch.cat([state["anchors"].long()[:, None], tok[:, :-1].long()], dim=1)
            base = U + (W1f[prev.reshape(-1)] @ W2f).view(R, g, V)
        else:
            base = U
        T = torch.empty((R, g + 1, V), dtype=tdt, device=dev)
        T[:, :g] = (base + torch.randn((R, g, V), generator=gen, device=dev) * sig[:g, None]).to(tdt)
        T[:, g] = (state["Ub"].float() + torch.randn((R, V), generator=gen, device=dev) * sig[g]).to(tdt)
        return T

    out = []
    for t in range(warmup + rounds):
        state["U"] = backbone(t)
        state["anchors"] = loop.anchors.clone()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

        def target_timed(tt, tok):
            ev[1].record()        # the draft's kernels are before this point on the stream
            T = target(tt, tok)
            ev[2].record()        # the target logits are built
            return T

        torch.cuda.synchronize()
        ev[0].record()
        r = loop.round(state["U"], target_timed)
        ev[3].record()
        torch.cuda.synchronize()
        t_draft = ev[0].elapsed_time(ev[1]) / 1e3
        t_verify = ev[2].elapsed_time(ev[3]) / 1e3
        if t < warmup:
            continue
        n_acc = r["n_accept"].cpu().numpy()
        a = r["a"].cpu().numpy().astype(np.float64)
        tau = float((n_acc + 1).mean())
        pred = float((1.0 + a.sum(axis=1)).mean())   # expected tau with every position verified
        ms = (t_draft + t_verify) * 1e3
        out.append({"round": t - warmup, "tau": round(tau, 3), "tau_from_cstar": round(pred, 3),
                    "ms_draft": round(t_draft * 1e3, 3), "ms_verify": round(t_verify * 1e3, 3),
                    "L_us_per_token": round(ms * 1e3 / tau, 2),
                    "alg1_lengths_mean": round(float(r["lengths"].float().mean().cpu()), 3)})
    tau = np.mean([o["tau"] for o in out])
    ms = np.mean([o["ms_draft"] + o["ms_verify"] for o in out])
    return {"metric": "multi-round decoding: tau per round and L = (T_draft + T_verify) / tau",
            "unit": "us per token", "value": round(ms * 1e3 / tau, 2), "higher_is_better": False,
            "n_gpus": 1, "rounds": rounds, "warmup": warmup, "data": "synthetic",
            "config": {"workload": cfg.name, "R": R, "gamma": g, "V": V},
            "mean_tau": round(float(tau), 3),
            "mean_tau_from_cstar": round(float(np.mean([o["tau_from_cstar"] for o in out])), 3),
            "mean_ms_per_round": round(float(ms), 3), "per_round": out}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="high_concurrency")
    ap.add_argument("--cpu-requests", type=int, default=0,
                    help="requests in the CPU oracle's all-thread sample (default: the whole batch)")
    ap.add_argument("--cpu-requests-1t", type=int, default=8,
                    help="requests in the CPU oracle's one-thread sample")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="steps timed one by one after streaming 1 GiB through the caches (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: build profiles/traffic.json from the two counter runs "
                         "(rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE of this script with "
                         "--calibrate-copy 1024)")
    ap.add_argument("--rounds", type=int, default=0,
                    help="run this many rounds of multi-round decoding instead (one JSON line)")
    ap.add_argument("--memory-probe", action="store_true",
                    help="measure read bandwidth against working-set size instead (one JSON line)")
    ap.add_argument("--scheduler-variants", action="store_true",
                    help="time the production scheduler, static threshold and acceptance "
                         "statistics instead of the round (one JSON line of its own)")
    args = ap.parse_args()
    if args.write_traffic:
        cmd = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {c} --output-format csv -d "
               "$REPO/gpurun_out/prof/{d} -o bench -- python3 $REPO/bench.py --steps 2 --warmup 1 "
               "--no-cpu-baseline --cold-steps 5 --calibrate-copy 1024")
        write_traffic(args.write_traffic[0], args.write_traffic[1], 1024,
                      (cmd.format(c="FETCH_SIZE", d="fetch"), cmd.format(c="WRITE_SIZE", d="write")))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path shards over requests with no exchange except one all-gather "
              "for the scheduler; the library runs on one GPU).", file=sys.stderr)
        sys.exit(2)

    import torch
    from draft_sampling_verification_w1_amd import dspark, synth

    cfg = synth.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dspark.lib()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
    if args.memory_probe:
        print(json.dumps(memory_probe()), flush=True)
        return
    if args.scheduler_variants:
        print(json.dumps(scheduler_variants(cfg, dspark, synth, args.steps, args.warmup)), flush=True)
        return
    if args.rounds:
        print(json.dumps(decode_rounds(cfg, dspark, synth, args.rounds, args.warmup)), flush=True)
        return
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t0 = time.time()
    W1, W2 = synth.weights(cfg)
    U, Ub = synth.backbone(cfg)
    anchors = synth.anchors(cfg)
    sps = synth.sps_table(cfg)
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")
    dU, dW1, dW2 = to_dev(U), to_dev(W1), to_dev(W2)
    dA, dSPS = to_dev(anchors), to_dev(sps)
    W2p = dspark.pack_w2(dW2, cfg.V)
    p = dspark.problem(cfg.R, cfg.gamma, cfg.V, tdt, cfg.seed)
    ws = dspark.workspace(p, dev)
    R, g = cfg.R, cfg.gamma
    d_out = (torch.empty((R, g), dtype=torch.int32, device=dev),
             torch.empty((R, g), dtype=torch.float64, device=dev),
             torch.empty((R, g), dtype=torch.float64, device=dev))
    v_out = {"cstar": torch.empty((R, g), dtype=torch.float32, device=dev),
             "n_accept": torch.empty(R, dtype=torch.int32, device=dev),
             "out_token": torch.empty(R, dtype=torch.int32, device=dev),
             "accept_mask": None, "lse_t": None}
    s_out = {"a": torch.empty((R, g), dtype=torch.float32, device=dev),
             "lengths": torch.empty(R, dtype=torch.int32, device=dev),
             "stats": torch.empty(4, dtype=torch.float64, device=dev), "theta_path": None}

    tok = dspark.draft_step(dU, dW1, W2p, dA, cfg.seed, ws=ws, out=d_out)[0].cpu().numpy()
    t0 = time.time()
    T = build_target(cfg, synth, U, Ub, W1, W2, anchors, tok)
    dT = to_dev(T)
    log(f"[bench] target logits built in {time.time() - t0:.1f}s")

    scheduled = cfg.confidence_H > 0
    if scheduled:
        h, w = synth.confidence_inputs(cfg)
        dH, dWc = to_dev(h), to_dev(w)
        dTemps = to_dev(synth.sts_temperatures(cfg))
        c_out = torch.empty((R, g), dtype=torch.float32, device=dev)
        del h

    def step():
        tk, ls, lq = dspark.draft_step(dU, dW1, W2p, dA, cfg.seed, ws=ws, out=d_out)
        if scheduled:   # the head's confidences set the lengths that verify checks
            dspark.confidence(dH, dWc, dTemps, dW1, dA, tk, out=c_out)
            sch = dspark.schedule(c_out, dSPS, out=s_out, with_path=False)
            dspark.verify(dU, dW1, W2p, dA, tk, ls, lq, dT, sch["lengths"], cfg.seed, ws=ws,
                          out=v_out, with_mask=False, with_lse_t=False)
        else:
            v = dspark.verify(dU, dW1, W2p, dA, tk, ls, lq, dT, None, cfg.seed, ws=ws, out=v_out,
                              with_mask=False, with_lse_t=False)
            dspark.schedule(v["cstar"], dSPS, out=s_out, with_path=False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / args.steps
    positions = R * g * args.steps
    value = positions / elapsed
    log(f"[bench] {args.steps} steps: {ms:.3f} ms/step, {value / 1e6:.3f} M positions/s")

    # cold: before each step a 512 MiB copy (1 GiB of traffic) evicts the 256 MB
    # Infinity Cache and the L2s; each step is timed alone with events on the
    # stream the library launches on (torch's current stream)
    cold_ms = None
    if args.cold_steps > 0:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.cold_steps)]
        for e0, e1 in ev:
            dst.copy_(src)
            e0.record()
            step()
            e1.record()
        torch.cuda.synchronize()
        cold = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        cold_ms = cold[len(cold) // 2]
        del src, dst
        log(f"[bench] cold (caches flushed before each step): median {cold_ms:.3f} ms/step")

    # the same steps again with per-kernel HIP-event timing on the launch stream
    dspark.timing_enable(True)
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof_ms = (time.perf_counter() - t1) * 1e3 / args.steps
    dspark.timing_enable(False)
    kern = dspark.timing_report()
    n_acc = v_out["n_accept"].cpu().numpy()
    lengths = s_out["lengths"].cpu().numpy() if scheduled else np.full(R, g)
    n_bonus = int((n_acc == lengths).sum())
    per_step = {k: (c / args.steps, ms_tot / args.steps) for k, (c, ms_tot) in kern.items()}
    dom = max(per_step, key=lambda k: per_step[k][1])
    launches, dom_ms = per_step[dom]
    avg_s = dom_ms / launches * 1e-3
    n_rows = int(lengths.sum())
    nb = algorithmic_bytes(dom, cfg, n_bonus, n_rows)
    traffic = measured_traffic(dom)
    achieved = nb / avg_s / 1e9
    path_b = path_bytes(cfg, n_bonus, n_rows)
    log("[bench] per-step kernel time (ms): " +
        ", ".join(f"{k} {v[1]:.3f} ({v[0]:.0f}x)" for k, v in sorted(per_step.items(), key=lambda x: -x[1][1])))

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "R": R, "gamma": g, "V": cfg.V, "rank": cfg.rank,
                   "step": ("draft_step + confidence + schedule(c) + verify(scheduled lengths)"
                            if scheduled else
                            "draft_step + verify(all gamma positions) + schedule(c*)"),
                   "path_hbm_bytes": int(path_b),
                   "path_hbm_frac": round(path_b / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4)},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": int(nb),
                     "avg_launch_us": round(avg_s * 1e6, 2),
                     # measured bytes (FETCH + WRITE) per launch over the same launch time
                     "traffic_GBps": None if traffic is None else round(traffic / avg_s / 1e9, 1)},
        "kernels_ms_per_step": {k: round(v[1], 4) for k, v in per_step.items()},
        "profiled_ms_per_step": round(prof_ms, 4),
        "mean_accepted": round(float(n_acc.mean()), 3),
    }
    if cold_ms is not None:
        result["cold"] = {"ms_per_step": round(cold_ms, 4),
                          "positions_per_s": round(R * g / (cold_ms * 1e-3), 1),
                          "steps": args.cold_steps,
                          "how": "median of single steps, each after a 512 MiB device copy"}
    if scheduled:
        result["mean_scheduled_length"] = round(float(lengths.mean()), 3)
    if not args.no_cpu_baseline:
        n_cpu = min(args.cpu_requests or R, R)
        n_1t = min(args.cpu_requests_1t, R)
        log(f"[bench] CPU oracle on {n_cpu} requests (all threads), {n_1t} (one thread) ...")
        inp = {"U": U, "W1": W1, "W2": W2, "anchors": anchors}
        result["cpu_baseline"] = cpu_baseline(cfg, synth, inp, T, n_cpu, n_1t)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
