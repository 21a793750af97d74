"""Benchmark of one DSpark draft -> schedule -> verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]

Workload (default): R = 64 requests, block gamma = 7, vocabulary V = 151936,
Markov rank r = 512, bf16 Markov factors, fp32 logits, per-request
temperature drawn from {0.6, 0.7, 1.0}, confidence sigmoid(N(1, 1)),
fixed-length verify (K = R * gamma), seeded synthetic inputs (synth).

A step is the whole hot path on inputs resident in HBM: dspark_draft_block
(gamma positions) + dspark_schedule + dspark_verify over the scheduled target
rows.  The target model's forward is outside the path: its output rows are
gathered once before timing (the schedule is deterministic given c and K).

Timing: W untimed warmup steps, then K timed steps bracketed by
torch.cuda.synchronize().  Each timed step is preceded by a 1 GiB read of an
unrelated buffer, which evicts the 256 MB Infinity Cache (MALL) and the L2s
with clean lines, so every step starts cold as it would after a target
forward; the step's own time is taken with HIP events on the library's
stream and the eviction is excluded.  A second pass of K steps times the
dominant kernel with events around each launch, and a back-to-back loop
gives the warm-cache rate for context.

Prints ONE JSON line.  `roofline` is for the dominant kernel (the fused Markov
bias + softmax statistics kernel: bias_seg16 for bf16 weights and R <= 64,
bias_seg64 above, bias_seg32_f32 for fp32 weights), timed with HIP events
recorded by the library around each launch; `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft+verify positions/sec (R×gamma) and achieved HBM GB/s at V=151936"
HBM_PEAK_GBPS = 8000.0
# committed FETCH_SIZE / WRITE_SIZE summaries of the fused kernel, per workload
TRAFFIC_FILES = {3: os.path.join(ROOT, "profiles", "bias_seg16_config3_traffic.txt"),
                 5: os.path.join(ROOT, "profiles", "bias_seg64_config5_traffic.txt")}


def tile_kernel(R, wdtype):
    """Name of the fused bias kernel that a batch runs on."""
    if wdtype != "bf16":
        return "bias_seg32_f32"
    return "bias_seg16" if R <= 64 else "bias_seg64"


def algorithmic_bytes(R, gamma, V, rank, wbytes, n_rows):
    """Bytes the method must move per step: U once, the verify target rows
    once, W2 once per draft position, and the gathered W1 rows."""
    per_pos_tile = wbytes * V * rank + 4 * R * V + wbytes * R * rank
    step = gamma * per_pos_tile + 4 * n_rows * V
    return step, per_pos_tile


def load_traffic(config, kernel):
    """HBM bytes per launch of the fused bias kernel from the committed
    counter summary of this workload, or None when there is none, it covers
    another kernel, or its kernel sources have changed since the counters
    were taken."""
    from draft_verify_sampling_bias_amd import profsum
    path = TRAFFIC_FILES.get(config)
    if path is None or not os.path.exists(path):
        return None
    t = profsum.read_traffic(path)
    if not t.get("kernel", "").startswith(kernel + "<"):
        return None
    if t.get("kernel_source_sha256_16") != profsum.tile_source_hash():
        return None
    return int(t["bytes_per_launch"])


class HipTimingEvents:
    """Raw HIP timing events created with hipEventDisableSystemFence: no
    system-scope cache write-back / invalidate when they complete, so an
    event pair attached to a kernel dispatch times the kernel alone."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import ctypes
        self._c = ctypes
        self._hip = ctypes.CDLL("libamdhip64.so")
        self.handles = []
        for _ in range(n):
            ev = ctypes.c_void_p()
            rc = self._hip.hipEventCreateWithFlags(ctypes.byref(ev), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.handles.append(ev.value)

    def elapsed_ms(self, i, j):
        ms = self._c.c_float()
        rc = self._hip.hipEventElapsedTime(self._c.byref(ms), self._c.c_void_p(self.handles[i]),
                                          self._c.c_void_p(self.handles[j]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for h in self.handles:
            self._hip.hipEventDestroy(self._c.c_void_p(h))
        self.handles = []


def cpu_baseline(inp, n_sample, seed=0, conf_min=None, capacity_sps=None, sts=None):
    """The CPU oracle on a bounded sample of requests (single BLAS thread),
    with the same scheduler as the GPU step (with capacity_sps: the capacity
    from the survival, then the top-K schedule with it; with sts = (logits,
    calibration logits, calibration counts): the temperatures fitted once
    outside the timing, then the calibrated confidence in each step)."""
    import oracle
    from threadpoolctl import threadpool_limits
    rng = np.random.default_rng(seed)
    reqs = sorted(rng.choice(inp.R, size=min(n_sample, inp.R), replace=False).tolist())
    conf = inp.c
    with threadpool_limits(limits=1):
        tau = oracle.sts_fit(sts[1], sts[2]).tau if sts is not None else None
        t0 = time.perf_counter()
        if sts is not None:
            conf = oracle.sts_apply(sts[0], tau)
        d = oracle.draft_block(inp.U, inp.W1, inp.W2, inp.wdtype, inp.anchor, inp.temp, inp.u_draft,
                               requests=reqs)
        y = np.where(d.y < 0, 0, d.y)
        if capacity_sps is not None:
            cap = oracle.capacity(oracle.survival(conf), capacity_sps)
            s = oracle.schedule(conf, cap.K, inp.anchor, y)
        elif conf_min is None:
            s = oracle.schedule(conf, inp.K, inp.anchor, y)
        else:
            s = oracle.schedule_cutoff(conf, conf_min, inp.anchor, y)
        t1 = time.perf_counter()
        # the row gather stands in for the target forward (not timed, as on the GPU)
        rows = inp.target[s.row_req.astype(np.int64), s.row_pos.astype(np.int64)]
        t2 = time.perf_counter()
        oracle.verify(rows, s.row_offsets, inp.U, inp.W1, inp.W2, inp.wdtype, inp.anchor, y, d.q_tok,
                      inp.temp, inp.u_accept, inp.u_final, requests=reqs)
        t3 = time.perf_counter()
    el = (t1 - t0) + (t3 - t2)
    return dict(value=len(reqs) * inp.gamma / el, unit="positions/s", cores=1, kind="oracle",
                sample=f"{len(reqs)} of {inp.R} requests (all {inp.gamma} positions, full V) plus the "
                       f"full-batch schedule; fp64 NumPy, 1 BLAS thread; {el:.1f} s",
                seconds=round(el, 2))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--cpu-sample", type=int, default=64)
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--no-warm", action="store_true", help="skip the back-to-back warm loop")
    ap.add_argument("--conf-min", type=float, default=None,
                    help="schedule with the static confidence cutoff at this conf_min instead of the top-K "
                         "scheduler with the configuration's capacity K")
    ap.add_argument("--capacity", action="store_true",
                    help="hardware-aware capacity: each step runs dspark_capacity on the previous step's "
                         "survival with a synthetic bucketed step-rate table, and the schedule uses the "
                         "capacity that call produced (the lag: K is known on the host ahead of the step)")
    ap.add_argument("--sts", action="store_true",
                    help="sequential temperature scaling: each step calibrates the confidence logits with "
                         "temperatures fitted once (dspark_sts_fit on synthetic calibration blocks, before "
                         "timing) and schedules on the calibrated confidence (dspark_sts_apply)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the step once in a HIP graph (torch.cuda.CUDAGraph) and time its replays; "
                         "every shape is fixed ahead, so the captured step needs no host work")
    ap.add_argument("--no-pack", action="store_true",
                    help="read W2 itself instead of its fragment-packed copy (dspark_pack_w2)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()

    ws_env = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or ws_env != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(request sharding across GPUs is a design note, not built)"}))
        sys.exit(2)

    import torch
    import draft_verify_sampling_bias_amd as ds
    import synth

    dev = torch.device("cuda:0")
    if args.copy_calib:
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 3}))
        return

    inp = synth.make_config(args.config)
    R, gamma, V, rank = inp.R, inp.gamma, inp.V, inp.rank
    wbytes = 2 if inp.wdtype == "bf16" else 4

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    if inp.wdtype == "bf16":
        W1 = torch.from_numpy(inp.W1.view(np.int16)).to(dev).view(torch.bfloat16)
        W2 = torch.from_numpy(inp.W2.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        W1, W2 = up(inp.W1), up(inp.W2)
    U, anchor, temp = up(inp.U), up(inp.anchor), up(inp.temp)
    u_draft, u_accept, u_final, c = up(inp.u_draft), up(inp.u_accept), up(inp.u_final), up(inp.c)
    target_full = up(inp.target)

    # the fragment-packed copy of W2 that the 16-row path reads, made once as
    # at model load (before and outside any timing)
    use_pack = inp.wdtype == "bf16" and R <= 64 and not args.no_pack
    W2p = ds.dspark_pack_w2(W2) if use_pack else None

    stream = torch.cuda.current_stream(dev)
    # outputs and workspaces allocated once
    y = torch.empty((R, gamma), dtype=torch.int32, device=dev)
    q_tok = torch.empty((R, gamma), dtype=torch.float32, device=dev)
    q_stats = torch.empty((R, gamma, 2), dtype=torch.float32, device=dev)
    wd = ds.W_BF16 if inp.wdtype == "bf16" else ds.W_F32
    ws_d = torch.empty(ds.draft_workspace_bytes(R, gamma, V, rank, wd), dtype=torch.uint8, device=dev)
    n_acc = torch.empty(R, dtype=torch.int32, device=dev)
    out_tok = torch.empty(R, dtype=torch.int32, device=dev)
    p_tok = torch.empty((R, gamma), dtype=torch.float32, device=dev)

    cutoff = args.conf_min is not None
    if cutoff and args.capacity:
        raise SystemExit("--conf-min and --capacity are alternative schedulers")
    # sequential temperature scaling: confidence logits of this batch, and the
    # temperatures fitted once on calibration blocks (an offline step)
    z_step = tau = None
    if args.sts:
        z_step = up(synth.make_calibration(7000 + args.config, R, gamma)[0])
        zc, nc, _ = synth.make_calibration(7100 + args.config, 20000, gamma)
        tau = ds.dspark_sts_fit(up(zc), up(nc))
        c = ds.dspark_sts_apply(z_step, tau)
    # hardware-aware capacity: the step rate table and the capacity outputs;
    # K_sched is the capacity the schedule uses
    K_sched = inp.K
    sps = cap_out = None
    if args.capacity:
        sps = up(synth.sps_table(R * (gamma + 1) + 1))
        cap_out = dict(K=torch.empty(1, dtype=torch.int32, device=dev),
                       expected=torch.empty(1, dtype=torch.float64, device=dev),
                       theta=torch.empty(1, dtype=torch.float64, device=dev))
        # an earlier step's survival (the inputs repeat, so every step has
        # the same) gives the capacity of the steps that follow
        ds.dspark_draft_block(U, W1, W2, anchor, temp, u_draft, out=(y, q_tok, q_stats), workspace=ws_d,
                              W2_packed=W2p)
        first = ds.dspark_schedule(c, R * gamma, anchor, y)
        ds.dspark_capacity(first["a"], sps, out=cap_out)
        K_sched = int(cap_out["K"].item())

    n_rows = R * (gamma + 1) if cutoff else ds.dspark_schedule_rows(R, gamma, K_sched)
    sch = dict(a=torch.empty((R, gamma), dtype=torch.float32, device=dev),
               l=torch.empty(R, dtype=torch.int32, device=dev),
               row_offsets=torch.empty(R + 1, dtype=torch.int32, device=dev),
               row_req=torch.empty(n_rows, dtype=torch.int32, device=dev),
               row_pos=torch.empty(n_rows, dtype=torch.int32, device=dev),
               row_tok=torch.empty(n_rows, dtype=torch.int32, device=dev),
               expected_tokens=torch.empty(1, dtype=torch.float32, device=dev))
    if args.capacity:
        sch["a"].copy_(first["a"])

    # target rows of the (deterministic) schedule: the stand-in for the target forward
    def schedule():
        if args.sts:
            ds.dspark_sts_apply(z_step, tau, out=c)
        if cutoff:
            ds.dspark_schedule_cutoff(c, args.conf_min, anchor, y, out=sch)
        else:
            if args.capacity:
                # the capacity for a later step, from the survival the
                # previous step left in sch["a"]; not read back in the step
                ds.dspark_capacity(sch["a"], sps, out=cap_out)
            ds.dspark_schedule(c, K_sched, anchor, y, out=sch)

    ds.dspark_draft_block(U, W1, W2, anchor, temp, u_draft, out=(y, q_tok, q_stats), workspace=ws_d, W2_packed=W2p)
    schedule()
    n_rows = int(sch["row_offsets"][R].item())
    rows = target_full[sch["row_req"][:n_rows].long(), sch["row_pos"][:n_rows].long()].contiguous()
    del target_full
    ws_v = torch.empty(ds.verify_workspace_bytes(R, gamma, V, rank, wd, n_rows), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(prof=None):
        ds.dspark_draft_block(U, W1, W2, anchor, temp, u_draft, out=(y, q_tok, q_stats), workspace=ws_d,
                              prof_events=prof, W2_packed=W2p)
        schedule()
        ds.dspark_verify(rows, sch["row_offsets"], U, W1, W2, anchor, temp, y, q_tok, q_stats, u_accept, u_final,
                         out=(n_acc, out_tok, p_tok), workspace=ws_v, W2_packed=W2p)

    # cache eviction between steps: READ 1 GiB of unrelated data (a write
    # would leave dirty lines whose write-back lands in the next kernel)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty(1, dtype=torch.float32, device=dev)

    def evict():
        torch.sum(flush, dim=0, out=sink)

    for _ in range(args.warmup):
        evict()
        step()
    torch.cuda.synchronize()

    # the measured step: the eager calls, or the replay of their capture
    run = step
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            step()
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=cap):
                step()
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        run = graph.replay
        for _ in range(args.warmup):
            evict()
            run()
        torch.cuda.synchronize()

    K = args.steps
    positions = R * gamma * K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    kev = HipTimingEvents(2 * gamma * K)

    # (1) the measured steps: cold caches, no events inside the step
    t0 = time.perf_counter()
    for i in range(K):
        evict()
        ev[i][0].record(stream)
        run()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall_cold = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in ev]
    tot_ms = float(np.sum(step_ms))
    value = positions / (tot_ms / 1e3)

    # (2) the dominant kernel alone: the library attaches a start / stop event
    # pair to each fused bias dispatch (hipExtLaunchKernel), so each interval
    # is that kernel's execution time; same cache state as pass (1)
    for i in range(K):
        evict()
        step(kev.handles[2 * gamma * i: 2 * gamma * (i + 1)])
    torch.cuda.synchronize()
    tile_ms = [kev.elapsed_ms(2 * gamma * i + 2 * k, 2 * gamma * i + 2 * k + 1) for i in range(K) for k in range(gamma)]
    kev.close()

    # (3) context: back-to-back steps with warm caches
    warm = None
    if not args.no_warm:
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(K):
            run()
        torch.cuda.synchronize()
        wall_warm = time.perf_counter() - t1
        warm = dict(value=positions / wall_warm, ms_per_step=wall_warm / K * 1e3)

    bytes_step, bytes_tile = algorithmic_bytes(R, gamma, V, rank, wbytes, n_rows)
    kernel = tile_kernel(R, inp.wdtype)
    ms_per_step = tot_ms / K
    tile_avg_ms = float(np.mean(tile_ms))
    tile_gbps = bytes_tile / (tile_avg_ms / 1e3) / 1e9
    step_gbps = bytes_step / (ms_per_step / 1e3) / 1e9

    cpu = None
    if not args.skip_cpu:
        cpu = cpu_baseline(inp, args.cpu_sample, conf_min=args.conf_min,
                           capacity_sps=synth.sps_table(R * (gamma + 1) + 1) if args.capacity else None,
                           sts=(synth.make_calibration(7000 + args.config, R, gamma)[0],
                                *synth.make_calibration(7100 + args.config, 20000, gamma)[:2]) if args.sts else None)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; logits, Markov factors, uniforms and confidences drawn by synth)",
        "config": {
            "workload": f"config{args.config}: R={R} gamma={gamma} V={V} r={rank} {inp.wdtype} W1/W2, fp32 logits, "
                        + ("confidence calibrated by sequential temperature scaling, " if args.sts else "")
                        + (f"static confidence cutoff conf_min={args.conf_min} ({n_rows} rows)" if cutoff else
                           f"hardware-aware capacity K={K_sched} from the previous step's survival and a "
                           f"bucketed step-rate table ({n_rows} rows)" if args.capacity else
                           f"{'fixed-length' if inp.K >= R * gamma else 'scheduled'} verify "
                           f"(K={inp.K}, {n_rows} rows)"),
            "R": R, "gamma": gamma, "V": V, "rank": rank, "weights": inp.wdtype, "K": K_sched,
            "W2_layout": "fragment-packed copy (dspark_pack_w2, made once before timing)" if use_pack
            else "row-major",
            "verify_rows": n_rows, "parallelism": "single GPU",
        },
        "hbm_gbps": round(step_gbps, 1),
        "hbm_frac": round(step_gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": int(bytes_step),
        "timing": "sum of per-step HIP-event intervals; caches evicted by a 1 GiB read before each step (excluded)"
                  + ("; the step is the replay of its HIP-graph capture" if args.graph else ""),
        "wall_s_timed_loop": round(wall_cold, 4),
        "step_ms_p10_p50_p90": [round(float(x), 4) for x in np.percentile(step_ms, [10, 50, 90])],
        "warm_back_to_back": None if warm is None else {k: round(v, 4) for k, v in warm.items()},
        "roofline": {
            "kernel": f"{kernel} (fused Markov bias GEMM + softmax statistics, one launch per draft position)",
            "bound": "hbm",
            "achieved": round(tile_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(tile_gbps / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic(args.config, kernel),
            "avg_launch_us": round(tile_avg_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": int(bytes_tile),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
