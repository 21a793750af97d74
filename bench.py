"""Benchmark of one DSpark draft -> schedule -> verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--policy greedy|sampled]
    python bench.py --sweep capacity|sts     (size sweeps of the off-step kernels, for a kernel trace)
    python bench.py --head rnn               (the RNN sequential head instead of the Markov head)

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
recorded by the library around each launch; `calls_us` gives each call's
time per step (a separate pass with events between the calls);
`acceptance` the accept rate by draft position and the tokens emitted per
request and verify pass; `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload, on one host core and on all of them (processes
over request chunks, the schedule in the parent), before the GPU is used.
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
TRAFFIC_FILES = {2: os.path.join(ROOT, "profiles", "bias_seg16_config2_traffic.txt"),
                 3: os.path.join(ROOT, "profiles", "bias_seg16_config3_traffic.txt"),
                 5: os.path.join(ROOT, "profiles", "bias_seg64_config5_traffic.txt")}


def tile_kernel(R, wdtype):
    """Name of the fused bias kernel that a batch runs on."""
    if wdtype != "bf16":
        return "bias_seg32_f32"
    return "bias_seg16" if R <= 64 else "bias_seg64"


def algorithmic_bytes(R, gamma, V, rank, wbytes, n_rows, rnn=False):
    """Bytes the method must move per step: U once, the verify target rows
    once, W2 once per draft position, and the gathered W1 rows (RNN head:
    the fp32 states instead; the state update's own reads of A, rank x rank,
    and of W1 rows are counted per position as well)."""
    h_bytes = 4 * R * rank if rnn else wbytes * R * rank
    per_pos_tile = wbytes * V * rank + 4 * R * V + h_bytes
    state = (wbytes * rank * rank + wbytes * R * rank + 8 * R * rank) if rnn else 0
    step = gamma * (per_pos_tile + state) + 4 * n_rows * V
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


# inputs of the all-cores oracle leg, set in the parent before its worker
# processes are forked (copy-on-write; the workers read them, never write)
_POOL = {}


def _oracle_draft(inp, reqs, rnn):
    import oracle
    if rnn is None:
        return oracle.draft_block(inp.U, inp.W1, inp.W2, inp.wdtype, inp.anchor, inp.temp, inp.u_draft,
                                  requests=reqs)
    return oracle.rnn_draft_block(inp.U, inp.W1, inp.W2, rnn[0], inp.wdtype, rnn[1], inp.anchor, inp.temp,
                                  inp.u_draft, requests=reqs)


def _oracle_draft_chunk(reqs):
    from threadpoolctl import threadpool_limits
    P = _POOL
    with threadpool_limits(limits=1):
        d = _oracle_draft(P["inp"], reqs, P["rnn"])
    return reqs, d.y[reqs], d.q_tok[reqs], (d.h[reqs] if d.h is not None else None), len(d.flags)


def _oracle_verify_chunk(job):
    import oracle
    from threadpoolctl import threadpool_limits
    reqs, y, q_tok, h = job
    P = _POOL
    inp = P["inp"]
    with threadpool_limits(limits=1):
        v = oracle.verify(P["rows"], P["row_offsets"], inp.U, inp.W1, inp.W2, inp.wdtype, inp.anchor, y, q_tok,
                          inp.temp, inp.u_accept, inp.u_final, requests=reqs, h_states=h)
    return len(v.flags)


def _host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = os.cpu_count() or 1
    return dict(cpu_count=os.cpu_count(), allowed=allowed, model=model)


def cpu_baseline(inp, n_sample, seed=0, conf_min=None, capacity_sps=None, sts=None, max_procs=16, rnn=None):
    """The CPU oracle, unmodified, on a bounded sample of requests of the same
    workload, timed twice: on one host core (BLAS on one thread, the process
    pinned to one core) and on all allowed cores (up to max_procs worker
    processes over request chunks, BLAS on one thread each; the schedule in
    the parent, as the global top-K needs every request's survival).  The
    scheduler is the GPU step's (with capacity_sps: the capacity from the
    survival, then the top-K schedule with it; with sts = (logits,
    calibration logits, calibration counts): temperatures fitted once outside
    the timing, then the calibrated confidence in each step).  The row gather
    stands in for the target forward and is not timed, as on the GPU.  Must
    run before this process touches the GPU (the workers are forked).  With
    rnn = (A, act) the drafter is the RNN head."""
    import multiprocessing as mp

    import oracle
    from threadpoolctl import threadpool_limits
    rng = np.random.default_rng(seed)
    reqs = sorted(rng.choice(inp.R, size=min(n_sample, inp.R), replace=False).tolist())
    host = _host_cpu()

    def sched(conf, y):
        if capacity_sps is not None:
            cap = oracle.capacity(oracle.survival(conf), capacity_sps)
            return oracle.schedule(conf, cap.K, inp.anchor, y)
        if conf_min is None:
            return oracle.schedule(conf, inp.K, inp.anchor, y)
        return oracle.schedule_cutoff(conf, conf_min, inp.anchor, y)

    tau = None
    if sts is not None:
        with threadpool_limits(limits=1):
            tau = oracle.sts_fit(sts[1], sts[2]).tau

    # (1) one core
    old_aff = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
    if old_aff:
        os.sched_setaffinity(0, {min(old_aff)})
    try:
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            conf = oracle.sts_apply(sts[0], tau) if sts is not None else inp.c
            d = _oracle_draft(inp, reqs, rnn)
            y = np.where(d.y < 0, 0, d.y)
            sch = sched(conf, y)
            t1 = time.perf_counter()
            rows = inp.target[sch.row_req.astype(np.int64), sch.row_pos.astype(np.int64)]
            t2 = time.perf_counter()
            v = oracle.verify(rows, sch.row_offsets, inp.U, inp.W1, inp.W2, inp.wdtype, inp.anchor, y, d.q_tok,
                              inp.temp, inp.u_accept, inp.u_final, requests=reqs, h_states=d.h)
            t3 = time.perf_counter()
    finally:
        if old_aff:
            os.sched_setaffinity(0, old_aff)
    el1 = (t1 - t0) + (t3 - t2)
    flags = dict(draft=len(d.flags), verify=len(v.flags))

    # (2) all allowed cores: the same sample split into one chunk per process
    n_proc = max(1, min(host["allowed"], max_procs, len(reqs)))
    chunks = [c.tolist() for c in np.array_split(np.asarray(reqs), n_proc) if len(c)]
    _POOL.clear()
    _POOL.update(inp=inp, rows=rows, row_offsets=sch.row_offsets, rnn=rnn)
    ctx = mp.get_context("fork")
    with ctx.Pool(n_proc) as pool:
        pool.map(abs, range(n_proc))  # workers up before timing
        t0 = time.perf_counter()
        conf = oracle.sts_apply(sts[0], tau) if sts is not None else inp.c
        y_all = np.zeros((inp.R, inp.gamma), np.int32)
        q_all = np.full((inp.R, inp.gamma), np.nan)
        h_all = np.zeros((inp.R, inp.gamma, inp.rank)) if rnn is not None else None
        for rq, yy, qq, hh, _ in pool.map(_oracle_draft_chunk, chunks):
            y_all[rq] = yy
            q_all[rq] = qq
            if hh is not None:
                h_all[rq] = hh
        sch2 = sched(conf, y_all)
        t1 = time.perf_counter()
        # the rows were gathered above (row_req / row_pos do not depend on y)
        assert np.array_equal(sch2.row_offsets, sch.row_offsets)
        t2 = time.perf_counter()
        pool.map(_oracle_verify_chunk, [(c, y_all, q_all, h_all) for c in chunks])
        t3 = time.perf_counter()
    _POOL.clear()
    eln = (t1 - t0) + (t3 - t2)
    pos = len(reqs) * inp.gamma
    return dict(value=pos / eln, unit="positions/s", cores=n_proc, kind="oracle",
                sample=f"{len(reqs)} of {inp.R} requests (all {inp.gamma} positions, full V) plus the "
                       f"full-batch schedule; fp64 NumPy, 1 BLAS thread per process; {n_proc} processes over "
                       f"request chunks: {eln:.2f} s; one core: {el1:.2f} s",
                seconds=round(eln, 2),
                single_core=dict(value=pos / el1, cores=1, seconds=round(el1, 2)),
                host=host, oracle_flags=flags)


CAPACITY_SIZES = [(1, 1), (64, 7), (256, 5), (1024, 5), (1024, 16)]
STS_SIZES = [(2000, 7), (8192, 7), (8193, 7), (20000, 1), (20000, 7), (24576, 7), (40000, 7)]
SWEEP_REPEATS = 3


def sweep(which):
    """Size sweep of an off-step kernel (dspark_capacity or dspark_sts_fit):
    each size is called SWEEP_REPEATS times on seeded synthetic inputs and one
    line per size is printed, so that a kernel trace (rocprofv3
    --kernel-trace) can be matched to its sizes by call order."""
    import torch
    import draft_verify_sampling_bias_amd as ds
    import synth
    if which == "capacity":
        for R, gamma in CAPACITY_SIZES:
            rng = np.random.default_rng(R * 31 + gamma)
            c = (1 / (1 + np.exp(-rng.normal(1, 1, (R, gamma))))).astype(np.float32)
            a = torch.from_numpy(np.cumprod(c, axis=1).astype(np.float32)).cuda()
            sps = torch.from_numpy(synth.sps_table(R * (gamma + 1) + 1)).cuda()
            for _ in range(SWEEP_REPEATS):
                out = ds.dspark_capacity(a, sps)
            torch.cuda.synchronize()
            print(f"capacity R={R} gamma={gamma} candidates={R * gamma} K={int(out['K'].item())}", flush=True)
    else:
        for N, gamma in STS_SIZES:
            z, n_acc, _ = synth.make_calibration(5, N, gamma)
            zd, nd = torch.from_numpy(z).cuda(), torch.from_numpy(n_acc).cuda()
            for _ in range(SWEEP_REPEATS):
                tau = ds.dspark_sts_fit(zd, nd)
            torch.cuda.synchronize()
            print(f"sts_fit N={N} gamma={gamma} tau={np.round(tau.cpu().numpy(), 4).tolist()}", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--policy", default=None, choices=["greedy", "sampled"],
                    help="the greedy or the sampled run of configs 1 and 2 (default: the configuration's first)")
    ap.add_argument("--sweep", default=None, choices=["capacity", "sts"],
                    help="only run a size sweep of dspark_capacity or dspark_sts_fit (durations from a kernel "
                         "trace: one line is printed per size, in call order)")
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
    ap.add_argument("--head", default="markov", choices=["markov", "rnn"],
                    help="the drafter's sequential head: Markov (bias W2 . W1[prev]) or RNN (bias W2 h_k, "
                         "h_k = tanh(A h_{k-1} + W1[prev]), A from synth.make_rnn_A; bf16 with R <= 64 only)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()

    ws_env = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or ws_env != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(request sharding across GPUs is a design note, not built)"}))
        sys.exit(2)

    import synth

    if args.sweep:
        sweep(args.sweep)
        return
    inp = None
    cpu = None
    rnn = None
    if not args.copy_calib:
        inp = synth.make_config(args.config, args.policy)
        if args.head == "rnn":
            if inp.wdtype != "bf16" or inp.R > 64:
                raise SystemExit("--head rnn runs on the 16-row path only (bf16 weights, R <= 64)")
            rnn = (synth.make_rnn_A(1000 + args.config, inp.rank), 1)
        # the CPU oracle runs first: its all-cores leg forks worker
        # processes, which must happen before this process uses the GPU
        if not args.skip_cpu:
            R_, g_ = inp.R, inp.gamma
            cpu = cpu_baseline(inp, args.cpu_sample, conf_min=args.conf_min,
                               capacity_sps=synth.sps_table(R_ * (g_ + 1) + 1) if args.capacity else None,
                               sts=(synth.make_calibration(7000 + args.config, R_, g_)[0],
                                    *synth.make_calibration(7100 + args.config, 20000, g_)[:2])
                               if args.sts else None, rnn=rnn)

    import torch
    import draft_verify_sampling_bias_amd as ds

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
    # RNN head: the recurrence matrix and the state buffer (written by the
    # draft, read by the verify)
    A_d = h_buf = None
    if rnn is not None:
        A_d = torch.from_numpy(rnn[0].view(np.int16)).to(dev).view(torch.bfloat16)
        h_buf = torch.empty((R, gamma, rank), dtype=torch.float32, device=dev)
    rk = dict(A=A_d, act=rnn[1], h=h_buf) if rnn is not None else {}

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
    ws_d = torch.empty(ds.draft_workspace_bytes(R, gamma, V, rank, wd, head=ds.HEAD_RNN if rnn else ds.HEAD_MARKOV,
                                                act=rnn[1] if rnn else 0), dtype=torch.uint8, device=dev)
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
                              W2_packed=W2p, **rk)
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

    ds.dspark_draft_block(U, W1, W2, anchor, temp, u_draft, out=(y, q_tok, q_stats), workspace=ws_d, W2_packed=W2p,
                          **rk)
    schedule()
    n_rows = int(sch["row_offsets"][R].item())
    rows = target_full[sch["row_req"][:n_rows].long(), sch["row_pos"][:n_rows].long()].contiguous()
    del target_full
    ws_v = torch.empty(ds.verify_workspace_bytes(R, gamma, V, rank, wd, n_rows,
                                                 head=ds.HEAD_RNN if rnn else ds.HEAD_MARKOV),
                       dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(prof=None):
        ds.dspark_draft_block(U, W1, W2, anchor, temp, u_draft, out=(y, q_tok, q_stats), workspace=ws_d,
                              prof_events=prof, W2_packed=W2p, **rk)
        schedule()
        ds.dspark_verify(rows, sch["row_offsets"], U, W1, W2, anchor, temp, y, q_tok, q_stats, u_accept, u_final,
                         out=(n_acc, out_tok, p_tok), workspace=ws_v, W2_packed=W2p, h=h_buf)

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

    # (3) each call's time: events between the calls of the step (a pass of
    # its own, as the events add a little to the step); eager calls only
    cev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for i in range(K):
        evict()
        cev[i][0].record(stream)
        ds.dspark_draft_block(U, W1, W2, anchor, temp, u_draft, out=(y, q_tok, q_stats), workspace=ws_d,
                              W2_packed=W2p, **rk)
        cev[i][1].record(stream)
        schedule()
        cev[i][2].record(stream)
        ds.dspark_verify(rows, sch["row_offsets"], U, W1, W2, anchor, temp, y, q_tok, q_stats, u_accept, u_final,
                         out=(n_acc, out_tok, p_tok), workspace=ws_v, W2_packed=W2p, h=h_buf)
        cev[i][3].record(stream)
    torch.cuda.synchronize()
    calls_us = {name: round(float(np.mean([cev[i][j].elapsed_time(cev[i][j + 1]) for i in range(K)])) * 1e3, 2)
                for j, name in enumerate(("draft", "schedule", "verify"))}

    # acceptance of the step (the inputs are the same every step): rate by
    # draft position among the requests that verified it and reached it
    # (every earlier draft accepted), and tokens emitted per request and
    # verify pass (accepted drafts + the correction or bonus)
    n_acc_h = n_acc.cpu().numpy().astype(np.int64)
    l_h = sch["l"].cpu().numpy().astype(np.int64)
    by_pos = []
    for k in range(gamma):
        reached = int(np.sum((l_h > k) & (n_acc_h >= k)))
        acc = int(np.sum((l_h > k) & (n_acc_h > k)))
        by_pos.append(dict(position=k, reached=reached, accepted=acc,
                           rate=round(acc / reached, 4) if reached else None))
    acceptance = dict(by_position=by_pos, tokens_per_request_per_pass=round(float(np.mean(n_acc_h + 1)), 4),
                      accepted_drafts=int(n_acc_h.sum()), verified_drafts=int(l_h.sum()),
                      greedy_requests=int(np.sum(inp.temp <= 0)))

    # (4) context: back-to-back steps with warm caches
    warm = None
    if not args.no_warm:
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(K):
            run()
        torch.cuda.synchronize()
        wall_warm = time.perf_counter() - t1
        warm = dict(value=positions / wall_warm, ms_per_step=wall_warm / K * 1e3)

    bytes_step, bytes_tile = algorithmic_bytes(R, gamma, V, rank, wbytes, n_rows, rnn=rnn is not None)
    kernel = tile_kernel(R, inp.wdtype)
    ms_per_step = tot_ms / K
    tile_avg_ms = float(np.mean(tile_ms))
    tile_gbps = bytes_tile / (tile_avg_ms / 1e3) / 1e9
    step_gbps = bytes_step / (ms_per_step / 1e3) / 1e9

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
                        + ("RNN head (tanh, A from synth.make_rnn_A), " if rnn else "")
                        + (f"{args.policy} requests, " if args.policy else "")
                        + ("confidence calibrated by sequential temperature scaling, " if args.sts else "")
                        + (f"static confidence cutoff conf_min={args.conf_min} ({n_rows} rows)" if cutoff else
                           f"hardware-aware capacity K={K_sched} from the previous step's survival and a "
                           f"bucketed step-rate table ({n_rows} rows)" if args.capacity else
                           f"{'fixed-length' if inp.K >= R * gamma else 'scheduled'} verify "
                           f"(K={inp.K}, {n_rows} rows)"),
            "R": R, "gamma": gamma, "V": V, "rank": rank, "weights": inp.wdtype, "K": K_sched, "head": args.head,
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
        "calls_us": calls_us,
        "acceptance": acceptance,
        "roofline": {
            "kernel": f"{kernel} (fused Markov bias GEMM + softmax statistics, one launch per draft position"
                      + ("; RNN state as two bf16 planes, two MFMAs per k-step)" if rnn else ")"),
            "bound": "hbm",
            "achieved": round(tile_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(tile_gbps / HBM_PEAK_GBPS, 4),
            "traffic": None if rnn else load_traffic(args.config, kernel),
            "avg_launch_us": round(tile_avg_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": int(bytes_tile),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
