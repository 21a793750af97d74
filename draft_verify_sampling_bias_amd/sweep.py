"""Size sweeps of the off-step kernels, for a kernel trace.

    python -m draft_verify_sampling_bias_amd.sweep capacity   # dspark_capacity
    python -m draft_verify_sampling_bias_amd.sweep sts        # dspark_sts_fit

Each size is called a few times on seeded synthetic inputs; the durations
come from the profiler (rocprofv3 --kernel-trace), one line per size is
printed so that a trace can be matched to its size by call order.
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

CAPACITY_SIZES = [(1, 1), (64, 7), (256, 5), (1024, 5), (1024, 16)]
STS_SIZES = [(2000, 7), (8192, 7), (8193, 7), (20000, 1), (20000, 7), (24576, 7), (40000, 7)]
REPEATS = 3


def sweep_capacity():
    import torch
    import synth
    import draft_verify_sampling_bias_amd as ds
    for R, gamma in CAPACITY_SIZES:
        rng = np.random.default_rng(R * 31 + gamma)
        c = (1 / (1 + np.exp(-rng.normal(1, 1, (R, gamma))))).astype(np.float32)
        a = torch.from_numpy(np.cumprod(c, axis=1).astype(np.float32)).cuda()
        sps = torch.from_numpy(synth.sps_table(R * (gamma + 1) + 1)).cuda()
        for _ in range(REPEATS):
            out = ds.dspark_capacity(a, sps)
        torch.cuda.synchronize()
        print(f"capacity R={R} gamma={gamma} candidates={R * gamma} K={int(out['K'].item())}", flush=True)


def sweep_sts():
    import torch
    import synth
    import draft_verify_sampling_bias_amd as ds
    for N, gamma in STS_SIZES:
        z, n_acc, _ = synth.make_calibration(5, N, gamma)
        zd, nd = torch.from_numpy(z).cuda(), torch.from_numpy(n_acc).cuda()
        for _ in range(REPEATS):
            tau = ds.dspark_sts_fit(zd, nd)
        torch.cuda.synchronize()
        print(f"sts_fit N={N} gamma={gamma} tau={np.round(tau.cpu().numpy(), 4).tolist()}", flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("which", choices=["capacity", "sts"])
    a = ap.parse_args(argv)
    sweep_capacity() if a.which == "capacity" else sweep_sts()


if __name__ == "__main__":
    main()
