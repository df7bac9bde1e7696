#!/usr/bin/env python3
"""Monte-Carlo study of the imbalance score: grouped (MoGE) routing vs a global top-K.

The TechWalker page (section 一) defines the imbalance score of a batch as the gap
between the busiest and the idlest device's load and reports, from Monte-Carlo
simulation, that a conventional top-K router almost always has a positive score,
while grouped routing (the N experts split into M equal groups, one per device,
K' = K/M experts taken from every group) has a score of zero by construction.

This script repeats that experiment on the GPU path: for every (N, M, K, T) and
score distribution it draws seeded batches of router scores, routes them both
ways through the C ABI (moge_route with M groups, and with one group for the
global top-K), counts the (token, expert) pairs per group with moge_permute, and
reports IS = (max_g load_g - min_g load_g) / T over the trials, and the busiest
group's load over the balanced load T*K/M: when a device's expert time grows with
its row count, that ratio is how much longer the step takes than under grouped
routing, where every group carries exactly T*K/M rows.

Usage: python imbalance_study.py [--trials 64] [--quick]
Prints one JSON line per configuration and a markdown table.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def draw_scores(T: int, N: int, seed: int, dist: str) -> np.ndarray:
    """Seeded router scores [T, N] float32: iid N(0,1), or the same plus a Zipf(1.2)
    popularity prior -1.2 ln(e + 1) over the experts."""
    from synth import inputs as S
    s = S.normal_tensor((T, N), 1.0, seed, 100 + N, "f32")
    if dist == "zipf":
        s = (s + S.zipf_bias(N, 1.2)[None, :]).astype(np.float32)
    return s


class Router:
    """moge_route + moge_permute on the GPU for one (N, M, K, T)."""

    def __init__(self, moge, N: int, M: int, K: int, T: int):
        import torch
        self.moge, self.torch = moge, torch
        # d, inter and dtype do not enter routing; they only have to be valid
        self.dims = {m: moge.make_dims(T, 256, N, m, K // m, 256, 0, moge.MOGE_F32) for m in (M, 1)}
        self.N, self.M, self.K, self.T = N, M, K, T
        dev = "cuda"
        self.idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.gate = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.counts = torch.empty((N,), dtype=torch.int32, device=dev)
        self.offsets = torch.empty((N + 1,), dtype=torch.int32, device=dev)
        self.gcounts = torch.empty((M,), dtype=torch.int32, device=dev)
        self.sorted_pair = torch.empty((T * K,), dtype=torch.int32, device=dev)
        self.pair_row = torch.empty((T * K,), dtype=torch.int32, device=dev)
        self.ws = torch.empty(max(moge.workspace_size(d) for d in self.dims.values()),
                              dtype=torch.uint8, device=dev)

    def group_loads(self, scores_dev, m: int) -> np.ndarray:
        """Per-group (token, expert) counts over the M device groups for routing
        with m groups (m = M: grouped; m = 1: global top-K)."""
        moge, d = self.moge, self.dims[m]
        moge.route(d, scores_dev, self.idx, self.gate)
        gc = self.gcounts if m == self.M else self.torch.empty((1,), dtype=self.torch.int32,
                                                               device="cuda")
        moge.permute(d, self.idx, None, self.counts, self.offsets, gc, self.sorted_pair,
                     self.pair_row, None, self.ws)
        counts = self.counts.cpu().numpy().astype(np.int64)
        return counts.reshape(self.M, self.N // self.M).sum(axis=1)

    def imbalance(self, scores: np.ndarray, with_peak: bool = False) -> tuple:
        """(IS grouped, IS global) for one batch, plus the global router's busiest
        group load over T*K/M when with_peak is set."""
        s = self.torch.from_numpy(scores).cuda()
        out = []
        for m in (self.M, 1):
            loads = self.group_loads(s, m)
            out.append(float(loads.max() - loads.min()) / self.T)
        if with_peak:
            out.append(float(loads.max()) * self.M / (self.T * self.K))
        return tuple(out)


def sweep(quick: bool):
    if quick:
        return [(64, 8, 8, T) for T in (16, 256)]
    cfgs = []
    for N, M in ((64, 8), (64, 4), (128, 8), (128, 16), (256, 16)):
        for kp in (1, 2):
            for T in (16, 64, 256, 1024, 4096, 16384):
                cfgs.append((N, M, M * kp, T))
    return cfgs


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--trials", type=int, default=64)
    ap.add_argument("--quick", action="store_true", help="two small configurations only")
    args = ap.parse_args()
    import sparse_moe_layer_moge_amd as moge
    rows = []
    for dist in ("iid", "zipf"):
        for (N, M, K, T) in sweep(args.quick):
            r = Router(moge, N, M, K, T)
            grp, glb, peak = [], [], []
            for trial in range(args.trials):
                a, b, c = r.imbalance(draw_scores(T, N, 1000 * trial + T, dist), with_peak=True)
                grp.append(a)
                glb.append(b)
                peak.append(c)
            glb = np.array(glb)
            rec = {"dist": dist, "N": N, "M": M, "K": K, "T": T, "trials": args.trials,
                   "moge_max_IS": max(grp), "global_mean_IS": round(float(glb.mean()), 4),
                   "global_p50_IS": round(float(np.percentile(glb, 50)), 4),
                   "global_p95_IS": round(float(np.percentile(glb, 95)), 4),
                   "global_frac_IS_gt_0": round(float((glb > 0).mean()), 4),
                   "global_busiest_over_balanced": round(float(np.mean(peak)), 3)}
            rows.append(rec)
            print(json.dumps(rec), flush=True)
    print("\n| scores | N | M | K | T | MoGE max IS | global top-K mean IS | p95 | P(IS > 0) "
          "| busiest / balanced |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['dist']} | {r['N']} | {r['M']} | {r['K']} | {r['T']} | {r['moge_max_IS']:g} | "
              f"{r['global_mean_IS']} | {r['global_p95_IS']} | {r['global_frac_IS_gt_0']} | "
              f"{r['global_busiest_over_balanced']} |")
    return 0


if __name__ == "__main__":
    sys.exit(main())
