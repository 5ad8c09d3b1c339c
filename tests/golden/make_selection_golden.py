"""Write the oracle's block selection for a full-size workload to tests/golden/<workload>_selection.json.

Calls only the oracle (``oracle.block_masses`` and ``oracle.select_blocks``) on the seeded numpy
inputs of ``synth``; nothing here touches the GPU path.  For every block row it records the
number of kept blocks, a CRC32 of the ascending kept columns (int32, little endian) and the row's
tie margin: the smaller of (a) the relative mass gap between the last kept and the first dropped
non-forced block and (b) the distance of the cumulative kept mass from the target, in units of
T_I.  A GPU row whose set differs from the oracle's is a tie only where that margin is <= 1e-6.

Workloads whose tau is not fixed (the long-context one) get tau by bisection on the exact masses
so that the kept-block density nnzb / C is as close as possible to the workload's target density,
as the long-context configuration asks ("tau tuned per seed to roughly 5% density").

Usage:  python tests/golden/make_selection_golden.py --workload long_131k --seeds 0 1 2 [--procs 8]
"""
from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import sys
import time
import zlib

for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, "1")

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

_G = {}


def _row_masses(job):
    b, seq_start, n, I = job
    M, _ = oracle.block_masses(_G["Q"], _G["K"], seq_start, n, I, _G["B"])
    return b, M


def _select_all(Ms, rows, tau, H_s):
    return [oracle.select_blocks(M, I, float(H_s * n_rows), tau) for M, (I, n_rows) in zip(Ms, rows)]


def _margin(M, sel, I, T_I, tau):
    kept = set(sel["kept"])
    dropped = [M[J] for J in range(I + 1) if J not in kept]
    gaps = [abs(sel["cum"] - tau * T_I) / T_I]
    if sel["cum_before_last"] is not None:
        gaps.append(abs(sel["cum_before_last"] - tau * T_I) / T_I)
    if sel["last_mass"] is not None and dropped:
        m_last = sel["last_mass"]
        gaps.append(abs(m_last - max(dropped)) / max(m_last, 1e-300))
    return float(min(gaps))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--seeds", type=int, nargs="+", default=[0])
    ap.add_argument("--procs", type=int, default=8)
    args = ap.parse_args()
    wl = synth.WORKLOADS[args.workload]
    path = os.path.join(HERE, f"{args.workload}_selection.json")
    out = json.load(open(path)) if os.path.exists(path) else {}
    out.update({"workload": args.workload, "B": wl.B, "H_s": wl.H_s,
                "generator": "synth.make_layer_inputs(workload, seed, layer=0) (numpy)",
                "written_by": "tests/golden/make_selection_golden.py (oracle only)",
                "row_order": "sequences in order, block rows I = 0.. within each"})
    out.setdefault("seeds", {})
    for seed in args.seeds:
        t0 = time.time()
        x = synth.make_layer_inputs(wl, seed)
        cu, B = x["cu_seqlens"], wl.B
        jobs, rows = [], []
        for sq in range(len(cu) - 1):
            n = int(cu[sq + 1] - cu[sq])
            for I in range((n + B - 1) // B):
                jobs.append((len(jobs), int(cu[sq]), n, I))
                rows.append((I, min(n, (I + 1) * B) - I * B))
        _G.update(Q=x["q_s"], K=x["k_s"], B=B)
        Ms = [None] * len(jobs)
        order = sorted(jobs, key=lambda j: -(j[3] + 1) * j[2])    # largest rows first
        with mp.get_context("fork").Pool(args.procs) as pool:
            for k, (b, M) in enumerate(pool.imap_unordered(_row_masses, order)):
                Ms[b] = M
                if k % 64 == 0:
                    print(f"seed {seed}: {k + 1}/{len(jobs)} block rows, {time.time() - t0:.0f} s", flush=True)
        C = sum(I + 1 for I, _ in rows)
        if wl.tau is not None:
            tau = float(np.float32(wl.tau))
        else:
            lo, hi = 1e-6, 1.0
            target = wl.target_density
            for _ in range(40):
                mid = float(np.float32(0.5 * (lo + hi)))
                dens = sum(len(s["kept"]) for s in _select_all(Ms, rows, mid, wl.H_s)) / C
                if dens < target:
                    lo = mid
                else:
                    hi = mid
                if hi - lo < 1e-7:
                    break
            cands = [float(np.float32(lo)), float(np.float32(hi))]
            dens = [sum(len(s["kept"]) for s in _select_all(Ms, rows, t, wl.H_s)) / C for t in cands]
            tau = cands[int(np.argmin([abs(d - target) for d in dens]))]
        sels = _select_all(Ms, rows, tau, wl.H_s)
        counts, crcs, margins = [], [], []
        for b, s in enumerate(sels):
            I, n_rows = rows[b]
            kept = np.asarray(sorted(s["kept"]), dtype="<i4")
            counts.append(int(kept.size))
            crcs.append(f"{zlib.crc32(kept.tobytes()):08x}")
            margins.append(_margin(Ms[b], s, I, float(wl.H_s * n_rows), tau))
        nnzb = int(sum(counts))
        out["seeds"][str(seed)] = {"tau": tau, "nnzb": nnzb, "n_causal": C, "density": nnzb / C,
                                   "counts": counts, "crc32": crcs,
                                   "tie_margin": [float(f"{m:.3e}") for m in margins]}
        print(f"seed {seed}: tau {tau:.7g} nnzb {nnzb} density {nnzb / C:.4f} "
              f"({time.time() - t0:.0f} s)", flush=True)
        with open(path, "w") as f:
            json.dump(out, f, separators=(",", ":"))
            f.write("\n")


if __name__ == "__main__":
    main()
