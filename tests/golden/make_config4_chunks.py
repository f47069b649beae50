"""Writes config4_chunks.npz: the oracle's action chunk for every sample of the batch-32 ragged
suffix-denoise workload (DM0-base action expert, prefix lengths 600..1100, 10 Euler steps),
from the seeded inputs.  Only the oracle and the seeded input generators run here.

    python -m tests.golden.make_config4_chunks [processes]

Samples are independent, so they are spread over worker processes (one BLAS thread each).
The file also keeps the prefix lengths and a fingerprint of the inputs, which the GPU test
compares with the inputs it regenerates, and the test recomputes two samples live.
"""
import multiprocessing as mp
import os
import sys
from pathlib import Path

import numpy as np

import oracle as O
from dual_expert_merged_amd import inputs
from dual_expert_merged_amd.configs import workload

OUT = Path(__file__).with_name("config4_chunks.npz")
_STATE = {}


def fingerprint(x1, kc, vc, lens):
    """A few sums that change if the seeded generators change."""
    return np.array([x1.sum(), kc[0, :, :, :8].sum(), vc[-1, :, :, :8].sum(), kc[:, -1, -1, :16].sum(),
                     float(lens.sum())], dtype=np.float64)


def _load():
    wl = workload(4)
    aw = inputs.make_action_weights(wl)
    kc, vc = inputs.make_kv_cache(wl)
    x1 = inputs.make_noise(wl)
    lens = inputs.make_prefix_lens(wl)
    return wl, aw, kc, vc, x1, lens


def _one(b):
    from threadpoolctl import threadpool_limits
    wl, aw, kc, vc, x1, lens = _STATE["d"]
    P = int(lens[b])
    with threadpool_limits(1):
        return b, O.suffix_denoise(x1[b], aw, kc[:, b, :, :P], vc[:, b, :, :P], wl.shape, wl.steps)


def main(nproc):
    _STATE["d"] = _load()          # inherited by the forked workers
    wl, aw, kc, vc, x1, lens = _STATE["d"]
    chunks = np.zeros(x1.shape, dtype=np.float64)
    with mp.get_context("fork").Pool(nproc) as pool:
        for b, c in pool.imap_unordered(_one, range(wl.batch)):
            chunks[b] = c
            print(f"sample {b} (P={lens[b]}) done", flush=True)
    np.savez_compressed(OUT, chunks=chunks.astype(np.float32), lens=lens,
                        fingerprint=fingerprint(x1, kc, vc, lens))
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else max(1, (os.cpu_count() or 2) // 2))
