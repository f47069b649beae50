"""GPU parity at the largest prefix the library takes (P_cap <= 65536) against the float64 oracle.

- tiny fp32 model, B = 2 with prefixes 65536 (the maximum) and 40001, 4 Euler steps: the key
  range splits into the maximum of 16 chunks of ~4100 keys each (the merge holds every chunk's
  statistics in registers), RoPE runs to position 65585; bound ||gpu - oracle||_inf /
  ||oracle||_inf <= 1e-4 per sample.
- DM0-base shapes with 2 layers, bf16, B = 2 with prefixes 16384 and 9001, 3 Euler steps: the
  bf16 attention kernel over 16 chunks of ~1050 keys; chunk bounds max abs <= 2e-2, mean abs
  <= 2e-3.
"""
import dataclasses

import numpy as np
import pytest

import oracle as O
from dual_expert_merged_amd import inputs
from dual_expert_merged_amd.configs import workload
from tests.gpu_harness import Gpu, err_stats, rel_inf

pytestmark = pytest.mark.gpu


def _run(wl, lens):
    aw = inputs.make_action_weights(wl)
    kc, vc = inputs.make_kv_cache(wl)
    x1 = inputs.make_noise(wl)
    gpu = Gpu(wl, None, aw)
    k, v = gpu.cache_to_device(kc, vc)
    got = gpu.denoise(k, v, lens, x1, wl.steps)
    refs = [O.suffix_denoise(x1[b], aw, kc[:, b, :, :int(lens[b])], vc[:, b, :, :int(lens[b])], wl.shape, wl.steps)
            for b in range(wl.batch)]
    return got, refs


@pytest.mark.timeout(600)
def test_tiny_fp32_at_the_largest_prefix():
    lens = np.array([65536, 40001], dtype=np.int32)
    wl = dataclasses.replace(workload(1), batch=2, prefix_len=65536)
    print(f"case: tiny fp32 denoise B=2 P_cap=65536 lens {lens.tolist()} steps {wl.steps}", flush=True)
    got, refs = _run(wl, lens)
    for b in range(2):
        e = rel_inf(got[b], refs[b])
        print(f"sample {b} (P={lens[b]}): rel inf err {e:.3e}", flush=True)
        assert e <= 1e-4, (b, e)


@pytest.mark.timeout(600)
def test_dm0_base_bf16_two_layers_long_prefix():
    lens = np.array([16384, 9001], dtype=np.int32)
    wl = dataclasses.replace(workload(3), shape=dataclasses.replace(workload(3).shape, n_layers=2), batch=2,
                             prefix_len=16384, steps=3)
    print(f"case: DM0-base shapes, 2 layers, bf16 denoise B=2 P_cap=16384 lens {lens.tolist()} steps 3", flush=True)
    got, refs = _run(wl, lens)
    for b in range(2):
        mx, mean = err_stats(got[b], refs[b])
        print(f"sample {b} (P={lens[b]}): max abs err {mx:.3e}, mean abs err {mean:.3e}", flush=True)
        assert mx <= 2e-2 and mean <= 2e-3, (b, mx, mean)
