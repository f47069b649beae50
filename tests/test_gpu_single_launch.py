"""GPU parity of the single-launch batch-1 suffix denoise (the DM0-base action expert at batch 1
runs as one kernel launch per chunk; persist.hip) against the float64 oracle, over the prefix
lengths it accepts (none, one token, a ragged tail, the DM0 prefix, the largest), and against the
multi-kernel sequence on the same inputs.  Bounds: the final action chunk within max abs 2e-2 and
mean abs 2e-3 of the oracle; replays and repeated runs bitwise equal."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from dual_expert_merged_amd import binding as bd
from dual_expert_merged_amd import inputs
from dual_expert_merged_amd.configs import workload
from tests.gpu_harness import Gpu, err_stats

pytestmark = pytest.mark.gpu
CHUNK_MAX, CHUNK_MEAN = 2e-2, 2e-3


@pytest.fixture(scope="module")
def dm0():
    wl = workload(3)
    aw = inputs.make_action_weights(wl)
    return wl, aw


def _cache(wl, P_cap, seed):
    s = wl.shape
    rng = np.random.default_rng([77, P_cap, seed])
    shape = (s.n_layers, 1, s.n_kv_heads, P_cap, s.head_dim)
    k = inputs.round_to(rng.standard_normal(shape, dtype=np.float32), s.dtype)
    v = inputs.round_to(rng.standard_normal(shape, dtype=np.float32), s.dtype)
    x1 = rng.standard_normal((1, s.chunk, s.action_dim), dtype=np.float32)
    return k, v, x1


@pytest.mark.parametrize("P,P_cap", [(816, 816), (0, 64), (1, 16), (333, 400), (960, 960)])
def test_single_launch_matches_oracle(dm0, P, P_cap):
    wl, aw = dm0
    print(f"case: single-launch denoise B=1 P={P} P_cap={P_cap}", flush=True)
    kc, vc, x1 = _cache(wl, P_cap, P)
    if P < P_cap:  # rows past the prefix hold values the kernel must never use
        kc[:, :, :, P:] = np.nan
        vc[:, :, :, P:] = np.nan
    gpu = Gpu(wl, None, aw)
    k, v = gpu.cache_to_device(kc, vc)
    got = gpu.denoise(k, v, [P], x1, wl.steps)
    ref = O.suffix_denoise(x1[0], aw, kc[:, 0, :, :P], vc[:, 0, :, :P], wl.shape, wl.steps)
    mx, mean = err_stats(got[0], ref)
    print(f"P={P}: max abs err {mx:.3e}, mean abs err {mean:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert mx <= CHUNK_MAX and mean <= CHUNK_MEAN, (mx, mean)


def test_single_launch_agrees_with_multi_kernel_and_replays(dm0):
    wl, aw = dm0
    print("case: single-launch vs multi-kernel, B=1 P=816, eager and graph", flush=True)
    kc, vc = inputs.make_kv_cache(wl)
    x1 = inputs.make_noise(wl)
    lens = inputs.make_prefix_lens(wl)
    single = Gpu(wl, None, aw)
    multi = Gpu(wl, None, aw)
    multi.ctx = bd.Context(wl.shape, 0, bd.DM_FLAG_MULTI_KERNEL)
    k, v = single.cache_to_device(kc, vc)
    a = single.denoise(k, v, lens, x1, wl.steps)
    b = multi.denoise(k, v, lens, x1, wl.steps)
    mx, mean = err_stats(a, b)
    print(f"single vs multi: max {mx:.3e} mean {mean:.3e}", flush=True)
    assert mx <= CHUNK_MAX and mean <= CHUNK_MEAN
    again = single.denoise(k, v, lens, x1, wl.steps)
    np.testing.assert_array_equal(again, a)  # deterministic
    replays = single.denoise(k, v, lens, x1, wl.steps, graph=True, replays=3)
    for r in replays:
        np.testing.assert_array_equal(r, a)  # graph replay == eager, every replay


def test_single_launch_one_euler_step_and_short_stack(dm0):
    """N = 1 and a 3-layer stack: the first step's embedding, one velocity reduce and the output
    written after the only step."""
    wl, aw = dm0
    s = dataclasses.replace(wl.shape, n_layers=3)
    wl3 = dataclasses.replace(wl, shape=s)
    body3 = aw.body.layers(0, 3)
    aw3 = dataclasses.replace(aw, body=body3)
    print("case: single-launch denoise, 3 layers, N=1 and N=2", flush=True)
    kc, vc, x1 = _cache(wl3, 816, 5)
    gpu = Gpu(wl3, None, aw3)
    k, v = gpu.cache_to_device(kc, vc)
    for N in (1, 2):
        got = gpu.denoise(k, v, [700], x1, N)
        ref = O.suffix_denoise(x1[0], aw3, kc[:, 0, :, :700], vc[:, 0, :, :700], s, N)
        mx, mean = err_stats(got[0], ref)
        print(f"N={N}: max {mx:.3e} mean {mean:.3e}", flush=True)
        assert mx <= CHUNK_MAX and mean <= CHUNK_MEAN
