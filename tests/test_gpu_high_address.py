"""Regression test for the scalar-based key/value copies of the bf16 attention kernel: it builds
each stage's 64-bit source address from two 32-bit words that went through the lane broadcast,
and a low word >= 2^31 once sign-extended into the high word (a faulting address).  Here the
K/V caches are placed where every low address word is >= 2^31, and the denoise must match the
float64 oracle (chunk bound max abs 2e-2, mean abs 2e-3).  The host side of the same split is
checked by tests/test_addr_words.py."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from dual_expert_merged_amd import inputs
from dual_expert_merged_amd.configs import BF16, ModelShape, workload
from tests.gpu_harness import Gpu, err_stats

pytestmark = pytest.mark.gpu
LOW_HALF = 1 << 31


def _placed(buf, off, like):
    n = like.numel() * like.element_size()
    return buf[off:off + n].view(torch.bfloat16).view(like.shape)


def test_denoise_with_caches_at_high_low_words():
    shape = ModelShape(n_layers=2, vlm_hidden=256, act_hidden=256, vlm_ffn=512, act_ffn=512, n_q_heads=4,
                       n_kv_heads=2, head_dim=128, action_dim=32, chunk=50, dtype=BF16)
    lens = np.array([200, 131], dtype=np.int32)
    wl = dataclasses.replace(workload(3), shape=shape, batch=2, prefix_len=208, steps=2)
    print(f"case: bf16 head-dim-128 denoise B=2 lens {lens.tolist()} with K/V at low address words >= 2^31",
          flush=True)
    aw = inputs.make_action_weights(wl)
    kc, vc = inputs.make_kv_cache(wl)
    x1 = inputs.make_noise(wl)
    gpu = Gpu(wl, None, aw)
    k0, v0 = gpu.cache_to_device(kc, vc)
    need = 2 * k0.numel() * k0.element_size()
    buf = torch.empty(LOW_HALF + 2 * need + 8192, dtype=torch.uint8, device="cuda")
    a = buf.data_ptr()
    lo = a & 0xFFFFFFFF
    if lo >= LOW_HALF and lo + need + 256 <= 1 << 32:
        target = (a + 255) // 256 * 256
    else:
        target = (a >> 32 << 32) + LOW_HALF
        if target < a:
            target += 1 << 32
    off = target - a
    assert 0 <= off and off + need <= buf.numel()
    k = _placed(buf, off, k0)
    v = _placed(buf, off + k0.numel() * k0.element_size(), v0)
    k.copy_(k0)
    v.copy_(v0)
    for t in (k, v):
        first, last = t.data_ptr(), t.data_ptr() + t.numel() * t.element_size() - 1
        assert (first & 0xFFFFFFFF) >= LOW_HALF and (first >> 32) == (last >> 32), hex(first)
    print(f"K at {k.data_ptr():#x}, V at {v.data_ptr():#x}", flush=True)
    del k0, v0
    got = gpu.denoise(k, v, lens, x1, wl.steps)
    for b in range(2):
        P = int(lens[b])
        ref = O.suffix_denoise(x1[b], aw, kc[:, b, :, :P], vc[:, b, :, :P], shape, wl.steps)
        mx, mean = err_stats(got[b], ref)
        print(f"sample {b} (P={P}): max abs err {mx:.3e}, mean abs err {mean:.3e}", flush=True)
        assert mx <= 2e-2 and mean <= 2e-3, (b, mx, mean)
