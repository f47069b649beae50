"""GPU parity of the per-head QK-norm switch (page "DM0 paper definition vs. Dexbotic code",
section 1: Qwen3 experts, whose attention RMS-normalises each query and key head before RoPE)
against the float64 oracle on the same seeded inputs.

Bounds: the tiny fp32 model ||gpu - oracle||_inf / ||oracle||_inf <= 1e-4 for the prefill K/V,
one merged layer and the denoise chunk; a small bf16 model's first-layer K/V ||.||_inf-relative
<= 1e-2 (one layer, as for the unnormalised path); the DM0-base bf16 chunk max abs <= 2e-2,
mean abs <= 2e-3.  The flag without gains is rejected.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from dual_expert_merged_amd import binding as bd
from dual_expert_merged_amd import inputs
from dual_expert_merged_amd.configs import BF16, ModelShape, workload
from tests.gpu_harness import Gpu, dev_lens, err_stats, np32, rel_inf

pytestmark = pytest.mark.gpu


def test_qknorm_tiny_fp32_prefill_layer_and_denoise():
    wl = workload(8)
    lens = inputs.make_prefix_lens(wl)
    s = wl.shape
    print(f"case: QK-norm tiny fp32, prefill + merged layer + denoise, B={wl.batch} lens {lens.tolist()}", flush=True)
    vlm = inputs.make_vlm_weights(wl)
    aw = inputs.make_action_weights(wl)
    emb = inputs.make_prefix_embeds(wl)
    x1 = inputs.make_noise(wl)
    gpu = Gpu(wl, vlm, aw)
    k, v = gpu.prefill(emb, lens)
    kn, vn = np32(k), np32(v)
    refs = {}
    for b in range(wl.batch):
        P = int(lens[b])
        rk, rv, _ = O.prefill_kv(emb[b, :P], vlm, s)
        refs[b] = (rk, rv)
        for l in range(s.n_layers):
            assert rel_inf(kn[l, b, :, :P], rk[l]) <= 1e-4 and rel_inf(vn[l, b, :, :P], rv[l]) <= 1e-4, (b, l)
    print("prefill K/V of both samples within 1e-4", flush=True)
    got = gpu.denoise(k, v, lens, x1, wl.steps)
    for b in range(wl.batch):
        ref = O.suffix_denoise(x1[b], aw, refs[b][0], refs[b][1], s, wl.steps)
        e = rel_inf(got[b], ref)
        print(f"denoise sample {b}: rel inf err {e:.3e}", flush=True)
        assert e <= 1e-4, (b, e)
    # one merged layer of both experts with QK-norm
    rng = np.random.default_rng(80)
    P = wl.prefix_len
    h_pre = rng.standard_normal((1, P, s.vlm_hidden)).astype(np.float32)
    h_suf = rng.standard_normal((1, s.chunk, s.act_hidden)).astype(np.float32)
    hp, hs, kl, vl = gpu.merged_layer(1, h_pre, h_suf, [P])
    rp, rs, rk, rv = O.merged_layer(h_pre[0], h_suf[0], vlm, aw.body, 1, s)
    for name, g, r in (("h_prefix", hp[0], rp), ("h_suffix", hs[0], rs), ("k", kl[0], rk.transpose(1, 0, 2)),
                       ("v", vl[0], rv.transpose(1, 0, 2))):
        e = rel_inf(g, r)
        print(f"merged layer {name}: rel inf err {e:.3e}", flush=True)
        assert e <= 1e-4, (name, e)


def test_qknorm_small_bf16_prefill():
    shape = ModelShape(n_layers=2, vlm_hidden=256, act_hidden=128, vlm_ffn=768, act_ffn=384, n_q_heads=4,
                       n_kv_heads=2, head_dim=32, action_dim=32, chunk=50, dtype=BF16, qk_norm=True)
    wl = dataclasses.replace(workload(8), shape=shape)
    lens = np.array([64, 23], dtype=np.int32)
    print(f"case: QK-norm small bf16 prefill lens {lens.tolist()}", flush=True)
    vlm = inputs.make_vlm_weights(wl)
    emb = inputs.make_prefix_embeds(wl)
    gpu = Gpu(wl, vlm, None)
    k, v = gpu.prefill(emb, lens)
    kn, vn = np32(k), np32(v)
    for b in range(2):
        P = int(lens[b])
        rk, rv, _ = O.prefill_kv(emb[b, :P], vlm, shape)
        ek, ev = rel_inf(kn[0, b, :, :P], rk[0]), rel_inf(vn[0, b, :, :P], rv[0])
        print(f"sample {b} layer 0: K rel inf {ek:.3e}, V rel inf {ev:.3e}", flush=True)
        assert ek <= 1e-2 and ev <= 1e-2, (b, ek, ev)


@pytest.mark.timeout(600)
def test_qknorm_dm0_base_bf16_b2_and_b1():
    wl = workload(9)
    s = wl.shape
    lens = inputs.make_prefix_lens(wl)
    print(f"case: QK-norm DM0-base bf16 denoise B={wl.batch} and B=1, P={wl.prefix_len}", flush=True)
    aw = inputs.make_action_weights(wl)
    kc, vc = inputs.make_kv_cache(wl)
    x1 = inputs.make_noise(wl)
    gpu = Gpu(wl, None, aw)
    k, v = gpu.cache_to_device(kc, vc)
    got = gpu.denoise(k, v, lens, x1, wl.steps)
    refs = [O.suffix_denoise(x1[b], aw, kc[:, b], vc[:, b], s, wl.steps) for b in range(wl.batch)]
    for b in range(wl.batch):
        mx, mean = err_stats(got[b], refs[b])
        print(f"sample {b}: max abs err {mx:.3e}, mean abs err {mean:.3e}", flush=True)
        assert mx <= 2e-2 and mean <= 2e-3, (b, mx, mean)
    # batch 1: the single launch does not take QK-norm, the kernel sequence runs
    kb, vb = gpu.cache_to_device(kc[:, :1], vc[:, :1])
    one = gpu.denoise(kb, vb, lens[:1], x1[:1], wl.steps)
    mx, mean = err_stats(one[0], refs[0])
    print(f"B=1: max abs err {mx:.3e}, mean abs err {mean:.3e}", flush=True)
    assert mx <= 2e-2 and mean <= 2e-3


def test_qknorm_flag_needs_gains():
    wl = workload(8)
    print("case: QK-norm argument checks", flush=True)
    s = wl.shape
    aw = inputs.make_action_weights(dataclasses.replace(wl, shape=dataclasses.replace(s, qk_norm=False)))
    kc, vc = inputs.make_kv_cache(wl)
    lens = inputs.make_prefix_lens(wl)
    ctx = bd.Context(s, 0)
    da = bd.DeviceAction(aw, s.dtype)  # no q_norm / k_norm
    k, v = bd.to_device(kc, torch.float32), bd.to_device(vc, torch.float32)
    x = torch.from_numpy(inputs.make_noise(wl)).cuda()
    ws = ctx.workspace(bd.OP_DENOISE, wl.batch, wl.prefix_len)
    with pytest.raises(bd.DMError) as e:
        ctx.suffix_denoise(da, k, v, dev_lens(lens), x, wl.steps, ws)
    assert e.value.status == bd.DM_ERR_INVALID_ARG
    ctx.close()
