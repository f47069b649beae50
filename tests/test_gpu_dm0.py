"""GPU parity at the DM0-base shapes (bf16 weights and activations, fp32 accumulation,
hidden 2048 / 1024, FFN 6144 / 3072, 16 query heads over 8 KV heads of dim 128, chunk 50,
action dim 32) against the float64 oracle on the same seeded inputs.

Bounds: the final action chunk must satisfy max |gpu - oracle| <= 2e-2 and
mean |gpu - oracle| <= 2e-3.  One layer's outputs (hidden streams, its K/V) are held to
||gpu - oracle||_inf / ||oracle||_inf <= 1e-2 (five bf16 half-ulps: bf16 rounds to 2^-9
relative, and each stored K/V or hidden update has been rounded once or twice).  The KV cache
of a 28-layer prefill carries, at layer l, the rounding of l earlier bf16 layers in its hidden
state, so it is checked for drift only: each layer's K/V within ||.||_inf-relative 2e-2 and a
mean absolute error within 1e-2 of the reference's RMS (already layer 0 sits near 2e-3: the
stored value and the normalised GEMM input are each rounded once, mean |delta| ~ 2^-10).  The
per-layer accuracy of the same kernels is pinned by the one-layer test, and the chunk computed
from that cache is held to the chunk bounds.
"""
import numpy as np
import pytest
import torch

import oracle as O
from dual_expert_merged_amd import inputs
from dual_expert_merged_amd.configs import workload
from tests.gpu_harness import Gpu, err_stats, np32, rel_inf

pytestmark = pytest.mark.gpu
CHUNK_MAX, CHUNK_MEAN, INTER_REL, DEEP_REL, DEEP_MEAN = 2e-2, 2e-3, 1e-2, 2e-2, 1e-2


def _chunk_ok(got, ref, what):
    mx, mean = err_stats(got, ref)
    print(f"{what}: max abs err {mx:.3e}, mean abs err {mean:.3e}", flush=True)
    assert mx <= CHUNK_MAX and mean <= CHUNK_MEAN, (what, mx, mean)


def test_one_merged_layer_bf16():
    wl = workload(2)
    print("case: one DM0-base merged layer bf16, P=816", flush=True)
    s = wl.shape
    vlm = inputs.make_vlm_weights(wl)
    aw = inputs.make_action_weights(wl)
    gpu = Gpu(wl, vlm, aw)
    h_pre = inputs.make_prefix_embeds(wl)
    h_suf = inputs.make_suffix_hidden(wl)
    hp, hs, k, v = gpu.merged_layer(0, h_pre, h_suf, [wl.prefix_len])
    rp, rs, rk, rv = O.merged_layer(h_pre[0], h_suf[0], vlm, aw.body, 0, s)
    for name, g, r in (("h_prefix", hp[0], rp), ("h_suffix", hs[0], rs),
                       ("k_prefix", k[0], rk.transpose(1, 0, 2)), ("v_prefix", v[0], rv.transpose(1, 0, 2))):
        e = rel_inf(g, r)
        print(f"{name}: rel inf err {e:.3e}, max/mean abs {err_stats(g, r)}", flush=True)
        assert e <= INTER_REL, (name, e)


@pytest.fixture(scope="module")
def cfg3():
    wl = workload(3)
    aw = inputs.make_action_weights(wl)
    k, v = inputs.make_kv_cache(wl)
    x1 = inputs.make_noise(wl)
    return wl, aw, k, v, x1


def test_suffix_denoise_b1_bf16(cfg3):
    wl, aw, kc, vc, x1 = cfg3
    print("case: 28-layer suffix denoise bf16 B=1 P=816 N=10 eager+graph", flush=True)
    gpu = Gpu(wl, None, aw)
    k, v = gpu.cache_to_device(kc, vc)
    lens = inputs.make_prefix_lens(wl)
    eager = gpu.denoise(k, v, lens, x1, wl.steps)
    ref = O.suffix_denoise(x1[0], aw, kc[:, 0], vc[:, 0], wl.shape, wl.steps)
    _chunk_ok(eager[0], ref, "config-3 chunk")
    replays = gpu.denoise(k, v, lens, x1, wl.steps, graph=True, replays=3)
    for r in replays:
        np.testing.assert_array_equal(r, eager)


def test_suffix_denoise_b32_ragged_bf16():
    wl = workload(4)
    lens = inputs.make_prefix_lens(wl)
    print(f"case: suffix denoise bf16 B=32 ragged P in [{lens.min()},{lens.max()}] cap {wl.prefix_len}", flush=True)
    aw = inputs.make_action_weights(wl)
    kc, vc = inputs.make_kv_cache(wl)
    x1 = inputs.make_noise(wl)
    gpu = Gpu(wl, None, aw)
    k, v = gpu.cache_to_device(kc, vc)
    got = gpu.denoise(k, v, lens, x1, wl.steps)
    samples = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 31})
    for b in samples:
        ref = O.suffix_denoise(x1[b], aw, kc[:, b, :, :lens[b]], vc[:, b, :, :lens[b]], wl.shape, wl.steps)
        _chunk_ok(got[b], ref, f"config-4 sample {b} (P={lens[b]})")
    # Batch invariance: the sample run alone takes the batch-1 kernels (skinny GEMMs,
    # split-key attention with bf16 partials), the batch the tiled ones, so the two agree to the
    # bf16 bound rather than bit for bit; each is held to the oracle bound on its own.
    b = samples[0]
    kb, vb = gpu.cache_to_device(kc[:, b:b + 1], vc[:, b:b + 1])
    alone = gpu.denoise(kb, vb, lens[b:b + 1], x1[b:b + 1], wl.steps)
    ref = O.suffix_denoise(x1[b], aw, kc[:, b, :, :lens[b]], vc[:, b, :, :lens[b]], wl.shape, wl.steps)
    _chunk_ok(alone[0], ref, f"config-4 sample {b} alone at B=1")
    mx, mean = err_stats(alone[0], got[b])
    print(f"batch invariance sample {b}: max {mx:.3e} mean {mean:.3e}", flush=True)
    assert mx <= CHUNK_MAX and mean <= CHUNK_MEAN


def test_suffix_denoise_b3_ragged_split_keys_bf16():
    """Three samples of the batch-32 workload (shortest, longest, one between): few enough
    workgroups that attention splits every sample's keys into chunks, so the shorter samples
    have chunks past their keys and chunks straddling the prefix/action boundary."""
    wl = workload(4)
    lens_all = inputs.make_prefix_lens(wl)
    pick = [int(np.argmin(lens_all)), int(np.argmax(lens_all)), 7]
    lens = lens_all[pick]
    print(f"case: suffix denoise bf16 B=3 ragged P={list(lens)} cap {wl.prefix_len}", flush=True)
    aw = inputs.make_action_weights(wl)
    kc, vc = inputs.make_kv_cache(wl)
    x1 = inputs.make_noise(wl)
    gpu = Gpu(wl, None, aw)
    k, v = gpu.cache_to_device(kc[:, pick], vc[:, pick])
    got = gpu.denoise(k, v, lens, x1[pick], wl.steps)
    for i, b in enumerate(pick):
        ref = O.suffix_denoise(x1[b], aw, kc[:, b, :, :lens[i]], vc[:, b, :, :lens[i]], wl.shape, wl.steps)
        _chunk_ok(got[i], ref, f"config-4 sample {b} (P={lens[i]}) in a batch of 3")


def test_suffix_denoise_b16_ragged_bf16():
    """Sixteen samples of the batch-32 workload (800 action rows): the mid-size plans, 128 x 128
    QKV tiles with a partial last row tile, 128 x 256 gate/up tiles, residual projections split
    four ways over K with the separate reduce, and attention keys split in two chunks."""
    wl = workload(4)
    lens_all = inputs.make_prefix_lens(wl)
    pick = list(range(16))
    lens = lens_all[pick]
    print(f"case: suffix denoise bf16 B=16 ragged P in [{lens.min()},{lens.max()}] cap {wl.prefix_len}", flush=True)
    aw = inputs.make_action_weights(wl)
    kc, vc = inputs.make_kv_cache(wl)
    x1 = inputs.make_noise(wl)
    gpu = Gpu(wl, None, aw)
    k, v = gpu.cache_to_device(kc[:, pick], vc[:, pick])
    got = gpu.denoise(k, v, lens, x1[pick], wl.steps)
    for i in sorted({int(np.argmin(lens)), int(np.argmax(lens)), 15}):
        ref = O.suffix_denoise(x1[i], aw, kc[:, i, :, :lens[i]], vc[:, i, :, :lens[i]], wl.shape, wl.steps)
        _chunk_ok(got[i], ref, f"config-4 sample {i} (P={lens[i]}) in a batch of 16")


def test_suffix_denoise_empty_and_longest_prefix_bf16():
    """Batch of two at the DM0 shapes: one sample with no prefix token (its queries see the 50
    action keys only; every later key chunk of it is empty) and one with the longest prefix."""
    wl = workload(4)
    lens_all = inputs.make_prefix_lens(wl)
    b_long = int(np.argmax(lens_all))
    pick = [0, b_long]
    lens = np.array([0, lens_all[b_long]], dtype=lens_all.dtype)
    print(f"case: suffix denoise bf16 B=2 P={[int(p) for p in lens]} cap {wl.prefix_len}", flush=True)
    aw = inputs.make_action_weights(wl)
    kc, vc = inputs.make_kv_cache(wl)
    x1 = inputs.make_noise(wl)
    gpu = Gpu(wl, None, aw)
    k, v = gpu.cache_to_device(kc[:, pick], vc[:, pick])
    got = gpu.denoise(k, v, lens, x1[pick], wl.steps)
    for i, b in enumerate(pick):
        ref = O.suffix_denoise(x1[b], aw, kc[:, b, :, :lens[i]], vc[:, b, :, :lens[i]], wl.shape, wl.steps)
        _chunk_ok(got[i], ref, f"config-4 sample {b} with P={lens[i]}")


def test_prefill_then_denoise_bf16():
    wl = workload(5)
    print("case: 28-layer VLM prefill bf16 B=8 P=816, then suffix denoise", flush=True)
    s = wl.shape
    vlm = inputs.make_vlm_weights(wl)
    aw = inputs.make_action_weights(wl)
    emb = inputs.make_prefix_embeds(wl)
    x1 = inputs.make_noise(wl)
    lens = inputs.make_prefix_lens(wl)
    gpu = Gpu(wl, vlm, aw)
    k, v = gpu.prefill(emb, lens)
    got = gpu.denoise(k, v, lens, x1, wl.steps)
    kn, vn = np32(k), np32(v)
    b = 5
    rk, rv, _ = O.prefill_kv(emb[b], vlm, s)
    for l in range(s.n_layers):
        for name, g, r in (("K", kn[l, b], rk[l]), ("V", vn[l, b], rv[l])):
            e = rel_inf(g, r)
            mean_rel = err_stats(g, r)[1] / float(np.sqrt(np.mean(r * r)))
            print(f"prefill sample {b} layer {l} {name}: rel inf err {e:.3e}, mean abs / rms {mean_rel:.3e}",
                  flush=True)
            assert e <= DEEP_REL and mean_rel <= DEEP_MEAN, (l, name, e, mean_rel)
    ref = O.suffix_denoise(x1[b], aw, rk, rv, s, wl.steps)
    _chunk_ok(got[b], ref, f"config-5 sample {b} chunk")


def test_prefill_ragged_prefix_bf16():
    """Ragged prefix lengths through the batch-8 prefill (8 x 816 rows: large GEMM tiles that
    straddle samples and hold rows past a sample's length, down to a one-token prefix): the K/V
    rows of the shortest samples against the oracle, every row at or past a length left
    untouched, then the denoise on that cache."""
    wl = workload(5)
    s = wl.shape
    lens = np.array([816, 613, 700, 1, 816, 655, 777, 802], dtype=np.int32)
    print(f"case: 28-layer VLM prefill bf16 B=8 ragged P={[int(p) for p in lens]} cap {wl.prefix_len}", flush=True)
    vlm = inputs.make_vlm_weights(wl)
    aw = inputs.make_action_weights(wl)
    emb = inputs.make_prefix_embeds(wl).copy()
    for b in range(wl.batch):
        emb[b, lens[b]:] = 0.0
    x1 = inputs.make_noise(wl)
    gpu = Gpu(wl, vlm, aw)
    k, v = gpu.prefill(emb, lens)  # the harness zero-fills the caches first
    kn, vn = np32(k), np32(v)
    for b in range(wl.batch):
        assert not np.any(kn[:, b, :, lens[b]:]) and not np.any(vn[:, b, :, lens[b]:]), f"rows past P={lens[b]} written"
    refs = {}
    for b in (3, 1):
        rk, rv, _ = O.prefill_kv(emb[b, :lens[b]], vlm, s)
        refs[b] = (rk, rv)
        for l in range(s.n_layers):
            for name, g, r in (("K", kn[l, b, :, :lens[b]], rk[l]), ("V", vn[l, b, :, :lens[b]], rv[l])):
                e = rel_inf(g, r)
                mean_rel = err_stats(g, r)[1] / float(np.sqrt(np.mean(r * r)))
                assert e <= DEEP_REL and mean_rel <= DEEP_MEAN, (b, l, name, e, mean_rel)
        print(f"prefill sample {b} (P={lens[b]}): K/V of all {s.n_layers} layers within bounds", flush=True)
    got = gpu.denoise(k, v, lens, x1, wl.steps)
    for b in (3, 1):
        ref = O.suffix_denoise(x1[b], aw, refs[b][0], refs[b][1], s, wl.steps)
        _chunk_ok(got[b], ref, f"config-5 ragged sample {b} (P={lens[b]}) chunk")
