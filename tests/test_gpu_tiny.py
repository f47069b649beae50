"""GPU parity on the tiny fp32 merged-attention model: every op of the HIP path against the
float64 oracle on the same seeded inputs, bound ||gpu - oracle||_inf / ||oracle||_inf <= 1e-4
per output tensor; plus closed forms (zero queries, constant velocity), ragged batches,
graph replay and determinism.  Shapes: 2 layers, hidden 256 / 128, 4 query heads over 2 KV
heads of dim 32, FFN 768 / 384, prefix 64, chunk 50, action dim 32, 4 Euler steps."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from dual_expert_merged_amd import binding as bd
from dual_expert_merged_amd import inputs
from dual_expert_merged_amd.configs import workload
from tests.gpu_harness import Gpu, dev_lens, err_stats, np32, rel_inf

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module")
def cfg1():
    wl = workload(1)
    vlm = inputs.make_vlm_weights(wl)
    aw = inputs.make_action_weights(wl)
    return wl, vlm, aw, Gpu(wl, vlm, aw)


def _ragged(wl, lens, P_cap=None):
    """The tiny model with B = len(lens) samples of the given prefix lengths."""
    return dataclasses.replace(wl, batch=len(lens), prefix_len=P_cap or max(lens))


def test_merged_layer_matches_oracle(cfg1):
    wl, vlm, aw, gpu = cfg1
    print("case: merged layer, tiny fp32, B=1, P=64", flush=True)
    s = wl.shape
    rng = np.random.default_rng(100)
    P = wl.prefix_len
    h_pre = rng.standard_normal((1, P, s.vlm_hidden)).astype(np.float32)
    h_suf = rng.standard_normal((1, s.chunk, s.act_hidden)).astype(np.float32)
    for layer in range(s.n_layers):
        hp, hs, k, v = gpu.merged_layer(layer, h_pre, h_suf, [P])
        rp, rs, rk, rv = O.merged_layer(h_pre[0], h_suf[0], vlm, aw.body, layer, s)
        assert rel_inf(hp[0], rp) <= TOL, rel_inf(hp[0], rp)
        assert rel_inf(hs[0], rs) <= TOL, rel_inf(hs[0], rs)
        assert rel_inf(k[0], rk.transpose(1, 0, 2)) <= TOL
        assert rel_inf(v[0], rv.transpose(1, 0, 2)) <= TOL


def test_merged_layer_ragged_batch(cfg1):
    """Several samples with ragged prefixes (1, a tile boundary, a ragged tail, the cap);
    prefix rows past a sample's length are left untouched."""
    wl, vlm, aw, gpu = cfg1
    s = wl.shape
    lens = [64, 1, 33, 50, 17]
    print(f"case: merged layer ragged lens={lens}", flush=True)
    P_cap = 64
    rng = np.random.default_rng(101)
    h_pre = rng.standard_normal((len(lens), P_cap, s.vlm_hidden)).astype(np.float32)
    h_suf = rng.standard_normal((len(lens), s.chunk, s.act_hidden)).astype(np.float32)
    hp, hs, k, v = gpu.merged_layer(1, h_pre, h_suf, lens)
    for b, P in enumerate(lens):
        rp, rs, rk, rv = O.merged_layer(h_pre[b, :P], h_suf[b], vlm, aw.body, 1, s)
        assert rel_inf(hp[b, :P], rp) <= TOL
        assert rel_inf(hs[b], rs) <= TOL
        assert rel_inf(k[b, :, :P], rk.transpose(1, 0, 2)) <= TOL
        assert rel_inf(v[b, :, :P], rv.transpose(1, 0, 2)) <= TOL
        np.testing.assert_array_equal(hp[b, P:], h_pre[b, P:])
        assert np.all(k[b, :, P:] == 0)


def test_zero_queries_average_visible_values(cfg1):
    """W_q = 0 makes every score equal, so each attention output is the mean of the values the
    block mask lets it see.  With W_o = I (hidden = Hq*D) and W_gate = 0 (the MLP adds 0) a
    prefix row's update is the mean of its sample's prefix values, read back from k/v_out."""
    wl, vlm, aw, gpu = cfg1
    s = dataclasses.replace(wl.shape, vlm_hidden=128, vlm_ffn=384)
    wl2 = dataclasses.replace(wl, shape=s)
    v2 = inputs.make_expert(wl2, inputs.VLM_W, 128, 384)
    qd = s.n_q_heads * s.head_dim
    for w in (v2,):
        w.w_qkv[:, :qd] = 0
        w.w_o[:] = np.eye(128, dtype=np.float32)[None]
        w.w_gate[:] = 0
    g2 = Gpu(wl2, v2, aw)
    lens = [64, 23]
    print(f"case: zero-query closed form lens={lens}", flush=True)
    rng = np.random.default_rng(102)
    h_pre = rng.standard_normal((2, 64, 128)).astype(np.float32)
    h_suf = rng.standard_normal((2, s.chunk, s.act_hidden)).astype(np.float32)
    hp, hs, k, v = g2.merged_layer(0, h_pre, h_suf, lens)
    G = s.n_q_heads // s.n_kv_heads
    for b, P in enumerate(lens):
        upd = (hp[b, :P] - h_pre[b, :P]).reshape(P, s.n_q_heads, s.head_dim)
        for h in range(s.n_q_heads):
            mean = v[b, h // G, :P].astype(np.float64).mean(0)
            np.testing.assert_allclose(upd[:, h], np.broadcast_to(mean, (P, s.head_dim)), rtol=0, atol=2e-5)


def test_prefill_matches_oracle(cfg1):
    wl, vlm, aw, gpu = cfg1
    s = wl.shape
    lens = [64, 40, 7]
    print(f"case: prefill tiny lens={lens}", flush=True)
    wl3 = _ragged(wl, lens, 64)
    emb = np.random.default_rng(103).standard_normal((3, 64, s.vlm_hidden)).astype(np.float32)
    k, v = gpu.prefill(emb, lens)
    k, v = np32(k), np32(v)
    for b, P in enumerate(lens):
        rk, rv, _ = O.prefill_kv(emb[b, :P], vlm, s)
        assert rel_inf(k[:, b, :, :P], rk) <= TOL, rel_inf(k[:, b, :, :P], rk)
        assert rel_inf(v[:, b, :, :P], rv) <= TOL
        assert np.all(k[:, b, :, P:] == 0)


def test_denoise_matches_oracle_eager_and_graph(cfg1):
    wl, vlm, aw, gpu = cfg1
    s = wl.shape
    print("case: denoise tiny B=1 eager+graph", flush=True)
    emb = inputs.make_prefix_embeds(wl)
    x1 = inputs.make_noise(wl)
    rk, rv, _ = O.prefill_kv(emb[0], vlm, s)
    ref = O.suffix_denoise(x1[0], aw, rk, rv, s, wl.steps)
    k, v = gpu.cache_to_device(rk[:, None].astype(np.float32), rv[:, None].astype(np.float32))
    lens = [wl.prefix_len]
    eager = gpu.denoise(k, v, lens, x1, wl.steps)
    assert rel_inf(eager[0], ref) <= TOL, rel_inf(eager[0], ref)
    replays = gpu.denoise(k, v, lens, x1, wl.steps, graph=True, replays=3)
    for r in replays:
        np.testing.assert_array_equal(r, eager)  # graph replay == eager, bit for bit, every replay


def test_end_to_end_prefill_then_denoise(cfg1):
    wl, vlm, aw, gpu = cfg1
    s = wl.shape
    print("case: end-to-end tiny prefill+denoise", flush=True)
    emb = inputs.make_prefix_embeds(wl)
    x1 = inputs.make_noise(wl)
    k, v = gpu.prefill(emb, [wl.prefix_len])
    got = gpu.denoise(k, v, [wl.prefix_len], x1, wl.steps)
    ref = O.euler_integrate(x1[0], lambda x, t: O.velocity_joint(x, t, aw, vlm, emb[0], s), wl.steps)
    assert rel_inf(got[0], ref) <= TOL, rel_inf(got[0], ref)


def test_ragged_denoise_and_batch_invariance(cfg1):
    """Ragged batch against the oracle per sample; each sample also equals itself run alone
    (B = 1 takes the split-key attention path, the batch does not)."""
    wl, vlm, aw, gpu = cfg1
    s = wl.shape
    lens = [64, 1, 31, 64, 45, 2, 63, 16]
    print(f"case: ragged denoise lens={lens}", flush=True)
    B, P_cap = len(lens), 64
    rng = np.random.default_rng(104)
    L, Hkv, D = s.n_layers, s.n_kv_heads, s.head_dim
    kc = np.zeros((L, B, Hkv, P_cap, D), np.float32)
    vc = np.zeros_like(kc)
    for b, P in enumerate(lens):
        kc[:, b, :, :P] = rng.standard_normal((L, Hkv, P, D))
        vc[:, b, :, :P] = rng.standard_normal((L, Hkv, P, D))
    x1 = rng.standard_normal((B, s.chunk, s.action_dim)).astype(np.float32)
    k, v = gpu.cache_to_device(kc, vc)
    got = gpu.denoise(k, v, lens, x1, 3)
    for b, P in enumerate(lens):
        ref = O.suffix_denoise(x1[b], aw, kc[:, b, :, :P], vc[:, b, :, :P], s, 3)
        assert rel_inf(got[b], ref) <= TOL, (b, rel_inf(got[b], ref))
    for b in (1, 4):
        kb, vb = gpu.cache_to_device(kc[:, b:b + 1], vc[:, b:b + 1])
        alone = gpu.denoise(kb, vb, [lens[b]], x1[b:b + 1], 3)
        np.testing.assert_allclose(alone[0], got[b], rtol=0, atol=1e-5)


def test_empty_prefix_in_ragged_batch(cfg1):
    """Samples with no prefix token (P_b = 0) attend to the action chunk only; a batch mixing
    them with full prefixes matches the oracle per sample."""
    wl, vlm, aw, gpu = cfg1
    s = wl.shape
    lens = [0, 64, 0, 5]
    print(f"case: ragged denoise with empty prefixes lens={lens}", flush=True)
    B, P_cap = len(lens), 64
    rng = np.random.default_rng(105)
    L, Hkv, D = s.n_layers, s.n_kv_heads, s.head_dim
    kc = rng.standard_normal((L, B, Hkv, P_cap, D)).astype(np.float32)  # rows past P_b are never read
    vc = rng.standard_normal((L, B, Hkv, P_cap, D)).astype(np.float32)
    x1 = rng.standard_normal((B, s.chunk, s.action_dim)).astype(np.float32)
    k, v = gpu.cache_to_device(kc, vc)
    got = gpu.denoise(k, v, lens, x1, 3)
    for b, P in enumerate(lens):
        ref = O.suffix_denoise(x1[b], aw, kc[:, b, :, :P], vc[:, b, :, :P], s, 3)
        assert rel_inf(got[b], ref) <= TOL, (b, rel_inf(got[b], ref))


def test_constant_velocity_closed_form(cfg1):
    """W_out = 0, b_out = c: v = c whatever the layers compute, so x_0 = x_1 - c."""
    wl, vlm, aw, gpu = cfg1
    s = wl.shape
    print("case: constant velocity", flush=True)
    aw2 = dataclasses.replace(aw, w_out=np.zeros_like(aw.w_out),
                              b_out=np.linspace(-1, 1, s.action_dim).astype(np.float32))
    g2 = Gpu(wl, None, aw2)
    rng = np.random.default_rng(105)
    kc = rng.standard_normal((s.n_layers, 1, s.n_kv_heads, 64, s.head_dim)).astype(np.float32)
    x1 = rng.standard_normal((1, s.chunk, s.action_dim)).astype(np.float32)
    k, v = g2.cache_to_device(kc, kc)
    got = g2.denoise(k, v, [64], x1, 7)
    np.testing.assert_allclose(got, x1 - aw2.b_out[None, None, :], rtol=0, atol=1e-5)


def test_determinism(cfg1):
    wl, vlm, aw, gpu = cfg1
    print("case: determinism", flush=True)
    emb = inputs.make_prefix_embeds(wl)
    x1 = inputs.make_noise(wl)
    k, v = gpu.prefill(emb, [64])
    a = gpu.denoise(k, v, [64], x1, wl.steps)
    k2, v2 = gpu.prefill(emb, [64])
    assert torch.equal(k, k2) and torch.equal(v, v2)
    b = gpu.denoise(k2, v2, [64], x1, wl.steps)
    np.testing.assert_array_equal(a, b)


def test_plan_rejects_other_step_count(cfg1):
    wl, vlm, aw, gpu = cfg1
    s = wl.shape
    print("case: plan step mismatch", flush=True)
    kc = np.zeros((s.n_layers, 1, s.n_kv_heads, 64, s.head_dim), np.float32)
    k, v = gpu.cache_to_device(kc, kc)
    ws = gpu.ctx.workspace(bd.OP_DENOISE, 1, 64)
    x = torch.zeros((1, s.chunk, s.action_dim), device="cuda")
    plan = gpu.ctx.denoise_plan(gpu.aw, k, v, dev_lens([64]), x, 4, ws)
    with pytest.raises(bd.DMError) as e:
        plan.launch(5)
    assert e.value.status == bd.DM_ERR_PLAN_MISMATCH
    plan.close()
    with pytest.raises(bd.DMError) as e:
        gpu.ctx.suffix_denoise(gpu.aw, k, v, dev_lens([64]), x, 4, ws[:100])
    assert e.value.status == bd.DM_ERR_WORKSPACE


def test_one_action_token_per_sample(cfg1):
    """chunk = 1: every GEMM row tile of four rows spans four samples (the epilogues' sample and
    token of each row), ragged prefixes, against the oracle per sample."""
    wl, vlm, aw, _ = cfg1
    s = dataclasses.replace(wl.shape, chunk=1)
    wl1 = dataclasses.replace(wl, shape=s)
    lens = [64, 3, 0, 17, 40]
    print(f"case: tiny fp32 chunk=1 B=5 lens={lens}", flush=True)
    B, P_cap = len(lens), 64
    rng = np.random.default_rng(106)
    L, Hkv, D = s.n_layers, s.n_kv_heads, s.head_dim
    kc = rng.standard_normal((L, B, Hkv, P_cap, D)).astype(np.float32)
    vc = rng.standard_normal((L, B, Hkv, P_cap, D)).astype(np.float32)
    x1 = rng.standard_normal((B, 1, s.action_dim)).astype(np.float32)
    g = Gpu(wl1, vlm, aw)
    k, v = g.cache_to_device(kc, vc)
    got = g.denoise(k, v, lens, x1, 3)
    for b, P in enumerate(lens):
        ref = O.suffix_denoise(x1[b], aw, kc[:, b, :, :P], vc[:, b, :, :P], s, 3)
        assert rel_inf(got[b], ref) <= TOL, (b, rel_inf(got[b], ref))
    # one merged layer with one action token per sample
    h_pre = rng.standard_normal((B, P_cap, s.vlm_hidden)).astype(np.float32)
    h_suf = rng.standard_normal((B, 1, s.act_hidden)).astype(np.float32)
    hp, hs, kk, vv = g.merged_layer(0, h_pre, h_suf, lens)
    for b, P in enumerate(lens):
        rp, rs, rk, rv = O.merged_layer(h_pre[b, :P], h_suf[b], vlm, aw.body, 0, s)
        assert rel_inf(hs[b], rs) <= TOL, (b, rel_inf(hs[b], rs))
        if P:
            assert rel_inf(hp[b, :P], rp) <= TOL
            assert rel_inf(kk[b, :, :P], rk.transpose(1, 0, 2)) <= TOL


def test_prefix_capacity_one(cfg1):
    """P_cap = 1: one prefix row per sample (four samples per GEMM row tile), prefill and one
    merged layer for B = 5 with prefixes of 0 or 1 tokens."""
    wl, vlm, aw, gpu = cfg1
    s = wl.shape
    lens = [1, 0, 1, 1, 0]
    print(f"case: tiny fp32 P_cap=1 B=5 lens={lens}", flush=True)
    B = len(lens)
    rng = np.random.default_rng(107)
    emb = rng.standard_normal((B, 1, s.vlm_hidden)).astype(np.float32)
    k, v = gpu.prefill(emb, lens)
    k, v = np32(k), np32(v)
    for b, P in enumerate(lens):
        if P:
            rk, rv, _ = O.prefill_kv(emb[b, :P], vlm, s)
            assert rel_inf(k[:, b, :, :P], rk) <= TOL, (b, rel_inf(k[:, b, :, :P], rk))
            assert rel_inf(v[:, b, :, :P], rv) <= TOL
        else:
            assert not np.any(k[:, b]) and not np.any(v[:, b])
    h_suf = rng.standard_normal((B, s.chunk, s.act_hidden)).astype(np.float32)
    hp, hs, kk, vv = gpu.merged_layer(1, emb, h_suf, lens)
    for b, P in enumerate(lens):
        rp, rs, rk, rv = O.merged_layer(emb[b, :P], h_suf[b], vlm, aw.body, 1, s)
        assert rel_inf(hs[b], rs) <= TOL, (b, rel_inf(hs[b], rs))
        if P:
            assert rel_inf(hp[b, :P], rp) <= TOL
        else:
            np.testing.assert_array_equal(hp[b], emb[b])
