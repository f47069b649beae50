"""Pins of the oracle's per-head QK-norm switch (page "DM0 paper definition vs. Dexbotic code",
section 1: the experts are Qwen3 stacks; Qwen3 attention RMS-normalises every query and key head
vector with a learned gain before RoPE).

  * loop twin: with QK-norm gains on both experts, the cached denoise equals the pure-Python
    joint stack of oracle/naive.py (which normalises each head vector in scalar loops);
  * zero query gain: every query head is 0, so the attention averages the visible value rows;
  * scale invariance: scaling the query and key weight rows by 2^k leaves the output unchanged up
    to the eps term of the norm;
  * a planted mistake (norm after RoPE instead of before) breaks the loop twin.
"""
import numpy as np
import pytest

import oracle as O
import oracle.dm_oracle as OD
from oracle import naive
from tests import tiny

TOL = 1e-12


def _model(seed, L=2, Hv=16, Ha=8, Fv=24, Fa=12, A=3):
    sh = tiny.shape()
    rng = np.random.default_rng(seed)
    vlm = tiny.expert(rng, L, Hv, Fv, sh)
    aw = tiny.action(rng, L, Ha, Fa, A, sh)
    for w in (vlm, aw.body):
        w.q_norm = 1.0 + 0.3 * rng.standard_normal((L, sh.head_dim))
        w.k_norm = 1.0 + 0.3 * rng.standard_normal((L, sh.head_dim))
    return sh, vlm, aw, rng


def test_qknorm_cached_denoise_matches_naive_joint_twin():
    sh, vlm, aw, rng = _model(50)
    P, S, A, N = 5, 3, 3, 3
    x_pre = rng.standard_normal((P, 16))
    x1 = rng.standard_normal((S, A))
    kc, vc, _ = O.prefill_kv(x_pre, vlm, sh)
    got = O.suffix_denoise(x1, aw, kc, vc, sh, N)
    ref = naive.denoise_joint(x1, aw, vlm, x_pre, sh, N)
    np.testing.assert_allclose(got, np.array(ref), rtol=0, atol=TOL)


def test_zero_query_gain_averages_visible_values():
    sh, vlm, aw, rng = _model(51)
    vlm.q_norm[0] = 0.0
    aw.body.q_norm[0] = 0.0
    P, S = 5, 3
    h_pre, h_suf = rng.standard_normal((P, 16)), rng.standard_normal((S, 8))
    qp, kp, vp = O.expert_qkv(h_pre, vlm, 0, sh, np.arange(P))
    qs, ks, vs = O.expert_qkv(h_suf, aw.body, 0, sh, P + np.arange(S))
    assert not np.any(qp) and not np.any(qs)
    o = O.gqa_attention(np.concatenate([qp, qs]), np.concatenate([kp, ks]), np.concatenate([vp, vs]),
                        O.merged_visibility(P, S))
    V = np.concatenate([vp, vs])
    g = sh.n_q_heads // sh.n_kv_heads
    for h in range(sh.n_q_heads):
        want_pre = V[:P, h // g].mean(axis=0)
        want_suf = V[:, h // g].mean(axis=0)
        np.testing.assert_allclose(o[:P].reshape(P, sh.n_q_heads, -1)[:, h], np.tile(want_pre, (P, 1)), atol=1e-12)
        np.testing.assert_allclose(o[P:].reshape(S, sh.n_q_heads, -1)[:, h], np.tile(want_suf, (S, 1)), atol=1e-12)


def test_query_key_row_scale_cancels():
    sh, vlm, aw, rng = _model(52)
    P, S, A = 5, 3, 3
    x_pre = rng.standard_normal((P, 16))
    x = rng.standard_normal((S, A))
    kc, vc, _ = O.prefill_kv(x_pre, vlm, sh)
    v1 = O.velocity_cached(x, 0.6, aw, kc, vc, sh)
    qk = (sh.n_q_heads + sh.n_kv_heads) * sh.head_dim
    aw.body.w_qkv = aw.body.w_qkv.copy()
    aw.body.w_qkv[:, :qk] *= 8.0
    v2 = O.velocity_cached(x, 0.6, aw, kc, vc, sh)
    np.testing.assert_allclose(v2, v1, rtol=0, atol=1e-6)
    assert not np.array_equal(v2, v1)  # only the eps term of the norm differs


def test_norm_after_rope_is_caught(monkeypatch):
    sh, vlm, aw, rng = _model(53)
    P, S, A, N = 4, 3, 3, 2
    x_pre = rng.standard_normal((P, 16))
    x1 = rng.standard_normal((S, A))
    ref = np.array(naive.denoise_joint(x1, aw, vlm, x_pre, sh, N))

    def wrong(n, w, l, shape, pos):
        T, Hq, Hkv, D = n.shape[0], shape.n_q_heads, shape.n_kv_heads, shape.head_dim
        qkv = O.linear(n, w.w_qkv[l])
        q = O.rope(qkv[:, :Hq * D].reshape(T, Hq, D), pos, shape.rope_base)
        k = O.rope(qkv[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D), pos, shape.rope_base)
        return (O.rms_norm(q, w.q_norm[l], shape.rms_eps), O.rms_norm(k, w.k_norm[l], shape.rms_eps),
                qkv[:, (Hq + Hkv) * D:].reshape(T, Hkv, D))

    monkeypatch.setattr(OD, "project_qkv", wrong)
    kc, vc, _ = O.prefill_kv(x_pre, vlm, sh)
    got = O.suffix_denoise(x1, aw, kc, vc, sh, N)
    assert not np.allclose(got, ref, atol=1e-9)
