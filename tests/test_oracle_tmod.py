"""Pins of the oracle's time-modulated action expert (page "DM0.5: High-Performance Embodied
VLA and OpenDM Open Source Introduction", section 5.2: time_mlp_in / time_mlp_out and a time
modulator in every layer).

  * loop twin: the cached, time-modulated denoise equals the pure-Python joint stack (prefix and
    action tokens through every layer, modulated action expert) of oracle/naive.py;
  * identity modulation: a modulator whose output is the constant (gain - 1, 0, 1) for each norm
    reproduces the unmodulated expert without the additive time embedding;
  * zero gates: every sublayer drops out, so the velocity is the modulated head applied to
    action_in_proj alone;
  * the modulation depends on t: two times give different velocities, one time twice the same.
"""
from types import SimpleNamespace

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
    aw.tmod = tiny.time_mod(rng, L, Ha)
    return sh, vlm, aw, rng


def test_tmod_cached_denoise_matches_naive_joint_twin():
    sh, vlm, aw, rng = _model(40)
    P, S, A, N = 5, 3, 3, 3
    x_pre = rng.standard_normal((P, 16))
    x1 = rng.standard_normal((S, A))
    kc, vc, _ = O.prefill_kv(x_pre, vlm, sh)
    got = O.suffix_denoise(x1, aw, kc, vc, sh, N)
    ref = naive.denoise_joint_tmod(x1, aw, vlm, x_pre, sh, N)
    np.testing.assert_allclose(got, np.array(ref), rtol=0, atol=TOL)


def test_identity_modulation_is_the_plain_expert_without_time_embedding(monkeypatch):
    sh, vlm, aw, rng = _model(41)
    L, H = aw.body.w_qkv.shape[0], aw.w_in.shape[0]
    tm = aw.tmod
    tm.w_mod = np.zeros_like(tm.w_mod)
    tm.w_fmod = np.zeros_like(tm.w_fmod)
    for l in range(L):
        tm.b_mod[l] = np.concatenate([aw.body.attn_norm[l] - 1, np.zeros(H), np.ones(H),
                                      aw.body.mlp_norm[l] - 1, np.zeros(H), np.ones(H)])
    tm.b_fmod = np.concatenate([aw.final_norm - 1, np.zeros(H)])
    P, S, A = 6, 3, 3
    kc, vc, _ = O.prefill_kv(rng.standard_normal((P, 16)), vlm, sh)
    x = rng.standard_normal((S, A))
    got = [O.velocity_cached(x, t, aw, kc, vc, sh) for t in (1.0, 0.3)]
    plain = SimpleNamespace(**{k: v for k, v in vars(aw).items() if k != "tmod"})
    monkeypatch.setattr(OD, "time_embedding", lambda t, H, base: np.zeros(H))
    for g, t in zip(got, (1.0, 0.3)):
        np.testing.assert_allclose(g, O.velocity_cached(x, t, plain, kc, vc, sh), rtol=0, atol=1e-12)


def test_zero_gates_leave_only_the_head():
    sh, vlm, aw, rng = _model(42)
    L, H = aw.body.w_qkv.shape[0], aw.w_in.shape[0]
    tm = aw.tmod
    tm.w_mod[:, 2 * H:3 * H] = 0.0
    tm.w_mod[:, 5 * H:6 * H] = 0.0
    tm.b_mod[:, 2 * H:3 * H] = 0.0
    tm.b_mod[:, 5 * H:6 * H] = 0.0
    P, S, A = 4, 3, 3
    kc, vc, _ = O.prefill_kv(rng.standard_normal((P, 16)), vlm, sh)
    x = rng.standard_normal((S, A))
    t = 0.7
    got = O.velocity_cached(x, t, aw, kc, vc, sh)
    # by hand: embed, then the final modulated norm and the out-projection
    te = naive.time_emb(t, H, sh.time_base)
    z = [sum(tm.w_in[i][k] * te[k] for k in range(H)) + tm.b_in[i] for i in range(H)]
    c = [sum(tm.w_out[i][k] * z[k] / (1 + np.exp(-z[k])) for k in range(H)) + tm.b_out[i] for i in range(H)]
    sc = [ci / (1 + np.exp(-ci)) for ci in c]
    fm = [sum(tm.w_fmod[i][k] * sc[k] for k in range(H)) + tm.b_fmod[i] for i in range(2 * H)]
    for s in range(S):
        h = [sum(aw.w_in[i][a] * x[s][a] for a in range(A)) + aw.b_in[i] for i in range(H)]
        r = np.sqrt(sum(v * v for v in h) / H + sh.rms_eps)
        n = [h[i] / r * (1 + fm[i]) + fm[H + i] for i in range(H)]
        for a in range(A):
            want = sum(aw.w_out[a][i] * n[i] for i in range(H)) + aw.b_out[a]
            assert abs(got[s, a] - want) < 1e-12


def test_modulation_depends_on_time():
    sh, vlm, aw, rng = _model(43)
    kc, vc, _ = O.prefill_kv(rng.standard_normal((4, 16)), vlm, sh)
    x = rng.standard_normal((3, 3))
    v1 = O.velocity_cached(x, 1.0, aw, kc, vc, sh)
    assert np.array_equal(v1, O.velocity_cached(x, 1.0, aw, kc, vc, sh))
    assert not np.allclose(v1, O.velocity_cached(x, 0.4, aw, kc, vc, sh), atol=1e-6)


@pytest.mark.parametrize("what", ["gate on the wrong sublayer", "shift before the scale", "scale without the 1 +"])
def test_planted_mistakes_break_the_loop_twin(monkeypatch, what):
    """Each pin above must fail for a plausible mistake planted in the oracle."""
    sh, vlm, aw, rng = _model(44)
    P, S, A, N = 4, 3, 3, 2
    x_pre = rng.standard_normal((P, 16))
    x1 = rng.standard_normal((S, A))
    kc, vc, _ = O.prefill_kv(x_pre, vlm, sh)
    ref = np.array(naive.denoise_joint_tmod(x1, aw, vlm, x_pre, sh, N))
    real = OD.layer_modulation
    if what == "gate on the wrong sublayer":
        monkeypatch.setattr(OD, "layer_modulation", lambda c, tm, l: (lambda m: [m[0], m[1], m[5], m[3], m[4], m[2]])(real(c, tm, l)))
    elif what == "shift before the scale":
        monkeypatch.setattr(OD, "ada_rms_norm", lambda h, s, b, eps: (lambda x: (x + b) / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * (1 + s))(np.asarray(h, float)))
    else:
        monkeypatch.setattr(OD, "ada_rms_norm", lambda h, s, b, eps: O.rms_norm(h, s, eps) + b)
    got = O.suffix_denoise(x1, aw, kc, vc, sh, N)
    assert not np.allclose(got, ref, atol=1e-9), what
