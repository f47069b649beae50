"""Pins of the oracle against what the pages and mathematics fix (no GPU, no HIP library).

Each test pins part of oracle/ to something other than itself: an independently written
pure-Python twin, closed forms, invariants, or a PyTorch CPU library routine.
Passages: "DM0 paper definition vs. Dexbotic code", section 1 (merged layer); "DM0.5:
High-Performance Embodied VLA and OpenDM Open Source Introduction", sections 5.1-5.3.
"""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import naive
from tests import tiny

TOL = 1e-12


def _tiny_model(seed=0, L=2, Hv=16, Ha=8, Fv=24, Fa=12, A=3, sh=None):
    sh = sh or tiny.shape()
    rng = np.random.default_rng(seed)
    vlm = tiny.expert(rng, L, Hv, Fv, sh)
    aw = tiny.action(rng, L, Ha, Fa, A, sh)
    return sh, vlm, aw, rng


# ---------------------------------------------------------------- P2: brute force twin

def test_naive_twin_merged_layer():
    sh, vlm, aw, rng = _tiny_model(1)
    P, S = 5, 3
    h_pre = rng.standard_normal((P, 16))
    h_suf = rng.standard_normal((S, 8))
    for l in range(2):
        a = O.merged_layer(h_pre, h_suf, vlm, aw.body, l, sh)
        b = naive.merged_layer(h_pre, h_suf, vlm, aw.body, l, sh)
        np.testing.assert_allclose(a[0], np.array(b[0]), rtol=0, atol=TOL)
        np.testing.assert_allclose(a[1], np.array(b[1]), rtol=0, atol=TOL)
        np.testing.assert_allclose(a[2], np.array(b[2]), rtol=0, atol=TOL)
        np.testing.assert_allclose(a[3], np.array(b[3]), rtol=0, atol=TOL)


def test_naive_twin_denoise_joint():
    sh, vlm, aw, rng = _tiny_model(2)
    P, S, A, N = 4, 3, 3, 3
    x_pre = rng.standard_normal((P, 16))
    x1 = rng.standard_normal((S, A))
    ref = naive.denoise_joint(x1, aw, vlm, x_pre, sh, N)
    got = O.euler_integrate(x1, lambda x, t: O.velocity_joint(x, t, aw, vlm, x_pre, sh), N)
    np.testing.assert_allclose(got, np.array(ref), rtol=0, atol=TOL)


# ---------------------------------------------------------------- P1: joint == cached

def test_joint_equals_prefill_plus_cached_suffix():
    """The merged stack over [prefix ; action] with the block mask equals prefill of the prefix
    alone followed by the action expert attending over the cached K/V."""
    sh, vlm, aw, rng = _tiny_model(3)
    P, S, A = 6, 4, 3
    x_pre = rng.standard_normal((P, 16))
    x = rng.standard_normal((S, A))
    kc, vc, h_last = O.prefill_kv(x_pre, vlm, sh)
    for t in (1.0, 0.55, 0.1):
        vj = O.velocity_joint(x, t, aw, vlm, x_pre, sh)
        vcached = O.velocity_cached(x, t, aw, kc, vc, sh)
        np.testing.assert_allclose(vcached, vj, rtol=0, atol=TOL)
    # the prefix rows of the joint stack never see the action tokens
    h_pre, h_suf = x_pre, rng.standard_normal((S, 8))
    for l in range(2):
        h_pre, h_suf, kp, vp = O.merged_layer(h_pre, h_suf, vlm, aw.body, l, sh)
        np.testing.assert_allclose(kp.transpose(1, 0, 2), kc[l], rtol=0, atol=TOL)
        np.testing.assert_allclose(vp.transpose(1, 0, 2), vc[l], rtol=0, atol=TOL)
    np.testing.assert_allclose(h_pre, h_last, rtol=0, atol=TOL)


def test_denoise_cached_matches_naive_joint():
    sh, vlm, aw, rng = _tiny_model(4)
    P, S, A, N = 5, 3, 3, 4
    x_pre = rng.standard_normal((P, 16))
    x1 = rng.standard_normal((S, A))
    kc, vc, _ = O.prefill_kv(x_pre, vlm, sh)
    got = O.suffix_denoise(x1, aw, kc, vc, sh, N)
    ref = naive.denoise_joint(x1, aw, vlm, x_pre, sh, N)
    np.testing.assert_allclose(got, np.array(ref), rtol=0, atol=TOL)


def test_batch_helper_slices_each_sample_to_its_length():
    sh, vlm, aw, rng = _tiny_model(5)
    L, Hkv, D, S, A = 2, 2, 4, 3, 3
    lens = np.array([3, 6, 5])
    Pcap = 8
    kc = rng.standard_normal((L, 3, Hkv, Pcap, D))
    vc = rng.standard_normal((L, 3, Hkv, Pcap, D))
    kc[:, 0, :, 3:] = 1e3  # padding must never be read
    x1 = rng.standard_normal((3, S, A))
    out = O.suffix_denoise_batch(x1, aw, kc, vc, lens, sh, 2)
    for b in range(3):
        ref = O.suffix_denoise(x1[b], aw, kc[:, b, :, :lens[b]], vc[:, b, :, :lens[b]], sh, 2)
        np.testing.assert_array_equal(out[b], ref)


# ---------------------------------------------------------------- P3, P4: attention closed forms

def test_softmax_rows_sum_to_one_v_ones():
    rng = np.random.default_rng(6)
    P, S, Hq, Hkv, D = 7, 3, 4, 2, 8
    q = rng.standard_normal((P + S, Hq, D)) * 3
    k = rng.standard_normal((P + S, Hkv, D)) * 3
    v = np.ones((P + S, Hkv, D))
    o = O.gqa_attention(q, k, v, O.merged_visibility(P, S))
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=TOL)


def test_zero_queries_average_visible_values():
    rng = np.random.default_rng(7)
    P, S, Hq, Hkv, D = 6, 4, 4, 2, 8
    q = np.zeros((P + S, Hq, D))
    k = rng.standard_normal((P + S, Hkv, D))
    v = rng.standard_normal((P + S, Hkv, D))
    o = O.gqa_attention(q, k, v, O.merged_visibility(P, S)).reshape(P + S, Hq, D)
    for h in range(Hq):
        kv = h // 2
        np.testing.assert_allclose(o[:P, h], np.broadcast_to(v[:P, kv].mean(0), (P, D)),
                                   rtol=0, atol=TOL)
        np.testing.assert_allclose(o[P:, h], np.broadcast_to(v[:, kv].mean(0), (S, D)),
                                   rtol=0, atol=TOL)


def test_block_mask_structure():
    vis = O.merged_visibility(3, 2)
    want = np.array([[1, 1, 1, 0, 0],
                     [1, 1, 1, 0, 0],
                     [1, 1, 1, 0, 0],
                     [1, 1, 1, 1, 1],
                     [1, 1, 1, 1, 1]], dtype=bool)
    np.testing.assert_array_equal(vis, want)


# ---------------------------------------------------------------- P5, P6: integrator

def test_constant_velocity_closed_form():
    sh, vlm, aw, rng = _tiny_model(8)
    c = rng.standard_normal(3)
    aw.w_out = np.zeros_like(aw.w_out)
    aw.b_out = c
    P, S, N = 4, 3, 7
    kc = rng.standard_normal((2, 2, P, 4))
    vc = rng.standard_normal((2, 2, P, 4))
    x1 = rng.standard_normal((S, 3))
    got = O.suffix_denoise(x1, aw, kc, vc, sh, N)
    np.testing.assert_allclose(got, x1 - c[None, :], rtol=0, atol=1e-13)


@pytest.mark.parametrize("N", [1, 2, 3, 10, 25])
def test_linear_path_is_integrated_exactly(N):
    """With v(x, t) = (x - a)/t the flow x_t = t eps + (1 - t) a is linear in t, so Euler from
    x_1 = eps with t_k = 1 - k/N and x <- x - v/N lands on a exactly."""
    rng = np.random.default_rng(9)
    a = rng.standard_normal((5, 3))
    eps = rng.standard_normal((5, 3))
    seen = []

    def vel(x, t):
        seen.append(t)
        np.testing.assert_allclose(x, t * eps + (1 - t) * a, rtol=0, atol=1e-12)
        return (x - a) / t

    got = O.euler_integrate(eps, vel, N)
    np.testing.assert_allclose(got, a, rtol=0, atol=1e-12)
    np.testing.assert_allclose(seen, [1 - k / N for k in range(N)], rtol=0, atol=0)


# ---------------------------------------------------------------- P7: GQA

def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(10)
    T, Hq, Hkv, D = 9, 8, 2, 4
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    vis = O.merged_visibility(6, 3)
    g = Hq // Hkv
    mha = O.gqa_attention(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), vis)
    np.testing.assert_allclose(O.gqa_attention(q, k, v, vis), mha, rtol=0, atol=TOL)


# ---------------------------------------------------------------- P8: RoPE

def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(11)
    u = rng.standard_normal((5, 3, 8))
    np.testing.assert_allclose(O.rope(u, np.zeros(5), 1e6), u, rtol=0, atol=0)
    r = O.rope(u, np.arange(5) * 37 + 3, 1e6)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(u, axis=-1),
                               rtol=0, atol=TOL)


def test_rope_pair_is_planar_rotation():
    """For each i the pair (u_i, u_{i+D/2}) is rotated by angle p * base^(-2i/D)."""
    rng = np.random.default_rng(12)
    D, base, p = 8, 1e6, 13
    u = rng.standard_normal((1, 1, D))
    r = O.rope(u, np.array([p]), base)[0, 0]
    for i in range(D // 2):
        ang = p * base ** (-2 * i / D)
        rot = np.array([[np.cos(ang), -np.sin(ang)], [np.sin(ang), np.cos(ang)]])
        want = rot @ np.array([u[0, 0, i], u[0, 0, i + D // 2]])
        np.testing.assert_allclose([r[i], r[i + D // 2]], want, rtol=0, atol=TOL)


def test_rope_relative_position_shift_invariance():
    rng = np.random.default_rng(13)
    T, Hq, Hkv, D = 7, 4, 2, 8
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    vis = O.merged_visibility(4, 3)
    pos = np.arange(T)
    ref = O.gqa_attention(O.rope(q, pos, 1e6), O.rope(k, pos, 1e6), v, vis)
    for c in (1, 50, 777):
        got = O.gqa_attention(O.rope(q, pos + c, 1e6), O.rope(k, pos + c, 1e6), v, vis)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)


# ---------------------------------------------------------------- P9: library cross-check

def _torch_layer(x, W, l, sh, mask, pos):
    """A standard pre-norm GQA transformer layer built from PyTorch CPU library routines."""
    F = torch.nn.functional
    t = lambda a: torch.as_tensor(np.asarray(a), dtype=torch.float64)
    x = t(x)
    Hq, Hkv, D = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    T = x.shape[0]
    n = F.rms_norm(x, (x.shape[1],), weight=t(W.attn_norm[l]), eps=sh.rms_eps)
    y = F.linear(n, t(W.w_qkv[l]))
    q = y[:, :Hq * D].reshape(T, Hq, D)
    k = y[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D)
    v = y[:, (Hq + Hkv) * D:].reshape(T, Hkv, D)
    inv = sh.rope_base ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
    rot = torch.polar(torch.ones(T, D // 2, dtype=torch.float64),
                      torch.as_tensor(pos, dtype=torch.float64)[:, None] * inv[None, :])

    def rope(u):  # the pair (u_i, u_{i+D/2}) as one complex number, times e^{i p theta}
        z = torch.complex(u[..., :D // 2], u[..., D // 2:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], dim=-1)

    q, k = rope(q), rope(k)
    o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                       v.transpose(0, 1)[None], attn_mask=torch.as_tensor(mask),
                                       enable_gqa=True)
    o = o[0].transpose(0, 1).reshape(T, Hq * D)
    h = x + F.linear(o, t(W.w_o[l]))
    m = F.rms_norm(h, (h.shape[1],), weight=t(W.mlp_norm[l]), eps=sh.rms_eps)
    return (h + F.linear(F.silu(F.linear(m, t(W.w_gate[l]))) * F.linear(m, t(W.w_up[l])),
                         t(W.w_down[l]))).numpy()


@pytest.mark.parametrize("P,S", [(6, 3), (5, 0)])
def test_merged_layer_with_identical_experts_is_one_masked_layer(P, S):
    """Identical expert weights and widths: the merged layer is one ordinary pre-norm layer over
    the concatenated sequence under the block mask (S = 0: a plain bidirectional layer)."""
    sh = tiny.shape()
    rng = np.random.default_rng(14)
    W = tiny.expert(rng, 1, 16, 24, sh)
    x = rng.standard_normal((P + S, 16))
    ref = _torch_layer(x, W, 0, sh, O.merged_visibility(P, S), np.arange(P + S))
    hp, hs, _, _ = O.merged_layer(x[:P], x[P:], W, W, 0, sh)
    np.testing.assert_allclose(np.concatenate([hp, hs]), ref, rtol=0, atol=1e-11)


def test_rmsnorm_closed_form():
    g = np.array([1.5, -0.5, 2.0, 1.0])
    eps = 1e-6
    for c in (3.0, -0.25, 1e-4):
        got = O.rms_norm(np.full((1, 4), c), g, eps)[0]
        np.testing.assert_allclose(got, np.sign(c) * g * abs(c) / np.sqrt(c * c + eps),
                                   rtol=1e-15, atol=0)


def test_time_embedding_closed_form():
    H = 8
    np.testing.assert_array_equal(O.time_embedding(0.0, H, 1e4), [0, 0, 0, 0, 1, 1, 1, 1])
    t = 0.7
    te = O.time_embedding(t, H, 1e4)
    np.testing.assert_allclose(te[0], np.sin(t), rtol=0, atol=0)
    np.testing.assert_allclose(te[4], np.cos(t), rtol=0, atol=0)
    np.testing.assert_allclose(te[3], np.sin(t * 1e4 ** (-6 / 8)), rtol=0, atol=0)
    np.testing.assert_allclose(te[:4] ** 2 + te[4:] ** 2, 1.0, rtol=0, atol=1e-15)


def test_suffix_embed_and_head_by_hand():
    sh, vlm, aw, rng = _tiny_model(15)
    x = rng.standard_normal((2, 3))
    h = O.suffix_embed(x, 0.0, aw, sh)
    for s in range(2):
        for i in range(8):
            want = sum(aw.w_in[i, a] * x[s, a] for a in range(3)) + aw.b_in[i] + (1.0 if i >= 4 else 0.0)
            assert abs(h[s, i] - want) < TOL
    v = O.velocity_head(h, aw, sh)
    for s in range(2):
        r = np.sqrt(np.mean(h[s] ** 2) + sh.rms_eps)
        for a in range(3):
            want = sum(aw.w_out[a, i] * h[s, i] / r * aw.final_norm[i] for i in range(8)) + aw.b_out[a]
            assert abs(v[s, a] - want) < TOL


# ---------------------------------------------------------------- FP8 E4M3

def test_e4m3_matches_torch_cast_in_range():
    rng = np.random.default_rng(16)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.05, 1, 30, 150)])
    x = x[np.abs(x) <= 448].astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.e4m3_round(x), ref)


def test_e4m3_grid_saturation_and_ties():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    vals = codes.to(torch.float64).numpy()
    finite = vals[np.isfinite(vals)]
    np.testing.assert_array_equal(O.e4m3_round(finite), finite)       # every code is a fixed point
    assert O.e4m3_round(np.array([448.0]))[0] == 448.0
    assert O.e4m3_round(np.array([1e6, -500.0, 464.0]))[0:2].tolist() == [448.0, -448.0]
    assert O.e4m3_round(np.array([464.0]))[0] == 448.0                 # tie 448|480 -> even
    assert O.e4m3_round(np.array([2.0 ** -10]))[0] == 0.0              # tie 0|2^-9 -> even (0)
    assert O.e4m3_round(np.array([3 * 2.0 ** -10]))[0] == 2.0 ** -8    # tie 2^-9|2^-8 -> even
    assert O.e4m3_round(np.array([1.0625]))[0] == 1.0                   # tie 1|1.125 -> even
    assert O.e4m3_round(np.array([1.1875]))[0] == 1.25


def test_fp8_linear_is_exact_scaled_integer_product():
    rng = np.random.default_rng(17)
    a = rng.standard_normal((5, 64))
    w = rng.standard_normal((7, 64)) * 0.02
    wq, ws = O.fp8_quantize_rows(w)
    assert np.all(np.abs(wq).max(axis=1) == 448.0)
    assert np.all(np.abs(wq * ws[:, None] - w) <= np.abs(w) * 2 ** -4 + ws[:, None] * 2.0 ** -10)
    y = O.fp8_linear(a, wq, ws)
    aq, r = O.fp8_quantize_rows(a)
    for m in range(5):
        for n in range(7):
            want = sum(aq[m, k] * wq[n, k] for k in range(64)) * r[m] * ws[n]
            assert abs(y[m, n] - want) <= 1e-12 * abs(want) + 1e-15
    # quantisation error stays within the E4M3 half-step bound of the row scale
    np.testing.assert_allclose(y, a @ w.T, rtol=0, atol=0.2)
