"""CPU pins of the training-step oracle (oracle/train.py: one flow-matching step on one merged
layer, page "DM0.5: High-Performance Embodied VLA and OpenDM Open Source Introduction",
section 5.3, with the knowledge-insulation switch of page "DM0 paper definition vs. Dexbotic
code", section 1).

1. Every gradient equals torch.autograd's on a float64 forward written here from the same
   definitions (torch ops, not the oracle), with and without knowledge insulation.
2. Central finite differences of the oracle's own loss agree with its gradients.
3. Closed forms: x_t at t = 0 and 1, u_t; an empty mask gives loss 0 and zero gradients; with
   w_out = 0 the velocity is b_out, the loss is sum(mask (b_out - u)^2) / sum(mask) and every
   gradient but b_out's is zero.
4. The training forward's velocity equals the inference oracle's (merged_layer then
   velocity_head on the same tokens).
5. Knowledge insulation leaves the action gradients unchanged and zeroes the VLM ones.
A planted mistake (a sign flip in the oracle's RMSNorm backward) fails pin 1.
"""
import copy
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from oracle import train as T
from dual_expert_merged_amd import inputs
from dual_expert_merged_amd.configs import workload

L_IDX = 1


def _case(B=3, P=24):
    wl = dataclasses.replace(workload(1), batch=B, prefix_len=P, ragged=(1, P))
    vlm = inputs.make_vlm_weights(wl)
    aw = inputs.make_action_weights(wl)
    tb = inputs.make_train_batch(wl)
    return wl, vlm, aw, tb


def _torch_loss(wl, vlm, aw, tb, ki):
    """The loss as a float64 torch graph; returns (loss, dict of leaf tensors by gradient name)."""
    s = wl.shape
    Hq, Hkv, D, e = s.n_q_heads, s.n_kv_heads, s.head_dim, s.rms_eps
    t64 = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    body = aw.body
    P_ = {"attn_norm": t64(body.attn_norm[L_IDX]), "w_qkv": t64(body.w_qkv[L_IDX]), "w_o": t64(body.w_o[L_IDX]),
          "mlp_norm": t64(body.mlp_norm[L_IDX]), "w_gate": t64(body.w_gate[L_IDX]), "w_up": t64(body.w_up[L_IDX]),
          "w_down": t64(body.w_down[L_IDX]), "w_in": t64(aw.w_in), "b_in": t64(aw.b_in),
          "final_norm": t64(aw.final_norm), "w_out": t64(aw.w_out), "b_out": t64(aw.b_out),
          "vlm_attn_norm": t64(vlm.attn_norm[L_IDX]), "vlm_w_qkv": t64(vlm.w_qkv[L_IDX]), "h_pre": t64(tb.h_pre)}

    def rms(x, g):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + e) * g

    def rot(u, pos):  # rotate-half RoPE, u [T, heads, D]
        half = D // 2
        th = s.rope_base ** (-2.0 * torch.arange(half, dtype=torch.float64) / D)
        ang = torch.tensor(pos, dtype=torch.float64)[:, None] * th[None, :]
        c, sn = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
        u1, u2 = u[..., :half], u[..., half:]
        return torch.cat([u1 * c - u2 * sn, u2 * c + u1 * sn], dim=-1)

    Ha = aw.w_in.shape[0]
    total = torch.zeros((), dtype=torch.float64)
    for b in range(wl.batch):
        Pb = int(tb.lens[b])
        a, eps = torch.tensor(tb.a[b], dtype=torch.float64), torch.tensor(tb.eps[b], dtype=torch.float64)
        tt = float(tb.t[b])
        x, u = tt * eps + (1 - tt) * a, eps - a
        i = torch.arange(Ha // 2, dtype=torch.float64)
        w = s.time_base ** (-2.0 * i / Ha)
        tau = torch.cat([torch.sin(tt * w), torch.cos(tt * w)])
        h0 = x @ P_["w_in"].T + P_["b_in"] + tau
        S = x.shape[0]
        n_p = rms(P_["h_pre"][b, :Pb], P_["vlm_attn_norm"])
        kv = n_p @ P_["vlm_w_qkv"][Hq * D:].T
        k_p = rot(kv[:, :Hkv * D].reshape(Pb, Hkv, D), np.arange(Pb))
        v_p = kv[:, Hkv * D:].reshape(Pb, Hkv, D)
        if ki:
            k_p, v_p = k_p.detach(), v_p.detach()
        n1 = rms(h0, P_["attn_norm"])
        qkv = n1 @ P_["w_qkv"].T
        pos = Pb + np.arange(S)
        q = rot(qkv[:, :Hq * D].reshape(S, Hq, D), pos)
        k = rot(qkv[:, Hq * D:(Hq + Hkv) * D].reshape(S, Hkv, D), pos)
        v = qkv[:, (Hq + Hkv) * D:].reshape(S, Hkv, D)
        K, V = torch.cat([k_p, k]), torch.cat([v_p, v])
        heads = []
        for h in range(Hq):
            g = h // (Hq // Hkv)
            p = torch.softmax(q[:, h] @ K[:, g].T / np.sqrt(D), dim=-1)
            heads.append(p @ V[:, g])
        o = torch.cat(heads, dim=1)
        h1 = h0 + o @ P_["w_o"].T
        n2 = rms(h1, P_["mlp_norm"])
        gt = n2 @ P_["w_gate"].T
        h2 = h1 + (gt * torch.sigmoid(gt) * (n2 @ P_["w_up"].T)) @ P_["w_down"].T
        vel = rms(h2, P_["final_norm"]) @ P_["w_out"].T + P_["b_out"]
        m = torch.tensor(tb.mask[b], dtype=torch.float64)
        total = total + (m * (vel - u) ** 2).sum()
    return total / float(tb.mask.sum()), P_


def _rel(a, b):
    n = max(np.abs(b).max(), 1e-300)
    return float(np.abs(np.asarray(a) - np.asarray(b)).max() / n)


@pytest.mark.parametrize("ki", [True, False])
def test_gradients_match_autograd(ki):
    wl, vlm, aw, tb = _case()
    loss, g = T.train_step(tb.h_pre, tb.lens, tb.a, tb.eps, tb.t, tb.mask, vlm, aw, L_IDX, wl.shape, ki=ki)
    tl, leaves = _torch_loss(wl, vlm, aw, tb, ki)
    tl.backward()
    assert abs(loss - tl.item()) <= 1e-12 * abs(tl.item())
    for name in T.GRAD_NAMES:
        ref = leaves[name].grad
        ref = np.zeros(g[name].shape) if ref is None else ref.numpy()
        if ki and name in ("vlm_attn_norm", "vlm_w_qkv", "h_pre"):
            assert not np.any(g[name]) and not np.any(ref), name
            continue
        assert np.abs(ref).max() > 0, name
        assert _rel(g[name], ref) <= 1e-9, (name, _rel(g[name], ref))


def test_planted_norm_backward_sign_fails_the_autograd_pin(monkeypatch):
    wl, vlm, aw, tb = _case(B=1)
    good = T._norm_bwd

    def flipped(x, g, dy, eps):
        dx, dg = good(x, g, dy, eps)
        r = T._rstd(x, eps)
        return dx + 2 * x * r ** 3 * np.sum(dy * g * x, axis=-1, keepdims=True) / x.shape[-1], dg

    monkeypatch.setattr(T, "_norm_bwd", flipped)
    _, g = T.train_step(tb.h_pre, tb.lens, tb.a, tb.eps, tb.t, tb.mask, vlm, aw, L_IDX, wl.shape, ki=False)
    tl, leaves = _torch_loss(wl, vlm, aw, tb, False)
    tl.backward()
    assert _rel(g["w_in"], leaves["w_in"].grad.numpy()) > 1e-3


def _f64_copy(vlm, aw):
    cv = copy.deepcopy(vlm)
    ca = copy.deepcopy(aw)
    for obj in (cv, ca.body, ca):
        for f in dataclasses.fields(obj):
            v = getattr(obj, f.name)
            if isinstance(v, np.ndarray):
                setattr(obj, f.name, v.astype(np.float64))
    return cv, ca


def test_finite_differences():
    wl, vlm, aw, tb = _case(B=2, P=12)
    vlm, aw = _f64_copy(vlm, aw)
    h_pre = tb.h_pre.astype(np.float64)
    loss, g = T.train_step(h_pre, tb.lens, tb.a, tb.eps, tb.t, tb.mask, vlm, aw, L_IDX, wl.shape, ki=False)
    rng = np.random.default_rng(3)
    where = {"attn_norm": (aw.body.attn_norm, L_IDX), "w_qkv": (aw.body.w_qkv, L_IDX), "w_o": (aw.body.w_o, L_IDX),
             "mlp_norm": (aw.body.mlp_norm, L_IDX), "w_gate": (aw.body.w_gate, L_IDX), "w_up": (aw.body.w_up, L_IDX),
             "w_down": (aw.body.w_down, L_IDX), "w_in": (aw.w_in, None), "b_in": (aw.b_in, None),
             "final_norm": (aw.final_norm, None), "w_out": (aw.w_out, None), "b_out": (aw.b_out, None),
             "vlm_attn_norm": (vlm.attn_norm, L_IDX), "vlm_w_qkv": (vlm.w_qkv, L_IDX), "h_pre": (h_pre, None)}
    h = 1e-5
    for name, (arr, l) in where.items():
        view = arr[l] if l is not None else arr
        grad = g[name]
        # coordinates with a gradient: the largest one and two random ones (h_pre: valid rows)
        flat = [int(np.argmax(np.abs(grad)))] + [int(i) for i in rng.integers(0, grad.size, 2)]
        if name == "vlm_w_qkv":
            Hq, D = wl.shape.n_q_heads, wl.shape.head_dim
            flat[1:] = [int(i) for i in rng.integers(Hq * D * grad.shape[1], grad.size, 2)]
        if name == "h_pre":
            flat[1:] = [int(np.ravel_multi_index((0, i, j), grad.shape))
                        for i, j in zip(rng.integers(0, tb.lens[0], 2), rng.integers(0, grad.shape[2], 2))]
        for i in flat:
            idx = np.unravel_index(i, view.shape)
            old = view[idx]
            view[idx] = old + h
            lp, _ = T.train_step(h_pre, tb.lens, tb.a, tb.eps, tb.t, tb.mask, vlm, aw, L_IDX, wl.shape, ki=False)
            view[idx] = old - h
            lm, _ = T.train_step(h_pre, tb.lens, tb.a, tb.eps, tb.t, tb.mask, vlm, aw, L_IDX, wl.shape, ki=False)
            view[idx] = old
            fd = (lp - lm) / (2 * h)
            # truncation O(h^2) relative to the gradient's scale, plus the rounding noise of
            # two loss values divided by 2h (a few ulp of the loss each)
            noise = 8 * np.finfo(np.float64).eps * abs(loss) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * np.abs(grad).max() + noise, (name, idx, fd, grad[idx])


def test_interpolation_closed_forms():
    a = np.array([[0.5, -1.0]])
    eps = np.array([[2.0, 0.25]])
    x1, u = T.fm_interpolate(a, eps, 1.0)
    x0, _ = T.fm_interpolate(a, eps, 0.0)
    np.testing.assert_array_equal(x1, eps)
    np.testing.assert_array_equal(x0, a)
    np.testing.assert_array_equal(u, eps - a)
    xh, _ = T.fm_interpolate(a, eps, 0.25)
    np.testing.assert_allclose(xh, [[0.875, -0.6875]], rtol=0, atol=1e-15)


def test_empty_mask_and_zero_out_projection():
    wl, vlm, aw, tb = _case(B=2)
    empty = np.zeros_like(tb.mask)
    loss, g = T.train_step(tb.h_pre, tb.lens, tb.a, tb.eps, tb.t, empty, vlm, aw, L_IDX, wl.shape, ki=False)
    assert loss == 0.0 and all(not np.any(v) for v in g.values())
    aw0 = dataclasses.replace(aw, w_out=np.zeros_like(aw.w_out))
    loss, g = T.train_step(tb.h_pre, tb.lens, tb.a, tb.eps, tb.t, tb.mask, vlm, aw0, L_IDX, wl.shape, ki=False)
    u = tb.eps.astype(np.float64) - tb.a
    err = aw.b_out.astype(np.float64)[None, None, :] - u
    n = tb.mask.sum()
    assert abs(loss - np.sum(tb.mask * err ** 2) / n) <= 1e-13 * loss
    ref = np.sum(2 * tb.mask * err, axis=(0, 1)) / n
    assert np.abs(g["b_out"] - ref).max() <= 1e-13 * np.abs(ref).max()
    assert np.abs(g["w_out"]).max() > 0  # dW_out = dv^T nf still flows
    for name in T.GRAD_NAMES:
        if name not in ("b_out", "w_out"):
            assert not np.any(g[name]), name


def test_training_velocity_equals_the_inference_oracle():
    wl, vlm, aw, tb = _case(B=1)
    P = int(tb.lens[0])
    x, _ = T.fm_interpolate(tb.a[0], tb.eps[0], float(tb.t[0]))
    v = T.velocity(tb.h_pre[0, :P], x, float(tb.t[0]), vlm, aw, L_IDX, wl.shape)
    h_suf = O.suffix_embed(x, float(tb.t[0]), aw, wl.shape)
    _, h2, _, _ = O.merged_layer(tb.h_pre[0, :P], h_suf, vlm, aw.body, L_IDX, wl.shape)
    np.testing.assert_allclose(v, O.velocity_head(h2, aw, wl.shape), rtol=1e-12, atol=1e-14)


def test_knowledge_insulation_changes_only_the_vlm_side():
    wl, vlm, aw, tb = _case()
    l1, g1 = T.train_step(tb.h_pre, tb.lens, tb.a, tb.eps, tb.t, tb.mask, vlm, aw, L_IDX, wl.shape, ki=True)
    l0, g0 = T.train_step(tb.h_pre, tb.lens, tb.a, tb.eps, tb.t, tb.mask, vlm, aw, L_IDX, wl.shape, ki=False)
    assert l1 == l0
    for name in T.GRAD_NAMES:
        if name in ("vlm_attn_norm", "vlm_w_qkv", "h_pre"):
            assert not np.any(g1[name]) and np.abs(g0[name]).max() > 0, name
        else:
            np.testing.assert_array_equal(g1[name], g0[name])
    # the VLM's query rows never reach the loss in one layer; rows past each prefix get nothing
    Hq, D = wl.shape.n_q_heads, wl.shape.head_dim
    assert not np.any(g0["vlm_w_qkv"][:Hq * D])
    for b in range(wl.batch):
        assert not np.any(g0["h_pre"][b, tb.lens[b]:])
