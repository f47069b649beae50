"""Oracle: one flow-matching training step on one dual-expert merged layer, float64 numpy,
forward and a hand-derived backward.

TEST INFRASTRUCTURE ONLY, like dm_oracle: tests, the smoke check and the benchmark's CPU leg
may use it; it shares no code with the HIP path.

Sources (the pages), cited by title and section:
  [FM]  "DM0.5: High-Performance Embodied VLA and OpenDM Open Source Introduction", section 5.3:
        training interpolates x_t = t*eps + (1-t)*a between the real chunk a and noise eps, the
        regression target is u_t = eps - a, and the loss is the mean squared error between the
        predicted velocity v(x_t, t | c) and u_t taken only over the valid action dimensions and
        time slices (an action mask).
  [KI]  "DM0 paper definition vs. Dexbotic code" (dregs-remover.com news 27019), section 1: the
        paper forbids the action expert's gradient from reaching the VLM (knowledge
        insulation), while the public code does not detach the prefix K/V, so there the action
        loss reaches the VLM through them.  Both graphs are offered: ``ki=True`` treats the
        prefix K/V as constants, ``ki=False`` back-propagates through them.
  [DM0], [SFX]: the merged layer and the action head, as in dm_oracle.

Readings where the pages are silent:
  - the step covers ONE merged layer l: action_in_proj + time embedding, layer l of both
    experts, the final norm and action_out_proj; one layer's prefix outputs never reach the
    action tokens (they read only the prefix K/V), so the prefix queries, the VLM's
    O-projection and MLP are not formed;
  - loss = sum(mask * (v - u)^2) / sum(mask) over the whole batch (the mean over the valid
    entries; 0 with no valid entry); mask holds 0 / 1 per (sample, time slice, action dim);
  - t is one time per sample in [0, 1]; the library draws no random numbers, so eps is an input;
  - gradients are those of this loss with respect to every parameter on its path: the action
    expert's layer-l tensors, the action head (w_in, b_in, final_norm, w_out, b_out) and, with
    ki=False, the VLM expert's layer-l attention-norm gain and K/V projection rows (its query
    rows get zero) plus the prefix hidden input h_pre.
"""
import numpy as np

from .dm_oracle import f64, gqa_attention, linear, rope, silu, time_embedding


def fm_interpolate(a, eps, t):
    """[FM]: x_t = t eps + (1 - t) a and the target velocity u_t = eps - a."""
    a, eps = f64(a), f64(eps)
    return t * eps + (1.0 - t) * a, eps - a


def _rstd(x, eps):
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _norm_bwd(x, g, dy, eps):
    """Gradients of y = x r g, r = (mean(x^2) + eps)^-1/2 (rows of x): (dx, dg)."""
    r = _rstd(x, eps)
    gd = dy * g
    H = x.shape[-1]
    dx = r * gd - x * r ** 3 * np.sum(gd * x, axis=-1, keepdims=True) / H
    return dx, np.sum(dy * x * r, axis=0)


def _dsilu(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def _forward(h_pre, x, t, vlm, aw, l, shape):
    """One sample's forward; returns (v, saved) with what the backward needs."""
    Hq, Hkv, D, eps = shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.rms_eps
    P, S = h_pre.shape[0], x.shape[0]
    sv = {"h_pre": h_pre, "x": x}
    # prefix K/V: the VLM expert's pre-norm and its key / value rows, RoPE on the keys
    n_p = h_pre * _rstd(h_pre, eps) * f64(vlm.attn_norm[l])
    kv_p = linear(n_p, f64(vlm.w_qkv[l])[Hq * D:])
    k_p, v_p = kv_p[:, :Hkv * D].reshape(P, Hkv, D), kv_p[:, Hkv * D:].reshape(P, Hkv, D)
    sv["n_p"] = n_p
    pos_p, pos_s = np.arange(P), P + np.arange(S)
    k_p = rope(k_p, pos_p, shape.rope_base)
    # action tokens: action_in_proj + time embedding, then the action expert's layer l
    body = aw.body
    h0 = linear(x, aw.w_in, aw.b_in) + time_embedding(t, aw.w_in.shape[0], shape.time_base)[None, :]
    n1 = h0 * _rstd(h0, eps) * f64(body.attn_norm[l])
    qkv = linear(n1, body.w_qkv[l])
    q = rope(qkv[:, :Hq * D].reshape(S, Hq, D), pos_s, shape.rope_base)
    k_s = rope(qkv[:, Hq * D:(Hq + Hkv) * D].reshape(S, Hkv, D), pos_s, shape.rope_base)
    v_s = qkv[:, (Hq + Hkv) * D:].reshape(S, Hkv, D)
    K, V = np.concatenate([k_p, k_s]), np.concatenate([v_p, v_s])
    o = gqa_attention(q, K, V, np.ones((S, P + S), dtype=bool))  # action rows see every key
    h1 = h0 + linear(o, body.w_o[l])
    n2 = h1 * _rstd(h1, eps) * f64(body.mlp_norm[l])
    gt, up = linear(n2, body.w_gate[l]), linear(n2, body.w_up[l])
    act = silu(gt) * up
    h2 = h1 + linear(act, body.w_down[l])
    nf = h2 * _rstd(h2, eps) * f64(aw.final_norm)
    v = linear(nf, aw.w_out, aw.b_out)
    sv.update(h0=h0, n1=n1, q=q, K=K, V=V, o=o, h1=h1, n2=n2, gt=gt, up=up, act=act, h2=h2, nf=nf,
              pos_p=pos_p, pos_s=pos_s)
    return v, sv


def velocity(h_pre, x, t, vlm, aw, l, shape):
    """v(x_t, t | c) of one sample after one merged layer (the training forward)."""
    return _forward(f64(h_pre), f64(x), float(t), vlm, aw, l, shape)[0]


def _backward(dv, sv, vlm, aw, l, shape, ki, g):
    """Accumulates one sample's parameter gradients into g; returns dh_pre (None with ki)."""
    Hq, Hkv, D, eps = shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.rms_eps
    body = aw.body
    S, P = sv["x"].shape[0], sv["h_pre"].shape[0]
    # head: v = nf W_out^T + b_out, nf = rmsnorm(h2) * final_norm
    g["w_out"] += dv.T @ sv["nf"]
    g["b_out"] += dv.sum(axis=0)
    dh2, dgf = _norm_bwd(sv["h2"], f64(aw.final_norm), dv @ f64(aw.w_out), eps)
    g["final_norm"] += dgf
    # MLP: h2 = h1 + (silu(gt) * up) W_down^T
    g["w_down"] += dh2.T @ sv["act"]
    dact = dh2 @ f64(body.w_down[l])
    dgt = dact * sv["up"] * _dsilu(sv["gt"])
    dup = dact * silu(sv["gt"])
    g["w_gate"] += dgt.T @ sv["n2"]
    g["w_up"] += dup.T @ sv["n2"]
    dn2 = dgt @ f64(body.w_gate[l]) + dup @ f64(body.w_up[l])
    dx2, dg2 = _norm_bwd(sv["h1"], f64(body.mlp_norm[l]), dn2, eps)
    g["mlp_norm"] += dg2
    dh1 = dh2 + dx2
    # O-projection: h1 = h0 + o W_o^T
    g["w_o"] += dh1.T @ sv["o"]
    do = (dh1 @ f64(body.w_o[l])).reshape(S, Hq, D)
    # attention of the action rows over [prefix ; action] keys, per query head
    q, K, V = sv["q"], sv["K"], sv["V"]
    grp = Hq // Hkv
    dq = np.zeros_like(q)
    dK, dV = np.zeros_like(K), np.zeros_like(V)
    for h in range(Hq):
        kv = h // grp
        s = q[:, h, :] @ K[:, kv, :].T / np.sqrt(D)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dp = do[:, h, :] @ V[:, kv, :].T
        dV[:, kv, :] += p.T @ do[:, h, :]
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True)) / np.sqrt(D)
        dq[:, h, :] = ds @ K[:, kv, :]
        dK[:, kv, :] += ds.T @ q[:, h, :]
    # RoPE is a rotation: its transpose rotates back (positions negated)
    dq = rope(dq, -sv["pos_s"], shape.rope_base)
    dk_s = rope(dK[P:], -sv["pos_s"], shape.rope_base)
    dqkv = np.concatenate([dq.reshape(S, Hq * D), dk_s.reshape(S, Hkv * D), dV[P:].reshape(S, Hkv * D)], axis=1)
    g["w_qkv"] += dqkv.T @ sv["n1"]
    dx1, dg1 = _norm_bwd(sv["h0"], f64(body.attn_norm[l]), dqkv @ f64(body.w_qkv[l]), eps)
    g["attn_norm"] += dg1
    dh0 = dh1 + dx1
    g["w_in"] += dh0.T @ sv["x"]
    g["b_in"] += dh0.sum(axis=0)
    if ki:
        return None
    # without knowledge insulation: through the prefix K/V into the VLM's layer l
    dk_p = rope(dK[:P], -sv["pos_p"], shape.rope_base)
    dkv = np.concatenate([dk_p.reshape(P, Hkv * D), dV[:P].reshape(P, Hkv * D)], axis=1)
    g["vlm_w_qkv"][Hq * D:] += dkv.T @ sv["n_p"]
    dh_pre, dgv = _norm_bwd(sv["h_pre"], f64(vlm.attn_norm[l]), dkv @ f64(vlm.w_qkv[l])[Hq * D:], eps)
    g["vlm_attn_norm"] += dgv
    return dh_pre


GRAD_NAMES = ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down",
              "w_in", "b_in", "final_norm", "w_out", "b_out", "vlm_attn_norm", "vlm_w_qkv", "h_pre")


def train_step(h_pre, lens, a, eps, t, mask, vlm, aw, l, shape, ki=True):
    """One training step on merged layer l for a batch: h_pre [B, P_cap, Hv] (rows >= lens[b]
    unused), a / eps / mask [B, S, A], t [B].  Returns (loss, grads) with grads a dict over
    GRAD_NAMES of float64 arrays shaped like the parameters of one layer (h_pre: like h_pre,
    zero in rows >= lens[b]; the VLM entries and h_pre are all zero with ki)."""
    body = aw.body
    B = a.shape[0]
    mask = f64(mask)
    n_valid = float(mask.sum())
    g = {"attn_norm": np.zeros(body.attn_norm.shape[1]), "w_qkv": np.zeros(body.w_qkv.shape[1:]),
         "w_o": np.zeros(body.w_o.shape[1:]), "mlp_norm": np.zeros(body.mlp_norm.shape[1]),
         "w_gate": np.zeros(body.w_gate.shape[1:]), "w_up": np.zeros(body.w_up.shape[1:]),
         "w_down": np.zeros(body.w_down.shape[1:]), "w_in": np.zeros(aw.w_in.shape),
         "b_in": np.zeros(aw.b_in.shape), "final_norm": np.zeros(aw.final_norm.shape),
         "w_out": np.zeros(aw.w_out.shape), "b_out": np.zeros(aw.b_out.shape),
         "vlm_attn_norm": np.zeros(vlm.attn_norm.shape[1]), "vlm_w_qkv": np.zeros(vlm.w_qkv.shape[1:]),
         "h_pre": np.zeros(np.shape(h_pre))}
    loss = 0.0
    for b in range(B):
        P = int(lens[b])
        x, u = fm_interpolate(a[b], eps[b], float(t[b]))
        v, sv = _forward(f64(h_pre[b, :P]), x, float(t[b]), vlm, aw, l, shape)
        err = v - u
        loss += float(np.sum(mask[b] * err * err))
        if n_valid > 0:
            dh_pre = _backward(2.0 * mask[b] * err / n_valid, sv, vlm, aw, l, shape, ki, g)
            if dh_pre is not None:
                g["h_pre"][b, :P] = dh_pre
    return (loss / n_valid if n_valid > 0 else 0.0), g
