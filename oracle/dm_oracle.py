"""Oracle: the DM0-style dual-expert merged-attention path written out plainly in float64 numpy.

TEST INFRASTRUCTURE ONLY.  A slow, obviously correct CPU reference for the HIP library; only
tests, the smoke check and the benchmark's CPU-baseline leg may use it.  It shares no code with
the HIP path and imports nothing from the package.

Sources (the pages), cited by title and section:
  [DM0]   "DM0 paper definition vs. Dexbotic code" (dregs-remover.com news 27019), section 1,
          key architecture conclusion: per layer each expert makes its own Q/K/V, they are
          joined along the sequence axis for one attention and split back; each expert then
          applies its own O-projection, residual and MLP.  Shapes: 28-layer Qwen3 experts,
          hidden 2048 (VLM) and 1024 (action), 16 query heads, 8 KV heads, head dim 128,
          action dim 32, chunk 50.
  [PFX]   "DM0.5: High-Performance Embodied VLA and OpenDM Open Source Introduction",
          section 5.1 (prefix): the prefix is encoded once and its per-layer KV cache is reused
          by every later action-generation step.
  [SFX]   same page, section 5.2 (suffix): action_in_proj lifts the action chunk to the expert
          width, the expert attends to the prefix KV cache, action_out_proj maps back to the
          velocity field v(x_t, t | c).
  [FM]    same page, section 5.3 (flow matching): x_t = t*eps + (1-t)*a with target
          u_t = eps - a; inference starts from random x_1 and Euler-integrates the velocity over
          diffusion_steps (default 10) to the action chunk.
  [FP8]   same page, section 6.3: the prefix MLP gate/up/down GEMMs run in FP8 E4M3 with
          scales and wider accumulation.
  [TMOD]  same page, section 5.2 (DM0.5 action expert): time_mlp_in / time_mlp_out turn the
          flow-matching time into a modulation signal, and a time modulator in every layer tells
          the action expert where on the noisy trajectory it is.
Constants the pages leave open are fixed by the workload definitions (RMSNorm eps 1e-6, RoPE
base 1e6, FFN 6144/3072, block mask "prefix bidirectional, suffix sees prefix and suffix").
Readings taken where the pages are silent are marked "reading:" below.

Conventions: hidden states are [T, H]; weights use the [out, in] layout; per-head tensors are
[T, heads, D]; a KV cache for one sample is [L, Hkv, P, D].  ``shape`` is any object with the
attributes n_q_heads, n_kv_heads, head_dim, rms_eps, rope_base, time_base; expert weights are
any object with stacked per-layer arrays attn_norm, w_qkv, w_o, mlp_norm, w_gate, w_up, w_down.
"""
import numpy as np

E4M3_MAX = 448.0


def f64(x):
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------- primitives

def rms_norm(x, gain, eps):
    """Pre-norm of a Qwen3 block: x / sqrt(mean(x^2) + eps) * gain, over the last axis."""
    x = f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * f64(gain)


def linear(x, w, b=None):
    """y = x W^T (+ b) with W in the [out, in] layout."""
    y = f64(x) @ f64(w).T
    return y if b is None else y + f64(b)


def silu(z):
    return z / (1.0 + np.exp(-z))


def rope(u, pos, base):
    """Rotary position embedding, rotate-half pairing (i, i + D/2), theta_i = base^(-2i/D).

    reading: the pages only say the experts are Qwen3; Qwen3 uses this rotate-half form.
    u: [T, heads, D]; pos: [T] integer positions.  Applied to queries and keys only.
    """
    u = f64(u)
    D = u.shape[-1]
    half = D // 2
    i = np.arange(half, dtype=np.float64)
    theta = f64(base) ** (-2.0 * i / D)
    ang = f64(pos)[:, None] * theta[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    u1, u2 = u[..., :half], u[..., half:]
    return np.concatenate([u1 * c - u2 * s, u2 * c + u1 * s], axis=-1)


def gqa_attention(q, k, v, visible):
    """Grouped-query softmax attention, [DM0] section 1 (16 query heads over 8 KV heads).

    q: [Tq, Hq, D]; k, v: [Tk, Hkv, D]; visible: [Tq, Tk] bool.  Returns [Tq, Hq*D] with column
    index h*D + d.  reading: query head h reads KV head h // (Hq/Hkv) (contiguous groups);
    scores are scaled by 1/sqrt(D).
    """
    q, k, v = f64(q), f64(k), f64(v)
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    out = np.empty((Tq, Hq, D))
    for h in range(Hq):
        kv = h // g
        s = (q[:, h, :] @ k[:, kv, :].T) / np.sqrt(D)
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        out[:, h, :] = p @ v[:, kv, :]
    return out.reshape(Tq, Hq * D)


def merged_visibility(P, S):
    """Block mask of the merged sequence [prefix ; action]: prefix rows see the prefix
    (bidirectional), action rows see prefix and action rows (bidirectional among themselves)."""
    vis = np.zeros((P + S, P + S), dtype=bool)
    vis[:P, :P] = True
    vis[P:, :] = True
    return vis


# ----------------------------------------------------------------------------- FP8 E4M3

def e4m3_round(x):
    """Nearest OCP E4M3 (e4m3fn) value: 3 mantissa bits, exponent bias 7, smallest normal 2^-6,
    subnormal step 2^-9, largest finite 448; ties to even; magnitudes above 448 saturate."""
    x = f64(x)
    a = np.abs(x)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))      # a = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -6).astype(np.float64)  # binade exponent, subnormals use 2^-6
    step = np.exp2(e - 3.0)
    r = np.round(a / step) * step                  # numpy rounds half to even
    r = np.minimum(r, E4M3_MAX)
    return np.where(a > 0, np.sign(x) * r, 0.0)


def bf16_round(x):
    """Nearest bfloat16 value of each float64: 8 significant bits, ties to even.  Used where the
    FP8 branch quantises a tensor that a bf16 model holds (reading below); the values met there
    are far inside bfloat16's normal range, so subnormals and overflow are not handled."""
    m, e = np.frexp(f64(x))                        # x = m * 2^e, |m| in [0.5, 1)
    return np.ldexp(np.round(m * 256.0), e - 8)    # numpy rounds half to even


def fp8_quantize_rows(m):
    """Per-row symmetric scale s = max|row| / 448 (1 for an all-zero row) and the E4M3 codes'
    values row / s.  Used for weights (per output channel) and activations (per token)."""
    m = f64(m)
    amax = np.max(np.abs(m), axis=-1)
    s = np.where(amax > 0, amax / E4M3_MAX, 1.0)
    return e4m3_round(m / s[..., None]), s


def fp8_linear(a, wq, ws):
    """[FP8] y[m, n] = r_m * s_n * sum_k a_q[m, k] * w_q[n, k] with per-token dynamic activation
    scales r and per-output-channel weight scales s; the sum is exact in float64."""
    aq, r = fp8_quantize_rows(a)
    return (aq @ f64(wq).T) * r[:, None] * f64(ws)[None, :]


# ----------------------------------------------------------------------------- one expert

def expert_qkv(h, w, l, shape, pos):
    """[DM0] section 1: an expert's own pre-norm and Q/K/V projections, RoPE on Q and K."""
    return project_qkv(rms_norm(h, w.attn_norm[l], shape.rms_eps), w, l, shape, pos)


def project_qkv(n, w, l, shape, pos):
    """Q/K/V projections of the normalised tokens n, RoPE on Q and K.  Experts with per-head
    QK-norm gains (``q_norm``, ``k_norm`` [L, D], not None) normalise every query and key head
    vector first: [DM0] names Qwen3 experts, whose attention applies an RMSNorm over each head's
    D dims (one gain vector per layer shared by the heads, the layers' eps) before RoPE."""
    T = n.shape[0]
    Hq, Hkv, D = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    qkv = linear(n, w.w_qkv[l])
    q = qkv[:, :Hq * D].reshape(T, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].reshape(T, Hkv, D)
    if getattr(w, "q_norm", None) is not None:
        q = rms_norm(q, w.q_norm[l], shape.rms_eps)
        k = rms_norm(k, w.k_norm[l], shape.rms_eps)
    return rope(q, pos, shape.rope_base), rope(k, pos, shape.rope_base), v


def mlp(m, w, l, fp8=None):
    """SwiGLU MLP down(silu(gate m) * up m) of the normalised input m.  fp8: optional
    (wq_gate, s_gate, wq_up, s_up, wq_down, s_down) for layer l, runs the three GEMMs as in
    [FP8] (``mlp_fp8`` with m itself as the quantised operand)."""
    if fp8 is None:
        return linear(silu(linear(m, w.w_gate[l])) * linear(m, w.w_up[l]), w.w_down[l])
    return mlp_fp8(m, np.ones(f64(m).shape[0]), fp8)


def mlp_fp8(n, inv_rms, fp8):
    """[FP8] SwiGLU MLP of the normalised input m = inv_rms[:, None] * n with the three GEMMs on
    E4M3 codes: n is quantised per token for gate and up, and their outputs are scaled by
    inv_rms (a positive factor per token commutes with per-token quantisation, so in exact
    arithmetic this equals quantising m); the dequantised gate output goes through silu and
    multiplies the up output; that product is quantised per token for down.
    reading: the tensors quantised are those a bf16 model holds at those two points: the
    gain-scaled residual n = h * g, whose 1/rms is applied after the GEMM, and the SwiGLU
    product; each is rounded to bfloat16 before its scale and E4M3 codes are taken, so every
    code is decided from the value the model stores."""
    gq, gs, uq, us, dq, ds = fp8
    n16 = bf16_round(n)
    r = f64(inv_rms)[:, None]
    act = silu(r * fp8_linear(n16, gq, gs)) * (r * fp8_linear(n16, uq, us))
    return fp8_linear(bf16_round(act), dq, ds)


def expert_finish(h, o, w, l, shape, fp8=None):
    """[DM0] section 1: after the joint attention each expert applies its own O-projection and
    residual, then its own pre-norm SwiGLU MLP and residual."""
    h = f64(h) + linear(o, w.w_o[l])
    if fp8 is None:
        return h + mlp(rms_norm(h, w.mlp_norm[l], shape.rms_eps), w, l)
    inv_rms = 1.0 / np.sqrt(np.mean(h * h, axis=-1) + shape.rms_eps)
    return h + mlp_fp8(h * f64(w.mlp_norm[l]), inv_rms, fp8)


def merged_layer(h_pre, h_suf, vlm, act, l, shape):
    """One dual-expert merged-attention layer, [DM0] section 1.

    h_pre: [P, Hv] VLM-expert tokens, h_suf: [S, Ha] action tokens.  Prefix position j is j,
    action token s sits at P + s (reading: positions continue after the prefix).
    Returns (h_pre', h_suf', k_pre, v_pre) with the prefix's post-RoPE K/V [P, Hkv, D].
    """
    P, S = h_pre.shape[0], h_suf.shape[0]
    qp, kp, vp = expert_qkv(h_pre, vlm, l, shape, np.arange(P))
    qs, ks, vs = expert_qkv(h_suf, act, l, shape, P + np.arange(S))
    o = gqa_attention(np.concatenate([qp, qs]), np.concatenate([kp, ks]),
                      np.concatenate([vp, vs]), merged_visibility(P, S))
    return (expert_finish(h_pre, o[:P], vlm, l, shape),
            expert_finish(h_suf, o[P:], act, l, shape), kp, vp)


# ----------------------------------------------------------------------------- prefix / suffix

def prefill_kv(x_pre, vlm, shape, fp8_mlp=None):
    """[PFX]: run the VLM expert alone over the prefix (bidirectional) and keep every layer's
    post-RoPE K and V.  Returns (k_cache, v_cache) as [L, Hkv, P, D] and the final hidden.
    fp8_mlp: optional list over layers of the [FP8] tuples of ``mlp``."""
    h = f64(x_pre)
    P = h.shape[0]
    ks, vs = [], []
    for l in range(vlm.w_qkv.shape[0]):
        q, k, v = expert_qkv(h, vlm, l, shape, np.arange(P))
        ks.append(k.transpose(1, 0, 2))
        vs.append(v.transpose(1, 0, 2))
        o = gqa_attention(q, k, v, np.ones((P, P), dtype=bool))
        h = expert_finish(h, o, vlm, l, shape, None if fp8_mlp is None else fp8_mlp[l])
    return np.stack(ks), np.stack(vs), h


def time_embedding(t, H, base):
    """reading: additive sinusoidal time embedding of width H, tau_i = sin(t w_i) and
    tau_{i+H/2} = cos(t w_i) with w_i = base^(-2i/H), t in [0, 1] unscaled."""
    i = np.arange(H // 2, dtype=np.float64)
    w = f64(base) ** (-2.0 * i / H)
    return np.concatenate([np.sin(t * w), np.cos(t * w)])


def suffix_embed(x, t, aw, shape):
    """[SFX] action_in_proj (with bias) of the chunk plus the time embedding, broadcast over
    the S action tokens."""
    H = aw.w_in.shape[0]
    return linear(x, aw.w_in, aw.b_in) + time_embedding(t, H, shape.time_base)[None, :]


def velocity_head(h, aw, shape):
    """[SFX] action_out_proj: final RMSNorm (reading: Qwen3 stacks end with one) then the
    out-projection with bias, giving v(x_t, t | c) of shape [S, A]."""
    return linear(rms_norm(h, aw.final_norm, shape.rms_eps), aw.w_out, aw.b_out)


def velocity_cached(x, t, aw, k_cache, v_cache, shape):
    """v(x_t, t | c) for one sample with the prefix already encoded, [PFX] + [SFX].

    k_cache, v_cache: [L, Hkv, P, D] for this sample (P its own prefix length).  Every action
    layer attends over [cache(l) ; its own K/V]; action rows see all P + S keys.  Action weights
    with a ``tmod`` attribute that is not None take the time-modulated expert instead.
    """
    if getattr(aw, "tmod", None) is not None:
        return velocity_cached_tmod(x, t, aw, k_cache, v_cache, shape)
    S = x.shape[0]
    P = k_cache.shape[2]
    pos = P + np.arange(S)
    h = suffix_embed(x, t, aw, shape)
    body = aw.body
    for l in range(body.w_qkv.shape[0]):
        q, k, v = expert_qkv(h, body, l, shape, pos)
        K = np.concatenate([f64(k_cache[l]).transpose(1, 0, 2), k])
        V = np.concatenate([f64(v_cache[l]).transpose(1, 0, 2), v])
        o = gqa_attention(q, K, V, np.ones((S, P + S), dtype=bool))
        h = expert_finish(h, o, body, l, shape)
    return velocity_head(h, aw, shape)


# ----------------------------------------------------------------------------- time modulation

def time_condition(t, tm, H, base):
    """[TMOD] the modulation signal of flow time t: c = time_mlp_out(silu(time_mlp_in(tau(t)))).
    reading: tau is the sinusoidal embedding of ``time_embedding`` (width H), both MLP layers
    are H -> H linears with biases and SiLU between them."""
    return linear(silu(linear(time_embedding(t, H, base), tm.w_in, tm.b_in)), tm.w_out, tm.b_out)


def layer_modulation(c, tm, l):
    """[TMOD] layer l's time modulator.  reading: one linear map of silu(c) gives, for each of the
    layer's two pre-norms (attention, then MLP), a scale, a shift and a residual gate (6 H
    values, in that order)."""
    return np.split(linear(silu(c), tm.w_mod[l], tm.b_mod[l]), 6)


def final_modulation(c, tm):
    """[TMOD] reading: the norm before action_out_proj is modulated the same way (scale, shift)."""
    return np.split(linear(silu(c), tm.w_fmod, tm.b_fmod), 2)


def ada_rms_norm(h, scale, shift, eps):
    """reading: a time-modulated RMSNorm replaces the learned gain by the modulation:
    x / sqrt(mean(x^2) + eps) * (1 + scale) + shift."""
    x = f64(h)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * (1.0 + f64(scale)) + f64(shift)


def velocity_cached_tmod(x, t, aw, k_cache, v_cache, shape):
    """v(x_t, t | c) of the time-modulated action expert ([TMOD], [PFX] + [SFX]): action_in_proj
    without the additive time embedding (the modulation replaces it); in every layer the two
    pre-norms are modulated and each sublayer's output enters the residual times its gate,
    h += gate * sublayer(ada_rms_norm(h)); the final norm is modulated too."""
    S = x.shape[0]
    P = k_cache.shape[2]
    pos = P + np.arange(S)
    body, tm = aw.body, aw.tmod
    eps = shape.rms_eps
    c = time_condition(t, tm, aw.w_in.shape[0], shape.time_base)
    h = linear(x, aw.w_in, aw.b_in)
    for l in range(body.w_qkv.shape[0]):
        s1, b1, g1, s2, b2, g2 = layer_modulation(c, tm, l)
        q, k, v = project_qkv(ada_rms_norm(h, s1, b1, eps), body, l, shape, pos)
        K = np.concatenate([f64(k_cache[l]).transpose(1, 0, 2), k])
        V = np.concatenate([f64(v_cache[l]).transpose(1, 0, 2), v])
        o = gqa_attention(q, K, V, np.ones((S, P + S), dtype=bool))
        h = h + g1 * linear(o, body.w_o[l])
        h = h + g2 * mlp(ada_rms_norm(h, s2, b2, eps), body, l)
    sf, bf = final_modulation(c, tm)
    return linear(ada_rms_norm(h, sf, bf, eps), aw.w_out, aw.b_out)


def velocity_joint(x, t, aw, vlm, x_pre, shape):
    """v(x_t, t | c) computed the long way: the full stack of merged layers over
    [prefix ; action tokens] with the block mask, nothing cached."""
    h_pre = f64(x_pre)
    h_suf = suffix_embed(x, t, aw, shape)
    for l in range(vlm.w_qkv.shape[0]):
        h_pre, h_suf, _, _ = merged_layer(h_pre, h_suf, vlm, aw.body, l, shape)
    return velocity_head(h_suf, aw, shape)


def euler_integrate(x1, velocity, N):
    """[FM] inference: start from x at t = 1 and take N explicit Euler steps to t = 0.

    reading: the printed update x_{t-dt} = x_t + v dt is garbled in sign; with u = eps - a and
    noise at t = 1 the step towards data is x <- x - v / N, with v evaluated at
    t_k = 1 - k/N (computed, not accumulated) for k = 0 .. N-1.
    """
    x = f64(x1)
    for k in range(N):
        t = 1.0 - k / N
        x = x - velocity(x, t) / N
    return x


def suffix_denoise(x1, aw, k_cache, v_cache, shape, N):
    """One sample's action chunk: Euler over v(x, t | c) with the cached prefix."""
    return euler_integrate(x1, lambda x, t: velocity_cached(x, t, aw, k_cache, v_cache, shape), N)


def suffix_denoise_batch(x1, aw, k_cache, v_cache, lens, shape, N, samples=None):
    """x1 [B, S, A]; caches [L, B, Hkv, P_cap, D]; lens [B].  Samples are independent; returns
    {b: chunk} for the requested samples (all by default)."""
    samples = range(x1.shape[0]) if samples is None else samples
    return {b: suffix_denoise(x1[b], aw, k_cache[:, b, :, :lens[b]], v_cache[:, b, :, :lens[b]],
                              shape, N) for b in samples}
