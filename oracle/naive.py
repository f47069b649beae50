"""Oracle twin in pure-Python loops for tiny shapes.

TEST INFRASTRUCTURE ONLY.  Written independently of dm_oracle.py (scalar loops, an explicit
-inf mask matrix, explicit [out][in] weight indexing) so that a dropped term, a wrong sign or
index, or a transposed operand in either one shows up as a mismatch between the two.
It follows the same passages as dm_oracle.py: "DM0 paper definition vs. Dexbotic code",
section 1 (merged layer), and "DM0.5: High-Performance Embodied VLA and OpenDM Open Source
Introduction", sections 5.1-5.3 (prefix cache, action expert, Euler sampling).
All arguments are nested Python lists or numpy arrays indexed element by element.
"""
import math

NEG_INF = float("-inf")


def matvec(W, x, b=None):
    """y[n] = sum_k W[n][k] x[k] (+ b[n])."""
    out = []
    for n in range(len(W)):
        acc = 0.0
        for k in range(len(x)):
            acc += float(W[n][k]) * float(x[k])
        out.append(acc + (float(b[n]) if b is not None else 0.0))
    return out


def rmsnorm(x, g, eps):
    ss = 0.0
    for v in x:
        ss += float(v) * float(v)
    inv = 1.0 / math.sqrt(ss / len(x) + eps)
    return [float(x[i]) * inv * float(g[i]) for i in range(len(x))]


def rotate(vec, p, base):
    D = len(vec)
    half = D // 2
    out = [0.0] * D
    for i in range(half):
        th = base ** (-2.0 * i / D)
        c, s = math.cos(p * th), math.sin(p * th)
        out[i] = vec[i] * c - vec[i + half] * s
        out[i + half] = vec[i + half] * c + vec[i] * s
    return out


def heads(row, n, D):
    return [row[j * D:(j + 1) * D] for j in range(n)]


def qkv_token(hrow, W, l, pos, sh):
    """Per-token pre-norm, Q/K/V projections, RoPE on Q and K.  Returns per-head lists."""
    return qkv_normed(rmsnorm(hrow, W.attn_norm[l], sh.rms_eps), W, l, pos, sh)


def qkv_normed(n, W, l, pos, sh):
    """Q/K/V projections of an already normalised token, RoPE on Q and K (after the per-head
    RMSNorm of q and k when the expert has QK-norm gains)."""
    Hq, Hkv, D = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    y = matvec(W.w_qkv[l], n)
    qh, kh = heads(y[:Hq * D], Hq, D), heads(y[Hq * D:(Hq + Hkv) * D], Hkv, D)
    if getattr(W, "q_norm", None) is not None:
        qh = [rmsnorm(v, W.q_norm[l], sh.rms_eps) for v in qh]
        kh = [rmsnorm(v, W.k_norm[l], sh.rms_eps) for v in kh]
    q = [rotate(v, pos, sh.rope_base) for v in qh]
    k = [rotate(v, pos, sh.rope_base) for v in kh]
    v = heads(y[(Hq + Hkv) * D:], Hkv, D)
    return q, k, v


def attend(Q, K, V, mask, sh):
    """Q: per query token a list of Hq head vectors; K, V: per key token lists of Hkv head
    vectors; mask[i][j] True when key j is visible to query i.  Returns per query token the
    concatenation of its Hq head outputs."""
    Hq, Hkv, D = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    out = []
    for i in range(len(Q)):
        row = []
        for h in range(Hq):
            kvh = (h * Hkv) // Hq
            sc = []
            for j in range(len(K)):
                if mask[i][j]:
                    d = 0.0
                    for e in range(D):
                        d += Q[i][h][e] * K[j][kvh][e]
                    sc.append(d / math.sqrt(D))
                else:
                    sc.append(NEG_INF)
            mx = max(sc)
            ex = [math.exp(s - mx) if s != NEG_INF else 0.0 for s in sc]
            tot = sum(ex)
            for e in range(D):
                acc = 0.0
                for j in range(len(K)):
                    acc += ex[j] * V[j][kvh][e]
                row.append(acc / tot)
        out.append(row)
    return out


def finish_token(hrow, orow, W, l, sh):
    """Own O-projection + residual, then own pre-norm SwiGLU MLP + residual."""
    a = matvec(W.w_o[l], orow)
    h = [float(hrow[i]) + a[i] for i in range(len(hrow))]
    m = rmsnorm(h, W.mlp_norm[l], sh.rms_eps)
    g = matvec(W.w_gate[l], m)
    u = matvec(W.w_up[l], m)
    act = [g[i] / (1.0 + math.exp(-g[i])) * u[i] for i in range(len(g))]
    d = matvec(W.w_down[l], act)
    return [h[i] + d[i] for i in range(len(h))]


def merged_layer(h_pre, h_suf, vlm, act, l, sh):
    P, S = len(h_pre), len(h_suf)
    Q, K, V = [], [], []
    for j in range(P):
        q, k, v = qkv_token(h_pre[j], vlm, l, j, sh)
        Q.append(q); K.append(k); V.append(v)
    for s in range(S):
        q, k, v = qkv_token(h_suf[s], act, l, P + s, sh)
        Q.append(q); K.append(k); V.append(v)
    mask = [[(i >= P) or (j < P) for j in range(P + S)] for i in range(P + S)]
    O = attend(Q, K, V, mask, sh)
    new_pre = [finish_token(h_pre[j], O[j], vlm, l, sh) for j in range(P)]
    new_suf = [finish_token(h_suf[s], O[P + s], act, l, sh) for s in range(S)]
    kp = [K[j] for j in range(P)]
    vp = [V[j] for j in range(P)]
    return new_pre, new_suf, kp, vp


def time_emb(t, H, base):
    half = H // 2
    out = [0.0] * H
    for i in range(half):
        w = base ** (-2.0 * i / H)
        out[i] = math.sin(t * w)
        out[i + half] = math.cos(t * w)
    return out


def velocity_joint(x, t, aw, vlm, x_pre, sh):
    """Velocity of the whole joint stack for one sample (prefix + action tokens)."""
    H = len(aw.w_in)
    te = time_emb(t, H, sh.time_base)
    h_suf = []
    for s in range(len(x)):
        e = matvec(aw.w_in, x[s], aw.b_in)
        h_suf.append([e[i] + te[i] for i in range(H)])
    h_pre = [[float(v) for v in row] for row in x_pre]
    for l in range(len(vlm.w_qkv)):
        h_pre, h_suf, _, _ = merged_layer(h_pre, h_suf, vlm, aw.body, l, sh)
    return [matvec(aw.w_out, rmsnorm(r, aw.final_norm, sh.rms_eps), aw.b_out) for r in h_suf]


def denoise_joint(x1, aw, vlm, x_pre, sh, N):
    x = [[float(v) for v in row] for row in x1]
    for k in range(N):
        t = 1.0 - k / N
        v = velocity_joint(x, t, aw, vlm, x_pre, sh)
        x = [[x[s][a] - v[s][a] / N for a in range(len(x[s]))] for s in range(len(x))]
    return x


# ---------------------------------------------------------------------- time-modulated action expert
# Same page, section 5.2 (DM0.5): time_mlp_in / time_mlp_out give a modulation signal c(t); every
# layer's modulator turns silu(c) into scale, shift and gate for each of its two pre-norms.

def silu(v):
    return v / (1.0 + math.exp(-v))


def time_condition(t, tm, H, base):
    z = matvec(tm.w_in, time_emb(t, H, base), tm.b_in)
    return matvec(tm.w_out, [silu(v) for v in z], tm.b_out)


def modulation(c, W, b, parts):
    y = matvec(W, [silu(v) for v in c], b)
    H = len(c)
    return [y[j * H:(j + 1) * H] for j in range(parts)]


def ada_norm(x, scale, shift, eps):
    ss = 0.0
    for v in x:
        ss += float(v) * float(v)
    inv = 1.0 / math.sqrt(ss / len(x) + eps)
    return [float(x[i]) * inv * (1.0 + float(scale[i])) + float(shift[i]) for i in range(len(x))]


def finish_token_tmod(hrow, orow, W, l, sh, mods):
    """Gated O-projection residual, modulated pre-norm, gated SwiGLU MLP residual."""
    s1, b1, g1, s2, b2, g2 = mods
    a = matvec(W.w_o[l], orow)
    h = [float(hrow[i]) + float(g1[i]) * a[i] for i in range(len(hrow))]
    m = ada_norm(h, s2, b2, sh.rms_eps)
    g = matvec(W.w_gate[l], m)
    u = matvec(W.w_up[l], m)
    act = [g[i] / (1.0 + math.exp(-g[i])) * u[i] for i in range(len(g))]
    d = matvec(W.w_down[l], act)
    return [h[i] + float(g2[i]) * d[i] for i in range(len(h))]


def velocity_joint_tmod(x, t, aw, vlm, x_pre, sh):
    """Joint stack (prefix + action tokens) with the time-modulated action expert; the VLM
    expert is unchanged and no additive time embedding is used."""
    tm = aw.tmod
    H = len(aw.w_in)
    c = time_condition(t, tm, H, sh.time_base)
    h_suf = [matvec(aw.w_in, x[s], aw.b_in) for s in range(len(x))]
    h_pre = [[float(v) for v in row] for row in x_pre]
    P, S = len(h_pre), len(h_suf)
    for l in range(len(vlm.w_qkv)):
        mods = modulation(c, tm.w_mod[l], tm.b_mod[l], 6)
        Q, K, V = [], [], []
        for j in range(P):
            q, k, v = qkv_token(h_pre[j], vlm, l, j, sh)
            Q.append(q); K.append(k); V.append(v)
        for s in range(S):
            q, k, v = qkv_normed(ada_norm(h_suf[s], mods[0], mods[1], sh.rms_eps), aw.body, l, P + s, sh)
            Q.append(q); K.append(k); V.append(v)
        mask = [[(i >= P) or (j < P) for j in range(P + S)] for i in range(P + S)]
        O = attend(Q, K, V, mask, sh)
        h_pre = [finish_token(h_pre[j], O[j], vlm, l, sh) for j in range(P)]
        h_suf = [finish_token_tmod(h_suf[s], O[P + s], aw.body, l, sh, mods) for s in range(S)]
    sf, bf = modulation(c, tm.w_fmod, tm.b_fmod, 2)
    return [matvec(aw.w_out, ada_norm(r, sf, bf, sh.rms_eps), aw.b_out) for r in h_suf]


def denoise_joint_tmod(x1, aw, vlm, x_pre, sh, N):
    x = [[float(v) for v in row] for row in x1]
    for k in range(N):
        t = 1.0 - k / N
        v = velocity_joint_tmod(x, t, aw, vlm, x_pre, sh)
        x = [[x[s][a] - v[s][a] / N for a in range(len(x[s]))] for s in range(len(x))]
    return x
