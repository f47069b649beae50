"""CPU pins of the oracle's FP8 MLP (page "DM0.5: High-Performance Embodied VLA and OpenDM Open
Source Introduction", section 6.3: the prefix MLP's gate, up and down GEMMs in FP8 E4M3 with
scales and wide accumulation).

1. Exactness on the grid.  When the MLP input rows are E4M3 values times a power of two whose
   largest entry is 448 times that power, and the weights are E4M3 codes with power-of-two row
   scales, per-token quantisation of the input is lossless; the inputs below are built so the
   SwiGLU product is such a row too, and silu is the identity on every gate value met (each is 0
   or at least 448, where 1 + exp(-g) rounds to 1).  The FP8 MLP must then equal the plain
   float64 MLP exactly.  Two more hand-built rows fix the rounding of the SwiGLU product: a value
   234 times its token's scale (nearest E4M3 value 240; truncation gives 224) and a value just
   above the 224|240 tie whose bfloat16 rounding lands on the tie (the reading that codes are
   decided from the bf16 tensor the model holds: 224; from the float64 value: 240).
2. Planted mistakes.  A copy of the FP8 MLP with switchable mistakes reproduces the oracle with no
   switch set and misses the exact values with each one: silu on the unscaled gate accumulator,
   silu on the up branch, a neighbouring token's scale, the scale taken over the wrong axis, a
   wrong E4M3 maximum, no quantisation of the SwiGLU product, truncating instead of rounding,
   codes decided from float64 instead of bfloat16 values.
3. RMSNorm's 1/rms after the GEMM: quantising the gain-scaled residual and scaling the GEMM
   outputs by a power-of-two 1/rms equals quantising the normalised input, bit for bit.
4. The end-to-end bound separates FP8 from bf16.  On the FP8 fixture (MLP weights x 4, layer 0's
   O-projection zero), a CPU emulation of a correct FP8 MLP in the kernels' precision (float32
   sums, bfloat16 stored tensors, h * gain as the quantised operand) lands within a third of the
   FP8-oracle-vs-bf16-oracle distance of layer 1's K/V; the same emulation with a bf16 MLP does
   not.
"""
import numpy as np
import pytest
import torch

import oracle as O
from tests import fp8_fixture as fx

E4 = 448.0


def p2(e):
    return np.exp2(np.asarray(e, dtype=np.float64))


# ---------------------------------------------------------------- bfloat16 rounding

def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(31)
    x = np.concatenate([rng.standard_normal(100000) * s for s in (1e-6, 1e-2, 1.0, 1e3, 1e7)]).astype(np.float32)
    # exact ties: 9 significant bits with the last one set
    ties = (np.arange(1, 2000, dtype=np.float32) * 2 + 1) * np.float32(2.0 ** -9) + 256
    x = np.concatenate([x, ties, -ties, np.float32([0.0, 1.0, -2.5])])
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(O.bf16_round(x), ref)


# ---------------------------------------------------------------- exact on the E4M3 grid

def _weights(codes, exps):
    """(codes, power-of-two row scales, dequantised matrix)."""
    codes = np.asarray(codes, dtype=np.float64)
    s = p2(exps)
    return codes, s, codes * s[:, None]


def case_grid():
    """4 tokens, hidden 8, FFN 4: every SwiGLU entry is +-7 * 2^z, so every tensor is on the grid."""
    k = np.array([0, 3, -2, 5])                              # token scale exponents, neighbours differ
    c = np.zeros((4, 8))
    c[:, 0] = [2.0 ** -7, 2.0 ** -5, 0.0, 2.0 ** -8]            # feeds the gate
    c[:, 1] = [2.0 ** -3, -2.0 ** -6, 2.0, -2.0 ** -4]          # feeds up
    c[:, 2] = [E4, -E4, E4, -E4]                              # sets the token scale 2^k
    filler = [-0.01171875, 2.0 ** -9, 13.0, -96.0, 0.6875]    # E4M3 codes incl. two subnormals
    for t in range(4):
        c[t, 3:] = np.roll(filler, t)
    m = c * p2(k)[:, None]
    G = np.zeros((4, 8))
    G[:, 0] = [E4, 224.0, E4, 112.0]
    U = np.zeros((4, 8))
    U[:, 1] = [1.0, -0.5, 2.0, 0.25]
    Dn = np.array([[1, -1.5, 0.875, 3.25], [-6, 0.0625, 20, -0.3125], [0.013671875, 1, -1, 2.5],
                   [-0.75, 40, 0.5, -9], [2, 2, -0.125, 0.4375], [-28, 0.1875, 1.25, -1],
                   [0.625, -3.5, 7, 0.09375], [1.5, -0.02734375, -12, 5]])
    return m, _weights(G, [8, 10, 12, 9]), _weights(U, [0, -2, 3, 1]), _weights(Dn, [-3, 0, 2, -1, 4, 1, -2, 0])


def _plain_mlp_identity_silu(m, g, u, d):
    """float64 MLP where silu is the identity: gate values are 0 or so large that 1 + exp(-g) == 1."""
    gv, uv = m @ g[2].T, m @ u[2].T
    assert np.all((gv == 0) | (1.0 + np.exp(-gv) == 1.0)), "gate values must be 0 or make 1 + exp(-g) round to 1"
    act = gv * uv
    nz = act[np.any(act != 0, axis=1)]
    rows = np.max(np.abs(nz), axis=1, keepdims=True)
    assert np.all((nz == 0) | (np.abs(nz) >= rows * 2.0 ** -14)), "SwiGLU entries must stay in E4M3's normal range"
    return act @ d[2].T


def case_round_nearest():
    """One token: SwiGLU product (14976, 28672) = (234, 448) x 64 -> codes (240, 448)."""
    m = np.array([[1.0, 1.0, E4, 0.6875, -13.0, 2.0 ** -9, 96.0, -0.01171875]])
    G = np.zeros((2, 8)); G[0, 0], G[1, 0] = 1.125, E4                     # gate 72 and 28672
    U = np.zeros((2, 8)); U[0, 1], U[1, 1] = 1.625, 1.0                    # up 208 and 1
    Dn = np.array([[3.0, -0.5], [0.25, 1.75], [-10.0, 0.0546875]])
    want_act = np.array([[240.0 * 64, 28672.0]])
    return m, _weights(G, [6, 6]), _weights(U, [7, 0]), _weights(Dn, [0, -4, 2]), want_act


def case_bf16_tie():
    """One token: gate 29 + 2^-6, up 8: SwiGLU 232.125 (bf16: 232, the 224|240 tie -> 224)."""
    m = np.array([[1.0, 1.0, 2.0 ** -6, E4, -13.0, 0.6875, 2.0 ** -9, 96.0]])
    G = np.zeros((2, 8)); G[0, :3] = [28.0, 1.0, 1.0]; G[1, 0] = E4
    U = np.zeros((2, 8)); U[0, 0], U[1, 0] = 8.0, 1.0
    Dn = np.array([[1.0, -2.0], [0.375, 0.5], [-4.5, 1.0]])
    want_act = np.array([[224.0, 448.0]])
    return m, _weights(G, [0, 0]), _weights(U, [0, 0]), _weights(Dn, [1, -3, 0]), want_act


def _tuple(g, u, d):
    return (g[0], g[1], u[0], u[1], d[0], d[1])


def _cases():
    m, g, u, d = case_grid()
    yield "grid", m, _tuple(g, u, d), _plain_mlp_identity_silu(m, g, u, d)
    for name, (m, g, u, d, want_act) in (("round-nearest", case_round_nearest()), ("bf16-tie", case_bf16_tie())):
        yield name, m, _tuple(g, u, d), want_act @ d[2].T


def test_oracle_fp8_mlp_exact_on_grid():
    for name, m, t, want in _cases():
        got = O.mlp(m, None, 0, fp8=t)
        assert np.array_equal(got, want), (name, got, want)


def test_oracle_bf16_mlp_agrees_on_grid_case():
    m, g, u, d = case_grid()
    w = type("W", (), {"w_gate": g[2][None], "w_up": u[2][None], "w_down": d[2][None]})
    np.testing.assert_array_equal(O.mlp(m, w, 0), _plain_mlp_identity_silu(m, g, u, d))


def test_fp8_mlp_takes_rms_after_the_gemm_exactly_for_powers_of_two():
    """mlp_fp8(n, 1/rms) quantises n and scales the GEMM outputs; for a power-of-two 1/rms per
    token that equals quantising the normalised input itself, bit for bit (bf16 rounding, the
    per-token scale and the E4M3 codes are all invariant under power-of-two scaling)."""
    rng = np.random.default_rng(33)
    n = rng.standard_normal((6, 64)) * 3
    inv = p2(rng.integers(-6, 6, size=6))
    t = (O.e4m3_round(rng.standard_normal((40, 64)) * 50), p2(rng.integers(-12, -8, 40)),
         O.e4m3_round(rng.standard_normal((40, 64)) * 50), p2(rng.integers(-12, -8, 40)),
         O.e4m3_round(rng.standard_normal((64, 40)) * 50), p2(rng.integers(-12, -8, 64)))
    got = O.mlp_fp8(n, inv, t)
    want = O.mlp(inv[:, None] * n, None, 0, fp8=t)
    assert np.array_equal(got, want)
    # and it is not the same as forgetting the factor
    assert not np.allclose(O.mlp_fp8(n, np.ones(6), t), want)


# ---------------------------------------------------------------- planted mistakes

def _trunc_e4m3(x):
    a = np.abs(x)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
    step = np.exp2(e - 3)
    return np.sign(x) * np.minimum(np.floor(a / step) * step, E4)


def mlp_fp8_variant(m, t, *, silu_acc=False, silu_up=False, neighbour=False, col_scale=False, qmax=E4,
                    quant_act=True, trunc=False, bf16=True):
    """The FP8 MLP with one switchable mistake at a time (no switch: the oracle's arithmetic)."""
    gq, gs, uq, us, dq, ds = t

    def quant(a):
        a = O.bf16_round(a) if bf16 else np.asarray(a, np.float64)
        amax = np.max(np.abs(a), axis=0 if col_scale else 1)
        s = np.where(amax > 0, amax / qmax, 1.0)
        s = np.broadcast_to(s[None, :] if col_scale else s[:, None], a.shape)
        q = (_trunc_e4m3 if trunc else O.e4m3_round)(a / s)
        if neighbour:
            s = np.roll(s, 1, axis=0)
        return q, s

    def lin(a, wq, ws, quantise=True, acc_fn=None):
        if not quantise:
            return a @ (wq * ws[:, None]).T
        q, s = quant(a)
        if col_scale:   # a column scale cannot be pulled out of the sum: dequantise first
            return (q * s) @ (wq * ws[:, None]).T
        acc = q @ wq.T
        if acc_fn is not None:
            acc = acc_fn(acc)
        return acc * s[:, :1] * ws[None, :]

    g = lin(m, gq, gs, acc_fn=O.silu if silu_acc else None)
    u = lin(m, uq, us)
    if not silu_acc:
        g = g if silu_up else O.silu(g)
    if silu_up:
        u = O.silu(u)
    return lin(O.bf16_round(g * u) if bf16 else g * u, dq, ds, quantise=quant_act)


MISTAKES = {
    "silu on the unscaled gate accumulator": dict(silu_acc=True),
    "silu on the up branch": dict(silu_up=True),
    "previous token's scale": dict(neighbour=True),
    "scale per input column": dict(col_scale=True),
    "E4M3 maximum taken as 240": dict(qmax=240.0),
    "SwiGLU product not quantised": dict(quant_act=False),
    "truncating E4M3 rounding": dict(trunc=True),
    "codes decided from float64 values": dict(bf16=False),
}


def test_variant_without_mistakes_is_the_oracle():
    for name, m, t, want in _cases():
        assert np.array_equal(mlp_fp8_variant(m, t), want), name
        assert np.array_equal(mlp_fp8_variant(m, t), O.mlp(m, None, 0, fp8=t)), name


@pytest.mark.parametrize("mistake", list(MISTAKES))
def test_each_planted_mistake_misses_an_exact_value(mistake):
    missed = [name for name, m, t, want in _cases() if not np.array_equal(mlp_fp8_variant(m, t, **MISTAKES[mistake]), want)]
    assert missed, f"no case detects: {mistake}"


# ---------------------------------------------------------------- the end-to-end bound discriminates

def _b16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _rows32(x):
    amax = np.max(np.abs(x), axis=1)
    s = np.where(amax > 0, amax / np.float32(448), np.float32(1)).astype(np.float32)
    return O.e4m3_round((x / s[:, None]).astype(np.float32)).astype(np.float32), s


def _emulated_layer1_kv(emb, w, shape, fp8):
    """Layer 1's K/V in the kernels' precision: float32 arithmetic, bfloat16 stored tensors
    (normalised inputs, SwiGLU product, residual, K/V), FP8 or bf16 MLP.  Layer 0's O-projection
    is zero in the fixture, so its attention does not reach the residual."""
    f32 = np.float32
    h = emb.astype(f32)
    n = _b16(h * w.mlp_norm[0].astype(f32))                  # the GEMM operand: h * gain in bf16
    inv = (1 / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + f32(shape.rms_eps))).astype(f32)
    if fp8 is not None:
        gq, gs, uq, us, dq, ds = (a.astype(f32) for a in fp8)
        a, r = _rows32(n)
        g = (a @ gq.T) * r[:, None] * gs * inv
        u = (a @ uq.T) * r[:, None] * us * inv
        a2, r2 = _rows32(_b16(g / (1 + np.exp(-g)) * u))
        d = (a2 @ dq.T) * r2[:, None] * ds
    else:
        g, u = (n @ w.w_gate[0].T.astype(f32)) * inv, (n @ w.w_up[0].T.astype(f32)) * inv
        d = _b16(g / (1 + np.exp(-g)) * u) @ w.w_down[0].T.astype(f32)
    h1 = _b16(h + d)
    n1 = _b16(h1 / np.sqrt(np.mean(h1 * h1, axis=1, keepdims=True) + f32(shape.rms_eps)) * w.attn_norm[1].astype(f32))
    qkv = n1 @ w.w_qkv[1].T.astype(f32)
    P, Hq, Hkv, D = h.shape[0], shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    k = O.rope(qkv[:, Hq * D:(Hq + Hkv) * D].reshape(P, Hkv, D), np.arange(P), shape.rope_base)
    v = qkv[:, (Hq + Hkv) * D:].reshape(P, Hkv, D)
    return _b16(k.transpose(1, 0, 2)), _b16(v.transpose(1, 0, 2))


def test_fp8_bound_separates_fp8_from_bf16():
    wl, vlm, emb, lens = fx.fixture()
    t = fx.fp8_tuples(vlm)
    for b, P in enumerate(lens):
        e = emb[b, :P]
        k8, v8, _ = O.prefill_kv(e, vlm, wl.shape, fp8_mlp=t)
        k16, v16, _ = O.prefill_kv(e, vlm, wl.shape)
        ke, ve = _emulated_layer1_kv(e, vlm, wl.shape, t[0])
        kb, vb = _emulated_layer1_kv(e, vlm, wl.shape, None)
        for name, r8, r16, good, bad in (("K", k8[1], k16[1], ke, kb), ("V", v8[1], v16[1], ve, vb)):
            eff = fx.distances(r16, r8)
            ok, wrong = fx.distances(good, r8), fx.distances(bad, r8)
            rms = float(np.sqrt(np.mean(r8 * r8)))
            print(f"sample {b} {name}: FP8 effect mean/rms {eff[0] / rms:.3e}; emulated FP8 at "
                  f"{ok[0] / eff[0]:.3f} / {ok[1] / eff[1]:.3f} of it, emulated bf16 MLP at "
                  f"{wrong[0] / eff[0]:.3f} / {wrong[1] / eff[1]:.3f} (mean / max)")
            assert eff[0] > 10 * 2.0 ** -9 * rms, "FP8 rounding must dominate bf16 noise on the fixture"
            assert ok[0] <= eff[0] / 3 and ok[1] <= eff[1] / 3, (b, name, ok, eff)
            assert not (wrong[0] <= eff[0] / 3 and wrong[1] <= eff[1] / 3), (b, name, wrong, eff)
