"""Tiny seeded shapes and weights for the oracle's self-tests (numpy only)."""
from types import SimpleNamespace

import numpy as np


def shape(Hq=4, Hkv=2, D=4, eps=1e-6, rope_base=1e6, time_base=1e4):
    return SimpleNamespace(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, rms_eps=eps,
                           rope_base=rope_base, time_base=time_base)


def expert(rng, L, H, F, sh, std=0.3):
    qkv = (sh.n_q_heads + 2 * sh.n_kv_heads) * sh.head_dim
    qd = sh.n_q_heads * sh.head_dim
    return SimpleNamespace(
        attn_norm=1.0 + 0.1 * rng.standard_normal((L, H)),
        w_qkv=std * rng.standard_normal((L, qkv, H)),
        w_o=std * rng.standard_normal((L, H, qd)),
        mlp_norm=1.0 + 0.1 * rng.standard_normal((L, H)),
        w_gate=std * rng.standard_normal((L, F, H)),
        w_up=std * rng.standard_normal((L, F, H)),
        w_down=std * rng.standard_normal((L, H, F)),
    )


def action(rng, L, H, F, A, sh, std=0.3):
    return SimpleNamespace(
        body=expert(rng, L, H, F, sh, std),
        w_in=std * rng.standard_normal((H, A)),
        b_in=std * rng.standard_normal(H),
        final_norm=1.0 + 0.1 * rng.standard_normal(H),
        w_out=std * rng.standard_normal((A, H)),
        b_out=std * rng.standard_normal(A),
    )


def time_mod(rng, L, H, std=0.3):
    """Time-modulation weights: time MLP (H -> H -> H) and per-layer / final modulators."""
    return SimpleNamespace(
        w_in=std * rng.standard_normal((H, H)), b_in=std * rng.standard_normal(H),
        w_out=std * rng.standard_normal((H, H)), b_out=std * rng.standard_normal(H),
        w_mod=std * rng.standard_normal((L, 6 * H, H)), b_mod=std * rng.standard_normal((L, 6 * H)),
        w_fmod=std * rng.standard_normal((2 * H, H)), b_fmod=std * rng.standard_normal(2 * H),
    )
