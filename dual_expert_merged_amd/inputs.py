"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module draws random numbers and rounds them to the storage precision of a workload;
it holds none of the method's arithmetic. Both the oracle (in tests and the CPU baseline)
and the GPU path receive exactly the arrays produced here.

Recipe (every draw uses ``numpy.random.default_rng([config_id, stream, layer, tensor])``):
  * stream 0: VLM-expert weights, stream 1: action-expert weights, stream 2: prefix
    embeddings, stream 3: prefix KV cache, stream 4: noise x at t=1, stream 5: ragged prefix
    lengths, stream 6: action-token hidden states fed straight into a single merged layer.
  * linear weights N(0, 0.02); norm gains 1 + N(0, 0.02); in/out projection biases N(0, 0.02);
    embeddings, KV cache and noise N(0, 1).  Draws are float32 standard normals.
  * bf16 workloads round every tensor to bfloat16 with round-to-nearest-even; the arrays keep
    float32 storage holding those exactly representable values.  Norm gains, biases and the
    in/out projections are float32 tensors of the action head; they are rounded too so every
    input of a bf16 workload is a bf16 value.
  * ragged prefix lengths are integers drawn uniformly from [lo, hi] inclusive.
  * per-head QK-norm gains (QK-norm models, tensors 7 and 8 of each expert's stream): 1 + N(0, 0.1).
  * time-modulated action expert (stream 1, tensors 5..12): time MLP weights N(0, 0.05) and
    biases N(0, 0.02); modulator weights N(0, 0.005); modulator biases N(0, 0.02) for the scales
    and shifts and 1 + N(0, 0.02) for the gates; all rounded like the other weights.
  * a training batch (stream 7, ``make_train_batch``): the prefix hidden input of the merged
    layer N(0, 1) in the rows below each sample's prefix length (zero past it), the real action
    chunk a uniform in [-1, 1], the noise eps N(0, 1), one time t per sample uniform in [0, 1],
    and an action mask that keeps the first S_b time slices and the first A_b action dims of
    sample b, with S_b uniform in [S/2, S] and A_b uniform in [A/2, A] (the last sample keeps
    all of them); float32, rounded like the other inputs of the workload.
"""
from dataclasses import dataclass

import numpy as np

from .configs import BF16, F32, Workload

VLM_W, ACT_W, PREFIX, KV, NOISE, LENS, SUFFIX_H, TRAIN = range(8)
T_ATTN_NORM, T_QKV, T_O, T_MLP_NORM, T_GATE, T_UP, T_DOWN, T_Q_NORM, T_K_NORM = range(9)
T_W_IN, T_B_IN, T_FINAL_NORM, T_W_OUT, T_B_OUT = range(5)
T_TM_W_IN, T_TM_B_IN, T_TM_W_OUT, T_TM_B_OUT, T_TM_W_MOD, T_TM_B_MOD, T_TM_W_FMOD, T_TM_B_FMOD = range(5, 13)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((u + r) >> np.uint64(16)).astype(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if dtype == F32:
        return x
    if dtype == BF16:
        return bf16_values(bf16_bits(x))
    raise ValueError(dtype)


def _rng(cfg, stream, layer, tensor):
    return np.random.default_rng([cfg, stream, layer, tensor])


def _normal(cfg, stream, layer, tensor, shape, std=1.0, mean=0.0):
    x = _rng(cfg, stream, layer, tensor).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


@dataclass
class ExpertWeights:
    """All layers of one expert, stacked on a leading layer axis, PyTorch Linear layout [out][in]."""
    attn_norm: np.ndarray   # [L, H]
    w_qkv: np.ndarray       # [L, (Hq + 2 Hkv) D, H]: query heads, then key heads, then value heads
    w_o: np.ndarray         # [L, H, Hq D]
    mlp_norm: np.ndarray    # [L, H]
    w_gate: np.ndarray      # [L, F, H]
    w_up: np.ndarray        # [L, F, H]
    w_down: np.ndarray      # [L, H, F]
    q_norm: np.ndarray = None   # [L, D] per-head QK-norm gains (QK-norm models only)
    k_norm: np.ndarray = None   # [L, D]

    def layers(self, lo, hi):
        """Layers lo .. hi-1 (absent optional gains stay absent)."""
        return ExpertWeights(*(None if getattr(self, f) is None else getattr(self, f)[lo:hi]
                               for f in self.__dataclass_fields__))

    def layer(self, l):
        return self.layers(l, l + 1)

    @property
    def n_layers(self):
        return self.w_qkv.shape[0]


@dataclass
class TimeModWeights:
    """Time modulation of the action expert: time MLP and per-layer / final modulators."""
    w_in: np.ndarray        # [Ha, Ha] time_mlp_in
    b_in: np.ndarray        # [Ha]
    w_out: np.ndarray       # [Ha, Ha] time_mlp_out
    b_out: np.ndarray       # [Ha]
    w_mod: np.ndarray       # [L, 6 Ha, Ha]: attention scale, shift, gate, MLP scale, shift, gate
    b_mod: np.ndarray       # [L, 6 Ha]
    w_fmod: np.ndarray      # [2 Ha, Ha]: final-norm scale, shift
    b_fmod: np.ndarray      # [2 Ha]


@dataclass
class ActionWeights:
    body: ExpertWeights
    w_in: np.ndarray        # [Ha, A]
    b_in: np.ndarray        # [Ha]
    final_norm: np.ndarray  # [Ha]
    w_out: np.ndarray       # [A, Ha]
    b_out: np.ndarray       # [A]
    tmod: TimeModWeights = None


def make_expert(wl: Workload, stream: int, hidden: int, ffn: int, n_layers=None) -> ExpertWeights:
    s = wl.shape
    L = s.n_layers if n_layers is None else n_layers
    dt = s.dtype
    qkv = s.qkv_rows
    qd = s.n_q_heads * s.head_dim
    c = wl.config_id

    def stack(tensor, shape, **kw):
        return np.stack([round_to(_normal(c, stream, l, tensor, shape, **kw), dt) for l in range(L)])

    return ExpertWeights(
        attn_norm=stack(T_ATTN_NORM, (hidden,), std=0.02, mean=1.0),
        w_qkv=stack(T_QKV, (qkv, hidden), std=0.02),
        w_o=stack(T_O, (hidden, qd), std=0.02),
        mlp_norm=stack(T_MLP_NORM, (hidden,), std=0.02, mean=1.0),
        w_gate=stack(T_GATE, (ffn, hidden), std=0.02),
        w_up=stack(T_UP, (ffn, hidden), std=0.02),
        w_down=stack(T_DOWN, (hidden, ffn), std=0.02),
        q_norm=stack(T_Q_NORM, (s.head_dim,), std=0.1, mean=1.0) if s.qk_norm else None,
        k_norm=stack(T_K_NORM, (s.head_dim,), std=0.1, mean=1.0) if s.qk_norm else None,
    )


def make_vlm_weights(wl: Workload) -> ExpertWeights:
    return make_expert(wl, VLM_W, wl.shape.vlm_hidden, wl.shape.vlm_ffn)


def make_action_weights(wl: Workload) -> ActionWeights:
    s = wl.shape
    body = make_expert(wl, ACT_W, s.act_hidden, s.act_ffn)
    L, c, dt = s.n_layers, wl.config_id, s.dtype
    H, A = s.act_hidden, s.action_dim
    tmod = None
    if s.time_mod:
        # modulators: scale and shift biases N(0, 0.02), gate biases 1 + N(0, 0.02), weights
        # N(0, 0.005) (modulations of about +-0.1 at hidden 1024); the time MLP's weights N(0, 0.05)
        # so that c(t) varies visibly with t
        gate_mean = np.tile(np.repeat([0.0, 0.0, 1.0], H), 2).astype(np.float32)
        tmod = TimeModWeights(
            w_in=round_to(_normal(c, ACT_W, L, T_TM_W_IN, (H, H), std=0.05), dt),
            b_in=round_to(_normal(c, ACT_W, L, T_TM_B_IN, (H,), std=0.02), dt),
            w_out=round_to(_normal(c, ACT_W, L, T_TM_W_OUT, (H, H), std=0.05), dt),
            b_out=round_to(_normal(c, ACT_W, L, T_TM_B_OUT, (H,), std=0.02), dt),
            w_mod=np.stack([round_to(_normal(c, ACT_W, l, T_TM_W_MOD, (6 * H, H), std=0.005), dt) for l in range(L)]),
            b_mod=np.stack([round_to(_normal(c, ACT_W, l, T_TM_B_MOD, (6 * H,), std=0.02) + gate_mean, dt)
                            for l in range(L)]),
            w_fmod=round_to(_normal(c, ACT_W, L, T_TM_W_FMOD, (2 * H, H), std=0.005), dt),
            b_fmod=round_to(_normal(c, ACT_W, L, T_TM_B_FMOD, (2 * H,), std=0.02), dt),
        )
    return ActionWeights(
        body=body,
        w_in=round_to(_normal(c, ACT_W, L, T_W_IN, (H, A), std=0.02), dt),
        b_in=round_to(_normal(c, ACT_W, L, T_B_IN, (H,), std=0.02), dt),
        final_norm=round_to(_normal(c, ACT_W, L, T_FINAL_NORM, (H,), std=0.02, mean=1.0), dt),
        w_out=round_to(_normal(c, ACT_W, L, T_W_OUT, (A, H), std=0.02), dt),
        b_out=round_to(_normal(c, ACT_W, L, T_B_OUT, (A,), std=0.02), dt),
        tmod=tmod,
    )


def make_prefix_lens(wl: Workload) -> np.ndarray:
    if wl.ragged is None:
        return np.full(wl.batch, wl.prefix_len, dtype=np.int32)
    lo, hi = wl.ragged
    lens = _rng(wl.config_id, LENS, 0, 0).integers(lo, hi + 1, size=wl.batch)
    assert lens.max() <= wl.prefix_len
    return lens.astype(np.int32)


def make_prefix_embeds(wl: Workload) -> np.ndarray:
    """[B, P_cap, Hv]; rows at or past a sample's prefix length are zero padding."""
    s = wl.shape
    lens = make_prefix_lens(wl)
    out = np.zeros((wl.batch, wl.prefix_len, s.vlm_hidden), dtype=np.float32)
    for b in range(wl.batch):
        out[b, :lens[b]] = round_to(_normal(wl.config_id, PREFIX, b, 0, (lens[b], s.vlm_hidden)),
                                    s.dtype)
    return out


def make_kv_cache(wl: Workload):
    """Post-RoPE prefix K and V, [L, B, Hkv, P_cap, D] each; padding positions are zero."""
    s = wl.shape
    lens = make_prefix_lens(wl)
    shape = (s.n_layers, wl.batch, s.n_kv_heads, wl.prefix_len, s.head_dim)
    k = np.zeros(shape, dtype=np.float32)
    v = np.zeros(shape, dtype=np.float32)
    for l in range(s.n_layers):
        for b in range(wl.batch):
            P = lens[b]
            kv_shape = (s.n_kv_heads, P, s.head_dim)
            k[l, b, :, :P] = round_to(_normal(wl.config_id, KV, l, 2 * b, kv_shape), s.dtype)
            v[l, b, :, :P] = round_to(_normal(wl.config_id, KV, l, 2 * b + 1, kv_shape), s.dtype)
    return k, v


def make_noise(wl: Workload) -> np.ndarray:
    """x at t=1, [B, S, A] float32 (the action state is always float32)."""
    s = wl.shape
    return _normal(wl.config_id, NOISE, 0, 0, (wl.batch, s.chunk, s.action_dim))


def make_suffix_hidden(wl: Workload) -> np.ndarray:
    """Action-token hidden states [B, S, Ha] fed straight into a single merged layer."""
    s = wl.shape
    return round_to(_normal(wl.config_id, SUFFIX_H, 0, 0, (wl.batch, s.chunk, s.act_hidden)),
                    s.dtype)


@dataclass
class TrainBatch:
    """Inputs of one flow-matching training step on a merged layer."""
    h_pre: np.ndarray   # [B, P_cap, Hv] prefix hidden entering the layer (zero past lens[b])
    lens: np.ndarray    # [B] int32 prefix lengths
    a: np.ndarray       # [B, S, A] real action chunk
    eps: np.ndarray     # [B, S, A] noise
    t: np.ndarray       # [B] flow-matching time per sample
    mask: np.ndarray    # [B, S, A] 1 on valid (time slice, action dim), else 0


def make_train_batch(wl: Workload) -> TrainBatch:
    s = wl.shape
    B, S, A, P = wl.batch, s.chunk, s.action_dim, wl.prefix_len
    c = wl.config_id
    lens = make_prefix_lens(wl)
    h_pre = np.zeros((B, P, s.vlm_hidden), dtype=np.float32)
    for b in range(B):
        h_pre[b, :lens[b]] = round_to(_normal(c, TRAIN, b, 0, (lens[b], s.vlm_hidden)), s.dtype)
    a = round_to(_rng(c, TRAIN, 0, 1).uniform(-1.0, 1.0, (B, S, A)).astype(np.float32), s.dtype)
    eps = round_to(_normal(c, TRAIN, 0, 2, (B, S, A)), s.dtype)
    t = _rng(c, TRAIN, 0, 3).uniform(0.0, 1.0, B).astype(np.float32)
    lim = _rng(c, TRAIN, 0, 4)
    s_b = lim.integers(S // 2, S + 1, size=B)
    a_b = lim.integers(A // 2, A + 1, size=B)
    s_b[-1], a_b[-1] = S, A
    mask = np.zeros((B, S, A), dtype=np.float32)
    for b in range(B):
        mask[b, :s_b[b], :a_b[b]] = 1.0
    return TrainBatch(h_pre, lens, a, eps, t, mask)
