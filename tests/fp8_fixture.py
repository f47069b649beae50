"""Seeded inputs of the FP8-MLP prefill checks (CPU discrimination test and GPU parity test).

A 2-layer small model (VLM hidden 256, FFN 768, 4 query / 2 KV heads of 32) over three ragged
prefixes.  Two changes to the seeded weights make FP8 rounding the dominant difference at
layer 1's K/V:
  * the gate, up and down weights are multiplied by 4 (a power of two, so every weight stays a
    bf16 value): the MLP's output then outweighs the residual and the E4M3 rounding of its
    operands moves layer 1's K/V by about 5 % of their RMS;
  * layer 0's O-projection is zero, so the residual entering layer 0's MLP is the bf16
    embedding itself: the MLP input is then the same bf16 tensor on every correct
    implementation, and the FP8 codes decided from it agree.
"""
from dataclasses import replace

import numpy as np

import oracle as O
from dual_expert_merged_amd import inputs
from dual_expert_merged_amd.configs import BF16, FP8, ModelShape, workload

MLP_SCALE = 4.0
LENS = (64, 41, 7)


def small_fp8_workload():
    shape = ModelShape(n_layers=2, vlm_hidden=256, act_hidden=128, vlm_ffn=768, act_ffn=384, n_q_heads=4,
                       n_kv_heads=2, head_dim=32, action_dim=32, chunk=50, dtype=BF16, vlm_mlp_dtype=FP8)
    return replace(workload(5), shape=shape, batch=len(LENS), prefix_len=max(LENS))


def fixture():
    """(workload, VLM weights, prefix embeddings [B, P_cap, H], lens)."""
    wl = small_fp8_workload()
    w = inputs.make_vlm_weights(wl)
    w_o = w.w_o.copy()
    w_o[0] = 0.0
    vlm = replace(w, w_gate=w.w_gate * MLP_SCALE, w_up=w.w_up * MLP_SCALE, w_down=w.w_down * MLP_SCALE, w_o=w_o)
    return wl, vlm, inputs.make_prefix_embeds(wl), np.array(LENS, dtype=np.int32)


def fp8_tuples(vlm):
    """The oracle's per-layer FP8 weights: (codes' values, scales) of gate, up and down."""
    out = []
    for l in range(vlm.w_qkv.shape[0]):
        gq, gs = O.fp8_quantize_rows(vlm.w_gate[l])
        uq, us = O.fp8_quantize_rows(vlm.w_up[l])
        dq, ds = O.fp8_quantize_rows(vlm.w_down[l])
        out.append((gq, gs, uq, us, dq, ds))
    return out


def distances(got, ref):
    """(mean |got - ref|, max |got - ref|)."""
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    return float(d.mean()), float(d.max())
