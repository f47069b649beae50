"""GPU parity of the flow-matching training step on one merged layer (dm_train_merged_layer;
page "DM0.5: High-Performance Embodied VLA and OpenDM Open Source Introduction", section 5.3,
and the knowledge-insulation switch of page "DM0 paper definition vs. Dexbotic code",
section 1) against the float64 oracle (oracle/train.py) on the same seeded inputs.

The step computes in float32 throughout, so the bounds are float32 ones:
  - tiny fp32 model, B = 3 with prefix lengths 0, 17 and 24 (P_cap 24), layer 1, with and
    without knowledge insulation: the loss within 1e-5 relative, every gradient tensor within
    1e-4 of the oracle relative to that tensor's largest magnitude;
  - DM0-base shapes (one layer, bf16 weights widened exactly), B = 2 with prefixes 816 and 431
    and the benchmarked B = 1 with prefix 816, with and without knowledge insulation: the loss
    and every gradient within 1e-4 of the oracle relative to the tensor's largest magnitude,
    the bound stated for float32 paths (measured: at most 1.6e-6, from float32 sums over up to
    6528 rows and softmax rows of up to 866 keys);
  - an empty mask gives loss 0 and all-zero gradients; argument checks.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import train as T
from dual_expert_merged_amd import binding as bd
from dual_expert_merged_amd import inputs
from dual_expert_merged_amd.configs import workload
from tests.gpu_harness import dev_lens

pytestmark = pytest.mark.gpu


def _run(wl, vlm, aw, tb, layer, ki, mask=None):
    s = wl.shape
    ctx = bd.Context(s, 0)
    dvlm = bd.DeviceExpert(vlm, s.dtype)
    daw = bd.DeviceAction(aw, s.dtype)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    B, P_cap = tb.h_pre.shape[0], tb.h_pre.shape[1]
    shapes = {"attn_norm": aw.body.attn_norm.shape[1:], "w_qkv": aw.body.w_qkv.shape[1:], "w_o": aw.body.w_o.shape[1:],
              "mlp_norm": aw.body.mlp_norm.shape[1:], "w_gate": aw.body.w_gate.shape[1:], "w_up": aw.body.w_up.shape[1:],
              "w_down": aw.body.w_down.shape[1:], "w_in": aw.w_in.shape, "b_in": aw.b_in.shape,
              "final_norm": aw.final_norm.shape, "w_out": aw.w_out.shape, "b_out": aw.b_out.shape,
              "vlm_attn_norm": vlm.attn_norm.shape[1:], "vlm_w_qkv": vlm.w_qkv.shape[1:], "h_prefix": tb.h_pre.shape}
    grads = {n: torch.full(tuple(shp), float("nan"), dtype=torch.float32, device="cuda") for n, shp in shapes.items()}
    loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    ws = ctx.workspace(bd.OP_TRAIN, B, P_cap)
    ctx.train_merged_layer(dvlm, daw, layer, dev(tb.h_pre), dev_lens(tb.lens), dev(tb.a), dev(tb.eps), dev(tb.t),
                           dev(tb.mask if mask is None else mask), ki, loss, grads, ws)
    torch.cuda.synchronize()
    out = {n: g.cpu().numpy() for n, g in grads.items()}
    ctx.close()
    return float(loss.item()), out


def _compare(wl, vlm, aw, tb, layer, ki, tol_loss, tol):
    ref_loss, ref = T.train_step(tb.h_pre, tb.lens, tb.a, tb.eps, tb.t, tb.mask, vlm, aw, layer, wl.shape, ki=ki)
    loss, got = _run(wl, vlm, aw, tb, layer, ki)
    e = abs(loss - ref_loss) / abs(ref_loss)
    print(f"ki={ki}: loss {loss:.6e} (oracle {ref_loss:.6e}, rel err {e:.2e})", flush=True)
    assert e <= tol_loss
    for name in T.GRAD_NAMES:
        g = got["h_prefix" if name == "h_pre" else name]
        r = ref[name]
        assert np.isfinite(g).all(), name
        if not np.any(r):
            assert not np.any(g), name  # exact zeros (insulated VLM side, query rows, padding rows)
            continue
        err = float(np.abs(g - r).max() / np.abs(r).max())
        print(f"  {name:14s} max |g| {np.abs(r).max():.3e}  rel err {err:.2e}", flush=True)
        assert err <= tol, (name, err)


@pytest.mark.parametrize("ki", [False, True])
def test_train_step_tiny_fp32(ki):
    wl = dataclasses.replace(workload(1), batch=3, prefix_len=24, ragged=(1, 24))
    print(f"case: training step, tiny fp32, B=3 P_cap=24, layer 1, knowledge insulation {ki}", flush=True)
    vlm = inputs.make_vlm_weights(wl)
    aw = inputs.make_action_weights(wl)
    tb = inputs.make_train_batch(wl)
    tb.lens[:] = [0, 17, 24]  # an empty prefix, a ragged one and a full one
    tb.h_pre[0] = 0.0
    tb.h_pre[1, 17:] = 0.0
    _compare(wl, vlm, aw, tb, 1, ki, 1e-5, 1e-4)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("ki", [False, True])
@pytest.mark.parametrize("lens", [(816, 431), (816,)], ids=["B2", "B1"])
def test_train_step_dm0_base_one_layer_bf16(ki, lens):
    """B = 2 (816 / 431) and the benchmarked B = 1, P = 816, whose products split K differently
    (the prefix products four ways instead of two)."""
    wl = dataclasses.replace(workload(2), batch=len(lens))
    print(f"case: training step, DM0-base one layer (bf16 weights), B={len(lens)} prefixes {list(lens)}, "
          f"knowledge insulation {ki}", flush=True)
    vlm = inputs.make_vlm_weights(wl)
    aw = inputs.make_action_weights(wl)
    tb = inputs.make_train_batch(wl)
    tb.lens[:] = lens
    for b, n in enumerate(lens):
        tb.h_pre[b, n:] = 0.0
    _compare(wl, vlm, aw, tb, 0, ki, 1e-4, 1e-4)


@pytest.mark.timeout(600)
def test_train_step_results_ordered_on_the_callers_stream():
    """The step forks part of its work (the prefix K/V projection, the MLP and O weight gradients,
    the prefix backward) onto the context's side stream and joins it back: copies enqueued on the
    caller's stream right after the call see every gradient finished (each starts as NaN), two
    calls give the same bits, and both equal the values after a device-wide synchronisation."""
    wl = workload(2)
    print("case: training step, DM0-base one layer, B=1, P=816, read on the caller's (non-default) stream", flush=True)
    s = wl.shape
    vlm, aw, tb = inputs.make_vlm_weights(wl), inputs.make_action_weights(wl), inputs.make_train_batch(wl)
    ctx = bd.Context(s, 0)
    dvlm, daw = bd.DeviceExpert(vlm, s.dtype), bd.DeviceAction(aw, s.dtype)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    args = (dev(tb.h_pre), dev_lens(tb.lens), dev(tb.a), dev(tb.eps), dev(tb.t), dev(tb.mask))
    shapes = {"w_qkv": aw.body.w_qkv.shape[1:], "w_o": aw.body.w_o.shape[1:], "w_gate": aw.body.w_gate.shape[1:],
              "w_up": aw.body.w_up.shape[1:], "w_down": aw.body.w_down.shape[1:], "attn_norm": aw.body.attn_norm.shape[1:],
              "mlp_norm": aw.body.mlp_norm.shape[1:], "w_in": aw.w_in.shape, "b_in": aw.b_in.shape,
              "final_norm": aw.final_norm.shape, "w_out": aw.w_out.shape, "b_out": aw.b_out.shape,
              "vlm_attn_norm": vlm.attn_norm.shape[1:], "vlm_w_qkv": vlm.w_qkv.shape[1:], "h_prefix": tb.h_pre.shape}
    ws = ctx.workspace(bd.OP_TRAIN, 1, tb.h_pre.shape[1])
    st = torch.cuda.Stream()
    snaps = []
    for _ in range(2):
        grads = {n: torch.full(tuple(shp), float("nan"), dtype=torch.float32, device="cuda") for n, shp in shapes.items()}
        loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            ctx.train_merged_layer(dvlm, daw, 0, *args, False, loss, grads, ws, stream=st)
            snap = {n: g.clone() for n, g in grads.items()}  # same stream, right after the call
            snap["loss"] = loss.clone()
        st.synchronize()
        torch.cuda.synchronize()
        for n, t in snap.items():
            assert not torch.isnan(t).any(), n
            final = loss if n == "loss" else grads[n]
            assert torch.equal(t, final), n
        snaps.append({n: t.cpu() for n, t in snap.items()})
    for n in snaps[0]:
        assert torch.equal(snaps[0][n], snaps[1][n]), n
    ctx.close()
    print("training step: results complete on the caller's stream, two calls bitwise equal", flush=True)


def test_train_step_empty_mask_and_argument_checks():
    wl = dataclasses.replace(workload(1), batch=2, prefix_len=16, ragged=(1, 16))
    print("case: training step, empty mask and argument checks", flush=True)
    vlm = inputs.make_vlm_weights(wl)
    aw = inputs.make_action_weights(wl)
    tb = inputs.make_train_batch(wl)
    loss, got = _run(wl, vlm, aw, tb, 0, False, mask=np.zeros_like(tb.mask))
    assert loss == 0.0
    for name, g in got.items():
        assert not np.any(g), name
    s = wl.shape
    ctx = bd.Context(s, 0)
    dvlm, daw = bd.DeviceExpert(vlm, s.dtype), bd.DeviceAction(aw, s.dtype)
    z = lambda *shape: torch.zeros(shape, dtype=torch.float32, device="cuda")
    B, P_cap, S, A = 2, 16, s.chunk, s.action_dim
    args = (z(B, P_cap, s.vlm_hidden), dev_lens(tb.lens), z(B, S, A), z(B, S, A), z(B), z(B, S, A))
    ws = ctx.workspace(bd.OP_TRAIN, B, P_cap)
    grads = {"attn_norm": z(s.act_hidden), "w_qkv": z(s.qkv_rows, s.act_hidden),
             "w_o": z(s.act_hidden, s.n_q_heads * s.head_dim), "mlp_norm": z(s.act_hidden),
             "w_gate": z(s.act_ffn, s.act_hidden), "w_up": z(s.act_ffn, s.act_hidden),
             "w_down": z(s.act_hidden, s.act_ffn), "w_in": z(s.act_hidden, A), "b_in": z(s.act_hidden),
             "final_norm": z(s.act_hidden), "w_out": z(A, s.act_hidden), "b_out": z(A)}
    loss = z(1)
    with pytest.raises(bd.DMError) as e:  # no VLM gradients without knowledge insulation
        ctx.train_merged_layer(dvlm, daw, 0, *args, False, loss, grads, ws)
    assert e.value.status == bd.DM_ERR_INVALID_ARG
    with pytest.raises(bd.DMError) as e:
        ctx.train_merged_layer(dvlm, daw, s.n_layers, *args, True, loss, grads, ws)
    assert e.value.status == bd.DM_ERR_SHAPE
    ctx.train_merged_layer(dvlm, daw, 0, *args, True, loss, grads, ws)  # insulated: no VLM gradients needed
    torch.cuda.synchronize()
    ctx.close()
    ctx2 = bd.Context(dataclasses.replace(s, qk_norm=True), 0)
    with pytest.raises(bd.DMError) as e:
        ctx2.train_merged_layer(dvlm, daw, 0, *args, True, loss, grads, ctx2.workspace(bd.OP_TRAIN, B, P_cap))
    assert e.value.status == bd.DM_ERR_UNSUPPORTED
    ctx2.close()
