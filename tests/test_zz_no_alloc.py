"""dm_suffix_denoise_noalloc (the denoise with its workspace in the library's static device
buffer) against dm_suffix_denoise with a caller workspace, on the same inputs: two calls in a row,
the second on a smaller input (the buffer then still holds the first call's contents), each
bitwise equal to the workspace entry point's result; and a size past the buffer rejected on
the host before any launch."""
import numpy as np
import pytest
import torch

from dual_expert_merged_amd import binding as bd
from dual_expert_merged_amd import inputs
from dual_expert_merged_amd.configs import workload
from tests.gpu_harness import dev_lens

pytestmark = pytest.mark.gpu
SCRATCH = 32 << 20


def _case(ctx, da, kc, vc, lens, x1, steps):
    k = bd.to_device(kc, torch.bfloat16)
    v = bd.to_device(vc, torch.bfloat16)
    ld = dev_lens(lens)
    B, P_cap = k.shape[1], k.shape[3]
    need = ctx.workspace_bytes(bd.OP_DENOISE, B, P_cap)
    print(f"case: noalloc denoise B={B} P_cap={P_cap} lens {list(lens)}: workspace {need} bytes", flush=True)
    assert 0 < need <= SCRATCH
    x_ws = torch.from_numpy(np.ascontiguousarray(x1)).cuda()
    x_na = x_ws.clone()
    ws = ctx.workspace(bd.OP_DENOISE, B, P_cap)
    ctx.suffix_denoise(da, k, v, ld, x_ws, steps, ws)
    ctx.suffix_denoise_noalloc(da, k, v, ld, x_na, steps)
    torch.cuda.synchronize()
    a, b = x_ws.cpu().numpy(), x_na.cpu().numpy()
    assert np.isfinite(a).all()
    diff = int(np.sum(a != b))
    print(f"B={B}: {diff} of {a.size} values differ between the two entry points", flush=True)
    assert diff == 0


def test_noalloc_matches_workspace_entry_point_twice():
    wl = workload(3)
    s = wl.shape
    aw = inputs.make_action_weights(wl)
    kc, vc = inputs.make_kv_cache(wl)
    x1 = inputs.make_noise(wl)
    ctx = bd.Context(s, 0)
    da = bd.DeviceAction(aw, s.dtype)
    # first call: two samples (the multi-kernel sequence), the cache duplicated with a shorter
    # second prefix
    k2 = np.concatenate([kc, kc], axis=1)
    v2 = np.concatenate([vc, vc], axis=1)
    x2 = np.concatenate([x1, x1[:, ::-1]], axis=0)
    _case(ctx, da, k2, v2, np.array([816, 500], np.int32), x2, wl.steps)
    # second call, smaller: one sample with a 400-row cache (the single launch)
    _case(ctx, da, kc[:, :, :, :400], vc[:, :, :, :400], np.array([333], np.int32), x1, wl.steps)
    ctx.close()


def test_noalloc_rejects_sizes_past_the_buffer():
    wl = workload(4)
    ctx = bd.Context(wl.shape, 0)
    B, P_cap = 32, wl.prefix_len
    need = ctx.workspace_bytes(bd.OP_DENOISE, B, P_cap)
    print(f"case: noalloc denoise B={B} P_cap={P_cap} needs {need} bytes", flush=True)
    assert need > SCRATCH
    da = bd.DeviceAction(inputs.make_action_weights(wl), wl.shape.dtype)
    s = wl.shape
    k = torch.zeros((s.n_layers, B, s.n_kv_heads, P_cap, s.head_dim), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((B, s.chunk, s.action_dim), dtype=torch.float32, device="cuda")
    with pytest.raises(bd.DMError) as e:
        ctx.suffix_denoise_noalloc(da, k, k, dev_lens(np.full(B, 600, np.int32)), x, wl.steps)
    assert e.value.status == bd.DM_ERR_WORKSPACE, e.value
    print(f"rejected: {e.value}", flush=True)
    ctx.close()
