"""Runs the HIP library on seeded workloads for the GPU parity tests (through the C ABI)."""
import numpy as np
import torch

from dual_expert_merged_amd import binding as bd
from dual_expert_merged_amd import inputs


def dev_lens(lens):
    return torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()


def np32(t):
    return t.detach().float().cpu().numpy()


class Gpu:
    """One context + device-resident weights for a workload."""

    def __init__(self, wl, vlm=None, aw=None):
        self.wl = wl
        self.shape = wl.shape
        self.ctx = bd.Context(wl.shape)
        self.td = bd.torch_dtype(wl.shape.dtype)
        fp8 = wl.shape.vlm_mlp_dtype != wl.shape.dtype
        self.vlm = bd.DeviceExpert(vlm, wl.shape.dtype, fp8_mlp=fp8) if vlm is not None else None
        self.aw = bd.DeviceAction(aw, wl.shape.dtype) if aw is not None else None

    def cache_to_device(self, k, v):
        return bd.to_device(k, self.td), bd.to_device(v, self.td)

    def denoise(self, k, v, lens, x, steps, graph=False, replays=1):
        """k, v: device caches [L][B][Hkv][P_cap][D]; x numpy [B][S][A]; returns numpy chunk."""
        B, P_cap = k.shape[1], k.shape[3]
        ws = self.ctx.workspace(bd.OP_DENOISE, B, P_cap)
        xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
        ld = dev_lens(lens)
        if not graph:
            self.ctx.suffix_denoise(self.aw, k, v, ld, xd, steps, ws)
            torch.cuda.synchronize()
            return xd.cpu().numpy()
        x0 = xd.clone()
        plan = self.ctx.denoise_plan(self.aw, k, v, ld, xd, steps, ws)
        outs = []
        for _ in range(replays):
            xd.copy_(x0)
            plan.launch()
            torch.cuda.synchronize()
            outs.append(xd.cpu().numpy())
        plan.close()
        return outs if replays > 1 else outs[0]

    def prefill(self, embeds, lens):
        B, P_cap = embeds.shape[0], embeds.shape[1]
        s = self.shape
        shape = (s.n_layers, B, s.n_kv_heads, P_cap, s.head_dim)
        k = torch.zeros(shape, dtype=self.td, device="cuda")
        v = torch.zeros(shape, dtype=self.td, device="cuda")
        ws = self.ctx.workspace(bd.OP_PREFILL, B, P_cap)
        e = torch.from_numpy(np.ascontiguousarray(embeds, dtype=np.float32)).cuda()
        self.ctx.prefill_kv(self.vlm, e, dev_lens(lens), k, v, ws)
        torch.cuda.synchronize()
        return k, v

    def merged_layer(self, layer, h_pre, h_suf, lens, want_kv=True):
        B, P_cap = h_pre.shape[0], h_pre.shape[1]
        s = self.shape
        hp = torch.from_numpy(np.ascontiguousarray(h_pre, dtype=np.float32)).cuda()
        hs = torch.from_numpy(np.ascontiguousarray(h_suf, dtype=np.float32)).cuda()
        ko = vo = None
        if want_kv:
            ko = torch.zeros((B, s.n_kv_heads, P_cap, s.head_dim), dtype=self.td, device="cuda")
            vo = torch.zeros_like(ko)
        ws = self.ctx.workspace(bd.OP_MERGED_LAYER, B, P_cap)
        self.ctx.merged_layer(self.vlm, self.aw.body if self.aw is not None else None, layer, hp, hs,
                              dev_lens(lens), ws, ko, vo)
        torch.cuda.synchronize()
        return np32(hp), np32(hs), (np32(ko) if want_kv else None), (np32(vo) if want_kv else None)


def rel_inf(got, ref):
    """||got - ref||_inf / ||ref||_inf."""
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / np.max(np.abs(ref)))


def err_stats(got, ref):
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    return float(d.max()), float(d.mean())
