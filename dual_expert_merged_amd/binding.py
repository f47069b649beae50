"""ctypes binding of libdm.so (include/dm.h): argument marshalling only.

Every computation runs in the HIP library; this module turns PyTorch device tensors into the
pointers, sizes and stream handle the C ABI takes, and raises DMError on a non-OK status.
The library must be built (``python -m dual_expert_merged_amd.build``); if it is missing the
first call raises, there is no fallback.
"""
import ctypes as C
import os

import numpy as np
import torch

from .configs import BF16, F32, FP8, ModelShape

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdm.so")

DM_OK, DM_ERR_INVALID_ARG, DM_ERR_SHAPE, DM_ERR_UNSUPPORTED, DM_ERR_WORKSPACE, DM_ERR_PLAN_MISMATCH, DM_ERR_HIP = \
    0, -1, -2, -3, -4, -5, -6
STATUS_NAMES = {0: "DM_OK", -1: "DM_ERR_INVALID_ARG", -2: "DM_ERR_SHAPE", -3: "DM_ERR_UNSUPPORTED",
                -4: "DM_ERR_WORKSPACE", -5: "DM_ERR_PLAN_MISMATCH", -6: "DM_ERR_HIP"}
DM_F32, DM_BF16, DM_FP8_E4M3 = 0, 1, 2
DM_FLAG_MULTI_KERNEL = 1
DM_FLAG_TIME_MODULATION = 2
DM_TMOD_MAX_STEPS = 16
DM_FLAG_QK_NORM = 4
OP_PREFILL, OP_MERGED_LAYER, OP_DENOISE, OP_TRAIN = 0, 1, 2, 3
_DT = {F32: DM_F32, BF16: DM_BF16, FP8: DM_FP8_E4M3}
EXPORTS = ["dm_version", "dm_last_error", "dm_ctx_create", "dm_ctx_destroy", "dm_workspace_bytes",
           "dm_prefill_kv", "dm_merged_layer", "dm_suffix_denoise", "dm_denoise_plan_create",
           "dm_denoise_plan_launch", "dm_denoise_plan_destroy", "dm_quantize_fp8_rows", "dm_suffix_denoise_noalloc",
           "dm_engine_create", "dm_engine_contract_get", "dm_engine_run", "dm_engine_replay", "dm_engine_buffers",
           "dm_engine_destroy", "dm_train_merged_layer"]


TRAIN_GRAD_FIELDS = ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down", "w_in", "b_in",
                     "final_norm", "w_out", "b_out", "vlm_attn_norm", "vlm_w_qkv", "h_prefix")


class TrainGradsC(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in TRAIN_GRAD_FIELDS]


ENGINE_CONTRACT_FIELDS = ("batch", "prefix_cap", "num_steps", "chunk", "action_dim", "vlm_hidden")


class EngineContractC(C.Structure):
    _fields_ = [(n, C.c_int) for n in ENGINE_CONTRACT_FIELDS]


class EngineRequestC(C.Structure):
    _fields_ = [("batch", C.c_int), ("prefix_cap", C.c_int), ("num_steps", C.c_int),
                ("prefix_embeds", C.c_void_p), ("prefix_lens", C.c_void_p), ("noise", C.c_void_p),
                ("actions", C.c_void_p)]


class DMError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Config(C.Structure):
    _fields_ = [("n_layers", C.c_int), ("vlm_hidden", C.c_int), ("act_hidden", C.c_int),
                ("vlm_ffn", C.c_int), ("act_ffn", C.c_int), ("n_q_heads", C.c_int),
                ("n_kv_heads", C.c_int), ("head_dim", C.c_int), ("action_dim", C.c_int),
                ("chunk", C.c_int), ("rms_eps", C.c_float), ("rope_base", C.c_float),
                ("dtype", C.c_int), ("vlm_mlp_dtype", C.c_int), ("flags", C.c_int)]


class ExpertWeightsC(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up",
                                          "w_down", "s_gate", "s_up", "s_down", "q_norm", "k_norm")]


TMOD_FIELDS = ("w_in", "b_in", "w_out", "b_out", "w_mod", "b_mod", "w_fmod", "b_fmod")


class TimeModC(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in TMOD_FIELDS]


class ActionWeightsC(C.Structure):
    _fields_ = [("body", ExpertWeightsC)] + [(n, C.c_void_p) for n in ("w_in", "b_in", "final_norm",
                                                                       "w_out", "b_out")] + \
               [("tmod", C.POINTER(TimeModC))]


_lib = None


def lib():
    """Load libdm.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m dual_expert_merged_amd.build")
        L = C.CDLL(LIB_PATH)
        vp, i, sz = C.c_void_p, C.c_int, C.c_size_t
        L.dm_version.restype = C.c_char_p
        L.dm_last_error.restype = C.c_char_p
        L.dm_ctx_create.argtypes = [C.POINTER(Config), i, C.POINTER(vp)]
        L.dm_ctx_destroy.argtypes = [vp]
        L.dm_ctx_destroy.restype = None
        L.dm_workspace_bytes.argtypes = [vp, i, i, i]
        L.dm_workspace_bytes.restype = sz
        L.dm_prefill_kv.argtypes = [vp, C.POINTER(ExpertWeightsC), vp, vp, i, i, vp, vp, vp, sz, vp]
        L.dm_merged_layer.argtypes = [vp, C.POINTER(ExpertWeightsC), C.POINTER(ExpertWeightsC), i, vp, vp, vp,
                                      i, i, vp, vp, vp, sz, vp]
        L.dm_suffix_denoise.argtypes = [vp, C.POINTER(ActionWeightsC), vp, vp, vp, i, i, vp, i, vp, sz, vp]
        L.dm_denoise_plan_create.argtypes = [vp, C.POINTER(ActionWeightsC), vp, vp, vp, i, i, vp, i, vp, sz, vp,
                                             C.POINTER(vp)]
        L.dm_denoise_plan_launch.argtypes = [vp, i, vp]
        L.dm_denoise_plan_destroy.argtypes = [vp]
        L.dm_denoise_plan_destroy.restype = None
        L.dm_quantize_fp8_rows.argtypes = [vp, vp, vp, i, i, vp]
        L.dm_suffix_denoise_noalloc.argtypes = [vp, C.POINTER(ActionWeightsC), vp, vp, vp, i, i, vp, i, vp]
        L.dm_engine_create.argtypes = [vp, C.POINTER(ExpertWeightsC), C.POINTER(ActionWeightsC), i, i, i, vp,
                                       C.POINTER(vp)]
        L.dm_engine_contract_get.argtypes = [vp, C.POINTER(EngineContractC)]
        L.dm_engine_run.argtypes = [vp, C.POINTER(EngineRequestC), vp]
        L.dm_engine_replay.argtypes = [vp, vp]
        L.dm_engine_buffers.argtypes = [vp, C.POINTER(vp), C.POINTER(vp), C.POINTER(vp)]
        L.dm_train_merged_layer.argtypes = [vp, C.POINTER(ExpertWeightsC), C.POINTER(ActionWeightsC), i, vp, vp, i,
                                            i, vp, vp, vp, vp, i, vp, C.POINTER(TrainGradsC), vp, sz, vp]
        L.dm_engine_destroy.argtypes = [vp]
        L.dm_engine_destroy.restype = None
        for name in EXPORTS:
            if name not in ("dm_version", "dm_last_error", "dm_ctx_destroy", "dm_workspace_bytes",
                            "dm_denoise_plan_destroy", "dm_engine_destroy"):
                getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def check(status):
    if status != DM_OK:
        raise DMError(status, lib().dm_last_error().decode(errors="replace"))


def ptr(t):
    """Device (or host) address of a tensor, None for None."""
    return None if t is None else C.c_void_p(t.data_ptr())


def stream_handle(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def make_config(shape: ModelShape, flags: int = 0) -> Config:
    return Config(shape.n_layers, shape.vlm_hidden, shape.act_hidden, shape.vlm_ffn, shape.act_ffn,
                  shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.action_dim, shape.chunk,
                  shape.rms_eps, shape.rope_base, _DT[shape.dtype], _DT[shape.vlm_mlp_dtype], flags)


def torch_dtype(dtype: str):
    return {F32: torch.float32, BF16: torch.bfloat16}[dtype]


def to_device(a: np.ndarray, dtype=torch.float32, device="cuda"):
    """Copy a numpy array (float32 holding values of `dtype`) to the device, converted exactly."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device).to(dtype).contiguous()


class DeviceExpert:
    """One expert's stacked weights resident on the device, plus the C struct pointing at them.

    fp8_mlp: keep gate/up/down as E4M3 codes with per-output-channel scales, quantised on the
    device by dm_quantize_fp8_rows from the weight-dtype matrices (bf16 only)."""

    def __init__(self, w, dtype, device="cuda", fp8_mlp=False):
        td = torch_dtype(dtype)
        self.t = {
            "attn_norm": to_device(w.attn_norm, torch.float32, device),
            "w_qkv": to_device(w.w_qkv, td, device),
            "w_o": to_device(w.w_o, td, device),
            "mlp_norm": to_device(w.mlp_norm, torch.float32, device),
            "w_gate": to_device(w.w_gate, td, device),
            "w_up": to_device(w.w_up, td, device),
            "w_down": to_device(w.w_down, td, device),
        }
        scales = [None, None, None]
        if fp8_mlp:
            if td != torch.bfloat16:
                raise DMError(DM_ERR_INVALID_ARG, "the FP8 MLP needs bf16 weights")
            for i, k in enumerate(("w_gate", "w_up", "w_down")):
                codes, s = quantize_fp8_rows(self.t[k])
                self.t[k], self.t["s" + k[1:]] = codes, s
                scales[i] = ptr(s)
            torch.cuda.current_stream().synchronize()
        qk = [None, None]
        if getattr(w, "q_norm", None) is not None:  # per-head QK-norm gains (float32)
            for i, k in enumerate(("q_norm", "k_norm")):
                self.t[k] = to_device(getattr(w, k), torch.float32, device)
                qk[i] = ptr(self.t[k])
        self.c = ExpertWeightsC(*(ptr(self.t[k]) for k in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate",
                                                            "w_up", "w_down")), *scales, *qk)


class DeviceAction:
    """Action-expert weights on the device.  With aw.tmod set (the time-modulated expert) the
    modulator matrices are kept in the weight dtype, the time MLP and all biases in float32."""

    def __init__(self, aw, dtype, device="cuda"):
        self.body = DeviceExpert(aw.body, dtype, device)
        self.t = {k: to_device(getattr(aw, k), torch.float32, device)
                  for k in ("w_in", "b_in", "final_norm", "w_out", "b_out")}
        tm = getattr(aw, "tmod", None)
        self.tm = None
        tmod_c = None
        if tm is not None:
            wd = torch_dtype(dtype)
            self.tm = {k: to_device(getattr(tm, k), wd if k in ("w_mod", "w_fmod") else torch.float32, device)
                       for k in TMOD_FIELDS}
            self.tmod_c = TimeModC(*(ptr(self.tm[k]) for k in TMOD_FIELDS))
            tmod_c = C.pointer(self.tmod_c)
        self.c = ActionWeightsC(self.body.c, *(ptr(self.t[k]) for k in ("w_in", "b_in", "final_norm", "w_out",
                                                                         "b_out")), tmod_c)


class Context:
    """A libdm context for one model shape on one device."""

    def __init__(self, shape: ModelShape, device: int = 0, flags: int = 0):
        self.shape = shape
        self.device = device
        if getattr(shape, "time_mod", False):
            flags |= DM_FLAG_TIME_MODULATION
        if getattr(shape, "qk_norm", False):
            flags |= DM_FLAG_QK_NORM
        self.cfg = make_config(shape, flags)
        h = C.c_void_p()
        self._destroy = lib().dm_ctx_destroy  # bound now: module globals may be gone when __del__ runs at exit
        check(lib().dm_ctx_create(C.byref(self.cfg), device, C.byref(h)))
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            self._destroy(self.h)
            self.h = None

    __del__ = close

    def workspace_bytes(self, op, B, P_cap):
        return lib().dm_workspace_bytes(self.h, op, B, P_cap)

    def workspace(self, op, B, P_cap):
        n = self.workspace_bytes(op, B, P_cap)
        if n == 0:
            raise DMError(DM_ERR_INVALID_ARG, "dm_workspace_bytes returned 0")
        return torch.empty(n, dtype=torch.uint8, device=f"cuda:{self.device}")

    def prefill_kv(self, vlm: DeviceExpert, prefix_embeds, lens, k_cache, v_cache, ws, stream=None):
        B, P_cap = prefix_embeds.shape[0], prefix_embeds.shape[1]
        check(lib().dm_prefill_kv(self.h, C.byref(vlm.c), ptr(prefix_embeds), ptr(lens), B, P_cap, ptr(k_cache),
                                  ptr(v_cache), ptr(ws), ws.numel(), stream_handle(stream)))

    def merged_layer(self, vlm: DeviceExpert, act: DeviceExpert, layer, h_prefix, h_suffix, lens, ws,
                     k_out=None, v_out=None, stream=None):
        B, P_cap = h_prefix.shape[0], h_prefix.shape[1]
        check(lib().dm_merged_layer(self.h, C.byref(vlm.c), C.byref(act.c), layer, ptr(h_prefix), ptr(h_suffix),
                                    ptr(lens), B, P_cap, ptr(k_out), ptr(v_out), ptr(ws), ws.numel(),
                                    stream_handle(stream)))

    def suffix_denoise(self, aw: DeviceAction, k_cache, v_cache, lens, x, num_steps, ws, stream=None):
        B, P_cap = k_cache.shape[1], k_cache.shape[3]
        check(lib().dm_suffix_denoise(self.h, C.byref(aw.c), ptr(k_cache), ptr(v_cache), ptr(lens), B, P_cap,
                                      ptr(x), num_steps, ptr(ws), ws.numel(), stream_handle(stream)))

    def suffix_denoise_noalloc(self, aw: DeviceAction, k_cache, v_cache, lens, x, num_steps, stream=None):
        B, P_cap = k_cache.shape[1], k_cache.shape[3]
        check(lib().dm_suffix_denoise_noalloc(self.h, C.byref(aw.c), ptr(k_cache), ptr(v_cache), ptr(lens), B, P_cap,
                                              ptr(x), num_steps, stream_handle(stream)))

    def train_merged_layer(self, vlm: DeviceExpert, aw: DeviceAction, layer, h_prefix, lens, actions, noise, t, mask,
                           knowledge_insulation, loss, grads, ws, stream=None):
        """One flow-matching training step on merged layer `layer`; `grads` maps the names in
        TRAIN_GRAD_FIELDS to float32 device tensors (absent names pass NULL); `loss` is a
        one-element float32 device tensor."""
        B, P_cap = h_prefix.shape[0], h_prefix.shape[1]
        gc = TrainGradsC(*(ptr(grads.get(n)) for n in TRAIN_GRAD_FIELDS))
        check(lib().dm_train_merged_layer(self.h, C.byref(vlm.c), C.byref(aw.c), layer, ptr(h_prefix), ptr(lens), B,
                                          P_cap, ptr(actions), ptr(noise), ptr(t), ptr(mask),
                                          1 if knowledge_insulation else 0, ptr(loss), C.byref(gc), ptr(ws),
                                          ws.numel(), stream_handle(stream)))

    def denoise_plan(self, aw: DeviceAction, k_cache, v_cache, lens, x, num_steps, ws, stream=None):
        B, P_cap = k_cache.shape[1], k_cache.shape[3]
        h = C.c_void_p()
        check(lib().dm_denoise_plan_create(self.h, C.byref(aw.c), ptr(k_cache), ptr(v_cache), ptr(lens), B, P_cap,
                                           ptr(x), num_steps, ptr(ws), ws.numel(), stream_handle(stream),
                                           C.byref(h)))
        return Plan(h, num_steps, keep=(aw, k_cache, v_cache, lens, x, ws))


class Plan:
    """A captured denoise graph; keeps the tensors it was captured with alive."""

    def __init__(self, handle, steps, keep):
        self._destroy = lib().dm_denoise_plan_destroy  # bound now, as in Context
        self.h = handle
        self.steps = steps
        self.keep = keep

    def launch(self, num_steps=None, stream=None):
        check(lib().dm_denoise_plan_launch(self.h, self.steps if num_steps is None else num_steps,
                                           stream_handle(stream)))

    def close(self):
        if getattr(self, "h", None):
            self._destroy(self.h)
            self.h = None

    __del__ = close


class Engine:
    """A fixed-contract engine: static device buffers and one captured prefill + denoise graph.
    Keeps the weight objects it was created from alive."""

    def __init__(self, ctx: "Context", vlm: "DeviceExpert", aw: "DeviceAction", B, P_cap, num_steps, stream=None):
        self._destroy = lib().dm_engine_destroy  # bound now, as in Context
        self.h = None
        h = C.c_void_p()
        check(lib().dm_engine_create(ctx.h, C.byref(vlm.c), C.byref(aw.c), B, P_cap, num_steps,
                                     stream_handle(stream), C.byref(h)))
        self.h = h
        self.keep = (ctx, vlm, aw)

    def contract(self):
        c = EngineContractC()
        check(lib().dm_engine_contract_get(self.h, C.byref(c)))
        return {n: getattr(c, n) for n in ENGINE_CONTRACT_FIELDS}

    def run(self, prefix_embeds, prefix_lens, noise, actions, batch=None, prefix_cap=None, num_steps=None,
            stream=None):
        """One request from host numpy arrays (float32 embeds / noise / actions, int32 lengths);
        the claimed shape defaults to the arrays' own, num_steps to the contract's."""
        for a, dt in ((prefix_embeds, np.float32), (prefix_lens, np.int32), (noise, np.float32), (actions, np.float32)):
            if a is not None and (a.dtype != dt or not a.flags.c_contiguous):
                raise ValueError("request arrays must be C-contiguous float32 (lengths int32)")
        k = self.contract()
        req = EngineRequestC(
            prefix_embeds.shape[0] if batch is None else batch,
            prefix_embeds.shape[1] if prefix_cap is None else prefix_cap,
            k["num_steps"] if num_steps is None else num_steps,
            *(None if a is None else C.c_void_p(a.ctypes.data) for a in (prefix_embeds, prefix_lens, noise, actions)))
        check(lib().dm_engine_run(self.h, C.byref(req), stream_handle(stream)))

    def replay(self, stream=None):
        check(lib().dm_engine_replay(self.h, stream_handle(stream)))

    def buffers(self):
        """Device addresses (ints) of the static prefix embeddings, prefix lengths and x."""
        e, l, x = C.c_void_p(), C.c_void_p(), C.c_void_p()
        check(lib().dm_engine_buffers(self.h, C.byref(e), C.byref(l), C.byref(x)))
        return e.value, l.value, x.value

    def close(self):
        if getattr(self, "h", None):
            self._destroy(self.h)
            self.h = None

    __del__ = close


def quantize_fp8_rows(src, stream=None):
    """E4M3 codes [rows][cols] (uint8) and per-row scales (float32) of a bf16 matrix."""
    rows, cols = src.shape[-2] if src.dim() > 1 else 1, src.shape[-1]
    rows = src.numel() // cols
    dst = torch.empty(src.shape, dtype=torch.uint8, device=src.device)
    scales = torch.empty(src.shape[:-1], dtype=torch.float32, device=src.device)
    check(lib().dm_quantize_fp8_rows(ptr(src), ptr(dst), ptr(scales), rows, cols, stream_handle(stream)))
    return dst, scales
