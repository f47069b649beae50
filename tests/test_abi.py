"""The C-ABI library: it loads, exports every entry point include/dm.h declares, and rejects bad
arguments on the host before any HIP call (CPU only: no compute call is made)."""
import ctypes as C
import os
import re

import pytest

from dual_expert_merged_amd import binding as bd
from dual_expert_merged_amd.configs import DM0_BASE, TINY
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "dm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("dm_prefill_kv", "dm_merged_layer", "dm_suffix_denoise", "dm_denoise_plan_create",
                     "dm_denoise_plan_launch", "dm_denoise_plan_destroy"):
        assert required in names
    assert sorted(bd.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    lib = bd.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert b"gfx950" in lib.dm_version()


def _cfg(**kw):
    c = bd.make_config(TINY)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 48, bd.DM_ERR_UNSUPPORTED),
    ("n_kv_heads", 3, bd.DM_ERR_SHAPE),
    ("act_hidden", 100, bd.DM_ERR_SHAPE),
    ("vlm_ffn", 0, bd.DM_ERR_SHAPE),
    ("action_dim", 65, bd.DM_ERR_UNSUPPORTED),
    ("action_dim", 30, bd.DM_ERR_UNSUPPORTED),
    ("chunk", 0, bd.DM_ERR_UNSUPPORTED),
    ("dtype", 7, bd.DM_ERR_UNSUPPORTED),
    ("vlm_mlp_dtype", bd.DM_FP8_E4M3, bd.DM_ERR_UNSUPPORTED),  # FP8 MLP needs a bf16 model
    ("rms_eps", 0.0, bd.DM_ERR_INVALID_ARG),
    ("n_layers", 0, bd.DM_ERR_SHAPE),
    ("flags", 8, bd.DM_ERR_INVALID_ARG),
])
def test_bad_config_rejected_before_any_hip_call(field, value, status):
    lib = bd.lib()
    h = C.c_void_p()
    cfg = _cfg(**{field: value})
    assert lib.dm_ctx_create(C.byref(cfg), 0, C.byref(h)) == status
    assert not h.value
    assert len(lib.dm_last_error()) > 0


def test_null_arguments_rejected():
    lib = bd.lib()
    assert lib.dm_ctx_create(None, 0, None) == bd.DM_ERR_INVALID_ARG
    assert lib.dm_workspace_bytes(None, bd.OP_DENOISE, 1, 816) == 0
    assert lib.dm_suffix_denoise(None, None, None, None, None, 1, 816, None, 10, None, 0, None) == bd.DM_ERR_INVALID_ARG
    assert lib.dm_prefill_kv(None, None, None, None, 1, 816, None, None, None, 0, None) == bd.DM_ERR_INVALID_ARG
    assert lib.dm_merged_layer(None, None, None, 0, None, None, None, 1, 816, None, None, None, 0,
                               None) == bd.DM_ERR_INVALID_ARG
    assert lib.dm_denoise_plan_launch(None, 10, None) == bd.DM_ERR_INVALID_ARG
    assert lib.dm_quantize_fp8_rows(None, None, None, 4, 4, None) == bd.DM_ERR_INVALID_ARG
    assert b"NULL" in lib.dm_last_error()
    lib.dm_ctx_destroy(None)
    lib.dm_denoise_plan_destroy(None)


def test_engine_null_arguments_rejected():
    lib = bd.lib()
    h = C.c_void_p()
    assert lib.dm_engine_create(None, None, None, 8, 816, 10, None, None) == bd.DM_ERR_INVALID_ARG
    assert lib.dm_engine_create(None, None, None, 8, 816, 10, None, C.byref(h)) == bd.DM_ERR_INVALID_ARG
    assert h.value is None
    assert lib.dm_engine_contract_get(None, C.byref(bd.EngineContractC())) == bd.DM_ERR_INVALID_ARG
    assert lib.dm_engine_run(None, C.byref(bd.EngineRequestC()), None) == bd.DM_ERR_INVALID_ARG
    assert lib.dm_engine_replay(None, None) == bd.DM_ERR_INVALID_ARG
    assert lib.dm_engine_buffers(None, None, None, None) == bd.DM_ERR_INVALID_ARG
    lib.dm_engine_destroy(None)


def test_engine_structs_match_the_header():
    text = open(HEADER).read()
    con = text[text.index("int batch;       /* B */"):text.index("} dm_engine_contract;")]
    assert tuple(re.findall(r"int (\w+);", con)) == bd.ENGINE_CONTRACT_FIELDS
    req = text[text.index("int batch, prefix_cap, num_steps;"):text.index("} dm_engine_request;")]
    names = ["batch", "prefix_cap", "num_steps"] + re.findall(r"\*\s*(\w+);", req)
    assert [f[0] for f in bd.EngineRequestC._fields_] == names


def test_train_null_arguments_rejected_and_grads_struct_matches_the_header():
    lib = bd.lib()
    g = bd.TrainGradsC()
    assert lib.dm_train_merged_layer(None, None, None, 0, None, None, 1, 816, None, None, None, None, 1, None,
                                     C.byref(g), None, 0, None) == bd.DM_ERR_INVALID_ARG
    assert lib.dm_workspace_bytes(None, bd.OP_TRAIN, 1, 816) == 0
    text = open(HEADER).read()
    body = text[text.index("float *attn_norm, *w_qkv, *w_o"):text.index("} dm_train_grads;")]
    body = re.sub(r"/\*.*?\*/", "", body)
    names = re.findall(r"\*(\w+)", body)
    assert tuple(names) == bd.TRAIN_GRAD_FIELDS
    assert [f[0] for f in bd.TrainGradsC._fields_] == list(names)


def test_dm0_base_config_is_accepted_by_validation():
    # a good config fails only at the device query on a machine without a GPU
    lib = bd.lib()
    h = C.c_void_p()
    cfg = bd.make_config(DM0_BASE)
    st = lib.dm_ctx_create(C.byref(cfg), 0, C.byref(h))
    if st == bd.DM_OK:
        lib.dm_ctx_destroy(h)
    else:
        assert st == bd.DM_ERR_HIP or st == bd.DM_ERR_INVALID_ARG, st
        assert b"hipGetDeviceCount" in lib.dm_last_error() or b"device" in lib.dm_last_error()


def test_time_modulation_needs_hidden_at_most_1024():
    h = C.c_void_p()
    cfg = _cfg(flags=bd.DM_FLAG_TIME_MODULATION, act_hidden=2048)
    assert bd.lib().dm_ctx_create(C.byref(cfg), 0, C.byref(h)) == bd.DM_ERR_UNSUPPORTED


def test_action_weights_struct_matches_the_header():
    """dm_action_weights ends with the tmod pointer after the five head tensors."""
    text = open(HEADER).read()
    body = text[text.index("dm_expert_weights body;"):text.index("} dm_action_weights;")]
    names = re.findall(r"\*\s*(\w+);", body)
    assert names == ["w_in", "b_in", "final_norm", "w_out", "b_out", "tmod"]
    assert [f[0] for f in bd.ActionWeightsC._fields_] == ["body"] + names
    tm = text[text.index("typedef struct {\n  const float *w_in;    /* [H][H] time_mlp_in */"):text.index("} dm_time_modulation;")]
    assert re.findall(r"\*\s*(\w+);", tm) == list(bd.TMOD_FIELDS)


def test_expert_weights_struct_matches_the_header():
    text = open(HEADER).read()
    body = text[text.index("const float *attn_norm; /* [L][H] */"):text.index("} dm_expert_weights;")]
    names = re.findall(r"\*\s*(\w+);", body)
    assert [f[0] for f in bd.ExpertWeightsC._fields_] == names
    assert names[-2:] == ["q_norm", "k_norm"]
