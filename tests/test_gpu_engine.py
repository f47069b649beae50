"""GPU tests of the fixed-contract engine (page "DM0.5: High-Performance Embodied VLA and OpenDM
Open Source Introduction", section 6.5: capture once over fixed-shape static buffers, copy each
new observation in, replay once; section 9.1: model-core against request latency).

- tiny fp32, B=3 ragged prefix 1-64, 4 steps: the engine's chunk against the float64 oracle
  (prefix encoding + denoise of every sample) ||gpu - oracle||_inf / ||oracle||_inf <= 1e-4,
  the contract it reports, and every rejection (shape claims that differ from the contract,
  prefix lengths outside 0..P_cap, missing buffers) leaving the output untouched;
- the same with per-head QK-norm (both experts);
- DM0-base bf16, B=2, prefix 816 / 523: two successive requests with different inputs, each
  bitwise equal to dm_prefill_kv followed by dm_suffix_denoise on the same inputs (the calls the
  other GPU tests hold to the oracle), and model-core replays between them changing nothing
  the next request sees;
- the FP8-MLP prefill (DM0-base, B = 2) and the time-modulated expert (tiny, B = 3): two
  requests each, bitwise equal to the separate calls;
- DM0-base bf16 at B = 1 (prefix 816, then 300 under the same 816 cap), where the captured
  denoise is the single-launch kernel: two requests bitwise equal to the separate calls.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from dual_expert_merged_amd import binding as bd
from dual_expert_merged_amd import inputs
from dual_expert_merged_amd.configs import FP8, workload
from tests.gpu_harness import Gpu, rel_inf

pytestmark = pytest.mark.gpu


def _engine(gpu, wl):
    return bd.Engine(gpu.ctx, gpu.vlm, gpu.aw, wl.batch, wl.prefix_len, wl.steps)


def _oracle_chunks(wl, vlm, aw, emb, lens, x1):
    out = []
    for b in range(wl.batch):
        P = int(lens[b])
        rk, rv, _ = O.prefill_kv(emb[b, :P], vlm, wl.shape)
        out.append(O.suffix_denoise(x1[b], aw, rk, rv, wl.shape, wl.steps))
    return out


def _tiny_case(wl, label):
    lens = inputs.make_prefix_lens(wl)
    print(f"case: engine, {label}, B={wl.batch} lens {lens.tolist()} P_cap={wl.prefix_len} steps={wl.steps}",
          flush=True)
    vlm = inputs.make_vlm_weights(wl)
    aw = inputs.make_action_weights(wl)
    emb = inputs.make_prefix_embeds(wl)
    x1 = inputs.make_noise(wl)
    gpu = Gpu(wl, vlm, aw)
    eng = _engine(gpu, wl)
    got = np.zeros_like(x1)
    eng.run(emb, lens, x1, got)
    for b, ref in enumerate(_oracle_chunks(wl, vlm, aw, emb, lens, x1)):
        e = rel_inf(got[b], ref)
        print(f"sample {b} (P={lens[b]}): rel inf err {e:.3e}", flush=True)
        assert e <= 1e-4, (b, e)
    return eng, emb, lens, x1, got


def test_engine_tiny_fp32_matches_oracle_and_rejects_off_contract_requests():
    wl = dataclasses.replace(workload(1), batch=3, ragged=(1, 64))
    eng, emb, lens, x1, got = _tiny_case(wl, "tiny fp32")
    s = wl.shape
    assert eng.contract() == {"batch": 3, "prefix_cap": 64, "num_steps": 4, "chunk": s.chunk,
                              "action_dim": s.action_dim, "vlm_hidden": s.vlm_hidden}
    out = np.full_like(x1, 7.0)
    cases = [
        (dict(batch=2), bd.DM_ERR_PLAN_MISMATCH),        # another batch
        (dict(prefix_cap=32), bd.DM_ERR_PLAN_MISMATCH),  # another prefix bucket
        (dict(num_steps=5), bd.DM_ERR_PLAN_MISMATCH),    # another step count needs another capture
    ]
    for claim, status in cases:
        with pytest.raises(bd.DMError) as e:
            eng.run(emb, lens, x1, out, **claim)
        assert e.value.status == status, claim
    for bad in (-1, 65):
        bad_lens = lens.copy()
        bad_lens[1] = bad
        with pytest.raises(bd.DMError) as e:
            eng.run(emb, bad_lens, x1, out)
        assert e.value.status == bd.DM_ERR_SHAPE, bad
    with pytest.raises(bd.DMError) as e:
        eng.run(emb, lens, None, out)
    assert e.value.status == bd.DM_ERR_INVALID_ARG
    np.testing.assert_array_equal(out, np.full_like(x1, 7.0))  # nothing was copied back
    print("every off-contract request rejected, output untouched", flush=True)
    again = np.zeros_like(x1)
    eng.run(emb, lens, x1, again)
    np.testing.assert_array_equal(again, got)
    e_ptr, l_ptr, x_ptr = eng.buffers()
    assert e_ptr and l_ptr and x_ptr and len({e_ptr, l_ptr, x_ptr}) == 3
    eng.close()


def test_engine_tiny_qk_norm_matches_oracle():
    wl = workload(8)
    eng, *_ = _tiny_case(wl, "tiny fp32 with per-head QK-norm")
    eng.close()


@pytest.mark.timeout(600)
def test_engine_dm0_base_bf16_equals_separate_calls_over_two_requests():
    wl = dataclasses.replace(workload(5), batch=2)
    s = wl.shape
    lens_a = np.array([816, 523], dtype=np.int32)
    print(f"case: engine, DM0-base bf16 B=2 P_cap=816 lens {lens_a.tolist()} then reversed, 10 steps", flush=True)
    vlm = inputs.make_vlm_weights(wl)
    aw = inputs.make_action_weights(wl)
    emb_a = inputs.make_prefix_embeds(dataclasses.replace(wl, batch=2))
    emb_a[1, 523:] = 0.0
    x_a = inputs.make_noise(wl)
    # a second request: the samples swapped, fresh noise
    emb_b = np.ascontiguousarray(emb_a[::-1])
    lens_b = np.ascontiguousarray(lens_a[::-1])
    x_b = np.random.default_rng(5).standard_normal(x_a.shape).astype(np.float32)
    gpu = Gpu(wl, vlm, aw)
    eng = _engine(gpu, wl)
    for name, emb, lens, x in (("A", emb_a, lens_a, x_a), ("B", emb_b, lens_b, x_b)):
        got = np.zeros_like(x)
        eng.run(emb, lens, x, got)
        k, v = gpu.prefill(emb, lens)
        ref = gpu.denoise(k, v, lens, x, wl.steps)
        del k, v
        torch.cuda.empty_cache()
        diff = float(np.abs(got - ref).max())
        print(f"request {name}: max |engine - separate calls| = {diff:.3e}", flush=True)
        np.testing.assert_array_equal(got, ref)
        assert np.isfinite(got).all() and np.abs(got).max() > 0
        for _ in range(2):  # model-core replays over whatever the buffers hold
            eng.replay()
        torch.cuda.synchronize()
    eng.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("variant", ["fp8_mlp", "time_modulation"])
def test_engine_equals_separate_calls_for_model_variants(variant):
    """The engine captures whatever the context's model is: the FP8-MLP prefill (DM0-base, B=2,
    prefixes 816 / 300) and the time-modulated action expert (tiny fp32, B=3 ragged); two
    requests each, bitwise equal to dm_prefill_kv followed by dm_suffix_denoise."""
    if variant == "fp8_mlp":
        wl = dataclasses.replace(workload(5), batch=2,
                                 shape=dataclasses.replace(workload(5).shape, vlm_mlp_dtype=FP8))
        lens_a = np.array([816, 300], dtype=np.int32)
    else:
        wl = dataclasses.replace(workload(6), kind="prefill_denoise")
        lens_a = inputs.make_prefix_lens(wl)
    print(f"case: engine, {variant}, B={wl.batch} P_cap={wl.prefix_len} lens {lens_a.tolist()}", flush=True)
    vlm = inputs.make_vlm_weights(wl)
    aw = inputs.make_action_weights(wl)
    emb_a = inputs.make_prefix_embeds(wl)
    x_a = inputs.make_noise(wl)
    emb_b = np.ascontiguousarray(emb_a[::-1])
    lens_b = np.ascontiguousarray(lens_a[::-1])
    x_b = np.random.default_rng(9).standard_normal(x_a.shape).astype(np.float32)
    gpu = Gpu(wl, vlm, aw)
    eng = _engine(gpu, wl)
    for name, emb, lens, x in (("A", emb_a, lens_a, x_a), ("B", emb_b, lens_b, x_b)):
        got = np.zeros_like(x)
        eng.run(emb, lens, x, got)
        k, v = gpu.prefill(emb, lens)
        ref = gpu.denoise(k, v, lens, x, wl.steps)
        del k, v
        torch.cuda.empty_cache()
        print(f"request {name}: max |engine - separate calls| = {float(np.abs(got - ref).max()):.3e}", flush=True)
        np.testing.assert_array_equal(got, ref)
        assert np.isfinite(got).all()
    eng.close()


@pytest.mark.timeout(600)
def test_engine_dm0_base_batch1_single_launch_equals_separate_calls():
    wl = dataclasses.replace(workload(5), batch=1)
    vlm = inputs.make_vlm_weights(wl)
    aw = inputs.make_action_weights(wl)
    emb = inputs.make_prefix_embeds(wl)
    x_a = inputs.make_noise(wl)
    x_b = np.random.default_rng(11).standard_normal(x_a.shape).astype(np.float32)
    emb_b = emb.copy()
    emb_b[0, 300:] = 0.0
    print("case: engine, DM0-base bf16 B=1 P_cap=816, requests with prefix 816 then 300, 10 steps", flush=True)
    gpu = Gpu(wl, vlm, aw)
    eng = _engine(gpu, wl)
    for name, e, lens, x in (("A", emb, np.array([816], dtype=np.int32), x_a),
                             ("B", emb_b, np.array([300], dtype=np.int32), x_b)):
        got = np.zeros_like(x)
        eng.run(e, lens, x, got)
        k, v = gpu.prefill(e, lens)
        ref = gpu.denoise(k, v, lens, x, wl.steps)
        del k, v
        torch.cuda.empty_cache()
        print(f"request {name}: max |engine - separate calls| = {float(np.abs(got - ref).max()):.3e}", flush=True)
        np.testing.assert_array_equal(got, ref)
        assert np.isfinite(got).all() and np.abs(got).max() > 0
    eng.close()
