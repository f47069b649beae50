"""The seeded input generator: rounding, determinism and the workload recipe (CPU only)."""
import numpy as np
import torch

from dual_expert_merged_amd import inputs
from dual_expert_merged_amd.configs import WORKLOADS, workload


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s for s in (1e-3, 1, 300)])
    # ties: values exactly halfway between two bf16 numbers
    base = rng.standard_normal(1000).astype(np.float32)
    ties = ((base.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(inputs.bf16_bits(x), ref)
    np.testing.assert_array_equal(inputs.round_to(x, "bf16"),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_rounded():
    wl = workload(1)
    a = inputs.make_action_weights(wl)
    b = inputs.make_action_weights(wl)
    np.testing.assert_array_equal(a.body.w_qkv, b.body.w_qkv)
    np.testing.assert_array_equal(a.w_out, b.w_out)
    s = wl.shape
    assert a.body.w_qkv.shape == (2, (4 + 4) * 32, 128)
    assert a.body.w_down.shape == (2, 128, 384)
    assert abs(a.body.w_qkv.std() - 0.02) < 2e-3
    assert abs(a.body.attn_norm.mean() - 1.0) < 1e-2
    wl2 = workload(2)
    v = inputs.make_vlm_weights(wl2)
    assert v.w_gate.dtype == np.float32 and v.w_gate.shape == (1, 6144, 2048)
    np.testing.assert_array_equal(inputs.round_to(v.w_gate[0, :4], "bf16"), v.w_gate[0, :4])


def test_ragged_lengths_and_padding():
    wl = workload(4)
    lens = inputs.make_prefix_lens(wl)
    assert lens.shape == (32,) and lens.min() >= 600 and lens.max() <= 1100
    assert wl.prefix_len == 1104 and wl.prefix_len % 16 == 0
    assert len(set(lens.tolist())) > 20
    small = workload(4, batch=3, shape=workload(1).shape, prefix_len=1104)
    k, v = inputs.make_kv_cache(small)
    l3 = inputs.make_prefix_lens(small)
    for b in range(3):
        assert np.all(k[:, b, :, l3[b]:] == 0) and np.all(k[:, b, :, :l3[b]] != 0)


def test_every_workload_has_its_shapes():
    assert WORKLOADS[3].shape.n_layers == 28 and WORKLOADS[3].steps == 10
    assert WORKLOADS[2].shape.n_layers == 1 and WORKLOADS[2].prefix_len == 816
    assert WORKLOADS[5].batch == 8 and WORKLOADS[1].shape.dtype == "f32"
    x = inputs.make_noise(WORKLOADS[3])
    assert x.shape == (1, 50, 32) and x.dtype == np.float32
