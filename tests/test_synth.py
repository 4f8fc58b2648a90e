"""The seeded input generator: determinism, distributions and storage formats."""
import numpy as np
import torch

import synth
from synth import configs


def test_draws_are_counter_based_and_thread_independent():
    a = synth.normal_f32(0, 4, (300000,), 1.0)
    b = synth.normal_f32(0, 4, (1000,), 1.0, first=200000)
    assert np.array_equal(a[200000:201000], b)
    c = synth.normal_f32(1, 4, (1000,), 1.0)
    assert not np.array_equal(a[:1000], c)
    u = synth.raw_u64(0, 4, 10)
    assert np.array_equal(u, synth.raw_u64(0, 4, 10))


def test_normal_moments():
    z = synth.normal_f32(0, 11, (2_000_000,), 1.0).astype(np.float64)
    assert abs(z.mean()) < 3e-3
    assert abs(z.std() - 1.0) < 3e-3
    assert abs(np.mean(z ** 4) - 3.0) < 0.03           # Gaussian kurtosis
    u = synth.uniform_f64(0, 12, 200000)
    assert u.min() > 0.0 and u.max() < 1.0 and abs(u.mean() - 0.5) < 3e-3


def test_bf16_storage_matches_torch_cast():
    f = synth.normal_f32(3, 5, (100000,), 0.7)
    b = synth.normal_bf16(3, 5, (100000,), 0.7)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_fp8_rows_match_torch_cast_and_scale_rule():
    codes, scales = synth.normal_fp8_rows(2, 6, (64, 512), 0.05)
    f = synth.normal_f32(2, 6, (64, 512), 0.05)
    amax = np.abs(f).max(axis=1)
    assert np.array_equal(scales, (amax / np.float32(448.0)).astype(np.float32))
    v = (f / scales[:, None]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    inside = np.abs(v) < 448.0
    assert np.array_equal(codes[inside], ref[inside])
    assert np.all((codes[~inside] & 0x7F) == 0x7E)       # saturated to +-448
    assert np.all((codes & 0x7F) != 0x7F)                # never NaN


def test_mxfp4_rows_follow_the_mx_scale_rule_and_nearest_codes():
    codes, scales = synth.normal_mxfp4_rows(2, 7, (16, 256), 0.05)
    f = synth.normal_f32(2, 7, (16, 256), 0.05).astype(np.float64)
    blocks = f.reshape(16, 8, 32)
    amax = np.abs(blocks).max(axis=2)
    # X - 127 = floor(log2(amax)) - 2: each block's largest value over 2^(X-127) is in [4, 8)
    r = amax / np.ldexp(1.0, scales.astype(np.int64) - 127)
    assert np.all((r >= 4.0) & (r < 8.0))
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    v = blocks / np.ldexp(1.0, scales.astype(np.int64) - 127)[:, :, None]
    d = np.abs(np.abs(v)[..., None] - mags)                     # distance to each magnitude
    best = d.min(axis=-1, keepdims=True)
    tie_even = np.where(d == best, np.arange(8) % 2, 9)         # among the nearest, the even code
    m = np.where((d == best).sum(-1) > 1, np.argmin(tie_even, axis=-1), np.argmin(d, axis=-1))
    ref = (m | np.where(v < 0, 8, 0)).reshape(16, 256).astype(np.uint8)
    got = np.stack([codes & 15, codes >> 4], axis=-1).reshape(16, 256)
    assert np.array_equal(got, ref)


def test_permutation_is_a_permutation():
    p = synth.permutation(0, 9, 512)
    assert sorted(p.tolist()) == list(range(512))
    assert not np.array_equal(p, np.arange(512))


def test_recipes_have_the_stated_shapes():
    cfg = configs.CONFIGS["tiny"]
    L = configs.make_layer(cfg)
    assert L["w_gate_up"].shape == (16, 256, 256) and L["w_down"].shape == (16, 256, 128)
    assert L["router_b"] is None and L["I_s"] == 0
    x = configs.make_tokens(cfg, 4)
    assert x.shape == (4, 256) and x.dtype == np.uint16
    assert np.array_equal(configs.make_tokens(cfg, 2), x[:2])   # prefixes agree across T
    c3 = configs.with_shape(configs.CONFIGS["flash_next_fp8"], E=8)
    L3 = configs.make_layer(c3)
    assert L3["w_gate_up"].dtype == np.uint8 and L3["s_gate_up"].shape == (8, 1024)
    assert L3["s_down"].shape == (8, 2048) and L3["shared_s_down"].shape == (2048,)
    zb = configs.zipf_bias(256, 1.1, 0.1795)
    assert zb.shape == (256,) and zb.max() < 0


def test_replicas_differ():
    cfg = configs.with_shape(configs.CONFIGS["tiny"], E=4)
    a = configs.make_layer(cfg, replica=0)
    b = configs.make_layer(cfg, replica=1)
    assert not np.array_equal(a["w_gate_up"], b["w_gate_up"])
