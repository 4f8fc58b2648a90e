"""Synthetic layer recipes: shapes, value distributions and seeds of the workloads.

Each recipe stands in for a layer the pages run on real weights (which are not
available here): the Qwen3.6-35B-A3B MoE layer of "Qwen3.6-35B-A3B on NVIDIA GB10" and
"Qwen3.6-35B-A3B for NInfer", and the Qwen3.8-Flash-Next layer of the veloGB10 README
("The model": 512 routed experts, top-10, plus a shared expert).  Sizes are synthetic
stand-ins of the same shape; all values are seeded draws (see ``synth.c``).

Distributions (N(0, s) means standard deviation s; fan_in is the length of the
contraction each weight row takes part in):
  x          bf16  N(0, 1)                        [T][H]
  router_w   fp32  N(0, 0.02)                     [E][H]
  router_b   fp32  N(0, 0.5) per expert, or a Zipf bias, or none
  w_gate_up  N(0, 1/sqrt(H))                      [E][2I][H]  rows [0,I) gate, [I,2I) up
  w_down     N(0, 1/sqrt(I))                      [E][H][I]
  shared_*   same law with I_s                    [2I_s][H], [H][I_s]
  shared_gate_w fp32 N(0, 0.02)                   [H]
Weights are bf16, or OCP E4M3FN codes with one fp32 scale per output row (amax/448).

Zipf variant: b_e = beta * ln p_{pi(e)}, p_r proportional to r^(-s) over ranks r = 1..E,
pi a seeded permutation; beta is the value ``calibrate_zipf.py`` found so that the
seed-0, T=32 draw leaves about 40% of the experts untouched.
"""
from dataclasses import dataclass, replace
import math

import numpy as np

from . import normal_bf16, normal_f32, normal_fp8_rows, normal_mxfp4_rows, permutation

TAG_X, TAG_RW, TAG_RB, TAG_GU, TAG_DN, TAG_SGU, TAG_SDN, TAG_SG, TAG_PERM = range(1, 10)
REPLICA_STRIDE = 100


@dataclass(frozen=True)
class LayerConfig:
    name: str
    H: int
    E: int
    k: int
    I: int
    I_s: int          # 0: no shared expert
    wtype: str        # 'bf16' | 'fp8' | 'fp8a8' (fp8 weights; the prefill path also quantises activations)
                      # | 'mxfp4' (4-bit E2M1 codes with an E8M0 scale per 32 values; decode path only)
    bias: str         # 'none' | 'normal' | 'zipf'
    BM: int
    bias_std: float = 0.5
    zipf_s: float = 1.1
    zipf_beta: float = 0.0
    router_std: float = 0.02
    renormalize: bool = True


# beta fixed by synth/calibrate_zipf.py (seed 0, T = 32): see that script's output.
ZIPF_BETA = 0.1795  # seed 0, T=32: 39.8% of 256 experts untouched

CONFIGS = {
    # tiny parity case: T=4, H=256, 16 experts, top-2, I=128, no shared expert, BM=16
    "tiny": LayerConfig("tiny", H=256, E=16, k=2, I=128, I_s=0, wtype="bf16", bias="none", BM=16),
    # Qwen3.6-35B-A3B-like decode / verify layer: T in {1, 8} (and 32 for two 16-position blocks)
    "qwen36_a3b": LayerConfig("qwen36_a3b", H=2048, E=256, k=8, I=512, I_s=512, wtype="bf16", bias="normal", BM=16),
    # same layer with a Zipf(1.1) expert popularity realised through the router bias
    "qwen36_a3b_zipf": LayerConfig("qwen36_a3b_zipf", H=2048, E=256, k=8, I=512, I_s=512, wtype="bf16",
                                   bias="zipf", BM=16, zipf_beta=ZIPF_BETA),
    # Qwen3.8-Flash-Next-like layer with fp8 e4m3 weights and per-row scales: T in {1, 6}
    "flash_next_fp8": LayerConfig("flash_next_fp8", H=2048, E=512, k=10, I=512, I_s=512, wtype="fp8",
                                  bias="normal", BM=16),
    # prefill chunk: the Qwen3.6-like shapes at T=4096 with an unbiased router, BM=64
    "prefill": LayerConfig("prefill", H=2048, E=256, k=8, I=512, I_s=512, wtype="bf16", bias="none", BM=64),
    # the prefill chunk with fp8 e4m3 experts (row scales), the same shapes
    "prefill_fp8": LayerConfig("prefill_fp8", H=2048, E=256, k=8, I=512, I_s=512, wtype="fp8", bias="none", BM=64),
    # the T=8 verify layer with MXFP4 routed and shared experts (4-bit decode GEMV)
    "qwen36_a3b_mxfp4": LayerConfig("qwen36_a3b_mxfp4", H=2048, E=256, k=8, I=512, I_s=512, wtype="mxfp4",
                                    bias="normal", BM=16),
    # the same fp8 experts with fp8 activations (one scale per token row and per h row)
    "prefill_fp8a8": LayerConfig("prefill_fp8a8", H=2048, E=256, k=8, I=512, I_s=512, wtype="fp8a8", bias="none",
                                 BM=64),
}

# Token counts each recipe is run at.
TOKENS = {"tiny": (4,), "qwen36_a3b": (1, 8, 32), "qwen36_a3b_zipf": (32,), "flash_next_fp8": (1, 6),
          "prefill": (4096,), "prefill_fp8": (4096,), "prefill_fp8a8": (4096,), "qwen36_a3b_mxfp4": (1, 8)}


def _tag(tid, replica):
    return tid + REPLICA_STRIDE * replica


def _weights(cfg, seed, tid, replica, shape, std):
    if cfg.wtype == "bf16":
        return normal_bf16(seed, _tag(tid, replica), shape, std), None
    if cfg.wtype == "mxfp4":
        return normal_mxfp4_rows(seed, _tag(tid, replica), shape, std)
    return normal_fp8_rows(seed, _tag(tid, replica), shape, std)


def zipf_bias(E, s, beta, seed=0, replica=0):
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    perm = permutation(seed, _tag(TAG_PERM, replica), E)
    return (beta * np.log(p[perm])).astype(np.float32)


def make_layer(cfg, seed=0, replica=0, with_experts=True):
    """Host arrays of one layer replica (dict).  ``with_experts=False`` skips the expert banks."""
    H, E, I, I_s = cfg.H, cfg.E, cfg.I, cfg.I_s
    L = dict(name=cfg.name, H=H, E=E, k=cfg.k, I=I, I_s=I_s, wtype=cfg.wtype, BM=cfg.BM,
             renormalize=cfg.renormalize)
    L["router_w"] = normal_f32(seed, _tag(TAG_RW, replica), (E, H), cfg.router_std)
    if cfg.bias == "normal":
        L["router_b"] = normal_f32(seed, _tag(TAG_RB, replica), (E,), cfg.bias_std)
    elif cfg.bias == "zipf":
        L["router_b"] = zipf_bias(E, cfg.zipf_s, cfg.zipf_beta, seed, replica)
    else:
        L["router_b"] = None
    if with_experts:
        L["w_gate_up"], L["s_gate_up"] = _weights(cfg, seed, TAG_GU, replica, (E, 2 * I, H), 1.0 / math.sqrt(H))
        L["w_down"], L["s_down"] = _weights(cfg, seed, TAG_DN, replica, (E, H, I), 1.0 / math.sqrt(I))
        if I_s > 0:
            L["shared_w_gate_up"], L["shared_s_gate_up"] = _weights(cfg, seed, TAG_SGU, replica, (2 * I_s, H),
                                                                    1.0 / math.sqrt(H))
            L["shared_w_down"], L["shared_s_down"] = _weights(cfg, seed, TAG_SDN, replica, (H, I_s),
                                                              1.0 / math.sqrt(I_s))
    if I_s > 0:
        L["shared_gate_w"] = normal_f32(seed, _tag(TAG_SG, replica), (H,), 0.02)
    return L


def make_tokens(cfg, T, seed=0, replica=0):
    """bf16 tokens [T][H]; token t of a T-token draw equals token t of any longer draw."""
    return normal_bf16(seed, _tag(TAG_X, replica), (T, cfg.H), 1.0)


def with_shape(cfg, **kw):
    """A copy of a recipe with some fields changed (for edge-case tests)."""
    return replace(cfg, **kw)
