"""Parity of the HIP path with the CPU oracle, through the C ABI (GPU only).

Bars: routing ids and every alignment array bit-exact; router weights within 1e-6;
logits within 1e-5 (1 + |L|) of fp64; layer output relL2 <= 1e-3 (bf16 weights) or
<= 5e-3 (fp8 weights) and max-abs <= 1e-2 max|ref|; bitwise identical output run to run.
The oracle routes from the logits the device produced, so a legitimate fp32 near-tie
cannot flip an expert between the two sides; the logits are checked separately.
"""
import hashlib
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from synth import configs
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import speculative_verify_moe_amd  # noqa: F401  (fails loudly if the library is missing)
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------- top-k routing

ROUTE_CASES = [
    # name, T, E, k, kind, renorm
    ("tiny", 4, 16, 2, "normal", True),
    ("qwen36_T8", 8, 256, 8, "normal", True),
    ("flash_T6", 6, 512, 10, "normal", True),
    ("prefill_T4096", 4096, 256, 8, "normal", True),
    ("ties", 100, 64, 8, "ties", True),
    ("E1024_k32", 33, 1024, 32, "normal", True),
    ("E1", 5, 1, 1, "normal", True),
    ("E100_ragged_lanes", 37, 100, 7, "normal", True),
    ("no_renorm", 19, 256, 8, "normal", False),
    ("spread", 7, 300, 5, "wide", True),
]


def _logits(kind, T, E, seed):
    rng = np.random.default_rng(seed)
    if kind == "ties":
        return rng.choice(np.array([-1.0, -0.0, 0.0, 1.0], np.float32), size=(T, E))
    if kind == "wide":
        return (rng.standard_normal((T, E)) * 30).astype(np.float32)
    return rng.standard_normal((T, E)).astype(np.float32)


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: c[0])
def test_route_topk_bit_exact(case):
    from speculative_verify_moe_amd import moe_route_topk
    name, T, E, k, kind, renorm = case
    _say(f"[route] {name} T={T} E={E} k={k}")
    lg = _logits(kind, T, E, zlib.crc32(name.encode()) % 1000)
    ids, w = moe_route_topk(torch.from_numpy(lg).cuda(), k, renormalize=renorm)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.route_topk(lg, k, renorm)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.max(np.abs(w.cpu().numpy().astype(np.float64) - w_ref)) <= 1e-6


# ---------------------------------------------------------------- alignment

ALIGN_CASES = [
    # name, T, k, E, BM, extra capacity blocks
    ("tiny", 4, 2, 16, 16, 0),
    ("qwen36_T8", 8, 8, 256, 16, 0),
    ("qwen36_T32", 32, 8, 256, 16, 3),
    ("flash_T6", 6, 10, 512, 16, 0),
    ("one_block_max", 64, 16, 1024, 32, 0),
    ("bm128", 50, 8, 64, 128, 1),
    ("prefill_T4096", 4096, 8, 256, 64, 0),
    ("prefill_flash", 4096, 10, 512, 64, 2),
    ("large_ragged", 1337, 3, 200, 16, 1),
    ("E1", 300, 1, 1, 64, 0),
    # the multi-block alignment just past the one-block size, 1024 experts, and every slot in
    # one of 16 hot experts (long runs of equal ids across the chunks)
    ("chunks_1025", 205, 5, 37, 16, 0),
    ("chunks_16385", 3277, 5, 300, 32, 1),
    ("chunks_E1024", 4096, 8, 1024, 64, 0),
    ("chunks_hot", 4096, 8, 256, 64, 0, 16),
]


@pytest.mark.parametrize("case", ALIGN_CASES, ids=lambda c: c[0])
def test_align_bit_exact(case):
    from speculative_verify_moe_amd import moe_align, moe_align_capacity
    name, T, k, E, BM, extra = case[:6]
    hot = case[6] if len(case) > 6 else E  # the experts the slots are drawn from
    _say(f"[align] {name} T={T} k={k} E={E} BM={BM}")
    rng = np.random.default_rng(T * 7 + E)
    ids = np.stack([rng.permutation(hot)[:k] for _ in range(T)]).astype(np.int32)
    cap = moe_align_capacity(T, k, E, BM) + extra * BM
    got = moe_align(torch.from_numpy(ids).cuda(), E, BM, cap=cap)
    torch.cuda.synchronize()
    ref = oracle.align(ids, E, BM, cap)
    assert np.array_equal(got["sorted_ids"].cpu().numpy(), ref["sorted_ids"])
    assert np.array_equal(got["block_expert"].cpu().numpy(), ref["block_expert"])
    assert np.array_equal(got["expert_counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(got["expert_offsets"].cpu().numpy(), ref["offsets"])
    assert int(got["num_padded"].cpu().numpy()[0]) == ref["num_padded"]


def test_align_of_device_routing_at_prefill_size():
    """Route then align on the device at T=4096; both stages bit-exact."""
    from speculative_verify_moe_amd import moe_align, moe_route_topk
    lg = _logits("normal", 4096, 256, 5)
    ids, _ = moe_route_topk(torch.from_numpy(lg).cuda(), 8)
    al = moe_align(ids, 256, 64)
    torch.cuda.synchronize()
    ids_ref, _ = oracle.route_topk(lg, 8)
    ref = oracle.align(ids_ref, 256, 64, al["cap"])
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.array_equal(al["sorted_ids"].cpu().numpy(), ref["sorted_ids"])


# ---------------------------------------------------------------- whole layer

LAYER_CASES = [
    # name, recipe, T: every output element of every token is compared with the oracle
    ("tiny_T4", "tiny", 4),
    ("tiny_T1", "tiny", 1),
    ("tiny_T9", "tiny", 9),
    ("tiny_T64", "tiny", 64),
    ("tiny_T65_prefill", "tiny", 65),
    ("tiny_T100_prefill", "tiny", 100),
    ("tiny_T600_prefill", "tiny", 600),
    ("qwen36_T1", "qwen36_a3b", 1),
    ("qwen36_T8", "qwen36_a3b", 8),
    ("qwen36_T5", "qwen36_a3b", 5),
    ("qwen36_T16", "qwen36_a3b", 16),
    ("qwen36_T32", "qwen36_a3b", 32),
    ("qwen36_zipf_T32", "qwen36_a3b_zipf", 32),
    ("qwen36_T64", "qwen36_a3b", 64),
    ("qwen36_T40", "qwen36_a3b", 40),
    ("flash_fp8_T1", "flash_next_fp8", 1),
    ("flash_fp8_T6", "flash_next_fp8", 6),
    ("flash_fp8_T16", "flash_next_fp8", 16),
    ("prefill_T4096", "prefill", 4096),
    ("prefill_T200", "prefill", 200),
    ("prefill_fp8_T4096", "prefill_fp8", 4096),
    ("prefill_fp8_T200", "prefill_fp8", 200),
    ("qwen36_mxfp4_T1", "qwen36_a3b_mxfp4", 1),
    ("qwen36_mxfp4_T8", "qwen36_a3b_mxfp4", 8),
    ("qwen36_mxfp4_T16", "qwen36_a3b_mxfp4", 16),
    ("qwen36_mxfp4_T32", "qwen36_a3b_mxfp4", 32),
    ("qwen36_mxfp4_T48", "qwen36_a3b_mxfp4", 48),
    ("flash_fp8_T40", "flash_next_fp8", 40),
    ("prefill_fp8a8_T4096", "prefill_fp8a8", 4096),
    ("prefill_fp8a8_T200", "prefill_fp8a8", 200),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=lambda c: c[0])
def test_layer_parity(case):
    name, recipe, T = case
    _say(f"[layer] {name} recipe={recipe} T={T}")
    cfg = configs.CONFIGS[recipe]
    L = G.host_layer(cfg)
    x = configs.make_tokens(cfg, T)
    rep = {}
    G.check_layer(L, x, report=rep)
    G.say_margin(name, rep)
    if cfg.wtype == "fp8a8" and not G.runs_decode_path(T, cfg.k):
        _check_act8_is_quantised(L, x, rep)


def test_layer_tiny_variants():
    """Ragged and degenerate shapes at the tiny size: k = E, k = 1, one expert, shared expert of
    a different width, no renormalisation, H not a multiple of 512."""
    variants = [dict(k=16), dict(k=1), dict(E=1, k=1), dict(I_s=64, bias="normal"), dict(I_s=192),
                dict(renormalize=False, I_s=128), dict(H=192, I=64), dict(H=128, I=256, I_s=64)]
    for v in variants:
        for T in (3, 70):
            cfg = configs.with_shape(configs.CONFIGS["tiny"], **v)
            if T > 64 and (cfg.H % 128 != 0):
                continue
            _say(f"[layer-variant] {v} T={T}")
            L = configs.make_layer(cfg, seed=11)
            x = configs.make_tokens(cfg, T, seed=11)
            rep = {}
            G.check_layer(L, x, report=rep)
            G.say_margin(f"tiny{v}_T{T}", rep)


def test_fp8_prefill_tiny_shapes():
    """fp8 weights on the prefill (MFMA) path at the tiny size: ragged T, with and without a
    shared expert, a shared width different from I."""
    for v in (dict(wtype="fp8"), dict(wtype="fp8", I_s=128, bias="normal"), dict(wtype="fp8", I_s=64, k=4)):
        for T in (65, 100, 600):
            cfg = configs.with_shape(configs.CONFIGS["tiny"], **v)
            _say(f"[fp8-prefill] {v} T={T}")
            L = configs.make_layer(cfg, seed=5)
            x = configs.make_tokens(cfg, T, seed=5)
            rep = {}
            G.check_layer(L, x, report=rep)
            G.say_margin(f"tiny{v}_T{T}", rep)


def _check_act8_is_quantised(L, x, rep):
    """The fp8-activation result sits much closer to the fp8-activation oracle than to the
    weights-only one: the quantisation decisions (codes and scales) are the oracle's."""
    ref_w8 = oracle.moe_layer(x, dict(L, wtype="fp8"), rep["ids"], rep["w"], tokens=rep["tokens"], rounding=True)
    d_a8 = np.linalg.norm(rep["got"] - rep["ref"])
    d_q = np.linalg.norm(rep["ref"] - ref_w8)
    assert d_q > 0 and d_a8 <= 0.1 * d_q, f"device-oracle distance {d_a8:.3e} vs quantisation effect {d_q:.3e}"


def test_fp8_activations_follow_the_oracle_quantisation():
    """A ragged chunk (200 tokens) of the fp8-activation layer; the 4096-token chunk runs the
    same check inside its layer case."""
    cfg = configs.CONFIGS["prefill_fp8a8"]
    _say("[fp8a8] quantisation decisions T=200")
    L = G.host_layer(cfg)
    x = configs.make_tokens(cfg, 200)
    rep = {}
    G.check_layer(L, x, report=rep)
    _check_act8_is_quantised(L, x, rep)


def test_fp8a8_prefill_tiny_shapes():
    """fp8 weights and fp8 activations on the prefill path at the tiny size: ragged T, with and
    without a shared expert; the decode path of the same bank streams bf16 activations."""
    for v in (dict(wtype="fp8a8"), dict(wtype="fp8a8", I_s=128, bias="normal"), dict(wtype="fp8a8", I_s=256, k=4)):
        for T in (6, 65, 100, 600):
            cfg = configs.with_shape(configs.CONFIGS["tiny"], **v)
            _say(f"[fp8a8-prefill] {v} T={T}")
            L = configs.make_layer(cfg, seed=5)
            x = configs.make_tokens(cfg, T, seed=5)
            rep = {}
            G.check_layer(L, x, report=rep)
            G.say_margin(f"tiny{v}_T{T}", rep)
            if not G.runs_decode_path(T, cfg.k):
                _check_act8_is_quantised(L, x, rep)


def test_mxfp4_tiny_shapes():
    """MXFP4 experts at the tiny size: one token to a full decode block, with and without a
    shared expert, k = 1, and H not a multiple of 512; a prefill chunk is refused."""
    from speculative_verify_moe_amd import MoeError, moe_layer_forward
    for v in (dict(wtype="mxfp4"), dict(wtype="mxfp4", I_s=64, bias="normal"), dict(wtype="mxfp4", k=1),
              dict(wtype="mxfp4", H=192, I=64, I_s=128)):
        for T in (1, 4, 64):
            cfg = configs.with_shape(configs.CONFIGS["tiny"], **v)
            _say(f"[mxfp4] {v} T={T}")
            L = configs.make_layer(cfg, seed=6)
            rep = {}
            G.check_layer(L, configs.make_tokens(cfg, T, seed=6), report=rep)
            G.say_margin(f"tiny{v}_T{T}", rep)
    cfg = configs.with_shape(configs.CONFIGS["tiny"], wtype="mxfp4")
    D = G.device_layer(configs.make_layer(cfg, seed=6))
    with pytest.raises(MoeError, match="decode path only"):
        moe_layer_forward(G.to_dev_bf16(configs.make_tokens(cfg, 100, seed=6)), D)


def test_fp8a8_needs_inter_multiple_of_128_on_the_prefill_path():
    from speculative_verify_moe_amd import MoeError, moe_layer_forward
    cfg = configs.with_shape(configs.CONFIGS["tiny"], wtype="fp8a8", I=64)
    D = G.device_layer(configs.make_layer(cfg, seed=1))
    x = G.to_dev_bf16(configs.make_tokens(cfg, 100, seed=1))
    with pytest.raises(MoeError, match="inter % 128"):
        moe_layer_forward(x, D)


def test_zero_tokens_is_a_no_op():
    from speculative_verify_moe_amd import moe_layer_forward
    cfg = configs.CONFIGS["tiny"]
    D = G.device_layer(G.host_layer(cfg))
    x = torch.empty((0, cfg.H), dtype=torch.bfloat16, device="cuda")
    out = moe_layer_forward(x, D)
    torch.cuda.synchronize()
    assert out.shape == (0, cfg.H)


def test_zero_input_gives_zero_output():
    cfg = configs.with_shape(configs.CONFIGS["tiny"], I_s=64)
    L = configs.make_layer(cfg, seed=2)
    x = np.zeros((5, cfg.H), np.uint16)
    out, _, _, _ = G.run_layer(L, x)
    assert np.all((out & 0x7FFF) == 0)


# ---------------------------------------------------------------- determinism, batch invariance

def _digest(bits):
    return hashlib.sha256(bits.tobytes()).hexdigest()


@pytest.mark.parametrize("recipe,T,runs", [("qwen36_a3b", 8, 20), ("flash_next_fp8", 6, 10), ("prefill", 4096, 5),
                                           ("qwen36_a3b_mxfp4", 8, 10),
                                           ("prefill_fp8a8", 4096, 3),
                                           ("prefill_fp8", 4096, 3)])
def test_bitwise_deterministic(recipe, T, runs):
    from speculative_verify_moe_amd import moe_layer_forward
    _say(f"[determinism] {recipe} T={T} runs={runs}")
    cfg = configs.CONFIGS[recipe]
    D = G.device_layer(G.host_layer(cfg))
    x = G.to_dev_bf16(configs.make_tokens(cfg, T))
    digests = set()
    for _ in range(runs):
        out = moe_layer_forward(x, D)
        torch.cuda.synchronize()
        digests.add(_digest(G.bf16_bits(out)))
    assert len(digests) == 1


BATCH_INVARIANCE_CASES = [
    # recipe, T, four-kernel path forced
    ("qwen36_a3b", 8, False), ("qwen36_a3b_mxfp4", 8, False), ("flash_next_fp8", 6, False),
    ("qwen36_a3b", 16, False), ("qwen36_a3b", 32, False), ("qwen36_a3b", 64, False),
    ("qwen36_a3b_zipf", 32, False), ("qwen36_a3b_mxfp4", 32, False), ("qwen36_a3b_mxfp4", 48, False),
    ("flash_next_fp8", 40, False), ("flash_next_fp8", 16, False), ("qwen36_a3b_zipf", 16, False),
    ("qwen36_a3b", 8, True), ("qwen36_a3b", 32, True), ("flash_next_fp8", 6, True), ("qwen36_a3b_mxfp4", 8, True),
]


@pytest.mark.parametrize("recipe,T,four", BATCH_INVARIANCE_CASES)
def test_verify_block_rows_equal_single_token_calls(recipe, T, four):
    """Row t of a T-token verify-block call is bitwise the one-token call on token t (decode
    path), whichever decode kernels each call takes; with ``four`` both run as four kernels."""
    import speculative_verify_moe_amd as moe
    from speculative_verify_moe_amd import moe_layer_forward
    _say(f"[batch-invariance] {recipe} T={T} four_kernel={four}")
    cfg = configs.CONFIGS[recipe]
    D = G.device_layer(G.host_layer(cfg))
    xb = configs.make_tokens(cfg, T)
    x = G.to_dev_bf16(xb)
    if four:
        moe.moe_set_option(moe.MOE_OPT_DECODE_FUSED, 0)
    try:
        block = G.bf16_bits(moe_layer_forward(x, D))
        for t in range(T):
            one = G.bf16_bits(moe_layer_forward(x[t:t + 1].contiguous(), D))
            assert np.array_equal(one[0], block[t]), f"row {t}"
    finally:
        moe.moe_set_option(moe.MOE_OPT_DECODE_FUSED, 1)


# ---------------------------------------------------------------- experts entry point

@pytest.mark.parametrize("recipe,T,BM", [("tiny", 4, 16), ("qwen36_a3b", 8, 16), ("tiny", 300, 64),
                                         ("prefill", 4096, 64), ("tiny", 130, 128), ("prefill_fp8", 4096, 64),
                                         ("prefill_fp8a8", 4096, 64), ("qwen36_a3b_mxfp4", 8, 16)])
def test_experts_forward_parity(recipe, T, BM):
    from speculative_verify_moe_amd import moe_align, moe_experts_forward, moe_route_topk
    _say(f"[experts] {recipe} T={T} BM={BM}")
    cfg = configs.CONFIGS[recipe]
    L = G.host_layer(cfg)
    xb = configs.make_tokens(cfg, T)
    lg = oracle.router_logits(xb, L["router_w"], L["router_b"]).astype(np.float32)
    ids, w = moe_route_topk(torch.from_numpy(lg).cuda(), cfg.k)
    al = moe_align(ids, cfg.E, BM)
    D = G.device_layer(L)
    routed = D.routed
    out = moe_experts_forward(G.to_dev_bf16(xb), routed, cfg.k, w, al, BM)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.route_topk(lg, cfg.k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    Lr = dict(G.oracle_layer_for_path(L, T), I_s=0)
    ref = oracle.moe_layer(xb, Lr, ids_ref, w_ref, rounding=True)
    got = G.bf16_values(G.bf16_bits(out))
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    mx = np.max(np.abs(got - ref))
    G.say_margin(f"experts_{recipe}_T{T}_BM{BM}", dict(rel_l2=rel, max_abs=mx, max_ref=np.max(np.abs(ref)),
                                                      wtype=Lr["wtype"]))
    assert rel <= G.TOL[Lr["wtype"]]
    assert mx <= G.MAX_ABS[Lr["wtype"]] * np.max(np.abs(ref))


# ---------------------------------------------------------------- the two decode paths

# (recipe, shape overrides, T, whether the fused kernel takes it): the fused kernel keeps the
# tokens and h in LDS (up to ~16 tokens at these widths) and, for MXFP4, whole 512-element
# lane groups; a 4-bit H of 512 or 1536 leaves lane groups past the row
_FOUR_KERNEL_CASES = [("tiny", {}, 4, True), ("tiny", {}, 64, True), ("qwen36_a3b", {}, 8, True),
                      # 16 tokens: top-k and alignment in one block; 17: top-k over the chip first
                      ("tiny", {}, 16, True), ("tiny", {}, 17, True), ("qwen36_a3b", {}, 17, False),
                      ("qwen36_a3b", {}, 1, True), ("qwen36_a3b", {}, 32, False), ("flash_next_fp8", {}, 6, True),
                      # 12 and 16 tokens: the fused kernel's h rows wrap around its LDS ring
                      ("qwen36_a3b", {}, 12, True), ("qwen36_a3b", {}, 16, True), ("flash_next_fp8", {}, 16, True),
                      ("qwen36_a3b_mxfp4", {}, 16, True),
                      # the ring without a shared expert
                      ("tiny", dict(H=2048, E=64, k=8, I=512, I_s=0), 16, True),
                      ("qwen36_a3b_mxfp4", {}, 8, True), ("qwen36_a3b_mxfp4", {}, 1, True),
                      ("tiny", dict(wtype="mxfp4"), 4, False),
                      ("tiny", dict(wtype="mxfp4", H=512, I=512, I_s=512, bias="normal"), 8, True),
                      ("tiny", dict(wtype="mxfp4", H=1536, I=512, I_s=512, k=4), 5, True),
                      ("tiny", dict(wtype="mxfp4", H=1024, I=512, I_s=0), 3, True)]


@pytest.mark.parametrize("recipe,shape,T,expect_fused", _FOUR_KERNEL_CASES)
def test_four_kernel_decode_path_matches_oracle_and_fused(recipe, shape, T, expect_fused):
    """MOE_OPT_DECODE_FUSED = 0 runs the decode block as four kernels; it must pass the same
    bars and give bitwise the same output and routing as the fused cooperative kernel."""
    import speculative_verify_moe_amd as moe
    _say(f"[four-kernel] {recipe} {shape} T={T}")
    cfg = configs.with_shape(configs.CONFIGS[recipe], **shape) if shape else configs.CONFIGS[recipe]
    L = G.host_layer(cfg) if not shape else configs.make_layer(cfg, seed=9)
    x = configs.make_tokens(cfg, T)
    D = G.device_layer(L)
    assert ("decode-fused" in moe.moe_describe_plan(T, D)) == expect_fused
    if expect_fused:
        G.check_layer(L, x)
    fused = G.run_layer(L, x)
    moe.moe_set_option(moe.MOE_OPT_DECODE_FUSED, 0)
    try:
        assert "decode-fused" not in moe.moe_describe_plan(T, D)
        G.check_layer(L, x)
        four = G.run_layer(L, x)
    finally:
        moe.moe_set_option(moe.MOE_OPT_DECODE_FUSED, 1)
    assert np.array_equal(fused[0], four[0]), "outputs differ between the fused and four-kernel paths"
    assert np.array_equal(fused[2], four[2]) and np.array_equal(fused[3], four[3])
    assert np.array_equal(fused[1], four[1])



def test_alternating_inputs_on_one_workspace():
    """Two different token blocks alternate on one workspace; every call must equal the
    oracle-checked result of its own input (no value may survive from the previous call)."""
    from speculative_verify_moe_amd import moe_layer_forward, moe_layer_workspace_size
    for recipe, T in (("qwen36_a3b", 8), ("flash_next_fp8", 6), ("tiny", 4)):
        cfg = configs.CONFIGS[recipe]
        L = G.host_layer(cfg)
        D = G.device_layer(L)
        xa_b = configs.make_tokens(cfg, T, replica=1)
        xb_b = configs.make_tokens(cfg, T, replica=2)
        ref_a = G.check_layer(L, xa_b)
        ref_b = G.check_layer(L, xb_b)
        xa, xb = G.to_dev_bf16(xa_b), G.to_dev_bf16(xb_b)
        ws = torch.zeros((moe_layer_workspace_size(T, D),), dtype=torch.uint8, device="cuda")
        outs = []
        for i in range(12):
            outs.append(moe_layer_forward(xa if i % 2 == 0 else xb, D, ws=ws))
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(G.bf16_bits(o), ref_a if i % 2 == 0 else ref_b), f"{recipe} call {i}"


@pytest.mark.gpu
def test_concurrent_prefill_calls_from_two_threads():
    """Two host threads, each on its own stream and workspace, run prefill layers at the same time.
    Both calls' shared experts go through the device's one second stream (a lock spans each
    call's fork to join); every output equals the single-threaded result bitwise."""
    import threading
    from speculative_verify_moe_amd import moe_layer_forward, moe_layer_workspace_size
    cfg = configs.CONFIGS["prefill"]
    T = 200
    L = G.host_layer(cfg)
    D = G.device_layer(L)
    xs = [G.to_dev_bf16(configs.make_tokens(cfg, T, replica=r)) for r in (1, 2)]
    refs = [G.bf16_bits(moe_layer_forward(x, D)) for x in xs]
    torch.cuda.synchronize()
    results, errors = [None, None], []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                ws = torch.zeros((moe_layer_workspace_size(T, D),), dtype=torch.uint8, device="cuda")
                outs = [moe_layer_forward(xs[i], D, ws=ws) for _ in range(8)]
            s.synchronize()
            results[i] = [G.bf16_bits(o) for o in outs]
        except Exception as e:  # reported below, on the test's thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for i in range(2):
        for j, o in enumerate(results[i]):
            assert np.array_equal(o, refs[i]), f"thread {i} call {j}"


@pytest.mark.gpu
@pytest.mark.parametrize("recipe,T", [("qwen36_a3b", 8), ("flash_next_fp8", 6), ("qwen36_a3b", 32), ("prefill", 200)])
def test_graph_replays_equal_eager(recipe, T):
    """A layer call captured in a HIP graph: every replay (inputs changed in place between
    replays, eager calls on the same workspace in between) equals the eager result bitwise.
    The fused kernel's barrier tokens continue from the workspace, so replays need no reset."""
    from speculative_verify_moe_amd import moe_layer_forward, moe_layer_workspace_size
    cfg = configs.CONFIGS[recipe]
    L = G.host_layer(cfg)
    D = G.device_layer(L)
    xa = G.to_dev_bf16(configs.make_tokens(cfg, T, replica=1))
    xb = G.to_dev_bf16(configs.make_tokens(cfg, T, replica=2))
    ws = torch.zeros((moe_layer_workspace_size(T, D),), dtype=torch.uint8, device="cuda")
    ref_a = G.bf16_bits(moe_layer_forward(xa, D, ws=ws))
    ref_b = G.bf16_bits(moe_layer_forward(xb, D, ws=ws))
    x_static = xa.clone()
    out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # first use on this stream outside the capture
        moe_layer_forward(x_static, D, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe_layer_forward(x_static, D, out=out, ws=ws)
    torch.cuda.synchronize()
    for i in range(6):
        x_static.copy_(xa if i % 2 == 0 else xb)
        g.replay()
        torch.cuda.synchronize()
        got = G.bf16_bits(out)
        assert np.array_equal(got, ref_a if i % 2 == 0 else ref_b), f"{recipe} T={T} replay {i}"
        eager = G.bf16_bits(moe_layer_forward(xb, D, ws=ws))
        torch.cuda.synchronize()
        assert np.array_equal(eager, ref_b), f"{recipe} T={T} eager call after replay {i}"


# ---------------------------------------------------------------- the fused kernel's waits

@pytest.mark.parametrize("recipe,T", [("qwen36_a3b", 8), ("qwen36_a3b", 1), ("flash_next_fp8", 6),
                                      ("qwen36_a3b_mxfp4", 8), ("tiny", 64), ("tiny", 3), ("qwen36_a3b", 16),
                                      ("qwen36_a3b_mxfp4", 16)])
def test_fused_waits_never_give_up(recipe, T):
    """Normal use of the fused decode kernel: over many calls on one workspace no wait gives up
    (the workspace's status word stays 0) and every output is finite and the same."""
    import speculative_verify_moe_amd as moe
    _say(f"[status] {recipe} T={T}")
    cfg = configs.CONFIGS[recipe]
    D = G.device_layer(G.host_layer(cfg))
    assert "decode-fused" in moe.moe_describe_plan(T, D)
    x = G.to_dev_bf16(configs.make_tokens(cfg, T))
    ws = torch.zeros((moe.moe_layer_workspace_size(T, D),), dtype=torch.uint8, device="cuda")
    outs = [moe.moe_layer_forward(x, D, ws=ws) for _ in range(40)]
    torch.cuda.synchronize()
    assert moe.moe_workspace_status(ws) == 0
    first = G.bf16_bits(outs[0])
    assert np.all(np.isfinite(G.bf16_values(first)))
    for o in outs[1:]:
        assert np.array_equal(G.bf16_bits(o), first)


def test_one_workspace_serves_calls_of_every_size():
    """Fused decode blocks, four-kernel decode blocks and prefill chunks take turns on one
    zeroed workspace: every call equals the same call on a workspace of its own, bitwise, and
    no fused wait gives up."""
    import speculative_verify_moe_amd as moe
    cfg = configs.CONFIGS["qwen36_a3b"]
    D = G.device_layer(G.host_layer(cfg))
    sizes = (8, 32, 100, 3, 64, 1)
    xs = {T: G.to_dev_bf16(configs.make_tokens(cfg, T, replica=T)) for T in sizes}
    refs = {}
    for T in sizes:
        ws_own = torch.zeros((moe.moe_layer_workspace_size(T, D),), dtype=torch.uint8, device="cuda")
        refs[T] = G.bf16_bits(moe.moe_layer_forward(xs[T], D, ws=ws_own))
    ws = torch.zeros((max(moe.moe_layer_workspace_size(T, D) for T in sizes),), dtype=torch.uint8, device="cuda")
    for rnd in range(3):
        for T in sizes:
            _say(f"[shared-workspace] round {rnd} T={T}: {moe.moe_describe_plan(T, D).split()[0]}")
            got = G.bf16_bits(moe.moe_layer_forward(xs[T], D, ws=ws))
            assert np.array_equal(got, refs[T]), f"round {rnd} T={T}"
    assert moe.moe_workspace_status(ws) == 0
