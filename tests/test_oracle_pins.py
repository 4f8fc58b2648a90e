"""Pins of the fp64 CPU oracle against things other than itself.

Every check here compares the oracle with an independent construction: values worked by
hand (``tests/golden``), closed forms, library routines (torch casts, torch's SiLU,
scipy's softmax, Python's sort), brute force over all experts with masked gates, or
invariants that any correct result must satisfy.  ``test_oracle_mutants.py`` plants
mistakes in a copy of the oracle and checks that this file catches each of them.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from synth import configs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- helpers (independent of the oracle)

def bf16_codes_to_f64(codes):
    """bf16 bit patterns -> float64 through torch's own bfloat16 type."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def bf16_rne_bits(v):
    """float64 -> nearest-even bfloat16 value (float64), by integer rounding of the double's bits.

    Valid for zero and for magnitudes in the bf16 normal range, which is all these tests use."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    u = v.view(np.uint64).copy()
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    u = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    return u.view(np.float64)


def fp8_codes_to_f64(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def silu_np(g):
    return g * scipy.special.expit(g)


def brute_topk(logits_row, k):
    """Rank by Python's sort with key (NaN last, -logit, index)."""
    order = sorted(range(len(logits_row)),
                   key=lambda e: (1 if math.isnan(logits_row[e]) else 0,
                                  0.0 if math.isnan(logits_row[e]) else -float(logits_row[e]), e))
    return order[:k]


def brute_align(ids, E, BM, cap):
    """Alignment built by sorting (expert, slot) pairs, then laying segments out with padding."""
    flat = [int(v) for v in np.asarray(ids).ravel()]
    n = len(flat)
    pairs = sorted((e, i) for i, e in enumerate(flat))
    sorted_ids = [n] * cap
    block_expert = [-1] * (cap // BM)
    counts = [0] * E
    offsets = [0] * (E + 1)
    pos = 0
    for e in range(E):
        mine = [i for (ee, i) in pairs if ee == e]
        counts[e] = len(mine)
        offsets[e] = pos
        for r, i in enumerate(mine):
            sorted_ids[pos + r] = i
        seg = -(-len(mine) // BM) * BM
        for b in range(pos // BM, (pos + seg) // BM):
            block_expert[b] = e
        pos += seg
    offsets[E] = pos
    return dict(sorted_ids=np.array(sorted_ids, np.int32), block_expert=np.array(block_expert, np.int32),
                counts=np.array(counts, np.int32), offsets=np.array(offsets, np.int32), num_padded=pos)


def dense_masked_layer(x, L, gates, rounding):
    """Every token through EVERY expert, weighted by a gate vector that is zero off the top-k.

    bf16 weights only.  Uses numpy einsum contractions; rounding points (when asked) use
    bf16_rne_bits."""
    rnd = bf16_rne_bits if rounding else (lambda a: a)
    I, I_s = L["I"], L.get("I_s", 0)
    X = bf16_codes_to_f64(x)
    Wgu = bf16_codes_to_f64(L["w_gate_up"])
    Wd = bf16_codes_to_f64(L["w_down"])
    G = np.einsum("th,erh->ter", X, Wgu[:, :I, :])
    U = np.einsum("th,erh->ter", X, Wgu[:, I:, :])
    Hh = rnd(silu_np(G) * U)
    Y = rnd(np.einsum("ter,eor->teo", Hh, Wd))
    out = np.einsum("te,teo->to", gates, Y)
    if I_s > 0:
        Sgu = bf16_codes_to_f64(L["shared_w_gate_up"])
        Sd = bf16_codes_to_f64(L["shared_w_down"])
        gam = scipy.special.expit(X @ L["shared_gate_w"].astype(np.float64))
        Hs = rnd(silu_np(X @ Sgu[:I_s].T) * (X @ Sgu[I_s:].T))
        Ys = rnd(Hs @ Sd.T)
        out = out + gam[:, None] * Ys
    return rnd(out)


def gates_from_topk(ids, w, E):
    g = np.zeros((ids.shape[0], E))
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            g[t, ids[t, j]] = w[t, j]
    return g


def routed(x, L, k, renormalize=True):
    lg = oracle.router_logits(x, L["router_w"], L["router_b"]).astype(np.float32)
    return oracle.route_topk(lg, k, renormalize)


# ---------------------------------------------------------------- number formats

def test_bf16_value_matches_torch_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bf16_codes_to_f64(codes)
    got = oracle.bf16_value(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(ref[~both_nan], got[~both_nan])


def test_bf16_round_matches_torch_on_fp32_exact_values():
    rng = np.random.default_rng(1)
    f = rng.standard_normal(4000).astype(np.float32) * np.float32(3.0)
    u = f.view(np.uint32)
    # force exact ties (low half == 0x8000) on a quarter, with both parities of the kept lsb
    u[:1000] = (u[:1000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    f = u.view(np.float32)
    special = np.array([0.0, -0.0, 1e-40, -1e-40, 3e38, 3.3895313e38, 1.0, -2.5], dtype=np.float32)
    f = np.concatenate([f, special])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(f.astype(np.float64))
    assert np.array_equal(ref, got)


def test_bf16_round_is_a_single_rounding_from_double():
    # 1 + 2^-8 is an exact tie between 1 and 1 + 2^-7: ties to even -> 1.0
    assert oracle.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    # a hair above the tie must round up; rounding via float32 first would give 1.0
    assert oracle.bf16_round(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81
    assert oracle.bf16_round(np.array([-(1.0 + 3 * 2.0 ** -8)]))[0] == 0xBF82  # tie -> even (…82)


def test_fp8_value_all_codes_closed_form_and_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.fp8_value(codes)
    ref = fp8_codes_to_f64(codes)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            assert math.isnan(got[c]) and math.isnan(ref[c])
            continue
        closed = (2.0 ** -6) * m / 8 if e == 0 else (2.0 ** (e - 7)) * (1 + m / 8)
        closed = -closed if s else closed
        assert got[c] == closed == ref[c], c
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def _fp8_finite_table():
    """(codes, values) of every finite E4M3FN code, from torch's own float8 type."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    return codes, fp8_codes_to_f64(codes)


def _fp8_brute_encode(v):
    """Nearest finite code by search over all codes; a tie goes to the even mantissa."""
    codes, vals = _fp8_finite_table()
    d = np.abs(vals - float(v))
    best = d.min()
    cand = [int(c) for c, dd in zip(codes, d) if dd == best]
    if len(cand) > 1:  # +0 / -0, or a true tie between neighbours
        same_sign = [c for c in cand if (c >> 7) == (1 if math.copysign(1.0, v) < 0 else 0)]
        cand = same_sign or cand
        cand = [c for c in cand if c & 1 == 0] or cand
    return cand[0]


def _fp8_test_values(seed=0):
    rng = np.random.default_rng(seed)
    codes, vals = _fp8_finite_table()
    pos = np.unique(vals[vals > 0])
    mids = (pos[:-1] + pos[1:]) / 2  # exact ties (representable in fp32)
    v = [0.0, -0.0, 448.0, 448.5, 464.0, 470.0, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -6 - 2.0 ** -11]
    v += list(mids) + list(-mids)
    v += [np.nextafter(np.float32(m), np.float32(0)) for m in mids[::3]]
    v += [np.nextafter(np.float32(m), np.float32(1e9)) for m in mids[::3]]
    v += list(np.exp(rng.uniform(np.log(2.0 ** -12), np.log(600.0), 400)) * rng.choice([-1, 1], 400))
    return np.array(v, dtype=np.float32)


def test_fp8_encode_is_the_nearest_code_with_ties_to_even():
    v = _fp8_test_values()
    got = oracle.fp8_encode(v)
    for a, c in zip(v, got):
        assert c == _fp8_brute_encode(a), (float(a), int(c))


def test_fp8_encode_matches_torch_cast_in_range():
    v = _fp8_test_values(1)
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.fp8_encode(v), ref)


def test_fp8_encode_round_trips_every_finite_code():
    codes, vals = _fp8_finite_table()
    np.testing.assert_array_equal(oracle.fp8_encode(vals.astype(np.float32)), codes)


def test_activation_scale_is_the_least_power_of_two_covering_the_row():
    a = np.array([[28.0, 1.0, -2.0, 0.5], [0.0, -3.0, 1.5, 2.0], [0.0, 0.0, 0.0, 0.0],
                  [28.5, 1.0, 0.0, 0.0], [448.0, -1.0, 0.0, 0.0], [449.0, 0.0, 0.0, 0.0]])
    q, s = oracle.quantise_rows(a)
    # 28 = 448 / 16 exactly; 3 <= 448 / 128 = 3.5 but > 448 / 256; 28.5 > 448 / 16; 449 > 448
    np.testing.assert_array_equal(s, [2.0 ** -4, 2.0 ** -7, 1.0, 2.0 ** -3, 1.0, 2.0])
    # row 0: 28, 1, -2, 0.5 times 16 -> 448, 16, -32, 8 (codes 0x7E, 0x58, 0xE0, 0x50)
    np.testing.assert_array_equal(q[0], [0x7E, 0x58, 0xE0, 0x50])
    # row 1: -3 * 128 = -384 (0xFC), 1.5 * 128 = 192 (0x74), 2 * 128 = 256 (0x78)
    np.testing.assert_array_equal(q[1], [0x00, 0xFC, 0x74, 0x78])
    np.testing.assert_array_equal(q[2], 0)
    for r in range(a.shape[0]):
        assert np.abs(a[r]).max() <= 448.0 * s[r] and not np.abs(a[r]).max() <= 224.0 * s[r] or s[r] == 1.0


def _torch_fp8_dequant(v, s):
    """v / s (exact: s is a power of two) to the nearest e4m3 through torch's float8 cast, times s."""
    qv = torch.from_numpy((np.float32(v) / np.float32(s)).astype(np.float32)).to(torch.float8_e4m3fn)
    return qv.to(torch.float64).numpy() * float(s)


def _bf16_bits(v):
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _act8_expert(seed, up_weight=1.0):
    """One fp8 expert and one token on which every quantisation step can be followed by hand:
    x sits on the e4m3 grid times 2^-4 with amax 28 = 448 / 16 (scale 1/16 exactly); the gate
    rows pick x[1] = 16 with weight 4 (g = 64, and silu(64) == 64 in fp64); up row r picks
    x[src[r]] with weight wu[r] (row 0: x[0] = 28 with weight 1; the others ``up_weight``), so
    h_r = 64 * wu[r] * x[src[r]] exactly and the h row's amax is 64 * 28 (scale 4)."""
    rng = np.random.default_rng(seed)
    H, I = 64, 64
    codes, vals = _fp8_finite_table()
    ok = vals[(np.abs(vals) <= 256) & (np.abs(vals) >= 2.0 ** -3)]
    xv = rng.choice(ok, H) / 16.0
    xv[0], xv[1], xv[2] = 28.0, 16.0, 1.0
    x = _bf16_bits(xv)
    assert np.array_equal(bf16_codes_to_f64(x), xv)
    enc = {float(v): int(c) for c, v in zip(codes, vals)}
    w_gu = np.zeros((2 * I, H), np.uint8)
    w_gu[:I, 1] = enc[4.0]
    src = rng.integers(1, H, I)  # only row 0 reads x[0] = 28
    src[0], src[1] = 0, 2
    wu = np.full(I, up_weight)
    wu[0] = 1.0
    w_gu[I + np.arange(I), src] = [enc[float(v)] for v in wu]
    s_gu = np.ones(2 * I, np.float32)
    w_d = rng.choice(codes[(codes & 0x7F) < 0x70], (H, I)).astype(np.uint8)
    s_d = rng.uniform(0.5, 2.0, H).astype(np.float32)
    return xv, x, src, wu, w_gu, w_d, s_gu, s_d


def test_fp8_activations_are_exact_on_the_scaled_grid():
    for seed in range(3):
        _, x, _, _, w_gu, w_d, s_gu, s_d = _act8_expert(seed)
        a8 = oracle.expert(x, w_gu, w_d, s_gu, s_d, wtype="fp8a8", rounding=True)
        w8 = oracle.expert(x, w_gu, w_d, s_gu, s_d, wtype="fp8", rounding=True)
        np.testing.assert_array_equal(a8, w8)


def test_fp8_token_quantisation_against_torch_fp8_cast():
    """x[2] moved off the grid: the fp8a8 expert equals the weights-only fp8 expert on the token
    that torch's e4m3 cast makes of it (every later step stays exact)."""
    for seed in range(3):
        xv, x, _, _, w_gu, w_d, s_gu, s_d = _act8_expert(seed)
        xv2 = xv.copy()
        xv2[2] = float(bf16_codes_to_f64(_bf16_bits([1.03]))[0])
        x2 = _bf16_bits(xv2)
        xq = _torch_fp8_dequant(xv2, 2.0 ** -4)
        assert xq[2] != xv2[2] and np.array_equal(xq[[0, 1]], xv2[[0, 1]])
        a8 = oracle.expert(x2, w_gu, w_d, s_gu, s_d, wtype="fp8a8", rounding=True)
        w8 = oracle.expert(_bf16_bits(xq), w_gu, w_d, s_gu, s_d, wtype="fp8", rounding=True)
        np.testing.assert_array_equal(a8, w8)
    # up weight 1.5 puts h off the token's grid: the token is quantised before h is formed
    # (x[2] = 1.1 -> 1.125, h_1 = 96 * 1.125 = 108 -> 112; from 1.1 it would be 105.6 -> 104)
    for seed in range(3):
        xv, x, _, _, w_gu, w_d, s_gu, s_d = _act8_expert(seed, up_weight=1.5)
        xv2 = xv.copy()
        xv2[2] = float(bf16_codes_to_f64(_bf16_bits([1.1]))[0])
        xq = _torch_fp8_dequant(xv2, 2.0 ** -4)
        assert xq[2] == 1.125
        np.testing.assert_array_equal(
            oracle.expert(_bf16_bits(xv2), w_gu, w_d, s_gu, s_d, wtype="fp8a8", rounding=True),
            oracle.expert(_bf16_bits(xq), w_gu, w_d, s_gu, s_d, wtype="fp8a8", rounding=True))


def test_fp8_h_quantisation_against_torch_fp8_cast():
    """Up weight 1.125 puts h off the grid (x stays on it): the down sums run over torch's e4m3
    cast of h / s_h times s_h, s_h = 4 (the h row's amax is 448 * 4)."""
    for seed in range(3):
        xv, x, src, wu, w_gu, w_d, s_gu, s_d = _act8_expert(seed, up_weight=1.125)
        h = 64.0 * wu * xv[src]
        assert np.abs(h).max() == 64.0 * 28.0
        s_h = 4.0  # amax 64 * 28 = 448 * 4
        hq = _torch_fp8_dequant(h, s_h)
        assert not np.array_equal(hq, h)
        ref = (fp8_codes_to_f64(w_d) @ hq) * s_d.astype(np.float64)
        got = oracle.expert(x, w_gu, w_d, s_gu, s_d, wtype="fp8a8", rounding=False)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=0)


# ---------------------------------------------------------------- MXFP4 (4-bit experts)

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # OCP MX v1.0, the E2M1 magnitudes by code


def test_fp4_value_all_codes():
    codes = np.arange(16, dtype=np.uint8)
    got = oracle.fp4_value(codes)
    ref = np.array(E2M1 + [-v for v in E2M1])
    np.testing.assert_array_equal(got, ref)
    assert math.copysign(1.0, got[8]) < 0  # -0


def test_e8m0_value_is_a_power_of_two():
    X = np.arange(256, dtype=np.uint8)
    got = oracle.e8m0_value(X)
    np.testing.assert_array_equal(got[:255], [math.ldexp(1.0, int(x) - 127) for x in range(255)])
    assert math.isnan(got[255])


def mxfp4_dequant(codes, scales):
    """[rows][L/2] code bytes (low nibble first) and [rows][L/32] E8M0 bytes -> [rows][L] float64,
    by a table and numpy's ldexp (independent of the oracle)."""
    lut = np.array(E2M1 + [-v for v in E2M1])
    lo = lut[codes & 15]
    hi = lut[codes >> 4]
    vals = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return vals * np.repeat(sc, 32, axis=-1)


def test_single_mxfp4_expert_is_textbook_swiglu_on_dequantised_weights():
    cfg = configs.with_shape(configs.CONFIGS["tiny"], E=1, k=1, wtype="mxfp4")
    L = configs.make_layer(cfg, seed=8)
    x = configs.make_tokens(cfg, 3, seed=8)
    got = oracle.moe_layer(x, L, np.zeros((3, 1), np.int32), np.ones((3, 1)), rounding=False)
    Wgu = mxfp4_dequant(L["w_gate_up"][0], L["s_gate_up"][0])
    Wd = mxfp4_dequant(L["w_down"][0], L["s_down"][0])
    ref = _torch_swiglu(torch.from_numpy(bf16_codes_to_f64(x)), torch.from_numpy(Wgu), torch.from_numpy(Wd),
                        cfg.I).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_mxfp4_layer_with_shared_equals_dense_dequantised():
    cfg = configs.with_shape(configs.CONFIGS["tiny"], wtype="mxfp4", I_s=64, k=2)
    L = configs.make_layer(cfg, seed=9)
    x = configs.make_tokens(cfg, 4, seed=9)
    ids, w = oracle.route_topk(oracle.router_logits(x, L["router_w"]).astype(np.float32), cfg.k)
    got = oracle.moe_layer(x, L, ids, w, rounding=False)
    X = torch.from_numpy(bf16_codes_to_f64(x))
    ref = np.zeros_like(got)
    for t in range(4):
        for j in range(cfg.k):
            e = ids[t, j]
            y = _torch_swiglu(X[t:t + 1], torch.from_numpy(mxfp4_dequant(L["w_gate_up"][e], L["s_gate_up"][e])),
                              torch.from_numpy(mxfp4_dequant(L["w_down"][e], L["s_down"][e])), cfg.I).numpy()[0]
            ref[t] += w[t, j] * y
    z = (bf16_codes_to_f64(x) @ L["shared_gate_w"].astype(np.float64))
    ys = _torch_swiglu(X, torch.from_numpy(mxfp4_dequant(L["shared_w_gate_up"], L["shared_s_gate_up"])),
                       torch.from_numpy(mxfp4_dequant(L["shared_w_down"], L["shared_s_down"])), cfg.I_s).numpy()
    ref += scipy.special.expit(z)[:, None] * ys
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


def test_fp8a8_layer_is_the_fp8a8_experts_combined():
    cfg = configs.with_shape(configs.CONFIGS["tiny"], wtype="fp8a8", I_s=32, k=2)
    L = configs.make_layer(cfg, seed=12)
    x = configs.make_tokens(cfg, 3, seed=12)
    ids, w = oracle.route_topk(oracle.router_logits(x, L["router_w"]).astype(np.float32), cfg.k)
    got = oracle.moe_layer(x, L, ids, w, rounding=False)
    z = oracle.shared_gate_logits(x, L["shared_gate_w"])
    for t in range(3):
        ref = sum(w[t, j] * oracle.expert(x[t], L["w_gate_up"][ids[t, j]], L["w_down"][ids[t, j]],
                                          L["s_gate_up"][ids[t, j]], L["s_down"][ids[t, j]], "fp8a8", False)
                  for j in range(cfg.k))
        ref = ref + scipy.special.expit(z[t]) * oracle.expert(x[t], L["shared_w_gate_up"], L["shared_w_down"],
                                                                L["shared_s_gate_up"], L["shared_s_down"], "fp8a8",
                                                                False)
        np.testing.assert_allclose(got[t], ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- routing

def _golden_route_cases():
    cases = []
    with open(os.path.join(GOLDEN, "route_worked.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, k, lg, ids, w = [p.strip() for p in line.split("|")]
            cases.append((name, int(k), [float(v) for v in lg.split()], [int(v) for v in ids.split()],
                          None if w == "-" else [float(v) for v in w.split()]))
    return cases


@pytest.mark.parametrize("case", _golden_route_cases(), ids=lambda c: c[0])
def test_route_golden(case):
    _, k, lg, ids_ref, w_ref = case
    ids, w = oracle.route_topk(np.array([lg], dtype=np.float32), k)
    assert ids[0].tolist() == ids_ref
    if w_ref is not None:
        np.testing.assert_allclose(w[0], w_ref, rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed", range(6))
def test_route_brute_force_random_and_ties(seed):
    rng = np.random.default_rng(seed)
    for trial in range(30):
        E = int(rng.integers(1, 17))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 5))
        if trial % 2:
            lg = rng.choice(np.array([-1.0, -0.0, 0.0, 1.0], np.float32), size=(T, E))
        else:
            lg = rng.standard_normal((T, E)).astype(np.float32)
        ids, w = oracle.route_topk(lg, k)
        for t in range(T):
            assert ids[t].tolist() == brute_topk(lg[t].tolist(), k)
            sel = lg[t, ids[t]].astype(np.float64)
            p = scipy.special.softmax(sel)
            np.testing.assert_allclose(w[t], p, rtol=1e-13, atol=0)
            assert abs(w[t].sum() - 1.0) < 1e-12


def test_route_closed_form_k2():
    rng = np.random.default_rng(7)
    lg = rng.standard_normal((50, 9)).astype(np.float32)
    ids, w = oracle.route_topk(lg, 2)
    for t in range(50):
        l0, l1 = float(lg[t, ids[t, 0]]), float(lg[t, ids[t, 1]])
        assert l0 >= l1
        assert abs(w[t, 0] - 1.0 / (1.0 + math.exp(l1 - l0))) < 1e-15


def test_route_without_renormalisation_is_plain_softmax():
    rng = np.random.default_rng(8)
    lg = rng.standard_normal((10, 12)).astype(np.float32)
    ids, w = oracle.route_topk(lg, 3, renormalize=False)
    full = scipy.special.softmax(lg.astype(np.float64), axis=1)
    for t in range(10):
        np.testing.assert_allclose(w[t], full[t, ids[t]], rtol=1e-13)


def test_router_logits_against_torch_matmul():
    cfg = configs.CONFIGS["tiny"]
    L = configs.make_layer(cfg)
    x = configs.make_tokens(cfg, 4)
    b = np.linspace(-1, 1, cfg.E).astype(np.float32)
    ref = torch.from_numpy(bf16_codes_to_f64(x)) @ torch.from_numpy(L["router_w"].astype(np.float64)).T
    ref = ref.numpy() + b.astype(np.float64)
    got = oracle.router_logits(x, L["router_w"], b)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    z = oracle.shared_gate_logits(x, L["router_w"][0])
    np.testing.assert_allclose(z, ref[:, 0] - b[0], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- alignment

def _check_align_invariants(al, ids, E, BM, cap):
    flat = np.asarray(ids).ravel()
    n = flat.size
    s = al["sorted_ids"]
    off = al["offsets"]
    assert off[0] == 0 and al["num_padded"] == off[E] <= cap
    real = s[s != n]
    assert sorted(real.tolist()) == list(range(n))                     # bijection onto the slots
    assert np.array_equal(al["counts"], np.bincount(flat, minlength=E))  # histogram
    assert (s == n).sum() == cap - n                                    # sentinels
    for e in range(E):
        seg = s[off[e]:off[e + 1]]
        assert (off[e + 1] - off[e]) % BM == 0
        assert (off[e + 1] - off[e]) == -(-al["counts"][e] // BM) * BM
        body = seg[:al["counts"][e]]
        assert np.all(flat[body] == e) and np.all(np.diff(body) > 0)   # right expert, ascending
        assert np.all(seg[al["counts"][e]:] == n)
        assert np.all(al["block_expert"][off[e] // BM:off[e + 1] // BM] == e)
    assert np.all(al["block_expert"][off[E] // BM:] == -1)


def test_align_golden():
    vals = {}
    with open(os.path.join(GOLDEN, "align_worked.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, v = line.split(":")
                vals[key.strip()] = [int(a) for a in v.split()]
    T, k, E, BM, cap = vals["T"][0], vals["k"][0], vals["E"][0], vals["BM"][0], vals["capacity"][0]
    ids = np.array(vals["ids"], np.int32).reshape(T, k)
    assert oracle.align_capacity(T, k, E, BM) == cap
    al = oracle.align(ids, E, BM, cap)
    for key in ("counts", "offsets", "sorted_ids", "block_expert"):
        assert al[key].tolist() == vals[key], key
    assert al["num_padded"] == vals["num_padded"][0]


@pytest.mark.parametrize("seed", range(5))
def test_align_brute_force_and_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(20):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 30))
        BM = int(rng.choice([1, 2, 4, 16, 64]))
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        cap = oracle.align_capacity(T, k, E, BM)
        al = oracle.align(ids, E, BM, cap)
        ref = brute_align(ids, E, BM, cap)
        for key in ("sorted_ids", "block_expert", "counts", "offsets"):
            assert np.array_equal(al[key], ref[key]), key
        assert al["num_padded"] == ref["num_padded"]
        _check_align_invariants(al, ids, E, BM, cap)


def test_align_capacity_is_tight_for_the_worst_case():
    # every slot on a distinct expert, one slot each: each segment is one slot plus BM-1 padding
    for T, k, E, BM in [(2, 4, 64, 16), (8, 8, 256, 16), (3, 2, 4, 4), (64, 10, 512, 16)]:
        n = T * k
        ids = (np.arange(n) % E).reshape(T, k).astype(np.int32)
        cap = oracle.align_capacity(T, k, E, BM)
        al = oracle.align(ids, E, BM, cap)
        assert al["num_padded"] <= cap
        touched = min(E, n)
        assert cap == -(-(n + touched * (BM - 1)) // BM) * BM
    with pytest.raises(ValueError):
        oracle.align(np.array([[0, 1]], np.int32), 2, 16, 16)


# ---------------------------------------------------------------- experts and layer

@pytest.mark.parametrize("rounding", [False, True])
def test_layer_equals_dense_masked_gates(rounding):
    cfg = configs.CONFIGS["tiny"]
    L = configs.make_layer(cfg)
    x = configs.make_tokens(cfg, 4)
    ids, w = routed(x, L, cfg.k)
    got = oracle.moe_layer(x, L, ids, w, rounding=rounding)
    ref = dense_masked_layer(x, L, gates_from_topk(ids, w, cfg.E), rounding)
    if rounding:
        assert np.array_equal(got, ref)
    else:
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("rounding", [False, True])
def test_layer_with_shared_equals_dense_masked_gates(rounding):
    cfg = configs.with_shape(configs.CONFIGS["tiny"], I_s=64, k=3, bias="normal")
    L = configs.make_layer(cfg, seed=3)
    x = configs.make_tokens(cfg, 5, seed=3)
    ids, w = routed(x, L, cfg.k)
    got = oracle.moe_layer(x, L, ids, w, rounding=rounding)
    ref = dense_masked_layer(x, L, gates_from_topk(ids, w, cfg.E), rounding)
    if rounding:
        assert np.array_equal(got, ref)
    else:
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("wtype", ["bf16", "fp8a8", "mxfp4"])
@pytest.mark.parametrize("rounding", [False, True])
def test_threaded_layer_is_bitwise_the_single_threaded_one(wtype, rounding):
    """The token list split over host threads gives bitwise the one-thread result, for any
    thread count (more threads than tokens included) and any order of the token list."""
    cfg = configs.with_shape(configs.CONFIGS["tiny"], I_s=64, k=3, bias="normal", wtype=wtype)
    L = configs.make_layer(cfg, seed=7)
    x = configs.make_tokens(cfg, 29, seed=7)
    ids, w = routed(x, L, cfg.k)
    tokens = np.random.default_rng(7).permutation(29)[:23].astype(np.int32)
    tokens = np.concatenate([tokens, tokens[:4]])  # repeated tokens too
    one = oracle.moe_layer(x, L, ids, w, tokens=tokens, rounding=rounding, threads=1)
    for n in (2, 3, 8, 27, 40):
        st = {}
        got = oracle.moe_layer(x, L, ids, w, tokens=tokens, rounding=rounding, threads=n, stats=st)
        assert st["threads"] == min(n, len(tokens))
        assert np.array_equal(got.view(np.uint64), one.view(np.uint64)), f"{n} threads"


def test_layer_k_equals_E_is_dense_soft_moe():
    cfg = configs.with_shape(configs.CONFIGS["tiny"], E=6, k=6)
    L = configs.make_layer(cfg, seed=4)
    x = configs.make_tokens(cfg, 3, seed=4)
    lg = oracle.router_logits(x, L["router_w"], None).astype(np.float32)
    ids, w = oracle.route_topk(lg, 6)
    soft = scipy.special.softmax(lg.astype(np.float64), axis=1)   # all experts, plain softmax
    got = oracle.moe_layer(x, L, ids, w, rounding=False)
    ref = dense_masked_layer(x, L, soft, rounding=False)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_layer_k1_is_the_chosen_expert_exactly():
    cfg = configs.with_shape(configs.CONFIGS["tiny"], k=1)
    L = configs.make_layer(cfg, seed=5)
    x = configs.make_tokens(cfg, 4, seed=5)
    ids, w = routed(x, L, 1)
    assert np.all(w == 1.0)
    got = oracle.moe_layer(x, L, ids, w, rounding=True)
    for t in range(4):
        e = ids[t, 0]
        y = oracle.expert(x[t], L["w_gate_up"][e], L["w_down"][e], rounding=True)
        assert np.array_equal(got[t], y)


def _torch_swiglu(X, Wgu, Wd, I):
    g = X @ Wgu[:I].T
    u = X @ Wgu[I:].T
    return (torch.nn.functional.silu(g) * u) @ Wd.T


def test_single_expert_is_textbook_swiglu():
    cfg = configs.with_shape(configs.CONFIGS["tiny"], E=1, k=1)
    L = configs.make_layer(cfg, seed=6)
    x = configs.make_tokens(cfg, 4, seed=6)
    ids = np.zeros((4, 1), np.int32)
    w = np.ones((4, 1))
    got = oracle.moe_layer(x, L, ids, w, rounding=False)
    X = torch.from_numpy(bf16_codes_to_f64(x))
    ref = _torch_swiglu(X, torch.from_numpy(bf16_codes_to_f64(L["w_gate_up"][0])),
                        torch.from_numpy(bf16_codes_to_f64(L["w_down"][0])), cfg.I).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_single_fp8_expert_is_textbook_swiglu_on_dequantised_weights():
    cfg = configs.with_shape(configs.CONFIGS["tiny"], E=1, k=1, wtype="fp8")
    L = configs.make_layer(cfg, seed=7)
    x = configs.make_tokens(cfg, 3, seed=7)
    got = oracle.moe_layer(x, L, np.zeros((3, 1), np.int32), np.ones((3, 1)), rounding=False)
    Wgu = fp8_codes_to_f64(L["w_gate_up"][0]) * L["s_gate_up"][0].astype(np.float64)[:, None]
    Wd = fp8_codes_to_f64(L["w_down"][0]) * L["s_down"][0].astype(np.float64)[:, None]
    ref = _torch_swiglu(torch.from_numpy(bf16_codes_to_f64(x)), torch.from_numpy(Wgu), torch.from_numpy(Wd),
                        cfg.I).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_fp8_layer_with_shared_equals_dense_dequantised():
    cfg = configs.with_shape(configs.CONFIGS["tiny"], wtype="fp8", I_s=32, k=2)
    L = configs.make_layer(cfg, seed=8)
    x = configs.make_tokens(cfg, 3, seed=8)
    ids, w = routed(x, L, 2)
    got = oracle.moe_layer(x, L, ids, w, rounding=False)
    X = torch.from_numpy(bf16_codes_to_f64(x))
    ref = np.zeros_like(got)
    for t in range(3):
        for j in range(2):
            e = ids[t, j]
            Wgu = fp8_codes_to_f64(L["w_gate_up"][e]) * L["s_gate_up"][e].astype(np.float64)[:, None]
            Wd = fp8_codes_to_f64(L["w_down"][e]) * L["s_down"][e].astype(np.float64)[:, None]
            ref[t] += w[t, j] * _torch_swiglu(X[t:t + 1], torch.from_numpy(Wgu), torch.from_numpy(Wd), cfg.I)[0].numpy()
    Sgu = fp8_codes_to_f64(L["shared_w_gate_up"]) * L["shared_s_gate_up"].astype(np.float64)[:, None]
    Sd = fp8_codes_to_f64(L["shared_w_down"]) * L["shared_s_down"].astype(np.float64)[:, None]
    gam = torch.sigmoid(X @ torch.from_numpy(L["shared_gate_w"].astype(np.float64)))
    ref += (gam[:, None] * _torch_swiglu(X, torch.from_numpy(Sgu), torch.from_numpy(Sd), 32)).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_zero_tokens_give_exact_zero():
    cfg = configs.with_shape(configs.CONFIGS["tiny"], I_s=32)
    L = configs.make_layer(cfg)
    x = np.zeros((3, cfg.H), np.uint16)
    ids = np.array([[0, 1], [2, 3], [4, 5]], np.int32)
    got = oracle.moe_layer(x, L, ids, np.full((3, 2), 0.5))
    assert np.all(got == 0.0)


def test_zero_down_weights_leave_only_the_shared_term():
    cfg = configs.with_shape(configs.CONFIGS["tiny"], I_s=32)
    L = configs.make_layer(cfg, seed=9)
    L["w_down"] = np.zeros_like(L["w_down"])
    x = configs.make_tokens(cfg, 4, seed=9)
    ids, w = routed(x, L, 2)
    got = oracle.moe_layer(x, L, ids, w, rounding=False)
    X = torch.from_numpy(bf16_codes_to_f64(x))
    gam = torch.sigmoid(X @ torch.from_numpy(L["shared_gate_w"].astype(np.float64)))
    ys = _torch_swiglu(X, torch.from_numpy(bf16_codes_to_f64(L["shared_w_gate_up"])),
                       torch.from_numpy(bf16_codes_to_f64(L["shared_w_down"])), 32)
    np.testing.assert_allclose(got, (gam[:, None] * ys).numpy(), rtol=1e-12, atol=1e-13)


def test_token_permutation_permutes_the_output():
    cfg = configs.with_shape(configs.CONFIGS["tiny"], I_s=32)
    L = configs.make_layer(cfg, seed=10)
    x = configs.make_tokens(cfg, 6, seed=10)
    ids, w = routed(x, L, 2)
    out = oracle.moe_layer(x, L, ids, w)
    p = np.array([3, 0, 5, 1, 4, 2])
    out_p = oracle.moe_layer(x[p], L, ids[p], w[p])
    assert np.array_equal(out_p, out[p])
    sub = oracle.moe_layer(x, L, ids, w, tokens=np.array([4, 1], np.int32))
    assert np.array_equal(sub, out[[4, 1]])


def test_rounded_layer_is_within_bf16_error_of_the_exact_one():
    cfg = configs.CONFIGS["tiny"]
    L = configs.make_layer(cfg)
    x = configs.make_tokens(cfg, 4)
    ids, w = routed(x, L, 2)
    r = oracle.moe_layer(x, L, ids, w, rounding=True)
    u = oracle.moe_layer(x, L, ids, w, rounding=False)
    rel = np.linalg.norm(r - u) / np.linalg.norm(u)
    assert 1e-4 < rel < 1e-2
    assert np.array_equal(bf16_rne_bits(r), r)   # outputs are bf16 values
