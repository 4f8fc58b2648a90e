"""Helpers shared by the GPU tests: layer construction (cached), device<->host views, and the
comparison of one layer call against the CPU oracle."""
import functools

import numpy as np
import torch

import oracle
from synth import configs

# relL2 bars.  MXFP4 weights decode exactly on both sides (E2M1 codes times a power of two),
# which leaves the error sources of bf16 -- fp32 against fp64 sums and the three bf16
# roundings -- so it takes the bf16 bar.  fp8 weights keep the 5e-3 their type is allowed;
# fp8 activations add one e4m3 rounding per activation (measured worst case 1.79e-3).
TOL = {"bf16": 1e-3, "fp8": 5e-3, "fp8a8": 5e-3, "mxfp4": 1e-3}
# max-abs bars, as a fraction of max |ref|: 1e-2, except fp8 activations, whose h codes can
# differ from the oracle's: the device's h (fp32 sums rounded to bf16) can differ from the
# oracle's by one bf16 step, which now and then moves an h code by one e4m3 step or a row's
# scale by one binade, and one slot's output then moves by a percent or two of max |ref|
# (measured worst cases: 8.2e-3 over the 4096-token chunk, 1.41e-2 for a 600-token chunk of the
# tiny layer, whose 128-wide h rows give a single code more weight).
MAX_ABS = {"bf16": 1e-2, "fp8": 1e-2, "fp8a8": 3e-2, "mxfp4": 1e-2}


def runs_decode_path(T, k):
    """The library's dispatch: T <= 64 tokens with T*k <= 1024 slots take the GEMV path."""
    return T <= 64 and T * k <= 1024


def oracle_layer_for_path(L, T):
    """fp8a8 banks quantise activations on the prefill path only; decode streams the same
    weights with bf16 activations (the fp8 reading)."""
    if L["wtype"] == "fp8a8" and runs_decode_path(T, L["k"]):
        return dict(L, wtype="fp8")
    return L


def bf16_bits(t):
    """bf16 CUDA tensor -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_dev_bf16(bits, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


@functools.lru_cache(maxsize=4)
def _experts(H, E, I, I_s, wtype, seed, replica):
    cfg = configs.LayerConfig("cache", H=H, E=E, k=1, I=I, I_s=I_s, wtype=wtype, bias="none", BM=16)
    return configs.make_layer(cfg, seed=seed, replica=replica)


def host_layer(cfg, seed=0, replica=0):
    """Host layer dict; expert banks of equal shape and seed are generated once and shared."""
    L = configs.make_layer(cfg, seed=seed, replica=replica, with_experts=False)
    ex = _experts(cfg.H, cfg.E, cfg.I, cfg.I_s, cfg.wtype, seed, replica)
    for key in ("w_gate_up", "w_down", "s_gate_up", "s_down", "shared_w_gate_up", "shared_w_down",
                "shared_s_gate_up", "shared_s_down"):
        if key in ex:
            L[key] = ex[key]
    return L


_dev_cache = {}


def device_layer(L):
    from speculative_verify_moe_amd import Layer
    key = (L["name"], L["H"], L["E"], L["k"], L["I"], L["I_s"], L["wtype"], id(L["w_gate_up"]))
    if key not in _dev_cache:
        if len(_dev_cache) >= 3:
            _dev_cache.clear()
            torch.cuda.empty_cache()
        # the entry keeps L alive, so the id() in the key cannot be reused while cached
        _dev_cache[key] = (L, Layer.from_host(L))
    return _dev_cache[key][1]


def run_layer(L, x_bits):
    """One moe_layer_forward call; returns host copies of out bits, logits, ids, w."""
    from speculative_verify_moe_amd import moe_layer_forward
    D = device_layer(L)
    x = to_dev_bf16(x_bits)
    T = x_bits.shape[0]
    logits = torch.empty((T, L["E"]), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, L["k"]), dtype=torch.int32, device="cuda")
    w = torch.empty((T, L["k"]), dtype=torch.float32, device="cuda")
    out = moe_layer_forward(x, D, logits_out=logits, ids_out=ids, w_out=w)
    torch.cuda.synchronize()
    return bf16_bits(out), logits.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


def say_margin(name, rep):
    """One line per compared case: the measured relL2 and max-abs (as a fraction of max |ref|)
    beside their bars."""
    wt = rep.get("wtype")
    frac = rep["max_abs"] / max(rep["max_ref"], 1e-300)
    print(f"[margin] {name} wtype={wt} relL2={rep['rel_l2']:.3e} bar={TOL[wt]:.0e} "
          f"maxabs/max|ref|={frac:.3e} bar={MAX_ABS[wt]:.0e}", flush=True)


def check_layer(L, x_bits, tokens=None, report=None):
    """Compare one layer call with the oracle.  Routing: bit-exact ids from the device logits,
    weights within 1e-6; logits within 1e-5 (1 + |L|) of fp64; output relL2 / max-abs bars."""
    out_bits, lg, ids, w = run_layer(L, x_bits)
    T = x_bits.shape[0]
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = np.asarray(tokens, dtype=np.int32)
    # logits against fp64 on the sampled tokens
    L64 = oracle.router_logits(x_bits[tokens], L["router_w"], L["router_b"])
    err = np.abs(lg[tokens].astype(np.float64) - L64)
    assert np.all(err <= 1e-5 * (1.0 + np.abs(L64))), f"logit error {err.max()}"
    # routing from the device logits: ids exact for every token, weights within 1e-6
    ids_ref, w_ref = oracle.route_topk(lg, L["k"], L.get("renormalize", True))
    assert np.array_equal(ids, ids_ref), "top-k ids differ from the oracle"
    assert np.max(np.abs(w.astype(np.float64) - w_ref)) <= 1e-6
    # layer output on the sampled tokens, routed as the device routed
    ref = oracle.moe_layer(x_bits, oracle_layer_for_path(L, T), ids_ref, w_ref, tokens=tokens, rounding=True)
    got = bf16_values(out_bits[tokens])
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    mx = np.max(np.abs(got - ref))
    Lref = oracle_layer_for_path(L, T)
    tol = TOL[Lref["wtype"]]
    if report is not None:
        report.update(rel_l2=rel, max_abs=mx, max_ref=np.max(np.abs(ref)), ref=ref, got=got, ids=ids_ref, w=w_ref,
                      tokens=tokens, wtype=Lref["wtype"])
    assert rel <= tol, f"relL2 {rel:.3e} > {tol}"
    mtol = MAX_ABS[Lref["wtype"]]
    assert mx <= mtol * np.max(np.abs(ref)), f"max-abs {mx:.3e} > {mtol} * {np.max(np.abs(ref)):.3e}"
    return out_bits
