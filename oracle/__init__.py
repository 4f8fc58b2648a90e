"""fp64 CPU oracle of the routed MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library (``speculative_verify_moe_amd``)
never does, and the two share no code.  The arithmetic lives in ``oracle.c``; this
module only marshals numpy arrays into it.

Every function here mirrors one C function; the passages each one follows are cited
in ``oracle.c``.  All pins of the oracle live in ``tests/test_oracle_pins.py``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB_PATH = os.environ.get("MOE_ORACLE_LIB", _build.LIB)
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"oracle library {_LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_round.restype = ctypes.c_uint16
        lib.oracle_bf16_round.argtypes = [ctypes.c_double]
        lib.oracle_fp8_value.restype = ctypes.c_double
        lib.oracle_fp8_value.argtypes = [ctypes.c_uint8]
        lib.oracle_fp8_encode.restype = ctypes.c_uint8
        lib.oracle_fp8_encode.argtypes = [ctypes.c_float]
        lib.oracle_fp4_value.restype = ctypes.c_double
        lib.oracle_fp4_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e8m0_value.restype = ctypes.c_double
        lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        lib.oracle_quantise_row.restype = ctypes.c_double
        lib.oracle_quantise_row.argtypes = [_I, _P, _P]
        lib.oracle_router_logits.restype = None
        lib.oracle_router_logits.argtypes = [_I, _I, _I, _P, _P, _P, _P]
        lib.oracle_shared_gate_logits.restype = None
        lib.oracle_shared_gate_logits.argtypes = [_I, _I, _P, _P, _P]
        lib.oracle_route_topk.restype = None
        lib.oracle_route_topk.argtypes = [_I, _I, _I, _I, _P, _P, _P]
        lib.oracle_align_capacity.restype = _I64
        lib.oracle_align_capacity.argtypes = [_I, _I, _I, _I]
        lib.oracle_align.restype = _I
        lib.oracle_align.argtypes = [_I, _I, _I, _I, _I64, _P, _P, _P, _P, _P, _P]
        lib.oracle_moe_layer.restype = None
        lib.oracle_moe_layer.argtypes = [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                                         _I, _P, _P, _P, _P, _P, _I, _P, _I, _P]
        lib.oracle_moe_layer_mt.restype = _I
        lib.oracle_moe_layer_mt.argtypes = [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                                            _I, _P, _P, _P, _P, _P, _I, _P, _I, _P, _I]
        lib.oracle_expert.restype = None
        lib.oracle_expert.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P, _I, _P]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def lib_path():
    return _LIB_PATH


def default_threads():
    """Host threads the layer oracle uses by default: the CPUs this process may run on, at
    most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------- number formats

def bf16_value(codes):
    """Exact value of bfloat16 bit patterns (uint16 array) as float64."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint16)
    return np.array([lib.oracle_bf16_value(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


def bf16_round(values):
    """Nearest-even bfloat16 bit patterns of float64 values (single rounding)."""
    lib = _load()
    v = np.asarray(values, dtype=np.float64)
    return np.array([lib.oracle_bf16_round(float(a)) for a in v.ravel()], dtype=np.uint16).reshape(v.shape)


def fp8_value(codes):
    """Value of OCP E4M3FN codes (uint8 array) as float64."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_fp8_value(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


def fp8_encode(values):
    """Nearest OCP E4M3FN codes (ties to an even mantissa, saturating at 448) of fp32 values."""
    lib = _load()
    v = np.asarray(values, dtype=np.float32)
    return np.array([lib.oracle_fp8_encode(float(a)) for a in v.ravel()], dtype=np.uint8).reshape(v.shape)


def quantise_rows(a):
    """Per-row fp8 quantisation of activations a [n][L] (fp32-representable values):
    (codes [n][L] uint8, scales [n] float64)."""
    lib = _load()
    a = _c(np.atleast_2d(a), np.float64)
    q = np.empty(a.shape, dtype=np.uint8)
    s = np.empty((a.shape[0],), dtype=np.float64)
    for i in range(a.shape[0]):
        s[i] = lib.oracle_quantise_row(a.shape[1], _ptr(a[i]), _ptr(q[i]))
    return q, s


WTYPES = {"bf16": 0, "fp8": 1, "fp8a8": 2, "mxfp4": 3}


def fp4_value(codes):
    """Value of E2M1 codes (the low 4 bits of uint8) as float64."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_fp4_value(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


def e8m0_value(codes):
    """Value of E8M0 scale bytes as float64."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e8m0_value(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


# ---------------------------------------------------------------- routing

def router_logits(x, w_r, b_r=None):
    """fp64 logits [T][E] of bf16 tokens x [T][H] (uint16) against fp32 router rows w_r [E][H]."""
    lib = _load()
    x = _c(x, np.uint16)
    w_r = _c(w_r, np.float32)
    b_r = _c(b_r, np.float32)
    T, H = x.shape
    E = w_r.shape[0]
    out = np.empty((T, E), dtype=np.float64)
    lib.oracle_router_logits(T, H, E, _ptr(x), _ptr(w_r), _ptr(b_r), _ptr(out))
    return out


def shared_gate_logits(x, w_sg):
    lib = _load()
    x = _c(x, np.uint16)
    w_sg = _c(w_sg, np.float32)
    T, H = x.shape
    out = np.empty((T,), dtype=np.float64)
    lib.oracle_shared_gate_logits(T, H, _ptr(x), _ptr(w_sg), _ptr(out))
    return out


def route_topk(logits, k, renormalize=True):
    """Top-k ids [T][k] int32 and gate weights [T][k] float64 from fp32 logits [T][E]."""
    lib = _load()
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib.oracle_route_topk(T, E, k, 1 if renormalize else 0, _ptr(lg), _ptr(ids), _ptr(w))
    return ids, w


# ---------------------------------------------------------------- alignment

def align_capacity(T, k, E, BM):
    return int(_load().oracle_align_capacity(T, k, E, BM))


def align(ids, E, BM, cap=None):
    """Alignment of ids [T][k]: dict of sorted_ids, block_expert, counts, offsets, num_padded."""
    lib = _load()
    ids = _c(ids, np.int32)
    T, k = ids.shape
    if cap is None:
        cap = align_capacity(T, k, E, BM)
    sorted_ids = np.empty((cap,), dtype=np.int32)
    block_expert = np.empty((cap // BM,), dtype=np.int32)
    counts = np.empty((E,), dtype=np.int32)
    offsets = np.empty((E + 1,), dtype=np.int32)
    num_padded = np.empty((1,), dtype=np.int32)
    rc = lib.oracle_align(T, k, E, BM, cap, _ptr(ids), _ptr(sorted_ids), _ptr(block_expert), _ptr(counts),
                          _ptr(offsets), _ptr(num_padded))
    if rc != 0:
        raise ValueError("capacity too small for the padded alignment")
    return dict(sorted_ids=sorted_ids, block_expert=block_expert, counts=counts, offsets=offsets,
                num_padded=int(num_padded[0]))


# ---------------------------------------------------------------- experts and layer

def _bank_arrays(layer, prefix):
    wtype = WTYPES[layer["wtype"]]
    wdt = np.uint16 if wtype == 0 else np.uint8
    gu = _c(layer[prefix + "w_gate_up"], wdt)
    dn = _c(layer[prefix + "w_down"], wdt)
    sdt = np.uint8 if wtype == 3 else np.float32
    sgu = _c(layer.get(prefix + "s_gate_up"), sdt) if wtype != 0 else None
    sd = _c(layer.get(prefix + "s_down"), sdt) if wtype != 0 else None
    return wtype, gu, dn, sgu, sd


def moe_layer(x, layer, ids, w, tokens=None, rounding=True, threads=None, stats=None):
    """Layer output [n_tok][H] float64 for the given routing (ids [T][k], w [T][k]).

    ``layer`` is a dict with H, E, k, I, I_s, wtype ('bf16' | 'fp8' | 'fp8a8': fp8 weights with
    fp8 activations, each row quantised with its own scale) and the weight arrays
    (w_gate_up [E][2I][H], w_down [E][H][I], optional s_gate_up/s_down for fp8, and
    shared_w_gate_up, shared_w_down, shared_s_*, shared_gate_w when I_s > 0).
    ``tokens`` selects which tokens to compute (default: all).  With ``rounding`` the
    outputs are bf16-representable values (bf16 at h, at each expert output and at the end).
    ``threads`` splits the tokens over that many host threads (default: default_threads());
    every token is computed by the same code, so the result does not depend on it.  A dict
    passed as ``stats`` receives the number of threads used.
    """
    lib = _load()
    x = _c(x, np.uint16)
    T, H = x.shape
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    k = ids.shape[1]
    E, I, I_s = layer["E"], layer["I"], layer.get("I_s", 0)
    wtype, gu, dn, sgu, sd = _bank_arrays(layer, "")
    if I_s > 0:
        _, sgu_w, sdn_w, ssgu, ssd = _bank_arrays(layer, "shared_")
        wsg = _c(layer["shared_gate_w"], np.float32)
    else:
        sgu_w = sdn_w = ssgu = ssd = wsg = None
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = _c(tokens, np.int32)
    out = np.empty((len(tokens), H), dtype=np.float64)
    nth = default_threads() if threads is None else int(threads)
    args = (T, H, E, k, I, wtype, _ptr(x), _ptr(gu), _ptr(dn), _ptr(sgu), _ptr(sd), _ptr(ids), _ptr(w),
            I_s, _ptr(sgu_w), _ptr(sdn_w), _ptr(ssgu), _ptr(ssd), _ptr(wsg), len(tokens), _ptr(tokens),
            1 if rounding else 0, _ptr(out))
    if nth <= 1:
        lib.oracle_moe_layer(*args)
        used = 1
    else:
        used = lib.oracle_moe_layer_mt(*args, nth)
    if stats is not None:
        stats["threads"] = used
    return out


def expert(x_t, w_gate_up, w_down, s_gate_up=None, s_down=None, wtype="bf16", rounding=True):
    """One token x_t [H] (bf16 bits) through one expert (w_gate_up [2I][H], w_down [H][I])."""
    lib = _load()
    wt = WTYPES[wtype]
    wdt = np.uint16 if wt == 0 else np.uint8
    x_t = _c(x_t, np.uint16)
    gu = _c(w_gate_up, wdt)
    dn = _c(w_down, wdt)
    H = x_t.shape[0]
    I = gu.shape[0] // 2
    sdt = np.uint8 if wt == 3 else np.float32
    sgu = _c(s_gate_up, sdt)
    sdn = _c(s_down, sdt)
    y = np.empty((H,), dtype=np.float64)
    lib.oracle_expert(H, I, wt, _ptr(x_t), _ptr(gu), _ptr(dn), _ptr(sgu), _ptr(sdn), 1 if rounding else 0, _ptr(y))
    return y
