"""ctypes binding of the C ABI in ``include/moe.h`` (libmoe_mi355x.so).

Marshalling only: every step of the layer runs in the HIP kernels of the library.
Tensors are torch CUDA (ROCm) tensors; bf16 values are ``torch.bfloat16`` tensors,
fp8 codes ``torch.uint8``; work goes on the current torch stream.  There is no
fallback: importing this module without the built library raises.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build()); the MoE layer has no CPU fallback")

_lib = ctypes.CDLL(LIB_PATH)

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_MISALIGNED, MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE = range(6)
MOE_W_BF16, MOE_W_FP8_E4M3, MOE_W_FP8_E4M3_A8, MOE_W_MXFP4 = 0, 1, 2, 3
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t


class _Bank(ctypes.Structure):
    _fields_ = [("wtype", _I32), ("num_experts", _I32), ("hidden", _I32), ("inter", _I32),
                ("w_gate_up", _P), ("w_down", _P), ("s_gate_up", _P), ("s_down", _P), ("mx_gate_up", _P),
                ("mx_down", _P)]


class _Layer(ctypes.Structure):
    _fields_ = [("hidden", _I32), ("num_experts", _I32), ("top_k", _I32), ("renormalize", _I32),
                ("router_w", _P), ("router_b", _P), ("routed", _Bank), ("shared", _Bank), ("shared_gate_w", _P)]


EXPORTS = {
    "moe_align_capacity": (_SZ, [_I32, _I32, _I32, _I32]),
    "moe_align_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "moe_route_topk": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "moe_align": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_experts_workspace_size": (_SZ, [_I32, _I32, ctypes.POINTER(_Bank), _I32]),
    "moe_experts_forward": (ctypes.c_int, [_P, _I32, ctypes.POINTER(_Bank), _I32, _P, _P, _P, _P, _P, _I32, _I64,
                                           _P, _P, _SZ, _P]),
    "moe_layer_workspace_size": (_SZ, [_I32, ctypes.POINTER(_Layer)]),
    "moe_layer_forward": (ctypes.c_int, [_P, _I32, ctypes.POINTER(_Layer), _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_layer_forward_noalloc": (ctypes.c_int, [_P, _I32, ctypes.POINTER(_Layer), _P, _P, _P, _P, _P]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_workspace_status_offset": (_SZ, []),
    "moe_describe_plan": (ctypes.c_char_p, [_I32, ctypes.POINTER(_Layer)]),
    "moe_set_stage_events": (ctypes.c_int, [ctypes.POINTER(_P), _I32]),
    "moe_set_option": (ctypes.c_int, [_I32, _I32]),
    "moe_measure_stream_read": (ctypes.c_int, [_P, _SZ, _I32, _I32, _P, _P]),
}
for _name, (_res, _args) in EXPORTS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class MoeError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"status {status}: {message}")
        self.status = status


def _check(status):
    if status != MOE_OK:
        raise MoeError(status, _lib.moe_last_error().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _workspace(nbytes, device):
    return torch.empty((max(int(nbytes), 1),), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ layer descriptors

class Bank:
    """A bank of n experts: w_gate_up [n][2I][H], w_down [n][H][I] (bf16, or uint8 fp8 codes
    with fp32 row scales s_gate_up [n][2I], s_down [n][H]).  ``act8`` (fp8 banks only): the
    prefill path quantises the activations too (MOE_W_FP8_E4M3_A8).  ``mxfp4``: uint8 code bytes
    w_gate_up [n][2I][H/2], w_down [n][H][I/2] with uint8 E8M0 block scales s_gate_up
    [n][2I][H/32], s_down [n][H][I/32] (MOE_W_MXFP4).  Holds the tensors alive."""

    def __init__(self, w_gate_up, w_down, s_gate_up=None, s_down=None, act8=False, mxfp4=False):
        self.w_gate_up, self.w_down, self.s_gate_up, self.s_down = w_gate_up, w_down, s_gate_up, s_down
        fp8 = w_gate_up.dtype == torch.uint8 and not mxfp4
        if act8 and not fp8:
            raise ValueError("act8 needs fp8 (uint8) weights")
        if mxfp4:
            self.wtype = MOE_W_MXFP4
        else:
            self.wtype = (MOE_W_FP8_E4M3_A8 if act8 else MOE_W_FP8_E4M3) if fp8 else MOE_W_BF16
        gu = w_gate_up if w_gate_up.dim() == 3 else w_gate_up.unsqueeze(0)
        self.num_experts, two_i, self.hidden = gu.shape
        if mxfp4:
            self.hidden *= 2
        self.inter = two_i // 2
        _dev(w_gate_up, torch.uint8 if (fp8 or mxfp4) else torch.bfloat16, "w_gate_up")
        _dev(w_down, w_gate_up.dtype, "w_down")
        if fp8:
            _dev(s_gate_up, torch.float32, "s_gate_up")
            _dev(s_down, torch.float32, "s_down")
        if mxfp4:
            _dev(s_gate_up, torch.uint8, "s_gate_up")
            _dev(s_down, torch.uint8, "s_down")

    def struct(self):
        mx = self.wtype == MOE_W_MXFP4
        return _Bank(self.wtype, self.num_experts, self.hidden, self.inter, _ptr(self.w_gate_up), _ptr(self.w_down),
                     None if mx else _ptr(self.s_gate_up), None if mx else _ptr(self.s_down),
                     _ptr(self.s_gate_up) if mx else None, _ptr(self.s_down) if mx else None)


class Layer:
    """One MoE layer: router_w [E][H] fp32, router_b [E] or None, routed Bank, optional shared
    Bank (one expert) with shared_gate_w [H] fp32, top_k and renormalize."""

    def __init__(self, router_w, router_b, routed, top_k, shared=None, shared_gate_w=None, renormalize=True):
        self.router_w = _dev(router_w, torch.float32, "router_w")
        self.router_b = None if router_b is None else _dev(router_b, torch.float32, "router_b")
        self.routed, self.shared, self.top_k, self.renormalize = routed, shared, int(top_k), bool(renormalize)
        self.shared_gate_w = None if shared_gate_w is None else _dev(shared_gate_w, torch.float32, "shared_gate_w")
        self.hidden, self.num_experts = routed.hidden, routed.num_experts
        self._s = _Layer(self.hidden, self.num_experts, self.top_k, 1 if self.renormalize else 0, _ptr(self.router_w),
                         _ptr(self.router_b), routed.struct(),
                         shared.struct() if shared is not None else _Bank(0, 0, self.hidden, 0, None, None, None, None,
                                                                           None, None),
                         _ptr(self.shared_gate_w))

    @property
    def struct(self):
        return self._s

    @classmethod
    def from_host(cls, L, device="cuda"):
        """Upload a host layer (the dict the synthetic recipes build) to the device."""
        def bf16(a):
            return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(device)

        def wt(a):
            return bf16(a) if a.dtype.name == "uint16" else torch.from_numpy(a).to(device)

        def f32(a):
            return None if a is None else torch.from_numpy(a).to(device)

        act8 = L.get("wtype") == "fp8a8"
        mx = L.get("wtype") == "mxfp4"
        routed = Bank(wt(L["w_gate_up"]), wt(L["w_down"]), f32(L.get("s_gate_up")), f32(L.get("s_down")), act8, mx)
        shared = None
        if L.get("I_s", 0) > 0:
            shared = Bank(wt(L["shared_w_gate_up"]), wt(L["shared_w_down"]), f32(L.get("shared_s_gate_up")),
                          f32(L.get("shared_s_down")), act8, mx)
        return cls(f32(L["router_w"]), f32(L.get("router_b")), routed, L["k"], shared,
                   f32(L.get("shared_gate_w")), L.get("renormalize", True))


# ------------------------------------------------------------------ entry points

def moe_align_capacity(T, k, E, BM):
    return int(_lib.moe_align_capacity(T, k, E, BM))


def moe_align_workspace_size(T, k, E):
    return int(_lib.moe_align_workspace_size(T, k, E))


def moe_experts_workspace_size(T, k, routed, BM):
    s = routed.struct()
    return int(_lib.moe_experts_workspace_size(T, k, ctypes.byref(s), BM))


def moe_layer_workspace_size(T, layer):
    return int(_lib.moe_layer_workspace_size(T, ctypes.byref(layer.struct)))


def moe_last_error():
    return _lib.moe_last_error().decode()


def moe_workspace_status(ws):
    """The workspace's count of fused-kernel waits that gave up (0 in normal use); reads the
    word on the device (synchronises with the current stream)."""
    off = int(_lib.moe_workspace_status_offset())
    return int(ws[off:off + 4].view(torch.int32).item())


def moe_describe_plan(T, layer):
    return _lib.moe_describe_plan(T, ctypes.byref(layer.struct)).decode()


MOE_OPT_DECODE_FUSED = 1


def moe_set_option(key, value):
    _check(_lib.moe_set_option(key, value))


def stage_event_handles(events):
    """The HIP handles of a list of torch.cuda.Event(enable_timing=True), as the host array the
    measurement hook takes (build it once, outside a timed loop)."""
    handles = []
    for ev in events:
        if ev.cuda_event == 0:      # torch creates the HIP event lazily
            ev.record()
        handles.append(ctypes.c_void_p(ev.cuda_event))
    return (_P * len(handles))(*handles), len(handles)


def moe_set_stage_events(events):
    """events: list of torch.cuda.Event(enable_timing=True), the (array, n) pair that
    stage_event_handles returns, or None to turn the hook off.  Stage i of each following
    moe_layer_forward on this thread takes events 2i (start of its first kernel) and 2i+1
    (end of its last)."""
    if not events:
        _check(_lib.moe_set_stage_events(None, 0))
        return
    arr, n = events if isinstance(events, tuple) else stage_event_handles(events)
    _check(_lib.moe_set_stage_events(arr, n))


def moe_measure_stream_read(buf, blocks, depth, sink=None):
    """One streaming read of the whole device tensor buf (a measurement aid, no part of the
    layer) on the current stream; returns the sink tensor (one uint32 checksum per block)."""
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty((blocks,), dtype=torch.int32, device=buf.device)
    _check(_lib.moe_measure_stream_read(_ptr(buf), nbytes, blocks, depth, _ptr(sink), _stream()))
    return sink


def moe_route_topk(logits, k, renormalize=True, topk_ids=None, topk_w=None):
    """Top-k routing of fp32 logits [T][E]: returns (ids [T][k] int32, w [T][k] fp32)."""
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _dev(topk_ids, torch.int32, "topk_ids")
    _dev(topk_w, torch.float32, "topk_w")
    _check(_lib.moe_route_topk(_ptr(logits), T, E, k, 1 if renormalize else 0, _ptr(topk_ids), _ptr(topk_w),
                               _stream()))
    return topk_ids, topk_w


def moe_align(topk_ids, E, BM, cap=None, out=None, ws=None):
    """Alignment of ids [T][k]: dict of sorted_ids, block_expert, expert_counts, expert_offsets, num_padded."""
    _dev(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    dev = topk_ids.device
    if cap is None:
        cap = moe_align_capacity(T, k, E, BM)
    if out is None:
        out = dict(sorted_ids=torch.empty((cap,), dtype=torch.int32, device=dev),
                   block_expert=torch.empty((cap // BM,), dtype=torch.int32, device=dev),
                   expert_counts=torch.empty((E,), dtype=torch.int32, device=dev),
                   expert_offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
                   num_padded=torch.empty((1,), dtype=torch.int32, device=dev))
    need = moe_align_workspace_size(T, k, E)
    if ws is None and need > 0:
        ws = _workspace(need, dev)
    _check(_lib.moe_align(_ptr(topk_ids), T, k, E, BM, cap, _ptr(out["sorted_ids"]), _ptr(out["block_expert"]),
                          _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]), _ptr(out["num_padded"]), _ptr(ws),
                          0 if ws is None else ws.numel(), _stream()))
    out["cap"] = cap
    return out


def moe_experts_forward(x, routed, k, topk_w, alignment, BM, out=None, ws=None):
    """Routed experts + combine (no shared expert) for bf16 x [T][H] given the routing and its alignment."""
    _dev(x, torch.bfloat16, "x")
    T, H = x.shape
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    s = routed.struct()
    need = int(_lib.moe_experts_workspace_size(T, k, ctypes.byref(s), BM))
    if ws is None:
        ws = _workspace(need, x.device)
    _check(_lib.moe_experts_forward(_ptr(x), T, ctypes.byref(s), k, _ptr(topk_w), _ptr(alignment["sorted_ids"]),
                                    _ptr(alignment["block_expert"]), _ptr(alignment["expert_counts"]),
                                    _ptr(alignment["expert_offsets"]), BM, alignment["cap"], _ptr(out), _ptr(ws),
                                    ws.numel(), _stream()))
    return out


def moe_layer_forward(x, layer, out=None, logits_out=None, ids_out=None, w_out=None, ws=None):
    """The whole layer for bf16 x [T][H]; returns out [T][H] bf16."""
    _dev(x, torch.bfloat16, "x")
    T, H = x.shape
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _dev(out, torch.bfloat16, "out")
    for t, dt, name in ((logits_out, torch.float32, "logits_out"), (ids_out, torch.int32, "ids_out"),
                        (w_out, torch.float32, "w_out")):
        if t is not None:
            _dev(t, dt, name)
    if ws is None:
        ws = torch.zeros((max(moe_layer_workspace_size(T, layer), 1),), dtype=torch.uint8, device=x.device)
    _check(_lib.moe_layer_forward(_ptr(x), T, ctypes.byref(layer.struct), _ptr(out), _ptr(logits_out), _ptr(ids_out),
                                  _ptr(w_out), _ptr(ws), ws.numel(), _stream()))
    return out


def moe_layer_forward_noalloc(x, layer, out=None, logits_out=None, ids_out=None, w_out=None):
    """The whole layer with the library's static device scratch instead of a workspace (the C
    entry point allocates nothing; only a missing ``out`` is allocated here, by torch)."""
    _dev(x, torch.bfloat16, "x")
    T, H = x.shape
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _dev(out, torch.bfloat16, "out")
    for t, dt, name in ((logits_out, torch.float32, "logits_out"), (ids_out, torch.int32, "ids_out"),
                        (w_out, torch.float32, "w_out")):
        if t is not None:
            _dev(t, dt, name)
    _check(_lib.moe_layer_forward_noalloc(_ptr(x), T, ctypes.byref(layer.struct), _ptr(out), _ptr(logits_out),
                                          _ptr(ids_out), _ptr(w_out), _stream()))
    return out
