"""ctypes binding of libmoe.so (include/moe.h): argument marshalling only.

Every step of the layer runs in the HIP kernels of libmoe.so; this module converts torch device
tensors to raw pointers and the current torch stream to a hipStream_t. PyTorch supplies device
memory (weights, activations, outputs, workspace) and streams, nothing else. If the library is
missing, loading raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_F32 = 0
MOE_BF16 = 1
MOE_FP8_E4M3 = 2  # bf16 x and router; FP8 E4M3 expert weights with fp32 per-row scales
MOE_MXFP4 = 3  # bf16 x and router; MXFP4 expert weights (packed E2M1 codes, E8M0 bytes per 32)
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "mxfp4": MOE_MXFP4}
WEIGHT_KEYS = ("router_w", "router_bias", "gate_up", "down", "shared_gate_up", "shared_down",
               "gate_up_scale", "down_scale", "shared_gate_up_scale", "shared_down_scale")

EXPORTS = ("moe_create", "moe_destroy", "moe_workspace_bytes", "moe_workspace_state_bytes",
           "moe_route", "moe_bucket",
           "moe_forward", "moe_forward_noalloc", "moe_forward_plan", "moe_forward_timed",
           "moe_status_str")


class moe_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class moe_weights(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in WEIGHT_KEYS]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so and declare its signatures. Raises if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m sparse_moe_routing_amd.build`"
                           " (there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.moe_create.argtypes = [ctypes.POINTER(moe_config), ctypes.POINTER(moe_weights),
                               ctypes.POINTER(ctypes.c_void_p)]
    lib.moe_create.restype = ctypes.c_int
    lib.moe_destroy.argtypes = [P]
    lib.moe_destroy.restype = None
    lib.moe_workspace_bytes.argtypes = [P, I32]
    lib.moe_workspace_bytes.restype = SZ
    lib.moe_workspace_state_bytes.argtypes = [P]
    lib.moe_workspace_state_bytes.restype = SZ
    lib.moe_route.argtypes = [P, P, P, I32, P, P, P, P, P, SZ, P]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_bucket.argtypes = [P, P, I32, P, P, P, P, SZ, P]
    lib.moe_bucket.restype = ctypes.c_int
    lib.moe_forward.argtypes = [P, P, I32, P, P, P, P, P, SZ, P]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [P, P, I32, P, P, P, P, P]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_forward_plan.argtypes = [P, I32, I32, ctypes.POINTER(I32),
                                     ctypes.POINTER(ctypes.c_char_p), I32]
    lib.moe_forward_plan.restype = ctypes.c_int
    lib.moe_forward_timed.argtypes = [P, P, I32, P, P, P, P, P, SZ, P, P, I32]
    lib.moe_forward_timed.restype = ctypes.c_int
    lib.moe_status_str.argtypes = [ctypes.c_int]
    lib.moe_status_str.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = load().moe_status_str(status).decode()
        super().__init__(f"{what}: {msg} ({status})")


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class MoeLayer:
    """A context over device weight tensors (borrowed: the tensors are kept alive here).

    weights: dict with router_w [R][H], router_bias [R] fp32 or None, gate_up [E][2I][H],
    down [E][H][I], shared_gate_up [2Is][H] or None, shared_down [H][Is] or None, and for "fp8"
    the row scales gate_up_scale [E][2I], down_scale [E][H], shared_gate_up_scale [2Is] and
    shared_down_scale [H] (fp32) next to uint8 FP8 E4M3 codes, for "mxfp4" packed E2M1 codes
    ([E][2I][H/2] ...) with E8M0 scale bytes gate_up_scale [E][2I][H/32], down_scale
    [E][H][I/32], shared_gate_up_scale [2Is][H/32], shared_down_scale [H][Is/32]; bf16 weights
    may be torch.bfloat16 or 16-bit integer tensors holding the bf16 bits.
    """

    def __init__(self, hidden, num_experts, inter, shared_inter, max_tokens, dtype, weights,
                 top_k=8):
        self.lib = load()
        self.cfg = moe_config(hidden, num_experts, top_k, inter, shared_inter, max_tokens,
                              DTYPES[dtype])
        self._keep = dict(weights)
        w = moe_weights(*((None if weights.get(k) is None else weights[k].data_ptr())
                          for k in WEIGHT_KEYS))
        ctx = ctypes.c_void_p()
        _check(self.lib.moe_create(ctypes.byref(self.cfg), ctypes.byref(w), ctypes.byref(ctx)),
               "moe_create")
        self.ctx = ctx
        self.hidden, self.num_experts = hidden, num_experts
        self.shared_inter = shared_inter
        self.rows = num_experts + (1 if shared_inter > 0 else 0)

    def close(self):
        if getattr(self, "ctx", None):
            self.lib.moe_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, T: int) -> int:
        return int(self.lib.moe_workspace_bytes(self.ctx, T))

    def state_bytes(self) -> int:
        """Size of the workspace's leading state region (zero before the first call, left zero
        by every call)."""
        return int(self.lib.moe_workspace_state_bytes(self.ctx))

    def workspace(self, T: int, device="cuda"):
        """A workspace for calls of up to T tokens. It starts zeroed: the library keeps arrival
        counters and work-queue words in its leading state region, which must be zero before the
        first call and which every call leaves at zero."""
        import torch
        return torch.zeros(max(self.workspace_bytes(T), 256), dtype=torch.uint8, device=device)

    def route(self, x=None, logits=None, T=None, ws=None, want_logits=True, stream=None):
        """(logits [T][R] or None, ids [T][8], w [T][8], g [T] or None) from x or given logits."""
        import torch
        src = x if x is not None else logits
        T = src.shape[0] if T is None else T
        dev = src.device
        ids = torch.empty((T, 8), dtype=torch.int32, device=dev)
        w = torch.empty((T, 8), dtype=torch.float32, device=dev)
        g = torch.empty((T,), dtype=torch.float32, device=dev) if self.shared_inter > 0 else None
        z = torch.empty((T, self.rows), dtype=torch.float32, device=dev) if want_logits else None
        ws = self.workspace(T, dev) if ws is None else ws
        _check(self.lib.moe_route(self.ctx, _ptr(x), _ptr(logits), T, _ptr(z), _ptr(ids),
                                  _ptr(w), _ptr(g), _ptr(ws), ws.numel(), _stream(stream)),
               "moe_route")
        return z, ids, w, g

    def bucket(self, ids, ws=None, stream=None):
        """(counts [E], offsets [E+1], perm [T*8]) for ids [T][8]."""
        import torch
        T = ids.shape[0]
        dev = ids.device
        counts = torch.empty((self.num_experts,), dtype=torch.int32, device=dev)
        offsets = torch.empty((self.num_experts + 1,), dtype=torch.int32, device=dev)
        perm = torch.empty((T * 8,), dtype=torch.int32, device=dev)
        ws = self.workspace(T, dev) if ws is None else ws
        _check(self.lib.moe_bucket(self.ctx, _ptr(ids), T, _ptr(counts), _ptr(offsets),
                                   _ptr(perm), _ptr(ws), ws.numel(), _stream(stream)),
               "moe_bucket")
        return counts, offsets, perm

    def forward(self, x, routing=None, y=None, ws=None, stream=None, events=None):
        """y [T][H] fp32; routing = (ids, w, g) to use a given routing, else routed from x."""
        import torch
        T = x.shape[0]
        dev = x.device
        y = torch.empty((T, self.hidden), dtype=torch.float32, device=dev) if y is None else y
        ws = self.workspace(T, dev) if ws is None else ws
        ids = w = g = None
        if routing is not None:
            ids, w, g = routing
        if events is None:
            _check(self.lib.moe_forward(self.ctx, _ptr(x), T, _ptr(ids), _ptr(w), _ptr(g),
                                        _ptr(y), _ptr(ws), ws.numel(), _stream(stream)),
                   "moe_forward")
        else:
            arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
            _check(self.lib.moe_forward_timed(self.ctx, _ptr(x), T, _ptr(ids), _ptr(w), _ptr(g),
                                              _ptr(y), _ptr(ws), ws.numel(), _stream(stream),
                                              arr, len(events)), "moe_forward_timed")
        return y

    def forward_noalloc(self, x, routing=None, y=None, stream=None):
        """moe_forward_noalloc: as forward, with the library's static scratch as workspace."""
        import torch
        T = x.shape[0]
        y = torch.empty((T, self.hidden), dtype=torch.float32, device=x.device) if y is None else y
        ids = w = g = None
        if routing is not None:
            ids, w, g = routing
        _check(self.lib.moe_forward_noalloc(self.ctx, _ptr(x), T, _ptr(ids), _ptr(w), _ptr(g),
                                            _ptr(y), _stream(stream)), "moe_forward_noalloc")
        return y

    def plan(self, T: int, routing_given: bool = False):
        """Names of the kernels moe_forward enqueues for T tokens, in order."""
        n = ctypes.c_int32()
        names = (ctypes.c_char_p * 16)()
        _check(self.lib.moe_forward_plan(self.ctx, T, int(routing_given), ctypes.byref(n), names,
                                         16), "moe_forward_plan")
        return [names[i].decode() for i in range(n.value)]


def device_weights(layer: dict, device="cuda") -> dict:
    """Copy a numpy layer (sparse_moe_routing_amd.inputs.make_layer) to device tensors."""
    import numpy as np
    import torch

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return {k: dev(layer.get(k)) for k in WEIGHT_KEYS + ("x",)}


def layer_from_numpy(layer: dict, max_tokens: int, device="cuda"):
    """(MoeLayer, device tensors) for a numpy layer from sparse_moe_routing_amd.inputs."""
    w = layer["workload"]
    t = device_weights(layer, device)
    m = MoeLayer(w.hidden, w.num_experts, w.inter, w.shared_inter, max_tokens, w.dtype, t)
    return m, t
