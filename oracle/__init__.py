"""Plain fp64 CPU oracle for the sparse MoE layer (ctypes wrapper over moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package; the library under ``sparse_moe_routing_amd`` never does, and the two
share no code. Every function here only marshals numpy arrays into the C oracle, whose header
states what each step computes and which passage of the pages it follows
("feat(windows): integrate upstream Qwen3.8 DFlash2 support - #8", the small-T MoE router
commit message).

bf16 tensors are passed as ``numpy.uint16`` arrays holding the raw bf16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

F32 = 0
BF16 = 1
FP8 = 2  # expert weights only: OCP FP8 E4M3 codes (numpy.uint8) with fp32 per-row scales
MXFP4 = 3  # expert weights only: OCP MXFP4, packed E2M1 codes with E8M0 scale bytes per 32

_lock = threading.Lock()
_lib = None


def build(out_path: str = _LIB_PATH, defines: tuple[str, ...] = ()) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-Werror", "-Wno-unused-parameter"]
    cmd += [f"-D{d}" for d in defines]
    tmp = out_path + f".tmp{os.getpid()}"
    cmd += [_SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if needed) an oracle shared library and declare its signatures."""
    global _lib
    if path is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(_LIB_PATH) or (
                        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
                    build()
                _lib = _declare(ctypes.CDLL(_LIB_PATH))
            return _lib
    return _declare(ctypes.CDLL(path))


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.c_void_p
    i = ctypes.c_int
    lib.oracle_logits.argtypes = [i, i, i, i, P, P, P, P]
    lib.oracle_select.argtypes = [i, i, i, P, i, i, P, P, P]
    lib.oracle_bucket.argtypes = [i, i, P, P, P, P]
    lib.oracle_forward.argtypes = [i, P, i, i, i, i, i, i, i, P, P, P, P, P, P, P, P, P]
    lib.oracle_forward_w.argtypes = [i, P, i, i, i, i, i, i, i, i, P, P, P, P, P, P, P, P, P, P,
                                     P, P, P]
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    for f in (lib.oracle_e2m1_value, lib.oracle_e8m0_value):
        f.argtypes = [ctypes.c_uint8]
        f.restype = ctypes.c_double
    for f in (lib.oracle_logits, lib.oracle_select, lib.oracle_bucket, lib.oracle_forward,
              lib.oracle_forward_w, lib.oracle_num_threads):
        f.restype = ctypes.c_int
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs must be float32 or uint16 (bf16 bits), got {a.dtype}")


class Oracle:
    """Bound view of one oracle build (the default build, or a planted-mistake variant)."""

    def __init__(self, lib: ctypes.CDLL | None = None):
        self.lib = lib if lib is not None else load()

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        """Threads of the oracle's later parallel regions (the baseline timing only)."""
        self.lib.oracle_set_num_threads(int(n))

    def logits(self, x: np.ndarray, router_w: np.ndarray, bias: np.ndarray | None = None):
        """z[t][r] = fp32(sum_h W[r][h] x[t][h] + b[r]) with fp64 accumulation."""
        x = np.ascontiguousarray(x)
        router_w = np.ascontiguousarray(router_w)
        dt = _dtype_code(x)
        assert _dtype_code(router_w) == dt
        T, H = x.shape
        R = router_w.shape[0]
        assert router_w.shape[1] == H
        if bias is not None:
            bias = np.ascontiguousarray(bias, dtype=np.float32)
            assert bias.shape == (R,)
        z = np.empty((T, R), dtype=np.float32)
        rc = self.lib.oracle_logits(T, H, R, dt, _ptr(x), _ptr(router_w), _ptr(bias), _ptr(z))
        if rc:
            raise ValueError("oracle_logits rejected its arguments")
        return z

    def select(self, z: np.ndarray, num_experts: int, has_gate: bool, k: int = 8):
        """Top-k ids under the total order, softmax weights (fp64), sigmoid gate (fp64)."""
        z = np.ascontiguousarray(z, dtype=np.float32)
        T, stride = z.shape
        ids = np.empty((T, k), dtype=np.int32)
        w = np.empty((T, k), dtype=np.float64)
        g = np.empty((T,), dtype=np.float64)
        rc = self.lib.oracle_select(T, num_experts, stride, _ptr(z), int(bool(has_gate)), k,
                                    _ptr(ids), _ptr(w), _ptr(g))
        if rc:
            raise ValueError("oracle_select rejected its arguments")
        return ids, w, (g if has_gate else None)

    def bucket(self, ids: np.ndarray, num_experts: int):
        """Stable counting sort of the flattened pair indices by expert id."""
        flat = np.ascontiguousarray(ids, dtype=np.int32).ravel()
        n = flat.size
        counts = np.empty((num_experts,), dtype=np.int32)
        offsets = np.empty((num_experts + 1,), dtype=np.int32)
        perm = np.empty((n,), dtype=np.int32)
        rc = self.lib.oracle_bucket(n, num_experts, _ptr(flat), _ptr(counts), _ptr(offsets),
                                    _ptr(perm))
        if rc:
            raise ValueError("oracle_bucket rejected its arguments")
        return counts, offsets, perm

    def forward(self, layer, ids: np.ndarray, w: np.ndarray, g: np.ndarray | None,
                tokens=None) -> np.ndarray:
        """y[j] for each token tokens[j] (all tokens when None), fp64, from the given routing."""
        x = layer["x"]
        T, H = x.shape
        E = layer["num_experts"]
        I = layer["inter"]
        Is = layer["shared_inter"]
        dt = _dtype_code(x)
        if tokens is None:
            tokens = np.arange(T, dtype=np.int32)
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        k = ids.shape[1]
        w = np.ascontiguousarray(w, dtype=np.float64)
        if g is not None:
            g = np.ascontiguousarray(g, dtype=np.float64)
        y = np.empty((tokens.size, H), dtype=np.float64)
        sgu = layer.get("shared_gate_up") if Is > 0 else None
        sdn = layer.get("shared_down") if Is > 0 else None
        if layer["gate_up"].dtype == np.uint8:
            # FP8 E4M3 codes with fp32 per-row scales, or MXFP4 packed codes with E8M0 scale bytes
            mx = layer.get("dtype") == "mxfp4"
            st = np.uint8 if mx else np.float32

            def sc_arr(a):
                return None if a is None else np.ascontiguousarray(a, dtype=st)
            sc = [sc_arr(layer.get(n)) for n in ("gate_up_scale", "down_scale",
                                                 "shared_gate_up_scale", "shared_down_scale")]
            rc = self.lib.oracle_forward_w(tokens.size, _ptr(tokens), T, H, E, I, Is, k, dt,
                                           MXFP4 if mx else FP8,
                                           _ptr(x), _ptr(layer["gate_up"]), _ptr(layer["down"]),
                                           _ptr(sgu), _ptr(sdn), *[_ptr(a) for a in sc],
                                           _ptr(ids), _ptr(w), _ptr(g), _ptr(y))
        else:
            rc = self.lib.oracle_forward(tokens.size, _ptr(tokens), T, H, E, I, Is, k, dt,
                                         _ptr(x), _ptr(layer["gate_up"]), _ptr(layer["down"]),
                                         _ptr(sgu), _ptr(sdn), _ptr(ids), _ptr(w), _ptr(g),
                                         _ptr(y))
        if rc:
            raise ValueError("oracle_forward rejected its arguments")
        return y

    def e4m3_value(self, code: int) -> float:
        """The value of one OCP FP8 E4M3 code (NaN for the two NaN codes)."""
        return float(self.lib.oracle_e4m3_value(int(code)))

    def e2m1_value(self, code: int) -> float:
        """The value of one FP4 E2M1 code (the low four bits of `code`)."""
        return float(self.lib.oracle_e2m1_value(int(code)))

    def e8m0_value(self, b: int) -> float:
        """The value of one E8M0 scale byte (NaN for 0xFF)."""
        return float(self.lib.oracle_e8m0_value(int(b)))

    def route(self, layer, logits_override=None):
        """Logits (fp32), then selection on them: the plain path from x to (ids, w, g)."""
        z = self.logits(layer["x"], layer["router_w"], layer.get("router_bias"))
        if logits_override is not None:
            z = logits_override
        ids, w, g = self.select(z, layer["num_experts"], layer["shared_inter"] > 0)
        return z, ids, w, g


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
