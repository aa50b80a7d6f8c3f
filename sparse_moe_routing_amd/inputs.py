"""Seeded synthetic workloads for the sparse MoE layer.

This module only draws and stores inputs; it holds none of the layer's arithmetic. The tests
feed the same arrays to the CPU oracle and to the HIP library, and the benchmark uses the same
shapes. numpy and the standard library only (no torch), so it imports anywhere.

Shapes and value distributions follow the five workloads the layer is measured on: the
decode and speculative-verify rounds of T = batch x (draft + 1) tokens described on the page
"feat(windows): integrate upstream Qwen3.8 DFlash2 support - #8" (T=4 at batch 1, T=32 at
batch 8, both with three draft tokens; a prefill chunk of 8192 tokens), with Qwen-family MoE
sizes: hidden 2048, 256 experts, top-8, expert and shared-expert intermediate 512.

Recipe (all draws from ``numpy.random.default_rng(seed)``, PCG64, ``standard_normal`` in
float32):
  1. router weight [E+1][H] (row E is the shared-expert gate row), scaled by 1/sqrt(H);
  2. only when the workload has a router bias: bias[E] scaled by sqrt(2) (variance 2); the
     gate row's bias is 0;
  3. for e = 0..E-1 in order: gate [I][H] and up [I][H] scaled by 1/sqrt(H), then down [H][I]
     scaled by 1/sqrt(I);
  4. shared expert: gate [Is][H], up [Is][H] (1/sqrt(H)), down [H][Is] (1/sqrt(Is));
  5. x [T][H], unscaled N(0, 1).
bf16 workloads round every draw to bf16 with round-to-nearest-even and store the raw bits as
uint16. fp8 workloads store x and the router weight as bf16 and quantize each expert weight row
(routed and shared, gate, up and down alike) to OCP FP8 E4M3 codes (uint8) with one float32
scale per row: scale = max|row| / 448 (1 for an all-zero row), code = the E4M3 value nearest to
v / scale (ties to the even code), so the row's largest magnitude becomes 448; the scales are
stored next to the codes as gate_up_scale [E][2I], down_scale [E][H], shared_gate_up_scale
[2Is], shared_down_scale [H]. gate and up are stored stacked as gate_up [E][2I][H] (gate rows first); down is
[E][H][I] (the nn.Linear convention: output rows, input columns contiguous).
mxfp4 workloads quantize the same expert weight rows to OCP MXFP4 (the Open Compute Project's
Microscaling formats): each block of 32 consecutive weights of a row shares one E8M0 scale byte
b (scale 2^(b - 127)), chosen as 2^(floor(log2(max|block|)) - 2) (the largest E2M1 magnitude is
6 = 1.5 * 2^2; an all-zero block takes b = 127), and each weight becomes the FP4 E2M1 code nearest
to v / scale (ties to the even code, magnitudes above 6 saturate to 6). Codes are packed two per
byte along the row, the even column in the low nibble: gate_up [E][2I][H/2], down [E][H][I/2],
shared [2Is][H/2], [H][Is/2]; the scale bytes are gate_up_scale [E][2I][H/32], down_scale
[E][H][I/32], shared_gate_up_scale [2Is][H/32], shared_down_scale [H][Is/32].

Tie tokens: selected tokens have every router score replaced by the nearest multiple of 0.25
(ties to even), which forces equal logits across experts; those tokens are routed from the given
logits rather than from x.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    hidden: int
    num_experts: int
    top_k: int
    inter: int
    shared_inter: int
    dtype: str            # "f32" or "bf16": storage type of x and of every weight; "fp8": x and
                          # the router in bf16, expert weights as FP8 E4M3 codes + row scales;
                          # "mxfp4": as fp8 with MXFP4 expert weights (E2M1 + E8M0 per 32)
    bias_std: float = 0.0  # > 0: per-expert router bias ~ N(0, bias_std^2)
    tie_every: int = 0     # > 0: tokens t with t % tie_every == 0 get tie-quantized logits
    seed: int = 0


WORKLOADS = (
    Workload("tiny_fp32_t4", 4, 64, 16, 8, 32, 32, "f32", tie_every=2, seed=0),
    Workload("decode_b1_t4", 4, 2048, 256, 8, 512, 512, "bf16", seed=1),
    Workload("decode_b8_t32", 32, 2048, 256, 8, 512, 512, "bf16", seed=2),
    Workload("verify_skewed_t192", 192, 2048, 256, 8, 512, 512, "bf16", bias_std=2.0 ** 0.5,
             seed=3),
    Workload("prefill_t8192", 8192, 2048, 256, 8, 512, 512, "bf16", tie_every=10, seed=4),
    # the same rounds with FP8 E4M3 expert weights (x and router in bf16)
    Workload("decode_b1_t4_fp8", 4, 2048, 256, 8, 512, 512, "fp8", seed=11),
    Workload("decode_b8_t32_fp8", 32, 2048, 256, 8, 512, 512, "fp8", seed=12),
    Workload("verify_skewed_t192_fp8", 192, 2048, 256, 8, 512, 512, "fp8",
             bias_std=2.0 ** 0.5, seed=13),
    Workload("prefill_t8192_fp8", 8192, 2048, 256, 8, 512, 512, "fp8", tie_every=10, seed=14),
    # and with MXFP4 expert weights
    Workload("decode_b1_t4_mxfp4", 4, 2048, 256, 8, 512, 512, "mxfp4", seed=21),
    Workload("decode_b8_t32_mxfp4", 32, 2048, 256, 8, 512, 512, "mxfp4", seed=22),
    Workload("verify_skewed_t192_mxfp4", 192, 2048, 256, 8, 512, 512, "mxfp4",
             bias_std=2.0 ** 0.5, seed=23),
    Workload("prefill_t8192_mxfp4", 8192, 2048, 256, 8, 512, 512, "mxfp4", tie_every=10,
             seed=24),
)
BY_NAME = {w.name: w for w in WORKLOADS}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the raw uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bits to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes of float32 values (nearest, ties to the even code; magnitudes above the
    largest finite value 448 saturate to it). Sign bit, then 4 exponent bits (bias 7) and 3
    mantissa bits; exponent field 0 holds the subnormal multiples of 2^-9."""
    a = np.asarray(a, dtype=np.float32)
    sign = (a.view(np.uint32) >> np.uint32(24)).astype(np.uint8) & np.uint8(0x80)
    v = np.minimum(np.abs(a), np.float32(448.0))
    # normal range (v >= 2^-6): round the float32 significand to 3 bits, nearest-even; a carry
    # into the exponent falls out of the integer add
    b = v.view(np.uint32)
    b = b + np.uint32(0x7FFFF) + ((b >> np.uint32(20)) & np.uint32(1))
    ex = (b >> np.uint32(23)).astype(np.int32) - 127
    code_n = ((ex + 7) << 3) | ((b >> np.uint32(20)) & np.uint32(7)).astype(np.int32)
    # subnormal range: multiples of 2^-9 (8 * 2^-9 is 2^-6, whose code is 8)
    code_s = np.rint(v * np.float32(512.0)).astype(np.int32)
    code = np.where(v >= np.float32(2.0 ** -6), code_n, code_s)
    return code.astype(np.uint8) | sign


def quantize_rows_e4m3(v: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row FP8 E4M3 quantization of a float32 matrix [..., rows, cols]: (codes, scales)."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.max(np.abs(v), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return f32_to_e4m3_codes(v / scale[..., None]), scale


def f32_to_e2m1_codes(a: np.ndarray) -> np.ndarray:
    """FP4 E2M1 codes (uint8, 0..15) of float32 values: the nearest of the eight magnitudes
    0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the even code, magnitudes above 6 saturated to 6; the sign
    in bit 3 (zero is code 0). Sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent
    field 0 holds 0 and the subnormal 0.5."""
    a = np.asarray(a, dtype=np.float32)
    v = np.abs(a)
    # from 1 up: round the float32 significand to 1 bit, nearest-even (a carry moves the exponent)
    b = v.view(np.uint32)
    b = b + np.uint32(0x1FFFFF) + ((b >> np.uint32(22)) & np.uint32(1))
    ex = (b >> np.uint32(23)).astype(np.int32) - 127
    code_n = np.where(ex > 2, 7, ((ex + 1) << 1) | ((b >> np.uint32(22)) & np.uint32(1)).astype(np.int32))
    # below 1: multiples of 0.5 (2 * 0.5 is 1.0, whose code is 2); rint rounds ties to even
    code_s = np.rint(v * np.float32(2.0)).astype(np.int32)
    code = np.where(v >= np.float32(1.0), code_n, code_s)
    return (code | np.where(np.signbit(a) & (code > 0), 8, 0)).astype(np.uint8)


def quantize_blocks_mxfp4(v: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """MXFP4 quantization of a float32 matrix [..., rows, cols] (cols a multiple of 32):
    (packed codes [..., rows, cols / 2], E8M0 scale bytes [..., rows, cols / 32])."""
    v = np.asarray(v, dtype=np.float32)
    blocks = v.reshape(v.shape[:-1] + (v.shape[-1] // 32, 32))
    amax = np.max(np.abs(blocks), axis=-1)
    _, ex = np.frexp(amax)  # amax = m * 2^ex with m in [0.5, 1): floor(log2(amax)) = ex - 1
    e = np.clip(ex.astype(np.int32) - 1 - 2, -127, 127)
    e = np.where(amax > 0, e, 0)
    scale_b = (e + 127).astype(np.uint8)
    x = np.ldexp(blocks, -e[..., None]).astype(np.float32)  # exact: a power-of-two scale
    codes = f32_to_e2m1_codes(x).reshape(v.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, scale_b


def _draw(rng, shape, scale, dtype):
    v = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        v *= np.float32(scale)
    if dtype in ("fp8", "mxfp4"):  # activations and the router stay bf16 in these workloads
        dtype = "bf16"
    return f32_to_bf16_bits(v) if dtype == "bf16" else v


def _draw_w(rng, shape, scale, dtype):
    """An expert weight block: as _draw, or (codes, per-row scales) for fp8, or (packed codes,
    block scale bytes) for mxfp4."""
    if dtype == "mxfp4":
        return quantize_blocks_mxfp4(_draw(rng, shape, scale, "f32"))
    if dtype != "fp8":
        return _draw(rng, shape, scale, dtype), None
    return quantize_rows_e4m3(_draw(rng, shape, scale, "f32"))


def make_layer(w: Workload, tokens: int | None = None, seed: int | None = None) -> dict:
    """Draw one layer (weights + x) following the recipe above.

    ``tokens`` overrides T (the weights do not depend on T; x is drawn last).
    """
    T = w.tokens if tokens is None else tokens
    rng = np.random.default_rng(w.seed if seed is None else seed)
    H, E, I, Is = w.hidden, w.num_experts, w.inter, w.shared_inter
    R = E + (1 if Is > 0 else 0)
    st = np.uint16 if w.dtype == "bf16" else np.float32
    layer = {"workload": w, "num_experts": E, "inter": I, "shared_inter": Is, "top_k": w.top_k,
             "dtype": w.dtype}
    layer["router_w"] = _draw(rng, (R, H), H ** -0.5, w.dtype)
    if w.bias_std > 0:
        b = np.zeros((R,), dtype=np.float32)
        b[:E] = rng.standard_normal((E,), dtype=np.float32) * np.float32(w.bias_std)
        layer["router_bias"] = b
    else:
        layer["router_bias"] = None
    mx = w.dtype == "mxfp4"
    fp8 = w.dtype == "fp8" or mx  # scaled one-byte storage
    if fp8:
        st = np.uint8
    pk = 2 if mx else 1  # elements per stored byte
    gate_up = np.empty((E, 2 * I, H // pk), dtype=st)
    down = np.empty((E, H, I // pk), dtype=st)
    gu_s = (np.empty((E, 2 * I, H // 32), np.uint8) if mx else
            np.empty((E, 2 * I), np.float32) if fp8 else None)
    dn_s = (np.empty((E, H, I // 32), np.uint8) if mx else
            np.empty((E, H), np.float32) if fp8 else None)
    for e in range(E):
        gate_up[e, :I], sg = _draw_w(rng, (I, H), H ** -0.5, w.dtype)
        gate_up[e, I:], su = _draw_w(rng, (I, H), H ** -0.5, w.dtype)
        down[e], sd = _draw_w(rng, (H, I), I ** -0.5, w.dtype)
        if fp8:
            gu_s[e, :I], gu_s[e, I:], dn_s[e] = sg, su, sd
    layer["gate_up"] = gate_up
    layer["down"] = down
    layer["gate_up_scale"] = gu_s
    layer["down_scale"] = dn_s
    if Is > 0:
        sgu = np.empty((2 * Is, H // pk), dtype=st)
        sgu[:Is], sg = _draw_w(rng, (Is, H), H ** -0.5, w.dtype)
        sgu[Is:], su = _draw_w(rng, (Is, H), H ** -0.5, w.dtype)
        layer["shared_gate_up"] = sgu
        layer["shared_down"], sd = _draw_w(rng, (H, Is), Is ** -0.5, w.dtype)
        layer["shared_gate_up_scale"] = np.concatenate([sg, su]) if fp8 else None
        layer["shared_down_scale"] = sd
    else:
        layer["shared_gate_up"] = None
        layer["shared_down"] = None
        layer["shared_gate_up_scale"] = None
        layer["shared_down_scale"] = None
    layer["x"] = _draw(rng, (T, H), 1.0, w.dtype)
    return layer


def draw_x(w: Workload, tokens: int, seed: int) -> np.ndarray:
    """A fresh activation batch [tokens][H] of the workload's storage type."""
    rng = np.random.default_rng(seed)
    return _draw(rng, (tokens, w.hidden), 1.0, w.dtype)


def tie_tokens(w: Workload, tokens: int | None = None) -> np.ndarray:
    """Indices of the tokens whose logits are tie-quantized."""
    T = w.tokens if tokens is None else tokens
    if w.tie_every <= 0:
        return np.zeros((0,), dtype=np.int64)
    return np.arange(0, T, w.tie_every, dtype=np.int64)


def tie_quantize(z: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Copy of z with the given rows rounded to multiples of 0.25 (ties to even)."""
    q = np.array(z, dtype=np.float32, copy=True)
    if len(rows):
        q[rows] = np.round(q[rows] * np.float32(4.0)) / np.float32(4.0)
    return q


def sample_tokens(T: int, n: int, seed: int = 1234, must=()) -> np.ndarray:
    """A sorted, seeded sample of min(n, T) distinct token indices including the first and last
    tokens and any indices in ``must``."""
    if T <= n:
        return np.arange(T, dtype=np.int32)
    rng = np.random.default_rng(seed)
    pick = set(int(t) for t in must if 0 <= t < T)
    pick.update((0, T - 1))
    rest = rng.choice(T, size=max(0, n - len(pick)), replace=False)
    pick.update(int(t) for t in rest)
    return np.array(sorted(pick)[:max(n, len(pick))], dtype=np.int32)
