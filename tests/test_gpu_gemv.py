"""GPU parity of the vector-ALU decode expert kernels (gateup_gemv + down_rows) against the CPU
oracle, element by element, through the C ABI.

Contexts here are created with MOE_GEMV_MAX_TOKENS=64 so that every decode round up to 64 tokens
takes the vector-ALU kernels (whatever the library's default boundary), at the token counts of the
pages' operator sweep and CPU-reference check (1, 2, 19, 20, 46, 47) and at the decode rounds
(4, 32) and the limit (64), with ragged groups (experts holding 1 .. 5 tokens) and several shapes
(weight rows of 1, 2 and 4 kilobytes; intermediate rows of 1 and 2 kilobytes; no shared expert, a
wider shared expert). Bars as everywhere: y within |gpu - oracle| <= 1e-3 + 1e-2 |oracle|.
"""
import contextlib
import os

import numpy as np
import pytest

import oracle as oracle_mod
from sparse_moe_routing_amd import binding, inputs

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-3, 1e-2


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def orc():
    return oracle_mod.default()


@contextlib.contextmanager
def gemv_limit(value):
    """Contexts created inside take the vector-ALU gate/up up to `value` tokens."""
    saved = {k: os.environ.get(k) for k in ("MOE_GEMV_MAX_TOKENS",)}
    os.environ["MOE_GEMV_MAX_TOKENS"] = str(value)
    try:
        yield
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def assert_close(gpu, ref, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bad = np.abs(gpu - ref) > ATOL + RTOL * np.abs(ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first "
                             f"{[(tuple(i), gpu[tuple(i)], ref[tuple(i)]) for i in idx]}")


def x_device(a):
    torch = _torch()
    a = a.view(np.int16) if a.dtype == np.uint16 else a
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def routing_device(ids, w, g):
    torch = _torch()
    return (torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(),
            torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda(),
            None if g is None else torch.from_numpy(np.ascontiguousarray(g, np.float32)).cuda())


_DECODE = {}


def decode_layer():
    """The T=4 decode workload's weights (H 2048, 256 experts, I = I_s = 512) with a context whose
    decode rounds all run the vector-ALU kernels."""
    if "m" not in _DECODE:
        layer = inputs.make_layer(inputs.BY_NAME["decode_b1_t4"])
        with gemv_limit(64):
            m, t = binding.layer_from_numpy(layer, max_tokens=64)
        _DECODE.update(layer=layer, m=m, t=t)
    return _DECODE["layer"], _DECODE["m"], _DECODE["t"]


@pytest.mark.parametrize("T", [1, 2, 4, 19, 20, 32, 46, 47, 64])
def test_gemv_decode_shapes(orc, T):
    """Every output at the decode shapes: from the oracle's routing and from x (routing checked
    against the oracle's; a token whose ids differ must sit at a near-tie and is left out)."""
    torch = _torch()
    layer, m, t = decode_layer()
    assert m.plan(T)[-2:] == ["gateup_gemv", "down_rows"], m.plan(T)
    w = layer["workload"]
    x_np = inputs.draw_x(w, T, seed=700 + T)
    x = x_device(x_np)
    lay = dict(layer)
    lay["x"] = x_np
    z_o = orc.logits(x_np, layer["router_w"], None)
    ids_o, w_o, g_o = orc.select(z_o, w.num_experts, True)
    y_given = m.forward(x, routing=routing_device(ids_o, w_o, g_o))
    y_int = m.forward(x)
    _, ids, _, _ = m.route(x=x, want_logits=False)
    torch.cuda.synchronize()
    y_o = orc.forward(lay, ids_o, w_o, g_o)
    assert_close(y_given.cpu().numpy(), y_o, f"T={T} (oracle routing)")
    same = (ids.cpu().numpy() == ids_o).all(1)
    assert same.sum() >= T - max(1, T // 50)
    assert_close(y_int.cpu().numpy()[same], y_o[same], f"T={T} (from x)")


# (H, E, I, Is, token counts): rows of 1, 2 and 4 KB, intermediate of 1 and 2 KB, the shared
# expert absent or wider, few experts (several tokens per expert: batches of the gate/up kernel)
GEMV_SHAPES = [
    (512, 16, 512, 512, (1, 7, 33, 64)),
    (1024, 32, 1024, 512, (3, 20, 64)),
    (2048, 8, 512, 1024, (2, 17, 64)),     # 8 experts: every token selects all of them
    (1024, 64, 512, 0, (5, 46)),          # no shared expert
]


def small_layer(H, E, I, Is, T, seed):
    rng = np.random.default_rng(seed)

    def draw(shape, scale):
        return inputs.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))

    return {"num_experts": E, "inter": I, "shared_inter": Is,
            "router_w": draw((E + (1 if Is else 0), H), H ** -0.5), "router_bias": None,
            "gate_up": draw((E, 2 * I, H), H ** -0.5), "down": draw((E, H, I), I ** -0.5),
            "shared_gate_up": draw((2 * Is, H), H ** -0.5) if Is else None,
            "shared_down": draw((H, Is), Is ** -0.5) if Is else None,
            "x": draw((T, H), 1.0)}


@pytest.mark.parametrize("shape", GEMV_SHAPES, ids=lambda s: f"H{s[0]}-E{s[1]}-I{s[2]}-Is{s[3]}")
def test_gemv_shapes(orc, shape):
    torch = _torch()
    H, E, I, Is, Ts = shape
    layer = small_layer(H, E, I, Is, 64, seed=H + E + I + Is + 5)
    t = binding.device_weights(layer)
    with gemv_limit(64):
        m = binding.MoeLayer(H, E, I, Is, 64, "bf16", t)
    ws = m.workspace(64)
    for T in Ts:
        assert m.plan(T)[-2:] == ["gateup_gemv", "down_rows"], (shape, T, m.plan(T))
        lay = dict(layer)
        lay["x"] = layer["x"][:T]
        x = t["x"][:T].contiguous()
        z_o = orc.logits(lay["x"], layer["router_w"], None)
        ids_o, w_o, g_o = orc.select(z_o, E, Is > 0)
        y = m.forward(x, routing=routing_device(ids_o, w_o, g_o), ws=ws)
        torch.cuda.synchronize()
        assert int(ws[:m.state_bytes()].view(torch.int32).abs().sum()) == 0
        assert_close(y.cpu().numpy(), orc.forward(lay, ids_o, w_o, g_o), f"{shape} T={T}")


def test_gemv_batch_invariance_bitwise():
    """A token's output bits do not depend on the batch it comes in, on the vector-ALU path."""
    torch = _torch()
    layer, m, t = decode_layer()
    x = x_device(inputs.draw_x(layer["workload"], 64, seed=9))
    y64 = m.forward(x)
    y4 = m.forward(x[:4].contiguous())
    y1 = m.forward(x[9:10].contiguous())
    y33 = m.forward(x[31:64].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y64[:4], y4) and torch.equal(y64[9:10], y1) and torch.equal(y64[31:], y33)


def test_gemv_out_of_range_ids_add_nothing(orc):
    torch = _torch()
    layer, m, t = decode_layer()
    w = layer["workload"]
    T = 20
    x_np = inputs.draw_x(w, T, seed=71)
    lay = dict(layer)
    lay["x"] = x_np
    z_o = orc.logits(x_np, layer["router_w"], None)
    ids_o, w_o, g_o = orc.select(z_o, w.num_experts, True)
    bad = np.random.default_rng(3).random(ids_o.shape) < 0.25
    ids_bad = np.where(bad, np.int32(-3), ids_o)
    y = m.forward(x_device(x_np), routing=routing_device(ids_bad, w_o, g_o))
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), orc.forward(lay, ids_o, np.where(bad, 0.0, w_o), g_o),
                 "out-of-range ids")


# ------------------------------------------------------------------ quantized weights (FP8, MXFP4)
# The vector-ALU gate/up widens each lane's stored weights to the same eight bf16 operands the
# bf16 kernel reads at that lane, so on weights a bf16 context holds exactly (every MXFP4 weight;
# FP8 under power-of-two row scales) its outputs are the bf16 kernel's bits.
from test_gpu_parity import quantized_pair, quantized_small_layer  # noqa: E402


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_gemv_quantized_equals_bf16_of_decoded_weights_bitwise(fmt):
    torch = _torch()
    H, E, I, Is, Tmax = 1024, 16, 512, 512, 64
    q, b = quantized_pair(fmt, H, E, I, Is, Tmax, seed=51 if fmt == "fp8" else 52)
    tq, tb = binding.device_weights(q), binding.device_weights(b)
    with gemv_limit(64):
        mq = binding.MoeLayer(H, E, I, Is, Tmax, fmt, tq)
        mb = binding.MoeLayer(H, E, I, Is, Tmax, "bf16", tb)
    for T in (1, 4, 19, 32, 64):
        assert mq.plan(T)[-2:] == ["gateup_gemv", "down_rows"], (fmt, T, mq.plan(T))
        x = tb["x"][:T].contiguous()
        yq = mq.forward(x)
        yb = mb.forward(x)
        torch.cuda.synchronize()
        assert torch.isfinite(yb).all(), (fmt, T)
        diff = (yq != yb).nonzero()
        assert diff.numel() == 0, (fmt, T, diff[:5].tolist())


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("shape", [(1024, 32, 512, 512), (2048, 16, 1024, 512), (512, 64, 512, 0)],
                         ids=lambda s: f"H{s[0]}-E{s[1]}-I{s[2]}-Is{s[3]}")
def test_gemv_quantized_oracle(orc, fmt, shape):
    """Quantized layers of normal draws on the vector-ALU path against the oracle, every output,
    from the oracle's routing, at ragged token counts."""
    torch = _torch()
    H, E, I, Is = shape
    layer = quantized_small_layer(fmt, H, E, I, Is or I, 64, seed=H + E + I + Is)
    if not Is:  # no shared expert: its weights and gate row dropped
        for k in ("shared_gate_up", "shared_down", "shared_gate_up_scale", "shared_down_scale"):
            layer[k] = None
        layer["shared_inter"] = 0
        layer["router_w"] = layer["router_w"][:E]
    t = binding.device_weights(layer)
    with gemv_limit(64):
        m = binding.MoeLayer(H, E, I, Is, 64, fmt, t)
    ws = m.workspace(64)
    for T in (1, 4, 20, 47, 64):
        assert m.plan(T)[-2:] == ["gateup_gemv", "down_rows"], (fmt, shape, T, m.plan(T))
        lay = dict(layer)
        lay["x"] = layer["x"][:T]
        z_o = orc.logits(lay["x"], layer["router_w"], None)
        ids_o, w_o, g_o = orc.select(z_o, E, Is > 0)
        y = m.forward(t["x"][:T].contiguous(), routing=routing_device(ids_o, w_o, g_o), ws=ws)
        torch.cuda.synchronize()
        assert int(ws[:m.state_bytes()].view(torch.int32).abs().sum()) == 0
        assert_close(y.cpu().numpy(), orc.forward(lay, ids_o, w_o, g_o), f"{fmt} {shape} T={T}")


def test_down_rows_groups_past_the_stage(orc):
    """The default decode plan (matrix-core gate/up, down_rows) with groups of up to 8 tokens:
    with 8 experts every token selects all of them, so every group past T = 4 has members beyond
    the four whose h rows a ring stage holds; every output against the oracle."""
    torch = _torch()
    H, E, I, Is = 1024, 8, 512, 512
    layer = small_layer(H, E, I, Is, 64, seed=88)
    t = binding.device_weights(layer)
    m = binding.MoeLayer(H, E, I, Is, 64, "bf16", t)
    ws = m.workspace(64)
    for T in (5, 8, 9, 17, 33, 64):
        assert m.plan(T)[-2:] == ["gateup", "down_rows"], (T, m.plan(T))
        lay = dict(layer)
        lay["x"] = layer["x"][:T]
        z_o = orc.logits(lay["x"], layer["router_w"], None)
        ids_o, w_o, g_o = orc.select(z_o, E, True)
        y = m.forward(t["x"][:T].contiguous(), routing=routing_device(ids_o, w_o, g_o), ws=ws)
        y_int = m.forward(t["x"][:T].contiguous(), ws=ws)
        torch.cuda.synchronize()
        y_o = orc.forward(lay, ids_o, w_o, g_o)
        assert_close(y.cpu().numpy(), y_o, f"E=8 T={T}")
        assert_close(y_int.cpu().numpy(), y_o, f"E=8 T={T} (from x)")  # every token: all 8
