"""Pins for the CPU oracle (no GPU): each check compares the oracle with something other than
itself - a library sort, closed forms, integer-exact arithmetic, a numpy/scipy SwiGLU, stable
argsort - and the planted-mistake builds show that every pin rejects a plausible error.

The layer follows the small-T MoE router commit message on the page "feat(windows): integrate
upstream Qwen3.8 DFlash2 support - #8": top-8 under the order (larger logit first, the lower
expert id on equal logits), softmax over the eight selected logits, a sigmoid shared-expert gate,
and a double-precision CPU reference checked at T = 1, 2, 19, 20, 46, 47, 768 and 4097.
"""
import math
import os
import tempfile

import numpy as np
import pytest
import scipy.special

import oracle as oracle_mod
from sparse_moe_routing_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers
def library_order(z_row: np.ndarray, E: int) -> np.ndarray:
    """Full order of experts by numpy's lexsort: primary key -z ascending (NaN sorts last),
    secondary key the id ascending. -0.0 and +0.0 compare equal in numpy's sort."""
    v = z_row[:E].astype(np.float64)
    return np.lexsort((np.arange(E), -v))


def tuple_sort_order(z_row, E):
    """A second brute force: Python's stable sort over (is_nan, -value, id) tuples."""
    keys = []
    for e in range(E):
        v = float(z_row[e])
        keys.append((math.isnan(v), 0.0 if math.isnan(v) else -v, e))
    return [k[2] for k in sorted(keys)]


def numpy_swiglu(x64, gu, dn, I):
    """Independent SwiGLU: np.matmul and scipy's logistic function."""
    a = x64 @ gu[:I].T
    u = x64 @ gu[I:].T
    h = a * scipy.special.expit(a) * u
    return h @ dn.T


def widen(a):
    if a.dtype == np.uint16:
        return inputs.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def tiny_layer(rng, T=3, H=16, E=8, I=8, Is=8, dtype="f32"):
    st = np.uint16 if dtype == "bf16" else np.float32

    def d(shape, s):
        v = (rng.standard_normal(shape) * s).astype(np.float32)
        return inputs.f32_to_bf16_bits(v) if dtype == "bf16" else v.astype(st)

    R = E + (1 if Is else 0)
    layer = {"num_experts": E, "inter": I, "shared_inter": Is, "top_k": 8, "dtype": dtype,
             "router_w": d((R, H), H ** -0.5), "router_bias": None,
             "gate_up": d((E, 2 * I, H), H ** -0.5), "down": d((E, H, I), I ** -0.5),
             "x": d((T, H), 1.0)}
    if Is:
        layer["shared_gate_up"] = d((2 * Is, H), H ** -0.5)
        layer["shared_down"] = d((H, Is), Is ** -0.5)
    else:
        layer["shared_gate_up"] = layer["shared_down"] = None
    return layer


def tie_heavy_logits(rng, T, E, gate=True):
    grid = np.array([-1.0, -0.75, -0.5, -0.25, -0.0, 0.0, 0.25, 0.5, 0.75, 1.0], np.float32)
    z = grid[rng.integers(0, len(grid), size=(T, E + (1 if gate else 0)))]
    return z.astype(np.float32)


# ----------------------------------------------------------------------------- pins
def pin_select_vs_library_sort(orc):
    rng = np.random.default_rng(11)
    for E in (8, 9, 16, 64, 256):
        for kind in ("normal", "ties", "special"):
            T = 40
            if kind == "normal":
                z = rng.standard_normal((T, E + 1)).astype(np.float32)
            elif kind == "ties":
                z = tie_heavy_logits(rng, T, E)
            else:
                z = tie_heavy_logits(rng, T, E)
                specials = np.array([np.nan, np.inf, -np.inf, -0.0, 0.0], np.float32)
                mask = rng.random((T, E + 1)) < 0.15
                z[mask] = specials[rng.integers(0, len(specials), size=mask.sum())]
            ids, w, g = orc.select(z, E, True)
            for t in range(T):
                lib = library_order(z[t], E)[:8]
                tup = tuple_sort_order(z[t], E)[:8]
                assert list(ids[t]) == list(lib), (E, kind, t, z[t], ids[t], lib)
                assert list(ids[t]) == tup


def pin_select_special_cases(orc):
    E = 256
    # all-equal logits: ids 0..7, weights exactly 1/8
    z = np.full((2, E + 1), 0.3, np.float32)
    z[1] = -0.0
    ids, w, g = orc.select(z, E, True)
    assert (ids == np.arange(8)).all()
    assert (w == 0.125).all()
    # distinct ascending logits, then a known permutation of the experts
    base = np.arange(E, dtype=np.float32) / 16.0
    rng = np.random.default_rng(5)
    perm = rng.permutation(E)
    z = np.zeros((2, E + 1), np.float32)
    z[0, :E] = base
    z[1, perm] = base  # expert perm[e] carries value base[e]
    ids, w, g = orc.select(z, E, True)
    want0 = np.arange(E - 1, E - 9, -1)
    assert (ids[0] == want0).all()
    assert (ids[1] == perm[want0]).all()
    assert np.array_equal(w[0], w[1])


def pin_weights_closed_form(orc):
    E = 16
    for L in (0.0, 0.5, 1.0, 3.0, -2.0):
        z = np.full((1, E + 1), -10.0, np.float32)
        z[0, 5] = L
        z[0, [1, 2, 3, 7, 9, 11, 13]] = 0.0
        ids, w, g = orc.select(z, E, True)
        if L > 0:
            assert ids[0, 0] == 5 and list(ids[0, 1:]) == [1, 2, 3, 7, 9, 11, 13]
            assert abs(w[0, 0] - math.exp(L) / (math.exp(L) + 7)) < 1e-12
            for k in range(1, 8):
                assert abs(w[0, k] - 1 / (math.exp(L) + 7)) < 1e-12
        assert abs(w[0].sum() - 1.0) < 1e-12
        assert (np.diff(w[0]) <= 1e-15).all()
    rng = np.random.default_rng(7)
    z = (rng.standard_normal((64, 257)) * 3).astype(np.float32)
    ids, w, g = orc.select(z, 256, True)
    assert np.abs(w.sum(1) - 1).max() < 1e-12
    assert (np.diff(w, axis=1) <= 1e-15).all()
    # reference softmax via scipy over the selected logits
    sel = np.take_along_axis(z[:, :256].astype(np.float64), ids, axis=1)
    assert np.abs(w - scipy.special.softmax(sel, axis=1)).max() < 1e-14
    # equivalently: the full softmax over all 256 experts renormalised to the selected eight
    full = scipy.special.softmax(z[:, :256].astype(np.float64), axis=1)
    fsel = np.take_along_axis(full, ids, axis=1)
    assert np.abs(w - fsel / fsel.sum(1, keepdims=True)).max() < 1e-12


def pin_gate(orc):
    E = 16
    z = np.zeros((4, E + 1), np.float32)
    z[:, E] = [0.0, np.inf, -np.inf, 2.0]
    _, _, g = orc.select(z, E, True)
    assert g[0] == 0.5 and g[1] == 1.0 and g[2] == 0.0
    assert abs(g[3] - scipy.special.expit(2.0)) < 1e-15
    rng = np.random.default_rng(3)
    z = rng.standard_normal((32, E + 1)).astype(np.float32)
    _, _, g = orc.select(z, E, True)
    assert np.abs(g - scipy.special.expit(z[:, E].astype(np.float64))).max() < 1e-15


def pin_logits_integer_exact(orc):
    rng = np.random.default_rng(9)
    for dtype in ("f32", "bf16"):
        T, H, R = 7, 96, 17
        xi = rng.integers(-8, 9, size=(T, H))
        wi = rng.integers(-8, 9, size=(R, H))
        bi = rng.integers(-64, 65, size=(R,))
        scale_w, scale_b = 2.0 ** -6, 2.0 ** -6
        xf = xi.astype(np.float32)
        wf = (wi * scale_w).astype(np.float32)
        bf = (bi * scale_b).astype(np.float32)
        if dtype == "bf16":
            xf, wf = inputs.f32_to_bf16_bits(xf), inputs.f32_to_bf16_bits(wf)
        z = orc.logits(xf, wf, bf)
        exact = (xi @ wi.T + bi[None, :]).astype(np.float64) * scale_w  # integers times 2^-6
        assert np.array_equal(z.astype(np.float64), exact), dtype


def pin_logits_random_vs_matmul(orc):
    rng = np.random.default_rng(10)
    layer = tiny_layer(rng, T=9, H=64, E=16, I=8, Is=8, dtype="bf16")
    b = rng.standard_normal(17).astype(np.float32)
    z = orc.logits(layer["x"], layer["router_w"], b)
    ref = widen(layer["x"]) @ widen(layer["router_w"]).T + b.astype(np.float64)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert (np.abs(z - ref) <= ulp).all()


def pin_bucket_vs_argsort(orc):
    rng = np.random.default_rng(12)
    for T, E in ((1, 16), (5, 16), (47, 256), (300, 256)):
        ids = np.stack([rng.permutation(E)[:8] for _ in range(T)]).astype(np.int32)
        counts, offsets, perm = orc.bucket(ids, E)
        flat = ids.ravel()
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
        assert np.array_equal(perm, np.argsort(flat, kind="stable"))


def pin_ffn_dense_equivalence(orc):
    """E = 8 identical experts: all eight are selected, the weights sum to 1, so the routed part
    equals one plain SwiGLU; with the shared expert the gate scales a second plain SwiGLU."""
    rng = np.random.default_rng(13)
    for dtype in ("f32", "bf16"):
        layer = tiny_layer(rng, T=5, H=32, E=8, I=12, Is=10, dtype=dtype)
        layer["gate_up"][:] = layer["gate_up"][0]
        layer["down"][:] = layer["down"][0]
        z, ids, w, g = orc.route(layer)
        assert sorted(ids[0]) == list(range(8))
        y = orc.forward(layer, ids, w, g)
        x64 = widen(layer["x"])
        routed = numpy_swiglu(x64, widen(layer["gate_up"][0]), widen(layer["down"][0]), 12)
        shared = numpy_swiglu(x64, widen(layer["shared_gate_up"]), widen(layer["shared_down"]), 10)
        ref = routed + g[:, None] * shared
        assert np.abs(y - ref).max() < 1e-12 * max(1.0, np.abs(ref).max()), dtype


def pin_ffn_shared_alone_and_zero(orc):
    rng = np.random.default_rng(14)
    layer = tiny_layer(rng, T=4, H=32, E=16, I=8, Is=8, dtype="f32")
    layer["down"][:] = 0.0
    layer["router_w"][16] = 0.0  # gate logit 0 -> g = 1/2
    z, ids, w, g = orc.route(layer)
    assert (g == 0.5).all()
    y = orc.forward(layer, ids, w, g)
    x64 = widen(layer["x"])
    ref = 0.5 * numpy_swiglu(x64, widen(layer["shared_gate_up"]), widen(layer["shared_down"]), 8)
    assert np.abs(y - ref).max() < 1e-12
    layer["x"][:] = 0.0
    z, ids, w, g = orc.route(layer)
    y = orc.forward(layer, ids, w, g)
    assert (y == 0.0).all()


def pin_ffn_routed_mixture(orc):
    """Distinct experts: y = sum_k w_k SwiGLU_{id_k}(x) + g SwiGLU_s(x) with numpy SwiGLUs."""
    rng = np.random.default_rng(15)
    for dtype in ("f32", "bf16"):
        layer = tiny_layer(rng, T=6, H=24, E=16, I=8, Is=4, dtype=dtype)
        z, ids, w, g = orc.route(layer)
        y = orc.forward(layer, ids, w, g, tokens=np.array([5, 0, 3], np.int32))
        x64 = widen(layer["x"])
        for j, t in enumerate((5, 0, 3)):
            ref = np.zeros(24)
            for k in range(8):
                e = ids[t, k]
                ref += w[t, k] * numpy_swiglu(x64[t:t + 1], widen(layer["gate_up"][e]),
                                              widen(layer["down"][e]), 8)[0]
            ref += g[t] * numpy_swiglu(x64[t:t + 1], widen(layer["shared_gate_up"]),
                                       widen(layer["shared_down"]), 4)[0]
            assert np.abs(y[j] - ref).max() < 1e-12, (dtype, t)


def pin_golden_hand_example(orc):
    path = os.path.join(GOLDEN, "select_hand.txt")
    rec = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, val = line.split(":", 1)
        rec[key.strip()] = val.strip()
    z1 = np.array([float(v) for v in rec["logits"].split()], np.float32)
    z2 = np.array([float(v) for v in rec["logits2"].split()], np.float32)
    ids, w, g = orc.select(np.stack([z1, z2]), 16, True)
    assert list(ids[0]) == [int(v) for v in rec["ids"].split()]
    assert list(ids[1]) == [int(v) for v in rec["ids2"].split()]
    env = {"exp": math.exp}
    S = eval(rec["S_expr"], env)
    env["S"] = S
    want = [eval(e.strip(), env) for e in rec["w2_exprs"].split(";")]
    assert np.abs(w[1] - np.array(want)).max() < 1e-12
    assert abs(g[1] - float(rec["g2_approx"])) < 1e-7


def pin_e4m3_values(orc):
    """The OCP FP8 E4M3 code points that the format's definition fixes: zero and negative zero,
    the smallest subnormal 2^-9, the smallest normal 2^-6, 1, 2, 1.875, the largest finite 448,
    NaN at S.1111.111 and no infinities; positive codes 0x00..0x7E strictly increasing and the
    negative half their mirror."""
    v = orc.e4m3_value
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x00)) == 1.0
    assert v(0x80) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9
    assert v(0x08) == 2.0 ** -6 and v(0x38) == 1.0 and v(0x40) == 2.0 and v(0x3F) == 1.875
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    pos = [v(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(pos, pos[1:]))
    assert all(v(0x80 | c) == -pos[c] for c in range(1, 0x7F))
    assert len(set(pos)) == 127 and all(math.isfinite(x) for x in pos)


def pin_e4m3_quantizer_round_trip(orc):
    """The input quantizer (nearest code, ties to the even code) maps every finite code value
    back to its code and every midpoint between neighbours to the even one of the two."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = np.array([orc.e4m3_value(int(c)) for c in codes], np.float32)
    assert np.array_equal(inputs.f32_to_e4m3_codes(vals), codes)
    pos = np.array([orc.e4m3_value(c) for c in range(0x7F)], np.float64)
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    got = inputs.f32_to_e4m3_codes(mid).astype(np.int64)
    lo = np.arange(126)
    assert np.all((got == lo) | (got == lo + 1)) and np.all(got % 2 == 0)
    assert inputs.f32_to_e4m3_codes(np.array([1e6, -1e6], np.float32)).tolist() == [0x7E, 0xFE]


def pin_fp8_forward_equals_bf16(orc):
    """FP8 weights with power-of-two row scales are exactly bf16 values (E4M3 has 3 mantissa bits),
    so the oracle's FP8 forward must equal its bf16 forward on those values, with every row's
    own scale (each row of gate, up and down gets a different power of two)."""
    rng = np.random.default_rng(31)
    T, H, E, I, Is = 3, 32, 8, 16, 24
    lay16 = {"num_experts": E, "inter": I, "shared_inter": Is, "top_k": 8, "dtype": "bf16"}
    lay8 = dict(lay16, dtype="fp8")

    def block(rows, cols):
        codes = rng.integers(0, 256, size=(rows, cols)).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x38  # no NaN codes
        scale = (2.0 ** rng.integers(-12, -4, size=rows)).astype(np.float32)
        vals = np.array([[orc.e4m3_value(int(c)) for c in r] for r in codes], np.float64)
        bits = inputs.f32_to_bf16_bits((vals * scale[:, None]).astype(np.float32))
        assert np.array_equal(inputs.bf16_bits_to_f32(bits), (vals * scale[:, None]).astype(np.float32))
        return codes, scale, bits

    gu8, gus, gu16 = zip(*[block(2 * I, H) for _ in range(E)])
    dn8, dns, dn16 = zip(*[block(H, I) for _ in range(E)])
    sgu8, sgus, sgu16 = block(2 * Is, H)
    sdn8, sdns, sdn16 = block(H, Is)
    x = inputs.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    lay16.update(x=x, gate_up=np.stack(gu16), down=np.stack(dn16), shared_gate_up=sgu16,
                 shared_down=sdn16)
    lay8.update(x=x, gate_up=np.stack(gu8), down=np.stack(dn8), shared_gate_up=sgu8,
                shared_down=sdn8, gate_up_scale=np.stack(gus), down_scale=np.stack(dns),
                shared_gate_up_scale=sgus, shared_down_scale=sdns)
    ids = np.stack([rng.permutation(E) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, E))
    w /= w.sum(1, keepdims=True)
    g = rng.random(T)
    y16 = orc.forward(lay16, ids, w, g)
    y8 = orc.forward(lay8, ids, w, g)
    assert np.abs(y8 - y16).max() <= 1e-12 * max(1.0, np.abs(y16).max())


# FP4 E2M1 magnitudes of codes 0..7 as the Open Compute Project's Microscaling (MX) formats
# specification lists them for its FP4 element type (codes 8..15: the same with the sign bit set)
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def pin_e2m1_values(orc):
    """Every FP4 E2M1 code against the MX specification's table: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and
    their negatives (code 8 is negative zero); no infinities or NaN."""
    for c in range(16):
        v = orc.e2m1_value(c)
        want = E2M1_TABLE[c & 7] * (-1.0 if c & 8 else 1.0)
        assert v == want and math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0), (c, v, want)


def pin_e8m0_values(orc):
    """E8M0 scale bytes: an exponent with bias 127 and no mantissa (0x7F is 1, 0x80 is 2, 0x00 the
    smallest 2^-127, 0xFE the largest 2^127), and 0xFF is NaN."""
    assert orc.e8m0_value(0x7F) == 1.0 and orc.e8m0_value(0x80) == 2.0
    assert orc.e8m0_value(0x7E) == 0.5 and orc.e8m0_value(0x7C) == 0.125
    assert orc.e8m0_value(0x00) == math.ldexp(1.0, -127)
    assert orc.e8m0_value(0xFE) == math.ldexp(1.0, 127)
    assert math.isnan(orc.e8m0_value(0xFF))


def pin_mxfp4_quantizer_nearest(orc):
    """The MXFP4 input quantizer against brute force on small blocks: each block's scale is
    2^(floor(log2 max|block|) - 2), and each weight's code is, of all sixteen codes, the one whose
    value times that scale is nearest to the weight (ties to the even code, beyond 6 saturated);
    the packing puts the even column in the low nibble."""
    rng = np.random.default_rng(41)
    v = (rng.standard_normal((6, 64)) * 2.0 ** rng.integers(-8, 3, size=(6, 1))).astype(np.float32)
    v[1, :32] = 0.0  # an all-zero block
    v[2, 5] = 0.0  # a zero inside a block
    # exact midpoints between neighbouring magnitudes (times the block's scale)
    sc3 = 2.0 ** (math.frexp(float(np.abs(v[3, :32]).max()))[1] - 1 - 2)
    v[3, 1:8] = (np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * sc3).astype(np.float32)
    packed, sb = inputs.quantize_blocks_mxfp4(v)
    assert packed.shape == (6, 32) and sb.shape == (6, 2)
    codes = np.stack([packed & 15, packed >> 4], axis=-1).reshape(6, 64)
    for r in range(6):
        for blk in range(2):
            seg = v[r, 32 * blk:32 * blk + 32].astype(np.float64)
            amax = np.abs(seg).max()
            want_b = 127 if amax == 0 else math.frexp(amax)[1] - 1 - 2 + 127
            assert sb[r, blk] == want_b, (r, blk, sb[r, blk], want_b)
            scale = orc.e8m0_value(int(sb[r, blk]))
            vals = [orc.e2m1_value(c) * scale for c in range(16)]
            for i, x in enumerate(seg):
                d = [abs(x - q) for q in vals]
                best = min(d)
                cands = [c for c in range(16) if d[c] == best]
                mags = sorted(set(c & 7 for c in cands))
                # the even magnitude code on a tie; zero is code 0
                m = mags[0] if len(mags) == 1 else [c for c in mags if c % 2 == 0][0]
                want = 0 if m == 0 else (m | (8 if x < 0 else 0))
                assert codes[r, 32 * blk + i] == want, (r, blk, i, x, codes[r, 32 * blk + i], want)


def pin_mxfp4_forward_equals_bf16(orc):
    """MXFP4 weights are bf16 values (E2M1 has one mantissa bit, E8M0 is a power of two), so the
    oracle's MXFP4 forward must equal its bf16 forward on the same values. The codes and scale
    bytes are encoded here from the specification's table, independently of the oracle, with a
    different scale on every block of every gate, up and down row."""
    rng = np.random.default_rng(43)
    T, H, E, I, Is = 3, 64, 8, 32, 64
    lay16 = {"num_experts": E, "inter": I, "shared_inter": Is, "top_k": 8, "dtype": "bf16"}
    lay4 = dict(lay16, dtype="mxfp4")
    table = np.array(E2M1_TABLE + [-t for t in E2M1_TABLE])

    def block(rows, cols):
        codes = rng.integers(0, 16, size=(rows, cols)).astype(np.uint8)
        sbytes = rng.integers(127 - 12, 127 - 2, size=(rows, cols // 32)).astype(np.uint8)
        vals = table[codes] * np.ldexp(1.0, sbytes.astype(np.int64) - 127).repeat(32, axis=1)
        bits = inputs.f32_to_bf16_bits(vals.astype(np.float32))
        assert np.array_equal(inputs.bf16_bits_to_f32(bits).astype(np.float64), vals)
        packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
        return packed, sbytes, bits

    gu4, gus, gu16 = zip(*[block(2 * I, H) for _ in range(E)])
    dn4, dns, dn16 = zip(*[block(H, I) for _ in range(E)])
    sgu4, sgus, sgu16 = block(2 * Is, H)
    sdn4, sdns, sdn16 = block(H, Is)
    x = inputs.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    lay16.update(x=x, gate_up=np.stack(gu16), down=np.stack(dn16), shared_gate_up=sgu16,
                 shared_down=sdn16)
    lay4.update(x=x, gate_up=np.stack(gu4), down=np.stack(dn4), shared_gate_up=sgu4,
                shared_down=sdn4, gate_up_scale=np.stack(gus), down_scale=np.stack(dns),
                shared_gate_up_scale=sgus, shared_down_scale=sdns)
    ids = np.stack([rng.permutation(E) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, E))
    w /= w.sum(1, keepdims=True)
    g = rng.random(T)
    y16 = orc.forward(lay16, ids, w, g)
    y4 = orc.forward(lay4, ids, w, g)
    assert np.abs(y4 - y16).max() <= 1e-12 * max(1.0, np.abs(y16).max())


PINS = [pin_select_vs_library_sort, pin_select_special_cases, pin_weights_closed_form, pin_gate,
        pin_logits_integer_exact, pin_logits_random_vs_matmul, pin_bucket_vs_argsort,
        pin_ffn_dense_equivalence, pin_ffn_shared_alone_and_zero, pin_ffn_routed_mixture,
        pin_golden_hand_example, pin_e4m3_values, pin_e4m3_quantizer_round_trip,
        pin_fp8_forward_equals_bf16, pin_e2m1_values, pin_e8m0_values,
        pin_mxfp4_quantizer_nearest, pin_mxfp4_forward_equals_bf16]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(oracle, pin):
    pin(oracle)


def test_oracle_p2_token_counts(oracle):
    """The token counts at which the pages' double-precision reference checks the op; the oracle's
    selection must agree with the library sort at each of them (E = 256, ties included)."""
    rng = np.random.default_rng(21)
    for T in (1, 2, 19, 20, 46, 47, 768, 4097):
        z = tie_heavy_logits(rng, T, 256) if T % 2 else rng.standard_normal((T, 257)).astype(np.float32)
        ids, w, g = oracle.select(z, 256, True)
        check = sorted(set([0, T - 1]) | set(rng.integers(0, T, size=min(T, 16)).tolist()))
        for t in check:
            assert list(ids[t]) == list(library_order(z[t], 256)[:8])
        assert np.abs(w.sum(1) - 1).max() < 1e-12


# ----------------------------------------------------------------------------- planted mistakes
PLANTS = {
    "ORACLE_PLANT_TIE_HIGH_ID": [pin_select_vs_library_sort, pin_select_special_cases,
                                 pin_golden_hand_example],
    "ORACLE_PLANT_SHIFT_ID8": [pin_select_vs_library_sort, pin_select_special_cases,
                               pin_golden_hand_example],
    "ORACLE_PLANT_SWAP_W67": [pin_weights_closed_form, pin_golden_hand_example],
    "ORACLE_PLANT_SWAP_GATE_UP": [pin_ffn_dense_equivalence, pin_ffn_routed_mixture],
    "ORACLE_PLANT_DROP_BIAS": [pin_logits_integer_exact, pin_logits_random_vs_matmul],
    "ORACLE_PLANT_E4M3_BIAS8": [pin_e4m3_values, pin_e4m3_quantizer_round_trip],
    "ORACLE_PLANT_UP_SCALE_ROW": [pin_fp8_forward_equals_bf16, pin_mxfp4_forward_equals_bf16],
    "ORACLE_PLANT_E8M0_BIAS128": [pin_e8m0_values, pin_mxfp4_forward_equals_bf16],
    "ORACLE_PLANT_FP4_HIGH_FIRST": [pin_mxfp4_forward_equals_bf16],
    "ORACLE_PLANT_E2M1_BIAS2": [pin_e2m1_values, pin_mxfp4_forward_equals_bf16],
}


@pytest.fixture(scope="module")
def plant_dir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("plant", sorted(PLANTS))
def test_planted_mistake_is_caught(plant, plant_dir):
    path = os.path.join(plant_dir, f"lib_{plant}.so")
    oracle_mod.build(path, defines=(plant,))
    bad = oracle_mod.Oracle(oracle_mod.load(path))
    for pin in PLANTS[plant]:
        with pytest.raises(AssertionError):
            pin(bad)


def test_workload_recipe_shapes():
    w = inputs.BY_NAME["tiny_fp32_t4"]
    layer = inputs.make_layer(w)
    assert layer["router_w"].shape == (17, 64) and layer["router_w"].dtype == np.float32
    assert layer["gate_up"].shape == (16, 64, 64)
    assert layer["down"].shape == (16, 64, 32)
    assert layer["x"].shape == (4, 64)
    again = inputs.make_layer(w)
    assert np.array_equal(layer["gate_up"], again["gate_up"])
    assert list(inputs.tie_tokens(w)) == [0, 2]
    # bf16 rounding: nearest-even on a few exact cases
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0], np.float32)
    back = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(v))
    assert list(back) == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 0.0]
    q = inputs.tie_quantize(np.array([[0.1, -0.1, 0.375, 0.125, 1.3]], np.float32), np.array([0]))
    assert list(q[0]) == [0.0, 0.0, 0.5, 0.0, 1.25] and np.signbit(q[0, 1])


def test_oracle_under_sanitizers(plant_dir):
    """Every oracle entry point (bf16, FP8 and MXFP4 forwards, logits, selection, bucketing, the
    format decoders) runs clean under AddressSanitizer and UndefinedBehaviorSanitizer: the oracle
    source is compiled into tests/sanitize_oracle.c's driver with both sanitizers (serial: no
    OpenMP runtime in the sanitized build), any invalid access or undefined operation aborts."""
    import shutil
    import subprocess
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    here = os.path.dirname(os.path.abspath(__file__))
    exe = os.path.join(plant_dir, "sanitize_oracle")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror", "-Wno-unused-parameter",
           "-Wno-unknown-pragmas", os.path.join(here, "sanitize_oracle.c"),
           os.path.join(os.path.dirname(here), "oracle", "moe_oracle.c"), "-o", exe, "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("checksum ") and "ERROR" not in r.stderr, r.stderr
