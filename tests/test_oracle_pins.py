"""Pins for the CPU oracle: each test checks it against something other than itself.

Pins used (and what each would catch):
* the FP4 E2M1 table of the OCP MX spec and the E8M0 powers of two (wrong code
  table, wrong bias, sign of zero);
* hand-built MXFP4 bytes (nibble order, scale block index);
* library routines on tiny inputs: numpy float64 matmul for the router and both
  expert GEMMs, a stable sort for top-k, scipy's softmax (dropped bias, transposed
  operand, wrong index, wrong softmax scope);
* closed-form SwiGLU identities and clamp behaviour (wrong clamp side, wrong
  alpha, missing +1);
* constructed experts whose outputs are known exactly: identity gate rows on a
  non-square shape (orientation, gate/up interleave), zero up rows with up bias
  -1 (interleave, bias inside the weighted sum), doubled down scales (linearity);
* the layer invariant that only routed experts matter (ZeroModels GPT-OSS page,
  "MXFP4 experts": routed-only and full-bank evaluation give identical results).
"""
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from workloads import CONFIGS, make_inputs, f32_from_bf16_bits, bf16_bits_from_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- element formats

def test_e2m1_table_matches_ocp_spec():
    table = _read_table("e2m1_table.txt")
    assert len(table) == 16
    for code_s, val_s in table:
        code, want = int(code_s), float(val_s)
        got = oracle.e2m1(code)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_e2m1_sign_symmetry_and_exact_in_bf16():
    for c in range(8):
        assert oracle.e2m1(c | 8) == -oracle.e2m1(c)
        assert math.copysign(1, oracle.e2m1(c | 8)) == -1.0
    # every e2m1 value times every scale in the workloads' range is a bf16 value
    vals = np.array([oracle.e2m1(c) * oracle.e8m0(s) for c in range(16) for s in range(115, 130)],
                    dtype=np.float32)
    assert np.array_equal(f32_from_bf16_bits(bf16_bits_from_f32(vals)), vals)


def test_e8m0_powers_of_two():
    assert oracle.e8m0(127) == 1.0
    assert oracle.e8m0(128) == 2.0
    assert oracle.e8m0(126) == 0.5
    assert oracle.e8m0(119) == 1.0 / 256
    assert oracle.e8m0(124) == 0.125
    assert oracle.e8m0(121) == 1.0 / 64          # 2^-6, lowest tiny-config scale
    assert oracle.e8m0(125) == 0.25              # 2^-2, highest tiny-config scale
    assert oracle.e8m0(0) == 2.0 ** -127
    assert oracle.e8m0(254) == 2.0 ** 127
    assert math.isnan(oracle.e8m0(255))
    for s in range(0, 254):
        assert oracle.e8m0(s) * 2.0 == oracle.e8m0(s + 1)


def test_dequant_hand_bytes():
    for byte_s, scale_s, even_s, odd_s in _read_table("mxfp4_bytes.txt"):
        blocks = np.full((1, 16), int(byte_s, 16), dtype=np.uint8)
        scales = np.array([[int(scale_s)]], dtype=np.uint8)
        w = oracle.dequant(blocks, scales)
        assert w.shape == (1, 32)
        even, odd = float(even_s), float(odd_s)
        assert np.all(w[0, 0::2] == even) and np.all(w[0, 1::2] == odd)
        assert np.all(np.signbit(w[0, 0::2]) == (math.copysign(1, even) < 0))
        assert np.all(np.signbit(w[0, 1::2]) == (math.copysign(1, odd) < 0))


def test_dequant_scale_block_index_and_row_stride():
    # rows x cols = 3 x 96: three scale blocks per row; each block a different scale
    blocks = np.full((3, 48), 0x22, dtype=np.uint8)          # every weight code 2 = 1.0
    scales = np.array([[127, 128, 129], [126, 127, 128], [120, 121, 122]], dtype=np.uint8)
    w = oracle.dequant(blocks, scales)
    for r in range(3):
        for b in range(3):
            assert np.all(w[r, 32 * b:32 * (b + 1)] == 2.0 ** (int(scales[r, b]) - 127))


# ---------------------------------------------------------------- router, top-k, softmax

def test_router_matches_numpy_matmul():
    inp = make_inputs(CONFIGS["tiny"], seed=3)
    logits, abs_sum = oracle.router(inp["x"], inp["router_w"], inp["router_b"], with_abs_sum=True)
    x = f32_from_bf16_bits(inp["x"]).astype(np.float64)
    wr = f32_from_bf16_bits(inp["router_w"]).astype(np.float64)
    br = f32_from_bf16_bits(inp["router_b"]).astype(np.float64)
    ref = x @ wr.T + br
    np.testing.assert_allclose(logits, ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(abs_sum, np.abs(x) @ np.abs(wr).T + np.abs(br), rtol=1e-13)


@pytest.mark.parametrize("E,k", [(4, 2), (8, 1), (32, 4), (128, 4), (256, 8), (5, 5)])
def test_topk_matches_stable_sort(E, k):
    rng = np.random.default_rng(E * 10 + k)
    logits = rng.standard_normal((50, E))
    logits[:, 1] = logits[:, 3] if E > 3 else logits[:, 1]      # exact ties
    idx, w = oracle.topk_softmax(logits, k)
    for t in range(logits.shape[0]):
        want = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        assert list(idx[t]) == want
        np.testing.assert_allclose(w[t], scipy.special.softmax(logits[t, want]), rtol=1e-14)
        assert abs(w[t].sum() - 1.0) < 1e-14


def test_topk_ties_go_to_lower_index():
    logits = np.array([[0.5, 1.0, 1.0, 1.0, 0.2, 1.0]])
    idx, w = oracle.topk_softmax(logits, 3)
    assert list(idx[0]) == [1, 2, 3]
    assert np.all(w == 1.0 / 3)


def test_softmax_special_cases():
    logits = np.array([[3.0, -1.0, 2.0, 0.0]])
    idx, w = oracle.topk_softmax(logits, 1)
    assert idx[0, 0] == 0 and w[0, 0] == 1.0
    idx, w = oracle.topk_softmax(np.zeros((1, 4)), 4)
    assert list(idx[0]) == [0, 1, 2, 3] and np.all(w == 0.25)
    # the k=2 weights of a logit gap d are sigmoid(d) and sigmoid(-d)
    idx, w = oracle.topk_softmax(np.array([[0.0, math.log(3.0), -5.0]]), 2)
    assert list(idx[0]) == [1, 0]
    np.testing.assert_allclose(w[0], [0.75, 0.25], rtol=1e-15)


def test_router_tie_fixture_duplicated_rows():
    cfg = CONFIGS["tiny"].with_(E=6, k=3)
    inp = make_inputs(cfg, seed=5)
    inp["router_w"][4] = inp["router_w"][1]
    inp["router_b"][4] = inp["router_b"][1]
    inp["router_w"][5] = inp["router_w"][1]
    inp["router_b"][5] = inp["router_b"][1]
    logits = oracle.router(inp["x"], inp["router_w"], inp["router_b"])
    assert np.array_equal(logits[:, 1], logits[:, 4])
    idx, _ = oracle.topk_softmax(logits, 3)
    for t in range(cfg.T):
        sel = list(idx[t])
        if 4 in sel:
            assert 1 in sel and sel.index(1) < sel.index(4)
        if 5 in sel:
            assert 4 in sel and sel.index(4) < sel.index(5)


# ---------------------------------------------------------------- SwiGLU

def test_swiglu_closed_forms():
    a, lim = 1.702, 7.0
    for up in (-3.0, 0.0, 2.5):
        assert oracle.swiglu(0.0, up) == 0.0                       # gate 0
    for gate in (-9.0, 0.3, 5.0, 12.0):
        assert oracle.swiglu(gate, -1.0) == 0.0                    # up + 1 = 0
    # sigmoid(alpha * g) = 3/4 at g = ln(3) / alpha
    g = math.log(3.0) / a
    assert oracle.swiglu(g, 1.0) == pytest.approx(2.0 * g * 0.75, rel=1e-15)
    assert oracle.swiglu(g, 0.0) == pytest.approx(g * 0.75, rel=1e-15)
    # sigmoid(z) + sigmoid(-z) = 1  =>  f(g, u) - f(-g, u) = (u + 1) g  for |g| <= limit
    for g, u in ((0.7, 0.2), (3.3, -2.0), (6.9, 6.9), (1.0, -6.5)):
        assert oracle.swiglu(g, u) - oracle.swiglu(-g, u) == pytest.approx((u + 1) * g, rel=1e-14)


def test_swiglu_clamps():
    # gate clamped above at the limit; up clamped on both sides
    assert oracle.swiglu(10.0, 10.0) == oracle.swiglu(7.0, 7.0)
    assert oracle.swiglu(7.5, 2.0) == oracle.swiglu(7.0, 2.0)
    assert oracle.swiglu(2.0, 20.0) == oracle.swiglu(2.0, 7.0)
    assert oracle.swiglu(6.5, -8.0) == oracle.swiglu(6.5, -7.0)
    # gate is NOT clamped below: -10 differs from -7
    assert oracle.swiglu(-10.0, -10.0) != oracle.swiglu(-7.0, -10.0)
    assert oracle.swiglu(-10.0, 3.0) < 0.0 and oracle.swiglu(-10.0, 3.0) > -1e-5
    # large clamped gate: sigmoid(11.914) ~ 1  =>  value just below (u + 1) * 7
    v = oracle.swiglu(7.0, 7.0)
    assert 56.0 - 1e-3 < v < 56.0


def test_swiglu_matches_high_precision():
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 40
    for g, u in ((1.0, 0.0), (-1.0, 2.0), (7.0, 7.0), (6.5, -7.0), (2.0, 7.0), (-10.0, -7.0),
                 (-10.0, 3.0), (0.123, -0.456)):
        gg, uu = min(g, 7.0), min(max(u, -7.0), 7.0)
        ref = (mpmath.mpf(uu) + 1) * gg / (1 + mpmath.exp(-mpmath.mpf("1.702") * gg))
        assert oracle.swiglu(g, u) == pytest.approx(float(ref), rel=2e-15, abs=1e-300)


# ---------------------------------------------------------------- experts and layer

def _np_layer(inp, k, alpha=1.702, limit=7.0):
    """The layer from library routines (numpy matmul, stable sort, scipy softmax)
    on the oracle's pinned dequantization and SwiGLU."""
    x = f32_from_bf16_bits(inp["x"]).astype(np.float64)
    wr = f32_from_bf16_bits(inp["router_w"]).astype(np.float64)
    br = f32_from_bf16_bits(inp["router_b"]).astype(np.float64)
    wgu = oracle.dequant(inp["gu_blocks"], inp["gu_scales"])        # [E, 2I, H]
    wdn = oracle.dequant(inp["dn_blocks"], inp["dn_scales"])        # [E, H, I]
    bgu = f32_from_bf16_bits(inp["gu_bias"]).astype(np.float64)
    bdn = f32_from_bf16_bits(inp["dn_bias"]).astype(np.float64)
    logits = x @ wr.T + br
    T, H = x.shape
    y = np.zeros((T, H))
    sw = np.vectorize(lambda g, u: oracle.swiglu(g, u, alpha, limit))
    for t in range(T):
        sel = sorted(range(wr.shape[0]), key=lambda e: (-logits[t, e], e))[:k]
        w = scipy.special.softmax(logits[t, sel])
        for j, e in enumerate(sel):
            gu = wgu[e] @ x[t] + bgu[e]
            h = sw(gu[0::2], gu[1::2])
            y[t] += w[j] * (wdn[e] @ h + bdn[e])
    return y


@pytest.mark.parametrize("H,I,E,k", [(64, 64, 4, 2), (96, 64, 5, 2), (64, 128, 4, 3)])
def test_layer_matches_library_composition(H, I, E, k):
    cfg = CONFIGS["tiny"].with_(H=H, I=I, E=E, k=k)
    inp = make_inputs(cfg, seed=11)
    out = oracle.forward(inp, k, intermediates=True)
    ref = _np_layer(inp, k)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


def _identity_experts(H, I, E):
    """Gate rows 2i carry 1.0 at column i; up rows are zero; down row d carries
    1.0 at column d (d < I). Scales 127 (x1)."""
    gu = np.zeros((E, 2 * I, H), dtype=np.uint8)     # nibble codes before packing
    for i in range(min(I, H)):
        gu[:, 2 * i, i] = 2                           # code 2 = 1.0
    dn = np.zeros((E, H, I), dtype=np.uint8)
    for d in range(min(H, I)):
        dn[:, d, d] = 2

    def pack(codes):
        return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)

    return pack(gu), pack(dn)


@pytest.mark.parametrize("H,I", [(96, 64), (64, 128)])
def test_identity_experts_non_square(H, I):
    cfg = CONFIGS["tiny"].with_(H=H, I=I, E=4, k=2)
    inp = make_inputs(cfg, seed=2)
    gu, dn = _identity_experts(H, I, 4)
    inp["gu_blocks"], inp["dn_blocks"] = gu, dn
    inp["gu_scales"][:] = 127
    inp["dn_scales"][:] = 127
    inp["gu_bias"][:] = 0
    out = oracle.forward(inp, 2, intermediates=True)
    x = f32_from_bf16_bits(inp["x"]).astype(np.float64)
    bdn = f32_from_bf16_bits(inp["dn_bias"]).astype(np.float64)
    for t in range(cfg.T):
        for j in range(2):
            e = out["idx"][t, j]
            h_want = np.zeros(I)
            for i in range(min(I, H)):
                h_want[i] = oracle.swiglu(x[t, i], 0.0)
            assert np.array_equal(out["h"][t, j], h_want)
            o_want = bdn[e].copy()
            o_want[:min(H, I)] += h_want[:min(H, I)]
            assert np.array_equal(out["o"][t, j], o_want)


def test_interleave_fixture_zero_up_rows():
    """Up rows (odd rows of gate_up) all code 0 and up bias -1  =>  h = 0, so
    y = sum_j w_j * b_dn[e_j] exactly. Reading the gate/up halves the other way
    round (or as contiguous halves) gives a different y."""
    cfg = CONFIGS["tiny"].with_(H=64, I=96, E=4, k=2)
    inp = make_inputs(cfg, seed=9)
    inp["gu_blocks"].reshape(4, 2 * 96, 32)[:, 1::2, :] = 0
    minus_one = bf16_bits_from_f32(np.array([-1.0], dtype=np.float32))[0]
    inp["gu_bias"][:, 1::2] = minus_one
    out = oracle.forward(inp, 2, intermediates=True)
    assert np.all(out["h"] == 0.0)
    bdn = f32_from_bf16_bits(inp["dn_bias"]).astype(np.float64)
    for t in range(cfg.T):
        want = np.zeros(64)
        for j in range(2):
            want = want + out["w"][t, j] * bdn[out["idx"][t, j]]
        assert np.array_equal(out["y"][t], want)


def test_only_routed_experts_matter():
    cfg = CONFIGS["tiny"].with_(E=6, k=2, T=4)
    inp = make_inputs(cfg, seed=4)
    base = oracle.forward(inp, 2)
    used = set(base["idx"].ravel().tolist())
    unused = [e for e in range(6) if e not in used]
    assert unused
    rng = np.random.default_rng(0)
    for e in unused:
        inp["gu_blocks"][e] = rng.integers(0, 256, inp["gu_blocks"][e].shape, dtype=np.uint8)
        inp["dn_blocks"][e] = rng.integers(0, 256, inp["dn_blocks"][e].shape, dtype=np.uint8)
        inp["dn_scales"][e] = 127
        inp["gu_bias"][e] = 0x3F80
    again = oracle.forward(inp, 2)
    assert np.array_equal(base["y"], again["y"])


def test_down_scale_doubling_doubles_output():
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg, seed=8)
    base = oracle.forward(inp, cfg.k)
    inp["dn_scales"] = inp["dn_scales"] + 1
    b = f32_from_bf16_bits(inp["dn_bias"]) * np.float32(2.0)
    inp["dn_bias"] = bf16_bits_from_f32(b)
    twice = oracle.forward(inp, cfg.k)
    assert np.array_equal(twice["y"], 2.0 * base["y"])


def test_token_subset_is_independent():
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg, seed=1)
    full = oracle.forward(inp, cfg.k)
    part = oracle.forward(inp, cfg.k, tokens=[5, 2])
    assert np.array_equal(part["y"], full["y"][[5, 2]])
    assert np.array_equal(part["idx"], full["idx"][[5, 2]])


# --------------------------------------------------------------------------- Pre-LN RMSNorm
# MLX README "Architecture Details" (RMSNorm, Pre-LN placement) and ZM "API" (norm_eps 1e-5):
# xn = bf16(x / sqrt(mean(x^2) + eps) * gamma), block output y = x + layer(xn).

def _bf16_nearest_exact(v: float) -> int:
    """Round a double to bf16 by exact rational arithmetic (ties to even): the bit pattern."""
    from fractions import Fraction
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    fv = Fraction(v)
    m, e = math.frexp(abs(v))          # |v| = m 2^e, 0.5 <= m < 1
    ulp = Fraction(2) ** (e - 8)
    lo = (abs(fv) // ulp) * ulp
    hi = lo + ulp
    dlo, dhi = abs(fv) - lo, hi - abs(fv)
    if dlo < dhi:
        r = lo
    elif dhi < dlo:
        r = hi
    else:                               # tie: the one with an even last kept bit
        r = lo if (lo / ulp) % 2 == 0 else hi
    f = np.float32(float(r) if v > 0 else -float(r))
    return int(f.view(np.uint32) >> 16)


def test_bf16_rounding_ties_to_even():
    cases = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 1.0 + 2.0 ** -8 + 2.0 ** -30,
             3.0, -0.0, 0.0, 1e-3, 123.456, -7.0 + 2.0 ** -6]
    for v in cases:
        assert oracle.bf16_round(v) == _bf16_nearest_exact(v), v
    assert oracle.bf16_round(1.0 + 2.0 ** -8) == 0x3F80          # tie -> even (down)
    assert oracle.bf16_round(1.0 + 3 * 2.0 ** -8) == 0x3F82      # tie -> even (up)
    rng = np.random.default_rng(7)
    for v in rng.standard_normal(300) * 10.0 ** rng.integers(-3, 4, 300):
        assert oracle.bf16_round(float(v)) == _bf16_nearest_exact(float(v))


def test_rmsnorm_closed_form_constant_rows():
    H = 96
    gamma = np.full(H, 0x3F80, dtype=np.uint16)                   # 1.0
    for c in (0.5, 1.0, 3.0, -2.25):
        x = np.full((1, H), bf16_bits_from_f32(np.float32(c)), dtype=np.uint16)
        for eps in (0.0, 1e-5, 0.25):
            xn, ex = oracle.rmsnorm(x, gamma, eps, with_exact=True)
            ref = c / math.sqrt(c * c + eps)
            np.testing.assert_allclose(ex, ref, rtol=2e-16, atol=0)
            assert (xn == _bf16_nearest_exact(ref)).all()
            if eps == 0.0:
                assert (xn == (0x3F80 if c > 0 else 0xBF80)).all()   # exactly +-1


def test_rmsnorm_matches_numpy_and_exact_rounding():
    cfg = CONFIGS["tiny"].with_(H=96)
    inp = make_inputs(cfg, seed=11, T=5, parts=("x", "norm_w"))
    x = f32_from_bf16_bits(inp["x"]).astype(np.float64)
    g = f32_from_bf16_bits(inp["norm_w"]).astype(np.float64)
    xn, ex = oracle.rmsnorm(inp["x"], inp["norm_w"], 1e-5, with_exact=True)
    ref = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-5) * g
    np.testing.assert_allclose(ex, ref, rtol=1e-14, atol=0)
    for t in range(5):
        for h in range(0, 96, 7):
            assert xn[t, h] == _bf16_nearest_exact(float(ex[t, h]))


def test_rmsnorm_scale_invariance_without_eps():
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg, seed=12, T=4, parts=("x", "norm_w"))
    xf = f32_from_bf16_bits(inp["x"])
    for j in (-3, 2, 5):
        xs = bf16_bits_from_f32(xf * np.float32(2.0 ** j))        # exact: a power of two
        assert (oracle.rmsnorm(xs, inp["norm_w"], 0.0) == oracle.rmsnorm(inp["x"], inp["norm_w"], 0.0)).all()


def test_prenorm_block_is_residual_plus_layer_of_normalized_rows():
    cfg = CONFIGS["tiny"]
    inp = make_inputs(cfg, seed=13)
    out = oracle.forward_prenorm(inp, cfg.k, eps=1e-5)
    xn = oracle.rmsnorm(inp["x"], inp["norm_w"], 1e-5)
    plain = oracle.forward(dict(inp, x=xn), cfg.k)
    np.testing.assert_array_equal(out["idx"], plain["idx"])
    np.testing.assert_allclose(out["y"] - f32_from_bf16_bits(inp["x"]), plain["y"], rtol=0, atol=1e-12)
    # gamma = 0 normalizes every row to zero: the layer then sees only its biases
    zero = oracle.forward_prenorm(dict(inp, norm_w=np.zeros_like(inp["norm_w"])), cfg.k)
    assert (f32_from_bf16_bits(zero["xn"]) == 0.0).all()          # (+-0: the sign of x survives)


# ---------------------------------------------------------------- expert-major mode

def _modes_agree(inp, k, tokens=None, alpha=1.702, limit=7.0, rel=1e-12):
    a = oracle.forward(inp, k, tokens=tokens, alpha=alpha, limit=limit, intermediates=True)
    b = oracle.forward_expert_major(inp, k, tokens=tokens, alpha=alpha, limit=limit, intermediates=True)
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_array_equal(a["w"], b["w"])
    np.testing.assert_array_equal(a["logits"], b["logits"])
    for key in ("h", "o", "y"):
        d = np.linalg.norm((a[key] - b[key]).reshape(a[key].shape[0], -1), axis=1)
        n = np.linalg.norm(a[key].reshape(a[key].shape[0], -1), axis=1)
        assert np.all(d <= rel * n), (key, float((d / n).max()))
    return a, b


@pytest.mark.parametrize("H,I,E,k,T", [(64, 64, 4, 2, 8), (96, 64, 5, 2, 40), (64, 128, 3, 3, 17),
                                       (64, 64, 1, 1, 6), (64, 96, 256, 8, 11)])
def test_expert_major_equals_brute_mode_small(H, I, E, k, T):
    """The two oracle modes compute the same definitions: identical routing, and h, o, y
    equal to double rounding (only the order inside the dot products differs); non-square
    shapes, one expert with k = 1, k = E and the largest E and k."""
    cfg = CONFIGS["tiny"].with_(H=H, I=I, E=E, k=k)
    _modes_agree(make_inputs(cfg, seed=11, T=T), k)


def test_expert_major_equals_brute_mode_decode_shapes():
    """The 20B-shaped decode (T = 1) and a token subset of the skewed batched decode, where
    several tokens share experts and an expert's tokens come from different slots."""
    cfg = CONFIGS["decode_20b"]
    _modes_agree(make_inputs(cfg, seed=1), cfg.k, rel=1e-6)
    cfg = CONFIGS["batched_decode_20b"]
    a, _ = _modes_agree(make_inputs(cfg, seed=1), cfg.k, tokens=[0, 5, 9, 17, 33, 63], rel=1e-6)
    assert len(np.unique(a["idx"])) < a["idx"].size     # experts shared between tokens


def test_expert_major_interleave_fixture():
    """Zero up rows with up bias -1: every h is 0, so y = sum_j w_j b_dn[e_j] in this mode too."""
    cfg = CONFIGS["tiny"].with_(H=64, I=96, E=4, k=2)
    inp = make_inputs(cfg, seed=9, T=12)
    inp["gu_blocks"].reshape(4, 2 * 96, 32)[:, 1::2, :] = 0
    inp["gu_bias"][:, 1::2] = bf16_bits_from_f32(np.array([-1.0], dtype=np.float32))[0]
    out = oracle.forward_expert_major(inp, cfg.k, intermediates=True)
    assert np.all(out["h"] == 0.0)
    b_dn = f32_from_bf16_bits(inp["dn_bias"]).astype(np.float64)
    want = np.zeros((12, 64))
    for j in range(cfg.k):
        want += out["w"][:, j:j + 1] * b_dn[out["idx"][:, j]]
    np.testing.assert_allclose(out["y"], want, rtol=1e-15, atol=0)


def test_swiglu_n_matches_scalar():
    rng = np.random.default_rng(4)
    g = rng.standard_normal(1000) * 10
    u = rng.standard_normal(1000) * 10
    h = oracle.swiglu_n(g, u)
    assert np.array_equal(h, np.array([oracle.swiglu(a, b) for a, b in zip(g, u)]))
