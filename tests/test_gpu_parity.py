"""GPU parity: every step of the HIP path against the CPU oracle, through the C ABI.

Bars: dequantized weights, top-k indices and the permutation bit-exact; routing
weights within 1e-6 relative; h, o and y within per-token relative L2 1e-2 and
per-element 5e-2 * rms (see gpu_util). Inputs are the seeded workloads (tiny, the
GPT-OSS-20B decode / batched decode / 4k prefill shapes and the 120B-shaped prefill)
plus fixtures: non-square H != I, duplicated router rows (ties), zero up rows
(gate/up interleave), maximal E and k, and ragged token counts on both sides of the
decode/prefill switch. Full-size configs run in the same launch configuration as the
benchmark and are compared on every token (the 4096-token and 120B-shaped workloads against
the oracle's expert-major mode).
"""
import ctypes

import numpy as np
import pytest
import torch

import mxfp4_mixture_experts_router_amd as moe
import oracle
from workloads import CONFIGS, make_inputs, f32_from_bf16_bits, bf16_bits_from_f32

from gpu_util import (assert_close_rows, bf16_bits, bf16_to_f64, check_selection, decode_h8, decode_mx8, dev,
                      host_permutation, to_dev, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import os
    if not os.path.exists(moe.library_path()):
        from mxfp4_mixture_experts_router_amd import build
        build.build()
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    moe.load_library()
    yield
    torch.cuda.synchronize()


def _reference(inp, cfg, tokens, **kw):
    """The oracle's layer for ``tokens``: the brute mode up to the work of 64 tokens of the
    GPT-OSS shape, the expert-major mode (pinned to it on CPU) beyond, so that the full-size
    workloads are compared on every token."""
    big = len(tokens) * cfg.H * cfg.I > 64 * 2880 * 2880
    fn = oracle.forward_expert_major if big else oracle.forward
    return fn(inp, cfg.k, tokens=tokens, alpha=cfg.alpha, limit=cfg.limit, **kw)


def _sample(T, n, seed=0):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, n - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s))


def _forward(inp_d, k, cfg, **kw):
    return moe.moe_forward(inp_d["x"], inp_d["router_w"], inp_d["router_b"], inp_d["gu_blocks"],
                           inp_d["gu_scales"], inp_d["gu_bias"], inp_d["dn_blocks"],
                           inp_d["dn_scales"], inp_d["dn_bias"], k, cfg.alpha, cfg.limit, **kw)


# ----------------------------------------------------------------------------- dequant

def _oracle_bf16_bits(blocks, scales):
    ref = oracle.dequant(blocks, scales).astype(np.float32)
    bits = bf16_bits_from_f32(ref)
    assert np.array_equal(f32_from_bf16_bits(bits), ref)     # exact in bf16
    return bits


def test_dequant_every_byte_and_scale():
    scales_range = np.arange(2, 253, dtype=np.uint8)            # supported scale bytes
    rows = scales_range.size
    blocks = np.tile(np.arange(256, dtype=np.uint8), (rows, 1))   # every byte, every row
    scales = np.repeat(scales_range[:, None], 512 // 32, axis=1)
    want = _oracle_bf16_bits(blocks, scales)
    got = bf16_bits(moe.dequant(to_dev(blocks), to_dev(scales)))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("name", ["tiny", "decode_20b"])
def test_dequant_expert_banks(name):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, parts=("gu_blocks", "gu_scales", "dn_blocks", "dn_scales"))
    e = cfg.E - 1
    for b, s in (("gu_blocks", "gu_scales"), ("dn_blocks", "dn_scales")):
        want = _oracle_bf16_bits(inp[b][e], inp[s][e])
        got = bf16_bits(moe.dequant(to_dev(inp[b][e]), to_dev(inp[s][e])))
        np.testing.assert_array_equal(got, want)
    # a whole bank in one call (rows = E * R)
    want = _oracle_bf16_bits(inp["dn_blocks"][:2], inp["dn_scales"][:2])
    got = bf16_bits(moe.dequant(to_dev(inp["dn_blocks"][:2]), to_dev(inp["dn_scales"][:2])))
    np.testing.assert_array_equal(got, want)


# ----------------------------------------------------------------------------- route

def _check_route(cfg, inp):
    ref_logits, abs_sum = oracle.router(inp["x"], inp["router_w"], inp["router_b"], with_abs_sum=True)
    ref_idx, ref_w = oracle.topk_softmax(ref_logits, cfg.k)
    ref = {"logits": ref_logits, "abs_sum": abs_sum, "idx": ref_idx, "w": ref_w}
    d = upload(inp)
    idx, w, logits = moe.route(d["x"], d["router_w"], d["router_b"], cfg.k, return_logits=True)
    idx, w, logits = idx.cpu().numpy(), w.cpu().numpy(), logits.cpu().numpy()
    ok = check_selection(idx, ref, cfg.H, cfg.k)
    np.testing.assert_allclose(w[ok], ref_w[ok], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
    err = np.abs(logits.astype(np.float64) - ref_logits)
    assert np.all(err <= 2.0 ** -23 * np.abs(ref_logits) + 1e-10 * abs_sum)
    return idx, ok


@pytest.mark.parametrize("name", ["tiny", "decode_20b", "batched_decode_20b", "prefill_20b",
                                  "prefill_120b"])
def test_route_matches_oracle(name):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, parts=("x", "router_w", "router_b"))
    _, ok = _check_route(cfg, inp)
    assert ok.mean() > 0.99


@pytest.mark.parametrize("T", [1, 16, 17, 300])
def test_route_ties_go_to_lower_index(T):
    cfg = CONFIGS["tiny"].with_(E=8, k=3, H=96)
    inp = make_inputs(cfg, seed=5, T=T, parts=("x", "router_w", "router_b"))
    for dup in (5, 6, 7):
        inp["router_w"][dup] = inp["router_w"][2]
        inp["router_b"][dup] = inp["router_b"][2]
    idx, _ = _check_route(cfg, inp)
    d = upload(inp)
    _, _, logits = moe.route(d["x"], d["router_w"], d["router_b"], cfg.k, return_logits=True)
    lg = logits.cpu().numpy()
    assert np.array_equal(lg[:, 2], lg[:, 5]) and np.array_equal(lg[:, 2], lg[:, 7])
    for t in range(T):
        sel = list(idx[t])
        for hi in (5, 6, 7):
            if hi in sel:
                assert 2 in sel and sel.index(2) < sel.index(hi)


def test_route_max_experts_and_k():
    cfg = CONFIGS["tiny"].with_(E=256, k=8, H=64)
    inp = make_inputs(cfg, seed=3, T=40, parts=("x", "router_w", "router_b"))
    _check_route(cfg, inp)


# ----------------------------------------------------------------------------- permute

def _random_routing(T, E, k, seed, skew=0.0):
    """k distinct experts per token, drawn without replacement with skewed probabilities
    (Gumbel top-k of log p: the same distribution as sequential draws without replacement)."""
    rng = np.random.default_rng(seed)
    logp = skew * rng.standard_normal(E)
    keys = logp[None, :] + rng.gumbel(size=(T, E))
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    return idx, w


PERMUTE_CASES = [(1, 32, 4, 0.0), (64, 32, 4, 2.0), (4096, 32, 4, 0.0), (2048, 128, 4, 1.0),
                 (333, 256, 8, 3.0), (1025, 4, 4, 0.0), (500, 16, 1, 5.0), (4097, 32, 4, 0.0),
                 (5000, 64, 4, 1.0),
                 (32, 256, 8, 0.0),        # 256 pairs: one block of the many-workgroup permute
                 (4100, 32, 4, 0.0),       # 65 blocks: the first with the scan pass
                 (20000, 256, 8, 2.0),     # 625 blocks, E = 256, k = 8
                 (65536, 32, 4, 1.0),      # 1024 blocks, a whole scan chunk
                 (65537, 32, 4, 1.0),      # 1025 blocks: a second scan chunk of one entry
                 (300000, 128, 4, 2.0),    # 4688 blocks: five scan chunks, the last ragged
                 (70000, 1, 1, 0.0),       # one expert: every pair keeps its place
                 (9000, 3, 2, 1.0)]        # 71 blocks, an odd expert count


@pytest.mark.parametrize("multi_block", [False, True], ids=["one_workgroup", "multi_block"])
@pytest.mark.parametrize("T,E,k,skew", PERMUTE_CASES)
def test_permute_is_a_stable_sort(T, E, k, skew, multi_block):
    # one workgroup: T k = 16384 pairs and fewer are sorted in LDS, more take the direct path;
    # multi_block: the histogram (+ scan above 64 blocks) + scatter kernels every forward of
    # the grouped sequence runs
    idx, w = _random_routing(T, E, k, seed=T + E, skew=skew)
    offsets, sorted_token, order, slot_row = host_permutation(idx, E)
    g_off, g_tok, g_w, g_slot = moe.permute(to_dev(idx), to_dev(w), E, multi_block=multi_block)
    np.testing.assert_array_equal(g_off.cpu().numpy(), offsets)
    np.testing.assert_array_equal(g_tok.cpu().numpy(), sorted_token)
    np.testing.assert_array_equal(g_w.cpu().numpy(), w.reshape(-1)[order])
    np.testing.assert_array_equal(g_slot.cpu().numpy(), slot_row)


# ----------------------------------------------------------------------------- grouped experts

def _grouped_case(cfg, T, seed):
    inp = make_inputs(cfg, seed=seed, T=T)
    tokens = np.arange(T)
    ref = _reference(inp, cfg, tokens, intermediates=True)
    return inp, tokens, ref, ref["idx"], ref["w"]


@pytest.mark.parametrize("name,T,H,I,E,k", [
    ("tiny", 8, 64, 64, 4, 2), ("tiny", 200, 96, 64, 5, 2), ("tiny", 333, 64, 128, 3, 2),
    ("prefill_20b", 4096, 2880, 2880, 32, 4), ("prefill_120b", 2048, 2880, 2880, 128, 4)])
def test_expert_up_and_down_grouped(name, T, H, I, E, k):
    """Every row of h and o, and every token of y, against the oracle."""
    cfg = CONFIGS[name].with_(H=H, I=I, E=E, k=k)
    inp, tokens, ref, idx, w = _grouped_case(cfg, T, seed=7)
    offsets, sorted_token, order, slot_row = host_permutation(idx, E)
    d = upload(inp)
    x8 = moe.quantize_act(d["x"])
    h8 = moe.expert_up(x8, T, d["gu_blocks"], d["gu_scales"], d["gu_bias"], to_dev(offsets),
                       to_dev(sorted_token), k, cfg.alpha, cfg.limit)
    rows = slot_row.reshape(T, k)[tokens]                      # [n, k] sorted rows of the sample
    h_np = decode_h8(h8, T * k, I)
    assert_close_rows(h_np[rows.reshape(-1)], ref["h"].reshape(-1, I), "h")
    # down: feed the oracle's h (rounded to bf16, then to h8 on the GPU) so this step is
    # checked on its own
    h_in = np.zeros((T * k, I), dtype=np.uint16)
    h_in[rows.reshape(-1)] = bf16_bits_from_f32(ref["h"].reshape(-1, I).astype(np.float32))
    sorted_w = w.reshape(-1)[order].astype(np.float32)
    o = moe.expert_down(moe.quantize_h(to_dev(h_in)), T, d["dn_blocks"], d["dn_scales"], d["dn_bias"],
                        to_dev(offsets), to_dev(sorted_w), k)
    o_np = o.cpu().numpy().astype(np.float64)[rows.reshape(-1)]
    want = (ref["o"] * ref["w"][:, :, None]).reshape(-1, H)
    assert_close_rows(o_np, want, "o")
    # combine of the GPU's o: the sampled tokens' y against the oracle
    y = bf16_to_f64(moe.combine(o, to_dev(slot_row), k))
    assert_close_rows(y[tokens], ref["y"], "y from combine")


@pytest.mark.parametrize("R,K", [(1, 32), (37, 96), (300, 2880)])
def test_quantize_act_is_exact_for_bf16(R, K):
    """hi + lo reproduces every bf16 value whose block's largest magnitude is within 2^13 of
    it; the rest (far below the block maximum) keep their error under 2^-21 of that maximum."""
    rng = np.random.default_rng(R * 1000 + K)
    x = (rng.standard_normal((R, K // 32, 32)) * np.exp2(rng.integers(-20, 20, size=(R, K // 32, 1)))).reshape(R, K)
    x[0, :32] = 0.0                                            # an all-zero block
    if K >= 64:
        x[0, 32:64] *= np.exp2(rng.integers(-24, 1, size=32))  # a wide dynamic range
    bits = bf16_bits_from_f32(x.astype(np.float32))
    xv = f32_from_bf16_bits(bits).astype(np.float64)
    q8 = moe.quantize_act(to_dev(bits))
    got = decode_mx8(q8, R, K)
    bmax = np.abs(xv.reshape(R, K // 32, 32)).max(axis=2, keepdims=True)
    bmax = np.repeat(bmax, 32, axis=2).reshape(R, K)
    near = np.abs(xv) >= bmax * 2.0 ** -13
    assert np.array_equal(got[near], xv[near])
    assert np.all(np.abs(got - xv) <= bmax * 2.0 ** -21)


@pytest.mark.parametrize("R,K", [(1, 32), (37, 96), (300, 2880), (129, 160), (5, 1056)])
def test_quantize_h_is_mx8_with_group_major_scales(R, K):
    """The h8 matrix holds the same data rows as the mx8 one, and byte b % 16 of word r of
    scale group b // 16 is the mx8 hi scale of row r's block b (every lo scale is hi - 4)."""
    rng = np.random.default_rng(R + K)
    x = (rng.standard_normal((R, K // 32, 32)) * np.exp2(rng.integers(-30, 30, size=(R, K // 32, 1)))).reshape(R, K)
    bits = to_dev(bf16_bits_from_f32(x.astype(np.float32)))
    q8 = moe.quantize_act(bits).cpu().numpy()
    h8 = moe.quantize_h(bits).cpu().numpy()
    nb, G, S = K // 32, (K + 511) // 512, (K // 32 + 15) // 16 * 16
    assert np.array_equal(h8[: 2 * R * K], q8[: 2 * R * K])
    sc = q8[2 * R * K: 2 * R * K + 2 * R * S].reshape(2 * R, S)[:, :nb].astype(np.int64)
    assert np.array_equal(sc[1::2], sc[0::2] - 4)
    grp = h8[2 * R * K: 2 * R * K + 16 * R * G].reshape(G, R, 16).transpose(1, 0, 2).reshape(R, 16 * G)[:, :nb]
    assert np.array_equal(grp, sc[0::2])
    assert np.array_equal(decode_h8(h8, R, K), decode_mx8(q8, R, K))


# ----------------------------------------------------------------------------- whole layer

FORWARD_CASES = [
    # (config, T override, H, I, E, k, tokens compared)
    ("tiny", None, None, None, None, None, 64),
    ("tiny", 1, 96, 64, 5, 2, 64),          # non-square, decode path
    ("tiny", 64, 64, 128, 4, 3, 64),        # non-square, largest decode batch
    ("tiny", 65, 96, 64, 5, 2, 65),         # non-square, smallest prefill batch
    ("tiny", 300, 64, 128, 3, 2, 300),      # few experts: several ragged m-tiles each
    ("tiny", 17, 64, 64, 256, 8, 17),       # maximal E and k, decode path
    ("tiny", 5, 96, 64, 5, 2, 5),           # non-square, batched decode: a partly filled 64-row tile
    ("tiny", 140, 64, 64, 256, 8, 140),     # maximal E and k, prefill path
    ("tiny", 2, 64, 64, 1, 1, 2),           # one expert, k = 1 (weight 1), few-token path
    ("tiny", 9, 64, 64, 1, 1, 9),           # one expert, batched decode path
    # batched decode with runs of several weight tiles per pair group (127 tiles in runs of 2,
    # the last run one tile; 125 tiles in runs of 3, the last run two)
    ("tiny", 64, 64, 4064, 1, 1, 64),
    ("tiny", 48, 64, 4000, 2, 2, 48),
    ("tiny", 70, 64, 64, 1, 1, 70),         # one expert, prefill path
    ("tiny", 9, 64, 64, 3, 3, 9),           # k = E: every expert routed
    ("tiny", 70, 96, 64, 3, 3, 70),         # k = E, prefill path
    ("tiny", 3, 4128, 64, 4, 2, 3),         # H > 4096 at few tokens: the grouped sequence
    ("tiny", 17, 4128, 64, 4, 2, 17),
    ("tiny", 3, 64, 4128, 4, 2, 3),         # I > 4096 at few tokens: the grouped sequence
    ("tiny", 17, 64, 4128, 4, 2, 17),
    # the router over slices of H (few 16-token groups, E >= 64): 4 slices (the last one empty
    # at H = 96), 2 slices
    ("tiny", 300, 256, 64, 64, 4, 300),
    ("tiny", 1100, 96, 64, 128, 4, 1100),
    ("tiny", 2100, 128, 64, 64, 2, 2100),
    # more than 64 blocks of 256 routed pairs: the permutation's scan pass
    ("tiny", 9000, 64, 64, 4, 2, 9000),
    ("tiny", 4500, 64, 96, 128, 4, 4500),
    ("tiny", 1, 3104, 64, 4, 2, 1),         # T = 1 at widths past 3072
    ("tiny", 1, 64, 3072, 4, 4, 1),
    ("tiny", 1, 64, 3104, 2, 2, 1),
    ("decode_20b", None, None, None, None, None, 1),
    ("decode_20b", 2, None, None, None, None, 2),
    ("batched_decode_20b", None, None, None, None, None, 64),
    ("prefill_20b", None, None, None, None, None, 4096),
    ("prefill_120b", None, None, None, None, None, 2048),
    # one GPU's shard of the 20B layer on eight GPUs (tensor-parallel decode, expert-parallel prefill)
    ("decode_20b_tp8", None, None, None, None, None, 1),
    ("batched_decode_20b_tp8", None, None, None, None, None, 64),
    ("prefill_20b_ep8", None, None, None, None, None, 2048),
]


@pytest.mark.parametrize("name,T,H,I,E,k,n_cmp", FORWARD_CASES)
def test_forward_matches_oracle(name, T, H, I, E, k, n_cmp):
    cfg = CONFIGS[name]
    over = {key: v for key, v in dict(H=H, I=I, E=E, k=k).items() if v is not None}
    cfg = cfg.with_(**over)
    T = cfg.T if T is None else T
    inp = make_inputs(cfg, seed=1, T=T)
    tokens = _sample(T, n_cmp, seed=T)
    ref = _reference(inp, cfg, tokens)
    d = upload(inp)
    y, idx, w = _forward(d, cfg.k, cfg, return_topk=True)
    y_np = bf16_to_f64(y)[tokens]
    idx_np = idx.cpu().numpy()[tokens]
    ok = check_selection(idx_np, ref, cfg.H, cfg.k)
    np.testing.assert_allclose(w.cpu().numpy()[tokens][ok], ref["w"][ok], rtol=1e-6, atol=1e-7)
    assert_close_rows(y_np[ok], ref["y"][ok], f"y ({name}, T={T})")
    # determinism: a second call is bit-identical
    y2 = _forward(d, cfg.k, cfg)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("T", [3, 100])
def test_forward_interleave_fixture(T):
    """Up rows all zero and up bias -1: every h is 0, so y = sum_j w_j * b_dn[e_j]."""
    cfg = CONFIGS["tiny"].with_(H=64, I=96, E=4, k=2)
    inp = make_inputs(cfg, seed=9, T=T)
    inp["gu_blocks"].reshape(4, 2 * 96, 32)[:, 1::2, :] = 0
    inp["gu_bias"][:, 1::2] = bf16_bits_from_f32(np.array([-1.0], dtype=np.float32))[0]
    ref = oracle.forward(inp, cfg.k)
    y = bf16_to_f64(_forward(upload(inp), cfg.k, cfg))
    assert_close_rows(y, ref["y"], "interleave fixture")


@pytest.mark.parametrize("T", [1, 64, 65, 1000])
def test_forward_tie_fixture(T):
    cfg = CONFIGS["tiny"].with_(E=8, k=3, H=64, I=64)
    inp = make_inputs(cfg, seed=21, T=T)
    for dup in (3, 6):
        inp["router_w"][dup] = inp["router_w"][1]
        inp["router_b"][dup] = inp["router_b"][1]
    tokens = _sample(T, 64, seed=1)
    ref = oracle.forward(inp, cfg.k, tokens=tokens)
    y, idx, _ = _forward(upload(inp), cfg.k, cfg, return_topk=True)
    np.testing.assert_array_equal(idx.cpu().numpy()[tokens], ref["idx"])
    assert_close_rows(bf16_to_f64(y)[tokens], ref["y"], "tie fixture")


class _HipEvents:
    """hipEvent_t handles from the HIP runtime this process already loaded."""

    def __init__(self):
        import ctypes
        import re
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                m = re.search(r"(/\S*libamdhip64\.so\S*)", line)
                if m:
                    path = m.group(1)
                    break
        self.c = ctypes
        self.lib = ctypes.CDLL(path or "libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            ev = self.c.c_void_p()
            assert self.lib.hipEventCreate(self.c.byref(ev)) == 0
            evs.append(ev.value)
        return evs

    def elapsed_ms(self, a, b):
        ms = self.c.c_float()
        assert self.lib.hipEventElapsedTime(self.c.byref(ms), self.c.c_void_p(a), self.c.c_void_p(b)) == 0
        return ms.value

    def destroy(self, evs):
        for ev in evs:
            self.lib.hipEventDestroy(self.c.c_void_p(ev))


@pytest.mark.parametrize("T,launches,prenorm,H,I,E", [
    (1, 3, False, 64, 64, 4), (3, 3, False, 64, 64, 4), (4, 4, False, 64, 64, 4), (17, 4, False, 64, 64, 4),
    (65, 5, False, 64, 64, 4), (1, 3, True, 64, 64, 4), (17, 4, True, 64, 64, 4), (65, 6, True, 64, 64, 4),
    # H or I above 4096: the grouped sequence at any token count
    (3, 5, False, 4128, 64, 4), (17, 5, False, 64, 4128, 4), (3, 6, True, 4128, 64, 4), (17, 6, True, 64, 4128, 4),
    # the router in two kernels (slices of H, then the top-k): still one stage
    (300, 5, False, 128, 64, 64), (300, 6, True, 128, 64, 64),
    # the permute in three kernels (histogram, scan, scatter): still one stage
    (9000, 5, False, 64, 64, 4)])
def test_forward_timed_matches_forward(T, launches, prenorm, H, I, E):
    import ctypes
    cfg = CONFIGS["tiny"].with_(H=H, I=I, E=E)
    inp = upload(make_inputs(cfg, seed=5, T=T))
    norm = dict(norm_weight=inp["norm_w"], norm_eps=1e-5) if prenorm else {}
    y_ref = _forward(inp, cfg.k, cfg, **norm)
    H, I, E = cfg.H, cfg.I, cfg.E
    shape = moe._shape(T, H, I, E, cfg.k, cfg.alpha, cfg.limit)
    ws = torch.empty(max(moe.workspace_bytes(T, H, I, E, cfg.k), 256), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(y_ref)
    hip = _HipEvents()
    evs = hip.create(2 * moe.MAX_LAUNCHES)
    arr = (ctypes.c_void_p * len(evs))(*evs)
    n = ctypes.c_int(-1)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    lib = moe.load_library()
    tail = (P(inp["router_w"]), P(inp["router_b"]), P(inp["gu_blocks"]), P(inp["gu_scales"]), P(inp["gu_bias"]),
            P(inp["dn_blocks"]), P(inp["dn_scales"]), P(inp["dn_bias"]), P(y), None, None, P(ws), ws.numel(),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), arr, len(evs), ctypes.byref(n))
    if prenorm:
        st = lib.moe_mxfp4_forward_prenorm_timed(ctypes.byref(shape), P(inp["x"]), P(inp["norm_w"]), 1e-5, *tail)
    else:
        st = lib.moe_mxfp4_forward_timed(ctypes.byref(shape), P(inp["x"]), *tail)
    assert st == 0, moe.load_library().moe_mxfp4_last_error()
    torch.cuda.synchronize()
    assert n.value == launches
    # each kernel's own start / end events: positive durations, in launch order
    for i in range(n.value):
        assert hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) > 0
        if i:
            assert hip.elapsed_ms(evs[2 * i - 1], evs[2 * i]) >= 0
    hip.destroy(evs)
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))


def test_forward_zero_tokens():
    cfg = CONFIGS["tiny"]
    inp = upload(make_inputs(cfg, T=0))
    y = _forward(inp, cfg.k, cfg)
    assert y.shape == (0, cfg.H)


# ----------------------------------------------------------------------------- pre-norm block

def _rms_rows(R, C, seed):
    """bf16 rows of mixed scale: N(0, 1) rows, rows scaled by 2^-20 and 2^20, a constant row
    and a row of zeros (eps keeps it finite: every output is zero)."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((R, C)).astype(np.float32)
    if R >= 5:
        v[1] *= 2.0 ** -20
        v[2] *= 2.0 ** 20
        v[3] = 0.75
        v[4] = 0.0
    g = (1.0 + 0.1 * rng.standard_normal(C)).astype(np.float32)
    return bf16_bits_from_f32(v), bf16_bits_from_f32(g)


def _near_bf16_tie(exact: np.ndarray) -> np.ndarray:
    """Where a value lies within 2^-40 relative of a midpoint between two bf16 numbers: only
    there may a different (correct to the last bits of a double) sum of squares change the
    rounding."""
    m, e = np.frexp(exact)
    frac = np.abs(np.ldexp(m, 8)) % 1.0
    return np.abs(frac - 0.5) < 2.0 ** -40 * 256


@pytest.mark.parametrize("R,C,eps", [(1, 2880, 1e-5), (37, 96, 1e-5), (300, 2880, 1e-5), (6, 8, 1e-5),
                                     (5, 4104, 1e-5), (9, 2880, 0.0), (5, 2880, 1e-2)])
def test_rmsnorm_matches_oracle(R, C, eps):
    x, g = _rms_rows(R, C, seed=R + C)
    if eps == 0.0:
        x[4] = x[0]                       # no zero row without eps
    want, exact = oracle.rmsnorm(x, g, eps, with_exact=True)
    got = bf16_bits(moe.rmsnorm(to_dev(x), to_dev(g), eps))
    bad = got != want
    assert not np.any(bad & ~_near_bf16_tie(exact)), np.argwhere(bad)[:8]
    assert bad.sum() <= 2


PRENORM_CASES = [
    # (config, T override, H, I, E, k, tokens compared); the residual is added by the last
    # kernel of each launch sequence: the down-projection (T < 4), the slot combine (4..64),
    # the prefill combine (> 64)
    ("tiny", None, None, None, None, None, 64),
    ("tiny", 1, 96, 64, 5, 2, 1),
    ("tiny", 3, 96, 64, 5, 2, 3),
    ("tiny", 5, 96, 64, 5, 2, 5),
    ("tiny", 65, 96, 64, 5, 2, 65),
    ("tiny", 5, 3616, 64, 4, 2, 5),         # H > 3584 from 4 tokens: the RMSNorm kernel of its own
    ("tiny", 3, 4128, 64, 4, 2, 3),         # H > 4096 at few tokens: RMSNorm kernel + grouped sequence
    ("tiny", 17, 64, 4128, 4, 2, 17),       # I > 4096 at few tokens: RMSNorm kernel + grouped sequence
    ("decode_20b", None, None, None, None, None, 1),
    ("batched_decode_20b", None, None, None, None, None, 64),
    ("prefill_20b", None, None, None, None, None, 4096),
    ("prefill_120b", None, None, None, None, None, 2048),
    # one GPU's shard of the 20B layer on eight GPUs (tensor-parallel decode, expert-parallel prefill)
    ("decode_20b_tp8", None, None, None, None, None, 1),
    ("batched_decode_20b_tp8", None, None, None, None, None, 64),
    ("prefill_20b_ep8", None, None, None, None, None, 2048),
]


@pytest.mark.parametrize("name,T,H,I,E,k,n_cmp", PRENORM_CASES)
def test_forward_prenorm_matches_oracle(name, T, H, I, E, k, n_cmp):
    cfg = CONFIGS[name]
    over = {key: v for key, v in dict(H=H, I=I, E=E, k=k).items() if v is not None}
    cfg = cfg.with_(**over)
    T = cfg.T if T is None else T
    inp = make_inputs(cfg, seed=3, T=T)
    tokens = _sample(T, n_cmp, seed=T + 1)
    eps = 1e-5
    big = len(tokens) * cfg.H * cfg.I > 64 * 2880 * 2880
    ref_fn = oracle.forward_prenorm_expert_major if big else oracle.forward_prenorm
    ref = ref_fn(inp, cfg.k, tokens=tokens, alpha=cfg.alpha, limit=cfg.limit, eps=eps)
    d = upload(inp)
    y, idx, w = _forward(d, cfg.k, cfg, return_topk=True, norm_weight=d["norm_w"], norm_eps=eps)
    # the normalized rows the layer ran on
    xn = bf16_bits(moe.rmsnorm(d["x"], d["norm_w"], eps))[tokens]
    np.testing.assert_array_equal(xn, ref["xn"])
    idx_np = idx.cpu().numpy()[tokens]
    ok = check_selection(idx_np, ref, cfg.H, cfg.k)
    np.testing.assert_allclose(w.cpu().numpy()[tokens][ok], ref["w"][ok], rtol=1e-6, atol=1e-7)
    assert_close_rows(bf16_to_f64(y)[tokens][ok], ref["y"][ok], f"prenorm y ({name}, T={T})")
    # the residual: y - x is the layer's output on xn, so it must also match the plain layer
    # run on the oracle's xn (to the tolerance of one more bf16 rounding of y)
    d_n = dict(d, x=to_dev(np.ascontiguousarray(oracle.rmsnorm(inp["x"], inp["norm_w"], eps))))
    y_plain = _forward(d_n, cfg.k, cfg)
    x_np = bf16_to_f64(d["x"])[tokens]
    diff = bf16_to_f64(y)[tokens] - x_np - bf16_to_f64(y_plain)[tokens]
    bound = 2.0 ** -8 * (np.abs(bf16_to_f64(y)[tokens]) + np.abs(bf16_to_f64(y_plain)[tokens]))
    assert np.all(np.abs(diff) <= bound + 1e-30)


# ----------------------------------------------------------------------------- dequantized bank

BANK_CASES = [
    # (config, T override, H, I, E, k, tokens compared)
    ("tiny", None, None, None, None, None, 64),
    ("tiny", 1, 96, 64, 5, 2, 1),           # contraction tail (96 = 64 + 32), partial column tile
    ("tiny", 65, 96, 160, 5, 2, 65),        # both projections with a contraction tail
    ("tiny", 300, 64, 128, 3, 2, 300),      # several ragged row tiles per expert
    ("tiny", 140, 64, 64, 256, 8, 140),     # maximal E and k
    ("batched_decode_20b", None, None, None, None, None, 64),
    ("prefill_20b", None, None, None, None, None, 4096),
    ("prefill_120b", None, None, None, None, None, 2048),
    # one GPU's shard of the 20B layer on eight GPUs (tensor-parallel decode, expert-parallel prefill)
    ("decode_20b_tp8", None, None, None, None, None, 1),
    ("batched_decode_20b_tp8", None, None, None, None, None, 64),
    ("prefill_20b_ep8", None, None, None, None, None, 2048),
]


@pytest.mark.parametrize("name,T,H,I,E,k,n_cmp", BANK_CASES)
def test_forward_dequantized_matches_oracle(name, T, H, I, E, k, n_cmp):
    """The dequantize-once variant against the oracle, and the pages' invariant that it agrees
    with the routed-only packed path: identical routing, outputs within the same bar."""
    cfg = CONFIGS[name]
    over = {key: v for key, v in dict(H=H, I=I, E=E, k=k).items() if v is not None}
    cfg = cfg.with_(**over)
    T = cfg.T if T is None else T
    inp = make_inputs(cfg, seed=2, T=T)
    tokens = _sample(T, n_cmp, seed=T + 2)
    ref = _reference(inp, cfg, tokens)
    d = upload(inp)
    gu_w, dn_w = moe.dequantize_bank(d["gu_blocks"], d["gu_scales"], d["dn_blocks"], d["dn_scales"])
    y, idx, w = moe.moe_forward_dequantized(d["x"], d["router_w"], d["router_b"], gu_w, d["gu_bias"], dn_w,
                                            d["dn_bias"], cfg.k, cfg.alpha, cfg.limit, return_topk=True)
    idx_np = idx.cpu().numpy()[tokens]
    ok = check_selection(idx_np, ref, cfg.H, cfg.k)
    np.testing.assert_allclose(w.cpu().numpy()[tokens][ok], ref["w"][ok], rtol=1e-6, atol=1e-7)
    y_np = bf16_to_f64(y)[tokens]
    assert_close_rows(y_np[ok], ref["y"][ok], f"dequantized bank y ({name}, T={T})")
    y_p, idx_p, _ = _forward(d, cfg.k, cfg, return_topk=True)
    assert torch.equal(idx, idx_p)
    assert_close_rows(y_np, bf16_to_f64(y_p)[tokens], f"dequantized vs packed ({name}, T={T})")
    y2 = moe.moe_forward_dequantized(d["x"], d["router_w"], d["router_b"], gu_w, d["gu_bias"], dn_w,
                                     d["dn_bias"], cfg.k, cfg.alpha, cfg.limit)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.gpu
def test_clock_probe_reports_a_plausible_clock():
    """The benchmark's clock probe: shader cycles against the constant 100 MHz counter give a
    clock between 0.5 and 3 GHz on every workgroup."""
    lib = moe.load_library()
    blocks = 512
    buf = torch.zeros(2 * blocks, dtype=torch.int64, device=dev())
    assert lib.moe_mxfp4_clock_probe(ctypes.c_void_p(buf.data_ptr()), blocks, 50000, None) == 0
    torch.cuda.synchronize()
    c = buf.view(blocks, 2).cpu().numpy().astype(np.float64)
    assert np.all(c[:, 1] > 0)
    mhz = 100.0 * c[:, 0] / c[:, 1]
    assert np.all((mhz > 500) & (mhz < 3000)), (mhz.min(), mhz.max())
