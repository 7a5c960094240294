"""Helpers for the GPU parity tests: upload seeded inputs, host-side expected
permutations, and the comparison rules.

Comparison rules (the layer's outputs are bf16; the oracle is IEEE double):
* integer outputs (top-k indices, permutation) must match exactly;
* a token's selection is compared exactly when the oracle's margin between the k-th
  and (k+1)-th logits exceeds the worst-case double summation error of both sides
  (4 * gamma_{H+1} * max_e sum_h |x_h W_eh|, gamma_n = n u / (1 - n u), u = 2^-53);
  inside that margin any valid top-k is accepted and the token is left out of the
  output comparison (the count is reported);
* float outputs: per token, relative L2 error ||y - y_ref|| / ||y_ref|| <= 1e-2, and
  every element |y - y_ref| <= 5e-2 * rms(y_ref[t]).
"""
from __future__ import annotations

import numpy as np
import torch

REL_L2 = 1e-2
ELEM = 5e-2
U64 = 2.0 ** -53


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    """Host numpy -> device tensor; uint16 bf16 bit patterns become torch.bfloat16."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(torch.bfloat16)
    t = torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    return t if dtype is None else t.to(dtype)


def upload(inp) -> dict:
    return {k: to_dev(v) for k, v in inp.items()}


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_permutation(idx: np.ndarray, E: int):
    """Stable sort of the (token, slot) pairs by expert (numpy's stable argsort)."""
    flat = idx.reshape(-1).astype(np.int64)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    k = idx.shape[1]
    sorted_token = (order // k).astype(np.int32)
    slot_row = np.empty_like(order)
    slot_row[order] = np.arange(order.size)
    return offsets, sorted_token, order, slot_row.astype(np.int32)


def _e4m3_table() -> np.ndarray:
    """Values of the 256 OCP E4M3 codes (0x7f / 0xff: NaN)."""
    t = np.empty(256, dtype=np.float64)
    for b in range(256):
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        t[b] = np.nan if (b & 0x7F) == 0x7F else (-mag if s else mag)
    return t


E4M3 = _e4m3_table()


def decode_mx8(q8, R: int, K: int) -> np.ndarray:
    """Values [R, K] of an mx8 activation matrix (layout in moe_mxfp4.h): per 32-element
    block, hi * 2^(s_hi - 127) + lo * 2^(s_lo - 127)."""
    q = np.asarray(q8.cpu().numpy() if hasattr(q8, "cpu") else q8, dtype=np.uint8)
    S = ((K // 32) + 15) // 16 * 16
    data = q[: 2 * R * K].reshape(2 * R, K)
    sc = q[2 * R * K: 2 * R * K + 2 * R * S].reshape(2 * R, S)[:, : K // 32].astype(np.int64)
    mult = np.ldexp(1.0, np.repeat(sc, 32, axis=1) - 127)
    v = E4M3[data] * mult
    return v[0::2] + v[1::2]


def decode_h8(q8, R: int, K: int) -> np.ndarray:
    """Values [R, K] of an h8 matrix (mx8 data rows; hi scales group-major, byte b % 16 of
    word r of group b // 16; lo scale = hi - 4; layout in moe_mxfp4.h)."""
    q = np.asarray(q8.cpu().numpy() if hasattr(q8, "cpu") else q8, dtype=np.uint8)
    nb, G = K // 32, (K + 511) // 512
    data = q[: 2 * R * K].reshape(2 * R, K)
    grp = q[2 * R * K: 2 * R * K + 16 * R * G].reshape(G, R, 16)
    s_hi = grp.transpose(1, 0, 2).reshape(R, 16 * G)[:, :nb].astype(np.int64)
    hi = E4M3[data[0::2]] * np.ldexp(1.0, np.repeat(s_hi, 32, axis=1) - 127)
    lo = E4M3[data[1::2]] * np.ldexp(1.0, np.repeat(s_hi - 4, 32, axis=1) - 127)
    return hi + lo


def gamma(n: int) -> float:
    return n * U64 / (1 - n * U64)


def selection_tolerance(H: int, abs_sum: np.ndarray) -> np.ndarray:
    """Per-token band within which two logits may be ordered either way by the GPU path:
    the error bound of any fp64 summation order of H+1 terms, plus the selection key's
    resolution (logits closer than 2^-44 relative count as equal there; 2^-43 covers both
    sides)."""
    return (4 * gamma(H + 1) + 2.0 ** -43) * abs_sum.max(axis=1)


def decided_tokens(ref: dict, H: int, k: int) -> np.ndarray:
    """Mask of tokens whose top-k set is fixed beyond the summation-error margin."""
    logits, abs_sum = ref["logits"], ref["abs_sum"]
    E = logits.shape[1]
    if k == E:
        return np.ones(logits.shape[0], dtype=bool)
    srt = -np.sort(-logits, axis=1)
    margin = srt[:, k - 1] - srt[:, k]
    return margin > selection_tolerance(H, abs_sum)


def check_selection(gpu_idx: np.ndarray, ref: dict, H: int, k: int):
    """Exact match on decided tokens; a valid top-k on the others. Returns the mask
    of tokens whose outputs can be compared."""
    decided = decided_tokens(ref, H, k)
    np.testing.assert_array_equal(gpu_idx[decided], ref["idx"][decided])
    tau = selection_tolerance(H, ref["abs_sum"])
    for t in np.nonzero(~decided)[0]:
        sel = set(gpu_idx[t].tolist())
        assert len(sel) == k
        l = ref["logits"][t]
        lo = min(l[list(sel)])
        hi = max([l[e] for e in range(l.size) if e not in sel], default=-np.inf)
        assert lo >= hi - tau[t]
    return decided & np.all(gpu_idx == ref["idx"], axis=1)


def assert_close_rows(got: np.ndarray, want: np.ndarray, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    diff = got - want
    num = np.linalg.norm(diff, axis=-1)
    den = np.linalg.norm(want, axis=-1)
    rel = num / np.maximum(den, 1e-300)
    rms = den / np.sqrt(want.shape[-1])
    elem = np.max(np.abs(diff), axis=-1) / np.maximum(rms, 1e-300)
    worst = int(np.argmax(rel))
    assert rel.max() <= REL_L2, f"{what}: rel-L2 {rel.max():.3e} at row {worst}"
    assert elem.max() <= ELEM, f"{what}: max|d|/rms {elem.max():.3e} at row {int(np.argmax(elem))}"
    return float(rel.max()), float(elem.max())
