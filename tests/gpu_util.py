"""Helpers for the GPU parity tests: host <-> device copies and the acceptance rules."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda:0"


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t.view(dtype) if dtype is not None else t


def dev_bf16(a_u16: np.ndarray) -> torch.Tensor:
    return dev(a_u16.view(np.int16), torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


E4M3 = None


def e4m3_table(orc) -> np.ndarray:
    global E4M3
    if E4M3 is None:
        E4M3 = np.array([orc.e4m3_to_f64(c) for c in range(256)], np.float64)
    return E4M3


def e4m3_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of e4m3fn above |v| (2^-9 in the subnormal range)."""
    a = np.abs(v)
    return np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-30))) - 3))


def assert_close(got: np.ndarray, want: np.ndarray, rtol=1e-2, atol=1e-2, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    bad = np.abs(got - want) > atol + rtol * np.abs(want)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements off; first at {tuple(i)}: "
                             f"got {got[tuple(i)]}, want {want[tuple(i)]}")


def assert_fp8_close(orc, codes_g, scales_g, codes_o, scales_o, group=64, what="fp8"):
    """fp8 rows/outputs: each scale (amax/448 of a float group) within the float
    tolerance rtol 1e-2, and each dequantised GPU value within one e4m3 ULP (at the
    oracle's code) of the oracle's, plus what the scale difference itself moves."""
    tab = e4m3_table(orc)
    assert_close(scales_g, scales_o, rtol=1e-2, atol=0, what=what + " scales")
    sg = np.repeat(np.asarray(scales_g, np.float64), group, axis=-1).reshape(codes_g.shape)
    so = np.repeat(np.asarray(scales_o, np.float64), group, axis=-1).reshape(codes_o.shape)
    co, cg = tab[codes_o], tab[codes_g]
    vg = cg * sg
    vo = co * so
    # vg - vo = (cg - co) * so + cg * (sg - so): one code step plus the scale difference
    lim = e4m3_ulp(co) * so + np.abs(cg) * np.abs(sg - so) + 1e-30
    bad = np.abs(vg - vo) > lim * (1 + 1e-6)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} codes beyond one ULP; first at {tuple(i)}: "
                             f"got {vg[tuple(i)]} (code {codes_g[tuple(i)]}), want {vo[tuple(i)]} "
                             f"(code {codes_o[tuple(i)]})")


def assert_fp4_close(orc, rows_g, rows_o, dim, what="fp4"):
    """MXFP4 rows: the rounding decisions sit on fp32 values that differ from the
    oracle's fp64 ones in the last bits, so an element code, or at a power-of-two
    edge of a block's maximum its scale, may differ.  At least 99.5% of the
    elements must decode to the oracle's value, and every element must lie within
    one E2M1 grid step of it at its own magnitude: with X the larger of the two
    block scales and r = max(|got|, |want|) / X, the step is 0.5 X below r = 2,
    X below r = 4 and 2 X above."""
    vg = orc.decode_rows(rows_g, dim, orc.FP4)
    vo = orc.decode_rows(rows_o, dim, orc.FP4)
    eg = rows_g[..., dim // 2:dim // 2 + dim // 32].astype(np.int64)
    eo = rows_o[..., dim // 2:dim // 2 + dim // 32].astype(np.int64)
    X = np.repeat(np.ldexp(1.0, np.maximum(eg, eo) - 127), 32, axis=-1)
    r = np.maximum(np.abs(vg), np.abs(vo)) / X
    step = np.where(r < 2.0, 0.5, np.where(r < 4.0, 1.0, 2.0)) * X
    bad = np.abs(vg - vo) > step
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements beyond one grid step; first at "
                             f"{tuple(i)}: got {vg[tuple(i)]}, want {vo[tuple(i)]}")
    same = float(np.mean(vg == vo))
    assert same >= 0.995, f"{what}: only {same:.4f} of the elements match the oracle's code"


def assert_topk_equivalent(got: np.ndarray, want: np.ndarray, scores: np.ndarray, kth: np.ndarray, what="topk"):
    """Same id sets, except swaps among ids whose oracle scores lie within
    1e-4 * max(1, |kth|) of the oracle's k-th score; ascending order, -1 padding."""
    for n in range(got.shape[0]):
        g = got[n]
        w = want[n]
        gv, wv = g[g >= 0], w[w >= 0]
        assert len(gv) == len(wv), f"{what}[{n}]: {len(gv)} ids, oracle {len(wv)}"
        assert np.all(g[len(gv):] == -1), f"{what}[{n}]: padding not -1"
        assert np.all(np.diff(gv) > 0), f"{what}[{n}]: ids not strictly ascending"
        extra = np.setdiff1d(gv, wv)
        missing = np.setdiff1d(wv, gv)
        if len(extra) == 0 and len(missing) == 0:
            continue
        tol = 1e-4 * max(1.0, abs(kth[n]))
        for i in np.concatenate([extra, missing]):
            assert 0 <= i < scores.shape[1], f"{what}[{n}]: id {i} not a candidate"
            assert abs(scores[n, i] - kth[n]) <= tol, (
                f"{what}[{n}]: id {i} (score {scores[n, i]}) differs, k-th score {kth[n]}")
