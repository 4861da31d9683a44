"""Pins of the CPU fp64 oracle against things other than itself.

Each ``pin_*`` function takes an oracle instance and raises AssertionError on a mismatch, so the same
pins run against the real oracle (the tests below) and against deliberately broken copies of it
(``test_planted_mistakes_are_caught``), which shows that a plausible mistake anywhere in the oracle
fails at least one pin.

What pins what:
  * hand-worked cases (tests/golden/hand_cases.json, derived by hand from the equations of the page
    "aclnnMaskedCausalConv1dBackward", section 功能说明 / function description);
  * the page's call example (section 调用示例): S=1, B=2, H=384, FLOAT16, all inputs zero;
  * PyTorch CPU fp64 autograd of the causal depthwise conv1d forward (a library routine whose
    gradient is exactly this backward);
  * the adjoint identity <F(x,w), gY> = <x, gradX> = <w, gradWeight>;
  * invariants: sign/scale equivariance, linearity, batch permutation, column independence,
    null mask == all-true mask, all-false mask -> zeros;
  * the codec: all 65536 patterns of both formats against numpy/torch decoding, round trips, and
    encoding against numpy's float64->float16 cast and a brute-force nearest-even search.
"""
from __future__ import annotations

import json
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from synth import workloads as wls

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "hand_cases.json")
TD = {"bf16": torch.bfloat16, "fp16": torch.float16}


# -- helpers independent of the oracle ---------------------------------------------------------------
def to_bits(values, dtype: str) -> np.ndarray:
    """Encode with torch's own cast (independent of the oracle's encoder)."""
    t = torch.tensor(np.asarray(values, dtype=np.float64)).to(TD[dtype])
    return t.view(torch.int16).numpy().view(np.uint16)


def from_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode with torch's own cast (independent of the oracle's decoder)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TD[dtype])
    return t.to(torch.float64).numpy()


def random_case(S, B, H, dtype="bf16", mask=("bernoulli", 0.7), seed=3):
    wl = synth.custom(S, B, H, dtype=dtype, mask=mask, seed=seed)
    inp = wls.host_inputs(wl)
    m = inp["mask"]
    return (wls.bits(inp["gy"]), wls.bits(inp["x"]), wls.bits(inp["w"]),
            None if m is None else m.numpy())


def torch_autograd(gy64, x64, w64, mask):
    """Gradients of y = mask * causal_depthwise_conv1d(x, w) by PyTorch CPU fp64 autograd; the
    window W is w64's first dimension."""
    S, B, H = x64.shape
    W = w64.shape[0]
    xt = torch.from_numpy(x64).permute(1, 2, 0).contiguous().requires_grad_(True)  # [B,H,S]
    wt = torch.from_numpy(w64).t().contiguous().unsqueeze(1).requires_grad_(True)  # [H,1,W]
    y = F.conv1d(xt, wt, padding=W - 1, groups=H)[..., :S]
    if mask is not None:
        y = y * torch.from_numpy(mask.astype(np.float64))[:, None, :]
    y.backward(torch.from_numpy(gy64).permute(1, 2, 0).contiguous())
    gx = xt.grad.permute(2, 0, 1).contiguous().numpy()
    gw = wt.grad.squeeze(1).t().contiguous().numpy()
    return gx, gw


SHAPES = [(1, 2, 5), (2, 3, 4), (3, 1, 7), (7, 3, 5), (33, 2, 6), (40, 4, 64)]


# -- pins --------------------------------------------------------------------------------------------
def pin_hand_cases(orc):
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        for dtype in ("bf16", "fp16"):
            gy = to_bits(c["gY"], dtype)
            x = to_bits(c["x"], dtype)
            w = to_bits(c["w"], dtype)
            m = None if c["mask"] is None else np.array(c["mask"], dtype=np.uint8)
            r = orc.backward(dtype, gy, x, w, m)
            exp_gx = np.array(c["gX"], dtype=np.float64)
            exp_gw = np.array(c["gW"], dtype=np.float64)
            tag = f"{c['name']}/{dtype}"
            assert np.array_equal(r["gx64"], exp_gx), (tag, r["gx64"], exp_gx)
            assert np.array_equal(r["gw64"], exp_gw), (tag, r["gw64"], exp_gw)
            assert np.array_equal(from_bits(r["gx16"], dtype), exp_gx), tag
            assert np.array_equal(from_bits(r["gw16"], dtype), exp_gw), tag
            np.testing.assert_allclose(r["gwrss"] ** 2, np.array(c["gW_sumsq"], float),
                                       rtol=1e-12, err_msg=tag)


FWD_GOLDEN = os.path.join(HERE, "golden", "forward_hand_cases.json")


def pin_forward_hand_cases(orc):
    for c in json.load(open(FWD_GOLDEN))["cases"]:
        for dtype in ("bf16", "fp16"):
            x = to_bits(c["x"], dtype)
            w = to_bits(c["w"], dtype)
            m = None if c["mask"] is None else np.array(c["mask"], dtype=np.uint8)
            r = orc.forward16(dtype, x, w, m)
            exp = np.array(c["y"], dtype=np.float64)
            tag = f"{c['name']}/{dtype}"
            assert np.array_equal(r["y64"], exp), (tag, r["y64"], exp)
            assert np.array_equal(from_bits(r["y16"], dtype), exp), tag


WIN_GOLDEN = os.path.join(HERE, "golden", "window_hand_cases.json")


def pin_window_hand_cases(orc):
    for c in json.load(open(WIN_GOLDEN))["cases"]:
        for dtype in ("bf16", "fp16"):
            tag = f"{c['name']}/{dtype}"
            m = None if c["mask"] is None else np.array(c["mask"], dtype=np.uint8)
            x, w = to_bits(c["x"], dtype), to_bits(c["w"], dtype)
            assert w.shape[0] == c["W"], tag
            if c["op"] == "forward":
                r = orc.forward16(dtype, x, w, m)
                exp = np.array(c["y"], dtype=np.float64)
                assert np.array_equal(r["y64"], exp), (tag, r["y64"], exp)
                assert np.array_equal(from_bits(r["y16"], dtype), exp), tag
                continue
            r = orc.backward(dtype, to_bits(c["gY"], dtype), x, w, m)
            exp_gx, exp_gw = np.array(c["gX"], np.float64), np.array(c["gW"], np.float64)
            assert np.array_equal(r["gx64"], exp_gx), (tag, r["gx64"], exp_gx)
            assert np.array_equal(r["gw64"], exp_gw), (tag, r["gw64"], exp_gw)
            assert np.array_equal(from_bits(r["gx16"], dtype), exp_gx), tag
            assert np.array_equal(from_bits(r["gw16"], dtype), exp_gw), tag
            np.testing.assert_allclose(r["gwrss"] ** 2, np.array(c["gW_sumsq"], float),
                                       rtol=1e-12, err_msg=tag)


def pin_window_autograd_and_adjoint(orc):
    """W != 3 against PyTorch autograd of conv1d(kernel W, padding W-1) and the adjoint
    identity <F(x,w), gY> = <x, gradX> = <w, gradWeight>."""
    for W in (1, 2, 4):
        for n, (S, B, H) in enumerate(SHAPES):
            wl = synth.custom(S, B, H, "bf16", ("bernoulli", 0.7), seed=130 + n, W=W)
            inp = wls.host_inputs(wl)
            gy, x, w = wls.bits(inp["gy"]), wls.bits(inp["x"]), wls.bits(inp["w"])
            m = None if inp["mask"] is None else inp["mask"].numpy()
            assert w.shape == (W, H)
            gy64, x64, w64 = (from_bits(a, "bf16") for a in (gy, x, w))
            r = orc.backward("bf16", gy, x, w, m)
            gx_ref, gw_ref = torch_autograd(gy64, x64, w64, m)
            sx = max(1.0, float(np.abs(gx_ref).max()))
            assert np.allclose(r["gx64"], gx_ref, rtol=0, atol=1e-13 * sx), (W, S, B, H)
            sw = max(1.0, float(np.abs(gw_ref).max()))
            assert np.allclose(r["gw64"], gw_ref, rtol=0, atol=1e-12 * sw), (W, S, B, H)
            y = orc.forward(x64, w64, m)
            lhs, mid = float(np.sum(y * gy64)), float(np.sum(x64 * r["gx64"]))
            rhs = float(np.sum(w64 * r["gw64"]))
            scale = float(np.sum(np.abs(y * gy64))) + 1e-300
            assert abs(lhs - mid) <= 1e-12 * scale and abs(lhs - rhs) <= 1e-12 * scale, (W, S)


VARLEN_GOLDEN = os.path.join(HERE, "golden", "varlen_hand_cases.json")


def pin_varlen_hand_cases(orc):
    for c in json.load(open(VARLEN_GOLDEN))["cases"]:
        cu = np.array(c["cu"], dtype=np.int64)
        m = None if c["mask"] is None else np.array(c["mask"], dtype=np.uint8)
        for dtype in ("bf16", "fp16"):
            tag = f"{c['name']}/{dtype}"
            x, w = to_bits(c["x"], dtype), to_bits(c["w"], dtype)
            if c["op"] == "forward":
                r = orc.forward16_varlen(dtype, x, w, cu, m)
                exp = np.array(c["y"], np.float64)
                assert np.array_equal(r["y64"], exp), (tag, r["y64"], exp)
                assert np.array_equal(from_bits(r["y16"], dtype), exp), tag
                continue
            r = orc.backward_varlen(dtype, to_bits(c["gY"], dtype), x, w, cu, m)
            exp_gx, exp_gw = np.array(c["gX"], np.float64), np.array(c["gW"], np.float64)
            assert np.array_equal(r["gx64"], exp_gx), (tag, r["gx64"], exp_gx)
            assert np.array_equal(r["gw64"], exp_gw), (tag, r["gw64"], exp_gw)
            assert np.array_equal(from_bits(r["gx16"], dtype), exp_gx), tag
            np.testing.assert_allclose(r["gwrss"] ** 2, np.array(c["gW_sumsq"], float),
                                       rtol=1e-12, err_msg=tag)


def pin_varlen_equals_padded(orc):
    """The packed layout computes what the padded [S,B,H] layout computes with a per-batch valid
    prefix mask (lengths = the sequence lengths), on the valid tokens: the same gradX there and the
    same gradWeight; likewise for the forward. The padded oracle is pinned independently above."""
    rng = np.random.default_rng(5)
    for W in (1, 2, 3, 4):
        for lens in ([5, 1, 3], [7], [2, 0, 6, 4, 1], [1, 1, 1, 1]):
            B, S, H = len(lens), max(lens), 6
            T = int(sum(lens))
            cu = np.cumsum(lens).astype(np.int64)
            gyp = rng.standard_normal((S, B, H))
            xp = rng.standard_normal((S, B, H))
            w = to_bits(rng.standard_normal((W, H)) * 0.5, "bf16")
            tok = rng.random((S, B)) < 0.8  # an extra per-token mask
            valid = np.arange(S)[:, None] < np.array(lens)[None, :]
            gyp16, xp16 = to_bits(gyp, "bf16"), to_bits(xp, "bf16")
            mask_pad = (valid & tok).T.astype(np.uint8)  # [B,S]
            order = [(b, i) for b in range(B) for i in range(lens[b])]
            pack = lambda a: np.stack([a[i, b] for b, i in order]) if order else a[:0, 0]
            gyv, xv = pack(gyp16), pack(xp16)
            mv = np.array([tok[i, b] for b, i in order], np.uint8)
            rp = orc.backward("bf16", gyp16, xp16, w, mask_pad)
            rv = orc.backward_varlen("bf16", gyv, xv, w, cu, mv)
            assert np.array_equal(rv["gx64"], pack(rp["gx64"])), (W, lens)
            scale = np.maximum(rp["gwrss"], 1e-300)
            assert np.all(np.abs(rv["gw64"] - rp["gw64"]) <= 1e-12 * scale), (W, lens)
            yp = orc.forward(from_bits(xp16, "bf16"), from_bits(w, "bf16"), mask_pad)
            yv = orc.forward_varlen(from_bits(xv, "bf16"), from_bits(w, "bf16"), cu, mv)
            assert np.array_equal(yv, pack(yp)), (W, lens)


def pin_call_example(orc):
    # Call example on the page: S=1, B=2, H=192*2, W=3, FLOAT16, every input (and the bool mask)
    # zero-filled. Whatever the print format, the gradients must be zero.
    S, B, H = 1, 2, 384
    z = np.zeros((S, B, H), np.uint16)
    for mask in (np.zeros((B, S), np.uint8), None):
        r = orc.backward("fp16", z, z, np.zeros((3, H), np.uint16), mask)
        assert np.all(from_bits(r["gx16"], "fp16") == 0.0)
        assert np.all(from_bits(r["gw16"], "fp16") == 0.0)
        assert np.all(r["gx64"] == 0.0) and np.all(r["gw64"] == 0.0)


def pin_autograd(orc):
    for n, (S, B, H) in enumerate(SHAPES):
        for dtype, mask in (("bf16", ("bernoulli", 0.7)), ("fp16", ("null",)),
                            ("bf16", ("prefix",))):
            gy, x, w, m = random_case(S, B, H, dtype, mask, seed=11 + n)
            r = orc.backward(dtype, gy, x, w, m)
            gx_ref, gw_ref = torch_autograd(from_bits(gy, dtype), from_bits(x, dtype),
                                            from_bits(w, dtype), m)
            sx = max(1.0, float(np.abs(gx_ref).max()))
            assert np.allclose(r["gx64"], gx_ref, rtol=0, atol=1e-13 * sx), (S, B, H, dtype)
            sw = max(1.0, float(np.abs(gw_ref).max()))
            assert np.allclose(r["gw64"], gw_ref, rtol=0, atol=1e-12 * sw), (S, B, H, dtype)


def pin_adjoint(orc):
    for n, (S, B, H) in enumerate(SHAPES):
        gy, x, w, m = random_case(S, B, H, "bf16", ("bernoulli", 0.6), seed=50 + n)
        gy64, x64, w64 = (from_bits(a, "bf16") for a in (gy, x, w))
        y = orc.forward(x64, w64, m)
        r = orc.backward("bf16", gy, x, w, m)
        lhs = float(np.sum(y * gy64))
        mid = float(np.sum(x64 * r["gx64"]))
        rhs = float(np.sum(w64 * r["gw64"]))
        scale = float(np.sum(np.abs(y * gy64))) + 1e-300
        assert abs(lhs - mid) <= 1e-12 * scale, (S, B, H, lhs, mid)
        assert abs(lhs - rhs) <= 1e-12 * scale, (S, B, H, lhs, rhs)


def pin_forward(orc):
    # The forward used by the adjoint pin is itself pinned to torch's conv1d.
    for n, (S, B, H) in enumerate(SHAPES):
        _, x, w, m = random_case(S, B, H, "bf16", ("bernoulli", 0.5), seed=70 + n)
        x64, w64 = from_bits(x, "bf16"), from_bits(w, "bf16")
        y = orc.forward(x64, w64, m)
        xt = torch.from_numpy(x64).permute(1, 2, 0)
        wt = torch.from_numpy(w64).t().contiguous().unsqueeze(1)
        ref = F.conv1d(xt, wt, padding=2, groups=H)[..., :S] * torch.from_numpy(
            m.astype(np.float64))[:, None, :]
        ref = ref.permute(2, 0, 1).numpy()
        assert np.allclose(y, ref, rtol=0, atol=1e-13 * max(1.0, np.abs(ref).max()))


def pin_invariants(orc):
    S, B, H = 19, 3, 8
    gy, x, w, m = random_case(S, B, H, "bf16", ("bernoulli", 0.7), seed=91)
    base = orc.backward("bf16", gy, x, w, m)
    # null mask == explicit all-true mask, bit for bit
    r_null = orc.backward("bf16", gy, x, w, None)
    r_true = orc.backward("bf16", gy, x, w, np.ones((B, S), np.uint8))
    for k in ("gx16", "gw16", "gx64", "gw64"):
        assert np.array_equal(r_null[k], r_true[k]), k
    # any nonzero byte counts as true
    r_255 = orc.backward("bf16", gy, x, w, np.full((B, S), 255, np.uint8))
    assert np.array_equal(r_255["gx16"], r_true["gx16"])
    # all-false mask -> exact zeros
    r0 = orc.backward("bf16", gy, x, w, np.zeros((B, S), np.uint8))
    assert np.all(r0["gx64"] == 0) and np.all(r0["gw64"] == 0)
    # sign flip of gradY negates both gradients exactly (flip the sign bit)
    neg = gy ^ np.uint16(0x8000)
    rn = orc.backward("bf16", neg, x, w, m)
    assert np.array_equal(rn["gx64"], -base["gx64"]) and np.array_equal(rn["gw64"], -base["gw64"])
    # scaling gradY by 2 (exponent + 1) doubles both exactly
    g2 = to_bits(from_bits(gy, "bf16") * 2.0, "bf16")
    r2 = orc.backward("bf16", g2, x, w, m)
    assert np.array_equal(r2["gx64"], 2 * base["gx64"]) and np.array_equal(r2["gw64"], 2 * base["gw64"])
    # linearity in gradY: split gradY into two disjoint parts
    pick = (np.arange(gy.size).reshape(gy.shape) * 7919) % 3 == 0
    ga = np.where(pick, gy, 0).astype(np.uint16)
    gb = np.where(pick, 0, gy).astype(np.uint16)
    ra, rb = orc.backward("bf16", ga, x, w, m), orc.backward("bf16", gb, x, w, m)
    assert np.allclose(ra["gx64"] + rb["gx64"], base["gx64"], rtol=0, atol=1e-13)
    assert np.allclose(ra["gw64"] + rb["gw64"], base["gw64"], rtol=0, atol=1e-12)
    # permuting the batch permutes gradX and leaves gradWeight unchanged
    perm = np.array([2, 0, 1])
    rp = orc.backward("bf16", gy[:, perm], x[:, perm], w, m[perm])
    assert np.array_equal(rp["gx64"], base["gx64"][:, perm])
    assert np.allclose(rp["gw64"], base["gw64"], rtol=0, atol=1e-12)
    # columns are independent: a column subset gives the same bits
    hs = np.array([6, 1, 3])
    rc = orc.backward("bf16", gy[:, :, hs], x[:, :, hs], w[:, hs], m)
    assert np.array_equal(rc["gx16"], base["gx16"][:, :, hs])
    assert np.array_equal(rc["gw64"], base["gw64"][:, hs])
    # the stencil only looks ahead: changing the last row leaves gradX rows < S-3 untouched
    gz = gy.copy()
    gz[-1] ^= np.uint16(0x8000)
    rz = orc.backward("bf16", gz, x, w, m)
    assert np.array_equal(rz["gx64"][: S - 3], base["gx64"][: S - 3])


def _all_patterns():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def pin_codec_decode(orc):
    pats = _all_patterns()
    for dtype in ("fp16", "bf16"):
        got = orc.decode(dtype, pats)
        if dtype == "fp16":
            ref = pats.view(np.float16).astype(np.float64)
        else:
            ref = from_bits(pats, "bf16")
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), dtype
        assert np.array_equal(got[~nan], ref[~nan]), dtype
        # signed zeros decode with their sign
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), dtype


def pin_codec_roundtrip(orc):
    pats = _all_patterns()
    for dtype in ("fp16", "bf16"):
        vals = from_bits(pats, dtype)
        ok = ~np.isnan(vals)
        back = orc.encode(dtype, vals[ok])
        assert np.array_equal(back, pats[ok]), dtype


def _fp16_specials():
    v = [0.0, -0.0, 65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001,
         3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11,
         1.0 + 2.0 ** -11 + 2.0 ** -40, 2049.0, 2051.0, -2049.0, 1e-9, -1e-9]
    return np.array(v, dtype=np.float64)


def pin_codec_encode_fp16(orc):
    rng = np.random.default_rng(5)
    v = np.concatenate([
        rng.standard_normal(20000) * 3.0,
        rng.standard_normal(5000) * 1e-5,  # subnormal range
        rng.uniform(-65000, 65000, 5000),
        # exact midpoints between neighbouring fp16 values: ties must go to even
        ((np.arange(1, 4000, dtype=np.float64) + 0.5) * 2.0 ** -10) * np.where(
            np.arange(1, 4000) % 2 == 0, 1.0, -1.0),
        _fp16_specials(),
    ])
    got = orc.encode("fp16", v)
    with np.errstate(over="ignore"):  # 65520 and above round to infinity, as they should
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def pin_codec_encode_bf16(orc):
    rng = np.random.default_rng(6)
    # (a) float32-representable inputs against torch's float32 -> bfloat16 cast
    v32 = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-39,
                          rng.standard_normal(2000) * 1e30]).astype(np.float32)
    got = orc.encode("bf16", v32.astype(np.float64))
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    # (b) arbitrary doubles against a brute-force nearest-even search over all finite bf16 values
    pats = _all_patterns()
    vals = from_bits(pats, "bf16")
    fin = np.isfinite(vals) & ~((vals == 0) & np.signbit(vals))
    order = np.argsort(vals[fin], kind="stable")
    sv, sp = vals[fin][order], pats[fin][order]
    mids = (sv[:-1] + sv[1:]) / 2  # exact in fp64
    v = np.concatenate([rng.standard_normal(4000) * 2.0 ** rng.integers(-130, 120, 4000),
                        mids[rng.integers(0, len(mids), 3000)],
                        np.nextafter(mids[rng.integers(0, len(mids), 1000)], np.inf),
                        np.nextafter(mids[rng.integers(0, len(mids), 1000)], -np.inf)])
    v = v[np.abs(v) < sv[-1]]
    k = np.clip(np.searchsorted(sv, v), 1, len(sv) - 1)
    lo, hi = sv[k - 1], sv[k]
    pick_hi = (hi - v < v - lo) | ((hi - v == v - lo) & (sp[k] % 2 == 0))
    ref = np.where(pick_hi, sp[k], sp[k - 1])
    got = orc.encode("bf16", v)
    same = got == ref
    # +0/-0: the search returns +0 for values that round to zero from below
    zero = (from_bits(ref, "bf16") == 0) & (from_bits(got, "bf16") == 0)
    assert np.all(same | zero)


def _rows_run(orc, dtype, gy, x, w, m, cuts):
    """The row-range oracle over consecutive ranges split at `cuts`: (gradX bits, fp64 sums, sums
    of squared terms)."""
    S, B, H = gy.shape
    W = w.shape[0]
    acc = np.zeros((W, H)), np.zeros((W, H))
    parts = []
    edges = [0, *cuts, S]
    for r0, r1 in zip(edges[:-1], edges[1:]):
        parts.append(orc.backward_rows(dtype, S, r0, r1, gy[r0:min(r1 + W - 1, S)], x[r0:r1], w, m,
                                       acc[0], acc[1]))
    return np.concatenate(parts), acc[0], acc[1]


def pin_rows_hand_cases(orc):
    """The row-range entry point on the hand-worked cases, one row per range: every gradX value and
    the gradWeight sums are the derived ones."""
    for c in json.load(open(GOLDEN))["cases"]:
        for dtype in ("bf16", "fp16"):
            gy, x, w = to_bits(c["gY"], dtype), to_bits(c["x"], dtype), to_bits(c["w"], dtype)
            m = None if c["mask"] is None else np.array(c["mask"], dtype=np.uint8)
            gx16, gw, sq = _rows_run(orc, dtype, gy, x, w, m, list(range(1, gy.shape[0])))
            tag = f"{c['name']}/{dtype}"
            assert np.array_equal(from_bits(gx16, dtype), np.array(c["gX"], float)), tag
            assert np.array_equal(gw, np.array(c["gW"], float)), tag
            assert np.array_equal(sq, np.array(c["gW_sumsq"], float)), tag


def pin_rows_equal_whole(orc):
    """Consecutive row ranges (of every length from 1, ending anywhere, with and without a mask,
    1-4 taps) give the whole-tensor oracle's gradX bit for bit and its gradWeight sums up to fp64
    reordering (the whole-tensor oracle is pinned independently above)."""
    for W in (1, 2, 3, 4):
        for mask in (("bernoulli", 0.7), ("null",)):
            gy, x, w, m = random_case(23, 3, 24, "bf16", mask, seed=30 + W)
            w = to_bits(np.resize(from_bits(w, "bf16"), (W, 24)), "bf16")
            whole = orc.backward("bf16", gy, x, w, m)
            for cuts in ([], [1], [22], [5, 6, 7, 20], list(range(1, 23)), [3, 11, 21]):
                gx16, gw, sq = _rows_run(orc, "bf16", gy, x, w, m, cuts)
                tag = (W, mask[0], cuts)
                assert np.array_equal(gx16, whole["gx16"]), tag
                scale = np.maximum(whole["gwrss"], 1e-300)
                assert np.all(np.abs(gw - whole["gw64"]) <= 1e-12 * scale), tag
                np.testing.assert_allclose(np.sqrt(sq), whole["gwrss"], rtol=1e-12, err_msg=str(tag))


PINS = [pin_hand_cases, pin_rows_hand_cases, pin_rows_equal_whole, pin_forward_hand_cases, pin_window_hand_cases,
        pin_window_autograd_and_adjoint, pin_varlen_hand_cases, pin_varlen_equals_padded,
        pin_call_example, pin_autograd, pin_adjoint, pin_forward, pin_invariants,
        pin_codec_decode, pin_codec_roundtrip, pin_codec_encode_fp16, pin_codec_encode_bf16]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_threads_reported(orc):
    assert orc.num_threads() >= 1


def test_result_independent_of_thread_count(tmp_path):
    """The oracle splits h across threads; each thread owns its outputs, so 1 thread == N threads."""
    code = (
        "import numpy as np, oracle, sys; sys.path.insert(0, '.');\n"
        "from tests.test_oracle import random_case\n"
        "gy,x,w,m = random_case(17, 3, 40, 'bf16', ('bernoulli', 0.7), seed=5)\n"
        "r = oracle.get().backward('bf16', gy, x, w, m)\n"
        "np.save(sys.argv[1], np.concatenate([r['gx64'].ravel(), r['gw64'].ravel()]))\n"
    )
    root = os.path.dirname(HERE)
    outs = []
    for t in ("1", "5"):
        out = str(tmp_path / f"r{t}.npy")
        env = dict(os.environ, OMP_NUM_THREADS=t)
        subprocess.run(["python", "-c", code, out], check=True, cwd=root, env=env)
        outs.append(np.load(out))
    assert np.array_equal(outs[0], outs[1])


def test_set_num_threads_keeps_results(orc):
    """The thread-count setter (used to time the oracle on one thread) changes no result."""
    gy, x, w, m = random_case(23, 2, 40, "fp16", ("bernoulli", 0.6), seed=8)
    n0 = orc.num_threads()
    try:
        orc.set_num_threads(1)
        assert orc.num_threads() == 1
        a = orc.backward("fp16", gy, x, w, m)
        orc.set_num_threads(max(n0, 3))
        b = orc.backward("fp16", gy, x, w, m)
    finally:
        orc.set_num_threads(n0)
    assert np.array_equal(a["gx64"], b["gx64"]) and np.array_equal(a["gw64"], b["gw64"])
    assert np.array_equal(a["gx16"], b["gx16"]) and np.array_equal(a["gw16"], b["gw16"])


# -- planted mistakes ------------------------------------------------------------------------------
MUTANTS = [
    ("tap orientation reversed", "wd[(W - 1 - k) * H + h]", "wd[k * H + h]"),
    ("mask index not transposed", "mask[j * S + i] != 0) ? 1.0 : 0.0;\n    return",
     "mask[i * B + j] != 0) ? 1.0 : 0.0;\n    return"),
    ("mask polarity inverted", "mask[j * S + i] != 0) ? 1.0 : 0.0;\n    return",
     "mask[j * S + i] == 0) ? 1.0 : 0.0;\n    return"),
    ("padding wraps around", "if (i >= S) return 0.0;", "if (i >= S) i -= S;"),
    ("gradWeight tap shift", "grad_y_masked(gyd, mask, S, B, H, i + W - 1 - k, j, h) * xd",
     "grad_y_masked(gyd, mask, S, B, H, i + k, j, h) * xd"),
    ("gradX drops the last tap",
     "for (int k = 0; k < W; ++k) {\n                    acc += grad_y_masked",
     "for (int k = 0; k < W - 1; ++k) {\n                    acc += grad_y_masked"),
    ("gradWeight skips the first batch", "for (int64_t j = 0; j < B; ++j) {\n                for (int64_t i = 0; i < S; ++i) {\n                    const double term",
     "for (int64_t j = 1; j < B; ++j) {\n                for (int64_t i = 0; i < S; ++i) {\n                    const double term"),
    ("encoder rounds ties away from zero", "(frac == 0.5 && fmod(r, 2.0) != 0.0)", "(frac == 0.5)"),
    ("encoder truncates", "if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;", ""),
    ("decoder subnormal scale off", "ldexp((double)f, 1 - bias - pb)", "ldexp((double)f, -bias - pb)"),
    ("decoder bias off by one", "e - bias - pb);", "e - bias - pb + 1);"),
    ("gradWeight rss uses |term|", "sq += term * term;", "sq += fabs(term);"),
    ("forward taps reversed", "acc += w[k * H + h] * x[", "acc += w[(W - 1 - k) * H + h] * x["),
    ("forward shifted one row back", "const int64_t src = i - (W - 1) + k;",
     "const int64_t src = i - W + k;"),
    ("forward ignores the mask", "y[(i * B + j) * H + h] = m * acc;", "y[(i * B + j) * H + h] = acc;"),
    ("gradX window stuck at 3 taps",
     "for (int k = 0; k < W; ++k) {\n                    acc += grad_y_masked",
     "for (int k = 0; k < W && k < 3; ++k) {\n                    acc += grad_y_masked"),
    ("varlen gradX reads across a sequence end", "if (r >= end) break;", "if (r >= T) break;"),
    ("varlen forward reads before a sequence start", "if (src < start) continue;",
     "if (src < 0) continue;"),
    ("varlen gradWeight crosses sequences", "if (r >= end) continue;", "if (r >= T) continue;"),
    ("forward window stuck at 3 taps",
     "for (int k = 0; k < W; ++k) {\n                    const int64_t src",
     "for (int k = 0; k < W && k < 3; ++k) {\n                    const int64_t src"),
    ("varlen gradX ignores the token mask",
     "mask[r] != 0) ? 1.0 : 0.0;\n                    acc += m * gyd",
     "mask[r] != 0) ? 1.0 : 1.0;\n                    acc += m * gyd"),
    ("varlen gradX masks by the output token",
     "if (r >= end) break;\n                    const double m = (mask == NULL || mask[r] != 0)",
     "if (r >= end) break;\n                    const double m = (mask == NULL || mask[t] != 0)"),
    ("varlen gradWeight ignores the token mask",
     "mask[r] != 0) ? 1.0 : 0.0;\n                    const double term",
     "mask[r] != 0) ? 1.0 : 1.0;\n                    const double term"),
    ("varlen forward ignores the token mask",
     "mask[t] != 0) ? 1.0 : 0.0;\n                y[t * H + h] = m * acc;",
     "mask[t] != 0) ? 1.0 : 1.0;\n                y[t * H + h] = m * acc;"),
    ("row ranges cut the window at the range end", "#define GYM(i, j) ((i) >= S ? 0.0",
     "#define GYM(i, j) ((i) >= r1 ? 0.0"),
    ("row ranges shift the gradWeight tap", "GYM(i + W - 1 - k, j) * xd", "GYM(i + k, j) * xd"),
    ("row ranges read the mask untransposed", "mask[(j) * S + (i)]", "mask[(i) * B + (j)]"),
    ("row ranges overwrite the caller's sums", "if (gw_acc) gw_acc[k * H + h] += acc;",
     "if (gw_acc) gw_acc[k * H + h] = acc;"),
    ("encoder saturates on overflow",
     "if (field >= (double)inf_field) return (uint16_t)(sign | inf_field);",
     "if (field >= (double)inf_field) return (uint16_t)(sign | (inf_field - 1u));"),
]


def test_planted_mistakes_are_caught(tmp_path):
    src = open(os.path.join(os.path.dirname(HERE), "oracle", "mccb_oracle.c")).read()
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    missed = []
    for name, old, new in MUTANTS:
        assert src.count(old) >= 1, f"mutant '{name}' does not apply"
        msrc = tmp_path / f"m{len(name)}_{abs(hash(name)) % 10**6}.c"
        msrc.write_text(src.replace(old, new, 1))
        lib = oracle.build(str(msrc), str(msrc) + ".so")
        orc = oracle.Oracle(lib)
        failed = []
        for pin in PINS:
            try:
                pin(orc)
            except AssertionError:
                failed.append(pin.__name__)
        if not failed:
            missed.append(name)
    assert not missed, f"no pin catches: {missed}"
