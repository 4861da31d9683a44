"""C-ABI checks that need no GPU: the library loads, exports every function include/mccb.h
declares, validates arguments on the host (before any HIP call) with the error classes of the page's
return-code table, and plans tiles as a pure function of the shape.

Every call below that passes made-up pointer values is one that validation must reject; a call that
got past validation would reach a kernel launch, so each such call asserts a validation code.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import masked_depthwise_causal_amd as mdc
from masked_depthwise_causal_amd import build as mbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mccb.h")

BF16, FP16 = mdc.MCCB_BF16, mdc.MCCB_FP16
OK, NULLPTR, INVALID, SHAPE = mdc.MCCB_OK, mdc.MCCB_ERR_PARAM_NULLPTR, mdc.MCCB_ERR_PARAM_INVALID, \
    mdc.MCCB_ERR_SHAPE
VALIDATION_CODES = {NULLPTR, INVALID, SHAPE}

# Made-up, widely separated, 256-byte aligned "device addresses" (never dereferenced).
GB = 1 << 30
GY, X, W, M, GX, GW, WS = (0x7F0000000000 + k * 64 * GB for k in range(7))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mccb_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("mccb_get_workspace_size", "mccb_backward", "mccb_forward"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = mdc.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", mbuild.LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mccb_\w+)", out))
    assert set(declared_functions()) <= exported


def _ws(S, B, H, dt=BF16):
    return mdc.mccb_get_workspace_size(S, B, H, dt)


def call(gy=GY, x=X, w=W, m=M, gx=GX, gw=GW, S=64, B=2, H=384, dt=BF16, ws=WS, wsz=None,
         stream=None):
    if wsz is None:
        wsz = _ws(S, B, H, dt) if dt in (BF16, FP16) else 0
    rc = mdc.mccb_backward(gy, x, w, m, gx, gw, S, B, H, dt, ws, wsz, stream)
    assert rc in VALIDATION_CODES, f"call passed validation with fake pointers (rc={rc})"
    return rc


@pytest.mark.parametrize("which", ["gy", "x", "w", "gx", "gw"])
def test_null_required_pointer(which):
    assert call(**{which: None}) == NULLPTR


def test_null_workspace_when_required():
    assert call(ws=None) == NULLPTR


def test_null_size_out_pointer():
    rc = mdc.lib().mccb_get_workspace_size(64, 2, 384, BF16, None)
    assert rc == NULLPTR
    assert mdc.lib().mccb_get_plan(64, 2, 384, BF16, None) == NULLPTR


@pytest.mark.parametrize("dt", [-1, 2, 7])
def test_bad_dtype(dt):
    assert call(dt=dt, wsz=1 << 40) == INVALID
    out = ctypes.c_uint64(0)
    assert mdc.lib().mccb_get_workspace_size(64, 2, 384, dt, ctypes.byref(out)) == INVALID


@pytest.mark.parametrize("S,B,H", [
    (64, 0, 384), (64, 33, 384), (0, 2, 384), (-5, 2, 384), (524288, 2, 384), (16385, 32, 384),
    (64, 2, 320), (64, 2, 24640), (64, 2, 400), (64, 2, 448 + 32), (1, 1, 0), (2 ** 40, 1, 384)])
def test_shape_out_of_range(S, B, H):
    out = ctypes.c_uint64(0)
    assert mdc.lib().mccb_get_workspace_size(S, B, H, BF16, ctypes.byref(out)) == SHAPE
    assert call(S=S, B=B, H=H, wsz=1 << 40) == SHAPE


@pytest.mark.parametrize("S,B,H", [(1, 1, 384), (524288, 1, 384), (16384, 32, 5120),
                                   (262144, 2, 24576), (1, 32, 24576), (3, 7, 448)])
def test_shape_limits_accepted(S, B, H):
    # the limits themselves are valid (constraints section: B 1..32, B*S 1..512K, H 384..24576);
    # one strip of one batch needs no workspace (the fused kernel writes gradWeight itself)
    p = mdc.mccb_get_plan(S, B, H, BF16)
    assert (_ws(S, B, H) == 0) == (B == 1 and p["n_strips"] == 1)


def test_workspace_too_small():
    need = _ws(64, 2, 384)
    assert call(wsz=need - 1) == INVALID
    assert call(wsz=0) == INVALID


@pytest.mark.parametrize("which", ["gy", "x", "w", "gx", "gw", "ws"])
def test_misaligned_pointer(which):
    base = {"gy": GY, "x": X, "w": W, "gx": GX, "gw": GW, "ws": WS}[which]
    assert call(**{which: base + 8}) == INVALID


@pytest.mark.parametrize("case", [
    dict(gx=GY), dict(gx=X + 1024), dict(gx=W), dict(gw=GX + 256), dict(gw=X), dict(gw=W),
    dict(ws=GY + 4096), dict(ws=GX), dict(ws=GW), dict(gx=M - 512)])
def test_overlapping_buffers(case):
    assert call(**case) == INVALID


# -- mccb_backward_noalloc: same validation, no workspace, a fixed scratch limit -----------------
def ncall(gy=GY, x=X, w=W, m=M, gx=GX, gw=GW, S=64, B=2, H=384, dt=BF16, stream=None):
    rc = mdc.mccb_backward_noalloc(gy, x, w, m, gx, gw, S, B, H, dt, stream)
    assert rc in VALIDATION_CODES | {mdc.MCCB_ERR_SCRATCH_LIMIT}, \
        f"no-alloc call passed validation with fake pointers (rc={rc})"
    return rc


@pytest.mark.parametrize("which", ["gy", "x", "w", "gx", "gw"])
def test_noalloc_null_required_pointer(which):
    assert ncall(**{which: None}) == NULLPTR


@pytest.mark.parametrize("dt", [-1, 2])
def test_noalloc_bad_dtype(dt):
    assert ncall(dt=dt) == INVALID


@pytest.mark.parametrize("S,B,H", [(64, 0, 384), (64, 2, 320), (16385, 32, 384)])
def test_noalloc_shape_out_of_range(S, B, H):
    assert ncall(S=S, B=B, H=H) == SHAPE


@pytest.mark.parametrize("which", ["gy", "x", "w", "gx", "gw"])
def test_noalloc_misaligned_pointer(which):
    base = {"gy": GY, "x": X, "w": W, "gx": GX, "gw": GW}[which]
    assert ncall(**{which: base + 8}) == INVALID


@pytest.mark.parametrize("case", [dict(gx=GY), dict(gx=X + 1024), dict(gw=GX + 256),
                                  dict(gw=W), dict(gx=M - 512)])
def test_noalloc_overlapping_buffers(case):
    assert ncall(**case) == INVALID


def test_noalloc_scratch_limit():
    # the headline shape fits the fixed scratch; S=262144 B=2 H=24576 does not and is refused
    # before anything is enqueued (the limit is checked after the shape, before any HIP call)
    limit = mdc.MCCB_NOALLOC_SCRATCH_BYTES
    assert limit == 64 << 20
    assert re.search(r"#define\s+MCCB_NOALLOC_SCRATCH_BYTES\s+\(64ull << 20\)",
                     open(HEADER).read())
    assert _ws(16384, 32, 5120) <= limit
    assert _ws(262144, 2, 24576) > limit
    assert ncall(S=262144, B=2, H=24576) == mdc.MCCB_ERR_SCRATCH_LIMIT
    assert "SCRATCH" in mdc.mccb_status_string(mdc.MCCB_ERR_SCRATCH_LIMIT)


Y = GX  # the forward's output slot


def fcall(x=X, w=W, m=M, y=Y, S=64, B=2, H=384, dt=BF16, stream=None):
    rc = mdc.mccb_forward(x, w, m, y, S, B, H, dt, stream)
    assert rc in VALIDATION_CODES, f"forward call passed validation with fake pointers (rc={rc})"
    return rc


@pytest.mark.parametrize("which", ["x", "w", "y"])
def test_forward_null_required_pointer(which):
    assert fcall(**{which: None}) == NULLPTR


@pytest.mark.parametrize("dt", [-1, 2])
def test_forward_bad_dtype(dt):
    assert fcall(dt=dt) == INVALID


@pytest.mark.parametrize("S,B,H", [(64, 0, 384), (64, 33, 384), (0, 2, 384), (524288, 2, 384),
                                   (64, 2, 320), (64, 2, 24640), (64, 2, 400)])
def test_forward_shape_out_of_range(S, B, H):
    assert fcall(S=S, B=B, H=H) == SHAPE


@pytest.mark.parametrize("which", ["x", "w", "y"])
def test_forward_misaligned_pointer(which):
    base = {"x": X, "w": W, "y": Y}[which]
    assert fcall(**{which: base + 8}) == INVALID


@pytest.mark.parametrize("case", [dict(y=X), dict(y=X + 2048), dict(y=W - 256), dict(y=M - 512),
                                  dict(x=Y + 64 * 2 * 384 * 2 - 16)])
def test_forward_overlapping_buffers(case):
    assert fcall(**case) == INVALID


def test_plan_is_pure_and_consistent():
    for (S, B, H, dt) in [(64, 1, 384, BF16), (4096, 4, 4096, BF16), (8192, 8, 8192, FP16),
                          (16384, 32, 5120, BF16), (262144, 2, 24576, BF16), (1, 1, 384, FP16),
                          (1000, 3, 448, BF16)]:
        p1 = mdc.mccb_get_plan(S, B, H, dt)
        p2 = mdc.mccb_get_plan(S, B, H, dt)
        assert p1 == p2
        C = B * H
        if S <= 64:  # the tall layout: one strip, which one round of 8 ring waves covers
            assert p1["n_strips"] == 1 and p1["waves_per_block"] == 8
            assert p1["rows_per_round"] == 64 >= p1["rows_per_strip"]
        else:
            assert p1["rows_per_strip"] % p1["rows_per_round"] == 0
        assert p1["rows_per_round"] % p1["rows_per_turn"] == 0
        assert p1["n_strips"] == -(-S // p1["rows_per_strip"])
        assert p1["n_col_blocks"] == -(-C // p1["cols_per_block"])
        direct = B == 1 and p1["n_strips"] == 1  # gradWeight written by the fused kernel
        assert p1["workspace_size"] == (0 if direct else p1["n_strips"] * 3 * C * 8)
        assert p1["workspace_size"] == _ws(S, B, H, dt)
        # the plan does not depend on the dtype
        other = FP16 if dt == BF16 else BF16
        assert mdc.mccb_get_plan(S, B, H, other) == p1


def test_wide_layout_tiles_rows_an_odd_number_of_times():
    """The wide layouts (column groups 16 or 32 KiB apart) on every row length they cover: the
    block's super-chunk (groups x spacing) fits a whole, odd number of times in a row, preferring
    4 x 16 KiB, then 4 x 32 KiB, then 3 x 32 KiB; rows with no such tiling (a whole number of
    256 KiB, or none of the three) take 4 x 16 KiB. Contiguous launches; the plan reports them."""
    K = 1024
    seen = set()
    for C in range(32768, 786432 + 1, 4096):  # rows of 64 KiB .. 1.5 MiB, whole 8 KiB
        B = next(b for b in range(1, 33) if C % b == 0 and C // b <= 24576 and (C // b) % 64 == 0)
        p = mdc.mccb_get_plan(1024, B, C // B, BF16)
        L = 2 * C
        odd = [(g, sp) for g, sp in ((4, 16 * K), (4, 32 * K), (3, 32 * K))
               if L % (g * sp) == 0 and (L // (g * sp)) % 2 == 1]
        g, sp = odd[0] if odd else (4, 16 * K)
        assert (p["waves_per_block"], p["group_spacing"], p["cols_per_block"]) == (g, sp, 256 * g), \
            (C, B, p)
        assert p["n_col_blocks"] == -(-C // p["cols_per_block"])
        seen.add((g, sp, bool(odd)))
    assert seen == {(4, 16 * K, True), (4, 32 * K, True), (3, 32 * K, True), (4, 16 * K, False)}
    # the workloads' rows: 320 KiB -> 4 x 16, 128 KiB -> 4 x 32, 96 KiB -> 3 x 32; narrower rows
    # take a ring layout (adjacent groups)
    for (S, B, H, dt, sp, g) in [(16384, 32, 5120, BF16, 16 * K, 4), (8192, 8, 8192, FP16, 32 * K, 4),
                                 (262144, 2, 24576, BF16, 32 * K, 3), (4096, 4, 4096, BF16, 0, 4),
                                 (64, 1, 384, BF16, 0, 8)]:
        p = mdc.mccb_get_plan(S, B, H, dt)
        assert (p["group_spacing"], p["waves_per_block"]) == (sp, g), (S, B, H, p)


# Strips of the fused kernel are at most this many rows: the plan aims for strips of 1024 rows and
# the kernel's mask staging is sized for that bound (a whole number of 16-row rounds).
MAX_STRIP_ROWS = 1024


def test_plan_strip_bounds_over_many_shapes():
    rng = np.random.default_rng(11)
    shapes = [(S, B, 384) for S in (1, 2, 15, 16, 17, 127, 128, 129, 1023, 1024, 1025, 1040, 2047,
                                    2048, 2049, 4095, 4096, 4097, 16383, 16384) for B in (1, 32)]
    shapes += [(262144, 2, 24576), (524288, 1, 384), (16384, 32, 24576)]
    for _ in range(200):
        B = int(rng.integers(1, 33))
        S = int(rng.integers(1, 524288 // B + 1))
        shapes.append((S, B, 64 * int(rng.integers(6, 385))))
    for S, B, H in shapes:
        p = mdc.mccb_get_plan(S, B, H, BF16)
        T = p["rows_per_strip"]
        assert 1 <= T <= MAX_STRIP_ROWS, (S, B, H, T)
        assert T % 16 == 0 or T >= S, (S, B, H, T)
        assert p["n_strips"] == -(-S // T)
        # no more strips than 128-row strips would make (the floor on strip length)
        assert p["n_strips"] <= max(1, -(-S // 128)), (S, B, H, T)


def test_workspace_stays_small_at_the_headline_shape():
    # fp64 partials, written once and read once: below 1 % of the 16.1 GB streamed at
    # S=16384, B=32, H=5120, so at most 2 % extra traffic
    assert _ws(16384, 32, 5120) < 0.01 * 3 * 16384 * 32 * 5120 * 2


def test_status_strings():
    for code in (OK, NULLPTR, INVALID, SHAPE, mdc.MCCB_ERR_RUNTIME, 12345):
        s = mdc.mccb_status_string(code)
        assert isinstance(s, str) and s
    assert "NULLPTR" in mdc.mccb_status_string(NULLPTR)
    assert "SHAPE" in mdc.mccb_status_string(SHAPE)


def test_python_binding_raises_on_bad_shape():
    with pytest.raises(mdc.MccbError) as e:
        mdc.mccb_get_workspace_size(64, 2, 100, BF16)
    assert e.value.status == SHAPE


# -- strided inputs (mccb_*_ex) ------------------------------------------------------------------
def strides(S=64, B=2, H=384, gy=None, x=None, w=None, m=None):
    st = mdc.Strides()
    st.gradY[:] = gy or [B * H, H, 1]
    st.x[:] = x or [B * H, H, 1]
    st.weight[:] = w or [H, 1]
    st.mask[:] = m or [S, 1]
    return st


def xcall(gy=GY, x=X, w=W, m=M, gx=GX, gw=GW, S=64, B=2, H=384, taps=3, dt=BF16, st=None, ws=WS,
          wsz=1 << 40):
    rc = mdc.mccb_backward_ex(gy, x, w, m, gx, gw, S, B, H, taps, dt, st, ws, wsz, None)
    assert rc in VALIDATION_CODES, f"strided call passed validation with fake pointers (rc={rc})"
    return rc


def test_ex_null_strides_is_the_contiguous_layout():
    assert mdc.mccb_get_workspace_size_ex(GY, X, W, 64, 2, 384, 3, BF16, None) == _ws(64, 2, 384)
    assert mdc.mccb_get_workspace_size_ex(GY, X, W, 64, 2, 384, 3, BF16, strides()) == _ws(64, 2, 384)
    assert mdc.mccb_forward_get_workspace_size_ex(X, W, 64, 2, 384, 3, BF16, None) == 0


def test_ex_workspace_packs_only_what_cannot_be_read_in_place():
    S, B, H = 64, 2, 384
    base, nb = _ws(S, B, H), S * B * H * 2
    # [B,S,H] storage viewed as [S,B,H]: channels contiguous, strides even -> read in place
    perm = [H, S * H, 1]
    assert mdc.mccb_get_workspace_size_ex(GY, X, W, S, B, H, 3, BF16, strides(gy=perm, x=perm)) == base
    # channels strided -> gradY packed after the 256-aligned partials
    st = strides(gy=[B * H * 2, H * 2, 2])
    assert mdc.mccb_get_workspace_size_ex(GY, X, W, S, B, H, 3, BF16, st) == -(-base // 256) * 256 + nb
    # a base that is only 2-byte aligned cannot feed 4-byte lane loads -> x packed
    assert mdc.mccb_get_workspace_size_ex(GY, X + 2, W, S, B, H, 3, BF16, None) == \
        -(-base // 256) * 256 + nb
    # a transposed weight is packed (3*H elements)
    got = mdc.mccb_get_workspace_size_ex(GY, X, W, S, B, H, 3, BF16, strides(w=[1, 3]))
    assert got == -(-base // 256) * 256 + 3 * H * 2
    # forward: in place needs row/batch strides that are multiples of 8 and a 16-byte base
    assert mdc.mccb_forward_get_workspace_size_ex(X, W, S, B, H, 3, BF16, strides(x=perm)) == 0
    assert mdc.mccb_forward_get_workspace_size_ex(X + 8, W, S, B, H, 3, BF16, None) == nb
    assert mdc.mccb_forward_get_workspace_size_ex(X, W, S, B, H, 3, BF16,
                                                  strides(x=[B * H + 2, H, 1])) == nb


def test_ex_lane_width_decides_in_place_reads():
    """The in-place rule follows the fused kernel's lane width: 8 bytes on shapes with S > 64 and
    B*H at least 32768 and a multiple of 4096, 4 bytes elsewhere. Even strides and a 4-byte (not 8-byte)
    aligned base are read in place on a 4-byte-lane shape and packed on an 8-byte-lane shape."""
    for S, B, H, wide in [(128, 8, 4096, True), (128, 12, 4096, True), (64, 8, 4096, False),
                          (128, 3, 4096, False), (128, 7, 4672, False), (128, 7, 5120, False),
                          (128, 32, 1152, True)]:
        base, nb = _ws(S, B, H), S * B * H * 2
        packed = -(-base // 256) * 256 + nb
        gy4 = GY + 4  # 4-byte aligned, not 8
        got = mdc.mccb_get_workspace_size_ex(gy4, X, W, S, B, H, 3, BF16, None)
        assert got == (packed if wide else base), (S, B, H)
        # row and batch strides of 2 elements more than contiguous: multiples of 2, not of 4
        st = strides(S, B, H, gy=[B * (H + 2), H + 2, 1])
        got = mdc.mccb_get_workspace_size_ex(GY, X, W, S, B, H, 3, BF16, st)
        assert got == (packed if wide else base), (S, B, H)
        # W = 4 takes the same lanes (the workspace holds 4 taps of partials)
        base4 = mdc.mccb_get_workspace_size_ex(GY, X, W, S, B, H, 4, BF16, None)
        got = mdc.mccb_get_workspace_size_ex(gy4, X, W, S, B, H, 4, BF16, None)
        assert got == (-(-base4 // 256) * 256 + nb if wide else base4), (S, B, H)


@pytest.mark.parametrize("which", ["gy", "x", "w", "gx", "gw"])
def test_ex_null_required_pointer(which):
    assert xcall(**{which: None}) == NULLPTR


@pytest.mark.parametrize("field,idx", [("gradY", 0), ("gradY", 2), ("x", 1), ("weight", 0),
                                       ("mask", 1)])
def test_ex_negative_stride(field, idx):
    st = strides()
    getattr(st, field)[idx] = -1
    assert xcall(st=st) == INVALID
    if field != "mask":
        with pytest.raises(mdc.MccbError):
            mdc.mccb_get_workspace_size_ex(GY, X, W, 64, 2, 384, 3, BF16, st)


def test_ex_element_misaligned_input():
    assert xcall(x=X + 1) == INVALID
    assert xcall(gy=GY + 3) == INVALID
    assert xcall(w=W + 1) == INVALID


def test_ex_extent_overflow():
    assert xcall(st=strides(gy=[1 << 60, 384, 1])) == INVALID


def test_ex_outputs_must_not_overlap_strided_extents():
    S, B, H = 64, 2, 384
    # gradY stored [B,S,H]: its extent is the whole S*B*H block starting at GY
    perm = [H, S * H, 1]
    assert xcall(st=strides(gy=perm), gx=GY + S * H * 2) == INVALID
    # a transposed mask [S,B] spans S*B bytes from M
    assert xcall(st=strides(m=[1, B]), gw=M + 16) == INVALID
    assert xcall(ws=X + 1024) == INVALID


def test_ex_workspace_too_small():
    need = mdc.mccb_get_workspace_size_ex(GY, X, W, 64, 2, 384, 3, BF16, strides(gy=[768, 384, 2]))
    assert xcall(st=strides(gy=[768, 384, 2]), wsz=need - 1) == INVALID


def test_forward_ex_validation():
    def f(**kw):
        args = dict(x=X, w=W, m=M, y=GX, S=64, B=2, H=384, taps=3, dt=BF16, st=None, ws=WS,
                    wsz=1 << 40)
        args.update(kw)
        rc = mdc.mccb_forward_ex(args["x"], args["w"], args["m"], args["y"], args["S"], args["B"],
                                 args["H"], args["taps"], args["dt"], args["st"], args["ws"],
                                 args["wsz"], None)
        assert rc in VALIDATION_CODES, f"strided forward passed validation (rc={rc})"
        return rc
    assert f(x=None) == NULLPTR
    assert f(st=strides(x=[768, -384, 1])) == INVALID
    assert f(x=X + 1) == INVALID
    assert f(y=X) == INVALID
    assert f(y=GX + 8) == INVALID  # output stays 16-byte aligned
    assert f(x=X + 2, ws=None) == NULLPTR  # packing needed, no workspace
    assert f(S=0) == SHAPE
    assert f(taps=0) == SHAPE
    assert f(taps=5) == SHAPE


# -- window taps W (mccb_*_ex) ----------------------------------------------------------------
@pytest.mark.parametrize("taps", [0, -1, 5, 64])
def test_ex_taps_out_of_range(taps):
    assert xcall(taps=taps) == SHAPE
    with pytest.raises(mdc.MccbError) as e:
        mdc.mccb_get_workspace_size_ex(GY, X, W, 64, 2, 384, taps, BF16, None)
    assert e.value.status == SHAPE


@pytest.mark.parametrize("taps", [1, 2, 3, 4])
def test_ex_workspace_scales_with_taps(taps):
    # fp64 partials [n_strips][W][B*H]; the strips do not depend on W
    for (S, B, H) in [(64, 2, 384), (16384, 32, 5120), (262144, 2, 24576)]:
        p = mdc.mccb_get_plan(S, B, H, BF16)
        got = mdc.mccb_get_workspace_size_ex(GY, X, W, S, B, H, taps, BF16, None)
        assert got == p["n_strips"] * taps * B * H * 8


def test_ex_weight_extent_follows_taps():
    # a [4,H] weight reaches 4*H elements: an output placed right after 3*H of them overlaps
    H = 384
    assert xcall(taps=4, gw=W + 3 * H * 2 + 256 - (3 * H * 2) % 256) == INVALID
    assert xcall(taps=4, gx=W + 3 * H * 2) == INVALID


# -- packed variable-length layout (mccb_varlen_*) --------------------------------------------------
CU = 0x7F0000000000 + 7 * 64 * GB


def vcall(gy=GY, x=X, w=W, m=M, cu=CU, gx=GX, gw=GW, T=100, nseq=3, H=384, taps=3, dt=BF16, ws=WS,
          wsz=1 << 40):
    rc = mdc.mccb_varlen_backward(gy, x, w, m, cu, gx, gw, T, nseq, H, taps, dt, ws, wsz, None)
    assert rc in VALIDATION_CODES, f"varlen call passed validation with fake pointers (rc={rc})"
    return rc


def test_varlen_workspace_sizes():
    T, H = 1000, 384
    p = mdc.mccb_get_plan(T, 1, H, BF16)
    got = mdc.mccb_varlen_get_workspace_size(T, 4, H, 3, BF16)
    assert got == -(-p["workspace_size"] // 256) * 256 + T  # partials, then one byte per token
    assert mdc.mccb_varlen_forward_get_workspace_size(T, 4, H, 2, BF16) == -(-T // 256) * 256 + T


@pytest.mark.parametrize("which", ["gy", "x", "w", "cu", "gx", "gw", "ws"])
def test_varlen_null_pointer(which):
    assert vcall(**{which: None}) == NULLPTR


@pytest.mark.parametrize("kw", [dict(T=0), dict(T=524289), dict(nseq=0), dict(H=320), dict(taps=5),
                                dict(taps=0)])
def test_varlen_shape_out_of_range(kw):
    assert vcall(**kw) == SHAPE


def test_varlen_validation():
    assert vcall(dt=2) == INVALID
    assert vcall(cu=CU + 4) == INVALID  # int64 array must be 8-byte aligned
    assert vcall(x=X + 8) == INVALID
    need = mdc.mccb_varlen_get_workspace_size(100, 3, 384, 3, BF16)
    assert vcall(wsz=need - 1) == INVALID
    assert vcall(gx=CU - 64) == INVALID  # gradX overlapping cu_seqlens
    assert vcall(ws=X + 4096) == INVALID
    rc = mdc.mccb_varlen_forward(X, W, M, CU, X + 4096, 100, 3, 384, 3, BF16, WS, 1 << 40, None)
    assert rc == INVALID  # y overlapping x
    rc = mdc.mccb_varlen_forward(X, W, M, None, GX, 100, 3, 384, 3, BF16, WS, 1 << 40, None)
    assert rc == NULLPTR


def test_binding_passes_workspace_bytes_of_any_dtype():
    """The binding hands the library the workspace's size in bytes (numel * element size), and
    refuses a non-contiguous workspace or one on another device."""
    import torch

    cpu = torch.device("cpu")
    assert mdc._ws_bytes(torch.empty(10, dtype=torch.uint8), cpu) == 10
    assert mdc._ws_bytes(torch.empty(10, dtype=torch.float32), cpu) == 40
    with pytest.raises(ValueError):
        mdc._ws_bytes(torch.empty(20, dtype=torch.uint8)[::2], cpu)
    with pytest.raises(ValueError):
        mdc._ws_bytes(torch.empty(10, dtype=torch.uint8), torch.device("meta"))
