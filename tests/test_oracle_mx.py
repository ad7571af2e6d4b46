"""Pins of the oracle's MXFP8 codec (E4M3 elements, 32-element blocks, e8m0
block scales; MXFP8 support is named on the first page, section 三)."""
import os
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.slow
def test_e4m3_encoder_exhaustive(tmp_path):
    oracle.lib()
    exe = tmp_path / "mx_exhaustive"
    subprocess.run(["gcc", "-O2", "-fopenmp", os.path.join(HERE, "mx_exhaustive.c"), "-o", str(exe),
                    "-L", os.path.dirname(oracle.LIB_PATH), "-loracle", "-lm",
                    f"-Wl,-rpath,{os.path.dirname(oracle.LIB_PATH)}"], check=True)
    p = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "mismatches: 0" in p.stdout


def test_e4m3_table():
    v = oracle.e4m3_values()
    assert v[0x7e] == 448.0 and v[0xfe] == -448.0
    assert np.isnan(v[0x7f]) and np.isnan(v[0xff])
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[0x38] == 1.0
    pos = v[:0x7f]
    assert np.all(np.diff(pos) > 0)
    # every finite code round-trips
    for c in list(range(0x7f)) + list(range(0x80, 0xff)):
        got = oracle.e4m3_encode(v[c])
        assert got == c or (c == 0x80 and got == 0x80), (c, got)


def test_e4m3_rounding_and_saturation():
    enc = oracle.e4m3_encode
    assert enc(1.0 + 1 / 16) == 0x38  # halfway 1 and 1.125: to even (1.0)
    assert enc(1.0 + 3 / 16) == 0x3a  # halfway 1.125 and 1.25: to even (1.25)
    assert enc(460.0) == 0x7e and enc(1e30) == 0x7e and enc(float("inf")) == 0x7e
    assert enc(-1e30) == 0xfe
    assert enc(2.0 ** -10) == 0x00  # half of the smallest subnormal: to even (0)
    assert enc(1.5 * 2.0 ** -9) == 0x02  # halfway 1 and 2 units: to even (2)
    assert enc(-0.0) == 0x80
    assert enc(float("nan")) == 0x7f


def test_scale_rule():
    sc = oracle.mx_scale_code
    assert sc(0.0) == 0
    for amax in [1e-30, 3e-5, 0.02, 0.75, 1.0, 1.5, 448.0, 511.0, 1e30]:
        s = sc(amax) - 127
        # floor rule: 2^(s+8) <= amax < 2^(s+9)
        assert 2.0 ** (s + 8) <= amax < 2.0 ** (s + 9), (amax, s)


def test_quantize_rows_properties():
    rng = np.random.default_rng(0)
    a = rng.standard_normal((64, 128)).astype(np.float32) * np.float32(3.0)
    a[5, 32:64] = 0.0  # an all-zero block
    codes, scales = oracle.mx_quantize(a, axis=0)
    assert scales[5, 1] == 0 and not np.any(codes[5, 32:64] & 0x7f)
    deq = oracle.mx_dequantize_rows(codes, scales)
    for r in range(0, 64, 7):
        for b in range(4):
            blk = a[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            s = int(scales[r, b]) - 127
            assert 2.0 ** (s + 8) <= amax < 2.0 ** (s + 9)
            # round to nearest: error at most half a step of the binade, and
            # never more than the saturation loss
            err = np.abs(deq[r, 32 * b:32 * b + 32] - blk)
            step = np.ldexp(1.0, np.maximum(np.floor(np.log2(np.maximum(np.abs(blk), 1e-300))) - 3,
                                            -9 + s) .astype(np.int64))
            sat = np.maximum(np.abs(blk) - 448.0 * 2.0 ** s, 0)
            assert np.all(err <= np.maximum(step / 2, sat) * (1 + 1e-12))


def test_quantize_cols_groups_and_padding():
    rng = np.random.default_rng(1)
    offsets = np.array([0, 40, 40, 103, 135], dtype=np.int32)  # an empty group, ragged tails
    a = rng.standard_normal((135, 64)).astype(np.float32)
    codes, scales = oracle.mx_quantize(a, axis=1, offsets=offsets)
    assert scales.shape == (2 + 0 + 2 + 1, 64)
    # Blocks restart at each group: block 1 of group 0 covers rows 32..39 only.
    amax = np.abs(a[32:40]).max(axis=0)
    assert np.array_equal(scales[1], np.array([oracle.mx_scale_code(v) for v in amax]))
    # Same rows as a stand-alone matrix quantised row-wise after transposing
    # give the same codes (blocks are the same 32 values).
    seg = a[40:72]  # group 2, first block: rows 40..71
    c_t, s_t = oracle.mx_quantize(np.ascontiguousarray(seg.T), axis=0)
    assert np.array_equal(c_t.T, codes[40:72]) and np.array_equal(s_t[:, 0], scales[2])
    deq = oracle.mx_dequantize_cols(codes, scales, offsets)
    # half-step rounding (2^-4 relative) or, with the floor scale rule,
    # saturation of values in [448, 512) * 2^s (at most 1/8 relative)
    np.testing.assert_allclose(deq, a, rtol=0.125, atol=2.0 ** -10 * 2.0 ** (int(scales.max()) - 127))
    assert np.mean(np.abs(deq - a) <= 2.0 ** -4 * np.abs(a) + 1e-6) > 0.98
