"""The fp8 (OCP E4M3) input recipe shared by the fp8 attention tests: decoding and rounding of the codes are
pinned to the format's definition and to torch's float8_e4m3fn conversion (a different implementation)."""
import numpy as np
import pytest

import synthetic as syn


def test_e4m3_values_by_definition():
    v = syn.E4M3_VALUES
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x38] == 1.0 and v[0xB8] == -1.0          # exponent 7 = bias, mantissa 0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0      # largest finite: 2^8 * 1.75
    assert v[0x08] == 2.0 ** -6                         # smallest normal
    assert v[0x01] == 2.0 ** -9                         # smallest subnormal: 2^-6 * 1/8
    assert v[0x07] == 2.0 ** -6 * 7 / 8
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.sum(np.isnan(v)) == 2 and np.all(np.isfinite(v[~np.isnan(v)]))
    pos = v[:127]
    assert np.all(np.diff(pos) > 0)                     # codes 0..126 increase


def test_e4m3_matches_torch_float8():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    nan = np.isnan(tv)
    assert np.array_equal(nan, np.isnan(syn.E4M3_VALUES))
    assert np.array_equal(tv[~nan], syn.E4M3_VALUES[~nan])
    r = np.random.default_rng(0)
    x = np.clip(r.standard_normal(100000) * 60, -448, 448).astype(np.float32)
    mid = (syn.E4M3_VALUES[:126] + syn.E4M3_VALUES[1:127]) / 2  # exact ties between neighbouring codes
    x = np.concatenate([x, mid.astype(np.float32), -mid.astype(np.float32),
                        np.array([0.0, -0.0, 448.0, -448.0, 1e-12], np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(syn.fp8_e4m3_bits(x), ref)


def test_e4m3_rounding_saturates_and_ties_to_even():
    assert syn.fp8_e4m3_bits(np.array([1000.0, -1e9]))[0] == 0x7E
    assert syn.fp8_e4m3_bits(np.array([-1e9]))[0] == 0xFE
    # between 1.0 (0x38, even) and 1.125 (0x39): the midpoint goes to 1.0; between 1.125 and 1.25 to 1.25
    assert syn.fp8_e4m3_bits(np.array([1.0625]))[0] == 0x38
    assert syn.fp8_e4m3_bits(np.array([1.1875]))[0] == 0x3A
    assert syn.fp8_e4m3_bits(np.array([np.nan]))[0] == 0x7F


def test_fp8_inputs_dequantise_within_half_a_step():
    w = syn.scaled(syn.WORKLOADS["dense_1024"], B=2, H=3, N=200, T=64, tv=(20, 64), side=1)
    base = syn.attention_inputs(syn.scaled(w, dtype="f32"))
    f = syn.attention_inputs_fp8(w)
    for r in ("q", "k_img", "k_txt"):
        desc = f["q_descale"] if r == "q" else f["k_descale"]
        sc = desc.astype(np.float64)[:, :, None, None]
        assert np.array_equal(f[r], syn.E4M3_VALUES[f[r + "_fp8"]] * sc)
        # relative error of E4M3 is at most 2^-4 for normal values (3 mantissa bits)
        big = np.abs(base[r]) > 2.0 ** -6 * sc
        assert np.all(np.abs(f[r] - base[r])[big] <= 2.0 ** -4 * np.abs(base[r])[big] + 1e-30)
    # one factor per head for K: the largest |k| over image and text keys of each head maps to 448
    kall = np.concatenate([f["k_img_fp8"], f["k_txt_fp8"]], axis=2)
    assert np.all((kall & 0x7F).reshape(2, 3, -1).max(axis=2) == 0x7E)
