"""Pins of the oracle's FP8 (e4m3) decoding, which the FP8 forward's parity
rests on: FP8 attention is the oracle's attention on the decoded codes times
their descale factors, so a wrong decode would move the reference.

* hand-worked codes of the format's definition (tests/golden/e4m3_codes.json:
  subnormals, the smallest normal, the bias, the largest finite value, signs,
  NaN);
* all 256 codes against torch's float8_e4m3fn type (an independent
  implementation of the same format);
* e4m3 rounding of exactly representable fp32 values decodes back to them.
"""
import json
import math
import os

import numpy as np
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _value(s):
    if s == "NaN":
        return math.nan
    if s == "-0":
        return -0.0
    if "^" in s:
        coef, _, exp = s.partition("2^")
        c = float(coef.rstrip("*")) if coef else 1.0
        return c * 2.0 ** int(exp)
    return float(s)


def test_hand_worked_codes():
    d = json.load(open(os.path.join(HERE, "golden", "e4m3_codes.json")))
    codes = np.array([int(c["code"], 16) for c in d["codes"]], np.uint8)
    want = np.array([_value(c["value"]) for c in d["codes"]])
    got = oracle.e4m3_to_f64(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zero is kept
    assert math.copysign(1.0, got[1]) == -1.0


def test_all_codes_match_torch_float8():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.isnan(got).sum() == 2  # 0x7f and 0xff only


def test_round_trip_of_representable_values():
    vals = np.array([0.0, 1.0, -2.5, 0.015625, 448.0, -0.001953125, 96.0, 0.40625])
    codes = torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn)
    back = oracle.e4m3_to_f64(codes.view(torch.uint8).numpy())
    assert np.array_equal(back, vals)


def test_fp8_attention_reference_is_attention_on_decoded_values():
    """The FP8 reference used by the GPU tests: attention_fwd on
    decode(codes) * descale. Checked here against a plain numpy softmax of
    the same products (a different evaluation of the same definition)."""
    r = np.random.default_rng(3)
    x = [r.standard_normal((1, 9, 2, 8)).astype(np.float32) for _ in range(3)]
    codes, scales = [], []
    for t in x:
        s = float(np.abs(t).max()) / 384.0
        codes.append(torch.from_numpy(t / s).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
        scales.append(s)
    q, k, v = (oracle.e4m3_to_f64(c) * s for c, s in zip(codes, scales))
    for causal in (False, True):
        o, lse = oracle.attention_fwd(q, k, v, 0.3, causal)
        for h in range(2):
            sc = 0.3 * q[0, :, h] @ k[0, :, h].T
            if causal:
                sc = np.where(np.tril(np.ones((9, 9), bool)), sc, -np.inf)
            m = sc.max(1, keepdims=True)
            p = np.exp(sc - m)
            assert np.allclose(o[0, :, h], (p / p.sum(1, keepdims=True)) @ v[0, :, h],
                               atol=1e-13, rtol=0)
            assert np.allclose(lse[0, h], (m + np.log(p.sum(1, keepdims=True)))[:, 0],
                               atol=1e-13, rtol=0)


def _decoder_variant(bias=7, sub_exp=-6, nan=True, sign=True):
    """A copy of the decoder with one planted mistake (for the test below)."""
    def dec(codes):
        c = np.ascontiguousarray(codes).view(np.uint8).astype(np.int64)
        s = np.where(c >> 7, -1.0, 1.0) if sign else np.ones(c.shape)
        e = (c >> 3) & 15
        m = (c & 7).astype(np.float64)
        v = s * np.where(e == 0, (m / 8.0) * 2.0 ** sub_exp,
                         (1.0 + m / 8.0) * np.ldexp(1.0, (e - bias).astype(np.int64)))
        return np.where((e == 15) & (m == 7), np.nan, v) if nan else v
    return dec


def test_planted_decoder_mistakes_fail_the_golden_codes(monkeypatch):
    for kw in ({"bias": 8}, {"sub_exp": -7}, {"nan": False}, {"sign": False}):
        monkeypatch.setattr(oracle, "e4m3_to_f64", _decoder_variant(**kw))
        try:
            test_hand_worked_codes()
        except AssertionError:
            continue
        raise AssertionError("golden codes did not catch %s" % kw)
