"""The oracle against the hand-derived worked examples under tests/golden/ (their
headers give the derivation and the passages they follow) and against the
stored config-1 regression anchor."""

import os

import numpy as np

import synth  # noqa: F401
from oracle import codecs, fp8, nvfp4

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read(name):
    rows = {}
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            rows.setdefault(key, []).append(vals)
    return rows


def _bf16(vals):
    return codecs.f32_to_bf16_bits_rne(np.array([float(v) for v in vals], np.float32))


def test_nvfp4_hand_example():
    g = _read("nvfp4_hand_example.txt")
    w = np.stack([_bf16(r) for r in g["w"]])
    assert np.array_equal(codecs.bf16_bits_to_f32(w).astype(np.float64),
                          np.array([[float(v) for v in r] for r in g["w"]]))   # inputs exact in bf16
    codes, scales, S = nvfp4.quantize(w)
    assert S == np.float32(float(g["S"][0][0]))
    assert np.array_equal(scales, np.array([[int(v, 16) for v in r] for r in g["scales"]], np.uint8))
    want = np.array([[int(v) for v in r] for r in g["codes"]], np.uint8)
    assert np.array_equal(nvfp4.unpack_codes(codes), want)


def test_fp8_activation_hand_example():
    g = _read("fp8_act_hand_example.txt")
    vals = [float(v) for v in g["x"][0]]
    x = np.zeros((1, 128), np.float32)
    x[0, :len(vals)] = vals
    xb = codecs.f32_to_bf16_bits_rne(x)
    assert np.array_equal(codecs.bf16_bits_to_f32(xb), x)
    codes, s = fp8.quantize_act(xb)
    assert s[0, 0] == np.float32(float(g["s"][0][0]))
    want = [int(v, 16) for v in g["codes"][0]]
    assert list(codes[0, :len(want)]) == want
    assert (codes[0, len(want):] == 0).all()


def test_config1_regression_anchor():
    import importlib.util
    spec = importlib.util.spec_from_file_location("mk", os.path.join(GOLD, "make_config1_digest.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    with open(os.path.join(GOLD, "config1_digest.txt")) as f:
        assert mk.digest() == f.read()
