"""Pins for oracle/norm.py: RMSNorm of the residual stream and the BF16 rounding of its
output, against closed forms and library routines (torch's float64 rms_norm and its
BF16 cast)."""
import numpy as np
import torch

import synth
from oracle import norm as N
from oracle.formats import bf16_to_f64


def test_bf16_rounding_matches_torch_cast_and_ties_to_even():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.normal(size=20000) * np.exp(rng.normal(size=20000) * 8),
                        2.0 ** -130 * rng.normal(size=200)])            # BF16 subnormals
    want = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # torch rounds FP64 -> FP32 -> BF16; compare on values that are exact in FP32
    v32 = v.astype(np.float32).astype(np.float64)
    assert np.array_equal(N.to_bf16_bits(v32), want)
    # ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> the even mantissa (1.0);
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6 -> 1 + 2^-6
    t = N.to_bf16_bits(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)]))
    assert list(t) == [0x3F80, 0x3F82, 0xBF80]


def test_rms_norm_closed_forms():
    H = 64
    g = synth.to_bf16_bits(np.linspace(-2, 2, H))
    gv = bf16_to_f64(g)
    r = synth.to_bf16_bits(np.array([[3.0] * H, [-0.5] * H]))
    x = N.rms_norm(r, g, 0.0)                 # a constant row c: c / |c| * gamma
    assert np.array_equal(x[0], gv) and np.array_equal(x[1], -gv)
    eps = 0.25
    x = N.rms_norm(r, g, eps)                 # c / sqrt(c^2 + eps) * gamma
    assert np.allclose(x[0], 3.0 / np.sqrt(9.0 + eps) * gv, rtol=1e-15, atol=0)
    # one nonzero element v in a row of H: mean = v^2 / H
    r1 = np.zeros((1, H), np.uint16)
    r1[0, 5] = synth.to_bf16_bits(np.array([2.0]))[0]
    x = N.rms_norm(r1, g, 0.0)
    assert np.isclose(x[0, 5], np.sqrt(H) * gv[5], rtol=1e-15) and np.count_nonzero(x) == 1


def test_rms_norm_matches_torch_float64():
    rng = np.random.default_rng(5)
    r = synth.to_bf16_bits(rng.normal(size=(6, 512)) * 3)
    g = synth.to_bf16_bits(1 + 0.1 * rng.normal(size=512))
    eps = 1e-5
    want = torch.nn.functional.rms_norm(torch.from_numpy(bf16_to_f64(r)), (512,),
                                        weight=torch.from_numpy(bf16_to_f64(g)), eps=eps).numpy()
    assert np.allclose(N.rms_norm(r, g, eps), want, rtol=1e-14, atol=1e-15)


def test_residual_out_is_the_plain_sum():
    r = synth.to_bf16_bits(np.array([[1.5, -2.0, 0.0]]))
    y = np.array([[0.25, 1e-3, -7.0]])
    assert np.array_equal(N.residual_out(r, y), [[1.75, -2.0 + 1e-3, -7.0]])
