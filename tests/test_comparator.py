"""The parity comparator (tests/harness.py, block_errors) on the CPU.

It must accept what a correct float32 kernel produces and reject small
systematic errors that the stated bar's absolute clause (4e-3 * max|y|) alone
would let through on a block with outlier channels: a dropped rank-16 patch of
sigma 0.02, and a phase whose angle delta * theta_j is formed as a float32
product.  Each "GPU" output here is an emulation in numpy float32 of the
arithmetic the kernels do, rounded to bfloat16 by the oracle's rounding of that
float32 value; the oracle's own outputs are the reference.
"""

from dataclasses import replace

import numpy as np
import pytest

from oracle import kamera_oracle as ko
from tests import harness as H
from workloads import SINGLE_FRAME, bits, make_inputs


@pytest.fixture(scope="module")
def block():
    # one (layer, key stream) block of the single-frame workload: 1024 tokens
    # x 512 features with 5% of the columns scaled by 8, rank 16, sigma 0.02,
    # and the largest shift of its range
    w = replace(SINGLE_FRAME, name="cmp", num_layers=1)
    inp = make_inputs(w, "cpu", seed=1234)
    lay, _ = H.layouts(w)
    x = bits(inp["src"][0][0, 0])
    u = bits(inp["u"][0][0, 0])
    v = bits(inp["v"][0][0, 0])
    delta = 8192
    want = ko.reuse_block_bits(x, delta, u, v, lay, rotate=True)
    y = ko.reuse_f64(ko.bf16_bits_to_f64(x), delta, ko.bf16_bits_to_f64(u), ko.bf16_bits_to_f64(v), lay,
                     rotate=True)
    return dict(lay=lay, x=x, u=u, v=v, delta=delta, want=want, y=y)


def emulate_f32(b, *, patch=True, phase="f64"):
    """R(delta) x + U V^T the way a float32 kernel computes it, rounded once
    from float32 to bfloat16.  phase="f64": the angle delta*theta_j in float64,
    then cos/sin rounded to float32; phase="f32": the angle as a float32
    product (the mistake the comparator must catch)."""
    lay = b["lay"]
    x = ko.bf16_bits_to_f64(b["x"]).astype(np.float32)
    ia, ib, j = ko.rope_pairs(lay)
    theta = np.power(np.float64(lay.rope_base), -2.0 * np.arange(lay.rope_dim // 2) / lay.rope_dim)
    if phase == "f64":
        phi = np.float64(b["delta"]) * theta
    else:
        phi = (np.float32(b["delta"]) * theta.astype(np.float32)).astype(np.float64)
    c = np.cos(phi).astype(np.float32)[j]
    s = np.sin(phi).astype(np.float32)[j]
    out = x.copy()
    a_, b_ = x[:, ia], x[:, ib]
    out[:, ia] = a_ * c - b_ * s
    out[:, ib] = b_ * c + a_ * s
    if patch:
        u = ko.bf16_bits_to_f64(b["u"]).astype(np.float32)
        v = ko.bf16_bits_to_f64(b["v"]).astype(np.float32)
        out = out + u @ v.T
    return ko.f64_to_bf16_bits(out.astype(np.float64))


def old_bar_passes(got, b):
    """The stated bar alone: 1 ulp or |gpu - y| <= 4e-3 * max|y| per element."""
    ulp = np.abs(H.ordinal(got) - H.ordinal(b["want"]))
    err = np.abs(ko.bf16_bits_to_f64(got) - b["y"])
    return bool(((ulp <= 1) | (err <= H.REL_TOL * np.max(np.abs(b["y"])))).all())


def test_accepts_a_correct_float32_kernel(block):
    got = emulate_f32(block)
    touched = np.ones(block["want"].shape[1], bool)
    assert H.block_errors(got, block["want"], block["y"], touched) == []
    assert H.block_errors(block["want"], block["want"], block["y"], touched) == []


def test_rejects_a_dropped_patch(block):
    got = emulate_f32(block, patch=False)
    touched = np.ones(block["want"].shape[1], bool)
    assert old_bar_passes(got, block), "the planted error should be one the stated bar alone misses"
    assert H.block_errors(got, block["want"], block["y"], touched)


@pytest.mark.parametrize("delta", [8192, -4096])
def test_rejects_a_float32_phase(block, delta):
    # the ends of the single-frame workload's shift range
    lay, x, u, v = block["lay"], block["x"], block["u"], block["v"]
    b = dict(block, delta=delta, want=ko.reuse_block_bits(x, delta, u, v, lay, rotate=True),
             y=ko.reuse_f64(ko.bf16_bits_to_f64(x), delta, ko.bf16_bits_to_f64(u), ko.bf16_bits_to_f64(v), lay,
                            rotate=True))
    touched = np.ones(b["want"].shape[1], bool)
    assert H.block_errors(emulate_f32(b), b["want"], b["y"], touched) == []
    got = emulate_f32(b, phase="f32")
    assert old_bar_passes(got, b), "the planted error should be one the stated bar alone misses"
    assert H.block_errors(got, b["want"], b["y"], touched)


def test_rejects_copied_columns_that_differ(block):
    got = block["want"].copy()
    touched = np.ones(block["want"].shape[1], bool)
    touched[:8] = False
    got[3, 2] ^= 1
    assert any("copied" in e for e in H.block_errors(got, block["want"], block["y"], touched))


def test_rejects_one_two_ulp_miss_on_a_large_value(block):
    want, y = block["want"], block["y"]
    touched = np.ones(want.shape[1], bool)
    k = np.unravel_index(np.argmax(np.abs(y)), y.shape)
    got = want.copy()
    # two steps up the monotone integer line of the value's magnitude
    got[k] = np.uint16(want[k] + 2) if (want[k] & 0x7FFF) < 0x7F7E else np.uint16(want[k] - 2)
    errs = H.block_errors(got, want, y, touched)
    assert any("2^-10" in e for e in errs), errs
