"""Planted mistakes in the oracle fail its pins.

Each case below changes one expression of oracle.c the way a plausible slip
would (eps outside the root, the sigmoid's sign, the filter's kh/kw index
order, a dropped channel, a shifted padding offset, the mean's sign, a lost
stride, a dropped beta, an off-by-one output extent), builds that copy, and
runs a battery of pins taken from test_oracle.py's families -- brute force on
tiny shapes, torch's CPU conv2d/batch_norm/silu in fp64, the BatchNorm
identity case and SiLU facts -- through it. Every planted mistake must fail at
least one pin, and the unaltered source must pass them all. The mistakes are
planted in the oracle, on the CPU; nothing here touches a GPU.
"""
import math

import numpy as np
import pytest

import oracle

from test_oracle import _brute_conv, _tiny_shapes

MUTATIONS = {
    "eps_outside_root": ("return gamma * (t - mean) / sqrt(var + eps) + beta;",
                         "return gamma * (t - mean) / (sqrt(var) + eps) + beta;"),
    "sigmoid_sign": ("double sig = 1.0 / (1.0 + exp(-v));", "double sig = 1.0 / (1.0 + exp(v));"),
    "kh_kw_swapped": ("((k * g->kh + r) * g->kw + s) * g->C_in",
                      "((k * g->kw + s) * g->kh + r) * g->C_in"),
    "dropped_channel": ("for (int c = 0; c < g->C_in; ++c)", "for (int c = 1; c < g->C_in; ++c)"),
    "shifted_padding": ("long long ih = p * g->stride - g->pad + r;",
                        "long long ih = p * g->stride - g->pad + r + (g->pad > 0);"),
    "mean_sign": ("return gamma * (t - mean) / sqrt(var + eps) + beta;",
                  "return gamma * (t + mean) / sqrt(var + eps) + beta;"),
    "stride_ignored_in_w": ("long long iw = q * g->stride - g->pad + s;",
                            "long long iw = q - g->pad + s;"),
    "beta_dropped": ("return gamma * (t - mean) / sqrt(var + eps) + beta;",
                     "return gamma * (t - mean) / sqrt(var + eps);"),
    "extent_off_by_one": ("return (in + 2 * pad - k) / stride + 1;",
                          "return (in + 2 * pad - k + 1) / stride + 1;"),
}


def _pin_brute_force():
    rng = np.random.default_rng(3)
    for shape in _tiny_shapes(24, 11):
        N, H, W, C_in, C_out, kh, kw, s, p = shape
        x = rng.standard_normal((N, H, W, C_in))
        w = rng.standard_normal((C_out, kh, kw, C_in))
        got = oracle.conv2d(x, w, s, p)
        ref = _brute_conv(x, w, s, p)
        assert got.shape == ref.shape, shape
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def _pin_torch():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(5)
    C = 5
    for (kh, kw, s, p) in [(3, 3, 1, 1), (3, 5, 2, 2), (1, 1, 1, 0)]:
        x = rng.standard_normal((2, 9, 8, 4))
        w = rng.standard_normal((C, kh, kw, 4))
        g, b = rng.uniform(0.5, 1.5, C), rng.standard_normal(C)
        m, v = rng.standard_normal(C), rng.uniform(0.5, 2.0, C)
        got = oracle.conv_bn_silu(x, w, g, b, m, v, 1e-3, s, p)
        t = F.conv2d(torch.from_numpy(x).permute(0, 3, 1, 2),
                     torch.from_numpy(w).permute(0, 3, 1, 2), stride=s, padding=p)
        t = F.batch_norm(t, torch.from_numpy(m), torch.from_numpy(v), torch.from_numpy(g),
                         torch.from_numpy(b), training=False, eps=1e-3)
        ref = F.silu(t).permute(0, 2, 3, 1).numpy()
        assert got.shape == ref.shape
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def _pin_bn_identity():
    rng = np.random.default_rng(2)
    t = rng.standard_normal((20, 4))
    var = rng.uniform(0.5, 2.0, 4)
    mean = rng.standard_normal(4)
    out = oracle.batchnorm(t, np.sqrt(var + 1e-5), mean, mean, var, 1e-5)
    np.testing.assert_allclose(out, t, rtol=0, atol=1e-13)


def _pin_silu():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    v = np.linspace(-10, 10, 201)
    np.testing.assert_allclose(oracle.silu(-v), oracle.silu(v) - v, rtol=0, atol=1e-13)
    from scipy.special import lambertw
    w1e = float(lambertw(1.0 / math.e).real)
    assert abs(oracle.silu(np.array([-1.0 - w1e]))[0] + w1e) < 1e-15


PINS = [_pin_brute_force, _pin_torch, _pin_bn_identity, _pin_silu]


def _failing_pins():
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError) as e:
            failed.append("%s: %s" % (pin.__name__, str(e).splitlines()[0] if str(e) else "fail"))
    return failed


def test_unaltered_oracle_passes_the_battery(tmp_path):
    with oracle.altered(oracle.source(), str(tmp_path)):
        assert _failing_pins() == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(tmp_path, name):
    old, new = MUTATIONS[name]
    src = oracle.source()
    assert src.count(old) == 1, "mutation site not found: %r" % old
    with oracle.altered(src.replace(old, new), str(tmp_path)):
        failed = _failing_pins()
    assert failed, "planted mistake %s passed every pin" % name
