"""Pins for the fp64 CPU oracle, against things other than the oracle itself.

Each pin is chosen so a plausible slip in the oracle (a dropped tap or
channel, a flipped kernel, a swapped kh/kw, asymmetric padding, eps outside
the root, a wrong sign in the sigmoid) fails at least one test:
  * brute force on tiny shapes with an explicitly padded copy and a different
    loop nest (channels outermost, math.fsum);
  * closed forms (all-ones inputs count in-bounds taps; one-hot inputs read
    the filter back in place; a centred delta filter is the identity);
  * library routines for special cases (1x1 conv is a matmul; torch's CPU
    conv2d / batch_norm / silu in fp64);
  * linearity, the BatchNorm fold identity, the BatchNorm identity case;
  * SiLU facts: SiLU(0) = 0, SiLU(-v) = SiLU(v) - v, and its minimum
    -W(1/e) at v = -1 - W(1/e) (W = Lambert W).
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from conv2d_batchnorm_silu_amd.inputs import WORKLOADS, make_inputs


def _rand(rng, shape):
    return rng.standard_normal(shape)


def _brute_conv(x, w, stride, pad):
    """Reference written independently: pad x with zeros explicitly, then loop
    output channel outermost and sum every window with math.fsum."""
    N, H, W, C = x.shape
    K, kh, kw, _ = w.shape
    xp = np.zeros((N, H + 2 * pad, W + 2 * pad, C))
    xp[:, pad:pad + H, pad:pad + W, :] = x
    P = (H + 2 * pad - kh) // stride + 1
    Q = (W + 2 * pad - kw) // stride + 1
    out = np.zeros((N, P, Q, K))
    for k in range(K):
        for n in range(N):
            for p in range(P):
                for q in range(Q):
                    win = xp[n, p * stride:p * stride + kh, q * stride:q * stride + kw, :]
                    out[n, p, q, k] = math.fsum((win * w[k]).ravel().tolist())
    return out


def _tiny_shapes(count, seed):
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < count:
        kh = int(rng.choice([1, 2, 3, 5]))
        kw = int(rng.choice([1, 2, 3, 5]))
        s = int(rng.choice([1, 2, 3]))
        p = int(rng.choice([0, 1, 2]))
        H, W = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        if H + 2 * p < kh or W + 2 * p < kw:
            continue
        shapes.append((int(rng.integers(1, 3)), H, W, int(rng.integers(1, 6)),
                       int(rng.integers(1, 6)), kh, kw, s, p))
    return shapes


@pytest.mark.parametrize("shape", _tiny_shapes(160, 7))
def test_conv_matches_brute_force(shape):
    N, H, W, C_in, C_out, kh, kw, s, p = shape
    rng = np.random.default_rng(hash(shape) & 0xFFFF)
    x = _rand(rng, (N, H, W, C_in))
    w = _rand(rng, (C_out, kh, kw, C_in))
    got = oracle.conv2d(x, w, s, p, threads=2)
    ref = _brute_conv(x, w, s, p)
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def _taps_in_bounds(o, stride, pad, k, n_in):
    return sum(1 for r in range(k) if 0 <= o * stride - pad + r < n_in)


@pytest.mark.parametrize("name", ["tiny_f32_3x3", "stem3x3s2_k16", "conv7x7_c64_k64"])
def test_conv_all_ones_counts_taps(name):
    wl = WORKLOADS[name]
    # Small batch, full spatial geometry of the workload.
    H, W, C = wl.H, wl.W, min(wl.C_in, 4)
    x = np.ones((1, H, W, C))
    w = np.ones((2, wl.kh, wl.kw, C))
    got = oracle.conv2d(x, w, wl.stride, wl.pad)
    assert got.shape == (1, wl.P, wl.Q, 2)
    for p in range(wl.P):
        rows = _taps_in_bounds(p, wl.stride, wl.pad, wl.kh, H)
        for q in range(wl.Q):
            cols = _taps_in_bounds(q, wl.stride, wl.pad, wl.kw, W)
            assert got[0, p, q, 0] == got[0, p, q, 1] == C * rows * cols


def test_conv_all_ones_known_values():
    # 224x224 RGB, 3x3, stride 2, pad 1: corner window holds 2x2 taps, interior 3x3.
    got = oracle.conv2d(np.ones((1, 224, 224, 3)), np.ones((1, 3, 3, 3)), 2, 1)
    assert got[0, 0, 0, 0] == 12 and got[0, 5, 7, 0] == 27 and got[0, 111, 111, 0] == 27
    # 56x56x64, 7x7, pad 3: corner 4x4 taps, interior 7x7.
    got = oracle.conv2d(np.ones((1, 56, 56, 64)), np.ones((1, 7, 7, 64)), 1, 3)
    assert got[0, 0, 0, 0] == 1024 and got[0, 20, 20, 0] == 64 * 49 and got[0, 55, 0, 0] == 1024


@pytest.mark.parametrize("kh,kw,s,p", [(3, 3, 1, 1), (2, 3, 2, 1), (5, 1, 1, 2), (3, 5, 3, 2)])
def test_conv_one_hot_reads_filter_in_place(kh, kw, s, p):
    rng = np.random.default_rng(11)
    N, H, W, C_in, C_out = 2, 7, 8, 3, 4
    w = _rand(rng, (C_out, kh, kw, C_in))
    n0, h0, w0, c0 = 1, 4, 3, 2
    x = np.zeros((N, H, W, C_in))
    x[n0, h0, w0, c0] = 1.0
    got = oracle.conv2d(x, w, s, p)
    P, Q = got.shape[1:3]
    for n, pp, qq, k in itertools.product(range(N), range(P), range(Q), range(C_out)):
        r, t = h0 - pp * s + p, w0 - qq * s + p
        want = w[k, r, t, c0] if (n == n0 and 0 <= r < kh and 0 <= t < kw) else 0.0
        assert got[n, pp, qq, k] == want


def test_conv_centred_delta_is_identity():
    rng = np.random.default_rng(3)
    C = 5
    x = _rand(rng, (2, 9, 6, C))
    w = np.zeros((C, 3, 3, C))
    for c in range(C):
        w[c, 1, 1, c] = 1.0
    np.testing.assert_array_equal(oracle.conv2d(x, w, 1, 1), x)


@pytest.mark.parametrize("C_in,C_out", [(64, 256), (3, 16), (17, 33)])
def test_conv_1x1_is_matmul(C_in, C_out):
    rng = np.random.default_rng(C_in)
    x = _rand(rng, (3, 5, 7, C_in))
    w = _rand(rng, (C_out, 1, 1, C_in))
    got = oracle.conv2d(x, w, 1, 0)
    ref = (x.reshape(-1, C_in) @ w.reshape(C_out, C_in).T).reshape(3, 5, 7, C_out)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_conv_linearity():
    rng = np.random.default_rng(5)
    x1, x2 = _rand(rng, (2, 6, 7, 4)), _rand(rng, (2, 6, 7, 4))
    w1, w2 = _rand(rng, (3, 3, 3, 4)), _rand(rng, (3, 3, 3, 4))
    a, b = 0.75, -1.5
    lhs = oracle.conv2d(a * x1 + b * x2, w1, 2, 1)
    rhs = a * oracle.conv2d(x1, w1, 2, 1) + b * oracle.conv2d(x2, w1, 2, 1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    lhs = oracle.conv2d(x1, a * w1 + b * w2, 2, 1)
    rhs = a * oracle.conv2d(x1, w1, 2, 1) + b * oracle.conv2d(x1, w2, 2, 1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_against_torch_cpu_fp64():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    for name in ["tiny_f32_3x3"]:
        wl = WORKLOADS[name]
        d = make_inputs(wl)
        got = oracle.conv_bn_silu(d["x"], d["w"], d["gamma"], d["beta"], d["mean"], d["var"],
                                  float(d["eps"]), wl.stride, wl.pad)
        xt = torch.from_numpy(d["x"].astype(np.float64)).permute(0, 3, 1, 2)
        wt = torch.from_numpy(d["w"].astype(np.float64)).permute(0, 3, 1, 2)
        t = F.conv2d(xt, wt, stride=wl.stride, padding=wl.pad)
        t = F.batch_norm(t, torch.from_numpy(d["mean"].astype(np.float64)),
                         torch.from_numpy(d["var"].astype(np.float64)),
                         torch.from_numpy(d["gamma"].astype(np.float64)),
                         torch.from_numpy(d["beta"].astype(np.float64)),
                         training=False, eps=float(d["eps"]))
        ref = F.silu(t).permute(0, 2, 3, 1).numpy()
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # Non-square windows and strides, fp64 random data.
    rng = np.random.default_rng(9)
    for (kh, kw, s, p) in [(3, 5, 2, 2), (7, 7, 1, 3), (1, 1, 2, 0)]:
        x = _rand(rng, (2, 11, 10, 6))
        w = _rand(rng, (5, kh, kw, 6))
        ref = F.conv2d(torch.from_numpy(x).permute(0, 3, 1, 2),
                       torch.from_numpy(w).permute(0, 3, 1, 2), stride=s, padding=p)
        np.testing.assert_allclose(oracle.conv2d(x, w, s, p), ref.permute(0, 2, 3, 1).numpy(),
                                   rtol=1e-12, atol=1e-12)


def test_batchnorm_identity_case():
    rng = np.random.default_rng(2)
    t = _rand(rng, (50, 6))
    var = rng.uniform(0.5, 2.0, 6)
    mean = _rand(rng, 6)
    eps = 1e-5
    gamma = np.sqrt(var + eps)
    out = oracle.batchnorm(t, gamma, mean, mean, var, eps)
    np.testing.assert_allclose(out, t, rtol=0, atol=4e-15 * (1 + np.abs(t).max() + np.abs(mean).max()))


def test_batchnorm_fold_identity():
    """The per-channel fold scale = gamma/sqrt(var+eps), bias = beta - mean*scale
    gives the same values as the unfolded form (to fp64 rounding)."""
    rng = np.random.default_rng(4)
    C = 9
    t = _rand(rng, (40, C)) * 3
    gamma, beta = rng.uniform(0.5, 1.5, C), _rand(rng, C)
    mean, var = _rand(rng, C), rng.uniform(0.5, 2.0, C)
    eps = 1e-5
    scale = gamma / np.sqrt(var + eps)
    bias = beta - mean * scale
    np.testing.assert_allclose(oracle.batchnorm(t, gamma, beta, mean, var, eps), t * scale + bias,
                               rtol=1e-13, atol=1e-13)


def test_batchnorm_against_torch():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(6)
    t = _rand(rng, (3, 4, 5, 7))
    g, b, m, v = rng.uniform(0.5, 1.5, 7), _rand(rng, 7), _rand(rng, 7), rng.uniform(0.5, 2, 7)
    ref = F.batch_norm(torch.from_numpy(t).permute(0, 3, 1, 2), torch.from_numpy(m),
                       torch.from_numpy(v), torch.from_numpy(g), torch.from_numpy(b),
                       training=False, eps=1e-3).permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(oracle.batchnorm(t, g, b, m, v, 1e-3), ref, rtol=1e-13, atol=1e-13)


def test_silu_facts():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    v = np.linspace(-30, 30, 6001)
    s = oracle.silu(v)
    np.testing.assert_allclose(oracle.silu(-v), s - v, rtol=0, atol=1e-13)
    from scipy.special import lambertw
    w1e = float(lambertw(1.0 / math.e).real)
    vmin = -1.0 - w1e
    smin = oracle.silu(np.array([vmin]))[0]
    assert abs(smin - (-w1e)) < 1e-15
    assert s.min() >= smin - 1e-15
    big = np.array([40.0, 100.0, 700.0])
    np.testing.assert_allclose(oracle.silu(big) / big, 1.0, rtol=1e-15)
    neg = oracle.silu(np.array([-800.0, -1e4]))
    assert np.all(neg == 0.0) and not np.any(np.isnan(neg))
    # Logistic form, checked against torch in fp64.
    torch = pytest.importorskip("torch")
    ref = torch.nn.functional.silu(torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(s, ref, rtol=1e-14, atol=1e-15)


def test_fused_equals_composition_and_sampling():
    wl = WORKLOADS["tiny_f32_3x3"]
    d = make_inputs(wl)
    args = (d["gamma"], d["beta"], d["mean"], d["var"], float(d["eps"]))
    fused = oracle.conv_bn_silu(d["x"], d["w"], *args, wl.stride, wl.pad)
    comp = oracle.silu(oracle.batchnorm(oracle.conv2d(d["x"], d["w"], wl.stride, wl.pad), *args))
    np.testing.assert_array_equal(fused, comp)
    idx = np.array([0, 1, 17, 255, 1000, fused.size - 1])
    np.testing.assert_array_equal(
        oracle.conv_bn_silu_at(d["x"], d["w"], *args, wl.stride, wl.pad, idx), fused.ravel()[idx])


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(8)
    x = _rand(rng, (3, 13, 11, 5))
    w = _rand(rng, (6, 3, 3, 5))
    outs = [oracle.conv2d(x, w, 1, 1, threads=t) for t in (1, 2, 3, 8)]
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


def test_out_extent_of_workloads():
    want = {"tiny_f32_3x3": 16, "conv1x1_c64_k256": 56, "conv3x3_c128_k128": 28,
            "stem3x3s2_k16": 112, "stem3x3s2_k24": 112, "conv7x7_c64_k64": 56}
    for name, P in want.items():
        wl = WORKLOADS[name]
        assert oracle.out_extent(wl.H, wl.kh, wl.stride, wl.pad) == P == wl.P
    assert oracle.out_extent(2, 5, 1, 1) == 0
    assert oracle.out_extent(2, 5, 1, 2) == 2


def test_rejects_bad_geometry():
    with pytest.raises(ValueError):
        oracle.conv2d(np.zeros((1, 2, 2, 1)), np.zeros((1, 5, 5, 1)), 1, 0)
    with pytest.raises(ValueError):
        oracle.conv2d(np.zeros((1, 4, 4, 2)), np.zeros((1, 3, 3, 3)), 1, 0)


# ---- training-mode batch norm (batch statistics) ----

def _train_case(seed, shape=(3, 9, 7, 5), C_out=6, k=3, stride=1, pad=1, shift=0.0):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=shape) + shift
    w = rng.normal(size=(C_out, k, k, shape[3])) / np.sqrt(k * k * shape[3])
    gamma = rng.uniform(0.5, 1.5, C_out)
    beta = rng.normal(0.0, 0.3, C_out)
    rm = rng.normal(0.0, 0.3, C_out)
    rv = rng.uniform(0.5, 2.0, C_out)
    return x, w, gamma, beta, rm, rv, stride, pad


def test_train_matches_torch_batch_norm():
    """torch CPU fp64 conv2d + batch_norm(training=True) + silu, including the
    running-estimate update (a library cross-check of every output)."""
    import torch
    import torch.nn.functional as F
    for seed, (stride, pad, mom) in enumerate([(1, 1, 0.1), (2, 0, 0.3), (1, 2, 1.0)]):
        x, w, g, b, rm, rv, _, _ = _train_case(40 + seed, stride=stride, pad=pad)
        eps = 1e-5
        got = oracle.conv_bn_silu_train(x, w, g, b, eps, stride, pad, rm, rv, mom)
        xt = torch.from_numpy(x).permute(0, 3, 1, 2)
        wt = torch.from_numpy(w).permute(0, 3, 1, 2)
        t = F.conv2d(xt, wt, stride=stride, padding=pad)
        rmt, rvt = torch.from_numpy(rm.copy()), torch.from_numpy(rv.copy())
        bn = F.batch_norm(t, rmt, rvt, torch.from_numpy(g), torch.from_numpy(b), training=True,
                          momentum=mom, eps=eps)
        ref = F.silu(bn).permute(0, 2, 3, 1).numpy()
        np.testing.assert_allclose(got["y"], ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got["running_mean"], rmt.numpy(), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(got["running_var"], rvt.numpy(), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(got["mean"], t.mean(dim=(0, 2, 3)).numpy(), rtol=1e-12,
                                   atol=1e-14)
        np.testing.assert_allclose(got["var"], t.var(dim=(0, 2, 3), unbiased=False).numpy(),
                                   rtol=1e-12, atol=1e-14)


def test_train_normalises_each_channel():
    """gamma = 1, beta = 0: before SiLU every channel has mean 0 and variance
    var/(var + eps) over the batch (the defining property of the transform);
    undoing SiLU is not needed -- the stage entries give the pre-SiLU values."""
    x, w, _, _, _, _, s, p = _train_case(50, shift=3.0)
    C = w.shape[0]
    got = oracle.conv_bn_silu_train(x, w, np.ones(C), np.zeros(C), 1e-5, s, p)
    t = oracle.conv2d(x, w, s, p)
    z = oracle.batchnorm(t, np.ones(C), np.zeros(C), got["mean"], got["var"], 1e-5).reshape(-1, C)
    np.testing.assert_allclose(z.mean(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(z.var(axis=0), got["var"] / (got["var"] + 1e-5), rtol=1e-10)
    np.testing.assert_array_equal(got["y"], oracle.silu(z.reshape(t.shape)))


def test_train_constant_channel_gives_beta():
    """A channel whose conv output is the same everywhere has variance 0, so
    its normalised value is 0 and the output is silu(beta) exactly."""
    x = np.ones((2, 4, 4, 3))
    w = np.ones((2, 1, 1, 3))
    w[1] *= -0.5
    beta = np.array([0.25, -1.5])
    got = oracle.conv_bn_silu_train(x, w, np.array([1.3, 0.7]), beta, 1e-5, 1, 0)
    np.testing.assert_array_equal(got["var"], 0.0)
    np.testing.assert_array_equal(got["y"][..., 0], oracle.silu(np.full((2, 4, 4), 0.25)))
    np.testing.assert_array_equal(got["y"][..., 1], oracle.silu(np.full((2, 4, 4), -1.5)))


def test_train_needs_two_values_per_channel():
    with pytest.raises(ValueError):
        oracle.conv_bn_silu_train(np.ones((1, 1, 1, 2)), np.ones((3, 1, 1, 2)), np.ones(3),
                                  np.zeros(3), 1e-5, 1, 0)


def test_train_with_batch_stats_equals_inference_path():
    """Feeding the batch statistics to the inference path reproduces the
    training output bit for bit (same stages, same order)."""
    x, w, g, b, _, _, s, p = _train_case(51)
    got = oracle.conv_bn_silu_train(x, w, g, b, 1e-5, s, p)
    inf = oracle.conv_bn_silu(x, w, g, b, got["mean"], got["var"], 1e-5, s, p)
    np.testing.assert_array_equal(got["y"], inf)


# ---- other epilogue activations ----

def test_gelu_pins():
    """GELU(v) = v * Phi(v): zero at zero, GELU(v) - GELU(-v) = v (since
    Phi(v) + Phi(-v) = 1), Phi(1) and Phi(-3) from scipy's normal CDF, the
    limits, and torch's exact GELU."""
    import torch
    from scipy.stats import norm
    assert oracle.gelu(np.array([0.0]))[0] == 0.0
    v = np.linspace(-8, 8, 1601)
    np.testing.assert_allclose(oracle.gelu(v) - oracle.gelu(-v), v, rtol=0, atol=1e-14)
    np.testing.assert_allclose(oracle.gelu(np.array([1.0, -3.0])),
                               [norm.cdf(1.0), -3.0 * norm.cdf(-3.0)], rtol=1e-14)
    assert abs(oracle.gelu(np.array([12.0]))[0] - 12.0) < 1e-15
    assert abs(oracle.gelu(np.array([-12.0]))[0]) < 1e-30
    ref = torch.nn.functional.gelu(torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(oracle.gelu(v), ref, rtol=1e-14, atol=1e-15)


def test_relu_pins():
    import torch
    v = np.random.default_rng(3).normal(size=1000) * 3
    np.testing.assert_array_equal(oracle.relu(v) - oracle.relu(-v), v)
    assert (oracle.relu(v)[v < 0] == 0).all()
    np.testing.assert_array_equal(oracle.relu(v), torch.relu(torch.from_numpy(v)).numpy())


def test_conv_bn_act_matches_torch_and_silu_path():
    """conv_bn_act against torch CPU fp64 conv2d + batch_norm + relu / gelu /
    nothing; with silu it is the fused oracle bit for bit."""
    import torch
    import torch.nn.functional as F
    wl = WORKLOADS["tiny_f32_3x3"]
    d = make_inputs(wl)
    args = (d["gamma"], d["beta"], d["mean"], d["var"], float(d["eps"]), wl.stride, wl.pad)
    xt = torch.from_numpy(d["x"].astype(np.float64)).permute(0, 3, 1, 2)
    wt = torch.from_numpy(d["w"].astype(np.float64)).permute(0, 3, 1, 2)
    bn = F.batch_norm(F.conv2d(xt, wt, stride=wl.stride, padding=wl.pad),
                      *(torch.from_numpy(d[k].astype(np.float64)) for k in ("mean", "var")),
                      torch.from_numpy(d["gamma"].astype(np.float64)),
                      torch.from_numpy(d["beta"].astype(np.float64)), training=False,
                      eps=float(d["eps"]))
    for act, fn in (("relu", F.relu), ("gelu", F.gelu), ("none", lambda t: t)):
        ref = fn(bn).permute(0, 2, 3, 1).numpy()
        np.testing.assert_allclose(oracle.conv_bn_act(d["x"], d["w"], *args, act), ref,
                                   rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(oracle.conv_bn_act(d["x"], d["w"], *args, "silu"),
                                  oracle.conv_bn_silu(d["x"], d["w"], *args))


def test_conv_bn_act_at_matches_full():
    for name in ("tiny_f32_3x3", "stem3x3s2_k16"):
        wl = WORKLOADS[name].scaled(N=1, H=9, W=11) if name != "tiny_f32_3x3" else WORKLOADS[name]
        d = make_inputs(wl)
        args = (d["gamma"], d["beta"], d["mean"], d["var"], float(d["eps"]), wl.stride, wl.pad)
        for act in ("relu", "gelu", "none", "silu"):
            full = oracle.conv_bn_act(d["x"], d["w"], *args, act)
            idx = np.random.default_rng(1).integers(0, full.size, 300)
            np.testing.assert_allclose(oracle.conv_bn_act_at(d["x"], d["w"], *args, act, idx),
                                       full.ravel()[idx], rtol=1e-13, atol=1e-14)


def test_fp8_e4m3_rounding():
    """Hand-worked values (0.3 -> 5/16, a tie 3*2^-10 -> 2^-8, subnormals,
    the largest finite 448, 464 the tie above it) and torch's float8_e4m3fn
    cast on a dense sweep of values."""
    import torch
    got = oracle.round_fp8_e4m3(np.array([1.0, 0.3, -3.3, 2**-9, 3 * 2**-10, 2**-10, 448.0,
                                           0.0, 17.0, 19.0]))
    np.testing.assert_array_equal(got, [1.0, 0.3125, -3.25, 2**-9, 2**-8, 0.0, 448.0, 0.0, 16.0,
                                        20.0])
    assert np.isnan(oracle.round_fp8_e4m3(np.array([470.0]))[0])
    v = np.concatenate([np.linspace(-440, 440, 20001), np.linspace(-0.05, 0.05, 4001),
                        np.random.default_rng(5).normal(size=5000) * 4])
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(oracle.round_fp8_e4m3(v.astype(np.float32)), ref)


def test_residual_add():
    """The residual enters once, additively: zero residual gives conv_bn_act,
    the result is linear in the residual, and a wrong shape is rejected."""
    wl = WORKLOADS["tiny_f32_3x3"]
    d = make_inputs(wl)
    args = (d["gamma"], d["beta"], d["mean"], d["var"], float(d["eps"]), wl.stride, wl.pad)
    base = oracle.conv_bn_act(d["x"], d["w"], *args, "silu")
    rng = np.random.default_rng(2)
    r1, r2 = rng.normal(size=base.shape), rng.normal(size=base.shape)
    z = oracle.conv_bn_act_residual(d["x"], d["w"], *args, "silu", np.zeros_like(base))
    np.testing.assert_array_equal(z, base)
    a = oracle.conv_bn_act_residual(d["x"], d["w"], *args, "silu", r1 + r2)
    b = oracle.conv_bn_act_residual(d["x"], d["w"], *args, "silu", r1)
    np.testing.assert_allclose(a - b, r2, rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.conv_bn_act_residual(d["x"], d["w"], *args, "silu", np.zeros(3))
