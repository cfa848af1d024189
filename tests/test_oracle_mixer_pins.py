"""Pins of the token-mixer oracle (oracle/mixer.py) to facts outside it:
library routines that compute the same functions (PyTorch's grouped conv1d,
SiLU, log-sigmoid and RMS norm in float64), closed forms (a one-hot tap is a
pure shift; a norm's output has a known length) and invariances.  Each pin
would catch a plausible slip: a reversed tap order, a convolution that looks
ahead, a norm over the wrong axis, a sum where a mean belongs."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import mixer

rng = np.random.default_rng


def _x(shape, seed=0):
    return rng(seed).standard_normal(shape)


def test_causal_conv_matches_grouped_conv1d():
    """Depthwise causal convolution = conv1d with one group per channel, the
    taps reversed (conv1d correlates), K - 1 zeros in front, first T outputs."""
    B, H, T, D, K = 2, 3, 11, 5, mixer.TAPS
    x = _x((B, H, T, D), 1)
    taps = _x((H, D, K), 2)
    ref = F.conv1d(torch.from_numpy(x).permute(0, 1, 3, 2).reshape(B, H * D, T),
                   torch.from_numpy(taps[..., ::-1].copy()).reshape(H * D, 1, K),
                   padding=K - 1, groups=H * D)[..., :T]
    ref = ref.reshape(B, H, D, T).permute(0, 1, 3, 2).numpy()
    np.testing.assert_allclose(mixer.causal_conv(x, taps), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("lag", [0, 1, 3])
def test_one_hot_tap_is_a_causal_shift(lag):
    """Tap `lag` alone: every token takes the value `lag` steps back, and the
    first `lag` tokens (before the sequence start) are zero."""
    H, T, D = 2, 9, 4
    x = _x((1, H, T, D), 3)
    taps = np.zeros((H, D, mixer.TAPS))
    taps[..., lag] = 1.0
    y = mixer.causal_conv(x, taps)
    np.testing.assert_array_equal(y[..., :lag, :], 0.0)
    np.testing.assert_array_equal(y[..., lag:, :], x[..., :T - lag, :])


def test_conv_never_sees_later_tokens():
    """Changing token t changes no output before t."""
    x = _x((1, 2, 12, 3), 4)
    taps = _x((2, 3, mixer.TAPS), 5)
    y0 = mixer.causal_conv(x, taps)
    x2 = x.copy()
    x2[..., 7, :] += 1.0
    y1 = mixer.causal_conv(x2, taps)
    np.testing.assert_array_equal(y0[..., :7, :], y1[..., :7, :])
    assert np.all(np.abs(y1[..., 7:11, :] - y0[..., 7:11, :]).max(axis=-1) > 0)


def test_activations_match_library_routines():
    x = _x((1000,), 6) * 8
    np.testing.assert_allclose(mixer.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=0)
    np.testing.assert_allclose(mixer.log_sigmoid(x), F.logsigmoid(torch.from_numpy(x)).numpy(),
                               rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(mixer.sigmoid(x), torch.sigmoid(torch.from_numpy(x)).numpy(),
                               rtol=1e-14, atol=0)
    # and at extremes: no overflow, log sigmoid(-800) = -800, log sigmoid(800) ~ -exp(-800)
    ext = np.array([-800.0, 800.0, 0.0])
    ls = mixer.log_sigmoid(ext)
    assert ls[0] == -800.0 and -1e-300 < ls[1] <= 0.0 and abs(ls[2] + np.log(2.0)) < 1e-15
    np.testing.assert_allclose(np.exp(mixer.log_sigmoid(x)) + np.exp(mixer.log_sigmoid(-x)), 1.0,
                               rtol=1e-14)


def test_l2norm_length_and_axis():
    """Rows over the last axis come out with squared length s / (s + eps),
    s the input's squared length; scaling a row by c changes it only through
    eps: l2norm(c x) = l2norm(x) * sqrt((s + eps) / (s + eps / c^2))."""
    x = _x((3, 4, 7, 16), 7)
    y = mixer.l2norm(x)
    s = np.sum(x * x, axis=-1)
    np.testing.assert_allclose(np.sum(y * y, axis=-1), s / (s + mixer.EPS), rtol=1e-13)
    c = 1e3
    np.testing.assert_allclose(mixer.l2norm(c * x),
                               y * np.sqrt((s + mixer.EPS) / (s + mixer.EPS / c**2))[..., None],
                               rtol=1e-13)


def test_rms_norm_matches_library_and_mean_square():
    x = _x((2, 3, 5, 32), 8)
    wgt = _x((32,), 9)
    ref = F.rms_norm(torch.from_numpy(x), (32,), torch.from_numpy(wgt), eps=mixer.EPS).numpy()
    np.testing.assert_allclose(mixer.rms_norm(x, wgt), ref, rtol=1e-13)
    y = mixer.rms_norm(x, np.ones(32))
    m = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), m / (m + mixer.EPS), rtol=1e-13)


def test_epilogue_is_norm_times_gate():
    """With the gate logits large the SiLU gate is the identity (silu(z) -> z
    for z >> 0), and with them at zero the output is zero."""
    o = _x((1, 2, 4, 16), 10)
    wgt = np.ones(16)
    g_big = np.full(o.shape, 60.0)
    np.testing.assert_allclose(mixer.epilogue(o, g_big, wgt), mixer.rms_norm(o, wgt) * 60.0, rtol=1e-14)
    np.testing.assert_array_equal(mixer.epilogue(o, np.zeros(o.shape), wgt), 0.0)


def _fd_check(f, inputs, cotangent, grads, seed, h=1e-6):
    """Central differences of <cotangent, f(inputs)> along random directions,
    against the inner product of the returned gradients with them."""
    r = rng(seed)
    for _ in range(3):
        dirs = [r.standard_normal(np.shape(x)) for x in inputs]
        plus = [x + h * d for x, d in zip(inputs, dirs)]
        minus = [x - h * d for x, d in zip(inputs, dirs)]
        fd = (np.sum(cotangent * f(*plus)) - np.sum(cotangent * f(*minus))) / (2 * h)
        an = sum(np.sum(gr * d) for gr, d in zip(grads, dirs))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)


@pytest.mark.parametrize("l2", [True, False])
def test_stream_backward_finite_differences(l2):
    """Reverse mode of conv -> SiLU (-> L2 norm) against central differences
    of the forward (which the autograd path does not use)."""
    H, T, D = 2, 9, 6
    x = _x((1, H, T, D), 11)
    taps = _x((H, D, mixer.TAPS), 12) * 0.5
    dy = _x((1, H, T, D), 13)
    gx, gw = mixer.stream_bwd(x, taps, dy, l2)
    assert gx.shape == x.shape and gw.shape == taps.shape

    def f(x_, w_):
        y = mixer.silu(mixer.causal_conv(x_, w_))
        return mixer.l2norm(y) if l2 else y
    _fd_check(f, [x, taps], dy, [gx, gw], 14)


def test_epilogue_backward_finite_differences():
    o = _x((1, 2, 5, 8), 15)
    g = _x((1, 2, 5, 8), 16)
    wgt = 1.0 + 0.1 * _x((8,), 17)
    dy = _x((1, 2, 5, 8), 18)
    go, gg, gw = mixer.epilogue_bwd(o, g, wgt, dy)
    _fd_check(mixer.epilogue, [o, g, wgt], dy, [go, gg, gw], 19)


def test_stream_backward_is_anticausal():
    """The gradient of token t's input collects only outputs t .. t+3."""
    H, T, D = 1, 12, 4
    x = _x((1, H, T, D), 20)
    taps = _x((H, D, mixer.TAPS), 21)
    dy = np.zeros((1, H, T, D))
    dy[..., 6, :] = 1.0
    gx, _ = mixer.stream_bwd(x, taps, dy, False)
    assert np.all(gx[..., 7:, :] == 0.0) and np.all(gx[..., :3, :] == 0.0)
    assert np.all(np.abs(gx[..., 3:7, :]).max(axis=-1) > 0)
