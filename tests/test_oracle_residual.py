"""Pins for the oracle's sublayer epilogue (post-norm and residual update).

The page "Welcome Beam: a 501B open model you can own, customize, and scale",
section "Residual Stream", normalises every sublayer output and adds it to
the stream at step s with weight 1/sqrt(s) while the stream keeps weight
sqrt((s-1)/s); the squares of the two weights sum to one so the stream keeps
a constant scale.  The norm is read as RMSNorm with a per-channel gain.
Pinned by torch's own rms_norm (step 1, where the stream is replaced), by
closed forms (a zero sublayer output leaves sqrt((s-1)/s) of the stream; a
zero stream gives an output of RMS sqrt(ms/(ms+eps))/sqrt(s)), by the scale
of the stream for orthogonal inputs, and by the norm's scale invariance."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).normal(size=shape) * scale).astype(np.float32)


def test_step_one_is_torch_rms_norm(oracle_mod):
    T, H, eps = 16, 512, 1e-5
    o = _rand((T, H), 0, 3.0)
    g = _rand((H,), 1) + 1.0
    res = _rand((T, H), 2)  # ignored at step 1: the stream keeps weight 0
    got = oracle_mod.residual_norm(o, g, eps, 1, res)
    want = F.rms_norm(torch.from_numpy(o).double(), (H,), torch.from_numpy(g).double(), eps)
    np.testing.assert_allclose(got, want.numpy(), rtol=2e-6, atol=2e-6)


@pytest.mark.parametrize("step", [2, 3, 10, 104])
def test_zero_output_keeps_the_stream_weight(oracle_mod, step):
    T, H = 4, 256
    res = _rand((T, H), 3)
    got = oracle_mod.residual_norm(np.zeros((T, H), np.float32), np.ones(H, np.float32), 1e-6,
                                   step, res)
    np.testing.assert_array_equal(got, np.float32(np.sqrt(np.float32((step - 1) / step))) * res)


@pytest.mark.parametrize("step", [2, 5, 104])
def test_zero_stream_has_closed_form_rms(oracle_mod, step):
    T, H, eps = 8, 1024, 0.5  # a large eps so that dropping it would show
    o = _rand((T, H), 4, 0.7)
    got = oracle_mod.residual_norm(o, np.ones(H, np.float32), eps, step, np.zeros((T, H), np.float32))
    ms = (o.astype(np.float64) ** 2).mean(axis=1)
    want = np.sqrt(ms / (ms + eps)) / np.sqrt(step)
    np.testing.assert_allclose(np.sqrt((got.astype(np.float64) ** 2).mean(axis=1)), want, rtol=1e-5)


@pytest.mark.parametrize("step", [2, 7, 52])
def test_orthogonal_inputs_keep_the_stream_scale(oracle_mod, step):
    """With the normalised output orthogonal to the stream and both of RMS 1,
    the new stream has RMS 1: the two weights' squares sum to one."""
    T, H = 6, 2048
    res = _rand((T, H), 5)
    res /= np.sqrt((res.astype(np.float64) ** 2).mean(axis=1, keepdims=True)).astype(np.float32)
    o = _rand((T, H), 6).astype(np.float64)
    r64 = res.astype(np.float64)
    o -= (o * r64).sum(axis=1, keepdims=True) / (r64 * r64).sum(axis=1, keepdims=True) * r64
    got = oracle_mod.residual_norm(o.astype(np.float32), np.ones(H, np.float32), 1e-12, step, res)
    rms = np.sqrt((got.astype(np.float64) ** 2).mean(axis=1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-5)


def test_norm_ignores_the_scale_of_the_output(oracle_mod):
    T, H = 4, 512
    o = _rand((T, H), 7)
    g = _rand((H,), 8)
    res = _rand((T, H), 9)
    base = oracle_mod.residual_norm(o, g, 1e-12, 3, res)
    for c in (2.5, 1000.0):
        np.testing.assert_allclose(oracle_mod.residual_norm(o * np.float32(c), g, 1e-12, 3, res),
                                   base, rtol=1e-5, atol=1e-6)


def test_bad_arguments_rejected(oracle_mod):
    o = np.ones((2, 64), np.float32)
    g = np.ones(64, np.float32)
    with pytest.raises(ValueError):
        oracle_mod.residual_norm(o, g, 0.0, 2, o)
    with pytest.raises(ValueError):
        oracle_mod.residual_norm(o, g, 1e-6, 0, o)
