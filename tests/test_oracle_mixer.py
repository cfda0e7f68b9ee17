"""CPU pins for the oracle of the mixer steps beside the scan (oracle.mixer):
the causal conv1d + bias + SiLU with its conv state, and the gated group
RMSNorm.  Each is tied to library routines (numpy.convolve, scipy.special.expit)
and to invariants, not to a re-typed formula."""
import numpy as np
import pytest
import scipy.special

from oracle import mixer


def test_silu_against_expit():
    v = np.linspace(-60.0, 60.0, 2001)
    np.testing.assert_allclose(mixer.silu(v), v * scipy.special.expit(v), rtol=1e-15, atol=1e-300)


def test_conv_equals_numpy_convolve_per_channel():
    """Without state, each channel is numpy.convolve of the input with the
    reversed kernel (the causal part), then bias and SiLU."""
    rng = np.random.default_rng(0)
    b, L, D, K = 2, 37, 5, 4
    x = rng.standard_normal((b, L, D))
    w = rng.standard_normal((D, K))
    bias = rng.standard_normal(D)
    out, _ = mixer.conv1d(x, w, bias)
    for r in range(b):
        for c in range(D):
            pre = np.convolve(x[r, :, c], w[c, ::-1])[:L] + bias[c]
            np.testing.assert_allclose(out[r, :, c], pre * scipy.special.expit(pre), rtol=1e-13)


def test_conv_identity_tap():
    """Weight (0, 0, 0, 1) and no bias: silu of the input itself."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 9, 3))
    w = np.zeros((3, 4)); w[:, 3] = 1.0
    out, _ = mixer.conv1d(x, w)
    np.testing.assert_allclose(out, x * scipy.special.expit(x), rtol=1e-14)


@pytest.mark.parametrize("cut", [1, 2, 3, 10])
def test_conv_state_splits_a_sequence(cut):
    """Two calls chained through the conv state equal one call over the whole
    sequence (the state carries the last K-1 inputs)."""
    rng = np.random.default_rng(cut)
    b, L, D = 2, 13, 6
    x = rng.standard_normal((b, L, D))
    w = rng.standard_normal((D, 4)); bias = rng.standard_normal(D)
    s0 = rng.standard_normal((b, D, 3))
    full, sf = mixer.conv1d(x, w, bias, s0)
    a, s1 = mixer.conv1d(x[:, :cut], w, bias, s0)
    c, s2 = mixer.conv1d(x[:, cut:], w, bias, s1)
    np.testing.assert_allclose(np.concatenate([a, c], axis=1), full, rtol=1e-13)
    np.testing.assert_allclose(s2, sf, rtol=0, atol=0)


def test_conv_update_equals_last_token():
    rng = np.random.default_rng(4)
    b, L, D = 3, 8, 5
    x = rng.standard_normal((b, L, D))
    w = rng.standard_normal((D, 4)); bias = rng.standard_normal(D)
    full, sf = mixer.conv1d(x, w, bias)
    pre, sp = mixer.conv1d(x[:, :-1], w, bias)
    o, s = mixer.conv1d_update(x[:, -1], w, bias, sp)
    np.testing.assert_allclose(o, full[:, -1], rtol=1e-13)
    np.testing.assert_allclose(s, sf, rtol=0, atol=0)


def test_conv_packing_equals_separate_sequences():
    """A row packing two sequences equals the two sequences run alone (the
    second from a zero state), and the carried state is the second one's."""
    rng = np.random.default_rng(5)
    L1, L2, D = 6, 9, 4
    x = rng.standard_normal((1, L1 + L2, D))
    w = rng.standard_normal((D, 4)); bias = rng.standard_normal(D)
    s0 = rng.standard_normal((1, D, 3))
    seq = np.array([[0] * L1 + [1] * L2], dtype=np.int32)
    packed, sp = mixer.conv1d(x, w, bias, s0, seq_idx=seq)
    a, _ = mixer.conv1d(x[:, :L1], w, bias, s0)
    c, sc = mixer.conv1d(x[:, L1:], w, bias)
    np.testing.assert_allclose(packed, np.concatenate([a, c], axis=1), rtol=1e-13)
    np.testing.assert_allclose(sp, sc, rtol=0, atol=0)


def test_gated_norm_constant_group_closed_form():
    """A group whose gated values are all v: each output is v / sqrt(v^2 + eps)."""
    y = np.full((2, 8), 3.0)
    z = np.full((2, 8), 2.0)
    v = 3.0 * 2.0 * scipy.special.expit(2.0)
    out = mixer.gated_rmsnorm(y, z, np.ones(8), group=4, eps=1e-6)
    np.testing.assert_allclose(out, np.full((2, 8), v / np.sqrt(v * v + 1e-6)), rtol=1e-14)


def test_gated_norm_unit_rms_and_scale_invariance():
    """With weight 1 the mean square of each group's output is ms/(ms + eps);
    scaling y scales nothing (up to eps); groups do not mix."""
    rng = np.random.default_rng(7)
    y = rng.standard_normal((5, 1024)); z = rng.standard_normal((5, 1024))
    out = mixer.gated_rmsnorm(y, z, np.ones(1024), group=512, eps=1e-6)
    v = (y * z * scipy.special.expit(z)).reshape(5, 2, 512)
    ms = np.mean(v * v, axis=-1)
    np.testing.assert_allclose(np.mean(out.reshape(5, 2, 512) ** 2, axis=-1), ms / (ms + 1e-6), rtol=1e-12)
    out2 = mixer.gated_rmsnorm(1e3 * y, z, np.ones(1024), group=512, eps=0.0)
    out3 = mixer.gated_rmsnorm(y, z, np.ones(1024), group=512, eps=0.0)
    np.testing.assert_allclose(out2, out3, rtol=1e-12)
    y2 = y.copy(); y2[:, :512] *= 7.0
    np.testing.assert_allclose(mixer.gated_rmsnorm(y2, z, np.ones(1024), 512, 0.0)[:, 512:],
                               out3[:, 512:], rtol=1e-13)


def test_gated_norm_weight_is_elementwise():
    rng = np.random.default_rng(8)
    y = rng.standard_normal((3, 512)); z = rng.standard_normal((3, 512)); w = rng.standard_normal(512)
    np.testing.assert_allclose(mixer.gated_rmsnorm(y, z, w, 512),
                               mixer.gated_rmsnorm(y, z, np.ones(512), 512) * w, rtol=1e-14)


def test_split_is_the_scan_layout():
    H, P, G, N = 2, 3, 1, 4
    out = np.arange(2 * 5 * (H * P + 2 * G * N), dtype=np.float64).reshape(2, 5, -1)
    x, Bm, Cm = mixer.split_xbc(out, H, P, G, N)
    assert x[1, 2, 1, 0] == out[1, 2, 3] and Bm[0, 4, 0, 3] == out[0, 4, 9] and Cm[1, 0, 0, 0] == out[1, 0, 10]


# ------------------------------------------------------ planted mistakes

MUTATIONS = {
    "taps_reversed": ("acc += src * w[None, None, :, k]", "acc += src * w[None, None, :, K - 1 - k]"),
    "no_bias": ("acc += np.asarray(bias, dtype=np.float64)[None, None, :]", "acc += 0.0"),
    "no_silu": ("return silu(acc), new_state", "return acc, new_state"),
    "state_newest_first": ("ext = np.concatenate([np.transpose(st, (0, 2, 1)), xbc], axis=1)",
                           "ext = np.concatenate([np.transpose(st, (0, 2, 1))[:, ::-1], xbc], axis=1)"),
    "no_sequence_mask": ("if j >= 0 and seq[r, j] != seq[r, t]:", "if False:"),
    "gate_swapped": ("v = y * silu(z)\n    shape", "v = z * silu(y)\n    shape"),
    "no_sqrt": ("out = (vg / np.sqrt(ms + eps)).reshape(shape)", "out = (vg / (ms + eps)).reshape(shape)"),
    "mean_over_groups": ("ms = np.mean(vg * vg, axis=-1, keepdims=True)",
                         "ms = np.mean(vg * vg, axis=(-2, -1), keepdims=True)"),
    "silu_sign": ("return v * np.where(v >= 0,", "return v * np.where(v < 0,"),
}

PINS = [test_silu_against_expit, test_conv_equals_numpy_convolve_per_channel, test_conv_identity_tap,
        lambda: test_conv_state_splits_a_sequence(2), test_conv_update_equals_last_token,
        test_conv_packing_equals_separate_sequences, test_gated_norm_constant_group_closed_form,
        test_gated_norm_unit_rms_and_scale_invariance, test_gated_norm_weight_is_elementwise]


def _failures(module):
    global mixer
    saved = mixer
    mixer = module
    bad = 0
    try:
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                bad += 1
    finally:
        mixer = saved
    return bad


def test_mixer_pins_catch_planted_mistakes(tmp_path):
    import importlib.util
    import inspect
    src = inspect.getsource(mixer)
    assert _failures(mixer) == 0
    for name, (old, new) in MUTATIONS.items():
        assert src.count(old) == 1, name
        path = tmp_path / ("mixer_%s.py" % name)
        path.write_text(src.replace(old, new))
        spec = importlib.util.spec_from_file_location("mixer_%s" % name, path)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        assert _failures(mod) > 0, "mutation %s went undetected" % name
