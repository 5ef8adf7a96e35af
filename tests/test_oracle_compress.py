"""Pins of the oracle's CSA2 compressor (gated softmax pooling over a window's m
tokens, RMS normalisation, forward RoPE on the trailing channels) to special
cases that reduce to library routines or to exact permutations. CPU only."""
import numpy as np
import torch

import oracle as O


def _rms(x, g, eps):
    t = torch.from_numpy(np.asarray(x, np.float64))
    return torch.nn.functional.rms_norm(t, (t.shape[-1],), torch.from_numpy(np.asarray(g, np.float64)), eps).numpy()


def _data(B, m, D, seed):
    rng = np.random.default_rng(seed)
    kv = rng.standard_normal((B, m, D)).astype(np.float32)
    gate = (rng.standard_normal((B, m, D)) * 2).astype(np.float32)
    g = rng.uniform(0.5, 1.5, D).astype(np.float32)
    return kv, gate, g


def test_one_token_window_is_the_normalised_kv():
    kv, gate, g = _data(3, 1, 512, 1)
    np.testing.assert_allclose(O.compress(kv, gate, g, 1e-6), _rms(kv[:, 0], g, 1e-6), rtol=1e-6, atol=1e-7)


def test_equal_gates_give_the_normalised_mean():
    # the mean-of-pairs stand-in of the CSA2 workload is this case at m = 2
    for m in (2, 4, 128):
        kv, gate, g = _data(2, m, 256, m)
        gate[:] = gate[:, :1]                                  # equal over the window, any value per channel
        np.testing.assert_allclose(O.compress(kv, gate, g, 1e-6), _rms(kv.astype(np.float64).mean(1), g, 1e-6),
                                   rtol=2e-6, atol=1e-6)


def test_a_dominant_gate_selects_its_token_and_weights_sum_to_one():
    kv, gate, g = _data(2, 4, 128, 5)
    gate[:, 2] += 200.0
    np.testing.assert_allclose(O.compress(kv, gate, g, 1e-6), _rms(kv[:, 2], g, 1e-6), rtol=1e-6, atol=1e-7)
    kv2 = np.repeat(kv[:, :1], 4, axis=1)                      # the same kv in every token: gates do not matter
    np.testing.assert_allclose(O.compress(kv2, gate, g, 1e-6), _rms(kv2[:, 0], g, 1e-6), rtol=1e-6, atol=1e-7)


def test_no_weight_means_ones_and_eps_enters_the_mean_square():
    kv, gate, _ = _data(1, 2, 64, 7)
    kv *= 1e-4                                                 # mean square ~1e-8: eps matters
    a = O.compress(kv, gate, None, 1e-6)
    gm = np.exp(gate - gate.max(1, keepdims=True))
    p = (gm * kv).sum(1) / gm.sum(1)
    np.testing.assert_allclose(a, _rms(p, np.ones(64), 1e-6), rtol=1e-5, atol=1e-7)
    assert not np.allclose(a, _rms(p, np.ones(64), 0.0), rtol=1e-3)


def test_forward_rope_on_the_trailing_channels():
    B, m, D, r = 2, 2, 128, 32
    kv, gate, g = _data(B, m, D, 9)
    base = O.compress(kv, gate, g, 1e-6)
    zero = np.zeros((B, r // 2, 2), np.float32)
    zero[..., 0] = 1.0
    assert np.array_equal(O.compress(kv, gate, g, 1e-6, rope_cs=zero), base)   # zero angle: no change
    quarter = np.zeros((B, r // 2, 2), np.float32)
    quarter[..., 1] = 1.0                                      # 90 degrees: (x1, x2) -> (-x2, x1)
    q = O.compress(kv, gate, g, 1e-6, rope_cs=quarter)
    x1, x2 = base[:, D - r:D - r // 2], base[:, D - r // 2:]
    assert np.array_equal(q[:, :D - r], base[:, :D - r])
    np.testing.assert_array_equal(q[:, D - r:D - r // 2], -x2)
    np.testing.assert_array_equal(q[:, D - r // 2:], x1)
    th = np.random.default_rng(3).uniform(0, 6.3, (B, r // 2))
    cs = np.stack([np.cos(th), np.sin(th)], -1).astype(np.float32)
    t = O.compress(kv, gate, g, 1e-6, rope_cs=cs)
    n0 = np.hypot(x1, x2)
    n1 = np.hypot(t[:, D - r:D - r // 2], t[:, D - r // 2:])
    np.testing.assert_allclose(n1, n0, rtol=1e-6, atol=1e-7)  # a rotation keeps pair norms


def test_masked_gates_drop_their_tokens():
    """A gate of -inf takes its token out of the channel's softmax: masking tokens
    gives the same entry as a window without them (per channel)."""
    kv, gate, g = _data(2, 4, 96, 11)
    masked = gate.copy()
    masked[0, 0] = -np.inf                                     # sequence 0: token 0 masked everywhere
    masked[1, 1:3] = -np.inf                                   # sequence 1: tokens 1 and 2 masked
    got = O.compress(kv, masked, g, 1e-6)
    assert np.all(np.isfinite(got))
    np.testing.assert_array_equal(got[:1], O.compress(kv[:1, 1:], gate[:1, 1:], g, 1e-6))
    keep = [0, 3]
    np.testing.assert_array_equal(got[1:], O.compress(kv[1:, keep], gate[1:, keep], g, 1e-6))
