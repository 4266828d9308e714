"""Pins of the oracle's attention against things other than itself: torch's
float64 scaled_dot_product_attention (a library routine), closed forms
(constant V, Q = 0, a single visible key, one dominant key) and invariances
of softmax attention (V + c, a common shift of the keys, key permutations,
causal independence from later keys)."""
import numpy as np
import pytest
import torch

import oracle
from epilogue_gemm_amd import inputs


def _vals(bits, fmt):
    return oracle.decode_array(fmt, np.asarray(bits).astype(np.uint32))


def _bits(vals, fmt):
    return oracle.encode_array(fmt, np.asarray(vals, np.float64).reshape(-1)).astype(np.uint16)


def _torch_ref(q, k, v, causal):
    # [B, S, H, D] -> [B, H, S, D] for torch, and back
    qt, kt, vt = (torch.from_numpy(x).transpose(1, 2) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal)
    return o.transpose(1, 2).contiguous().numpy()


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,S,H,D", [(2, 37, 3, 16), (1, 64, 2, 64), (3, 5, 1, 8)])
def test_matches_torch_sdpa_f64(fmt, causal, B, S, H, D):
    d = inputs.attention_inputs(B, S, H, D, fmt, seed=S + D)
    q, k, v = (_vals(d[n], fmt).reshape(B, S, H, D) for n in ("Q", "K", "V"))
    y, o = oracle.attention(d["Q"], d["K"], d["V"], B, S, H, D, fmt, causal)
    ref = _torch_ref(q, k, v, causal)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)
    assert np.array_equal(o.reshape(-1), _bits(y.reshape(-1), fmt))


def test_closed_forms():
    B, S, H, D, fmt = 1, 16, 2, 8, "f16"
    rng = np.random.default_rng(1)
    q = rng.standard_normal((B, S, H, D))
    k = rng.standard_normal((B, S, H, D))
    c = np.array([0.5, -1.0, 2.0, 0.25, 0.0, 3.0, -0.75, 1.5])
    v_const = np.broadcast_to(c, (B, S, H, D)).copy()
    Qb, Kb, Vc = _bits(q, fmt), _bits(k, fmt), _bits(v_const, fmt)
    for causal in (False, True):
        # every value row equal: the output is that row
        y, _ = oracle.attention(Qb, Kb, Vc, B, S, H, D, fmt, causal)
        assert np.allclose(y, v_const, rtol=1e-14, atol=1e-14)
    # Q = 0: uniform weights over the visible keys
    v = rng.standard_normal((B, S, H, D))
    Vb = _bits(v, fmt)
    vv = _vals(Vb, fmt).reshape(B, S, H, D)
    y, _ = oracle.attention(np.zeros_like(Qb), Kb, Vb, B, S, H, D, fmt, False)
    assert np.allclose(y, np.broadcast_to(vv.mean(axis=1, keepdims=True), y.shape), rtol=1e-13, atol=1e-14)
    y, _ = oracle.attention(np.zeros_like(Qb), Kb, Vb, B, S, H, D, fmt, True)
    cummean = np.cumsum(vv, axis=1) / np.arange(1, S + 1).reshape(1, S, 1, 1)
    assert np.allclose(y, cummean, rtol=1e-13, atol=1e-14)
    # causal query 0 sees key 0 only: exactly V[0]
    y, _ = oracle.attention(Qb, Kb, Vb, B, S, H, D, fmt, True)
    assert np.array_equal(y[:, 0], vv[:, 0])
    # S = 1: O = V
    y, _ = oracle.attention(Qb[: H * D], Kb[: H * D], Vb[: H * D], 1, 1, H, D, fmt, False)
    assert np.array_equal(y.reshape(-1), vv[:, :1].reshape(-1))


def test_dominant_key_and_scale():
    # q = a e0 and key 3 = b e0 with a b / sqrt(D) = 48: weight of every other
    # key (scores 0) is e^-48 relative, so O = V[3] to ~1e-20; with the scale
    # left out (a b = 48 sqrt(D)) the margin would differ by sqrt(D)
    B, S, H, D, fmt = 1, 8, 1, 16, "f16"
    q = np.zeros((B, S, H, D))
    k = np.zeros((B, S, H, D))
    q[0, :, 0, 0] = 16.0
    k[0, 3, 0, 0] = 12.0  # 16 * 12 / 4 = 48
    v = np.arange(S * D, dtype=np.float64).reshape(B, S, H, D) / 64
    y, _ = oracle.attention(_bits(q, fmt), _bits(k, fmt), _bits(v, fmt), B, S, H, D, fmt, False)
    w_other = np.exp(-48.0) / (1 + 7 * np.exp(-48.0))
    want = (1 - 7 * w_other) * v[0, 3, 0] + w_other * (v[0, :, 0].sum(axis=0) - v[0, 3, 0])
    assert np.allclose(y[0, :, 0], np.broadcast_to(want, (S, D)), rtol=1e-14, atol=1e-15)
    # with a smaller product the weights follow softmax(score / sqrt(D)) exactly
    k[0, 3, 0, 0] = 1.0  # score 16 / 4 = 4 for key 3, 0 elsewhere
    y, _ = oracle.attention(_bits(q, fmt), _bits(k, fmt), _bits(v, fmt), B, S, H, D, fmt, False)
    w3 = np.exp(4.0) / (np.exp(4.0) + 7)
    want = w3 * v[0, 3, 0] + (1 - w3) / 7 * (v[0, :, 0].sum(axis=0) - v[0, 3, 0])
    assert np.allclose(y[0, 0, 0], want, rtol=1e-13)


def test_invariances():
    B, S, H, D, fmt = 2, 24, 2, 16, "bf16"
    d = inputs.attention_inputs(B, S, H, D, fmt, seed=9)
    q, k, v = (_vals(d[n], fmt).reshape(B, S, H, D) for n in ("Q", "K", "V"))
    y0, _ = oracle.attention(d["Q"], d["K"], d["V"], B, S, H, D, fmt, False)
    # every key shifted by the same vector t changes all scores of a query by
    # q . t / sqrt(D): the softmax, hence O, is unchanged (t exact in bf16)
    t = np.zeros(D)
    t[0] = 2.0
    k_t = _bits(k + t, fmt)
    if np.array_equal(_vals(k_t, fmt).reshape(B, S, H, D), k + t):
        yt, _ = oracle.attention(d["Q"], k_t, d["V"], B, S, H, D, fmt, False)
        assert np.allclose(yt, y0, rtol=1e-11, atol=1e-12)
    # permuting keys and values together (full attention) leaves O unchanged
    perm = np.random.default_rng(2).permutation(S)
    kp = k[:, perm].copy()
    vp = v[:, perm].copy()
    yp, _ = oracle.attention(d["Q"], _bits(kp, fmt), _bits(vp, fmt), B, S, H, D, fmt, False)
    assert np.allclose(yp, y0, rtol=1e-12, atol=1e-13)
    # causal: query i does not depend on keys/values after i
    yc, _ = oracle.attention(d["Q"], d["K"], d["V"], B, S, H, D, fmt, True)
    k2, v2 = k.copy(), v.copy()
    k2[:, S // 2:] *= -3.0
    v2[:, S // 2:] += 5.0
    yc2, _ = oracle.attention(d["Q"], _bits(k2, fmt), _bits(v2, fmt), B, S, H, D, fmt, True)
    assert np.array_equal(yc2[:, : S // 2], yc[:, : S // 2])
    assert not np.allclose(yc2[:, S // 2:], yc[:, S // 2:])


def test_value_shift_adds_the_shift():
    # O(Q, K, V + c) = O(Q, K, V) + c for a constant row c (the weights sum to
    # 1); V on a grid of quarters so that V + c is exact in fp16
    B, S, H, D, fmt = 1, 32, 2, 8, "f16"
    d = inputs.attention_inputs(B, S, H, D, fmt, seed=4)
    v = np.random.default_rng(4).integers(-8, 9, (B, S, H, D)) / 4.0
    c = np.array([1.0, -2.0, 0.5, 4.0, -0.25, 8.0, 2.0, -1.0])
    v_bits, vc_bits = _bits(v, fmt), _bits(v + c, fmt)
    assert np.array_equal(_vals(vc_bits, fmt).reshape(B, S, H, D), v + c)
    for causal in (False, True):
        y0, _ = oracle.attention(d["Q"], d["K"], v_bits, B, S, H, D, fmt, causal)
        y1, _ = oracle.attention(d["Q"], d["K"], vc_bits, B, S, H, D, fmt, causal)
        assert np.allclose(y1 - y0, np.broadcast_to(c, y0.shape), rtol=0, atol=1e-13)


def test_rows_match_full_run_and_bad_arguments():
    B, S, H, D, fmt = 2, 40, 3, 16, "f16"
    d = inputs.attention_inputs(B, S, H, D, fmt, seed=8)
    y, o = oracle.attention(d["Q"], d["K"], d["V"], B, S, H, D, fmt, True)
    rng = np.random.default_rng(0)
    rb, ri, rh = rng.integers(0, B, 50), rng.integers(0, S, 50), rng.integers(0, H, 50)
    yr, orow = oracle.attention(d["Q"], d["K"], d["V"], B, S, H, D, fmt, True, rows=(rb, ri, rh))
    assert np.array_equal(yr, y[rb, ri, rh]) and np.array_equal(orow, o[rb, ri, rh])
    with pytest.raises(ValueError):
        oracle.attention(d["Q"], d["K"], d["V"], B, S, H, D + 1, fmt, True)
    with pytest.raises(ValueError):
        oracle.attention(d["Q"], d["K"], d["V"], B, S, H, D, fmt, True, rows=([0], [S], [0]))
