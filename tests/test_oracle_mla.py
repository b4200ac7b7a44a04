"""Pins of the oracle's MLA decode attention with weight absorption (section
09 of the reader.mx article "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型").  The
article checks its absorbed path against explicit K/V reconstruction; the
pins do the same with an independent float64 formulation.  CPU only."""
import numpy as np
import pytest

import oracle


def _cfg(H=4, kvl=64, nope=24, rope=8, vdim=32):
    return oracle.MlaConfig(H, kvl, nope, rope, vdim, float(1.0 / np.sqrt(nope + rope)))


def _inputs(c, S, T, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, c.H, c.nope + c.rope)).astype(np.float32)
    kv_b = (rng.standard_normal((c.H * (c.nope + c.vdim), c.kvl)) * 0.2).astype(np.float32)
    L = rng.standard_normal((T, c.kvl)).astype(np.float32)
    R = rng.standard_normal((T, c.rope)).astype(np.float32)
    return q, kv_b, L, R


def _explicit(c, q, kv_b, L, R):
    """Rebuild every head's keys and values from the latent, then ordinary
    causal softmax attention (float64)."""
    S, T = q.shape[0], L.shape[0]
    W = kv_b.astype(np.float64).reshape(c.H, c.nope + c.vdim, c.kvl)
    Lf, Rf = L.astype(np.float64), R.astype(np.float64)
    K_nope = np.einsum("hdi,ti->thd", W[:, :c.nope], Lf)          # [T][H][nope]
    V = np.einsum("hvi,ti->thv", W[:, c.nope:], Lf)               # [T][H][vdim]
    out = np.zeros((S, c.H, c.vdim))
    for s in range(S):
        n = T - S + 1 + s
        for h in range(c.H):
            k = np.concatenate([K_nope[:n, h], Rf[:n]], axis=1)   # rope key shared by heads
            a = k @ q[s, h].astype(np.float64) * c.scale
            p = np.exp(a - a.max())
            p /= p.sum()
            out[s, h] = p @ V[:n, h]
    return out


@pytest.mark.parametrize("S,T", [(1, 1), (1, 37), (3, 50)])
def test_absorbed_equals_explicit_kv(S, T):
    c = _cfg()
    q, kv_b, L, R = _inputs(c, S, T, seed=T)
    ctx = oracle.mla_decode(c, q, kv_b, L, R)
    ref = _explicit(c, q, kv_b, L, R)
    assert np.abs(ctx - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())


def test_single_row_and_uniform_scores():
    c = _cfg()
    q, kv_b, L, R = _inputs(c, 1, 9, seed=3)
    W = kv_b.astype(np.float64).reshape(c.H, c.nope + c.vdim, c.kvl)
    # one visible row: softmax weight 1, ctx = W_UV L[0]
    ctx1 = oracle.mla_decode(c, q, kv_b, L[:1], R[:1])
    assert np.allclose(ctx1[0], np.einsum("hvi,i->hv", W[:, c.nope:], L[0].astype(np.float64)),
                       rtol=1e-5, atol=1e-6)
    # zero query: uniform weights, ctx = W_UV mean(L)
    ctx0 = oracle.mla_decode(c, np.zeros_like(q), kv_b, L, R)
    mean = L.astype(np.float64).mean(axis=0)
    assert np.allclose(ctx0[0], np.einsum("hvi,i->hv", W[:, c.nope:], mean), rtol=1e-5, atol=1e-6)


def test_causal_window():
    # query s of S sees rows t < T - S + 1 + s: changing later rows leaves it alone
    c = _cfg()
    S, T = 3, 20
    q, kv_b, L, R = _inputs(c, S, T, seed=5)
    a = oracle.mla_decode(c, q, kv_b, L, R)
    L2, R2 = L.copy(), R.copy()
    L2[T - 1] += 5.0
    R2[T - 1] -= 5.0
    b = oracle.mla_decode(c, q, kv_b, L2, R2)
    assert np.array_equal(a[:S - 1], b[:S - 1])
    assert not np.array_equal(a[S - 1], b[S - 1])


def test_rope_key_shifts_scores():
    # a rope-only query: scores come from R alone, the latent does not matter
    c = _cfg()
    q, kv_b, L, R = _inputs(c, 1, 12, seed=6)
    q[:, :, :c.nope] = 0.0
    ctx = oracle.mla_decode(c, q, kv_b, L, R)
    ref = _explicit(c, q, kv_b, L, R)
    assert np.allclose(ctx, ref, rtol=1e-5, atol=1e-6)
