"""The chunkwise WY refactoring (what the HIP kernels compute) against the stepwise oracle."""

import numpy as np
import pytest

import oracle
from tests.chunked_model import backward as chunk_bwd
from tests.chunked_model import forward as chunk_fwd


def _inputs(seed, T, Dk, Dv, s0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, Dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, Dv))
    b = 1 / (1 + np.exp(-rng.standard_normal((T, Dk))))
    w = 1 / (1 + np.exp(-rng.standard_normal((T, Dv))))
    la = -np.log1p(np.exp(rng.standard_normal((T, Dk)) - 2))
    S0 = 0.3 * rng.standard_normal((Dk, Dv)) if s0 else np.zeros((Dk, Dv))
    return q, k, v, la, b, w, S0


def _as4(x):
    return x[None, :, None, :]


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-300, np.sqrt(np.mean(b * b))))


@pytest.mark.parametrize("C,T", [(1, 9), (7, 23), (16, 64), (16, 37), (32, 70), (64, 130)])
def test_chunked_forward_equals_stepwise(C, T):
    q, k, v, la, b, w, S0 = _inputs(C * 1000 + T, T, 16, 8)
    o, ST, _ = chunk_fwd(q, k, v, la, b, w, S0, C)
    o_ref, S_ref = oracle.forward(_as4(q), _as4(k), _as4(v), _as4(la), _as4(b), _as4(w), S0[None, None])
    assert rel(o, o_ref[0, :, 0]) < 1e-12
    assert rel(ST, S_ref[0, 0]) < 1e-12


@pytest.mark.parametrize("C,T", [(1, 7), (7, 23), (16, 40), (32, 64)])
@pytest.mark.parametrize("with_dS", [False, True])
def test_chunked_backward_equals_reverse_mode(C, T, with_dS):
    q, k, v, la, b, w, S0 = _inputs(C * 31 + T, T, 8, 6)
    rng = np.random.default_rng(5)
    dO = rng.standard_normal(v.shape)
    dS = rng.standard_normal(S0.shape) if with_dS else None
    g = chunk_bwd(q, k, v, la, b, w, S0, dO, dS, C)
    ref = oracle.backward(_as4(q), _as4(k), _as4(v), _as4(la), _as4(b), _as4(w), S0[None, None], _as4(dO),
                          None if dS is None else dS[None, None])
    for key in ("dq", "dk", "db", "dlog_alpha", "dv", "dw"):
        assert rel(g[key], ref[key][0, :, 0]) < 1e-10, key
    assert rel(g["dS0"], ref["dS0"][0, 0]) < 1e-10


def test_wy_inverse_is_unit_lower_triangular_inverse():
    q, k, v, la, b, w, S0 = _inputs(3, 64, 16, 8)
    g = np.cumsum(la, axis=0)
    Kh = np.exp(g) * b * k
    Kt = k / np.exp(g)
    A = np.tril(Kh @ Kt.T, -1)
    T = np.linalg.inv(np.eye(64) + A)
    assert np.allclose(np.triu(T, 1), 0, atol=1e-14)
    assert np.allclose(np.diag(T), 1, atol=1e-14)
    assert np.max(np.abs(T @ (np.eye(64) + A) - np.eye(64))) < 1e-12
