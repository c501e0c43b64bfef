"""Pins of the oracle's codec fit (CPU only): mu and W_down from the leading right singular vectors
of the mean-removed activation rows (pith.science paper page, "What carries the argument").

S1 recovers a planted subspace exactly (projector, mean, singular values of the planted factor,
exact reconstruction of every row) in both stacking modes; S2 checks Eckart-Young (the residual
energy equals the discarded eigenvalues of the covariance, from a different routine); S3 matches
the covariance eigenvectors; S4 checks the conventions (orthonormal, descending, sign); S5 ties
the fitted W_up blocks to the oracle's encode and decode.  Planted mistakes caught: a missing
centring (S1, S2), left instead of right vectors or a transposed block (S1, S5), the wrong
stacking order (S1), ascending order or no sign fix (S4).
"""
import numpy as np
import pytest

from looped_transformer_kv_amd import synth
from oracle import oracle as O


def _unstack(mode, A, T, H, d):
    """Stacked rows [G][n][X] -> trajectory rows [n][T][H][d] (the inverse of the stacking)."""
    G, n, X = A.shape
    if mode == 1:
        return A[0].reshape(n, T, H, d)
    return np.transpose(A.reshape(H, n, T, d), (1, 2, 0, 3))


def _planted(mode, T=3, H=2, d=8, r=4, n=200, seed=0, noise=0.0):
    rng = np.random.default_rng(seed)
    G = 1 if mode == 1 else H
    X = T * (H * d if mode == 1 else d)
    W0 = np.stack([np.linalg.qr(rng.standard_normal((X, r)))[0] for _ in range(G)])
    mu0 = 2.0 * rng.standard_normal((G, X))
    c = rng.standard_normal((G, n, r)) * (3.0 * 0.6 ** np.arange(r))
    A = mu0[:, None, :] + np.einsum("gnr,gxr->gnx", c, W0) + noise * rng.standard_normal((G, n, X))
    return _unstack(mode, A, T, H, d), A, W0, mu0, c


@pytest.mark.parametrize("mode", [0, 1])
def test_s1_planted_subspace(mode):
    T, H, d, r = 3, 2, 8, 4
    x, A, W0, mu0, c = _planted(mode, T, H, d, r)
    mu, Wd, Wup, sig = O.fit_svd(mode, T, H, d, r, x)
    G = Wd.shape[0]
    for g in range(G):
        assert np.max(np.abs(Wd[g] @ Wd[g].T - W0[g] @ W0[g].T)) < 1e-10
        assert np.max(np.abs(mu[g] - (mu0[g] + c[g].mean(0) @ W0[g].T))) < 1e-12
        cc = c[g] - c[g].mean(0)
        assert np.allclose(sig[g], np.linalg.svd(cc, compute_uv=False), rtol=1e-10, atol=0)
        rec = mu[g] + ((A[g] - mu[g]) @ Wd[g]) @ Wd[g].T
        assert np.max(np.abs(rec - A[g])) < 1e-10


@pytest.mark.parametrize("mode", [0, 1])
def test_s2_eckart_young(mode):
    T, H, d, r = 3, 2, 8, 4
    x, A, _, _, _ = _planted(mode, T, H, d, r, seed=1, noise=0.3)
    mu, Wd, _, sig = O.fit_svd(mode, T, H, d, r, x)
    for g in range(Wd.shape[0]):
        Ac = A[g] - A[g].mean(0)
        ev = np.sort(np.linalg.eigvalsh(Ac.T @ Ac))[::-1]
        resid = Ac - (Ac @ Wd[g]) @ Wd[g].T
        assert abs(np.sum(resid ** 2) - np.sum(ev[r:])) < 1e-8 * np.sum(ev)
        assert np.allclose(sig[g] ** 2, ev[:r], rtol=1e-9, atol=0)


@pytest.mark.parametrize("mode", [0, 1])
def test_s3_covariance_eigenvectors(mode):
    T, H, d, r = 2, 2, 8, 5
    x, A, _, _, _ = _planted(mode, T, H, d, r, seed=2, noise=0.2)
    _, Wd, _, _ = O.fit_svd(mode, T, H, d, r, x)
    for g in range(Wd.shape[0]):
        Ac = A[g] - A[g].mean(0)
        w, V = np.linalg.eigh(Ac.T @ Ac)
        V = V[:, ::-1][:, :r]
        # same vectors up to sign
        assert np.max(np.abs(np.abs(np.sum(V * Wd[g], axis=0)) - 1.0)) < 1e-9


def test_s4_conventions():
    x, _, _, _, _ = _planted(0, seed=3, noise=0.1)
    _, Wd, Wup, sig = O.fit_svd(0, 3, 2, 8, 4, x)
    for g in range(Wd.shape[0]):
        assert np.max(np.abs(Wd[g].T @ Wd[g] - np.eye(4))) < 1e-12
        assert np.all(np.diff(sig[g]) <= 0)
        for j in range(4):
            k = np.argmax(np.abs(Wd[g][:, j]))
            assert Wd[g][k, j] > 0


@pytest.mark.parametrize("mode", [0, 1])
def test_s5_blocks_with_encode_and_decode(mode):
    """W_up,t are W_down's blocks: encoding a planted row and decoding it at every loop through the
    oracle's decode (one cached token, attention weight 1) returns the row's loop-t vectors."""
    T, H, d, r = 3, 2, 8, 4
    x, _, _, _, _ = _planted(mode, T, H, d, r, n=60, seed=4)
    mu, Wd, Wup, _ = O.fit_svd(mode, T, H, d, r, x)
    ck = O.encode(mode, T, H, d, r, Wd, mu, x[:1])                  # [1][G][r]
    G = Wd.shape[0]
    P = 4
    pool = np.zeros((1, G, P, r))
    pool[0, :, 0, :] = ck[0]
    bt = np.zeros((1, 1), dtype=np.int32)
    lens = np.ones(1, dtype=np.int32)
    q = np.zeros((1, H, d))
    for t in range(T):
        out = O.decode(mode, T, H, d, r, r, t, Wup, Wup, mu, mu, pool, pool, bt, lens, P, q)
        assert np.max(np.abs(out[0] - x[0, t])) < 1e-10


def test_fit_rows_follow_the_staging_layout():
    cfg = synth.Config("fit", L=1, H=2, d=8, T=3, r_k=4, r_v=4, B=1, N=1, dtype="f64", cid=150)
    x = synth.chunk_staging(cfg, 0, synth.AX_K, 1, 50)[0]          # [n][T][H][d]
    A = O.stack_rows(0, x)
    assert A.shape == (2, 50, 24)
    assert np.array_equal(A[1, 7, 8:16], x[7, 1, 1])               # head 1, loop 1
    A2 = O.stack_rows(1, x)
    assert np.array_equal(A2[0, 7, 16 + 8:16 + 16], x[7, 1, 1])    # (t, h, i) order
