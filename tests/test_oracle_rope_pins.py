"""Pins of the oracle's rotary path (CPU only): decode with the rotation applied after
reconstruction.

The pages' free-parameter ledger records the assumption behind it: a token keeps one position
at every recurrence step, so the rotation can be applied to the reconstructed pre-rotation K.
The rotation itself is RoFormer's (cited by the pages): pair m of the rotated dimensions turns by
pos * theta^(-2m / rot_dims).  Planted-mistake coverage: a flipped sine, a wrong frequency law or
position breaks R2/R5; a wrong pairing breaks R2/R4; forgetting to rotate the self key or using
the wrong position for it breaks R5; touching the unrotated tail breaks R3.
"""
import math

import numpy as np
import pytest

from looped_transformer_kv_amd import synth
from oracle import brute
from oracle import oracle as O
import tinycase


def _problem(mode, seed, d=8, H=2, ragged=True, q_gain=3.0):
    cfg = synth.Config("rope", L=1, H=H, d=d, T=2, r_k=3, r_v=4, B=3, N=9, mode=mode,
                       dtype="f64", page=4, cid=90 + seed)
    p = tinycase.make(cfg, ragged=ragged, q_gain=q_gain)
    return cfg, p


def _decode_rope(cfg, p, t, with_self, **kw):
    ks, vs = p.self_kv(t) if with_self else (None, None)
    return O.decode_rope(cfg.mode, cfg.T, cfg.H, cfg.d, cfg.r_k, cfg.r_v, t, p.W_up_k, p.W_up_v,
                         p.mu_k, p.mu_v, p.k_pool, p.v_pool, p.block_table, p.seq_lens,
                         cfg.page, p.q[t], ks, vs, **kw)


# ---- R1: no rotated dimensions is exactly the pinned decode ------------------------------------
@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("with_self", [False, True])
def test_r1_zero_rotation_is_plain_decode(mode, with_self):
    cfg, p = _problem(mode, 0)
    for t in range(cfg.T):
        ks, vs = p.self_kv(t) if with_self else (None, None)
        base = O.decode(mode, cfg.T, cfg.H, cfg.d, cfg.r_k, cfg.r_v, t, p.W_up_k, p.W_up_v,
                        p.mu_k, p.mu_v, p.k_pool, p.v_pool, p.block_table, p.seq_lens, cfg.page,
                        p.q[t], ks, vs)
        assert np.array_equal(_decode_rope(cfg, p, t, with_self, rot_dims=0), base)


# ---- R2: closed-form rotations -----------------------------------------------------------------
def test_r2_closed_form_values():
    # one pair turned by one radian: (1, 0) -> (cos 1, sin 1)
    y = O.rope_rotate([1.0, 0.0], 2, 0, 10000.0, 1.0)
    assert np.allclose(y, [0.5403023058681398, 0.8414709848078965], rtol=0, atol=1e-15)
    # d = 4, theta = 10^4: pair 0 has frequency 1, pair 1 frequency 10^(-2) (exponent -2m/rot)
    # half split pairs (0, 2) and (1, 3); at position 100 pair 1 turns by exactly one radian and
    # pair 0 by 100 radians
    y = O.rope_rotate([0.0, 1.0, 0.0, 0.0], 4, 0, 10000.0, 100.0)
    assert np.allclose(y, [0.0, math.cos(1.0), 0.0, math.sin(1.0)], rtol=0, atol=1e-15)
    y = O.rope_rotate([0.0, 0.0, 1.0, 0.0], 4, 0, 10000.0, 100.0)
    assert np.allclose(y, [-math.sin(100.0), 0.0, math.cos(100.0), 0.0], rtol=0, atol=1e-14)
    # interleaved pairs (0, 1) and (2, 3)
    y = O.rope_rotate([0.0, 0.0, 1.0, 0.0], 4, 1, 10000.0, 100.0)
    assert np.allclose(y, [0.0, 0.0, math.cos(1.0), math.sin(1.0)], rtol=0, atol=1e-15)
    # a quarter turn of pair 0 (position pi/2) maps e0 to e1 (half split: e_half)
    y = O.rope_rotate([1.0, 0.0, 0.0, 0.0], 4, 1, 10000.0, math.pi / 2)
    assert np.allclose(y, [0.0, 1.0, 0.0, 0.0], rtol=0, atol=1e-15)


# ---- R3: it is a rotation: orthogonal, additive in position, identity at 0 ---------------------
@pytest.mark.parametrize("style", [0, 1])
def test_r3_rotation_group_properties(style):
    rng = np.random.default_rng(3)
    d, rot, theta = 12, 8, 500.0
    x = rng.standard_normal(d)
    for pos in (0.0, 1.0, 37.0, 4095.0):
        y = O.rope_rotate(x, rot, style, theta, pos)
        assert abs(np.linalg.norm(y) - np.linalg.norm(x)) < 1e-12
        assert np.array_equal(y[rot:], x[rot:])                      # tail untouched
    assert np.array_equal(O.rope_rotate(x, rot, style, theta, 0.0), x)
    a, b = 13.0, 29.0
    ab = O.rope_rotate(O.rope_rotate(x, rot, style, theta, b), rot, style, theta, a)
    assert np.max(np.abs(ab - O.rope_rotate(x, rot, style, theta, a + b))) < 1e-12
    back = O.rope_rotate(O.rope_rotate(x, rot, style, theta, a), rot, style, theta, -a)
    assert np.max(np.abs(back - x)) < 1e-13


# ---- R4: the two pairings are the same rotation in permuted coordinates -------------------------
@pytest.mark.parametrize("mode", [0, 1])
def test_r4_half_split_equals_interleaved_after_permutation(mode):
    cfg, p = _problem(mode, 1)
    d, rot, H = cfg.d, cfg.d, cfg.H
    half = rot // 2
    # interleaved coordinate 2m <- half-split m, 2m + 1 <- half-split m + half
    perm = np.empty(d, dtype=np.int64)
    perm[0::2] = np.arange(half)
    perm[1::2] = np.arange(half) + half
    # permute every head slice of the key side (W_up^K columns, mu^K, q, k_self); V stays
    cols = np.concatenate([h * d + perm for h in range(H if mode == 1 else 1)])
    Wk2 = p.W_up_k[..., cols]
    mk = p.mu_k.reshape(p.mu_k.shape[0], cfg.T, -1)[..., cols].reshape(p.mu_k.shape)
    t = 1
    ks, vs = p.self_kv(t)
    q2 = p.q[t][..., perm]
    ks2 = np.ascontiguousarray(ks)[..., perm]
    args = (mode, cfg.T, H, d, cfg.r_k, cfg.r_v, t)
    a = O.decode_rope(*args, p.W_up_k, p.W_up_v, p.mu_k, p.mu_v, p.k_pool, p.v_pool,
                      p.block_table, p.seq_lens, cfg.page, p.q[t], ks, vs, theta=50.0, style=0)
    b = O.decode_rope(*args, Wk2, p.W_up_v, mk, p.mu_v, p.k_pool, p.v_pool, p.block_table,
                      p.seq_lens, cfg.page, q2, ks2, vs, theta=50.0, style=1)
    assert np.max(np.abs(a - b)) < 1e-12
    # and the rotation matters: without it the output differs
    c = O.decode_rope(*args, p.W_up_k, p.W_up_v, p.mu_k, p.mu_v, p.k_pool, p.v_pool,
                      p.block_table, p.seq_lens, cfg.page, p.q[t], ks, vs, rot_dims=0)
    assert np.max(np.abs(a - c)) > 1e-3


# ---- R5: brute force on tiny ragged inputs (separate NumPy formulation) ------------------------
@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("style", [0, 1])
@pytest.mark.parametrize("with_self", [False, True])
@pytest.mark.parametrize("rot", [8, 4])
def test_r5_brute_force_tiny(mode, style, with_self, rot):
    cfg, p = _problem(mode, 2 + style)
    p.seq_lens[0] = 0
    ck = tinycase.logical_latents(p.k_pool, p.block_table, p.seq_lens, cfg.page)
    cv = tinycase.logical_latents(p.v_pool, p.block_table, p.seq_lens, cfg.page)
    for t in range(cfg.T):
        ks, vs = p.self_kv(t) if with_self else (None, None)
        out = _decode_rope(cfg, p, t, with_self, theta=30.0, rot_dims=rot, style=style)
        ref = brute.decode_rope(mode, cfg.T, cfg.H, cfg.d, t, p.W_up_k, p.W_up_v, p.mu_k,
                                p.mu_v, ck, cv, p.seq_lens, p.q[t],
                                None if ks is None else np.ascontiguousarray(ks),
                                None if vs is None else np.ascontiguousarray(vs),
                                theta=30.0, rot_dims=rot, style=style)
        assert np.max(np.abs(out - ref)) < 1e-12
