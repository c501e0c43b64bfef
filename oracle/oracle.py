"""ctypes front end of the fp64 C oracle (lla_oracle.c).

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the benchmark's CPU-baseline leg,
never by the product path.  Every argument is converted to a contiguous float64 / int32 numpy
array first, so the C code sees exactly the values it is given.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        i, dbl, lng = ctypes.c_int, ctypes.c_double, ctypes.c_long
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_compression_ratio.restype = ctypes.c_double
        L.oracle_compression_ratio.argtypes = [i, i, i, i, i, i]
        L.oracle_decode.restype = ctypes.c_int
        L.oracle_decode.argtypes = [i, i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, ip, ip, i, i, i,
                                    dp, dp, dp, lng, dbl, dp]
        L.oracle_rope_rotate.restype = ctypes.c_int
        L.oracle_rope_rotate.argtypes = [dp, i, i, dbl, dbl]
        L.oracle_decode_rope.restype = ctypes.c_int
        L.oracle_decode_rope.argtypes = [i, i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, ip, ip, i, i,
                                         i, dp, dp, dp, lng, dbl, dbl, i, i, dp]
        L.oracle_prefill.restype = ctypes.c_int
        L.oracle_prefill.argtypes = [i, i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, ip, ip, i, i, i,
                                     i, ip, dp, dp, dp, lng, dbl, dp]
        L.oracle_encode.restype = ctypes.c_int
        L.oracle_encode.argtypes = [i, i, i, i, i, dp, dp, dp, i, dp]
        L.oracle_append.restype = ctypes.c_int
        L.oracle_append.argtypes = [i, i, dp, i, ip, ip, i, i, dp]
        L.oracle_flat_attn.restype = ctypes.c_int
        L.oracle_flat_attn.argtypes = [i, i, dp, dp, ip, ip, i, i, i, dp, dp, dp, lng, dbl, dp]
        _lib = L
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a, kind=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(kind))


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def compression_ratio(mode, T, H, d, r_k, r_v) -> float:
    return float(lib().oracle_compression_ratio(mode, T, H, d, r_k, r_v))


def decode(mode, T, H, d, r_k, r_v, t, W_up_k, W_up_v, mu_k, mu_v, k_pool, v_pool,
           block_table, seq_lens, P, q, k_self=None, v_self=None, scale=None):
    """Decode attention of loop t over the paged latent cache; returns out [B][H][d] (fp64).
    k_self / v_self are [B][H][d] arrays (any strides; copied densely, so the C stride is H*d)."""
    block_table = _i32(block_table)
    seq_lens = _i32(seq_lens)
    B, max_pages = block_table.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    arrs = [_f64(a) for a in (W_up_k, W_up_v, mu_k, mu_v, k_pool, v_pool, q, k_self, v_self)]
    out = np.zeros((B, H, d), dtype=np.float64)
    rc = lib().oracle_decode(mode, T, H, d, r_k, r_v, t, *[_p(a) for a in arrs[:6]],
                             _p(block_table, ctypes.c_int32), _p(seq_lens, ctypes.c_int32),
                             B, P, max_pages, _p(arrs[6]), _p(arrs[7]), _p(arrs[8]),
                             H * d, float(scale), _p(out))
    if rc != 0:
        raise RuntimeError(f"oracle_decode failed ({rc})")
    return out


def rope_rotate(x, rot_dims, style, theta, pos):
    """A copy of the vector x with its first rot_dims entries rotated to position pos."""
    y = np.array(x, dtype=np.float64, copy=True)
    rc = lib().oracle_rope_rotate(_p(y), int(rot_dims), int(style), float(theta), float(pos))
    if rc != 0:
        raise RuntimeError(f"oracle_rope_rotate failed ({rc})")
    return y


def decode_rope(mode, T, H, d, r_k, r_v, t, W_up_k, W_up_v, mu_k, mu_v, k_pool, v_pool,
                block_table, seq_lens, P, q, k_self=None, v_self=None, scale=None,
                theta=10000.0, rot_dims=None, style=0):
    """decode() with the rotation applied after reconstruction: cached K_hat(j) at position j,
    k_self at position seq_lens[b]; q as given.  rot_dims defaults to d."""
    block_table = _i32(block_table)
    seq_lens = _i32(seq_lens)
    B, max_pages = block_table.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if rot_dims is None:
        rot_dims = d
    arrs = [_f64(a) for a in (W_up_k, W_up_v, mu_k, mu_v, k_pool, v_pool, q, k_self, v_self)]
    out = np.zeros((B, H, d), dtype=np.float64)
    rc = lib().oracle_decode_rope(mode, T, H, d, r_k, r_v, t, *[_p(a) for a in arrs[:6]],
                                  _p(block_table, ctypes.c_int32), _p(seq_lens, ctypes.c_int32),
                                  B, P, max_pages, _p(arrs[6]), _p(arrs[7]), _p(arrs[8]),
                                  H * d, float(scale), float(theta), int(rot_dims), int(style),
                                  _p(out))
    if rc != 0:
        raise RuntimeError(f"oracle_decode_rope failed ({rc})")
    return out


def prefill(mode, T, H, d, r_k, r_v, t, W_up_k, W_up_v, mu_k, mu_v, k_pool, v_pool,
            block_table, seq_lens, P, q, k_new, v_new, n_new, scale=None):
    """Chunked prefill attention of loop t: q, k_new, v_new [B][Pn][H][d]; new token i of
    sequence b attends to its cached context (reconstructed) and to new tokens 0..i.  Returns
    out [B][Pn][H][d] (fp64), zero in rows i >= n_new[b]."""
    block_table = _i32(block_table)
    seq_lens = _i32(seq_lens)
    n_new = _i32(n_new)
    B, max_pages = block_table.shape
    q = _f64(q)
    Pn = q.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    arrs = [_f64(a) for a in (W_up_k, W_up_v, mu_k, mu_v, k_pool, v_pool, k_new, v_new)]
    out = np.zeros((B, Pn, H, d), dtype=np.float64)
    rc = lib().oracle_prefill(mode, T, H, d, r_k, r_v, t, *[_p(a) for a in arrs[:6]],
                              _p(block_table, ctypes.c_int32), _p(seq_lens, ctypes.c_int32),
                              B, P, max_pages, Pn, _p(n_new, ctypes.c_int32), _p(q),
                              _p(arrs[6]), _p(arrs[7]), H * d, float(scale), _p(out))
    if rc != 0:
        raise RuntimeError(f"oracle_prefill failed ({rc})")
    return out


def encode(mode, T, H, d, r, W_down, mu, x):
    """c = (x - mu) W_down for one axis; x is the staging buffer [B][T][H][d]; returns [B][G][r]."""
    x = _f64(x)
    B = x.shape[0]
    G = 1 if mode == 1 else H
    c = np.zeros((B, G, r), dtype=np.float64)
    rc = lib().oracle_encode(mode, T, H, d, r, _p(_f64(W_down)), _p(_f64(mu)), _p(x), B, _p(c))
    if rc != 0:
        raise RuntimeError(f"oracle_encode failed ({rc})")
    return c


def append(c, write_pos, block_table, P, pool):
    """Returns a copy of the fp64 pool with c[b] written at logical position write_pos[b]."""
    c = _f64(c)
    B, G, r = c.shape
    block_table = _i32(block_table)
    pool = np.array(pool, dtype=np.float64, copy=True, order="C")
    rc = lib().oracle_append(G, r, _p(c), B, _p(_i32(write_pos), ctypes.c_int32),
                             _p(block_table, ctypes.c_int32), P, block_table.shape[1], _p(pool))
    if rc != 0:
        raise RuntimeError("oracle_append: write position outside the block table")
    return pool


def flat_attn(H, d, k_pool, v_pool, block_table, seq_lens, P, q, k_self=None, v_self=None,
              scale=None):
    """Softmax attention over an uncompressed paged loop-t cache; returns [B][H][d]."""
    block_table = _i32(block_table)
    seq_lens = _i32(seq_lens)
    B, max_pages = block_table.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    arrs = [_f64(a) for a in (k_pool, v_pool, q, k_self, v_self)]
    out = np.zeros((B, H, d), dtype=np.float64)
    rc = lib().oracle_flat_attn(H, d, _p(arrs[0]), _p(arrs[1]), _p(block_table, ctypes.c_int32),
                                _p(seq_lens, ctypes.c_int32), B, P, max_pages, _p(arrs[2]),
                                _p(arrs[3]), _p(arrs[4]), H * d, float(scale), _p(out))
    if rc != 0:
        raise RuntimeError(f"oracle_flat_attn failed ({rc})")
    return out


def encode_prefill(mode, T, H, d, r, W_down, mu, x, write_pos, n_new, block_table, P, pool):
    """Bulk encode and append of a chunk: x is the chunk's staging [B][Pn][T][H][d]; row i of
    sequence b (i < n_new[b]) is encoded as one token (encode above) and written at logical
    position write_pos[b] + i (append above).  Returns (c [B][Pn][G][r], the updated fp64 pool);
    c is zero in rows i >= n_new[b]."""
    x = _f64(x)
    B, Pn = x.shape[:2]
    G = 1 if mode == 1 else H
    c = encode(mode, T, H, d, r, W_down, mu, x.reshape((B * Pn,) + x.shape[2:]))
    c = c.reshape(B, Pn, G, r)
    n = np.clip(_i32(n_new), 0, Pn)
    block_table = _i32(block_table)
    rows = [(b, i) for b in range(B) for i in range(int(n[b]))]
    if rows:
        bs = np.array([b for b, _ in rows])
        pos = np.array([int(write_pos[b]) + i for b, i in rows], dtype=np.int32)
        pool = append(np.stack([c[b, i] for b, i in rows]), pos, block_table[bs], P, pool)
    else:
        pool = np.array(pool, dtype=np.float64, copy=True)
    for b in range(B):
        c[b, int(n[b]):] = 0.0
    return c, pool


def stack_rows(mode, x):
    """Trajectory rows x [n][T][H][d] -> stacked vectors [G][n][X], in the order the encode uses
    (per head: (t, i) of head g; LLA-2D: (t, h, i))."""
    x = _f64(x)
    n, T, H, d = x.shape
    if mode == 1:
        return x.reshape(1, n, T * H * d)
    return np.ascontiguousarray(np.transpose(x, (2, 0, 1, 3)).reshape(H, n, T * d))


def fit_svd(mode, T, H, d, r, x):
    """Codec initialisation by truncated SVD of the mean-removed activations (pith.science
    paper page, "What carries the argument"): per group, mu = mean of the stacked rows,
    W_down = the r leading right singular vectors of the centred stacked matrix (columns in
    decreasing singular value; sign fixed so each column's entry of largest magnitude is
    positive), W_up,t = the transpose of W_down's rows t*D_g .. (t+1)*D_g - 1.
    x: rows [n][T][H][d].  Returns (mu [G][X], W_down [G][X][r], W_up [T][G][r][D_g],
    sigma [G][r])."""
    A = stack_rows(mode, x)
    G, n, X = A.shape
    Dg = X // T
    mu = A.mean(axis=1)
    Wd = np.empty((G, X, r))
    sig = np.empty((G, r))
    for g in range(G):
        _, s, vt = np.linalg.svd(A[g] - mu[g][None, :], full_matrices=False)
        V = vt[:r].T.copy()
        for j in range(r):
            k = int(np.argmax(np.abs(V[:, j])))
            if V[k, j] < 0:
                V[:, j] = -V[:, j]
        Wd[g] = V
        sig[g] = s[:r]
    Wup = np.ascontiguousarray(np.transpose(Wd.reshape(G, T, Dg, r), (1, 0, 3, 2)))
    return mu, Wd, Wup, sig
