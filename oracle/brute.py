"""Independent NumPy brute force of the LLA codec and decode attention, for tiny inputs.

TEST INFRASTRUCTURE ONLY.  Written separately from lla_oracle.c (whole-tensor reshapes and
einsum instead of explicit loops) so the two can pin each other.  Latents here are in logical
order [B][N][G][r] (no paging); lengths mask the tail.

Follows the pages on Looped Latent Attention (arXiv 2607.15456): pith.science paper page,
"What carries the argument" (encode c = (x - mu) W_down, reconstruct x_hat_t = c W_up,t + mu_t,
attention unchanged) and the abstract (per-head default, LLA-2D folds the heads).
"""
import numpy as np


def stack(mode, x):
    """Staging [B][T][H][d] -> stacked, un-centred vectors [B][G][X] ((t, h, i) order for 2D)."""
    B, T, H, d = x.shape
    if mode == 1:
        return x.reshape(B, 1, T * H * d)
    return np.transpose(x, (0, 2, 1, 3)).reshape(B, H, T * d)


def encode(mode, W_down, mu, x):
    xs = stack(mode, np.asarray(x, dtype=np.float64))
    return np.einsum("bgx,gxr->bgr", xs - mu[None], W_down)


def reconstruct(t, c, W_up, mu, T):
    """c [B][N][G][r], W_up [T][G][r][Dg], mu [G][X] -> [B][N][G][Dg] for loop t."""
    Dg = W_up.shape[-1]
    mu_t = mu.reshape(mu.shape[0], T, Dg)[:, t, :]
    return np.einsum("bngr,grk->bngk", c, W_up[t]) + mu_t[None, None]


def attention(q, K, V, lens, k_self=None, v_self=None, scale=None):
    """q [B][H][d]; K, V [B][N][H][d]; positions j >= lens[b] are masked out."""
    B, N, H, d = K.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    s = scale * np.einsum("bhd,bnhd->bhn", q, K)
    mask = np.arange(N)[None, :] < np.asarray(lens)[:, None]  # [B][N]
    s = np.where(mask[:, None, :], s, -np.inf)
    if k_self is not None:
        s = np.concatenate([s, scale * np.einsum("bhd,bhd->bh", q, k_self)[..., None]], axis=-1)
        V = np.concatenate([V, v_self[:, None]], axis=1)
    m = np.max(s, axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(s - m)
    Z = w.sum(-1, keepdims=True)
    p = w / np.where(Z > 0, Z, 1.0)
    return np.einsum("bhn,bnhd->bhd", p, V)


def decode(mode, T, H, d, t, W_up_k, W_up_v, mu_k, mu_v, ck, cv, lens, q, k_self=None,
           v_self=None, scale=None):
    B, N = ck.shape[:2]
    K = reconstruct(t, ck, W_up_k, mu_k, T).reshape(B, N, H, d)
    V = reconstruct(t, cv, W_up_v, mu_v, T).reshape(B, N, H, d)
    return attention(q, K, V, lens, k_self, v_self, scale)


def rotation_matrix(d, rot_dims, style, theta, pos):
    """The d x d rotary matrix of position pos (RoFormer's rotation, cited by the pages), built
    as a block matrix: the identity with a 2 x 2 rotation block [[cos, -sin], [sin, cos]] placed
    on each rotated pair of coordinates; y = R x."""
    R = np.eye(d)
    half = rot_dims // 2
    for m in range(half):
        ang = pos * theta ** (-2.0 * m / rot_dims)
        a, b = (m, m + half) if style == 0 else (2 * m, 2 * m + 1)
        R[a, a], R[a, b] = np.cos(ang), -np.sin(ang)
        R[b, a], R[b, b] = np.sin(ang), np.cos(ang)
    return R


def decode_rope(mode, T, H, d, t, W_up_k, W_up_v, mu_k, mu_v, ck, cv, lens, q, k_self=None,
                v_self=None, scale=None, theta=10000.0, rot_dims=None, style=0):
    """decode() with each cached key rotated to its position j and the self key to lens[b]."""
    if rot_dims is None:
        rot_dims = d
    B, N = ck.shape[:2]
    K = reconstruct(t, ck, W_up_k, mu_k, T).reshape(B, N, H, d)
    V = reconstruct(t, cv, W_up_v, mu_v, T).reshape(B, N, H, d)
    Rj = np.stack([rotation_matrix(d, rot_dims, style, theta, j) for j in range(N)])  # [N][d][d]
    K = np.einsum("nij,bnhj->bnhi", Rj, K)
    if k_self is not None:
        Rs = np.stack([rotation_matrix(d, rot_dims, style, theta, n) for n in lens])   # [B][d][d]
        k_self = np.einsum("bij,bhj->bhi", Rs, k_self)
    return attention(q, K, V, lens, k_self, v_self, scale)


def prefill(mode, T, H, d, t, W_up_k, W_up_v, mu_k, mu_v, ck, cv, lens, q, k_new, v_new, n_new,
            scale=None):
    """Chunked prefill: q, k_new, v_new [B][Pn][H][d]; query i sees cached j < lens[b] and new
    i' <= i (a causal mask over the concatenated key axis).  Rows i >= n_new[b] are zero."""
    B, N = ck.shape[:2]
    Pn = q.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    K = np.concatenate([reconstruct(t, ck, W_up_k, mu_k, T).reshape(B, N, H, d), k_new], axis=1)
    V = np.concatenate([reconstruct(t, cv, W_up_v, mu_v, T).reshape(B, N, H, d), v_new], axis=1)
    s = scale * np.einsum("bihd,bjhd->bhij", q, K)                  # [B][H][Pn][N + Pn]
    j = np.arange(N + Pn)
    cached = j[None, :] < np.asarray(lens)[:, None]                  # [B][N + Pn]
    causal = (j[None, :] >= N) & (j[None, :] - N <= np.arange(Pn)[:, None])  # [Pn][N + Pn]
    ok = cached[:, None, None, :] | causal[None, None, :, :]
    s = np.where(ok, s, -np.inf)
    w = np.exp(s - s.max(-1, keepdims=True))
    p = w / w.sum(-1, keepdims=True)
    out = np.einsum("bhij,bjhd->bihd", p, V)
    live = np.arange(Pn)[None, :] < np.asarray(n_new)[:, None]
    return np.where(live[..., None, None], out, 0.0)
