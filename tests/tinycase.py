"""Builds complete seeded decode problems (fp64 values, already quantised to the storage dtype)
from the synthetic generators, for the oracle pins and the GPU parity tests."""
from dataclasses import dataclass
from typing import Optional

import numpy as np

from looped_transformer_kv_amd import synth


@dataclass
class Problem:
    cfg: synth.Config
    layer: int
    B: int
    n_pages: int
    W_down_k: np.ndarray
    W_up_k: np.ndarray
    mu_k: np.ndarray
    W_down_v: np.ndarray
    W_up_v: np.ndarray
    mu_v: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    x_k: np.ndarray          # staging [B][T][H][d]
    x_v: np.ndarray
    q: dict                  # t -> [B][H][d]

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if self.B else 0

    def self_kv(self, t):
        """Self key/value of loop t: views into the staging buffers (batch stride T*H*d)."""
        return self.x_k[:, t], self.x_v[:, t]


def make(cfg: synth.Config, layer: int = 0, B: Optional[int] = None, N: Optional[int] = None,
         ragged: bool = False, q_gain: float = 1.0, loud_tokens: int = 0, salt: int = 0,
         lens: Optional[np.ndarray] = None) -> Problem:
    B = cfg.B if B is None else B
    N = cfg.N if N is None else N
    c = synth.scaled(cfg, B=B, N=N)
    max_pages = c.max_pages
    n_pages = B * max_pages
    Wdk, Wuk, muk = synth.codec(c, layer, synth.AX_K)
    Wdv, Wuv, muv = synth.codec(c, layer, synth.AX_V)
    kp = synth.latent_pool(c, layer, synth.AX_K, n_pages)
    vp = synth.latent_pool(c, layer, synth.AX_V, n_pages)
    bt = synth.block_table(c, B, max_pages, salt)
    if lens is None:
        lens = synth.seq_lens(c, B, N, ragged, salt)
    lens = np.asarray(lens, dtype=np.int32)
    if loud_tokens:
        # a few cached tokens with 8x larger K latents, so a peaked softmax singles them out
        g = synth.rng(c, synth.K_POS, layer, salt)
        for b in range(B):
            if lens[b] == 0:
                continue
            for j in g.integers(0, lens[b], size=loud_tokens):
                page = bt[b, j // c.page]
                kp[page, :, j % c.page, :] = synth.quantize(8.0 * kp[page, :, j % c.page, :],
                                                            c.dtype)
    xk = synth.staging(c, layer, synth.AX_K, B, salt)
    xv = synth.staging(c, layer, synth.AX_V, B, salt)
    q = {t: synth.queries(c, layer, t, B, q_gain) for t in range(c.T)}
    return Problem(c, layer, B, n_pages, Wdk, Wuk, muk, Wdv, Wuv, muv, kp, vp, bt, lens, xk, xv,
                   q)


def logical_latents(pool, block_table, lens, P):
    """Gather a paged pool [n_pages][G][P][r] into logical order [B][N][G][r] (N = max len),
    zero beyond each sequence's length."""
    B = block_table.shape[0]
    N = int(np.max(lens)) if B else 0
    G, r = pool.shape[1], pool.shape[3]
    out = np.zeros((B, N, G, r))
    for b in range(B):
        for j in range(int(lens[b])):
            out[b, j] = pool[block_table[b, j // P], :, j % P, :]
    return out
