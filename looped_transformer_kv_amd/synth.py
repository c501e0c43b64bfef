"""Seeded synthetic inputs for the LLA decode path, shared by the tests, the benchmark and smoke().

This module draws random numbers and lays them out; it holds none of the method's arithmetic
(no encode, reconstruction or attention).  Both the HIP library and the fp64 oracle receive the
values produced here (the oracle after an exact upcast to fp64).

Recipe (synthetic stand-ins for Ouro / Huginn activations, which are not available):
  * W_down[g] (X x r, X = T*D_g): Q of the reduced QR of an i.i.d. N(0,1) matrix, columns
    sign-fixed so diag(R) > 0 (orthonormal columns, as an SVD initialisation gives).
  * W_up[t][g] (r x D_g) = the transpose of W_down[g]'s rows t*D_g .. (t+1)*D_g - 1, i.e. the
    codec at its SVD initialisation, where the up-projection is the down-projection's transpose.
  * mu[g] ~ N(0, 0.1^2), length X.
  * latent component i ~ N(0, decay^i)   (decay 0.6, or 0.8 for the many-loop block).
  * q ~ N(0, 1).  Staging trajectories x (and hence the current token's loop-t self key/value)
    ~ N(0, s^2) with s^2 = sum_i decay^i / X + 0.01, the per-element energy of a cached vector.
  * block tables: a seeded random permutation of the physical pages (tests paging for real).
  * prefill chunks: Pn new tokens per sequence with queries ~ N(0, 1) and trajectories ~ N(0, s^2)
    as above; ragged chunk sizes are uniform in [0, Pn] with the two ends always present.
Floating inputs are drawn in fp64 and cast once to fp32, then to bf16 with round-to-nearest-even.
"""
from dataclasses import dataclass, replace

import numpy as np

ROOT_SEED = 1234


@dataclass(frozen=True)
class Config:
    name: str
    L: int            # layers
    H: int            # heads
    d: int            # head dim
    T: int            # loops
    r_k: int
    r_v: int
    B: int            # batch (sequences)
    N: int            # cached tokens per sequence
    mode: int = 0     # 0 per-head codec, 1 LLA-2D
    dtype: str = "bf16"
    decay: float = 0.6
    page: int = 64    # tokens per page
    cid: int = 0      # seed namespace

    @property
    def G(self):
        return 1 if self.mode == 1 else self.H

    @property
    def Dg(self):
        return self.H * self.d if self.mode == 1 else self.d

    @property
    def X(self):
        return self.T * self.Dg

    @property
    def max_pages(self):
        # one page of headroom so the token appended after the N cached ones has a slot
        return (self.N + 1 + self.page - 1) // self.page


# The workloads: shapes of the pages' models (Ouro-1.4B / 2.6B at T = 4, Huginn-3.5B at 32 loops)
# at the compression points the pages discuss (21.3x, 4x, 64x LLA-2D, 32x).
CONFIGS = {
    "tiny_f32": Config("tiny_f32", L=1, H=2, d=64, T=4, r_k=8, r_v=16, B=1, N=256,
                       dtype="f32", cid=1),
    "ouro14_21x": Config("ouro14_21x", L=24, H=16, d=128, T=4, r_k=16, r_v=32, B=32, N=4096,
                         cid=2),
    "ouro14_21x_cap": Config("ouro14_21x_cap", L=24, H=16, d=128, T=4, r_k=16, r_v=32, B=768,
                             N=4096, cid=3),
    "ouro14_4x": Config("ouro14_4x", L=24, H=16, d=128, T=4, r_k=96, r_v=160, B=64, N=4096,
                        cid=6),
    "ouro26_2d_64x": Config("ouro26_2d_64x", L=48, H=16, d=128, T=4, r_k=96, r_v=160, B=16,
                            N=16384, mode=1, cid=4),
    "huginn_32x": Config("huginn_32x", L=4, H=32, d=128, T=32, r_k=96, r_v=160, B=64, N=4096,
                         decay=0.8, cid=5),
}


def scaled(cfg: Config, **kw) -> Config:
    """Same codec and distributions, smaller batch / context (for tests the oracle can check)."""
    return replace(cfg, **kw)


def rng(cfg: Config, *keys) -> np.random.Generator:
    ss = np.random.SeedSequence([ROOT_SEED, cfg.cid] + [int(k) for k in keys])
    return np.random.Generator(np.random.PCG64(ss))


# kinds of draws (seed keys)
K_CODEC, K_MU, K_LAT, K_Q, K_X, K_PAGES, K_LENS, K_POS, K_PQ, K_PX, K_PN = range(11)
AX_K, AX_V = 0, 1


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16 (round to nearest even); returns the raw uint16 bit patterns."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def quantize(a: np.ndarray, dtype: str) -> np.ndarray:
    """Values exactly representable in the storage dtype (returned as fp64)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(f64_to_bf16_bits(a))
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def orthonormal(g: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    Q, R = np.linalg.qr(g.standard_normal((rows, cols)))
    sgn = np.sign(np.diag(R))
    sgn[sgn == 0] = 1.0
    return Q * sgn[None, :]


def codec(cfg: Config, layer: int, axis: int):
    """(W_down [G][X][r], W_up [T][G][r][D_g], mu [G][X]) in fp64, already quantised."""
    r = cfg.r_k if axis == AX_K else cfg.r_v
    Wd = np.empty((cfg.G, cfg.X, r))
    mu = np.empty((cfg.G, cfg.X))
    for g in range(cfg.G):
        Wd[g] = orthonormal(rng(cfg, K_CODEC, layer, g, axis), cfg.X, r)
        mu[g] = 0.1 * rng(cfg, K_MU, layer, g, axis).standard_normal(cfg.X)
    Wup = np.ascontiguousarray(
        np.transpose(Wd.reshape(cfg.G, cfg.T, cfg.Dg, r), (1, 0, 3, 2)))  # [T][G][r][Dg]
    return quantize(Wd, cfg.dtype), quantize(Wup, cfg.dtype), quantize(mu, cfg.dtype)


def latent_sigma(cfg: Config, r: int) -> np.ndarray:
    return np.sqrt(cfg.decay ** np.arange(r))


def latent_pool(cfg: Config, layer: int, axis: int, n_pages: int) -> np.ndarray:
    """Host-drawn latent pool [n_pages][G][P][r] (every slot filled, used or not)."""
    r = cfg.r_k if axis == AX_K else cfg.r_v
    g = rng(cfg, K_LAT, layer, axis)
    c = g.standard_normal((n_pages, cfg.G, cfg.page, r)) * latent_sigma(cfg, r)
    return quantize(c, cfg.dtype)


def block_table(cfg: Config, B: int, max_pages: int, salt: int = 0) -> np.ndarray:
    perm = rng(cfg, K_PAGES, salt).permutation(B * max_pages).astype(np.int32)
    return perm.reshape(B, max_pages)


def seq_lens(cfg: Config, B: int, N: int, ragged: bool = False, salt: int = 0) -> np.ndarray:
    if not ragged:
        return np.full(B, N, dtype=np.int32)
    return rng(cfg, K_LENS, salt).integers(1, N + 1, size=B).astype(np.int32)


def queries(cfg: Config, layer: int, t: int, B: int, gain: float = 1.0) -> np.ndarray:
    q = gain * rng(cfg, K_Q, layer, t).standard_normal((B, cfg.H, cfg.d))
    return quantize(q, cfg.dtype)


def staging(cfg: Config, layer: int, axis: int, B: int, salt: int = 0) -> np.ndarray:
    """Current tokens' loop trajectories x [B][T][H][d] for one axis."""
    r = cfg.r_k if axis == AX_K else cfg.r_v
    s = np.sqrt(np.sum(cfg.decay ** np.arange(r)) / cfg.X + 0.01)
    x = s * rng(cfg, K_X, layer, axis, salt).standard_normal((B, cfg.T, cfg.H, cfg.d))
    return quantize(x, cfg.dtype)


def chunk_queries(cfg: Config, layer: int, t: int, B: int, Pn: int,
                  gain: float = 1.0) -> np.ndarray:
    """Loop-t queries of a chunk of Pn new tokens per sequence, [B][Pn][H][d]."""
    q = gain * rng(cfg, K_PQ, layer, t).standard_normal((B, Pn, cfg.H, cfg.d))
    return quantize(q, cfg.dtype)


def chunk_staging(cfg: Config, layer: int, axis: int, B: int, Pn: int,
                  salt: int = 0) -> np.ndarray:
    """Loop trajectories of a chunk of Pn new tokens per sequence, [B][Pn][T][H][d] for one axis
    (same per-element spread as the single-token staging)."""
    r = cfg.r_k if axis == AX_K else cfg.r_v
    s = np.sqrt(np.sum(cfg.decay ** np.arange(r)) / cfg.X + 0.01)
    x = s * rng(cfg, K_PX, layer, axis, salt).standard_normal((B, Pn, cfg.T, cfg.H, cfg.d))
    return quantize(x, cfg.dtype)


def chunk_counts(cfg: Config, B: int, Pn: int, ragged: bool = False, salt: int = 0) -> np.ndarray:
    """New tokens per sequence in a chunk: all Pn, or ragged in [0, Pn] (ends included)."""
    if not ragged:
        return np.full(B, Pn, dtype=np.int32)
    n = rng(cfg, K_PN, salt).integers(0, Pn + 1, size=B).astype(np.int32)
    if B >= 2:
        n[0], n[-1] = 0, Pn
    return n


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    """Upload exactly-representable fp64 values in the storage dtype (torch tensor)."""
    import torch
    if dtype == "bf16":
        bits = f64_to_bf16_bits(a).view(np.int16)
        return torch.from_numpy(bits).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(device)


def from_device(t) -> np.ndarray:
    """Exact fp64 copy of a bf16 / fp32 torch tensor."""
    import torch
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.to(torch.float64).numpy()


def device_latent_pool(cfg: Config, layer: int, axis: int, n_pages: int, device="cuda"):
    """Latent pool drawn on the device (for multi-GB pools): torch Philox, seeded per
    (config, layer, axis), components scaled by their standard deviations, cast to bf16."""
    import torch
    r = cfg.r_k if axis == AX_K else cfg.r_v
    gen = torch.Generator(device=device)
    gen.manual_seed(ROOT_SEED * 1_000_003 + cfg.cid * 10_007 + layer * 13 + axis)
    sig = torch.tensor(latent_sigma(cfg, r), dtype=torch.float32, device=device)
    out = torch.empty((n_pages, cfg.G, cfg.page, r), dtype=torch.bfloat16, device=device)
    step = max(1, (1 << 27) // max(1, cfg.G * cfg.page * r))  # ~128M elements per chunk
    for p0 in range(0, n_pages, step):
        p1 = min(n_pages, p0 + step)
        x = torch.randn((p1 - p0, cfg.G, cfg.page, r), generator=gen, device=device,
                        dtype=torch.float32)
        out[p0:p1] = (x * sig).to(torch.bfloat16)
    return out
