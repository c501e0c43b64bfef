"""GPU parity of the codec fit (lla_fit_svd) against the fp64 oracle (numpy SVD of the centred,
stacked rows), through the C ABI.

Inputs are planted low-rank trajectories (mean + factor x orthonormal basis + noise, factor
variances decaying like the latent spectrum) rounded to bf16; the oracle fits the exact bf16
values.  Bar: mu and W_down within the bf16 bar (2e-2 max + 1e-3) with W_down's columns matched
up to the sign only where the sign decision is ambiguous (two entries of equal magnitude), the
singular values to 1e-3 relative, the fitted subspaces' projectors to 1e-2, and W_up equal to
W_down's blocks bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

from looped_transformer_kv_amd import lla, synth
from oracle import oracle as O
from gpucase import assert_close

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _planted(mode, T, H, d, r_true, n, seed, noise=0.02, decay=0.8):
    rng = np.random.default_rng(seed)
    G = 1 if mode == 1 else H
    X = T * (H * d if mode == 1 else d)
    A = np.empty((G, n, X))
    for g in range(G):
        W0 = np.linalg.qr(rng.standard_normal((X, r_true)))[0]
        c = rng.standard_normal((n, r_true)) * np.sqrt(decay ** np.arange(r_true))
        A[g] = 0.1 * rng.standard_normal(X) + c @ W0.T + noise * rng.standard_normal((n, X))
    if mode == 1:
        x = A[0].reshape(n, T, H, d)
    else:
        x = np.transpose(A.reshape(H, n, T, d), (1, 2, 0, 3))
    return synth.quantize(x, "bf16")


CASES = {                                    # (mode, T, H, d, r, n[, factor decay[, iters]])
    "per_head_X128_r16": (0, 2, 2, 64, 16, 3000),
    "lla2d_X256_r16": (1, 2, 2, 64, 16, 3000),
    "ouro14_X512_r16": (0, 4, 2, 128, 16, 4096),
    "ouro14_X512_r32": (0, 4, 2, 128, 32, 4096),
    "odd_rank_r13": (0, 2, 2, 64, 13, 700),
    # block widths r + 8 of 16, 56 and 72 columns (the kernels' 1, 4 and 5 column tiles); the
    # larger ranks get a slower spectrum so every planted direction stays well above the noise
    "r8_block16": (0, 2, 2, 64, 8, 2000),
    "r48_block56": (0, 2, 2, 64, 48, 3000, 0.95),
    "r64_block72": (0, 2, 1, 128, 64, 3000, 0.95),
    # the 4x codec's ranks: blocks of 104 and 168 columns (7 and 11 column tiles), per head and
    # LLA-2D; a slow spectrum keeps all r + 12 planted directions above the noise, and the
    # smaller gaps between them get more iterations
    "r96_block104": (0, 4, 1, 128, 96, 4096, 0.985, 120),
    "r160_block168": (0, 4, 1, 128, 160, 6000, 0.985, 150),
    "lla2d_r96": (1, 4, 2, 64, 96, 4096, 0.985, 120),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fit_matches_oracle(gpu, name):
    mode, T, H, d, r, n, *rest = CASES[name]
    x = _planted(mode, T, H, d, r + 12, n, seed=len(name), decay=rest[0] if rest else 0.8)
    iters = rest[1] if len(rest) > 1 else 40
    codec = lla.make_codec(mode, T, H, d, r, r, lla.LLA_BF16)
    G = 1 if mode == 1 else H
    X = T * (H * d if mode == 1 else d)
    Dg = X // T
    ws_bytes = lla.lla_fit_plan(codec, r, n)
    ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device=gpu)
    xd = synth.to_device(x, "bf16", gpu)
    mu = torch.empty((G, X), dtype=torch.bfloat16, device=gpu)
    Wd = torch.empty((G, X, r), dtype=torch.bfloat16, device=gpu)
    Wu = torch.empty((T, G, r, Dg), dtype=torch.bfloat16, device=gpu)
    sig = torch.empty((G, r), dtype=torch.float32, device=gpu)
    say(f"fit {name}: n={n} X={X} r={r} workspace={ws_bytes >> 20} MiB")
    lla.lla_fit_svd(codec, r, xd, n, iters, mu, Wd, Wu, sig, ws)
    torch.cuda.synchronize()
    mu_o, Wd_o, Wu_o, sig_o = O.fit_svd(mode, T, H, d, r, x)
    mu_g, Wd_g, Wu_g = synth.from_device(mu), synth.from_device(Wd), synth.from_device(Wu)
    sig_g = sig.cpu().double().numpy()
    assert_close(mu_g, mu_o, "bf16", f"{name} mu")
    assert np.max(np.abs(sig_g - sig_o) / sig_o) < 1e-3, f"{name} sigma"
    # W_up is exactly the blocks of W_down
    assert np.array_equal(Wu_g, np.transpose(Wd_g.reshape(G, T, Dg, r), (1, 0, 3, 2)))
    for g in range(G):
        P_g = Wd_g[g] @ Wd_g[g].T
        P_o = Wd_o[g] @ Wd_o[g].T
        assert np.linalg.norm(P_g - P_o, 2) < 1e-2, f"{name} g={g} subspace"
        ref = Wd_o[g].copy()
        for j in range(r):
            # the sign convention is a decision on the largest magnitude: where the two largest
            # magnitudes of a column are within rounding of each other either sign is valid
            top2 = np.sort(np.abs(ref[:, j]))[-2:]
            gtop2 = np.sort(np.abs(Wd_g[g][:, j]))[-2:]
            ambiguous = (top2[1] - top2[0] < 1e-2 * top2[1] or
                         gtop2[1] - gtop2[0] < 1e-2 * gtop2[1])
            if ambiguous:
                ref[:, j] *= np.sign(np.dot(ref[:, j], Wd_g[g][:, j]))
            else:
                k = int(np.argmax(np.abs(Wd_g[g][:, j])))
                assert Wd_g[g][k, j] > 0, f"{name}: sign convention, column {j}"
        assert_close(Wd_g[g], ref, "bf16", f"{name} W_down g={g}")
