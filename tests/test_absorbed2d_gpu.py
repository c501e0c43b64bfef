"""The all-heads absorbed LLA-2D decode (lla_decode_attn_absorbed on plan kernel 4: one workgroup
per (sequence, context split) serves every head) against the oracle's explicit reconstruction
(exact up to rounding without a rotation; the oracle pin P5 checks that identity).

Covered: every (d, r_k, r_v) the kernel takes, head counts 1..16 (fewer than 16 heads leave
zero-padded MMA columns), ragged and empty sequences, the self term on and off, several context
splits, boundary needles aimed at one head (the 16-token score blocks, the 32-token chunks, the
128-token split unit, split edges and the last token), the headline LLA-2D shape at full size,
and bitwise determinism.  Bar: bf16 max|gpu - oracle| <= 2e-2 max|oracle| + 1e-3.
"""
import sys

import numpy as np
import pytest
import torch

from looped_transformer_kv_amd import lla, synth
import gpucase
import tinycase
from gpucase import assert_close, tol

pytestmark = pytest.mark.gpu

# (d, r_k, r_v, H): every rank pair with r_k % 32 == 0 at both head dims, several head counts
SHAPES = [(128, 96, 160, 16), (64, 96, 160, 16), (128, 96, 160, 7), (128, 32, 32, 16),
          (64, 32, 32, 2), (128, 32, 64, 5), (64, 32, 64, 16), (128, 64, 64, 1), (64, 64, 64, 9),
          (128, 64, 128, 16), (64, 64, 128, 3)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _cfg(i, d, r_k, r_v, H, T=4):
    return synth.Config(f"abs2d_{d}_{r_k}_{r_v}_h{H}", L=1, H=H, d=d, T=T, r_k=r_k, r_v=r_v,
                        B=3, N=1, mode=1, cid=400 + i)


def _check_plan(dp, B, lens):
    plan = dp.layer.absorbed_plan
    assert plan.kernel == 4
    assert plan.splits * plan.tokens_per_split >= int(max(lens))
    return plan


@pytest.mark.parametrize("with_self", [True, False], ids=["self", "noself"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"d{d}_r{a}_{b}_h{h}" for d, a, b, h in SHAPES])
def test_absorbed2d_small(gpu, shape, with_self):
    cfg = _cfg(SHAPES.index(shape), *shape)
    lens = np.array([0, 1, 263, 300, 31, 129], dtype=np.int32)
    p = tinycase.make(cfg, B=len(lens), N=300, lens=lens)
    dp = gpucase.DeviceProblem(p)
    plan = _check_plan(dp, len(lens), lens)
    for t in (0, cfg.T - 1):
        say(f"absorbed 2D {cfg.name} self={with_self} splits={plan.splits} t={t}")
        got = dp.decode(t, with_self, absorbed=True)
        ref = dp.oracle_decode(t, with_self)
        assert_close(got, ref, "bf16", f"{cfg.name} self={with_self} t={t}")
        if not with_self:
            assert np.all(got[0] == 0.0)                    # empty context, no self term


def test_absorbed2d_many_splits_and_tails(gpu):
    """Two long sequences (9 and 6 splits of 128 tokens) and short ones in the same call."""
    cfg = synth.scaled(synth.CONFIGS["ouro26_2d_64x"], B=4, N=1100)
    lens = np.array([1100, 701, 5, 128], dtype=np.int32)
    p = tinycase.make(cfg, B=4, N=1100, lens=lens)
    dp = gpucase.DeviceProblem(p)
    plan = _check_plan(dp, 4, lens)
    assert plan.splits == 9 and plan.tokens_per_split == 128
    for t in (1, 3):
        say(f"absorbed 2D split tails t={t}")
        assert_close(dp.decode(t, True, absorbed=True), dp.oracle_decode(t, True), "bf16",
                     f"split tails t={t}")


def _plant_2d(p, t, b, pos, head, margin=25.0):
    """Overwrite cached token `pos` of sequence b with a key latent aligned with head `head`'s
    absorbed query, so that its score for that head beats every other by `margin`, and scale its
    value latent by 8."""
    c = p.cfg
    scale = 1.0 / np.sqrt(c.d)
    page, slot = p.block_table[b, pos // c.page], pos % c.page
    qh = p.q[t][b, head]
    W = p.W_up_k[t, 0][:, head * c.d:(head + 1) * c.d]        # [r_k][d]
    mu = p.mu_k[0, t * c.Dg + head * c.d: t * c.Dg + (head + 1) * c.d]
    u = W @ qh
    L = int(p.seq_lens[b])
    lat = np.stack([p.k_pool[p.block_table[b, j // c.page], 0, j % c.page] for j in range(L)])
    others = scale * np.abs((lat @ W + mu) @ qh).max()
    self_s = scale * abs(float(qh @ p.x_k[b, t, head]))
    alpha = (margin + others + self_s + scale * abs(float(mu @ qh))) / (scale * np.linalg.norm(u))
    p.k_pool[page, 0, slot, :] = synth.quantize(alpha * u / np.linalg.norm(u), "bf16")
    # the latent spans all heads, so one head's slice of a value moves little; a louder value
    # latent makes the needle's pull on the output far larger than the bar
    p.v_pool[page, 0, slot, :] = synth.quantize(8.0 * p.v_pool[page, 0, slot, :], "bf16")


@pytest.mark.parametrize("group", [0, 1])
def test_absorbed2d_needles(gpu, group):
    """One decisive token per sequence, aimed at one head, at the kernel's boundaries: score block
    edges 15/16, chunk edges 31/32 and 63, split edges (128-token splits: 127/128/129, 255/256,
    383/384, 511/512), the first and the last token."""
    cfg = synth.scaled(synth.CONFIGS["ouro26_2d_64x"], B=8, N=700)
    positions = [[0, 15, 16, 31, 32, 127, 128, 129], [255, 256, 383, 384, 511, 512, 699, 63]][group]
    B = len(positions)
    lens = np.full(B, 700, dtype=np.int32)
    t = 2
    p = tinycase.make(cfg, B=B, N=700, lens=lens, q_gain=8.0)
    ref_without = gpucase.DeviceProblem(p).oracle_decode(t, True)
    heads = [(3 * b + group) % cfg.H for b in range(B)]
    for b, pos in enumerate(positions):
        _plant_2d(p, t, b, pos, heads[b])
    dp = gpucase.DeviceProblem(p)
    plan = _check_plan(dp, B, lens)
    say(f"absorbed 2D needles {positions} heads {heads} splits={plan.splits}")
    ref = dp.oracle_decode(t, True)
    bound = tol("bf16")(ref)
    for b in range(B):
        moved = np.max(np.abs(ref[b, heads[b]] - ref_without[b, heads[b]]))
        assert moved > 10 * bound, f"needle at {positions[b]} moves the oracle by {moved:.3e}"
    got = dp.decode(t, True, absorbed=True)
    assert_close(got, ref, "bf16", f"absorbed 2D needles {positions}")


def test_absorbed2d_deterministic(gpu):
    cfg = synth.scaled(synth.CONFIGS["ouro26_2d_64x"], B=5, N=900)
    p = tinycase.make(cfg, B=5, N=900, ragged=True)
    dp = gpucase.DeviceProblem(p)
    a = dp.decode(1, True, absorbed=True)
    b = dp.decode(1, True, absorbed=True)
    assert np.array_equal(a, b)


def test_absorbed2d_full_size(gpu):
    """ouro26_2d_64x at its full batch and context (B = 16, 16384 tokens, 32 splits): the sampled
    oracle on the last sequence, and the reconstructing kernel on every output, both within the
    bar."""
    from test_parity_gpu import _full_layer, _sampled_oracle
    cfg = synth.CONFIGS["ouro26_2d_64x"]
    layer, host = _full_layer(cfg, gpu)
    assert layer.absorbed_plan.kernel == 4
    sel = [cfg.B - 1]
    xk = synth.staging(cfg, 0, synth.AX_K, cfg.B)
    xv = synth.staging(cfg, 0, synth.AX_V, cfg.B)
    xkd, xvd = synth.to_device(xk, "bf16", gpu), synth.to_device(xv, "bf16", gpu)
    ws = layer.workspace(gpu)
    t = cfg.T - 1
    q = synth.queries(cfg, 0, t, cfg.B)
    qd = synth.to_device(q, "bf16", gpu)
    outs = []
    for absorbed in (False, True):
        out = torch.full((cfg.B, cfg.H, cfg.d), float("nan"), dtype=torch.bfloat16, device=gpu)
        run = layer.decode_absorbed if absorbed else layer.decode
        say(f"2D full size absorbed={absorbed} splits="
            f"{(layer.absorbed_plan if absorbed else layer.plan).splits}")
        run(t, qd, out, ws, xkd[:, t], xvd[:, t], cfg.T * cfg.H * cfg.d)
        torch.cuda.synchronize()
        outs.append(synth.from_device(out))
    say("2D full size: oracle on the last sequence")
    ref = _sampled_oracle(cfg, layer, host, sel, t, q, xk[:, t], xv[:, t])
    assert_close(outs[1][sel], ref, "bf16", "absorbed 2D full size vs oracle")
    assert_close(outs[1], outs[0], "bf16", "absorbed 2D vs reconstructing kernel")
