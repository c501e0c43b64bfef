"""Boundary needles: one decisive cached token (its key aligned with the query, the query scaled
x 8) placed at every boundary the kernels tile by: the first and last token of a 32-token chunk,
of a 64-token page, of a context split (tokens_per_split), of a 256-token prefill step and of
the sequence.  With the configs' near-uniform softmax a dropped or double-counted token moves the
output by far less than the parity bar; a needle moves it by far more, so an off-by-one at any of
these boundaries fails here.  Each case also asserts that power on the oracle itself: removing
the needle must change the oracle's output by more than 10 times the bar.

Covered: lla_decode_attn, lla_decode_attn_absorbed and lla_decode_attn_rope (both pairings) with
one context split and with several, and both passes of lla_prefill_attn (needles in the cached
context, and in the chunk on and just past the causal diagonal).
Bar: bf16 max|gpu - oracle| <= 2e-2 max|oracle| + 1e-3.
"""
import sys

import numpy as np
import pytest
import torch

from looped_transformer_kv_amd import lla, synth
from oracle import oracle as O
import gpucase
import tinycase
from gpucase import Chunk, assert_close, tol

pytestmark = pytest.mark.gpu
CFG = synth.CONFIGS["ouro14_21x"]
MARGIN = 25.0          # needle score above every other score (natural-log units)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _rotate_back(q, pos, style, theta=10000.0):
    """q rotated by -pos (RoFormer rotation, pair m turns by pos * theta^(-2m/d)), so that
    <q, R_pos k> = <R_pos^T q, k>; used only to aim a needle under the rotary decode."""
    d = q.shape[-1]
    out = np.array(q, dtype=np.float64)
    for m in range(d // 2):
        i, j = (2 * m, 2 * m + 1) if style else (m, m + d // 2)
        phi = -pos * theta ** (-2.0 * m / d)
        c, s = np.cos(phi), np.sin(phi)
        out[..., i], out[..., j] = q[..., i] * c - q[..., j] * s, q[..., i] * s + q[..., j] * c
    return out


def _plant(p, t, b, pos, q_bh, rope_style=None):
    """Overwrite cached token `pos` of sequence b with a key latent aligned with q (per head), so
    that its score beats every other score of that sequence by MARGIN; returns the old latents."""
    c = p.cfg
    scale = 1.0 / np.sqrt(c.d)
    page, slot = p.block_table[b, pos // c.page], pos % c.page
    old = p.k_pool[page, :, slot, :].copy()
    for h in range(c.H):
        W = p.W_up_k[t, h]                                    # [r_k][d]
        mu = p.mu_k[h, t * c.d:(t + 1) * c.d]
        qa = q_bh[h] if rope_style is None else _rotate_back(q_bh[h], pos, rope_style)
        u = W @ qa
        L = int(p.seq_lens[b])
        lat = np.stack([p.k_pool[p.block_table[b, j // c.page], h, j % c.page] for j in range(L)])
        others = scale * np.abs((lat @ W + mu) @ qa).max()    # upper bound on the other scores
        self_s = scale * abs(float(q_bh[h] @ p.x_k[b, t, h]))
        alpha = (MARGIN + others + self_s + scale * abs(float(mu @ qa))) / (scale * np.linalg.norm(u))
        p.k_pool[page, h, slot, :] = synth.quantize(alpha * u / np.linalg.norm(u), "bf16")
    return old


def _check_power(ref_with, ref_without, sel, what):
    for b in sel:
        moved = np.max(np.abs(ref_with[b] - ref_without[b]))
        bound = tol("bf16")(ref_with)
        assert moved > 10 * bound, f"{what}: needle in sequence {b} moves the oracle by only {moved:.3e}"


def _decode_case(lens, needles, form, t=1):
    """needles: {sequence: position}.  Returns nothing; asserts parity and power."""
    B = len(lens)
    p = tinycase.make(CFG, B=B, N=int(max(lens)), lens=np.asarray(lens, np.int32), q_gain=8.0)
    rope = None
    if form.startswith("rope"):
        rope = lla.lla_rope(10000.0, CFG.d, 0 if form == "rope_half" else 1)
    base = gpucase.DeviceProblem(p)
    ref_without = (base.oracle_decode_rope(t, rope, True) if rope is not None
                   else base.oracle_decode(t, True))
    for b, pos in needles.items():
        _plant(p, t, b, pos, p.q[t][b], None if rope is None else rope.style)
    dp = gpucase.DeviceProblem(p)
    plan = dp.layer.plan
    say(f"needles {form} splits={plan.splits} tps={plan.tokens_per_split} {needles}")
    if rope is not None:
        ref = dp.oracle_decode_rope(t, rope, True)
        got = dp.decode(t, True, rope=rope)
    else:
        ref = dp.oracle_decode(t, True)
        got = dp.decode(t, True, absorbed=form == "absorbed")
    _check_power(ref, ref_without, needles, form)
    assert_close(got, ref, "bf16", f"needles {form} {needles}")
    return plan


FORMS = ["plain", "absorbed", "rope_half", "rope_interleaved"]


@pytest.mark.parametrize("form", FORMS)
def test_decode_needles_one_split(gpu, form):
    """32 sequences (one split each): needles at chunk edges 31/32, page edges 63/64, the edges of
    each wave's chunk group (127/128, 255/256), the first and the last cached token, including
    sequences whose last chunk holds a single token."""
    pairs = [(300, 0), (300, 31), (300, 32), (300, 63), (300, 64), (300, 127), (300, 128),
             (300, 255), (300, 256), (300, 299), (257, 256), (33, 32), (64, 63), (1, 0), (65, 64),
             (129, 128), (32, 31)]
    lens = [L for L, _ in pairs] + [300] * (32 - len(pairs))
    needles = {b: pos for b, (_, pos) in enumerate(pairs)}
    plan = _decode_case(lens, needles, form)
    assert plan.splits == 1


@pytest.mark.parametrize("group", [0, 1, 2])
@pytest.mark.parametrize("form", FORMS)
def test_decode_needles_split_context(gpu, form, group):
    """4 sequences of 1100 tokens: the plan splits the context (tokens_per_split 256); needles at
    every split edge (tps - 1, tps, tps + 1, ...) and the last token."""
    lens = [1100, 1100, 1100, 1100]
    positions = [[255, 256, 257, 1099], [511, 512, 0, 767], [768, 1023, 1024, 1025]][group]
    plan = _decode_case(lens, dict(enumerate(positions)), form)
    assert plan.splits > 1 and plan.tokens_per_split == 256


# ------------------------------------------------------------------ prefill
def _prefill_power(ch, t, rows, ref_with, what):
    """The oracle without the planted keys differs by > 10x the bar on the aimed query rows."""
    ref_without = ch.oracle_with(t, *ch.saved)
    bound = tol("bf16")(ref_with)
    for b, i in rows:
        moved = np.max(np.abs(ref_with[b, i] - ref_without[b, i]))
        assert moved > 10 * bound, f"{what}: row ({b},{i}) moves by only {moved:.3e}"


class NeedleChunk(Chunk):
    def oracle_with(self, t, k_pool, xk):
        p, c = self.p, self.cfg
        return O.prefill(c.mode, c.T, c.H, c.d, c.r_k, c.r_v, t, p.W_up_k, p.W_up_v, p.mu_k,
                         p.mu_v, k_pool, p.v_pool, p.block_table, p.seq_lens, c.page, self.q[t],
                         xk[:, :, t], self.xv[:, :, t], self.n_new)

    def upload(self):
        self.dp.k_pool.copy_(synth.to_device(self.p.k_pool, "bf16", self.gpu))
        self.xkd = synth.to_device(self.xk, "bf16", self.gpu)
        torch.cuda.synchronize()


PREFILL_CODECS = ["ouro14_21x", "ouro14_4x"]    # two passes (r <= 32); fused kernel (96 / 160)


@pytest.mark.parametrize("codec", PREFILL_CODECS)
def test_prefill_needles_cached_pass(gpu, codec):
    """Needles in the cached context (latents) at tile edges 31/32, 256-token step edges 255/256,
    the first and the last cached token; each aimed at one query row of the chunk."""
    cfg = synth.CONFIGS[codec]
    t = 2
    lens = [300, 300, 300, 300, 257, 300]
    pos = [0, 31, 32, 255, 256, 299]
    aim = [0, 5, 63, 64, 1, 100]                       # query row each needle is aimed at
    ch = NeedleChunk(cfg, len(lens), 300, 128, lens, [128] * len(lens), gpu, q_gain=8.0)
    ch.saved = (ch.p.k_pool.copy(), ch.xk.copy())
    for b in range(len(lens)):
        _plant(ch.p, t, b, pos[b], ch.q[t][b, aim[b]])
    ch.upload()
    say(f"prefill {codec} cached-pass needles at {pos}")
    ref = ch.oracle(t)
    _prefill_power(ch, t, list(enumerate(aim)), ref, "cached pass")
    ch.check(ch.run(t), ref, "prefill cached-pass needles")


@pytest.mark.parametrize("codec", PREFILL_CODECS)
def test_prefill_needles_chunk_pass(gpu, codec):
    """Needles among the chunk's own keys at chunk positions 0, 31, 32, 255, 256 and the last live
    row, each aimed at the query on the causal diagonal (it must be seen) and, in a second
    sequence, at the query just before it (it must not be)."""
    cfg = synth.CONFIGS[codec]
    t = 1
    Pn = 300
    pos = [0, 31, 32, 255, 256, 299]
    B = 2 * len(pos)
    lens = [200] * B
    ch = NeedleChunk(cfg, B, 200, Pn, lens, [Pn] * B, gpu, q_gain=8.0)
    ch.saved = (ch.p.k_pool.copy(), ch.xk.copy())
    scale = 1.0 / np.sqrt(cfg.d)
    seen = []
    for k, i0 in enumerate(pos):
        for b, i1 in ((2 * k, i0), (2 * k + 1, max(i0 - 1, 0))):
            if b == 2 * k + 1 and i0 == 0:
                continue                                  # no query before the first row
            qa = ch.q[t][b, i1]                           # [H][d]
            n = np.linalg.norm(qa, axis=-1, keepdims=True)
            # every other score of row i1 is at most scale |q| |k|; beat it by MARGIN
            kmax = np.abs(ch.xk[b, :, t]).max() * np.sqrt(cfg.d)
            alpha = (MARGIN + scale * n * kmax + 50.0) / (scale * n)
            ch.xk[b, i0, t] = synth.quantize(alpha * qa / n, "bf16")
            if b == 2 * k:
                seen.append((b, i1))
    ch.upload()
    say(f"prefill {codec} chunk-pass needles at {pos}")
    ref = ch.oracle(t)
    _prefill_power(ch, t, seen, ref, "chunk pass")
    ch.check(ch.run(t), ref, "prefill chunk-pass needles")
