"""GPU parity of the chunked prefill (lla_prefill_attn) and the bulk encode (lla_encode_chunk),
through the C ABI, against the fp64 oracle on seeded inputs.

Bar (as for decode): bf16 max|gpu - oracle| <= 2e-2 max|oracle| + 1e-3 over the live rows; rows
past a sequence's chunk size must stay untouched.  Small cases span two query blocks of 256,
several 32-token tiles of cached context and of chunk, ragged tails, empty contexts and empty
chunks, for every (d, r_k, r_v) the library accepts: the two-pass kernels of ranks up to 32 and
the fused kernel of the wider pairs, per-head and LLA-2D.  The full-size cases run the benchmark's
launch (the codec's batch x 4096 cached tokens, a chunk of 512) and check sampled sequences.
"""
import sys

import numpy as np
import pytest
import torch

from looped_transformer_kv_amd import lla, synth
from looped_transformer_kv_amd.runtime import LatentLayer
from oracle import oracle as O
import gpucase
import tinycase
from gpucase import Chunk, assert_close

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# codec shapes the prefill kernel instantiates: (mode, H, d, T, r_k, r_v)
SHAPES = {
    "ouro14_21x": synth.CONFIGS["ouro14_21x"],
    "h4_d128_2d_r32": synth.Config("pf_2d", L=1, H=4, d=128, T=2, r_k=32, r_v=32, B=1, N=1,
                                   mode=1, cid=140),
    "h2_d64_r16": synth.Config("pf_d64", L=1, H=2, d=64, T=3, r_k=16, r_v=16, B=1, N=1, cid=141),
    "h2_d64_2d_r16_32": synth.Config("pf_d64_2d", L=1, H=2, d=64, T=2, r_k=16, r_v=32, B=1, N=1,
                                     mode=1, cid=142),
    "h4_d128_r16_16": synth.Config("pf_d128_r16", L=1, H=4, d=128, T=4, r_k=16, r_v=16, B=1, N=1,
                                   cid=143),
    "h2_d64_r32_32": synth.Config("pf_d64_r32", L=1, H=2, d=64, T=4, r_k=32, r_v=32, B=1, N=1,
                                  cid=144),
    # the fused kernel of the wider rank pairs
    "h2_d128_r96_160": synth.Config("pf_d128_r96", L=1, H=2, d=128, T=4, r_k=96, r_v=160, B=1,
                                    N=1, cid=145),
    "h4_d128_2d_r96_160": synth.Config("pf_2d_r96", L=1, H=4, d=128, T=2, r_k=96, r_v=160, B=1,
                                       N=1, mode=1, cid=146),
    "h2_d64_r96_160": synth.Config("pf_d64_r96", L=1, H=2, d=64, T=3, r_k=96, r_v=160, B=1, N=1,
                                   cid=147),
    "h2_d128_r32_64": synth.Config("pf_d128_r32_64", L=1, H=2, d=128, T=4, r_k=32, r_v=64, B=1,
                                   N=1, cid=148),
    "h3_d64_2d_r32_64": synth.Config("pf_d64_2d_r32_64", L=1, H=3, d=64, T=2, r_k=32, r_v=64,
                                     B=1, N=1, mode=1, cid=149),
    "h2_d128_2d_r64_64": synth.Config("pf_d128_2d_r64", L=1, H=2, d=128, T=4, r_k=64, r_v=64,
                                      B=1, N=1, mode=1, cid=150),
    "h2_d64_r64_64": synth.Config("pf_d64_r64", L=1, H=2, d=64, T=4, r_k=64, r_v=64, B=1, N=1,
                                  cid=151),
    "h2_d128_r64_128": synth.Config("pf_d128_r64_128", L=1, H=2, d=128, T=3, r_k=64, r_v=128,
                                    B=1, N=1, cid=152),
    "h2_d64_r64_128": synth.Config("pf_d64_r64_128", L=1, H=2, d=64, T=4, r_k=64, r_v=128, B=1,
                                   N=1, cid=153),
}



@pytest.mark.parametrize("shape", list(SHAPES))
def test_prefill_small(gpu, shape):
    """Two query blocks (Pn = 300), ragged cached lengths including 0 and a partial tile, ragged
    chunk sizes including 0 and Pn."""
    cfg = SHAPES[shape]
    lens, n_new = [0, 137, 64], [300, 0, 77]
    ch = Chunk(cfg, 3, 137, 300, lens, n_new, gpu)
    for t in sorted({0, cfg.T - 1}):
        for strided in (True, False):
            say(f"prefill {shape} t={t} strided={strided} lens={lens} n_new={n_new}")
            ch.check(ch.run(t, strided), ch.oracle(t), f"{shape} t={t}")


@pytest.mark.parametrize("codec", ["ouro14_21x", "ouro14_4x"])
@pytest.mark.parametrize("variant", ["peaked", "long_context", "tiny_chunks"])
def test_prefill_variants(gpu, variant, codec):
    """The headline codec (two passes) and the 4x codec (ranks 96 / 160: the fused kernel)."""
    cfg = synth.CONFIGS[codec]
    if variant == "peaked":            # sharp softmax: q x 8
        ch = Chunk(cfg, 2, 500, 64, [500, 31], [64, 33], gpu, q_gain=8.0)
    elif variant == "long_context":    # context much longer than the chunk
        ch = Chunk(cfg, 2, 2000, 40, [2000, 1999], [40, 1], gpu)
    else:                              # one-token and two-token chunks, empty context
        ch = Chunk(cfg, 4, 70, 2, [0, 70, 1, 33], [1, 2, 2, 1], gpu)
    t = cfg.T - 1
    say(f"prefill {codec} {variant}")
    ch.check(ch.run(t), ch.oracle(t), f"{codec} {variant}")


def test_prefill_single_token_chunk_matches_decode(gpu):
    """A chunk of one token is the decode step with that token as its self term (oracle pin F1):
    the prefill kernel and the decode kernel both meet the oracle on the same inputs."""
    cfg = SHAPES["ouro14_21x"]
    ch = Chunk(cfg, 3, 300, 1, [300, 5, 0], [1, 1, 1], gpu)
    c = ch.cfg
    t = 1
    say("prefill one-token chunk vs decode")
    got = ch.run(t)[:, 0]
    ref = ch.oracle(t)[:, 0]
    assert_close(got, ref, "bf16", "prefill, one token")
    out = torch.empty((3, c.H, c.d), dtype=torch.bfloat16, device=gpu)
    layer = ch.dp.layer
    layer.decode(t, ch.qd[t][:, 0].contiguous(), out, layer.workspace(gpu), ch.xkd[:, 0, t],
                 ch.xvd[:, 0, t], c.T * c.H * c.d)
    torch.cuda.synchronize()
    assert_close(synth.from_device(out), ref, "bf16", "decode with the chunk token as self")


def _check_encode_chunk(gpu, shape, B, N, Pn, lens, n_new, shapes=None):
    """lla_encode_chunk: c against the oracle; the pool holds c rounded once at write_pos + i for
    live rows only; every other slot keeps its bytes."""
    cfg = (shapes or SHAPES)[shape]
    ch = Chunk(cfg, B, N, Pn, lens, n_new, gpu)
    c, p = ch.cfg, ch.p
    wpos_h = p.seq_lens.copy()
    wpos = torch.from_numpy(wpos_h).to(gpu)
    ck = torch.full((B, Pn, c.G, c.r_k), float("nan"), dtype=torch.float32, device=gpu)
    cv = torch.full((B, Pn, c.G, c.r_v), float("nan"), dtype=torch.float32, device=gpu)
    kb, vb = synth.from_device(ch.dp.k_pool), synth.from_device(ch.dp.v_pool)
    say(f"encode_chunk {shape} B={B} Pn={Pn}")
    ch.dp.layer.encode_chunk(Pn, ch.nd, ch.xkd, ch.xvd, wpos, ck, cv)
    torch.cuda.synchronize()
    live = np.arange(Pn)[None, :] < ch.n_new[:, None]
    for axis, cgpu, W, mu, r, before, pool, x in (
            (0, ck, p.W_down_k, p.mu_k, c.r_k, kb, ch.dp.k_pool, ch.xk),
            (1, cv, p.W_down_v, p.mu_v, c.r_v, vb, ch.dp.v_pool, ch.xv)):
        got = cgpu.double().cpu().numpy()
        ref, _ = O.encode_prefill(c.mode, c.T, c.H, c.d, r, W, mu, x, wpos_h, ch.n_new,
                                  p.block_table, c.page, before)
        assert np.all(np.isnan(got[~live])), f"axis {axis}: rows past the chunk were written"
        assert_close(got[live], ref[live], "bf16", f"{shape} c axis {axis}")
        # the pool: the rounding of the kernel's own c, at write_pos + i, live rows only
        stored = synth.quantize(np.nan_to_num(got), "bf16")
        expect = before.copy()
        for b in range(B):
            for i in range(int(ch.n_new[b])):
                pos = wpos_h[b] + i
                expect[p.block_table[b, pos // c.page], :, pos % c.page] = stored[b, i]
        after = synth.from_device(pool)
        assert np.array_equal(after, expect), f"{shape} axis {axis}: pool differs"


@pytest.mark.parametrize("shape,Pn", [("ouro14_21x", 70), ("h4_d128_2d_r32", 70),
                                      ("ouro14_21x", 100), ("h2_d64_r16", 100)])
def test_encode_chunk(gpu, shape, Pn):
    """A few hundred rows: the split-axis kernel."""
    _check_encode_chunk(gpu, shape, 3, 90, Pn, [90, 0, 33], [Pn, 0, 41])


# codecs whose bulk encode takes the wide-rank GEMM (both ranks multiples of 32, one >= 64, at
# least 1024 rows): per head and LLA-2D, stacked axes from 128 (2 chunks of 64) to 4096
# (32 loops, the Huginn shape per head)
WIDE_ENCODE = {
    "ouro14_4x": (synth.CONFIGS["ouro14_4x"], 4, 70, 512, [70, 0, 33, 64], [512, 300, 0, 511]),
    "2d_h4_r96_160": (synth.Config("enc_2d", L=1, H=4, d=128, T=4, r_k=96, r_v=160, B=1, N=1,
                                   mode=1, cid=160), 4, 40, 300, [40, 7, 0, 31], [300, 299, 1, 0]),
    "t32_h2_r96_160": (synth.Config("enc_t32", L=1, H=2, d=128, T=32, r_k=96, r_v=160, B=1,
                                    N=1, cid=161), 2, 64, 512, [64, 5], [512, 480]),
    "d64_r32_64": (synth.Config("enc_d64", L=1, H=2, d=64, T=2, r_k=32, r_v=64, B=1, N=1,
                                cid=162), 8, 20, 128, [20, 0, 3, 19, 17, 1, 7, 8],
                   [128, 127, 0, 64, 128, 1, 99, 128]),
    "2d_d128_r64_64": (synth.Config("enc_2d64", L=1, H=2, d=128, T=2, r_k=64, r_v=64, B=1, N=1,
                                    mode=1, cid=163), 4, 10, 256, [10, 0, 5, 9], [256, 200, 256, 3]),
    "d128_r64_128": (synth.Config("enc_r128", L=1, H=2, d=128, T=3, r_k=64, r_v=128, B=1, N=1,
                                  cid=164), 4, 10, 256, [10, 1, 0, 9], [256, 255, 100, 256]),
}


@pytest.mark.parametrize("name", list(WIDE_ENCODE))
def test_encode_chunk_wide_ranks(gpu, name):
    """Thousands of rows of the wider rank pairs: the GEMM kernel (W_down staged per 64-element
    chunk, rows centred on the way), with empty, full and ragged chunks, writes starting
    mid-page and rows past a chunk left alone."""
    cfg, B, N, Pn, lens, n_new = WIDE_ENCODE[name]
    assert B * Pn >= 1024 and max(lens) <= N
    _check_encode_chunk(gpu, name, B, N, Pn, lens, n_new, shapes={name: cfg})


def test_encode_chunk_row_streaming(gpu):
    """4096 rows of a short stacked axis over 16 heads (256 workgroups, one per CU): the
    row-streaming kernel, with empty, full and ragged chunks and writes starting mid-page."""
    _check_encode_chunk(gpu, "ouro14_21x", 8, 64, 512, [64, 0, 33, 5, 64, 17, 40, 1],
                        [512, 0, 512, 300, 7, 511, 512, 64])


@pytest.mark.parametrize("codec", ["ouro14_21x", "ouro14_4x", "ouro26_2d_64x"])
def test_prefill_bench_shape_sampled(gpu, codec):
    """The benchmark's launch on each codec it times prefill for: the codec's batch x 4096 cached
    tokens, a chunk of 512, all 16 heads (per-head codecs at ranks 16 / 32 and 96 / 160, and the
    LLA-2D codec); the oracle checks three sampled sequences."""
    cfg = synth.CONFIGS[codec]
    B, N, Pn = cfg.B, cfg.N, 512
    cfgp = synth.scaled(cfg, N=N + Pn)
    max_pages = cfgp.max_pages
    n_pages = B * max_pages
    Wdk, Wuk, muk = synth.codec(cfg, 0, synth.AX_K)
    Wdv, Wuv, muv = synth.codec(cfg, 0, synth.AX_V)
    kpool = synth.device_latent_pool(cfg, 0, synth.AX_K, n_pages, gpu)
    vpool = synth.device_latent_pool(cfg, 0, synth.AX_V, n_pages, gpu)
    bt = synth.block_table(cfgp, B, max_pages)
    lens = synth.seq_lens(cfg, B, N)
    up = lambda a: synth.to_device(a, "bf16", gpu)
    cd = lla.make_codec(cfg.mode, cfg.T, cfg.H, cfg.d, cfg.r_k, cfg.r_v, lla.LLA_BF16)
    layer = LatentLayer(cd, up(Wdk), up(Wdv), up(Wuk), up(Wuv), up(muk), up(muv), kpool, vpool,
                        torch.from_numpy(bt).to(gpu), torch.from_numpy(lens).to(gpu), cfg.page, N)
    t = cfg.T - 1
    q = synth.chunk_queries(cfg, 0, t, B, Pn)
    xk = synth.chunk_staging(cfg, 0, synth.AX_K, B, Pn)
    xv = synth.chunk_staging(cfg, 0, synth.AX_V, B, Pn)
    n_new = np.full(B, Pn, dtype=np.int32)
    xkd, xvd = up(xk), up(xv)
    out = torch.empty((B, Pn, cfg.H, cfg.d), dtype=torch.bfloat16, device=gpu)
    say(f"prefill full size {codec} B={B} N={N} Pn={Pn}")
    layer.prefill(t, Pn, torch.from_numpy(n_new).to(gpu), up(q), xkd[:, :, t], xvd[:, :, t], out,
                  new_stride=cfg.T * cfg.H * cfg.d)
    torch.cuda.synchronize()
    got = synth.from_device(out)
    assert np.all(np.isfinite(got))
    sel = [0, B // 2, B - 1]
    pages = np.unique(bt[sel])
    remap = {int(pg): i for i, pg in enumerate(pages)}
    bt2 = np.vectorize(lambda x: remap[int(x)])(bt[sel]).astype(np.int32)
    idx = torch.from_numpy(pages.astype(np.int64)).to(gpu)
    kp = synth.from_device(kpool.index_select(0, idx))
    vp = synth.from_device(vpool.index_select(0, idx))
    say(f"prefill full size: oracle on sequences {sel}")
    ref = O.prefill(cfg.mode, cfg.T, cfg.H, cfg.d, cfg.r_k, cfg.r_v, t, Wuk, Wuv, muk, muv, kp, vp, bt2,
                    lens[sel], cfg.page, q[sel], xk[sel][:, :, t], xv[sel][:, :, t], n_new[sel])
    assert_close(got[sel], ref, "bf16", f"prefill full size {codec}")
