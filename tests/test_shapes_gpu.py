"""GPU parity for every shape the C ABI accepts, and for the exact launches the benchmark times.

Decode: each (d_head, r_k, r_v) that lla_decode_attn, _absorbed and _rope accept (the library's
supported-shape check is read through a probe call, so a pair added to it without a test here fails
test_every_accepted_decode_shape_is_listed) against the fp64 oracle, with ragged lengths
including 0 and 1, a self term, and loops 0 and T - 1.  Encode: the benchmark's
lla_encode_append_layers launch (32 sequences, all 24 layers, each layer with its own block
table) read back slot by slot against oracle encode.  Flat comparator: the benchmark's
lla_ref_attn launch (32 sequences x 4096 tokens, one split) on sampled sequences.

Bar: bf16 max|gpu - oracle| <= 2e-2 max|oracle| + 1e-3.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

from looped_transformer_kv_amd import lla, synth
from looped_transformer_kv_amd.runtime import LatentLayer
from oracle import oracle as O
import gpucase
import tinycase
from gpucase import assert_close

DECODE_PAIRS = [(16, 16), (16, 32), (32, 32), (32, 64), (64, 64), (64, 128), (96, 160)]
HEAD_DIMS = [64, 128]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _accepts(d, r_k, r_v):
    """Whether lla_decode_attn accepts a bf16 per-head codec of this shape (validation only: the
    call is made with a zero batch, so nothing is launched)."""
    codec = lla.make_codec(0, 4, 2, d, r_k, r_v, lla.LLA_BF16)
    buf = 0x10000                                # never dereferenced: batch 0 enqueues nothing
    params = lla.lla_params(buf, buf, buf, buf, buf, buf)
    cache = lla.lla_cache(buf, buf, buf, buf, 0, 64, 8, 8, 256)
    st = lla.lib().lla_decode_attn(ctypes.byref(codec), ctypes.byref(params),
                                   ctypes.byref(cache), 0, buf, None, None, 0, 0.1, buf, None, 0,
                                   None)
    return st != lla.LLA_ERR_UNSUPPORTED


def test_every_accepted_decode_shape_is_listed():
    """The shapes below are exactly the ones the library accepts (per-head, bf16, T = 4)."""
    for d in (32, 64, 96, 128):
        for rk in (8, 16, 24, 32, 48, 64, 96, 128, 160):
            for rv in (8, 16, 24, 32, 48, 64, 96, 128, 160, 192):
                if d not in (64, 128) or rk > 4 * d or rv > 4 * d:
                    continue
                listed = (rk, rv) in DECODE_PAIRS
                assert _accepts(d, rk, rv) == listed, (d, rk, rv)


def _cfg(d, r_k, r_v, mode=0):
    # T = 4 keeps X = T * D_g >= r for every pair at d = 64
    return synth.Config(f"shape_d{d}_{r_k}_{r_v}_m{mode}", L=1, H=4 if mode == 0 else 2, d=d,
                        T=4, r_k=r_k, r_v=r_v, B=3, N=1, mode=mode,
                        cid=300 + 10 * HEAD_DIMS.index(d) + DECODE_PAIRS.index((r_k, r_v)) +
                        100 * mode)


def _problem(cfg, q_gain=1.0):
    B, N = 3, 300
    lens = synth.seq_lens(cfg, B, N, ragged=True, salt=11)
    lens[0], lens[1] = 0, 1
    lens[2] = 263                                     # partial last chunk
    p = tinycase.make(cfg, B=B, N=N, lens=lens, q_gain=q_gain)
    return p, gpucase.DeviceProblem(p)


@pytest.mark.gpu
@pytest.mark.parametrize("form", ["plain", "absorbed", "rope_half", "rope_interleaved"])
@pytest.mark.parametrize("pair", DECODE_PAIRS, ids=[f"r{a}_{b}" for a, b in DECODE_PAIRS])
@pytest.mark.parametrize("d", HEAD_DIMS)
def test_decode_every_shape(gpu, d, pair, form):
    cfg = _cfg(d, *pair)
    p, dp = _problem(cfg)
    for t in (0, cfg.T - 1):
        say(f"decode d={d} r={pair} {form} lens={list(p.seq_lens)} t={t}")
        if form.startswith("rope"):
            rope = lla.lla_rope(10000.0, d, 0 if form == "rope_half" else 1)
            got = dp.decode(t, True, rope=rope)
            ref = dp.oracle_decode_rope(t, rope, True)
        else:
            got = dp.decode(t, True, absorbed=form == "absorbed")
            ref = dp.oracle_decode(t, True)
        assert_close(got, ref, "bf16", f"d={d} r={pair} {form} t={t}")


@pytest.mark.gpu
@pytest.mark.parametrize("style", [0, 1])
@pytest.mark.parametrize("pair", [(16, 16), (16, 32)], ids=["r16_16", "r16_32"])
@pytest.mark.parametrize("d", HEAD_DIMS)
def test_rope_odd_head_count(gpu, d, pair, style):
    """Rotary decode of a rank-16 key codec with an odd head count: the kernel that serves two
    heads per wave needs an even count, so these calls take the one-head-per-workgroup kernel."""
    cfg = synth.Config(f"rope_odd_d{d}_{pair[0]}_{pair[1]}", L=1, H=3, d=d, T=4, r_k=pair[0],
                       r_v=pair[1], B=3, N=1, mode=0,
                       cid=500 + 10 * HEAD_DIMS.index(d) + DECODE_PAIRS.index(pair))
    p, dp = _problem(cfg)
    rope = lla.lla_rope(10000.0, d, style)
    for t in (0, cfg.T - 1):
        say(f"rope odd heads d={d} r={pair} style={style} lens={list(p.seq_lens)} t={t}")
        assert_close(dp.decode(t, True, rope=rope), dp.oracle_decode_rope(t, rope, True), "bf16",
                     f"odd heads d={d} r={pair} style={style} t={t}")


@pytest.mark.gpu
@pytest.mark.parametrize("form", ["plain", "absorbed", "rope_half"])
@pytest.mark.parametrize("pair", [(16, 32), (32, 64), (96, 160)],
                         ids=["r16_32", "r32_64", "r96_160"])
@pytest.mark.parametrize("d", HEAD_DIMS)
def test_decode_shapes_lla2d(gpu, d, pair, form):
    """The same instantiations serve LLA-2D codecs (one latent over all heads)."""
    cfg = _cfg(d, *pair, mode=1)
    p, dp = _problem(cfg)
    t = cfg.T - 1
    say(f"decode 2D d={d} r={pair} {form} lens={list(p.seq_lens)}")
    if form == "rope_half":
        rope = lla.lla_rope(10000.0, d, 0)
        assert_close(dp.decode(t, True, rope=rope), dp.oracle_decode_rope(t, rope, True), "bf16",
                     f"2D d={d} r={pair} {form}")
    else:
        assert_close(dp.decode(t, True, absorbed=form == "absorbed"), dp.oracle_decode(t, True),
                     "bf16", f"2D d={d} r={pair} {form}")


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_shapes_cover_the_accepted_set(d):
    """Every (d, r_k, r_v) lla_prefill_attn accepts has a small-case parity test above (a
    validation-only probe: nothing is launched)."""
    from test_prefill_gpu import SHAPES
    tested = {(c.d, c.r_k, c.r_v) for c in SHAPES.values()}
    for rk in (8, 16, 32, 48, 64, 96):
        for rv in (8, 16, 32, 48, 64, 128, 160):
            codec = lla.make_codec(0, 4, 2, d, rk, rv, lla.LLA_BF16)
            st = lla.lib().lla_prefill_attn(ctypes.byref(codec), None, None, 0, 0, None, None,
                                             None, None, 0, 0.1, None, None)
            accepted = st != lla.LLA_ERR_UNSUPPORTED
            assert accepted == ((d, rk, rv) in tested), (d, rk, rv, st)


# ------------------------------------------------------------------ the benchmark's encode launch
@pytest.mark.gpu
def test_bench_encode_launch_against_oracle(gpu):
    """lla_encode_append_layers exactly as the benchmark calls it (headline codec, 32 sequences,
    24 layers, each with its own codec, pools and block table, write position 4096): every written
    slot holds bf16(c) with c within the bar of the oracle's encode, and no other slot changes."""
    cfg = synth.CONFIGS["ouro14_21x"]
    B, L, N = cfg.B, cfg.L, cfg.N
    max_pages = cfg.max_pages
    n_pages = B * max_pages
    layers, host = [], []
    for l in range(L):
        Wdk, Wuk, muk = synth.codec(cfg, l, synth.AX_K)
        Wdv, Wuv, muv = synth.codec(cfg, l, synth.AX_V)
        kp = torch.zeros((n_pages, cfg.G, cfg.page, cfg.r_k), dtype=torch.bfloat16, device=gpu)
        vp = torch.zeros((n_pages, cfg.G, cfg.page, cfg.r_v), dtype=torch.bfloat16, device=gpu)
        bt = synth.block_table(cfg, B, max_pages, salt=100 + l)        # distinct per layer
        lens = np.full(B, N, dtype=np.int32)
        up = lambda a: synth.to_device(a, "bf16", gpu)
        codec = lla.make_codec(0, cfg.T, cfg.H, cfg.d, cfg.r_k, cfg.r_v, lla.LLA_BF16)
        layers.append(LatentLayer(codec, up(Wdk), up(Wdv), up(Wuk), up(Wuv), up(muk), up(muv), kp,
                                  vp, torch.from_numpy(bt).to(gpu), torch.from_numpy(lens).to(gpu),
                                  cfg.page, N))
        xk = synth.staging(cfg, l, synth.AX_K, B)
        xv = synth.staging(cfg, l, synth.AX_V, B)
        host.append(dict(Wdk=Wdk, Wdv=Wdv, muk=muk, muv=muv, bt=bt, xk=xk, xv=xv,
                         xkd=up(xk), xvd=up(xv)))
    pos = torch.full((B,), N, dtype=torch.int32, device=gpu)
    say(f"encode_append_layers: {L} layers, batch {B}")
    LatentLayer.encode_append_layers(layers, [h["xkd"] for h in host], [h["xvd"] for h in host],
                                     pos)
    torch.cuda.synchronize()
    slot = N % cfg.page
    for l in range(L):
        h = host[l]
        page = torch.from_numpy(h["bt"][:, N // cfg.page].astype(np.int64)).to(gpu)
        for axis, r in ((0, cfg.r_k), (1, cfg.r_v)):
            pool = layers[l].tensors["v_pool" if axis else "k_pool"]
            ref = O.encode(0, cfg.T, cfg.H, cfg.d, r, h["Wdv"] if axis else h["Wdk"],
                           h["muv"] if axis else h["muk"], h["xv"] if axis else h["xk"])
            got = synth.from_device(pool.index_select(0, page)[:, :, slot, :])   # [B][G][r]
            assert_close(got, ref, "bf16", f"layer {l} axis {axis} written slots")
            # nothing but the written slots changed: the pools started at zero
            written = int(torch.count_nonzero(pool.index_select(0, page)[:, :, slot, :]))
            assert int(torch.count_nonzero(pool)) == written, f"layer {l} axis {axis}"


# ------------------------------------------------------------------ the benchmark's flat launch
@pytest.mark.gpu
def test_bench_flat_launch_sampled(gpu):
    """lla_ref_attn at the benchmark's shape (32 sequences x 4096 cached tokens, 16 heads, d 128,
    one split), pools drawn on the device, checked on sampled sequences against the oracle."""
    cfg = synth.CONFIGS["ouro14_21x"]
    B, N, H, d, P = 32, cfg.N, cfg.H, cfg.d, cfg.page
    max_pages = cfg.max_pages
    n_pages = B * max_pages
    gen = torch.Generator(device=gpu)
    gen.manual_seed(4242)
    kf = (0.12 * torch.randn((n_pages, H, P, d), generator=gen, device=gpu)).to(torch.bfloat16)
    vf = (0.12 * torch.randn((n_pages, H, P, d), generator=gen, device=gpu)).to(torch.bfloat16)
    bt = synth.block_table(cfg, B, max_pages, salt=77)
    lens = np.full(B, N, dtype=np.int32)
    btd, ld = torch.from_numpy(bt).to(gpu), torch.from_numpy(lens).to(gpu)
    flat = lla.make_cache(kf, vf, btd, ld, P, N)
    plan = lla.lla_ref_plan(H, d, lla.LLA_BF16, flat)
    assert plan.splits == 1
    ws = torch.empty(max(4, plan.workspace_bytes // 4), dtype=torch.float32, device=gpu)
    q = synth.quantize(synth.rng(cfg, 91, 0).standard_normal((B, H, d)), "bf16")
    out = torch.empty((B, H, d), dtype=torch.bfloat16, device=gpu)
    say("flat comparator at the benchmark shape")
    lla.lla_ref_attn(H, d, lla.LLA_BF16, flat, synth.to_device(q, "bf16", gpu), None, None, 0,
                     1.0 / np.sqrt(d), out, ws)
    torch.cuda.synchronize()
    got = synth.from_device(out)
    sel = [0, 13, B - 1]
    pages = np.unique(bt[sel])
    remap = {int(p): i for i, p in enumerate(pages)}
    bt2 = np.vectorize(lambda x: remap[int(x)])(bt[sel]).astype(np.int32)
    idx = torch.from_numpy(pages.astype(np.int64)).to(gpu)
    kp = synth.from_device(kf.index_select(0, idx))
    vp = synth.from_device(vf.index_select(0, idx))
    ref = O.flat_attn(H, d, kp, vp, bt2, lens[sel], P, q[sel])
    assert_close(got[sel], ref, "bf16", "flat comparator, benchmark launch")


F32_SHAPES = [(64, 8, 16), (64, 12, 20), (128, 16, 32), (128, 24, 8)]


@pytest.mark.gpu
@pytest.mark.parametrize("shape", F32_SHAPES, ids=[f"d{d}_r{a}_{b}" for d, a, b in F32_SHAPES])
def test_decode_f32_shapes(gpu, shape):
    """fp32 codecs: the kernel built for the 8/16 codec at d = 64 and the one with runtime ranks
    (any other pair), with ragged lengths including 0 and 1, a self term, loops 0 and T - 1, and
    several context splits."""
    d, r_k, r_v = shape
    cfg = synth.Config(f"f32_d{d}_{r_k}_{r_v}", L=1, H=2, d=d, T=4, r_k=r_k, r_v=r_v, B=3, N=1,
                       mode=0, dtype="f32", cid=700 + F32_SHAPES.index(shape))
    p, dp = _problem(cfg)
    assert dp.layer.plan.splits > 1
    for t in (0, cfg.T - 1):
        say(f"f32 decode d={d} r=({r_k},{r_v}) lens={list(p.seq_lens)} t={t} "
            f"splits={dp.layer.plan.splits}")
        assert_close(dp.decode(t, True), dp.oracle_decode(t, True), "f32",
                     f"f32 d={d} r=({r_k},{r_v}) t={t}")
