"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on seeded inputs.

Bar: bf16 max|gpu - oracle| <= 2e-2 max|oracle| + 1e-3; fp32 <= 1e-4 max|oracle|.
Small cases span several 32-token chunks, several context splits and a ragged tail; full-size
cases run the exact launch configuration of the benchmark and check sampled sequences.
"""
import sys

import numpy as np
import pytest
import torch

from looped_transformer_kv_amd import lla, synth
from looped_transformer_kv_amd.runtime import LatentLayer
from oracle import brute
from oracle import oracle as O
import gpucase
import tinycase
from gpucase import assert_close

pytestmark = pytest.mark.gpu

BF16_CFGS = ["ouro14_21x", "ouro14_4x", "ouro26_2d_64x", "huginn_32x"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------ tiny fp32 configuration
def test_tiny_f32_four_loops_encode_append_and_readback(gpu):
    """All T loops over 256 cached tokens, then encode+append of the new token, then a decode at
    length N+1 that must see the appended latent."""
    cfg = synth.CONFIGS["tiny_f32"]
    p = tinycase.make(cfg)
    dp = gpucase.DeviceProblem(p)
    for t in range(cfg.T):
        say(f"tiny_f32 decode t={t}")
        assert_close(dp.decode(t), dp.oracle_decode(t), "f32", f"tiny_f32 t={t}")
    B, N = p.B, cfg.N
    pos = torch.full((B,), N, dtype=torch.int32, device=gpu)
    ck = torch.empty((B, cfg.G, cfg.r_k), dtype=torch.float32, device=gpu)
    cv = torch.empty((B, cfg.G, cfg.r_v), dtype=torch.float32, device=gpu)
    kb, vb = synth.from_device(dp.k_pool), synth.from_device(dp.v_pool)
    say("tiny_f32 encode_append")
    dp.layer.encode_append(dp.x_k, dp.x_v, pos, ck, cv)
    torch.cuda.synchronize()
    for axis, cgpu, W, mu, r, before, pool in (
            (0, ck, p.W_down_k, p.mu_k, cfg.r_k, kb, dp.k_pool),
            (1, cv, p.W_down_v, p.mu_v, cfg.r_v, vb, dp.v_pool)):
        ref = O.encode(cfg.mode, cfg.T, cfg.H, cfg.d, r, W, mu, p.x_v if axis else p.x_k)
        c = cgpu.double().cpu().numpy()
        assert_close(c, ref, "f32", f"encode axis {axis}")
        after = synth.from_device(pool)
        expect = O.append(c, np.full(B, N, np.int32), p.block_table, cfg.page, before)
        assert np.array_equal(after, expect)   # fp32 pool: the slot holds c exactly
    dp.seq_lens += 1
    p.seq_lens = p.seq_lens + 1
    dp.layer.set_max_seq_len(N + 1)
    kp, vp = synth.from_device(dp.k_pool), synth.from_device(dp.v_pool)
    for t in (0, cfg.T - 1):
        say(f"tiny_f32 decode after append t={t}")
        ref = dp.oracle_decode(t, k_pool=kp, v_pool=vp)
        assert_close(dp.decode(t), ref, "f32", f"tiny_f32 post-append t={t}")


# ------------------------------------------------------------------ bf16, reduced sizes
def _small(name):
    cfg = synth.CONFIGS[name]
    B = 2 if cfg.mode == 1 else 3
    return cfg, B, 300


@pytest.mark.parametrize("variant", ["plain", "ragged", "peaked", "noself"])
@pytest.mark.parametrize("name", BF16_CFGS)
def test_bf16_decode_small(gpu, name, variant):
    cfg, B, N = _small(name)
    lens = None
    if variant == "ragged":
        lens = synth.seq_lens(cfg, B, N, ragged=True, salt=3)
        lens[0], lens[1] = 0, 1   # empty context and a single token
    p = tinycase.make(cfg, B=B, N=N, lens=lens, q_gain=8.0 if variant == "peaked" else 1.0,
                      loud_tokens=3 if variant == "peaked" else 0)
    dp = gpucase.DeviceProblem(p)
    with_self = variant != "noself"
    for t in sorted({0, 1, cfg.T - 1}):
        say(f"{name}/{variant} B={B} lens={list(p.seq_lens)} t={t}")
        gpu_out = dp.decode(t, with_self)
        ref = dp.oracle_decode(t, with_self)
        assert_close(gpu_out, ref, "bf16", f"{name}/{variant} t={t}")


@pytest.mark.parametrize("name", BF16_CFGS)
def test_bf16_empty_context(gpu, name):
    cfg = synth.CONFIGS[name]
    p = tinycase.make(cfg, B=2, N=64, lens=np.zeros(2, np.int32))
    dp = gpucase.DeviceProblem(p)
    say(f"{name} empty context")
    assert np.all(dp.decode(0, with_self=False) == 0.0)
    out = dp.decode(0, with_self=True)
    assert np.array_equal(out, p.x_v[:, 0])   # softmax over the self term alone


@pytest.mark.parametrize("name", BF16_CFGS + ["tiny_f32"])
def test_encode_append(gpu, name):
    cfg = synth.CONFIGS[name]
    B = 70 if cfg.mode == 0 else 5    # > 64 rows exercises the batch tiling
    N = 100
    p = tinycase.make(cfg, B=B, N=N)
    dp = gpucase.DeviceProblem(p)
    pos_h = np.full(B, N, dtype=np.int32)
    pos_h[1] = 3                       # overwrite an existing slot
    pos_h[2] = -1                      # skipped
    pos = torch.from_numpy(pos_h).to(gpu)
    ck = torch.zeros((B, cfg.G, cfg.r_k), dtype=torch.float32, device=gpu)
    cv = torch.zeros((B, cfg.G, cfg.r_v), dtype=torch.float32, device=gpu)
    kb, vb = synth.from_device(dp.k_pool), synth.from_device(dp.v_pool)
    say(f"{name} encode_append B={B}")
    dp.layer.encode_append(dp.x_k, dp.x_v, pos, ck, cv)
    torch.cuda.synchronize()
    for axis, cgpu, W, mu, r, before, pool in (
            (0, ck, p.W_down_k, p.mu_k, cfg.r_k, kb, dp.k_pool),
            (1, cv, p.W_down_v, p.mu_v, cfg.r_v, vb, dp.v_pool)):
        ref = O.encode(cfg.mode, cfg.T, cfg.H, cfg.d, r, W, mu, p.x_v if axis else p.x_k)
        c = cgpu.double().cpu().numpy()
        assert_close(c, ref, "bf16" if cfg.dtype == "bf16" else "f32", f"{name} c axis {axis}")
        # the pool holds c rounded once to the storage dtype, at the written slots only
        stored = synth.quantize(c, cfg.dtype)
        keep = pos_h >= 0
        expect = O.append(stored[keep], pos_h[keep], p.block_table[keep], cfg.page, before)
        after = synth.from_device(pool)
        assert np.array_equal(after, expect), f"{name} axis {axis}: pool differs"


@pytest.mark.parametrize("name", ["ouro14_4x", "ouro26_2d_64x"])
def test_encode_append_wide_ranks_many_sequences(gpu, name):
    """A decode-step encode over 1024 sequences at ranks 96 / 160 takes the bulk-encode GEMM (one
    row per sequence): c against the oracle, the pool against O.append of c rounded once; then
    lla_encode_append_layers over two layers (each layer through the same single-call path)
    writes bitwise what one call per layer writes."""
    cfg = synth.CONFIGS[name]
    B, N = 1024, 8
    dps = [gpucase.DeviceProblem(tinycase.make(cfg, layer=l, B=B, N=N, salt=l)) for l in range(2)]
    p, dp = dps[0].p, dps[0]
    pos_h = np.full(B, N, dtype=np.int32)
    pos_h[1] = 3                       # overwrite an existing slot
    pos_h[2] = -1                      # skipped
    pos_h[5] = 1 << 20                 # past the block table: skipped
    pos = torch.from_numpy(pos_h).to(gpu)
    ck = torch.zeros((B, cfg.G, cfg.r_k), dtype=torch.float32, device=gpu)
    cv = torch.zeros((B, cfg.G, cfg.r_v), dtype=torch.float32, device=gpu)
    before = [(synth.from_device(d.k_pool), synth.from_device(d.v_pool)) for d in dps]
    say(f"{name} encode_append B={B} (bulk-encode GEMM)")
    dp.layer.encode_append(dp.x_k, dp.x_v, pos, ck, cv)
    torch.cuda.synchronize()
    keep = (pos_h >= 0) & (pos_h < p.block_table.shape[1] * cfg.page)
    for axis, cgpu, W, mu, r, kb, pool in (
            (0, ck, p.W_down_k, p.mu_k, cfg.r_k, before[0][0], dp.k_pool),
            (1, cv, p.W_down_v, p.mu_v, cfg.r_v, before[0][1], dp.v_pool)):
        ref = O.encode(cfg.mode, cfg.T, cfg.H, cfg.d, r, W, mu, p.x_v if axis else p.x_k)
        c = cgpu.double().cpu().numpy()
        assert_close(c, ref, "bf16", f"{name} c axis {axis}")
        stored = synth.quantize(c, "bf16")
        expect = O.append(stored[keep], pos_h[keep], p.block_table[keep], cfg.page, kb)
        assert np.array_equal(synth.from_device(pool), expect), f"{name} axis {axis}: pool differs"
    single = [(synth.from_device(d.k_pool), synth.from_device(d.v_pool)) for d in dps[:1]]
    dps[1].layer.encode_append(dps[1].x_k, dps[1].x_v, pos)
    torch.cuda.synchronize()
    single.append((synth.from_device(dps[1].k_pool), synth.from_device(dps[1].v_pool)))
    for d, (kb, vb) in zip(dps, before):
        d.k_pool.copy_(synth.to_device(kb, "bf16", gpu))
        d.v_pool.copy_(synth.to_device(vb, "bf16", gpu))
    torch.cuda.synchronize()
    say(f"{name}: encode_append_layers over 2 layers, B={B}")
    LatentLayer.encode_append_layers([d.layer for d in dps], [d.x_k for d in dps],
                                     [d.x_v for d in dps], pos)
    torch.cuda.synchronize()
    for l, d in enumerate(dps):
        assert np.array_equal(synth.from_device(d.k_pool), single[l][0]), f"layer {l} K pool"
        assert np.array_equal(synth.from_device(d.v_pool), single[l][1]), f"layer {l} V pool"


@pytest.mark.parametrize("name,n_layers", [("ouro14_21x", 3), ("ouro14_21x", 35),
                                           ("ouro26_2d_64x", 2), ("tiny_f32", 2)])
def test_encode_append_layers_matches_single_calls(gpu, name, n_layers):
    """lla_encode_append_layers writes bitwise what one lla_encode_append per layer writes:
    several layers' codecs and pools, shared positions (one overwrite, one skipped slot); 35
    layers take two launches of the multi-layer kernel, fp32 codecs go layer by layer."""
    cfg = synth.CONFIGS[name]
    B = 32 if cfg.mode == 0 else 4
    N = 100
    # salt = layer: every layer gets its own block-table permutation (and staging rows)
    dps = [gpucase.DeviceProblem(tinycase.make(cfg, layer=l, B=B, N=N, salt=l))
           for l in range(n_layers)]
    assert not np.array_equal(dps[0].p.block_table, dps[1].p.block_table)
    pos_h = np.full(B, N, dtype=np.int32)
    pos_h[1] = 3
    pos_h[2] = -1
    pos = torch.from_numpy(pos_h).to(gpu)
    before = [(synth.from_device(dp.k_pool), synth.from_device(dp.v_pool)) for dp in dps]
    say(f"{name}: {n_layers} single encode_append calls")
    for dp in dps:
        dp.layer.encode_append(dp.x_k, dp.x_v, pos)
    torch.cuda.synchronize()
    single = [(synth.from_device(dp.k_pool), synth.from_device(dp.v_pool)) for dp in dps]
    for dp, (kb, vb) in zip(dps, before):
        dp.k_pool.copy_(synth.to_device(kb, cfg.dtype, gpu))
        dp.v_pool.copy_(synth.to_device(vb, cfg.dtype, gpu))
    torch.cuda.synchronize()
    say(f"{name}: one encode_append_layers call over {n_layers} layers")
    LatentLayer.encode_append_layers([dp.layer for dp in dps], [dp.x_k for dp in dps],
                                     [dp.x_v for dp in dps], pos)
    torch.cuda.synchronize()
    for l, dp in enumerate(dps):
        assert np.array_equal(synth.from_device(dp.k_pool), single[l][0]), f"layer {l} K pool"
        assert np.array_equal(synth.from_device(dp.v_pool), single[l][1]), f"layer {l} V pool"
    assert not np.array_equal(single[0][0], before[0][0]), "the single calls wrote nothing"


# ------------------------------------------------------------------ flat comparator
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_flat_ref_attn_vs_oracle(gpu, dtype):
    cfg = synth.scaled(synth.CONFIGS["ouro14_21x"], dtype=dtype)
    B, N, H, d, P = 4, 333, cfg.H, cfg.d, cfg.page
    g = np.random.default_rng(11)
    max_pages = (N + P - 1) // P
    n_pages = B * max_pages
    kf = synth.quantize(0.3 * g.standard_normal((n_pages, H, P, d)), dtype)
    vf = synth.quantize(0.3 * g.standard_normal((n_pages, H, P, d)), dtype)
    bt = synth.block_table(cfg, B, max_pages, salt=9)
    lens = np.array([N, 1, 0, 200], dtype=np.int32)
    q = synth.quantize(g.standard_normal((B, H, d)), dtype)
    ks = synth.quantize(0.3 * g.standard_normal((B, H, d)), dtype)
    vs = synth.quantize(0.3 * g.standard_normal((B, H, d)), dtype)
    up = lambda a: synth.to_device(a, dtype)
    kd, vd, btd, ld = up(kf), up(vf), torch.from_numpy(bt).to(gpu), torch.from_numpy(lens).to(gpu)
    flat = lla.make_cache(kd, vd, btd, ld, P, int(lens.max()))
    code = gpucase.CODE_DT[dtype]
    plan = lla.lla_ref_plan(H, d, code, flat)
    ws = torch.empty(max(4, plan.workspace_bytes // 4), dtype=torch.float32, device=gpu)
    for with_self in (False, True):
        out = torch.full((B, H, d), float("nan"), dtype=gpucase.TORCH_DT[dtype], device=gpu)
        say(f"flat {dtype} self={with_self}")
        lla.lla_ref_attn(H, d, code, flat, up(q), up(ks) if with_self else None,
                         up(vs) if with_self else None, 0, 1.0 / np.sqrt(d), out, ws)
        torch.cuda.synchronize()
        ref = O.flat_attn(H, d, kf, vf, bt, lens, P, q, ks if with_self else None,
                          vs if with_self else None)
        assert_close(synth.from_device(out), ref, dtype, f"flat {dtype} self={with_self}")


def test_flat_equals_latent_on_materialised_reconstructions_f32(gpu):
    """lla_ref_attn over explicitly reconstructed (fp32) K/V equals lla_decode_attn."""
    cfg = synth.CONFIGS["tiny_f32"]
    p = tinycase.make(cfg, B=2, N=200, ragged=True)
    dp = gpucase.DeviceProblem(p)
    t = 2
    ck = tinycase.logical_latents(p.k_pool, p.block_table, p.seq_lens, cfg.page)
    cv = tinycase.logical_latents(p.v_pool, p.block_table, p.seq_lens, cfg.page)
    Nmax = ck.shape[1]
    K = brute.reconstruct(t, ck, p.W_up_k, p.mu_k, cfg.T).reshape(p.B, Nmax, cfg.H, cfg.d)
    V = brute.reconstruct(t, cv, p.W_up_v, p.mu_v, cfg.T).reshape(p.B, Nmax, cfg.H, cfg.d)
    fk = np.zeros((p.n_pages, cfg.H, cfg.page, cfg.d))
    fv = np.zeros_like(fk)
    for b in range(p.B):
        for j in range(int(p.seq_lens[b])):
            fk[p.block_table[b, j // cfg.page], :, j % cfg.page] = K[b, j]
            fv[p.block_table[b, j // cfg.page], :, j % cfg.page] = V[b, j]
    # keep the pool tensors alive: the cache struct holds raw device pointers only
    fkd, fvd = synth.to_device(fk, "f32"), synth.to_device(fv, "f32")
    flat = lla.make_cache(fkd, fvd, dp.block_table, dp.seq_lens, cfg.page, p.max_seq_len)
    plan = lla.lla_ref_plan(cfg.H, cfg.d, lla.LLA_F32, flat)
    ws = torch.empty(max(4, plan.workspace_bytes // 4), dtype=torch.float32, device=gpu)
    out = torch.empty((p.B, cfg.H, cfg.d), dtype=torch.float32, device=gpu)
    lla.lla_ref_attn(cfg.H, cfg.d, lla.LLA_F32, flat, dp.q[t], dp.x_k[:, t], dp.x_v[:, t],
                     cfg.T * cfg.H * cfg.d, 1.0 / np.sqrt(cfg.d), out, ws)
    torch.cuda.synchronize()
    lat = dp.decode(t)
    assert_close(out.double().cpu().numpy(), lat, "f32", "flat vs latent")


# ------------------------------------------------------------------ determinism, error paths
def test_decode_is_deterministic(gpu):
    cfg = synth.CONFIGS["ouro14_21x"]
    p = tinycase.make(cfg, B=4, N=1000, ragged=True)
    dp = gpucase.DeviceProblem(p)
    a, b = dp.decode(1), dp.decode(1)
    assert np.array_equal(a, b)


def test_invalid_arguments_enqueue_nothing(gpu):
    cfg = synth.CONFIGS["ouro14_21x"]
    p = tinycase.make(cfg, B=1, N=1024)   # one sequence: the context is split, partials needed
    dp = gpucase.DeviceProblem(p)
    L = dp.layer
    assert L.plan.splits > 1 and L.plan.workspace_bytes > 0
    out = torch.full((1, cfg.H, cfg.d), 7.0, dtype=torch.bfloat16, device=gpu)
    ws = L.workspace(gpu)
    q = dp.q[0]
    call = lambda **kw: lla.lla_decode_attn(
        kw.get("codec", L.codec), L.params, kw.get("cache", L.cache), kw.get("t", 0), q,
        kw.get("ks", None), kw.get("vs", None), 0, 0.1, out, kw.get("ws", ws),
        kw.get("wsb", None), check=False)
    assert call(t=cfg.T) == lla.LLA_ERR_SHAPE
    assert call(t=-1) == lla.LLA_ERR_SHAPE
    assert call(ks=dp.x_k) == lla.LLA_ERR_NULL
    assert call(ws=None, wsb=0) == lla.LLA_ERR_WORKSPACE
    assert call(wsb=8) == lla.LLA_ERR_WORKSPACE
    bad = lla.make_codec(0, cfg.T, cfg.H, cfg.d, 8, 16, lla.LLA_BF16)
    assert call(codec=bad) == lla.LLA_ERR_UNSUPPORTED
    bad = lla.make_codec(0, cfg.T, cfg.H, cfg.d, cfg.r_k, cfg.r_v, 9)
    assert call(codec=bad) == lla.LLA_ERR_DTYPE
    c2 = lla.make_cache(dp.k_pool, dp.v_pool, dp.block_table, dp.seq_lens, 48, 1024)
    assert call(cache=c2) == lla.LLA_ERR_SHAPE
    torch.cuda.synchronize()
    assert torch.all(out.float() == 7.0)


# ------------------------------------------------------------------ full sizes, sampled outputs
FULL = ["ouro14_21x", "ouro14_4x", "huginn_32x", "ouro26_2d_64x", "ouro14_21x_cap"]


def _full_layer(cfg, gpu):
    """One layer of a configuration at its full batch and context, pools drawn on the device."""
    B, N = cfg.B, cfg.N
    max_pages = cfg.max_pages
    n_pages = B * max_pages
    Wdk, Wuk, muk = synth.codec(cfg, 0, synth.AX_K)
    Wdv, Wuv, muv = synth.codec(cfg, 0, synth.AX_V)
    kpool = synth.device_latent_pool(cfg, 0, synth.AX_K, n_pages, gpu)
    vpool = synth.device_latent_pool(cfg, 0, synth.AX_V, n_pages, gpu)
    bt = synth.block_table(cfg, B, max_pages)
    lens = synth.seq_lens(cfg, B, N)
    up = lambda a: synth.to_device(a, cfg.dtype, gpu)
    codec = lla.make_codec(cfg.mode, cfg.T, cfg.H, cfg.d, cfg.r_k, cfg.r_v, lla.LLA_BF16)
    layer = LatentLayer(codec, up(Wdk), up(Wdv), up(Wuk), up(Wuv), up(muk), up(muv), kpool, vpool,
                        torch.from_numpy(bt).to(gpu), torch.from_numpy(lens).to(gpu), cfg.page,
                        N)
    host = dict(Wuk=Wuk, Wuv=Wuv, muk=muk, muv=muv, bt=bt, lens=lens)
    return layer, host


def _sampled_oracle(cfg, layer, host, sel, t, q, ks, vs, rope=None):
    """Oracle on the sequences in `sel`, from a read-back of exactly their pages."""
    bt = host["bt"][sel]
    pages = np.unique(bt)
    remap = {int(pg): i for i, pg in enumerate(pages)}
    bt2 = np.vectorize(lambda x: remap[int(x)])(bt).astype(np.int32)
    idx = torch.from_numpy(pages.astype(np.int64)).to(layer.tensors["k_pool"].device)
    kp = synth.from_device(layer.tensors["k_pool"].index_select(0, idx))
    vp = synth.from_device(layer.tensors["v_pool"].index_select(0, idx))
    if rope is not None:
        return O.decode_rope(cfg.mode, cfg.T, cfg.H, cfg.d, cfg.r_k, cfg.r_v, t, host["Wuk"],
                             host["Wuv"], host["muk"], host["muv"], kp, vp, bt2,
                             host["lens"][sel], cfg.page, q[sel], ks[sel], vs[sel],
                             theta=rope.theta, rot_dims=rope.rot_dims, style=rope.style)
    return O.decode(cfg.mode, cfg.T, cfg.H, cfg.d, cfg.r_k, cfg.r_v, t, host["Wuk"], host["Wuv"],
                    host["muk"], host["muv"], kp, vp, bt2, host["lens"][sel], cfg.page, q[sel],
                    ks[sel], vs[sel])


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(gpu, name):
    cfg = synth.CONFIGS[name]
    say(f"{name}: full size B={cfg.B} N={cfg.N} (one layer)")
    layer, host = _full_layer(cfg, gpu)
    sel = [cfg.B - 1] if cfg.mode == 1 else [0, cfg.B // 2, cfg.B - 1]
    xk = synth.staging(cfg, 0, synth.AX_K, cfg.B)
    xv = synth.staging(cfg, 0, synth.AX_V, cfg.B)
    xkd, xvd = synth.to_device(xk, "bf16", gpu), synth.to_device(xv, "bf16", gpu)
    ws = layer.workspace(gpu)
    for t in sorted({0, cfg.T - 1}):
        q = synth.queries(cfg, 0, t, cfg.B)
        out = torch.empty((cfg.B, cfg.H, cfg.d), dtype=torch.bfloat16, device=gpu)
        say(f"{name}: decode t={t} splits={layer.plan.splits}")
        layer.decode(t, synth.to_device(q, "bf16", gpu), out, ws, xkd[:, t], xvd[:, t],
                     cfg.T * cfg.H * cfg.d)
        torch.cuda.synchronize()
        got = synth.from_device(out)
        assert np.all(np.isfinite(got))
        say(f"{name}: oracle on sequences {sel}")
        ref = _sampled_oracle(cfg, layer, host, sel, t, q, xk[:, t], xv[:, t])
        assert_close(got[sel], ref, "bf16", f"{name} t={t}")


# ------------------------------------------------------------------ read-bandwidth probe
@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (3 << 20) + 16 * 7])
def test_stream_read_reads_every_word(gpu, nbytes):
    """The probe behind the read ceiling: the XOR of its per-workgroup sink entries equals the XOR
    of every 32-bit word of the buffer."""
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(gpu)
    sink = torch.zeros(512, dtype=torch.int32, device=gpu)
    say(f"stream_read {nbytes} bytes")
    lla.lla_stream_read(buf, sink)
    torch.cuda.synchronize()
    expect = np.bitwise_xor.reduce(host)
    assert int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))) == int(expect)


# ------------------------------------------------------------------ absorbed-attention decode
@pytest.mark.parametrize("variant", ["plain", "ragged", "peaked", "noself"])
@pytest.mark.parametrize("name", BF16_CFGS)
def test_absorbed_decode_small(gpu, name, variant):
    """lla_decode_attn_absorbed against the oracle's explicit reconstruction (exact up to rounding
    without a rotation; the oracle pin P5 checks the identity itself)."""
    cfg, B, N = _small(name)
    lens = None
    if variant == "ragged":
        lens = synth.seq_lens(cfg, B, N, ragged=True, salt=3)
        lens[0], lens[1] = 0, 1
    p = tinycase.make(cfg, B=B, N=N, lens=lens, q_gain=8.0 if variant == "peaked" else 1.0,
                      loud_tokens=3 if variant == "peaked" else 0)
    dp = gpucase.DeviceProblem(p)
    with_self = variant != "noself"
    for t in sorted({0, cfg.T - 1}):
        say(f"absorbed {name}/{variant} B={B} lens={list(p.seq_lens)} t={t}")
        got = dp.decode(t, with_self, absorbed=True)
        assert_close(got, dp.oracle_decode(t, with_self), "bf16", f"absorbed {name}/{variant} t={t}")


def test_absorbed_split_context_and_empty(gpu):
    """A single long sequence (the plan splits the context; partials go through combine) and an
    all-empty batch without self term (zeros)."""
    cfg = synth.CONFIGS["ouro14_21x"]
    p = tinycase.make(cfg, B=1, N=1500, ragged=False)
    dp = gpucase.DeviceProblem(p)
    assert dp.layer.plan.splits > 1
    say(f"absorbed split context splits={dp.layer.plan.splits}")
    assert_close(dp.decode(1, True, absorbed=True), dp.oracle_decode(1, True), "bf16",
                 "absorbed split")
    p = tinycase.make(cfg, B=2, N=64, lens=np.zeros(2, np.int32))
    dp = gpucase.DeviceProblem(p)
    say("absorbed empty context")
    assert np.all(dp.decode(0, with_self=False, absorbed=True) == 0.0)


def test_absorbed_matches_reconstructing_kernel_full_size(gpu):
    """Headline shape at full size: the absorbed kernel agrees with the oracle on sampled
    sequences, and with the reconstructing kernel everywhere within the same bar."""
    cfg = synth.CONFIGS["ouro14_21x"]
    layer, host = _full_layer(cfg, gpu)
    sel = [0, cfg.B // 2, cfg.B - 1]
    xk = synth.staging(cfg, 0, synth.AX_K, cfg.B)
    xv = synth.staging(cfg, 0, synth.AX_V, cfg.B)
    xkd, xvd = synth.to_device(xk, "bf16", gpu), synth.to_device(xv, "bf16", gpu)
    ws = layer.workspace(gpu)
    t = cfg.T - 1
    q = synth.queries(cfg, 0, t, cfg.B)
    qd = synth.to_device(q, "bf16", gpu)
    outs = []
    for absorbed in (False, True):
        out = torch.empty((cfg.B, cfg.H, cfg.d), dtype=torch.bfloat16, device=gpu)
        run = layer.decode_absorbed if absorbed else layer.decode
        say(f"full size absorbed={absorbed}")
        run(t, qd, out, ws, xkd[:, t], xvd[:, t], cfg.T * cfg.H * cfg.d)
        torch.cuda.synchronize()
        outs.append(synth.from_device(out))
    ref = _sampled_oracle(cfg, layer, host, sel, t, q, xk[:, t], xv[:, t])
    assert_close(outs[1][sel], ref, "bf16", "absorbed full size vs oracle")
    assert_close(outs[1], outs[0], "bf16", "absorbed vs reconstructing kernel")


# ------------------------------------------------------------------ rotation after reconstruction
@pytest.mark.parametrize("style", [0, 1])
@pytest.mark.parametrize("variant", ["plain", "ragged", "noself"])
@pytest.mark.parametrize("name", BF16_CFGS)
def test_rope_decode_small(gpu, name, variant, style):
    """lla_decode_attn_rope against the oracle's explicit reconstruction + rotation."""
    cfg, B, N = _small(name)
    lens = None
    if variant == "ragged":
        lens = synth.seq_lens(cfg, B, N, ragged=True, salt=3)
        lens[0], lens[1] = 0, 1
    p = tinycase.make(cfg, B=B, N=N, lens=lens)
    dp = gpucase.DeviceProblem(p)
    rope = lla.lla_rope(10000.0, cfg.d, style)
    with_self = variant != "noself"
    for t in sorted({0, cfg.T - 1}):
        say(f"rope {name}/{variant} style={style} B={B} lens={list(p.seq_lens)} t={t}")
        got = dp.decode(t, with_self, rope=rope)
        assert_close(got, dp.oracle_decode_rope(t, rope, with_self), "bf16",
                     f"rope {name}/{variant}/{style} t={t}")


def test_rope_fast_rotation(gpu):
    """theta = 10 over 4000 positions: the pairs past the first 16 turn up to ~356 revolutions,
    beyond the range the hardware sine and cosine take unreduced, so the rotary decode reduces
    every pair group's angle (the instantiation the 10^4-theta workloads never launch)."""
    cfg = synth.CONFIGS["ouro14_21x"]
    p = tinycase.make(cfg, B=2, N=4000, lens=np.array([4000, 2345], dtype=np.int32))
    dp = gpucase.DeviceProblem(p)
    for style in (0, 1):
        rope = lla.lla_rope(10.0, cfg.d, style)
        say(f"rope theta 10 style={style} splits={dp.layer.plan.splits}")
        assert_close(dp.decode(1, True, rope=rope), dp.oracle_decode_rope(1, rope, True), "bf16",
                     f"rope theta 10 style {style}")


def test_rope_split_context_long_positions(gpu):
    """One sequence of 4000 tokens (positions up to 4000, split context: the rotated self score
    reaches combine through the partial record), with a self term."""
    cfg = synth.CONFIGS["ouro14_21x"]
    p = tinycase.make(cfg, B=1, N=4000)
    dp = gpucase.DeviceProblem(p)
    assert dp.layer.plan.splits > 1
    for style in (0, 1):
        rope = lla.lla_rope(10000.0, cfg.d, style)
        say(f"rope split context splits={dp.layer.plan.splits} style={style}")
        assert_close(dp.decode(2, True, rope=rope), dp.oracle_decode_rope(2, rope, True), "bf16",
                     f"rope split style {style}")


def test_rope_full_size_sampled(gpu):
    cfg = synth.CONFIGS["ouro14_21x"]
    layer, host = _full_layer(cfg, gpu)
    sel = [0, cfg.B - 1]
    xk = synth.staging(cfg, 0, synth.AX_K, cfg.B)
    xv = synth.staging(cfg, 0, synth.AX_V, cfg.B)
    xkd, xvd = synth.to_device(xk, "bf16", gpu), synth.to_device(xv, "bf16", gpu)
    ws = layer.workspace(gpu)
    t = 1
    q = synth.queries(cfg, 0, t, cfg.B)
    rope = lla.lla_rope(10000.0, cfg.d, 0)
    out = torch.empty((cfg.B, cfg.H, cfg.d), dtype=torch.bfloat16, device=gpu)
    say("rope full size")
    layer.decode_rope(t, rope, synth.to_device(q, "bf16", gpu), out, ws, xkd[:, t], xvd[:, t],
                      cfg.T * cfg.H * cfg.d)
    torch.cuda.synchronize()
    got = synth.from_device(out)
    assert np.all(np.isfinite(got))
    ref = _sampled_oracle(cfg, layer, host, sel, t, q, xk[:, t], xv[:, t], rope=rope)
    assert_close(got[sel], ref, "bf16", "rope full size")


# ------------------------------------------------------------------ head dim 64
# d_head = 64 instantiations (the rotary path then has a single 32-pair tile per lane)
D64_CFGS = {
    "h4_d64_r16_32": synth.Config("d64_r16_32", L=1, H=4, d=64, T=3, r_k=16, r_v=32, B=3, N=1,
                                  cid=150),
    "h4_d64_r64_128": synth.Config("d64_r64_128", L=1, H=4, d=64, T=2, r_k=64, r_v=128, B=3,
                                   N=1, cid=151),
    "h4_d64_2d_r32_64": synth.Config("d64_2d_r32_64", L=1, H=4, d=64, T=2, r_k=32, r_v=64, B=2,
                                     N=1, mode=1, cid=152),
}


@pytest.mark.parametrize("style", [0, 1])
@pytest.mark.parametrize("name", list(D64_CFGS))
def test_head_dim_64_decode_forms(gpu, name, style):
    """The reconstructing, absorbed and rotary decodes at d_head = 64 against the oracle, ragged
    lengths including 0 and 1, with a self term; the rotary decode in both styles."""
    cfg = D64_CFGS[name]
    B, N = cfg.B, 300
    lens = synth.seq_lens(cfg, B, N, ragged=True, salt=5)
    lens[0], lens[1] = 0, 1
    p = tinycase.make(cfg, B=B, N=N, lens=lens)
    dp = gpucase.DeviceProblem(p)
    rope = lla.lla_rope(10000.0, cfg.d, style)
    for t in sorted({0, cfg.T - 1}):
        say(f"d64 {name} style={style} B={B} lens={list(p.seq_lens)} t={t}")
        if style == 0:
            ref = dp.oracle_decode(t, True)
            assert_close(dp.decode(t, True), ref, "bf16", f"d64 {name} t={t}")
            assert_close(dp.decode(t, True, absorbed=True), ref, "bf16",
                         f"d64 absorbed {name} t={t}")
        assert_close(dp.decode(t, True, rope=rope), dp.oracle_decode_rope(t, rope, True), "bf16",
                     f"d64 rope {name}/{style} t={t}")


# ------------------------------------------------------------------ partial rotation
@pytest.mark.parametrize("style", [0, 1])
@pytest.mark.parametrize("rot", ["none", "quarter", "half", "all_but_two"])
@pytest.mark.parametrize("name", ["ouro14_21x", "h4_d64_r16_32"])
def test_rope_partial_rotation(gpu, name, rot, style):
    """Rotation of the first rot_dims head dims only (the rest untouched), against the oracle's
    rotary decode with the same rot_dims: ragged lengths including 0 and 1, a self term."""
    cfg = synth.CONFIGS[name] if name in synth.CONFIGS else D64_CFGS[name]
    rd = {"none": 0, "quarter": cfg.d // 4, "half": cfg.d // 2, "all_but_two": cfg.d - 2}[rot]
    B, N = 3, 300
    lens = synth.seq_lens(cfg, B, N, ragged=True, salt=13)
    lens[0], lens[1] = 0, 1
    p = tinycase.make(cfg, B=B, N=N, lens=lens)
    dp = gpucase.DeviceProblem(p)
    rope = lla.lla_rope(10000.0, rd, style)
    for t in sorted({0, cfg.T - 1}):
        say(f"rope partial {name} rot_dims={rd} style={style} lens={list(p.seq_lens)} t={t}")
        assert_close(dp.decode(t, True, rope=rope), dp.oracle_decode_rope(t, rope, True), "bf16",
                     f"rope partial {name} rot={rd} style={style} t={t}")


def test_rope_partial_rotation_split_context(gpu):
    """Partial rotation over a split context (positions up to 4000, the rotated self score reaches
    combine through the partial record)."""
    cfg = synth.CONFIGS["ouro14_21x"]
    p = tinycase.make(cfg, B=1, N=4000)
    dp = gpucase.DeviceProblem(p)
    assert dp.layer.plan.splits > 1
    for rd, style in ((64, 0), (32, 1)):
        rope = lla.lla_rope(10000.0, rd, style)
        say(f"rope partial split context rot_dims={rd} style={style}")
        assert_close(dp.decode(1, True, rope=rope), dp.oracle_decode_rope(1, rope, True), "bf16",
                     f"rope partial split rot={rd} style={style}")
