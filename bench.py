#!/usr/bin/env python3
"""Benchmark of the LLA decode hot path on one MI355X.

One step = one decode step of a weight-tied looped model on the Ouro-1.4B-like 21.3x workload:
24 layers, 16 heads, d_head 128, T = 4 loops, per-head codec r_k = 16 / r_v = 32, bf16 latents,
batch 32, 4096 cached tokens per sequence.  In loop-major order (loop t outer, layer inner) every
(layer, loop) runs lla_decode_attn over that layer's whole latent cache (96 calls, each on a
distinct 201 MB layer cache, so the 256 MB Infinity Cache cannot serve repeats), then one
lla_encode_append_layers call encodes and appends the new token for all 24 layers.  Each step
decodes against the same 4096 cached tokens and appends at slot 4096, so every timed step does
identical work.

value      cached token-loops per second for the whole step (B * N * T * L per step)
roofline   the decode kernel: latent bytes per launch / its average launch time (HIP events
           around the decode segment of every timed step), against MI355X's 8 TB/s; for the
           LLA-2D workload (matrix-core bound) the literal reconstruct-path flops against the
           2.5 PFLOP/s dense bf16 peak, with the latent bandwidth alongside
read_ceiling  a plain streaming read (lla_stream_read) of exactly one decode call's latent bytes,
           launched T x L times back to back in one HIP graph over L distinct buffers, on the
           same run: the achievable read rate for a call of this size, against which the latent
           bandwidth is also given
cpu_baseline  the fp64 oracle on the host cores, on a bounded sample of the same step (median of
           3 runs)
tiny_f32   the tiny fp32 configuration (1 layer, 2 heads, d_head 64, 4 loops, 256 tokens): its
           per-call decode and encode+append times (launch-latency bound)
flat_ref   the uncompressed loop-t comparator (lla_ref_attn) at batch <= 32 on the same GPU
Inputs are synthetic (seeded) and resident in HBM before timing starts.  --workload selects
another of the configured shapes (the default is the one the metric is quoted on).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LLA decode-attn latent HBM GB/s (% of peak) + cached token·loops/s at 1 GPU"
UNIT = "cached token·loops/s"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# exponentials per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz at half the fp32 issue rate
EXP_PEAK_PER_S = 256 * 4 * 16 * 2.4e9 / 2
WORKLOAD = "ouro14_21x"
DESCRIBE = {
    "ouro14_21x": "Ouro-1.4B-like looped decode step at 21.3x",
    "ouro14_21x_cap": "Ouro-1.4B-like 21.3x capacity point (batch 768)",
    "ouro14_4x": "Ouro-1.4B-like looped decode step, 4x codec",
    "ouro26_2d_64x": "Ouro-2.6B-like LLA-2D decode step at 64x",
    "huginn_32x": "Huginn-like 32-loop decode step at 32x",
}
# oracle sample (sequences) per workload: about 10-30 s of fp64 work per (layer, loop) call
CPU_SAMPLE_SEQS = {"ouro14_21x": 32, "ouro14_21x_cap": 32, "ouro14_4x": 8,
                   "ouro26_2d_64x": 1, "huginn_32x": 4}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_bf16_ouro14_21x_traffic.txt")
MFMA_FILE = os.path.join(ROOT, "profiles", "decode_bf16_ouro14_21x_mfma.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "looped_transformer_kv_amd", "csrc", f)
                  for f in ("decode_bf16.hip", "lla_internal.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded(path, key):
    """A figure from a committed rocprofv3 summary under profiles/, or None when the file is
    missing or was taken on a different version of the decode kernel's source."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def recorded_traffic():
    """HBM bytes per decode launch (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's)."""
    return recorded(TRAFFIC_FILE, "traffic_bytes_per_launch")


def recorded_mfma_util():
    """The decode kernel's matrix-core busy fraction (rocprofv3 MfmaUtil, headline shape)."""
    v = recorded(MFMA_FILE, "mfma_util_percent_median")
    return None if v is None else round(v / 100.0, 4)


def build_layers(cfg, dev, n_layers):
    import torch
    from looped_transformer_kv_amd import lla, synth
    from looped_transformer_kv_amd.runtime import LatentLayer

    B, N = cfg.B, cfg.N
    n_pages = B * cfg.max_pages
    bt = torch.from_numpy(synth.block_table(cfg, B, cfg.max_pages)).to(dev)
    lens = torch.full((B,), N, dtype=torch.int32, device=dev)
    codec = lla.make_codec(cfg.mode, cfg.T, cfg.H, cfg.d, cfg.r_k, cfg.r_v, lla.LLA_BF16)
    layers, host = [], []
    for l in range(n_layers):
        Wdk, Wuk, muk = synth.codec(cfg, l, synth.AX_K)
        Wdv, Wuv, muv = synth.codec(cfg, l, synth.AX_V)
        up = lambda a: synth.to_device(a, "bf16", dev)
        kp = synth.device_latent_pool(cfg, l, synth.AX_K, n_pages, dev)
        vp = synth.device_latent_pool(cfg, l, synth.AX_V, n_pages, dev)
        layers.append(LatentLayer(codec, up(Wdk), up(Wdv), up(Wuk), up(Wuv), up(muk), up(muv),
                                  kp, vp, bt, lens, cfg.page, N))
        host.append(dict(Wdk=Wdk, Wdv=Wdv, Wuk=Wuk, Wuv=Wuv, muk=muk, muv=muv))
    return layers, host, bt, lens


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


CPU_RUNS = 3


def cpu_baseline(cfg, layers, host, bt, q, xk, xv, budget_s):
    """The fp64 oracle, timed on this host's cores, on a sample of the step: CPU_RUNS runs, each
    over whole layers (all T decode calls, then the layer's encode+append) of the first
    CPU_SAMPLE_SEQS sequences (all of them for the default workload) for about budget_s /
    CPU_RUNS seconds; the value is the median run's rate."""
    import numpy as np
    import torch
    from looped_transformer_kv_amd import synth
    from oracle import oracle as O

    B, N, T = cfg.B, cfg.N, cfg.T
    nb = min(B, CPU_SAMPLE_SEQS.get(cfg.name, B))
    # the sampled sequences' pages only, renumbered
    pages = bt[:nb].reshape(-1)
    bt_h = np.arange(pages.numel(), dtype=np.int32).reshape(nb, -1)
    lens = np.full(nb, N, dtype=np.int32)
    pos = np.full(nb, N, dtype=np.int32)
    rates, layer_counts, l = [], [], 0
    for run in range(CPU_RUNS):
        spent, done_layers = 0.0, 0
        while spent < budget_s / CPU_RUNS:
            li = l % len(layers)
            kp = synth.from_device(torch.index_select(layers[li].tensors["k_pool"], 0, pages))
            vp = synth.from_device(torch.index_select(layers[li].tensors["v_pool"], 0, pages))
            xk_h, xv_h = synth.from_device(xk[li][:nb]), synth.from_device(xv[li][:nb])
            q_h = [synth.from_device(q[t][li][:nb]) for t in range(T)]
            hd = host[li]
            t0 = time.perf_counter()
            for t in range(T):
                O.decode(cfg.mode, T, cfg.H, cfg.d, cfg.r_k, cfg.r_v, t, hd["Wuk"], hd["Wuv"],
                         hd["muk"], hd["muv"], kp, vp, bt_h, lens, cfg.page, q_h[t], xk_h[:, t],
                         xv_h[:, t])
            ck = O.encode(cfg.mode, T, cfg.H, cfg.d, cfg.r_k, hd["Wdk"], hd["muk"], xk_h)
            cv = O.encode(cfg.mode, T, cfg.H, cfg.d, cfg.r_v, hd["Wdv"], hd["muv"], xv_h)
            O.append(ck, pos, bt_h, cfg.page, kp)
            O.append(cv, pos, bt_h, cfg.page, vp)
            spent += time.perf_counter() - t0
            done_layers += 1
            l += 1
        rates.append(done_layers * nb * N * T / spent)
        layer_counts.append(done_layers)
        log(f"cpu_baseline: run {run}: {done_layers} layers in {spent:.1f} s")
    order = sorted(range(CPU_RUNS), key=lambda i: rates[i])
    med = order[CPU_RUNS // 2]
    return {"value": rates[med], "unit": UNIT, "cores": O.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "runs": [round(r, 1) for r in rates],
            "sample": f"median of {CPU_RUNS} runs; each run: whole layers of one decode step "
                      f"({layer_counts[med]} in the median run) over {nb} of {B} sequences x {N} "
                      f"cached tokens: all {T} loops of decode attention, then encode+append; "
                      f"fp64"}


def read_ceiling(dev, nbytes, calls, n_bufs, reps=5):
    """The achievable read bandwidth for a call of the decode's size: lla_stream_read of nbytes,
    launched `calls` times back to back in one HIP graph over n_bufs distinct buffers (as the
    decode step reads distinct layer caches), best of `reps` replays."""
    import torch
    from looped_transformer_kv_amd import lla

    bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(n_bufs)]
    for b in bufs:
        b.fill_(1)
    sink = torch.zeros(512, dtype=torch.int32, device=dev)

    def run():
        for i in range(calls):
            lla.lla_stream_read(bufs[i % n_bufs], sink)

    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e3 / calls)
    del bufs, g
    torch.cuda.empty_cache()
    gbs = nbytes / (best * 1e-6) / 1e9
    return {"kernel": "lla_stream_read", "bytes_per_call": nbytes, "calls_per_graph": calls,
            "us_per_call": round(best, 3), "GBps": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def flat_comparator(cfg, dev, steps):
    """lla_ref_attn over uncompressed loop-t K/V slices at batch min(B, 32), rotating over 4
    distinct slices (4.3 GB at the default shape) so the Infinity Cache cannot serve repeats."""
    import torch
    from looped_transformer_kv_amd import lla, synth

    B, N, H, d = min(cfg.B, 32), cfg.N, cfg.H, cfg.d
    n_pages = B * cfg.max_pages
    bt = torch.from_numpy(synth.block_table(cfg, B, cfg.max_pages)).to(dev)
    lens = torch.full((B,), N, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    slices = []
    for _ in range(4):
        kf = (0.12 * torch.randn((n_pages, H, cfg.page, d), generator=gen, device=dev)).to(
            torch.bfloat16)
        vf = (0.12 * torch.randn((n_pages, H, cfg.page, d), generator=gen, device=dev)).to(
            torch.bfloat16)
        slices.append((kf, vf, lla.make_cache(kf, vf, bt, lens, cfg.page, N)))
    plan = lla.lla_ref_plan(H, d, lla.LLA_BF16, slices[0][2])
    ws = torch.empty(max(4, plan.workspace_bytes // 4), dtype=torch.float32, device=dev)
    q = torch.randn((B, H, d), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    scale = 1.0 / math.sqrt(d)
    for i in range(4):
        lla.lla_ref_attn(H, d, lla.LLA_BF16, slices[i][2], q, None, None, 0, scale, out, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    calls = 4 * steps
    e0.record()
    for i in range(calls):
        lla.lla_ref_attn(H, d, lla.LLA_BF16, slices[i % 4][2], q, None, None, 0, scale, out, ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    flat_bytes = B * N * H * d * 2 * 2
    gbs = flat_bytes / (us * 1e-6) / 1e9
    del slices
    torch.cuda.empty_cache()
    return {"kernel": "lla_ref_attn (flat loop-t cache)", "batch": B, "context": N,
            "us_per_call": round(us, 2), "bytes_per_call": flat_bytes,
            "achieved_GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "splits": plan.splits}


def tiny_leg(dev, reps=50):
    """The tiny fp32 configuration: T decode calls (with the self term) and one encode+append,
    each graph-launched `reps` times back to back; per-call times."""
    import numpy as np
    import torch
    from looped_transformer_kv_amd import lla, synth
    from looped_transformer_kv_amd.runtime import LatentLayer

    cfg = synth.CONFIGS["tiny_f32"]
    B, N, T, H, d = cfg.B, cfg.N, cfg.T, cfg.H, cfg.d
    n_pages = B * cfg.max_pages
    up = lambda a: synth.to_device(a, "f32", dev)
    Wdk, Wuk, muk = synth.codec(cfg, 0, synth.AX_K)
    Wdv, Wuv, muv = synth.codec(cfg, 0, synth.AX_V)
    codec = lla.make_codec(0, T, H, d, cfg.r_k, cfg.r_v, lla.LLA_F32)
    layer = LatentLayer(codec, up(Wdk), up(Wdv), up(Wuk), up(Wuv), up(muk), up(muv),
                        up(synth.latent_pool(cfg, 0, synth.AX_K, n_pages)),
                        up(synth.latent_pool(cfg, 0, synth.AX_V, n_pages)),
                        torch.from_numpy(synth.block_table(cfg, B, cfg.max_pages)).to(dev),
                        torch.full((B,), N, dtype=torch.int32, device=dev), cfg.page, N)
    q = [up(synth.queries(cfg, 0, t, B)) for t in range(T)]
    xk = up(synth.staging(cfg, 0, synth.AX_K, B))
    xv = up(synth.staging(cfg, 0, synth.AX_V, B))
    out = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    ws = layer.workspace(dev)
    pos = torch.full((B,), N, dtype=torch.int32, device=dev)

    def dec():
        for _ in range(reps):
            for t in range(T):
                layer.decode(t, q[t], out, ws, xk[:, t], xv[:, t], T * H * d)

    def enc():
        for _ in range(reps):
            layer.encode_append(xk, xv, pos)

    res = {}
    for name, fn, calls in (("decode", dec, reps * T), ("encode_append", enc, reps)):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / calls)
        res[name + "_us_per_call"] = round(float(np.median(times)), 3)
    return {"config": "tiny_f32: 1 layer, 2 heads, d_head 64, T 4, r 8/16, batch 1, 256 tokens, "
                      "fp32", "splits": layer.plan.splits, **res}


PREFILL_CHUNK = 512
# (r_k, r_v) pairs lla_prefill_attn serves (d_head 64 or 128): two passes up to 32, one fused
# kernel above
PREFILL_RANKS = {(16, 16), (16, 32), (32, 32), (32, 64), (64, 64), (64, 128), (96, 160)}


def prefill_leg(cfg, layers, dev, launch, steps, warmup):
    """Chunked prefill on the same layers: a chunk of PREFILL_CHUNK new tokens per sequence after
    the N cached ones, all L layers x T loops of lla_prefill_attn, then one lla_encode_chunk per
    layer.  Inputs are fresh device draws (q ~ N(0, 1), chunk trajectories with the staging
    spread).  The chunk's latents are written at positions 0 .. chunk - 1, which the block table
    holds (overwriting cached values changes no timing)."""
    import torch
    from looped_transformer_kv_amd import synth

    B, N, T, H, d = cfg.B, cfg.N, cfg.T, cfg.H, cfg.d
    L, Pn = len(layers), PREFILL_CHUNK
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.ROOT_SEED + 7)
    xs = math.sqrt(sum(cfg.decay ** i for i in range(cfg.r_k)) / cfg.X + 0.01)
    qc = [torch.randn((B, Pn, H, d), generator=gen, device=dev).to(torch.bfloat16)
          for _ in range(T)]
    xkc = (xs * torch.randn((B, Pn, T, H, d), generator=gen, device=dev)).to(torch.bfloat16)
    xvc = (xs * torch.randn((B, Pn, T, H, d), generator=gen, device=dev)).to(torch.bfloat16)
    n_new = torch.full((B,), Pn, dtype=torch.int32, device=dev)
    wpos = torch.zeros((B,), dtype=torch.int32, device=dev)
    outc = torch.empty((B, Pn, H, d), dtype=torch.bfloat16, device=dev)
    stride = T * H * d

    def attn_all():
        for t in range(T):
            for l in range(L):
                layers[l].prefill(t, Pn, n_new, qc[t], xkc[:, :, t], xvc[:, :, t], outc,
                                  new_stride=stride)

    def enc_all():
        for l in range(L):
            layers[l].encode_chunk(Pn, n_new, xkc, xvc, wpos)

    attn_all()
    enc_all()
    torch.cuda.synchronize()
    run_a, run_e = attn_all, enc_all
    if launch == "hip_graph":
        ga, ge = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(ga):
            attn_all()
        with torch.cuda.graph(ge):
            enc_all()
        run_a, run_e = ga.replay, ge.replay
    for _ in range(warmup):
        run_a()
        run_e()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(steps):
        run_a()
    ev[1].record()
    for _ in range(steps):
        run_e()
    ev[2].record()
    torch.cuda.synchronize()
    attn_us = ev[0].elapsed_time(ev[1]) * 1e3 / (steps * T * L)
    enc_us = ev[1].elapsed_time(ev[2]) * 1e3 / (steps * L)
    # work of one call: every query against its cached context and its causal part of the chunk.
    # What binds is the vector ALU, whose irreducible part is one exponential per visible pair:
    # EXP_PEAK_PER_S is the chip's rate of those (transcendentals issue at half the fp32 rate).
    pairs = B * H * (Pn * N + Pn * (Pn + 1) // 2)
    exp_rate = pairs / (attn_us * 1e-6)
    # matrix-core work of the latent-space formulation: q' = c W_up,t^K q and the expansion
    # O_lat W_up,t^V once per query, 2 (r_k + r_v) per cached pair, 4d per causal chunk pair.
    # At ranks above 32 this is what binds (the fused kernel: ~6x the flops per exponential).
    flops = (B * H * Pn * 2 * d * (cfg.r_k + cfg.r_v) + B * H * Pn * N * 2 * (cfg.r_k + cfg.r_v) +
             B * H * Pn * (Pn + 1) // 2 * 4 * d)
    tflops = flops / (attn_us * 1e-6) / 1e12
    enc_bytes = sum(B * Pn * T * H * d * 2 + cfg.G * cfg.X * r * 2 + cfg.G * cfg.X * 2 +
                    B * Pn * cfg.G * r * 2 for r in (cfg.r_k, cfg.r_v))
    step_s = (attn_us * T * L + enc_us * L) * 1e-6
    return {"kernel": "lla_prefill_attn + lla_encode_chunk", "chunk": Pn, "cached": N,
            "attn_us_per_call": round(attn_us, 3), "pairs_per_call": pairs,
            "pairs_per_s": round(exp_rate, 1),
            "frac_of_exp_peak": round(exp_rate / EXP_PEAK_PER_S, 4),
            "mfma_flops_per_call": flops, "TFLOPs": round(tflops, 1),
            "frac_of_bf16_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "bound": "mfma" if max(cfg.r_k, cfg.r_v) > 32 else "exp",
            "encode_chunk_us_per_call": round(enc_us, 3),
            "encode_chunk_bytes_per_call": enc_bytes,
            "encode_chunk_GBps": round(enc_bytes / (enc_us * 1e-6) / 1e9, 1),
            "prefill_tokens_per_s": round(B * Pn / step_s, 1)}


FIT_ITERS = 40
FIT_MAX_BYTES = 8 << 30        # staged rows per axis: B x N rows, capped at 8 GiB of bf16


def fit_leg(cfg, dev, steps):
    """Codec fit of one layer (both axes) from n = B x N rows of staged trajectories, at most
    FIT_MAX_BYTES per axis (Huginn's 32 loops x 32 heads make a row 256 KB: 32768 rows there)
    (lla_fit_svd, FIT_ITERS steps of subspace iteration).  The rows are i.i.d. draws with the
    staging spread: the work per call does not depend on the data."""
    import torch
    from looped_transformer_kv_amd import lla, synth

    T, H, d = cfg.T, cfg.H, cfg.d
    n = min(cfg.B * cfg.N, FIT_MAX_BYTES // (T * H * d * 2))
    codec = lla.make_codec(cfg.mode, T, H, d, cfg.r_k, cfg.r_v, lla.LLA_BF16)
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.ROOT_SEED + 11)
    xs = math.sqrt(sum(cfg.decay ** i for i in range(cfg.r_k)) / cfg.X + 0.01)
    x = []
    for _ in range(2):
        xa = torch.empty((n, T, H, d), dtype=torch.bfloat16, device=dev)
        for i in range(0, n, 8192):                 # fp32 draws a slice at a time
            j = min(n, i + 8192)
            xa[i:j] = (xs * torch.randn((j - i, T, H, d), generator=gen, device=dev)).to(
                torch.bfloat16)
        x.append(xa)
    G, X, Dg = cfg.G, cfg.X, cfg.Dg
    outs, wss = [], []
    for r in (cfg.r_k, cfg.r_v):
        outs.append((torch.empty((G, X), dtype=torch.bfloat16, device=dev),
                     torch.empty((G, X, r), dtype=torch.bfloat16, device=dev),
                     torch.empty((T, G, r, Dg), dtype=torch.bfloat16, device=dev)))
        wss.append(torch.empty(lla.lla_fit_plan(codec, r, n) // 4 + 4, dtype=torch.float32,
                               device=dev))

    def run():
        for ax, r in enumerate((cfg.r_k, cfg.r_v)):
            mu, Wd, Wu = outs[ax]
            lla.lla_fit_svd(codec, r, x[ax], n, FIT_ITERS, mu, Wd, Wu, None, wss[ax])

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    cov_flops = 2 * 2 * n * X * X * G           # A^T A of both axes (full X x X)
    return {"kernel": "lla_fit_svd (K and V of one layer)", "rows": n, "iters": FIT_ITERS,
            "ms_per_layer": round(ms, 3), "covariance_flops": cov_flops,
            "covariance_TFLOPs_over_call": round(cov_flops / (ms * 1e-3) / 1e12, 1),
            "staged_bytes": 2 * n * T * H * d * 2}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time budget for the CPU baseline (0 disables it)")
    ap.add_argument("--no-flat", action="store_true", help="skip the flat comparator")
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of HIP graphs")
    ap.add_argument("--workload", default=WORKLOAD, choices=sorted(DESCRIBE),
                    help="shape to time (default: the one the metric is quoted on)")
    ap.add_argument("--layers", type=int, default=0,
                    help="build only this many layers (0: all; the step then covers them)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the read-ceiling probe")
    ap.add_argument("--no-absorbed", action="store_true",
                    help="skip timing the absorbed-attention decode (lla_decode_attn_absorbed)")
    ap.add_argument("--no-rope", action="store_true",
                    help="skip timing the decode with rotation after reconstruction "
                         "(lla_decode_attn_rope, theta 10^4, whole-head half-split pairs)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip timing the chunked prefill (lla_prefill_attn, a chunk of "
                         f"{PREFILL_CHUNK} after the cached context, then lla_encode_chunk)")
    ap.add_argument("--no-fit", action="store_true",
                    help="skip timing the codec fit (lla_fit_svd of one layer's K and V from "
                         "B x N staged rows)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (the reference "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written":
                          dst.numel() * 4, "launches": 3}), flush=True)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the LLA decode path is measured on a single MI355X and has no multi-GPU mode.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from looped_transformer_kv_amd import lla, synth
    from looped_transformer_kv_amd.runtime import LatentLayer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    lla.lib()
    cfg = synth.CONFIGS[args.workload]
    B, N, T, H, d = cfg.B, cfg.N, cfg.T, cfg.H, cfg.d
    L = min(cfg.L, args.layers) if args.layers > 0 else cfg.L

    ceiling = None
    if not args.no_ceiling:
        log("measuring the read ceiling at the call's size")
        ceiling = read_ceiling(dev, B * N * cfg.G * (cfg.r_k + cfg.r_v) * 2, T * L, L)
    log(f"building {L} layers of {cfg.name} (batch {B}, context {N}) on {dev}")
    layers, host, bt, lens = build_layers(cfg, dev, L)
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.ROOT_SEED)
    q = [[torch.randn((B, H, d), generator=gen, device=dev).to(torch.bfloat16) for _ in range(L)]
         for _ in range(T)]
    xs = math.sqrt(sum(cfg.decay ** i for i in range(cfg.r_k)) / cfg.X + 0.01)
    xk = [(xs * torch.randn((B, T, H, d), generator=gen, device=dev)).to(torch.bfloat16)
          for _ in range(L)]
    xv = [(xs * torch.randn((B, T, H, d), generator=gen, device=dev)).to(torch.bfloat16)
          for _ in range(L)]
    write_pos = torch.full((B,), N, dtype=torch.int32, device=dev)
    out = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)
    plan = layers[0].plan
    ws = layers[0].workspace(dev)
    stride = T * H * d

    def decode_all():
        for t in range(T):
            for l in range(L):
                layers[l].decode(t, q[t][l], out, ws, xk[l][:, t], xv[l][:, t], stride)

    def encode_all():
        LatentLayer.encode_append_layers(layers, xk, xv, write_pos)

    decode_all()
    encode_all()
    torch.cuda.synchronize()
    launch = "eager"
    if not args.eager:
        try:
            g_dec, g_enc = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_dec):
                decode_all()
            with torch.cuda.graph(g_enc):
                encode_all()
            run_dec, run_enc, launch = g_dec.replay, g_enc.replay, "hip_graph"
        except Exception as e:  # capture unsupported: fall back to eager launches
            log(f"graph capture failed ({e}); timing eager launches")
    if launch == "eager":
        run_dec, run_enc = decode_all, encode_all

    for _ in range(args.warmup):
        run_dec()
        run_enc()
    torch.cuda.synchronize()

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(K):
        ev[k][0].record()
        run_dec()
        ev[k][1].record()
        run_enc()
    end.record()
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / K
    dec_us = sum(a.elapsed_time(b) for a, b in ev) * 1e3 / (K * T * L)
    enc_us = (step_ms * 1e3 - dec_us * T * L) / L

    latent_bytes = B * N * cfg.G * (cfg.r_k + cfg.r_v) * 2
    achieved = latent_bytes / (dec_us * 1e-6) / 1e9
    # literal reconstruct path per call: every cached token expanded for K and V, plus attention
    flops = B * N * (cfg.G * 2 * (cfg.r_k + cfg.r_v) * cfg.Dg + 4 * H * d)
    tflops = flops / (dec_us * 1e-6) / 1e12
    token_loops = B * N * T * L
    # encode: staging rows, W_down and mu read, latents written, both axes
    enc_bytes = sum(B * T * H * d * 2 + cfg.G * cfg.X * r * 2 + cfg.G * cfg.X * 2 + B * cfg.G * r * 2
                    for r in (cfg.r_k, cfg.r_v))
    if cfg.mode == 1:   # matrix-core bound: the roofline is the expansion's flops
        roofline = {"bound": "mfma", "achieved": round(tflops, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": recorded_traffic() if cfg.name == WORKLOAD else None}
    result = {
        "metric": METRIC,
        "value": token_loops / (step_ms * 1e-3),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {DESCRIBE[cfg.name]}, {L} layers x {T} loops "
                        f"of LLA decode attention + one {L}-layer encode/append call",
            "mode": "lla_2d" if cfg.mode == 1 else "per_head",
            "layers": L, "heads": H, "d_head": d, "loops": T, "r_k": cfg.r_k, "r_v": cfg.r_v,
            "compression": round(lla.lla_compression_ratio(layers[0].codec), 3),
            "global_batch": B, "seq_len": N, "page_size": cfg.page,
            "splits": plan.splits, "launch": launch, "parallelism": "none (1 GPU)",
        },
        "roofline": roofline,
        "read_ceiling": ceiling,
        "decode_us_per_call": round(dec_us, 3),
        "decode_latent_bytes_per_call": latent_bytes,
        "decode_latent_GBps": round(achieved, 1),
        "decode_frac_of_hbm_peak": round(achieved / HBM_PEAK_GBS, 4),
        "decode_frac_of_read_ceiling": round(achieved / ceiling["GBps"], 4) if ceiling else None,
        "decode_flops_per_call": flops,
        "decode_TFLOPs": round(tflops, 2),
        "decode_mfma_busy_frac": recorded_mfma_util() if cfg.name == WORKLOAD else None,
        "decode_token_loops_per_s_per_call": round(B * N / (dec_us * 1e-6), 1),
        "encode_us_per_layer": round(enc_us, 3),
        "encode_bytes_per_layer": enc_bytes,
        "encode_GBps": round(enc_bytes / (enc_us * 1e-6) / 1e9, 1),
    }
    def time_variant(run_one):
        """Per-call time of `run_one(t, l)` over the whole step (T x L calls), graph-launched
        like the main decode."""
        def all_calls():
            for t in range(T):
                for l in range(L):
                    run_one(t, l)
        all_calls()
        torch.cuda.synchronize()
        run = all_calls
        if launch == "hip_graph":
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                all_calls()
            run = g.replay
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(K):
            run()
        a1.record()
        torch.cuda.synchronize()
        us = a0.elapsed_time(a1) * 1e3 / (K * T * L)
        gbs = latent_bytes / (us * 1e-6) / 1e9
        return {"us_per_call": round(us, 3), "latent_GBps": round(gbs, 1),
                "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                "frac_of_read_ceiling": round(gbs / ceiling["GBps"], 4) if ceiling else None,
                "token_loops_per_s_per_call": round(B * N / (us * 1e-6), 1)}

    if not args.no_absorbed:
        log("timing the absorbed-attention decode")
        result["absorbed"] = {"kernel": "lla_decode_attn_absorbed", **time_variant(
            lambda t, l: layers[l].decode_absorbed(t, q[t][l], out, ws, xk[l][:, t], xv[l][:, t],
                                                   stride))}
    if not args.no_rope:
        log("timing the decode with rotation after reconstruction")
        rope = lla.lla_rope(10000.0, d, 0)
        result["rope"] = {"kernel": "lla_decode_attn_rope", "theta": 10000.0, "rot_dims": d,
                          "style": "half_split", **time_variant(
            lambda t, l: layers[l].decode_rope(t, rope, q[t][l], out, ws, xk[l][:, t],
                                               xv[l][:, t], stride))}
    if not args.no_prefill and (cfg.r_k, cfg.r_v) in PREFILL_RANKS:
        log("timing the chunked prefill")
        result["prefill"] = prefill_leg(cfg, layers, dev, launch, K, args.warmup)
    if not args.no_fit and cfg.X % 128 == 0 and cfg.X <= 8192 and max(cfg.r_k, cfg.r_v) <= 160:
        log("timing the codec fit")
        result["fit"] = fit_leg(cfg, dev, 3)
    log("timing the tiny fp32 configuration")
    result["tiny_f32"] = tiny_leg(dev)
    if not args.no_flat:
        log("timing the flat comparator")
        result["flat_ref"] = flat_comparator(cfg, dev, max(5, K))
    if args.cpu_seconds > 0:
        log("timing the oracle on the host cores")
        result["cpu_baseline"] = cpu_baseline(cfg, layers, host, bt, q, xk, xv, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
