"""GPU tests of two contracts of the C ABI that parity against the oracle does not reach.

* Out-of-range page ids.  A block-table entry outside [0, n_pages) inside a sequence's visible
  range makes that sequence's outputs NaN and never faults; every other sequence's outputs are
  bitwise those of a run with a valid table, and entries past a sequence's length are never read.
  Covered for the reconstructing, absorbed (per head and the all-heads LLA-2D kernel) and rotary
  decodes (bf16), the fp32 decode and the chunked prefill.  An encode whose write position lands on such a page writes nothing for that
  row and leaves every other write as it was.
* HIP-graph replay.  Decode (plain, absorbed, rotary), encode-append (one layer or many) and
  prefill captured once and replayed several times, with eager work and synchronisations between
  the replays, give bitwise the eager results on every replay (the benchmark times graph
  launches).
"""
import sys

import numpy as np
import pytest
import torch

from looped_transformer_kv_amd import lla, synth
from looped_transformer_kv_amd.runtime import LatentLayer
import gpucase
import tinycase
from gpucase import Chunk

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _same(a, b):
    return np.array_equal(a, b, equal_nan=True)


# ------------------------------------------------------------------ out-of-range page ids
DECODE_KINDS = {"decode": "ouro14_21x", "absorbed": "ouro14_21x", "rope": "ouro14_21x",
                "decode_2d": "ouro26_2d_64x", "absorbed_2d": "ouro26_2d_64x", "f32": "tiny_f32"}


@pytest.mark.parametrize("kind", list(DECODE_KINDS))
def test_bad_page_ids_poison_only_their_sequence(gpu, kind):
    cfg = synth.CONFIGS[DECODE_KINDS[kind]]
    N = 300
    lens = np.array([N, 250, 130, 200], dtype=np.int32)
    p = tinycase.make(cfg, B=4, N=N, lens=lens)
    dp = gpucase.DeviceProblem(p)
    P = cfg.page
    rope = lla.lla_rope(10000.0, cfg.d, 0) if kind == "rope" else None
    t = cfg.T - 1

    def run():
        return dp.decode(t, True, absorbed=kind.startswith("absorbed"), rope=rope)

    say(f"bad pages {kind} ({cfg.name}): clean run")
    clean = run()
    assert np.all(np.isfinite(clean))
    bt0 = dp.block_table.clone()
    dp.block_table[1, 0] = p.n_pages                        # first page, past the pool
    dp.block_table[3, (lens[3] - 1) // P] = -7              # last visible page, negative
    dp.block_table[2, (lens[2] - 1) // P + 1] = p.n_pages + 9   # past sequence 2's length
    say(f"bad pages {kind}: poisoned table")
    got = run()
    dp.block_table.copy_(bt0)
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[3])), "bad page did not poison"
    assert _same(got[[0, 2]], clean[[0, 2]]), "other sequences changed"


@pytest.mark.parametrize("codec", ["ouro14_21x", "ouro14_4x"])
def test_bad_page_ids_in_prefill(gpu, codec):
    """Two passes (ranks up to 32) and the fused kernel (96 / 160)."""
    cfg = synth.CONFIGS[codec]
    lens, n_new = [200, 150, 90, 64], [70, 50, 0, 33]
    ch = Chunk(cfg, B=4, N=200, Pn=70, lens=lens, n_new=n_new, gpu=gpu)
    P, t = ch.cfg.page, 1
    say(f"bad pages prefill {codec}: clean run")
    clean = ch.run(t)
    bt0 = ch.dp.block_table.clone()
    ch.dp.block_table[1, 1] = ch.p.n_pages                  # inside the cached context
    ch.dp.block_table[2, 0] = -1                            # a sequence with an empty chunk
    ch.dp.block_table[3, (lens[3] + n_new[3]) // P + 1] = -3   # past the chunk's positions
    say(f"bad pages prefill {codec}: poisoned table")
    got = ch.run(t)
    ch.dp.block_table.copy_(bt0)
    assert np.all(np.isnan(got[1, :n_new[1]])), "bad page did not poison"
    assert _same(got[[0, 2, 3]], clean[[0, 2, 3]]), "other sequences changed"
    assert np.all(np.isnan(got[1, n_new[1]:])), "rows past the chunk were written"


@pytest.mark.parametrize("name", ["ouro14_21x", "tiny_f32"])
def test_bad_page_at_append_position_writes_nothing(gpu, name):
    cfg = synth.CONFIGS[name]
    B, N = 6, 100
    p = tinycase.make(cfg, B=B, N=N)
    dp = gpucase.DeviceProblem(p)
    P = cfg.page
    pos_h = np.full(B, N, dtype=np.int32)
    pos = torch.from_numpy(pos_h).to(gpu)
    before = [synth.from_device(dp.k_pool), synth.from_device(dp.v_pool)]
    say(f"{name} append: clean run")
    dp.layer.encode_append(dp.x_k, dp.x_v, pos)
    torch.cuda.synchronize()
    clean = [synth.from_device(dp.k_pool), synth.from_device(dp.v_pool)]
    dp.k_pool.copy_(synth.to_device(before[0], cfg.dtype, gpu))
    dp.v_pool.copy_(synth.to_device(before[1], cfg.dtype, gpu))
    bt0 = dp.block_table.clone()
    page = int(p.block_table[2, N // P])
    dp.block_table[2, N // P] = p.n_pages + 1
    say(f"{name} append: sequence 2's page out of range")
    dp.layer.encode_append(dp.x_k, dp.x_v, pos)
    torch.cuda.synchronize()
    dp.block_table.copy_(bt0)
    for ax in (0, 1):
        expect = clean[ax].copy()
        expect[page, :, N % P] = before[ax][page, :, N % P]    # sequence 2's row stays unwritten
        got = synth.from_device(dp.k_pool if ax == 0 else dp.v_pool)
        assert np.array_equal(got, expect), f"axis {ax}: pool differs"


def test_bad_page_in_chunk_encode_writes_nothing_there(gpu):
    cfg = synth.CONFIGS["ouro14_21x"]
    lens, n_new = [0, 40, 100], [70, 70, 30]
    ch = Chunk(cfg, B=3, N=100, Pn=70, lens=lens, n_new=n_new, gpu=gpu)
    P = ch.cfg.page
    wpos_h = np.array(lens, dtype=np.int32)
    wpos = torch.from_numpy(wpos_h).to(gpu)
    dp = ch.dp
    before = [synth.from_device(dp.k_pool), synth.from_device(dp.v_pool)]
    say("chunk encode: clean run")
    dp.layer.encode_chunk(ch.Pn, ch.nd, ch.xkd, ch.xvd, wpos)
    torch.cuda.synchronize()
    clean = [synth.from_device(dp.k_pool), synth.from_device(dp.v_pool)]
    dp.k_pool.copy_(synth.to_device(before[0], "bf16", gpu))
    dp.v_pool.copy_(synth.to_device(before[1], "bf16", gpu))
    bt0 = dp.block_table.clone()
    lp = (wpos_h[1] + n_new[1] - 1) // P                   # the page of sequence 1's last row
    page = int(ch.p.block_table[1, lp])
    dp.block_table[1, lp] = -2
    say("chunk encode: sequence 1's last page out of range")
    dp.layer.encode_chunk(ch.Pn, ch.nd, ch.xkd, ch.xvd, wpos)
    torch.cuda.synchronize()
    dp.block_table.copy_(bt0)
    rows = [j for j in range(wpos_h[1], wpos_h[1] + n_new[1]) if j // P == lp]
    assert rows
    for ax in (0, 1):
        expect = clean[ax].copy()
        for j in rows:
            expect[page, :, j % P] = before[ax][page, :, j % P]
        got = synth.from_device(dp.k_pool if ax == 0 else dp.v_pool)
        assert np.array_equal(got, expect), f"axis {ax}: pool differs"


# ------------------------------------------------------------------ HIP-graph replay
def test_graph_replay_matches_eager(gpu):
    cfg = synth.CONFIGS["ouro14_21x"]
    p = tinycase.make(cfg, B=3, N=300, ragged=True)
    dp = gpucase.DeviceProblem(p)
    ch = Chunk(cfg, B=3, N=150, Pn=70, lens=[150, 64, 0], n_new=[70, 21, 40], gpu=gpu)
    t = 2
    ws = dp.layer.workspace(gpu)
    q = dp.q[t]
    ks, vs, stride = dp.x_k[:, t], dp.x_v[:, t], cfg.T * cfg.H * cfg.d
    pos = torch.full((3,), 300, dtype=torch.int32, device=gpu)
    out_d = torch.empty((3, cfg.H, cfg.d), dtype=torch.bfloat16, device=gpu)
    out_a = torch.empty_like(out_d)
    out_r = torch.empty_like(out_d)
    rope = lla.lla_rope(10000.0, cfg.d, 0)
    ck = torch.empty((3, cfg.G, cfg.r_k), dtype=torch.float32, device=gpu)
    cv = torch.empty((3, cfg.G, cfg.r_v), dtype=torch.float32, device=gpu)
    out_p = torch.empty((3, ch.Pn, cfg.H, cfg.d), dtype=torch.bfloat16, device=gpu)
    kn, vn = ch.xkd[:, :, t], ch.xvd[:, :, t]

    def work():
        dp.layer.decode(t, q, out_d, ws, ks, vs, stride)
        dp.layer.decode_absorbed(t, q, out_a, ws, ks, vs, stride)
        dp.layer.decode_rope(t, rope, q, out_r, ws, ks, vs, stride)
        dp.layer.encode_append(dp.x_k, dp.x_v, pos, ck, cv)
        ch.dp.layer.prefill(t, ch.Pn, ch.nd, ch.qd[t], kn, vn, out_p, new_stride=stride)

    outs = (out_d, out_a, out_r, ck, cv, out_p)

    def snap():
        return [synth.from_device(o) for o in outs]

    def poison():
        for o in outs:
            o.fill_(float("nan"))

    say("graph replay: eager reference")
    poison()
    work()
    torch.cuda.synchronize()
    ref = snap()
    pools = [synth.from_device(dp.k_pool), synth.from_device(dp.v_pool)]
    g = torch.cuda.CUDAGraph()
    poison()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    other = torch.empty_like(out_d)
    for rep in range(3):
        poison()
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = snap()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert _same(a, b), f"replay {rep}: output {i} differs from eager"
        assert np.array_equal(synth.from_device(dp.k_pool), pools[0])
        assert np.array_equal(synth.from_device(dp.v_pool), pools[1])
        # eager work of the program itself between replays
        dp.layer.decode(0, dp.q[0], other, ws, dp.x_k[:, 0], dp.x_v[:, 0], stride)
        _ = float(other.float().abs().sum())
        torch.cuda.synchronize()


def test_graph_replay_of_multi_layer_encode(gpu):
    """lla_encode_append_layers captured once writes, on every replay, the pools of its eager
    call (the pools are put back to their earlier contents before each replay)."""
    cfg = synth.CONFIGS["ouro14_21x"]
    dps = [gpucase.DeviceProblem(tinycase.make(cfg, layer=l, B=5, N=120)) for l in range(3)]
    pos = torch.tensor([120, 7, -1, 64, 119], dtype=torch.int32, device=gpu)
    pools = [p for dp in dps for p in (dp.k_pool, dp.v_pool)]
    before = [p.clone() for p in pools]

    def work():
        LatentLayer.encode_append_layers([dp.layer for dp in dps], [dp.x_k for dp in dps],
                                         [dp.x_v for dp in dps], pos)

    def restore():
        for p, b in zip(pools, before):
            p.copy_(b)

    say("multi-layer encode: eager reference")
    work()
    torch.cuda.synchronize()
    ref = [synth.from_device(p) for p in pools]
    assert any(not np.array_equal(r, synth.from_device(b)) for r, b in zip(ref, before))
    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        torch.cuda.synchronize()
        say(f"multi-layer encode: graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for i, (p, r) in enumerate(zip(pools, ref)):
            assert np.array_equal(synth.from_device(p), r), f"replay {rep}: pool {i} differs"
        _ = float(dps[0].x_k.float().abs().sum())     # eager work between replays
        torch.cuda.synchronize()


def test_graph_replay_of_absorbed_2d(gpu):
    """The all-heads absorbed LLA-2D decode (three kernels) captured once gives bitwise its eager
    result on every replay."""
    cfg = synth.CONFIGS["ouro26_2d_64x"]
    p = tinycase.make(cfg, B=3, N=700, ragged=True)
    dp = gpucase.DeviceProblem(p)
    assert dp.layer.absorbed_plan.kernel == 4 and dp.layer.absorbed_plan.splits > 1
    t = 1
    ws = dp.layer.workspace(gpu)
    ks, vs, stride = dp.x_k[:, t], dp.x_v[:, t], cfg.T * cfg.H * cfg.d
    out = torch.empty((3, cfg.H, cfg.d), dtype=torch.bfloat16, device=gpu)

    def work():
        dp.layer.decode_absorbed(t, dp.q[t], out, ws, ks, vs, stride)

    say("absorbed 2D graph: eager reference")
    out.fill_(float("nan"))
    work()
    torch.cuda.synchronize()
    ref = synth.from_device(out)
    assert np.all(np.isfinite(ref))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        ws.fill_(float("nan"))                      # stale workspace must not leak into a replay
        torch.cuda.synchronize()
        say(f"absorbed 2D graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert _same(synth.from_device(out), ref), f"replay {rep} differs from eager"
        dp.layer.decode(0, dp.q[0], out, ws, dp.x_k[:, 0], dp.x_v[:, 0], stride)   # eager work
        torch.cuda.synchronize()


def test_graph_replay_of_wide_prefill(gpu):
    """The fused prefill kernel of the wide ranks (LLA-2D, 96 / 160) captured once gives bitwise
    its eager result on every replay."""
    cfg = synth.CONFIGS["ouro26_2d_64x"]
    ch = Chunk(cfg, B=3, N=300, Pn=90, lens=[300, 45, 0], n_new=[90, 33, 60], gpu=gpu)
    t = 2
    out = torch.empty((3, ch.Pn, cfg.H, cfg.d), dtype=torch.bfloat16, device=gpu)
    kn, vn, stride = ch.xkd[:, :, t], ch.xvd[:, :, t], cfg.T * cfg.H * cfg.d

    def work():
        ch.dp.layer.prefill(t, ch.Pn, ch.nd, ch.qd[t], kn, vn, out, new_stride=stride)

    say("wide prefill graph: eager reference")
    out.fill_(float("nan"))
    work()
    torch.cuda.synchronize()
    ref = synth.from_device(out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"wide prefill graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert _same(synth.from_device(out), ref), f"replay {rep} differs from eager"
        ch.dp.layer.prefill(0, ch.Pn, ch.nd, ch.qd[0], ch.xkd[:, :, 0], ch.xvd[:, :, 0], out,
                            new_stride=stride)               # eager work between replays
        torch.cuda.synchronize()
