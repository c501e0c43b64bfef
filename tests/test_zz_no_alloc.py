"""lla_decode_attn_noalloc (the decode entry point that allocates nothing: its context-split
partials live in the library's own per-device scratch array) against lla_decode_attn with a
caller workspace, through the C ABI: two split-context calls in a row, the second smaller, then a
single-split call; each output equals the workspace entry point's bit for bit (same kernels, same
arithmetic) and meets the oracle within the bf16 bar.  A plan needing more than the array's
4 MiB is refused before anything is enqueued.
"""
import sys

import numpy as np
import pytest
import torch

from looped_transformer_kv_amd import lla, synth
import gpucase
import tinycase
from gpucase import assert_close

pytestmark = pytest.mark.gpu
CFG = synth.CONFIGS["ouro14_21x"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _noalloc(dp, t):
    p, c = dp.p, dp.p.cfg
    out = torch.full((p.B, c.H, c.d), float("nan"), dtype=torch.bfloat16, device=dp.device)
    L = dp.layer
    lla.lla_decode_attn_noalloc(L.codec, L.params, L.cache, t, dp.q[t], dp.x_k[:, t],
                                dp.x_v[:, t], c.T * c.H * c.d, 1.0 / np.sqrt(c.d), out)
    torch.cuda.synchronize()
    return synth.from_device(out)


@pytest.mark.parametrize("t", [0, 3])
def test_noalloc_equals_workspace_entry_point(gpu, t):
    cases = [dict(B=1, N=3000, lens=None),                       # 16 heads x S splits
             dict(B=2, N=700, lens=np.array([700, 333], np.int32)),   # smaller, ragged
             dict(B=32, N=300, lens=None)]                       # one split: no partials
    for k, cs in enumerate(cases):
        p = tinycase.make(CFG, B=cs["B"], N=cs["N"], lens=cs["lens"], salt=k)
        dp = gpucase.DeviceProblem(p)
        plan = dp.layer.plan
        assert (plan.splits > 1) == (k < 2)
        say(f"noalloc case {k}: B={p.B} lens={list(p.seq_lens)} splits={plan.splits} "
            f"partials {plan.workspace_bytes} B t={t}")
        ref_ws = dp.decode(t)
        got = _noalloc(dp, t)
        assert np.array_equal(got, ref_ws), f"case {k}: differs from lla_decode_attn"
        assert_close(got, dp.oracle_decode(t), "bf16", f"noalloc case {k} t={t}")


def test_noalloc_refuses_plans_beyond_its_scratch(gpu):
    """One sequence per (batch, head) row over a very long context: the plan's partials exceed
    the 4 MiB array, so the call returns LLA_ERR_WORKSPACE and the output stays untouched."""
    c = CFG
    N = 1 << 20
    P = c.page
    max_pages = N // P + 1
    dummy = torch.zeros(16, dtype=torch.bfloat16, device=gpu)
    bt = torch.zeros((31, max_pages), dtype=torch.int32, device=gpu)
    lens = torch.full((31,), N, dtype=torch.int32, device=gpu)
    cache = lla.make_cache(dummy, dummy, bt, lens, P, N, n_pages=1)
    codec = lla.make_codec(0, c.T, c.H, c.d, c.r_k, c.r_v, lla.LLA_BF16)
    assert lla.lla_decode_plan(codec, cache).workspace_bytes > (4 << 20)
    params = lla.make_params(dummy, dummy, dummy, dummy, dummy, dummy)
    q = torch.zeros((31, c.H, c.d), dtype=torch.bfloat16, device=gpu)
    out = torch.full((31, c.H, c.d), 7.0, dtype=torch.bfloat16, device=gpu)
    st = lla.lla_decode_attn_noalloc(codec, params, cache, 0, q, None, None, 0, 0.1, out,
                                     check=False)
    torch.cuda.synchronize()
    assert st == lla.LLA_ERR_WORKSPACE
    assert torch.all(out.float() == 7.0)
