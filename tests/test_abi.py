"""The C ABI on the CPU: liblla.so loads, exports every function include/lla.h declares, and its
host-only helpers and argument validation behave (nothing here launches a kernel)."""
import ctypes
import os
import re
from fractions import Fraction

import pytest

from looped_transformer_kv_amd import lla, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("lla_decode_attn", "lla_encode_append", "lla_ref_attn"):
        assert must in names


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports_declared_symbol(name):
    L = lla.lib()
    assert hasattr(L, name), f"liblla.so does not export {name}"


def test_package_has_no_fallback():
    # the binding refuses to run without the library rather than computing anywhere else
    assert os.path.exists(lla.LIB_PATH)
    src = open(os.path.join(ROOT, "looped_transformer_kv_amd", "lla.py")).read()
    assert "oracle" not in src.replace("no fallback", "")


def _codec(c):
    return lla.make_codec(c.mode, c.T, c.H, c.d, c.r_k, c.r_v,
                          lla.LLA_F32 if c.dtype == "f32" else lla.LLA_BF16)


@pytest.mark.parametrize("name", sorted(synth.CONFIGS))
def test_ratio_and_byte_accounting(name):
    c = synth.CONFIGS[name]
    codec = _codec(c)
    rho = lla.lla_compression_ratio(codec)
    exact = Fraction(2 * c.T * c.d * (c.H if c.mode else 1), c.r_k + c.r_v)
    assert rho == float(exact)
    elt = 4 if c.dtype == "f32" else 2
    lat = lla.lla_latent_bytes_per_token(codec)
    flat = lla.lla_flat_bytes_per_token(codec)
    assert lat == c.G * (c.r_k + c.r_v) * elt
    assert flat == 2 * c.T * c.H * c.d * elt
    assert Fraction(flat, lat) == exact      # the reduction is exact


def test_ratio_rejects_invalid_codec():
    assert lla.lla_compression_ratio(lla.make_codec(0, 4, 16, 96, 16, 32, 1)) == 0.0
    assert lla.lla_latent_bytes_per_token(lla.make_codec(0, 0, 16, 128, 16, 32, 1)) == 0


def test_decode_plan_covers_the_context():
    c = synth.CONFIGS["ouro14_21x"]
    cache = lla.lla_cache(None, None, None, None, c.B, c.page, c.max_pages, c.B * c.max_pages,
                          c.N)
    plan = lla.lla_decode_plan(_codec(c), cache)
    assert plan.kernel == 1
    assert plan.splits * plan.tokens_per_split >= c.N
    assert (plan.splits - 1) * plan.tokens_per_split < c.N
    assert plan.tokens_per_split % 128 == 0
    # a single split is finished inside the latent kernel; more need fp32 partials
    expect = 0 if plan.splits == 1 else c.B * c.H * plan.splits * (c.d + 4) * 4
    assert plan.workspace_bytes == expect
    small = lla.lla_cache(None, None, None, None, 1, c.page, c.max_pages, c.max_pages, c.N)
    plan = lla.lla_decode_plan(_codec(c), small)
    assert plan.splits > 1 and plan.workspace_bytes == c.H * plan.splits * (c.d + 4) * 4



@pytest.mark.parametrize("B,N", [(32, 4096), (1, 4096), (768, 4096), (3, 300), (0, 0)])
def test_decode_workspace_size_matches_plan(B, N):
    c = synth.CONFIGS["ouro14_21x"]
    max_pages = max(1, (N + 1 + c.page - 1) // c.page)
    cache = lla.lla_cache(None, None, None, None, B, c.page, max_pages, max(1, B * max_pages), N)
    plan = lla.lla_decode_plan(_codec(c), cache)
    assert lla.lla_decode_workspace_size(_codec(c), cache) == plan.workspace_bytes
    L = lla.lib()
    out = ctypes.c_size_t(12345)
    assert L.lla_decode_workspace_size(ctypes.byref(_codec(c)), ctypes.byref(cache), None) == \
        lla.LLA_ERR_NULL
    bad = lla.make_codec(0, 4, 16, 96, 16, 32, 1)          # d_head 96: invalid codec
    assert L.lla_decode_workspace_size(ctypes.byref(bad), ctypes.byref(cache),
                                       ctypes.byref(out)) == lla.LLA_ERR_SHAPE
    assert out.value == 12345                              # untouched on error
    assert L.lla_decode_workspace_size(ctypes.byref(_codec(c)), None,
                                       ctypes.byref(out)) == lla.LLA_ERR_NULL

def test_absorbed_plan():
    """lla_decode_absorbed_plan: kernel 4 (all heads per workgroup, splits per sequence) for LLA-2D
    codecs with <= 16 heads, r_k % 32 == 0 and r_v % 16 == 0; the plain decode plan otherwise."""
    c = synth.CONFIGS["ouro26_2d_64x"]
    cache = lla.lla_cache(None, None, None, None, c.B, c.page, c.max_pages, c.B * c.max_pages, c.N)
    plan = lla.lla_decode_absorbed_plan(_codec(c), cache)
    assert (plan.kernel, plan.splits, plan.tokens_per_split) == (4, 32, 512)
    rk, rv, B, S = c.r_k, c.r_v, c.B, 32
    up = lambda n: (n + 63) // 64 * 64
    floats = up(B * 16 * rk) + 2 * up(B * 16) + up(B * S * 16 * rv) + up(B * S * 16 * 2)
    assert plan.workspace_bytes == 4 * floats
    for mode, H, rk, rv in ((0, 16, 96, 160), (1, 32, 96, 160), (1, 16, 16, 32)):
        codec = lla.make_codec(mode, 4, H, 128, rk, rv, lla.LLA_BF16)
        a = lla.lla_decode_absorbed_plan(codec, cache)
        b = lla.lla_decode_plan(codec, cache)
        assert (a.kernel, a.splits, a.tokens_per_split, a.workspace_bytes) == \
            (b.kernel, b.splits, b.tokens_per_split, b.workspace_bytes)
    L = lla.lib()
    assert L.lla_decode_absorbed_plan(ctypes.byref(_codec(c)), ctypes.byref(cache), None) == \
        lla.LLA_ERR_NULL


FAKE = 0x10000   # never dereferenced: every call below fails validation first


def _no_gpu():
    # the calls below carry fake device pointers; they must never reach a real device
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation checks run only where no GPU is visible")


def _status(**kw):
    c = synth.CONFIGS["ouro14_21x"]
    codec = kw.get("codec", _codec(c))
    params = lla.lla_params(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    # one sequence of up to 4096 tokens: the plan splits the context, so a workspace is needed
    cache = kw.get("cache", lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 64, 4096))
    L = lla.lib()
    return L.lla_decode_attn(ctypes.byref(codec) if codec is not None else None,
                             ctypes.byref(params), ctypes.byref(cache), kw.get("t", 0),
                             kw.get("q", FAKE), kw.get("ks", None), kw.get("vs", None), 0, 0.1,
                             FAKE, kw.get("ws", None), kw.get("wsb", 0), None)


def test_validation_codes_without_launch():
    _no_gpu()
    c = synth.CONFIGS["ouro14_21x"]
    default = lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 64, 4096)
    assert lla.lla_decode_plan(_codec(c), default).workspace_bytes > 0
    assert _status(codec=None) == lla.LLA_ERR_NULL
    assert _status(t=4) == lla.LLA_ERR_SHAPE
    assert _status(q=None) == lla.LLA_ERR_NULL
    assert _status(ks=FAKE) == lla.LLA_ERR_NULL                     # k_self without v_self
    assert _status(codec=lla.make_codec(0, 4, 16, 128, 16, 32, 5)) == lla.LLA_ERR_DTYPE
    assert _status(codec=lla.make_codec(0, 4, 16, 128, 8, 32, 1)) == lla.LLA_ERR_UNSUPPORTED
    assert _status(codec=lla.make_codec(0, 4, 16, 128, 600, 32, 1)) == lla.LLA_ERR_SHAPE
    assert _status(cache=lla.lla_cache(FAKE + 2, FAKE, FAKE, FAKE, 1, 64, 64, 64, 4096)) == \
        lla.LLA_ERR_ALIGN
    assert _status(cache=lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 64, 4097)) == \
        lla.LLA_ERR_SHAPE                                                # max_seq_len > pages*P
    assert _status(cache=lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 1, 48, 86, 86, 4096)) == \
        lla.LLA_ERR_SHAPE                                                # P not a multiple of 32
    assert _status() == lla.LLA_ERR_WORKSPACE                            # no workspace
    assert _status(ws=FAKE + 4, wsb=1 << 20) == lla.LLA_ERR_ALIGN
    # 2^21 pages x 16 heads x 64 slots = 2^31 pool rows: past the kernels' 32-bit row index
    huge = lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 1 << 21, 4096)
    assert _status(cache=huge) == lla.LLA_ERR_UNSUPPORTED
    assert _status(cache=lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 1, 64, 64, (1 << 21) - 1,
                                       4096)) == lla.LLA_ERR_WORKSPACE   # one page fewer is fine
    L = lla.lib()
    assert L.lla_ref_attn(16, 128, lla.LLA_BF16, ctypes.byref(huge), FAKE, None, None, 0, 0.1,
                          FAKE, None, 0, None) == lla.LLA_ERR_UNSUPPORTED


def test_status_strings():
    for s in range(8):
        assert lla.lla_status_str(s)
    assert lla.lla_version().count(".") == 2


def test_stream_read_validation_without_launch():
    _no_gpu()
    L = lla.lib()
    assert L.lla_stream_read(None, 16, FAKE, None) == lla.LLA_ERR_NULL
    assert L.lla_stream_read(FAKE, 16, None, None) == lla.LLA_ERR_NULL
    assert L.lla_stream_read(FAKE + 8, 16, FAKE, None) == lla.LLA_ERR_ALIGN
    assert L.lla_stream_read(FAKE, 16, FAKE + 2, None) == lla.LLA_ERR_ALIGN
    assert L.lla_stream_read(FAKE, 24, FAKE, None) == lla.LLA_ERR_SHAPE
    assert L.lla_stream_read(FAKE, 0, FAKE, None) == lla.LLA_OK        # nothing to read


def test_absorbed_validation_without_launch():
    _no_gpu()
    c = synth.CONFIGS["ouro14_21x"]
    L = lla.lib()
    params = lla.lla_params(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    cache = lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 64, 4096)

    def call(codec, ws=None, wsb=0):
        return L.lla_decode_attn_absorbed(ctypes.byref(codec), ctypes.byref(params),
                                          ctypes.byref(cache), 0, FAKE, None, None, 0, 0.1, FAKE,
                                          ws, wsb, None)
    # fp32 codecs have no absorbed kernel; the rest validates like lla_decode_attn
    assert call(lla.make_codec(0, 4, 16, 128, 16, 32, lla.LLA_F32)) == lla.LLA_ERR_DTYPE
    assert call(lla.make_codec(0, 4, 16, 128, 8, 32, lla.LLA_BF16)) == lla.LLA_ERR_UNSUPPORTED
    assert call(_codec(c)) == lla.LLA_ERR_WORKSPACE


def test_rope_validation_without_launch():
    _no_gpu()
    c = synth.CONFIGS["ouro14_21x"]
    L = lla.lib()
    params = lla.lla_params(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    cache = lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 64, 4096)
    ws = FAKE            # validation stops before the workspace would be read

    def call(rope, codec=None, wsb=1 << 30):
        codec = codec or _codec(c)
        return L.lla_decode_attn_rope(ctypes.byref(codec), ctypes.byref(params),
                                      ctypes.byref(cache), 0,
                                      None if rope is None else ctypes.byref(rope), FAKE, None,
                                      None, 0, 0.1, FAKE, ws, wsb, None)
    assert call(None) == lla.LLA_ERR_NULL
    assert call(lla.lla_rope(10000.0, 128, 0), lla.make_codec(0, 4, 16, 128, 16, 32,
                                                              lla.LLA_F32)) == lla.LLA_ERR_DTYPE
    assert call(lla.lla_rope(1.0, 128, 0)) == lla.LLA_ERR_SHAPE
    assert call(lla.lla_rope(10000.0, 128, 2)) == lla.LLA_ERR_SHAPE
    assert call(lla.lla_rope(10000.0, 130, 0)) == lla.LLA_ERR_SHAPE     # wider than the head
    assert call(lla.lla_rope(10000.0, 63, 0)) == lla.LLA_ERR_SHAPE      # odd
    assert call(lla.lla_rope(10000.0, -2, 1)) == lla.LLA_ERR_SHAPE
    assert call(lla.lla_rope(10000.0, 64, 0), wsb=0) == lla.LLA_ERR_WORKSPACE   # partial: valid
    assert call(lla.lla_rope(10000.0, 128, 0), wsb=0) == lla.LLA_ERR_WORKSPACE


def test_prefill_validation_without_launch():
    _no_gpu()
    c = synth.CONFIGS["ouro14_21x"]
    L = lla.lib()
    params = lla.lla_params(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    cache = lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 64, 4096)

    def call(codec=None, t=0, chunk=8, n_new=FAKE, stride=0, q=FAKE, cache_=None):
        codec = codec or _codec(c)
        return L.lla_prefill_attn(ctypes.byref(codec), ctypes.byref(params),
                                  ctypes.byref(cache_ or cache), t, chunk, n_new, q, FAKE, FAKE,
                                  stride, 0.1, FAKE, None)
    assert call(lla.make_codec(0, 4, 16, 128, 16, 32, lla.LLA_F32)) == lla.LLA_ERR_DTYPE
    assert call(lla.make_codec(0, 4, 16, 128, 96, 128, lla.LLA_BF16)) == lla.LLA_ERR_UNSUPPORTED
    assert call(lla.make_codec(0, 4, 16, 128, 32, 128, lla.LLA_BF16)) == lla.LLA_ERR_UNSUPPORTED
    assert call(n_new=None) == lla.LLA_ERR_NULL
    assert call(t=4) == lla.LLA_ERR_SHAPE
    assert call(chunk=-1) == lla.LLA_ERR_SHAPE
    assert call(stride=16 * 128 - 8) == lla.LLA_ERR_SHAPE          # shorter than a row
    assert call(stride=16 * 128 + 4) == lla.LLA_ERR_SHAPE          # not a multiple of 8
    assert call(chunk=1 << 14, stride=1 << 17) == lla.LLA_ERR_SHAPE  # row offsets past 2^31
    assert call(q=FAKE + 8) == lla.LLA_ERR_ALIGN
    odd_pages = lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 1, 48, 64, 64, 3072)
    assert call(cache_=odd_pages) == lla.LLA_ERR_SHAPE
    # 2^21 pages x 16 heads x 64 slots = 2^31 pool rows: past the kernels' 32-bit row index
    huge = lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 1 << 21, 4096)
    assert call(cache_=huge) == lla.LLA_ERR_UNSUPPORTED
    assert call(chunk=0) == lla.LLA_OK                              # nothing to do
    empty = lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 0, 64, 64, 64, 0)
    assert call(cache_=empty) == lla.LLA_OK


def test_encode_chunk_validation_without_launch():
    _no_gpu()
    c = synth.CONFIGS["ouro14_21x"]
    L = lla.lib()
    params = lla.lla_params(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    cache = lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 64, 4096)

    def call(chunk=8, n_new=FAKE, x=FAKE):
        return L.lla_encode_chunk(ctypes.byref(_codec(c)), ctypes.byref(params),
                                  ctypes.byref(cache), chunk, n_new, x, FAKE, FAKE, None, None,
                                  None)
    assert call(n_new=None) == lla.LLA_ERR_NULL
    assert call(chunk=-1) == lla.LLA_ERR_SHAPE
    assert call(chunk=(1 << 30) + 1) == lla.LLA_ERR_SHAPE
    assert call(x=None) == lla.LLA_ERR_NULL
    assert call(x=FAKE + 8) == lla.LLA_ERR_ALIGN
    assert call(chunk=0) == lla.LLA_OK


def test_fit_validation_without_launch():
    _no_gpu()
    L = lla.lib()
    bf = lla.make_codec(0, 4, 16, 128, 16, 32, lla.LLA_BF16)
    sz = ctypes.c_size_t(0)
    assert L.lla_fit_plan(ctypes.byref(bf), 16, 4096, ctypes.byref(sz)) == lla.LLA_OK
    need = sz.value
    assert need > 0
    assert L.lla_fit_plan(ctypes.byref(bf), 16, 4096, None) == lla.LLA_ERR_NULL
    f32 = lla.make_codec(0, 4, 16, 128, 16, 32, lla.LLA_F32)
    assert L.lla_fit_plan(ctypes.byref(f32), 16, 4096, ctypes.byref(sz)) == lla.LLA_ERR_DTYPE
    assert L.lla_fit_plan(ctypes.byref(bf), 0, 4096, ctypes.byref(sz)) == lla.LLA_ERR_SHAPE
    assert L.lla_fit_plan(ctypes.byref(bf), 161, 4096, ctypes.byref(sz)) == \
        lla.LLA_ERR_UNSUPPORTED
    odd = lla.make_codec(0, 3, 16, 64, 16, 32, lla.LLA_BF16)          # X = 192
    assert L.lla_fit_plan(ctypes.byref(odd), 16, 4096, ctypes.byref(sz)) == \
        lla.LLA_ERR_UNSUPPORTED
    assert L.lla_fit_plan(ctypes.byref(bf), 16, 24, ctypes.byref(sz)) == lla.LLA_ERR_SHAPE

    def call(ws=FAKE, wsb=need, x=FAKE, iters=10):
        return L.lla_fit_svd(ctypes.byref(bf), 16, x, 4096, iters, FAKE, FAKE, FAKE, None, ws,
                             wsb, None)
    assert call(wsb=need - 4) == lla.LLA_ERR_WORKSPACE
    assert call(ws=None) == lla.LLA_ERR_NULL
    assert call(x=FAKE + 8) == lla.LLA_ERR_ALIGN
    assert call(iters=-1) == lla.LLA_ERR_SHAPE


def test_encode_layers_validation_without_launch():
    _no_gpu()
    c = synth.CONFIGS["ouro14_21x"]
    codec = _codec(c)
    L = lla.lib()
    params = lla.lla_params(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    cache = lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 64, 4096)

    def call(n=2, caches=None, xk=FAKE, prm=params, wp=FAKE):
        m = max(n, 1)
        pa = (lla.lla_params * m)(*[prm] * m)
        ca = caches if caches is not None else (lla.lla_cache * m)(*[cache] * m)
        xs = (ctypes.c_void_p * m)(*[xk] * m)
        return L.lla_encode_append_layers(ctypes.byref(codec), n, pa, ca, xs, xs, wp, None)
    assert call(n=-1) == lla.LLA_ERR_SHAPE
    assert call(n=0) == lla.LLA_OK                                   # nothing to do
    assert call(wp=None) == lla.LLA_ERR_NULL
    assert call(xk=None) == lla.LLA_ERR_NULL
    assert call(xk=FAKE + 8) == lla.LLA_ERR_ALIGN
    assert call(prm=lla.lla_params(FAKE, None, FAKE, FAKE, FAKE, FAKE)) == lla.LLA_ERR_NULL
    other_batch = lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 2, 64, 64, 64, 4096)
    assert call(caches=(lla.lla_cache * 2)(cache, other_batch)) == lla.LLA_ERR_SHAPE
    other_pages = lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 65, 4096)
    assert call(caches=(lla.lla_cache * 2)(cache, other_pages)) == lla.LLA_ERR_SHAPE
    empty = lla.lla_cache(FAKE, FAKE, FAKE, FAKE, 0, 64, 64, 64, 0)
    assert call(caches=(lla.lla_cache * 2)(empty, empty)) == lla.LLA_OK   # empty batch
    bad_codec = lla.make_codec(0, 4, 16, 128, 16, 32, 5)
    m = 2
    assert L.lla_encode_append_layers(ctypes.byref(bad_codec), m, (lla.lla_params * m)(params, params),
                                      (lla.lla_cache * m)(cache, cache),
                                      (ctypes.c_void_p * m)(FAKE, FAKE),
                                      (ctypes.c_void_p * m)(FAKE, FAKE), FAKE, None) == \
        lla.LLA_ERR_DTYPE
