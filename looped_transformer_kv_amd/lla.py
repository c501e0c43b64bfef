"""Thin ctypes binding of liblla.so (include/lla.h): argument marshalling only.

Every computation runs in the library's HIP kernels.  Functions carry the C names; tensors are
passed as raw device pointers (`tensor.data_ptr()`), streams as raw hipStream_t handles (default:
torch's current stream).  A missing library is an error, never a fallback.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblla.so")

LLA_OK, LLA_ERR_NULL, LLA_ERR_SHAPE, LLA_ERR_DTYPE, LLA_ERR_ALIGN, LLA_ERR_WORKSPACE, \
    LLA_ERR_UNSUPPORTED, LLA_ERR_HIP = range(8)
LLA_F32, LLA_BF16 = 0, 1
LLA_PER_HEAD, LLA_2D = 0, 1


class LLAError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {lla_status_str(status)} (status {status})")


class lla_codec(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("T", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("d_head", ctypes.c_int32), ("r_k", ctypes.c_int32), ("r_v", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class lla_params(ctypes.Structure):
    _fields_ = [("W_down_k", ctypes.c_void_p), ("W_down_v", ctypes.c_void_p),
                ("W_up_k", ctypes.c_void_p), ("W_up_v", ctypes.c_void_p),
                ("mu_k", ctypes.c_void_p), ("mu_v", ctypes.c_void_p)]


class lla_cache(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("n_pages", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32)]


class lla_rope(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_float), ("rot_dims", ctypes.c_int32), ("style", ctypes.c_int32)]


class lla_plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("tokens_per_split", ctypes.c_int32), ("waves_per_block", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]


_lib = None


def lib():
    """The loaded liblla.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m "
                              "looped_transformer_kv_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_size_t)
        L.lla_compression_ratio.restype = ctypes.c_double
        L.lla_compression_ratio.argtypes = [P(lla_codec)]
        L.lla_latent_bytes_per_token.restype = sz
        L.lla_latent_bytes_per_token.argtypes = [P(lla_codec)]
        L.lla_flat_bytes_per_token.restype = sz
        L.lla_flat_bytes_per_token.argtypes = [P(lla_codec)]
        L.lla_decode_plan.restype = i32
        L.lla_decode_plan.argtypes = [P(lla_codec), P(lla_cache), P(lla_plan)]
        L.lla_decode_absorbed_plan.restype = i32
        L.lla_decode_absorbed_plan.argtypes = [P(lla_codec), P(lla_cache), P(lla_plan)]
        L.lla_decode_workspace_size.restype = i32
        L.lla_decode_workspace_size.argtypes = [P(lla_codec), P(lla_cache), P(sz)]
        L.lla_decode_attn.restype = i32
        L.lla_decode_attn.argtypes = [P(lla_codec), P(lla_params), P(lla_cache), i32, vp, vp, vp,
                                      i64, f32, vp, vp, sz, vp]
        L.lla_decode_attn_noalloc.restype = i32
        L.lla_decode_attn_noalloc.argtypes = [P(lla_codec), P(lla_params), P(lla_cache), i32, vp,
                                              vp, vp, i64, f32, vp, vp]
        L.lla_decode_attn_rope.restype = i32
        L.lla_decode_attn_rope.argtypes = [P(lla_codec), P(lla_params), P(lla_cache), i32,
                                           P(lla_rope), vp, vp, vp, i64, f32, vp, vp, sz, vp]
        L.lla_decode_attn_absorbed.restype = i32
        L.lla_decode_attn_absorbed.argtypes = [P(lla_codec), P(lla_params), P(lla_cache), i32, vp,
                                               vp, vp, i64, f32, vp, vp, sz, vp]
        L.lla_encode_append.restype = i32
        L.lla_encode_append.argtypes = [P(lla_codec), P(lla_params), P(lla_cache), vp, vp, vp, vp,
                                        vp, vp]
        L.lla_encode_chunk.restype = i32
        L.lla_encode_append_layers.restype = i32
        L.lla_encode_append_layers.argtypes = [P(lla_codec), i32, P(lla_params), P(lla_cache),
                                               P(vp), P(vp), vp, vp]
        L.lla_encode_chunk.argtypes = [P(lla_codec), P(lla_params), P(lla_cache), i32, vp, vp, vp,
                                       vp, vp, vp, vp]
        L.lla_prefill_attn.restype = i32
        L.lla_prefill_attn.argtypes = [P(lla_codec), P(lla_params), P(lla_cache), i32, i32, vp, vp,
                                       vp, vp, i64, f32, vp, vp]
        L.lla_fit_plan.restype = i32
        L.lla_fit_plan.argtypes = [P(lla_codec), i32, i64, P(sz)]
        L.lla_fit_svd.restype = i32
        L.lla_fit_svd.argtypes = [P(lla_codec), i32, vp, i64, i32, vp, vp, vp, vp, vp, sz, vp]
        L.lla_ref_plan.restype = i32
        L.lla_ref_plan.argtypes = [i32, i32, i32, P(lla_cache), P(lla_plan)]
        L.lla_ref_attn.restype = i32
        L.lla_ref_attn.argtypes = [i32, i32, i32, P(lla_cache), vp, vp, vp, i64, f32, vp, vp, sz,
                                   vp]
        L.lla_stream_read.restype = i32
        L.lla_stream_read.argtypes = [vp, sz, vp, vp]
        L.lla_status_str.restype = ctypes.c_char_p
        L.lla_status_str.argtypes = [i32]
        L.lla_version.restype = ctypes.c_char_p
        L.lla_version.argtypes = []
        _lib = L
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn, status, check):
    if check and status != LLA_OK:
        raise LLAError(fn, status)
    return status


# ------------------------------------------------------------------ struct builders
def make_codec(mode, T, n_heads, d_head, r_k, r_v, dtype) -> lla_codec:
    return lla_codec(mode, T, n_heads, d_head, r_k, r_v, dtype)


def make_params(W_down_k=None, W_down_v=None, W_up_k=None, W_up_v=None, mu_k=None,
                mu_v=None) -> lla_params:
    return lla_params(_ptr(W_down_k), _ptr(W_down_v), _ptr(W_up_k), _ptr(W_up_v), _ptr(mu_k),
                      _ptr(mu_v))


def make_cache(k_pool, v_pool, block_table, seq_lens, page_size, max_seq_len, batch=None,
               max_pages=None, n_pages=None) -> lla_cache:
    """Pools [n_pages][G|H][P][r|d]; block_table [B][max_pages] int32; seq_lens [B] int32."""
    if batch is None:
        batch = block_table.shape[0]
    if max_pages is None:
        max_pages = block_table.shape[1]
    if n_pages is None:
        n_pages = k_pool.shape[0]
    return lla_cache(_ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), batch,
                     page_size, max_pages, n_pages, max_seq_len)


# ------------------------------------------------------------------ entry points (C names)
def lla_compression_ratio(codec: lla_codec) -> float:
    return float(lib().lla_compression_ratio(ctypes.byref(codec)))


def lla_latent_bytes_per_token(codec: lla_codec) -> int:
    return int(lib().lla_latent_bytes_per_token(ctypes.byref(codec)))


def lla_flat_bytes_per_token(codec: lla_codec) -> int:
    return int(lib().lla_flat_bytes_per_token(ctypes.byref(codec)))


def lla_decode_plan(codec: lla_codec, cache: lla_cache) -> lla_plan:
    plan = lla_plan()
    _check("lla_decode_plan",
           lib().lla_decode_plan(ctypes.byref(codec), ctypes.byref(cache), ctypes.byref(plan)),
           True)
    return plan


def lla_decode_absorbed_plan(codec: lla_codec, cache: lla_cache) -> lla_plan:
    plan = lla_plan()
    _check("lla_decode_absorbed_plan",
           lib().lla_decode_absorbed_plan(ctypes.byref(codec), ctypes.byref(cache),
                                          ctypes.byref(plan)), True)
    return plan


def lla_decode_workspace_size(codec: lla_codec, cache: lla_cache) -> int:
    out = ctypes.c_size_t(0)
    _check("lla_decode_workspace_size", lib().lla_decode_workspace_size(
        ctypes.byref(codec), ctypes.byref(cache), ctypes.byref(out)), True)
    return int(out.value)


def lla_decode_attn(codec, params, cache, t, q, k_self, v_self, self_stride, scale, out,
                    workspace, workspace_bytes=None, stream=None, check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().lla_decode_attn(ctypes.byref(codec), ctypes.byref(params), ctypes.byref(cache),
                               int(t), _ptr(q), _ptr(k_self), _ptr(v_self), int(self_stride),
                               float(scale), _ptr(out), _ptr(workspace), int(workspace_bytes),
                               _stream(stream))
    return _check("lla_decode_attn", st, check)


def lla_decode_attn_noalloc(codec, params, cache, t, q, k_self, v_self, self_stride, scale, out,
                            stream=None, check=True) -> int:
    """lla_decode_attn without a workspace (the library's own per-device scratch array)."""
    st = lib().lla_decode_attn_noalloc(ctypes.byref(codec), ctypes.byref(params),
                                       ctypes.byref(cache), int(t), _ptr(q), _ptr(k_self),
                                       _ptr(v_self), int(self_stride), float(scale), _ptr(out),
                                       _stream(stream))
    return _check("lla_decode_attn_noalloc", st, check)


def lla_decode_attn_rope(codec, params, cache, t, rope, q, k_self, v_self, self_stride, scale,
                         out, workspace, workspace_bytes=None, stream=None, check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().lla_decode_attn_rope(ctypes.byref(codec), ctypes.byref(params), ctypes.byref(cache),
                                    int(t), ctypes.byref(rope), _ptr(q), _ptr(k_self),
                                    _ptr(v_self), int(self_stride), float(scale), _ptr(out),
                                    _ptr(workspace), int(workspace_bytes), _stream(stream))
    return _check("lla_decode_attn_rope", st, check)


def lla_decode_attn_absorbed(codec, params, cache, t, q, k_self, v_self, self_stride, scale, out,
                             workspace, workspace_bytes=None, stream=None, check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().lla_decode_attn_absorbed(ctypes.byref(codec), ctypes.byref(params),
                                        ctypes.byref(cache), int(t), _ptr(q), _ptr(k_self),
                                        _ptr(v_self), int(self_stride), float(scale), _ptr(out),
                                        _ptr(workspace), int(workspace_bytes), _stream(stream))
    return _check("lla_decode_attn_absorbed", st, check)


def lla_encode_append(codec, params, cache, x_k, x_v, write_pos, c_k_out=None, c_v_out=None,
                      stream=None, check=True) -> int:
    st = lib().lla_encode_append(ctypes.byref(codec), ctypes.byref(params), ctypes.byref(cache),
                                 _ptr(x_k), _ptr(x_v), _ptr(write_pos), _ptr(c_k_out),
                                 _ptr(c_v_out), _stream(stream))
    return _check("lla_encode_append", st, check)


def lla_encode_append_layers(codec, params, caches, x_k, x_v, write_pos, stream=None,
                             check=True) -> int:
    """Encode and append for len(params) layers in one call: params and caches are sequences of
    lla_params / lla_cache, x_k and x_v sequences of staging tensors (or device pointers)."""
    n = len(params)
    assert len(caches) == n and len(x_k) == n and len(x_v) == n
    pa = (lla_params * n)(*params)
    ca = (lla_cache * n)(*caches)
    xk = (ctypes.c_void_p * n)(*[_ptr(x) for x in x_k])
    xv = (ctypes.c_void_p * n)(*[_ptr(x) for x in x_v])
    st = lib().lla_encode_append_layers(ctypes.byref(codec), int(n), pa, ca, xk, xv,
                                        _ptr(write_pos), _stream(stream))
    return _check("lla_encode_append_layers", st, check)


def lla_encode_chunk(codec, params, cache, chunk, n_new, x_k, x_v, write_pos, c_k_out=None,
                     c_v_out=None, stream=None, check=True) -> int:
    st = lib().lla_encode_chunk(ctypes.byref(codec), ctypes.byref(params), ctypes.byref(cache),
                                int(chunk), _ptr(n_new), _ptr(x_k), _ptr(x_v), _ptr(write_pos),
                                _ptr(c_k_out), _ptr(c_v_out), _stream(stream))
    return _check("lla_encode_chunk", st, check)


def lla_prefill_attn(codec, params, cache, t, chunk, n_new, q, k_new, v_new, new_stride, scale,
                     out, stream=None, check=True) -> int:
    st = lib().lla_prefill_attn(ctypes.byref(codec), ctypes.byref(params), ctypes.byref(cache),
                                int(t), int(chunk), _ptr(n_new), _ptr(q), _ptr(k_new),
                                _ptr(v_new), int(new_stride), float(scale), _ptr(out),
                                _stream(stream))
    return _check("lla_prefill_attn", st, check)


def lla_fit_plan(codec, r, n) -> int:
    out = ctypes.c_size_t(0)
    _check("lla_fit_plan", lib().lla_fit_plan(ctypes.byref(codec), int(r), int(n),
                                              ctypes.byref(out)), True)
    return int(out.value)


def lla_fit_svd(codec, r, x, n, iters, mu, W_down, W_up, sigma, workspace, workspace_bytes=None,
                stream=None, check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().lla_fit_svd(ctypes.byref(codec), int(r), _ptr(x), int(n), int(iters), _ptr(mu),
                           _ptr(W_down), _ptr(W_up), _ptr(sigma), _ptr(workspace),
                           int(workspace_bytes), _stream(stream))
    return _check("lla_fit_svd", st, check)


def lla_ref_plan(n_heads, d_head, dtype, flat: lla_cache) -> lla_plan:
    plan = lla_plan()
    _check("lla_ref_plan", lib().lla_ref_plan(n_heads, d_head, dtype, ctypes.byref(flat),
                                              ctypes.byref(plan)), True)
    return plan


def lla_ref_attn(n_heads, d_head, dtype, flat, q, k_self, v_self, self_stride, scale, out,
                 workspace, workspace_bytes=None, stream=None, check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().lla_ref_attn(n_heads, d_head, dtype, ctypes.byref(flat), _ptr(q), _ptr(k_self),
                            _ptr(v_self), int(self_stride), float(scale), _ptr(out),
                            _ptr(workspace), int(workspace_bytes), _stream(stream))
    return _check("lla_ref_attn", st, check)


def lla_stream_read(buf, sink, nbytes=None, stream=None, check=True) -> int:
    """Stream `nbytes` (default: all) of the device tensor `buf` once (a read-bandwidth probe);
    workgroup w stores the XOR of the 32-bit words it read in sink[w] (an int32 device tensor of
    at least 512 entries)."""
    if nbytes is None:
        nbytes = buf.numel() * buf.element_size()
    st = lib().lla_stream_read(_ptr(buf), int(nbytes), _ptr(sink), _stream(stream))
    return _check("lla_stream_read", st, check)


def lla_status_str(status: int) -> str:
    return lib().lla_status_str(int(status)).decode()


def lla_version() -> str:
    return lib().lla_version().decode()
