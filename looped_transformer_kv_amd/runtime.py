"""Device-side containers around the C ABI: one layer's codec parameters and paged latent cache.

torch is used only to allocate device memory and to name streams; every computation is a call
into liblla.so through `lla`.
"""
import math

from . import lla


def dtype_code(torch_dtype) -> int:
    import torch
    if torch_dtype == torch.bfloat16:
        return lla.LLA_BF16
    if torch_dtype == torch.float32:
        return lla.LLA_F32
    raise ValueError(f"unsupported dtype {torch_dtype}")


class LatentLayer:
    """Codec parameters ([G][X][r] W_down, [T][G][r][D_g] W_up, [G][X] mu per axis) and a paged
    latent cache ([n_pages][G][P][r] pools, [B][max_pages] block table, [B] lengths) of one layer.
    """

    def __init__(self, codec: lla.lla_codec, W_down_k, W_down_v, W_up_k, W_up_v, mu_k, mu_v,
                 k_pool, v_pool, block_table, seq_lens, page_size: int, max_seq_len: int):
        self.codec = codec
        self.tensors = dict(W_down_k=W_down_k, W_down_v=W_down_v, W_up_k=W_up_k, W_up_v=W_up_v,
                            mu_k=mu_k, mu_v=mu_v, k_pool=k_pool, v_pool=v_pool,
                            block_table=block_table, seq_lens=seq_lens)
        self.params = lla.make_params(W_down_k, W_down_v, W_up_k, W_up_v, mu_k, mu_v)
        self.page_size = page_size
        self.set_max_seq_len(max_seq_len)

    def set_max_seq_len(self, max_seq_len: int):
        t = self.tensors
        self.cache = lla.make_cache(t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    self.page_size, max_seq_len)
        self.plan = lla.lla_decode_plan(self.codec, self.cache)
        self.absorbed_plan = lla.lla_decode_absorbed_plan(self.codec, self.cache)

    def workspace(self, device):
        """One workspace for every decode entry point (the larger of the two plans)."""
        import torch
        need = max(self.plan.workspace_bytes, self.absorbed_plan.workspace_bytes)
        n = max(4, (need + 3) // 4)
        return torch.empty(n, dtype=torch.float32, device=device)

    def decode(self, t, q, out, workspace, k_self=None, v_self=None, self_stride=0, scale=None,
               stream=None, check=True):
        if scale is None:
            scale = 1.0 / math.sqrt(self.codec.d_head)
        return lla.lla_decode_attn(self.codec, self.params, self.cache, t, q, k_self, v_self,
                                   self_stride, scale, out, workspace, stream=stream, check=check)

    def decode_rope(self, t, rope, q, out, workspace, k_self=None, v_self=None, self_stride=0,
                    scale=None, stream=None, check=True):
        """Decode with the rotation after reconstruction (lla_decode_attn_rope); same workspace."""
        if scale is None:
            scale = 1.0 / math.sqrt(self.codec.d_head)
        return lla.lla_decode_attn_rope(self.codec, self.params, self.cache, t, rope, q, k_self,
                                        v_self, self_stride, scale, out, workspace,
                                        stream=stream, check=check)

    def decode_absorbed(self, t, q, out, workspace, k_self=None, v_self=None, self_stride=0,
                        scale=None, stream=None, check=True):
        """The same attention in the latent space (lla_decode_attn_absorbed); the workspace of
        `workspace()` covers its plan."""
        if scale is None:
            scale = 1.0 / math.sqrt(self.codec.d_head)
        return lla.lla_decode_attn_absorbed(self.codec, self.params, self.cache, t, q, k_self,
                                            v_self, self_stride, scale, out, workspace,
                                            stream=stream, check=check)

    def encode_append(self, x_k, x_v, write_pos, c_k_out=None, c_v_out=None, stream=None,
                      check=True):
        return lla.lla_encode_append(self.codec, self.params, self.cache, x_k, x_v, write_pos,
                                     c_k_out, c_v_out, stream=stream, check=check)

    @staticmethod
    def encode_append_layers(layers, x_k, x_v, write_pos, stream=None, check=True):
        """lla_encode_append for every layer of `layers` in one call (lla_encode_append_layers);
        x_k[i], x_v[i] are layer i's staging tensors."""
        return lla.lla_encode_append_layers(layers[0].codec, [L.params for L in layers],
                                            [L.cache for L in layers], x_k, x_v, write_pos,
                                            stream=stream, check=check)

    def prefill(self, t, chunk, n_new, q, k_new, v_new, out, new_stride=0, scale=None,
                stream=None, check=True):
        """Chunked prefill attention of loop t (lla_prefill_attn): q, out [B][chunk][H][d]."""
        if scale is None:
            scale = 1.0 / math.sqrt(self.codec.d_head)
        return lla.lla_prefill_attn(self.codec, self.params, self.cache, t, chunk, n_new, q,
                                    k_new, v_new, new_stride, scale, out, stream=stream,
                                    check=check)

    def encode_chunk(self, chunk, n_new, x_k, x_v, write_pos, c_k_out=None, c_v_out=None,
                     stream=None, check=True):
        """Bulk encode and append of a chunk (lla_encode_chunk): x [B][chunk][T][H][d]."""
        return lla.lla_encode_chunk(self.codec, self.params, self.cache, chunk, n_new, x_k, x_v,
                                    write_pos, c_k_out, c_v_out, stream=stream, check=check)
