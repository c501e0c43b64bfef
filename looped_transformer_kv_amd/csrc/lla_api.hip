// lla_api.hip -- the C ABI of liblla.so (declared in include/lla.h): argument validation, split
// planning and kernel launches.  No allocation, no global mutable state, no host synchronisation.
#include <cstdint>

#include <cmath>
#include <mutex>
#include <vector>

#include "lla_internal.h"

namespace lla {
size_t decode_f32_lds_bytes(int d, int r_k, int r_v);
}

using namespace lla;

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr size_t kMaxDynLds = 64 * 1024;

struct Shape {
    int G, Dg;
    long X;
};

Shape shape_of(const lla_codec *c) {
    Shape s;
    s.G = c->mode == LLA_2D ? 1 : c->n_heads;
    s.Dg = c->mode == LLA_2D ? c->n_heads * c->d_head : c->d_head;
    s.X = (long)c->T * s.Dg;
    return s;
}

size_t elt_size(int dtype) { return dtype == LLA_BF16 ? 2 : 4; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

lla_status check_codec(const lla_codec *c) {
    if (!c) return LLA_ERR_NULL;
    if (c->dtype != LLA_F32 && c->dtype != LLA_BF16) return LLA_ERR_DTYPE;
    if (c->mode != LLA_PER_HEAD && c->mode != LLA_2D) return LLA_ERR_SHAPE;
    if (c->T < 1 || c->T > 64 || c->n_heads < 1 || c->n_heads > 4096) return LLA_ERR_SHAPE;
    if (c->d_head != 64 && c->d_head != 128) return LLA_ERR_SHAPE;
    const long X = shape_of(c).X;
    if (c->r_k < 1 || c->r_v < 1 || c->r_k > X || c->r_v > X) return LLA_ERR_SHAPE;
    return LLA_OK;
}

// Pools, block table and sizes of a paged cache.  seq_lens is required only for decode.
lla_status check_cache(const lla_cache *k, bool need_lens) {
    if (!k) return LLA_ERR_NULL;
    if (!k->k_pool || !k->v_pool || !k->block_table || (need_lens && !k->seq_lens))
        return LLA_ERR_NULL;
    if (k->batch < 0 || k->page_size < 1 || k->max_pages < 1 || k->n_pages < 1 ||
        k->max_seq_len < 0 || (long)k->max_seq_len > (long)k->max_pages * k->page_size)
        return LLA_ERR_SHAPE;
    if (!aligned16(k->k_pool) || !aligned16(k->v_pool)) return LLA_ERR_ALIGN;
    return LLA_OK;
}

// Workgroups a decode call aims for: context splits are added until B*H*S reaches it (two
// workgroups of four waves per compute unit on the 256-CU chip).
constexpr int kTargetBlocks = 512;

// Context splits: enough workgroups to fill the chip, each covering a multiple of `unit`
// tokens and at most `max_tps` tokens.
void split_plan(int rows, int max_len, int unit, int max_tps, lla_plan *p,
                int target = kTargetBlocks) {
    const int chunks = (max_len + unit - 1) / unit;
    int S = (target + rows - 1) / (rows > 0 ? rows : 1);
    const int S_min = (max_len + max_tps - 1) / max_tps;
    if (S > chunks) S = chunks;
    if (S < S_min) S = S_min;
    if (S < 1) S = 1;
    int tps = (max_len + S - 1) / S;
    tps = ((tps + unit - 1) / unit) * unit;
    if (tps < unit) tps = unit;
    S = (max_len + tps - 1) / tps;
    if (S < 1) S = 1;
    p->splits = S;
    p->tokens_per_split = tps;
}

lla_status decode_plan(const lla_codec *c, const lla_cache *k, lla_plan *p) {
    const bool bf16 = c->dtype == LLA_BF16;
    p->kernel = bf16 ? 1 : 2;
    p->waves_per_block = 4;
    // fp32 caches (small configurations) split in 32-token units: each split's workgroup rebuilds
    // its tokens one per thread, so short contexts need several splits to use more than a few CUs
    split_plan(k->batch * c->n_heads, k->max_seq_len, bf16 ? 32 * 4 : 32,
               bf16 ? 32 * kMaxChunksPerSplit : (1 << 30), p);
    // a single-split bf16 plan finishes in the latent kernel and needs no partials
    const bool direct = bf16 && p->splits == 1;
    p->workspace_bytes = direct ? 0 : (size_t)k->batch * c->n_heads * p->splits *
                                          (c->d_head + kPartialPad) * sizeof(float);
    return LLA_OK;
}

// Workgroups the all-heads absorbed LLA-2D kernel aims for (two of four waves per compute unit).
constexpr int kAbs2dTargetBlocks = 512;

// lla_decode_attn_absorbed: LLA-2D codecs the all-heads kernel takes split each sequence's
// context on its own (one workgroup per (sequence, split) serves every head); its workspace holds
// q~, the per-split latent partials and their (max, sum).  Every other codec: lla_decode_plan.
lla_status absorbed_plan(const lla_codec *c, const lla_cache *k, lla_plan *p) {
    if (!(c->dtype == LLA_BF16 && absorbed2d_supported(c->mode == LLA_2D ? 1 : 0, c->n_heads,
                                                       c->d_head, c->r_k, c->r_v)))
        return decode_plan(c, k, p);
    p->kernel = 4;
    p->waves_per_block = 4;
    split_plan(k->batch, k->max_seq_len, 32 * 4, 32 * kMaxChunksPerSplit, p, kAbs2dTargetBlocks);
    if (p->splits > kMaxAbs2dSplits) return LLA_ERR_UNSUPPORTED;
    p->workspace_bytes = abs2d_layout(k->batch, p->splits, c->r_k, c->r_v).total * sizeof(float);
    return LLA_OK;
}

lla_status ref_plan(int H, int d, int dtype, const lla_cache *k, lla_plan *p) {
    (void)d;
    (void)dtype;
    p->kernel = 3;
    p->waves_per_block = 4;
    split_plan(k->batch * H, k->max_seq_len, 32 * 4, 32 * kMaxChunksPerSplit, p);
    p->workspace_bytes = (size_t)k->batch * H * p->splits * (d + kPartialPad) * sizeof(float);
    return LLA_OK;
}

lla_status check_workspace(const lla_plan &p, void *ws, size_t bytes) {
    if (p.workspace_bytes == 0) return LLA_OK;
    if (!ws || bytes < p.workspace_bytes) return LLA_ERR_WORKSPACE;
    if (!aligned16(ws)) return LLA_ERR_ALIGN;
    return LLA_OK;
}

}  // namespace

extern "C" {

double lla_compression_ratio(const lla_codec *c) {
    if (check_codec(c) != LLA_OK) return 0.0;
    const double flat = 2.0 * c->T * c->d_head * (c->mode == LLA_2D ? c->n_heads : 1);
    return flat / (double)(c->r_k + c->r_v);
}

size_t lla_latent_bytes_per_token(const lla_codec *c) {
    if (check_codec(c) != LLA_OK) return 0;
    return (size_t)shape_of(c).G * (c->r_k + c->r_v) * elt_size(c->dtype);
}

size_t lla_flat_bytes_per_token(const lla_codec *c) {
    if (check_codec(c) != LLA_OK) return 0;
    return (size_t)2 * c->T * c->n_heads * c->d_head * elt_size(c->dtype);
}

lla_status lla_decode_plan(const lla_codec *c, const lla_cache *k, lla_plan *p) {
    lla_status st = check_codec(c);
    if (st != LLA_OK) return st;
    if (!k || !p) return LLA_ERR_NULL;
    if (k->batch < 0 || k->max_seq_len < 0) return LLA_ERR_SHAPE;
    return decode_plan(c, k, p);
}

lla_status lla_decode_absorbed_plan(const lla_codec *c, const lla_cache *k, lla_plan *p) {
    lla_status st = check_codec(c);
    if (st != LLA_OK) return st;
    if (!k || !p) return LLA_ERR_NULL;
    if (k->batch < 0 || k->max_seq_len < 0) return LLA_ERR_SHAPE;
    return absorbed_plan(c, k, p);
}

lla_status lla_decode_workspace_size(const lla_codec *c, const lla_cache *k, size_t *bytes) {
    if (!bytes) return LLA_ERR_NULL;
    lla_plan p;
    const lla_status st = lla_decode_plan(c, k, &p);
    if (st != LLA_OK) return st;
    *bytes = p.workspace_bytes;
    return LLA_OK;
}

}  // extern "C"

namespace {

// Validation and kernel arguments shared by the latent decode entry points.  `bf16_only` rejects
// fp32 codecs (the absorbed and rotary kernels have no fp32 variant).
lla_status prepare_decode(const lla_codec *c, const lla_params *prm, const lla_cache *k, int32_t t,
                          const void *q, const void *k_self, const void *v_self,
                          int64_t self_stride, float scale, void *out, void *workspace,
                          size_t workspace_bytes, bool bf16_only, DecodeArgs *args,
                          lla_plan *plan, bool absorbed = false) {
    lla_status st = check_codec(c);
    if (st != LLA_OK) return st;
    if (!prm || !prm->W_up_k || !prm->W_up_v || !prm->mu_k || !prm->mu_v) return LLA_ERR_NULL;
    if ((st = check_cache(k, true)) != LLA_OK) return st;
    if (!q || !out || (k_self == nullptr) != (v_self == nullptr)) return LLA_ERR_NULL;
    if (t < 0 || t >= c->T || self_stride < 0) return LLA_ERR_SHAPE;
    const bool bf16 = c->dtype == LLA_BF16;
    if (bf16_only && !bf16) return LLA_ERR_DTYPE;
    if (bf16) {
        if (!decode_bf16_supported(c->d_head, c->r_k, c->r_v)) return LLA_ERR_UNSUPPORTED;
        if (k->page_size % 32 != 0) return LLA_ERR_SHAPE;
        // the kernels address a pool row (page, group, slot) with a signed 32-bit index
        if ((long)k->n_pages * shape_of(c).G * k->page_size > (1L << 31) - 1)
            return LLA_ERR_UNSUPPORTED;
        if (!aligned16(q) || !aligned16(prm->W_up_k) || !aligned16(prm->W_up_v))
            return LLA_ERR_ALIGN;
    } else if (decode_f32_lds_bytes(c->d_head, c->r_k, c->r_v) > kMaxDynLds) {
        return LLA_ERR_UNSUPPORTED;
    }
    if ((st = absorbed ? absorbed_plan(c, k, plan) : decode_plan(c, k, plan)) != LLA_OK)
        return st;
    if ((st = check_workspace(*plan, workspace, workspace_bytes)) != LLA_OK) return st;

    const Shape sh = shape_of(c);
    DecodeArgs &a = *args;
    a = DecodeArgs{};
    a.k_pool = k->k_pool;
    a.v_pool = k->v_pool;
    a.block_table = k->block_table;
    a.seq_lens = k->seq_lens;
    a.W_up_k = prm->W_up_k;
    a.W_up_v = prm->W_up_v;
    a.mu_k = prm->mu_k;
    a.mu_v = prm->mu_v;
    a.q = q;
    a.k_self = k_self;
    a.v_self = v_self;
    a.self_stride = self_stride ? self_stride : (int64_t)c->n_heads * c->d_head;
    a.out = out;
    a.ws = static_cast<float *>(workspace);
    a.B = k->batch;
    a.H = c->n_heads;
    a.G = sh.G;
    a.Dg = sh.Dg;
    a.T = c->T;
    a.t = t;
    a.r_k = c->r_k;
    a.r_v = c->r_v;
    a.P = k->page_size;
    a.max_pages = k->max_pages;
    a.n_pages = k->n_pages;
    a.max_seq_len = k->max_seq_len;
    a.S = plan->splits;
    a.tokens_per_split = plan->tokens_per_split;
    a.mode = c->mode;
    a.scale_log2 = scale * kLog2e;
    return LLA_OK;
}

}  // namespace

extern "C" {

lla_status lla_decode_attn(const lla_codec *c, const lla_params *prm, const lla_cache *k,
                           int32_t t, const void *q, const void *k_self, const void *v_self,
                           int64_t self_stride, float scale, void *out, void *workspace,
                           size_t workspace_bytes, void *stream) {
    DecodeArgs a;
    lla_plan plan;
    lla_status st = prepare_decode(c, prm, k, t, q, k_self, v_self, self_stride, scale, out,
                                   workspace, workspace_bytes, false, &a, &plan);
    if (st != LLA_OK) return st;
    if (k->batch == 0) return LLA_OK;
    const bool bf16 = c->dtype == LLA_BF16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = bf16 ? launch_decode_bf16(a, false, s) : launch_decode_f32(a, s);
    if (e != hipSuccess) return LLA_ERR_HIP;
    if (bf16 && plan.splits == 1) return LLA_OK;   // the latent kernel finished the output itself
    e = launch_combine(a, c->d_head, bf16, true, false, s);
    return e == hipSuccess ? LLA_OK : LLA_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------- decode without allocation
// lla_decode_attn_noalloc keeps its context-split partials in this file-scope device array
// instead of a caller workspace.  Each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, never the device memory: the
// device address comes from hipGetSymbolAddress, once per device, and only that address is used.
namespace lla {
constexpr size_t kScratchBytes = size_t(4) << 20;
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];
}  // namespace lla

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float *g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch` on each device

// The current device's copy of `scratch` (looked up on the first call on that device).
lla_status scratch_of_current_device(float **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LLA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(lla::scratch)) != hipSuccess || !p)
            return LLA_ERR_HIP;
        g_scratch_ptr[dev] = static_cast<float *>(p);
    }
    *out = g_scratch_ptr[dev];
    return LLA_OK;
}

}  // namespace

extern "C" {

lla_status lla_decode_attn_noalloc(const lla_codec *c, const lla_params *prm, const lla_cache *k,
                                   int32_t t, const void *q, const void *k_self,
                                   const void *v_self, int64_t self_stride, float scale, void *out,
                                   void *stream) {
    lla_plan plan;
    lla_status st = lla_decode_plan(c, k, &plan);
    if (st != LLA_OK) return st;
    if (plan.workspace_bytes > lla::kScratchBytes) return LLA_ERR_WORKSPACE;
    float *ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != LLA_OK) return st;
    return lla_decode_attn(c, prm, k, t, q, k_self, v_self, self_stride, scale, out, ws,
                           lla::kScratchBytes, stream);
}

lla_status lla_decode_attn_rope(const lla_codec *c, const lla_params *prm, const lla_cache *k,
                                int32_t t, const lla_rope *rope, const void *q,
                                const void *k_self, const void *v_self, int64_t self_stride,
                                float scale, void *out, void *workspace, size_t workspace_bytes,
                                void *stream) {
    if (!rope) return LLA_ERR_NULL;
    DecodeArgs a;
    lla_plan plan;
    lla_status st = prepare_decode(c, prm, k, t, q, k_self, v_self, self_stride, scale, out,
                                   workspace, workspace_bytes, true, &a, &plan);
    if (st != LLA_OK) return st;
    if (!(rope->theta > 1.0f) || !std::isfinite(rope->theta) ||
        (rope->style != 0 && rope->style != 1))
        return LLA_ERR_SHAPE;
    if (rope->rot_dims < 0 || rope->rot_dims > c->d_head || (rope->rot_dims & 1))
        return LLA_ERR_SHAPE;
    if (k->batch == 0) return LLA_OK;
    a.rope_log2_theta = std::log2(rope->theta);
    a.rope_style = rope->style;
    a.rope_rot = rope->rot_dims;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = decode_rope_heads_supported(a.mode, a.H, c->d_head, a.r_k, a.r_v)
                             ? launch_decode_rope_heads(a, s)
                             : launch_decode_bf16(a, true, s);
    if (e != hipSuccess) return LLA_ERR_HIP;
    if (plan.splits == 1) return LLA_OK;
    return launch_combine(a, c->d_head, true, true, true, s) == hipSuccess ? LLA_OK : LLA_ERR_HIP;
}

lla_status lla_decode_attn_absorbed(const lla_codec *c, const lla_params *prm,
                                    const lla_cache *k, int32_t t, const void *q,
                                    const void *k_self, const void *v_self, int64_t self_stride,
                                    float scale, void *out, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    DecodeArgs a;
    lla_plan plan;
    lla_status st = prepare_decode(c, prm, k, t, q, k_self, v_self, self_stride, scale, out,
                                   workspace, workspace_bytes, true, &a, &plan, true);
    if (st != LLA_OK) return st;
    if (k->batch == 0) return LLA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (plan.kernel == 4)
        return launch_decode_absorbed2d(a, s) == hipSuccess ? LLA_OK : LLA_ERR_HIP;
    if (launch_decode_absorbed(a, s) != hipSuccess) return LLA_ERR_HIP;
    if (plan.splits == 1) return LLA_OK;
    return launch_combine(a, c->d_head, true, true, false, s) == hipSuccess ? LLA_OK : LLA_ERR_HIP;
}

namespace {

// Shared by lla_encode_append (one row per sequence) and lla_encode_chunk (rps rows per
// sequence, n_rows live).
// Validation and kernel arguments of one layer's encode (both axes).
lla_status encode_args(const lla_codec *c, const lla_params *prm, const lla_cache *k, int rps,
                       const int32_t *n_rows, const void *x_k, const void *x_v,
                       const int32_t *write_pos, float *c_k_out, float *c_v_out,
                       EncodeArgs ax[2]) {
    lla_status st = check_codec(c);
    if (st != LLA_OK) return st;
    if (!prm || !prm->W_down_k || !prm->W_down_v || !prm->mu_k || !prm->mu_v) return LLA_ERR_NULL;
    if ((st = check_cache(k, false)) != LLA_OK) return st;
    if (!x_k || !x_v || !write_pos) return LLA_ERR_NULL;
    if (!aligned16(x_k) || !aligned16(x_v) || !aligned16(prm->mu_k) || !aligned16(prm->mu_v))
        return LLA_ERR_ALIGN;
    const Shape sh = shape_of(c);
    for (int axis = 0; axis < 2; ++axis) {
        EncodeArgs &a = ax[axis];
        a = EncodeArgs{};
        a.x = axis ? x_v : x_k;
        a.W_down = axis ? prm->W_down_v : prm->W_down_k;
        a.mu = axis ? prm->mu_v : prm->mu_k;
        a.pool = axis ? k->v_pool : k->k_pool;
        a.block_table = k->block_table;
        a.write_pos = write_pos;
        a.n_rows = n_rows;
        a.c_out = axis ? c_v_out : c_k_out;
        a.B = k->batch * rps;
        a.rps = rps;
        a.H = c->n_heads;
        a.G = sh.G;
        a.Dg = sh.Dg;
        a.T = c->T;
        a.d = c->d_head;
        a.r = axis ? c->r_v : c->r_k;
        a.P = k->page_size;
        a.max_pages = k->max_pages;
        a.n_pages = k->n_pages;
        a.mode = c->mode;
    }
    return LLA_OK;
}

lla_status encode_rows(const lla_codec *c, const lla_params *prm, const lla_cache *k, int rps,
                       const int32_t *n_rows, const void *x_k, const void *x_v,
                       const int32_t *write_pos, float *c_k_out, float *c_v_out, void *stream) {
    EncodeArgs ax[2];
    const lla_status st = encode_args(c, prm, k, rps, n_rows, x_k, x_v, write_pos, c_k_out,
                                      c_v_out, ax);
    if (st != LLA_OK) return st;
    if (k->batch == 0 || rps == 0) return LLA_OK;
    return launch_encode(ax[0], ax[1], c->dtype == LLA_BF16, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? LLA_OK
               : LLA_ERR_HIP;
}

}  // namespace

lla_status lla_encode_append(const lla_codec *c, const lla_params *prm, const lla_cache *k,
                             const void *x_k, const void *x_v, const int32_t *write_pos,
                             float *c_k_out, float *c_v_out, void *stream) {
    return encode_rows(c, prm, k, 1, nullptr, x_k, x_v, write_pos, c_k_out, c_v_out, stream);
}

lla_status lla_encode_append_layers(const lla_codec *c, int32_t n_layers,
                                    const lla_params *params, const lla_cache *caches,
                                    const void *const *x_k, const void *const *x_v,
                                    const int32_t *write_pos, void *stream) {
    if (n_layers < 0) return LLA_ERR_SHAPE;
    if (n_layers == 0) return LLA_OK;
    if (!params || !caches || !x_k || !x_v) return LLA_ERR_NULL;
    std::vector<EncodeArgs> ka(n_layers), va(n_layers);
    for (int i = 0; i < n_layers; ++i) {
        EncodeArgs ax[2];
        const lla_status st = encode_args(c, &params[i], &caches[i], 1, nullptr, x_k[i], x_v[i],
                                          write_pos, nullptr, nullptr, ax);
        if (st != LLA_OK) return st;
        const lla_cache &k = caches[i], &k0 = caches[0];
        // one batch, page geometry and set of write positions for every layer
        if (k.batch != k0.batch || k.page_size != k0.page_size || k.max_pages != k0.max_pages ||
            k.n_pages != k0.n_pages)
            return LLA_ERR_SHAPE;
        ka[i] = ax[0];
        va[i] = ax[1];
    }
    if (caches[0].batch == 0) return LLA_OK;
    return launch_encode_layers(ka.data(), va.data(), n_layers, c->dtype == LLA_BF16,
                                static_cast<hipStream_t>(stream)) == hipSuccess
               ? LLA_OK
               : LLA_ERR_HIP;
}

lla_status lla_encode_chunk(const lla_codec *c, const lla_params *prm, const lla_cache *k,
                            int32_t chunk, const int32_t *n_new, const void *x_k,
                            const void *x_v, const int32_t *write_pos, float *c_k_out,
                            float *c_v_out, void *stream) {
    if (!n_new) return LLA_ERR_NULL;
    if (chunk < 0 || (k && (long)k->batch * chunk > (1L << 30))) return LLA_ERR_SHAPE;
    return encode_rows(c, prm, k, chunk, n_new, x_k, x_v, write_pos, c_k_out, c_v_out, stream);
}

lla_status lla_prefill_attn(const lla_codec *c, const lla_params *prm, const lla_cache *k,
                            int32_t t, int32_t chunk, const int32_t *n_new, const void *q,
                            const void *k_new, const void *v_new, int64_t new_stride,
                            float scale, void *out, void *stream) {
    lla_status st = check_codec(c);
    if (st != LLA_OK) return st;
    if (c->dtype != LLA_BF16) return LLA_ERR_DTYPE;
    if (!prefill_supported(c->d_head, c->r_k, c->r_v)) return LLA_ERR_UNSUPPORTED;
    if (!prm || !prm->W_up_k || !prm->W_up_v || !prm->mu_k || !prm->mu_v) return LLA_ERR_NULL;
    if ((st = check_cache(k, true)) != LLA_OK) return st;
    if (!n_new || !q || !k_new || !v_new || !out) return LLA_ERR_NULL;
    if (t < 0 || t >= c->T || chunk < 0 || k->page_size % 32 != 0) return LLA_ERR_SHAPE;
    const long hd = (long)c->n_heads * c->d_head;
    if (new_stride == 0) new_stride = hd;
    if (new_stride < hd || new_stride % 8 != 0) return LLA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
        return LLA_ERR_ALIGN;
    if (k->batch == 0 || chunk == 0) return LLA_OK;
    const int qpb = prefill_queries_per_block();
    const long QB = ((long)chunk + qpb - 1) / qpb;
    if ((long)k->batch * c->n_heads * QB > (1L << 30) || (long)k->batch * chunk > (1L << 30))
        return LLA_ERR_SHAPE;
    // the kernel forms a chunk row's offset inside its sequence in 32-bit arithmetic
    if ((long)chunk * new_stride > (1L << 31) - 1) return LLA_ERR_SHAPE;
    const Shape sh = shape_of(c);
    // and a pool row (page, group, slot) as a signed 32-bit index
    if ((long)k->n_pages * sh.G * k->page_size > (1L << 31) - 1) return LLA_ERR_UNSUPPORTED;
    PrefillArgs a{};
    a.k_pool = k->k_pool;
    a.v_pool = k->v_pool;
    a.block_table = k->block_table;
    a.seq_lens = k->seq_lens;
    a.W_up_k = prm->W_up_k;
    a.W_up_v = prm->W_up_v;
    a.mu_k = prm->mu_k;
    a.mu_v = prm->mu_v;
    a.q = q;
    a.k_new = k_new;
    a.v_new = v_new;
    a.n_new = n_new;
    a.out = out;
    a.new_stride = new_stride;
    a.B = k->batch;
    a.H = c->n_heads;
    a.G = sh.G;
    a.Dg = sh.Dg;
    a.T = c->T;
    a.t = t;
    a.r_k = c->r_k;
    a.r_v = c->r_v;
    a.P = k->page_size;
    a.max_pages = k->max_pages;
    a.n_pages = k->n_pages;
    a.max_seq_len = k->max_seq_len;
    a.Pn = chunk;
    a.QB = (int)QB;
    a.mode = c->mode;
    a.scale_log2 = scale * kLog2e;
    return launch_prefill(a, static_cast<hipStream_t>(stream)) == hipSuccess ? LLA_OK
                                                                              : LLA_ERR_HIP;
}

lla_status lla_ref_plan(int32_t H, int32_t d, int32_t dtype, const lla_cache *k, lla_plan *p) {
    if (!k || !p) return LLA_ERR_NULL;
    if (dtype != LLA_F32 && dtype != LLA_BF16) return LLA_ERR_DTYPE;
    if (H < 1 || (d != 64 && d != 128) || k->batch < 0 || k->max_seq_len < 0)
        return LLA_ERR_SHAPE;
    return ref_plan(H, d, dtype, k, p);
}

lla_status lla_ref_attn(int32_t H, int32_t d, int32_t dtype, const lla_cache *k, const void *q,
                        const void *k_self, const void *v_self, int64_t self_stride, float scale,
                        void *out, void *workspace, size_t workspace_bytes, void *stream) {
    if (dtype != LLA_F32 && dtype != LLA_BF16) return LLA_ERR_DTYPE;
    if (H < 1 || H > 4096 || (d != 64 && d != 128)) return LLA_ERR_SHAPE;
    lla_status st = check_cache(k, true);
    if (st != LLA_OK) return st;
    if (!q || !out || (k_self == nullptr) != (v_self == nullptr)) return LLA_ERR_NULL;
    if (self_stride < 0 || k->page_size % 32 != 0) return LLA_ERR_SHAPE;
    // the kernel addresses a pool row (page, head, slot) with a signed 32-bit index
    if ((long)k->n_pages * H * k->page_size > (1L << 31) - 1) return LLA_ERR_UNSUPPORTED;
    lla_plan plan;
    ref_plan(H, d, dtype, k, &plan);
    if ((st = check_workspace(plan, workspace, workspace_bytes)) != LLA_OK) return st;
    if (k->batch == 0) return LLA_OK;
    DecodeArgs a{};
    a.k_pool = k->k_pool;
    a.v_pool = k->v_pool;
    a.block_table = k->block_table;
    a.seq_lens = k->seq_lens;
    a.q = q;
    a.k_self = k_self;
    a.v_self = v_self;
    a.self_stride = self_stride ? self_stride : (int64_t)H * d;
    a.out = out;
    a.ws = static_cast<float *>(workspace);
    a.B = k->batch;
    a.H = H;
    a.G = H;
    a.Dg = d;
    a.T = 1;
    a.t = 0;
    a.P = k->page_size;
    a.max_pages = k->max_pages;
    a.n_pages = k->n_pages;
    a.max_seq_len = k->max_seq_len;
    a.S = plan.splits;
    a.tokens_per_split = plan.tokens_per_split;
    a.mode = 0;
    a.scale_log2 = scale * kLog2e;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf16 = dtype == LLA_BF16;
    if (launch_flat(a, d, bf16, s) != hipSuccess) return LLA_ERR_HIP;
    return launch_combine(a, d, bf16, false, false, s) == hipSuccess ? LLA_OK : LLA_ERR_HIP;
}

lla_status lla_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
    if (!buf || !sink) return LLA_ERR_NULL;
    if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return LLA_ERR_ALIGN;
    if (bytes % 16 != 0) return LLA_ERR_SHAPE;
    if (bytes == 0) return LLA_OK;
    return launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream)) == hipSuccess
               ? LLA_OK
               : LLA_ERR_HIP;
}

const char *lla_status_str(lla_status s) {
    switch (s) {
        case LLA_OK: return "ok";
        case LLA_ERR_NULL: return "null pointer";
        case LLA_ERR_SHAPE: return "invalid shape or size";
        case LLA_ERR_DTYPE: return "invalid dtype";
        case LLA_ERR_ALIGN: return "buffer not 16-byte aligned";
        case LLA_ERR_WORKSPACE: return "workspace missing or too small";
        case LLA_ERR_UNSUPPORTED: return "shape not supported by the built kernels";
        case LLA_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

const char *lla_version(void) { return "0.1.0"; }

}  // extern "C"

namespace {

lla_status fit_check(const lla_codec *c, int32_t r, int64_t n, int *S, size_t *bytes) {
    lla_status st = check_codec(c);
    if (st != LLA_OK) return st;
    if (c->dtype != LLA_BF16) return LLA_ERR_DTYPE;
    const Shape sh = shape_of(c);
    if (r < 1 || r > sh.X) return LLA_ERR_SHAPE;
    if (r > kFitMaxCols - 8 || sh.X % 128 != 0 || sh.X > 8192) return LLA_ERR_UNSUPPORTED;
    if (n < fit_block_cols(r) + 1 || n > (int64_t)1 << 30) return LLA_ERR_SHAPE;
    *bytes = fit_workspace_floats(sh.G, (int)sh.X, r, (long)n, S) * sizeof(float);
    return LLA_OK;
}

}  // namespace

lla_status lla_fit_plan(const lla_codec *c, int32_t r, int64_t n, size_t *workspace_bytes) {
    if (!workspace_bytes) return LLA_ERR_NULL;
    int S;
    return fit_check(c, r, n, &S, workspace_bytes);
}

lla_status lla_fit_svd(const lla_codec *c, int32_t r, const void *x, int64_t n, int32_t iters,
                       void *mu, void *W_down, void *W_up, float *sigma, void *workspace,
                       size_t workspace_bytes, void *stream) {
    int S;
    size_t need;
    lla_status st = fit_check(c, r, n, &S, &need);
    if (st != LLA_OK) return st;
    if (iters < 0 || iters > 10000) return LLA_ERR_SHAPE;
    if (!x || !mu || !W_down || !W_up || !workspace) return LLA_ERR_NULL;
    if (workspace_bytes < need) return LLA_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(workspace)) return LLA_ERR_ALIGN;
    const Shape sh = shape_of(c);
    FitArgs a{};
    a.x = x;
    a.n = (long)n;
    a.T = c->T;
    a.H = c->n_heads;
    a.d = c->d_head;
    a.G = sh.G;
    a.X = (int)sh.X;
    a.r = r;
    a.rb = fit_block_cols(r);
    a.mode = c->mode;
    a.iters = iters;
    a.S = S;
    a.bf16 = 1;
    float *w = static_cast<float *>(workspace);
    a.part = w;
    w += (size_t)S * a.G * a.X * a.X;
    a.colsum = w;
    w += (size_t)S * a.G * a.X;
    a.C = w;
    w += (size_t)a.G * a.X * a.X;
    a.mu32 = w;
    w += (size_t)a.G * a.X;
    a.V = w;
    w += (size_t)a.G * a.X * a.rb;
    a.W = w;
    w += (size_t)a.G * a.X * a.rb;
    a.rot = reinterpret_cast<float4 *>(w);
    w += fit_rotation_floats(a.G, a.rb);
    a.order = reinterpret_cast<int *>(w);
    a.mu_out = mu;
    a.Wd_out = W_down;
    a.Wu_out = W_up;
    a.sigma = sigma;
    return launch_fit(a, static_cast<hipStream_t>(stream)) == hipSuccess ? LLA_OK : LLA_ERR_HIP;
}
