/*
 * lla.h -- C ABI of liblla.so, the MI355X (gfx950) Looped Latent Attention decode hot path.
 *
 * Method: "Looped Latent Attention: Cross-Loop KV Compression for Looped Transformers"
 * (O'Neill & Reid, arXiv 2607.15456).  Per layer, head and axis (K or V) a token's T loop-step
 * vectors are joined into one vector x; the cache keeps only the rank-r latent
 * c = (x - mu) W_down, loop t reads it back as x_hat_t = c W_up,t + mu_t, and attention is as before
 * (pith.science paper page, "What carries the argument").  Loop-specific K/V are rebuilt only when
 * attention reads them; the default codec is per head, LLA-2D folds all heads of a layer into one
 * latent per axis (abstract).  Compression rho = 2 T d_head / (r_k + r_v) (Eq. 4).
 *
 * Conventions shared by every entry point
 *   - Plain C: every pointer is a raw device pointer unless it says "host".  No torch types.
 *   - Ownership: the caller allocates and owns every buffer; the library allocates nothing and
 *     never frees anything.  Its only global mutable state belongs to lla_decode_attn_noalloc: a
 *     4 MiB device array per GPU and the host-side table of those arrays' addresses.
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 *     call returns without synchronising.
 *   - Errors: arguments are validated on the host before anything is enqueued; on a validation
 *     error the call returns the status and enqueues nothing.  LLA_ERR_HIP reports a failed launch.
 *     No C++ exception crosses the ABI.  Calls on disjoint buffers are thread-safe.
 *   - Loop index t is 0-based (the pages count loops 1..T).
 *   - Shapes.  H = n_heads, d = d_head, T = loops.  Per-head mode: G = H latent groups, D_g = d.
 *     LLA-2D mode: G = 1, D_g = H*d.  X = T*D_g is the stacked length.  Element type is
 *     codec->dtype (bf16 or fp32) for every floating buffer except the optional fp32 encode copies.
 *   - Stacking order of x (a reading: the pages say only "stacked"): per-head x[t*d + i] for head
 *     h; LLA-2D x[(t*H + h)*d + i].  mu_t is block t of mu (length D_g).
 *   - Out-of-range page ids in a block table make the affected outputs NaN (never a fault).
 *     Lengths are clamped to [0, max_seq_len].
 *   - Pool size: the bf16 decode entry points (lla_decode_attn, _absorbed, _rope) need
 *     n_pages * G * page_size < 2^31 pool rows, lla_ref_attn n_pages * H * page_size < 2^31;
 *     larger pools return LLA_ERR_UNSUPPORTED.
 */
#ifndef LLA_H
#define LLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LLA_OK = 0,
    LLA_ERR_NULL = 1,        /* a required pointer is NULL (or only one of k_self / v_self given) */
    LLA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
    LLA_ERR_DTYPE = 3,       /* unknown dtype */
    LLA_ERR_ALIGN = 4,       /* a buffer is not 16-byte aligned */
    LLA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than the size query returned */
    LLA_ERR_UNSUPPORTED = 6, /* valid, but no kernel is built for this shape */
    LLA_ERR_HIP = 7          /* a kernel launch failed */
} lla_status;

typedef enum { LLA_F32 = 0, LLA_BF16 = 1 } lla_dtype;
typedef enum { LLA_PER_HEAD = 0, LLA_2D = 1 } lla_mode;

/* Codec shape (host struct).  Supported: d_head in {64, 128}; 1 <= T <= 64; 1 <= r <= X.
 * bf16 decode: (r_k, r_v) in {(16,16), (16,32), (32,32), (32,64), (64,64), (64,128), (96,160)}.
 * fp32 decode: any r_k, r_v with (r_k + r_v) * d_head <= 16384.  Encode: any r. */
typedef struct {
    int32_t mode;      /* lla_mode */
    int32_t T;         /* loops per token */
    int32_t n_heads;   /* H (query heads = key/value heads) */
    int32_t d_head;    /* d */
    int32_t r_k, r_v;  /* latent ranks of the K and V codecs */
    int32_t dtype;     /* lla_dtype of every floating buffer */
} lla_codec;

/* Codec parameters of one layer (host struct of device pointers, row-major):
 *   W_down_{k,v} [G][X][r]           encode projection (encode only; may be NULL for decode)
 *   W_up_{k,v}   [T][G][r][D_g]      per-loop up-projection W_up,t
 *   mu_{k,v}     [G][X]              centring mean; mu_t = mu[g][t*D_g : (t+1)*D_g]           */
typedef struct {
    const void *W_down_k, *W_down_v;
    const void *W_up_k, *W_up_v;
    const void *mu_k, *mu_v;
} lla_params;

/* Paged cache of one layer (host struct of device pointers).
 *   latent pools: k_pool [n_pages][G][P][r_k], v_pool [n_pages][G][P][r_v]
 *   flat pools (lla_ref_attn):  [n_pages][H][P][d] each, one loop's uncompressed K / V
 *   block_table [batch][max_pages] int32: token j of sequence b is at page block_table[b][j/P],
 *   slot j%P.  seq_lens [batch] int32: cached tokens per sequence (never modified here; the
 *   caller increments it after lla_encode_append).  max_seq_len bounds every seq_lens entry and
 *   must satisfy max_seq_len <= max_pages * P; it sizes the split plan.
 *   page_size P: a multiple of 32 for the bf16 latent decode and for the flat comparator.    */
typedef struct {
    void *k_pool, *v_pool;
    const int32_t *block_table;
    const int32_t *seq_lens;
    int32_t batch, page_size, max_pages, n_pages, max_seq_len;
} lla_cache;

/* How a decode call is split across the GPU (reported for tests and benchmarks). */
typedef struct {
    int32_t kernel;           /* 1 bf16 MFMA latent kernel, 2 fp32 latent kernel, 3 flat kernel,
                                 4 all-heads absorbed LLA-2D kernel */
    int32_t splits;           /* context splits per (sequence, head); kernel 4: per sequence */
    int32_t tokens_per_split;
    int32_t waves_per_block;
    size_t workspace_bytes;   /* what the call needs (0 if none) */
} lla_plan;

/* Eq. 4 (pith.science paper page, "What carries the argument"): rho = 2 T d / (r_k + r_v) per
 * head and layer; for LLA-2D the latent covers all heads, rho = 2 T H d / (r_k + r_v).
 * Returns 0.0 for a NULL or invalid codec. */
double lla_compression_ratio(const lla_codec *codec);

/* Bytes one cached token occupies per layer in the latent cache: G * (r_k + r_v) * sizeof(dtype)
 * (0 for a NULL or invalid codec).  Times the token count it is the whole cache, and against
 * lla_flat_bytes_per_token it is exactly the reduction by rho: the arXiv abstract calls the
 * reduction exact, and the Figure 10 caption (maximum decode batch against context) has the
 * cache shrink by rho at every context length. */
size_t lla_latent_bytes_per_token(const lla_codec *codec);

/* Bytes the uncompressed loop-indexed cache would take per token and layer:
 * 2 * T * H * d * sizeof(dtype) (Figure 1: every loop keeps its own K_t, V_t). */
size_t lla_flat_bytes_per_token(const lla_codec *codec);

/* Split plan and workspace size of lla_decode_attn for this codec and cache (host call).  The
 * plan depends on the codec, batch, n_heads and max_seq_len only; _rope and _absorbed use it too. */
lla_status lla_decode_plan(const lla_codec *codec, const lla_cache *cache, lla_plan *plan);

/* Split plan and workspace size of lla_decode_attn_absorbed.  For a bf16 LLA-2D codec with
 * n_heads <= 16, r_k a multiple of 32 and r_v a multiple of 16 the call runs the all-heads kernel
 * (kernel 4): one workgroup per (sequence, context split) serves every head, so each latent is
 * read once per call; its workspace holds q~ for every (sequence, head) and each split's latent
 * partials, and grows with batch x splits x 16 x r_v floats.  Every other codec gets the plan of
 * lla_decode_plan.  Errors as lla_decode_plan; LLA_ERR_UNSUPPORTED if more than 1024 splits would
 * be needed. */
lla_status lla_decode_absorbed_plan(const lla_codec *codec, const lla_cache *cache,
                                    lla_plan *plan);

/* Workspace bytes lla_decode_attn (and _rope, _absorbed) needs for this codec and cache: the
 * workspace_bytes of lla_decode_plan (0 when the call needs none).  bytes NULL -> LLA_ERR_NULL;
 * otherwise the errors of lla_decode_plan, with *bytes untouched. */
lla_status lla_decode_workspace_size(const lla_codec *codec, const lla_cache *cache, size_t *bytes);

/*
 * Decode attention of loop t for every sequence and head of one layer, reading the latent cache
 * (arXiv abstract: K/V are reconstructed only when attention reads them; pith.science paper
 * page, "What carries the argument": x_hat_t = c W_up,t + mu_t, attention unchanged).
 * For each sequence b and head h:
 *   s_j  = scale * <q[b][h], K_hat_t(j)[h]>   for every cached token j < seq_lens[b]
 *   plus, when k_self/v_self are given, the current token's own loop-t key/value (a reading:
 *   the token attends to itself, as in a causal decoder);
 *   out[b][h] = sum_j softmax(s)_j V_hat_t(j)[h].
 * An empty context without a self term gives out = 0.
 *   q, out           [B][H][d]   (dtype; for bf16, q and W_up_{k,v} must be 16-byte aligned)
 *   k_self, v_self   rows at k_self + b*self_stride + h*d (dtype); both NULL or both set;
 *                    self_stride in elements, 0 means H*d
 *   workspace        device, >= plan.workspace_bytes (may be NULL if that is 0)
 * Reads W_up_{k,v} and mu_{k,v} of `params` only.
 */
lla_status lla_decode_attn(const lla_codec *codec, const lla_params *params,
                           const lla_cache *cache, int32_t t, const void *q, const void *k_self,
                           const void *v_self, int64_t self_stride, float scale, void *out,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * lla_decode_attn for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation and arguments,
 * minus the workspace.  Context-split partials go to a file-scope device array of the library
 * (4 MiB; each GPU the library runs on holds its own copy until the process ends), found with
 * hipGetSymbolAddress on the first call on each device; no call allocates or frees anything.
 * A plan whose workspace_bytes (lla_decode_plan) exceed 4 MiB returns LLA_ERR_WORKSPACE and
 * enqueues nothing; LLA_ERR_HIP if the device or the array's address cannot be obtained.  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU (concurrent streams,
 * threads) race and must be serialised by the caller.  Nothing in the array needs clearing:
 * every partial a call reads was written earlier in the same call.
 */
lla_status lla_decode_attn_noalloc(const lla_codec *codec, const lla_params *params,
                                   const lla_cache *cache, int32_t t, const void *q,
                                   const void *k_self, const void *v_self, int64_t self_stride,
                                   float scale, void *out, void *stream);

/* Rotary position embedding applied after reconstruction (see lla_decode_attn_rope).  The first
 * rot_dims head dims rotate: pair m (m < rot_dims/2) turns by pos * theta^(-2m/rot_dims); the
 * dims from rot_dims on are left as they are (rot_dims = d_head rotates the whole head,
 * rot_dims = 0 none). */
typedef struct {
    float theta;       /* base; > 1 */
    int32_t rot_dims;  /* rotated head dims: even, 0 <= rot_dims <= d_head */
    int32_t style;     /* 0: pairs (m, m + rot_dims/2) (half split); 1: pairs (2m, 2m + 1) */
} lla_rope;

/*
 * Decode attention with the rotation applied after reconstruction (the "full-RoPE" read path the
 * pages' free-parameter ledger describes: a token keeps one position at every recurrence step,
 * so each reconstructed pre-rotation key K_hat_t(j) = c_k(j) W_up,t^K + mu_t^K is rotated to its
 * position j; the rotation is RoFormer's, which the pages cite).  The current token's own key
 * k_self is rotated to its position seq_lens[b]; q is taken as given (the caller rotates it to
 * that same position); values are not rotated.  Otherwise as lla_decode_attn (same plan and
 * workspace).  The ledger fixes neither the rotated width nor the pairing, so rot_dims and style
 * are arguments.  bf16 codecs only (LLA_ERR_DTYPE); rope NULL -> LLA_ERR_NULL; theta <= 1, a
 * style other than 0/1, or rot_dims odd, negative or above d_head -> LLA_ERR_SHAPE.
 * Per-head codecs with r_k = 16, r_v 16 or 32 and an even head count run two heads per wave: the
 * rotated scores come from the per-position cosines and sines contracted with each head's pair
 * coefficients on the matrix core (bf16 operands, fp32 accumulation; each token's query over the
 * ranks rounded to bf16), and values are summed in latent space (bf16 weights, fp32 sums) and
 * expanded through W_up,t^V once, which equals the reconstruct-then-rotate attention up to
 * rounding.  Other codecs rotate in the same pair space one head per workgroup.
 */
lla_status lla_decode_attn_rope(const lla_codec *codec, const lla_params *params,
                                const lla_cache *cache, int32_t t, const lla_rope *rope,
                                const void *q, const void *k_self, const void *v_self,
                                int64_t self_stride, float scale, void *out, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Absorbed-attention decode (the form the editorial letter on the pith.science paper page for
 * "Looped Latent Attention" discusses): the same result as lla_decode_attn up to rounding, computed
 * in the latent space.  q~ = W_up,t^K q once per sequence and head; s_j = scale (<q~, c_k(j)> +
 * <q, mu_t^K>); c~ = sum_j softmax(s)_j c_v(j); out = c~ W_up,t^V + mu_t^V (plus the self term).
 * It is exact only while nothing acts between expansion and attention (no rotation); the per-token
 * work is r_k + r_v multiply-adds per head instead of the d x (r_k + r_v) of the expansion.
 * Arguments and layouts are those of lla_decode_attn; the plan and the workspace size are
 * lla_decode_absorbed_plan's (the same as lla_decode_plan's except for LLA-2D codecs the
 * all-heads kernel takes).  bf16 codecs only (LLA_ERR_DTYPE otherwise), with the same supported
 * (d_head, r_k, r_v).  The all-heads kernel enqueues three kernels (q~; the latent stream; the
 * merge of the splits with the expansion c~ W_up,t^V) and needs q 16-byte aligned.
 */
lla_status lla_decode_attn_absorbed(const lla_codec *codec, const lla_params *params,
                                    const lla_cache *cache, int32_t t, const void *q,
                                    const void *k_self, const void *v_self, int64_t self_stride,
                                    float scale, void *out, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * Encode and append (pith.science paper page, "What carries the argument": the loop-step vectors
 * joined into one, mean removed, projected: c = (x - mu) W_down).  For every sequence b, group g
 * and axis:
 *   c = (stack_g(x[b]) - mu[g]) W_down[g],  accumulated in fp32,
 *   written (rounded to the pool dtype, bf16 round-to-nearest-even) to the pool slot of logical
 *   position write_pos[b] (page block_table[b][pos/P], slot pos%P).
 *   x_k, x_v        staging [B][T][H][d] (dtype, 16-byte aligned; mu_k / mu_v too): the
 *                   token's K / V at every loop
 *   write_pos       device int32 [B]; positions >= max_pages*P or < 0 are skipped
 *   c_k_out/c_v_out optional device fp32 [B][G][r] copies of c before rounding (NULL = none)
 * Reads W_down_{k,v} and mu_{k,v} of `params`.  seq_lens is not read or modified.
 */
lla_status lla_encode_append(const lla_codec *codec, const lla_params *params,
                             const lla_cache *cache, const void *x_k, const void *x_v,
                             const int32_t *write_pos, float *c_k_out, float *c_v_out,
                             void *stream);

/*
 * Bulk encode and append of a chunk of new tokens (a prefill chunk), after its last loop: the same
 * operation as lla_encode_append (pith.science paper page, "What carries the argument":
 * c = (x - mu) W_down) over `chunk` rows per sequence.  Row i of sequence b (i < n_new[b]) is
 * encoded and written to the pool slot of logical position write_pos[b] + i.
 *   x_k, x_v        staging [B][chunk][T][H][d] (dtype, 16-byte aligned; mu_k / mu_v too)
 *   n_new           device int32 [B]: live rows per sequence (rows i >= n_new[b] are ignored)
 *   write_pos       device int32 [B]: position of row 0; positions outside the block table
 *                   (< 0 or >= max_pages*P) are skipped
 *   c_k_out/c_v_out optional device fp32 [B][chunk][G][r] copies of c before rounding, written
 *                   for live rows only (NULL = none)
 * Precision (bf16 codecs): fp32 accumulation of exact bf16 products; at 1024 rows or more with
 * both ranks multiples of 32 and one of them 64 or more, x - mu is formed in fp32 and rounded once
 * to bf16 before the product (relative 2^-9 per element, the class of the output's rounding).
 * chunk = 0 (or batch 0) enqueues nothing.  chunk < 0 or batch*chunk > 2^30 -> LLA_ERR_SHAPE;
 * n_new NULL -> LLA_ERR_NULL; otherwise validated like lla_encode_append.
 */
lla_status lla_encode_chunk(const lla_codec *codec, const lla_params *params,
                            const lla_cache *cache, int32_t chunk, const int32_t *n_new,
                            const void *x_k, const void *x_v, const int32_t *write_pos,
                            float *c_k_out, float *c_v_out, void *stream);

/*
 * Encode and append of the current token for several layers in one call: for each layer i,
 * exactly lla_encode_append(codec, &params[i], &caches[i], x_k[i], x_v[i], write_pos, NULL,
 * NULL, stream) (pith.science paper page for "Looped Latent Attention", "What carries the
 * argument": the per-layer encode on write), with one launch for up to 32 layers on the
 * matrix-core path.  After a decode step every layer's loop trajectories exist, so an engine
 * appends all layers at once.
 *   params, caches  host arrays of n_layers; every cache has the same batch, page_size,
 *                   max_pages and n_pages (else LLA_ERR_SHAPE); each has its own pools and
 *                   block table
 *   x_k, x_v        host arrays of n_layers device pointers, each as in lla_encode_append
 *   write_pos       device int32 [batch], shared by the layers
 * n_layers < 0 -> LLA_ERR_SHAPE; n_layers = 0 enqueues nothing.  Every layer is validated as in
 * lla_encode_append before anything is enqueued.  No fp32 copies of the latents.
 */
lla_status lla_encode_append_layers(const lla_codec *codec, int32_t n_layers,
                                    const lla_params *params, const lla_cache *caches,
                                    const void *const *x_k, const void *const *x_v,
                                    const int32_t *write_pos, void *stream);

/*
 * Chunked prefill attention for loop t.  The pages do not describe prefill; this is the decode
 * rule above applied to a chunk of new tokens at once: new token i of sequence b (i < n_new[b],
 * logical position seq_lens[b] + i) attends to every cached token j < seq_lens[b], reconstructed
 * through the codec as in lla_decode_attn, and causally to the chunk's own loop-t keys/values
 * i' <= i, which are taken as given (they are encoded with lla_encode_chunk after the last loop).
 *   s_j = scale <q[b][i][h], K_hat_t(j)[h]> (cached) or scale <q[b][i][h], k_new[b][i'][h]>;
 *   out[b][i][h] = sum softmax(s) V.
 *   q, out          [B][chunk][H][d] bf16, 16-byte aligned
 *   k_new, v_new    chunk rows: row (b, i) at + (b*chunk + i)*new_stride, head h at + h*d (bf16,
 *                   16-byte aligned); new_stride in elements, 0 means H*d, else a multiple of 8
 *                   and >= H*d (T*H*d reads loop t of a [B][chunk][T][H][d] staging buffer
 *                   offset by t*H*d)
 *   n_new           device int32 [B], clamped to [0, chunk]
 * Rows i >= n_new[b] of out are not written.  Ranks up to 32 run as two kernels whose partial
 * state passes through the live rows of out; the wider pairs run as one kernel.  In both cases out
 * must not overlap any input.  No workspace.  bf16 codecs only (LLA_ERR_DTYPE); d_head 64 or 128
 * with (r_k, r_v) in {(16,16), (16,32), (32,32), (32,64), (64,64), (64,128), (96,160)} and
 * n_pages * G * page_size < 2^31, else LLA_ERR_UNSUPPORTED; page_size a multiple of 32,
 * 0 <= t < T and chunk * new_stride < 2^31, else LLA_ERR_SHAPE.  chunk = 0 enqueues nothing.
 */
lla_status lla_prefill_attn(const lla_codec *codec, const lla_params *params,
                            const lla_cache *cache, int32_t t, int32_t chunk,
                            const int32_t *n_new, const void *q, const void *k_new,
                            const void *v_new, int64_t new_stride, float scale, void *out,
                            void *stream);

/*
 * Codec fit by truncated SVD (pith.science paper page for "Looped Latent Attention", "What
 * carries the argument": the codec's starting point comes from an SVD of activation data, W_down
 * spanning the leading right singular subspace).  For every group g, with a_j the stacked
 * vector of row j (the encode's stacking order) and n rows:
 *   mu[g] = mean_j a_j;   W_down[g] = the r leading right singular vectors of [a_j - mu], as
 *   columns in decreasing singular value, each column's entry of largest magnitude positive;
 *   W_up[t][g] = the transpose of W_down[g]'s rows t*D_g .. (t+1)*D_g - 1;
 *   sigma[g] (optional, fp32 [G][r]) = the r leading singular values.
 * Computed on the GPU as the centred covariance A^T A - n mu^T mu (matrix cores, fp32
 * accumulation of the exact bf16 inputs), `iters` steps of subspace iteration with r + 8 columns
 * (CholeskyQR2), then a Rayleigh-Ritz step (Jacobi rotations, applied to the basis as they are
 * logged); the result converges to the exact one as (lambda_{r+9} / lambda_r)^iters.  Outputs are
 * rounded once to bf16.
 *   x          rows [n][T][H][d] bf16 (e.g. a layer's staged K or V trajectories), 16-byte aligned
 *   mu         [G][X], W_down [G][X][r], W_up [T][G][r][D_g], bf16, caller-owned
 *   workspace  device, >= lla_fit_plan bytes, 16-byte aligned
 * bf16 codecs only (LLA_ERR_DTYPE); r in [1, 160] and X = T*D_g a multiple of 128 (at most 8192)
 * else LLA_ERR_UNSUPPORTED (r > X: LLA_ERR_SHAPE); n >= r + 9 (+1 if r is odd), <= 2^30;
 * 0 <= iters <= 10000.
 */
lla_status lla_fit_plan(const lla_codec *codec, int32_t r, int64_t n, size_t *workspace_bytes);
lla_status lla_fit_svd(const lla_codec *codec, int32_t r, const void *x, int64_t n,
                       int32_t iters, void *mu, void *W_down, void *W_up, float *sigma,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Split plan and workspace size of lla_ref_attn. */
lla_status lla_ref_plan(int32_t n_heads, int32_t d_head, int32_t dtype, const lla_cache *flat,
                        lla_plan *plan);

/*
 * Flat comparator: the same decode attention over an uncompressed loop-t cache (Figure 1 caption:
 * each recurrent step t contributes its own (K_t, V_t)).  `flat` describes pools
 * [n_pages][H][P][d] of loop t's keys and values; q, k_self, v_self, self_stride, scale, out and
 * the workspace are as in lla_decode_attn.  d_head in {64, 128}.
 */
lla_status lla_ref_attn(int32_t n_heads, int32_t d_head, int32_t dtype, const lla_cache *flat,
                        const void *q, const void *k_self, const void *v_self,
                        int64_t self_stride, float scale, void *out, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * Measurement helper (not an LLA operation): streams `bytes` of `buf` once from device memory.
 * Its time gives the achievable HBM read rate, the practical ceiling for the latent stream.
 * Workgroup w (at most 512 of them) stores the XOR of the 32-bit words it read in sink[w]; the
 * XOR of sink[0 .. 511] is the XOR of every word of the buffer if the caller zeroed sink first
 * (entries of workgroups that do not exist are left untouched).
 * buf: device, 16-byte aligned, bytes a multiple of 16 (0 enqueues nothing);
 * sink: device uint32 [512].
 */
lla_status lla_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* Static description of a status code. */
const char *lla_status_str(lla_status status);

/* Library version, "major.minor.patch". */
const char *lla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LLA_H */
