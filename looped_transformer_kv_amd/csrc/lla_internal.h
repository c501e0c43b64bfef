// lla_internal.h -- shared internals of liblla.so: kernel argument blocks, launchers and small
// device helpers for gfx950 (CDNA4, 64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lla.h"

namespace lla {

// Workgroup index -> work item, XCD-aware.  Consecutive workgroup ids are dispatched round-robin
// over the 8 XCDs of the chip, so id % 8 names the XCD.  With the plain order every XCD would
// serve a fixed subset of heads (head h sits at the same offset in every page, so each XCD's
// requests would hit a fixed subset of memory channels).  Transposing gives XCD x the
// contiguous work range [x n/8, (x+1) n/8): whole sequences, all heads.  Identity when n % 8 != 0.
__device__ __forceinline__ int xcd_work_item(int id, int n) {
    return (n & 7) ? id : (id & 7) * (n >> 3) + (id >> 3);
}


// ---------------------------------------------------------------- kernel argument blocks

// One decode call (latent or flat).  Pointers are device pointers; element type is bf16
// (stored as uint16_t) or fp32 according to the kernel instantiation.
struct DecodeArgs {
    const void *k_pool, *v_pool;     // latent: [n_pages][G][P][r]; flat: [n_pages][H][P][d]
    const int32_t *block_table;      // [B][max_pages]
    const int32_t *seq_lens;         // [B]
    const void *W_up_k, *W_up_v;     // [T][G][r][Dg]   (latent only)
    const void *mu_k, *mu_v;         // [G][X]          (latent only)
    const void *q;                   // [B][H][d]
    const void *k_self, *v_self;     // rows at + b*self_stride + h*d, or null
    int64_t self_stride;
    void *out;                       // [B][H][d]
    float *ws;                       // partials [B][H][S][d + 4]: o[d], m, l, -, -
    int B, H, G, Dg, T, t, r_k, r_v, P, max_pages, n_pages, max_seq_len;
    int S, tokens_per_split;
    int mode;                        // 0 per-head, 1 LLA-2D
    float scale_log2;                // softmax scale * log2(e): scores live in the log2 domain
    // rotation after reconstruction (lla_decode_attn_rope only): the first rope_rot head dims
    // rotate, pair m (m < rope_rot / 2) by pos * theta^(-2m / rope_rot); style 0 pairs
    // (m, m + rope_rot / 2), style 1 pairs (2m, 2m + 1); dims from rope_rot on stay put
    float rope_log2_theta;
    int rope_style;
    int rope_rot;
};

// One chunked prefill call (bf16).
struct PrefillArgs {
    const void *k_pool, *v_pool;     // latent pools [n_pages][G][P][r]
    const int32_t *block_table;      // [B][max_pages]
    const int32_t *seq_lens;         // [B]: cached tokens before the chunk
    const void *W_up_k, *W_up_v;     // [T][G][r][Dg]
    const void *mu_k, *mu_v;         // [G][X]
    const void *q;                   // [B][Pn][H][d]
    const void *k_new, *v_new;       // chunk rows at + (b*Pn + i)*new_stride + h*d
    const int32_t *n_new;            // [B]: chunk tokens per sequence (clamped to [0, Pn])
    void *out;                       // [B][Pn][H][d]
    int64_t new_stride;
    int B, H, G, Dg, T, t, r_k, r_v, P, max_pages, n_pages, max_seq_len;
    int Pn, QB;                      // chunk capacity; query blocks per (sequence, head)
    int mode;
    float scale_log2;
};

// One codec fit (bf16): workspace pointers are fp32 regions carved by the host.
constexpr int kFitMaxCols = 168;     // columns of the iterated block (r + 8, r <= 160)
constexpr int kFitSweeps = 12;       // Jacobi sweeps of the Rayleigh-Ritz step
struct FitArgs {
    const void *x;                   // trajectory rows [n][T][H][d]
    long n;
    int T, H, d, G, X, r, rb, mode, iters, S, bf16;
    float *part;                     // [S][G][X][X] partial A^T A (blocks bi <= bj)
    float *colsum;                   // [S][G][X] partial column sums
    float *C;                        // [G][X][X] centred covariance
    float *mu32;                     // [G][X]
    float *V, *W;                    // [G][X][rb] iterate and product
    void *mu_out, *Wd_out, *Wu_out;  // [G][X], [G][X][r], [T][G][r][X/T] in the codec dtype
    float *sigma;                    // optional [G][r]
    float4 *rot;                     // [G][sweeps][rb - 1][rb / 2] Jacobi rotations (c, s, p, q bits)
    int *order;                      // [G][kFitMaxCols] Ritz columns by decreasing eigenvalue
};

// One encode+append call.
struct EncodeArgs {
    const void *x;                   // staging rows [B][T][H][d] (B = rows)
    const void *W_down;              // [G][X][r]
    const void *mu;                  // [G][X]
    void *pool;                      // [n_pages][G][P][r]
    const int32_t *block_table;      // [sequences][max_pages]
    const int32_t *write_pos;        // [sequences]
    const int32_t *n_rows;           // optional [sequences]: live rows of each sequence
    float *c_out;                    // optional [B][G][r]
    int B, H, G, Dg, T, d, r, P, max_pages, n_pages, mode;
    int rps;                         // rows per sequence: row -> (row / rps, row % rps)
};

// Staging row `row` belongs to sequence seq = row / rps as its chunk index i = row % rps and is
// appended at pos = write_pos[seq] + i.  Returns whether the row is live (i < n_rows[seq]).
__device__ __forceinline__ bool encode_row(const EncodeArgs &a, int row, int &seq, int &pos) {
    seq = row / a.rps;
    const int i = row - seq * a.rps;
    pos = a.write_pos[seq] + i;
    return !a.n_rows || i < a.n_rows[seq];
}

// ---------------------------------------------------------------- launchers (host)
// Each returns hipSuccess or the launch error.  Shapes were validated by the caller.
hipError_t launch_decode_bf16(const DecodeArgs &a, bool rope, hipStream_t s);
hipError_t launch_decode_f32(const DecodeArgs &a, hipStream_t s);
// rotary decode, two heads per wave, scores on the matrix core (per-head codecs, even head count,
// r_k = 16, r_v 16 or 32, d 64 or 128); same plan, workspace and partial records as
// launch_decode_bf16(a, true, s)
bool decode_rope_heads_supported(int mode, int H, int d, int r_k, int r_v);
hipError_t launch_decode_rope_heads(const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_absorbed(const DecodeArgs &a, hipStream_t s);
hipError_t launch_flat(const DecodeArgs &a, int d, bool bf16, hipStream_t s);
constexpr int kStreamReadSlots = 512;   // sink entries of lla_stream_read (= its largest grid)
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st);
// self_in_record: the current token's score was computed by the decode kernel and stored in
// split 0's record (slot d + 2, log2 domain) instead of being formed here from q and k_self
hipError_t launch_combine(const DecodeArgs &a, int d, bool bf16, bool has_mu, bool self_in_record,
                          hipStream_t s);
hipError_t launch_encode(const EncodeArgs &k_axis, const EncodeArgs &v_axis, bool bf16,
                         hipStream_t s);
// n layers' encodes (per-layer K and V axis arguments that differ only in their pointers)
hipError_t launch_encode_layers(const EncodeArgs *k_axes, const EncodeArgs *v_axes, int n,
                                bool bf16, hipStream_t s);
bool decode_bf16_supported(int d, int r_k, int r_v);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);
bool prefill_supported(int d, int r_k, int r_v);
hipError_t launch_fit(FitArgs a, hipStream_t s);
size_t fit_workspace_floats(int G, int X, int r, long n, int *S_out);
size_t fit_rotation_floats(int G, int rb);
int fit_block_cols(int r);
int prefill_queries_per_block();

// Absorbed LLA-2D decode (decode_absorbed2d.hip): heads are the 16 columns of its MFMA tiles.
constexpr int kAbs2dHeads = 16;
constexpr int kMaxAbs2dSplits = 1024;
// Its workspace, in floats from the workspace base; every region starts 256-byte aligned.
struct Abs2dLayout {
    size_t qt;      // bf16 [B][2][16][r_k]: q~ (log2-scaled) as hi, lo
    size_t qm;      // [B][16]: <q, mu_t^K>, log2-scaled
    size_t self;    // [B][16]: the current token's own score (-inf without one)
    size_t part;    // [B][S][16][r_v]: per split, sum_j p_j c_v(j) relative to the split max
    size_t stat;    // [B][S][16][2]: split max, split sum of p
    size_t total;
};
__host__ __device__ inline Abs2dLayout abs2d_layout(int B, int S, int r_k, int r_v) {
    auto up = [](size_t n) { return (n + 63) & ~size_t(63); };
    Abs2dLayout L;
    L.qt = 0;
    L.qm = L.qt + up((size_t)B * kAbs2dHeads * r_k);
    L.self = L.qm + up((size_t)B * kAbs2dHeads);
    L.part = L.self + up((size_t)B * kAbs2dHeads);
    L.stat = L.part + up((size_t)B * S * kAbs2dHeads * r_v);
    L.total = L.stat + up((size_t)B * S * kAbs2dHeads * 2);
    return L;
}
bool absorbed2d_supported(int mode, int H, int d, int r_k, int r_v);
// a.S / a.tokens_per_split are the splits per sequence of the absorbed plan
hipError_t launch_decode_absorbed2d(const DecodeArgs &a, hipStream_t s);

constexpr int kPartialPad = 4;   // partial record = d + 4 floats (16-byte aligned records)
constexpr int kMaxChunksPerSplit = 512;   // 32-token chunks one latent-decode workgroup covers

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf2f(uint16_t u) {
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <typename TS> __device__ __forceinline__ float ld_elt(const TS *p);
template <> __device__ __forceinline__ float ld_elt<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float ld_elt<uint16_t>(const uint16_t *p) { return bf2f(*p); }

template <typename TS> __device__ __forceinline__ void st_elt(TS *p, float v);
template <> __device__ __forceinline__ void st_elt<float>(float *p, float v) { *p = v; }
template <> __device__ __forceinline__ void st_elt<uint16_t>(uint16_t *p, float v) { *p = f2bf(v); }

// Butterfly reductions over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// 2^x with 2^(-inf) = 0.
__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane permutations inside 16-lane rows (gfx9 encodings).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8-lane half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within each row

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Max over each 16-lane row, result in every lane of the row.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    v = fmaxf(v, dpp<kDppMirror>(v));
    return v;
}

// Sum over aligned groups of G lanes (G = 8, 16 or 32), result in every lane of the group.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G == 8 || G == 16 || G == 32, "group size");
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    if constexpr (G >= 16) v += dpp<kDppMirror>(v);
    if constexpr (G == 32) v += __shfl_xor(v, 16, 64);
    return v;
}

// x[l] + x[l ^ 32] in every lane (v_permlane32_swap).
__device__ __forceinline__ float add_swap32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace lla
