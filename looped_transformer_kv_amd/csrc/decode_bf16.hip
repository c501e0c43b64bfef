// decode_bf16.hip -- fused latent decode attention, bf16 storage, fp32 accumulation, gfx950 MFMA.
//
// Computes, for loop t, sequence b, head h (pith.science paper page for "Looped Latent Attention",
// section "What carries the argument": x_hat_t = c W_up,t + mu_t, attention unchanged; abstract:
// K/V rebuilt only when attention reads them):
//   K_hat(j) = c_k(j) W_up,t^K + mu_t^K,  s_j = scale <q, K_hat(j)>
//   V_hat(j) = c_v(j) W_up,t^V + mu_t^V,  out = sum_j softmax(s)_j V_hat(j)
// Both reconstructions are dense contractions over the latent rank, run per cached token on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation; the full K_hat / V_hat never leave registers.
// mu_t enters exactly, as constants: <q, mu_t^K> is added to every cached score and
// (sum_j p_j) mu_t^V to the output.
//
// Work decomposition: one workgroup per (sequence b, head h, context split s); its waves take
// 32-token chunks round-robin, each wave keeping the next chunks' latents in flight.  Latents go
// straight from HBM into MFMA operand registers (16 bytes per lane per 16 ranks; a chunk is one
// contiguous run per axis).  The split's page table and W_up,t are staged in LDS once.
//
// Small ranks (r_k, r_v <= 32): the attention weights ride on the expansion operands.
//   Scores: A = W_up,t^K transposed (d x r_k) with lane (l32, .)'s column i = 32M + l32 scaled by
//           q_i * scale * log2(e) and rounded to bf16, B = chunk latents (r_k x 32 tokens).  The
//           tiles of all 32-row groups of the head dim accumulate into one 32x32 tile whose row r
//           holds sum over M of q_i K_hat_i(j), i = 32M + r: 16 in-lane adds and one exchange
//           between lanes l and l^32 give token l32's score.
//   Values: A = chunk latents (32 tokens x r_v) with token j's row scaled by its softmax weight
//           p_j and rounded to bf16, B = W_up,t^V (r_v x d).  The p-weighted V_hat tiles add into
//           four persistent 32x32 accumulators across chunks; their 32 token rows are summed once
//           at the end.
//   Every cached token still gets its full d x r expansion on the matrix cores; the query and
//   the weights enter as operand scalings.  Rounding q_i W and p_j c_j to bf16 is the same
//   precision class as a bf16 K cache and bf16 softmax weights in a flat attention kernel.
// Larger ranks: explicit K_hat / V_hat tiles per chunk; scores are in-lane dot products with q
//   held in fp32, and p_j V_hat(j) accumulates into o with fp32 FMAs (p reaches the V tile's row
//   layout through 128 B of LDS).
// Online softmax in the log2 domain; the waves of a workgroup merge through LDS.  A single-split
// plan finishes the output here (self term and mu_t^V included); otherwise one (o, m, l) partial
// per split goes to combine.hip.
#include "lla_internal.h"

namespace lla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32x32x16(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// two fp32 -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// 8 bf16 times s, rounded back to bf16
__device__ __forceinline__ uint4 scale_bf16x8(uint4 w, float s) {
    const uint32_t in[4] = {w.x, w.y, w.z, w.w};
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = pk_bf16(__uint_as_float(in[i] << 16) * s, __uint_as_float(in[i] & 0xffff0000u) * s);
    return make_uint4(r[0], r[1], r[2], r[3]);
}

// Latent registers of one 32-token chunk (this lane's 16-byte slices).
template <int KK, int KV>
struct Chunk {
    uint4 k[KK], v[KV];
};

template <int D, int RK, int RV, bool ROPE>
struct Shape {
    static constexpr int MT = D / 32;                  // 32-column tiles over the head dim
    static constexpr int KK = RK / 16, KV = RV / 16;   // MFMA k-steps over the latent ranks
    // small ranks: the attention weights ride on the expansion operands (query on W_up^K, softmax
    // weight on the value latents) and V_hat accumulates in the matrix-core accumulators across
    // chunks; W_up operands live in registers.  Larger ranks: W_up operands from LDS, explicit
    // per-chunk V_hat tiles, query and output in VALU registers.
    static constexpr bool FUSED = !ROPE && KK <= 2 && KV <= 2;
    // larger ranks without rotation: chunks go through the explicit path two at a time, so each
    // W_up operand read from LDS feeds two MFMAs (one per chunk) and the LDS operand traffic per
    // token halves (one operand per MFMA would keep LDS at its peak rate)
    static constexpr bool PAIR = !FUSED && !ROPE && KK + KV > 4;
    static constexpr int WAVES = 4;
    static constexpr int DEPTH =
        KK + KV <= 3 ? 3 : (KK + KV <= 4 || PAIR ? 2 : 1);   // chunks in flight per wave
};

template <int D, int RK, int RV, bool ROPE>
constexpr int kThreads = 64 * Shape<D, RK, RV, ROPE>::WAVES;

// ROPE: the rotation follows reconstruction (lla_decode_attn_rope).  Every K_hat tile (mu_t
// included, through one more MFMA of the mu row against a row of ones) is rotated in registers
// to its token's position before the dot with q: with the rotation over all d head dims, every
// pair of a tile element is held by the same lane (half split: the same register of the tile
// d/2 ahead; interleaved: the neighbouring register).  The explicit path always runs.
template <int D, int RK, int RV, bool ROPE>
__global__ __attribute__((amdgpu_flat_work_group_size(1, kThreads<D, RK, RV, ROPE>)))
void decode_bf16_kernel(DecodeArgs a) {
    using SH = Shape<D, RK, RV, ROPE>;
    constexpr int MT = SH::MT, KK = SH::KK, KV = SH::KV, WAVES = SH::WAVES;
    constexpr bool FUSED = SH::FUSED, PAIR = SH::PAIR;
    constexpr int RKP = RK + 8, RVP = RV + 8;   // padded LDS rows (keeps 16-byte alignment)

    __shared__ __align__(16) uint16_t sWk[D * RKP];   // W_up,t^K transposed: [i][k]
    __shared__ __align__(16) uint16_t sWv[D * RVP];   // W_up,t^V transposed: [i][k]
    __shared__ __align__(16) float sP[WAVES][64];   // p of one chunk (two in the paired path)
    __shared__ __align__(16) float sQ[PAIR ? D : 4];   // paired path: q, log2-scaled
    __shared__ __align__(16) float sO[WAVES][D];
    __shared__ float sM[WAVES], sL[WAVES];
    __shared__ int sSlot[kMaxChunksPerSplit];         // chunk -> first token row in the pool
    // ROPE: A operands of the pair-space score MFMAs (tile T < PT: cosine part of pairs
    // 32T .. 32T + 31; PT + T: sine part), per k-step and bf16 term (hi, then lo for ranks up to
    // 32, where the matrix cores have room for the second term)
    constexpr int PT = ROPE ? MT / 2 : 1;
    constexpr int TERMS = KK <= 2 ? 2 : 1;
    __shared__ __align__(16) uint4 sAq[ROPE ? 2 * PT * KK * TERMS : 1][64];

    const int S = a.S;
    const int id = xcd_work_item(blockIdx.x, gridDim.x);
    const int s = id % S;
    const int h = (id / S) % a.H;
    const int b = id / (S * a.H);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h2 = lane >> 5;
    const int g = a.mode ? 0 : h;
    const int col0 = a.mode ? h * D : 0;

    // ---- this split's token range and its chunk -> pool row table
    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
    const int j_begin = s * a.tokens_per_split;
    const int j_end = min(j_begin + a.tokens_per_split, len);
    const int nchunks = j_end > j_begin ? (j_end - j_begin + 31) >> 5 : 0;
    const int32_t *bt = a.block_table + (size_t)b * a.max_pages;
    // chunk c -> first token row of its page slot; negative marks an invalid page id.  The
    // table read is clamped, so any c >= 0 reads in bounds (callers use c < nchunks).
    auto slot_of = [&](int c) {
        const int j = j_begin + 32 * c;
        const int page = bt[min(j / a.P, a.max_pages - 1)];
        const bool bad = (unsigned)page >= (unsigned)a.n_pages;
        const int row = ((bad ? 0 : page) * a.G + g) * a.P + j % a.P;
        return bad ? -row - 1 : row;
    };

    const uint16_t *kpool = static_cast<const uint16_t *>(a.k_pool);
    const uint16_t *vpool = static_cast<const uint16_t *>(a.v_pool);
    const int lane_k = l32 * RK + 8 * h2, lane_v = l32 * RV + 8 * h2;

    // chunk c at pool row `slot` (as from slot_of): token row (slot + l32), latent entries
    // 16ks + 8h2 .. +7.  Lanes past the sequence end read the chunk's last valid token instead
    // (its weight is zero), so within a chunk no slot beyond the sequence is read; a chunk past
    // the end (only ever prefetched, never used) reads its page slot's first row.
    auto load_slot = [&](int c, int slot, Chunk<KK, KV> &x) {
        const int row = __builtin_amdgcn_readfirstlane(slot < 0 ? -slot - 1 : slot);
        const int valid = j_end - (j_begin + 32 * c);
        const int tok = min(l32, max(valid - 1, 0));
        const uint16_t *kb = kpool + (size_t)row * RK;
        const uint16_t *vb = vpool + (size_t)row * RV;
        const int dk = lane_k + (tok - l32) * RK, dv = lane_v + (tok - l32) * RV;
#pragma unroll
        for (int ks = 0; ks < KK; ++ks)
            x.k[ks] = *reinterpret_cast<const uint4 *>(kb + dk + 16 * ks);
#pragma unroll
        for (int ks = 0; ks < KV; ++ks)
            x.v[ks] = *reinterpret_cast<const uint4 *>(vb + dv + 16 * ks);
    };
    auto load = [&](int c, Chunk<KK, KV> &x) { load_slot(c, sSlot[c], x); };
    // the key or the value half of load_slot, for refilling a buffer half as soon as it is consumed
    auto load_half = [&](int c, Chunk<KK, KV> &x, bool keys) {
        const int slot = sSlot[c];
        const int row = __builtin_amdgcn_readfirstlane(slot < 0 ? -slot - 1 : slot);
        const int valid = j_end - (j_begin + 32 * c);
        const int tok = min(l32, max(valid - 1, 0));
        if (keys) {
            const uint16_t *kb = kpool + (size_t)row * RK + lane_k + (tok - l32) * RK;
#pragma unroll
            for (int ks = 0; ks < KK; ++ks) x.k[ks] = *reinterpret_cast<const uint4 *>(kb + 16 * ks);
        } else {
            const uint16_t *vb = vpool + (size_t)row * RV + lane_v + (tok - l32) * RV;
#pragma unroll
            for (int ks = 0; ks < KV; ++ks) x.v[ks] = *reinterpret_cast<const uint4 *>(vb + 16 * ks);
        }
    };

    // ---- prologue.  A wave's vector loads complete in order, so the order of issue matters:
    // (1) page-table entries of this wave's first chunks, (2) every small set-up operand, raw
    // into registers, (3) the first latent chunks, and only then (4) the reductions and LDS
    // stores that wait on (2).  HBM streaming thus starts one page-table round trip after entry.
    constexpr int DEPTH = SH::DEPTH;
    constexpr int NT = 64 * WAVES;
    // Every load here is unconditional, at a clamped in-bounds index, so no branch separates
    // them (a load under a branch costs a full wait at the join).
    const int c_last = max(nchunks - 1, 0);
    int first[DEPTH];   // not clamped to the sequence: these reads need not wait for its length
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) first[i] = slot_of(wave + i * WAVES);

    // (2) W_up,t of this head's D columns.  Fused path: each lane loads its own MFMA operands
    // (rows 16ks + 8h2 + e, e = 0..7, of column 32 tile + l32) straight from memory, so no
    // workgroup-wide staging or barrier is needed.  Explicit path: 16-byte row pieces for the
    // transposed LDS copy (piece e is row e / (D/8), columns 8 (e % (D/8)) .. +7).
    const uint16_t *Wk = static_cast<const uint16_t *>(a.W_up_k) +
                         ((size_t)a.t * a.G + g) * RK * a.Dg + col0;
    const uint16_t *Wv = static_cast<const uint16_t *>(a.W_up_v) +
                         ((size_t)a.t * a.G + g) * RV * a.Dg + col0;
    uint16_t wkraw[FUSED ? MT * KK : 1][8], wvraw[FUSED ? MT * KV : 1][8];
    if constexpr (FUSED) {
#pragma unroll
        for (int M = 0; M < MT; ++M)
#pragma unroll
            for (int ks = 0; ks < KK; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    wkraw[M * KK + ks][e] = Wk[(size_t)(16 * ks + 8 * h2 + e) * a.Dg + 32 * M + l32];
#pragma unroll
        for (int N = 0; N < MT; ++N)
#pragma unroll
            for (int ks = 0; ks < KV; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    wvraw[N * KV + ks][e] = Wv[(size_t)(16 * ks + 8 * h2 + e) * a.Dg + 32 * N + l32];
    }
    constexpr int PK = RK * D / 8, PV = RV * D / 8;                 // pieces per matrix
    constexpr int UK = FUSED ? 1 : (PK + NT - 1) / NT;               // pieces per thread
    constexpr int UV = FUSED ? 1 : (PV + NT - 1) / NT;
    uint4 wpk[UK], wpv[UV];
    if constexpr (!FUSED) {
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int e = min(tid + u * NT, PK - 1);
            wpk[u] = *reinterpret_cast<const uint4 *>(Wk + (size_t)(e / (D / 8)) * a.Dg +
                                                      8 * (e % (D / 8)));
        }
#pragma unroll
        for (int u = 0; u < UV; ++u) {
            const int e = min(tid + u * NT, PV - 1);
            wpv[u] = *reinterpret_cast<const uint4 *>(Wv + (size_t)(e / (D / 8)) * a.Dg +
                                                      8 * (e % (D / 8)));
        }
    }
    // page table.  Fused path: this wave's own chunks c = wave + WAVES (lane + 64 u) only, as
    // only this wave reads them; explicit path: the whole split, block-wide.
    constexpr int US = FUSED ? (kMaxChunksPerSplit / WAVES + 63) / 64
                             : (kMaxChunksPerSplit + NT - 1) / NT;   // entries per thread
    int slot_reg[US];
#pragma unroll
    for (int u = 0; u < US; ++u)
        slot_reg[u] = slot_of(min(FUSED ? wave + WAVES * (lane + 64 * u) : tid + u * NT, c_last));
    // query, mu_t^K, and the current token's own loop-t key / value (single-split plans finish
    // the output here): element i = lane + 64 u of the head's d
    constexpr int UD = D / 64;
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) + ((size_t)b * a.H + h) * D;
    const uint16_t *muk = static_cast<const uint16_t *>(a.mu_k) +
                          (size_t)g * a.T * a.Dg + (size_t)a.t * a.Dg + col0;
    const bool has_self = a.k_self != nullptr;
    const bool self_here = S == 1 && has_self;
    const bool self_score = has_self && (S == 1 || ROPE);   // ROPE: stored for the combine
    const uint16_t *muvp = static_cast<const uint16_t *>(a.mu_v) +
                           (size_t)g * a.T * a.Dg + (size_t)a.t * a.Dg + col0;
    // without a self term these read q / mu_v instead and the values are dropped
    const uint16_t *ksp = self_score ? static_cast<const uint16_t *>(a.k_self) +
                                           (size_t)b * a.self_stride + (size_t)h * D
                                     : qp;
    const uint16_t *vsp = self_here ? static_cast<const uint16_t *>(a.v_self) +
                                          (size_t)b * a.self_stride + (size_t)h * D
                                    : muvp;
    // ROPE: the first R = rope_rot head dims rotate.  The rotation partner of element i < R
    // (half split: i +- R/2, interleaved: i ^ 1); elements from R on have none
    const int R = ROPE ? a.rope_rot : 0;
    auto partner = [&](int i) {
        if (i >= R) return i;
        return a.rope_style ? (i ^ 1) : (i < R / 2 ? i + R / 2 : i - R / 2);
    };
    uint16_t qv[UD], mkv[UD], ksv[UD], kpv[ROPE ? UD : 1];
#pragma unroll
    for (int u = 0; u < UD; ++u) {
        const int i = lane + 64 * u;
        qv[u] = qp[i];
        mkv[u] = muk[i];
        ksv[u] = ksp[i];
        if constexpr (ROPE) kpv[u] = ksp[partner(i)];
    }
    // element tid of the output (threads tid < D use them)
    const uint16_t vs_raw = vsp[tid % D], muv_raw = muvp[tid % D];
    // fused path: q_i for this lane's columns i = 32M + l32; explicit path: q rows
    // 32M + 8bb + 4h2 + 0..3 of the K tile
    uint16_t qcol[FUSED ? MT : 1];
    uint2 qrow[(FUSED || ROPE) ? 1 : MT][4];
#pragma unroll
    for (int M = 0; M < MT; ++M) {
        if constexpr (FUSED) {
            qcol[M] = qp[32 * M + l32];
        } else if constexpr (!ROPE) {
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
                qrow[M][bb] = *reinterpret_cast<const uint2 *>(qp + 32 * M + 8 * bb + 4 * h2);
        }
    }

    // (3) the first latent chunks of this wave (paired path: the first one; the second follows
    // once the W_up pieces are in LDS, so the two never hold registers at the same time)
    Chunk<KK, KV> buf[DEPTH];
#pragma unroll
    for (int i = 0; i < (PAIR ? 1 : DEPTH); ++i) load_slot(wave + i * WAVES, first[i], buf[i]);

    // (4) page table (and, explicit path, W_up,t transposed: [column][rank]) into LDS;
    // <q, mu_t^K>, <q, k_self>
#pragma unroll
    for (int u = 0; u < US; ++u) {
        const int c = FUSED ? wave + WAVES * (lane + 64 * u) : tid + u * NT;
        if (c < nchunks) sSlot[c] = slot_reg[u];
    }
#pragma unroll
    for (int u = 0; u < (FUSED ? 0 : UK); ++u) {
        const int e = tid + u * NT;
        if (e < PK) {
            const int k = e / (D / 8), i0 = 8 * (e % (D / 8));
            const uint32_t w[4] = {wpk[u].x, wpk[u].y, wpk[u].z, wpk[u].w};
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                sWk[(i0 + 2 * x) * RKP + k] = (uint16_t)(w[x] & 0xffffu);
                sWk[(i0 + 2 * x + 1) * RKP + k] = (uint16_t)(w[x] >> 16);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < (FUSED ? 0 : UV); ++u) {
        const int e = tid + u * NT;
        if (e < PV) {
            const int k = e / (D / 8), i0 = 8 * (e % (D / 8));
            const uint32_t w[4] = {wpv[u].x, wpv[u].y, wpv[u].z, wpv[u].w};
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                sWv[(i0 + 2 * x) * RVP + k] = (uint16_t)(w[x] & 0xffffu);
                sWv[(i0 + 2 * x + 1) * RVP + k] = (uint16_t)(w[x] >> 16);
            }
        }
    }
    if constexpr (PAIR) load_slot(wave + WAVES, first[1], buf[1]);
    // ROPE: revolutions per position of pair m, theta^(-2m/d) / (2 pi); the angle pos * f is
    // reduced to [0, 1) revolutions before the hardware sine / cosine
    // (pairs m >= R/2 stand for two unrotated dims: frequency 0)
    auto rope_rev = [&](int m) {
        return m < R / 2
                   ? exp2_(-2.0f * (float)m / (float)R * a.rope_log2_theta) * 0.15915494309189535f
                   : 0.f;
    };
    float qm, s_self = -INFINITY;   // log2-scaled
    {
        float am = 0.f, as = 0.f;
#pragma unroll
        for (int u = 0; u < UD; ++u) {
            am += bf2f(qv[u]) * bf2f(mkv[u]);
            float kk = bf2f(ksv[u]);
            if constexpr (ROPE) {
                // the current token's key turns to its position, seq_lens[b] (its first R dims)
                const int i = lane + 64 * u;
                if (i < R) {
                    const bool first = a.rope_style ? !(i & 1) : i < R / 2;
                    const int m = a.rope_style ? i >> 1 : (first ? i : i - R / 2);
                    const float rev = __builtin_amdgcn_fractf((float)len * rope_rev(m));
                    const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
                    const float kp = bf2f(kpv[u]);
                    kk = first ? kk * cs - kp * sn : kp * sn + kk * cs;
                }
            }
            as += bf2f(qv[u]) * kk;
        }
        // ROPE: mu_t^K is part of the rotated key, so it is not a constant of the scores
        qm = ROPE ? 0.f : wave_sum(am) * a.scale_log2;
        if (self_score) s_self = wave_sum(as) * a.scale_log2;
    }
    // explicit path: q rows in fp32, log2-scaled (the paired path reads them from LDS, to keep
    // its registers for the second chunk)
    if constexpr (PAIR) {
        if (tid < D) sQ[tid] = bf2f(qp[tid]) * a.scale_log2;
    }
    float qs[(FUSED || ROPE || PAIR) ? 1 : MT][16];
    if constexpr (!FUSED) {
#pragma unroll
        for (int M = 0; M < ((FUSED || ROPE || PAIR) ? 0 : MT); ++M)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const uint2 u = qrow[M][bb];
                qs[M][4 * bb + 0] = __uint_as_float(u.x << 16) * a.scale_log2;
                qs[M][4 * bb + 1] = __uint_as_float(u.x & 0xffff0000u) * a.scale_log2;
                qs[M][4 * bb + 2] = __uint_as_float(u.y << 16) * a.scale_log2;
                qs[M][4 * bb + 3] = __uint_as_float(u.y & 0xffff0000u) * a.scale_log2;
            }
        __syncthreads();   // W_up and the page table are shared by the workgroup
    }

    // W_up operands: K tile M / V tile N, k-step ks; lane (l32, h2) holds rows 16ks+8h2 .. +7
    // of column 32*tile + l32.
    auto wk_op = [&](int M, int ks) {
        return *reinterpret_cast<const uint4 *>(&sWk[(32 * M + l32) * RKP + 16 * ks + 8 * h2]);
    };
    auto wv_op = [&](int N, int ks) {
        return *reinterpret_cast<const uint4 *>(&sWv[(32 * N + l32) * RVP + 16 * ks + 8 * h2]);
    };
    // fused path: this lane's column i = 32M + l32 of W_up,t^K scaled by q_i (log2-scaled)
    uint4 wkq[FUSED ? MT * KK : 1], wvr[FUSED ? MT * KV : 1];
    if constexpr (FUSED) {
        auto pack8 = [](const uint16_t *v) {
            return make_uint4(v[0] | (uint32_t)v[1] << 16, v[2] | (uint32_t)v[3] << 16,
                              v[4] | (uint32_t)v[5] << 16, v[6] | (uint32_t)v[7] << 16);
        };
#pragma unroll
        for (int M = 0; M < MT; ++M) {
            const float qi = bf2f(qcol[M]) * a.scale_log2;
#pragma unroll
            for (int ks = 0; ks < KK; ++ks)
                wkq[M * KK + ks] = scale_bf16x8(pack8(wkraw[M * KK + ks]), qi);
        }
#pragma unroll
        for (int N = 0; N < MT; ++N)
#pragma unroll
            for (int ks = 0; ks < KV; ++ks) wvr[N * KV + ks] = pack8(wvraw[N * KV + ks]);
    }
    // ROPE: the score in pair space.  With R_j the rotation to token j's position, pair m
    // (head-dim elements i, i') contributes cos(phi_jm) (q_i x_i + q_i' x_i') +
    // sin(phi_jm) (q_i' x_i - q_i x_i') to <q, R_j x>.  Both brackets are linear in the key
    // x = c_k W_up,t^K + mu_t^K, so they come out of MFMAs: A = the pair coefficients over the
    // ranks (q_i W[k][i] + q_i' W[k][i'], resp. q_i' W[k][i] - q_i W[k][i'], log2-scaled, bf16;
    // hi + lo terms up to rank 32) against the chunk's latents, and one more MFMA adds the mu part (its three
    // bf16 terms in k-slots 0..2 of the lanes h2 = 0, against ones).  A lane then needs, per
    // pair, its angle's sine and cosine and two FMAs; the rotation style only changes which
    // elements form pair m.
    uint4 amu[ROPE ? 2 * PT : 1];
    uint4 bone = make_uint4(0, 0, 0, 0);
    float fr[ROPE ? PT * 16 : 1];
    if constexpr (ROPE) {
        // pair m: a rotated pair (m < R/2) or two unrotated dims R + 2k, R + 2k + 1 (k = m - R/2)
        // taken as a pair with angle 0, so every pair tile has the same form
        auto pair_elems = [&](int m, int &i, int &ip) {
            if (m >= R / 2) {
                i = R + 2 * (m - R / 2);
                ip = i + 1;
            } else if (a.rope_style) {
                i = 2 * m;
                ip = 2 * m + 1;
            } else {
                i = m;
                ip = m + R / 2;
            }
        };
        const float scl = a.scale_log2;
        for (int T = wave; T < 2 * PT; T += WAVES) {     // each wave builds whole tiles
            const int N = T % PT;
            const bool sine = T >= PT;
            int i, ip;
            pair_elems(32 * N + l32, i, ip);
            const float qi = bf2f(qp[i]), qip = bf2f(qp[ip]);
            const float ca = (sine ? qip : qi) * scl, cb = (sine ? -qi : qip) * scl;
#pragma unroll
            for (int ks = 0; ks < KK; ++ks) {
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const int k = 16 * ks + 8 * h2 + e;
                    const float v0 = ca * bf2f(sWk[i * RKP + k]) + cb * bf2f(sWk[ip * RKP + k]);
                    const float v1 = ca * bf2f(sWk[i * RKP + k + 1]) + cb * bf2f(sWk[ip * RKP + k + 1]);
                    const uint16_t h0 = f2bf(v0), h1 = f2bf(v1);
                    hi[e / 2] = h0 | (uint32_t)h1 << 16;
                    lo[e / 2] = f2bf(v0 - bf2f(h0)) | (uint32_t)f2bf(v1 - bf2f(h1)) << 16;
                }
                sAq[(T * KK + ks) * TERMS][lane] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                if (TERMS == 2) sAq[(T * KK + ks) * TERMS + 1][lane] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
            }
        }
#pragma unroll
        for (int T = 0; T < 2 * PT; ++T) {
            const int N = T % PT;
            int i, ip;
            pair_elems(32 * N + l32, i, ip);
            const float qi = bf2f(qp[i]), qip = bf2f(qp[ip]);
            const float mi = bf2f(muk[i]), mip = bf2f(muk[ip]);
            const float v = scl * (T >= PT ? qip * mi - qi * mip : qi * mi + qip * mip);
            const uint16_t t0 = f2bf(v);
            const float r1 = v - bf2f(t0);
            const uint16_t t1 = f2bf(r1);
            const uint16_t t2 = f2bf(r1 - bf2f(t1));
            amu[T] = h2 ? make_uint4(0u, 0u, 0u, 0u) : make_uint4(t0 | (uint32_t)t1 << 16, t2, 0u, 0u);
        }
        bone = h2 ? make_uint4(0u, 0u, 0u, 0u) : make_uint4(0x3F803F80u, 0x3F80u, 0u, 0u);
        // lane (l32, h2) holds pairs 32N + 8 (v / 4) + 4 h2 + v % 4 of pair tile N
#pragma unroll
        for (int k = 0; k < PT * 16; ++k)
            fr[k] = rope_rev(32 * (k / 16) + 8 * ((k % 16) / 4) + 4 * h2 + (k % 4));
        __syncthreads();                                 // the pair operands are shared
    }

    float m_run = -INFINITY, l_lane = 0.f;
    float o[FUSED ? 1 : MT];                  // explicit path: p-weighted V_hat, column 32N + l32
    f32x16 ov[FUSED ? MT : 1];                // fused path: sum over chunks of p-weighted V_hat
#pragma unroll
    for (int N = 0; N < (FUSED ? 1 : MT); ++N) o[N] = 0.f;
#pragma unroll
    for (int N = 0; N < (FUSED ? MT : 1); ++N) ov[N] = f32x16{};

    // online softmax (log2 domain) for this chunk's scores: returns token l32's weight.  The
    // running max only moves when some score of the chunk exceeds it; otherwise the rescale
    // factor is exactly 1 and the wave-wide max, the exp of the old max and the rescale are
    // skipped (a wave-uniform branch).
    auto softmax_step = [&](float sc) {
        if (__builtin_amdgcn_ballot_w64(sc > m_run) != 0) {
            const float r = row16_max(sc);   // the two 16-lane rows of a half hold all 32 scores
            const float cmax = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 0)),
                                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 16)));
            const float m_new = fmaxf(m_run, cmax);
            const float alpha = exp2_(m_run - m_new);
            l_lane *= alpha;
            if constexpr (FUSED) {
#pragma unroll
                for (int N = 0; N < MT; ++N)
#pragma unroll
                    for (int v = 0; v < 16; ++v) ov[N][v] *= alpha;
            } else {
#pragma unroll
                for (int N = 0; N < MT; ++N) o[N] *= alpha;
            }
            m_run = m_new;
        }
        const float p = exp2_(sc - m_run);
        l_lane += (h2 == 0 ? p : 0.f);
        return p;
    };

    // the same for two chunks at once (paired path): one running max over their 64 tokens; returns
    // the weights of token l32 of each chunk
    auto softmax_step2 = [&](float s0, float s1, float &p0, float &p1) {
        const float sm = fmaxf(s0, s1);
        if (__builtin_amdgcn_ballot_w64(sm > m_run) != 0) {
            const float r = row16_max(sm);
            const float cmax = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 0)),
                                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 16)));
            const float m_new = fmaxf(m_run, cmax);
            const float alpha = exp2_(m_run - m_new);
            l_lane *= alpha;
#pragma unroll
            for (int N = 0; N < (FUSED ? 0 : MT); ++N) o[N] *= alpha;
            m_run = m_new;
        }
        p0 = exp2_(s0 - m_run);
        p1 = exp2_(s1 - m_run);
        l_lane += (h2 == 0 ? p0 + p1 : 0.f);
    };

    // ---- fused path, in two stages so that the matrix core can work on the next chunk's scores
    // while the vector ALUs finish the current one.
    // Scores: A = q-scaled W_up^K transposed (d x r_k), B = chunk latents (r_k x 32 tokens); the
    // tiles of all 32-row groups of the head dim add into one accumulator, whose row r holds the
    // sum over M of q_i K_hat_i(j), i = 32M + r.
    auto kscore = [&](const Chunk<KK, KV> &x) {
        f32x16 acc = {};
#pragma unroll
        for (int M = 0; M < MT; ++M)
#pragma unroll
            for (int ks = 0; ks < KK; ++ks) acc = mfma32x32x16(wkq[M * KK + ks], x.k[ks], acc);
        return acc;
    };
    // Rest of chunk c: finish the dot, softmax, then the values.  A = chunk latents with token
    // l32's row scaled by its weight p (rounded to bf16), B = W_up^V (r_v x d): V_hat tiles of 32
    // token rows, already p-weighted, add into ov across chunks; the rows are summed at the end.
    auto finish = [&](int c, const f32x16 &acc, const Chunk<KK, KV> &x) {
        const int valid = j_end - (j_begin + 32 * c);   // >= 1, wave-uniform
        float t8[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) t8[v] = acc[v] + acc[v + 8];
#pragma unroll
        for (int v = 0; v < 4; ++v) t8[v] += t8[v + 4];
        float sc = add_swap32((t8[0] + t8[2]) + (t8[1] + t8[3])) + qm;
        if (l32 >= valid) sc = -INFINITY;
        if (sSlot[c] < 0) sc = __builtin_nanf("");
        const float p = softmax_step(sc);   // token l32's weight, in both lane halves
#pragma unroll
        for (int ks = 0; ks < KV; ++ks) {
            const uint4 xs = scale_bf16x8(x.v[ks], p);
#pragma unroll
            for (int N = 0; N < MT; ++N) ov[N] = mfma32x32x16(xs, wvr[N * KV + ks], ov[N]);
        }
    };

    // explicit path (larger ranks): one chunk, start to end
    // next >= 0: the chunk to refill x with, half by half as each half is consumed
    auto compute = [&](int c, Chunk<KK, KV> &x, int next) {
        const int valid = j_end - (j_begin + 32 * c);   // >= 1, wave-uniform
        {
            // ---- scores: K_hat tiles (d rows x 32 token columns) dotted with q per lane
            float sp[MT];                           // independent chains, one per tile
            if constexpr (ROPE) {
                // token l32 sits at position j_begin + 32c + l32
                const float pos = (float)(j_begin + 32 * c + l32);
#pragma unroll
                for (int N = 0; N < PT; ++N) {
                    f32x16 tc = mfma32x32x16(amu[N], bone, f32x16{});
                    f32x16 ts = mfma32x32x16(amu[PT + N], bone, f32x16{});
#pragma unroll
                    for (int ks = 0; ks < KK; ++ks)
#pragma unroll
                        for (int term = 0; term < TERMS; ++term) {
                            tc = mfma32x32x16(sAq[(N * KK + ks) * TERMS + term][lane], x.k[ks], tc);
                            ts = mfma32x32x16(sAq[((PT + N) * KK + ks) * TERMS + term][lane], x.k[ks], ts);
                        }
                    float ac = 0.f, as = 0.f;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const float rev = __builtin_amdgcn_fractf(pos * fr[16 * N + v]);
                        ac = fmaf(__builtin_amdgcn_cosf(rev), tc[v], ac);
                        as = fmaf(__builtin_amdgcn_sinf(rev), ts[v], as);
                    }
                    sp[N] = ac + as;
                }
#pragma unroll
                for (int M = PT; M < MT; ++M) sp[M] = 0.f;
            } else {
#pragma unroll
                for (int M = 0; M < MT; ++M) {
                    f32x16 acc = {};
#pragma unroll
                    for (int ks = 0; ks < KK; ++ks)
                        acc = mfma32x32x16(wk_op(M, ks), x.k[ks], acc);
                    sp[M] = 0.f;
#pragma unroll
                    for (int v = 0; v < 16; ++v) sp[M] += qs[M][v] * acc[v];
                }
            }
            float tot = sp[0];
#pragma unroll
            for (int M = 1; M < MT; ++M) tot += sp[M];
            if (next >= 0) load_half(next, x, true);   // the keys are consumed
            float sc = add_swap32(tot) + qm;        // token l32's score, in both lane halves
            if (l32 >= valid) sc = -INFINITY;
            if (sSlot[c] < 0) sc = __builtin_nanf("");

            // ---- V_hat tiles (32 token rows x d columns), issued before the softmax chain
            // (ROPE: one at a time after it, to keep the rotation's registers free)
            f32x16 vacc[ROPE ? 1 : MT];
            if constexpr (!ROPE) {
#pragma unroll
                for (int N = 0; N < MT; ++N) {
                    vacc[N] = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < KV; ++ks)
                        vacc[N] = mfma32x32x16(x.v[ks], wv_op(N, ks), vacc[N]);
                }
            }
            const float p = softmax_step(sc);

            // ---- p of tokens 8*(v/4) + 4*h2 + (v%4): the V tile's row layout, via LDS
            if (h2 == 0) sP[wave][l32] = p;
            __builtin_amdgcn_wave_barrier();
            float pr[16];
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const float4 t4 = *reinterpret_cast<const float4 *>(&sP[wave][8 * bb + 4 * h2]);
                pr[4 * bb + 0] = t4.x; pr[4 * bb + 1] = t4.y;
                pr[4 * bb + 2] = t4.z; pr[4 * bb + 3] = t4.w;
            }
#pragma unroll
            for (int N = 0; N < MT; ++N) {
                if constexpr (ROPE) {
                    f32x16 vt = {};
#pragma unroll
                    for (int ks = 0; ks < KV; ++ks) vt = mfma32x32x16(x.v[ks], wv_op(N, ks), vt);
#pragma unroll
                    for (int v = 0; v < 16; ++v) o[N] += pr[v] * vt[v];
                } else {
#pragma unroll
                    for (int v = 0; v < 16; ++v) o[N] += pr[v] * vacc[N][v];
                }
            }
            if (next >= 0) load_half(next, x, false);   // the values are consumed
            __builtin_amdgcn_wave_barrier();
        }
    };

    // paired explicit path: chunks c0 and c1 = c0 + WAVES (has1: c1 is one of this wave's chunks;
    // otherwise x1 is ignored, its tokens get weight 0).  Every W_up operand read from LDS feeds
    // one MFMA per chunk; the two chunks' scores share one softmax step, and the V_hat tiles are
    // built one column tile at a time after it
    // n0, n1 >= 0: the chunks to refill x0 and x1 with; each half is refilled as soon as it has
    // been consumed (keys after the scores, values after the V_hat tiles), so the next pair's loads
    // overlap this pair's remaining work
    auto compute2 = [&](int c0, Chunk<KK, KV> &x0, Chunk<KK, KV> &x1, bool has1, int n0, int n1) {
        const int c1 = has1 ? c0 + WAVES : c0;
        const int valid0 = j_end - (j_begin + 32 * c0);
        const int valid1 = has1 ? j_end - (j_begin + 32 * c1) : 0;
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int M = 0; M < MT; ++M) {
            f32x16 a0 = {}, a1 = {};
#pragma unroll
            for (int ks = 0; ks < KK; ++ks) {
                const uint4 w = wk_op(M, ks);
                a0 = mfma32x32x16(w, x0.k[ks], a0);
                a1 = mfma32x32x16(w, x1.k[ks], a1);
            }
            float u0 = 0.f, u1 = 0.f;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const float4 q4 = *reinterpret_cast<const float4 *>(&sQ[32 * M + 8 * bb + 4 * h2]);
                u0 += q4.x * a0[4 * bb] + q4.y * a0[4 * bb + 1] + q4.z * a0[4 * bb + 2] + q4.w * a0[4 * bb + 3];
                u1 += q4.x * a1[4 * bb] + q4.y * a1[4 * bb + 1] + q4.z * a1[4 * bb + 2] + q4.w * a1[4 * bb + 3];
            }
            t0 += u0;
            t1 += u1;
        }
        if (n0 >= 0) {
            load_half(n0, x0, true);
            load_half(n1, x1, true);
        }
        float sc0 = add_swap32(t0) + qm, sc1 = add_swap32(t1) + qm;
        if (l32 >= valid0) sc0 = -INFINITY;
        if (l32 >= valid1) sc1 = -INFINITY;
        if (sSlot[c0] < 0) sc0 = __builtin_nanf("");
        if (sSlot[c1] < 0) sc1 = __builtin_nanf("");
        float p0, p1;
        softmax_step2(sc0, sc1, p0, p1);
        if (h2 == 0) {
            sP[wave][l32] = p0;
            sP[wave][32 + l32] = p1;
        }
        __builtin_amdgcn_wave_barrier();
        // V_hat tiles; the weights of the tile's token rows 8 bb + 4 h2 + 0..3 come from LDS
#pragma unroll
        for (int N = 0; N < MT; ++N) {
            f32x16 v0 = {}, v1 = {};
#pragma unroll
            for (int ks = 0; ks < KV; ++ks) {
                const uint4 w = wv_op(N, ks);
                v0 = mfma32x32x16(x0.v[ks], w, v0);
                v1 = mfma32x32x16(x1.v[ks], w, v1);
            }
            float acc = 0.f;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const float4 u = *reinterpret_cast<const float4 *>(&sP[wave][8 * bb + 4 * h2]);
                acc += u.x * v0[4 * bb] + u.y * v0[4 * bb + 1] + u.z * v0[4 * bb + 2] + u.w * v0[4 * bb + 3];
            }
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const float4 u = *reinterpret_cast<const float4 *>(&sP[wave][32 + 8 * bb + 4 * h2]);
                acc += u.x * v1[4 * bb] + u.y * v1[4 * bb + 1] + u.z * v1[4 * bb + 2] + u.w * v1[4 * bb + 3];
            }
            o[(FUSED) ? 0 : N] += acc;
        }
        if (n0 >= 0) {
            load_half(n0, x0, false);
            load_half(n1, x1, false);
        }
        __builtin_amdgcn_wave_barrier();
    };

    // ---- main loop: chunks wave, wave + WAVES, ...  DEPTH chunks per wave are in flight: a
    // buffer is refilled with the chunk DEPTH rounds ahead as soon as it has been consumed.
    // Prefetch indices are clamped to the last chunk, so no load sits behind a data-dependent
    // branch and the wait counts stay exact.
    // Two workgroups share each CU and the SIMD issues from the older wave first, so left alone
    // the older workgroup runs ahead and the younger one finishes alone.  A wave's issue priority
    // therefore rises with the work it has left (in chunks), which keeps the pair in step.
    auto fair_prio = [](int left) {
        if (left > 12) __builtin_amdgcn_s_setprio(3);
        else if (left > 6) __builtin_amdgcn_s_setprio(2);
        else if (left > 3) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
    };
    if (wave < nchunks) {
        const int rounds = (nchunks - wave + WAVES - 1) / WAVES;   // chunks of this wave, >= 1
        int c = wave, r = 0;
        if constexpr (FUSED) {
            // the next chunk's scores go to the matrix core before this chunk's vector work
            f32x16 kacc = kscore(buf[0]);
            for (; r + DEPTH <= rounds; r += DEPTH) {
                fair_prio(rounds - r);
#pragma unroll
                for (int i = 0; i < DEPTH; ++i) {
                    const f32x16 knext = kscore(buf[(i + 1) % DEPTH]);
                    finish(c, kacc, buf[i]);
                    load(min(c + DEPTH * WAVES, nchunks - 1), buf[i]);
                    kacc = knext;
                    c += WAVES;
                }
            }
#pragma unroll
            for (int i = 0; i + 1 < DEPTH; ++i) {
                if (r + i < rounds) {
                    const f32x16 knext = kscore(buf[(i + 1) % DEPTH]);
                    finish(c, kacc, buf[i]);
                    kacc = knext;
                    c += WAVES;
                }
            }
        } else if constexpr (PAIR) {
            // buf[0], buf[1] hold chunks c, c + WAVES; both are refilled two rounds ahead
            for (; r + 2 <= rounds; r += 2) {
                fair_prio(rounds - r);
                compute2(c, buf[0], buf[1], true, min(c + 2 * WAVES, nchunks - 1),
                         min(c + 3 * WAVES, nchunks - 1));
                c += 2 * WAVES;
            }
            if (r < rounds) compute2(c, buf[0], buf[0], false, -1, -1);   // an odd last chunk
        } else {
            for (; r + DEPTH <= rounds; r += DEPTH) {
                fair_prio(rounds - r);
#pragma unroll
                for (int i = 0; i < DEPTH; ++i) {
                    // one chunk in flight: refill its buffer half by half inside compute (the
                    // next chunk's keys then load during this chunk's values); with more chunks in
                    // flight the whole buffer is refilled after it (measured faster there)
                    if constexpr (DEPTH == 1) {
                        compute(c, buf[i], min(c + DEPTH * WAVES, nchunks - 1));
                    } else {
                        compute(c, buf[i], -1);
                        load(min(c + DEPTH * WAVES, nchunks - 1), buf[i]);
                    }
                    c += WAVES;
                }
            }
            // the last rounds % DEPTH chunks are already in their buffers
#pragma unroll
            for (int i = 0; i + 1 < DEPTH; ++i) {
                if (r + i < rounds) {
                    compute(c, buf[i], -1);
                    c += WAVES;
                }
            }
        }
    }

    // ---- merge lanes, then waves, into this split's result
    const float l_w = wave_sum(l_lane);
    float of[MT];                              // column 32N + l32 of this wave's p-weighted sum
#pragma unroll
    for (int N = 0; N < MT; ++N) {
        if constexpr (FUSED) {
            float t = 0.f;                     // the 16 token rows this lane holds, then l ^ 32
#pragma unroll
            for (int v = 0; v < 16; ++v) t += ov[N][v];
            of[N] = add_swap32(t);
        } else {
            of[N] = add_swap32(o[N]);
        }
    }
    if (h2 == 0) {
#pragma unroll
        for (int N = 0; N < MT; ++N) sO[wave][32 * N + l32] = of[N];
    }
    if (lane == 0) {
        sM[wave] = m_run;
        sL[wave] = l_w;
    }
    // a single split finishes the output here (same arithmetic as combine.hip): the current
    // token's own loop-t key/value joins the softmax and (sum of cached weights) mu_t^V is added
    __syncthreads();
    if (tid < D) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sM[w]);
        if (S == 1) M = fmaxf(M, s_self);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                const float e = exp2_(sM[w] - M);
                L += sL[w] * e;
                O += sO[w][tid] * e;
            }
        }
        if (S == 1) {
            float res = 0.f;
            if (M != -INFINITY) {
                const float w_self = self_here ? exp2_(s_self - M) : 0.f;
                const float v_self = self_here ? bf2f(vs_raw) : 0.f;
                res = (O + L * bf2f(muv_raw) + w_self * v_self) / (L + w_self);
            }
            static_cast<uint16_t *>(a.out)[((size_t)b * a.H + h) * D + tid] = f2bf(res);
        } else {
            float *rec = a.ws + (((size_t)b * a.H + h) * S + s) * (D + kPartialPad);
            rec[tid] = O;
            if (tid == 0) {
                rec[D] = M;
                rec[D + 1] = L;
                if (ROPE && s == 0) rec[D + 2] = s_self;   // the rotated self score, for combine
            }
        }
    }
}

template <int D, int RK, int RV>
hipError_t launch_t(const DecodeArgs &a, bool rope, hipStream_t st) {
    const unsigned blocks = (unsigned)a.B * a.H * a.S;
    if (rope)
        hipLaunchKernelGGL((decode_bf16_kernel<D, RK, RV, true>), dim3(blocks),
                           dim3(64 * Shape<D, RK, RV, true>::WAVES), 0, st, a);
    else
        hipLaunchKernelGGL((decode_bf16_kernel<D, RK, RV, false>), dim3(blocks),
                           dim3(64 * Shape<D, RK, RV, false>::WAVES), 0, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, bool rope, hipStream_t st) {
#define LLA_CASE(RK, RV) \
    if (a.r_k == RK && a.r_v == RV) return launch_t<D, RK, RV>(a, rope, st);
    LLA_CASE(16, 16)
    LLA_CASE(16, 32)
    LLA_CASE(32, 32)
    LLA_CASE(32, 64)
    LLA_CASE(64, 64)
    LLA_CASE(64, 128)
    LLA_CASE(96, 160)
#undef LLA_CASE
    return hipErrorInvalidValue;
}

}  // namespace

bool decode_bf16_supported(int d, int r_k, int r_v) {
    if (d != 64 && d != 128) return false;
    const int pairs[][2] = {{16, 16}, {16, 32}, {32, 32}, {32, 64}, {64, 64}, {64, 128}, {96, 160}};
    for (auto &p : pairs)
        if (p[0] == r_k && p[1] == r_v) return true;
    return false;
}

hipError_t launch_decode_bf16(const DecodeArgs &a, bool rope, hipStream_t st) {
    const int d = a.mode ? a.Dg / a.H : a.Dg;
    if (d == 128) return launch_d<128>(a, rope, st);
    if (d == 64) return launch_d<64>(a, rope, st);
    return hipErrorInvalidValue;
}

}  // namespace lla
