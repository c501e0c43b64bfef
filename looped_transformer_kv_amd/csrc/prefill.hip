// prefill.hip -- chunked prefill attention over the latent cache, bf16 storage, gfx950 MFMA.
//
// A chunk of new tokens per sequence attends, for loop t, to the cached context through the codec
// (pith.science paper page for "Looped Latent Attention", "What carries the argument":
// x_hat_t = c W_up,t + mu_t, attention unchanged) and causally to the chunk's own loop-t keys and
// values, which are taken as given (they are encoded only after the last loop, like the decode
// step's own token).  New token i of sequence b sees cached j < seq_lens[b] and new i' <= i.
//
// Cached tokens are attended in latent space.  With no rotation, the codec's reconstruction is
// linear, so for a query q (scores in the log2 domain, c = scale log2(e)):
//   s_j = c <q, c_k(j) W_up,t^K + mu_t^K> = <q', c_k(j)> + c <q, mu_t^K>,  q' = c W_up,t^K q,
//   sum_j p_j V_hat(j) = (sum_j p_j c_v(j)) W_up,t^V + (sum_j p_j) mu_t^V,
// the identity the absorbed decode uses.  Per cached 32-token tile a wave then runs one score
// MFMA per 16 key ranks (A = the latent rows, B = q'^T) and two value MFMAs into a 32 x 32
// latent accumulator O_lat^T = C_v^T P^T (rank x query); the chunk's own tiles are ordinary flash
// attention over the given keys and values, and one online softmax spans both.
//
// Two passes, launched back to back on the caller's stream:
// * the cached pass (one workgroup of 8 waves per (sequence, head, block of 256 queries); wave w
//   owns queries [32w, 32w + 32) of the block) runs the online softmax over the cached tiles in
//   latent space and parks each query's partial state (O_lat, running max, weight sum) in its own
//   out row.  It holds only latent-sized state, so four waves share a SIMD, and it stages 8 tiles
//   per step with two steps of loads in flight, enough to cover HBM latency; its speed is then
//   set by the softmax's vector work and each wave's dependent chain per tile.
// * the chunk pass (same grid) starts from that state, O^T = W_up,t^V^T O_lat^T, runs ordinary
//   flash attention over the chunk's own tiles up to each query, adds (sum of cached weights)
//   mu_t^V, normalises and overwrites the row with the result.
// Every score tile is S^T (32 tokens x 32 queries, v_mfma_f32_32x32x16_bf16), so each lane holds
// 16 scores of one query: the softmax row statistics need in-lane reductions and one exchange
// between lanes l and l ^ 32, and every accumulator keeps one query per lane, so the online
// rescale is a per-lane multiply.  Tiles are staged in LDS in the lane layout of the MFMA
// operands (cached: the latent rows and the value latents transposed; chunk: key and value rows);
// LDS is double-buffered with one barrier per step.
// Precision: q', the latents, the chunk keys and values, the softmax weights and O_lat (rounded
// once, when parked) are bf16 MFMA operands (the precision class of a bf16 KV cache in a
// flash-attention kernel); scores, statistics and accumulators are fp32; out is rounded once (RNE).
#include "lla_internal.h"

namespace lla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ f32x16 mfma(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// two fp32 -> two bf16 (round to nearest even), lo in the low half
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// two 16-bit values, lo in the low half
__device__ __forceinline__ uint32_t pk16(short lo, short hi) {
    return static_cast<uint32_t>(static_cast<uint16_t>(lo)) | (static_cast<uint32_t>(static_cast<uint16_t>(hi)) << 16);
}

// elements 8s .. 8s + 7 of an accumulator as one 8 x bf16 operand
__device__ __forceinline__ uint4 pack8(const f32x16 &x, int s) {
    return make_uint4(pk_bf16(x[8 * s + 0], x[8 * s + 1]), pk_bf16(x[8 * s + 2], x[8 * s + 3]),
                      pk_bf16(x[8 * s + 4], x[8 * s + 5]), pk_bf16(x[8 * s + 6], x[8 * s + 7]));
}

// max(x[l], x[l ^ 32]) in every lane
__device__ __forceinline__ float max_swap32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

constexpr int PWAVES = 8;                  // waves per workgroup
constexpr int QWG = PWAVES * 32;           // queries per workgroup: one 32-query tile per wave
constexpr int CNS = 2;                     // chunk tiles in flight in the chunk pass
constexpr int CWAVES = 8;                  // waves per workgroup of the chunk pass
constexpr int CQWG = CWAVES * 32;          // queries per workgroup of the chunk pass
constexpr float kSlack = 8.f;              // lazy rescale threshold (log2 domain)
constexpr int kBufferWord3 = 0x00020000;   // word 3 of a raw (untyped, unswizzled) buffer resource

// An operand slot in LDS holds one 16-byte row per lane; a 16-byte pad after every 8 rows spreads
// the transposed 2-byte writes of the value operands over the banks (a group of 8 lanes still
// reads 128 contiguous bytes).
constexpr int kSlot = 72;                  // uint4 per operand slot
__device__ __forceinline__ int srow(int r) { return r + (r >> 3); }

// Query operands (B of a full-width score MFMA over the head dims): lane (l32, h2) holds query row
// wq0 + l32, k-step ks covers dims 32 (ks / 2) + 16 (ks % 2) + 4 h2 + {0..3} and + 8 + {0..3} (a
// permutation of the head dims that the chunk keys' LDS layout shares).  Rows past the chunk read
// the last valid row (their results are not stored).
template <int D>
__device__ __forceinline__ void load_query_operands(const PrefillArgs &a, int b, int h, int qrow,
                                                    int h2, uint4 (&qop)[D / 16]) {
    const uint16_t *row = static_cast<const uint16_t *>(a.q) + (((size_t)b * a.Pn + qrow) * a.H + h) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const int d0 = 32 * (ks >> 1) + 16 * (ks & 1) + 4 * h2;
        const uint2 lo = *reinterpret_cast<const uint2 *>(row + d0);
        const uint2 hi = *reinterpret_cast<const uint2 *>(row + d0 + 8);
        qop[ks] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
}

// This lane's half of <q, mu_t^K> (the dims of its query operands: k-step ks covers dims
// 16 ks + 4 h2 + {0..3} and 16 ks + 8 + 4 h2 + {0..3}); the partner lane h2 ^ 1 holds the other half.
template <int D>
__device__ __forceinline__ float query_dot_mu_k(const PrefillArgs &a, int g, int col0, int h2,
                                                const uint4 (&qop)[D / 16]) {
    const uint16_t *muk = static_cast<const uint16_t *>(a.mu_k) + (size_t)g * a.T * a.Dg +
                          (size_t)a.t * a.Dg + col0 + 4 * h2;
    float qm = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const uint2 lo = *reinterpret_cast<const uint2 *>(muk + 16 * ks);
        const uint2 hi = *reinterpret_cast<const uint2 *>(muk + 16 * ks + 8);
        const uint32_t mv[4] = {lo.x, lo.y, hi.x, hi.y};
        const uint32_t qv[4] = {qop[ks].x, qop[ks].y, qop[ks].z, qop[ks].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qm += __uint_as_float(qv[i] << 16) * __uint_as_float(mv[i] << 16);
            qm += __uint_as_float(qv[i] & 0xFFFF0000u) * __uint_as_float(mv[i] & 0xFFFF0000u);
        }
    }
    return qm;
}

// Partial softmax state of the cached pass, parked per query in that query's own out row until
// the chunk pass overwrites the row with its result: O_lat as bf16 in the lane order of the
// W_up,t^V MFMA's B operand (lane (query, h2), k-step ks at uint4 KV h2 + ks), then the running
// max and the weight sum (fp32).  32 KV + 8 <= 72 bytes, inside a row of 64 bf16.
__device__ __forceinline__ uint4 *state_row(const PrefillArgs &a, int b, int iq, int h, int D) {
    return reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.out) +
                                     (((size_t)b * a.Pn + iq) * a.H + h) * D);
}

// ================================================================ cached pass
template <int RK, int RV>
struct CShape {
    static constexpr int KK = RK / 16, KV = RV / 16;   // k-steps over the key / value ranks
    // 16-byte latent pieces (8 ranks of one token) of a cached tile: key pieces, then value pieces
    static constexpr int CPK = 32 * RK / 8, CPV = 32 * RV / 8, CP = CPK + CPV;
    // cached tiles per pipeline step: 8 (256 tokens), 4 when a tile has more pieces than 3 per
    // wave, which keeps the stage registers at 24
    static constexpr int CGT = CP > 192 ? 4 : 8;
    static constexpr int NP = CP * CGT / (64 * PWAVES);   // pieces per thread per step
    static constexpr int SL = KK + 2;                     // 1 KB operand slots per tile
    static_assert(CP * CGT % (64 * PWAVES) == 0, "whole pieces per thread");
    static_assert(CPK % 64 == 0, "each wave's pieces are all keys or all values");
    static_assert(RK <= 32 && RV <= 32, "one 32-row MFMA tile of latent ranks");
};

// Registers holding one step's latent pieces (this thread's) while they are in flight.
template <int N>
struct CStage {
    uint4 r[N];
    bool bad;                                  // uniform: a page id of the step was out of range
};

// One workgroup per (sequence, head, block of 256 queries), 8 waves, two workgroups per CU.
// Only the latent state (q', O_lat, max, sum) lives in registers, so four waves share a SIMD; a
// step stages 8 tiles (256 tokens; 4 at key and value ranks 32) through LDS and the next two
// steps' latents are in flight,
// enough bytes per CU to cover HBM latency.
template <int D, int RK, int RV>
__global__ __launch_bounds__(64 * PWAVES) __attribute__((amdgpu_waves_per_eu(4)))
void prefill_cached_kernel(PrefillArgs a) {
    using CS = CShape<RK, RV>;
    constexpr int KS = D / 16, KK = CS::KK, KV = CS::KV, NP = CS::NP, SL = CS::SL;
    constexpr int CP = CS::CP, CPK = CS::CPK, CGT = CS::CGT;
    using St = CStage<NP>;

    // per buffer and tile: slots [0, KK) the key latents (A of the score MFMA), [KK, KK + 2) the
    // value latents transposed (A of the value MFMA)
    __shared__ __align__(16) uint4 cbuf[2][CGT][SL][kSlot];
    __shared__ int sbad[PWAVES];
    // A operands of the q' MFMA (W_up,t^K at the query operand's dims), one k-step per slot
    __shared__ __align__(16) uint4 sWk[KS][kSlot];
    static_assert(KS <= PWAVES, "one operand slot per wave");

    const int id = xcd_work_item(blockIdx.x, gridDim.x);
    const int qb = id % a.QB;
    const int h = (id / a.QB) % a.H;
    const int b = id / (a.QB * a.H);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h2 = lane >> 5;
    const int g = a.mode ? 0 : h;
    const int col0 = a.mode ? h * D : 0;

    int nn = a.n_new[b];
    nn = nn < 0 ? 0 : (nn > a.Pn ? a.Pn : nn);
    const int q0 = qb * QWG;
    if (q0 >= nn) return;                               // the whole block is past the chunk
    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
    if (len == 0) return;                               // nothing cached: the chunk pass starts empty
    const int qend = min(nn, q0 + QWG);
    const int ctiles = (len + 31) >> 5;
    const int steps = (ctiles + CGT - 1) / CGT;
    const int wq0 = q0 + 32 * wave;
    const bool wlive = wq0 < qend;
    const float csc = a.scale_log2;

    // ---- q' = c W_up,t^K q for this wave's queries, on the matrix cores: q'^T = W q^T with
    // A = W_up,t^K (lane (rank l32, h2): the rank's row at the query operand's dims; ranks past
    // RK are zero), B = the query operands.  Lane (query, h2) gets ranks 8 (v / 4) + 4 h2 + v % 4,
    // which packs straight into the B operand of the score MFMA (k-step ks: ranks
    // 16 ks + 8 (e / 4) + 4 h2 + e % 4 at element e).  q mu_t^K (scaled) is one in-lane dot over
    // this lane's half of the dims plus an exchange.
    uint4 qlat[KK];
    float qmu;
    {
        // wave w < KS builds operand slot w (buffer loads: a fixed byte offset per lane plus a
        // scalar one per element); the workgroup shares the slots
        const uint16_t *Wk = static_cast<const uint16_t *>(a.W_up_k) +
                             ((size_t)a.t * a.G + g) * RK * a.Dg + col0;
        if (wave < KS) {
            const int ks = wave;
            const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t *>(Wk), 0, ((RK - 1) * a.Dg + D) * 2, kBufferWord3);
            const int wl = (min(l32, RK - 1) * a.Dg + 4 * h2) * 2;
            uint16_t w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint16_t v = __builtin_amdgcn_raw_buffer_load_b16(
                    wr, wl, (32 * (ks >> 1) + 16 * (ks & 1) + (e < 4 ? e : e + 4)) * 2, 0);
                w[e] = l32 < RK ? v : (uint16_t)0;
            }
            sWk[ks][srow(lane)] = make_uint4(w[0] | (uint32_t)w[1] << 16, w[2] | (uint32_t)w[3] << 16,
                                             w[4] | (uint32_t)w[5] << 16, w[6] | (uint32_t)w[7] << 16);
        }
        uint4 qop[KS];
        load_query_operands<D>(a, b, h, min(wq0 + l32, nn - 1), h2, qop);
        const float qm = query_dot_mu_k<D>(a, g, col0, h2, qop);
        __syncthreads();                                // the W_up,t^K slots
        f32x16 qa = {};
        const int rdw = srow(lane);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa = mfma(sWk[ks][rdw], qop[ks], qa);
#pragma unroll
        for (int v = 0; v < 16; ++v) qa[v] *= csc;
#pragma unroll
        for (int ks = 0; ks < KK; ++ks) qlat[ks] = pack8(qa, ks);
        qmu = (qm + __shfl_xor(qm, 32, 64)) * csc;
    }

    // ---- step inputs.  Piece p = tid + 512 x of step s belongs to tile 8 s + p / CP (clamped to
    // the last cached tile); within the tile, piece p' = p % CP is (token p' / (R / 8), clamped to
    // the last valid token; ranks 8 (p' % (R / 8)) .. + 7) of c_k (p' < CPK) or of c_v (p' - CPK),
    // in one page (P is a multiple of 32).  CP and CPK are multiples of 64, so a wave's pieces of
    // one slot are all keys or all values of one tile: the page lookup is scalar, per wave and
    // slot, and only the token and rank are per lane.
    const uint16_t *kp = static_cast<const uint16_t *>(a.k_pool);
    const uint16_t *vp = static_cast<const uint16_t *>(a.v_pool);
    const int32_t *bt = a.block_table + (size_t)b * a.max_pages;
    const int tpp = a.P >> 5;                           // tiles per page
    // tile / tpp = mulhi(tile, tmag) or one more (tile < 2^32)
    const uint32_t tmag = 0xFFFFFFFFu / (uint32_t)tpp;
    auto slot_tile = [&](int x) { return (64 * wave + 64 * PWAVES * x) / CP; };
    auto slot_key = [&](int x) { return (64 * wave + 64 * PWAVES * x) % CP < CPK; };
    auto lane_piece = [&](int x) { return ((64 * wave + 64 * PWAVES * x) % CP) + lane - (slot_key(x) ? 0 : CPK); };
    bool bad_w = false;                                 // uniform: this wave met a bad page id
    auto issue = [&](int s, St &st) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < NP; ++x) {
            const int tile = min(CGT * s + slot_tile(x), ctiles - 1);
            uint32_t pidx = __umulhi((uint32_t)tile, tmag);
            int toff = tile - (int)pidx * tpp;
            if (toff >= tpp) {
                toff -= tpp;
                ++pidx;
            }
            int page = bt[pidx];
            const bool ok = (unsigned)page < (unsigned)a.n_pages;
            st.bad |= !ok;
            page = ok ? page : 0;
            const int row = (page * a.G + g) * a.P + 32 * toff;   // pool row of the tile's token 0
            const int lim = len - 1 - 32 * tile;                   // >= 0: last valid token
            const bool key = slot_key(x);
            const int R = key ? RK : RV;
            const int pi = lane_piece(x);
            const int tok = pi / (R / 8), rank = 8 * (pi % (R / 8));
            const uint16_t *src = (key ? kp : vp) + (size_t)(row + min(tok, lim)) * R + rank;
            st.r[x] = *reinterpret_cast<const uint4 *>(src);
        }
    };

    // ---- write step s's pieces into LDS buffer `buf` in operand layout
    auto produce = [&](int s, St &st, int buf) __attribute__((always_inline)) {
        if (s >= steps) return;
        bad_w |= st.bad;
        st.bad = false;
#pragma unroll
        for (int x = 0; x < NP; ++x) {
            const int tg = slot_tile(x);
            const int pi = lane_piece(x);
            const uint4 w = st.r[x];
            if (slot_key(x)) {
                // A operand of the score MFMA, lane (token, h2) of k-step ks: ranks
                // 16 ks + 8 (e / 4) + 4 h2 + e % 4 at element e.  Ranks 8 p' .. + 3 of this piece
                // go to lane (token, 0), + 4 .. + 7 to lane (token, 1), elements 4 (p' % 2) .. + 3,
                // k-step p' / 2 (p' = rank / 8).
                const int tok = pi / (RK / 8), pq = pi % (RK / 8);
                uint2 *d0 = reinterpret_cast<uint2 *>(&cbuf[buf][tg][pq >> 1][srow(tok)]) + (pq & 1);
                uint2 *d1 =
                    reinterpret_cast<uint2 *>(&cbuf[buf][tg][pq >> 1][srow(32 + tok)]) + (pq & 1);
                *d0 = make_uint2(w.x, w.y);
                *d1 = make_uint2(w.z, w.w);
            } else {
                // A operand of the value MFMA, lane (rank, h2) of token k-step kj: tokens
                // 16 kj + 8 (e / 4) + 4 h2 + e % 4 at element e
                const int tok = pi / (RV / 8), rank = 8 * (pi % (RV / 8));
                const int kj = tok >> 4, rem = tok & 15;
                const int hh = (rem >> 2) & 1, e = 4 * (rem >> 3) + (rem & 3);
                const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int y = 0; y < 8; ++y) {
                    uint16_t *dst = reinterpret_cast<uint16_t *>(
                        &cbuf[buf][tg][KK + kj][srow(32 * hh + rank + y)]);
                    dst[e] = static_cast<uint16_t>(wd[y >> 1] >> (16 * (y & 1)));
                }
            }
        }
    };

    // ---- online softmax over the cached tokens (log2 domain), with the matrix cores doing the
    // per-score additions.  Scores are taken relative to a reference m_b: the score MFMA starts
    // from a bias MFMA that adds c q mu_t^K - m_b to every score (A = 1 at ranks 0..2 of lanes
    // h2 = 0, B = that bias split into three bf16 terms, whose sum is exact to 2^-27 relative),
    // so p = 2^sc needs no per-score add, and the weight sum is an MFMA of the packed weights
    // against ones (every lane gets its query's full sum).  Lazy rescale, guarded by that sum:
    // m_b moves (to the tile's max) only when a tile's weights sum past 2^32 (an overflowed
    // weight included), and the tile's weights are then recomputed; no weight the accumulators
    // take exceeds 2^32, and the result is exact after the final normalisation.  The first tile
    // sets m_b from its max.
    constexpr float kSumMax = 4294967296.f;             // 2^32
    const uint32_t one2 = 0x3F803F80u;                  // two bf16 ones
    const uint4 onesA = make_uint4(one2, one2, one2, one2);
    const uint4 biasA = h2 ? make_uint4(0u, 0u, 0u, 0u) : make_uint4(one2, 0x3F80u, 0u, 0u);
    auto bias_op = [&](float bv) __attribute__((always_inline)) {
        const uint16_t hi = f2bf(bv);
        const float r1 = bv - bf2f(hi);
        const uint16_t mid = f2bf(r1);
        const uint16_t lo = f2bf(r1 - bf2f(mid));
        return h2 ? make_uint4(0u, 0u, 0u, 0u)
                  : make_uint4(hi | (uint32_t)mid << 16, lo, 0u, 0u);
    };
    float m_b = 0.f, l_run = 0.f;
    bool started = false;                               // uniform: m_b has been set
    uint4 biasB = bias_op(qmu);
    f32x16 olat = {};
    const int rd = srow(lane);                          // this lane's operand row
    // move the reference to the tile's max (per query: both lanes agree); first: no history
    auto rebase = [&](f32x16 &sc, bool first) __attribute__((always_inline)) {
        float mx = sc[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sc[v]);
        float delta = max_swap32(mx);
        if (!first) delta = fmaxf(delta, 0.f);
        if (!(delta > -INFINITY)) delta = 0.f;          // all masked (or NaN): keep m_b
        const float alpha = first ? 0.f : exp2_(-delta);
        l_run *= alpha;
#pragma unroll
        for (int v = 0; v < 16; ++v) olat[v] *= alpha;
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[v] -= delta;
        m_b += delta;
        biasB = bias_op(qmu - m_b);
    };
    auto consume = [&](int s, int buf) __attribute__((always_inline)) {
        if (!wlive || s >= steps) return;
        const int nt = min(CGT, ctiles - CGT * s);
        for (int j = 0; j < nt; ++j) {
            const int j0 = 32 * (CGT * s + j);
            f32x16 sc = mfma(biasA, biasB, f32x16{});
#pragma unroll
            for (int ks = 0; ks < KK; ++ks) sc = mfma(cbuf[buf][j][ks][rd], qlat[ks], sc);
            // the last tile masks tokens past len.  Lane (query, h2), element v: token
            // 8 (v / 4) + 4 h2 + v % 4.
            if (j0 + 32 > len) {
                const int lm = len - 1 - j0 - 4 * h2;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (8 * (v >> 2) + (v & 3) > lm) sc[v] = -INFINITY;
            }
            if (!started) {
                rebase(sc, true);
                started = true;
            }
            f32x16 pr;
#pragma unroll
            for (int v = 0; v < 16; ++v) pr[v] = exp2_(sc[v]);
            uint4 p0 = pack8(pr, 0), p1 = pack8(pr, 1);
            f32x16 ls = mfma(onesA, p1, mfma(onesA, p0, f32x16{}));
            if (__builtin_amdgcn_ballot_w64(ls[0] > kSumMax) != 0) {
                rebase(sc, false);
#pragma unroll
                for (int v = 0; v < 16; ++v) pr[v] = exp2_(sc[v]);
                p0 = pack8(pr, 0);
                p1 = pack8(pr, 1);
                ls = mfma(onesA, p1, mfma(onesA, p0, f32x16{}));
            }
            olat = mfma(cbuf[buf][j][KK][rd], p0, olat);
            olat = mfma(cbuf[buf][j][KK + 1][rd], p1, olat);
            l_run += ls[0];
        }
    };

    // ---- pipeline: step i + 1 produced while step i is consumed; step i + 2's inputs in flight
    St s0, s1;
    s0.bad = s1.bad = false;
    issue(0, s0);
    issue(1, s1);
    produce(0, s0, 0);
    issue(2, s0);
    __syncthreads();
    for (int it = 0; it < steps; it += 2) {
        produce(it + 1, s1, 1);
        issue(it + 3, s1);
        consume(it, 0);
        __syncthreads();
        produce(it + 2, s0, 0);
        issue(it + 4, s0);
        consume(it + 1, 1);
        __syncthreads();
    }

    // ---- park the state in the query's out row (an out-of-range page anywhere in the cached
    // context makes the sum NaN)
    if (lane == 0) sbad[wave] = bad_w;
    __syncthreads();
    bool bad_any = false;
#pragma unroll
    for (int w = 0; w < PWAVES; ++w) bad_any |= sbad[w] != 0;
    if (!wlive) return;
    const int iq = wq0 + l32;
    if (iq >= qend) return;
    uint4 *st = state_row(a, b, iq, h, D);
#pragma unroll
    for (int ks = 0; ks < KV; ++ks) st[KV * h2 + ks] = pack8(olat, ks);
    if (h2 == 0)
        *reinterpret_cast<float2 *>(st + 2 * KV) =
            make_float2(m_b, bad_any ? __builtin_nanf("") : l_run);
}

// ================================================================ chunk pass
template <int D>
struct PShape {
    static constexpr int MT = D / 32;                  // 32-wide tiles of the head dim
    static constexpr int KS = D / 16;                  // k-steps of a full-width score MFMA
    // 16-byte pieces of a 32-token chunk tile per axis (32 rows x D / 8), per thread
    static constexpr int PIECES = 32 * D / 8;
    static constexpr int NEWP = (PIECES + 64 * CWAVES - 1) / (64 * CWAVES);
    static constexpr int NST = 2 * NEWP;               // stage registers per thread
    // value rows are kept as stored (token-major, each row padded to D + 16 elements so that the
    // four rows a transposed read touches fall in distinct banks) after the KS key slots
    static constexpr int VST = D + 16;
    static constexpr int VSLOTS = (32 * VST * 2 + 16 * kSlot - 1) / (16 * kSlot);
    static constexpr int SLOTS = KS + VSLOTS;          // 1 KB operand slots per LDS buffer
    static_assert(MT == 2 || MT == 4, "head dim 64 or 128");
};

// Registers holding one chunk tile's 16-byte pieces of the key and value rows while they are in
// flight (key pieces, then value pieces).
template <int N>
struct Stage {
    uint4 r[N];
};

// W_up,t^V, the A operand of the expansion O^T = W_up,t^V^T O_lat^T, staged once per workgroup in
// LDS as stored (rank-major rows of the head's D dims, each row padded to D + 16 elements so that
// the four rows a transposed read touches fall in distinct banks), with 16-byte loads by every
// thread.  Lane (dim, h2) of 32-dim tile n, k-step ks takes the dim's column at ranks
// 16 ks + 8 (e / 4) + 4 h2 + e % 4 (the order of O_lat's B operand) through two ds_read_b64_tr_b16.
template <int D>
constexpr int wv_stride() { return D + 16; }

template <int D, int RV>
__device__ __forceinline__ void stage_wv(const PrefillArgs &a, int g, int col0, int tid, int nthr,
                                         uint16_t *sWv) {
    constexpr int ST = wv_stride<D>(), PR = D / 8;            // 16-byte pieces per row
    const uint16_t *Wv = static_cast<const uint16_t *>(a.W_up_v) +
                         ((size_t)a.t * a.G + g) * RV * a.Dg + col0;
    for (int p = tid; p < RV * PR; p += nthr) {
        const int row = p / PR, c8 = p - row * PR;
        *reinterpret_cast<uint4 *>(sWv + row * ST + 8 * c8) =
            *reinterpret_cast<const uint4 *>(Wv + (size_t)row * a.Dg + 8 * c8);
    }
}

// the A operand of 32-dim tile n, k-step ks: lane (4 e' + m) of each 16-lane group addresses rank
// 16 ks + 4 h2 + e' (+ 8 for the second read) at dims 32 n + 16 ((lane / 16) % 2) + 4 m .. + 3
template <int D>
__device__ __forceinline__ uint4 wv_operand(const uint16_t *sWv, int n, int ks, int lane) {
    constexpr int ST = wv_stride<D>();
    const int h2 = lane >> 5;
    lds_char *p = (lds_char *)(sWv) +
                  ((16 * ks + 4 * h2 + ((lane & 15) >> 2)) * ST + 32 * n + 16 * ((lane >> 4) & 1) +
                   4 * (lane & 3)) * 2;
    const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 16 * ST));
    return make_uint4(pk16(r0[0], r0[1]), pk16(r0[2], r0[3]), pk16(r1[0], r1[1]), pk16(r1[2], r1[3]));
}

// Flash attention of a workgroup's queries [q0, qend) (8 waves, wave w owning 32 of them) over
// the chunk's own tiles up to each query, from the state the cached context left (oacc = the
// cached part in model space, unnormalised; m_run its reference in the log2 domain; l_run and
// l_lat this lane's share of the cached weight sum).  Then + (sum of cached weights) mu_t^V,
// normalise and store.  `expand` runs once, after the first chunk tile is in LDS: the two-pass
// form forms the cached part's expansion there, while its loads are in flight.
template <int D, typename Expand>
__device__ __forceinline__ void chunk_phase(const PrefillArgs &a, int b, int h, int g, int col0,
                                            int nn, int q0, int qend,
                                            uint4 (&sbuf)[2][PShape<D>::SLOTS][kSlot],
                                            const uint4 (&qop)[D / 16], f32x16 (&oacc)[D / 32],
                                            float m_run, float l_run, float l_lat, Expand expand) {
    using SH = PShape<D>;
    constexpr int MT = SH::MT, KS = SH::KS;
    constexpr int NEWP = SH::NEWP, NST = SH::NST;
    using St = Stage<NST>;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h2 = lane >> 5;
    const int tiles = (qend + 31) >> 5;                 // chunk tiles up to the last query
    const int wq0 = q0 + 32 * wave;                     // this wave's first query
    const bool wlive = wq0 < qend;
    const int iq = wq0 + l32;
    const float csc = a.scale_log2;

    // ---- tile inputs.  Chunk tile n: piece p = tid + 512 x of each axis is row 32n + (p % 128) / 4
    // (clamped to the last valid row), dims 32 (p / 128) + 8 (p % 4) .. + 7: a wave covers 16 rows
    // of one 32-dim tile, so the transposed value writes of half a wave fall in 16 distinct banks.
    // Slots [0, NEWP) hold key pieces, [NEWP, 2 NEWP) value pieces.
    const uint16_t *kn = static_cast<const uint16_t *>(a.k_new);
    const uint16_t *vn = static_cast<const uint16_t *>(a.v_new);
    auto piece_row = [](int pc) { return (pc & 127) >> 2; };
    auto piece_dim = [](int pc) { return 32 * (pc >> 7) + 8 * (pc & 3); };
    int pc_row[NST], pc_col[NST];
#pragma unroll
    for (int x = 0; x < NST; ++x) {
        const int pc = min(tid + 64 * CWAVES * (x % NEWP), SH::PIECES - 1);
        pc_row[x] = piece_row(pc);
        pc_col[x] = piece_dim(pc);
    }
    const uint16_t *kn_b = kn + (size_t)b * a.Pn * a.new_stride + (size_t)h * D;
    const uint16_t *vn_b = vn + (size_t)b * a.Pn * a.new_stride + (size_t)h * D;
    auto issue = [&](int tile, St &st) __attribute__((always_inline)) {
        tile = min(tile, tiles - 1);
        const int n0 = 32 * tile;
        const int rmax = nn - 1 - n0;
#pragma unroll
        for (int x = 0; x < NST; ++x) {
            const uint16_t *chk = (x < NEWP ? kn_b : vn_b) +
                                  (uint32_t)((n0 + min(pc_row[x], rmax)) * (int)a.new_stride +
                                             pc_col[x]);
            st.r[x] = *reinterpret_cast<const uint4 *>(chk);
        }
    };

    // ---- write tile `tile` into LDS buffer `buf` in operand layout
    auto produce = [&](int tile, const St &st, int buf) __attribute__((always_inline)) {
        if (tile >= tiles) return;
        // key piece (row jr, dims 8c .. 8c + 7): dims 8c + 4 hh + {0..3} are elements
        // 4 (c % 2) .. + 3 of lane 32 hh + jr in k-step 2 (c / 4) + (c / 2) % 2
#pragma unroll
        for (int x = 0; x < NEWP; ++x) {
            const int pc = tid + 64 * CWAVES * x;
            if (SH::PIECES % (64 * CWAVES) != 0 && pc >= SH::PIECES) break;
            const int jr = piece_row(pc), c8 = piece_dim(pc) >> 3;
            const int ks = 2 * (c8 >> 2) + ((c8 >> 1) & 1);
            const uint4 w = st.r[x];
            uint2 *d0 = reinterpret_cast<uint2 *>(&sbuf[buf][ks][srow(jr)]) + (c8 & 1);
            uint2 *d1 = reinterpret_cast<uint2 *>(&sbuf[buf][ks][srow(32 + jr)]) + (c8 & 1);
            *d0 = make_uint2(w.x, w.y);
            *d1 = make_uint2(w.z, w.w);
        }
        // value piece (row jr, dims 8p .. 8p + 7) -> its place in the token-major value rows
        uint16_t *vrow = reinterpret_cast<uint16_t *>(&sbuf[buf][KS][0]);
#pragma unroll
        for (int x = 0; x < NEWP; ++x) {
            const int pc = tid + 64 * CWAVES * x;
            if (SH::PIECES % (64 * CWAVES) != 0 && pc >= SH::PIECES) break;
            *reinterpret_cast<uint4 *>(vrow + piece_row(pc) * SH::VST + piece_dim(pc)) =
                st.r[NEWP + x];
        }
    };
    // the V^T operand of 32-dim tile n, token k-step kj: lane (dim, h2) holds tokens
    // 16 kj + 8 (e / 4) + 4 h2 + e % 4 at element e (the order of P^T), through two transposed
    // reads: lane (4 e' + m) of each 16-lane group addresses token 16 kj + 4 h2 + e' (+ 8) at dims
    // 32 n + 16 ((lane / 16) % 2) + 4 m .. + 3, and lane l gets dim 32 n + l % 32
    const uint32_t vtr = (uint32_t)(((4 * h2 + ((lane & 15) >> 2)) * SH::VST +
                                     16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2);
    auto vt_operand = [&](int buf, int n, int kj) __attribute__((always_inline)) {
        lds_char *p = (lds_char *)(&sbuf[buf][KS][0]) + vtr + (16 * kj * SH::VST + 32 * n) * 2;
        const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
        const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 16 * SH::VST));
        return make_uint4(pk16(r0[0], r0[1]), pk16(r0[2], r0[3]), pk16(r1[0], r1[1]),
                          pk16(r1[2], r1[3]));
    };

    // ---- online softmax over the chunk's tiles (log2 domain; raw q . k scores need * c), lazy
    // rescale
    const int wlast = min(wq0 + 31, qend - 1);          // this wave's last query
    const int rd = srow(lane);                          // this lane's operand row
    auto consume = [&](int tile, int buf) __attribute__((always_inline)) {
        if (!wlive || tile >= tiles) return;
        const int j0 = 32 * tile;
        if (j0 > wlast) return;                         // every token is after every query
        f32x16 sc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sc = mfma(sbuf[buf][ks][rd], qop[ks], sc);
        // tiles that reach past this wave's first query mask the tokens after each query.  Lane
        // (query, h2), element v: token 8 (v / 4) + 4 h2 + v % 4.
        if (j0 + 31 > wq0) {
            const int lim = wq0 + l32 - j0;             // last visible token
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if (8 * (v >> 2) + 4 * h2 + (v & 3) > lim) sc[v] = -INFINITY;
        }
        float mx = sc[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sc[v]);
        mx = max_swap32(mx) * csc;
        const float m_cand = fmaxf(m_run, mx);
        if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kSlack) != 0) {
            const float alpha = m_cand == -INFINITY ? 1.f : exp2_(m_run - m_cand);
            l_run *= alpha;
            l_lat *= alpha;
#pragma unroll
            for (int n = 0; n < MT; ++n)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[n][v] *= alpha;
            m_run = m_cand;
        }
        // softmax weights as the two bf16 B operands of the value MFMAs
        f32x16 pr;
        float ls = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            pr[v] = exp2_(fmaf(sc[v], csc, -m_run));
            ls += pr[v];
        }
        l_run += ls;
        const uint4 p0 = pack8(pr, 0), p1 = pack8(pr, 1);
#pragma unroll
        for (int n = 0; n < MT; ++n) {
            oacc[n] = mfma(vt_operand(buf, n, 0), p0, oacc[n]);
            oacc[n] = mfma(vt_operand(buf, n, 1), p1, oacc[n]);
        }
    };

    // ---- pipeline: tile i + 1 produced while tile i is consumed; the inputs of tiles i + 2 ..
    // i + 1 + CNS in flight (stage set j % CNS holds tile j)
    St S[CNS];
#pragma unroll
    for (int u = 0; u < CNS; ++u) issue(u, S[u]);
    produce(0, S[0], 0);
    issue(CNS, S[0]);
    __syncthreads();
    expand();
    // All CNS sub-steps run on every trip (a count that is not a multiple ends with empty ones):
    // a path that skips some of the loads would make the compiler wait on later loads too.
    for (int it = 0; it < tiles; it += CNS) {
#pragma unroll
        for (int u = 0; u < CNS; ++u) {
            St &nx = S[(u + 1) % CNS];
            produce(it + u + 1, nx, (it + u + 1) & 1);
            issue(it + u + 1 + CNS, nx);
            consume(it + u, (it + u) & 1);
            __syncthreads();
        }
    }

    // ---- + (sum of cached weights) mu_t^V; normalise and store
    if (!wlive) return;
    const uint16_t *muv = static_cast<const uint16_t *>(a.mu_v) + (size_t)g * a.T * a.Dg +
                          (size_t)a.t * a.Dg + col0;
    const float lat_w = l_lat + __shfl_xor(l_lat, 32, 64);
    const float inv = 1.f / (l_run + __shfl_xor(l_run, 32, 64));
    if (iq >= qend) return;
    uint16_t *row = static_cast<uint16_t *>(a.out) + (((size_t)b * a.Pn + iq) * a.H + h) * D;
#pragma unroll
    for (int n = 0; n < MT; ++n)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = 32 * n + 8 * q4 + 4 * h2;
            float o[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] = (oacc[n][4 * q4 + c] + lat_w * bf2f(muv[d0 + c])) * inv;
            const uint2 w = make_uint2(pk_bf16(o[0], o[1]), pk_bf16(o[2], o[3]));
            *reinterpret_cast<uint2 *>(row + d0) = w;
        }
}

// One workgroup of 8 waves (two per SIMD) per (sequence, head, block of 256 queries).  Starts from
// the cached pass's state (O^T = W_up,t^V^T O_lat^T, weights and max) and runs flash attention
// over the chunk's own tiles up to each query; normalises and stores.
template <int D, int RV>
__global__ __launch_bounds__(64 * CWAVES) void prefill_chunk_kernel(PrefillArgs a) {
    using SH = PShape<D>;
    constexpr int MT = SH::MT, KS = SH::KS, KV = RV / 16;

    // operand slots per buffer: [0, KS) for the keys (sK), [KS, KS + 2 MT) for the values (sV)
    __shared__ __align__(16) uint4 sbuf[2][SH::SLOTS][kSlot];
    // W_up,t^V, staged once per workgroup
    __shared__ __align__(16) uint16_t sWv[RV * wv_stride<D>()];

    const int id = xcd_work_item(blockIdx.x, gridDim.x);
    const int qb = id % a.QB;
    const int h = (id / a.QB) % a.H;
    const int b = id / (a.QB * a.H);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h2 = lane >> 5;
    const int g = a.mode ? 0 : h;
    const int col0 = a.mode ? h * D : 0;

    int nn = a.n_new[b];
    nn = nn < 0 ? 0 : (nn > a.Pn ? a.Pn : nn);
    const int q0 = qb * CQWG;
    if (q0 >= nn) return;                               // the whole block is past the chunk
    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
    const int qend = min(nn, q0 + CQWG);                 // this block's queries: [q0, qend)
    const int wq0 = q0 + 32 * wave;                     // this wave's first query
    const bool wlive = wq0 < qend;
    const int iq = wq0 + l32;

    uint4 qop[KS];
    load_query_operands<D>(a, b, h, min(iq, nn - 1), h2, qop);

    // ---- state after the cached tokens, parked by the cached pass in lane order: the W_up,t^V
    // expansion's B operand (O_lat), the max and the weight sum, which also scales mu_t^V later.
    // The sums live in the h2 = 0 lane (both lanes are added at the end); lanes of queries past
    // the block start empty.
    float m_run = -INFINITY, l_run = 0.f, l_lat = 0.f;
    f32x16 oacc[MT];
#pragma unroll
    for (int n = 0; n < MT; ++n) oacc[n] = f32x16{};
    uint4 lop[KV];
#pragma unroll
    for (int ks = 0; ks < KV; ++ks) lop[ks] = make_uint4(0u, 0u, 0u, 0u);
    if (wlive && len > 0) {
        float2 ml = make_float2(-INFINITY, 0.f);
        if (iq < qend) {
            const uint4 *st = state_row(a, b, iq, h, D);
#pragma unroll
            for (int ks = 0; ks < KV; ++ks) lop[ks] = st[KV * h2 + ks];
            ml = *reinterpret_cast<const float2 *>(st + 2 * KV);
        }
        m_run = ml.x;
        l_run = h2 ? 0.f : ml.y;
        l_lat = l_run;
    }
    if (len > 0) stage_wv<D, RV>(a, g, col0, tid, 64 * CWAVES, sWv);
    // the cached part back in model space, from the shared W_up,t^V operands
    chunk_phase<D>(a, b, h, g, col0, nn, q0, qend, sbuf, qop, oacc, m_run, l_run, l_lat,
                   [&]() __attribute__((always_inline)) {
                       if (wlive && len > 0) {
#pragma unroll
                           for (int n = 0; n < MT; ++n)
#pragma unroll
                               for (int ks = 0; ks < KV; ++ks)
                                   oacc[n] = mfma(wv_operand<D>(sWv, n, ks, lane), lop[ks], oacc[n]);
                       }
                   });
}

// ================================================================ wide ranks: one fused kernel
// Key and value ranks above 32 ((32, 64), (64, 64), (64, 128), (96, 160)): a query's latent state
// (O_lat, r_v values) no longer fits its out row, so the cached part and the chunk part run in
// one kernel and the state stays in registers.  Same grid and waves as the two passes (8 waves of
// 32 queries per (sequence, head, block of 256 queries)), at two waves per SIMD.
//  * cached part, per 32-token tile: r_k / 16 score MFMAs S^T = C_k q'^T (A: the key latents from
//    LDS in the lane order of that operand, B: q' from registers) and 2 r_v / 32 value MFMAs into
//    the rank x query accumulators O_lat^T += C_v^T P^T.  The value latents stay token-major in
//    LDS, in blocks of 16 tokens x 32 ranks, and come back transposed through ds_read_b64_tr_b16
//    (lane (rank, h2) gets four tokens of its rank per read); the tokens are taken in the order
//    the score MFMA leaves the softmax weights in (k-step kj, element e: token
//    16 kj + 8 (e / 4) + 4 h2 + e % 4), so P^T is packed in place.
//  * then O^T = W_up,t^V^T O_lat^T (O_lat rounded once to bf16), and the chunk part as in the
//    two-pass form.
template <int RK, int RV>
struct WShape {
    static constexpr int KK = RK / 16;                 // score k-steps
    static constexpr int RT = RV / 32;                 // 32-rank tiles of O_lat^T
    static constexpr int KV = RV / 16;                 // k-steps of the expansion
    // 16-byte pieces of a 32-token tile: keys (token p % 32, ranks 8 (p / 32) ..), then values
    static constexpr int CPK = 4 * RK, CPV = 4 * RV, CP = CPK + CPV;
    static constexpr int VOFF = KK * kSlot;            // value blocks of a staged tile (uint4)
    static constexpr int TILE = VOFF + 2 * RT * 64;    // uint4 per staged tile
    static_assert(RK % 32 == 0 && RV % 32 == 0, "whole 32-rank tiles");
};

template <int D, int RK, int RV>
__global__ __launch_bounds__(64 * PWAVES) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_wide_kernel(PrefillArgs a) {
    using WS = WShape<RK, RV>;
    using SH = PShape<D>;
    constexpr int KS = D / 16, MT = D / 32, KK = WS::KK, RT = WS::RT, KV = WS::KV;
    constexpr int CP = WS::CP, CPK = WS::CPK, TILE = WS::TILE, VOFF = WS::VOFF;
    constexpr int NPS = (CP + 64 * PWAVES - 1) / (64 * PWAVES);   // pieces per thread and tile
    constexpr int CBUF = 3 * TILE, PBUF = 2 * SH::SLOTS * kSlot;
    static_assert(CQWG == QWG, "the chunk part serves the same queries");

    // one LDS array: at its start the cached staging (three tile buffers), later the chunk
    // part's two tile buffers (the cached part's reads then take immediate offsets), then the
    // W_up,t^V operands
    constexpr int CB = CBUF > PBUF ? CBUF : PBUF;
    static_assert(RV * wv_stride<D>() % 8 == 0, "whole uint4 of staged W_up,t^V");
    __shared__ __align__(16) uint4 lds[CB + RV * wv_stride<D>() / 8];
    __shared__ int sbad[PWAVES];
    uint4 *const pool = lds;
    uint16_t *const sWv = reinterpret_cast<uint16_t *>(lds + CB);

    const int id = xcd_work_item(blockIdx.x, gridDim.x);
    const int qb = id % a.QB;
    const int h = (id / a.QB) % a.H;
    const int b = id / (a.QB * a.H);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h2 = lane >> 5;
    const int g = a.mode ? 0 : h;
    const int col0 = a.mode ? h * D : 0;

    int nn = a.n_new[b];
    nn = nn < 0 ? 0 : (nn > a.Pn ? a.Pn : nn);
    const int q0 = qb * QWG;
    if (q0 >= nn) return;                               // the whole block is past the chunk
    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
    const int qend = min(nn, q0 + QWG);
    const int wq0 = q0 + 32 * wave;
    const bool wlive = wq0 < qend;
    const float csc = a.scale_log2;
    const int rd = srow(lane);

    float m_run = -INFINITY, l_run = 0.f, l_lat = 0.f;
    f32x16 oacc[MT];
#pragma unroll
    for (int n = 0; n < MT; ++n) oacc[n] = f32x16{};

    if (len > 0) {
        // ---- tile inputs.  Piece p = 64 wave + 512 x + lane of tile n (clamped to the last cached
        // tile): p < CPK is key piece (token p % 32 (clamped to the last valid token), ranks
        // 8 (p / 32) .. + 7), else value piece u = p - CPK of block u / 64 = (kj RT + rt): token
        // 16 kj + (u % 64) / 4, ranks 32 rt + 8 (u % 4) .. + 7.  CPK is a multiple of 64, so a
        // wave's pieces of one slot are all keys or all values; the page lookup is scalar.
        const int ctiles = (len + 31) >> 5;
        const uint16_t *kp = static_cast<const uint16_t *>(a.k_pool);
        const uint16_t *vp = static_cast<const uint16_t *>(a.v_pool);
        const int32_t *bt = a.block_table + (size_t)b * a.max_pages;
        const int tpp = a.P >> 5;                       // tiles per page
        const uint32_t tmag = 0xFFFFFFFFu / (uint32_t)tpp;   // tile / tpp = mulhi or one more
        struct St {
            uint4 r[NPS];
            bool bad;                                   // uniform: a page id was out of range
        };
        bool bad_w = false;
        auto slot_base = [&](int x) { return 64 * wave + 64 * PWAVES * x; };
        auto issue = [&](int n, St &st) __attribute__((always_inline)) {
            const int tile = min(n, ctiles - 1);
            uint32_t pidx = __umulhi((uint32_t)tile, tmag);
            int toff = tile - (int)pidx * tpp;
            if (toff >= tpp) {
                toff -= tpp;
                ++pidx;
            }
            int page = bt[pidx];
            const bool ok = (unsigned)page < (unsigned)a.n_pages;
            st.bad |= !ok;
            page = ok ? page : 0;
            const int row = (page * a.G + g) * a.P + 32 * toff;
            const int lim = len - 1 - 32 * tile;
#pragma unroll
            for (int x = 0; x < NPS; ++x) {
                const int sp = slot_base(x);
                if (CP % (64 * PWAVES) != 0 && sp >= CP) break;
                const int pc = sp + lane;
                const uint16_t *src;
                if (sp < CPK) {
                    src = kp + (size_t)(row + min(pc & 31, lim)) * RK + 8 * (pc >> 5);
                } else {
                    const int u = pc - CPK, bi = u >> 6, w = u & 63;
                    const int tok = 16 * (bi / RT) + (w >> 2), c8 = 4 * (bi % RT) + (w & 3);
                    src = vp + (size_t)(row + min(tok, lim)) * RV + 8 * c8;
                }
                st.r[x] = *reinterpret_cast<const uint4 *>(src);
            }
        };
        // ---- tile n's pieces into LDS tile buffer `buf` (past the last tile: a copy of it, unused).
        // Key piece (token j, ranks 8c .. 8c + 7):
        // ranks 8c + 4 hh + {0..3} are elements 4 (c % 2) .. + 3 of lane (j, hh) in k-step c / 2
        // (padded operand slots); value pieces keep their place in the 1 KB block.
        auto produce = [&](int n, St &st, int buf) __attribute__((always_inline)) {
            bad_w |= st.bad;
            st.bad = false;
            uint4 *T = pool + buf * TILE;
#pragma unroll
            for (int x = 0; x < NPS; ++x) {
                const int sp = slot_base(x);
                if (CP % (64 * PWAVES) != 0 && sp >= CP) break;
                const int pc = sp + lane;
                const uint4 w = st.r[x];
                if (sp < CPK) {
                    const int j = pc & 31, c8 = pc >> 5;
                    uint2 *d0 = reinterpret_cast<uint2 *>(&T[(c8 >> 1) * kSlot + srow(j)]) + (c8 & 1);
                    uint2 *d1 =
                        reinterpret_cast<uint2 *>(&T[(c8 >> 1) * kSlot + srow(32 + j)]) + (c8 & 1);
                    *d0 = make_uint2(w.x, w.y);
                    *d1 = make_uint2(w.z, w.w);
                } else {
                    T[VOFF + pc - CPK] = w;
                }
            }
        };

        // the first two tiles' loads go out before the set-up below
        St s0, s1;
        s0.bad = s1.bad = false;
        issue(0, s0);
        issue(1, s1);
        stage_wv<D, RV>(a, g, col0, tid, 64 * PWAVES, sWv);

        // ---- q' = c W_up,t^K q (rank x query tiles on the matrix cores; A = the W_up,t^K rows at
        // the query operand's dims, straight from memory) and c <q, mu_t^K>.  Tile rt leaves lane
        // (query, h2) ranks 32 rt + 8 (v / 4) + 4 h2 + v % 4, which packs into the score MFMA's B
        // operand (k-step ks: ranks 16 ks + 8 (e / 4) + 4 h2 + e % 4).
        uint4 qlat[KK];
        float qmu;
        {
            uint4 qop[KS];
            load_query_operands<D>(a, b, h, min(wq0 + l32, nn - 1), h2, qop);
            const uint16_t *Wk = static_cast<const uint16_t *>(a.W_up_k) +
                                 ((size_t)a.t * a.G + g) * RK * a.Dg + col0 + 4 * h2;
#pragma unroll
            for (int rt = 0; rt < RK / 32; ++rt) {
                const uint16_t *wrow = Wk + (size_t)(32 * rt + l32) * a.Dg;
                f32x16 qa = {};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint2 lo = *reinterpret_cast<const uint2 *>(wrow + 16 * ks);
                    const uint2 hi = *reinterpret_cast<const uint2 *>(wrow + 16 * ks + 8);
                    qa = mfma(make_uint4(lo.x, lo.y, hi.x, hi.y), qop[ks], qa);
                }
#pragma unroll
                for (int v = 0; v < 16; ++v) qa[v] *= csc;
                qlat[2 * rt] = pack8(qa, 0);
                qlat[2 * rt + 1] = pack8(qa, 1);
            }
            const float qm = query_dot_mu_k<D>(a, g, col0, h2, qop);
            qmu = (qm + __shfl_xor(qm, 32, 64)) * csc;
        }

        // ---- online softmax over the cached tiles (log2 domain; scores relative to c <q, mu_t^K>,
        // which is the same for every cached token and joins the reference at the end).  Lazy
        // rescale guarded by the weight sums: m_lat is the first tile's max and moves (to a tile's
        // max) only when a lane's weights of one tile sum past 2^32 (an overflowed weight
        // included); that tile's weights are then recomputed, so no weight the accumulators take
        // exceeds 2^32 and the result is exact after the final normalisation.  The sums are taken
        // from the rounded bf16 weights the value MFMAs use.
        constexpr float kSumMax = 4294967296.f;         // 2^32
        f32x16 olat[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) olat[rt] = f32x16{};
        float m_lat = 0.f, l_sum = 0.f;
        bool started = false;                           // uniform: m_lat has been set
        // transposed reads: lane (4 e' + m) of each 16-lane group addresses token 4 h2 + e' (+ 8
        // for the second read) of the block at ranks 16 ((lane / 16) % 2) + 4 m .. + 3, and lane
        // l gets rank l % 32 of those four tokens
        const uint32_t vrd =
            (uint32_t)(((4 * h2 + ((lane & 15) >> 2)) * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2);
        // move the reference to the tile's max (both lanes of a query agree); first: no history
        auto rebase = [&](const f32x16 &sc, bool first) __attribute__((always_inline)) {
            float mx = sc[0];
#pragma unroll
            for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sc[v]);
            mx = max_swap32(mx);
            if (!(mx > -INFINITY)) return;              // all masked (or NaN): keep m_lat
            if (first) {
                m_lat = mx;
                return;
            }
            if (!(mx > m_lat)) return;
            const float alpha = exp2_(m_lat - mx);
            l_sum *= alpha;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int v = 0; v < 16; ++v) olat[rt][v] *= alpha;
            m_lat = mx;
        };
        const uint32_t one2 = 0x3F803F80u;              // two bf16 ones
        auto wsum = [&](const uint4 &p0, const uint4 &p1) __attribute__((always_inline)) {
            const uint32_t w[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[i]),
                                                      __builtin_bit_cast(bf16x2, one2), acc, false);
            return acc;
        };
        // score MFMAs of the tile in buffer `buf` (raw latent scores S^T, lane (query, h2))
        auto score = [&](int buf) __attribute__((always_inline)) {
            const uint4 *T = pool + buf * TILE;
            uint4 ka[KK];
#pragma unroll
            for (int ks = 0; ks < KK; ++ks) ka[ks] = T[ks * kSlot + rd];
            f32x16 sc = {};
#pragma unroll
            for (int ks = 0; ks < KK; ++ks) sc = mfma(ka[ks], qlat[ks], sc);
            return sc;
        };
        // Tile n (buffer `buf`), whose scores `scn` holds, then the inputs of tile n + 2 (into
        // buffer `pbuf`, from stage set `st`) and the loads of tile n + 4 (into `st`).  After two
        // rare uniform branches (the last tile's mask, the first tile's reference) the step is
        // branch-free code in two parts, which the compiler schedules together (fencing each MFMA
        // between the other instructions measured 3.5 % slower at 96/160, and fencing only the
        // second part 17 % slower):
        //  1. tile n + 1's key operands and tile n's value operands from LDS, tile n + 1's score
        //     MFMAs, each followed by its share of tile n's softmax;
        //  2. tile n's value MFMAs in pairs (block kj RT + rt holds tokens 16 kj .. + 15 of ranks
        //     32 rt .. + 31), tile n + 2's LDS writes and tile n + 4's loads between them.
        // Every wave runs every step (a wave whose queries are all past the chunk computes on
        // the chunk's last query and discards the result); the score MFMAs past the last tile
        // read a stale buffer and go unused.
        f32x16 scn = {};
        auto step = [&](int n, int buf, int nbuf, int pbuf, St &st) __attribute__((always_inline)) {
            f32x16 sc = scn;
            // the last tile masks tokens past len.  Lane (query, h2), element v: token
            // 8 (v / 4) + 4 h2 + v % 4.
            const int j0 = 32 * n;
            if (j0 + 32 > len) {
                const int lm = len - 1 - j0 - 4 * h2;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (8 * (v >> 2) + (v & 3) > lm) sc[v] = -INFINITY;
            }
            if (!started) {
                rebase(sc, true);
                started = true;
            }
            // ---- region 1: tile n + 1's key operands, then tile n's value operands from LDS
            const uint4 *Tn = pool + nbuf * TILE;
            uint4 ka[KK];
#pragma unroll
            for (int ks = 0; ks < KK; ++ks) ka[ks] = Tn[ks * kSlot + rd];
            uint4 va[2 * RT];
            lds_char *vb = (lds_char *)(pool + buf * TILE + VOFF) + vrd;
#pragma unroll
            for (int i = 0; i < 2 * RT; ++i) {
                lds_char *blk = vb + 1024 * i;
                const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)blk);
                const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(blk + 512));
                va[i] = make_uint4(pk16(r0[0], r0[1]), pk16(r0[2], r0[3]), pk16(r1[0], r1[1]),
                                   pk16(r1[2], r1[3]));
            }
            // tile n + 1's score MFMAs, each followed by its share of tile n's softmax (the
            // scheduler interleaves them with the value step below: no fences)
            f32x16 s2 = {}, pr;
#pragma unroll
            for (int i = 0; i < KK; ++i) {
                s2 = mfma(ka[i], qlat[i], s2);
#pragma unroll
                for (int v = 16 * i / KK; v < 16 * (i + 1) / KK; ++v) pr[v] = exp2_(sc[v] - m_lat);
            }
            scn = s2;
            uint4 p0 = pack8(pr, 0), p1 = pack8(pr, 1);
            float ls = wsum(p0, p1);
            if (__builtin_amdgcn_ballot_w64(ls > kSumMax) != 0) {
                rebase(sc, false);
#pragma unroll
                for (int v = 0; v < 16; ++v) pr[v] = exp2_(sc[v] - m_lat);
                p0 = pack8(pr, 0);
                p1 = pack8(pr, 1);
                ls = wsum(p0, p1);
            }
            l_sum += ls;
            // ---- region 2: the value MFMAs in pairs, with tile n + 2's LDS writes and tile n + 4's
            // loads between them
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                olat[rt] = mfma(va[rt], p0, olat[rt]);
                olat[rt] = mfma(va[RT + rt], p1, olat[rt]);
                if (rt == 0) produce(n + 2, st, pbuf);
                if (rt == (RT > 2 ? 2 : RT - 1)) issue(n + 4, st);
            }
        };

        // ---- pipeline over a ring of three LDS tile buffers (tile n in buffer n % 3): tile n's
        // step writes tile n + 2 into the buffer tile n - 1 has left (one barrier per tile) and
        // loads tile n + 4 (stage set n % 2)
        produce(0, s0, 0);
        issue(2, s0);
        produce(1, s1, 1);
        issue(3, s1);
        __syncthreads();
        scn = score(0);
        int bj = 0;                                     // j % 3
        auto nx3 = [](int x) { return x == 2 ? 0 : x + 1; };
        for (int j = 0; j < ctiles; j += 2) {
            const int b1 = nx3(bj), b2 = nx3(b1);
            step(j, bj, b1, b2, s0);
            __syncthreads();
            if (j + 1 < ctiles) step(j + 1, b1, b2, nx3(b2), s1);
            __syncthreads();
            bj = b2;
        }
        // an out-of-range page id anywhere in the cached context makes the outputs NaN
        if (lane == 0) sbad[wave] = bad_w;
        __syncthreads();
        bool bad_any = false;
#pragma unroll
        for (int w = 0; w < PWAVES; ++w) bad_any |= sbad[w] != 0;

        // ---- the cached part in model space: O^T = W_up,t^V^T O_lat^T
        if (wlive) {
            uint4 lop[KV];
#pragma unroll
            for (int ks = 0; ks < KV; ++ks) lop[ks] = pack8(olat[ks >> 1], ks & 1);
#pragma unroll
            for (int n = 0; n < MT; ++n)
#pragma unroll
                for (int ks = 0; ks < KV; ++ks)
                    oacc[n] = mfma(wv_operand<D>(sWv, n, ks, lane), lop[ks], oacc[n]);
        }
        m_run = m_lat + qmu;
        l_run = bad_any ? __builtin_nanf("") : l_sum;
        l_lat = l_run;
    }

    uint4 qop[KS];
    load_query_operands<D>(a, b, h, min(wq0 + l32, nn - 1), h2, qop);
    auto &sbuf = *reinterpret_cast<uint4 (*)[2][SH::SLOTS][kSlot]>(pool);
    chunk_phase<D>(a, b, h, g, col0, nn, q0, qend, sbuf, qop, oacc, m_run, l_run, l_lat,
                   []() {});
}

template <int D, int RK, int RV>
hipError_t launch_t(const PrefillArgs &a, hipStream_t st) {
    const unsigned blocks = (unsigned)a.B * a.H * a.QB;
    hipLaunchKernelGGL((prefill_cached_kernel<D, RK, RV>), dim3(blocks), dim3(64 * PWAVES), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    PrefillArgs c = a;
    c.QB = (a.Pn + CQWG - 1) / CQWG;
    const unsigned cblocks = (unsigned)a.B * a.H * c.QB;
    hipLaunchKernelGGL((prefill_chunk_kernel<D, RV>), dim3(cblocks), dim3(64 * CWAVES), 0, st, c);
    return hipGetLastError();
}

template <int D, int RK, int RV>
hipError_t launch_wide(const PrefillArgs &a, hipStream_t st) {
    const unsigned blocks = (unsigned)a.B * a.H * a.QB;
    hipLaunchKernelGGL((prefill_wide_kernel<D, RK, RV>), dim3(blocks),
                       dim3(64 * PWAVES), 0, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs &a, hipStream_t st) {
    if (a.r_k == 16 && a.r_v == 16) return launch_t<D, 16, 16>(a, st);
    if (a.r_k == 16 && a.r_v == 32) return launch_t<D, 16, 32>(a, st);
    if (a.r_k == 32 && a.r_v == 32) return launch_t<D, 32, 32>(a, st);
    if (a.r_k == 32 && a.r_v == 64) return launch_wide<D, 32, 64>(a, st);
    if (a.r_k == 64 && a.r_v == 64) return launch_wide<D, 64, 64>(a, st);
    if (a.r_k == 64 && a.r_v == 128) return launch_wide<D, 64, 128>(a, st);
    if (a.r_k == 96 && a.r_v == 160) return launch_wide<D, 96, 160>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace

int prefill_queries_per_block() { return QWG; }

bool prefill_supported(int d, int r_k, int r_v) {
    if (d != 64 && d != 128) return false;
    return (r_k == 16 && (r_v == 16 || r_v == 32)) || (r_k == 32 && (r_v == 32 || r_v == 64)) ||
           (r_k == 64 && (r_v == 64 || r_v == 128)) || (r_k == 96 && r_v == 160);
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st) {
    const int d = a.mode ? a.Dg / a.H : a.Dg;
    if (d == 128) return launch_d<128>(a, st);
    if (d == 64) return launch_d<64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace lla
