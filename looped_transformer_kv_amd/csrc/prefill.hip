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
// attention over the given keys and values.  Both kinds share one online softmax; at the end
// O^T += W_up,t^V^T O_lat^T (one MFMA per 16 value ranks and 32-dim tile) and (sum p) mu_t^V are
// added to the chunk part's accumulators.
//
// Layout of the work: one workgroup of 8 waves (two per SIMD) per (sequence, head, block of 256
// queries); wave w owns queries [32w, 32w + 32) of the block.  Every score tile is S^T (32 tokens
// x 32 queries, v_mfma_f32_32x32x16_bf16), so each lane holds 16 scores of one query: the softmax
// row statistics need in-lane reductions and one exchange between lanes l and l ^ 32, and every
// accumulator keeps one query per lane, so the online rescale is a per-lane multiply.  Tiles are
// staged in LDS in the lane layout of the MFMA operands (cached: the latent rows and the value
// latents transposed; chunk: key and value rows); LDS is double-buffered, one barrier per tile,
// and the inputs of tile i + 2 are in flight in registers meanwhile.
// Precision: q', the latents, the chunk keys and values, the softmax weights and O_lat are bf16
// MFMA operands (the precision class of a bf16 KV cache in a flash-attention kernel); scores,
// statistics and accumulators are fp32; out is rounded once (RNE).
#include "lla_internal.h"

namespace lla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// two fp32 -> two bf16 (round to nearest even), lo in the low half
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
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

constexpr int PWAVES = 8;                  // waves per workgroup (two per SIMD)
constexpr int QWG = PWAVES * 32;           // queries per workgroup: one 32-query tile per wave

template <int D, int RK, int RV>
struct PShape {
    static constexpr int MT = D / 32;                  // 32-wide tiles of the head dim
    static constexpr int KS = D / 16;                  // k-steps of a full-width score MFMA
    static constexpr int KK = RK / 16, KV = RV / 16;   // k-steps over the key / value ranks
    // 16-byte latent pieces (8 ranks of one token) of a cached tile: key pieces, then value pieces
    static constexpr int CPK = 32 * RK / 8, CPV = 32 * RV / 8, CP = CPK + CPV;
    // 16-byte pieces of a 32-token chunk tile per axis (32 rows x D / 8), per thread
    static constexpr int PIECES = 32 * D / 8;
    static constexpr int NEWP = (PIECES + 64 * PWAVES - 1) / (64 * PWAVES);
    static constexpr int NST = 2 * NEWP;               // stage registers per thread
    static constexpr int SLOTS = KS + 2 * MT;          // 1 KB operand slots per LDS buffer
    static_assert(CP <= 64 * PWAVES, "one latent piece per thread");
    static_assert(KK + 2 <= SLOTS, "cached operands fit a buffer");
    static_assert(MT == 2 || MT == 4, "head dim 64 or 128");
    static_assert(RK <= 32 && RV <= 32, "one 32-row MFMA tile of latent ranks");
};

// Registers holding one tile's inputs while they are in flight: for a cached tile the thread's
// latent piece (slot 0; threads past the pieces load a duplicate), for a chunk tile its 16-byte
// pieces of the chunk rows (key pieces, then value pieces).  Every slot is one unconditional
// 16-byte load whose address is chosen by the tile's kind, so the registers stay registers.
template <int N>
struct Stage {
    uint4 r[N];
    bool bad;                                // a cached tile whose page id is out of range
};

template <int D, int RK, int RV>
__global__ __launch_bounds__(64 * PWAVES) void prefill_kernel(PrefillArgs a) {
    using SH = PShape<D, RK, RV>;
    constexpr int MT = SH::MT, KS = SH::KS, KK = SH::KK, KV = SH::KV;
    constexpr int NEWP = SH::NEWP, NST = SH::NST;
    using St = Stage<NST>;

    // operand slots per buffer: a chunk tile uses [0, KS) for the keys (sK) and [KS, KS + 2 MT)
    // for the values (sV); a cached tile uses [0, KK) for the key latents and [KK, KK + 2) for the
    // value latents transposed
    __shared__ __align__(16) uint4 sbuf[2][SH::SLOTS][64];
    // each wave's query operands: used at set-up and by the few chunk tiles, so they wait in LDS
    // rather than in registers
    __shared__ __align__(16) uint4 sQ[PWAVES][KS][64];
    __shared__ int sBad[2];

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
    const int qend = min(nn, q0 + QWG);                 // this block's queries: [q0, qend)
    const int ctiles = (len + 31) >> 5;                 // cached tiles
    const int tiles = ctiles + ((qend + 31) >> 5);      // then chunk tiles up to the last query
    const int wq0 = q0 + 32 * wave;                     // this wave's first query
    const bool wlive = wq0 < qend;
    const float csc = a.scale_log2;

    const uint16_t *qp = static_cast<const uint16_t *>(a.q);
    const uint16_t *kp = static_cast<const uint16_t *>(a.k_pool);
    const uint16_t *vp = static_cast<const uint16_t *>(a.v_pool);
    const uint16_t *kn = static_cast<const uint16_t *>(a.k_new);
    const uint16_t *vn = static_cast<const uint16_t *>(a.v_new);
    const int32_t *bt = a.block_table + (size_t)b * a.max_pages;

    // ---- query operands (B of the full-width score MFMA): lane (l32, h2) holds query row
    // wq0 + l32, k-step ks covers dims 32 (ks / 2) + 16 (ks % 2) + 4 h2 + {0..3} and + 8 + {0..3}
    // (a permutation of the head dims that the chunk keys' layout shares).  Rows past the chunk
    // read the last valid row (their results are not stored).
    uint4 qop[KS];                                      // set-up only; then in sQ
    const int qrow = min(wq0 + l32, nn - 1);
    {
        const uint16_t *row = qp + (((size_t)b * a.Pn + qrow) * a.H + h) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = 32 * (ks >> 1) + 16 * (ks & 1) + 4 * h2;
            const uint2 lo = *reinterpret_cast<const uint2 *>(row + d0);
            const uint2 hi = *reinterpret_cast<const uint2 *>(row + d0 + 8);
            qop[ks] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
    }
    auto qdim = [&](int ks, int e) { return 32 * (ks >> 1) + 16 * (ks & 1) + 4 * h2 + (e < 4 ? e : e + 4); };

    // ---- q' = c W_up,t^K q for this wave's queries, on the matrix cores: q'^T = W q^T with
    // A = W_up,t^K (lane (rank l32, h2): the rank's row at the query operand's dims; ranks past
    // RK are zero), B = the query operands.  Lane (query, h2) gets ranks 8 (v / 4) + 4 h2 + v % 4,
    // which packs straight into the B operand of the cached score MFMA (k-step ks: ranks
    // 16 ks + 8 (e / 4) + 4 h2 + e % 4 at element e).  q mu_t^K (scaled) is one in-lane dot over
    // this lane's half of the dims plus an exchange.
    uint4 qlat[KK];
    float qmu;
    {
        const uint16_t *Wk = static_cast<const uint16_t *>(a.W_up_k) +
                             ((size_t)a.t * a.G + g) * RK * a.Dg + col0;
        const uint16_t *muk = static_cast<const uint16_t *>(a.mu_k) + (size_t)g * a.T * a.Dg +
                              (size_t)a.t * a.Dg + col0;
        const int rk = min(l32, RK - 1);
        f32x16 qa = {};
        float qm = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint16_t w[8];
            const uint32_t qv[4] = {qop[ks].x, qop[ks].y, qop[ks].z, qop[ks].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int dim = qdim(ks, e);
                w[e] = l32 < RK ? Wk[(size_t)rk * a.Dg + dim] : (uint16_t)0;
                qm += bf2f(static_cast<uint16_t>(qv[e >> 1] >> (16 * (e & 1)))) * bf2f(muk[dim]);
            }
            const uint4 wop = make_uint4(w[0] | (uint32_t)w[1] << 16, w[2] | (uint32_t)w[3] << 16,
                                         w[4] | (uint32_t)w[5] << 16, w[6] | (uint32_t)w[7] << 16);
            qa = mfma(wop, qop[ks], qa);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) qa[v] *= csc;
#pragma unroll
        for (int ks = 0; ks < KK; ++ks) qlat[ks] = pack8(qa, ks);
        qmu = (qm + __shfl_xor(qm, 32, 64)) * csc;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sQ[wave][ks][lane] = qop[ks];   // read by chunk tiles
    }

    // ---- tile inputs.  Cached tile c: piece p = tid < CP is (token 32c + p / (R / 8), clamped to
    // the last valid token; ranks 8 (p % (R / 8)) .. + 7) of c_k (p < CPK) or c_v, in one page
    // (P is a multiple of 32).  Chunk tile n: piece p = tid + 512 x of each axis is row
    // 32n + p / (D / 8) (clamped to the last valid row), dims 8 (p % (D / 8)) .. + 7; slots
    // [0, NEWP) hold key pieces, [NEWP, 2 NEWP) value pieces.  Addresses are a per-thread constant
    // plus a per-tile scalar.
    const int cp = min(tid, SH::CP - 1);
    const bool ckey = cp < SH::CPK;
    const int cR = ckey ? RK : RV;
    const int cpi = ckey ? cp : cp - SH::CPK;
    const int ctok = cpi / (cR / 8), crank = 8 * (cpi % (cR / 8));
    const uint16_t *cbase = (ckey ? kp : vp) + (size_t)g * a.P * cR + crank;
    const size_t cpage = (size_t)a.G * a.P * cR;
    int pc_row[NST], pc_col[NST];                       // chunk piece of each stage slot
#pragma unroll
    for (int x = 0; x < NST; ++x) {
        const int pc = min(tid + 64 * PWAVES * (x % NEWP), SH::PIECES - 1);
        pc_row[x] = pc / (D / 8);
        pc_col[x] = 8 * (pc % (D / 8));
    }
    const uint16_t *kn_b = kn + (size_t)b * a.Pn * a.new_stride + (size_t)h * D;
    const uint16_t *vn_b = vn + (size_t)b * a.Pn * a.new_stride + (size_t)h * D;
    auto issue = [&](int tile, St &st) __attribute__((always_inline)) {
        tile = min(tile, tiles - 1);
        const bool cached = tile < ctiles;
        int page = bt[min((32 * tile) / a.P, a.max_pages - 1)];
        st.bad = cached && (unsigned)page >= (unsigned)a.n_pages;
        page = (unsigned)page < (unsigned)a.n_pages ? page : 0;
        const uint16_t *lat = cbase + page * cpage +
                              (size_t)((32 * tile) % a.P + min(ctok, max(len - 1 - 32 * tile, 0))) * cR;
        // chunk: rows 32n + r, clamped to the last valid row
        const int n0 = 32 * (tile - ctiles);
        const int rmax = nn - 1 - n0;
#pragma unroll
        for (int x = 0; x < NST; ++x) {
            const uint16_t *chk = (x < NEWP ? kn_b : vn_b) +
                                  (uint32_t)((n0 + min(pc_row[x], rmax)) * (int)a.new_stride +
                                             pc_col[x]);
            st.r[x] = *reinterpret_cast<const uint4 *>(cached ? lat : chk);
        }
    };

    // ---- write tile `tile` into LDS buffer `buf` in operand layout
    auto produce = [&](int tile, const St &st, int buf) __attribute__((always_inline)) {
        if (tile >= tiles) return;
        if (tile < ctiles) {
            if (tid == 0) sBad[buf] = st.bad;
            if (tid >= SH::CP) return;
            const uint4 w = st.r[0];
            if (ckey) {
                // A operand of the cached score MFMA, lane (token, h2) of k-step ks: ranks
                // 16 ks + 8 (e / 4) + 4 h2 + e % 4 at element e.  Ranks 8 p' .. + 3 of this piece
                // go to lane (ctok, 0), + 4 .. + 7 to lane (ctok, 1), elements 4 (p' % 2) .. + 3,
                // k-step p' / 2 (p' = crank / 8).
                const int pq = crank >> 3;
                uint2 *d0 = reinterpret_cast<uint2 *>(&sbuf[buf][pq >> 1][ctok]) + (pq & 1);
                uint2 *d1 = reinterpret_cast<uint2 *>(&sbuf[buf][pq >> 1][32 + ctok]) + (pq & 1);
                *d0 = make_uint2(w.x, w.y);
                *d1 = make_uint2(w.z, w.w);
            } else {
                // A operand of the value MFMA, lane (rank, h2) of token k-step kj: tokens
                // 16 kj + 8 (e / 4) + 4 h2 + e % 4 at element e
                const int kj = ctok >> 4, rem = ctok & 15;
                const int hh = (rem >> 2) & 1, e = 4 * (rem >> 3) + (rem & 3);
                const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int y = 0; y < 8; ++y) {
                    uint16_t *dst = reinterpret_cast<uint16_t *>(
                        &sbuf[buf][KK + kj][32 * hh + crank + y]);
                    dst[e] = static_cast<uint16_t>(wd[y >> 1] >> (16 * (y & 1)));
                }
            }
        } else {
            // key piece (row jr, dims 8c .. 8c + 7): dims 8c + 4 hh + {0..3} are elements
            // 4 (c % 2) .. + 3 of lane 32 hh + jr in k-step 2 (c / 4) + (c / 2) % 2
#pragma unroll
            for (int x = 0; x < NEWP; ++x) {
                const int pc = tid + 64 * PWAVES * x;
                if (SH::PIECES % (64 * PWAVES) != 0 && pc >= SH::PIECES) break;
                const int jr = pc / (D / 8), c8 = pc % (D / 8);
                const int ks = 2 * (c8 >> 2) + ((c8 >> 1) & 1);
                const uint4 w = st.r[x];
                uint2 *d0 = reinterpret_cast<uint2 *>(&sbuf[buf][ks][jr]) + (c8 & 1);
                uint2 *d1 = reinterpret_cast<uint2 *>(&sbuf[buf][ks][32 + jr]) + (c8 & 1);
                *d0 = make_uint2(w.x, w.y);
                *d1 = make_uint2(w.z, w.w);
            }
            // value piece (row jr, dims 8p .. 8p + 7) -> the V^T operand of each dim: lane
            // (dim % 32, h2) of slot KS + 2 (dim / 32) + jr / 16 holds tokens 16 kj + 8 (e / 4) +
            // 4 h2 + e % 4 at element e
#pragma unroll
            for (int x = 0; x < NEWP; ++x) {
                const int pc = tid + 64 * PWAVES * x;
                if (SH::PIECES % (64 * PWAVES) != 0 && pc >= SH::PIECES) break;
                const int jr = pc / (D / 8), p8 = 8 * (pc % (D / 8));
                const int kj = jr >> 4, rem = jr & 15;
                const int hh = (rem >> 2) & 1, e = 4 * (rem >> 3) + (rem & 3);
                const uint4 w = st.r[NEWP + x];
                const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int y = 0; y < 8; ++y) {
                    const int dim = p8 + y;
                    uint16_t *dst = reinterpret_cast<uint16_t *>(
                        &sbuf[buf][KS + 2 * (dim >> 5) + kj][32 * hh + (dim & 31)]);
                    dst[e] = static_cast<uint16_t>(wd[y >> 1] >> (16 * (y & 1)));
                }
            }
        }
    };

    // ---- online softmax state of this wave's 32 queries (log2 domain): total and cached weight
    // sums, O^T accumulators per 32-dim tile (chunk values, later the reconstructed cached part)
    // and the latent accumulator O_lat^T (rank x query)
    float m_run = -INFINITY, l_run = 0.f, l_lat = 0.f;
    f32x16 oacc[MT], olat = {};
#pragma unroll
    for (int n = 0; n < MT; ++n) oacc[n] = f32x16{};

    // Cached scores leave the MFMA already scaled (q' carries c) and need + c q mu_t^K; chunk
    // scores are raw q . k and need * c: either way p = 2^(s scl + bias - m) is one FMA and one
    // exp2.  Lazy rescale: the accumulators are rescaled only when a lane's max grows by more
    // than kSlack (p <= 2^kSlack meanwhile, exact after the final normalisation by l).
    constexpr float kSlack = 8.f;
    const int wlast = min(wq0 + 31, qend - 1);          // this wave's last query

    auto consume = [&](int tile, int buf) __attribute__((always_inline)) {
        if (!wlive || tile >= tiles) return;
        const bool cached = tile < ctiles;
        const int j0 = cached ? 32 * tile : 32 * (tile - ctiles);
        if (!cached && j0 > wlast) return;                  // every token is after every query
        f32x16 sc = {};
        float scl, bias;
        if (cached) {
#pragma unroll
            for (int ks = 0; ks < KK; ++ks) sc = mfma(sbuf[buf][ks][lane], qlat[ks], sc);
            if (sBad[buf]) {
#pragma unroll
                for (int v = 0; v < 16; ++v) sc[v] = __builtin_nanf("");
            }
            scl = 1.f;
            bias = qmu;
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sc = mfma(sbuf[buf][ks][lane], sQ[wave][ks][lane], sc);
            scl = csc;
            bias = 0.f;
        }
        // edge tiles mask some score: the cached context's last tile, chunk tiles that reach past
        // this wave's first query.  Lane (query, h2), element v: token 8 (v / 4) + 4 h2 + v % 4.
        if (cached ? j0 + 32 > len : j0 + 31 > wq0) {
            const int lim = cached ? len - 1 - j0 : wq0 + l32 - j0;   // last visible token
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if (8 * (v >> 2) + 4 * h2 + (v & 3) > lim) sc[v] = -INFINITY;
        }
        float mx = sc[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sc[v]);
        mx = fmaf(max_swap32(mx), scl, bias);
        const float m_cand = fmaxf(m_run, mx);
        if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kSlack) != 0) {
            const float alpha = m_cand == -INFINITY ? 1.f : exp2_(m_run - m_cand);
            l_run *= alpha;
            l_lat *= alpha;
#pragma unroll
            for (int n = 0; n < MT; ++n)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[n][v] *= alpha;
#pragma unroll
            for (int v = 0; v < 16; ++v) olat[v] *= alpha;
            m_run = m_cand;
        }
        // softmax weights as the two bf16 B operands of the value MFMAs
        const float nb = bias - m_run;
        f32x16 pr;
        float ls = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            pr[v] = exp2_(fmaf(sc[v], scl, nb));
            ls += pr[v];
        }
        l_run += ls;
        const uint4 p0 = pack8(pr, 0), p1 = pack8(pr, 1);
        if (cached) {
            l_lat += ls;
            olat = mfma(sbuf[buf][KK][lane], p0, olat);
            olat = mfma(sbuf[buf][KK + 1][lane], p1, olat);
        } else {
            // (the value operands are read only now: a chunk tile is rare, registers are not)
#pragma unroll
            for (int n = 0; n < MT; ++n) {
                oacc[n] = mfma(sbuf[buf][KS + 2 * n][lane], p0, oacc[n]);
                oacc[n] = mfma(sbuf[buf][KS + 2 * n + 1][lane], p1, oacc[n]);
            }
        }
    };

    // ---- pipeline: tile i + 1 produced while tile i is consumed; tile i + 2's inputs in flight
    St s0, s1;
    issue(0, s0);
    issue(1, s1);
    produce(0, s0, 0);
    issue(2, s0);
    __syncthreads();
    auto step = [&](int it, St &next) __attribute__((always_inline)) {
        produce(it + 1, next, (it + 1) & 1);
        issue(it + 3, next);
        consume(it, it & 1);
        __syncthreads();
    };
    // Both half-steps run on every trip (an odd count ends with an empty step): a path that skips
    // the second half's loads would make the compiler wait on loads issued one step earlier
    // instead of two.
    for (int it = 0; it < tiles; it += 2) {
        step(it, s1);
        step(it + 1, s0);
    }

    // ---- the cached part back in model space: O^T += W_up,t^V^T O_lat^T (A: lane (dim, h2) of
    // 32-dim tile n holds the dim's column at ranks 16 ks + 8 (e / 4) + 4 h2 + e % 4, the order
    // O_lat's lanes pack in), then + (sum of cached weights) mu_t^V; normalise and store.
    if (!wlive) return;
    const uint16_t *Wv = static_cast<const uint16_t *>(a.W_up_v) +
                         ((size_t)a.t * a.G + g) * RV * a.Dg + col0;
    const uint16_t *muv = static_cast<const uint16_t *>(a.mu_v) + (size_t)g * a.T * a.Dg +
                          (size_t)a.t * a.Dg + col0;
    uint4 lop[KV];
#pragma unroll
    for (int ks = 0; ks < KV; ++ks) lop[ks] = pack8(olat, ks);
#pragma unroll
    for (int n = 0; n < MT; ++n) {
#pragma unroll
        for (int ks = 0; ks < KV; ++ks) {
            uint16_t w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                w[e] = Wv[(size_t)(16 * ks + 8 * (e >> 2) + 4 * h2 + (e & 3)) * a.Dg + 32 * n + l32];
            const uint4 wop = make_uint4(w[0] | (uint32_t)w[1] << 16, w[2] | (uint32_t)w[3] << 16,
                                         w[4] | (uint32_t)w[5] << 16, w[6] | (uint32_t)w[7] << 16);
            oacc[n] = mfma(wop, lop[ks], oacc[n]);
        }
    }
    const float lat_w = l_lat + __shfl_xor(l_lat, 32, 64);
    const float inv = 1.f / (l_run + __shfl_xor(l_run, 32, 64));
    const int iq = wq0 + l32;
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

template <int D, int RK, int RV>
hipError_t launch_t(const PrefillArgs &a, hipStream_t st) {
    const unsigned blocks = (unsigned)a.B * a.H * a.QB;
    hipLaunchKernelGGL((prefill_kernel<D, RK, RV>), dim3(blocks), dim3(64 * PWAVES), 0, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs &a, hipStream_t st) {
    if (a.r_k == 16 && a.r_v == 16) return launch_t<D, 16, 16>(a, st);
    if (a.r_k == 16 && a.r_v == 32) return launch_t<D, 16, 32>(a, st);
    if (a.r_k == 32 && a.r_v == 32) return launch_t<D, 32, 32>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace

int prefill_queries_per_block() { return QWG; }

bool prefill_supported(int d, int r_k, int r_v) {
    if (d != 64 && d != 128) return false;
    return (r_k == 16 && (r_v == 16 || r_v == 32)) || (r_k == 32 && r_v == 32);
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st) {
    const int d = a.mode ? a.Dg / a.H : a.Dg;
    if (d == 128) return launch_d<128>(a, st);
    if (d == 64) return launch_d<64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace lla
