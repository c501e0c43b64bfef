// prefill.hip -- chunked prefill attention over the latent cache, bf16 storage, gfx950 MFMA.
//
// A chunk of new tokens per sequence attends, for loop t, to the cached context through the codec
// (pith.science paper page for "Looped Latent Attention", "What carries the argument":
// x_hat_t = c W_up,t + mu_t, attention unchanged) and causally to the chunk's own loop-t keys and
// values, which are taken as given (they are encoded only after the last loop, like the decode
// step's own token).  New token i of sequence b sees cached j < seq_lens[b] and new i' <= i.
//
// This is flash attention whose K/V tiles are rebuilt from latents on the matrix cores:
//   K_hat tile (32 tokens x d) = c_k W_up,t^K + mu_t^K,   V_hat tile = c_v W_up,t^V + mu_t^V,
// each expanded once per workgroup and shared by all its queries, so the d x r expansion of a
// cached token is amortised over up to 256 queries.
//
// Layout of the work: one workgroup of 8 waves (two per SIMD) per (sequence, head, block of 256
// queries); wave w owns queries [32w, 32w + 32) of the block.  Per 32-token tile:
//   * the waves split the expansion (key tile w or value tile w - 4: one MFMA chain each, mu_t
//     entering exactly as one more k-step) and store the bf16 results in LDS directly in the lane
//     layout of the attention MFMAs' operands;
//     chunk tiles are copied into the same layout from the caller's rows;
//   * every wave computes S^T = K_hat Q^T (32 tokens x 32 queries per query tile, v_mfma 32x32x16,
//     K from LDS, Q^T in registers), so each lane holds 16 scores of one query: the softmax row
//     statistics need in-lane reductions and one exchange between lanes l and l ^ 32;
//   * P^T (bf16) is the B operand of O^T = V_hat^T P^T, whose lanes again hold one query each, so
//     the online-softmax rescale is a per-lane multiply.
// The head-dim order inside a k-step is permuted (the order the key expansion leaves in a lane);
// the query operand uses the same permutation, which leaves every dot product unchanged.
// LDS is double-buffered: tile i + 1 is produced while tile i is consumed, one barrier per tile;
// the latents (or chunk rows) of tile i + 2 are in flight in registers meanwhile.
// Precision: K_hat, V_hat and the softmax weights are rounded to bf16 for the MFMAs (the
// precision of a bf16 KV cache in a flash-attention kernel); scores, statistics and the output
// accumulate in fp32; out is rounded once (RNE).
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
    static constexpr int KS = D / 16;                  // k-steps of the score MFMA
    static constexpr int KK = RK / 16, KV = RV / 16;   // k-steps of the expansions
    static constexpr int KMAX = KK > KV ? KK : KV;    // k-steps of this wave's expansion job
    // 16-byte pieces of a 32-token chunk tile per axis (32 rows x D / 8), per thread
    static constexpr int PIECES = 32 * D / 8;
    static constexpr int NEWP = (PIECES + 64 * PWAVES - 1) / (64 * PWAVES);
    // stage registers per thread: the latent slices of its wave's job (a cached tile) or its
    // pieces of both axes (a chunk tile)
    static constexpr int NST = KMAX > 2 * NEWP ? KMAX : 2 * NEWP;
    static_assert(2 * MT <= PWAVES, "one expansion job per wave");
    static_assert(MT == 2 || MT == 4, "head dim 64 or 128");
};

// Registers holding one tile's inputs while they are in flight: for a cached tile the lane's
// latent slices (k-steps of c_k, then of c_v), for a chunk tile the thread's 16-byte pieces of the
// chunk rows (key pieces, then value pieces).  Every slot is one unconditional 16-byte load whose
// address is chosen by the tile's kind, so the registers stay registers.
template <int N>
struct Stage {
    uint4 r[N];
};

template <int D, int RK, int RV>
__global__ __launch_bounds__(64 * PWAVES) void prefill_kernel(PrefillArgs a) {
    using SH = PShape<D, RK, RV>;
    constexpr int MT = SH::MT, KS = SH::KS, KK = SH::KK, KV = SH::KV, KMAX = SH::KMAX;
    constexpr int NEWP = SH::NEWP, NST = SH::NST;
    using St = Stage<NST>;

    // operand tiles: sK[buf][k-step][lane], sV[buf][2N + kj][lane] (16 bytes each)
    __shared__ __align__(16) uint4 sK[2][KS][64];
    __shared__ __align__(16) uint4 sV[2][2 * MT][64];

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

    const uint16_t *qp = static_cast<const uint16_t *>(a.q);
    const uint16_t *kp = static_cast<const uint16_t *>(a.k_pool);
    const uint16_t *vp = static_cast<const uint16_t *>(a.v_pool);
    const uint16_t *kn = static_cast<const uint16_t *>(a.k_new);
    const uint16_t *vn = static_cast<const uint16_t *>(a.v_new);
    const int32_t *bt = a.block_table + (size_t)b * a.max_pages;

    // ---- this wave's expansion job: key tile `jt` (job < MT) or value tile `jt` (MT <= job < 2MT);
    // waves 2MT.. have none.  Both kinds take their W_up,t operand with the same lane layout:
    // lane (l32, h2) holds column col0 + 32 jt + l32 at ranks 16 ks + 8 h2 .. + 7 (the A operand
    // W^T of the key expansion, the B operand W of the value expansion).
    const int job = wave;
    const bool kjob = job < MT, vjob = job >= MT && job < 2 * MT;
    const int jt = kjob ? job : (vjob ? job - MT : 0);
    const int RJ = kjob ? RK : RV;
    const uint16_t *Wj = static_cast<const uint16_t *>(kjob ? a.W_up_k : a.W_up_v) +
                         ((size_t)a.t * a.G + g) * RJ * a.Dg + col0 + 32 * jt + l32;
    uint4 wj[KMAX];
#pragma unroll
    for (int ks = 0; ks < KMAX; ++ks) {
        const int k0 = min(16 * ks, RJ - 16) + 8 * h2;      // k-steps past RJ are unused
        uint16_t e[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) e[x] = Wj[(size_t)(k0 + x) * a.Dg];
        wj[ks] = make_uint4(e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16,
                            e[4] | (uint32_t)e[5] << 16, e[6] | (uint32_t)e[7] << 16);
    }
    // mu_t enters the expansion exactly through one more MFMA k-step: a key tile adds the mu row
    // (A, k-slot 0 of lanes h2 = 0: mu at this lane's dim) times a row of ones (B); a value tile
    // adds a column of ones (A) times the mu row (B).
    const uint16_t *muj = static_cast<const uint16_t *>(kjob ? a.mu_k : a.mu_v) +
                          (size_t)g * a.T * a.Dg + (size_t)a.t * a.Dg + col0 + 32 * jt + l32;
    const uint32_t mu_bits = h2 == 0 ? *muj : 0u;
    const uint4 mu_op = make_uint4(mu_bits, 0, 0, 0);
    const uint4 one_op = make_uint4(h2 == 0 ? 0x3F80u : 0u, 0, 0, 0);

    // ---- query operands (B of the score MFMA): lane (l32, h2) holds query row wq0 + 32u + l32,
    // k-step ks covers dims 32 (ks / 2) + 16 (ks % 2) + 4 h2 + {0..3} and + 8 + {0..3}.  Rows past
    // the chunk read the last valid row (their results are not stored).
    uint4 qop[KS];
    {
        const int i = min(wq0 + l32, nn - 1);
        const uint16_t *row = qp + (((size_t)b * a.Pn + i) * a.H + h) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = 32 * (ks >> 1) + 16 * (ks & 1) + 4 * h2;
            const uint2 lo = *reinterpret_cast<const uint2 *>(row + d0);
            const uint2 hi = *reinterpret_cast<const uint2 *>(row + d0 + 8);
            qop[ks] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
    }

    // ---- tile inputs.  Cached tile c: this wave's job's latents (c_k for a key job, c_v for a
    // value job) of token 32c + l32 (the last valid token past the end), in one page (P is a
    // multiple of 32); an out-of-range page id poisons the tile with NaN.  Chunk tile n: piece
    // p = tid + 512 x of each axis is row 32n + p / (D / 8) (clamped to the last valid row),
    // dims 8 (p % (D / 8)) .. + 7; slots [0, NEWP) hold key pieces, [NEWP, 2 NEWP) value pieces.
    // Addresses are a per-lane constant plus a per-tile scalar: a cached tile lies in one page at
    // slot (32c) % P, and a chunk piece's row offset inside its tile is fixed per thread.
    const uint16_t *pool_j = (kjob ? kp : vp) + (size_t)g * a.P * RJ + 8 * h2;
    const size_t page_elems = (size_t)a.G * a.P * RJ;
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
        // cached: token 32 tile + min(l32, last valid) in page bt[32 tile / P]
        int page = bt[min((32 * tile) / a.P, a.max_pages - 1)];
        page = (unsigned)page < (unsigned)a.n_pages ? page : 0;
        const uint16_t *lat = pool_j + page * page_elems +
                              (size_t)((32 * tile) % a.P + min(l32, max(len - 1 - 32 * tile, 0))) *
                                  RJ;
        // chunk: rows 32n + r, clamped to the last valid row
        const int n0 = 32 * (tile - ctiles);
        const int rmax = nn - 1 - n0;
#pragma unroll
        for (int x = 0; x < NST; ++x) {
            const uint16_t *chk = (x < NEWP ? kn_b : vn_b) +
                                  (uint32_t)((n0 + min(pc_row[x], rmax)) * (int)a.new_stride +
                                             pc_col[x]);
            const uint16_t *l = lat + min(16 * x, RJ - 16);
            st.r[x] = *reinterpret_cast<const uint4 *>(cached ? l : chk);
        }
    };

    // ---- write tile `tile` into LDS buffer `buf` in operand layout
    auto produce = [&](int tile, const St &st, int buf) __attribute__((always_inline)) {
        if (tile >= tiles) return;
        if (tile < ctiles) {
            // an out-of-range page id poisons the tile: mu becomes NaN (bf16 0x7FC0), which the
            // mu k-step spreads to every element
            const bool bad = (unsigned)bt[(32 * tile) / a.P] >= (unsigned)a.n_pages;
            const uint4 mu_t = make_uint4(bad && h2 == 0 ? 0x7FC0u : mu_op.x, 0, 0, 0);
            if (kjob) {
                // K_hat^T tile jt: D[m = dim][n = token]; lane (token l32, h2) gets dims
                // 32 jt + 8 (v / 4) + 4 h2 + v % 4, i.e. k-steps 2 jt (v < 8) and 2 jt + 1
                f32x16 acc = mfma(mu_t, one_op, f32x16{});
#pragma unroll
                for (int ks = 0; ks < KK; ++ks) acc = mfma(wj[ks], st.r[ks], acc);
                sK[buf][2 * jt][lane] = pack8(acc, 0);
                sK[buf][2 * jt + 1][lane] = pack8(acc, 1);
            } else if (vjob) {
                // V_hat tile jt: D[m = token][n = dim]; lane (dim l32, h2) gets tokens
                // 8 (v / 4) + 4 h2 + v % 4: token k-steps 0 (v < 8) and 1
                f32x16 acc = mfma(one_op, mu_t, f32x16{});
#pragma unroll
                for (int ks = 0; ks < KV; ++ks) acc = mfma(st.r[ks], wj[ks], acc);
                sV[buf][2 * jt][lane] = pack8(acc, 0);
                sV[buf][2 * jt + 1][lane] = pack8(acc, 1);
            }
        } else {
            // key piece (row jt, dims 8c .. 8c + 7): dims 8c + 4 hh + {0..3} are elements
            // 4 (c % 2) .. + 3 of lane 32 hh + jt in k-step 2 (c / 4) + (c / 2) % 2
#pragma unroll
            for (int x = 0; x < NEWP; ++x) {
                const int pc = tid + 64 * PWAVES * x;
                if (SH::PIECES % (64 * PWAVES) != 0 && pc >= SH::PIECES) break;
                const int jr = pc / (D / 8), c8 = pc % (D / 8);
                const int ks = 2 * (c8 >> 2) + ((c8 >> 1) & 1);
                const uint4 w = st.r[x];
                uint2 *d0 = reinterpret_cast<uint2 *>(&sK[buf][ks][jr]) + (c8 & 1);
                uint2 *d1 = reinterpret_cast<uint2 *>(&sK[buf][ks][32 + jr]) + (c8 & 1);
                *d0 = make_uint2(w.x, w.y);
                *d1 = make_uint2(w.z, w.w);
            }
            // value piece (row jt, dims 8p .. 8p + 7) -> the V^T operand of each dim: lane
            // (dim % 32, h2) of slot 2 (dim / 32) + jt / 16 holds tokens 16 kj + 8 (e / 4) + 4 h2 +
            // e % 4 at element e
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
                        &sV[buf][2 * (dim >> 5) + kj][32 * hh + (dim & 31)]);
                    dst[e] = static_cast<uint16_t>(wd[y >> 1] >> (16 * (y & 1)));
                }
            }
        }
    };

    // ---- online softmax state of this wave's 32 queries (log2 domain); O^T accumulators per
    // 32-dim tile
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 oacc[MT];
#pragma unroll
    for (int n = 0; n < MT; ++n) oacc[n] = f32x16{};

    // Scores stay raw (q . k) until the exponent: p = 2^(s c - m) with c = scale log2(e) is one FMA
    // and one exp2 per score; the running max m is kept in the scaled log2 domain.  Lazy rescale:
    // the accumulators are rescaled only when a lane's max grows by more than kSlack (p <= 2^kSlack
    // meanwhile, exact after the final normalisation by l).
    constexpr float kSlack = 8.f;
    const float csc = a.scale_log2;
    const int wlast = min(wq0 + 31, qend - 1);          // this wave's last query

    auto consume = [&](int tile, int buf) __attribute__((always_inline)) {
        if (!wlive) return;
        const bool cached = tile < ctiles;
        const int j0 = cached ? 32 * tile : 32 * (tile - ctiles);
        if (!cached && j0 > wlast) return;                  // every token is after every query
        uint4 kop[KS], vop[2 * MT];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kop[ks] = sK[buf][ks][lane];
        f32x16 sc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sc = mfma(kop[ks], qop[ks], sc);
        // the value operands take the key operands' registers
#pragma unroll
        for (int x = 0; x < 2 * MT; ++x) vop[x] = sV[buf][x][lane];
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
        mx = max_swap32(mx) * csc;
        const float m_cand = fmaxf(m_run, mx);
        if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kSlack) != 0) {
            const float alpha = m_cand == -INFINITY ? 1.f : exp2_(m_run - m_cand);
            l_run *= alpha;
#pragma unroll
            for (int n = 0; n < MT; ++n)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[n][v] *= alpha;
            m_run = m_cand;
        }
        // softmax weights as the two bf16 B operands of the value MFMAs
        const float nm = -m_run;
        f32x16 pr;
        float ls = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            pr[v] = exp2_(fmaf(sc[v], csc, nm));
            ls += pr[v];
        }
        l_run += ls;
        const uint4 p0 = pack8(pr, 0), p1 = pack8(pr, 1);
#pragma unroll
        for (int n = 0; n < MT; ++n) {
            oacc[n] = mfma(vop[2 * n], p0, oacc[n]);
            oacc[n] = mfma(vop[2 * n + 1], p1, oacc[n]);
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
    for (int it = 0; it < tiles; it += 2) {
        step(it, s1);
        if (it + 1 >= tiles) break;
        step(it + 1, s0);
    }

    // ---- normalise and store: lane (query, h2) holds dims 32n + 8a + 4 h2 + {0..3}
    if (!wlive) return;
    const int iq = wq0 + l32;
    const float inv = 1.f / (l_run + __shfl_xor(l_run, 32, 64));
    if (iq >= qend) return;
    uint16_t *row = static_cast<uint16_t *>(a.out) + (((size_t)b * a.Pn + iq) * a.H + h) * D;
#pragma unroll
    for (int n = 0; n < MT; ++n)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x16 &o = oacc[n];
            const uint2 w = make_uint2(pk_bf16(o[4 * q4] * inv, o[4 * q4 + 1] * inv),
                                       pk_bf16(o[4 * q4 + 2] * inv, o[4 * q4 + 3] * inv));
            *reinterpret_cast<uint2 *>(row + 32 * n + 8 * q4 + 4 * h2) = w;
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
