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
// Layout of the work: one workgroup of 4 waves per (sequence, head, block of 256 queries); wave w
// owns queries [64w, 64w + 64) of the block as two 32-query tiles.  Per 32-token tile:
//   * the waves split the expansion (key tile M and value tile N = one MFMA chain each) and store
//     the bf16 results in LDS directly in the lane layout of the attention MFMAs' operands;
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

constexpr int PWAVES = 4;                  // waves per workgroup
constexpr int QT = 2;                      // 32-query tiles per wave
constexpr int QWG = PWAVES * QT * 32;      // queries per workgroup

template <int D, int RK, int RV>
struct PShape {
    static constexpr int MT = D / 32;                  // 32-wide tiles of the head dim
    static constexpr int KS = D / 16;                  // k-steps of the score MFMA
    static constexpr int KK = RK / 16, KV = RV / 16;   // k-steps of the expansions
    static constexpr int NEWK = KS * 64 / (64 * PWAVES);        // chunk key pieces per thread
    static constexpr int NEWV = 32 * D / 8 / (64 * PWAVES);     // chunk value pieces per thread
    static constexpr int NST = (KK + KV > NEWK + NEWV) ? KK + KV : NEWK + NEWV;   // stage regs
    static_assert(MT == 2 || MT == 4, "head dim 64 or 128");
};

// Registers holding one tile's inputs while they are in flight: latent slices (cached tiles:
// k-steps of c_k, then of c_v) or chunk rows (new tiles: key pieces, then value pieces).
template <int N>
struct Stage {
    uint4 r[N];
};

template <int D, int RK, int RV>
__global__ __launch_bounds__(64 * PWAVES) void prefill_kernel(PrefillArgs a) {
    using SH = PShape<D, RK, RV>;
    constexpr int MT = SH::MT, KS = SH::KS, KK = SH::KK, KV = SH::KV;
    constexpr int NEWK = SH::NEWK, NEWV = SH::NEWV, NST = SH::NST;

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
    const int wq0 = q0 + 64 * wave;                     // this wave's first query
    const bool wlive = wq0 < qend;

    const uint16_t *qp = static_cast<const uint16_t *>(a.q);
    const uint16_t *kp = static_cast<const uint16_t *>(a.k_pool);
    const uint16_t *vp = static_cast<const uint16_t *>(a.v_pool);
    const uint16_t *kn = static_cast<const uint16_t *>(a.k_new);
    const uint16_t *vn = static_cast<const uint16_t *>(a.v_new);
    const int32_t *bt = a.block_table + (size_t)b * a.max_pages;

    // ---- expansion jobs of this wave: key tile mk and/or value tile nv (-1: none)
    const int mk = MT == 4 ? wave : (wave < 2 ? wave : -1);
    const int nv = MT == 4 ? wave : (wave >= 2 ? wave - 2 : -1);
    const int mkc = mk < 0 ? 0 : mk, nvc = nv < 0 ? 0 : nv;   // clamped for the (unused) loads
    // A operand of the key expansion: W_up,t^K transposed, lane (l32, h2) holds column
    // col0 + 32 mk + l32, ranks 16 ks + 8 h2 .. + 7.  B operand of the value expansion: W_up,t^V,
    // lane (l32, h2) holds column col0 + 32 nv + l32, the same ranks.
    const uint16_t *Wk = static_cast<const uint16_t *>(a.W_up_k) +
                         ((size_t)a.t * a.G + g) * RK * a.Dg + col0;
    const uint16_t *Wv = static_cast<const uint16_t *>(a.W_up_v) +
                         ((size_t)a.t * a.G + g) * RV * a.Dg + col0;
    uint4 wk[KK], wv[KV];
#pragma unroll
    for (int ks = 0; ks < KK; ++ks) {
        uint16_t e[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) e[x] = Wk[(size_t)(16 * ks + 8 * h2 + x) * a.Dg + 32 * mkc + l32];
        wk[ks] = make_uint4(e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16,
                            e[4] | (uint32_t)e[5] << 16, e[6] | (uint32_t)e[7] << 16);
    }
#pragma unroll
    for (int ks = 0; ks < KV; ++ks) {
        uint16_t e[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) e[x] = Wv[(size_t)(16 * ks + 8 * h2 + x) * a.Dg + 32 * nvc + l32];
        wv[ks] = make_uint4(e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16,
                            e[4] | (uint32_t)e[5] << 16, e[6] | (uint32_t)e[7] << 16);
    }
    // mu_t: the key tile's lane holds dims 32 mk + 8 (v / 4) + 4 h2 + v % 4; the value tile's
    // lane holds dim 32 nv + l32
    const uint16_t *muk = static_cast<const uint16_t *>(a.mu_k) +
                          (size_t)g * a.T * a.Dg + (size_t)a.t * a.Dg + col0;
    const uint16_t *muv = static_cast<const uint16_t *>(a.mu_v) +
                          (size_t)g * a.T * a.Dg + (size_t)a.t * a.Dg + col0;
    float mkv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) mkv[v] = bf2f(muk[32 * mkc + 8 * (v >> 2) + 4 * h2 + (v & 3)]);
    const float mvv = bf2f(muv[32 * nvc + l32]);

    // ---- query operands (B of the score MFMA): lane (l32, h2) holds query row wq0 + 32u + l32,
    // k-step ks covers dims 32 (ks / 2) + 16 (ks % 2) + 4 h2 + {0..3} and + 8 + {0..3}.  Rows past
    // the chunk read the last valid row (their results are not stored).
    uint4 qop[QT][KS];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
        const int i = min(wq0 + 32 * u + l32, nn - 1);
        const uint16_t *row = qp + (((size_t)b * a.Pn + i) * a.H + h) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = 32 * (ks >> 1) + 16 * (ks & 1) + 4 * h2;
            const uint2 lo = *reinterpret_cast<const uint2 *>(row + d0);
            const uint2 hi = *reinterpret_cast<const uint2 *>(row + d0 + 8);
            qop[u][ks] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
    }

    // ---- tile inputs.  Cached tile c: token 32c + l32 (the last valid token past the end) of
    // one page (P is a multiple of 32); an out-of-range page id poisons the tile with NaN.
    // Chunk tile n: rows 32n .. 32n + 31 of k_new / v_new (clamped to the last valid row).
    auto issue = [&](int tile, Stage<NST> &st) {
        tile = min(tile, tiles - 1);
        if (tile < ctiles) {
            const int j = min(32 * tile + l32, len - 1);
            int page = bt[(32 * tile) / a.P];
            page = (unsigned)page < (unsigned)a.n_pages ? page : 0;
            const size_t row = ((size_t)page * a.G + g) * a.P + j % a.P;
#pragma unroll
            for (int ks = 0; ks < KK; ++ks)
                st.r[ks] = *reinterpret_cast<const uint4 *>(kp + row * RK + 16 * ks + 8 * h2);
#pragma unroll
            for (int ks = 0; ks < KV; ++ks)
                st.r[KK + ks] = *reinterpret_cast<const uint4 *>(vp + row * RV + 16 * ks + 8 * h2);
        } else {
            const int n0 = 32 * (tile - ctiles);
#pragma unroll
            for (int x = 0; x < NEWK; ++x) {
                const int idx = tid + 64 * PWAVES * x;          // (k-step, lane) of the operand
                const int ks = idx >> 6, ln = idx & 63;
                const int i = min(n0 + (ln & 31), nn - 1);
                const int d0 = 32 * (ks >> 1) + 16 * (ks & 1) + 4 * (ln >> 5);
                const uint16_t *row = kn + ((size_t)b * a.Pn + i) * a.new_stride + (size_t)h * D;
                const uint2 lo = *reinterpret_cast<const uint2 *>(row + d0);
                const uint2 hi = *reinterpret_cast<const uint2 *>(row + d0 + 8);
                st.r[x] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
#pragma unroll
            for (int x = 0; x < NEWV; ++x) {
                const int idx = tid + 64 * PWAVES * x;          // (token, 8-dim piece)
                const int i = min(n0 + idx / (D / 8), nn - 1);
                const uint16_t *row = vn + ((size_t)b * a.Pn + i) * a.new_stride + (size_t)h * D;
                st.r[NEWK + x] = *reinterpret_cast<const uint4 *>(row + 8 * (idx % (D / 8)));
            }
        }
    };

    // ---- write tile `tile` into LDS buffer `buf` in operand layout
    auto produce = [&](int tile, const Stage<NST> &st, int buf) {
        if (tile >= tiles) return;
        if (tile < ctiles) {
            const int page = bt[(32 * tile) / a.P];
            const float poison = (unsigned)page < (unsigned)a.n_pages ? 0.f : __builtin_nanf("");
            if (mk >= 0) {
                // K_hat^T tile mk: D[m = dim][n = token]; lane (token l32, h2) gets dims
                // 32 mk + 8 (v / 4) + 4 h2 + v % 4, i.e. k-steps 2 mk (v < 8) and 2 mk + 1
                f32x16 acc = {};
#pragma unroll
                for (int ks = 0; ks < KK; ++ks) acc = mfma(wk[ks], st.r[ks], acc);
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[v] += mkv[v] + poison;
                sK[buf][2 * mk][lane] = pack8(acc, 0);
                sK[buf][2 * mk + 1][lane] = pack8(acc, 1);
            }
            if (nv >= 0) {
                // V_hat tile nv: D[m = token][n = dim]; lane (dim l32, h2) gets tokens
                // 8 (v / 4) + 4 h2 + v % 4: token k-steps 0 (v < 8) and 1
                f32x16 acc = {};
#pragma unroll
                for (int ks = 0; ks < KV; ++ks) acc = mfma(st.r[KK + ks], wv[ks], acc);
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[v] += mvv + poison;
                sV[buf][2 * nv][lane] = pack8(acc, 0);
                sV[buf][2 * nv + 1][lane] = pack8(acc, 1);
            }
        } else {
#pragma unroll
            for (int x = 0; x < NEWK; ++x) {
                const int idx = tid + 64 * PWAVES * x;
                sK[buf][idx >> 6][idx & 63] = st.r[x];
            }
            // value piece (token jt, dims 8p .. 8p + 7) -> the V^T operand of each dim: lane
            // (dim % 32, h2) of slot 2 (dim / 32) + jt / 16 holds tokens 16 kj + 8 (e / 4) + 4 h2 +
            // e % 4 at element e
#pragma unroll
            for (int x = 0; x < NEWV; ++x) {
                const int idx = tid + 64 * PWAVES * x;
                const int jt = idx / (D / 8), p8 = 8 * (idx % (D / 8));
                const int kj = jt >> 4, rem = jt & 15;
                const int hh = (rem >> 2) & 1, e = 4 * (rem >> 3) + (rem & 3);
                const uint4 w = st.r[NEWK + x];
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

    // ---- online softmax state per query tile (log2 domain); O^T accumulators per 32-dim tile
    float m_run[QT], l_run[QT];
    f32x16 oacc[QT][MT];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
        m_run[u] = -INFINITY;
        l_run[u] = 0.f;
#pragma unroll
        for (int n = 0; n < MT; ++n) oacc[u][n] = f32x16{};
    }

    auto consume = [&](int tile, int buf) {
        if (!wlive) return;
        const bool cached = tile < ctiles;
        const int j0 = cached ? 32 * tile : 32 * (tile - ctiles);
        if (!cached && j0 > min(wq0 + 63, qend - 1)) return;   // every token is after every query
        uint4 kop[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kop[ks] = sK[buf][ks][lane];
        f32x16 sacc[QT];
#pragma unroll
        for (int u = 0; u < QT; ++u) sacc[u] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int u = 0; u < QT; ++u) sacc[u] = mfma(kop[ks], qop[u][ks], sacc[u]);
        uint4 vop[2 * MT];
#pragma unroll
        for (int x = 0; x < 2 * MT; ++x) vop[x] = sV[buf][x][lane];

        uint4 pop[QT][2];
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            // lane (query, h2), element v: token j0 + 8 (v / 4) + 4 h2 + v % 4
            const int iq = wq0 + 32 * u + l32;
            const int lim = cached ? len - 1 - j0 : iq - j0;   // last visible token, tile-relative
            float sv[16];
            float mx = -INFINITY;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int j = 8 * (v >> 2) + 4 * h2 + (v & 3);
                sv[v] = j <= lim ? sacc[u][v] * a.scale_log2 : -INFINITY;
                mx = fmaxf(mx, sv[v]);
            }
            mx = max_swap32(mx);
            const float m_new = fmaxf(m_run[u], mx);
            if (__builtin_amdgcn_ballot_w64(m_new > m_run[u]) != 0) {
                const float alpha = exp2_(m_run[u] - m_new);
                l_run[u] *= alpha;
#pragma unroll
                for (int n = 0; n < MT; ++n)
#pragma unroll
                    for (int v = 0; v < 16; ++v) oacc[u][n][v] *= alpha;
                m_run[u] = m_new;
            }
            f32x16 p;
            float ls = 0.f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                p[v] = exp2_(sv[v] - m_run[u]);
                ls += p[v];
            }
            l_run[u] += ls;
            pop[u][0] = pack8(p, 0);
            pop[u][1] = pack8(p, 1);
        }
#pragma unroll
        for (int n = 0; n < MT; ++n)
#pragma unroll
            for (int kj = 0; kj < 2; ++kj)
#pragma unroll
                for (int u = 0; u < QT; ++u)
                    oacc[u][n] = mfma(vop[2 * n + kj], pop[u][kj], oacc[u][n]);
    };

    // ---- pipeline: tile i + 1 produced while tile i is consumed; tile i + 2's inputs in flight
    Stage<NST> s0, s1;
    issue(0, s0);
    issue(1, s1);
    produce(0, s0, 0);
    issue(2, s0);
    __syncthreads();
    auto step = [&](int it, Stage<NST> &next) {
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
    uint16_t *op = static_cast<uint16_t *>(a.out);
#pragma unroll
    for (int u = 0; u < QT; ++u) {
        const int iq = wq0 + 32 * u + l32;
        const float lsum = l_run[u] + __shfl_xor(l_run[u], 32, 64);
        const float inv = 1.f / lsum;
        if (iq >= qend) continue;
        uint16_t *row = op + (((size_t)b * a.Pn + iq) * a.H + h) * D;
#pragma unroll
        for (int n = 0; n < MT; ++n)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x16 &o = oacc[u][n];
                const uint2 w = make_uint2(pk_bf16(o[4 * q4] * inv, o[4 * q4 + 1] * inv),
                                           pk_bf16(o[4 * q4 + 2] * inv, o[4 * q4 + 3] * inv));
                *reinterpret_cast<uint2 *>(row + 32 * n + 8 * q4 + 4 * h2) = w;
            }
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
