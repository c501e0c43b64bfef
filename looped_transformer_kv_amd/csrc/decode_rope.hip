// decode_rope.hip -- rotary latent decode for key rank 16: two heads of one sequence per wave, each
// chunk's rotation sines and cosines computed once for both, scores on the matrix core.
//
// Computes what the rotary form of decode_bf16.hip computes (the rotation follows reconstruction:
// "Axiom & Free-Parameter Ledger" page, a token keeps its position at every recurrence step, so
// RoPE can be applied after reconstruction; pith.science "Looped Latent Attention", section "What
// carries the argument": x_hat_t = c W_up,t + mu_t):
//   s_j = scale <q, R_j K_hat(j)>,  K_hat(j) = c_k(j) W_up,t^K + mu_t^K
//   out = sum_j softmax(s)_j V_hat(j) (plus the current token's own key and value)
//
// Scores.  With pair m = (i, i') of the head dims and phi_jm token j's angle for it,
//   <q, R_j x> = sum_m cos(phi_jm) (q_i x_i + q_i' x_i') + sin(phi_jm) (q_i' x_i - q_i x_i'),
// and x = c_k W_up,t^K + mu_t^K is linear in the latent.  Per head, the coefficients of both
// brackets over the ranks (q_i W[k][i] + q_i' W[k][i'] and q_i' W[k][i] - q_i W[k][i'], and the
// same with mu_t^K in place of a W row) form a matrix A of (r_k + 1) rows over d pair-space
// columns (d/2 cosine columns, then d/2 sine columns).  For a chunk of 32 tokens the pair-space
// matrix Phi = [cos phi; sin phi] (d x 32) depends on the positions only, so it is built once per
// chunk for every head the wave serves, and one MFMA contraction per head, A Phi, gives each token
// its query over the latent ranks (and its mu term): the score is then a 16-term dot product with
// the token's latent.  Both MFMA operands are bf16 (A rounded once from fp32; Phi from the
// hardware sine and cosine), accumulation fp32; the token's query is rounded to bf16 for the dot
// (bf16 pairs, v_dot2_f32_bf16), the mu term stays fp32.
// Values.  The rotation leaves values alone, so sum_j p_j V_hat(j) = (sum_j p_j c_v(j)) W_up,t^V +
// (sum_j p_j) mu_t^V: the value latents, weighted by p rounded to bf16, accumulate in fp32 and
// are expanded once, at the end.
//
// Work decomposition: one workgroup of 8 waves per (sequence b, pair of heads, context split s),
// the same splits as the latent decode plan (B * H / 2 * S workgroups of 8 waves = the plan's
// B * H * S workgroups of 4).  Waves take 32-token chunks round-robin with two chunks of both
// heads' latents in flight; a single-split plan finishes the output here (self term and
// (sum p) mu_t^V included), otherwise one (o, m, l) partial per (head, split) goes to combine.hip,
// with the rotated self score in the first split's record.
#include <cmath>

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
__device__ __forceinline__ float lo_bf(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
// c + a.lo * b.lo + a.hi * b.hi over bf16 pairs, fp32 result (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                           c, false);
}

template <int D, int RK, int RV>
struct RopeShape {
    static_assert(RK == 16, "the score tile holds the 16 ranks and the mu row");
    static_assert(RV % 16 == 0 && RV <= 32, "value ranks");
    static constexpr int HG = 2;          // heads per wave
    static constexpr int WAVES = 8;
    static constexpr int KS = D / 16;     // MFMA k-steps over pair space: cosine half, sine half
    static constexpr int KC = KS / 2;     // k-steps of the cosine half
    static constexpr int NF = 8 * KC;     // pairs whose angle a lane computes (d/4)
    static constexpr int KV = RV / 16;    // 16-byte value latent slices per lane and head
    static constexpr int DEPTH = 2;       // chunks in flight per wave
};

// this lane's latent slices of one 32-token chunk, for both heads: keys (ranks 8 h2 .. +7),
// values (ranks 16 ks + 8 h2 .. +7)
template <int HG, int KV>
struct RopeChunk {
    uint4 k[HG];
    uint4 v[HG][KV];
};

// KF: the number of leading pair groups kc (pairs 16 kc .. 16 kc + 15) whose angles the chunk loop
// reduces to [0, 1) before the hardware sine and cosine, which take revolutions and are accurate
// for |x| <= 256.  Frequencies fall with m, so the groups that can pass 256 revolutions come
// first; the launcher picks KF = 1 when no position of the cache takes a pair m >= 16 that far,
// else KF = d / 32 (every group).
template <int D, int RK, int RV, int KF>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void decode_rope_kernel(DecodeArgs a) {
    using SH = RopeShape<D, RK, RV>;
    constexpr int HG = SH::HG, WAVES = SH::WAVES, KS = SH::KS, KC = SH::KC, NF = SH::NF;
    constexpr int KV = SH::KV, DEPTH = SH::DEPTH;
    constexpr int NT = 64 * WAVES;
    static_assert(kMaxChunksPerSplit <= 64 * WAVES, "one page-table entry per lane and wave");
    static_assert(HG * D <= NT, "one output element per thread");

    __shared__ __align__(16) uint4 sA[HG][KS][64];          // A operands (bf16), per k-step and lane
    constexpr int DP = D + 8;   // padded W_up^K rows: the A build's row-varying reads spread over banks
    __shared__ __align__(16) uint16_t sWk[HG][RK + 1][DP];  // W_up,t^K rows, then mu_t^K
    __shared__ __align__(16) uint16_t sQ[HG][D];
    __shared__ __align__(16) float sC[WAVES][HG][RV];       // each wave's p-weighted latent sums
    __shared__ __align__(16) float sCbar[HG][RV];
    __shared__ float sM[WAVES][HG], sL[WAVES][HG], sSelf[HG];
    __shared__ int sSlot[64 * WAVES];                       // chunk -> head h0's first pool row

    const int S = a.S, HP = a.H / HG;
    const int id = xcd_work_item(blockIdx.x, gridDim.x);
    const int s = id % S;
    const int hp = (id / S) % HP;
    const int b = id / (S * HP);
    const int h0 = HG * hp;                                  // heads h0 .. h0 + HG - 1
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h2 = lane >> 5;

    // ---- this split's token range and its chunk -> pool row table
    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
    const int j_begin = s * a.tokens_per_split;
    const int j_end = min(j_begin + a.tokens_per_split, len);
    const int nchunks = j_end > j_begin ? (j_end - j_begin + 31) >> 5 : 0;
    const int32_t *bt = a.block_table + (size_t)b * a.max_pages;
    // chunk c -> head h0's row of its first token (head h0 + e: e * P rows on, the next group of
    // the same page); negative marks an invalid page id.  The table read is clamped.
    auto slot_of = [&](int c) {
        const int j = j_begin + 32 * c;
        const int page = bt[min(j / a.P, a.max_pages - 1)];
        const bool bad = (unsigned)page >= (unsigned)a.n_pages;
        const int row = ((bad ? 0 : page) * a.G + h0) * a.P + j % a.P;
        return bad ? -row - 1 : row;
    };
    const uint16_t *kpool = static_cast<const uint16_t *>(a.k_pool);
    const uint16_t *vpool = static_cast<const uint16_t *>(a.v_pool);
    // chunk c at row `slot`: lanes past the sequence end read the chunk's last valid token (its
    // weight is zero); a chunk past the end (only ever prefetched) reads its page slot's first row
    auto load_slot = [&](int c, int slot, RopeChunk<HG, KV> &x) {
        const int row = __builtin_amdgcn_readfirstlane(slot < 0 ? -slot - 1 : slot);
        const int valid = j_end - (j_begin + 32 * c);
        const int tok = min(l32, max(valid - 1, 0));
#pragma unroll
        for (int e = 0; e < HG; ++e) {
            const size_t r = (size_t)(row + e * a.P + tok);
            x.k[e] = *reinterpret_cast<const uint4 *>(kpool + r * RK + 8 * h2);
#pragma unroll
            for (int ks = 0; ks < KV; ++ks)
                x.v[e][ks] = *reinterpret_cast<const uint4 *>(vpool + r * RV + 16 * ks + 8 * h2);
        }
    };
    auto load = [&](int c, RopeChunk<HG, KV> &x) { load_slot(c, sSlot[c], x); };

    // ---- prologue, in issue order: (1) the page-table entries of this wave's first chunks,
    // (2) every set-up operand raw into registers, (3) the first latent chunks, (4) LDS stores and
    // the work that waits on (2).  All loads are unconditional at clamped in-bounds indices.
    const int c_last = max(nchunks - 1, 0);
    int first[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) first[i] = slot_of(wave + i * WAVES);
    // this wave's chunks c = wave + WAVES * lane (entries past the split repeat its last chunk)
    const int slot_reg = slot_of(min(wave + WAVES * lane, c_last));

    // W_up,t^K of heads h0 .. h0 + HG - 1: consecutive groups, one contiguous block of
    // HG * r_k * d elements, in 16-byte pieces (W_up,t^V is read at the end, by the threads that
    // expand the value sums)
    const uint16_t *Wk = static_cast<const uint16_t *>(a.W_up_k) + ((size_t)a.t * a.G + h0) * RK * D;
    const uint16_t *Wv = static_cast<const uint16_t *>(a.W_up_v) + ((size_t)a.t * a.G + h0) * RV * D;
    constexpr int PWK = HG * RK * D / 8;
    constexpr int UWK = (PWK + NT - 1) / NT;
    uint4 wkp[UWK];
#pragma unroll
    for (int u = 0; u < UWK; ++u)
        wkp[u] = reinterpret_cast<const uint4 *>(Wk)[min(tid + u * NT, PWK - 1)];
    // element (e, i) = (tid / D, tid % D) of the heads' q and mu_t^K (the operands of the output
    // step, mu_t^V, the own key and value and W_up,t^V, are read after the chunk loop)
    const int oe = (tid % (HG * D)) / D, oi = tid % D;
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) + ((size_t)b * a.H + h0) * D;
    const size_t mu_off = (size_t)(h0 + oe) * a.T * a.Dg + (size_t)a.t * a.Dg + oi;
    const uint16_t q_raw = qp[oe * D + oi];
    const uint16_t mk_raw = static_cast<const uint16_t *>(a.mu_k)[mu_off];
    const int R = a.rope_rot;

    // (3) the first latent chunks of this wave.  The set-up loads above stay ahead of them: a
    // wave's loads complete in order, and the LDS stores below wait only for those.
    __builtin_amdgcn_sched_barrier(0);
    RopeChunk<HG, KV> buf[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) load_slot(wave + i * WAVES, first[i], buf[i]);

    // (4) LDS: page table, W_up,t, q and mu_t^K.  Every store is unconditional (threads past a
    // table's end write a copy of its last entry, the same value), so no load is moved into a
    // branch behind the latent burst.
    sSlot[wave + WAVES * lane] = slot_reg;
#pragma unroll
    for (int u = 0; u < UWK; ++u) {
        const int e = min(tid + u * NT, PWK - 1);   // element 8e of the [HG][RK][D] block
        *reinterpret_cast<uint4 *>(&sWk[(8 * e) / (RK * D)][((8 * e) / D) % RK][(8 * e) % D]) = wkp[u];
    }
    sQ[oe][oi] = q_raw;          // threads from HG * D on repeat (oe, oi) of thread tid - HG * D
    sWk[oe][RK][oi] = mk_raw;
    // revolutions per position of pair m, theta^(-2m/R) / (2 pi); pairs m >= R/2 stand for two
    // unrotated dims (frequency 0)
    const float kexp = R > 0 ? -2.0f * a.rope_log2_theta / (float)R : 0.f;
    auto rope_rev = [&](int m) {
        const float f = exp2_((float)m * kexp) * 0.15915494309189535f;
        return m < R / 2 ? f : 0.f;
    };
    // this lane's pairs: 16 kc + 8 h2 + e, kc < KC, e < 8 (the Phi rows it holds)
    float fr[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) fr[f] = rope_rev(16 * (f / 8) + 8 * h2 + f % 8);
    __syncthreads();

    // ---- A operands.  Row rho of the 32-row score tile: the MFMA result element v of lane
    // (l32, h2) is row 8 (v / 4) + 4 h2 + v % 4, so rank 8 h2 + v (v < 8) goes to that row, the
    // lane's key latent slice lines up with its elements 0..7, and mu_t^K takes element 8 of the
    // h2 = 0 lanes (row 16); the other rows are zero.  Column k of k-step ks: pair
    // m = 16 (ks % KC) + 8 h2 + e, cosine bracket for ks < KC, sine bracket after; log2-scaled.
    auto pair_elems = [&](int m, int &i, int &ip) {
        const bool rot = m < R / 2;
        const int i_rot = a.rope_style ? 2 * m : m;
        const int ip_rot = a.rope_style ? 2 * m + 1 : m + R / 2;
        const int i_flat = R + 2 * (m - R / 2);
        i = rot ? i_rot : i_flat;
        ip = rot ? ip_rot : i_flat + 1;
    };
    static_assert((HG * KS) % WAVES == 0, "whole k-steps per wave");
#pragma unroll
    for (int j = 0; j < HG * KS / WAVES; ++j) {              // each wave builds whole k-steps
        const int it = wave + WAVES * j;
        const int e = it / KS, ks = it % KS;
        const bool sine = ks >= KC;
        const int v = 4 * (l32 / 8) + l32 % 4, vh = (l32 / 4) % 2;   // row l32 = element v of half vh
        const int kap = v < 8 ? 8 * vh + v : (v == 8 && vh == 0 ? RK : -1);
        const int kr = max(kap, 0);
        const int m0 = 16 * (ks % KC) + 8 * h2;   // this lane's pairs m0 .. m0 + 7
        float cf[8];
        if ((R & 15) == 0) {
            // each group of 8 pairs is wholly rotated or wholly unrotated: 16-byte reads.  Half
            // split: elements m0.. and m0 + R/2..; interleaved (and unrotated): 2 m0 .. 2 m0 + 15
            const bool half = m0 < R / 2 && !a.rope_style;
            const int o0 = half ? m0 : 2 * m0, o1 = half ? m0 + R / 2 : 2 * m0 + 8;
            const uint4 w0 = *reinterpret_cast<const uint4 *>(&sWk[e][kr][o0]);
            const uint4 w1 = *reinterpret_cast<const uint4 *>(&sWk[e][kr][o1]);
            const uint4 q0 = *reinterpret_cast<const uint4 *>(&sQ[e][o0]);
            const uint4 q1 = *reinterpret_cast<const uint4 *>(&sQ[e][o1]);
            const uint32_t W[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            const uint32_t Q[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
            for (int y = 0; y < 8; ++y) {
                const uint32_t wa = W[y / 2], wb = W[4 + y / 2], qa = Q[y / 2], qb = Q[4 + y / 2];
                const float wi = half ? ((y & 1) ? hi_bf(wa) : lo_bf(wa)) : lo_bf(W[y]);
                const float wip = half ? ((y & 1) ? hi_bf(wb) : lo_bf(wb)) : hi_bf(W[y]);
                const float qi = half ? ((y & 1) ? hi_bf(qa) : lo_bf(qa)) : lo_bf(Q[y]);
                const float qip = half ? ((y & 1) ? hi_bf(qb) : lo_bf(qb)) : hi_bf(Q[y]);
                cf[y] = sine ? qip * wi - qi * wip : qi * wi + qip * wip;
            }
        } else {
#pragma unroll
            for (int y = 0; y < 8; ++y) {
                int i, ip;
                pair_elems(m0 + y, i, ip);
                const float qi = bf2f(sQ[e][i]), qip = bf2f(sQ[e][ip]);
                const float wi = bf2f(sWk[e][kr][i]), wip = bf2f(sWk[e][kr][ip]);
                cf[y] = sine ? qip * wi - qi * wip : qi * wi + qip * wip;
            }
        }
        uint32_t w[4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
            w[x] = pk_bf16(kap >= 0 ? cf[2 * x] * a.scale_log2 : 0.f,
                           kap >= 0 ? cf[2 * x + 1] * a.scale_log2 : 0.f);
        sA[e][ks][lane] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    __syncthreads();

    // ---- per-head running state: max (log2 domain), this lane's share of the weight sum, and
    // the p-weighted value latents of ranks 16 ks + 8 h2 + x (fp32)
    float m_run[HG], l_lane[HG], cb[HG][8 * KV];
#pragma unroll
    for (int e = 0; e < HG; ++e) {
        m_run[e] = -INFINITY;
        l_lane[e] = 0.f;
#pragma unroll
        for (int x = 0; x < 8 * KV; ++x) cb[e][x] = 0.f;
    }

    // the A operands of both heads stay in registers
    uint4 areg[HG][KS];
#pragma unroll
    for (int e = 0; e < HG; ++e)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) areg[e][ks] = sA[e][ks][lane];

    // one chunk, both heads
    auto compute = [&](int c, const RopeChunk<HG, KV> &x) {
        const int valid = j_end - (j_begin + 32 * c);   // >= 1, wave-uniform
        const bool bad = sSlot[c] < 0;
        // Phi for token l32 (position j_begin + 32c + l32), one cosine k-step and its sine
        // k-step at a time (element e of k-step kc: pair 16 kc + 8 h2 + e), each pair of k-steps
        // feeding both heads' MFMAs as soon as it is built
        const float pos = (float)(j_begin + 32 * c + l32);
        f32x16 acc[HG];
#pragma unroll
        for (int e = 0; e < HG; ++e) acc[e] = f32x16{};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            uint32_t cw[4], sw[4];
#pragma unroll
            for (int y = 0; y < 4; ++y) {
                float r0 = pos * fr[8 * kc + 2 * y], r1 = pos * fr[8 * kc + 2 * y + 1];
                if (kc < KF) {
                    r0 = __builtin_amdgcn_fractf(r0);
                    r1 = __builtin_amdgcn_fractf(r1);
                }
                cw[y] = pk_bf16(__builtin_amdgcn_cosf(r0), __builtin_amdgcn_cosf(r1));
                sw[y] = pk_bf16(__builtin_amdgcn_sinf(r0), __builtin_amdgcn_sinf(r1));
            }
            const uint4 pc = make_uint4(cw[0], cw[1], cw[2], cw[3]);
            const uint4 ps = make_uint4(sw[0], sw[1], sw[2], sw[3]);
#pragma unroll
            for (int e = 0; e < HG; ++e) acc[e] = mfma32x32x16(areg[e][kc], pc, acc[e]);
#pragma unroll
            for (int e = 0; e < HG; ++e) acc[e] = mfma32x32x16(areg[e][KC + kc], ps, acc[e]);
        }
#pragma unroll
        for (int e = 0; e < HG; ++e) {
            // the token's query over ranks 8 h2 .. + 7, rounded to bf16, against its latent slice
            // (bf16 pairs, v_dot2_f32_bf16); the mu term stays fp32
            const uint4 kx = x.k[e];
            float sp = (h2 == 0 ? acc[e][8] : 0.f);
            sp = dot2bf(pk_bf16(acc[e][0], acc[e][1]), kx.x, sp);
            sp = dot2bf(pk_bf16(acc[e][2], acc[e][3]), kx.y, sp);
            sp = dot2bf(pk_bf16(acc[e][4], acc[e][5]), kx.z, sp);
            sp = dot2bf(pk_bf16(acc[e][6], acc[e][7]), kx.w, sp);
            float sc = add_swap32(sp);                  // token l32's score, in both lane halves
            if (l32 >= valid) sc = -INFINITY;
            if (bad) sc = __builtin_nanf("");
            // online softmax (log2 domain); the running max only moves when a score exceeds it,
            // so the rescale is skipped otherwise (a wave-uniform branch)
            if (__builtin_amdgcn_ballot_w64(sc > m_run[e]) != 0) {
                const float r = row16_max(sc);
                const float cmax =
                    fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 0)),
                          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 16)));
                const float m_new = fmaxf(m_run[e], cmax);
                const float alpha = exp2_(m_run[e] - m_new);
                l_lane[e] *= alpha;
#pragma unroll
                for (int y = 0; y < 8 * KV; ++y) cb[e][y] *= alpha;
                m_run[e] = m_new;
            }
            const float p = exp2_(sc - m_run[e]);
            l_lane[e] += (h2 == 0 ? p : 0.f);
            // p (rounded to bf16) times each bf16 value latent, added in fp32: (p, 0) and (0, p)
            // against a latent pair pick its low and its high element (v_dot2_f32_bf16)
            const uint32_t plo = pk_bf16(p, 0.f), phi = pk_bf16(0.f, p);
#pragma unroll
            for (int ks = 0; ks < KV; ++ks) {
                const uint4 vx = x.v[e][ks];
                cb[e][8 * ks + 0] = dot2bf(plo, vx.x, cb[e][8 * ks + 0]);
                cb[e][8 * ks + 1] = dot2bf(phi, vx.x, cb[e][8 * ks + 1]);
                cb[e][8 * ks + 2] = dot2bf(plo, vx.y, cb[e][8 * ks + 2]);
                cb[e][8 * ks + 3] = dot2bf(phi, vx.y, cb[e][8 * ks + 3]);
                cb[e][8 * ks + 4] = dot2bf(plo, vx.z, cb[e][8 * ks + 4]);
                cb[e][8 * ks + 5] = dot2bf(phi, vx.z, cb[e][8 * ks + 5]);
                cb[e][8 * ks + 6] = dot2bf(plo, vx.w, cb[e][8 * ks + 6]);
                cb[e][8 * ks + 7] = dot2bf(phi, vx.w, cb[e][8 * ks + 7]);
            }
        }
    };

    // ---- main loop: chunks wave, wave + WAVES, ...; a buffer is refilled with the chunk DEPTH
    // rounds ahead as soon as it has been consumed (prefetch indices clamped to the last chunk).
    // Waves w and w + 4 share a SIMD; both serve the same two heads and keep the default issue
    // priority (raising it by the work left, as the one-head kernel does, measured ~0.2 us slower
    // here, and skewing the split towards the older wave ~4 us slower).
    if (wave < nchunks) {
        const int rounds = (nchunks - wave + WAVES - 1) / WAVES;   // >= 1
        int c = wave, r = 0;
        for (; r + DEPTH <= rounds; r += DEPTH) {
#pragma unroll
            for (int i = 0; i < DEPTH; ++i) {
                compute(c, buf[i]);
                load(min(c + DEPTH * WAVES, nchunks - 1), buf[i]);
                c += WAVES;
            }
        }
#pragma unroll
        for (int i = 0; i + 1 < DEPTH; ++i) {
            if (r + i < rounds) {
                compute(c, buf[i]);
                c += WAVES;
            }
        }
    }
    // operands of the output step, read only by the waves that use them (threads below HG * D
    // form the output, waves below HG the self scores), in flight during the merge below: this
    // thread's column of W_up,t^V, mu_t^V and own value (head h0 + oe, element oi), and the
    // current token's own key for head h0 + wave (lanes over d, rotation partners too).  The
    // waves past them, which the SIMDs' oldest-first issue usually leaves last, go straight to
    // the merge.
    const bool has_self = a.k_self != nullptr;
    const bool self_here = S == 1 && has_self;
    uint16_t wv_raw[RV], mv_raw = 0, vs_raw = 0;
    if (tid < HG * D) {
#pragma unroll
        for (int k = 0; k < RV; ++k) wv_raw[k] = Wv[((size_t)oe * RV + k) * D + oi];
        mv_raw = static_cast<const uint16_t *>(a.mu_v)[mu_off];
        if (self_here)
            vs_raw = static_cast<const uint16_t *>(a.v_self)[(size_t)b * a.self_stride +
                                                             (size_t)(h0 + oe) * D + oi];
    }
    // the rotated self score of head h0 + wave: the current token's key turns to position len
    if (wave < HG) {
        const int se = wave;
        auto partner = [&](int i) {
            if (i >= R) return i;
            return a.rope_style ? (i ^ 1) : (i < R / 2 ? i + R / 2 : i - R / 2);
        };
        float as = 0.f;
        if (has_self) {
            const uint16_t *ksp = static_cast<const uint16_t *>(a.k_self) +
                                  (size_t)b * a.self_stride + (size_t)(h0 + se) * D;
#pragma unroll
            for (int u = 0; u < D / 64; ++u) {
                const int i = lane + 64 * u;
                float kk = bf2f(ksp[i]);
                if (i < R) {
                    const bool first_el = a.rope_style ? !(i & 1) : i < R / 2;
                    const int m = a.rope_style ? i >> 1 : (first_el ? i : i - R / 2);
                    const float rev = __builtin_amdgcn_fractf((float)len * rope_rev(m));
                    const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
                    const float kp = bf2f(ksp[partner(i)]);
                    kk = first_el ? kk * cs - kp * sn : kp * sn + kk * cs;
                }
                as += bf2f(qp[se * D + i]) * kk;
            }
        }
        const float ss = wave_sum(as) * a.scale_log2;
        if (lane == 0) sSelf[wave] = has_self ? ss : -INFINITY;
    }

    // ---- merge: lanes (the 32 tokens of each half), then waves, then expand the latent sums
#pragma unroll
    for (int e = 0; e < HG; ++e) {
        const float lw = wave_sum(l_lane[e]);
#pragma unroll
        for (int y = 0; y < 8 * KV; ++y) cb[e][y] = group_sum<32>(cb[e][y]);
        if (l32 == 0) {
#pragma unroll
            for (int ks = 0; ks < KV; ++ks)
#pragma unroll
                for (int y = 0; y < 8; ++y) sC[wave][e][16 * ks + 8 * h2 + y] = cb[e][8 * ks + y];
        }
        if (lane == 0) {
            sM[wave][e] = m_run[e];
            sL[wave][e] = lw;
        }
    }
    __syncthreads();
    // the heads' maxima over the waves (and, single split, the self score)
    auto head_max = [&](int e) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sM[w][e]);
        if (S == 1) M = fmaxf(M, sSelf[e]);
        return M;
    };
    if (tid < HG * RV) {
        const int e = tid / RV, k = tid % RV;
        const float M = head_max(e);
        float C = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) C += sC[w][e][k] * exp2_(sM[w][e] - M);
        }
        sCbar[e][k] = C;
    }
    __syncthreads();
    if (tid < HG * D) {
        const float M = head_max(oe);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) L += sL[w][oe] * exp2_(sM[w][oe] - M);
#pragma unroll
            for (int k = 0; k < RV; ++k) O = fmaf(sCbar[oe][k], bf2f(wv_raw[k]), O);
        }
        const int h = h0 + oe;
        if (S == 1) {
            float res = 0.f;
            if (M != -INFINITY) {
                const float w_self = self_here ? exp2_(sSelf[oe] - M) : 0.f;
                const float v_self = self_here ? bf2f(vs_raw) : 0.f;
                res = (O + L * bf2f(mv_raw) + w_self * v_self) / (L + w_self);
            }
            static_cast<uint16_t *>(a.out)[((size_t)b * a.H + h) * D + oi] = f2bf(res);
        } else {
            float *rec = a.ws + (((size_t)b * a.H + h) * S + s) * (D + kPartialPad);
            rec[oi] = O;
            if (oi == 0) {
                rec[D] = M;
                rec[D + 1] = L;
                if (s == 0) rec[D + 2] = sSelf[oe];   // the rotated self score, for combine
            }
        }
    }
}

template <int D, int RK, int RV>
hipError_t launch_rope_t(const DecodeArgs &a, hipStream_t st) {
    using SH = RopeShape<D, RK, RV>;
    const unsigned blocks = (unsigned)a.B * (a.H / SH::HG) * a.S;
    // the fastest pair past group 0, m = 16: theta^(-32 / rot) / (2 pi) revolutions per position
    // (frequency 0 when it is not rotated); cached positions are below max_seq_len
    const int R = a.rope_rot;
    const double f16 = 16 < R / 2 ? std::exp2(-32.0 / R * a.rope_log2_theta) / (2.0 * M_PI) : 0.0;
    const bool first_only = (double)a.max_seq_len * f16 < 250.0;
    if (first_only)
        hipLaunchKernelGGL((decode_rope_kernel<D, RK, RV, 1>), dim3(blocks), dim3(64 * SH::WAVES), 0,
                           st, a);
    else
        hipLaunchKernelGGL((decode_rope_kernel<D, RK, RV, SH::KC>), dim3(blocks),
                           dim3(64 * SH::WAVES), 0, st, a);
    return hipGetLastError();
}

}  // namespace

bool decode_rope_heads_supported(int mode, int H, int d, int r_k, int r_v) {
    return mode == 0 && H % 2 == 0 && (d == 64 || d == 128) && r_k == 16 &&
           (r_v == 16 || r_v == 32);
}

hipError_t launch_decode_rope_heads(const DecodeArgs &a, hipStream_t st) {
    const int d = a.Dg;
    if (!decode_rope_heads_supported(a.mode, a.H, d, a.r_k, a.r_v)) return hipErrorInvalidValue;
    if (d == 128) return a.r_v == 16 ? launch_rope_t<128, 16, 16>(a, st) : launch_rope_t<128, 16, 32>(a, st);
    return a.r_v == 16 ? launch_rope_t<64, 16, 16>(a, st) : launch_rope_t<64, 16, 32>(a, st);
}

}  // namespace lla
