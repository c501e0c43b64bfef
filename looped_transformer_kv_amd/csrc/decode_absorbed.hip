// decode_absorbed.hip -- absorbed-attention decode over the latent cache, bf16 storage, fp32 math.
//
// The same attention as decode_bf16.hip (pith.science paper page for "Looped Latent Attention",
// "What carries the argument": x_hat_t = c W_up,t + mu_t, attention unchanged), computed in the
// latent space instead of reconstructing K_hat / V_hat per token (the absorbed form the
// editorial letter on the same page discusses; without a rotation between expansion and
// attention it is exact up to rounding):
//   q~  = W_up,t^K q                     (r_k values, once per sequence and head)
//   s_j = scale (<q~, c_k(j)> + <q, mu_t^K>)
//   c~  = sum_j softmax(s)_j c_v(j)      (r_v values)
//   out = c~ W_up,t^V + mu_t^V           (one expansion per sequence and head)
// Per cached token this moves G (r_k + r_v) bf16 values and does r_k + r_v multiply-adds per head:
// a pure latent-bandwidth kernel for every codec, LLA-2D included.
//
// Work decomposition: one workgroup of 4 waves per (sequence b, head h, context split s); the
// waves take 32-token chunks round-robin.  Lane mapping per chunk: a latent row of r bf16 values
// is NP = r / 8 pieces of 16 bytes; lane l reads piece l % NP of token (l / NP) + TPP * pass,
// TPP = 64 / NP tokens per pass, so every lane owns one fixed rank group for the whole call and
// a pass reads TPP consecutive rows (contiguous bytes).  Scores: each lane's 8-term partial dot
// goes to LDS and token j's lane sums its NP partials in a fixed order.  Values: each lane keeps
// 8 fp32 accumulators of p_j c_v(j) for its rank group; they are summed over lanes, then waves,
// in a fixed order at the end.  Online softmax in the log2 domain as in decode_bf16.hip; a
// single-split plan finishes the output here, otherwise (o, m, l) partials in the head-dim space
// go to combine.hip, exactly like the reconstructing kernel's.
#include "lla_internal.h"

namespace lla {
namespace {

template <int R>
struct Pieces {
    static constexpr int NP = R / 8;                    // 16-byte pieces per latent row
    static constexpr int TPP = 64 / NP;                 // tokens per pass
    static constexpr int ACT = TPP * NP;                // active lanes per pass
    static constexpr int PASSES = (32 + TPP - 1) / TPP; // passes per 32-token chunk
};

template <int PK, int PV>
struct AbsChunk {
    uint4 k[PK], v[PV];
};

template <int D, int RK, int RV>
__global__ __launch_bounds__(256) void absorbed_kernel(DecodeArgs a) {
    constexpr int WAVES = 4;
    using KP = Pieces<RK>;
    using VP = Pieces<RV>;
    constexpr int PK = KP::PASSES, PV = VP::PASSES;
    constexpr int DEPTH = PK + PV <= 4 ? 3 : (PK + PV <= 8 ? 2 : 1);   // chunks in flight per wave

    __shared__ float sQt[RK];                           // q~, log2-scaled
    __shared__ float sPart[WAVES][32][KP::NP + 1];      // per-token partial dots
    __shared__ float sP[WAVES][32];                     // the chunk's softmax weights
    __shared__ float sRed[WAVES][64][9];                // per-lane value accumulators
    __shared__ float sC[WAVES][RV];                     // per-wave c~
    __shared__ float sM[WAVES], sL[WAVES];
    __shared__ float sCbar[RV];
    __shared__ int sSlot[kMaxChunksPerSplit];

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

    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
    const int j_begin = s * a.tokens_per_split;
    const int j_end = min(j_begin + a.tokens_per_split, len);
    const int nchunks = j_end > j_begin ? (j_end - j_begin + 31) >> 5 : 0;
    const int32_t *bt = a.block_table + (size_t)b * a.max_pages;
    auto slot_of = [&](int c) {   // chunk c -> first token row; negative marks a bad page id
        const int j = j_begin + 32 * c;
        const int page = bt[min(j / a.P, a.max_pages - 1)];
        const bool bad = (unsigned)page >= (unsigned)a.n_pages;
        const int row = ((bad ? 0 : page) * a.G + g) * a.P + j % a.P;
        return bad ? -row - 1 : row;
    };

    const uint16_t *kpool = static_cast<const uint16_t *>(a.k_pool);
    const uint16_t *vpool = static_cast<const uint16_t *>(a.v_pool);
    // this lane's pieces: rank group and token within each pass
    const int gk = lane % KP::NP, tk0 = lane / KP::NP;
    const int gv = lane % VP::NP, tv0 = lane / VP::NP;
    // chunk c at pool row `slot`; tokens past the sequence end (or past the chunk, for inactive
    // lanes) re-read the chunk's last valid token, so nothing beyond a sequence is read
    auto load_slot = [&](int c, int slot, AbsChunk<PK, PV> &x) {
        const int row = __builtin_amdgcn_readfirstlane(slot < 0 ? -slot - 1 : slot);
        const int last = max(min(j_end - (j_begin + 32 * c), 32) - 1, 0);
        const uint16_t *kb = kpool + (size_t)row * RK;
        const uint16_t *vb = vpool + (size_t)row * RV;
#pragma unroll
        for (int u = 0; u < PK; ++u) {
            const int tok = min(tk0 + KP::TPP * u, last);
            x.k[u] = *reinterpret_cast<const uint4 *>(kb + tok * RK + 8 * gk);
        }
#pragma unroll
        for (int u = 0; u < PV; ++u) {
            const int tok = min(tv0 + VP::TPP * u, last);
            x.v[u] = *reinterpret_cast<const uint4 *>(vb + tok * RV + 8 * gv);
        }
    };

    // ---- prologue.  A wave's vector loads complete in order, so the set-up loads go out before
    // the latent burst and the arithmetic on them waits only for them: (1) the page-table entries
    // of this wave's first chunks, (2) the set-up operands raw into registers, (3) the first
    // latent chunks, (4) q~, <q, mu_t^K>, the self score and the LDS stores.  Every load is
    // unconditional at a clamped in-bounds index (a load under a branch waits at the join).
    const int c_last = max(nchunks - 1, 0);
    int first[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) first[i] = slot_of(wave + i * WAVES);
    // (2) q~[k] = <W_up,t^K row k (this head's columns), q>: thread t takes the 16-byte piece
    // pc = t % NPC of rows k = t / NPC + RPP p; the NPC pieces of a row sit in one aligned lane
    // group and are summed there.  <q, mu_t^K> and the self score: elements lane + 64 u per wave.
    constexpr int NPC = D / 8, RPP = 64 * WAVES / NPC, QPASS = (RK + RPP - 1) / RPP;
    constexpr int UD = D / 64;
    const int pc = tid % NPC, kr0 = tid / NPC;
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) + ((size_t)b * a.H + h) * D;
    const uint16_t *wk0 = static_cast<const uint16_t *>(a.W_up_k) +
                          ((size_t)a.t * a.G + g) * RK * a.Dg + col0 + 8 * pc;
    uint4 wq[QPASS];
#pragma unroll
    for (int p = 0; p < QPASS; ++p)
        wq[p] = *reinterpret_cast<const uint4 *>(wk0 + (size_t)min(kr0 + RPP * p, RK - 1) * a.Dg);
    const uint4 qpc = *reinterpret_cast<const uint4 *>(qp + 8 * pc);
    const uint16_t *muk = static_cast<const uint16_t *>(a.mu_k) + (size_t)g * a.T * a.Dg +
                          (size_t)a.t * a.Dg + col0;
    const bool self_here = S == 1 && a.k_self != nullptr;
    // without a self term this reads q again and the value is dropped
    const uint16_t *ksp = self_here ? static_cast<const uint16_t *>(a.k_self) +
                                          (size_t)b * a.self_stride + (size_t)h * D
                                    : qp;
    uint16_t qv[UD], mkv[UD], ksv[UD];
#pragma unroll
    for (int u = 0; u < UD; ++u) {
        qv[u] = qp[lane + 64 * u];
        mkv[u] = muk[lane + 64 * u];
        ksv[u] = ksp[lane + 64 * u];
    }
    constexpr int US = (kMaxChunksPerSplit + 64 * WAVES - 1) / (64 * WAVES);
    int slot_reg[US];
#pragma unroll
    for (int u = 0; u < US; ++u) slot_reg[u] = slot_of(min(tid + 64 * WAVES * u, c_last));
    __builtin_amdgcn_sched_barrier(0);

    // (3) the first latent chunks of this wave
    AbsChunk<PK, PV> buf[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) load_slot(wave + i * WAVES, first[i], buf[i]);

    // (4) the arithmetic on the set-up operands, and the LDS stores
    auto dot8 = [](const uint4 &x, const uint4 &y) {
        const uint32_t xv[4] = {x.x, x.y, x.z, x.w}, yv[4] = {y.x, y.y, y.z, y.w};
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc += __uint_as_float(xv[e] << 16) * __uint_as_float(yv[e] << 16);
            acc += __uint_as_float(xv[e] & 0xffff0000u) * __uint_as_float(yv[e] & 0xffff0000u);
        }
        return acc;
    };
#pragma unroll
    for (int p = 0; p < QPASS; ++p) {
        const float v = group_sum<NPC>(dot8(wq[p], qpc));
        const int k = kr0 + RPP * p;
        if (pc == 0 && k < RK) sQt[k] = v * a.scale_log2;
    }
    float qm, s_self = -INFINITY;   // <q, mu_t^K> and the self score, log2-scaled
    {
        float am = 0.f, as = 0.f;
#pragma unroll
        for (int u = 0; u < UD; ++u) {
            am += bf2f(qv[u]) * bf2f(mkv[u]);
            as += bf2f(qv[u]) * bf2f(ksv[u]);
        }
        qm = wave_sum(am) * a.scale_log2;
        const float ss = wave_sum(as) * a.scale_log2;
        if (self_here) s_self = ss;
    }
#pragma unroll
    for (int u = 0; u < US; ++u) {
        const int c = tid + 64 * WAVES * u;
        if (c < nchunks) sSlot[c] = slot_reg[u];
    }
    __syncthreads();
    float qt[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qt[e] = sQt[8 * gk + e];

    float m_run = -INFINITY, l_lane = 0.f;
    float cacc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) cacc[e] = 0.f;

    auto compute = [&](int c, const AbsChunk<PK, PV> &x) {
        const int valid = j_end - (j_begin + 32 * c);   // >= 1, wave-uniform
        // ---- partial dots of this lane's rank group, one per pass
#pragma unroll
        for (int u = 0; u < PK; ++u) {
            const uint32_t w[4] = {x.k[u].x, x.k[u].y, x.k[u].z, x.k[u].w};
            float d0 = 0.f, d1 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                d0 += qt[2 * e] * __uint_as_float(w[e] << 16);
                d1 += qt[2 * e + 1] * __uint_as_float(w[e] & 0xffff0000u);
            }
            const int tok = tk0 + KP::TPP * u;
            if (lane < KP::ACT && tok < 32) sPart[wave][tok][gk] = d0 + d1;
        }
        __builtin_amdgcn_wave_barrier();
        // ---- token l32's score (both lane halves), then the online softmax step
        float sc = qm;
#pragma unroll
        for (int q2 = 0; q2 < KP::NP; ++q2) sc += sPart[wave][l32][q2];
        if (l32 >= valid) sc = -INFINITY;
        if (sSlot[c] < 0) sc = __builtin_nanf("");
        if (__builtin_amdgcn_ballot_w64(sc > m_run) != 0) {
            const float r = row16_max(sc);
            const float cmax = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 0)),
                                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 16)));
            const float m_new = fmaxf(m_run, cmax);
            const float alpha = exp2_(m_run - m_new);
            l_lane *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) cacc[e] *= alpha;
            m_run = m_new;
        }
        const float p = exp2_(sc - m_run);
        l_lane += (h2 == 0 ? p : 0.f);
        if (h2 == 0) sP[wave][l32] = p;
        __builtin_amdgcn_wave_barrier();
        // ---- p-weighted value latents of this lane's rank group
#pragma unroll
        for (int u = 0; u < PV; ++u) {
            const int tok = tv0 + VP::TPP * u;
            const float pw = (lane < VP::ACT && tok < 32) ? sP[wave][min(tok, 31)] : 0.f;
            const uint32_t w[4] = {x.v[u].x, x.v[u].y, x.v[u].z, x.v[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                cacc[2 * e] += pw * __uint_as_float(w[e] << 16);
                cacc[2 * e + 1] += pw * __uint_as_float(w[e] & 0xffff0000u);
            }
        }
        __builtin_amdgcn_wave_barrier();
    };

    auto load = [&](int c, AbsChunk<PK, PV> &x) { load_slot(c, sSlot[c], x); };
    if (wave < nchunks) {
        const int rounds = (nchunks - wave + WAVES - 1) / WAVES;
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

    // ---- operands of the output step, which the threads below D form: column tid % D of
    // W_up,t^V, mu_t^V and the own value, issued now so that they arrive during the merge below
    // (value ranks up to 64; wider ones read the column during the expansion)
    constexpr bool EARLY_W = RV <= 64;
    const uint16_t *wv = static_cast<const uint16_t *>(a.W_up_v) +
                         ((size_t)a.t * a.G + g) * RV * a.Dg + col0 + tid % D;
    // every thread loads (column tid % D, no branch: a load under one would wait at the join);
    // without a self term the own-value read repeats mu_t^V and is dropped
    const uint16_t *muvp = static_cast<const uint16_t *>(a.mu_v) + (size_t)g * a.T * a.Dg +
                           (size_t)a.t * a.Dg + col0 + tid % D;
    const uint16_t *vsp = self_here ? static_cast<const uint16_t *>(a.v_self) +
                                          (size_t)b * a.self_stride + (size_t)h * D + tid % D
                                    : muvp;
    uint16_t wcol[EARLY_W ? RV : 1];
    if constexpr (EARLY_W) {
#pragma unroll
        for (int k = 0; k < RV; ++k) wcol[k] = wv[(size_t)k * a.Dg];
    }
    const uint16_t muv_raw = *muvp, vs_raw = *vsp;

    // ---- this wave's c~: sum the lanes of each rank group (tokens tv0 = 0, 1, ...), fixed order
#pragma unroll
    for (int e = 0; e < 8; ++e) sRed[wave][lane][e] = cacc[e];
    const float l_w = wave_sum(l_lane);
    __builtin_amdgcn_wave_barrier();
    for (int k = lane; k < RV; k += 64) {
        const int grp = k / 8, e = k % 8;
        float t = 0.f;
        for (int tt = 0; tt < VP::TPP; ++tt) t += sRed[wave][grp + VP::NP * tt][e];
        sC[wave][k] = t;
    }
    if (lane == 0) {
        sM[wave] = m_run;
        sL[wave] = l_w;
    }
    __syncthreads();
    // ---- merge the waves: c~ and the softmax sums
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sM[w]);
    for (int k = tid; k < RV; k += 64 * WAVES) {
        float t = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) t += sC[w][k] * exp2_(sM[w] - M);
        }
        sCbar[k] = t;
    }
    __syncthreads();
    if (tid < D) {
        float L = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) L += sL[w] * exp2_(sM[w] - M);
        }
        // O = c~ W_up,t^V (this head's column tid)
        float O = 0.f;
        if constexpr (EARLY_W) {
#pragma unroll
            for (int k = 0; k < RV; ++k) O += sCbar[k] * bf2f(wcol[k]);
        } else {
            for (int k = 0; k < RV; ++k) O += sCbar[k] * bf2f(wv[(size_t)k * a.Dg]);
        }
        if (S == 1) {
            const float Mf = fmaxf(M, s_self);
            float res = 0.f;
            if (Mf != -INFINITY) {
                const float e = M != -INFINITY ? exp2_(M - Mf) : 0.f;
                const float w_self = self_here ? exp2_(s_self - Mf) : 0.f;
                const float v_self = self_here ? bf2f(vs_raw) : 0.f;
                res = ((O + L * bf2f(muv_raw)) * e + w_self * v_self) / (L * e + w_self);
            }
            static_cast<uint16_t *>(a.out)[((size_t)b * a.H + h) * D + tid] = f2bf(res);
        } else {
            float *rec = a.ws + (((size_t)b * a.H + h) * S + s) * (D + kPartialPad);
            rec[tid] = O;
            if (tid == 0) {
                rec[D] = M;
                rec[D + 1] = L;
            }
        }
    }
}

template <int D, int RK, int RV>
hipError_t launch_t(const DecodeArgs &a, hipStream_t st) {
    const unsigned blocks = (unsigned)a.B * a.H * a.S;
    hipLaunchKernelGGL((absorbed_kernel<D, RK, RV>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t st) {
#define LLA_CASE(RK, RV) \
    if (a.r_k == RK && a.r_v == RV) return launch_t<D, RK, RV>(a, st);
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

hipError_t launch_decode_absorbed(const DecodeArgs &a, hipStream_t st) {
    const int d = a.mode ? a.Dg / a.H : a.Dg;
    if (d == 128) return launch_d<128>(a, st);
    if (d == 64) return launch_d<64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace lla
