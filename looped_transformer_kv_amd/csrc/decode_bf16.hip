// decode_bf16.hip -- fused latent decode attention, bf16 storage, fp32 accumulation, gfx950 MFMA.
//
// Computes, for loop t, sequence b, head h (pith.science paper page for "Looped Latent Attention",
// section "What carries the argument": x_hat_t = c W_up,t + mu_t, attention unchanged; abstract:
// K/V rebuilt only when attention reads them):
//   K_hat(j) = c_k(j) W_up,t^K (+ mu_t^K),  s_j = scale <q, K_hat(j)>
//   V_hat(j) = c_v(j) W_up,t^V (+ mu_t^V),  out = sum_j softmax(s)_j V_hat(j)
// Both reconstructions are real dense contractions over the latent rank, run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  mu_t enters exactly, as constants: <q, mu_t^K>
// is added to every cached score, and (sum_j p_j) mu_t^V is added by the combine kernel, so the
// MFMA tiles hold c W_up,t and the full K_hat / V_hat are never written anywhere.
//
// Work decomposition: one workgroup per (sequence b, head h, context split s); each of its waves
// takes 32-token chunks round-robin.  Per chunk and lane, latents are loaded straight from HBM
// into MFMA operand registers (16 bytes per lane, one contiguous span per chunk), so no LDS round
// trip is needed for the stream.
//   K side: A = W_up,t^K transposed (d x r_k), B = chunk latents (r_k x 32 tokens); the 32x32
//           result tile has tokens as columns, so <q, K_hat> is a 16-term in-lane dot product
//           plus one exchange between lane l and l^32.
//   V side: A = chunk latents (32 tokens x r_v), B = W_up,t^V (r_v x d); the tile has tokens as
//           rows, so p-weighted accumulation into o is in-lane; lanes l and l^32 are summed once
//           at the end.
// Online softmax in the log2 domain with one wave-wide max per chunk; the waves of a workgroup
// merge through LDS and write one (o, m, l) partial per split, finished by combine.hip.
#include <cstdlib>

#include "lla_internal.h"

namespace lla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32x32x16(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Latent registers of one 32-token chunk (this lane's 16-byte slices).
template <int KK, int KV>
struct Chunk {
    uint4 k[KK], v[KV];
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Eight fp32 values -> eight bf16 (round to nearest even, v_cvt_pk_bf16_f32) in one uint4.
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ uint4 pack8(const f32x16 &a, int base) {
    return make_uint4(pk_bf16(a[base + 0], a[base + 1]), pk_bf16(a[base + 2], a[base + 3]),
                      pk_bf16(a[base + 4], a[base + 5]), pk_bf16(a[base + 6], a[base + 7]));
}

template <int D, int RK, int RV, int WAVES, bool SMFMA>
__global__ __launch_bounds__(64 * WAVES)
__attribute__((amdgpu_waves_per_eu(SMFMA && RK + RV <= 64 ? 3 : 1)))
void decode_bf16_kernel(DecodeArgs a) {
    constexpr int MT = D / 32;                  // 32-column tiles over the head dim
    constexpr int KK = RK / 16, KV = RV / 16;   // MFMA k-steps over the latent ranks
    constexpr bool OCC3 = SMFMA && RK + RV <= 64;  // sized for 3 waves per SIMD
    constexpr bool WREG = !OCC3 && (KK + KV) * MT <= 16; // W_up operands kept in registers
    constexpr int RKP = RK + 8, RVP = RV + 8;   // padded LDS rows (keeps 16-byte alignment)

    __shared__ __align__(16) uint16_t sWk[D * RKP];   // W_up,t^K transposed: [i][k]
    __shared__ __align__(16) uint16_t sWv[D * RVP];   // W_up,t^V transposed: [i][k]
    __shared__ __align__(16) float sP[WAVES][32];
    __shared__ __align__(16) float sO[WAVES][D];
    __shared__ float sM[WAVES], sL[WAVES];
    __shared__ int sSlot[kMaxChunksPerSplit];         // chunk -> first token row in the pool

    const int S = a.S;
    const int id = blockIdx.x;
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
    {
        const int32_t *bt = a.block_table + (size_t)b * a.max_pages;
        for (int c = tid; c < nchunks; c += 64 * WAVES) {
            const int j = j_begin + 32 * c;
            const int page = bt[j / a.P];
            const bool bad = (unsigned)page >= (unsigned)a.n_pages;
            const int row = ((bad ? 0 : page) * a.G + g) * a.P + j % a.P;
            sSlot[c] = bad ? -row - 1 : row;   // negative marks an invalid page id
        }
    }

    // ---- stage W_up,t for this head's D columns, transposed, into LDS
    {
        const uint16_t *Wk = static_cast<const uint16_t *>(a.W_up_k) +
                             ((size_t)a.t * a.G + g) * RK * a.Dg + col0;
        const uint16_t *Wv = static_cast<const uint16_t *>(a.W_up_v) +
                             ((size_t)a.t * a.G + g) * RV * a.Dg + col0;
        for (int e = tid; e < RK * D; e += 64 * WAVES) {
            const int k = e / D, i = e - k * D;
            sWk[i * RKP + k] = Wk[(size_t)k * a.Dg + i];
        }
        for (int e = tid; e < RV * D; e += 64 * WAVES) {
            const int k = e / D, i = e - k * D;
            sWv[i * RVP + k] = Wv[(size_t)k * a.Dg + i];
        }
    }

    // ---- query in the K-tile row layout, pre-scaled by scale*log2(e); <q, mu_t^K>
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) + ((size_t)b * a.H + h) * D;
    // VALU scores: q rows 32M + 8bb + 4h2 + 0..3 of the K tile, fp32, pre-scaled.
    // MFMA scores: q as the A operand of S = q . K_hat^T, the same bf16 in every row m; k-slot
    // kk of lane half h2 in step (M, half) is d-row 32M + 16half + 8(kk/4) + 4h2 + kk%4, the
    // row the K_hat tile holds in element 8half + kk of that lane.
    float qs[SMFMA ? 1 : MT][16];
    uint4 qop[SMFMA ? MT : 1][2];
#pragma unroll
    for (int M = 0; M < MT; ++M)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const uint2 u = *reinterpret_cast<const uint2 *>(qp + 32 * M + 8 * bb + 4 * h2);
            if constexpr (SMFMA) {
                if (bb & 1) { qop[M][bb >> 1].z = u.x; qop[M][bb >> 1].w = u.y; }
                else        { qop[M][bb >> 1].x = u.x; qop[M][bb >> 1].y = u.y; }
            } else {
                qs[M][4 * bb + 0] = __uint_as_float(u.x << 16) * a.scale_log2;
                qs[M][4 * bb + 1] = __uint_as_float(u.x & 0xffff0000u) * a.scale_log2;
                qs[M][4 * bb + 2] = __uint_as_float(u.y << 16) * a.scale_log2;
                qs[M][4 * bb + 3] = __uint_as_float(u.y & 0xffff0000u) * a.scale_log2;
            }
        }
    float qm;
    {
        const uint16_t *muk = static_cast<const uint16_t *>(a.mu_k) +
                              (size_t)g * a.T * a.Dg + (size_t)a.t * a.Dg + col0;
        float acc = 0.f;
        for (int i = lane; i < D; i += 64) acc += bf2f(qp[i]) * bf2f(muk[i]);
        qm = wave_sum(acc) * a.scale_log2;
    }
    __syncthreads();

    // W_up operands: K tile M / V tile N, k-step ks; lane (l32, h2) holds rows 16ks+8h2 .. +7
    // of column 32*tile + l32.
    auto wk_op = [&](int M, int ks) {
        return *reinterpret_cast<const uint4 *>(&sWk[(32 * M + l32) * RKP + 16 * ks + 8 * h2]);
    };
    auto wv_op = [&](int N, int ks) {
        return *reinterpret_cast<const uint4 *>(&sWv[(32 * N + l32) * RVP + 16 * ks + 8 * h2]);
    };
    uint4 wkr[WREG ? MT * KK : 1], wvr[WREG ? MT * KV : 1];
    if constexpr (WREG) {
#pragma unroll
        for (int M = 0; M < MT; ++M)
#pragma unroll
            for (int ks = 0; ks < KK; ++ks) wkr[M * KK + ks] = wk_op(M, ks);
#pragma unroll
        for (int N = 0; N < MT; ++N)
#pragma unroll
            for (int ks = 0; ks < KV; ++ks) wvr[N * KV + ks] = wv_op(N, ks);
    }

    const uint16_t *kpool = static_cast<const uint16_t *>(a.k_pool);
    const uint16_t *vpool = static_cast<const uint16_t *>(a.v_pool);

    // 16-byte slices of chunk c: token row (slot + l32), latent entries 16ks + 8h2 .. +7
    auto load = [&](int c, Chunk<KK, KV> &x) {
        int row = sSlot[c];
        row = row < 0 ? -row - 1 : row;
        const uint16_t *ck = kpool + ((size_t)row + l32) * RK + 8 * h2;
        const uint16_t *cv = vpool + ((size_t)row + l32) * RV + 8 * h2;
#pragma unroll
        for (int ks = 0; ks < KK; ++ks) x.k[ks] = *reinterpret_cast<const uint4 *>(ck + 16 * ks);
#pragma unroll
        for (int ks = 0; ks < KV; ++ks) x.v[ks] = *reinterpret_cast<const uint4 *>(cv + 16 * ks);
    };

    float m_run = -INFINITY, l_lane = 0.f;
    float o[MT];
#pragma unroll
    for (int N = 0; N < MT; ++N) o[N] = 0.f;

    auto compute = [&](int c, Chunk<KK, KV> &x) {
        const int valid = j_end - (j_begin + 32 * c);   // >= 1, wave-uniform
        if (valid < 32) {
            // slots past the sequence end may hold anything (even NaN bit patterns)
            const bool keep = l32 < valid;
#pragma unroll
            for (int ks = 0; ks < KK; ++ks) x.k[ks] = keep ? x.k[ks] : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int ks = 0; ks < KV; ++ks) x.v[ks] = keep ? x.v[ks] : make_uint4(0, 0, 0, 0);
        }
        // K_hat tiles (d rows x 32 token columns) and the scores of this chunk
        f32x16 acc[MT];
#pragma unroll
        for (int M = 0; M < MT; ++M) {
            acc[M] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KK; ++ks)
                acc[M] = mfma32x32x16(WREG ? wkr[M * KK + ks] : wk_op(M, ks), x.k[ks], acc[M]);
        }
        float sc;                                   // token l32's score, in both lane halves
        if constexpr (SMFMA) {
            // K_hat (rounded to bf16) contracted with q on the matrix pipe: every row of the
            // result holds the 32 scores of the chunk, so no cross-lane step is needed.
            f32x16 sacc = {};
#pragma unroll
            for (int M = 0; M < MT; ++M) {
                sacc = mfma32x32x16(qop[M][0], pack8(acc[M], 0), sacc);
                sacc = mfma32x32x16(qop[M][1], pack8(acc[M], 8), sacc);
            }
            sc = sacc[0] * a.scale_log2 + qm;
        } else {
            float sp[MT];                           // independent chains, one per tile
#pragma unroll
            for (int M = 0; M < MT; ++M) {
                sp[M] = 0.f;
#pragma unroll
                for (int v = 0; v < 16; ++v) sp[M] += qs[M][v] * acc[M][v];
            }
            float tot = sp[0];
#pragma unroll
            for (int M = 1; M < MT; ++M) tot += sp[M];
            sc = add_swap32(tot) + qm;
        }
        if (valid < 32 && l32 >= valid) sc = -INFINITY;
        if (sSlot[c] < 0) sc = __builtin_nanf("");

        // V_hat tiles (32 token rows x d columns); independent of the softmax below, so the
        // matrix pipe works on them while the max / exp / p exchange runs
        f32x16 vacc[MT];
#pragma unroll
        for (int N = 0; N < MT; ++N) {
            vacc[N] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KV; ++ks)
                vacc[N] = mfma32x32x16(x.v[ks], WREG ? wvr[N * KV + ks] : wv_op(N, ks), vacc[N]);
        }

        // online softmax (log2 domain).  The running max only moves when some score of the
        // chunk exceeds it; otherwise the rescale factor is exactly 1 and the wave-wide max, the
        // exp of the old max and the rescale are skipped (a wave-uniform branch).
        if (__builtin_amdgcn_ballot_w64(sc > m_run) != 0) {
            // the two 16-lane rows of a lane half hold all 32 scores
            const float r = row16_max(sc);
            const float cmax = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 0)),
                                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 16)));
            const float m_new = fmaxf(m_run, cmax);
            const float alpha = exp2_(m_run - m_new);
            l_lane *= alpha;
#pragma unroll
            for (int N = 0; N < MT; ++N) o[N] *= alpha;
            m_run = m_new;
        }
        const float p = exp2_(sc - m_run);
        l_lane += (h2 == 0 ? p : 0.f);

        // p of tokens 8*(v/4) + 4*h2 + (v%4): the V tile's row layout
        if (h2 == 0) sP[wave][l32] = p;
        __builtin_amdgcn_wave_barrier();
        float pr[16];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const float4 t4 = *reinterpret_cast<const float4 *>(&sP[wave][8 * bb + 4 * h2]);
            pr[4 * bb + 0] = t4.x; pr[4 * bb + 1] = t4.y;
            pr[4 * bb + 2] = t4.z; pr[4 * bb + 3] = t4.w;
        }

        // p-weighted V_hat into o
#pragma unroll
        for (int N = 0; N < MT; ++N)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[N] += pr[v] * vacc[N][v];
        __builtin_amdgcn_wave_barrier();
    };

    // ---- main loop: chunks wave, wave + WAVES, ...; the next chunk's latents are in flight
    // while the current one is computed.  Prefetch indices are clamped, so the instruction
    // stream has no data-dependent branches around the loads.
    if constexpr (KK + KV <= 4) {
        // small ranks: 3 KB per wave-chunk, so keep a second chunk in flight
        if (wave < nchunks) {
            Chunk<KK, KV> A, Bq;
            int c = wave;
            load(c, A);
            load(min(c + WAVES, nchunks - 1), Bq);
            while (true) {
                compute(c, A);
                load(min(c + 2 * WAVES, nchunks - 1), A);
                c += WAVES;
                if (c >= nchunks) break;
                compute(c, Bq);
                load(min(c + 2 * WAVES, nchunks - 1), Bq);
                c += WAVES;
                if (c >= nchunks) break;
            }
        }
    } else {
        // large ranks: one chunk is already KK+KV 1-KB loads per wave; registers go to occupancy
        for (int c = wave; c < nchunks; c += WAVES) {
            Chunk<KK, KV> A;
            load(c, A);
            compute(c, A);
        }
    }

    // ---- merge lanes, then waves, into this split's partial
    const float l_w = wave_sum(l_lane);
#pragma unroll
    for (int N = 0; N < MT; ++N) o[N] = add_swap32(o[N]);
    if (h2 == 0) {
#pragma unroll
        for (int N = 0; N < MT; ++N) sO[wave][32 * N + l32] = o[N];
    }
    if (lane == 0) {
        sM[wave] = m_run;
        sL[wave] = l_w;
    }
    // a single split finishes the output here (same arithmetic as combine.hip): the current
    // token's own loop-t key/value joins the softmax and (sum of cached weights) mu_t^V is added
    float s_self = -INFINITY;
    const bool has_self = a.k_self != nullptr;
    if (S == 1 && has_self) {
        const uint16_t *ks = static_cast<const uint16_t *>(a.k_self) + (size_t)b * a.self_stride +
                             (size_t)h * D;
        float acc = 0.f;
        for (int i = lane; i < D; i += 64) acc += bf2f(qp[i]) * bf2f(ks[i]);
        s_self = wave_sum(acc) * a.scale_log2;
    }
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
                const uint16_t *muv = static_cast<const uint16_t *>(a.mu_v) +
                                      (size_t)g * a.T * a.Dg + (size_t)a.t * a.Dg + col0;
                float w_self = 0.f, v_self = 0.f;
                if (has_self) {
                    w_self = exp2_(s_self - M);
                    v_self = bf2f(static_cast<const uint16_t *>(a.v_self)[
                        (size_t)b * a.self_stride + (size_t)h * D + tid]);
                }
                res = (O + L * bf2f(muv[tid]) + w_self * v_self) / (L + w_self);
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

// Scores on the vector ALU (fp32 FMAs, default) or on the matrix pipe (LLA_SCORE_MFMA=1).
bool score_on_valu() {
    static const bool v = [] {
        const char *e = std::getenv("LLA_SCORE_MFMA");
        return !(e && e[0] == '1');
    }();
    return v;
}

template <int D, int RK, int RV, int WAVES>
hipError_t launch_t(const DecodeArgs &a, hipStream_t st) {
    const unsigned blocks = (unsigned)a.B * a.H * a.S;
    if (score_on_valu())
        hipLaunchKernelGGL((decode_bf16_kernel<D, RK, RV, WAVES, false>), dim3(blocks),
                           dim3(64 * WAVES), 0, st, a);
    else
        hipLaunchKernelGGL((decode_bf16_kernel<D, RK, RV, WAVES, true>), dim3(blocks),
                           dim3(64 * WAVES), 0, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t st) {
#define LLA_CASE(RK, RV) \
    if (a.r_k == RK && a.r_v == RV) return launch_t<D, RK, RV, 4>(a, st);
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

hipError_t launch_decode_bf16(const DecodeArgs &a, int waves, hipStream_t st) {
    (void)waves;
    const int d = a.mode ? a.Dg / a.H : a.Dg;
    if (d == 128) return launch_d<128>(a, st);
    if (d == 64) return launch_d<64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace lla
