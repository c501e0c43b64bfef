// flat.hip -- decode attention over an uncompressed, paged loop-t K/V cache (the comparator).
//
// The loop-indexed cache the latent store replaces (Figure 1 caption of "Looped Latent
// Attention": each recurrent step t contributes its own (K_t, V_t), so loop t's attention reads
// exactly those).  Pure HBM streaming at about one flop per byte, so this is a VALU kernel laid
// out for coalescing: a token's d-vector is read by D/8 (bf16) or D/4 (fp32) lanes with 16-byte
// loads, every lane group keeps its own online-softmax state (no cross-group traffic in the loop).
// A wave takes whole 32-token chunks; the split's page slots are resolved into LDS once, so a
// chunk's K and V (two contiguous runs) are requested with no dependent lookup in between.
#include "lla_internal.h"

namespace lla {
namespace {

template <int D, typename TS, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void flat_kernel(DecodeArgs a) {
    constexpr int EPL = 16 / sizeof(TS);    // elements per lane per 16-byte load
    constexpr int LPT = D / EPL;            // lanes per token
    constexpr int TPW = 64 / LPT;           // tokens per wave step
    constexpr int U = 32 / TPW;             // steps per 32-token chunk
    static_assert(LPT >= 1 && LPT <= 64 && 64 % LPT == 0 && U >= 1, "lane layout");

    __shared__ __align__(16) float sO[WAVES][D];
    __shared__ float sM[WAVES], sL[WAVES];
    __shared__ int sRow[kMaxChunksPerSplit];   // chunk -> first token row of its page slot

    const int S = a.S;
    const int id = xcd_work_item(blockIdx.x, gridDim.x);
    const int s = id % S;
    const int h = (id / S) % a.H;
    const int b = id / (S * a.H);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane / LPT, sub = lane % LPT;

    const TS *qp = static_cast<const TS *>(a.q) + ((size_t)b * a.H + h) * D + sub * EPL;
    float qv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] = ld_elt<TS>(qp + e) * a.scale_log2;

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
            const int row = ((bad ? 0 : page) * a.H + h) * a.P + j % a.P;
            sRow[c] = bad ? -row - 1 : row;   // negative marks an invalid page id
        }
    }
    __syncthreads();
    const TS *kpool = static_cast<const TS *>(a.k_pool);
    const TS *vpool = static_cast<const TS *>(a.v_pool);

    float m = -INFINITY, l = 0.f, o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;

    // each wave takes whole 32-token chunks (one page slot run), round-robin
    for (int c = wave; c < nchunks; c += WAVES) {
        int row = sRow[c];
        const bool bad = row < 0;
        row = bad ? -row - 1 : row;
        const int valid = j_end - (j_begin + 32 * c);   // >= 1
        const size_t base = (size_t)row * D + sub * EPL;
        uint4 kr[U], vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t off = base + (size_t)(u * TPW + grp) * D;
            kr[u] = *reinterpret_cast<const uint4 *>(kpool + off);
            vr[u] = *reinterpret_cast<const uint4 *>(vpool + off);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = u * TPW + grp < valid;
            const TS *kk = reinterpret_cast<const TS *>(&kr[u]);
            const TS *vv = reinterpret_cast<const TS *>(&vr[u]);
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) dot += qv[e] * ld_elt<TS>(kk + e);
            dot = group_sum<LPT>(dot);
            float sc = ok ? dot : -INFINITY;
            if (bad) sc = __builtin_nanf("");
            const float m_new = fmaxf(m, sc);
            const float alpha = (m == m_new) ? 1.f : exp2_(m - m_new);
            const float p = (sc == -INFINITY) ? 0.f : exp2_(sc - m_new);
            l = l * alpha + p;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                // slots past the sequence end may hold anything: never let them reach o
                const float v = ok ? ld_elt<TS>(vv + e) : 0.f;
                o[e] = o[e] * alpha + p * v;
            }
            m = m_new;
        }
    }

    // merge the lane groups of the wave (lanes that differ in the group bits)
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
        const float m2 = __shfl_xor(m, off, 64);
        const float l2 = __shfl_xor(l, off, 64);
        const float M = fmaxf(m, m2);
        const float e1 = (m == -INFINITY) ? 0.f : exp2_(m - M);
        const float e2 = (m2 == -INFINITY) ? 0.f : exp2_(m2 - M);
        l = l * e1 + l2 * e2;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float o2 = __shfl_xor(o[e], off, 64);
            o[e] = o[e] * e1 + o2 * e2;
        }
        m = M;
    }
    if (grp == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) sO[wave][sub * EPL + e] = o[e];
        if (sub == 0) {
            sM[wave] = m;
            sL[wave] = l;
        }
    }
    __syncthreads();
    for (int i = tid; i < D; i += 64 * WAVES) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sM[w]);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                const float e = exp2_(sM[w] - M);
                L += sL[w] * e;
                O += sO[w][i] * e;
            }
        }
        float *rec = a.ws + (((size_t)b * a.H + h) * S + s) * (D + kPartialPad);
        rec[i] = O;
        if (i == 0) {
            rec[D] = M;
            rec[D + 1] = L;
        }
    }
}

template <int D, typename TS>
hipError_t launch_t(const DecodeArgs &a, hipStream_t st) {
    const unsigned blocks = (unsigned)a.B * a.H * a.S;
    hipLaunchKernelGGL((flat_kernel<D, TS, 4>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_flat(const DecodeArgs &a, int d, bool bf16, hipStream_t st) {
    if (d == 128) return bf16 ? launch_t<128, uint16_t>(a, st) : launch_t<128, float>(a, st);
    if (d == 64) return bf16 ? launch_t<64, uint16_t>(a, st) : launch_t<64, float>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace lla
