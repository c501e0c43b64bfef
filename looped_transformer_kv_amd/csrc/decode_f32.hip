// decode_f32.hip -- latent decode attention with fp32 storage and fp32 arithmetic (VALU).
//
// Same operation as decode_bf16.hip (pith.science paper page for "Looped Latent Attention",
// "What carries the argument": x_hat_t = c W_up,t + mu_t; attention unchanged), for fp32 caches.
// There is no fp32-input MFMA shape that pays off at these ranks, and fp32 caches are small, so
// this kernel uses plain fp32 FMAs and keeps full fp32 accuracy throughout.
//
// One workgroup of 256 threads per (sequence, head, split).  W_up,t (this head's columns) and the
// scaled query sit in LDS.  Tokens are processed 256 at a time: each thread rebuilds one token's
// K_hat and scores it; the block then updates the running max, and for V each thread owns one
// output column and a stride of the block's tokens.
#include "lla_internal.h"

namespace lla {
namespace {

constexpr int kThreads = 256;

__device__ float block_reduce(float v, float *red, bool is_max) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = is_max ? wave_max(v) : wave_sum(v);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < kThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
    return r;
}

// RKC, RVC: the latent ranks when known at compile time (0: read from the arguments).  Known ranks
// let the rank loops unroll, so a token's latent row is read once into registers instead of once
// per head-dim element; the arithmetic and its order are the same either way.
template <int D, int RKC, int RVC>
__global__ __launch_bounds__(kThreads) void decode_f32_kernel(DecodeArgs a) {
    extern __shared__ float smem[];
    const int RK = RKC ? RKC : a.r_k, RV = RVC ? RVC : a.r_v;
    float *sWk = smem;               // [RK][D]
    float *sWv = sWk + RK * D;       // [RV][D]
    float *sQ = sWv + RV * D;        // [D]  q * scale * log2(e)
    float *sPb = sQ + D;             // [kThreads] softmax weights of the current token block
    float *sO = sPb + kThreads;      // [kThreads] partial output columns
    float *red = sO + kThreads;      // [8] reduction scratch

    const int S = a.S;
    const int id = xcd_work_item(blockIdx.x, gridDim.x);
    const int s = id % S;
    const int h = (id / S) % a.H;
    const int b = id / (S * a.H);
    const int tid = threadIdx.x;
    const int g = a.mode ? 0 : h;
    const int col0 = a.mode ? h * D : 0;

    const float *Wk = static_cast<const float *>(a.W_up_k) + ((size_t)a.t * a.G + g) * RK * a.Dg;
    const float *Wv = static_cast<const float *>(a.W_up_v) + ((size_t)a.t * a.G + g) * RV * a.Dg;
    for (int e = tid; e < RK * D; e += kThreads)
        sWk[e] = Wk[(size_t)(e / D) * a.Dg + col0 + e % D];
    for (int e = tid; e < RV * D; e += kThreads)
        sWv[e] = Wv[(size_t)(e / D) * a.Dg + col0 + e % D];
    const float *qp = static_cast<const float *>(a.q) + ((size_t)b * a.H + h) * D;
    const float *muk = static_cast<const float *>(a.mu_k) + (size_t)g * a.T * a.Dg +
                       (size_t)a.t * a.Dg + col0;
    float qmu = 0.f;
    for (int i = tid; i < D; i += kThreads) {
        sQ[i] = qp[i] * a.scale_log2;
        qmu += qp[i] * muk[i];
    }
    qmu = block_reduce(qmu, red, false) * a.scale_log2;   // contains __syncthreads

    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
    const int j_begin = s * a.tokens_per_split;
    const int j_end = min(j_begin + a.tokens_per_split, len);
    const float *kpool = static_cast<const float *>(a.k_pool);
    const float *vpool = static_cast<const float *>(a.v_pool);
    const int32_t *bt = a.block_table + (size_t)b * a.max_pages;

    constexpr int NP = kThreads / D;   // token strides per output column
    const int col = tid % D, part = tid / D;
    float m_run = -INFINITY, l_run = 0.f, o = 0.f;

    for (int jb = j_begin; jb < j_end; jb += kThreads) {
        const int j = jb + tid;
        float sc = -INFINITY;
        if (j < j_end) {
            int page = bt[j / a.P];
            const bool bad = (unsigned)page >= (unsigned)a.n_pages;
            page = bad ? 0 : page;
            const float *ck = kpool + (((size_t)page * a.G + g) * a.P + j % a.P) * RK;
            float dot = 0.f;
            for (int i = 0; i < D; ++i) {
                float kh = 0.f;
                for (int k = 0; k < RK; ++k) kh += ck[k] * sWk[k * D + i];
                dot += sQ[i] * kh;
            }
            sc = bad ? __builtin_nanf("") : dot + qmu;
        }
        const float m_new = fmaxf(m_run, block_reduce(sc, red, true));
        const float alpha = exp2_(m_run - m_new);
        const float p = exp2_(sc - m_new);
        const float psum = block_reduce(p, red, false);
        l_run = l_run * alpha + psum;
        m_run = m_new;
        sPb[tid] = p;
        __syncthreads();
        o *= alpha;
        const int nb = min(kThreads, j_end - jb);
        for (int jj = part; jj < nb; jj += NP) {
            const int jt = jb + jj;
            int page = bt[jt / a.P];
            page = (unsigned)page >= (unsigned)a.n_pages ? 0 : page;
            const float *cv = vpool + (((size_t)page * a.G + g) * a.P + jt % a.P) * RV;
            float vh = 0.f;
            for (int k = 0; k < RV; ++k) vh += cv[k] * sWv[k * D + col];
            o += sPb[jj] * vh;
        }
        __syncthreads();
    }
    sO[tid] = o;
    __syncthreads();
    if (tid < D) {
        float O = 0.f;
        for (int pp = 0; pp < NP; ++pp) O += sO[pp * D + tid];
        float *rec = a.ws + (((size_t)b * a.H + h) * S + s) * (D + kPartialPad);
        rec[tid] = O;
        if (tid == 0) {
            rec[D] = m_run;
            rec[D + 1] = l_run;
        }
    }
}

}  // namespace

size_t decode_f32_lds_bytes(int d, int r_k, int r_v) {
    return sizeof(float) * ((size_t)(r_k + r_v) * d + d + 2 * kThreads + 8);
}

hipError_t launch_decode_f32(const DecodeArgs &a, hipStream_t st) {
    const int d = a.mode ? a.Dg / a.H : a.Dg;
    const unsigned blocks = (unsigned)a.B * a.H * a.S;
    const size_t lds = decode_f32_lds_bytes(d, a.r_k, a.r_v);
    if (d == 64 && a.r_k == 8 && a.r_v == 16)   // the small fp32 codec of the tiny configuration
        hipLaunchKernelGGL((decode_f32_kernel<64, 8, 16>), dim3(blocks), dim3(kThreads), lds, st, a);
    else if (d == 128)
        hipLaunchKernelGGL((decode_f32_kernel<128, 0, 0>), dim3(blocks), dim3(kThreads), lds, st, a);
    else if (d == 64)
        hipLaunchKernelGGL((decode_f32_kernel<64, 0, 0>), dim3(blocks), dim3(kThreads), lds, st, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace lla
