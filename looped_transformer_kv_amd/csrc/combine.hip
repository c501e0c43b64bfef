// combine.hip -- merges the per-split (o, m, l) partials of a decode call and adds the terms that
// are constant over the cached tokens.
//
// Partials hold, in the log2 domain, m = max score, l = sum_j 2^(s_j - m) and
// o = sum_j 2^(s_j - m) (c_v(j) W_up,t) over one split's cached tokens.  With the current token's
// own loop-t key/value (a reading of the pages: the token attends to itself), the output is
//   out = (sum_s 2^(m_s - M) o_s  +  L mu_t^V  +  2^(s_self - M) v_self) / (L + 2^(s_self - M)),
//   L = sum_s 2^(m_s - M) l_s,
// i.e. softmax attention over V_hat(j) = c_v(j) W_up,t + mu_t (pith.science paper page for
// "Looped Latent Attention", "What carries the argument").  For the flat comparator mu is absent.
// An empty context without a self term yields 0.
#include "lla_internal.h"

namespace lla {
namespace {

template <int D, typename TS>
__global__ __launch_bounds__(D) void combine_kernel(DecodeArgs a, int has_mu, int self_in_record) {
    __shared__ float red[D / 64 + 1];
    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh % a.H;
    const int i = threadIdx.x, lane = i & 63, wave = i >> 6;
    const float *rec0 = a.ws + (size_t)bh * a.S * (D + kPartialPad);

    float M = -INFINITY;
    for (int s = 0; s < a.S; ++s) M = fmaxf(M, rec0[(size_t)s * (D + kPartialPad) + D]);

    const bool has_self = a.k_self != nullptr;
    float s_self = -INFINITY, v_self = 0.f;
    if (has_self && self_in_record) {
        s_self = rec0[D + 2];
        v_self = ld_elt<TS>(static_cast<const TS *>(a.v_self) + (size_t)b * a.self_stride +
                            (size_t)h * D + i);
        M = fmaxf(M, s_self);
    } else if (has_self) {
        const TS *qp = static_cast<const TS *>(a.q) + ((size_t)b * a.H + h) * D;
        const TS *ks = static_cast<const TS *>(a.k_self) + (size_t)b * a.self_stride +
                       (size_t)h * D;
        const TS *vs = static_cast<const TS *>(a.v_self) + (size_t)b * a.self_stride +
                       (size_t)h * D;
        float prod = wave_sum(ld_elt<TS>(qp + i) * ld_elt<TS>(ks + i));
        if (lane == 0) red[wave] = prod;
        __syncthreads();
        float dot = 0.f;
        for (int w = 0; w < D / 64; ++w) dot += red[w];
        s_self = dot * a.scale_log2;
        v_self = ld_elt<TS>(vs + i);
        M = fmaxf(M, s_self);
    }

    float res = 0.f;
    if (M != -INFINITY) {
        float L = 0.f, O = 0.f;
        for (int s = 0; s < a.S; ++s) {
            const float *rec = rec0 + (size_t)s * (D + kPartialPad);
            const float e = exp2_(rec[D] - M);
            L += rec[D + 1] * e;
            O += rec[i] * e;
        }
        float mu = 0.f;
        if (has_mu) {
            const int g = a.mode ? 0 : h;
            const int col0 = a.mode ? h * D : 0;
            mu = ld_elt<TS>(static_cast<const TS *>(a.mu_v) + (size_t)g * a.T * a.Dg +
                            (size_t)a.t * a.Dg + col0 + i);
        }
        const float w_self = has_self ? exp2_(s_self - M) : 0.f;
        res = (O + L * mu + w_self * v_self) / (L + w_self);
    }
    st_elt<TS>(static_cast<TS *>(a.out) + (size_t)bh * D + i, res);
}

}  // namespace

hipError_t launch_combine(const DecodeArgs &a, int d, bool bf16, bool has_mu, bool self_in_record,
                          hipStream_t st) {
    const unsigned blocks = (unsigned)a.B * a.H;
    const int hm = has_mu ? 1 : 0, sr = self_in_record ? 1 : 0;
    if (d == 128) {
        if (bf16)
            hipLaunchKernelGGL((combine_kernel<128, uint16_t>), dim3(blocks), dim3(128), 0, st, a, hm, sr);
        else
            hipLaunchKernelGGL((combine_kernel<128, float>), dim3(blocks), dim3(128), 0, st, a, hm, sr);
    } else if (d == 64) {
        if (bf16)
            hipLaunchKernelGGL((combine_kernel<64, uint16_t>), dim3(blocks), dim3(64), 0, st, a, hm, sr);
        else
            hipLaunchKernelGGL((combine_kernel<64, float>), dim3(blocks), dim3(64), 0, st, a, hm, sr);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace lla
