// encode.hip -- encode a finished token's loop trajectories into latents and append them.
//
// pith.science paper page for "Looped Latent Attention", "What carries the argument": for each
// layer, head and axis the T per-loop vectors are stacked and centred and projected,
// c = (x - mu) W_down.  LLA-2D (abstract) stacks all heads of the layer into one vector; the
// stacking order used here is (t, h, i), a reading, which makes the LLA-2D stacked vector of a
// token simply its contiguous [T][H][d] staging row.
//
// One workgroup per (group g, 64 output columns).  256 threads = 64 columns x 4 row groups; the
// batch is walked in tiles of 64 rows.  Centred stacked values are staged through LDS 64 elements
// at a time and W_down rows are read coalesced across the columns; accumulation is fp32 in a
// fixed order (increasing stacked index).  The result is rounded once to the pool dtype (bf16
// round-to-nearest-even) and written to the slot of logical position write_pos[b].
#include "lla_internal.h"

namespace lla {
namespace {

constexpr int KC = 64;   // output columns per block
constexpr int RG = 4;    // row groups per block
constexpr int BT = 64;   // batch rows per tile
constexpr int XC = 64;   // stacked elements per LDS stage

template <typename TS>
__global__ __launch_bounds__(KC * RG) void encode_kernel(EncodeArgs a) {
    __shared__ float sX[BT][XC + 1];
    const int g = blockIdx.x;
    const int tid = threadIdx.x;
    const int col = tid % KC, rg = tid / KC;
    const int k = blockIdx.y * KC + col;
    const size_t X = (size_t)a.T * a.Dg;
    const TS *x = static_cast<const TS *>(a.x);
    const TS *W = static_cast<const TS *>(a.W_down) + (size_t)g * X * a.r;
    const TS *mu = static_cast<const TS *>(a.mu) + (size_t)g * X;
    TS *pool = static_cast<TS *>(a.pool);

    for (int b0 = 0; b0 < a.B; b0 += BT) {
        const int nb = min(BT, a.B - b0);
        float acc[BT / RG];
#pragma unroll
        for (int i = 0; i < BT / RG; ++i) acc[i] = 0.f;
        for (size_t x0 = 0; x0 < X; x0 += XC) {
            const int nx = (int)min((size_t)XC, X - x0);
            __syncthreads();
            for (int e = tid; e < BT * XC; e += KC * RG) {
                const int bb = e / XC, xx = e % XC;
                float v = 0.f;
                if (bb < nb && xx < nx) {
                    const size_t xi = x0 + xx;
                    size_t off;
                    if (a.mode) {
                        off = (size_t)(b0 + bb) * X + xi;              // (t, h, i) order
                    } else {
                        const size_t t = xi / a.d, i = xi % a.d;        // (t, i) of head g
                        off = (((size_t)(b0 + bb) * a.T + t) * a.H + g) * a.d + i;
                    }
                    v = ld_elt<TS>(x + off) - ld_elt<TS>(mu + xi);
                }
                sX[bb][xx] = v;
            }
            __syncthreads();
            if (k < a.r) {
                for (int xx = 0; xx < nx; ++xx) {
                    const float w = ld_elt<TS>(W + (x0 + xx) * a.r + k);
#pragma unroll
                    for (int i = 0; i < BT / RG; ++i) acc[i] += sX[rg + RG * i][xx] * w;
                }
            }
        }
        if (k < a.r) {
#pragma unroll
            for (int i = 0; i < BT / RG; ++i) {
                const int bb = rg + RG * i;
                if (bb >= nb) continue;
                const int b = b0 + bb;
                if (a.c_out) a.c_out[((size_t)b * a.G + g) * a.r + k] = acc[i];
                const int pos = a.write_pos[b];
                if (pos < 0 || pos >= a.max_pages * a.P) continue;
                const int page = a.block_table[(size_t)b * a.max_pages + pos / a.P];
                if ((unsigned)page >= (unsigned)a.n_pages) continue;
                st_elt<TS>(pool + (((size_t)page * a.G + g) * a.P + pos % a.P) * a.r + k, acc[i]);
            }
        }
    }
}

}  // namespace

hipError_t launch_encode(const EncodeArgs &a, bool bf16, hipStream_t st) {
    const dim3 grid(a.G, (a.r + KC - 1) / KC);
    if (bf16)
        hipLaunchKernelGGL(encode_kernel<uint16_t>, grid, dim3(KC * RG), 0, st, a);
    else
        hipLaunchKernelGGL(encode_kernel<float>, grid, dim3(KC * RG), 0, st, a);
    return hipGetLastError();
}

}  // namespace lla
