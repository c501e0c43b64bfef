// encode.hip -- encode a finished token's loop trajectories into latents and append them.
//
// pith.science paper page for "Looped Latent Attention", "What carries the argument": for each
// layer, head and axis the T per-loop vectors are stacked and centred and projected,
// c = (x - mu) W_down.  LLA-2D (abstract) stacks all heads of the layer into one vector; the
// stacking order used here is (t, h, i), a reading, which makes the LLA-2D stacked vector of a
// token simply its contiguous [T][H][d] staging row.
//
// One launch covers both axes.  A workgroup of 256 threads owns (axis, group g, 32 latent
// columns, 8 sequences): thread (row, col) accumulates c[b0 + row][k0 + col].  The stacked axis
// is walked in stages of XC elements: the 8 centred stacked rows (x - mu, fp32) and the
// XC x 32 tile of W_down are staged through LDS with 16-byte coalesced loads, then each thread
// runs XC fp32 FMAs from LDS.  Accumulation order is fixed (increasing stacked index).  The result
// is rounded once to the pool dtype (bf16 round-to-nearest-even) and written to the slot of
// logical position write_pos[b]; the optional fp32 copy keeps the value before rounding.
#include "lla_internal.h"

namespace lla {
namespace {

constexpr int KC = 32;    // latent columns per workgroup
constexpr int BR = 8;     // sequences per workgroup
constexpr int XC = 256;   // stacked elements per LDS stage
constexpr int NT = KC * BR;

struct EncodePair {
    EncodeArgs ax[2];
    int blocks_k;         // workgroups of the K axis (the V axis follows)
};

template <typename TS>
__device__ __forceinline__ void load8(const TS *p, float *v);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t *p, float *v) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void load8<float>(const float *p, float *v) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename TS>
__global__ __launch_bounds__(NT) void encode_kernel(EncodePair pr) {
    __shared__ __align__(16) float sX[BR][XC];        // centred stacked rows
    __shared__ __align__(16) float sW[XC][KC + 1];    // W_down tile (fp32), padded rows

    int blk = blockIdx.x;
    const int axis = blk < pr.blocks_k ? 0 : 1;
    if (axis) blk -= pr.blocks_k;
    const EncodeArgs &a = pr.ax[axis];
    const int ktiles = (a.r + KC - 1) / KC;
    const int btiles = (a.B + BR - 1) / BR;
    const int kt = blk % ktiles;
    const int bt_ = (blk / ktiles) % btiles;
    const int g = blk / (ktiles * btiles);
    const int k0 = kt * KC, b0 = bt_ * BR;

    const int tid = threadIdx.x;
    const int col = tid % KC, row = tid / KC;
    const size_t X = (size_t)a.T * a.Dg;
    const TS *x = static_cast<const TS *>(a.x);
    const TS *W = static_cast<const TS *>(a.W_down) + (size_t)g * X * a.r;
    const TS *mu = static_cast<const TS *>(a.mu) + (size_t)g * X;

    float acc = 0.f;
    for (size_t x0 = 0; x0 < X; x0 += XC) {
        const int nx = (int)((X - x0) < (size_t)XC ? (X - x0) : (size_t)XC);   // multiple of 8
        __syncthreads();
        // centred rows: 8 consecutive stacked elements per thread-step (never crossing a d-row)
        for (int e = tid; e < BR * (XC / 8); e += NT) {
            const int br = e / (XC / 8), xx = (e % (XC / 8)) * 8;
            float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            const int b = b0 + br;
            if (b < a.B && xx < nx) {
                const size_t xi = x0 + xx;
                size_t off;
                if (a.mode) {
                    off = (size_t)b * X + xi;                      // (t, h, i) order
                } else {
                    const size_t t = xi / a.d, i = xi % a.d;       // (t, i) of head g
                    off = (((size_t)b * a.T + t) * a.H + g) * a.d + i;
                }
                float m[8];
                load8<TS>(x + off, v);
                load8<TS>(mu + xi, m);
#pragma unroll
                for (int q = 0; q < 8; ++q) v[q] -= m[q];
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) sX[br][xx + q] = v[q];
        }
        // W_down rows x0 .. x0+nx-1, columns k0 .. k0+31
        for (int e = tid; e < XC * KC; e += NT) {
            const int xx = e / KC, kk = e % KC;
            float w = 0.f;
            if (xx < nx && k0 + kk < a.r) w = ld_elt<TS>(W + (x0 + xx) * a.r + k0 + kk);
            sW[xx][kk] = w;
        }
        __syncthreads();
#pragma unroll 8
        for (int xx = 0; xx < nx; ++xx) acc += sX[row][xx] * sW[xx][col];
    }

    const int b = b0 + row, k = k0 + col;
    if (b >= a.B || k >= a.r) return;
    if (a.c_out) a.c_out[((size_t)b * a.G + g) * a.r + k] = acc;
    const int pos = a.write_pos[b];
    if (pos < 0 || pos >= a.max_pages * a.P) return;
    const int page = a.block_table[(size_t)b * a.max_pages + pos / a.P];
    if ((unsigned)page >= (unsigned)a.n_pages) return;
    st_elt<TS>(static_cast<TS *>(a.pool) + (((size_t)page * a.G + g) * a.P + pos % a.P) * a.r + k,
               acc);
}

int blocks_of(const EncodeArgs &a) {
    return a.G * ((a.r + KC - 1) / KC) * ((a.B + BR - 1) / BR);
}

}  // namespace

hipError_t launch_encode(const EncodeArgs &k_axis, const EncodeArgs &v_axis, bool bf16,
                         hipStream_t st) {
    EncodePair pr;
    pr.ax[0] = k_axis;
    pr.ax[1] = v_axis;
    pr.blocks_k = blocks_of(k_axis);
    const unsigned blocks = (unsigned)(pr.blocks_k + blocks_of(v_axis));
    if (bf16)
        hipLaunchKernelGGL(encode_kernel<uint16_t>, dim3(blocks), dim3(NT), 0, st, pr);
    else
        hipLaunchKernelGGL(encode_kernel<float>, dim3(blocks), dim3(NT), 0, st, pr);
    return hipGetLastError();
}

}  // namespace lla
