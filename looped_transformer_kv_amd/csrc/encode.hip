// encode.hip -- encode a finished token's loop trajectories into latents and append them.
//
// pith.science paper page for "Looped Latent Attention", "What carries the argument": a token's
// T loop-step vectors of one layer, head and axis are joined end to end into one vector x of
// length T d, the codec mean mu is subtracted and W_down maps the rest to the rank-r latent,
// c = (x - mu) W_down.  LLA-2D (abstract) stacks all heads of the layer into one vector; the
// stacking order used here is (t, h, i), a reading, which makes the LLA-2D stacked vector of a
// token simply its contiguous [T][H][d] staging row.
//
// One launch covers both axes.  bf16 caches use the matrix-core kernel below; fp32 caches use
// this vector kernel: a workgroup of 256 threads owns (axis, group g, 32 latent
// columns, 32 sequences); thread (row group rg, column col) accumulates the four outputs
// c[b0 + rg + 8i][k0 + col], i = 0..3, in four independent fp32 chains.  The stacked axis is
// walked in stages of XC elements: the centred stacked rows (x - mu, fp32) and the XC x 32 tile
// of W_down (storage dtype) are staged through LDS with 16-byte loads, and the next stage's loads
// are in flight while the current stage is multiplied.  Every output is summed in increasing
// stacked index.  The result is rounded once to the pool dtype (bf16 round-to-nearest-even) and
// written to the slot of logical position write_pos[b]; the optional fp32 copy keeps the value
// before rounding.  A chunk of several tokens per sequence (bulk encode after a prefill) is the
// same contraction over more rows: row i of sequence b goes to write_pos[b] + i, and rows past
// the sequence's chunk size are neither stored nor copied out.
#include "lla_internal.h"

namespace lla {
namespace {

constexpr int KC = 32;    // latent columns per workgroup
constexpr int RG = 8;     // row groups
constexpr int RPT = 4;    // rows per thread
constexpr int BR = RG * RPT;   // sequences per workgroup
constexpr int NT = KC * RG;

struct EncodePair {
    EncodeArgs ax[2];
    int blocks_k;         // workgroups of the K axis (the V axis follows)
    int rows;             // encode_mfma_kernel: rows per workgroup (32, 16, 8 or 4)
};

// 16 bytes of fp32 storage -> float values
__device__ __forceinline__ void unpack(const uint4 u, float *v) {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
}

// fp32 codecs (bf16 ones take encode_mfma_kernel below)
__global__ __launch_bounds__(NT) void encode_kernel(EncodePair pr) {
    using TS = float;
    constexpr int XC = 128;                              // 16 KB + 17 KB of LDS
    constexpr int EPV = 16 / sizeof(TS);                 // elements per 16-byte load
    constexpr int XL = BR * XC / EPV / NT;               // x loads per thread per stage
    constexpr int WL = XC * KC / EPV / NT;               // W loads per thread per stage
    constexpr int WROW = KC + 2 * EPV;                   // padded LDS row (keeps 16 B alignment)
    __shared__ __align__(16) float sX[BR][XC];
    __shared__ __align__(16) TS sW[XC][WROW];

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
    const int col = tid % KC, rg = tid / KC;
    const int X = a.T * a.Dg;
    const TS *x = static_cast<const TS *>(a.x);
    const TS *W = static_cast<const TS *>(a.W_down) + (size_t)g * X * a.r;
    const TS *mu = static_cast<const TS *>(a.mu) + (size_t)g * X;
    // W rows start 16-byte aligned when r is a multiple of the vector width
    const bool wvec = (a.r % EPV) == 0 && (reinterpret_cast<uintptr_t>(W) & 15) == 0;

    uint4 xr[XL], mr[XL], wr[WL];
    // issue the global loads of the stage starting at x0 (zeros outside the problem)
    auto fetch = [&](int x0) {
#pragma unroll
        for (int u = 0; u < XL; ++u) {
            const int e = tid + u * NT;
            const int br = e / (XC / EPV), xx = (e % (XC / EPV)) * EPV;
            const int b = b0 + br;
            xr[u] = mr[u] = make_uint4(0, 0, 0, 0);
            if (b < a.B && x0 + xx < X) {
                const int xi = x0 + xx;
                size_t off;
                if (a.mode) {
                    off = (size_t)b * X + xi;                               // (t, h, i) order
                } else {
                    const int t = xi / a.d, i = xi - t * a.d;               // (t, i) of head g
                    off = (((size_t)b * a.T + t) * a.H + g) * a.d + i;
                }
                xr[u] = *reinterpret_cast<const uint4 *>(x + off);
                mr[u] = *reinterpret_cast<const uint4 *>(mu + xi);
            }
        }
#pragma unroll
        for (int u = 0; u < WL; ++u) {
            const int e = tid + u * NT;
            const int xx = e / (KC / EPV), kk = (e % (KC / EPV)) * EPV;
            wr[u] = make_uint4(0, 0, 0, 0);
            const int xi = x0 + xx, k = k0 + kk;
            if (xi < X && k < a.r) {
                const TS *src = W + (size_t)xi * a.r + k;
                if (wvec && k + EPV <= a.r) {
                    wr[u] = *reinterpret_cast<const uint4 *>(src);
                } else {
                    TS tmp[EPV];
#pragma unroll
                    for (int q = 0; q < EPV; ++q) tmp[q] = (k + q < a.r) ? src[q] : TS(0);
                    wr[u] = *reinterpret_cast<const uint4 *>(tmp);
                }
            }
        }
    };
    // write the fetched stage into LDS (x centred in fp32, W in its storage type)
    auto stage = [&]() {
#pragma unroll
        for (int u = 0; u < XL; ++u) {
            const int e = tid + u * NT;
            const int br = e / (XC / EPV), xx = (e % (XC / EPV)) * EPV;
            float v[8], m[8];
            unpack(xr[u], v);
            unpack(mr[u], m);
#pragma unroll
            for (int q = 0; q < EPV; ++q) sX[br][xx + q] = v[q] - m[q];
        }
#pragma unroll
        for (int u = 0; u < WL; ++u) {
            const int e = tid + u * NT;
            const int xx = e / (KC / EPV), kk = (e % (KC / EPV)) * EPV;
            *reinterpret_cast<uint4 *>(&sW[xx][kk]) = wr[u];
        }
    };

    float acc[RPT] = {0.f, 0.f, 0.f, 0.f};
    fetch(0);
    for (int x0 = 0; x0 < X; x0 += XC) {
        __syncthreads();                 // previous stage fully consumed
        stage();
        __syncthreads();
        if (x0 + XC < X) fetch(x0 + XC); // next stage in flight during the FMAs below
        const int nx = min(XC, X - x0);
        for (int xx = 0; xx < nx; xx += 4) {
            float w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = ld_elt<TS>(&sW[xx + q][col]);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const float4 xv = *reinterpret_cast<const float4 *>(&sX[rg + RG * i][xx]);
                acc[i] += xv.x * w[0];
                acc[i] += xv.y * w[1];
                acc[i] += xv.z * w[2];
                acc[i] += xv.w * w[3];
            }
        }
    }

    const int k = k0 + col;
    if (k >= a.r) return;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int b = b0 + rg + RG * i;
        if (b >= a.B) continue;
        int seq, pos;
        if (!encode_row(a, b, seq, pos)) continue;           // row past its sequence's chunk
        if (a.c_out) a.c_out[((size_t)b * a.G + g) * a.r + k] = acc[i];
        if (pos < 0 || pos >= a.max_pages * a.P) continue;
        const int page = a.block_table[(size_t)seq * a.max_pages + pos / a.P];
        if ((unsigned)page >= (unsigned)a.n_pages) continue;
        st_elt<TS>(static_cast<TS *>(a.pool) + (((size_t)page * a.G + g) * a.P + pos % a.P) * a.r +
                       k,
                   acc[i]);
    }
}

int blocks_of(const EncodeArgs &a) {
    return a.G * ((a.r + KC - 1) / KC) * ((a.B + BR - 1) / BR);
}

// ---------------------------------------------------------------- bf16: matrix cores
// C = X W - 1 (mu W) per (axis, group): a dense contraction over the stacked axis, run on
// v_mfma_f32_32x32x16_bf16.  A workgroup owns the output rows of `rows` sequences (32, or 16, 8, 4
// when a batch is too small to fill the chip with 32-row tiles: the 32-row MFMA tile then repeats
// its rows and the workgroups of one column slice each read the whole W_down slice, from cache)
// by 32 latent columns; its EWAVES waves split the stacked axis into contiguous ranges of
// 16-element k-steps.
// Every lane loads its own operands straight from memory: A = staging rows (16 bytes per lane
// per k-step) and the mean mu (the same in every row), B = W_down rows 16ks + 8h2 + 0..7 of
// column c0 + l32 (eight 2-byte loads; a wave's loads cover whole 64-byte row segments).  Groups
// of EG k-steps are double-buffered.  Inputs stay exact bf16; x W and mu W accumulate in
// separate fp32 chains and are subtracted at the end; the waves' partial tiles are summed in a
// fixed order through LDS.  The append slots (write_pos, then the page table) are fetched at the
// start so that the stores at the end wait on nothing.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int EWAVES = 8;            // waves per workgroup
// word 3 of a raw (untyped, unswizzled) buffer resource
constexpr int kBufferWord3 = 0x00020000;
// k-steps per load group: four in the single-call kernel; one in the many-layer kernel, whose
// tiles leave each wave a few k-steps, so that its registers fit two workgroups per CU
constexpr int EGRP = 4, EGRP_LAYERS = 1;

__device__ __forceinline__ f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int EG>
struct EncOps {
    uint4 x[EG], m[EG];
    uint16_t w[EG][8];
};

// One workgroup's tile `blk` of axis `a` (RS rows per workgroup).
template <int EG>
__device__ __forceinline__ void encode_mfma_tile(const EncodeArgs a, int blk, const int RS) {
    __shared__ float sAcc[EWAVES][32][33];

    const int ctiles = (a.r + 31) / 32;
    const int rtiles = (a.B + RS - 1) / RS;
    const int ct = blk % ctiles;
    const int rt = (blk / ctiles) % rtiles;
    const int g = blk / (ctiles * rtiles);
    const int c0 = ct * 32, b0 = rt * RS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h2 = lane >> 5;
    const int X = a.T * a.Dg;
    const int nks = X / 16;                              // X is a multiple of 64
    const int per = (nks + EWAVES - 1) / EWAVES;
    const int ks0 = min(wave * per, nks), ks1 = min(ks0 + per, nks);

    // ---- append slots of this thread's outputs (rows tid / 32 and tid / 32 + 16 of the tile),
    // fetched first; the page-table reads wait only for the write positions
    constexpr int OUTS = 32 * 32 / (64 * EWAVES);        // outputs per thread
    int wpos[OUTS], wseq[OUTS], page[OUTS];
    bool wlive[OUTS];
#pragma unroll
    for (int o = 0; o < OUTS; ++o)
        wlive[o] = encode_row(a, min(b0 + (tid + 64 * EWAVES * o) / 32, a.B - 1), wseq[o],
                              wpos[o]);

    const uint16_t *x = static_cast<const uint16_t *>(a.x);
    const uint16_t *W = static_cast<const uint16_t *>(a.W_down) + (size_t)g * X * a.r;
    const uint16_t *mu = static_cast<const uint16_t *>(a.mu) + (size_t)g * X;
    const int brow = min(b0 + l32 % RS, a.B - 1);        // this lane's A-operand row (clamped)
    const int wcol = min(c0 + l32, a.r - 1);             // this lane's B-operand column (clamped)

    // Operands come through buffer loads: a fixed byte offset per lane (vector) plus an offset
    // uniform per k-step and element (scalar), so the loads take no per-element address
    // arithmetic; the resources span exactly the workgroup's rows, its group's W_down and mu
    // (out-of-range reads return zero).  d_head is 64 or 128, so a lane's 8 stacked elements
    // never cross a head-dim row.
    const size_t rowstride = a.mode ? (size_t)X : (size_t)a.T * a.H * a.d;   // staging row
    const int nrows = min(RS, a.B - b0);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(x + (size_t)b0 * rowstride), 0, (int)(nrows * rowstride * 2),
        kBufferWord3);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(W), 0, X * a.r * 2, kBufferWord3);
    const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(mu), 0, X * 2, kBufferWord3);
    const int xl = (int)((size_t)(brow - b0) * rowstride + 8 * h2) * 2;
    const int wl = (8 * h2 * a.r + wcol) * 2;
    const int ml = 16 * h2;
    const int dsh = a.d == 128 ? 7 : 6;

    // k-steps kg .. kg + EG - 1 of this wave; steps past its range load in bounds and are zeroed
    auto load_grp = [&](int kg, EncOps<EG> &op) {
#pragma unroll
        for (int j = 0; j < EG; ++j) {
            const int ks = min(kg + j, max(ks1 - 1, 0));
            int xo;                                             // the k-step's row offset
            if (a.mode) {
                xo = 16 * ks;                                          // (t, h, i) order
            } else {
                const int t = (16 * ks) >> dsh, i = (16 * ks) & (a.d - 1);   // (t, i) of head g
                xo = (t * a.H + g) * a.d + i;
            }
            op.x[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, xl, 2 * xo, 0));
            op.m[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(mr, ml, 32 * ks, 0));
#pragma unroll
            for (int e = 0; e < 8; ++e)
                op.w[j][e] = __builtin_amdgcn_raw_buffer_load_b16(wr, wl, (16 * ks + e) * a.r * 2, 0);
        }
    };
    f32x16 acc = {}, accmu = {};
    auto compute = [&](int kg, const EncOps<EG> &op) {
#pragma unroll
        for (int j = 0; j < EG; ++j) {
            const bool live = kg + j < ks1;
            const uint4 ax = live ? op.x[j] : make_uint4(0, 0, 0, 0);
            const uint4 am = live ? op.m[j] : make_uint4(0, 0, 0, 0);
            const uint16_t *w = op.w[j];
            const uint4 bw = make_uint4(w[0] | (uint32_t)w[1] << 16, w[2] | (uint32_t)w[3] << 16,
                                        w[4] | (uint32_t)w[5] << 16, w[6] | (uint32_t)w[7] << 16);
            acc = mfma32(ax, bw, acc);
            accmu = mfma32(am, bw, accmu);
        }
    };

    EncOps<EG> A, Bq;
    load_grp(ks0, A);
#pragma unroll
    for (int o = 0; o < OUTS; ++o) {
        const int pos = wpos[o];
        const int pi = min(max(pos, 0) / a.P, a.max_pages - 1);
        page[o] = a.block_table[(size_t)wseq[o] * a.max_pages + pi];
    }
    for (int kg = ks0; kg < ks1; kg += 2 * EG) {
        load_grp(kg + EG, Bq);
        compute(kg, A);
        if (kg + EG >= ks1) break;
        load_grp(kg + 2 * EG, A);
        compute(kg + EG, Bq);
    }

    // ---- partial tile (rows 8(v/4) + 4h2 + v%4, column l32) -> fixed-order sum over waves
#pragma unroll
    for (int v = 0; v < 16; ++v) sAcc[wave][8 * (v >> 2) + 4 * h2 + (v & 3)][l32] = acc[v] - accmu[v];
    __syncthreads();
#pragma unroll
    for (int o = 0; o < OUTS; ++o) {
        const int idx = tid + 64 * EWAVES * o;
        const int row = idx >> 5, col = idx & 31;
        const int bb = b0 + row, k = c0 + col;
        if (row >= RS || bb >= a.B || k >= a.r) continue;
        float c = 0.f;
#pragma unroll
        for (int w = 0; w < EWAVES; ++w) c += sAcc[w][row][col];
        const int pos = wpos[o];
        if (!wlive[o]) continue;                             // row past its sequence's chunk
        if (a.c_out) a.c_out[((size_t)bb * a.G + g) * a.r + k] = c;
        if (pos < 0 || pos >= a.max_pages * a.P) continue;
        if ((unsigned)page[o] >= (unsigned)a.n_pages) continue;
        static_cast<uint16_t *>(a.pool)[(((size_t)page[o] * a.G + g) * a.P + pos % a.P) * a.r +
                                        k] = f2bf(c);
    }
}

__global__ __launch_bounds__(64 * EWAVES) void encode_mfma_kernel(EncodePair pr) {
    int blk = blockIdx.x;
    const int axis = blk < pr.blocks_k ? 0 : 1;
    if (axis) blk -= pr.blocks_k;
    encode_mfma_tile<EGRP>(axis ? pr.ax[1] : pr.ax[0], blk, pr.rows);
}

// Several layers' encodes in one launch (the same tiles as encode_mfma_kernel, layer after
// layer): the fields every layer shares come from ax[], the per-layer pointers from the tables.
constexpr int kEncLayersMax = 32;    // layers per launch (the tables sit in the kernel arguments)
struct EncodeLayers {
    EncodeArgs ax[2];
    const void *src[kEncLayersMax][2][3];    // per layer and axis: staging x, W_down, mu
    void *pool[kEncLayersMax][2];
    const int32_t *block_table[kEncLayersMax];
    int blocks_k, blocks_layer, rows;
};

__global__ __launch_bounds__(64 * EWAVES) __attribute__((amdgpu_waves_per_eu(4)))
void encode_layers_kernel(EncodeLayers el) {
    const int layer = blockIdx.x / el.blocks_layer;
    int blk = blockIdx.x - layer * el.blocks_layer;
    const int axis = blk < el.blocks_k ? 0 : 1;
    if (axis) blk -= el.blocks_k;
    EncodeArgs a = el.ax[axis];
    a.x = el.src[layer][axis][0];
    a.W_down = el.src[layer][axis][1];
    a.mu = el.src[layer][axis][2];
    a.pool = el.pool[layer][axis];
    a.block_table = el.block_table[layer];
    encode_mfma_tile<EGRP_LAYERS>(a, blk, el.rows);
}

int mfma_blocks_of(const EncodeArgs &a, int rows) {
    return a.G * ((a.r + 31) / 32) * ((a.B + rows - 1) / rows);
}

// ---------------------------------------------------------------- bf16, many rows
// The bulk encode of a prefill chunk (thousands of rows): a workgroup owns (axis, group, 32 latent
// columns, 512 rows).  It stages its column slice of W_down transposed in LDS once (W^T[col][x]);
// each of its waves then streams whole rows: C^T = W^T X^T on v_mfma_f32_32x32x16_bf16 with
// A = W^T from LDS (16 bytes per lane per k-step) and B = X^T straight from the staging rows
// (16 bytes per lane per k-step), over the full stacked axis, so no partial tiles are exchanged.
// A lane's results are one row (its B column) at 16 latent columns, so its append slot is one
// lookup.  mu W is formed once per wave, in its own fp32 chain, and subtracted at the end.
constexpr int RWAVES = 4;            // waves per workgroup
constexpr int RXMAX = 512;           // largest stacked axis it serves (LDS: 32 x 520 bf16)
constexpr int RTILES = 16;           // 32-row tiles per workgroup
constexpr int RGRP = 8;              // k-steps per load group

__global__ __launch_bounds__(64 * RWAVES) void encode_rows_kernel(EncodePair pr) {
    __shared__ __align__(16) uint16_t sWt[32][RXMAX + 8];

    int blk = blockIdx.x;
    const int axis = blk < pr.blocks_k ? 0 : 1;
    if (axis) blk -= pr.blocks_k;
    const EncodeArgs a = axis ? pr.ax[1] : pr.ax[0];
    const int ctiles = (a.r + 31) / 32;
    const int rblocks = (a.B + 32 * RTILES - 1) / (32 * RTILES);
    const int ct = blk % ctiles;
    const int rb = (blk / ctiles) % rblocks;
    const int g = blk / (ctiles * rblocks);
    const int c0 = ct * 32;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h2 = lane >> 5;
    const int X = a.T * a.Dg;
    const int KS = X / 16;                               // X is a multiple of 64

    // ---- W^T slice into LDS: 8-column pieces of W_down rows (columns past r are zero)
    const uint16_t *W = static_cast<const uint16_t *>(a.W_down) + (size_t)g * X * a.r;
    for (int idx = tid; idx < X * 4; idx += 64 * RWAVES) {
        const int xr = idx >> 2, cg = 8 * (idx & 3);
        uint4 w = make_uint4(0, 0, 0, 0);
        if (c0 + cg < a.r) w = *reinterpret_cast<const uint4 *>(W + (size_t)xr * a.r + c0 + cg);
        const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            sWt[cg + e][xr] = static_cast<uint16_t>(wd[e >> 1] >> (16 * (e & 1)));
    }
    __syncthreads();
    auto wt = [&](int ks) {           // A operand: column l32, stacked 16 ks + 8 h2 .. + 7
        return *reinterpret_cast<const uint4 *>(&sWt[l32][16 * ks + 8 * h2]);
    };

    // ---- mu W (the same for every row): B = mu at stacked 16 ks + 8 h2 .. + 7
    const uint16_t *mu = static_cast<const uint16_t *>(a.mu) + (size_t)g * X;
    f32x16 muacc = {};
    for (int ks = 0; ks < KS; ++ks)
        muacc = mfma32(wt(ks), *reinterpret_cast<const uint4 *>(mu + 16 * ks + 8 * h2), muacc);

    // this wave's row tiles: r0 = 32 (rb RTILES + wave + RWAVES i).  The append slot of this
    // lane's row in every tile is fetched first, so the row stream below waits on nothing else.
    constexpr int TPW = RTILES / RWAVES;                 // row tiles per wave
    const uint16_t *x = static_cast<const uint16_t *>(a.x);
    int ntile = 0;
    while (ntile < TPW && 32 * (rb * RTILES + wave + RWAVES * ntile) < a.B) ++ntile;
    uint16_t *dst[TPW];
    bool live[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int rr = 32 * (rb * RTILES + wave + RWAVES * i) + l32;
        int seq, pos;
        live[i] = rr < a.B && encode_row(a, min(rr, a.B - 1), seq, pos);
        const bool store = live[i] && pos >= 0 && pos < a.max_pages * a.P;
        const int page = store ? a.block_table[(size_t)seq * a.max_pages + pos / a.P] : -1;
        dst[i] = (unsigned)page < (unsigned)a.n_pages
            ? static_cast<uint16_t *>(a.pool) + (((size_t)page * a.G + g) * a.P + pos % a.P) * a.r
            : nullptr;
    }
    // staging offset of stacked index k: k + t (H d - d) with t = k / d per head ((t, i) of head
    // g), plain k for LLA-2D ((t, h, i) order); d is a power of two
    const int dsh = 31 - __builtin_clz(a.d);
    const int tjump = a.mode ? 0 : (a.H - 1) * a.d;
    const int ngrp = (KS + RGRP - 1) / RGRP;
    const int nsteps = ntile * ngrp;
    // the stream of (tile, k-group) steps is double-buffered: the next group's rows are in
    // flight during the current group's MFMAs
    auto load = [&](int st, uint4 *xv) {
        st = min(st, max(nsteps - 1, 0));
        const int i = st / ngrp, k0 = RGRP * (st - i * ngrp);
        const int row = min(32 * (rb * RTILES + wave + RWAVES * i) + l32, a.B - 1);
        const uint16_t *xr = x + (a.mode ? (size_t)row * X : ((size_t)row * a.T * a.H + g) * a.d);
#pragma unroll
        for (int j = 0; j < RGRP; ++j) {
            const int k = 16 * min(k0 + j, KS - 1) + 8 * h2;
            xv[j] = *reinterpret_cast<const uint4 *>(xr + k + (k >> dsh) * tjump);
        }
    };
    f32x16 acc = {};
    auto step = [&](int st, const uint4 *xv) {
        const int i = st / ngrp, k0 = RGRP * (st - i * ngrp);
        if (k0 + RGRP <= KS) {
#pragma unroll
            for (int j = 0; j < RGRP; ++j) acc = mfma32(wt(k0 + j), xv[j], acc);
        } else {
#pragma unroll
            for (int j = 0; j < RGRP; ++j)
                if (k0 + j < KS) acc = mfma32(wt(k0 + j), xv[j], acc);
        }
        if (k0 + RGRP < KS) return;
        // tile done.  Lane (row, h2), element v: latent column c0 + 8 (v / 4) + 4 h2 + v % 4
        const int rr = 32 * (rb * RTILES + wave + RWAVES * i) + l32;
        const f32x16 res = acc;
        acc = f32x16{};
        bool lv = false;
        uint16_t *d = nullptr;
#pragma unroll
        for (int u = 0; u < TPW; ++u)
            if (u == i) { lv = live[u]; d = dst[u]; }
        if (!lv) return;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int col = c0 + 8 * q + 4 * h2;
            if (col >= a.r) continue;                    // r is a multiple of 8
            const float c[4] = {res[4 * q] - muacc[4 * q], res[4 * q + 1] - muacc[4 * q + 1],
                                res[4 * q + 2] - muacc[4 * q + 2],
                                res[4 * q + 3] - muacc[4 * q + 3]};
            if (a.c_out)
                *reinterpret_cast<float4 *>(a.c_out + ((size_t)rr * a.G + g) * a.r + col) =
                    make_float4(c[0], c[1], c[2], c[3]);
            if (d)
                *reinterpret_cast<uint2 *>(d + col) =
                    make_uint2((uint32_t)f2bf(c[0]) | (uint32_t)f2bf(c[1]) << 16,
                               (uint32_t)f2bf(c[2]) | (uint32_t)f2bf(c[3]) << 16);
        }
    };
    uint4 xa[RGRP], xb[RGRP];
    load(0, xa);
    for (int st = 0; st < nsteps; st += 2) {
        load(st + 1, xb);
        step(st, xa);
        if (st + 1 >= nsteps) break;
        load(st + 2, xa);
        step(st + 1, xb);
    }
}

// ---------------------------------------------------------------- bf16, many rows, wide ranks
// The bulk encode of a prefill chunk when both latent ranks are multiples of 32 (at least one 64
// or more): C^T = W_down^T (X - 1 mu)^T per (axis, group) as one GEMM on v_mfma_f32_32x32x16_bf16.
// A workgroup of GWAVES waves owns (axis, group, a block of `rows` rows) and every latent column of
// its axis; wave w owns the 32-row tile [32 w, 32 w + 32) of the block (waves past the block only
// help stage).  The stacked axis is walked in chunks of 128 (64 at r = 160):
//  * the chunk's W_down rows (chunk x r, row-major as stored) and mu values are staged in LDS by the
//    whole workgroup, double-buffered with one barrier per chunk, and W comes back through
//    ds_read_b64_tr_b16 as the A operand (lane (rank, h2) of k-step ks: stacked 16 ks + 8 h2 ..
//    + 7 of its rank; the four rows a 16-lane group reads fall in distinct banks, padding the LDS
//    row where r is a multiple of 64);
//  * the B operand, 8 consecutive stacked elements of one row, comes straight from the staging
//    row (16 bytes per lane, one chunk ahead) and is centred on the way: x - mu is formed in fp32
//    and rounded to bf16 (relative 2^-9 per element, the class of the latent's own bf16
//    rounding), so the rows need no separate mu W chain.
// A lane's result is one row at 16 latent columns per 32-column tile, so its append slot is one
// lookup, fetched before the stream.
constexpr int GWAVES = 8;            // waves per workgroup
constexpr int GKMIN = 64;            // the stacked axis is a multiple of this

template <int CT>
struct GShape {
    static constexpr int R = 32 * CT;                                    // latent columns
    // stacked elements per chunk: 128 (more bytes in flight per wave), 64 at r = 160, where the
    // larger chunk's registers spill
    static constexpr int GKC = CT >= 5 ? 64 : 128;
    static constexpr int GKS = GKC / 16;                                 // k-steps per chunk
    // LDS row of a staged W_down row (elements): padded when 2R bytes would map the four rows a
    // transposed read touches onto the same banks
    static constexpr int WST = R % 64 == 0 ? (R == 64 ? 72 : R + 16) : R;
    static constexpr int WP = GKC * R / 8;                               // 16-byte W pieces
    static constexpr int NPW = (WP + 64 * GWAVES - 1) / (64 * GWAVES);   // per thread
    static constexpr int BUF = GKC * WST + GKC;                          // W rows, then mu
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two fp32 -> two bf16 (round to nearest even), lo in the low half
__device__ __forceinline__ uint32_t pk2bf(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// 8 bf16 of x minus 8 bf16 of mu, in fp32, rounded once to 8 bf16
__device__ __forceinline__ uint4 centre8(const uint4 xv, const uint4 mv) {
    const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w}, ms[4] = {mv.x, mv.y, mv.z, mv.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = pk2bf(__uint_as_float(xs[i] << 16) - __uint_as_float(ms[i] << 16),
                     __uint_as_float(xs[i] & 0xFFFF0000u) - __uint_as_float(ms[i] & 0xFFFF0000u));
    return make_uint4(o[0], o[1], o[2], o[3]);
}

template <int CT>
__device__ __forceinline__ void encode_gemm_tile(const EncodeArgs a, int blk, int rows,
                                                 uint16_t *lds) {
    using GS = GShape<CT>;
    constexpr int R = GS::R, WST = GS::WST, NPW = GS::NPW, WP = GS::WP, BUF = GS::BUF;
    constexpr int GKC = GS::GKC, GKS = GS::GKS;
    const int X = a.T * a.Dg;
    const int rblocks = (a.B + rows - 1) / rows;
    const int rb = blk % rblocks, g = blk / rblocks;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h2 = lane >> 5;
    const bool wlive = 32 * wave < rows;                  // uniform
    const int rr = rb * rows + 32 * wave + l32;           // this lane's row
    const int row = min(rr, a.B - 1);                     // (clamped for the loads)
    const int nch = X / GKC;

    // ---- append slot of this lane's row, fetched first
    uint16_t *dst = nullptr;
    bool live = false;
    if (wlive && rr < a.B) {
        int seq, pos;
        live = encode_row(a, rr, seq, pos);
        if (live && pos >= 0 && pos < a.max_pages * a.P) {
            const int page = a.block_table[(size_t)seq * a.max_pages + pos / a.P];
            if ((unsigned)page < (unsigned)a.n_pages)
                dst = static_cast<uint16_t *>(a.pool) + (((size_t)page * a.G + g) * a.P + pos % a.P) * R;
        }
    }

    const uint16_t *W = static_cast<const uint16_t *>(a.W_down) + (size_t)g * X * R;
    const uint16_t *mu = static_cast<const uint16_t *>(a.mu) + (size_t)g * X;
    // staging offset of stacked index k: k + t (H d - d) with t = k / d per head ((t, i) of head
    // g), plain k for LLA-2D ((t, h, i) order); d is a power of two
    const int dsh = 31 - __builtin_clz(a.d);
    const int tjump = a.mode ? 0 : (a.H - 1) * a.d;
    const uint16_t *xr = static_cast<const uint16_t *>(a.x) +
                         (a.mode ? (size_t)row * X : ((size_t)row * a.T * a.H + g) * a.d);

    // ---- chunk c's W_down rows and mu into registers, then into LDS buffer `buf`
    struct WV {
        uint4 w[NPW];
        uint4 m;
    };
    auto wload = [&](int c) __attribute__((always_inline)) {
        WV v;
        const uint16_t *src = W + (size_t)c * GKC * R;
#pragma unroll
        for (int x = 0; x < NPW; ++x) {
            // the last slot clamps its piece (WP is a multiple of 64, so per wave)
            const int p = min(tid + 64 * GWAVES * x, WP - 1);
            v.w[x] = *reinterpret_cast<const uint4 *>(src + 8 * p);
        }
        v.m = *reinterpret_cast<const uint4 *>(mu + (size_t)c * GKC + 8 * (tid & (GKC / 8 - 1)));
        return v;
    };
    auto wstore = [&](int buf, const WV v) __attribute__((always_inline)) {
        uint16_t *b = lds + buf * BUF;
#pragma unroll
        for (int x = 0; x < NPW; ++x) {
            const int p = tid + 64 * GWAVES * x;
            if (WP % (64 * GWAVES) == 0 || 64 * wave + 64 * GWAVES * x < WP)
                *reinterpret_cast<uint4 *>(b + (p / (R / 8)) * WST + 8 * (p % (R / 8))) = v.w[x];
        }
        if (tid < GKC / 8) *reinterpret_cast<uint4 *>(b + GKC * WST + 8 * tid) = v.m;
    };
    // ---- chunk c's rows of this lane: stacked 64 c + 16 ks + 8 h2 .. + 7
    struct XV {
        uint4 v[GKS];
    };
    auto xload = [&](int c) __attribute__((always_inline)) {
        XV xv;
#pragma unroll
        for (int ks = 0; ks < GKS; ++ks) {
            const int k = GKC * c + 16 * ks + 8 * h2;
            xv.v[ks] = *reinterpret_cast<const uint4 *>(xr + k + (k >> dsh) * tjump);
        }
        return xv;
    };
    // transposed reads: lane (4 e' + m) of each 16-lane group addresses stacked row 8 h2 + e'
    // (+ 4 for the second read) at ranks 16 ((lane / 16) % 2) + 4 m .. + 3, and lane l gets rank
    // l % 32 of those four rows
    const uint32_t vrd =
        (uint32_t)(((8 * h2 + ((lane & 15) >> 2)) * WST + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2);
    f32x16 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x16{};
    auto compute = [&](int buf, const XV xv) __attribute__((always_inline)) {
        uint16_t *b = lds + buf * BUF;
        lds_char *wb = (lds_char *)b + vrd;
#pragma unroll
        for (int ks = 0; ks < GKS; ++ks) {
            // one k-step's operand reads at a time (hoisting them all would spill)
            __builtin_amdgcn_sched_barrier(0);
            const uint4 mv = *reinterpret_cast<const uint4 *>(b + GKC * WST + 16 * ks + 8 * h2);
            const uint4 bx = centre8(xv.v[ks], mv);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                lds_char *p0 = wb + (16 * ks * WST + 32 * ct) * 2;
                const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
                const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + 8 * WST));
                const uint4 av = make_uint4(
                    (uint32_t)(uint16_t)r0[0] | (uint32_t)(uint16_t)r0[1] << 16,
                    (uint32_t)(uint16_t)r0[2] | (uint32_t)(uint16_t)r0[3] << 16,
                    (uint32_t)(uint16_t)r1[0] | (uint32_t)(uint16_t)r1[1] << 16,
                    (uint32_t)(uint16_t)r1[2] | (uint32_t)(uint16_t)r1[3] << 16);
                acc[ct] = mfma32(av, bx, acc[ct]);
            }
        }
    };

    // ---- pipeline: chunk c + 1's W_down and rows in flight while chunk c is multiplied
    XV xa, xb;
    WV wv = wload(0);
    xa = xload(0);
    wstore(0, wv);
    __syncthreads();
    for (int c = 0; c < nch; c += 2) {
        const bool n1 = c + 1 < nch, n2 = c + 2 < nch;
        if (n1) {
            wv = wload(c + 1);
            xb = xload(c + 1);
        }
        if (wlive) compute(0, xa);
        if (n1) wstore(1, wv);
        __syncthreads();
        if (!n1) break;
        if (n2) {
            wv = wload(c + 2);
            xa = xload(c + 2);
        }
        if (wlive) compute(1, xb);
        if (n2) wstore(0, wv);
        __syncthreads();
    }

    // ---- result: lane (row, h2), element v of tile ct: latent column 32 ct + 8 (v / 4) + 4 h2 + v % 4
    if (!live) return;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int col = 32 * ct + 8 * q + 4 * h2;
            const float c0 = acc[ct][4 * q], c1 = acc[ct][4 * q + 1], c2 = acc[ct][4 * q + 2],
                        c3 = acc[ct][4 * q + 3];
            if (a.c_out)
                *reinterpret_cast<float4 *>(a.c_out + ((size_t)rr * a.G + g) * R + col) =
                    make_float4(c0, c1, c2, c3);
            if (dst) *reinterpret_cast<uint2 *>(dst + col) = make_uint2(pk2bf(c0, c1), pk2bf(c2, c3));
        }
}

struct EncodeGemm {
    EncodeArgs ax[2];
    int blocks_k;         // workgroups of the K axis (the V axis follows)
    int rows;             // rows per workgroup (32-row tiles: 256, 128 or 64)
};

template <int CTK, int CTV>
__global__ __launch_bounds__(64 * GWAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void encode_gemm_kernel(EncodeGemm eg) {
    constexpr int BUF = GShape<CTK>::BUF > GShape<CTV>::BUF ? GShape<CTK>::BUF : GShape<CTV>::BUF;
    __shared__ __align__(16) uint16_t lds[2 * BUF];
    int blk = blockIdx.x;
    if (blk < eg.blocks_k) {
        encode_gemm_tile<CTK>(eg.ax[0], blk, eg.rows, lds);
    } else {
        blk -= eg.blocks_k;
        encode_gemm_tile<CTV>(eg.ax[1], blk, eg.rows, lds);
    }
}

int gemm_blocks_of(const EncodeArgs &a, int rows) { return a.G * ((a.B + rows - 1) / rows); }

int rows_blocks_of(const EncodeArgs &a) {
    return a.G * ((a.r + 31) / 32) * ((a.B + 32 * RTILES - 1) / (32 * RTILES));
}

// The row-streaming kernel serves bf16 codecs with a short stacked axis, many rows, and 16-byte
// aligned rows of W_down; everything else takes encode_mfma_kernel.
bool rows_kernel_fits(const EncodeArgs &a) {
    const int X = a.T * a.Dg;
    return X <= RXMAX && a.B >= 256 && a.r % 8 == 0 &&
           (reinterpret_cast<uintptr_t>(a.W_down) & 15) == 0 &&
           (reinterpret_cast<uintptr_t>(a.mu) & 15) == 0 &&
           (reinterpret_cast<uintptr_t>(a.c_out) & 15) == 0;
}

// 32-row tiles unless that leaves CUs idle: a small batch is latency-bound, and more, shorter
// workgroups put more loads in flight
int rows_per_block(const EncodeArgs &k_axis, const EncodeArgs &v_axis, int layers) {
    for (int rows = 32; rows > 4; rows /= 2)
        if ((long)layers * (mfma_blocks_of(k_axis, rows) + mfma_blocks_of(v_axis, rows)) >= 256)
            return rows;
    return 4;
}

// The wide-rank GEMM serves bf16 bulk encodes of many rows when both ranks are multiples of 32
// with one of them 64 or more (the rank pairs (32,64), (64,64), (64,128), (96,160)), the stacked
// axis is a multiple of 64 and the operands are 16-byte aligned.
bool gemm_kernel_fits(const EncodeArgs &k, const EncodeArgs &v) {
    auto ok = [](const EncodeArgs &a) {
        return a.B >= 1024 && (a.T * a.Dg) % (a.r >= 160 ? GKMIN : 2 * GKMIN) == 0 &&
               a.r % 32 == 0 && a.r <= 160 &&
               (reinterpret_cast<uintptr_t>(a.x) & 15) == 0 &&
               (reinterpret_cast<uintptr_t>(a.W_down) & 15) == 0 &&
               (reinterpret_cast<uintptr_t>(a.mu) & 15) == 0 &&
               (reinterpret_cast<uintptr_t>(a.c_out) & 15) == 0;
    };
    const int pk = k.r / 32, pv = v.r / 32;
    const bool pair = (pk == 1 && pv == 2) || (pk == 2 && pv == 2) || (pk == 2 && pv == 4) ||
                      (pk == 3 && pv == 5);
    return pair && ok(k) && ok(v) && k.B == v.B;
}

template <int CTK, int CTV>
hipError_t launch_gemm_t(const EncodeGemm &eg, unsigned blocks, hipStream_t st) {
    hipLaunchKernelGGL((encode_gemm_kernel<CTK, CTV>), dim3(blocks), dim3(64 * GWAVES), 0, st, eg);
    return hipGetLastError();
}

hipError_t launch_gemm(const EncodeArgs &k_axis, const EncodeArgs &v_axis, hipStream_t st) {
    EncodeGemm eg;
    eg.ax[0] = k_axis;
    eg.ax[1] = v_axis;
    // a 32-row tile per wave unless that leaves the grid short of two workgroups per CU (LLA-2D:
    // one group)
    eg.rows = 32 * GWAVES;
    while (eg.rows > 32 * GWAVES / 4 &&
           gemm_blocks_of(k_axis, eg.rows) + gemm_blocks_of(v_axis, eg.rows) < 512)
        eg.rows /= 2;
    eg.blocks_k = gemm_blocks_of(k_axis, eg.rows);
    const unsigned blocks = (unsigned)(eg.blocks_k + gemm_blocks_of(v_axis, eg.rows));
    const int pk = k_axis.r / 32, pv = v_axis.r / 32;
    if (pk == 1 && pv == 2) return launch_gemm_t<1, 2>(eg, blocks, st);
    if (pk == 2 && pv == 2) return launch_gemm_t<2, 2>(eg, blocks, st);
    if (pk == 2 && pv == 4) return launch_gemm_t<2, 4>(eg, blocks, st);
    return launch_gemm_t<3, 5>(eg, blocks, st);
}

}  // namespace

hipError_t launch_encode_layers(const EncodeArgs *k_axes, const EncodeArgs *v_axes, int n,
                                bool bf16, hipStream_t st) {
    // when a single call would give any layer to another kernel (fp32 codecs; the row-streaming
    // kernel, which also depends on each layer's operand alignment), every layer goes through
    // the single-call launcher, so each pool is written exactly as a single call writes it
    bool per_layer = !bf16;
    for (int i = 0; i < n && !per_layer; ++i)
        per_layer = (rows_kernel_fits(k_axes[i]) && rows_kernel_fits(v_axes[i]) &&
                     rows_blocks_of(k_axes[i]) + rows_blocks_of(v_axes[i]) >= 256) ||
                    gemm_kernel_fits(k_axes[i], v_axes[i]);
    if (per_layer) {
        for (int i = 0; i < n; ++i) {
            const hipError_t e = launch_encode(k_axes[i], v_axes[i], bf16, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    for (int i0 = 0; i0 < n; i0 += kEncLayersMax) {
        const int m = n - i0 < kEncLayersMax ? n - i0 : kEncLayersMax;
        EncodeLayers el{};
        el.ax[0] = k_axes[i0];
        el.ax[1] = v_axes[i0];
        for (int j = 0; j < m; ++j) {
            const EncodeArgs &k = k_axes[i0 + j], &v = v_axes[i0 + j];
            el.src[j][0][0] = k.x;
            el.src[j][0][1] = k.W_down;
            el.src[j][0][2] = k.mu;
            el.src[j][1][0] = v.x;
            el.src[j][1][1] = v.W_down;
            el.src[j][1][2] = v.mu;
            el.pool[j][0] = k.pool;
            el.pool[j][1] = v.pool;
            el.block_table[j] = k.block_table;
        }
        el.rows = rows_per_block(el.ax[0], el.ax[1], m);
        el.blocks_k = mfma_blocks_of(el.ax[0], el.rows);
        el.blocks_layer = el.blocks_k + mfma_blocks_of(el.ax[1], el.rows);
        hipLaunchKernelGGL(encode_layers_kernel, dim3((unsigned)(m * el.blocks_layer)),
                           dim3(64 * EWAVES), 0, st, el);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_encode(const EncodeArgs &k_axis, const EncodeArgs &v_axis, bool bf16,
                         hipStream_t st) {
    if (bf16 && gemm_kernel_fits(k_axis, v_axis)) return launch_gemm(k_axis, v_axis, st);
    EncodePair pr;
    pr.ax[0] = k_axis;
    pr.ax[1] = v_axis;
    // the row-streaming kernel only pays when its grid fills the chip (a workgroup per CU);
    // fewer, longer row blocks lose to the split-axis kernel's many short ones
    if (bf16 && rows_kernel_fits(k_axis) && rows_kernel_fits(v_axis) &&
        rows_blocks_of(k_axis) + rows_blocks_of(v_axis) >= 256) {
        pr.blocks_k = rows_blocks_of(k_axis);
        const unsigned blocks = (unsigned)(pr.blocks_k + rows_blocks_of(v_axis));
        hipLaunchKernelGGL(encode_rows_kernel, dim3(blocks), dim3(64 * RWAVES), 0, st, pr);
    } else if (bf16) {
        pr.rows = rows_per_block(k_axis, v_axis, 1);
        pr.blocks_k = mfma_blocks_of(k_axis, pr.rows);
        const unsigned blocks = (unsigned)(pr.blocks_k + mfma_blocks_of(v_axis, pr.rows));
        hipLaunchKernelGGL(encode_mfma_kernel, dim3(blocks), dim3(64 * EWAVES), 0, st, pr);
    } else {
        pr.blocks_k = blocks_of(k_axis);
        const unsigned blocks = (unsigned)(pr.blocks_k + blocks_of(v_axis));
        hipLaunchKernelGGL(encode_kernel, dim3(blocks), dim3(NT), 0, st, pr);
    }
    return hipGetLastError();
}

}  // namespace lla
