// fit.hip -- codec fit by truncated SVD of the (mean-removed) activations, bf16, gfx950.
//
// pith.science paper page for "Looped Latent Attention", "What carries the argument": the codec
// starts from an SVD of activation data, W_down spanning the leading right singular subspace of
// the mean-removed activation matrix.  Per group g the
// activations are the stacked rows a_j (X = T D_g values per token, the encode's stacking order);
//   mu = mean_j a_j,   C = sum_j (a_j - mu)^T (a_j - mu) = A^T A - n mu^T mu   (X x X),
// and the right singular vectors of the centred matrix are C's eigenvectors.  The top r are found
// by subspace iteration on C with r + 8 columns, orthonormalised by CholeskyQR2 after every
// product, then a Rayleigh-Ritz step: H = V^T C V, its eigenvectors by parallel-order Jacobi
// sweeps, W_down = V Q in decreasing eigenvalue order, each column's entry of largest magnitude
// made positive, sigma = sqrt(eigenvalue), W_up,t = the transpose of W_down's rows t D_g ...
//
// Kernels, in launch order (host side in lla_api.hip):
//   fit_cov_kernel     A^T A on v_mfma_f32_32x32x16_bf16 over 128 x 128 blocks (bi <= bj) of C,
//                      rows split into S ranges; 32-row chunks of the two column strips are
//                      staged transposed in LDS; diagonal blocks also form column sums (a ones
//                      operand).  Exact bf16 inputs, fp32 accumulation, partials per split.
//   fit_reduce_kernel  C = sum over splits - n mu mu^T (both triangles), mu (fp32 and output).
//   fit_init_kernel    the start block: a counter-based hash per (g, i, c) (splitmix64).
//   fit_mul_kernel     W = C V (fp32), one workgroup per (g, 32 rows).
//   fit_orth_kernel    V = orth(W) by CholeskyQR2, one workgroup per group.
//   fit_ritz_kernel    Rayleigh-Ritz: H = V^T C V and its Jacobi rotations (logged), one
//                      workgroup per group.
//   fit_apply_kernel   the rotations applied to V's rows (W_down before signs), 32 rows each.
//   fit_out_kernel     column signs and the outputs, one workgroup per group.
#include "lla_internal.h"

#include <cmath>

namespace lla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

constexpr int CB = 128;          // covariance block edge
constexpr int CK = 64;           // rows per staged chunk
constexpr int FT = 256;          // threads of every fit kernel

// Stacked index k of row `row`, group g: staging offset ((row T + t) H + g) d + i per head with
// k = t d + i; row X + k for LLA-2D ((t, h, i) order).
__device__ __forceinline__ size_t stage_off(const FitArgs &a, int row, int g, int k) {
    if (a.mode) return (size_t)row * a.X + k;
    const int t = k / a.d;
    return (((size_t)row * a.T + t) * a.H + g) * a.d + (k - t * a.d);
}

// ---------------------------------------------------------------- A^T A and column sums
__global__ __launch_bounds__(FT) void fit_cov_kernel(FitArgs a) {
    __shared__ __align__(16) uint16_t sI[CB][CK + 8];   // strip of block row bi, [col][row]
    __shared__ __align__(16) uint16_t sJ[CB][CK + 8];   // strip of block column bj

    const int nb = a.X / CB;
    const int pairs = nb * (nb + 1) / 2;
    // work item (g, s, pair), pair fastest: the pairs of one (group, row range) are consecutive
    // items of one XCD and run together, so its L2 serves the strips they share
    int id = xcd_work_item(blockIdx.x, gridDim.x);
    int pr = id % pairs;
    id /= pairs;
    const int s = id % a.S;
    const int g = id / a.S;
    int bi = 0;                                          // pair -> (bi <= bj)
    while (pr >= nb - bi) { pr -= nb - bi; ++bi; }
    const int bj = bi + pr;
    const bool diag = bi == bj;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h2 = lane >> 5;
    const int ti = wave >> 1, tj = wave & 1;             // this wave's 64 x 64 sub-block
    const long per = (a.n + a.S - 1) / a.S;
    const int r0 = (int)min((long)a.n, per * s), r1 = (int)min((long)a.n, per * (s + 1));
    const uint16_t *x = static_cast<const uint16_t *>(a.x);

    // staging: slot u of thread tid holds the 16-byte piece of token tid % 32 + 32 (u % 2) of the
    // 64-row chunk and columns 8 cg .. + 7, cg = tid / 32 + 8 (u / 2), of each strip.  Written
    // transposed (sI[col][token]) one element per instruction: the 32 lanes of a half-wave write
    // consecutive tokens of one row; the second half-wave takes its elements rotated by four,
    // which puts its rows 12 apart from the first half's, i.e. on the other 16 banks (rows are 36
    // dwords apart).  Conflict-free.
    const int rr = tid & 31, hw = (tid >> 5) & 1;
    uint4 pi[4], pj[4];
    auto fetch = [&](int c0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int tok = c0 + rr + 32 * (u & 1);
            const int row = min(tok, max(r1 - 1, 0));
            const bool live = tok < r1;
            const int col = 8 * ((tid >> 5) + 8 * (u >> 1));
            pi[u] = live ? *reinterpret_cast<const uint4 *>(x + stage_off(a, row, g, CB * bi + col))
                         : make_uint4(0, 0, 0, 0);
            pj[u] = live ? *reinterpret_cast<const uint4 *>(x + stage_off(a, row, g, CB * bj + col))
                         : make_uint4(0, 0, 0, 0);
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int col = 8 * ((tid >> 5) + 8 * (u >> 1));
            const int tk = rr + 32 * (u & 1);
            const uint32_t wi[4] = {pi[u].x, pi[u].y, pi[u].z, pi[u].w};
            const uint32_t wj[4] = {pj[u].x, pj[u].y, pj[u].z, pj[u].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int er = (e + 4) & 7;                  // the rotated element (same parity)
                const int el = hw ? er : e;
                const uint32_t di = hw ? wi[er >> 1] : wi[e >> 1];
                const uint32_t dj = hw ? wj[er >> 1] : wj[e >> 1];
                sI[col + el][tk] = static_cast<uint16_t>(di >> (16 * (e & 1)));
                sJ[col + el][tk] = static_cast<uint16_t>(dj >> (16 * (e & 1)));
            }
        }
    };

    f32x16 acc[2][2] = {};
    f32x16 sum = {};
    const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
    fetch(r0);
    for (int c0 = r0; c0 < r1; c0 += CK) {
        __syncthreads();                                 // previous chunk consumed
        stage();
        __syncthreads();
        if (c0 + CK < r1) fetch(c0 + CK);                // next chunk in flight
#pragma unroll
        for (int ks = 0; ks < CK / 16; ++ks) {
            uint4 av[2], bv[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                av[m] = *reinterpret_cast<const uint4 *>(&sI[64 * ti + 32 * m + l32][16 * ks + 8 * h2]);
                bv[m] = *reinterpret_cast<const uint4 *>(&sJ[64 * tj + 32 * m + l32][16 * ks + 8 * h2]);
            }
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int nn = 0; nn < 2; ++nn) acc[m][nn] = mfma(av[m], bv[nn], acc[m][nn]);
            if (diag) {
                // column sums of the block's columns 32 wave ..: every row of D is the sum
                const uint4 cv = *reinterpret_cast<const uint4 *>(&sJ[32 * wave + l32][16 * ks + 8 * h2]);
                sum = mfma(ones, cv, sum);
            }
        }
    }
    // D[m = i][n = j]: lane (j = l32, h2), element v: i = 8 (v / 4) + 4 h2 + v % 4
    float *P = a.part + ((size_t)s * a.G + g) * a.X * a.X;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nn = 0; nn < 2; ++nn) {
            const int j = CB * bj + 64 * tj + 32 * nn + l32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int i = CB * bi + 64 * ti + 32 * m + 8 * (v >> 2) + 4 * h2 + (v & 3);
                P[(size_t)i * a.X + j] = acc[m][nn][v];
            }
        }
    if (diag && h2 == 0)
        a.colsum[((size_t)s * a.G + g) * a.X + CB * bj + 32 * wave + l32] = sum[0];
}

// ---------------------------------------------------------------- C = sum - n mu mu^T, mu
__global__ __launch_bounds__(FT) void fit_reduce_kernel(FitArgs a) {
    const size_t idx = (size_t)blockIdx.x * FT + threadIdx.x;
    const size_t per_g = (size_t)a.X * a.X;
    if (idx >= per_g * a.G) return;
    const int g = (int)(idx / per_g);
    const int i = (int)((idx % per_g) / a.X), j = (int)(idx % a.X);
    // only blocks with block row <= block column were computed: read (j, i) below the diagonal
    const bool swap = (i / CB) > (j / CB);
    const int ii = swap ? j : i, jj = swap ? i : j;
    float c = 0.f, si = 0.f, sj = 0.f;
    for (int s = 0; s < a.S; ++s) {
        c += a.part[(((size_t)s * a.G + g) * a.X + ii) * a.X + jj];
        si += a.colsum[((size_t)s * a.G + g) * a.X + i];
        sj += a.colsum[((size_t)s * a.G + g) * a.X + j];
    }
    const float inv_n = 1.f / (float)a.n;
    const float mi = si * inv_n, mj = sj * inv_n;
    a.C[idx] = c - (float)a.n * mi * mj;
    if (i == 0) {
        a.mu32[(size_t)g * a.X + j] = mj;
        if (a.bf16)
            static_cast<uint16_t *>(a.mu_out)[(size_t)g * a.X + j] = f2bf(mj);
        else
            static_cast<float *>(a.mu_out)[(size_t)g * a.X + j] = mj;
    }
}

// ---------------------------------------------------------------- subspace iteration
__device__ __forceinline__ float hash_unit(uint64_t k) {
    // splitmix64 finaliser (Steele, Lea, Flood 2014) -> uniform in [-1, 1)
    k += 0x9E3779B97F4A7C15ull;
    k = (k ^ (k >> 30)) * 0xBF58476D1CE4E5B9ull;
    k = (k ^ (k >> 27)) * 0x94D049BB133111EBull;
    k ^= k >> 31;
    return (float)(k >> 40) * (2.f / 16777216.f) - 1.f;
}

__global__ __launch_bounds__(FT) void fit_init_kernel(FitArgs a) {
    const size_t idx = (size_t)blockIdx.x * FT + threadIdx.x;
    if (idx >= (size_t)a.G * a.X * a.rb) return;
    a.W[idx] = hash_unit(idx);
}

// W = C V: workgroup (g, rows 32 q .. + 31).  64-wide k-chunks of C's rows (sC) and of V's rows
// (sV, row-major at pitch rb) pass through LDS, the next chunk's loads in flight while the current
// one is multiplied; thread (row tid / 8, columns tid % 8 + 8 u) accumulates in fp32.
// NB = ceil(rb / 16): every thread sums MU = 2 NB column slots (columns past rb read in-bounds
// LDS and are never stored), so the inner loop has no guard.
constexpr int MV = (64 * kFitMaxCols / 2 + FT - 1) / FT;  // float2 pieces of a V chunk per thread
template <int NB>
__global__ __launch_bounds__(FT) void fit_mul_kernel(FitArgs a) {
    constexpr int MU = 2 * NB;                            // column slots per thread
    __shared__ float sC[32][64 + 1];
    // + 16: the unguarded slots of the last rows reach 8 floats past a chunk of 64 x 72
    __shared__ __align__(8) float sV[64 * kFitMaxCols + 16];
    const int rows_per = a.X / 32;
    const int g = blockIdx.x / rows_per, q = blockIdx.x % rows_per;
    const int tid = threadIdx.x, rb = a.rb;
    const int il = tid / 8, c0 = tid % 8;
    const int nu = (rb - c0 + 7) / 8;                    // this thread's columns
    const float *C = a.C + ((size_t)g * a.X + 32 * q) * a.X;
    const float *V = a.V + (size_t)g * a.X * rb;
    const int npv = 64 * rb / 2;                          // float2 pieces per V chunk (rb even)
    float4 pc[2];
    float2 pv[MV];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {                    // C: 32 rows x 16 float4
            const int e = tid + FT * m;
            pc[m] = *reinterpret_cast<const float4 *>(C + (size_t)(e / 16) * a.X + k0 + 4 * (e % 16));
        }
#pragma unroll
        for (int m = 0; m < MV; ++m) {
            const int e = min(tid + FT * m, npv - 1);
            pv[m] = *reinterpret_cast<const float2 *>(V + (size_t)k0 * rb + 2 * e);
        }
    };
    float acc[MU] = {};
    fetch(0);
    for (int k0 = 0; k0 < a.X; k0 += 64) {
        __syncthreads();                                 // the previous chunk is consumed
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int e = tid + FT * m;
            float *d = &sC[e / 16][4 * (e % 16)];
            d[0] = pc[m].x; d[1] = pc[m].y; d[2] = pc[m].z; d[3] = pc[m].w;
        }
#pragma unroll
        for (int m = 0; m < MV; ++m) {
            const int e = tid + FT * m;
            if (e < npv) *reinterpret_cast<float2 *>(&sV[2 * e]) = pv[m];
        }
        __syncthreads();
        if (k0 + 64 < a.X) fetch(k0 + 64);
#pragma unroll 8
        for (int k = 0; k < 64; ++k) {
            const float cik = sC[il][k];
            const float *vr = &sV[k * rb + c0];
#pragma unroll
            for (int u = 0; u < MU; ++u) acc[u] += cik * vr[8 * u];
        }
    }
#pragma unroll
    for (int u = 0; u < MU; ++u)
        if (u < nu) a.W[((size_t)g * a.X + 32 * q + il) * rb + c0 + 8 * u] = acc[u];
}

constexpr int CR = 32;                                   // rows of a fit_apply_kernel block

// The orthonormalisation's LDS layout for NB 16-column tiles.  Blocks of up to 3 tiles (48
// columns, the small ranks) hold 16 NB columns per matrix row, form L^-1 in a second matrix (every
// column at once) and stream 64-row chunks; wider blocks hold kFitMaxCols columns, form the
// inverse in place (one matrix: 137 KB of LDS at 168 columns) and stream 32-row chunks.
template <int NB>
struct OrthCfg {
    static constexpr bool SMALL = NB <= 3;
    static constexpr int C = SMALL ? 16 * NB : kFitMaxCols;   // columns a matrix row holds
    static constexpr int P = C + 1;                           // LDS pitch (odd: rows read across
                                                              // lanes fall in different banks)
    static constexpr int OR = SMALL ? 64 : 32;                // rows of a streamed chunk
    static constexpr int CHE = (OR * C + FT - 1) / FT;        // chunk elements per thread
};

// OR-row chunks of an X x rb block (row-major, pitch rb) stream through sY; slot m of thread tid
// is chunk element tid + FT m (a chunk's rows are contiguous in memory), and the next chunk's
// loads are in flight while the current one is used.  X is a multiple of 64.
template <int NB>
struct ChunkStream {
    using CF = OrthCfg<NB>;
    int n, rb;
    float pre[CF::CHE];
    __device__ void init(int rb_) {
        rb = rb_;
        n = CF::OR * rb;
    }
    __device__ void fetch(const float *Y, int k0) {
#pragma unroll
        for (int m = 0; m < CF::CHE; ++m) {
            const int e = min((int)threadIdx.x + FT * m, n - 1);
            pre[m] = Y[(size_t)k0 * rb + e];
        }
    }
    __device__ void stage(float (*sY)[CF::P]) {
#pragma unroll
        for (int m = 0; m < CF::CHE; ++m) {
            const int e = (int)threadIdx.x + FT * m;
            if (e < n) sY[e / rb][e % rb] = pre[m];
        }
    }
};

// Cholesky factor L (lower, rb x rb, in LDS; zero above the diagonal) of the Gram matrix of the
// X x rb block Y (global).  Thread (tp, tq) of a 16 x 16 grid accumulates entries (tp + 16u,
// tq + 16v) over the row chunks.  A pivot below a tiny fraction of the trace is clamped
// (rank-deficient blocks stay finite).  NB = ceil(rb / 16) is a template parameter so the inner
// loops carry no guards (a guard per term would make every LDS read wait on its own).
template <int NB>
__device__ __forceinline__ void gram_cholesky(const FitArgs &a, const float *Y,
                                              float (*L)[OrthCfg<NB>::P],
                                              float (*sY)[OrthCfg<NB>::P]) {
    using CF = OrthCfg<NB>;
    const int rb = a.rb, tid = threadIdx.x;
    const int tp = tid >> 4, tq = tid & 15;
    float acc[NB][NB] = {};
    ChunkStream<NB> cs;
    cs.init(rb);
    cs.fetch(Y, 0);
    for (int k0 = 0; k0 < a.X; k0 += CF::OR) {
        __syncthreads();
        cs.stage(sY);
        __syncthreads();
        if (k0 + CF::OR < a.X) cs.fetch(Y, k0 + CF::OR);
#pragma unroll 4
        for (int k = 0; k < CF::OR; ++k) {
            float yp[NB], yq[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                yp[u] = sY[k][min(tp + 16 * u, CF::C)];
                yq[u] = sY[k][min(tq + 16 * u, CF::C)];
            }
#pragma unroll
            for (int u = 0; u < NB; ++u)
#pragma unroll
                for (int v = 0; v < NB; ++v) acc[u][v] += yp[u] * yq[v];
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NB; ++u)
#pragma unroll
        for (int v = 0; v < NB; ++v) {
            const int p = tp + 16 * u, q = tq + 16 * v;
            if (p < rb && q < rb) L[p][q] = q <= p ? acc[u][v] : 0.f;
        }
    __syncthreads();
    __shared__ float tr;
    __shared__ float sink[FT];                           // target of stores that must not land
    if (tid == 0) {
        float t = 0.f;
        for (int p = 0; p < rb; ++p) t += L[p][p];
        tr = t;
    }
    __syncthreads();
    // right-looking: pivot j, then its column, then the trailing lower triangle, each step O(1)
    // work per thread of the 16 x 16 grid
    const float floor_ = 1e-12f * tr + 1e-30f;
    for (int j = 0; j < rb; ++j) {
        if (tid == 0) L[j][j] = sqrtf(fmaxf(L[j][j], floor_));
        __syncthreads();
        if (tid > j && tid < rb) L[tid][j] /= L[j][j];
        __syncthreads();
        // the trailing lower entries (p >= q > j, below rb) are updated branch-free: every
        // visit stores, to a per-thread dummy slot when it is not such an entry, so no entry that
        // another thread reads in this phase is written
#pragma unroll
        for (int u = 0; u < NB; ++u)
#pragma unroll
            for (int v = 0; v < NB; ++v) {
                const int p = tp + 16 * u, q = tq + 16 * v;
                if (16 * NB > CF::C && (p >= CF::C || q >= CF::C)) continue;
                const bool upd = p > j && q > j && q <= p && p < rb;
                const float val = L[p][q] - L[p][j] * L[q][j];
                *(upd ? &L[p][q] : &sink[tid]) = val;
            }
        __syncthreads();
    }
}

// out = Y L^{-T}; then each chunk of Y is multiplied by L^{-1} in full.  out may alias Y: a chunk
// is read completely (and the next one fetched) before any of it is written.
// Small blocks: L^{-1} in Li by elimination on [L | I] (step j scales row j, then clears column j
// below it for every column at once, O(1) work per thread and step); 64-row chunks, thread
// (row tid / 4, columns tid % 4 + 4v).
// Wide blocks: L^{-1} overwrites L, column by column from the last:
// M[i][j] = -(sum_{k=j+1..i} M[i][k] L[k][j]) / L[j][j], where the columns k > j of M are already
// in place and L's column j is kept in sX; 32-row chunks, thread (row tid / 8, columns
// tid % 8 + 8v).  In both, all column slots are summed over k < rb (rows of the inverse past rb
// read in-bounds LDS and their sums are never stored; its upper triangle is zero), so the loop
// body has no guard.
template <int NB>
__device__ __forceinline__ void solve_rows(const FitArgs &a, const float *Y, float *out,
                                           float (*L)[OrthCfg<NB>::P],
                                           float (*Li)[OrthCfg<NB>::P],
                                           float (*sY)[OrthCfg<NB>::P]) {
    using CF = OrthCfg<NB>;
    constexpr int LN = CF::SMALL ? 4 : 8;                // lanes per chunk row
    constexpr int SV = 16 * NB / LN;                     // output column slots per thread
    const int rb = a.rb, tid = threadIdx.x;
    float (*M)[CF::P] = CF::SMALL ? Li : L;              // where L^{-1} ends up
    if constexpr (CF::SMALL) {
        const int tp = tid >> 4, tq = tid & 15;
        __shared__ float sink[FT];                       // target of stores that must not land
#pragma unroll
        for (int u = 0; u < NB; ++u)
#pragma unroll
            for (int v = 0; v < NB; ++v) {
                const int p = tp + 16 * u, q = tq + 16 * v;
                if (p < rb && q < rb) Li[p][q] = p == q ? 1.f : 0.f;
            }
        __syncthreads();
        for (int j = 0; j < rb; ++j) {
            if (tid <= j) Li[j][tid] /= L[j][j];
            __syncthreads();
#pragma unroll
            for (int u = 0; u < NB; ++u)
#pragma unroll
                for (int v = 0; v < NB; ++v) {
                    const int p = tp + 16 * u, c = tq + 16 * v;
                    const bool upd = p > j && p < rb && c <= j;
                    const float val = Li[p][c] - L[p][j] * Li[j][c];
                    *(upd ? &Li[p][c] : &sink[tid]) = val;   // dummy slot: see gram_cholesky
                }
            __syncthreads();
        }
    } else {
        __shared__ float sX[kFitMaxCols];
        for (int j = rb - 1; j >= 0; --j) {
            const float djj = 1.f / L[j][j];
            if (tid > j && tid < rb) sX[tid] = L[tid][j];
            __syncthreads();
            if (tid > j && tid < rb) {
                float sum = 0.f;
                for (int k = j + 1; k <= tid; ++k) sum += L[tid][k] * sX[k];
                L[tid][j] = -djj * sum;
            } else if (tid == j) {
                L[j][j] = djj;
            }
            __syncthreads();
        }
    }
    const int i = tid / LN, jq = tid % LN;
    const int nv = (rb - jq + LN - 1) / LN;
    ChunkStream<NB> cs;
    cs.init(rb);
    cs.fetch(Y, 0);
    for (int k0 = 0; k0 < a.X; k0 += CF::OR) {
        __syncthreads();                                 // the previous chunk is used
        cs.stage(sY);
        __syncthreads();
        if (k0 + CF::OR < a.X) cs.fetch(Y, k0 + CF::OR);
        float acc[SV] = {};
#pragma unroll 4
        for (int k = 0; k < rb; ++k) {
            const float y = sY[i][k];
#pragma unroll
            for (int v = 0; v < SV; ++v) acc[v] += y * M[min(jq + LN * v, CF::C - 1)][k];
        }
#pragma unroll
        for (int v = 0; v < SV; ++v)
            if (v < nv) out[(size_t)(k0 + i) * rb + jq + LN * v] = acc[v];
    }
}

// V = orth(W) by CholeskyQR2 (W L1^-T, then once more)
template <int NB>
__global__ __launch_bounds__(FT) void fit_orth_kernel(FitArgs a) {
    using CF = OrthCfg<NB>;
    __shared__ float L[CF::C][CF::P];
    __shared__ float Li[CF::SMALL ? CF::C : 1][CF::P];
    __shared__ float sY[CF::OR][CF::P];
    const int g = blockIdx.x;
    float *W = a.W + (size_t)g * a.X * a.rb;
    float *V = a.V + (size_t)g * a.X * a.rb;
    gram_cholesky<NB>(a, W, L, sY);
    solve_rows<NB>(a, W, V, L, Li, sY);
    __syncthreads();
    gram_cholesky<NB>(a, V, L, sY);
    solve_rows<NB>(a, V, V, L, Li, sY);
}

// Rayleigh-Ritz, first part: H = V^T W (W = C V), its eigenvectors by cyclic Jacobi sweeps.  Only
// H lives in LDS: each round's rotations (cos, sin and the column pair) are logged to the
// workspace, and fit_apply_kernel applies them to V's rows (V Q, Q never formed).  Also the order
// of the Ritz values (decreasing, ties by index) and sigma.
__global__ __launch_bounds__(FT) void fit_ritz_kernel(FitArgs a) {
    __shared__ float H[kFitMaxCols][kFitMaxCols + 1];
    __shared__ float rc[kFitMaxCols / 2], rs[kFitMaxCols / 2];
    __shared__ int rp[kFitMaxCols / 2], rq[kFitMaxCols / 2];
    const int g = blockIdx.x, rb = a.rb, tid = threadIdx.x;
    const float *V = a.V + (size_t)g * a.X * rb;
    const float *W = a.W + (size_t)g * a.X * rb;
    for (int e = tid; e < rb * rb; e += FT) {
        const int p = e / rb, q = e % rb;
        float s = 0.f;
        for (int k = 0; k < a.X; ++k) s += V[(size_t)k * rb + p] * W[(size_t)k * rb + q];
        H[p][q] = s;
    }
    __syncthreads();
    for (int e = tid; e < rb * rb; e += FT) {            // symmetrise
        const int p = e / rb, q = e % rb;
        if (p < q) {
            const float m = 0.5f * (H[p][q] + H[q][p]);
            H[p][q] = m;
            H[q][p] = m;
        }
    }
    __syncthreads();
    // cyclic Jacobi in round-robin order: rb - 1 rounds of rb / 2 disjoint pairs per sweep
    const int half = rb / 2;
    float4 *rot = a.rot + (size_t)g * kFitSweeps * (rb - 1) * half;
    for (int sweep = 0; sweep < kFitSweeps; ++sweep) {
        for (int round = 0; round < rb - 1; ++round) {
            if (tid < half) {
                // pair k of the round: positions k and rb - 1 - k of the rotating list, where
                // element 0 is fixed and the others rotate by `round`
                auto at = [&](int pos) { return pos == 0 ? 0 : 1 + (pos - 1 + round) % (rb - 1); };
                int p = at(tid), q = at(rb - 1 - tid);
                if (p > q) { const int t = p; p = q; q = t; }
                const float hpq = H[p][q];
                float c = 1.f, sn = 0.f;
                if (fabsf(hpq) > 1e-30f) {
                    const float th = (H[q][q] - H[p][p]) / (2.f * hpq);
                    const float t = (th >= 0.f ? 1.f : -1.f) / (fabsf(th) + sqrtf(th * th + 1.f));
                    c = 1.f / sqrtf(t * t + 1.f);
                    sn = t * c;
                }
                rp[tid] = p; rq[tid] = q; rc[tid] = c; rs[tid] = sn;
                rot[((size_t)sweep * (rb - 1) + round) * half + tid] =
                    make_float4(c, sn, __int_as_float(p), __int_as_float(q));
            }
            __syncthreads();
            for (int e = tid; e < half * rb; e += FT) {      // columns: H J
                const int k = e / rb, i = e % rb;
                const int p = rp[k], q = rq[k];
                const float c = rc[k], sn = rs[k];
                const float hp = H[i][p], hq = H[i][q];
                H[i][p] = c * hp - sn * hq;
                H[i][q] = sn * hp + c * hq;
            }
            __syncthreads();
            for (int e = tid; e < half * rb; e += FT) {      // rows: J^T H
                const int k = e / rb, j = e % rb;
                const int p = rp[k], q = rq[k];
                const float c = rc[k], sn = rs[k];
                const float hp = H[p][j], hq = H[q][j];
                H[p][j] = c * hp - sn * hq;
                H[q][j] = sn * hp + c * hq;
            }
            __syncthreads();
        }
    }
    // decreasing eigenvalue order (ties by index)
    if (tid < rb) {
        const float li = H[tid][tid];
        int rank = 0;
        for (int j = 0; j < rb; ++j) {
            const float lj = H[j][j];
            rank += (lj > li) || (lj == li && j < tid);
        }
        a.order[(size_t)g * kFitMaxCols + rank] = tid;
        if (a.sigma && rank < a.r) a.sigma[(size_t)g * a.r + rank] = sqrtf(fmaxf(li, 0.f));
    }
}

// Rayleigh-Ritz, second part: the logged rotations applied to 32 rows of V at a time (the rows of
// V Q, Q = the product of the rotations in order); the first r columns of V Q in Ritz order go to
// the workspace W (free once H is formed).  The next round's rotations load while this one is
// applied.
__global__ __launch_bounds__(FT) void fit_apply_kernel(FitArgs a) {
    __shared__ float sR[CR][kFitMaxCols + 1];
    __shared__ float4 sRot[2][kFitMaxCols / 2];
    const int rb = a.rb, tid = threadIdx.x, half = rb / 2;
    const int rows_per = a.X / CR;
    const int g = blockIdx.x / rows_per, r0 = (blockIdx.x % rows_per) * CR;
    const float *V = a.V + ((size_t)g * a.X + r0) * rb;
    for (int e = tid; e < CR * rb; e += FT) sR[e / rb][e % rb] = V[e];
    const int rounds = kFitSweeps * (rb - 1);
    const float4 *rot = a.rot + (size_t)g * rounds * half;
    float4 nxt = make_float4(1.f, 0.f, 0.f, 0.f);
    if (tid < half) nxt = rot[tid];
    for (int t = 0; t < rounds; ++t) {
        if (tid < half) sRot[t & 1][tid] = nxt;
        __syncthreads();                                 // this round's rotations and the rows
        if (tid < half && t + 1 < rounds) nxt = rot[(size_t)(t + 1) * half + tid];
        for (int e = tid; e < CR * half; e += FT) {
            const int row = e / half, k = e % half;
            const float4 r = sRot[t & 1][k];
            const int p = __float_as_int(r.z), q = __float_as_int(r.w);
            const float x = sR[row][p], y = sR[row][q];
            sR[row][p] = r.x * x - r.y * y;
            sR[row][q] = r.y * x + r.x * y;
        }
        __syncthreads();
    }
    const int *order = a.order + (size_t)g * kFitMaxCols;
    float *Y = a.W + ((size_t)g * a.X + r0) * rb;
    for (int e = tid; e < CR * a.r; e += FT) {
        const int row = e / a.r, c = e % a.r;
        Y[(size_t)row * rb + c] = sR[row][order[c]];
    }
}

// Outputs: each column's sign fixed so that its entry of largest magnitude (first on ties) is
// positive, then W_down and the W_up,t blocks in the codec dtype.
__global__ __launch_bounds__(FT) void fit_out_kernel(FitArgs a) {
    __shared__ float colsign[kFitMaxCols];
    const int g = blockIdx.x, rb = a.rb, tid = threadIdx.x;
    const float *Y = a.W + (size_t)g * a.X * rb;
    if (tid < a.r) {
        float best = -1.f;
        int arg = 0;
        for (int i = 0; i < a.X; ++i) {
            const float v = fabsf(Y[(size_t)i * rb + tid]);
            if (v > best) { best = v; arg = i; }
        }
        colsign[tid] = Y[(size_t)arg * rb + tid] < 0.f ? -1.f : 1.f;
    }
    __syncthreads();
    const int Dg = a.X / a.T;
    for (int e = tid; e < a.X * a.r; e += FT) {
        const int i = e / a.r, c = e % a.r;
        const float v = colsign[c] * Y[(size_t)i * rb + c];
        const size_t wd = ((size_t)g * a.X + i) * a.r + c;
        const int t = i / Dg, k = i - t * Dg;
        const size_t wu = (((size_t)t * a.G + g) * a.r + c) * Dg + k;
        if (a.bf16) {
            static_cast<uint16_t *>(a.Wd_out)[wd] = f2bf(v);
            static_cast<uint16_t *>(a.Wu_out)[wu] = f2bf(v);
        } else {
            static_cast<float *>(a.Wd_out)[wd] = v;
            static_cast<float *>(a.Wu_out)[wu] = v;
        }
    }
}

}  // namespace

size_t fit_workspace_floats(int G, int X, int r, long n, int *S_out) {
    const int nb = X / CB;
    const int pairs = nb * (nb + 1) / 2;
    int S = (1024 + G * pairs - 1) / (G * pairs);
    const long chunks = (n + CK - 1) / CK;
    if (S > chunks) S = (int)(chunks > 0 ? chunks : 1);
    if (S > 16) S = 16;
    if (S < 1) S = 1;
    if (S_out) *S_out = S;
    const int rb = fit_block_cols(r);
    return (size_t)S * G * X * X + (size_t)S * G * X + (size_t)G * X * X + (size_t)G * X +
           2 * (size_t)G * X * rb + fit_rotation_floats(G, rb) + (size_t)G * kFitMaxCols;
}

size_t fit_rotation_floats(int G, int rb) {
    return (size_t)G * kFitSweeps * (rb - 1) * (rb / 2) * 4;
}

int fit_block_cols(int r) {
    int rb = r + 8;
    rb += rb & 1;
    return rb > kFitMaxCols ? kFitMaxCols : rb;
}

template <int NB>
void launch_step(const FitArgs &a, bool mul, hipStream_t st) {
    if (mul)
        hipLaunchKernelGGL(fit_mul_kernel<NB>, dim3(a.G * (a.X / 32)), dim3(FT), 0, st, a);
    else
        hipLaunchKernelGGL(fit_orth_kernel<NB>, dim3(a.G), dim3(FT), 0, st, a);
}

// W = C V (mul) or V = orth(W), instantiated for NB = ceil(rb / 16)
void launch_iter(const FitArgs &a, bool mul, hipStream_t st) {
    switch ((a.rb + 15) / 16) {
    case 1: launch_step<1>(a, mul, st); break;
    case 2: launch_step<2>(a, mul, st); break;
    case 3: launch_step<3>(a, mul, st); break;
    case 4: launch_step<4>(a, mul, st); break;
    case 5: launch_step<5>(a, mul, st); break;
    case 6: launch_step<6>(a, mul, st); break;
    case 7: launch_step<7>(a, mul, st); break;
    case 8: launch_step<8>(a, mul, st); break;
    case 9: launch_step<9>(a, mul, st); break;
    case 10: launch_step<10>(a, mul, st); break;
    default: launch_step<11>(a, mul, st); break;
    }
}

hipError_t launch_fit(FitArgs a, hipStream_t st) {
    const int nb = a.X / CB;
    const int pairs = nb * (nb + 1) / 2;
    hipLaunchKernelGGL(fit_cov_kernel, dim3(a.G * pairs * a.S), dim3(FT), 0, st, a);
    const size_t cells = (size_t)a.G * a.X * a.X;
    hipLaunchKernelGGL(fit_reduce_kernel, dim3((unsigned)((cells + FT - 1) / FT)), dim3(FT), 0,
                       st, a);
    const size_t vcells = (size_t)a.G * a.X * a.rb;
    hipLaunchKernelGGL(fit_init_kernel, dim3((unsigned)((vcells + FT - 1) / FT)), dim3(FT), 0, st,
                       a);
    launch_iter(a, false, st);
    for (int it = 0; it < a.iters; ++it) {
        launch_iter(a, true, st);
        launch_iter(a, false, st);
    }
    launch_iter(a, true, st);
    hipLaunchKernelGGL(fit_ritz_kernel, dim3(a.G), dim3(FT), 0, st, a);
    hipLaunchKernelGGL(fit_apply_kernel, dim3(a.G * (a.X / CR)), dim3(FT), 0, st, a);
    hipLaunchKernelGGL(fit_out_kernel, dim3(a.G), dim3(FT), 0, st, a);
    return hipGetLastError();
}

}  // namespace lla
