// fit.hip -- codec fit from the top right singular vectors of the activations, bf16, gfx950.
//
// pith.science paper page for "Looped Latent Attention", "What carries the argument": the codec
// is initialised from the top right singular vectors of teacher activations.  Per group g the
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
//   fit_ritz_kernel    Rayleigh-Ritz and the outputs, one workgroup per group.
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
constexpr int CK = 32;           // rows per staged chunk
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
    int id = blockIdx.x;
    const int s = id % a.S;
    id /= a.S;
    int pr = id % pairs;
    const int g = id / pairs;
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

    // staging: thread tid loads the 16-byte piece (row tid / 16, columns 8 (tid % 16) ..) of each
    // strip, i.e. both strips are 32 rows x 128 columns = 512 pieces, two per thread each
    uint4 pi[2], pj[2];
    auto fetch = [&](int c0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int p = tid + FT * u;
            const int row = min(c0 + p / 16, max(r1 - 1, 0));
            const bool live = c0 + p / 16 < r1;
            const int col = 8 * (p % 16);
            pi[u] = live ? *reinterpret_cast<const uint4 *>(x + stage_off(a, row, g, CB * bi + col))
                         : make_uint4(0, 0, 0, 0);
            pj[u] = live ? *reinterpret_cast<const uint4 *>(x + stage_off(a, row, g, CB * bj + col))
                         : make_uint4(0, 0, 0, 0);
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int p = tid + FT * u;
            const int rr = p / 16, col = 8 * (p % 16);
            const uint32_t wi[4] = {pi[u].x, pi[u].y, pi[u].z, pi[u].w};
            const uint32_t wj[4] = {pj[u].x, pj[u].y, pj[u].z, pj[u].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sI[col + e][rr] = static_cast<uint16_t>(wi[e >> 1] >> (16 * (e & 1)));
                sJ[col + e][rr] = static_cast<uint16_t>(wj[e >> 1] >> (16 * (e & 1)));
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

// W = C V: workgroup (g, rows 32 q .. + 31); 64-wide k-chunks of C's rows and V's rows are staged
// in LDS with coalesced loads; thread (row tid / 8, columns tid % 8 + 8 u) accumulates in fp32
__global__ __launch_bounds__(FT) void fit_mul_kernel(FitArgs a) {
    __shared__ float sC[32][64 + 1];
    __shared__ float sV[64][kFitMaxCols + 1];
    const int rows_per = a.X / 32;
    const int g = blockIdx.x / rows_per, q = blockIdx.x % rows_per;
    const int tid = threadIdx.x;
    const int il = tid / 8, c0 = tid % 8;
    const float *C = a.C + ((size_t)g * a.X + 32 * q) * a.X;
    const float *V = a.V + (size_t)g * a.X * a.rb;
    float acc[kFitMaxCols / 8] = {};
    for (int k0 = 0; k0 < a.X; k0 += 64) {
        __syncthreads();
        for (int e = tid; e < 32 * 64; e += FT) sC[e / 64][e % 64] = C[(size_t)(e / 64) * a.X + k0 + e % 64];
        for (int e = tid; e < 64 * a.rb; e += FT)
            sV[e / a.rb][e % a.rb] = V[(size_t)k0 * a.rb + e];
        __syncthreads();
        for (int k = 0; k < 64; ++k) {
            const float cik = sC[il][k];
#pragma unroll
            for (int u = 0; u < kFitMaxCols / 8; ++u)
                if (c0 + 8 * u < a.rb) acc[u] += cik * sV[k][c0 + 8 * u];
        }
    }
#pragma unroll
    for (int u = 0; u < kFitMaxCols / 8; ++u)
        if (c0 + 8 * u < a.rb) a.W[((size_t)g * a.X + 32 * q + il) * a.rb + c0 + 8 * u] = acc[u];
}

// Cholesky factor L (lower, rb x rb, in LDS) of the Gram matrix of the X x rb block Y (global).
// The Gram matrix accumulates over 64-row chunks of Y staged in LDS.  A pivot below a tiny
// fraction of the trace is clamped (rank-deficient blocks stay finite).
__device__ void gram_cholesky(const FitArgs &a, const float *Y, float (*L)[kFitMaxCols + 1],
                              float (*sY)[kFitMaxCols + 1]) {
    const int rb = a.rb, tid = threadIdx.x;
    constexpr int PMAX = kFitMaxCols * (kFitMaxCols + 1) / 2;
    constexpr int PPT = (PMAX + FT - 1) / FT;            // pairs per thread
    float acc[PPT] = {};
    const int npairs = rb * (rb + 1) / 2;
    int pp[PPT], qq[PPT];
#pragma unroll
    for (int u = 0; u < PPT; ++u) {                      // pair e -> (p >= q)
        int e = tid + FT * u, p = 0;
        if (e >= npairs) e = 0;
        while (e >= p + 1) { e -= p + 1; ++p; }
        pp[u] = p;
        qq[u] = e;
    }
    for (int k0 = 0; k0 < a.X; k0 += 64) {
        __syncthreads();
        for (int e = tid; e < 64 * rb; e += FT) sY[e / rb][e % rb] = Y[(size_t)k0 * rb + e];
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
            if (tid + FT * u >= npairs) continue;
            float s = acc[u];
            for (int k = 0; k < 64; ++k) s += sY[k][pp[u]] * sY[k][qq[u]];
            acc[u] = s;
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PPT; ++u)
        if (tid + FT * u < npairs) L[pp[u]][qq[u]] = acc[u];
    __syncthreads();
    __shared__ float tr;
    if (tid == 0) {
        float t = 0.f;
        for (int p = 0; p < rb; ++p) t += L[p][p];
        tr = t;
    }
    __syncthreads();
    const float floor_ = 1e-12f * tr + 1e-30f;
    for (int j = 0; j < rb; ++j) {
        if (tid == 0) {
            float d = L[j][j];
            for (int k = 0; k < j; ++k) d -= L[j][k] * L[j][k];
            L[j][j] = sqrtf(fmaxf(d, floor_));
        }
        __syncthreads();
        for (int p = j + 1 + tid; p < rb; p += FT) {
            float v = L[p][j];
            for (int k = 0; k < j; ++k) v -= L[p][k] * L[j][k];
            L[p][j] = v / L[j][j];
        }
        __syncthreads();
    }
}

// out = Y L^{-T}.  L^{-1} (lower triangular) is formed in LDS, one column per thread by forward
// substitution; then every 64-row chunk of Y is staged in LDS and multiplied by L^{-T}
// (out[i][j] = sum_{k <= j} Y[i][k] Linv[j][k]).  out may alias Y: a chunk is read completely
// before any of it is written.
__device__ void solve_rows(const FitArgs &a, const float *Y, float *out,
                           float (*L)[kFitMaxCols + 1], float (*Li)[kFitMaxCols + 1],
                           float (*sY)[kFitMaxCols + 1]) {
    const int rb = a.rb, tid = threadIdx.x;
    if (tid < rb) {
        const int c = tid;
        for (int j = 0; j < rb; ++j) Li[j][c] = 0.f;
        Li[c][c] = 1.f / L[c][c];
        for (int j = c + 1; j < rb; ++j) {
            float s = 0.f;
            for (int k = c; k < j; ++k) s += L[j][k] * Li[k][c];
            Li[j][c] = -s / L[j][j];
        }
    }
    __syncthreads();
    for (int k0 = 0; k0 < a.X; k0 += 64) {
        for (int e = tid; e < 64 * rb; e += FT) sY[e / rb][e % rb] = Y[(size_t)k0 * rb + e];
        __syncthreads();
        for (int e = tid; e < 64 * rb; e += FT) {
            const int i = e / rb, j = e % rb;
            float s = 0.f;
            for (int k = 0; k <= j; ++k) s += sY[i][k] * Li[j][k];
            out[(size_t)(k0 + i) * rb + j] = s;
        }
        __syncthreads();
    }
}

// V = orth(W) by CholeskyQR2 (W L1^-T, then once more)
__global__ __launch_bounds__(FT) void fit_orth_kernel(FitArgs a) {
    __shared__ float L[kFitMaxCols][kFitMaxCols + 1];
    __shared__ float Li[kFitMaxCols][kFitMaxCols + 1];
    __shared__ float sY[64][kFitMaxCols + 1];
    const int g = blockIdx.x;
    float *W = a.W + (size_t)g * a.X * a.rb;
    float *V = a.V + (size_t)g * a.X * a.rb;
    gram_cholesky(a, W, L, sY);
    solve_rows(a, W, V, L, Li, sY);
    gram_cholesky(a, V, L, sY);
    solve_rows(a, V, V, L, Li, sY);
}

// Rayleigh-Ritz: H = V^T W (W = C V), Jacobi eigenvectors, sorted top r, outputs
__global__ __launch_bounds__(FT) void fit_ritz_kernel(FitArgs a) {
    __shared__ float H[kFitMaxCols][kFitMaxCols + 1];
    __shared__ float Q[kFitMaxCols][kFitMaxCols + 1];
    __shared__ float rc[kFitMaxCols / 2], rs[kFitMaxCols / 2];
    __shared__ int rp[kFitMaxCols / 2], rq[kFitMaxCols / 2];
    __shared__ int order[kFitMaxCols];
    __shared__ float colmax[kFitMaxCols];
    const int g = blockIdx.x, rb = a.rb, tid = threadIdx.x;
    const float *V = a.V + (size_t)g * a.X * rb;
    const float *W = a.W + (size_t)g * a.X * rb;
    for (int e = tid; e < rb * rb; e += FT) {
        const int p = e / rb, q = e % rb;
        float s = 0.f;
        for (int k = 0; k < a.X; ++k) s += V[(size_t)k * rb + p] * W[(size_t)k * rb + q];
        H[p][q] = s;
        Q[p][q] = p == q ? 1.f : 0.f;
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
            }
            __syncthreads();
            for (int e = tid; e < half * rb; e += FT) {      // columns: H J, Q J
                const int k = e / rb, i = e % rb;
                const int p = rp[k], q = rq[k];
                const float c = rc[k], sn = rs[k];
                const float hp = H[i][p], hq = H[i][q];
                H[i][p] = c * hp - sn * hq;
                H[i][q] = sn * hp + c * hq;
                const float qp = Q[i][p], qq = Q[i][q];
                Q[i][p] = c * qp - sn * qq;
                Q[i][q] = sn * qp + c * qq;
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
        order[rank] = tid;
    }
    __syncthreads();
    // W_down column c = V Q[:, order[c]]; written to the workspace W first for the sign pass
    float *Y = a.W + (size_t)g * a.X * rb;
    __syncthreads();                                     // every thread has read W for H
    for (int e = tid; e < a.X * a.r; e += FT) {
        const int i = e / a.r, c = e % a.r;
        const int src = order[c];
        float s = 0.f;
        for (int k = 0; k < rb; ++k) s += V[(size_t)i * rb + k] * Q[k][src];
        Y[(size_t)i * rb + c] = s;                       // W's rows are only read above
    }
    __threadfence_block();
    __syncthreads();
    // sign: the entry of largest magnitude (first on ties) of each column is positive
    if (tid < a.r) {
        float best = -1.f;
        int arg = 0;
        for (int i = 0; i < a.X; ++i) {
            const float v = fabsf(Y[(size_t)i * rb + tid]);
            if (v > best) { best = v; arg = i; }
        }
        colmax[tid] = Y[(size_t)arg * rb + tid] < 0.f ? -1.f : 1.f;
        if (a.sigma) a.sigma[(size_t)g * a.r + tid] = sqrtf(fmaxf(H[order[tid]][order[tid]], 0.f));
    }
    __syncthreads();
    const int Dg = a.X / a.T;
    for (int e = tid; e < a.X * a.r; e += FT) {
        const int i = e / a.r, c = e % a.r;
        const float v = colmax[c] * Y[(size_t)i * rb + c];
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
           2 * (size_t)G * X * rb;
}

int fit_block_cols(int r) {
    int rb = r + 8;
    rb += rb & 1;
    return rb > kFitMaxCols ? kFitMaxCols : rb;
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
    hipLaunchKernelGGL(fit_orth_kernel, dim3(a.G), dim3(FT), 0, st, a);
    for (int it = 0; it < a.iters; ++it) {
        hipLaunchKernelGGL(fit_mul_kernel, dim3(a.G * (a.X / 32)), dim3(FT), 0, st, a);
        hipLaunchKernelGGL(fit_orth_kernel, dim3(a.G), dim3(FT), 0, st, a);
    }
    hipLaunchKernelGGL(fit_mul_kernel, dim3(a.G * (a.X / 32)), dim3(FT), 0, st, a);
    hipLaunchKernelGGL(fit_ritz_kernel, dim3(a.G), dim3(FT), 0, st, a);
    return hipGetLastError();
}

}  // namespace lla
