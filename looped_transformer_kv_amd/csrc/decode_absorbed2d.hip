// decode_absorbed2d.hip -- absorbed-attention decode for LLA-2D codecs, all heads per workgroup.
//
// LLA-2D (arXiv abstract: the extreme-compression regime) keeps one latent per token, layer and
// axis for all heads, so the per-head decode workgroups of decode_absorbed.hip would each read
// the whole latent stream: H times the bytes the call needs.  Here one workgroup takes a context
// split of one sequence and serves every head from the same bytes.  The attention is the
// absorbed form (the editorial letter on the pith.science paper page for "Looped Latent
// Attention"; exact up to rounding while no rotation sits between expansion and attention):
//   q~_h = W_up,t^K[:, head h] q_h                  (r_k values per head)
//   s_hj = scale (<q~_h, c_k(j)> + <q_h, mu_t^K[h]>)
//   c~_h = sum_j softmax_h(s)_j c_v(j)              (r_v values per head)
//   out_h = c~_h W_up,t^V[:, head h] + mu_t^V[h]    (plus the current token's own key/value)
//
// Three launches:
//   1. absorb_q:  q~ (log2-scaled) for every (sequence, head), stored as a bf16 pair hi + lo
//                 (hi = bf16(q~), lo = bf16(q~ - hi): about 16 significant bits), <q, mu^K> and
//                 the current token's own score.
//   2. stream:    one workgroup of 4 waves per (sequence, split); the waves take 32-token chunks
//                 round-robin.  Per chunk, on the matrix cores (v_mfma_f32_16x16x32_bf16):
//                   scores  S[token][head] = C_k[token][:] . Q~[:][head]      (hi and lo terms)
//                   values  A[rank][head] += C_v^T[rank][token] . P[token][head] (hi and lo)
//                 The key latents are the A operand in their own row-major layout (lane l holds
//                 token l % 16, ranks 8 (l / 16) .. +7 of a 32-rank slice).  The value latents
//                 need the token index as the contraction index, so each chunk goes to a
//                 wave-private LDS block in token-major rows and comes back through
//                 ds_read_b64_tr_b16, which hands lane l rank l % 16 of four tokens.  The 32
//                 tokens are taken in the order k = 8 g + e -> token 16 (e / 4) + 4 g + e % 4
//                 (g = lane / 16), which is exactly where the score MFMA left each lane's
//                 softmax weights, so P never moves between lanes.  Each lane owns one head
//                 (lane % 16) for the whole call: its running max, its sum and its rows of the
//                 value accumulators.
//   3. combine:   one workgroup per (sequence, head) merges the splits' (c~, m, l), expands
//                 c~ W_up,t^V once, adds mu and the self term.
// Heads beyond H (H < 16) are zero columns.  Tokens past a sequence's end re-read its last token
// and get weight 0; an out-of-range page id makes that sequence's outputs NaN.
#include "lla_internal.h"

namespace lla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kWaves = 4;
#ifndef ABS2D_DEPTH
#define ABS2D_DEPTH 1
#endif
#ifndef ABS2D_OCC
#define ABS2D_OCC 2
#endif

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
    return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

// ---------------------------------------------------------------- 1. q~, <q, mu^K>, self score
// One workgroup per (sequence, head column).  Thread t owns the 8 head dims 8 (t % NPC) .. + 7
// (NPC = D / 8) of the rows k = t / NPC + RPP i; every load is issued before the first use, and
// each row's NPC partial dots are summed across the lanes of a DPP row group in a fixed order.
template <int D, int RK>
__global__ __launch_bounds__(256) void absorb_q_kernel(DecodeArgs a) {
    constexpr int NPC = D / 8;                 // 16-byte pieces per head slice of a row
    constexpr int RPP = 256 / NPC;             // rows per pass
    constexpr int PASSES = (RK + RPP - 1) / RPP;
    const Abs2dLayout L = abs2d_layout(a.B, a.S, RK, a.r_v);
    const int b = blockIdx.x / kAbs2dHeads, h = blockIdx.x % kAbs2dHeads;
    const int tid = threadIdx.x;
    uint16_t *hi = reinterpret_cast<uint16_t *>(a.ws + L.qt) + ((size_t)b * 2 * kAbs2dHeads + h) * RK;
    uint16_t *lo = hi + (size_t)kAbs2dHeads * RK;
    float *qm = a.ws + L.qm + (size_t)b * kAbs2dHeads + h;
    float *sself = a.ws + L.self + (size_t)b * kAbs2dHeads + h;
    if (h >= a.H) {                       // padding column
        if (tid < RK) hi[tid] = lo[tid] = 0;
        if (tid == 0) {
            *qm = 0.f;
            *sself = -INFINITY;
        }
        return;
    }
    const int pc = tid % NPC, kr = tid / NPC;
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) + ((size_t)b * a.H + h) * D;
    const uint16_t *wbase = static_cast<const uint16_t *>(a.W_up_k) + (size_t)a.t * RK * a.Dg +
                            (size_t)h * D + 8 * pc;
    uint4 w[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        const int k = min(kr + RPP * i, RK - 1);
        w[i] = *reinterpret_cast<const uint4 *>(wbase + (size_t)k * a.Dg);
    }
    const uint4 qq = *reinterpret_cast<const uint4 *>(qp + 8 * pc);
    // <q, mu_t^K> and the self score, same piece layout (element loads: mu and the self rows
    // carry no alignment requirement)
    auto load8 = [](const uint16_t *p) {
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = pack2(p[2 * e], p[2 * e + 1]);
        return uint4{v[0], v[1], v[2], v[3]};
    };
    uint4 mk = {0u, 0u, 0u, 0u}, ks = {0u, 0u, 0u, 0u};
    if (tid < NPC) {
        mk = load8(static_cast<const uint16_t *>(a.mu_k) + (size_t)a.t * a.Dg + (size_t)h * D +
                   8 * pc);
        if (a.k_self)
            ks = load8(static_cast<const uint16_t *>(a.k_self) + (size_t)b * a.self_stride +
                       (size_t)h * D + 8 * pc);
    }
    const uint32_t qv[4] = {qq.x, qq.y, qq.z, qq.w};
    auto dot8 = [&](const uint4 &x) {
        const uint32_t xv[4] = {x.x, x.y, x.z, x.w};
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc += __uint_as_float(xv[e] << 16) * __uint_as_float(qv[e] << 16);
            acc += __uint_as_float(xv[e] & 0xffff0000u) * __uint_as_float(qv[e] & 0xffff0000u);
        }
        return acc;
    };
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        const float v = group_sum<NPC>(dot8(w[i])) * a.scale_log2;
        const int k = kr + RPP * i;
        if (pc == 0 && k < RK) {
            const uint16_t vh = f2bf(v);
            hi[k] = vh;
            lo[k] = f2bf(v - bf2f(vh));
        }
    }
    if (tid < NPC) {                      // the first row group: lanes 0 .. NPC-1
        const float am = group_sum<NPC>(dot8(mk));
        const float as = group_sum<NPC>(dot8(ks));
        if (tid == 0) {
            *qm = am * a.scale_log2;
            *sself = a.k_self ? as * a.scale_log2 : -INFINITY;
        }
    }
}

// ---------------------------------------------------------------- 2. the latent stream
template <int RK, int RV>
struct Abs2dChunk {
    uint4 k[2][RK / 32];   // key latents: A operands of the two 16-token score blocks
    uint4 v[RV / 16];      // value latents: 16-byte pieces, 64 consecutive pieces per step
};

template <int RK, int RV, int DEPTH, int OCC>
__global__ __launch_bounds__(64 * kWaves, OCC) void absorbed2d_kernel(DecodeArgs a) {
    constexpr int NKK = RK / 32;                 // 32-rank slices of a key latent
    constexpr int NVB = RV / 16;                 // 16-rank blocks of a value latent
    constexpr int NPR = RV / 8;                  // 16-byte pieces per value row
    // LDS row stride in dwords: >= RV / 2 and = 8 mod 16, so the 16 rows a transposed read
    // touches (8 bytes x 4 lanes per row) fall on distinct banks in each half-wave
    constexpr int VSTR = (RV / 2) % 16 == 8 ? RV / 2 : RV / 2 + 8;
    static_assert(RK % 32 == 0 && RV % 16 == 0, "rank shapes");
    static_assert(32 * VSTR >= kAbs2dHeads * RV, "merge buffer fits the staging block");

    __shared__ __align__(16) uint32_t sV[kWaves][32 * VSTR];
    __shared__ float sM[kWaves][kAbs2dHeads], sL[kWaves][kAbs2dHeads];
    __shared__ int sSlot[kMaxChunksPerSplit];

    const Abs2dLayout lay = abs2d_layout(a.B, a.S, RK, RV);
    const int S = a.S;
    const int id = xcd_work_item(blockIdx.x, gridDim.x);
    const int s = id % S;
    const int b = id / S;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, g = lane >> 4;

    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_seq_len ? a.max_seq_len : len);
    const int j_begin = s * a.tokens_per_split;
    const int j_end = min(j_begin + a.tokens_per_split, len);
    const int nchunks = j_end > j_begin ? (j_end - j_begin + 31) >> 5 : 0;
    const int32_t *bt = a.block_table + (size_t)b * a.max_pages;
    auto slot_of = [&](int c) {   // chunk c -> pool row of its first token; negative: bad page
        const int j = j_begin + 32 * c;
        const int page = bt[min(j / a.P, a.max_pages - 1)];
        const bool bad = (unsigned)page >= (unsigned)a.n_pages;
        const int row = (bad ? 0 : page) * a.P + j % a.P;
        return bad ? -row - 1 : row;
    };

    const uint16_t *kpool = static_cast<const uint16_t *>(a.k_pool);
    const uint16_t *vpool = static_cast<const uint16_t *>(a.v_pool);
    auto load_slot = [&](int c, int slot, Abs2dChunk<RK, RV> &x) {
        const int row = __builtin_amdgcn_readfirstlane(slot < 0 ? -slot - 1 : slot);
        const int last = max(min(j_end - (j_begin + 32 * c), 32) - 1, 0);
        const uint16_t *kb = kpool + (size_t)row * RK;
        const uint16_t *vb = vpool + (size_t)row * RV;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int tok = min(16 * blk + c16, last);
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                x.k[blk][kk] = *reinterpret_cast<const uint4 *>(kb + tok * RK + 32 * kk + 8 * g);
        }
#pragma unroll
        for (int u = 0; u < NVB; ++u) {
            const int p = lane + 64 * u;
            const int tok = min(p / NPR, last);
            x.v[u] = *reinterpret_cast<const uint4 *>(vb + (tok * NPR + p % NPR) * 8);
        }
    };

    // ---- prologue.  A wave's vector loads complete in order, so the small loads go out before
    // the latent burst: (1) the page-table entries of this wave's first chunks, (2) the q~ operands,
    // <q, mu^K> and the table entries of this wave's own chunks (c = wave + kWaves * (lane + 64 u);
    // only this wave reads them, so no barrier is needed), (3) the first latent chunks.  Every
    // load is unconditional at a clamped in-bounds index (a load under a branch waits at the join).
    const int c_last = max(nchunks - 1, 0);
    int first[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) first[i] = slot_of(wave + i * kWaves);

    // B operands of the score MFMA: lane l holds head l % 16, ranks 32 kk + 8 g .. + 7
    bf16x8 qhi[NKK], qlo[NKK];
    {
        const uint16_t *qt = reinterpret_cast<const uint16_t *>(a.ws + lay.qt) +
                             ((size_t)b * 2 * kAbs2dHeads + c16) * RK + 8 * g;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            qhi[kk] = as_bf16x8(*reinterpret_cast<const uint4 *>(qt + 32 * kk));
            qlo[kk] = as_bf16x8(*reinterpret_cast<const uint4 *>(qt + kAbs2dHeads * RK + 32 * kk));
        }
    }
    const float qm = a.ws[lay.qm + (size_t)b * kAbs2dHeads + c16];
    constexpr int US = (kMaxChunksPerSplit / kWaves + 63) / 64;
    int slot_reg[US];
#pragma unroll
    for (int u = 0; u < US; ++u) slot_reg[u] = slot_of(min(wave + kWaves * (lane + 64 * u), c_last));
    __builtin_amdgcn_sched_barrier(0);

    Abs2dChunk<RK, RV> buf[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) load_slot(wave + i * kWaves, first[i], buf[i]);
#pragma unroll
    for (int u = 0; u < US; ++u) {
        const int c = wave + kWaves * (lane + 64 * u);
        if (c < nchunks) sSlot[c] = slot_reg[u];
    }

    float m_run = -INFINITY, l_lane = 0.f;
    f32x4 acc[NVB];
#pragma unroll
    for (int nb = 0; nb < NVB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint32_t *wv = sV[wave];
    // transposed-read addresses: this lane, as a source row of the read, names token
    // 16 hf + 4 g + c16 / 4 and ranks 16 nb + 4 (c16 % 4) .. + 3
    const uint32_t rd_base = (uint32_t)((4 * g + (c16 >> 2)) * VSTR * 4 + (c16 & 3) * 8);

    // scores of chunk c and its value latents to LDS; returns the 8 scores (log2 domain)
    auto stage = [&](int c, const Abs2dChunk<RK, RV> &x, f32x4 (&sc)[2]) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            sc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                sc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(x.k[blk][kk]), qhi[kk],
                                                                  sc[blk], 0, 0, 0);
                sc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(x.k[blk][kk]), qlo[kk],
                                                                  sc[blk], 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < NVB; ++u) {
            const int p = lane + 64 * u;
            *reinterpret_cast<uint4 *>(wv + (p / NPR) * VSTR + (p % NPR) * 4) = x.v[u];
        }
        __builtin_amdgcn_wave_barrier();
    };

    auto finish = [&](int c, f32x4 (&sc)[2]) {
        const int valid = j_end - (j_begin + 32 * c);   // >= 1, wave-uniform
        const bool bad = sSlot[c] < 0;
        float x[8];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * blk + 4 * g + i;
                float v = tok < valid ? sc[blk][i] + qm : -INFINITY;
                x[4 * blk + i] = bad ? __builtin_nanf("") : v;
            }
        float cm = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) cm = fmaxf(cm, x[e]);
        cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(cm), __float_as_uint(cm),
                                                         false, false);
        cm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        if (__builtin_amdgcn_ballot_w64(cm > m_run) != 0) {
            if (cm > m_run) {
                const float alpha = exp2_(m_run - cm);
                l_lane *= alpha;
#pragma unroll
                for (int nb = 0; nb < NVB; ++nb) acc[nb] *= alpha;
                m_run = cm;
            }
        }
        uint32_t ph[4], pl[4];
        float lsum = 0.f;
        const float mr = m_run == -INFINITY ? 0.f : m_run;   // no score yet: every p is 0
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float p0 = exp2_(x[e] - mr), p1 = exp2_(x[e + 1] - mr);
            lsum += p0 + p1;
            const uint16_t h0 = f2bf(p0), h1 = f2bf(p1);
            ph[e / 2] = pack2(h0, h1);
            pl[e / 2] = pack2(f2bf(p0 - bf2f(h0)), f2bf(p1 - bf2f(h1)));
        }
        l_lane += lsum;
        const bf16x8 Phi = __builtin_bit_cast(bf16x8, uint4{ph[0], ph[1], ph[2], ph[3]});
        const bf16x8 Plo = __builtin_bit_cast(bf16x8, uint4{pl[0], pl[1], pl[2], pl[3]});
        lds_char *base = (lds_char *)wv;
#pragma unroll
        for (int nb = 0; nb < NVB; ++nb) {
            const uint32_t off = rd_base + nb * 32;
            const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + off));
            const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(base + off + 16 * VSTR * 4));
            const uint4 vt = {pack2((uint16_t)r0[0], (uint16_t)r0[1]),
                              pack2((uint16_t)r0[2], (uint16_t)r0[3]),
                              pack2((uint16_t)r1[0], (uint16_t)r1[1]),
                              pack2((uint16_t)r1[2], (uint16_t)r1[3])};
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vt), Phi, acc[nb], 0, 0, 0);
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vt), Plo, acc[nb], 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
    };

    if (wave < nchunks) {
        int c = wave;
        for (;;) {
            bool done = false;
#pragma unroll
            for (int i = 0; i < DEPTH; ++i) {
                if (!done) {
                    f32x4 sc[2];
                    stage(c, buf[i], sc);
                    const int nxt = c + DEPTH * kWaves;
                    if (nxt < nchunks) load_slot(nxt, sSlot[nxt], buf[i]);
                    finish(c, sc);
                    c += kWaves;
                    done = c >= nchunks;
                }
            }
            if (done) break;
        }
    }

    // ---- merge the waves: per head, rescale to the common max and add, in wave order
    const float l_head = add_swap32(l_lane + __shfl_xor(l_lane, 16, 64));
    __syncthreads();                             // every wave is done with its staging block
    float *sAcc = reinterpret_cast<float *>(&sV[0][0]);   // [kWaves][16][RV] after the stream
    float *mine = sAcc + (size_t)wave * 32 * VSTR;
#pragma unroll
    for (int nb = 0; nb < NVB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[c16 * RV + 16 * nb + 4 * g + i] = acc[nb][i];
    if (g == 0) {
        sM[wave][c16] = m_run;
        sL[wave][c16] = l_head;
    }
    __syncthreads();
    float *part = a.ws + lay.part + ((size_t)b * S + s) * kAbs2dHeads * RV;
    for (int idx = tid; idx < kAbs2dHeads * RV; idx += 64 * kWaves) {
        const int h = idx / RV;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sM[w][h]);
        float v = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
                v += sAcc[(size_t)w * 32 * VSTR + idx] * exp2_(sM[w][h] - M);
        }
        part[idx] = v;
    }
    if (tid < kAbs2dHeads) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sM[w][tid]);
        float Lsum = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) Lsum += sL[w][tid] * exp2_(sM[w][tid] - M);
        }
        float *st = a.ws + lay.stat + (((size_t)b * S + s) * kAbs2dHeads + tid) * 2;
        st[0] = M;
        st[1] = Lsum;
    }
}

// ---------------------------------------------------------------- 3. merge splits and expand
// One workgroup of 256 threads per (sequence, head).  Two dependent rounds of loads: the W_up,t^V
// slice of the head (thread t: 8 columns 8 (t % NPC) .. + 7 of rows t / NPC + NKG i) together
// with the splits' (max, sum); then the splits' partial latents.  Every sum runs in a fixed
// order (splits by residue class, then the classes in order; rows by group, then the groups).
template <int D, int RV>
__global__ __launch_bounds__(256) void absorbed2d_combine_kernel(DecodeArgs a) {
    constexpr int NPC = D / 8;                     // 16-byte column pieces of a W row slice
    constexpr int NKG = 256 / NPC;                 // row groups
    constexpr int WROWS = (RV + NKG - 1) / NKG;    // rows per thread
    constexpr int NK4 = RV / 4;                    // float4 pieces of a partial latent
    constexpr int NSG = 256 / NK4;                 // split classes
    const Abs2dLayout lay = abs2d_layout(a.B, a.S, a.r_k, RV);
    const int b = blockIdx.x / a.H, h = blockIdx.x % a.H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int S = a.S;
    __shared__ float sW[kMaxAbs2dSplits];
    __shared__ __align__(16) float sRed[NKG * D > NSG * RV ? NKG * D : NSG * RV];
    __shared__ float sC[RV];
    __shared__ float sML[2];

    // ---- round 1: the W slice and the split statistics
    const int pc = tid % NPC, kg = tid / NPC;
    const uint16_t *wbase = static_cast<const uint16_t *>(a.W_up_v) + (size_t)a.t * RV * a.Dg +
                            (size_t)h * D + 8 * pc;
    uint4 w[WROWS];
#pragma unroll
    for (int i = 0; i < WROWS; ++i) {
        const int k = min(kg + NKG * i, RV - 1);
        w[i] = *reinterpret_cast<const uint4 *>(wbase + (size_t)k * a.Dg);
    }
    // split statistics, 4 per thread: (max, sum) of split 4 tid + j
    const float2 *st = reinterpret_cast<const float2 *>(a.ws + lay.stat) +
                       (size_t)b * S * kAbs2dHeads + h;
    // the first batch of partial latents goes out with round 1 as well (it does not depend on
    // the statistics): thread (class sg, piece k4) takes splits sg, sg + NSG, ...
    const float *part = a.ws + lay.part + ((size_t)b * S * kAbs2dHeads + h) * RV;
    constexpr int PB = 8;                          // partial loads in flight per thread
    const int k4 = tid % NK4, sg = tid / NK4;
    const bool pact = tid < NSG * NK4;
    float4 pv[PB];
#pragma unroll
    for (int j = 0; j < PB; ++j) {
        const int s = sg + NSG * j;
        pv[j] = (pact && s < S) ? *reinterpret_cast<const float4 *>(
                                      part + (size_t)s * kAbs2dHeads * RV + 4 * k4)
                                : float4{0.f, 0.f, 0.f, 0.f};
    }
    float2 sv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int s = 4 * tid + j;
        sv[j] = s < S ? st[(size_t)s * kAbs2dHeads] : float2{-INFINITY, 0.f};
    }
    float M = fmaxf(fmaxf(sv[0].x, sv[1].x), fmaxf(sv[2].x, sv[3].x));
    for (int s = 4 * 256 + tid; s < S; s += 256) M = fmaxf(M, st[(size_t)s * kAbs2dHeads].x);
    M = wave_max(M);
    if (lane == 0) sRed[tid >> 6] = M;
    __syncthreads();
    M = fmaxf(fmaxf(sRed[0], sRed[1]), fmaxf(sRed[2], sRed[3]));
    float Ls = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int s = 4 * tid + j;
        if (s < S) {
            const float wgt = M != -INFINITY ? exp2_(sv[j].x - M) : 0.f;
            sW[s] = wgt;
            Ls += sv[j].y * wgt;
        }
    }
    for (int s = 4 * 256 + tid; s < S; s += 256) {
        const float2 x = st[(size_t)s * kAbs2dHeads];
        const float wgt = M != -INFINITY ? exp2_(x.x - M) : 0.f;
        sW[s] = wgt;
        Ls += x.y * wgt;
    }
    Ls = wave_sum(Ls);
    __syncthreads();                               // sRed's maxima are read; sW is complete
    if (lane == 0) sRed[4 + (tid >> 6)] = Ls;
    __syncthreads();
    if (tid == 0) {
        sML[0] = M;
        sML[1] = (sRed[4] + sRed[5]) + (sRed[6] + sRed[7]);
    }
    // ---- round 2: the partial latents, weighted and summed per split class
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    if (pact) {
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const float wgt = sg + NSG * j < S ? sW[sg + NSG * j] : 0.f;
            acc.x += pv[j].x * wgt;
            acc.y += pv[j].y * wgt;
            acc.z += pv[j].z * wgt;
            acc.w += pv[j].w * wgt;
        }
        for (int s0 = sg + NSG * PB; s0 < S; s0 += NSG * PB) {
#pragma unroll
            for (int j = 0; j < PB; ++j) {
                const int s = s0 + NSG * j;
                pv[j] = s < S ? *reinterpret_cast<const float4 *>(
                                    part + (size_t)s * kAbs2dHeads * RV + 4 * k4)
                              : float4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int j = 0; j < PB; ++j) {
                const float wgt = s0 + NSG * j < S ? sW[s0 + NSG * j] : 0.f;
                acc.x += pv[j].x * wgt;
                acc.y += pv[j].y * wgt;
                acc.z += pv[j].z * wgt;
                acc.w += pv[j].w * wgt;
            }
        }
    }
    __syncthreads();                               // every thread is done with sRed's scalars
    if (pact) *reinterpret_cast<float4 *>(sRed + sg * RV + 4 * k4) = acc;
    __syncthreads();
    if (tid < RV) {
        float c = 0.f;
#pragma unroll
        for (int g = 0; g < NSG; ++g) c += sRed[g * RV + tid];
        sC[tid] = c;
    }
    __syncthreads();
    // ---- expansion O = c~ W_up,t^V (this head's columns)
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
    for (int i = 0; i < WROWS; ++i) {
        const int k = kg + NKG * i;
        const float c = k < RV ? sC[k] : 0.f;
        const uint32_t wv[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o[2 * e] += c * __uint_as_float(wv[e] << 16);
            o[2 * e + 1] += c * __uint_as_float(wv[e] & 0xffff0000u);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sRed[kg * D + 8 * pc + e] = o[e];
    __syncthreads();
    if (tid >= D) return;
    float O = 0.f;
#pragma unroll 8
    for (int g = 0; g < NKG; ++g) O += sRed[g * D + tid];
    const float Mx = sML[0], Lsum = sML[1];
    const float s_self = a.ws[lay.self + (size_t)b * kAbs2dHeads + h];
    const bool self_here = a.k_self != nullptr;
    const float Mf = fmaxf(Mx, s_self);
    float res = 0.f;
    if (Mf != -INFINITY) {
        const float e = Mx != -INFINITY ? exp2_(Mx - Mf) : 0.f;
        const float w_self = self_here ? exp2_(s_self - Mf) : 0.f;
        const float v_self = self_here ? bf2f(static_cast<const uint16_t *>(a.v_self)[
                                             (size_t)b * a.self_stride + (size_t)h * D + tid])
                                       : 0.f;
        const float mu = bf2f(static_cast<const uint16_t *>(a.mu_v)[(size_t)a.t * a.Dg +
                                                                   (size_t)h * D + tid]);
        res = ((O + Lsum * mu) * e + w_self * v_self) / (Lsum * e + w_self);
    }
    static_cast<uint16_t *>(a.out)[((size_t)b * a.H + h) * D + tid] = f2bf(res);
}

template <int D, int RK, int RV>
hipError_t launch_t(const DecodeArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((absorb_q_kernel<D, RK>), dim3(a.B * kAbs2dHeads), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((absorbed2d_kernel<RK, RV, ABS2D_DEPTH, ABS2D_OCC>), dim3(a.B * a.S),
                       dim3(64 * kWaves), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((absorbed2d_combine_kernel<D, RV>), dim3(a.B * a.H), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t st) {
#define LLA_CASE(RK, RV) \
    if (a.r_k == RK && a.r_v == RV) return launch_t<D, RK, RV>(a, st);
    LLA_CASE(32, 32)
    LLA_CASE(32, 64)
    LLA_CASE(64, 64)
    LLA_CASE(64, 128)
    LLA_CASE(96, 160)
#undef LLA_CASE
    return hipErrorInvalidValue;
}

}  // namespace

bool absorbed2d_supported(int mode, int H, int d, int r_k, int r_v) {
    return mode == 1 && H >= 1 && H <= kAbs2dHeads && (d == 64 || d == 128) && r_k % 32 == 0 &&
           r_v % 16 == 0 && decode_bf16_supported(d, r_k, r_v);
}

hipError_t launch_decode_absorbed2d(const DecodeArgs &a, hipStream_t st) {
    const int d = a.Dg / a.H;
    if (a.S < 1 || a.S > kMaxAbs2dSplits) return hipErrorInvalidValue;
    if (d == 128) return launch_d<128>(a, st);
    if (d == 64) return launch_d<64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace lla
