// bwd_la64.hip -- the backward of the plain second-order numerator as
// masked first-order maps, on the one-launch kernel of fwd_la64.hip.
//
// With L = sum_t <out_t, dout_t> and out_t = q_t^T (S_t C_t - G_t), the
// gradients are (Higher-order Linear Attention, paperlayer.ai summary sec. 4:
// the reverse-mode scan; the identity below is pinned against the oracle's
// autograd gradients on the CPU, tests/test_backward_algebra.py):
//   u_j = S_j q_j                 = LA (Q, K, K; g)
//   w_j = sum_{t>=j} g^(2(t-j)) q_t (dout_t . v_j)
//                                 = LA^rev (V, dO, Q; g^2)
//   dq  = LA (dO, V, U; g^2) + LA (W, K, K; g)
//   dk  = LA^rev (K, Q, W; g) + LA^rev (K, W, Q; g)
//   dv  = LA^rev (U, Q, dO; g^2)
// where LA (A, B, C; r)_t = sum_{s<=t} r^(t-s) (a_t . b_s) c_s and LA^rev the
// same over s >= t with r^(s-t).  dO, U and W are fp32; they enter the maps
// as bf16 pairs (hi = bf16(x), lo = bf16(x - hi)): dO split as it is staged,
// U and W written as pairs by the maps that form them.  U and the second part
// of dq share their keys, values and decay, so they are one launch with two
// sets of queries, and the two maps of dk are one launch whose carry is
// symmetric.  After W, the maps fall into two pairs that do not depend on
// each other, each pair one grid: three launches in all.
//
// With an initial state (S, C, m, G, h at position -1) and a gradient dF
// flowing into the final state, the same maps carry the states' terms.  With
// X' = S^T C - G and Y' = S^T m - h (the read-out of token t is (S_t q_t)^T
// C_t, every entry of S its own variable), p = n - 1 - t, and the final
// state's gradient folded into
//   D_S = dS_F + C_n dG_F^T + m_n dh_F^T,  D_C = dC_F + S_n dG_F,
//   D_m = dm_F + S_n dh_F,                 dX' = -dG_F,  dY' = -dh_F,
// the maps take carries at position -1 of their own direction:
//   U  = LA (Q, K, K; g)  from S_init               (final carry: S_n)
//   W  = LA^rev (V, dO, Q; g^2) from g^-2 dX'^T, plus g^(2p) dY'
//                                                   (final carry M_W)
//   dq = LA (W, K, K; g) from S_init^T + LA (dO, V, U; g^2) from X'_init^T
//        + g^p (D_C v_t + D_m)
//   dk = LA^rev (K, Q, W; g) + LA^rev (K, W, Q; g) from g^-1 D_S, whose
//        carry is symmetric                         (final carry M_K)
//   dv = LA^rev (U, Q, dO; g^2) from g^-2 dX' + g^p D_C^T q_t
// and the initial state's gradient is
//   dX'_0 = g^2 M_W^T,  dY'_0 = g^(2n) dY',  dS = g M_K + C dX'_0^T + m dY'_0^T,
//   dC = g^n D_C + S dX'_0,  dm = g^n D_m + S dY'_0,  dG = -dX'_0,  dh = -dY'_0
// (pinned against the oracle on the CPU, tests/test_backward_algebra.py).
// C_n comes from a map with keys Q and values V that forms no output, only
// its final carry, and m_n from a reduction of the decayed queries.
//
// Workspace: the first kCtrlBytes are the one-launch kernels' control block,
// then the flags of two maps, their aggregates, the pairs of U and W, and
// per head the states' matrices.  The call clears the control block and the
// flags itself (a fill kernel), so the backward workspace needs no
// initialisation, as for the chunked path.
#include "bf16_split.h"
#include "device_common.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kBw = 64;  // d = dv = chunk
constexpr int kMSplits = 8;  // token ranges of the decayed query sums
constexpr int kMat = kBw * kBw;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}


size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct BwdLaLayout {
    size_t flags, agg, uh, ul, wh, wl, state, total;
};

// the states' per-head matrices ([BH][64][64] fp32) and vectors ([BH][64])
struct ShardBufs {
    float *sinT, *xinT, *wc, *kc, *vc, *dc, *dcT, *sfin, *cfin, *mw, *mk;
    float *wb, *dm, *mpart;  // mpart: [BH][kMSplits][64]
};
constexpr int kShardMats = 11, kShardVecs = 2 + kMSplits;

ShardBufs shard_bufs(char *base, int BH) {
    float *f = reinterpret_cast<float *>(base);
    const size_t M = static_cast<size_t>(BH) * kMat, V = static_cast<size_t>(BH) * kBw;
    ShardBufs b{};
    float **mats[kShardMats] = {&b.sinT, &b.xinT, &b.wc, &b.kc, &b.vc, &b.dc, &b.dcT, &b.sfin, &b.cfin, &b.mw, &b.mk};
    for (int i = 0; i < kShardMats; ++i) *mats[i] = f + i * M;
    f += kShardMats * M;
    b.wb = f; b.dm = f + V; b.mpart = f + 2 * V;
    return b;
}

struct ShardArgs {
    int H, n;
    GammaTab gam;
    hla_state init;   // init.S null: the zero state
    hla_state dfin;   // dfin.S null: no gradient into the final state
    ShardBufs b;
};

__device__ __forceinline__ float bf16_word(const u32x4 &w, int e) {  // element e of 8 packed bf16
    const uint32_t x = w[e >> 1];
    return __uint_as_float((e & 1) ? (x & 0xFFFF0000u) : (x << 16));
}

// partial sum over token range sp of g^(n-1-t) q_t (for m_n): thread (rows
// tid/8 + 32i, columns 8 (tid % 8) ..), its loads issued together
__device__ __forceinline__ void msum_block(const uint16_t *q, int n, int H, GammaTab gam, float *mpart, int bh, int sp,
                                           float (*red)[kBw + 1]) {
    const int cg = threadIdx.x & 7, tr = threadIdx.x >> 3;
    const float lg = log2f(head_gamma(gam, bh % H));
    const int per = (n + kMSplits - 1) / kMSplits, t0 = sp * per, t1 = min(n, t0 + per);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int tb = t0; tb < t1; tb += 256) {
        u32x4 raw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = tb + tr + 32 * i;
            raw[i] = t < t1 ? *reinterpret_cast<const u32x4 *>(q + (static_cast<size_t>(bh) * n + t) * kBw + 8 * cg)
                            : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = tb + tr + 32 * i;
            const float w = t < t1 ? exp2f(static_cast<float>(n - 1 - t) * lg) : 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, bf16_word(raw[i], e), acc[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tr][8 * cg + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < kBw) {
        float sum = 0.0f;
        for (int i = 0; i < 32; ++i) sum += red[i][threadIdx.x];
        mpart[(static_cast<size_t>(bh) * kMSplits + sp) * kBw + threadIdx.x] = sum;
    }
}

// One launch clears the control block and the maps' flags (blocks from
// nsum on, a grid-stride fill) and, when the final state has a gradient,
// forms the query sums (the first nsum = BH kMSplits blocks, head-major):
// the two touch disjoint words and both finish before the first map.
__global__ __launch_bounds__(256) void k_clear_msum(uint32_t *p, size_t words, const uint16_t *q, int n, int H,
                                                    GammaTab gam, float *mpart, int nsum) {
    __shared__ float red[32][kBw + 1];
    const int b = blockIdx.x;
    if (b < nsum) {
        msum_block(q, n, H, gam, mpart, b / kMSplits, b % kMSplits, red);
        return;
    }
    const size_t stride = static_cast<size_t>(gridDim.x - nsum) * 256;
    for (size_t i = static_cast<size_t>(b - nsum) * 256 + threadIdx.x; i < words; i += stride) p[i] = 0u;
}

typedef float Lmat[kBw][kBw];  // a 64 x 64 matrix in LDS

// Thread tid of 256 owns the 4 x 4 block at rows r0 = 4 (tid / 16), columns
// c0 = 4 (tid % 16) of every 64 x 64 matrix it stages or forms.
struct Blk {
    int r0, c0;
};
__device__ __forceinline__ Blk blk_of(int tid) { return Blk{4 * (tid >> 4), 4 * (tid & 15)}; }

typedef f32x4 B4[4];  // a 4 x 4 block, by rows

__device__ __forceinline__ void ld_blk(const float *m, Blk b, B4 &x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = *reinterpret_cast<const f32x4 *>(m + (b.r0 + i) * kBw + b.c0);
}

__device__ __forceinline__ void st_blk(float *m, Blk b, const B4 &x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4 *>(m + (b.r0 + i) * kBw + b.c0) = x[i];
}

// the block of A^T B over LDS matrices: o[i][e] = sum_l A[l][r0 + i] B[l][c0 + e]
__device__ __forceinline__ void atb(const Lmat &A, const Lmat &B, Blk b, B4 &o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int l = 0; l < kBw; ++l) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(&A[l][b.r0]);
        const f32x4 x = *reinterpret_cast<const f32x4 *>(&B[l][b.c0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] += a[i] * x;
    }
}

// a block read from LDS, transposed or not
__device__ __forceinline__ void lds_blk(const Lmat &L, Blk b, bool transpose, B4 &x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (transpose) {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[i][e] = L[b.c0 + e][b.r0 + i];
        } else {
            x[i] = *reinterpret_cast<const f32x4 *>(&L[b.r0 + i][b.c0]);
        }
    }
}

// put a block into LDS, as it is or transposed
__device__ __forceinline__ void put_blk(Lmat &L, Blk b, const B4 &x, bool transpose) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (transpose) {
#pragma unroll
            for (int e = 0; e < 4; ++e) L[b.c0 + e][b.r0 + i] = x[i][e];
        } else {
            *reinterpret_cast<f32x4 *>(&L[b.r0 + i][b.c0]) = x[i];
        }
    }
}

constexpr int kPrepJobs = 3, kFinishJobs = 2;

// Per head (blockIdx.x) and job (blockIdx.y), the maps' carries and bias
// and the final state's folded terms (see the header); every load of a job
// is issued before its first use.
//   job 0: S_0^T (dq's first map), X'_0^T (its second), X'_0 = S_0^T C_0 - G_0
//   job 1: g^-1 D_S (dk), D_S = dS_F + C_n dG_F^T + m_n dh_F^T
//   job 2: D_C, D_C^T, D_m, W's and dv's carries -g^-2 dG_F^T, -g^-2 dG_F, W's bias -g^-2 dh_F
// Jobs 1 and 2 need S_n (sfin), C_n (cfin) and the query partials.
__global__ __launch_bounds__(256) void k_shard_prep(ShardArgs a) {
    __shared__ Lmat L[3];
    __shared__ float mnv[kBw], dhv[kBw];
    const int bh = blockIdx.x, job = blockIdx.y, tid = threadIdx.x;
    const Blk b = blk_of(tid);
    const float g = head_gamma(a.gam, bh % a.H), lg = log2f(g);
    const float ig2 = 1.0f / (g * g);
    const bool ini = a.init.S != nullptr, fin = a.dfin.S != nullptr;
    const size_t mo = static_cast<size_t>(bh) * kMat, vo = static_cast<size_t>(bh) * kBw;
    B4 x, y, z, d;
    if (job == 0) {
        if (!ini) return;
        ld_blk(a.init.S + mo, b, x);
        ld_blk(a.init.C + mo, b, y);
        ld_blk(a.init.G + mo, b, z);
        put_blk(L[0], b, x, false);  // S_0
        put_blk(L[1], b, y, false);  // C_0
        put_blk(L[2], b, z, true);   // G_0^T
        __syncthreads();
        lds_blk(L[0], b, true, x);
        st_blk(a.b.sinT + mo, b, x);
        atb(L[1], L[0], b, y);  // (C_0^T S_0)[r][c] = X'_0[c][r] + G_0[c][r]
        lds_blk(L[2], b, false, z);
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] -= z[i];
        st_blk(a.b.xinT + mo, b, y);
        return;
    }
    if (!fin) return;
    if (job == 1) {
        ld_blk(a.b.cfin + mo, b, x);
        ld_blk(a.dfin.G + mo, b, y);
        ld_blk(a.dfin.S + mo, b, d);
        if (tid < kBw) {  // m_n and dh_F
            float part[kMSplits];
#pragma unroll
            for (int sp = 0; sp < kMSplits; ++sp) part[sp] = a.b.mpart[vo * kMSplits + sp * kBw + tid];
            const float m0 = ini ? a.init.m[vo + tid] : 0.0f, dh = a.dfin.h[vo + tid];
            float mn = exp2f(static_cast<float>(a.n) * lg) * m0;
#pragma unroll
            for (int sp = 0; sp < kMSplits; ++sp) mn += part[sp];
            mnv[tid] = mn;
            dhv[tid] = dh;
        }
        put_blk(L[0], b, x, true);  // C_n^T
        put_blk(L[1], b, y, true);  // dG_F^T
        __syncthreads();
        atb(L[0], L[1], b, z);  // (C_n dG_F^T)[r][c]
        const f32x4 dh4 = *reinterpret_cast<const f32x4 *>(&dhv[b.c0]);
        const float ig = 1.0f / g;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = ig * (d[i] + z[i] + mnv[b.r0 + i] * dh4);
        st_blk(a.b.kc + mo, b, x);
        return;
    }
    ld_blk(a.b.sfin + mo, b, x);
    ld_blk(a.dfin.G + mo, b, y);
    ld_blk(a.dfin.C + mo, b, d);
    if (tid < kBw) dhv[tid] = a.dfin.h[vo + tid];
    put_blk(L[0], b, x, true);   // S_n^T
    put_blk(L[1], b, y, false);  // dG_F
    put_blk(L[2], b, d, false);  // dC_F
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] *= -ig2;
    st_blk(a.b.vc + mo, b, y);   // dv's carry: -g^-2 dG_F
    __syncthreads();
    atb(L[0], L[1], b, z);  // (S_n dG_F)[r][c]
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = d[i] + z[i];
    st_blk(a.b.dc + mo, b, x);   // D_C
    atb(L[1], L[0], b, z);  // (dG_F^T S_n^T)[r][c] = (S_n dG_F)[c][r]
    lds_blk(L[2], b, true, d);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = d[i] + z[i];
    st_blk(a.b.dcT + mo, b, x);  // D_C^T
    lds_blk(L[1], b, true, x);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] *= -ig2;
    st_blk(a.b.wc + mo, b, x);   // W's carry: -g^-2 dG_F^T
    if (tid < kBw) {
        float sh = 0.0f;
        for (int b2 = 0; b2 < kBw; ++b2) sh = fmaf(L[0][b2][tid], dhv[b2], sh);
        a.b.dm[vo + tid] = a.dfin.m[vo + tid] + sh;  // D_m
        a.b.wb[vo + tid] = -ig2 * dhv[tid];         // W's bias
    }
}

// dq_t += g^p (D_C v_t + D_m) and dv_t += g^p D_C^T q_t, p = n - 1 - t: per
// 64-token block, wave w forms features 16w.. on the MFMA as (M x^T)^T, so
// that a lane holds four consecutive features of one token (v and q are
// exact bf16, D_C enters as a bf16 pair).
__device__ __forceinline__ void corr_block(const uint16_t *q, const uint16_t *v, int n, int H, GammaTab gam,
                                           const float *dc, const float *dcT, const float *dm, float *dq, float *dv,
                                           int bh, int tb0) {
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int r = l & 15, g4 = l >> 4, c0 = 16 * wave;
    const float lg = log2f(head_gamma(gam, bh % H));
    const size_t mo = static_cast<size_t>(bh) * kMat, head = static_cast<size_t>(bh) * n;
    const u32x4 z4 = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int prod = 0; prod < 2; ++prod) {
        const uint16_t *x = prod == 0 ? v : q;  // out[t][c] = sum_k M[c][k] x_t[k]
        const float *M = prod == 0 ? dc : dcT;
        float *out = prod == 0 ? dq : dv;
        bf16x8 mh[2], ml[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {  // A operand: lane (g4, r) holds M[c0 + r][32 ks + 8 g4 ..]
            const float *row = M + mo + (c0 + r) * kBw + 32 * ks + 8 * g4;
            pair_operand(*reinterpret_cast<const f32x4 *>(row), *reinterpret_cast<const f32x4 *>(row + 4), mh[ks], ml[ks]);
        }
        const f32x4 add = prod == 0 ? *reinterpret_cast<const f32x4 *>(dm + static_cast<size_t>(bh) * kBw + c0 + 4 * g4)
                                    : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int t = tb0 + 16 * tb + r;  // this lane's token (B operand column and output row)
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const u32x4 raw = t < n ? *reinterpret_cast<const u32x4 *>(x + (head + t) * kBw + 32 * ks + 8 * g4) : z4;
                const bf16x8 xb = __builtin_bit_cast(bf16x8, raw);
                acc = mfma(mh[ks], xb, acc);
                acc = mfma(ml[ks], xb, acc);
            }
            if (t < n) {  // acc[e] = out[t][c0 + 4 g4 + e]
                f32x4 *o = reinterpret_cast<f32x4 *>(out + (head + t) * kBw + c0 + 4 * g4);
                *o += exp2f(static_cast<float>(n - 1 - t) * lg) * (acc + add);
            }
        }
    }
}

// The initial state's gradient (see the header) from M_W, M_K and the folded
// terms, per head and job:
//   job 0: dS = g M_K + g^2 C_0 M_W + m_0 dY'_0^T
//   job 1: dC = g^n D_C + g^2 S_0 M_W^T, dG = -g^2 M_W^T, dm = g^n D_m + S_0 dY'_0, dh = -dY'_0
__device__ __forceinline__ void finish_block(const ShardArgs &a, const hla_state &dinit, int bh, int job, Lmat *L,
                                             float *dyv) {
    const int tid = threadIdx.x;
    const Blk b = blk_of(tid);
    const float g = head_gamma(a.gam, bh % a.H), lg = log2f(g);
    const float g2 = g * g, gn = exp2f(static_cast<float>(a.n) * lg), g2n = gn * gn;
    const bool ini = a.init.S != nullptr, fin = a.dfin.S != nullptr;
    const size_t mo = static_cast<size_t>(bh) * kMat, vo = static_cast<size_t>(bh) * kBw;
    B4 x, y, w, m = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f},
                     f32x4{0.f, 0.f, 0.f, 0.f}};
    if (tid < kBw) dyv[tid] = fin ? -g2n * a.dfin.h[vo + tid] : 0.0f;  // dY'_0
    ld_blk(a.b.mw + mo, b, w);
    if (job == 0) {
        ld_blk(a.b.mk + mo, b, m);
        if (ini) {
            ld_blk(a.init.C + mo, b, x);
            put_blk(L[0], b, x, true);   // C_0^T
            put_blk(L[1], b, w, false);  // M_W
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = g * m[i];
        if (ini) {
            atb(L[0], L[1], b, y);
            const f32x4 dy4 = *reinterpret_cast<const f32x4 *>(&dyv[b.c0]);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] += g2 * y[i] + a.init.m[vo + b.r0 + i] * dy4;
        }
        st_blk(dinit.S + mo, b, x);
        return;
    }
    if (fin) ld_blk(a.b.dc + mo, b, m);
    if (ini) {
        ld_blk(a.init.S + mo, b, x);
        put_blk(L[0], b, x, true);  // S_0^T
    }
    put_blk(L[1], b, w, true);  // M_W^T
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = gn * m[i];  // zero without dF
    if (ini) {
        atb(L[0], L[1], b, y);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] += g2 * y[i];
    }
    st_blk(dinit.C + mo, b, x);
    lds_blk(L[1], b, false, x);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] *= -g2;
    st_blk(dinit.G + mo, b, x);
    if (tid < kBw) {
        float dmv = fin ? gn * a.b.dm[vo + tid] : 0.0f;
        if (ini && fin)
            for (int b2 = 0; b2 < kBw; ++b2) dmv = fmaf(L[0][b2][tid], dyv[b2], dmv);
        dinit.m[vo + tid] = dmv;
        dinit.h[vo + tid] = -dyv[tid];
        if (dinit.rho != nullptr && tid == 0) dinit.rho[bh] = 0.0f;
    }
}

__global__ __launch_bounds__(256) void k_shard_corr(const uint16_t *q, const uint16_t *v, int n, int H, GammaTab gam,
                                                    const float *dc, const float *dcT, const float *dm, float *dq,
                                                    float *dv) {
    corr_block(q, v, n, H, gam, dc, dcT, dm, dq, dv, blockIdx.x, blockIdx.y * kBw);
}

// Per head (blockIdx.x) and job (blockIdx.y).  A launch of its own: sharing a
// grid with the corrections above (its LDS and registers imposed on every
// block) made the pair 2.4 times slower than the two launches.
__global__ __launch_bounds__(256) void k_shard_finish(ShardArgs a, hla_state dinit) {
    __shared__ Lmat L[2];
    __shared__ float dyv[kBw];
    finish_block(a, dinit, blockIdx.x, blockIdx.y, L, dyv);
}

BwdLaLayout bwd_la_layout(int BH, int n) {
    const size_t pair = static_cast<size_t>(BH) * n * kBw * sizeof(uint16_t);
    BwdLaLayout L{};
    L.flags = kCtrlBytes;  // two maps' flags, then their aggregates
    L.agg = L.flags + 2 * la64_flag_bytes(BH, n);
    L.uh = align256(L.agg + 2 * la64_agg_bytes(BH, n));
    L.ul = align256(L.uh + pair);
    L.wh = align256(L.ul + pair);
    L.wl = align256(L.wh + pair);
    L.state = align256(L.wl + pair);
    L.total = L.state + (static_cast<size_t>(kShardMats) * kMat + static_cast<size_t>(kShardVecs) * kBw) *
                            static_cast<size_t>(BH) * sizeof(float);
    return L;
}

}  // namespace

bool la_backward_eligible(const BwdProblem &p) {
    const FwdProblem &f = p.f;
    if (!(f.dtype == HLA_BF16 && f.d == kBw && f.dv == kBw && f.w == kBw && f.n > 0 && f.ridge == 0.0f &&
          !f.normalize))
        return false;
    // the states' matrices are read and written 16 bytes at a time
    auto a16 = [](const hla_state &x) {
        auto al = [](const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; };
        return x.S == nullptr || (al(x.S) && al(x.C) && al(x.G));
    };
    if (!(a16(f.init) && a16(p.dfinal) && a16(p.dinit))) return false;
    const int nh = f.gam.per_head ? f.H : 1;
    for (int h = 0; h < nh; ++h)
        if (f.gam.g[h] < 0.75f) return false;
    return true;
}

size_t la_backward_workspace_bytes(int BH, int n) { return bwd_la_layout(BH, n).total; }

size_t backward_workspace_bytes(int BH, int n, int d, int dv, int w) {
    const size_t gen = generic_backward_workspace_bytes(BH, n, d, dv, w);
    if (!(d == kBw && dv == kBw && w == kBw && n > 0)) return gen;
    const size_t la = la_backward_workspace_bytes(BH, n);
    return gen > la ? gen : la;
}

hipError_t la_backward(const BwdProblem &p, hipStream_t st) {
    const FwdProblem &f = p.f;
    const int BH = f.B * f.H;
    const BwdLaLayout L = bwd_la_layout(BH, f.n);
    char *base = static_cast<char *>(f.ws);
    uint32_t *ctrl = reinterpret_cast<uint32_t *>(base);
    const size_t fb = la64_flag_bytes(BH, f.n), ab = la64_agg_bytes(BH, f.n);
    const LaSpace sa{reinterpret_cast<uint32_t *>(base + L.flags), reinterpret_cast<float *>(base + L.agg)};
    const LaSpace sb{reinterpret_cast<uint32_t *>(base + L.flags + fb), reinterpret_cast<float *>(base + L.agg + ab)};
    auto pair = [&](size_t off) { return reinterpret_cast<uint16_t *>(base + off); };
    uint16_t *uh = pair(L.uh), *ul = pair(L.ul), *wh = pair(L.wh), *wl = pair(L.wl);
    // the control block and both maps' flags start clear (every launch below
    // then leaves them valid for the next); with a final-state gradient the
    // same launch forms the decayed query sums
    const bool states = f.init.S != nullptr || p.dfinal.S != nullptr || p.dinit.S != nullptr;
    const bool ini = f.init.S != nullptr, fin = p.dfinal.S != nullptr, dini = p.dinit.S != nullptr;
    ShardArgs sh{};
    sh.H = f.H; sh.n = f.n; sh.gam = f.gam;
    if (ini) sh.init = f.init;
    if (fin) sh.dfin = p.dfinal;
    sh.b = shard_bufs(base + L.state, BH);
    const uint16_t *q16 = static_cast<const uint16_t *>(f.q), *v16 = static_cast<const uint16_t *>(f.v);
    const size_t words = (kCtrlBytes + 2 * fb) / sizeof(uint32_t);
    const int nsum = fin ? BH * kMSplits : 0;
    const size_t zb = (words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024;
    hipLaunchKernelGGL(k_clear_msum, dim3(static_cast<unsigned>(nsum + zb)), dim3(256), 0, st, ctrl, words, q16, f.n,
                       f.H, f.gam, sh.b.mpart, nsum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    auto map = [&](bool rev, bool gsq) {
        LaProblem m{};
        m.B = f.B; m.H = f.H; m.n = f.n; m.gam = f.gam;
        m.rev = rev; m.gsq = gsq;
        return m;
    };
    if (!states) {
        // W = LA^rev (V, dO, Q; g^2), as a pair
        LaProblem w = map(true, true);
        w.q = f.v; w.kf = p.dout; w.v = f.q; w.mode = 2; w.oh = wh; w.ol = wl;
        if ((e = la64_forward_in(w, ctrl, sa, st)) != hipSuccess) return e;
        // U = LA (Q, K, K; g), as a pair, and dq = LA (W, K, K; g): two sets of queries;
        // with dk = LA^rev (K, Q, W; g) + LA^rev (K, W, Q; g), the symmetric carry
        LaProblem u = map(false, false), dk = map(true, false);
        u.q = f.q; u.k = f.k; u.v = f.k; u.mode = 2; u.oh = uh; u.ol = ul;
        u.q2 = wh; u.q2l = wl; u.mode2 = 0; u.out2 = p.dq;
        dk.q = f.k; dk.k = f.q; dk.v = wh; dk.vl = wl; dk.mode = 0; dk.sym = true; dk.out = p.dk;
        if ((e = la64_forward_pair(u, sa, dk, sb, ctrl, st)) != hipSuccess) return e;
        // dq += LA (dO, V, U; g^2), with dv = LA^rev (U, Q, dO; g^2)
        LaProblem dq = map(false, true), dv = map(true, true);
        dq.qf = p.dout; dq.k = f.v; dq.v = uh; dq.vl = ul; dq.mode = 1; dq.out = p.dq;
        dv.q = uh; dv.ql = ul; dv.k = f.q; dv.vf = p.dout; dv.mode = 0; dv.out = p.dv;
        return la64_forward_pair(dq, sa, dv, sb, ctrl, st);
    }

    // ---- with states (the header's second identity) ----
    // U from S_0 (its final carry S_n), and C_n from a map that forms no output
    LaProblem u = map(false, false);
    u.q = f.q; u.k = f.k; u.v = f.k; u.mode = 2; u.oh = uh; u.ol = ul;
    u.init = ini ? f.init.S : nullptr;
    if (fin) {
        u.fin = sh.b.sfin;
        LaProblem cn = map(false, false);
        cn.q = f.q; cn.k = f.q; cn.v = f.v; cn.mode = 3; cn.init = ini ? f.init.C : nullptr; cn.fin = sh.b.cfin;
        if ((e = la64_forward_pair(u, sa, cn, sb, ctrl, st)) != hipSuccess) return e;
    } else if ((e = la64_forward_in(u, ctrl, sa, st)) != hipSuccess) {
        return e;
    }
    if (ini || fin) {
        hipLaunchKernelGGL(k_shard_prep, dim3(static_cast<unsigned>(BH), kPrepJobs), dim3(256), 0, st, sh);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // W from g^-2 dX'^T with the bias g^(2p) dY' (its final carry M_W)
    LaProblem w = map(true, true);
    w.q = f.v; w.kf = p.dout; w.v = f.q; w.mode = 2; w.oh = wh; w.ol = wl;
    if (fin) { w.init = sh.b.wc; w.bias = sh.b.wb; }
    if (dini) w.fin = sh.b.mw;
    if ((e = la64_forward_in(w, ctrl, sa, st)) != hipSuccess) return e;
    // dq = LA (W, K, K; g) from S_0^T, with dk from g^-1 D_S (its final carry M_K)
    LaProblem dq1 = map(false, false), dk = map(true, false);
    dq1.q = wh; dq1.ql = wl; dq1.k = f.k; dq1.v = f.k; dq1.mode = 0; dq1.out = p.dq;
    if (ini) dq1.init = sh.b.sinT;
    dk.q = f.k; dk.k = f.q; dk.v = wh; dk.vl = wl; dk.mode = 0; dk.sym = true; dk.out = p.dk;
    if (fin) dk.init = sh.b.kc;
    if (dini) dk.fin = sh.b.mk;
    if ((e = la64_forward_pair(dq1, sa, dk, sb, ctrl, st)) != hipSuccess) return e;
    // dq += LA (dO, V, U; g^2) from X'_0^T, with dv from g^-2 dX'
    LaProblem dq = map(false, true), dv = map(true, true);
    dq.qf = p.dout; dq.k = f.v; dq.v = uh; dq.vl = ul; dq.mode = 1; dq.out = p.dq;
    if (ini) dq.init = sh.b.xinT;
    dv.q = uh; dv.ql = ul; dv.k = f.q; dv.vf = p.dout; dv.mode = 0; dv.out = p.dv;
    if (fin) dv.init = sh.b.vc;
    if ((e = la64_forward_pair(dq, sa, dv, sb, ctrl, st)) != hipSuccess) return e;
    if (fin) {  // the final state's C and m terms
        hipLaunchKernelGGL(k_shard_corr, dim3(static_cast<unsigned>(BH), static_cast<unsigned>((f.n + kBw - 1) / kBw)),
                           dim3(256), 0, st, q16, v16, f.n, f.H, f.gam, sh.b.dc, sh.b.dcT, sh.b.dm, p.dq, p.dv);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (dini) {
        hipLaunchKernelGGL(k_shard_finish, dim3(static_cast<unsigned>(BH), kFinishJobs), dim3(256), 0, st, sh, p.dinit);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace hla
