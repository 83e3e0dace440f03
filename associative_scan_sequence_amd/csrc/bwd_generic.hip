// bwd_generic.hip -- chunked backward of the masked second-order HLA forward:
// gradients of sum_t <out_t, dout_t> with respect to q, k and v, for any
// d, dv, w in {16, 32, 64, 128} and fp32 or bf16 inputs, fp32 throughout.
//
// Higher-order Linear Attention, paperlayer.ai summary sec. 4 and 5 (the scan
// trains chunk-parallel; outputs and summaries are linear in the prefix
// states).  Written with the value rows widened by a constant 1 (V^ = [V | 1])
// and the upstream gradient of token t as g^_t = [dnum_t | dden_t] (dout and 0
// for the plain output; dout/den and -(dout . out)/den for the ratio), num and
// den are one linear map of V^ and the gradient is itself a masked
// second-order scan, run from the last token to the first:
//
//   u_j  = S_j q_j                                     (forward, kept per chunk)
//   Gb_j = sum_{t>=j} g^(2(t-j)) q_t g^_t^T            Cb_j: the same with g^(t-j)
//   (the Cb slots hold lambda Cb, plus the seed of a final-state gradient)
//   w_j  = Gb_j v^_j        T_i = sum_{j>=i} g^(j-i) (w_j q_j^T + q_j w_j^T)
//   dq_t = X^_t g^_t + S_t w_t + lambda (C^_t g^_t + Cb_t v^_t)
//   dk_i = T_i k_i          dv_j = Gb_j^T u_j + lambda Cb_j^T q_j   (first dv columns)
//
// Per chunk of L tokens (local t, s; e_t = g^(t+1), eh_t = g^(L-t); carries
// from the left (S0, X0, y0, C0, m0) of the forward, from the right Gb', Cb', T'):
//   Gam = Gn V^T + gd 1^T (masked s <= t)
//   W   = (Gam o D_{g^2})^T Q + diag(eh^2)(V Gbn'^T + 1 gbd'^T)
//   dQ  = diag(e^2)(Gn X0^T + gd y0^T) + (Gam o D_{g^2}) U + diag(e) W S0
//         + ((W K^T) o D_g o L) K + lambda [diag(e)(Gn C0^T + gd m0^T)
//         + (Gam o D_g) Q + (Gam o D_g)^T Q + diag(eh)(V Cbn'^T + 1 cbd'^T)]
//   dK  = ((K Q^T) o Mu) W + ((K W^T) o Mu) Q + diag(eh) K T'   (Mu = (D_g o L)^T)
//   dV  = P^T Gn + diag(eh^2) U Gbn' + lambda diag(eh) Q Cbn'     (P: the forward's matrix)
//   right carries: Gb <- Q^T diag(g^(2t)) G^ + g^(2L) Gb', Cb with g^t, g^L;
//                  T  <- W^T diag(g^t) Q + Q^T diag(g^t) W + g^L T'
//
// Kernels (one workgroup of 256 threads per chunk unless stated):
//   generic forward  left carries, U, out and den (into this call's workspace)
//   k_bwd_prep       per token: Gn, gd of the ratio
//   k_bwd_sums       Q^T diag(g^(2t)) G^ (and the ridge's g^t sums) -> right slot c
//   k_rprefix        per head, elementwise: slot c = g^(pL_c) slot c+1 + slot c
//   k_bwd_w          W (kept) and the exact T increment -> T slot c
//   k_bwd_dq, k_bwd_dk, k_bwd_dv
#include "device_common.h"
#include "hla_internal.h"
#include "tile_fp32.h"

namespace hla {
namespace {

constexpr int kThreads = tile::kThreads;
constexpr int kMaxW = tile::kMaxW;
using tile::gram;
using tile::max3;
using tile::mm;
using tile::Stage;
using tile::store_tile;

struct BwdArgs {
    int H, n, d, dv, w, nc;
    float ridge;
    int normalize;
    const void *q, *k, *v;
    const float *dout;
    float *gq, *gk, *gv;  // dq, dk, dv
    const float *S, *C, *m, *X, *y, *U;  // forward slots [BH][nc+1][..], U [BH][nc][w][d]
    const float *out, *den;              // forward output and denominator
    const float *Gn;                     // dnum rows: dout, or dout / den with the ratio
    float *Gw, *gd;                      // ratio only: Gn storage, and dden (else gd = null)
    float *RG, *rg, *RC, *rc, *T;        // right slots [BH][nc+1][..]; slot c = state at chunk c's start
    float *W;                            // [BH][nc][w][d]
    GammaTab gam;
    hla_state ini;                       // initial state (ini.S null: zero state)
    hla_state dini;                      // its gradient (dini.S null: not formed)
    hla_state dfin;                      // gradient flowing into the final state (dfin.S null: none)
    int cbar;                            // the C-bar slots are live (ridge, or dfin given)
};

__device__ __forceinline__ size_t slot(const BwdArgs &a, int bh, int c) {
    return static_cast<size_t>(bh) * (a.nc + 1) + c;
}

// g^k for k = 0..2w in LDS (each entry rounded once from powf)
__device__ __forceinline__ void pow_table(float *gt, float g, int w) {
    for (int k = threadIdx.x; k <= 2 * w; k += kThreads) gt[k] = gpow(g, k);
    __syncthreads();
}

// ---- ratio: Gn = dout / den, gd = -(dout . out) / den, one thread per token
template <int DV>
__global__ __launch_bounds__(kThreads) void k_bwd_prep(BwdArgs a, size_t tokens) {
    const size_t t = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (t >= tokens) return;
    const float inv = 1.0f / a.den[t];
    const float *g = a.dout + t * DV, *o = a.out + t * DV;
    float *gn = a.Gw + t * DV;
    float dot = 0.0f;
    for (int j = 0; j < DV; ++j) {
        dot += g[j] * o[j];
        gn[j] = g[j] * inv;
    }
    a.gd[t] = -dot * inv;
}

// ---- right-slot increments of chunk c: Q^T diag(g^(2t)) [Gn | gd], and with the
// ridge Q^T diag(g^t) [Gn | gd]; the last chunk also clears slot nc of every
// right-slot array
template <typename T, int D, int DV>
__global__ __launch_bounds__(kThreads) void k_bwd_sums(BwdArgs a) {
    constexpr int MR = D / 16, MC = DV / 16;
    __shared__ float gt[2 * kMaxW + 1];
    __shared__ Stage<max3(D, DV, 16)> st;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int s0 = c * a.w, L = min(a.w, a.n - s0);
    const float g = head_gamma(a.gam, bh % a.H);
    const size_t tok = static_cast<size_t>(bh) * a.n + s0;
    const T *q = static_cast<const T *>(a.q) + tok * D;
    const float *gn = a.Gn + tok * DV;
    const float *gd = a.gd ? a.gd + tok : nullptr;
    const bool cbar = a.cbar != 0;
    const float lam = a.ridge;
    const int tid = threadIdx.x;
    pow_table(gt, g, a.w);
    auto qe = [&](int t, int l) { return Elem<T>::get(q, static_cast<size_t>(t) * D + l); };
    auto gne = [&](int t, int col) { return gn[static_cast<size_t>(t) * DV + col]; };
    const size_t sl = slot(a, bh, c);
    {
        float aG[MR][MC] = {};
        mm<MR, MC, true>(aG, D, L, st, [&](int r, int t) { return gt[2 * t] * qe(t, r); }, gne);
        store_tile<MR, MC>(a.RG + sl * D * DV, D, DV, aG);
    }
    if (cbar) {  // lambda is folded into the C-bar increments
        float aC[MR][MC] = {};
        mm<MR, MC, true>(aC, D, L, st, [&](int r, int t) { return lam * gt[t] * qe(t, r); }, gne);
        store_tile<MR, MC>(a.RC + sl * D * DV, D, DV, aC);
    }
    tile::row_sums(D, gd ? L : 0, [&](int r, int t) { return gt[2 * t] * qe(t, r) * gd[t]; },
                   [&](int r, float x) { a.rg[sl * D + r] = x; });
    if (cbar)
        tile::row_sums(D, gd ? L : 0, [&](int r, int t) { return lam * gt[t] * qe(t, r) * gd[t]; },
                       [&](int r, float x) { a.rc[sl * D + r] = x; });
    if (c == a.nc - 1) {  // slot nc: nothing to the right of the last token
        const size_t se = slot(a, bh, a.nc);
        for (int i = tid; i < D * DV; i += kThreads) {
            a.RG[se * D * DV + i] = 0.0f;
            if (cbar) a.RC[se * D * DV + i] = 0.0f;
        }
        for (int i = tid; i < D * D; i += kThreads) a.T[se * D * D + i] = 0.0f;
        if (tid < D) {
            a.rg[se * D + tid] = 0.0f;
            if (cbar) a.rc[se * D + tid] = 0.0f;
        }
    }
}

// Right-to-left decayed prefix over the slots, elementwise:
// slot c = g^(power L_c) slot c+1 + slot c, for c = nc-1 .. 0.
struct RScan {
    float *base;
    int E;
};

__global__ __launch_bounds__(kThreads) void k_rprefix(BwdArgs a, RScan s0, RScan s1, int power) {
    const int bh = blockIdx.y;
    int e = blockIdx.x * kThreads + threadIdx.x;
    RScan sg = s0;
    if (e >= s0.E) {
        e -= s0.E;
        sg = s1;
        if (e >= s1.E) return;
    }
    const float g = head_gamma(a.gam, bh % a.H);
    const int Llast = a.n - (a.nc - 1) * a.w;
    const float rf = gpow(g, power * a.w), rl = gpow(g, power * Llast);
    float *p = sg.base + static_cast<size_t>(bh) * (a.nc + 1) * sg.E + e;
    float run = p[static_cast<size_t>(a.nc) * sg.E];
    // eight slot loads in flight per step (the scan itself is serial)
    int c = a.nc - 1;
    for (; c >= 7; c -= 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = p[static_cast<size_t>(c - u) * sg.E];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            run = (c - u == a.nc - 1 ? rl : rf) * run + x[u];
            p[static_cast<size_t>(c - u) * sg.E] = run;
        }
    }
    for (; c >= 0; --c) {
        float *sl = p + static_cast<size_t>(c) * sg.E;
        run = (c == a.nc - 1 ? rl : rf) * run + *sl;
        *sl = run;
    }
}

// ---- W = (Gam o D_{g^2})^T Q + diag(eh^2)(V Gbn'^T + 1 gbd'^T), kept; T increment
template <typename T, int D, int DV, int RT>
__global__ __launch_bounds__(kThreads) void k_bwd_w(BwdArgs a) {
    constexpr int MA = D / 16, BW = 16 * RT;
    constexpr int BUF = BW * kMaxW > D * D ? BW * kMaxW : D * D;
    __shared__ float buf[BUF];  // Gam2 (stride BW), then W rows (stride D), then A (D x D)
    __shared__ float gt[2 * kMaxW + 1];
    __shared__ Stage<max3(BW, D, DV)> st;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int s0 = c * a.w, L = min(a.w, a.n - s0);
    const float g = head_gamma(a.gam, bh % a.H);
    const size_t tok = static_cast<size_t>(bh) * a.n + s0;
    const T *q = static_cast<const T *>(a.q) + tok * D;
    const T *v = static_cast<const T *>(a.v) + tok * DV;
    const float *gn = a.Gn + tok * DV;
    const float *gd = a.gd ? a.gd + tok : nullptr;
    const size_t sr = slot(a, bh, c + 1);
    const float *RGn = a.RG + sr * D * DV, *rgd = a.rg + sr * D;
    const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    pow_table(gt, g, a.w);
    auto qe = [&](int t, int l) { return Elem<T>::get(q, static_cast<size_t>(t) * D + l); };
    auto ve = [&](int t, int l) { return Elem<T>::get(v, static_cast<size_t>(t) * DV + l); };
    // Gam2[t][s] = g^(2(t-s)) (gn_t . v_s + gd_t), s <= t
    gram<RT, DV>(buf, BW, L, st, [&](int t, int l) { return gn[static_cast<size_t>(t) * DV + l]; }, ve,
                 [&](int t, int s, float x) { return s <= t ? gt[2 * (t - s)] * (x + (gd ? gd[t] : 0.0f)) : 0.0f; });
    __syncthreads();
    // W[s][:] = sum_{t >= s} Gam2[t][s] q_t + eh_s^2 (Gbn' v_s + gbd')
    float wacc[RT][MA] = {};
    mm<RT, MA, true>(wacc, L, L, st, [&](int s, int t) { return buf[t * BW + s]; }, qe);
    mm<RT, MA, false>(wacc, L, DV, st, [&](int s, int l) { return gt[2 * (L - s)] * ve(s, l); },
                      [&](int l, int col) { return RGn[col * DV + l]; });
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int s = RT * ty + i;
        if (s >= L) continue;
#pragma unroll
        for (int j = 0; j < MA; ++j) wacc[i][j] += gt[2 * (L - s)] * rgd[MA * tx + j];
    }
    float *Wg = a.W + (static_cast<size_t>(bh) * a.nc + c) * a.w * D;
    store_tile<RT, MA>(Wg, L, D, wacc);
    store_tile<RT, MA>(buf, L, D, wacc);  // W rows, stride D (Gam2 reads ended in mm)
    __syncthreads();
    // T increment: A + A^T with A = sum_t g^t w_t q_t^T (d x d), so it is exactly symmetric
    float tacc[MA][MA] = {};
    mm<MA, MA, true>(tacc, D, L, st, [&](int r, int t) { return gt[t] * buf[t * D + r]; }, qe);
    store_tile<MA, MA>(buf, D, D, tacc);  // the W reads ended inside mm
    __syncthreads();
    {
        const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
        float *Tc = a.T + slot(a, bh, c) * D * D;
#pragma unroll
        for (int i = 0; i < MA; ++i)
#pragma unroll
            for (int j = 0; j < MA; ++j) {
                const int r = MA * ty + i, col = MA * tx + j;
                Tc[r * D + col] = tacc[i][j] + buf[col * D + r];
            }
    }
}

// ---- dQ
template <typename T, int D, int DV, int RT>
__global__ __launch_bounds__(kThreads) void k_bwd_dq(BwdArgs a) {
    constexpr int MA = D / 16, BW = 16 * RT;
    __shared__ float buf[BW * BW];
    __shared__ float gt[2 * kMaxW + 1];
    __shared__ Stage<max3(BW, D, DV)> st;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int s0 = c * a.w, L = min(a.w, a.n - s0);
    const float g = head_gamma(a.gam, bh % a.H);
    const float lam = a.ridge;
    const size_t tok = static_cast<size_t>(bh) * a.n + s0;
    const T *q = static_cast<const T *>(a.q) + tok * D;
    const T *k = static_cast<const T *>(a.k) + tok * D;
    const T *v = static_cast<const T *>(a.v) + tok * DV;
    const float *gn = a.Gn + tok * DV;
    const float *gd = a.gd ? a.gd + tok : nullptr;
    const float *U = a.U + (static_cast<size_t>(bh) * a.nc + c) * a.w * D;
    const float *Wc = a.W + (static_cast<size_t>(bh) * a.nc + c) * a.w * D;
    const size_t sl = slot(a, bh, c), sr = slot(a, bh, c + 1);
    const float *S0 = a.S + sl * D * D, *X0 = a.X + sl * D * DV, *y0 = a.y + sl * D;
    const float *C0 = a.C + sl * D * DV, *m0 = a.m + sl * D;
    const float *RCn = a.RC + sr * D * DV, *rcd = a.rc + sr * D;
    const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    pow_table(gt, g, a.w);
    auto qe = [&](int t, int l) { return Elem<T>::get(q, static_cast<size_t>(t) * D + l); };
    auto ke = [&](int t, int l) { return Elem<T>::get(k, static_cast<size_t>(t) * D + l); };
    auto ve = [&](int t, int l) { return Elem<T>::get(v, static_cast<size_t>(t) * DV + l); };
    auto gne = [&](int t, int l) { return gn[static_cast<size_t>(t) * DV + l]; };
    // Gam[t][s] = gn_t . v_s + gd_t for s <= t (no decay)
    gram<RT, DV>(buf, BW, L, st, gne, ve,
                 [&](int t, int s, float x) { return s <= t ? x + (gd ? gd[t] : 0.0f) : 0.0f; });
    __syncthreads();
    float acc[RT][MA] = {};
    // (Gam o D_{g^2}) U
    mm<RT, MA, false>(acc, L, L, st, [&](int t, int s) { return s <= t ? gt[2 * (t - s)] * buf[t * BW + s] : 0.0f; },
                      [&](int s, int col) { return U[s * D + col]; });
    if (lam != 0.0f) {  // lambda ((Gam o D_g) + (Gam o D_g)^T) Q
        mm<RT, MA, false>(acc, L, L, st,
                          [&](int t, int s) {
                              float x = s <= t ? gt[t - s] * buf[t * BW + s] : 0.0f;
                              if (s >= t) x += gt[s - t] * buf[s * BW + t];
                              return lam * x;
                          },
                          qe);
    }
    __syncthreads();  // Gam reads done
    // ((W K^T) o D_g o L) K
    gram<RT, D>(buf, BW, L, st, [&](int t, int l) { return Wc[t * D + l]; }, ke,
                [&](int t, int s, float x) { return s <= t ? gt[t - s] * x : 0.0f; });
    __syncthreads();
    mm<RT, MA, false>(acc, L, L, st, [&](int t, int s) { return buf[t * BW + s]; }, ke);
    // carries: e^2 (Gn X0^T + gd y0^T) + e W S0 + lambda [e (Gn C0^T + gd m0^T) + eh (V Cbn'^T + cbd')]
    mm<RT, MA, false>(acc, L, DV, st, [&](int t, int l) { return gt[2 * (t + 1)] * gne(t, l); },
                      [&](int l, int col) { return X0[col * DV + l]; });
    mm<RT, MA, false>(acc, L, D, st, [&](int t, int b) { return gt[t + 1] * Wc[t * D + b]; },
                      [&](int b, int col) { return S0[b * D + col]; });
    if (lam != 0.0f)
        mm<RT, MA, false>(acc, L, DV, st, [&](int t, int l) { return lam * gt[t + 1] * gne(t, l); },
                          [&](int l, int col) { return C0[col * DV + l]; });
    if (a.cbar)  // the C-bar slots already carry lambda
        mm<RT, MA, false>(acc, L, DV, st, [&](int t, int l) { return gt[L - t] * ve(t, l); },
                          [&](int l, int col) { return RCn[col * DV + l]; });
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int t = RT * ty + i;
        if (t >= L) continue;
        const float e = gt[t + 1], eh = gt[L - t], gdt = gd ? gd[t] : 0.0f;
#pragma unroll
        for (int j = 0; j < MA; ++j) {
            const int col = MA * tx + j;
            float x = e * e * gdt * y0[col];
            if (lam != 0.0f) x += lam * e * gdt * m0[col];
            if (a.cbar) x += eh * rcd[col];
            acc[i][j] += x;
        }
    }
    store_tile<RT, MA>(a.gq + tok * D, L, D, acc);
}

// ---- dK = ((K Q^T) o Mu) W + ((K W^T) o Mu) Q + diag(eh) K T'
template <typename T, int D, int DV, int RT>
__global__ __launch_bounds__(kThreads) void k_bwd_dk(BwdArgs a) {
    constexpr int MA = D / 16, BW = 16 * RT;
    __shared__ float buf[BW * BW];
    __shared__ float gt[2 * kMaxW + 1];
    __shared__ Stage<max3(BW, D, DV)> st;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int s0 = c * a.w, L = min(a.w, a.n - s0);
    const float g = head_gamma(a.gam, bh % a.H);
    const size_t tok = static_cast<size_t>(bh) * a.n + s0;
    const T *q = static_cast<const T *>(a.q) + tok * D;
    const T *k = static_cast<const T *>(a.k) + tok * D;
    const float *Wc = a.W + (static_cast<size_t>(bh) * a.nc + c) * a.w * D;
    const float *Tr = a.T + slot(a, bh, c + 1) * D * D;
    pow_table(gt, g, a.w);
    auto ke = [&](int t, int l) { return Elem<T>::get(k, static_cast<size_t>(t) * D + l); };
    auto qe = [&](int t, int l) { return Elem<T>::get(q, static_cast<size_t>(t) * D + l); };
    auto we = [&](int t, int l) { return Wc[t * D + l]; };
    auto upper = [&](int t, int s, float x) { return s >= t ? gt[s - t] * x : 0.0f; };
    float acc[RT][MA] = {};
    gram<RT, D>(buf, BW, L, st, ke, qe, upper);
    __syncthreads();
    mm<RT, MA, false>(acc, L, L, st, [&](int t, int s) { return buf[t * BW + s]; }, we);
    __syncthreads();
    gram<RT, D>(buf, BW, L, st, ke, we, upper);
    __syncthreads();
    mm<RT, MA, false>(acc, L, L, st, [&](int t, int s) { return buf[t * BW + s]; }, qe);
    mm<RT, MA, false>(acc, L, D, st, [&](int t, int b) { return gt[L - t] * ke(t, b); },
                      [&](int b, int col) { return Tr[b * D + col]; });
    store_tile<RT, MA>(a.gk + tok * D, L, D, acc);
}

// ---- dV = P^T Gn + diag(eh^2) U Gbn' + lambda diag(eh) Q Cbn'
template <typename T, int D, int DV, int RT>
__global__ __launch_bounds__(kThreads) void k_bwd_dv(BwdArgs a) {
    constexpr int MC = DV / 16, BW = 16 * RT;
    __shared__ float buf[BW * BW];
    __shared__ float gt[2 * kMaxW + 1];
    __shared__ Stage<max3(BW, D, DV)> st;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int s0 = c * a.w, L = min(a.w, a.n - s0);
    const float g = head_gamma(a.gam, bh % a.H);
    const float lam = a.ridge;
    const size_t tok = static_cast<size_t>(bh) * a.n + s0;
    const T *q = static_cast<const T *>(a.q) + tok * D;
    const float *gn = a.Gn + tok * DV;
    const float *U = a.U + (static_cast<size_t>(bh) * a.nc + c) * a.w * D;
    const size_t sr = slot(a, bh, c + 1);
    const float *RGn = a.RG + sr * D * DV, *RCn = a.RC + sr * D * DV;
    pow_table(gt, g, a.w);
    auto qe = [&](int t, int l) { return Elem<T>::get(q, static_cast<size_t>(t) * D + l); };
    // P[t][s] = g^(2(t-s)) (q_t . u_s) + lambda g^(t-s) (q_t . q_s), s <= t
    gram<RT, D>(buf, BW, L, st, qe, [&](int s, int l) { return U[s * D + l]; },
                [&](int t, int s, float x) { return s <= t ? gt[2 * (t - s)] * x : 0.0f; });
    __syncthreads();
    if (lam != 0.0f) {  // add the ridge part (each entry is read and written by its owner)
        gram<RT, D>(buf, BW, L, st, qe, qe,
                    [&](int t, int s, float x) { return s <= t ? buf[t * BW + s] + lam * gt[t - s] * x : 0.0f; });
        __syncthreads();
    }
    float acc[RT][MC] = {};
    mm<RT, MC, true>(acc, L, L, st, [&](int s, int t) { return buf[t * BW + s]; },
                     [&](int t, int col) { return gn[static_cast<size_t>(t) * DV + col]; });
    mm<RT, MC, false>(acc, L, D, st, [&](int s, int l) { return gt[2 * (L - s)] * U[s * D + l]; },
                      [&](int l, int col) { return RGn[l * DV + col]; });
    if (a.cbar)
        mm<RT, MC, false>(acc, L, D, st, [&](int s, int l) { return gt[L - s] * qe(s, l); },
                          [&](int l, int col) { return RCn[l * DV + col]; });
    store_tile<RT, MC>(a.gv + tok * DV, L, DV, acc);
}

// D[r][b] = dS_f[r][b] + sum_c C_n[r][c] dG_f[b][c] + m_n[r] dh_f[b]: the gradient
// reaching the final key moment S_n, directly and through G_n = S_n^T C_n - X_n
// (with C and G widened by their m and h columns).
template <int D, int DV>
__device__ __forceinline__ float fin_moment(const BwdArgs &a, int bh, int r, int b) {
    const size_t sn = slot(a, bh, a.nc), so = static_cast<size_t>(bh);
    const float *Cn = a.C + (sn * D + r) * DV, *dG = a.dfin.G + (so * D + b) * DV;
    float x = a.dfin.S[(so * D + r) * D + b] + a.m[sn * D + r] * a.dfin.h[so * D + b];
    for (int c = 0; c < DV; ++c) x += Cn[c] * dG[c];
    return x;
}

// ---- seeds of the right slots at position n from a gradient flowing into the
// final state, one workgroup per row r of every head (after k_bwd_sums has
// cleared slot nc, before the reverse prefixes).  The final state reaches the
// loss through X_n (G_n = S_n^T C_n - X_n), S_n and C_n, each a right carry
// read one token past the last one, hence the g^-1 and g^-2:
//   Gb slot nc   = -g^-2 dG_f          (widened by -g^-2 dh_f)
//   T slot nc    = g^-1 (D + D^T)      (D above)
//   Cb slot nc   = g^-1 (dC_f + S_n dG_f)   (widened by dm_f + S_n dh_f)
template <int D, int DV>
__global__ __launch_bounds__(kThreads) void k_bwd_seed(BwdArgs a) {
    const int r = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    const float g = head_gamma(a.gam, bh % a.H), gi = 1.0f / g, gi2 = gi * gi;
    const size_t sn = slot(a, bh, a.nc), so = static_cast<size_t>(bh);
    for (int b = tid; b < D; b += kThreads)
        a.T[(sn * D + r) * D + b] = gi * (fin_moment<D, DV>(a, bh, r, b) + fin_moment<D, DV>(a, bh, b, r));
    const float *Sr = a.S + (sn * D + r) * D;
    for (int c = tid; c <= DV; c += kThreads) {  // column DV: the m / h column
        const float *dgc = c < DV ? a.dfin.G + so * D * DV + c : a.dfin.h + so * D;
        const int ld = c < DV ? DV : 1;
        float y = c < DV ? a.dfin.C[(so * D + r) * DV + c] : a.dfin.m[so * D + r];
        for (int b = 0; b < D; ++b) y += Sr[b] * dgc[static_cast<size_t>(b) * ld];
        const float gs = -gi2 * dgc[static_cast<size_t>(r) * ld];
        if (c < DV) {
            a.RG[(sn * D + r) * DV + c] = gs;
            a.RC[(sn * D + r) * DV + c] = gi * y;
        } else {
            a.rg[sn * D + r] = gs;
            a.rc[sn * D + r] = gi * y;
        }
    }
}

// ---- per-chunk parts of sum_j g^(j+1) q_j w_j^T (the one-sided key-moment
// term of the initial-state gradient) into T slot c.  Runs after k_bwd_dk, the
// last reader of T; the last chunk clears slot nc, so an undecayed suffix sum
// over the slots leaves the total in slot 0.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_bwd_qw(BwdArgs a) {
    constexpr int MR = D / 16;
    __shared__ float gt[2 * kMaxW + 1];
    __shared__ Stage<max3(D, D, 16)> st;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int s0 = c * a.w, L = min(a.w, a.n - s0);
    const float g = head_gamma(a.gam, bh % a.H), base = gpow(g, s0);
    const size_t tok = static_cast<size_t>(bh) * a.n + s0;
    const T *q = static_cast<const T *>(a.q) + tok * D;
    const float *Wc = a.W + (static_cast<size_t>(bh) * a.nc + c) * a.w * D;
    pow_table(gt, g, a.w);
    float acc[MR][MR] = {};
    mm<MR, MR, true>(acc, D, L, st,
                     [&](int r, int t) { return base * gt[t + 1] * Elem<T>::get(q, static_cast<size_t>(t) * D + r); },
                     [&](int t, int b) { return Wc[t * D + b]; });
    store_tile<MR, MR>(a.T + slot(a, bh, c) * D * D, D, D, acc);
    if (c == a.nc - 1) {
        float *z = a.T + slot(a, bh, a.nc) * D * D;
        for (int i = threadIdx.x; i < D * D; i += kThreads) z[i] = 0.0f;
    }
}

// ---- gradient of the initial state (the state at position -1), one
// workgroup per row r of the d rows of every head (the token sum of dS is
// already in T slot 0).  With C' = [C | m] of the
// initial state (zero when none is given), Gb0' = [Gb_0 | gb_0] and
// Cb0' = [Cb_0 | cb_0] the right slots at token 0, and w_j the kept W rows:
//   dS[r][b]  = g^2 sum_c C'[r][c] Gb0'[b][c] + sum_j g^(j+1) q_j[r] w_j[b]
//   dC'[r][c] = g^2 (S Gb0')[r][c] + lambda g Cb0'[r][c]
//   (+ g^n D[r][b] in dS with a final-state gradient; its C' part arrives
//   through the seeded Cb slots, which also carry lambda)
//   dG'[r][c] = -g^2 Gb0'[r][c]              (G' = [G | h])
// The first two come from the read-out (S_t q_t)^T C_t of every token and the
// carry X = S C - G with X_{-1} scaled by g^(2(t+1)); S's entries count as
// independent variables.
template <typename T, int D, int DV>
__global__ __launch_bounds__(kThreads) void k_bwd_init(BwdArgs a, hla_state ini, hla_state dini) {
    const int r = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    const float g = head_gamma(a.gam, bh % a.H), g2 = g * g;
    const size_t s0 = slot(a, bh, 0);
    const float *Gb = a.RG + s0 * D * DV, *gb = a.rg + s0 * D;
    const bool cbar = a.cbar != 0;
    const size_t so = static_cast<size_t>(bh);
    if (tid < D) {
        const int b = tid;
        float x = a.T[(s0 * D + r) * D + b];  // sum_j g^(j+1) q_j w_j^T, from k_bwd_qw
        if (ini.S) {
            const float *Cr = ini.C + (so * D + r) * DV;
            float y = ini.m[so * D + r] * gb[b];
            for (int c = 0; c < DV; ++c) y += Cr[c] * Gb[static_cast<size_t>(b) * DV + c];
            x += g2 * y;
        }
        if (a.dfin.S) x += gpow(g, a.n) * fin_moment<D, DV>(a, bh, r, b);
        dini.S[(so * D + r) * D + b] = x;
    }
    for (int c = tid; c <= DV; c += kThreads) {  // column DV is the m / h column
        const float *gcol = c < DV ? Gb + c : gb;
        const int ld = c < DV ? DV : 1;
        float y = 0.0f;
        if (ini.S) {
            const float *Sr = ini.S + (so * D + r) * D;
            for (int b = 0; b < D; ++b) y += Sr[b] * gcol[static_cast<size_t>(b) * ld];
        }
        float x = g2 * y;
        if (cbar) x += g * (c < DV ? a.RC[(s0 * D + r) * DV + c] : a.rc[s0 * D + r]);
        const float gr = -g2 * gcol[static_cast<size_t>(r) * ld];
        if (c < DV) {
            dini.C[(so * D + r) * DV + c] = x;
            dini.G[(so * D + r) * DV + c] = gr;
        } else {
            dini.m[so * D + r] = x;
            dini.h[so * D + r] = gr;
        }
    }
    if (dini.rho && r == 0 && tid == 0) dini.rho[bh] = 0.0f;  // rho does not reach any output
}

__global__ __launch_bounds__(kThreads) void k_fill_zero(float *p, size_t count) {
    const size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i < count) p[i] = 0.0f;
}

template <typename T, int D, int DV>
hipError_t launch_bwd(const BwdArgs &a, int BH, hipStream_t st) {
    const dim3 blk(kThreads), grid(a.nc, BH);
    if (a.normalize) {
        const size_t tokens = static_cast<size_t>(BH) * a.n;
        hipLaunchKernelGGL((k_bwd_prep<DV>), dim3((tokens + kThreads - 1) / kThreads), blk, 0, st, a, tokens);
    }
    hipLaunchKernelGGL((k_bwd_sums<T, D, DV>), grid, blk, 0, st, a);
    if (a.dfin.S) hipLaunchKernelGGL((k_bwd_seed<D, DV>), dim3(D, BH), blk, 0, st, a);
    const RScan sG{a.RG, D * DV}, sg{a.rg, D}, sC{a.RC, D * DV}, sc{a.rc, D}, sT{a.T, D * D}, none{nullptr, 0};
    const int e1 = D * DV + D;
    hipLaunchKernelGGL(k_rprefix, dim3((e1 + kThreads - 1) / kThreads, BH), blk, 0, st, a, sG, sg, 2);
    if (a.cbar)
        hipLaunchKernelGGL(k_rprefix, dim3((e1 + kThreads - 1) / kThreads, BH), blk, 0, st, a, sC, sc, 1);
    // register tile: 4 x 4 per thread for chunks up to 64 tokens, 8 x 8 for 128
    if (a.w > 64) {
        hipLaunchKernelGGL((k_bwd_w<T, D, DV, 8>), grid, blk, 0, st, a);
    } else {
        hipLaunchKernelGGL((k_bwd_w<T, D, DV, 4>), grid, blk, 0, st, a);
    }
    hipLaunchKernelGGL(k_rprefix, dim3((D * D + kThreads - 1) / kThreads, BH), blk, 0, st, a, sT, none, 1);
    if (a.w > 64) {
        hipLaunchKernelGGL((k_bwd_dq<T, D, DV, 8>), grid, blk, 0, st, a);
        hipLaunchKernelGGL((k_bwd_dk<T, D, DV, 8>), grid, blk, 0, st, a);
        hipLaunchKernelGGL((k_bwd_dv<T, D, DV, 8>), grid, blk, 0, st, a);
    } else {
        hipLaunchKernelGGL((k_bwd_dq<T, D, DV, 4>), grid, blk, 0, st, a);
        hipLaunchKernelGGL((k_bwd_dk<T, D, DV, 4>), grid, blk, 0, st, a);
        hipLaunchKernelGGL((k_bwd_dv<T, D, DV, 4>), grid, blk, 0, st, a);
    }
    if (a.dini.S) {
        hipLaunchKernelGGL((k_bwd_qw<T, D>), grid, blk, 0, st, a);
        const RScan sQ{a.T, D * D};
        hipLaunchKernelGGL(k_rprefix, dim3((D * D + kThreads - 1) / kThreads, BH), blk, 0, st, a, sQ, none, 0);
        hipLaunchKernelGGL((k_bwd_init<T, D, DV>), dim3(D, BH), blk, 0, st, a, a.ini, a.dini);
    }
    return hipGetLastError();
}

template <typename T, int D>
hipError_t pick_dv(const BwdArgs &a, int BH, hipStream_t st) {
    switch (a.dv) {
        case 16: return launch_bwd<T, D, 16>(a, BH, st);
        case 32: return launch_bwd<T, D, 32>(a, BH, st);
        case 64: return launch_bwd<T, D, 64>(a, BH, st);
        case 128: return launch_bwd<T, D, 128>(a, BH, st);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t pick_d(const BwdArgs &a, int BH, hipStream_t st) {
    switch (a.d) {
        case 16: return pick_dv<T, 16>(a, BH, st);
        case 32: return pick_dv<T, 32>(a, BH, st);
        case 64: return pick_dv<T, 64>(a, BH, st);
        case 128: return pick_dv<T, 128>(a, BH, st);
    }
    return hipErrorInvalidValue;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct BwdLayout {
    size_t fwd, out, den, Gn, gd, RG, rg, RC, rc, T, W, total;
};

BwdLayout layout(int BH, int n, int d, int dv, int w) {
    const size_t nc = (static_cast<size_t>(n) + w - 1) / w;
    const size_t slots = static_cast<size_t>(BH) * (nc + 1), tok = static_cast<size_t>(BH) * n;
    BwdLayout L{};
    size_t off = 0;
    L.fwd = off; off = align256(off + generic_workspace_bytes(BH, n, d, dv, w));
    L.out = off; off = align256(off + tok * dv * sizeof(float));
    L.den = off; off = align256(off + tok * sizeof(float));
    L.Gn = off; off = align256(off + tok * dv * sizeof(float));
    L.gd = off; off = align256(off + tok * sizeof(float));
    L.RG = off; off = align256(off + slots * d * dv * sizeof(float));
    L.rg = off; off = align256(off + slots * d * sizeof(float));
    L.RC = off; off = align256(off + slots * d * dv * sizeof(float));
    L.rc = off; off = align256(off + slots * d * sizeof(float));
    L.T = off; off = align256(off + slots * d * d * sizeof(float));
    L.W = off; off = align256(off + static_cast<size_t>(BH) * nc * w * d * sizeof(float));
    L.total = off;
    return L;
}

}  // namespace

size_t generic_backward_workspace_bytes(int BH, int n, int d, int dv, int w) {
    return layout(BH, n, d, dv, w).total;
}

hipError_t generic_backward(const BwdProblem &p, hipStream_t st) {
    const FwdProblem &f = p.f;
    const int BH = f.B * f.H;
    if (f.nc == 0) return hipSuccess;
    const BwdLayout L = layout(BH, f.n, f.d, f.dv, f.w);
    char *base = static_cast<char *>(f.ws);
    // the forward: left carries, U, out and den
    FwdProblem fw = f;
    fw.ws = base + L.fwd;
    fw.ws_bytes = generic_workspace_bytes(BH, f.n, f.d, f.dv, f.w);
    fw.out = reinterpret_cast<float *>(base + L.out);
    fw.den = reinterpret_cast<float *>(base + L.den);
    fw.init = f.init;  // the left carries start from it (held constant)
    fw.fin = hla_state{};
    fw.carries_only = f.normalize ? 0 : 1;  // out and den only enter the ratio's gradient
    fw.own_prefix = 0;                      // the slots below are read as prefixes
    hipError_t e = generic_forward(fw, st);
    if (e != hipSuccess) return e;
    const GenericSlots sl = generic_slots(fw);
    BwdArgs a{};
    a.H = f.H; a.n = f.n; a.d = f.d; a.dv = f.dv; a.w = f.w; a.nc = f.nc;
    a.ridge = f.ridge; a.normalize = f.normalize;
    a.q = f.q; a.k = f.k; a.v = f.v;
    a.dout = p.dout; a.gq = p.dq; a.gk = p.dk; a.gv = p.dv;
    a.S = sl.S; a.C = sl.C; a.m = sl.m; a.X = sl.X; a.y = sl.y; a.U = sl.U;
    a.out = fw.out; a.den = fw.den;
    a.Gw = reinterpret_cast<float *>(base + L.Gn);
    a.gd = f.normalize ? reinterpret_cast<float *>(base + L.gd) : nullptr;
    a.Gn = f.normalize ? a.Gw : p.dout;
    a.RG = reinterpret_cast<float *>(base + L.RG);
    a.rg = reinterpret_cast<float *>(base + L.rg);
    a.RC = reinterpret_cast<float *>(base + L.RC);
    a.rc = reinterpret_cast<float *>(base + L.rc);
    a.T = reinterpret_cast<float *>(base + L.T);
    a.W = reinterpret_cast<float *>(base + L.W);
    a.gam = f.gam;
    a.ini = f.init;
    a.dini = p.dinit;
    a.dfin = p.dfinal;
    a.cbar = (f.ridge != 0.0f || p.dfinal.S) ? 1 : 0;
    if (f.dtype == HLA_BF16) return pick_d<uint16_t>(a, BH, st);
    return pick_d<float>(a, BH, st);
}

hipError_t zero_state_grad(const hla_state &s, int BH, int d, int dv, hipStream_t st) {
    const size_t N = static_cast<size_t>(BH);
    float *parts[6] = {s.S, s.C, s.m, s.G, s.h, s.rho};
    const size_t sizes[6] = {N * d * d, N * d * dv, N * d, N * d * dv, N * d, N};
    for (int i = 0; i < 6; ++i)
        if (parts[i] && sizes[i])
            hipLaunchKernelGGL(k_fill_zero, dim3((sizes[i] + kThreads - 1) / kThreads), dim3(kThreads), 0, st,
                               parts[i], sizes[i]);
    return hipGetLastError();
}

}  // namespace hla
