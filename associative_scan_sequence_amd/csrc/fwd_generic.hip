// fwd_generic.hip -- chunked masked second-order HLA forward for any
// supported width (d, dv, w in {16, 32, 64, 128}) and fp32 or bf16 inputs.
//
// Higher-order Linear Attention, paperlayer.ai summary sec. 4 and 5: token
// deltas feed an exclusive scan inside each chunk, every token forms its
// inclusive state and output, and chunk summaries are scanned with the same
// operator to give each chunk its carry-in.  The masked semidirect product
// (sec. 4.2) carries the cross term S_later C_earlier; here it is carried in
// the equivalent corrected form X = S C - G, y = S m - h, for which the
// per-token update is X_t = g^2 X_{t-1} + S_t q_t v_t^T (it follows from the
// G, h updates).  Splitting the scan into a linear pass over (S, C, m) and a
// second linear pass over (X, y) removes every state-by-state product from
// the inter-chunk scan:
//
//   per chunk c (L tokens, local index t, s; carry (S0, C0, m0, X0, y0)):
//     e_t = g^(t+1), f_s = g^(L-1-s), rho = g^L
//     A = (Q K^T) o D_g o L          (D_g[t,s] = g^(t-s), L: s <= t)
//     U = diag(e) Q S0 + A K         row s = S_{s} q_s (inclusive S times q)
//     P = (Q U^T) o D_{g^2} o L + lambda (Q Q^T) o D_g o L
//     num = P V + diag(e^2) Q X0 + lambda diag(e) Q C0
//     den = P 1 + diag(e^2) Q y0 + lambda diag(e) Q m0
//   carry:  S0' = rho S0 + K^T diag(f) K,  C0' = rho C0 + Q^T diag(f) V,
//           m0' = rho m0 + Q^T f,  X0' = rho^2 X0 + U^T diag(f^2) V,
//           y0' = rho^2 y0 + U^T f^2
//
// Kernels (one workgroup of 256 threads per chunk unless stated):
//   k_init_slot   per head: slot 0 = init (X = S C - G); without init (and
//                 n > 0) the scans write slot 0's zeros themselves
//   k_chunk_sums  K^T diag(f) K, Q^T diag(f) V, Q^T f     -> slot c+1
//   k_prefix      per head, elementwise: slot c+1 = rho^p slot c + slot c+1
//                 (not launched for a forward call with at most 16 chunks at
//                 d, dv <= 32: the kernels below then sum the slots, prefix_of)
//   k_chunk_uz    A, U (kept for the output pass), U^T diag(f^2) V, U^T f^2
//   k_chunk_out   P, num, den, ratio
//   k_final       per head: final (S, C, m), G = S C - X, h = S m - y, rho
// Everything is fp32; bf16 inputs are widened exactly on load.
#include "device_common.h"
#include "hla_internal.h"
#include "tile_fp32.h"

namespace hla {
namespace {

constexpr int kThreads = tile::kThreads;
constexpr int kMaxW = tile::kMaxW;

struct Slots {
    float *S, *C, *m, *X, *y;  // [BH][nc+1][...]: slot c = state before chunk c
    float *U;                  // [BH][nc][w][d]
};

struct GenArgs {
    int H, n, d, dv, w, nc;
    float ridge;
    int normalize;
    int carries_only;
    int own_prefix;  // the prefix scans are not launched: consumers sum the slots (see prefix_of)
    const void *q, *k, *v;
    float *out, *den;
    hla_state init, fin;
    Slots ws;
    GammaTab gam;
};

__device__ __forceinline__ size_t slot_index(const GenArgs &a, int bh, int slot) {
    return static_cast<size_t>(bh) * (a.nc + 1) + slot;
}

// Few chunks, narrow heads: the two prefix scans cost a launch each, more
// than the sums themselves.  Then the slots keep the chunks' own increments
// and each consumer forms the prefix it needs, slot c = the state before
// chunk c, with the scan kernel's recurrence in the same order (the same
// bits): run = slot 0 (the initial state, or zero), then run = r run + slot
// j+1 for j < c, with r = g^(power w), g^(power L_last) for the last chunk.
constexpr int kOwnPrefixChunks = 16;

template <int E>
__device__ void prefix_of(const GenArgs &a, int bh, const float *slots, int c, int power, float *dst) {
    const float g = head_gamma(a.gam, bh % a.H);
    const int Llast = a.n - (a.nc - 1) * a.w;
    const float rf = gpow(g, power * a.w), rl = gpow(g, power * Llast);
    const float *p = slots + slot_index(a, bh, 0) * E;
    for (int e = threadIdx.x; e < E; e += kThreads) {
        float x[kOwnPrefixChunks];  // every slot's load in flight at once
#pragma unroll
        for (int j = 0; j < kOwnPrefixChunks; ++j) x[j] = j < c ? p[static_cast<size_t>(j + 1) * E + e] : 0.0f;
        float run = a.init.S != nullptr ? p[e] : 0.0f;
#pragma unroll
        for (int j = 0; j < kOwnPrefixChunks; ++j)
            if (j < c) run = (j == a.nc - 1 ? rl : rf) * run + x[j];
        dst[e] = run;
    }
}

// Out = S*C - In and outv = S*m - inv for one head; S [D][D], C/In/Out [D][DV].
template <int D, int DV, int SR>
__device__ void s_times_c_minus(const float *S, const float *C, const float *In, float *Out,
                                const float *m, const float *inv, float *outv, tile::Stage<SR> &st) {
    constexpr int MR = D / 16, MC = DV / 16;
    const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    float acc[MR][MC] = {};
    tile::mm<MR, MC, false>(acc, D, D, st, [&](int r, int l) { return S[r * D + l]; },
                            [&](int l, int col) { return C[l * DV + col]; });
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int j = 0; j < MC; ++j) {
            const int o = (MR * ty + i) * DV + MC * tx + j;
            Out[o] = acc[i][j] - In[o];
        }
    tile::row_sums(D, D, [&](int r, int l) { return S[r * D + l] * m[l]; },
                   [&](int r, float s) { outv[r] = s - inv[r]; });
}

template <int D, int DV>
__global__ __launch_bounds__(kThreads) void k_init_slot(GenArgs a) {
    __shared__ tile::Stage<tile::max3(D, DV, 16)> st;
    const int bh = blockIdx.x;
    const size_t sl = slot_index(a, bh, 0);
    float *S = a.ws.S + sl * D * D, *C = a.ws.C + sl * D * DV, *m = a.ws.m + sl * D;
    float *X = a.ws.X + sl * D * DV, *y = a.ws.y + sl * D;
    const int tid = threadIdx.x;
    if (a.init.S == nullptr) {
        for (int i = tid; i < D * D; i += kThreads) S[i] = 0.0f;
        for (int i = tid; i < D * DV; i += kThreads) C[i] = 0.0f, X[i] = 0.0f;
        if (tid < D) m[tid] = 0.0f, y[tid] = 0.0f;
        return;
    }
    const float *iS = a.init.S + static_cast<size_t>(bh) * D * D;
    const float *iC = a.init.C + static_cast<size_t>(bh) * D * DV;
    const float *iG = a.init.G + static_cast<size_t>(bh) * D * DV;
    const float *im = a.init.m + static_cast<size_t>(bh) * D;
    const float *ih = a.init.h + static_cast<size_t>(bh) * D;
    for (int i = tid; i < D * D; i += kThreads) S[i] = iS[i];
    for (int i = tid; i < D * DV; i += kThreads) C[i] = iC[i];
    if (tid < D) m[tid] = im[tid];
    s_times_c_minus<D, DV>(iS, iC, iG, X, im, ih, y, st);
}

// K^T diag(f) K, Q^T diag(f) V and Q^T f of chunk c -> slot c+1 (products from
// LDS, tile_fp32.h).  The key moment is formed from sqrt(f_s) k_s on both
// sides: fma(x_a, x_b, acc) is the same operation for (a, b) and (b, a), so
// the moment (and every prefix of it) is exactly symmetric.
template <typename T, int D, int DV>
__global__ __launch_bounds__(kThreads) void k_chunk_sums(GenArgs a) {
    constexpr int MR = D / 16, MC = DV / 16;
    __shared__ float fs[kMaxW], hs[kMaxW];  // f_s = g^(L-1-s) and sqrt(f_s)
    __shared__ tile::Stage<tile::max3(D, DV, 16)> st;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int s0 = c * a.w, L = min(a.w, a.n - s0);
    const float g = head_gamma(a.gam, bh % a.H);
    const size_t tok = static_cast<size_t>(bh) * a.n + s0;
    const T *q = static_cast<const T *>(a.q) + tok * D;
    const T *k = static_cast<const T *>(a.k) + tok * D;
    const T *v = static_cast<const T *>(a.v) + tok * DV;
    const int tid = threadIdx.x;
    for (int i = tid; i < L; i += kThreads) {
        fs[i] = gpow(g, L - 1 - i);
        hs[i] = sqrtf(fs[i]);
    }
    __syncthreads();
    auto qe = [&](int t, int l) { return Elem<T>::get(q, static_cast<size_t>(t) * D + l); };
    auto ke = [&](int t, int l) { return Elem<T>::get(k, static_cast<size_t>(t) * D + l); };
    auto ve = [&](int t, int l) { return Elem<T>::get(v, static_cast<size_t>(t) * DV + l); };
    const size_t sl = slot_index(a, bh, c + 1);
    {
        float aS[MR][MR] = {};
        tile::mm<MR, MR, true>(aS, D, L, st, [&](int r, int t) { return hs[t] * ke(t, r); },
                               [&](int t, int col) { return hs[t] * ke(t, col); });
        tile::store_tile<MR, MR>(a.ws.S + sl * D * D, D, D, aS);
    }
    float aC[MR][MC] = {};
    tile::mm<MR, MC, true>(aC, D, L, st, [&](int r, int t) { return fs[t] * qe(t, r); }, ve);
    tile::store_tile<MR, MC>(a.ws.C + sl * D * DV, D, DV, aC);
    tile::row_sums(D, L, [&](int r, int t) { return fs[t] * qe(t, r); },
                   [&](int r, float x) { a.ws.m[sl * D + r] = x; });
}

// Exclusive-to-inclusive decayed prefix over the chunk slots, elementwise:
// slot c+1 = rho_c^power * slot c + slot c+1.  Up to three arrays per launch
// (their element ranges are concatenated along blockIdx.x).
struct ScanSeg {
    float *base;
    int E;
};

__global__ __launch_bounds__(kThreads) void k_prefix(GenArgs a, ScanSeg s0, ScanSeg s1,
                                                     ScanSeg s2, int power) {
    const int bh = blockIdx.y;
    int e = blockIdx.x * kThreads + threadIdx.x;
    ScanSeg seg = s0;
    if (e >= s0.E) {
        e -= s0.E;
        seg = s1;
        if (e >= s1.E) {
            e -= s1.E;
            seg = s2;
            if (e >= s2.E) return;
        }
    }
    if (a.nc == 0) return;
    const float g = head_gamma(a.gam, bh % a.H);
    const int Llast = a.n - (a.nc - 1) * a.w;
    const float rf = gpow(g, power * a.w), rl = gpow(g, power * Llast);
    float *p = seg.base + static_cast<size_t>(bh) * (a.nc + 1) * seg.E + e;
    if (a.init.S == nullptr) p[0] = 0.0f;  // the zero state before chunk 0
    float run = p[0];
    // eight slot loads in flight per step (the scan itself is serial)
    int c = 0;
    for (; c + 8 <= a.nc; c += 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = p[static_cast<size_t>(c + 1 + u) * seg.E];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            run = (c + u == a.nc - 1 ? rl : rf) * run + x[u];
            p[static_cast<size_t>(c + 1 + u) * seg.E] = run;
        }
    }
    for (; c < a.nc; ++c) {
        const float r = (c == a.nc - 1) ? rl : rf;
        float *slot = p + static_cast<size_t>(c + 1) * seg.E;
        run = r * run + *slot;
        *slot = run;
    }
}

// A, U (kept for the output pass), Z = U^T diag(f^2) V and z = U^T f^2 of chunk c
// (products from LDS, tile_fp32.h; RT x RT register tiles, 16 RT >= w)
template <typename T, int D, int DV, int RT>
__global__ __launch_bounds__(kThreads) void k_chunk_uz(GenArgs a) {
    constexpr int MC = D / 16, MZ = DV / 16, BW = 16 * RT;
    __shared__ float buf[BW * kMaxW];  // A (L x L, stride BW), then U rows (stride D)
    __shared__ float gt[2 * kMaxW + 1];
    __shared__ tile::Stage<tile::max3(BW, D, DV)> st;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int s0 = c * a.w, L = min(a.w, a.n - s0);
    const float g = head_gamma(a.gam, bh % a.H);
    const size_t tok = static_cast<size_t>(bh) * a.n + s0;
    const T *q = static_cast<const T *>(a.q) + tok * D;
    const T *k = static_cast<const T *>(a.k) + tok * D;
    const T *v = static_cast<const T *>(a.v) + tok * DV;
    constexpr bool OWN = D <= 32 && DV <= 32;  // the only widths that may skip the prefix scans
    __shared__ float own_s[OWN ? D * D : 1];
    const float *S0 = a.ws.S + slot_index(a, bh, c) * D * D;
    const int tid = threadIdx.x;
    for (int i = tid; i <= 2 * a.w; i += kThreads) gt[i] = gpow(g, i);
    if constexpr (OWN) {
        if (a.own_prefix) {
            prefix_of<D * D>(a, bh, a.ws.S, c, 1, own_s);
            S0 = own_s;
        }
    }
    __syncthreads();
    auto qe = [&](int t, int l) { return Elem<T>::get(q, static_cast<size_t>(t) * D + l); };
    auto ke = [&](int t, int l) { return Elem<T>::get(k, static_cast<size_t>(t) * D + l); };
    auto ve = [&](int t, int l) { return Elem<T>::get(v, static_cast<size_t>(t) * DV + l); };
    // A[t][s] = g^(t-s) (q_t . k_s) for s <= t
    tile::gram<RT, D>(buf, BW, L, st, qe, ke, [&](int t, int s, float x) { return s <= t ? gt[t - s] * x : 0.0f; });
    __syncthreads();
    // U[t][:] = e_t (S0 q_t) + sum_{s<=t} A[t][s] k_s, e_t = g^(t+1)
    float u[RT][MC] = {};
    tile::mm<RT, MC, false>(u, L, D, st, [&](int t, int l) { return gt[t + 1] * qe(t, l); },
                            [&](int l, int col) { return S0[l * D + col]; });
    tile::mm<RT, MC, false>(u, L, L, st, [&](int t, int s) { return buf[t * BW + s]; }, ke);
    float *Ug = a.ws.U + (static_cast<size_t>(bh) * a.nc + c) * a.w * D;
    tile::store_tile<RT, MC>(Ug, L, D, u);
    tile::store_tile<RT, MC>(buf, L, D, u);  // the A reads ended inside mm
    __syncthreads();
    // Z = U^T diag(f^2) V, f_s^2 = g^(2(L-1-s)); z = U^T f^2
    float z[MC][MZ] = {};
    tile::mm<MC, MZ, true>(z, D, L, st, [&](int r, int s) { return gt[2 * (L - 1 - s)] * buf[s * D + r]; }, ve);
    const size_t sl = slot_index(a, bh, c + 1);
    tile::store_tile<MC, MZ>(a.ws.X + sl * D * DV, D, DV, z);
    tile::row_sums(D, L, [&](int r, int s) { return gt[2 * (L - 1 - s)] * buf[s * D + r]; },
                   [&](int r, float x) { a.ws.y[sl * D + r] = x; });
}

// P, num, den and the ratio of chunk c (products from LDS, tile_fp32.h)
template <typename T, int D, int DV, int RT>
__global__ __launch_bounds__(kThreads) void k_chunk_out(GenArgs a) {
    constexpr int MC = DV / 16, BW = 16 * RT, PS = BW + 1;  // odd stride: row walks hit distinct banks
    __shared__ float P[BW * PS];
    __shared__ float gt[2 * kMaxW + 1], dens[kMaxW];
    __shared__ tile::Stage<tile::max3(BW, D, DV)> st;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int s0 = c * a.w, L = min(a.w, a.n - s0);
    const float g = head_gamma(a.gam, bh % a.H);
    const float lam = a.ridge;
    const size_t tok = static_cast<size_t>(bh) * a.n + s0;
    const T *q = static_cast<const T *>(a.q) + tok * D;
    const T *v = static_cast<const T *>(a.v) + tok * DV;
    const float *U = a.ws.U + (static_cast<size_t>(bh) * a.nc + c) * a.w * D;
    const size_t sl = slot_index(a, bh, c);
    const float *X0 = a.ws.X + sl * D * DV, *C0 = a.ws.C + sl * D * DV;
    const float *y0 = a.ws.y + sl * D, *m0 = a.ws.m + sl * D;
    constexpr bool OWN = D <= 32 && DV <= 32;  // the only widths that may skip the prefix scans
    __shared__ float own_x[OWN ? D * DV : 1], own_c[OWN ? D * DV : 1], own_y[OWN ? D : 1], own_m[OWN ? D : 1];
    const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    for (int i = tid; i <= 2 * a.w; i += kThreads) gt[i] = gpow(g, i);
    if constexpr (OWN) {
        if (a.own_prefix) {
            prefix_of<D * DV>(a, bh, a.ws.X, c, 2, own_x);
            prefix_of<D * DV>(a, bh, a.ws.C, c, 1, own_c);
            prefix_of<D>(a, bh, a.ws.y, c, 2, own_y);
            prefix_of<D>(a, bh, a.ws.m, c, 1, own_m);
            X0 = own_x; C0 = own_c; y0 = own_y; m0 = own_m;
        }
    }
    __syncthreads();
    auto qe = [&](int t, int l) { return Elem<T>::get(q, static_cast<size_t>(t) * D + l); };
    auto ve = [&](int t, int l) { return Elem<T>::get(v, static_cast<size_t>(t) * DV + l); };
    // P[t][s] = g^(2(t-s)) (q_t . u_s) + lambda g^(t-s) (q_t . q_s), s <= t
    tile::gram<RT, D>(P, PS, L, st, qe, [&](int s, int l) { return U[s * D + l]; },
                      [&](int t, int s, float x) { return s <= t ? gt[2 * (t - s)] * x : 0.0f; });
    if (lam != 0.0f) {  // each entry is read and written by the thread that owns it
        __syncthreads();
        tile::gram<RT, D>(P, PS, L, st, qe, qe,
                          [&](int t, int s, float x) { return s <= t ? P[t * PS + s] + lam * gt[t - s] * x : 0.0f; });
    }
    __syncthreads();
    // den_t = sum_s P[t][s] + e_t^2 (q_t . y0) + lambda e_t (q_t . m0)
    tile::row_sums(L, L, [&](int t, int s) { return s <= t ? P[t * PS + s] : 0.0f; },
                   [&](int t, float ps) { dens[t] = ps; });
    // (each row's fin runs on the lane that wrote its dens entry above)
    tile::row_sums(L, D,
                   [&](int t, int l) {
                       const float e = gt[t + 1];
                       return qe(t, l) * (e * e * y0[l] + lam * e * m0[l]);
                   },
                   [&](int t, float x) {
                       const float dn = dens[t] + x;
                       dens[t] = dn;
                       if (a.den) a.den[tok + t] = dn;
                   });
    __syncthreads();
    // num = P V + diag(e^2) Q X0 + lambda diag(e) Q C0
    float acc[RT][MC] = {};
    tile::mm<RT, MC, false>(acc, L, L, st, [&](int t, int s) { return P[t * PS + s]; }, ve);
    tile::mm<RT, MC, false>(acc, L, D, st, [&](int t, int l) { return gt[2 * (t + 1)] * qe(t, l); },
                            [&](int l, int col) { return X0[l * DV + col]; });
    if (lam != 0.0f)
        tile::mm<RT, MC, false>(acc, L, D, st, [&](int t, int l) { return lam * gt[t + 1] * qe(t, l); },
                                [&](int l, int col) { return C0[l * DV + col]; });
    float *out = a.out + tok * DV;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int t = RT * ty + i;
        if (t >= L) continue;
        const float dn = dens[t];
#pragma unroll
        for (int j = 0; j < MC; ++j) {
            const float num = acc[i][j];
            out[static_cast<size_t>(t) * DV + MC * tx + j] = a.normalize ? num / dn : num;
        }
    }
}

template <int D, int DV>
__global__ __launch_bounds__(kThreads) void k_final(GenArgs a) {
    __shared__ tile::Stage<tile::max3(D, DV, 16)> st;
    const int bh = blockIdx.x;
    const size_t sl = slot_index(a, bh, a.nc);
    const float *S = a.ws.S + sl * D * D, *C = a.ws.C + sl * D * DV, *m = a.ws.m + sl * D;
    const float *X = a.ws.X + sl * D * DV, *y = a.ws.y + sl * D;
    constexpr bool OWN = D <= 32 && DV <= 32;  // the only widths that may skip the prefix scans
    __shared__ float own_s[OWN ? D * D : 1], own_c[OWN ? D * DV : 1], own_x[OWN ? D * DV : 1];
    __shared__ float own_m[OWN ? D : 1], own_y[OWN ? D : 1];
    if constexpr (OWN) {
        if (a.own_prefix) {
            prefix_of<D * D>(a, bh, a.ws.S, a.nc, 1, own_s);
            prefix_of<D * DV>(a, bh, a.ws.C, a.nc, 1, own_c);
            prefix_of<D>(a, bh, a.ws.m, a.nc, 1, own_m);
            prefix_of<D * DV>(a, bh, a.ws.X, a.nc, 2, own_x);
            prefix_of<D>(a, bh, a.ws.y, a.nc, 2, own_y);
            S = own_s; C = own_c; m = own_m; X = own_x; y = own_y;
            __syncthreads();
        }
    }
    float *fS = a.fin.S + static_cast<size_t>(bh) * D * D;
    float *fC = a.fin.C + static_cast<size_t>(bh) * D * DV;
    float *fm = a.fin.m + static_cast<size_t>(bh) * D;
    const int tid = threadIdx.x;
    for (int i = tid; i < D * D; i += kThreads) fS[i] = S[i];
    for (int i = tid; i < D * DV; i += kThreads) fC[i] = C[i];
    if (tid < D) fm[tid] = m[tid];
    s_times_c_minus<D, DV>(S, C, X, a.fin.G + static_cast<size_t>(bh) * D * DV, m, y,
                           a.fin.h + static_cast<size_t>(bh) * D, st);
    if (tid == 0 && a.fin.rho) {
        const float g = head_gamma(a.gam, bh % a.H);
        const float r0 = (a.init.S && a.init.rho) ? a.init.rho[bh] : 1.0f;
        a.fin.rho[bh] = r0 * gpow(g, a.n);
    }
}

template <typename T, int D, int DV>
hipError_t launch_all(GenArgs a, int BH, hipStream_t st) {
    const dim3 blk(kThreads);
    // a forward call (not the backward's recompute, which reads the prefix
    // slots afterwards) with few chunks and narrow heads skips the scans
    a.own_prefix = a.own_prefix && !a.carries_only && a.nc <= kOwnPrefixChunks && D <= 32 && DV <= 32;
    if (a.init.S != nullptr || a.nc == 0) hipLaunchKernelGGL((k_init_slot<D, DV>), dim3(BH), blk, 0, st, a);
    if (a.nc > 0) {
        hipLaunchKernelGGL((k_chunk_sums<T, D, DV>), dim3(a.nc, BH), blk, 0, st, a);
        const ScanSeg sS{a.ws.S, D * D}, sC{a.ws.C, D * DV}, sm{a.ws.m, D};
        const int e1 = D * D + D * DV + D;
        if (!a.own_prefix)
            hipLaunchKernelGGL(k_prefix, dim3((e1 + kThreads - 1) / kThreads, BH), blk, 0, st, a, sS, sC, sm, 1);
        if (a.w > 64)
            hipLaunchKernelGGL((k_chunk_uz<T, D, DV, 8>), dim3(a.nc, BH), blk, 0, st, a);
        else
            hipLaunchKernelGGL((k_chunk_uz<T, D, DV, 4>), dim3(a.nc, BH), blk, 0, st, a);
        const ScanSeg sX{a.ws.X, D * DV}, sy{a.ws.y, D}, none{nullptr, 0};
        const int e2 = D * DV + D;
        if (!a.own_prefix)
            hipLaunchKernelGGL(k_prefix, dim3((e2 + kThreads - 1) / kThreads, BH), blk, 0, st, a, sX, sy, none, 2);
        if (a.carries_only) return hipGetLastError();
        if (a.w > 64)
            hipLaunchKernelGGL((k_chunk_out<T, D, DV, 8>), dim3(a.nc, BH), blk, 0, st, a);
        else
            hipLaunchKernelGGL((k_chunk_out<T, D, DV, 4>), dim3(a.nc, BH), blk, 0, st, a);
    }
    if (a.fin.S) hipLaunchKernelGGL((k_final<D, DV>), dim3(BH), blk, 0, st, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t pick_dv(const GenArgs &a, int BH, hipStream_t st) {
    switch (a.dv) {
        case 16: return launch_all<T, D, 16>(a, BH, st);
        case 32: return launch_all<T, D, 32>(a, BH, st);
        case 64: return launch_all<T, D, 64>(a, BH, st);
        case 128: return launch_all<T, D, 128>(a, BH, st);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t pick_d(const GenArgs &a, int BH, hipStream_t st) {
    switch (a.d) {
        case 16: return pick_dv<T, 16>(a, BH, st);
        case 32: return pick_dv<T, 32>(a, BH, st);
        case 64: return pick_dv<T, 64>(a, BH, st);
        case 128: return pick_dv<T, 128>(a, BH, st);
    }
    return hipErrorInvalidValue;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct WsLayout {
    size_t S, C, m, X, y, U, total;
};

WsLayout layout(int BH, int n, int d, int dv, int w) {
    const size_t nc = (static_cast<size_t>(n) + w - 1) / w;
    const size_t slots = static_cast<size_t>(BH) * (nc + 1);
    WsLayout L{};
    size_t off = 0;
    L.S = off; off = align256(off + slots * d * d * sizeof(float));
    L.C = off; off = align256(off + slots * d * dv * sizeof(float));
    L.m = off; off = align256(off + slots * d * sizeof(float));
    L.X = off; off = align256(off + slots * d * dv * sizeof(float));
    L.y = off; off = align256(off + slots * d * sizeof(float));
    L.U = off; off = align256(off + static_cast<size_t>(BH) * nc * w * d * sizeof(float));
    L.total = off;
    return L;
}

}  // namespace

size_t generic_workspace_bytes(int BH, int n, int d, int dv, int w) {
    return layout(BH, n, d, dv, w).total;
}

GenericSlots generic_slots(const FwdProblem &p) {
    const WsLayout L = layout(p.B * p.H, p.n, p.d, p.dv, p.w);
    char *base = static_cast<char *>(p.ws);
    return GenericSlots{reinterpret_cast<float *>(base + L.S), reinterpret_cast<float *>(base + L.C),
                        reinterpret_cast<float *>(base + L.m), reinterpret_cast<float *>(base + L.X),
                        reinterpret_cast<float *>(base + L.y), reinterpret_cast<float *>(base + L.U)};
}

hipError_t generic_forward(const FwdProblem &p, hipStream_t st) {
    const int BH = p.B * p.H;
    const WsLayout L = layout(BH, p.n, p.d, p.dv, p.w);
    char *base = static_cast<char *>(p.ws);
    GenArgs a{};
    a.H = p.H; a.n = p.n; a.d = p.d; a.dv = p.dv; a.w = p.w; a.nc = p.nc;
    a.ridge = p.ridge; a.normalize = p.normalize; a.carries_only = p.carries_only; a.own_prefix = p.own_prefix;
    a.q = p.q; a.k = p.k; a.v = p.v; a.out = p.out; a.den = p.den;
    a.init = p.init; a.fin = p.fin; a.gam = p.gam;
    a.ws.S = reinterpret_cast<float *>(base + L.S);
    a.ws.C = reinterpret_cast<float *>(base + L.C);
    a.ws.m = reinterpret_cast<float *>(base + L.m);
    a.ws.X = reinterpret_cast<float *>(base + L.X);
    a.ws.y = reinterpret_cast<float *>(base + L.y);
    a.ws.U = reinterpret_cast<float *>(base + L.U);
    if (p.dtype == HLA_BF16) return pick_d<uint16_t>(a, BH, st);
    return pick_d<float>(a, BH, st);
}

}  // namespace hla
