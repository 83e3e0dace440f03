// fwd_higher.hip -- chunked forward of the two other operators of
// Higher-order Linear Attention: the asymmetric variant (AHLA) and masked
// third order; any d, dv, w in {16, 32, 64, 128}, fp32 or bf16 inputs, fp32
// arithmetic (products of LDS tiles, tile_fp32.h).
//
// AHLA (paperlayer.ai summary sec. 6, 6.1, 6.2): the masked left-cascaded
// product Q (K^T Q)(K^T V), out_t = sum_{j<=t} sum_{i<=j} g^(t-i)
// (q_t.k_j)(q_j.k_i) v_i, is first-order causal attention applied twice.
// Per chunk (L tokens, local t, s; e_t = g^(t+1), f_s = g^(L-1-s),
// carry-in (P0, m0, E0, n0) = the state before the chunk):
//   A   = (Q K^T) o D_g o L
//   Y   = A V + diag(e) Q P0            row s = P_s^T q_s (inclusive P)
//   yd  = A 1 + diag(e) Q m0
//   num = A Y + diag(e) Q E0,  den = A yd + diag(e) Q n0
//   P0' = g^L P0 + K^T diag(f) V,  m0' = g^L m0 + K^T f
//   E0' = g^L E0 + K^T diag(f) Y,  n0' = g^L n0 + K^T diag(f) yd
// E's chunk increment uses P0 (through Y), so the scan runs in two linear
// passes: (P, m) first, then (E, n).
//
// Third order (sec. 7, 7.1, 7.3; no decay): out_t = q_t^T F_t with
// F_t = sum_{j<=t} S_j q_j q_j^T P_j, the masked A A^T A V.  Per chunk
// (carry-in (S0, P0, m0, F0, Fd0)):
//   A   = (Q K^T) o L
//   U   = A K + Q S0                     row s = S_s q_s
//   Y   = A V + Q P0,  yd = A 1 + Q m0   row s = P_s^T q_s, q_s . m_s
//   Pm  = (Q U^T) o L
//   num = Pm Y + Q F0,  den = Pm yd + Q Fd0
//   S0' = S0 + K^T K,  P0' = P0 + K^T V,  m0' = m0 + K^T 1
//   F0' = F0 + U^T Y,  Fd0' = Fd0 + U^T yd
// (the second-order chunk form with the first-order values Y in place of V).
//
// Kernels (one workgroup of 256 threads per chunk unless stated):
//   k_hi_init   per head: slot 0 = the initial state, or zeros
//   k_hi_sums   chunk sums of the first level (and K^T K) -> slot c+1
//   k_hi_scan   per head, elementwise: slot c+1 = g^L slot c + slot c+1
//   k_hi_mid    A (and U), Y, yd kept for the output pass; second-level sums
//   k_hi_out    the output and the denominator
//   k_hi_final  per head: the final state
#include "device_common.h"
#include "hla_internal.h"
#include "tile_fp32.h"

namespace hla {
namespace {

constexpr int kThreads = tile::kThreads;
constexpr int kMaxW = tile::kMaxW;

struct HiSlots {
    float *S;        // [BH][nc+1][d][d]   (third order)
    float *P, *m;    // [BH][nc+1][d][dv], [d]: first level
    float *E, *n;    // [BH][nc+1][d][dv], [d]: second level (AHLA E, n; third order F, Fd)
    float *U;        // [BH][nc][w][d]     (third order)
    float *Y, *yd;   // [BH][nc][w][dv], [w]
};

struct HiArgs {
    int H, n, d, dv, w, nc;
    int normalize;
    const void *q, *k, *v;
    float *out, *den;
    HiState init, fin;  // init.X1 == nullptr: zero state
    HiSlots ws;
    GammaTab gam;
};

__device__ __forceinline__ size_t hslot(const HiArgs &a, int bh, int c) {
    return static_cast<size_t>(bh) * (a.nc + 1) + c;
}

template <int D, int DV, bool THIRD>
__global__ __launch_bounds__(kThreads) void k_hi_init(HiArgs a) {
    const int bh = blockIdx.x, tid = threadIdx.x;
    const size_t sl = hslot(a, bh, 0);
    float *P = a.ws.P + sl * D * DV, *E = a.ws.E + sl * D * DV, *m = a.ws.m + sl * D, *nn = a.ws.n + sl * D;
    const bool z = a.init.X1 == nullptr;
    const size_t hd = static_cast<size_t>(bh);
    for (int i = tid; i < D * DV; i += kThreads) {
        P[i] = z ? 0.0f : a.init.X1[hd * D * DV + i];
        E[i] = z ? 0.0f : a.init.X2[hd * D * DV + i];
    }
    if (tid < D) {
        m[tid] = z ? 0.0f : a.init.v1[hd * D + tid];
        nn[tid] = z ? 0.0f : a.init.v2[hd * D + tid];
    }
    if constexpr (THIRD) {
        float *S = a.ws.S + sl * D * D;
        for (int i = tid; i < D * D; i += kThreads) S[i] = z ? 0.0f : a.init.S[hd * D * D + i];
    }
}

// K^T diag(f) V and K^T f (and, for third order, K^T K) of chunk c -> slot c+1.
// K^T K is formed from the same operand on both sides, so it is exactly
// symmetric (fma(x_a, x_b, acc) is the same operation for (a, b) and (b, a)).
template <typename T, int D, int DV, bool THIRD>
__global__ __launch_bounds__(kThreads) void k_hi_sums(HiArgs a) {
    constexpr int MR = D / 16, MC = DV / 16;
    __shared__ float fs[kMaxW];
    __shared__ tile::Stage<tile::max3(D, DV, 16)> st;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int s0 = c * a.w, L = min(a.w, a.n - s0);
    const float g = THIRD ? 1.0f : head_gamma(a.gam, bh % a.H);
    const size_t tok = static_cast<size_t>(bh) * a.n + s0;
    const T *k = static_cast<const T *>(a.k) + tok * D;
    const T *v = static_cast<const T *>(a.v) + tok * DV;
    const int tid = threadIdx.x;
    for (int i = tid; i < L; i += kThreads) fs[i] = gpow(g, L - 1 - i);
    __syncthreads();
    auto ke = [&](int t, int l) { return Elem<T>::get(k, static_cast<size_t>(t) * D + l); };
    auto ve = [&](int t, int l) { return Elem<T>::get(v, static_cast<size_t>(t) * DV + l); };
    const size_t sl = hslot(a, bh, c + 1);
    if constexpr (THIRD) {
        float aS[MR][MR] = {};
        tile::mm<MR, MR, true>(aS, D, L, st, [&](int r, int t) { return ke(t, r); }, ke);
        tile::store_tile<MR, MR>(a.ws.S + sl * D * D, D, D, aS);
    }
    float aP[MR][MC] = {};
    tile::mm<MR, MC, true>(aP, D, L, st, [&](int r, int t) { return fs[t] * ke(t, r); }, ve);
    tile::store_tile<MR, MC>(a.ws.P + sl * D * DV, D, DV, aP);
    tile::row_sums(D, L, [&](int r, int t) { return fs[t] * ke(t, r); },
                   [&](int r, float x) { a.ws.m[sl * D + r] = x; });
}

// Decayed prefix over the slots, elementwise: slot c+1 = g^L_c slot c + slot
// c+1, for up to three arrays (element ranges concatenated along blockIdx.x).
struct ScanArr {
    float *base;
    int E;
};

__global__ __launch_bounds__(kThreads) void k_hi_scan(HiArgs a, ScanArr s0, ScanArr s1, ScanArr s2, int third) {
    const int bh = blockIdx.y;
    int e = blockIdx.x * kThreads + threadIdx.x;
    ScanArr seg = s0;
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
    const float g = third ? 1.0f : head_gamma(a.gam, bh % a.H);
    const int Llast = a.n - (a.nc - 1) * a.w;
    const float rf = gpow(g, a.w), rl = gpow(g, Llast);
    float *p = seg.base + static_cast<size_t>(bh) * (a.nc + 1) * seg.E + e;
    float run = p[0];
    int c = 0;
    for (; c + 8 <= a.nc; c += 8) {  // eight slot loads in flight per step
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
        float *slot = p + static_cast<size_t>(c + 1) * seg.E;
        run = (c == a.nc - 1 ? rl : rf) * run + *slot;
        *slot = run;
    }
}

// A (and U), Y, yd of chunk c (kept for the output pass), then the second
// level's chunk sums: K^T diag(f) Y, K^T diag(f) yd (AHLA) or U^T Y, U^T yd
// (third order) -> slot c+1 of E, n.
template <typename T, int D, int DV, int RT, bool THIRD>
__global__ __launch_bounds__(kThreads) void k_hi_mid(HiArgs a) {
    constexpr int MD = D / 16, MV = DV / 16, BW = 16 * RT;
    __shared__ float buf[BW * kMaxW];  // A (L x L, stride BW), then Y rows (stride DV)
    __shared__ float gt[kMaxW + 1], ydl[kMaxW];
    __shared__ tile::Stage<tile::max3(BW, D, DV)> st;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int s0 = c * a.w, L = min(a.w, a.n - s0);
    const float g = THIRD ? 1.0f : head_gamma(a.gam, bh % a.H);
    const size_t tok = static_cast<size_t>(bh) * a.n + s0;
    const T *q = static_cast<const T *>(a.q) + tok * D;
    const T *k = static_cast<const T *>(a.k) + tok * D;
    const T *v = static_cast<const T *>(a.v) + tok * DV;
    const size_t sl = hslot(a, bh, c);
    const float *P0 = a.ws.P + sl * D * DV, *m0 = a.ws.m + sl * D;
    const size_t ck = static_cast<size_t>(bh) * a.nc + c;
    float *Yg = a.ws.Y + ck * a.w * DV, *ydg = a.ws.yd + ck * a.w;
    const int tid = threadIdx.x;
    for (int i = tid; i <= a.w; i += kThreads) gt[i] = gpow(g, i);
    __syncthreads();
    auto qe = [&](int t, int l) { return Elem<T>::get(q, static_cast<size_t>(t) * D + l); };
    auto ke = [&](int t, int l) { return Elem<T>::get(k, static_cast<size_t>(t) * D + l); };
    auto ve = [&](int t, int l) { return Elem<T>::get(v, static_cast<size_t>(t) * DV + l); };
    // A[t][s] = g^(t-s) (q_t . k_s), s <= t
    tile::gram<RT, D>(buf, BW, L, st, qe, ke, [&](int t, int s, float x) { return s <= t ? gt[t - s] * x : 0.0f; });
    __syncthreads();
    if constexpr (THIRD) {  // U = A K + Q S0, kept for the output pass
        const float *S0 = a.ws.S + sl * D * D;
        float u[RT][MD] = {};
        tile::mm<RT, MD, false>(u, L, D, st, qe, [&](int l, int col) { return S0[l * D + col]; });
        tile::mm<RT, MD, false>(u, L, L, st, [&](int t, int s) { return buf[t * BW + s]; }, ke);
        tile::store_tile<RT, MD>(a.ws.U + ck * a.w * D, L, D, u);
    }
    // Y = A V + diag(e) Q P0 (third order: e = 1)
    float y[RT][MV] = {};
    tile::mm<RT, MV, false>(y, L, D, st, [&](int t, int l) { return gt[t + 1] * qe(t, l); },
                            [&](int l, int col) { return P0[l * DV + col]; });
    tile::mm<RT, MV, false>(y, L, L, st, [&](int t, int s) { return buf[t * BW + s]; }, ve);
    // yd = A 1 + diag(e) Q m0 (each row's two sums on the same lane)
    tile::row_sums(L, L, [&](int t, int s) { return buf[t * BW + s]; }, [&](int t, float x) { ydl[t] = x; });
    tile::row_sums(L, D, [&](int t, int l) { return gt[t + 1] * qe(t, l) * m0[l]; },
                   [&](int t, float x) {
                       ydl[t] += x;
                       ydg[t] = ydl[t];
                   });
    tile::store_tile<RT, MV>(Yg, L, DV, y);
    __syncthreads();  // every A read done
    tile::store_tile<RT, MV>(buf, L, DV, y);
    __syncthreads();
    // second level: E increment = K^T diag(f) Y (third order: U^T Y), n likewise with yd
    const size_t sn = hslot(a, bh, c + 1);
    const float *Ug = THIRD ? a.ws.U + ck * a.w * D : nullptr;
    auto lhs = [&](int r, int s) {
        if constexpr (THIRD) return Ug[static_cast<size_t>(s) * D + r];
        else return gt[L - 1 - s] * ke(s, r);
    };
    float z[MD][MV] = {};
    tile::mm<MD, MV, true>(z, D, L, st, lhs, [&](int s, int col) { return buf[s * DV + col]; });
    tile::store_tile<MD, MV>(a.ws.E + sn * D * DV, D, DV, z);
    tile::row_sums(D, L, [&](int r, int s) { return lhs(r, s) * ydl[s]; },
                   [&](int r, float x) { a.ws.n[sn * D + r] = x; });
}

// the output and the denominator of chunk c
template <typename T, int D, int DV, int RT, bool THIRD>
__global__ __launch_bounds__(kThreads) void k_hi_out(HiArgs a) {
    constexpr int MV = DV / 16, BW = 16 * RT, PS = BW + 1;  // odd stride: row walks hit distinct banks
    __shared__ float M[BW * PS];
    __shared__ float gt[kMaxW + 1], dens[kMaxW];
    __shared__ tile::Stage<tile::max3(BW, D, DV)> st;
    const int c = blockIdx.x, bh = blockIdx.y;
    const int s0 = c * a.w, L = min(a.w, a.n - s0);
    const float g = THIRD ? 1.0f : head_gamma(a.gam, bh % a.H);
    const size_t tok = static_cast<size_t>(bh) * a.n + s0;
    const T *q = static_cast<const T *>(a.q) + tok * D;
    const T *k = static_cast<const T *>(a.k) + tok * D;
    const size_t sl = hslot(a, bh, c);
    const float *E0 = a.ws.E + sl * D * DV, *n0 = a.ws.n + sl * D;
    const size_t ck = static_cast<size_t>(bh) * a.nc + c;
    const float *Yg = a.ws.Y + ck * a.w * DV, *ydg = a.ws.yd + ck * a.w;
    const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    for (int i = tid; i <= a.w; i += kThreads) gt[i] = gpow(g, i);
    __syncthreads();
    auto qe = [&](int t, int l) { return Elem<T>::get(q, static_cast<size_t>(t) * D + l); };
    auto ke = [&](int t, int l) { return Elem<T>::get(k, static_cast<size_t>(t) * D + l); };
    // AHLA: M = A = (Q K^T) o D_g o L;  third order: M = (Q U^T) o L
    if constexpr (THIRD) {
        const float *Ug = a.ws.U + ck * a.w * D;
        tile::gram<RT, D>(M, PS, L, st, qe, [&](int s, int l) { return Ug[static_cast<size_t>(s) * D + l]; },
                          [&](int t, int s, float x) { return s <= t ? x : 0.0f; });
    } else {
        tile::gram<RT, D>(M, PS, L, st, qe, ke, [&](int t, int s, float x) { return s <= t ? gt[t - s] * x : 0.0f; });
    }
    __syncthreads();
    // den_t = sum_s M[t][s] yd_s + e_t (q_t . n0)
    tile::row_sums(L, L, [&](int t, int s) { return M[t * PS + s] * ydg[s]; },
                   [&](int t, float x) { dens[t] = x; });
    tile::row_sums(L, D, [&](int t, int l) { return gt[t + 1] * qe(t, l) * n0[l]; },
                   [&](int t, float x) {
                       const float dn = dens[t] + x;
                       dens[t] = dn;
                       if (a.den) a.den[tok + t] = dn;
                   });
    __syncthreads();
    // num = M Y + diag(e) Q E0
    float acc[RT][MV] = {};
    tile::mm<RT, MV, false>(acc, L, L, st, [&](int t, int s) { return M[t * PS + s]; },
                            [&](int s, int col) { return Yg[static_cast<size_t>(s) * DV + col]; });
    tile::mm<RT, MV, false>(acc, L, D, st, [&](int t, int l) { return gt[t + 1] * qe(t, l); },
                            [&](int l, int col) { return E0[l * DV + col]; });
    float *out = a.out + tok * DV;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int t = RT * ty + i;
        if (t >= L) continue;
        const float dn = dens[t];
#pragma unroll
        for (int j = 0; j < MV; ++j) {
            const float num = acc[i][j];
            out[static_cast<size_t>(t) * DV + MV * tx + j] = a.normalize ? num / dn : num;
        }
    }
}

template <int D, int DV, bool THIRD>
__global__ __launch_bounds__(kThreads) void k_hi_final(HiArgs a) {
    const int bh = blockIdx.x, tid = threadIdx.x;
    const size_t sl = hslot(a, bh, a.nc), hd = static_cast<size_t>(bh);
    for (int i = tid; i < D * DV; i += kThreads) {
        a.fin.X1[hd * D * DV + i] = a.ws.P[sl * D * DV + i];
        a.fin.X2[hd * D * DV + i] = a.ws.E[sl * D * DV + i];
    }
    if (tid < D) {
        a.fin.v1[hd * D + tid] = a.ws.m[sl * D + tid];
        a.fin.v2[hd * D + tid] = a.ws.n[sl * D + tid];
    }
    if constexpr (THIRD) {
        for (int i = tid; i < D * D; i += kThreads) a.fin.S[hd * D * D + i] = a.ws.S[sl * D * D + i];
    } else {
        if (tid == 0 && a.fin.rho) {
            const float g = head_gamma(a.gam, bh % a.H);
            const float r0 = (a.init.X1 && a.init.rho) ? a.init.rho[bh] : 1.0f;
            a.fin.rho[bh] = r0 * gpow(g, a.n);
        }
    }
}

template <typename T, int D, int DV, bool THIRD>
hipError_t launch(const HiArgs &a, int BH, hipStream_t st) {
    const dim3 blk(kThreads);
    hipLaunchKernelGGL((k_hi_init<D, DV, THIRD>), dim3(BH), blk, 0, st, a);
    if (a.nc > 0) {
        hipLaunchKernelGGL((k_hi_sums<T, D, DV, THIRD>), dim3(a.nc, BH), blk, 0, st, a);
        const ScanArr sP{a.ws.P, D * DV}, sm{a.ws.m, D}, sS{THIRD ? a.ws.S : nullptr, THIRD ? D * D : 0};
        const int e1 = D * DV + D + (THIRD ? D * D : 0);
        hipLaunchKernelGGL(k_hi_scan, dim3((e1 + kThreads - 1) / kThreads, BH), blk, 0, st, a, sP, sm, sS,
                           THIRD ? 1 : 0);
        if (a.w > 64) hipLaunchKernelGGL((k_hi_mid<T, D, DV, 8, THIRD>), dim3(a.nc, BH), blk, 0, st, a);
        else hipLaunchKernelGGL((k_hi_mid<T, D, DV, 4, THIRD>), dim3(a.nc, BH), blk, 0, st, a);
        const ScanArr sE{a.ws.E, D * DV}, sn{a.ws.n, D}, none{nullptr, 0};
        const int e2 = D * DV + D;
        hipLaunchKernelGGL(k_hi_scan, dim3((e2 + kThreads - 1) / kThreads, BH), blk, 0, st, a, sE, sn, none,
                           THIRD ? 1 : 0);
        if (a.w > 64) hipLaunchKernelGGL((k_hi_out<T, D, DV, 8, THIRD>), dim3(a.nc, BH), blk, 0, st, a);
        else hipLaunchKernelGGL((k_hi_out<T, D, DV, 4, THIRD>), dim3(a.nc, BH), blk, 0, st, a);
    }
    if (a.fin.X1) hipLaunchKernelGGL((k_hi_final<D, DV, THIRD>), dim3(BH), blk, 0, st, a);
    return hipGetLastError();
}

template <typename T, int D, bool THIRD>
hipError_t pick_dv(const HiArgs &a, int BH, hipStream_t st) {
    switch (a.dv) {
        case 16: return launch<T, D, 16, THIRD>(a, BH, st);
        case 32: return launch<T, D, 32, THIRD>(a, BH, st);
        case 64: return launch<T, D, 64, THIRD>(a, BH, st);
        case 128: return launch<T, D, 128, THIRD>(a, BH, st);
    }
    return hipErrorInvalidValue;
}

template <typename T, bool THIRD>
hipError_t pick_d(const HiArgs &a, int BH, hipStream_t st) {
    switch (a.d) {
        case 16: return pick_dv<T, 16, THIRD>(a, BH, st);
        case 32: return pick_dv<T, 32, THIRD>(a, BH, st);
        case 64: return pick_dv<T, 64, THIRD>(a, BH, st);
        case 128: return pick_dv<T, 128, THIRD>(a, BH, st);
    }
    return hipErrorInvalidValue;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct HiLayout {
    size_t S, P, m, E, n, U, Y, yd, total;
};

// Bytes of the flag region that follows the control block: the one-launch
// path's flags (none where that path cannot run), which no data overlaps.
// AHLA: the chained map's two flag sets side by side (one launch, so one
// epoch: they must not overlap); third order: the first-order map's flags
// and the second-order kernel's, which launch one after the other and share
// the region.
size_t flag_area(int BH, int n, int d, int dv, int w, bool third) {
    if (!(d == 64 && dv == 64 && w == 64 && n > 0)) return 0;
    const size_t fb = la64_flag_bytes(BH, n);
    if (!third) return align256(2 * fb);
    const size_t f2 = fast64_flag_bytes(BH, n);
    return align256(fb > f2 ? fb : f2);
}

// (the control block and the flag region of the one-launch path below come
// first; this path touches neither)
HiLayout layout(int BH, int n, int d, int dv, int w, bool third) {
    const size_t nc = (static_cast<size_t>(n) + w - 1) / w;
    const size_t slots = static_cast<size_t>(BH) * (nc + 1), chunks = static_cast<size_t>(BH) * nc;
    HiLayout L{};
    size_t off = kCtrlBytes + flag_area(BH, n, d, dv, w, third);
    L.S = off; off = align256(off + (third ? slots * d * d * sizeof(float) : 0));
    L.P = off; off = align256(off + slots * d * dv * sizeof(float));
    L.m = off; off = align256(off + slots * d * sizeof(float));
    L.E = off; off = align256(off + slots * d * dv * sizeof(float));
    L.n = off; off = align256(off + slots * d * sizeof(float));
    L.U = off; off = align256(off + (third ? chunks * w * d * sizeof(float) : 0));
    L.Y = off; off = align256(off + chunks * w * dv * sizeof(float));
    L.yd = off; off = align256(off + chunks * w * sizeof(float));
    L.total = off;
    return L;
}

// ---- one-launch path (bf16, d = dv = 64, chunk 64, numerator only, no states):
// AHLA = LA(Q, K, LA(Q, K, V)) and third order = HLA2(Q, K, LA(Q, K, V)) with
// LA the masked first-order map (fwd_la64.hip, decay g; g = 1 for third
// order) and HLA2 the second-order forward (k_fast64).  The intermediate
// values Y = LA(Q, K, V) are kept as bf16 hi + lo, and both maps are linear in
// their values: the second map (first order for AHLA, second order for third
// order) takes the pair as its values, in one launch.
// Workspace: control block, flag region, the one-launch kernels' data
// (shared: every launch leaves the control block valid for the next), Y hi,
// Y lo.
struct FastHiLayout {
    size_t flags, data, yh, yl, total;
};

// AHLA: the chained map's two sets of sums; third order: the first map's
// sums (or the second-order kernel's data, whichever is larger), then its
// output as a bf16 pair
FastHiLayout fast_layout(int BH, int n, bool third) {
    const size_t tok = static_cast<size_t>(BH) * n;
    FastHiLayout L{};
    L.flags = kCtrlBytes;
    L.data = L.flags + flag_area(BH, n, 64, 64, 64, third);
    if (!third) {
        L.yh = L.yl = 0;
        L.total = L.data + 2 * la64_agg_bytes(BH, n);
        return L;
    }
    const size_t la = la64_agg_bytes(BH, n), f64 = fast64_data_bytes(BH, n);
    L.yh = align256(L.data + (la > f64 ? la : f64));
    L.yl = align256(L.yh + tok * 64 * sizeof(uint16_t));
    L.total = L.yl + tok * 64 * sizeof(uint16_t);
    return L;
}

bool fast_eligible(const HiProblem &p) {
    if (!(p.dtype == HLA_BF16 && p.d == 64 && p.dv == 64 && p.w == 64 && p.n > 0 && !p.normalize &&
          p.den == nullptr && p.init.X1 == nullptr && p.fin.X1 == nullptr))
        return false;
    const int nh = p.gam.per_head ? p.H : 1;
    for (int h = 0; h < nh; ++h)
        if (p.gam.g[h] < 0.75f) return false;
    return true;
}

hipError_t fast_higher(const HiProblem &p, hipStream_t st) {
    const int BH = p.B * p.H;
    const FastHiLayout L = fast_layout(BH, p.n, p.third);
    char *base = static_cast<char *>(p.ws);
    uint32_t *ctrl = reinterpret_cast<uint32_t *>(base);
    char *flags = base + L.flags, *data = base + L.data;
    LaProblem la{};
    la.B = p.B; la.H = p.H; la.n = p.n; la.q = p.q; la.k = p.k; la.gam = p.gam;
    if (!p.third) {  // out = LA (Q, K, LA (Q, K, V)) in one launch
        const size_t fb = la64_flag_bytes(BH, p.n), ab = la64_agg_bytes(BH, p.n);
        const LaSpace s1{reinterpret_cast<uint32_t *>(flags), reinterpret_cast<float *>(data)};
        const LaSpace s2{reinterpret_cast<uint32_t *>(flags + fb), reinterpret_cast<float *>(data + ab)};
        la.v = p.v; la.out = p.out; la.mode = 0;
        return la64_chain(la, ctrl, s1, s2, st);
    }
    uint16_t *yh = reinterpret_cast<uint16_t *>(base + L.yh), *yl = reinterpret_cast<uint16_t *>(base + L.yl);
    // Y = LA(Q, K, V) as bf16 hi + lo
    la.v = p.v; la.oh = yh; la.ol = yl; la.mode = 2;
    hipError_t e = la64_forward_in(la, ctrl, LaSpace{reinterpret_cast<uint32_t *>(flags), reinterpret_cast<float *>(data)}, st);
    if (e != hipSuccess) return e;
    FwdProblem f{};  // the second-order map on the pair (hi, lo) at once
    f.B = p.B; f.H = p.H; f.n = p.n; f.d = 64; f.dv = 64; f.w = 64; f.nc = (p.n + 63) / 64;
    f.dtype = HLA_BF16; f.q = p.q; f.k = p.k; f.gam = p.gam;
    f.v = yh; f.vl = yl; f.out = p.out;
    return fast64_forward(f, ctrl, reinterpret_cast<uint32_t *>(flags), data, st);
}

}  // namespace

size_t higher_workspace_bytes(int BH, int n, int d, int dv, int w, bool third) {
    const size_t gen = layout(BH, n, d, dv, w, third).total;
    if (!(d == 64 && dv == 64 && w == 64 && n > 0)) return gen;
    const size_t fast = fast_layout(BH, n, third).total;
    return gen > fast ? gen : fast;
}

hipError_t higher_forward(const HiProblem &p, hipStream_t st) {
    if (fast_eligible(p)) return fast_higher(p, st);
    const int BH = p.B * p.H;
    const HiLayout L = layout(BH, p.n, p.d, p.dv, p.w, p.third);
    char *base = static_cast<char *>(p.ws);
    HiArgs a{};
    a.H = p.H; a.n = p.n; a.d = p.d; a.dv = p.dv; a.w = p.w; a.nc = (p.n + p.w - 1) / p.w;
    a.normalize = p.normalize;
    a.q = p.q; a.k = p.k; a.v = p.v; a.out = p.out; a.den = p.den;
    a.init = p.init; a.fin = p.fin; a.gam = p.gam;
    a.ws.S = reinterpret_cast<float *>(base + L.S);
    a.ws.P = reinterpret_cast<float *>(base + L.P);
    a.ws.m = reinterpret_cast<float *>(base + L.m);
    a.ws.E = reinterpret_cast<float *>(base + L.E);
    a.ws.n = reinterpret_cast<float *>(base + L.n);
    a.ws.U = reinterpret_cast<float *>(base + L.U);
    a.ws.Y = reinterpret_cast<float *>(base + L.Y);
    a.ws.yd = reinterpret_cast<float *>(base + L.yd);
    if (p.third) {
        if (p.dtype == HLA_BF16) return pick_d<uint16_t, true>(a, BH, st);
        return pick_d<float, true>(a, BH, st);
    }
    if (p.dtype == HLA_BF16) return pick_d<uint16_t, false>(a, BH, st);
    return pick_d<float, false>(a, BH, st);
}

}  // namespace hla
