// decode_higher.hip -- one streaming decode step of the asymmetric variant
// (AHLA) and of masked third-order HLA (the recurrences of fwd_higher.hip,
// one token per state).
//
// AHLA (paperlayer.ai summary sec. 6.1 and 6.3: strictly causal streaming
// with O(d dv) work and state per token), decay g:
//   P_t = g P + k v^T,  m_t = g m + k,  y = P_t^T q,  yd = q . m_t
//   E_t = g E + k y^T,  n_t = g n + yd k
//   num = E_t^T q = g E^T q + (q . k) y,  den = g (q . n) + (q . k) yd
// so P and E are each read once and written once (E^T q is taken from the
// old E while the new one is written).
// Third order (sec. 7.1 and 7.2: the strictly causal streaming kernel), no decay:
//   S_t = S + k k^T,  a = S_t q,  P_t = P + k v^T,  y = P_t^T q,
//   m_t = m + k,  yd = q . m_t,  F_t = F + a y^T,  Fd_t = Fd + yd a
//   num = F_t^T q = F^T q + (q . a) y,  den = q . Fd_t
// S (symmetric), P and F are each read once and written once.
//
// One workgroup of 256 threads per state; rows of each matrix are read as
// float4 with a row split over W/4 lanes, and column sums are reduced
// through LDS in a fixed order.
#include "device_common.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kThreads = 256;

struct HiDecArgs {
    int H, d, dv, normalize;
    const void *q, *k, *v;
    HiState st;
    float *out, *den;
    GammaTab gam;
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

template <int W>
__device__ __forceinline__ void reduce_cols(float4 p, float *red, float *dst) {
    constexpr int LPR = W / 4, RPI = kThreads / LPR;
    const int tid = threadIdx.x, c4 = tid % LPR, rg = tid / LPR;
    float *row = red + rg * W + c4 * 4;
    row[0] = p.x; row[1] = p.y; row[2] = p.z; row[3] = p.w;
    __syncthreads();
    if (tid < W) {
        float s = 0.0f;
#pragma unroll
        for (int g = 0; g < RPI; ++g) s += red[g * W + tid];
        dst[tid] = s;
    }
    __syncthreads();
}

// One pass over an R x W row-major matrix X: with old rows x_r, writes
// X_r <- alpha x_r + lr[r] * cv (cv a W-vector) and returns in dst the
// column sums sum_r wr[r] * (use_new ? new x_r : old x_r).
template <int R, int W>
__device__ __forceinline__ void stream_rows(float *X, float alpha, const float *lr, const float *cv,
                                            const float *wr, bool use_new, float *red, float *dst) {
    constexpr int LPR = W / 4, RPI = kThreads / LPR, IT = (R + RPI - 1) / RPI;
    const int tid = threadIdx.x, c4 = tid % LPR, r0 = tid / LPR;
    const float c0 = cv[c4 * 4], c1 = cv[c4 * 4 + 1], c2 = cv[c4 * 4 + 2], c3 = cv[c4 * 4 + 3];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 x[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int r = r0 + it * RPI;
        if (r < R) x[it] = *reinterpret_cast<const float4 *>(X + r * W + c4 * 4);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int r = r0 + it * RPI;
        if (r < R) {
            const float l = lr[r], w = wr[r];
            float4 y;
            y.x = alpha * x[it].x + l * c0;
            y.y = alpha * x[it].y + l * c1;
            y.z = alpha * x[it].z + l * c2;
            y.w = alpha * x[it].w + l * c3;
            *reinterpret_cast<float4 *>(X + r * W + c4 * 4) = y;
            const float4 s = use_new ? y : x[it];
            acc.x += w * s.x; acc.y += w * s.y; acc.z += w * s.z; acc.w += w * s.w;
        }
    }
    reduce_cols<W>(acc, red, dst);
}

template <typename T, int D, int DV, bool THIRD>
__global__ __launch_bounds__(kThreads) void k_decode_higher(HiDecArgs a) {
    __shared__ float qs[D], ks[D], as[D], ms[D], vs[DV], ys[DV], xs[DV];
    __shared__ float red[1024];
    __shared__ float scal[4];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
    const float g = THIRD ? 1.0f : head_gamma(a.gam, b % a.H);
    float *P = a.st.X1 + static_cast<size_t>(b) * D * DV;
    float *E = a.st.X2 + static_cast<size_t>(b) * D * DV;
    float *m = a.st.v1 + static_cast<size_t>(b) * D;
    float *n = a.st.v2 + static_cast<size_t>(b) * D;
    if (tid < D) {
        qs[tid] = Elem<T>::get(static_cast<const T *>(a.q), static_cast<size_t>(b) * D + tid);
        ks[tid] = Elem<T>::get(static_cast<const T *>(a.k), static_cast<size_t>(b) * D + tid);
    }
    if (tid < DV) vs[tid] = Elem<T>::get(static_cast<const T *>(a.v), static_cast<size_t>(b) * DV + tid);
    __syncthreads();
    if constexpr (THIRD) {  // S_t = S + k k^T, a = S_t q (column sums; S symmetric)
        stream_rows<D, D>(a.st.S + static_cast<size_t>(b) * D * D, 1.0f, ks, ks, qs, true, red, as);
    }
    // P_t = g P + k v^T, y = P_t^T q
    stream_rows<D, DV>(P, g, ks, vs, qs, true, red, ys);
    // m_t, the scalars yd = q . m_t, q . k, q . a (third order), q . n_{t-1}
    if (tid < D) {
        const float mt = g * m[tid] + ks[tid];
        m[tid] = mt;
        ms[tid] = mt;
    }
    __syncthreads();
    if (wv < 4) {
        float x = 0.0f;
        for (int i = lane; i < D; i += 64) {
            if (wv == 0) x += qs[i] * ms[i];
            else if (wv == 1) x += qs[i] * ks[i];
            else if (wv == 2) x += THIRD ? qs[i] * as[i] : 0.0f;
            else x += qs[i] * n[i];
        }
        x = wave_sum(x);
        if (lane == 0) scal[wv] = x;
    }
    __syncthreads();
    const float yd = scal[0], qk = scal[1], qa = scal[2], qn = scal[3];
    // second level: E_t = g E + k y^T (AHLA) / F_t = F + a y^T (third); x = E^T q of the old E
    stream_rows<D, DV>(E, g, THIRD ? as : ks, ys, qs, false, red, xs);
    if (tid < D) n[tid] = g * n[tid] + yd * (THIRD ? as[tid] : ks[tid]);
    if (tid < DV) {
        const float lead = THIRD ? qa : qk;  // q . (the vector the new row of E was scaled by)
        const float num = g * xs[tid] + lead * ys[tid];
        const float dn = g * qn + lead * yd;
        a.out[static_cast<size_t>(b) * DV + tid] = a.normalize ? num / dn : num;
        if (tid == 0) {
            if (a.den) a.den[b] = dn;
            if (!THIRD && a.st.rho) a.st.rho[b] *= g;
        }
    }
}

template <typename T, int D, bool THIRD>
hipError_t pick_dv(const HiDecArgs &a, int N, hipStream_t st) {
    switch (a.dv) {
        case 16: hipLaunchKernelGGL((k_decode_higher<T, D, 16, THIRD>), dim3(N), dim3(kThreads), 0, st, a); break;
        case 32: hipLaunchKernelGGL((k_decode_higher<T, D, 32, THIRD>), dim3(N), dim3(kThreads), 0, st, a); break;
        case 64: hipLaunchKernelGGL((k_decode_higher<T, D, 64, THIRD>), dim3(N), dim3(kThreads), 0, st, a); break;
        case 128: hipLaunchKernelGGL((k_decode_higher<T, D, 128, THIRD>), dim3(N), dim3(kThreads), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, bool THIRD>
hipError_t pick_d(const HiDecArgs &a, int N, hipStream_t st) {
    switch (a.d) {
        case 16: return pick_dv<T, 16, THIRD>(a, N, st);
        case 32: return pick_dv<T, 32, THIRD>(a, N, st);
        case 64: return pick_dv<T, 64, THIRD>(a, N, st);
        case 128: return pick_dv<T, 128, THIRD>(a, N, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t higher_decode(const HiDecodeProblem &p, hipStream_t st) {
    HiDecArgs a{};
    a.H = p.H; a.d = p.d; a.dv = p.dv; a.normalize = p.normalize;
    a.q = p.q; a.k = p.k; a.v = p.v; a.st = p.st; a.out = p.out; a.den = p.den; a.gam = p.gam;
    const int N = p.B * p.H;
    if (p.third) {
        if (p.dtype == HLA_BF16) return pick_d<uint16_t, true>(a, N, st);
        return pick_d<float, true>(a, N, st);
    }
    if (p.dtype == HLA_BF16) return pick_d<uint16_t, false>(a, N, st);
    return pick_d<float, false>(a, N, st);
}

}  // namespace hla
