// decode.hip -- one streaming decode step of masked second-order HLA.
//
// Higher-order Linear Attention, paperlayer.ai summary sec. 1-2 (constant-size
// state per head, O(d^2 + d dv) work per token) and gist.science explainer,
// Methodik item 1 (prefix summaries, cross summaries, masked output).  For one
// new token (q, k, v) and a state (S, C, m, G, h) at t-1, with decay g and
// ridge lambda:
//   r = k^T C_{t-1},  s = k . m_{t-1}
//   S_t = g S + k k^T,   C_t = g C + q v^T,   m_t = g m + q
//   G_t = g^2 G + g k r^T,   h_t = g^2 h + g s k
//   a = (S_t + lambda I) q
//   num = a^T C_t - q^T G_t = g (a^T C_{t-1}) + (a.q) v - g^2 (q^T G_{t-1}) - g (q.k) r
//   den = a . m_t - q . h_t
// The rewritten num lets each of S, C and G be read once and written once:
// the step is a pure stream over the state (about 2 * 4 * (d^2 + 2 d dv)
// bytes per state), so it is bound by HBM bandwidth.
//
// One workgroup of 256 threads per state.  Rows of each matrix are read as
// float4 with a row split over W/4 lanes, so every wave touches whole
// contiguous rows; column partial sums are reduced through LDS.  S must be
// symmetric (the method keeps it so): a = S_t q is formed column-wise, and
// for d >= 64 only the 32 x 32 tiles on and above the diagonal are read (at
// d = 128, 40 of 64 KB); each tile below it is written as the transpose of
// its partner through LDS.
#include "device_common.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kThreads = 256;

struct DecArgs {
    int H, d, dv;
    float ridge;
    int normalize;
    const void *q, *k, *v;
    hla_state st;
    float *out, *den;
    GammaTab gam;
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Column sums of per-thread float4 partials: thread (row group rg, column
// group c4) holds p; result[col] for col < W is written to dst.
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

template <typename T, int D, int DV>
__global__ __launch_bounds__(kThreads) void k_decode(DecArgs a) {
    __shared__ float qs[D], ks[D], ms[D], hs[D], as[D], vs[DV];
    __shared__ float rs[DV], acs[DV], qgs[DV];
    __shared__ float red[2 * 1024];
    // transposed copies of the tiles above the diagonal (d >= 64)
    __shared__ float tb[D >= 64 ? (D / 32) * (D / 32 - 1) / 2 : 1][32 * 33];
    __shared__ float scal[4];
    const int b = blockIdx.x;  // state index b*H + h
    const float g = head_gamma(a.gam, b % a.H), g2 = g * g, lam = a.ridge;
    const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
    float *S = a.st.S + static_cast<size_t>(b) * D * D;
    float *C = a.st.C + static_cast<size_t>(b) * D * DV;
    float *G = a.st.G + static_cast<size_t>(b) * D * DV;
    float *m = a.st.m + static_cast<size_t>(b) * D;
    float *h = a.st.h + static_cast<size_t>(b) * D;
    if (tid < D) {
        qs[tid] = Elem<T>::get(static_cast<const T *>(a.q), static_cast<size_t>(b) * D + tid);
        ks[tid] = Elem<T>::get(static_cast<const T *>(a.k), static_cast<size_t>(b) * D + tid);
        ms[tid] = m[tid];
        hs[tid] = h[tid];
    }
    if (tid < DV) vs[tid] = Elem<T>::get(static_cast<const T *>(a.v), static_cast<size_t>(b) * DV + tid);
    __syncthreads();

    // pass 1: S_t = g S + k k^T ; a = S_t q (column form, S symmetric)
    if constexpr (D >= 64) {
        // Tiles (I, J), I <= J, of 32 x 32; thread (row, c4) = (tid / 8, tid % 8)
        // holds elements (row, 4 c4 .. 4 c4 + 3) of each.  Column sums over a
        // tile give a[32 J + col]; the transposed tile (J, I), I < J, below
        // the diagonal gives a[32 I + row] as row sums.
        constexpr int NT = D / 32, NU = NT * (NT + 1) / 2, NOFF = NU - NT;
        const int row = tid >> 3, c4 = tid & 7;
        float4 x[NU];
        int ti[NU], tj[NU];
        {
            int u = 0;
#pragma unroll
            for (int I = 0; I < NT; ++I)
#pragma unroll
                for (int J = I; J < NT; ++J) {
                    ti[u] = I;
                    tj[u] = J;
                    ++u;
                }
        }
#pragma unroll
        for (int u = 0; u < NU; ++u)
            x[u] = *reinterpret_cast<const float4 *>(S + (32 * ti[u] + row) * D + 32 * tj[u] + c4 * 4);
        float4 accc[NT];
        float accr[NT];
#pragma unroll
        for (int J = 0; J < NT; ++J) {
            accc[J] = make_float4(0.f, 0.f, 0.f, 0.f);
            accr[J] = 0.0f;
        }
        int off = 0;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int I = ti[u], J = tj[u];
            const float kr = ks[32 * I + row], qr = qs[32 * I + row];
            const int cb = 32 * J + c4 * 4;
            float4 y;
            y.x = g * x[u].x + kr * ks[cb];
            y.y = g * x[u].y + kr * ks[cb + 1];
            y.z = g * x[u].z + kr * ks[cb + 2];
            y.w = g * x[u].w + kr * ks[cb + 3];
            *reinterpret_cast<float4 *>(S + (32 * I + row) * D + cb) = y;
            accc[J].x += y.x * qr; accc[J].y += y.y * qr; accc[J].z += y.z * qr; accc[J].w += y.w * qr;
            if (I < J) {  // the mirrored tile: row sums, and its transpose staged for the lower write
                accr[I] += (y.x * qs[cb] + y.y * qs[cb + 1]) + (y.z * qs[cb + 2] + y.w * qs[cb + 3]);
                float *t = tb[off];
                t[row * 33 + c4 * 4] = y.x;
                t[row * 33 + c4 * 4 + 1] = y.y;
                t[row * 33 + c4 * 4 + 2] = y.z;
                t[row * 33 + c4 * 4 + 3] = y.w;
                ++off;
            }
        }
        // column sums: over the 8 rows of this wave (lanes 8 apart), then the 4 waves
#pragma unroll
        for (int J = 0; J < NT; ++J) {
#pragma unroll
            for (int sh = 8; sh < 64; sh <<= 1) {
                accc[J].x += __shfl_xor(accc[J].x, sh, 64);
                accc[J].y += __shfl_xor(accc[J].y, sh, 64);
                accc[J].z += __shfl_xor(accc[J].z, sh, 64);
                accc[J].w += __shfl_xor(accc[J].w, sh, 64);
            }
            // row sums: over the 8 lanes of a row
#pragma unroll
            for (int sh = 1; sh < 8; sh <<= 1) accr[J] += __shfl_xor(accr[J], sh, 64);
        }
        if (lane < 8) {
#pragma unroll
            for (int J = 0; J < NT; ++J) {
                float *cs = red + (wv * NT + J) * 32 + c4 * 4;
                cs[0] = accc[J].x; cs[1] = accc[J].y; cs[2] = accc[J].z; cs[3] = accc[J].w;
            }
        }
        if (c4 == 0) {
#pragma unroll
            for (int I = 0; I < NT; ++I) red[1024 + 32 * I + row] = accr[I];
        }
        __syncthreads();
        // the lower tiles: row r2 of tile (J, I) is column r2 of tile (I, J)
        {
            int o = 0;
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int I = ti[u], J = tj[u];
                if (I < J) {
                    const float *t = tb[o];
                    float4 z;
                    z.x = t[(c4 * 4) * 33 + row];
                    z.y = t[(c4 * 4 + 1) * 33 + row];
                    z.z = t[(c4 * 4 + 2) * 33 + row];
                    z.w = t[(c4 * 4 + 3) * 33 + row];
                    *reinterpret_cast<float4 *>(S + (32 * J + row) * D + 32 * I + c4 * 4) = z;
                    ++o;
                }
            }
        }
        if (tid < D) {
            const int J = tid >> 5, col = tid & 31;
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < kThreads / 64; ++w) sum += red[(w * NT + J) * 32 + col];
            // row sums exist for tile rows above the last
            as[tid] = sum + (J < NT - 1 ? red[1024 + tid] : 0.0f) + lam * qs[tid];
        }
        __syncthreads();
        (void)NOFF;
    } else {
    {
        constexpr int LPR = D / 4, RPI = kThreads / LPR, IT = (D + RPI - 1) / RPI;
        const int c4 = tid % LPR, r0 = tid / LPR;
        const float k0 = ks[c4 * 4], k1 = ks[c4 * 4 + 1], k2 = ks[c4 * 4 + 2], k3 = ks[c4 * 4 + 3];
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        float4 x[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int r = r0 + it * RPI;
            if (r < D) x[it] = *reinterpret_cast<const float4 *>(S + r * D + c4 * 4);
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int r = r0 + it * RPI;
            if (r < D) {
                const float kr = ks[r], qr = qs[r];
                float4 y;
                y.x = g * x[it].x + kr * k0;
                y.y = g * x[it].y + kr * k1;
                y.z = g * x[it].z + kr * k2;
                y.w = g * x[it].w + kr * k3;
                *reinterpret_cast<float4 *>(S + r * D + c4 * 4) = y;
                acc.x += y.x * qr; acc.y += y.y * qr; acc.z += y.z * qr; acc.w += y.w * qr;
            }
        }
        reduce_cols<D>(acc, red, as);
        if (tid < D) as[tid] += lam * qs[tid];
        __syncthreads();
    }
    }
    // scalars: s = k . m_{t-1}, a.q, q.k
    if (wv < 3) {
        float x = 0.0f;
        for (int i = lane; i < D; i += 64) {
            if (wv == 0) x += ks[i] * ms[i];
            else if (wv == 1) x += as[i] * qs[i];
            else x += qs[i] * ks[i];
        }
        x = wave_sum(x);
        if (lane == 0) scal[wv] = x;
    }
    __syncthreads();
    // m_t, h_t, den
    if (tid < D) {
        const float mt = g * ms[tid] + qs[tid];
        const float ht = g2 * hs[tid] + g * scal[0] * ks[tid];
        m[tid] = mt;
        h[tid] = ht;
        ms[tid] = as[tid] * mt - qs[tid] * ht;  // den terms
    }
    __syncthreads();
    if (wv == 0) {
        float x = 0.0f;
        for (int i = lane; i < D; i += 64) x += ms[i];
        x = wave_sum(x);
        if (lane == 0) scal[3] = x;
    }
    // pass 2: r = k^T C_{t-1}, aC = a^T C_{t-1}; C_t = g C + q v^T
    {
        constexpr int LPR = DV / 4, RPI = kThreads / LPR, IT = (D + RPI - 1) / RPI;
        const int c4 = tid % LPR, r0 = tid / LPR;
        const float v0 = vs[c4 * 4], v1 = vs[c4 * 4 + 1], v2 = vs[c4 * 4 + 2], v3 = vs[c4 * 4 + 3];
        float4 pr = make_float4(0.f, 0.f, 0.f, 0.f), pa = pr;
        float4 x[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int r = r0 + it * RPI;
            if (r < D) x[it] = *reinterpret_cast<const float4 *>(C + r * DV + c4 * 4);
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int r = r0 + it * RPI;
            if (r < D) {
                const float kr = ks[r], ar = as[r], qr = qs[r];
                pr.x += kr * x[it].x; pr.y += kr * x[it].y; pr.z += kr * x[it].z; pr.w += kr * x[it].w;
                pa.x += ar * x[it].x; pa.y += ar * x[it].y; pa.z += ar * x[it].z; pa.w += ar * x[it].w;
                float4 y;
                y.x = g * x[it].x + qr * v0;
                y.y = g * x[it].y + qr * v1;
                y.z = g * x[it].z + qr * v2;
                y.w = g * x[it].w + qr * v3;
                *reinterpret_cast<float4 *>(C + r * DV + c4 * 4) = y;
            }
        }
        reduce_cols<DV>(pr, red, rs);
        reduce_cols<DV>(pa, red + 1024, acs);
    }
    // pass 3: qG = q^T G_{t-1}; G_t = g^2 G + g k r^T
    {
        constexpr int LPR = DV / 4, RPI = kThreads / LPR, IT = (D + RPI - 1) / RPI;
        const int c4 = tid % LPR, r0 = tid / LPR;
        const float r_0 = rs[c4 * 4], r_1 = rs[c4 * 4 + 1], r_2 = rs[c4 * 4 + 2], r_3 = rs[c4 * 4 + 3];
        float4 pq = make_float4(0.f, 0.f, 0.f, 0.f);
        float4 x[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int r = r0 + it * RPI;
            if (r < D) x[it] = *reinterpret_cast<const float4 *>(G + r * DV + c4 * 4);
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int r = r0 + it * RPI;
            if (r < D) {
                const float qr = qs[r], gk = g * ks[r];
                pq.x += qr * x[it].x; pq.y += qr * x[it].y; pq.z += qr * x[it].z; pq.w += qr * x[it].w;
                float4 y;
                y.x = g2 * x[it].x + gk * r_0;
                y.y = g2 * x[it].y + gk * r_1;
                y.z = g2 * x[it].z + gk * r_2;
                y.w = g2 * x[it].w + gk * r_3;
                *reinterpret_cast<float4 *>(G + r * DV + c4 * 4) = y;
            }
        }
        reduce_cols<DV>(pq, red, qgs);
    }
    // output
    if (tid < DV) {
        const float aq = scal[1], qk = scal[2], dn = scal[3];
        const float num = g * acs[tid] + aq * vs[tid] - g2 * qgs[tid] - g * qk * rs[tid];
        a.out[static_cast<size_t>(b) * DV + tid] = a.normalize ? num / dn : num;
    }
    if (tid == 0) {
        if (a.den) a.den[b] = scal[3];
        if (a.st.rho) a.st.rho[b] *= g;
    }
}

template <typename T, int D>
hipError_t pick_dv(const DecArgs &a, int N, hipStream_t st) {
    switch (a.dv) {
        case 16: hipLaunchKernelGGL((k_decode<T, D, 16>), dim3(N), dim3(kThreads), 0, st, a); break;
        case 32: hipLaunchKernelGGL((k_decode<T, D, 32>), dim3(N), dim3(kThreads), 0, st, a); break;
        case 64: hipLaunchKernelGGL((k_decode<T, D, 64>), dim3(N), dim3(kThreads), 0, st, a); break;
        case 128: hipLaunchKernelGGL((k_decode<T, D, 128>), dim3(N), dim3(kThreads), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t pick_d(const DecArgs &a, int N, hipStream_t st) {
    switch (a.d) {
        case 16: return pick_dv<T, 16>(a, N, st);
        case 32: return pick_dv<T, 32>(a, N, st);
        case 64: return pick_dv<T, 64>(a, N, st);
        case 128: return pick_dv<T, 128>(a, N, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t decode_step(const DecodeProblem &p, hipStream_t st) {
    DecArgs a{};
    a.H = p.H; a.d = p.d; a.dv = p.dv; a.ridge = p.ridge; a.normalize = p.normalize;
    a.q = p.q; a.k = p.k; a.v = p.v; a.st = p.st; a.out = p.out; a.den = p.den; a.gam = p.gam;
    const int N = p.B * p.H;
    if (p.dtype == HLA_BF16) return pick_d<uint16_t>(a, N, st);
    return pick_d<float>(a, N, st);
}

}  // namespace hla
