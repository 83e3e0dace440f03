// compose.hip -- batched masked semidirect-product composition of segment
// summaries (Higher-order Linear Attention, paperlayer.ai summary sec. 4.2;
// gist.science explainer, "Assoziative Operatoren": the composition of two
// segments adds the cross term of the later segment's key moment with the
// earlier segment's query-value accumulator).  Earlier segment a, later b:
//   S = rho_b S_a + S_b      C = rho_b C_a + C_b      m = rho_b m_a + m_b
//   G = rho_b^2 G_a + G_b + rho_b S_b C_a
//   h = rho_b^2 h_a + h_b + rho_b S_b m_a           rho = rho_a rho_b
// One workgroup per pair; the d x d x dv product S_b C_a is register-tiled
// (each thread owns a (d/16) x (dv/16) block of G) with S_b and C_a staged
// through LDS in slices of 16 along the contraction index.
#include "device_common.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kThreads = 256;

template <int D, int DV>
__global__ __launch_bounds__(kThreads) void k_compose(hla_state a, hla_state b, hla_state r) {
    constexpr int MR = D / 16, MC = DV / 16, KS = 16;
    __shared__ float sb[D][KS + 1], ca[KS][DV];
    __shared__ float mas[D];
    const int p = blockIdx.x, tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    const size_t oS = static_cast<size_t>(p) * D * D, oC = static_cast<size_t>(p) * D * DV;
    const size_t om = static_cast<size_t>(p) * D;
    const float ra = a.rho ? a.rho[p] : 1.0f, rb = b.rho ? b.rho[p] : 1.0f;
    const float *Sa = a.S + oS, *Sb = b.S + oS;
    const float *Ca = a.C + oC, *Cb = b.C + oC, *Ga = a.G + oC, *Gb = b.G + oC;
    for (int i = tid; i < D * D; i += kThreads) r.S[oS + i] = rb * Sa[i] + Sb[i];
    for (int i = tid; i < D * DV; i += kThreads) r.C[oC + i] = rb * Ca[i] + Cb[i];
    if (tid < D) {
        r.m[om + tid] = rb * a.m[om + tid] + b.m[om + tid];
        mas[tid] = a.m[om + tid];
    }
    float acc[MR][MC] = {};
    for (int l0 = 0; l0 < D; l0 += KS) {
        __syncthreads();
        for (int i = tid; i < D * KS; i += kThreads) sb[i / KS][i % KS] = Sb[(i / KS) * D + l0 + i % KS];
        for (int i = tid; i < KS * DV; i += kThreads) ca[i / DV][i % DV] = Ca[(l0 + i / DV) * DV + i % DV];
        __syncthreads();
#pragma unroll
        for (int l = 0; l < KS; ++l) {
            float sr[MR], cc[MC];
#pragma unroll
            for (int i = 0; i < MR; ++i) sr[i] = sb[ty + 16 * i][l];
#pragma unroll
            for (int j = 0; j < MC; ++j) cc[j] = ca[l][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < MR; ++i)
#pragma unroll
                for (int j = 0; j < MC; ++j) acc[i][j] += sr[i] * cc[j];
        }
    }
    const float rb2 = rb * rb;
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int j = 0; j < MC; ++j) {
            const size_t o = oC + (ty + 16 * i) * DV + tx + 16 * j;
            r.G[o] = rb2 * Ga[o - oC] + Gb[o - oC] + rb * acc[i][j];
        }
    __syncthreads();
    if (tid < D) {
        float x = 0.0f;
        for (int l = 0; l < D; ++l) x += Sb[tid * D + l] * mas[l];
        r.h[om + tid] = rb2 * a.h[om + tid] + b.h[om + tid] + rb * x;
    }
    if (tid == 0 && r.rho) r.rho[p] = ra * rb;
}

template <int D>
hipError_t pick_dv(int count, int dv, const hla_state &a, const hla_state &b, const hla_state &r,
                   hipStream_t st) {
    switch (dv) {
        case 16: hipLaunchKernelGGL((k_compose<D, 16>), dim3(count), dim3(kThreads), 0, st, a, b, r); break;
        case 32: hipLaunchKernelGGL((k_compose<D, 32>), dim3(count), dim3(kThreads), 0, st, a, b, r); break;
        case 64: hipLaunchKernelGGL((k_compose<D, 64>), dim3(count), dim3(kThreads), 0, st, a, b, r); break;
        case 128: hipLaunchKernelGGL((k_compose<D, 128>), dim3(count), dim3(kThreads), 0, st, a, b, r); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t state_compose(int count, int d, int dv, const hla_state &a, const hla_state &b,
                         const hla_state &r, hipStream_t st) {
    if (count == 0) return hipSuccess;
    switch (d) {
        case 16: return pick_dv<16>(count, dv, a, b, r, st);
        case 32: return pick_dv<32>(count, dv, a, b, r, st);
        case 64: return pick_dv<64>(count, dv, a, b, r, st);
        case 128: return pick_dv<128>(count, dv, a, b, r, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace hla
