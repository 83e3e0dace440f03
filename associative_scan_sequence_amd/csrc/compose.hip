// compose.hip -- batched masked semidirect-product composition of segment
// summaries (Higher-order Linear Attention, paperlayer.ai summary sec. 4.2;
// gist.science explainer, "Assoziative Operatoren": the composition of two
// segments adds the cross term of the later segment's key moment with the
// earlier segment's query-value accumulator).  Earlier segment a, later b:
//   S = rho_b S_a + S_b      C = rho_b C_a + C_b      m = rho_b m_a + m_b
//   G = rho_b^2 G_a + G_b + rho_b S_b C_a
//   h = rho_b^2 h_a + h_b + rho_b S_b m_a           rho = rho_a rho_b
// One workgroup (four waves) per pair.  The d x d x dv product enters G as
// G^T = C_a^T S_b^T on fp32 MFMA (v_mfma_f32_16x16x4_f32: fp32 products,
// fp32 accumulation, as exact as the plain fp32 sum).  C_a is staged in LDS
// with rows padded to dv + 4 floats, so the four lane groups of an operand
// read (rows 4 apart) fall on disjoint banks; S_b is read from memory once,
// in operand layout, and the S result is formed from the same reads.  Every
// input is read once and every output written once, so the kernel is bound
// by HBM bandwidth (the product is ~4 MFLOP per pair at d = dv = 128).
#include "device_common.h"
#include "hla_internal.h"

namespace hla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ void st4(float *p, const f32x4 &v) { *reinterpret_cast<f32x4 *>(p) = v; }

template <int D, int DV>
__global__ __launch_bounds__(kThreads) void k_compose(hla_state a, hla_state b, hla_state r) {
    constexpr int LDC = DV + 4;                  // padded C_a row, floats
    constexpr int NIB = D / 16, NJB = DV / 16;   // 16-row blocks of S_b, 16-column blocks of C_a
    constexpr int IBW = (NIB + 3) / 4;           // S_b row blocks per wave: wave + 4t
    __shared__ float ca[D * LDC];
    __shared__ float mas[D];
    const int p = blockIdx.x, tid = threadIdx.x;
    const int wave = tid >> 6, l = tid & 63, rr = l & 15, g = l >> 4;
    const size_t oS = static_cast<size_t>(p) * D * D, oC = static_cast<size_t>(p) * D * DV;
    const size_t om = static_cast<size_t>(p) * D;
    const float ra = a.rho ? a.rho[p] : 1.0f, rb = b.rho ? b.rho[p] : 1.0f;
    const float *Sa = a.S + oS, *Sb = b.S + oS;
    const float *Ca = a.C + oC, *Cb = b.C + oC, *Ga = a.G + oC, *Gb = b.G + oC;

    // ---- C = rho_b C_a + C_b, and C_a -> LDS (rows l, padded)
#pragma unroll 4
    for (int x = tid; x < D * DV / 4; x += kThreads) {
        const f32x4 c_a = ld4(Ca + 4 * x), c_b = ld4(Cb + 4 * x);
        st4(r.C + oC + 4 * x, rb * c_a + c_b);
        const int row = (4 * x) / DV, col = (4 * x) % DV;
        st4(&ca[row * LDC + col], c_a);
    }
    if (tid < D) {
        const float m_a = a.m[om + tid];
        mas[tid] = m_a;
        r.m[om + tid] = rb * m_a + b.m[om + tid];
    }
    __syncthreads();

    // ---- G^T tiles (rows j = 16jb + 4g + e, cols i = 16ib + rr) over k = l:
    // step s of block m pairs lane group g with l = 16m + 4g + s
    f32x4 acc[NJB][IBW];
    float hp[IBW];
#pragma unroll
    for (int t = 0; t < IBW; ++t) {
        hp[t] = 0.0f;
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) acc[jb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll 2
    for (int m = 0; m < D / 16; ++m) {
        const int l0 = 16 * m + 4 * g;
        f32x4 sb[IBW];
#pragma unroll
        for (int t = 0; t < IBW; ++t) {
            const int ib = wave + 4 * t;
            if (ib < NIB) {
                const int i = 16 * ib + rr;
                sb[t] = ld4(Sb + i * D + l0);
                const f32x4 s_a = ld4(Sa + i * D + l0);
                st4(r.S + oS + i * D + l0, rb * s_a + sb[t]);
                hp[t] += (sb[t][0] * mas[l0] + sb[t][1] * mas[l0 + 1]) + (sb[t][2] * mas[l0 + 2] + sb[t][3] * mas[l0 + 3]);
            }
        }
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const float cv = ca[(l0 + s4) * LDC + 16 * jb + rr];
#pragma unroll
                for (int t = 0; t < IBW; ++t)
                    if (wave + 4 * t < NIB) acc[jb][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(cv, sb[t][s4], acc[jb][t], 0, 0, 0);
            }
        }
    }

    // ---- G = rho_b^2 G_a + G_b + rho_b S_b C_a;  h = rho_b^2 h_a + h_b + rho_b S_b m_a
    const float rb2 = rb * rb;
#pragma unroll
    for (int t = 0; t < IBW; ++t) {
        const int ib = wave + 4 * t;
        if (ib < NIB) {
            const int i = 16 * ib + rr;
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const size_t o = static_cast<size_t>(i) * DV + 16 * jb + 4 * g;
                st4(r.G + oC + o, rb2 * ld4(Ga + o) + ld4(Gb + o) + rb * acc[jb][t]);
            }
            float x = hp[t];
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            if (g == 0) r.h[om + i] = rb2 * a.h[om + i] + b.h[om + i] + rb * x;
        }
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
