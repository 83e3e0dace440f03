// fwd_small.hip -- the masked second-order forward of short sequences
// (n <= 256, d and dv in {16, 32}) as two causal first-order maps, with no
// chunks and no carries.
//
// Higher-order Linear Attention, paperlayer.ai summary sec. 3.1 (the mask
// keeps j <= t) and sec. 4.3 (a fixed decay attenuates each step): the masked
// numerator q_t^T (S_t C_t - G_t) keeps, of all pairs of the key moment and
// the query-value moment, those whose key comes no later than its query:
// it is the sum of (q_t . k_i)(k_i . q_j) v_j over i <= j <= t, each term
// decayed by g^(2t - i - j).  Summing over i first gives two maps of the form
//   LA(A, B, C; r)_t = sum over s <= t of r^(t - s) (a_t . b_s) c_s:
//   U   = LA(Q, K, K; g)       (row j is S_j q_j),
//   out = LA(Q, U, V; g^2).
// The identity is checked in fp64 against the serial oracle on the CPU
// (tests/test_small_path_algebra.py).
//
// One workgroup of 256 threads forms a map's rows for 8 consecutive tokens
// of one head.  Thread (token tau = tid / 32, lane l = tid % 32) sums the
// terms s = l, l + 32, ... (s <= t) over LDS-staged rows of B and C, two
// rows per step; the 32 lanes of a token then add their partial sums across
// lanes.  A workgroup stages only the rows up to its last token.  At these lengths a launch is
// bound by latency (one staging pass, one summing pass, one reduction), not
// by its O(n^2 (d + dv)) fp32 FMA work.  Two launches: U (fp32) into the
// workspace, then the output.
#include "device_common.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kTok = 8;     // tokens per workgroup
constexpr int kLanes = 32;  // lanes per token
constexpr int kSmallMaxN = 256;

typedef uint32_t w4 __attribute__((ext_vector_type(4)));

// Staging of rows [0, rows) of a [n][D] row-major operand: 16-byte loads,
// at most kLoads per thread, all issued before the first LDS store.
template <typename T, int D>
struct Rows {
    static constexpr int kVec = 16 / static_cast<int>(sizeof(T));  // elements per load (D is a multiple)
    static constexpr int kLoads = kSmallMaxN * D / kVec / 256;
    w4 raw[kLoads];

    __device__ __forceinline__ void load(const T *src, int rows) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int e0 = (i * 256 + static_cast<int>(threadIdx.x)) * kVec;
            raw[i] = e0 < rows * D ? *reinterpret_cast<const w4 *>(src + e0) : w4{0u, 0u, 0u, 0u};
        }
    }
    // widened to fp32, into LDS rows of stride D + 4: 16-byte aligned, and
    // the consecutive rows that 16 consecutive lanes read with 16-byte loads
    // (lane l reads row l + 64 i) cover the 64 banks once (D = 16: rows 80
    // bytes apart; D = 32: 144)
    __device__ __forceinline__ void store(int rows, float *dst) const {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int e0 = (i * 256 + static_cast<int>(threadIdx.x)) * kVec;
            if (e0 >= rows * D) continue;
            const int r = e0 / D, c = e0 - r * D;
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                float x;
                if constexpr (sizeof(T) == 4) {
                    x = __uint_as_float(raw[i][e]);
                } else {  // bf16 -> fp32 is exact: the bits are the top half of the word
                    const uint32_t w = raw[i][e >> 1];
                    x = __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
                }
                dst[r * (D + 4) + c + e] = x;
            }
        }
    }
};

// y[t] = sum over s <= t of r^(t-s) (a_t . b_s) c_s for the 8 tokens of
// block blockIdx.y of head blockIdx.x; r = g^rexp.  a, b: [BH][n][DA];
// c: [BH][n][DC]; y: [BH][n][DC] fp32.
template <typename TA, typename TB, typename TC, int DA, int DC>
__global__ __launch_bounds__(256) void k_small_map(const TA *a, const TB *b, const TC *c, int n, int H,
                                                   GammaTab gam, float rexp, float *y) {
    __shared__ __align__(16) float sb[kSmallMaxN * (DA + 4)];
    __shared__ __align__(16) float sc[kSmallMaxN * (DC + 4)];
    const int bh = blockIdx.x, t0 = blockIdx.y * kTok;
    const int rows = min(n, t0 + kTok);
    const size_t head = static_cast<size_t>(bh) * n;
    Rows<TB, DA> rb;
    Rows<TC, DC> rc;
    rb.load(b + head * DA, rows);
    rc.load(c + head * DC, rows);
    const int tau = threadIdx.x / kLanes, l = threadIdx.x % kLanes, t = t0 + tau;
    const bool live = t < n;
    float at[DA];
#pragma unroll
    for (int k = 0; k < DA; ++k) at[k] = live ? Elem<TA>::get(a, (head + t) * DA + k) : 0.0f;
    // log2 of the decay per step (-inf for g = 0, whose zeroth power is taken as 1 below)
    const float lr = rexp * log2f(head_gamma(gam, bh % H));
    rb.store(rows, sb);
    rc.store(rows, sc);
    float acc[DC];
#pragma unroll
    for (int j = 0; j < DC; ++j) acc[j] = 0.0f;
    __syncthreads();
    if (live) {
        // two rows per step (s and s + 32, the second weighted 0 past t), each
        // dot product in four partial sums: independent chains to overlap
        for (int s = l; s <= t; s += 2 * kLanes) {
            const int s2 = s + kLanes <= t ? s + kLanes : s;
            const float4 *br = reinterpret_cast<const float4 *>(sb + s * (DA + 4));
            const float4 *br2 = reinterpret_cast<const float4 *>(sb + s2 * (DA + 4));
            float p[4] = {0.0f, 0.0f, 0.0f, 0.0f}, p2[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k4 = 0; k4 < DA / 4; ++k4) {
                const float4 x = br[k4], x2 = br2[k4];
                const float *a4 = at + 4 * k4;
                p[0] = fmaf(a4[0], x.x, p[0]); p[1] = fmaf(a4[1], x.y, p[1]);
                p[2] = fmaf(a4[2], x.z, p[2]); p[3] = fmaf(a4[3], x.w, p[3]);
                p2[0] = fmaf(a4[0], x2.x, p2[0]); p2[1] = fmaf(a4[1], x2.y, p2[1]);
                p2[2] = fmaf(a4[2], x2.z, p2[2]); p2[3] = fmaf(a4[3], x2.w, p2[3]);
            }
            float w = (p[0] + p[1]) + (p[2] + p[3]);
            float w2 = s2 != s ? (p2[0] + p2[1]) + (p2[2] + p2[3]) : 0.0f;
            if (lr != 0.0f) {
                const int e = t - s, e2 = t - s2;
                if (e != 0) w *= exp2f(static_cast<float>(e) * lr);
                if (e2 != 0) w2 *= exp2f(static_cast<float>(e2) * lr);
            }
            const float4 *cr = reinterpret_cast<const float4 *>(sc + s * (DC + 4));
            const float4 *cr2 = reinterpret_cast<const float4 *>(sc + s2 * (DC + 4));
#pragma unroll
            for (int j4 = 0; j4 < DC / 4; ++j4) {
                const float4 x = cr[j4], x2 = cr2[j4];
                float *c4 = acc + 4 * j4;
                c4[0] = fmaf(w2, x2.x, fmaf(w, x.x, c4[0])); c4[1] = fmaf(w2, x2.y, fmaf(w, x.y, c4[1]));
                c4[2] = fmaf(w2, x2.z, fmaf(w, x.z, c4[2])); c4[3] = fmaf(w2, x2.w, fmaf(w, x.w, c4[3]));
            }
        }
    }
    // the token's 32 lanes are 32 consecutive lanes of one wave
#pragma unroll
    for (int j = 0; j < DC; ++j) {
#pragma unroll
        for (int off = kLanes / 2; off >= 1; off >>= 1) acc[j] += __shfl_xor(acc[j], off, kLanes);
    }
    if (!live) return;
    float *yr = y + (head + t) * DC;
#pragma unroll
    for (int j = 0; j < DC; ++j)
        if (j % kLanes == l) yr[j] = acc[j];
}

template <typename T, int D, int DV>
hipError_t small_launch(const FwdProblem &p, float *u, hipStream_t st) {
    const int BH = p.B * p.H;
    const dim3 grid(static_cast<unsigned>(BH), static_cast<unsigned>((p.n + kTok - 1) / kTok));
    const T *q = static_cast<const T *>(p.q), *k = static_cast<const T *>(p.k), *v = static_cast<const T *>(p.v);
    hipLaunchKernelGGL((k_small_map<T, T, T, D, D>), grid, dim3(256), 0, st, q, k, k, p.n, p.H, p.gam, 1.0f, u);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_small_map<T, float, T, D, DV>), grid, dim3(256), 0, st, q, static_cast<const float *>(u),
                       v, p.n, p.H, p.gam, 2.0f, p.out);
    return hipGetLastError();
}

template <typename T>
hipError_t small_dispatch(const FwdProblem &p, float *u, hipStream_t st) {
    if (p.d == 16 && p.dv == 16) return small_launch<T, 16, 16>(p, u, st);
    if (p.d == 16 && p.dv == 32) return small_launch<T, 16, 32>(p, u, st);
    if (p.d == 32 && p.dv == 16) return small_launch<T, 32, 16>(p, u, st);
    return small_launch<T, 32, 32>(p, u, st);
}

}  // namespace

bool small_supported(const FwdProblem &p) {
    const bool wd = (p.d == 16 || p.d == 32) && (p.dv == 16 || p.dv == 32);
    return wd && p.n > 0 && p.n <= kSmallMaxN && p.ridge == 0.0f && !p.normalize && p.den == nullptr &&
           p.init.S == nullptr && p.fin.S == nullptr && (p.dtype == HLA_F32 || p.dtype == HLA_BF16);
}

size_t small_data_bytes(int BH, int n, int d) {
    return (static_cast<size_t>(BH) * n * d * sizeof(float) + 255) & ~static_cast<size_t>(255);
}

hipError_t small_forward(const FwdProblem &p, void *data, hipStream_t st) {
    float *u = static_cast<float *>(data);
    return p.dtype == HLA_BF16 ? small_dispatch<uint16_t>(p, u, st) : small_dispatch<float>(p, u, st);
}

}  // namespace hla
