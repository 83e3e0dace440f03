// decode_mq.hip -- the streaming decode step with a packed, shared key moment.
//
// Higher-order Linear Attention, paperlayer.ai summary sec. 5.2: sharing the
// key moment across the query heads of a group reduces the state from
// O(h d^2) to O(d^2 + h d dv), and packed symmetric storage of S further cuts
// bandwidth.  The key moment S = sum k k^T depends on the keys only, so query
// heads that share keys (and values: grouped / multi-query attention, one
// k, v per kv head) share one S; C, m, G, h stay per query head.  The step
// is the one of decode.hip (same update and output, per query head), with S
// read from the packed triangle.
//
// Packed layout of a d x d symmetric S (d = 32, 64, 128), d(d+1)/2 floats:
// the 32 x 32 tiles (I, J), I <= J, in row-major tile order; an
// off-diagonal tile is stored whole (1024 floats, row-major), a diagonal
// tile as its upper triangle (528 floats, row r holding columns r..31).
//
// Kernels:
//   k_decode_mq  one workgroup of 256 threads per query head: reads the
//                group's packed S_{t-1}, forms a = (g S_{t-1} + k k^T + lambda I) q,
//                streams C and G (read once, written once), writes m, h, out,
//                den.  With one query head per group it also writes S_t
//                (so S is read once and written once).
//   k_update_s   (groups of several heads) one workgroup per group, after every
//                head has read S_{t-1}: S_t = g S_{t-1} + k k^T in place; rho *= g.
#include "device_common.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kThreads = 256;
constexpr int TS = 32;                   // tile side
constexpr int kDiag = TS * (TS + 1) / 2;  // 528 floats per diagonal tile

struct MqArgs {
    int H, R, d, dv;  // query heads, query heads per group
    float ridge;
    int normalize;
    const void *q, *k, *v;
    hla_mq_state st;
    float *out, *den;
    GammaTab gam;
};

__host__ __device__ constexpr int tile_offset(int NT, int I, int J) {
    // tiles before row I of tiles, then within row I
    int off = 0;
    for (int i = 0; i < I; ++i) off += kDiag + (NT - 1 - i) * TS * TS;
    return off + (J == I ? 0 : kDiag + (J - I - 1) * TS * TS);
}

// (r, c), c >= r, of element e of a packed diagonal tile
__device__ __forceinline__ void diag_rc(int e, int &r, int &c) {
    // row r starts at r*TS - r(r-1)/2; invert, then correct by one either way
    int rr = static_cast<int>((2.0f * TS + 1.0f - sqrtf((2.0f * TS + 1.0f) * (2.0f * TS + 1.0f) - 8.0f * e)) * 0.5f);
    rr = rr < 0 ? 0 : (rr > TS - 1 ? TS - 1 : rr);
    if (rr + 1 < TS && (rr + 1) * TS - (rr + 1) * rr / 2 <= e) ++rr;
    if (rr * TS - rr * (rr - 1) / 2 > e) --rr;
    r = rr;
    c = rr + (e - (rr * TS - rr * (rr - 1) / 2));
}

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

// The query head a workgroup serves.  Workgroups are dealt round-robin to the
// eight XCDs (index mod 8), so the heads of a group are placed on one XCD,
// where its L2 serves the group's packed S to all of them (needs the number
// of groups to be a multiple of 8; otherwise the plain order).
__device__ __forceinline__ int head_of_block(int N, int R) {
    const int i = static_cast<int>(blockIdx.x);
    const int groups = N / R;
    if (R == 1 || groups % 8 != 0) return i;
    const int x = i % 8, j = i / 8;
    return (x + 8 * (j / R)) * R + j % R;
}

template <typename T, int D, int DV, bool WRITE_S>
__global__ __launch_bounds__(kThreads) void k_decode_mq(MqArgs a) {
    constexpr int NT = D / TS;
    __shared__ float qs[D], ks[D], ms[D], hs[D], as[D], vs[DV];
    __shared__ float rs[DV], acs[DV], qgs[DV];
    __shared__ float red[2 * 1024];
    __shared__ float dt[NT][TS * (TS + 1)];  // diagonal tiles expanded to full (updated values)
    __shared__ float scal[4];
    const int N = gridDim.x;
    const int b = head_of_block(N, a.R);  // query-head state index
    const int grp = b / a.R;              // kv-group index (= index of k, v, S)
    const float g = head_gamma(a.gam, b % a.H), g2 = g * g, lam = a.ridge;
    const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
    float *S = a.st.S + static_cast<size_t>(grp) * (D * (D + 1) / 2);
    float *C = a.st.C + static_cast<size_t>(b) * D * DV;
    float *G = a.st.G + static_cast<size_t>(b) * D * DV;
    float *m = a.st.m + static_cast<size_t>(b) * D;
    float *h = a.st.h + static_cast<size_t>(b) * D;
    if (tid < D) {
        qs[tid] = Elem<T>::get(static_cast<const T *>(a.q), static_cast<size_t>(b) * D + tid);
        ks[tid] = Elem<T>::get(static_cast<const T *>(a.k), static_cast<size_t>(grp) * D + tid);
        ms[tid] = m[tid];
        hs[tid] = h[tid];
    }
    if (tid < DV) vs[tid] = Elem<T>::get(static_cast<const T *>(a.v), static_cast<size_t>(grp) * DV + tid);
    __syncthreads();

    // ---- pass 1: a = S_t q with S_t = g S_{t-1} + k k^T (+ lambda q)
    // Off-diagonal tiles (I < J): thread (row, c4) = (tid / 8, tid % 8) holds
    // elements (row, 4 c4 .. +3); column sums give a[32J + col], row sums (the
    // mirrored tile) a[32I + row].  Diagonal tiles: expanded into LDS from the
    // packed triangle, then column sums over the full tile.
    const int row = tid >> 3, c4 = tid & 7;
    float4 accc[NT];
    float accr[NT];
#pragma unroll
    for (int J = 0; J < NT; ++J) {
        accc[J] = make_float4(0.f, 0.f, 0.f, 0.f);
        accr[J] = 0.0f;
    }
    // diagonal tiles: packed elements -> updated values -> both halves of the LDS tile
#pragma unroll
    for (int I = 0; I < NT; ++I) {
        float *P = S + tile_offset(NT, I, I);
        for (int e = tid; e < kDiag; e += kThreads) {
            int r, c;
            diag_rc(e, r, c);
            const float y = g * P[e] + ks[TS * I + r] * ks[TS * I + c];
            if (WRITE_S) P[e] = y;
            dt[I][r * (TS + 1) + c] = y;
            dt[I][c * (TS + 1) + r] = y;
        }
    }
    // off-diagonal tiles: float4 rows
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int J = I + 1; J < NT; ++J) {
            float *P = S + tile_offset(NT, I, J);
            const float4 x = *reinterpret_cast<const float4 *>(P + row * TS + c4 * 4);
            const float kr = ks[TS * I + row], qr = qs[TS * I + row];
            const int cb = TS * J + c4 * 4;
            float4 y;
            y.x = g * x.x + kr * ks[cb];
            y.y = g * x.y + kr * ks[cb + 1];
            y.z = g * x.z + kr * ks[cb + 2];
            y.w = g * x.w + kr * ks[cb + 3];
            if (WRITE_S) *reinterpret_cast<float4 *>(P + row * TS + c4 * 4) = y;
            accc[J].x += y.x * qr; accc[J].y += y.y * qr; accc[J].z += y.z * qr; accc[J].w += y.w * qr;
            accr[I] += (y.x * qs[cb] + y.y * qs[cb + 1]) + (y.z * qs[cb + 2] + y.w * qs[cb + 3]);
        }
    __syncthreads();  // diagonal tiles expanded
#pragma unroll
    for (int J = 0; J < NT; ++J) {
        const float qr = qs[TS * J + row];
        const float *t = dt[J] + row * (TS + 1) + c4 * 4;
        accc[J].x += t[0] * qr; accc[J].y += t[1] * qr; accc[J].z += t[2] * qr; accc[J].w += t[3] * qr;
    }
    // column sums over the 8 rows of a wave (lanes 8 apart), then the 4 waves;
    // row sums over the 8 lanes of a row
#pragma unroll
    for (int J = 0; J < NT; ++J) {
#pragma unroll
        for (int sh = 8; sh < 64; sh <<= 1) {
            accc[J].x += __shfl_xor(accc[J].x, sh, 64);
            accc[J].y += __shfl_xor(accc[J].y, sh, 64);
            accc[J].z += __shfl_xor(accc[J].z, sh, 64);
            accc[J].w += __shfl_xor(accc[J].w, sh, 64);
        }
#pragma unroll
        for (int sh = 1; sh < 8; sh <<= 1) accr[J] += __shfl_xor(accr[J], sh, 64);
    }
    if (lane < 8) {
#pragma unroll
        for (int J = 0; J < NT; ++J) {
            float *cs = red + (wv * NT + J) * TS + c4 * 4;
            cs[0] = accc[J].x; cs[1] = accc[J].y; cs[2] = accc[J].z; cs[3] = accc[J].w;
        }
    }
    if (c4 == 0) {
#pragma unroll
        for (int I = 0; I < NT; ++I) red[1024 + TS * I + row] = accr[I];
    }
    __syncthreads();
    if (tid < D) {
        const int J = tid / TS, col = tid % TS;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) sum += red[(w * NT + J) * TS + col];
        as[tid] = sum + (J < NT - 1 ? red[1024 + tid] : 0.0f) + lam * qs[tid];
    }
    __syncthreads();

    // ---- scalars: s = k . m_{t-1}, a . q, q . k
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
    // ---- pass 2: r = k^T C_{t-1}, aC = a^T C_{t-1}; C_t = g C + q v^T
    {
        constexpr int LPR = DV / 4, RPI = kThreads / LPR, IT = (D + RPI - 1) / RPI;
        const int cc = tid % LPR, r0 = tid / LPR;
        const float v0 = vs[cc * 4], v1 = vs[cc * 4 + 1], v2 = vs[cc * 4 + 2], v3 = vs[cc * 4 + 3];
        float4 pr = make_float4(0.f, 0.f, 0.f, 0.f), pa = pr;
        float4 x[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int r = r0 + it * RPI;
            if (r < D) x[it] = *reinterpret_cast<const float4 *>(C + r * DV + cc * 4);
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
                *reinterpret_cast<float4 *>(C + r * DV + cc * 4) = y;
            }
        }
        reduce_cols<DV>(pr, red, rs);
        reduce_cols<DV>(pa, red + 1024, acs);
    }
    // ---- pass 3: qG = q^T G_{t-1}; G_t = g^2 G + g k r^T
    {
        constexpr int LPR = DV / 4, RPI = kThreads / LPR, IT = (D + RPI - 1) / RPI;
        const int cc = tid % LPR, r0 = tid / LPR;
        const float r_0 = rs[cc * 4], r_1 = rs[cc * 4 + 1], r_2 = rs[cc * 4 + 2], r_3 = rs[cc * 4 + 3];
        float4 pq = make_float4(0.f, 0.f, 0.f, 0.f);
        float4 x[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int r = r0 + it * RPI;
            if (r < D) x[it] = *reinterpret_cast<const float4 *>(G + r * DV + cc * 4);
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
                *reinterpret_cast<float4 *>(G + r * DV + cc * 4) = y;
            }
        }
        reduce_cols<DV>(pq, red, qgs);
    }
    if (tid < DV) {
        const float aq = scal[1], qk = scal[2], dn = scal[3];
        const float num = g * acs[tid] + aq * vs[tid] - g2 * qgs[tid] - g * qk * rs[tid];
        a.out[static_cast<size_t>(b) * DV + tid] = a.normalize ? num / dn : num;
    }
    if (tid == 0) {
        if (a.den) a.den[b] = scal[3];
        if (WRITE_S && a.st.rho) a.st.rho[grp] *= g;
    }
}

// S_t = g S_{t-1} + k k^T on a group's packed S, in place; rho *= g
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_update_s(MqArgs a) {
    constexpr int NT = D / TS;
    __shared__ float ks[D];
    const int grp = blockIdx.x, tid = threadIdx.x;
    const float g = head_gamma(a.gam, (grp * a.R) % a.H);
    if (tid < D) ks[tid] = Elem<T>::get(static_cast<const T *>(a.k), static_cast<size_t>(grp) * D + tid);
    __syncthreads();
    float *S = a.st.S + static_cast<size_t>(grp) * (D * (D + 1) / 2);
#pragma unroll
    for (int I = 0; I < NT; ++I) {
        float *P = S + tile_offset(NT, I, I);
        for (int e = tid; e < kDiag; e += kThreads) {
            int r, c;
            diag_rc(e, r, c);
            P[e] = g * P[e] + ks[TS * I + r] * ks[TS * I + c];
        }
#pragma unroll
        for (int J = I + 1; J < NT; ++J) {
            float *Q = S + tile_offset(NT, I, J);
            const int r = tid >> 3, c4 = tid & 7;
            float4 x = *reinterpret_cast<const float4 *>(Q + r * TS + c4 * 4);
            const float kr = ks[TS * I + r];
            const int cb = TS * J + c4 * 4;
            x.x = g * x.x + kr * ks[cb];
            x.y = g * x.y + kr * ks[cb + 1];
            x.z = g * x.z + kr * ks[cb + 2];
            x.w = g * x.w + kr * ks[cb + 3];
            *reinterpret_cast<float4 *>(Q + r * TS + c4 * 4) = x;
        }
    }
    if (tid == 0 && a.st.rho) a.st.rho[grp] *= g;
}

// full <-> packed (count matrices); one workgroup per matrix
template <int D, bool PACK>
__global__ __launch_bounds__(kThreads) void k_pack(const float *src, float *dst) {
    constexpr int NT = D / TS;
    const size_t i = blockIdx.x;
    const float *full_in = src + i * D * D;
    const float *pk_in = src + i * (D * (D + 1) / 2);
    float *pk_out = dst + i * (D * (D + 1) / 2);
    float *full_out = dst + i * D * D;
    const int tid = threadIdx.x;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int J = I; J < NT; ++J) {
            const int off = tile_offset(NT, I, J);
            const int cnt = I == J ? kDiag : TS * TS;
            for (int e = tid; e < cnt; e += kThreads) {
                int r, c;
                if (I == J) diag_rc(e, r, c);
                else r = e / TS, c = e % TS;
                const int gr = TS * I + r, gc = TS * J + c;
                if (PACK) {
                    pk_out[off + e] = full_in[gr * D + gc];
                } else {
                    const float x = pk_in[off + e];
                    full_out[gr * D + gc] = x;
                    full_out[gc * D + gr] = x;
                }
            }
        }
}

template <typename T, int D>
hipError_t pick_dv(const MqArgs &a, int N, int groups, hipStream_t st) {
#define HLA_MQ_LAUNCH(DV)                                                                          \
    if (a.R == 1) hipLaunchKernelGGL((k_decode_mq<T, D, DV, true>), dim3(N), dim3(kThreads), 0, st, a); \
    else hipLaunchKernelGGL((k_decode_mq<T, D, DV, false>), dim3(N), dim3(kThreads), 0, st, a);
    switch (a.dv) {
        case 16: HLA_MQ_LAUNCH(16) break;
        case 32: HLA_MQ_LAUNCH(32) break;
        case 64: HLA_MQ_LAUNCH(64) break;
        case 128: HLA_MQ_LAUNCH(128) break;
        default: return hipErrorInvalidValue;
    }
#undef HLA_MQ_LAUNCH
    if (a.R > 1) hipLaunchKernelGGL((k_update_s<T, D>), dim3(groups), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t pick_d(const MqArgs &a, int N, int groups, hipStream_t st) {
    switch (a.d) {
        case 32: return pick_dv<T, 32>(a, N, groups, st);
        case 64: return pick_dv<T, 64>(a, N, groups, st);
        case 128: return pick_dv<T, 128>(a, N, groups, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t decode_step_mq(const DecodeMqProblem &p, hipStream_t st) {
    MqArgs a{};
    a.H = p.H; a.R = p.H / p.kv_heads; a.d = p.d; a.dv = p.dv; a.ridge = p.ridge; a.normalize = p.normalize;
    a.q = p.q; a.k = p.k; a.v = p.v; a.st = p.st; a.out = p.out; a.den = p.den; a.gam = p.gam;
    const int N = p.B * p.H, groups = p.B * p.kv_heads;
    if (p.dtype == HLA_BF16) return pick_d<uint16_t>(a, N, groups, st);
    return pick_d<float>(a, N, groups, st);
}

hipError_t key_moment_pack(int count, int d, const float *src, float *dst, bool pack, hipStream_t st) {
    if (count == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(count)), blk(kThreads);
    if (d == 32) {
        if (pack) hipLaunchKernelGGL((k_pack<32, true>), grid, blk, 0, st, src, dst);
        else hipLaunchKernelGGL((k_pack<32, false>), grid, blk, 0, st, src, dst);
    } else if (d == 64) {
        if (pack) hipLaunchKernelGGL((k_pack<64, true>), grid, blk, 0, st, src, dst);
        else hipLaunchKernelGGL((k_pack<64, false>), grid, blk, 0, st, src, dst);
    } else if (d == 128) {
        if (pack) hipLaunchKernelGGL((k_pack<128, true>), grid, blk, 0, st, src, dst);
        else hipLaunchKernelGGL((k_pack<128, false>), grid, blk, 0, st, src, dst);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hla
