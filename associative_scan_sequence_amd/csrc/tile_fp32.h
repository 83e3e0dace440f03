// tile_fp32.h -- fp32 products of chunk tiles for the generic (any-width)
// kernels, formed from LDS by a workgroup of 256 threads.
//
// Operands are staged in k-blocks of KB, transposed ([k][row], rows padded
// by 4 floats, sized to the largest row count the kernel stages); every thread owns a contiguous block of output rows (RM per
// thread, rows RM*ty ..) and columns (NC per thread, columns NC*tx ..), with
// ty = tid / 16 and tx = tid % 16, so its operand reads are 16-byte vectors.
// Operands are given as element functions (row, k) -> float; masks, decay
// factors and scales are folded into them.
#pragma once

#include <hip/hip_runtime.h>

namespace hla {
namespace tile {

constexpr int kThreads = 256;
constexpr int kMaxW = 128;  // largest row count of a staged operand
constexpr int KB = 32;

// ROWS: the largest row (or column) count a kernel stages
template <int ROWS>
struct alignas(16) Stage {
    float a[KB][ROWS + 4];
    float b[KB][ROWS + 4];
};

constexpr int max3(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }

template <int N>
__device__ __forceinline__ void read_vec(const float *p, float (&v)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const float4 x = *reinterpret_cast<const float4 *>(p + i);
            v[i] = x.x; v[i + 1] = x.y; v[i + 2] = x.z; v[i + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = p[i];
    }
}

// buf[t][s] (row stride BW) = fin(t, s, sum_{l<K} A(t, l) B(s, l)) for t, s < L;
// thread (ty, tx) forms rows RT*ty .. and columns RT*tx .. (RT*16 >= L).
template <int RT, int K, int SR, typename FA, typename FB, typename FF>
__device__ __forceinline__ void gram(float *buf, int BW, int L, Stage<SR> &st, FA A, FB B, FF fin) {
    const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    float acc[RT][RT] = {};
    for (int l0 = 0; l0 < K; l0 += KB) {
        for (int idx = tid; idx < L * KB; idx += kThreads) {  // k fastest: row-major operands
            const int row = idx / KB, kk = idx % KB;
            const bool in = l0 + kk < K;
            st.a[kk][row] = in ? A(row, l0 + kk) : 0.0f;
            st.b[kk][row] = in ? B(row, l0 + kk) : 0.0f;
        }
        __syncthreads();
        if (RT * ty < L && RT * tx < L) {
#pragma unroll 4
            for (int kk = 0; kk < KB; ++kk) {
                float av[RT], bv[RT];
                read_vec<RT>(&st.a[kk][RT * ty], av);
                read_vec<RT>(&st.b[kk][RT * tx], bv);
#pragma unroll
                for (int i = 0; i < RT; ++i)
#pragma unroll
                    for (int j = 0; j < RT; ++j) acc[i][j] += av[i] * bv[j];
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            const int t = RT * ty + i, s = RT * tx + j;
            if (t < L && s < L) buf[t * BW + s] = fin(t, s, acc[i][j]);
        }
}

// acc[i][j] += sum_{k<K} M(r_i, k) X(k, c_j) for rows r_i = RM*ty + i < nrows and
// columns c_j = NC*tx + j (16*NC columns).  ROWFAST stages M with the row index
// fastest (for M read as a transpose, M(r, k) = P[k][r]); else k fastest.
template <int RM, int NC, bool ROWFAST, int SR, typename FM, typename FX>
__device__ __forceinline__ void mm(float (&acc)[RM][NC], int nrows, int K, Stage<SR> &st, FM M, FX X) {
    constexpr int NCOL = 16 * NC;
    const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    for (int k0 = 0; k0 < K; k0 += KB) {
        if constexpr (ROWFAST) {
            for (int idx = tid; idx < nrows * KB; idx += kThreads) {
                const int row = idx % nrows, kk = idx / nrows;
                st.a[kk][row] = k0 + kk < K ? M(row, k0 + kk) : 0.0f;
            }
        } else {
            for (int idx = tid; idx < nrows * KB; idx += kThreads) {
                const int row = idx / KB, kk = idx % KB;
                st.a[kk][row] = k0 + kk < K ? M(row, k0 + kk) : 0.0f;
            }
        }
        for (int idx = tid; idx < KB * NCOL; idx += kThreads) {
            const int kk = idx / NCOL, col = idx % NCOL;
            st.b[kk][col] = k0 + kk < K ? X(k0 + kk, col) : 0.0f;
        }
        __syncthreads();
        if (RM * ty < nrows) {
#pragma unroll 4
            for (int kk = 0; kk < KB; ++kk) {
                float av[RM], xv[NC];
                read_vec<RM>(&st.a[kk][RM * ty], av);
                read_vec<NC>(&st.b[kk][NC * tx], xv);
#pragma unroll
                for (int i = 0; i < RM; ++i)
#pragma unroll
                    for (int j = 0; j < NC; ++j) acc[i][j] += av[i] * xv[j];
            }
        }
        __syncthreads();
    }
}

// dst[r][c] = acc for the rows and columns the thread owns in mm's layout
template <int RM, int NC>
__device__ __forceinline__ void store_tile(float *dst, int nrows, int width, const float (&acc)[RM][NC]) {
    const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
#pragma unroll
    for (int i = 0; i < RM; ++i) {
        const int r = RM * ty + i;
        if (r < nrows) {
#pragma unroll
            for (int j = 0; j < NC; ++j) dst[static_cast<size_t>(r) * width + NC * tx + j] = acc[i][j];
        }
    }
}

// fin(r, sum_{i<N} f(r, i)) for rows r < R, by all threads of the workgroup:
// four lanes per row, each summing every fourth term, then two shuffles (a
// fixed order, so the result is deterministic).  fin runs on one lane per row.
template <typename F, typename FIN>
__device__ __forceinline__ void row_sums(int R, int N, F f, FIN fin) {
    const int tid = threadIdx.x, part = tid & 3;
    for (int r0 = 0; r0 < R; r0 += kThreads / 4) {
        const int r = r0 + (tid >> 2);
        float s = 0.0f;
        if (r < R)
            for (int i = part; i < N; i += 4) s += f(r, i);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        if (r < R && part == 0) fin(r, s);
    }
}

}  // namespace tile
}  // namespace hla
