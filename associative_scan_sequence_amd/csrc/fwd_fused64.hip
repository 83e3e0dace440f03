// fwd_fused64.hip -- one-launch masked second-order HLA forward for
// d = dv = 64, chunk w = 64, bf16 q/k/v, on gfx950 MFMA.
//
// Method (Higher-order Linear Attention, paperlayer.ai summary sec. 4 and 5):
// inside each chunk the token-level exclusive scan is evaluated as masked
// w x w products, and chunk summaries are scanned to give carry-ins.  The
// carry is held in the corrected form (S, X = S C - G), for which
//   X_t = g^2 X_{t-1} + S_t q_t v_t^T,   num_t = q_t^T X_t,
// so both S and X are *linear* scans once S is known (see fwd_generic.hip
// for the per-chunk formulas).  Per chunk (local token indices t, s):
//   A   = (Q K^T) o D_g o L                       masked scores
//   U   = diag(e) Q S0 + A K                      row s = S_s q_s
//   P   = (Q U^T) o D_{g^2} o L
//   num = P V + diag(e^2) Q X0
//   S0 <- g^w S0 + K^T diag(f) K,   X0 <- g^2w X0 + U^T diag(f^2) V
//
// Parallel structure.  One workgroup owns a segment of up to four
// consecutive chunks of one head and runs two groups of four waves; group 0
// walks the segment's first two chunks and group 1 the last two, at the same
// time, so every SIMD holds two waves that hide each other's latency.  Group
// 1 starts from the key moment and X increment that group 0 accumulates,
// handed over through LDS.  Three phases, two device-wide rounds:
//   A: the segment's own key moment sum S_seg (chunk recurrence from 0);
//      publish it.  Round 1: wait for every earlier segment of the head and
//      sum their decayed S_seg -> the segment's S carry.
//   B: walk the chunks with the true S carry and a local X starting at 0:
//      all masked products, the local part of num (kept in registers), and
//      the segment's X increment Z_seg; publish it.  Round 2: sum the
//      decayed Z_seg of every earlier segment -> the segment's X carry.
//   C: add diag(e^2 g^(2*offset)) Q X_start to num and store.
// Both rounds are plain decayed sums of published aggregates (no serial
// chain between segments).  Workgroups take logical ids from a ticket
// counter, so a workgroup only waits on workgroups that started before it.
//
// Precision.  q, k, v are exact in bf16.  Every operand formed in fp32 (A,
// U, P, S0, X0, and f-scaled K) is split as x = hi + lo with hi = bf16(x),
// lo = bf16(x - hi); each such product is two bf16 MFMAs with fp32
// accumulation, leaving ~2^-16 relative operand error.
//
// MFMA: v_mfma_f32_16x16x32_bf16.  Lane l = 16 g + r holds A-operand row r,
// k = 8g..8g+7; B-operand column r, k = 8g..8g+7; accumulator rows 4g..4g+3
// of column r.  Each wave owns a 16-token slice of its group's chunk (or a
// 16-row slice of S and X), so most operands stay wave-private.
#include "device_common.h"
#include "hla_internal.h"

namespace hla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int W = 64;        // chunk width = d = dv
constexpr int LDR = 72;      // padded LDS row, in bf16 elements (144 bytes)
constexpr int kThreads = 512;  // two groups of four waves
constexpr int kPerGroup = 2;   // chunks per wave group
constexpr int kMaxL = 4;       // chunks per workgroup
constexpr int kSpinLimit = 1 << 22;

struct FusedArgs {
    int H, n, nc, P, L, BH;
    const uint16_t *q, *k, *v;
    float *out;
    uint32_t *ctrl;   // [0] ticket, [1] done, [2] epoch, [3] wait-timeout count
    uint32_t *flag1, *flag2;  // [BH * P]
    float *aggS, *aggZ;       // [BH * P][4096], in accumulator-tile order
    GammaTab gam;
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const __bf16 *base, int row, int col) {
    return *reinterpret_cast<const bf16x8 *>(base + row * LDR + col);
}

// hi = bf16(x), lo = bf16(x - hi), 4 values
__device__ __forceinline__ void split4(const f32x4 &x, uint2 &hi, uint2 &lo) {
    typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
    bf4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = static_cast<__bf16>(x[i]);
        l[i] = static_cast<__bf16>(x[i] - static_cast<float>(h[i]));
    }
    hi = *reinterpret_cast<uint2 *>(&h);
    lo = *reinterpret_cast<uint2 *>(&l);
}

__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hi[i] = static_cast<__bf16>(x[i]);
        lo[i] = static_cast<__bf16>(x[i] - static_cast<float>(hi[i]));
    }
}

__device__ __forceinline__ void st4(__bf16 *base, int row, int col, uint2 v) {
    *reinterpret_cast<uint2 *>(base + row * LDR + col) = v;
}

__device__ __forceinline__ uint32_t next_epoch(uint32_t e) { return e * 1664525u + 1013904223u; }

// Cross-workgroup hand-off without cache maintenance: aggregates and flags
// are written and read with agent-scope relaxed atomics, which gfx950 issues
// as device-coherent (sc1) accesses, so no L2 write-back or invalidate is
// needed.  The writer waits for its stores to complete (vmcnt 0) before the
// workgroup barrier that precedes the flag store; readers poll the flag and
// only then load the aggregate.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ }

__device__ bool wait_flag(const uint32_t *f, uint32_t want) {
    for (int it = 0; it < kSpinLimit; ++it) {
        if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want) return true;
        __builtin_amdgcn_s_sleep(2);
    }
    return false;
}

// 16 floats of this thread's accumulator tiles, stored and loaded as 16-byte
// device-coherent (sc1) buffer accesses.  Each aggregate slot is 16 KB; the
// thread's 64 bytes sit at byte offset 64 * tid.
constexpr int kSc1 = 16;  // cache policy: sc1 (device scope)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const float *slot) {
    // slot addresses are uniform across the wave; say so, so the descriptor is scalar
    const uint64_t addr = reinterpret_cast<uint64_t>(slot);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(addr)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(addr >> 32)));
    float *base = reinterpret_cast<float *>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, 16384, 0x00020000);
}

__device__ __forceinline__ void put16(const float *slot, int tid, const f32x4 (&x)[4]) {
    const __amdgpu_buffer_rsrc_t rs = slot_rsrc(slot);
#pragma unroll
    for (int b = 0; b < 4; ++b) __builtin_amdgcn_raw_buffer_store_b128(x[b], rs, 64 * tid + 16 * b, 0, kSc1);
}

// acc += sum over n slots of scale[i] * slot_i (this thread's 16 floats);
// all loads of a batch are issued before the first add.
template <int NB>
__device__ __forceinline__ void add_slots(f32x4 (&acc)[4], const float *const (&slots)[NB],
                                          const float (&scale)[NB], int n, int tid) {
    f32x4 v[NB][4];
#pragma unroll
    for (int s = 0; s < NB; ++s)
        if (s < n) {
            const __amdgpu_buffer_rsrc_t rs = slot_rsrc(slots[s]);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                v[s][b] = __builtin_amdgcn_raw_buffer_load_b128(rs, 64 * tid + 16 * b, 0, kSc1);
        }
#pragma unroll
    for (int s = 0; s < NB; ++s)
        if (s < n) {
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[b] += scale[s] * v[s][b];
        }
}

// LDS of one wave group: 8 padded 64 x 64 bf16 tiles (72 KB).
struct GroupLds {
    __bf16 KT[W * LDR];   // K^T [a][s]
    __bf16 VT[W * LDR];   // V^T [j][s]
    __bf16 APh[W * LDR];  // A then P, [t][s] (rows private to the owning wave)
    __bf16 APl[W * LDR];
    __bf16 Uh[W * LDR];   // staging: K rows (Uh) and V rows (Ul); then U [s][a]
    __bf16 Ul[W * LDR];
    __bf16 STh[W * LDR];  // S0 (symmetric, [a][b]) then X0^T ([j][a]) of the chunk
    __bf16 STl[W * LDR];
};

struct Smem {
    GroupLds grp[2];
    float pw[2 * W + 2];  // g^k, k = 0 .. 2W+1
    uint32_t misc[4];
};

__global__ __launch_bounds__(kThreads, 1) void k_fused64(FusedArgs a) {
    __shared__ Smem sm;
    const int tid = threadIdx.x, grp = tid >> 8, wt = tid & 255;
    const int w = wt >> 6, l = wt & 63, r = l & 15, g = l >> 4;
    GroupLds &G = sm.grp[grp];
    const int total = a.BH * a.P;

    // ---- logical workgroup id from the ticket counter, and the launch epoch
    if (tid == 0) {
        sm.misc[0] = __hip_atomic_fetch_add(&a.ctrl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.misc[1] = next_epoch(__hip_atomic_load(&a.ctrl[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    }
    __syncthreads();
    // wave-uniform (SGPR) copies, so slot addresses and buffer descriptors stay scalar
    const int ticket = __builtin_amdgcn_readfirstlane(static_cast<int>(sm.misc[0]));
    const uint32_t epoch = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sm.misc[1])));
    const int p = ticket / a.BH, bh = ticket % a.BH;
    const int c0 = p * a.L;
    const int Lseg = min(a.L, a.nc - c0);           // chunks in this segment (>= 1)
    const int jbase = kPerGroup * grp;               // first segment-local chunk of this group
    const int nmine = max(0, min(kPerGroup, Lseg - jbase));
    const float gam = head_gamma(a.gam, bh % a.H);
    const bool decay = gam != 1.0f;
    for (int i = tid; i < 2 * W + 2; i += kThreads) sm.pw[i] = gpow(gam, i);
    auto chunk_len = [&](int j) { return min(W, a.n - (c0 + j) * W); };
    int lenA = 0, lenB = 0;  // tokens covered by group 0 and group 1
    for (int j = 0; j < Lseg; ++j) (j < kPerGroup ? lenA : lenB) += chunk_len(j);

    // ---- issue every global load of this group's chunks up front
    uint4 kreg[kPerGroup][2], vreg[kPerGroup][2];
    bf16x8 qf[kPerGroup][2];
    const size_t head_tok = static_cast<size_t>(bh) * a.n;
    const int t = 16 * w + r;  // this lane's token (column of the transposed tiles)
#pragma unroll
    for (int jj = 0; jj < kPerGroup; ++jj) {
        const int c = c0 + jbase + jj;
        const int Lc = (jj < nmine) ? chunk_len(jbase + jj) : 0;
        const size_t tok0 = head_tok + static_cast<size_t>(c) * W;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int idx = wt + 256 * u, row = idx >> 3, cg = idx & 7;
            if (row < Lc) {
                kreg[jj][u] = *reinterpret_cast<const uint4 *>(a.k + (tok0 + row) * W + cg * 8);
                vreg[jj][u] = *reinterpret_cast<const uint4 *>(a.v + (tok0 + row) * W + cg * 8);
            } else {
                kreg[jj][u] = make_uint4(0, 0, 0, 0);
                vreg[jj][u] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (t < Lc) x = *reinterpret_cast<const uint4 *>(a.q + (tok0 + t) * W + 32 * ks + 8 * g);
            qf[jj][ks] = *reinterpret_cast<bf16x8 *>(&x);
        }
    }
    __syncthreads();  // pw ready

    // Staging a chunk: K rows (Uh) and V rows (Ul) are written row-major with
    // 16-byte stores; after a barrier every thread gathers 8 consecutive
    // tokens of one feature (conflict-free 2-byte reads along a row) into one
    // 16-byte row of K^T and V^T.
    auto stage_rows = [&](int jj, bool with_v) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int idx = wt + 256 * u, row = idx >> 3, cg = idx & 7;
            *reinterpret_cast<uint4 *>(&G.Uh[row * LDR + cg * 8]) = kreg[jj][u];
            if (with_v) *reinterpret_cast<uint4 *>(&G.Ul[row * LDR + cg * 8]) = vreg[jj][u];
        }
    };
    auto stage_transpose = [&](bool with_v) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int task = wt + 256 * u, f = task & 63, blk = task >> 6;
            bf16x8 x;
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = G.Uh[(8 * blk + i) * LDR + f];
            *reinterpret_cast<bf16x8 *>(&G.KT[f * LDR + 8 * blk]) = x;
            if (with_v) {
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] = G.Ul[(8 * blk + i) * LDR + f];
                *reinterpret_cast<bf16x8 *>(&G.VT[f * LDR + 8 * blk]) = x;
            }
        }
    };
    // acc[bb] (rows 16w.., cols 16bb..) = rho * acc + K^T diag(f) K over the staged chunk
    auto s_update = [&](f32x4 (&acc)[4], int Lc) {
        const float rho = sm.pw[Lc];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) acc[bb] *= rho;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 kt = ld8(G.KT, 16 * w + r, 32 * ks + 8 * g);
            bf16x8 kb[4];
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) kb[bb] = ld8(G.KT, 16 * bb + r, 32 * ks + 8 * g);
            if (!decay) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) acc[bb] = mfma(kt, kb[bb], acc[bb]);
            } else {
                float x[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int s = 32 * ks + 8 * g + i;
                    const float f = s < Lc ? sm.pw[Lc - 1 - s] : 0.0f;
                    x[i] = f * static_cast<float>(kt[i]);
                }
                bf16x8 h, lo;
                split8(x, h, lo);
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) acc[bb] = mfma(h, kb[bb], acc[bb]);
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) acc[bb] = mfma(lo, kb[bb], acc[bb]);
            }
        }
    };
    // a 16-float accumulator set <-> a float scratch area in LDS (group exchange)
    float *xch = reinterpret_cast<float *>(sm.grp[1].STh);  // 16 KB inside group 1's ST tiles
    auto put_xch = [&](const f32x4 (&x)[4]) {
#pragma unroll
        for (int b = 0; b < 4; ++b) *reinterpret_cast<f32x4 *>(xch + wt * 16 + 4 * b) = x[b];
    };
    auto get_xch = [&](f32x4 (&x)[4]) {
#pragma unroll
        for (int b = 0; b < 4; ++b) x[b] = *reinterpret_cast<const f32x4 *>(xch + wt * 16 + 4 * b);
    };
    const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};

    // ================= phase A: the segment's key moment sum ==================
    // Each group sums its own chunks; group 1 then adds group 0's sum.
    f32x4 sacc[4], part[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) sacc[bb] = zero4;
#pragma unroll
    for (int jj = 0; jj < kPerGroup; ++jj) {
        const bool valid = jj < nmine;
        if (valid) stage_rows(jj, false);
        __syncthreads();
        if (valid) stage_transpose(false);
        __syncthreads();
        if (valid) s_update(sacc, chunk_len(jbase + jj));
    }
    __syncthreads();  // group 1's ST tiles are free for the exchange
    if (grp == 0) put_xch(sacc);
    __syncthreads();
    const size_t slot = static_cast<size_t>(bh) * a.P + p;
    if (grp == 1) {
        get_xch(part);  // group 0's sum S_A
        f32x4 seg[4];
        const float rhoB = sm.pw[lenB];
#pragma unroll
        for (int b = 0; b < 4; ++b) seg[b] = rhoB * part[b] + sacc[b];
        put16(a.aggS + slot * 4096, wt, seg);
        wait_stores();
    }
    __syncthreads();
    if (tid == 0) __hip_atomic_store(&a.flag1[slot], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // ---- round 1: S carry = sum over earlier segments of g^(gap) S_seg
    const int seg_tokens = a.L * W;
    // carry = sum over earlier segments pp of g^(pwr * gap) * agg[pp] (gap = tokens
    // between).  The two groups each load every other predecessor and swap their
    // partial sums through LDS, so each aggregate is read once per workgroup.
    auto sum_earlier = [&](f32x4 (&acc)[4], const float *agg, int pwr) {
        constexpr int NB = 4;
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[b] = zero4;
        for (int p0 = grp; p0 < p; p0 += 2 * NB) {
            const float *slots[NB];
            float scale[NB];
            int cnt = 0;
#pragma unroll
            for (int s2 = 0; s2 < NB; ++s2) {
                const int pp = min(p0 + 2 * s2, p - 1);
                if (p0 + 2 * s2 < p) ++cnt;
                slots[s2] = agg + (static_cast<size_t>(bh) * a.P + pp) * 4096;
                scale[s2] = decay ? powf(gam, static_cast<float>(pwr * (p - 1 - pp) * seg_tokens)) : 1.0f;
            }
            add_slots<NB>(acc, slots, scale, cnt, wt);
        }
        float *mine = reinterpret_cast<float *>(sm.grp[grp].STh);
        const float *other = reinterpret_cast<const float *>(sm.grp[grp ^ 1].STh);
        __syncthreads();  // both ST areas free
#pragma unroll
        for (int b = 0; b < 4; ++b) *reinterpret_cast<f32x4 *>(mine + wt * 16 + 4 * b) = acc[b];
        __syncthreads();
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[b] += *reinterpret_cast<const f32x4 *>(other + wt * 16 + 4 * b);
    };
    for (int pp = tid; pp < p; pp += kThreads)
        if (!wait_flag(&a.flag1[static_cast<size_t>(bh) * a.P + pp], epoch))
            __hip_atomic_fetch_add(&a.ctrl[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    {
        f32x4 carry[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) carry[b] = zero4;
        sum_earlier(carry, a.aggS, 1);
        const float rhoA = sm.pw[lenA];
#pragma unroll
        for (int b = 0; b < 4; ++b) sacc[b] = grp == 0 ? carry[b] : rhoA * carry[b] + part[b];
    }
    __syncthreads();  // exchange area read; ST tiles may be written
    // S0 (symmetric) -> ST as hi/lo: element (row 16w+4g+i, col 16bb+r) stored at [16bb+r][16w+4g+i]
    auto write_s = [&]() {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            uint2 h, lo;
            split4(sacc[bb], h, lo);
            st4(G.STh, 16 * bb + r, 16 * w + 4 * g, h);
            st4(G.STl, 16 * bb + r, 16 * w + 4 * g, lo);
        }
    };
    f32x4 xacc[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) xacc[jb] = zero4;
    // X0 -> ST as hi/lo transposed: element (row a=16w+4g+i, col j=16jb+r) at [j][a]
    auto write_x = [&]() {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            uint2 h, lo;
            split4(xacc[jb], h, lo);
            st4(G.STh, 16 * jb + r, 16 * w + 4 * g, h);
            st4(G.STl, 16 * jb + r, 16 * w + 4 * g, lo);
        }
    };
    write_s();

    // ================= phase B: each group walks its chunks ===================
    // num keeps P V only; the X0 term of each chunk is added in phase C, so the
    // local X at the start of the group's second chunk is saved here.
    f32x4 num[kPerGroup][4];
    f32x4 xsave[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) xsave[b] = zero4;
#pragma unroll
    for (int jj = 0; jj < kPerGroup; ++jj) {
        const bool valid = jj < nmine;
        const bool x0_local_save = jj == 1;
        const int Lc = valid ? chunk_len(jbase + jj) : 0;
        if (valid) stage_rows(jj, true);
        __syncthreads();  // (1) rows staged; S0 of this chunk in ST
        // transposes, and P1: A^T[:, t] = K q_t, masked and decayed -> A rows.
        // All four key blocks are computed: the last wave needs all of them, so
        // skipping masked blocks in the others would not shorten the chunk.
        if (valid) {
            stage_transpose(true);
            f32x4 acc[4];
            bf16x8 kf[2][4];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) kf[ks][sb] = ld8(G.Uh, 16 * sb + r, 32 * ks + 8 * g);
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) acc[sb] = zero4;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) acc[sb] = mfma(kf[ks][sb], qf[jj][ks], acc[sb]);
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                if (decay) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int s = 16 * sb + 4 * g + i;
                        acc[sb][i] = (s <= t) ? sm.pw[t - s] * acc[sb][i] : 0.0f;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[sb][i] = (16 * sb + 4 * g + i <= t) ? acc[sb][i] : 0.0f;
                }
                uint2 h, lo;
                split4(acc[sb], h, lo);
                st4(G.APh, t, 16 * sb + 4 * g, h);
                st4(G.APl, t, 16 * sb + 4 * g, lo);
            }
        }
        __syncthreads();  // (2) K^T, V^T ready; staging rows consumed
        // P2: U^T[:, t] = e_t S0 q_t + K^T A^T[:, t]  -> U rows
        if (valid) {
            const float e = sm.pw[t + 1];
            f32x4 acc[4];
#pragma unroll
            for (int ab = 0; ab < 4; ++ab) acc[ab] = zero4;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 sh[4], sl[4];
#pragma unroll
                for (int ab = 0; ab < 4; ++ab) {
                    sh[ab] = ld8(G.STh, 16 * ab + r, 32 * ks + 8 * g);
                    sl[ab] = ld8(G.STl, 16 * ab + r, 32 * ks + 8 * g);
                }
#pragma unroll
                for (int ab = 0; ab < 4; ++ab) acc[ab] = mfma(sh[ab], qf[jj][ks], acc[ab]);
#pragma unroll
                for (int ab = 0; ab < 4; ++ab) acc[ab] = mfma(sl[ab], qf[jj][ks], acc[ab]);
            }
#pragma unroll
            for (int ab = 0; ab < 4; ++ab) acc[ab] *= e;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 ah = ld8(G.APh, t, 32 * ks + 8 * g);
                const bf16x8 al = ld8(G.APl, t, 32 * ks + 8 * g);
                bf16x8 kt[4];
#pragma unroll
                for (int ab = 0; ab < 4; ++ab) kt[ab] = ld8(G.KT, 16 * ab + r, 32 * ks + 8 * g);
#pragma unroll
                for (int ab = 0; ab < 4; ++ab) acc[ab] = mfma(kt[ab], ah, acc[ab]);
#pragma unroll
                for (int ab = 0; ab < 4; ++ab) acc[ab] = mfma(kt[ab], al, acc[ab]);
            }
#pragma unroll
            for (int ab = 0; ab < 4; ++ab) {
                uint2 h, lo;
                split4(acc[ab], h, lo);
                st4(G.Uh, t, 16 * ab + 4 * g, h);
                st4(G.Ul, t, 16 * ab + 4 * g, lo);
            }
        }
        __syncthreads();  // (3) all rows of U; S0 reads done
        // P3: P^T[:, t] = U q_t, masked, decayed by g^(2(t-s)) -> P rows (private)
        // P4: num^T[:, t] = V^T P^T[:, t]  (the X0 term is added in phase C)
        if (x0_local_save) xsave[0] = xacc[0], xsave[1] = xacc[1], xsave[2] = xacc[2], xsave[3] = xacc[3];
        if (valid) {
            {
                f32x4 acc[4];
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) acc[sb] = zero4;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    bf16x8 uh[4], ul[4];
#pragma unroll
                    for (int sb = 0; sb < 4; ++sb) {
                        uh[sb] = ld8(G.Uh, 16 * sb + r, 32 * ks + 8 * g);
                        ul[sb] = ld8(G.Ul, 16 * sb + r, 32 * ks + 8 * g);
                    }
#pragma unroll
                    for (int sb = 0; sb < 4; ++sb) acc[sb] = mfma(uh[sb], qf[jj][ks], acc[sb]);
#pragma unroll
                    for (int sb = 0; sb < 4; ++sb) acc[sb] = mfma(ul[sb], qf[jj][ks], acc[sb]);
                }
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) {
                    if (decay) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int s = 16 * sb + 4 * g + i;
                            acc[sb][i] = (s <= t) ? sm.pw[2 * (t - s)] * acc[sb][i] : 0.0f;
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[sb][i] = (16 * sb + 4 * g + i <= t) ? acc[sb][i] : 0.0f;
                    }
                    uint2 h, lo;
                    split4(acc[sb], h, lo);
                    st4(G.APh, t, 16 * sb + 4 * g, h);
                    st4(G.APl, t, 16 * sb + 4 * g, lo);
                }
            }
            f32x4 acc[4];
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) acc[jb] = zero4;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 ph = ld8(G.APh, t, 32 * ks + 8 * g);
                const bf16x8 pl = ld8(G.APl, t, 32 * ks + 8 * g);
                bf16x8 vt[4];
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) vt[jb] = ld8(G.VT, 16 * jb + r, 32 * ks + 8 * g);
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) acc[jb] = mfma(vt[jb], ph, acc[jb]);
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) acc[jb] = mfma(vt[jb], pl, acc[jb]);
            }
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) num[jj][jb] = acc[jb];
        } else {
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) num[jj][jb] = zero4;
        }
        // P5: S0 <- rho S0 + K^T diag(f) K (next chunk's S0 into ST; this chunk's
        // S0 was last read before barrier (3))
        // P6: X0 <- rho^2 X0 + (diag(f^2) U)^T V, with U read column-wise from its rows
        if (valid) {
            s_update(sacc, Lc);
            write_s();
            const float rho2 = sm.pw[2 * Lc];
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) xacc[jb] *= rho2;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float x[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int s = 32 * ks + 8 * g + i;
                    const float f2 = s < Lc ? sm.pw[2 * (Lc - 1 - s)] : 0.0f;
                    const int o = s * LDR + 16 * w + r;
                    x[i] = f2 * (static_cast<float>(G.Uh[o]) + static_cast<float>(G.Ul[o]));
                }
                bf16x8 uh, ul;
                split8(x, uh, ul);
                bf16x8 vt[4];
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) vt[jb] = ld8(G.VT, 16 * jb + r, 32 * ks + 8 * g);
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) xacc[jb] = mfma(uh, vt[jb], xacc[jb]);
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) xacc[jb] = mfma(ul, vt[jb], xacc[jb]);
            }
        }
        __syncthreads();  // (6) chunk done; LDS may be restaged
    }

    // ---- group 1 adds group 0's X increment; publish Z_seg; round 2: X carry
    if (grp == 0) put_xch(xacc);
    __syncthreads();
    if (grp == 1) {
        get_xch(part);  // group 0's increment Z_A
        f32x4 seg[4];
        const float rhoB2 = sm.pw[lenB] * sm.pw[lenB];  // lenB <= 2W: square the in-table power
#pragma unroll
        for (int b = 0; b < 4; ++b) seg[b] = rhoB2 * part[b] + xacc[b];
        put16(a.aggZ + slot * 4096, wt, seg);
        wait_stores();
    }
    __syncthreads();
    if (tid == 0) __hip_atomic_store(&a.flag2[slot], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int pp = tid; pp < p; pp += kThreads)
        if (!wait_flag(&a.flag2[static_cast<size_t>(bh) * a.P + pp], epoch))
            __hip_atomic_fetch_add(&a.ctrl[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    {
        f32x4 carry[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) carry[b] = zero4;
        sum_earlier(carry, a.aggZ, 2);
        const float rhoA2 = sm.pw[lenA] * sm.pw[lenA];
        // X at this group's start: the carry, or (group 1) carry decayed over group 0 plus Z_A
#pragma unroll
        for (int b = 0; b < 4; ++b) xacc[b] = grp == 0 ? carry[b] : rhoA2 * carry[b] + part[b];
    }
    // ================= phase C: add e_t^2 q_t^T X0 of each chunk and store ===
    // X0 of the group's chunk jj = g^(2*64*jj) X_start + (local X before chunk jj)
    const f32x4 xstart[4] = {xacc[0], xacc[1], xacc[2], xacc[3]};
#pragma unroll
    for (int jj = 0; jj < kPerGroup; ++jj) {
        __syncthreads();  // exchange area / previous X0 reads done
        const bool valid = jj < nmine;
        if (valid) {
            const float d2 = jj == 0 ? 1.0f : sm.pw[2 * chunk_len(jbase)] ;
#pragma unroll
            for (int b = 0; b < 4; ++b) xacc[b] = d2 * xstart[b] + (jj == 0 ? zero4 : xsave[b]);
            write_x();
        }
        __syncthreads();
        if (valid) {
            const int j = jbase + jj;
            const int Lc = chunk_len(j);
            const float e2 = sm.pw[2 * t + 2];
            float *orow = a.out + (head_tok + static_cast<size_t>(c0 + j) * W + t) * W;
            f32x4 acc[4];
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) acc[jb] = zero4;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 xh[4], xl[4];
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) {
                    xh[jb] = ld8(G.STh, 16 * jb + r, 32 * ks + 8 * g);
                    xl[jb] = ld8(G.STl, 16 * jb + r, 32 * ks + 8 * g);
                }
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) acc[jb] = mfma(xh[jb], qf[jj][ks], acc[jb]);
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) acc[jb] = mfma(xl[jb], qf[jj][ks], acc[jb]);
            }
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                const f32x4 o = num[jj][jb] + e2 * acc[jb];
                if (t < Lc)
                    *reinterpret_cast<float4 *>(orow + 16 * jb + 4 * g) = make_float4(o[0], o[1], o[2], o[3]);
            }
        }
    }

    // ---- the last workgroup resets the ticket and advances the epoch
    if (tid == 0) {
        // kernel completion publishes these to the next launch on the stream
        const uint32_t done = __hip_atomic_fetch_add(&a.ctrl[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == static_cast<uint32_t>(total - 1)) {
            __hip_atomic_store(&a.ctrl[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.ctrl[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.ctrl[2], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

bool fused64_supported(const FwdProblem &p) {
    return p.dtype == HLA_BF16 && p.d == 64 && p.dv == 64 && p.w == 64 && p.ridge == 0.0f &&
           !p.normalize && p.den == nullptr && p.init.S == nullptr && p.fin.S == nullptr &&
           p.n > 0;
}

void fused64_geometry(int BH, int nc, int *P, int *L) {
    // about one workgroup per CU; at most kMaxL chunks per workgroup
    int target = (256 + BH - 1) / BH;
    int l = (nc + target - 1) / target;
    l = l < 1 ? 1 : (l > kMaxL ? kMaxL : l);
    *L = l;
    *P = (nc + l - 1) / l;
}

size_t fused64_workspace_bytes(int BH, int n) {
    const int nc = (n + W - 1) / W;
    int P, L;
    fused64_geometry(BH, nc, &P, &L);
    const size_t slots = static_cast<size_t>(BH) * P;
    return align256(2 * slots * sizeof(uint32_t)) + 2 * slots * 4096 * sizeof(float);
}

hipError_t fused64_forward(const FwdProblem &p, uint32_t *ctrl, void *data, hipStream_t st) {
    FusedArgs a{};
    a.H = p.H; a.n = p.n; a.nc = p.nc; a.BH = p.B * p.H;
    fused64_geometry(a.BH, a.nc, &a.P, &a.L);
    a.q = static_cast<const uint16_t *>(p.q);
    a.k = static_cast<const uint16_t *>(p.k);
    a.v = static_cast<const uint16_t *>(p.v);
    a.out = p.out;
    a.ctrl = ctrl;
    const size_t slots = static_cast<size_t>(a.BH) * a.P;
    char *base = static_cast<char *>(data);
    a.flag1 = reinterpret_cast<uint32_t *>(base);
    a.flag2 = a.flag1 + slots;
    a.aggS = reinterpret_cast<float *>(base + align256(2 * slots * sizeof(uint32_t)));
    a.aggZ = a.aggS + slots * 4096;
    a.gam = p.gam;
    hipLaunchKernelGGL(k_fused64, dim3(static_cast<unsigned>(slots)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace hla
