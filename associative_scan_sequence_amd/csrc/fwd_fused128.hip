// fwd_fused128.hip -- one-launch masked second-order HLA forward for
// d = dv = 128, bf16 q/k/v, on gfx950 MFMA; long sequences over few heads.
//
// Method (Higher-order Linear Attention, paperlayer.ai summary sec. 4 and 5;
// the chunk algebra of fwd_fast64.hip): with the carry held as
// (S, X = S C - G), per 64-token chunk (local t, s; length L; e_t = g^(t+1),
// f_s = g^(L-1-s); Us = diag(f^2) U)
//   A   = (Q K^T) o D_g o L,   U = diag(e) Q S0 + A K,
//   num = P V + diag(e^2) Q X0,  P = (Q Us^T) o L scaled by 1/f_t^2 per row,
//   S0 <- g^L S0 + K^T diag(f) K,   X0 <- g^2L X0 + Us^T V.
// (The chunk width the caller names only changes rounding order: this
// kernel always works in 64-token chunks.)
//
// Segments.  A head of n tokens is cut into P segments of L chunks, one per
// workgroup.  Segment outputs need the carries (S0, X0) at the segment
// start.  S0 is a decayed sum of the earlier segments' key moments; X0 is a
// decayed sum of their X increments, and the X increment of a segment that
// starts from carry S0 is affine in S0:
//   Z = S0 Ct + Lz,   Ct = sum_s g^(2 Lseg - 1 - s) q_s v_s^T  (s = position
//   in the segment),  Lz = the X increment computed from a zero S carry.
// So each workgroup walks its segment twice.  Pass 1 starts from zero
// carries and yields the segment's key moment S_seg, Ct and Lz; S_seg is
// published (round 1), the S carry is summed from the earlier segments,
// Z = S0 Ct + Lz is formed (one fp32 product) and published (round 2), and
// the X carry is summed likewise.  Pass 2 walks again from the true carries
// and writes the outputs.  With P = 1 (many heads, or short sequences) pass
// 1 and both rounds are skipped.  Aggregates and flags are device-coherent
// (sc1) accesses and carry a launch epoch; segments are taken from a ticket
// counter in increasing order (see k_fused128).
//
// Layout.  512 threads = 8 waves; wave w owns feature block w (16 of 128):
// the columns b = 16w.. of S (= its rows, S being symmetric), the columns
// j = 16w.. of X and Ct, the rows b of U^T and the rows j of num^T.  Every
// state lives in registers as accumulator tiles (lane l = 16g + r holds rows
// 16ab+4g..+3 of column 16w+r), and enters a contraction over its row index
// directly as an operand: an accumulator pair (row blocks 2k, 2k+1) gives
// the k slots 8g+e <-> row 32k+4g+e (e < 4) or 32k+16+4g+(e-4), and the
// other operand (q) is read from LDS in the same slot order.  The masked
// 64 x 64 products (A, then P) are spread over the waves as tiles and pass
// through LDS.  Transposed operands (K^T, V^T, Us^T, Q^T) come from
// row-major LDS tiles through ds_read_b64_tr_b16.  Precision: every fp32
// operand is split into bf16 hi + lo (two MFMAs); the one fp32 x fp32
// product (S0 Ct) takes hi*hi + hi*lo + lo*hi.  Us enters P with a third
// term (x = hi + mid + lo to ~2^-26): q_t . Us_s cancels heavily when q_t is
// nearly orthogonal to S_s q_s (at t = s = 0 the value is (q.k)^2), and a
// two-term Us would leave an error of ~2^-18 / cos(q, S q) there.
#include "bf16_split.h"
#include "device_common.h"
#include "hla_internal.h"

namespace hla {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int W = 64;          // tokens per chunk
constexpr int D = 128;         // d = dv
constexpr int LDW = -1;        // 128-wide tiles: the shifted-row layout of off()
constexpr int LDN = 72;        // padded LDS row of 64 bf16 (144 bytes)
constexpr int kBlk128 = 2432;  // elements per 16-row block of a 128-wide tile
constexpr int kTile128 = 4 * kBlk128;  // a 64-row 128-wide tile
constexpr int kThreads = 512;  // eight waves
constexpr int kSpinLimit = 1 << 22;
constexpr int kSpinWord = 4;   // control word: spin limit of the bounded waits (0: kSpinLimit)
constexpr int kLine = 64;
constexpr int kTicketWord = kLine + 2;  // control word: next segment ticket (P > 1)
constexpr int kSlot = 16384;   // floats per published 128 x 128 aggregate
constexpr float kMinGamma = 0.75f;
constexpr int kStateMaxSegs = 256;  // state calls: at most one segment per CU of MI355X
static_assert(kCtrlBytes >= 2 * kLine * 4, "control block too small");

struct Args128 {
    int H, n, nc, P, L, BH, segs;  // segs = BH * P
    const uint16_t *q, *k, *v;
    float *out;
    uint32_t *ctrl;     // as in fwd_fast64.hip
    uint32_t *flags;    // [BH * P][2]
    float *aggS, *aggZ; // [BH * P][kSlot]
    GammaTab gam;
    // STATE variants only:
    float *aggC;         // [BH * P][kSlot] the segments' value moments C_seg
    float *aggV;         // [BH * P][2 * D] their y increments, then their query sums m_seg
    const float *iagg;   // [BH][3][kSlot] the initial S, X = S C - G and C in the slot layout, or null
    const float *iaggV;  // [BH][2 * D] its y = S m - h, then m
    const float *irho;   // initial rho [BH] or null (read as 1)
    hla_state fin;       // final state; fin.S null: not requested
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Element offset of (row, col) in a tile.  LD > 0: rows padded to LD
// elements.  LD == LDW (128-wide tiles): rows of 256 bytes in blocks of 16,
// row r of a block shifted by 32 (r & 3) + 272 b2 + 384 b3 bytes (b2, b3 its
// bits 2 and 3) and each block followed by 768 spare bytes.  The 16-byte slot
// a row starts in is then 2 (r & 3) + b2 + 8 b3 (mod 256 bytes): transposed
// reads (rows R..R+3 and R+8..R+11, 32 bytes each) and 8-byte row reads (16
// rows) hit every bank once, and since the shift depends only on row bits that
// are lane constants or compile-time in every access here, each address is a
// lane base plus an immediate (no per-access arithmetic, unlike an XOR swizzle).
template <int LD>
__device__ __forceinline__ int off(int row, int col) {
    if constexpr (LD > 0) return row * LD + col;
    return (row >> 4) * kBlk128 + (row & 15) * 128 + 16 * (row & 3) + 136 * ((row >> 2) & 1) +
           192 * ((row >> 3) & 1) + col;
}

template <int LD>
__device__ __forceinline__ bf16x8 ld8(const __bf16 *base, int row, int col) {
    return *reinterpret_cast<const bf16x8 *>(base + off<LD>(row, col));
}

// two 4-element pieces of one LDS row: slots 0..3 at col1, 4..7 at col2
template <int LD>
__device__ __forceinline__ bf16x8 ld44(const __bf16 *base, int row, int col1, int col2) {
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(base + off<LD>(row, col1));
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(base + off<LD>(row, col2));
    bf16x8 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = a[i];
        x[4 + i] = b[i];
    }
    return x;
}

// Transposed operand: lane (g, r) receives M[rb1 + e][col0 + r] (slots 8g+e,
// e < 4) and M[rb2 + e][col0 + r] (slots 8g+4+e).
template <int LD>
__device__ __forceinline__ bf16x8 tr8(const __bf16 *M, int rb1, int rb2, int col0, int r) {
    const int col = col0 + 4 * (r & 3);
    const __bf16 *p1 = M + off<LD>(rb1 + (r >> 2), col);
    const __bf16 *p2 = M + off<LD>(rb2 + (r >> 2), col);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p1));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p2));
    const bf16x4 ab = __builtin_bit_cast(bf16x4, a), bb = __builtin_bit_cast(bf16x4, b);
    bf16x8 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = ab[i];
        x[4 + i] = bb[i];
    }
    return x;
}

// scale the 8 slots of an operand whose slot e holds row (rb + e) or
// (rb + 4 + e - 4) by w(row), then split
template <typename F>
__device__ __forceinline__ void scaled_split(const bf16x8 &x, int rb, F wfun, bf16x8 &hi, bf16x8 &lo) {
    f32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a[e] = wfun(rb + e) * static_cast<float>(x[e]);
        b[e] = wfun(rb + 4 + e) * static_cast<float>(x[4 + e]);
    }
    pair_operand(a, b, hi, lo);
}

template <int LD>
__device__ __forceinline__ void st4(__bf16 *base, int row, int col, const bf16x4 &v) {
    *reinterpret_cast<bf16x4 *>(base + off<LD>(row, col)) = v;
}

__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ }

__device__ __forceinline__ uint32_t next_epoch(uint32_t e) { return e * 1664525u + 1013904223u; }

__device__ bool wait_flag(const uint32_t *f, uint32_t want, int spin) {
    for (int it = 0; it < spin; ++it) {
        if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// a carry whose inputs could not be waited for: NaN, so every output built on it is NaN
__device__ __forceinline__ void poison(f32x4 (&acc)[8]) {
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[b] = f32x4{nan, nan, nan, nan};
}

constexpr int kSc1 = 16;  // buffer cache policy: sc1 (device scope)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const float *slot) {
    const uint64_t addr = reinterpret_cast<uint64_t>(slot);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(addr)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(addr >> 32)));
    float *base = reinterpret_cast<float *>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, kSlot * 4, 0x00020000);
}

// a thread's 32 floats (8 tiles) <-> its 128 bytes of a 64 KB slot
__device__ __forceinline__ void put32(const float *slot, int tid, const f32x4 (&x)[8]) {
    const __amdgpu_buffer_rsrc_t rs = slot_rsrc(slot);
#pragma unroll
    for (int b = 0; b < 8; ++b) __builtin_amdgcn_raw_buffer_store_b128(x[b], rs, 128 * tid + 16 * b, 0, kSc1);
}

// acc += sum over earlier segments pp < p of scale(pp) * slot(pp)
template <typename F>
__device__ void add_slots(f32x4 (&acc)[8], const float *agg, int first, int p, int tid, F scale) {
    constexpr int NB = 4;
    for (int p0 = 0; p0 < p; p0 += NB) {
        f32x4 v[NB][8];
#pragma unroll
        for (int s = 0; s < NB; ++s)
            if (p0 + s < p) {
                const __amdgpu_buffer_rsrc_t rs = slot_rsrc(agg + static_cast<size_t>(first + p0 + s) * kSlot);
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    v[s][b] = __builtin_amdgcn_raw_buffer_load_b128(rs, 128 * tid + 16 * b, 0, kSc1);
            }
#pragma unroll
        for (int s = 0; s < NB; ++s)
            if (p0 + s < p) {
                const float sc = scale(p0 + s);
#pragma unroll
                for (int b = 0; b < 8; ++b) acc[b] += sc * v[s][b];
            }
    }
}

// acc = sum over earlier segments pp < p of scale(pp) * slot(pp)
template <typename F>
__device__ void sum_slots(f32x4 (&acc)[8], const float *agg, int first, int p, int tid, F scale) {
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    add_slots(acc, agg, first, p, tid, scale);
}

// one float of a published vector slot (device-coherent)
__device__ __forceinline__ void put_vec(const float *slot, int idx, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), slot_rsrc(slot), 4 * idx, 0, kSc1);
}
__device__ __forceinline__ float get_vec(const float *slot, int idx) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(slot_rsrc(slot), 4 * idx, 0, kSc1));
}

struct Smem128 {
    __bf16 K[kTile128];   // chunk rows [s][a]
    __bf16 V[kTile128];   // [s][j]
    __bf16 Q[kTile128];   // [t][a]
    __bf16 Uh[kTile128];  // Us rows [s][b]: hi, mid and a third term
    __bf16 Ul[kTile128];
    __bf16 Ux[kTile128];
    __bf16 Ah[W * LDN];  // masked scores A[t][i], then P[t][s], hi and lo
    __bf16 Al[W * LDN];
    float vec[2 * D];    // STATE: vectors exchanged between the waves
    uint32_t epoch;
    int ticket;    // the segment this workgroup holds (ticketed launches)
    uint32_t bad;  // nonzero: a wait of this segment gave up
};
// the S0 tiles of the Z product (128 rows, hi and lo) overlay K .. Uh
static_assert(4 * kTile128 >= 2 * (2 * kTile128), "S0 overlay does not fit");

// The ten unmasked (t-block, i-block) tiles of a 64 x 64 masked product,
// then the two masked tiles whose zeros a k-block read also covers.
// Entry idx of each table sits in bits 2idx, 2idx+1 of a constant, so the
// lookup is a shift of a wave-uniform index (no memory read):
//   tb = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3, 0, 2}, ib = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3, 1, 3}.
__device__ __forceinline__ void tri_tile(int idx, int &tb, int &ib) {
    constexpr uint32_t kTb = 0x8ffa94u, kIb = 0xde4910u;
    tb = static_cast<int>((kTb >> (2 * idx)) & 3u);
    ib = static_cast<int>((kIb >> (2 * idx)) & 3u);
}

// LOOP = false: one segment per workgroup (grid = segs: at most the CU count,
// or any count when each head is one segment); true: workgroups take
// segments until none is left (grid = CU count < segs).
// When the segments of a head wait on each other (P > 1), a workgroup takes
// its segments from a ticket counter (control word kTicketWord), so segment
// s is only ever held by a workgroup that is already running, and every
// earlier segment of its head was taken before it by a running workgroup
// that waits only on segments earlier still: the waits always end, whatever
// other streams keep resident on the device.  With P = 1 nothing waits and
// segment = workgroup index.
// A wait that still gives up (spin limit, or forced from the host through
// control word 4) makes the carry it was waiting for NaN: every output of
// the segment and of the later segments of its head that read the carry is
// then NaN, never a silently wrong number.
// STATE: an initial state enters the carries (a.iagg, prepared by
// k_fused128_init) and the last segment of each head forms the final state
// when a.fin.S is set.  For the final state every segment also sums, in pass
// 1, its value moment C_seg (whence Ct = g^T C_seg, T its token count), its
// query sum m_seg and its zero-carry y increment ly (column sums of Us); its
// y increment from the true carry is y_seg = S0 g^T m_seg + ly, by the same
// affine argument as Z.  C_seg, y_seg and m_seg are published with Z.  The
// last segment then has S and X at the sequence end in its registers after
// pass 2, and forms G = S C - X and h = S m - y from the summed C, m and y.
template <bool DECAY, bool LOOP, bool STATE>
__global__ __launch_bounds__(kThreads, 1) void k_fused128(Args128 a) {
    __shared__ Smem128 sm;
    const int tid = threadIdx.x, l = tid & 63, r = l & 15, g = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)

    // ---- launch epoch (flags of this launch carry it)
    if (tid == 0) sm.epoch = next_epoch(__hip_atomic_load(&a.ctrl[kLine + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    __syncthreads();
    const uint32_t epoch = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sm.epoch)));
    float lg = 0.0f;
    auto gp = [&](float e) { return DECAY ? __builtin_amdgcn_exp2f(e * lg) : 1.0f; };  // g^e
    const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
    auto seg_body = [&](const int seg) __attribute__((always_inline)) {
    const int bh = seg % a.BH, p = seg / a.BH;
    const size_t head_tok = static_cast<size_t>(bh) * a.n;
    lg = DECAY ? log2f(head_gamma(a.gam, bh % a.H)) : 0.0f;
    const int c0 = p * a.L;
    const int Lseg = min(a.L, a.nc - c0);
    const int seg_tokens = a.L * W;
    const size_t slot0 = static_cast<size_t>(bh) * a.P;
    const bool want_fin = STATE && a.fin.S != nullptr;
    const bool fin_seg = want_fin && p + 1 == a.P;  // this workgroup writes the head's final state
    const int T = min(a.n - c0 * W, a.L * W);       // tokens of this segment

    // ---- chunk inputs: each thread fetches two 16-byte pieces of q, k and v
    u32x4 pre[3][2];
    auto fetch = [&](int j) __attribute__((always_inline)) {  // chunk j of the segment
        // unconditional loads (rows past the chunk read the head's first row);
        // they are masked to zero when staged
        const int Lc = j < Lseg ? min(W, a.n - (c0 + j) * W) : 0;
        const size_t tok0 = head_tok + static_cast<size_t>(c0 + j) * W;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int idx = tid + kThreads * u, row = idx >> 4, cg = idx & 15;
            const size_t off = (row < Lc ? tok0 + row : head_tok) * D + cg * 8;
            pre[0][u] = *reinterpret_cast<const u32x4 *>(a.q + off);
            pre[1][u] = *reinterpret_cast<const u32x4 *>(a.k + off);
            pre[2][u] = *reinterpret_cast<const u32x4 *>(a.v + off);
        }
    };
    auto stage = [&](int Lc) __attribute__((always_inline)) {
        const u32x4 z = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int idx = tid + kThreads * u, row = idx >> 4, cg = idx & 15;
            const bool ok = row < Lc;
            *reinterpret_cast<u32x4 *>(&sm.Q[off<LDW>(row, cg * 8)]) = ok ? pre[0][u] : z;
            *reinterpret_cast<u32x4 *>(&sm.K[off<LDW>(row, cg * 8)]) = ok ? pre[1][u] : z;
            *reinterpret_cast<u32x4 *>(&sm.V[off<LDW>(row, cg * 8)]) = ok ? pre[2][u] : z;
        }
    };

    f32x4 sacc[8], xacc[8], cacc[8];  // S[a][b = 16w+r], X[a][j = 16w+r], Ct[a][j] (STATE: C_seg[a][j])
#pragma unroll
    for (int b = 0; b < 8; ++b) sacc[b] = xacc[b] = cacc[b] = zero4;
    // STATE, pass 1: m_seg and ly, entry 16w+r in row 0 (lanes 0-15) of a ones-operand product
    f32x4 macc = zero4, lyacc = zero4;
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(r == 0 ? 1.0f : 0.0f);

    // One walk over the segment.  OUT: pass 2 (outputs); else pass 1 (Ct too).
    auto walk = [&](auto out_tag) {
        constexpr bool OUT = decltype(out_tag)::value;
        fetch(0);
        int pos = 0;  // token offset of the chunk in the segment
        for (int jc = 0; jc < Lseg; ++jc) {
            const int Lc = min(W, a.n - (c0 + jc) * W);
            __syncthreads();  // (0) previous chunk's tile reads done
            stage(Lc);
            if (jc + 1 < Lseg) fetch(jc + 1);
            __syncthreads();  // (1) chunk tiles ready

            // -- masked scores A^T tiles -> A rows (hi/lo) in LDS
            for (int idx = w; idx < 12; idx += 8) {
                int tb, ib;
                tri_tile(idx, tb, ib);
                f32x4 at = zero4;
                if (idx < 10) {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        at = mfma(ld8<LDW>(sm.K, 16 * ib + r, 32 * ks + 8 * g),
                                  ld8<LDW>(sm.Q, 16 * tb + r, 32 * ks + 8 * g), at);
                    const int t = 16 * tb + r;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int i = 16 * ib + 4 * g + c;
                        at[c] = i <= t ? gp(static_cast<float>(t - i)) * at[c] : 0.0f;
                    }
                }
                bf16x4 h, lo;
                split4(at, h, lo);
                st4<LDN>(sm.Ah, 16 * tb + r, 16 * ib + 4 * g, h);
                st4<LDN>(sm.Al, 16 * tb + r, 16 * ib + 4 * g, lo);
            }
            // -- S0 q part of U^T (rows b = 16w.., all t), from the S registers
            f32x4 us_[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) us_[tb] = zero4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8 sh, sl;
                pair_operand(sacc[2 * kk], sacc[2 * kk + 1], sh, sl);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const bf16x8 qp = ld44<LDW>(sm.Q, 16 * tb + r, 32 * kk + 4 * g, 32 * kk + 16 + 4 * g);
                    us_[tb] = mfma(sh, qp, us_[tb]);
                    us_[tb] = mfma(sl, qp, us_[tb]);
                }
            }
            __syncthreads();  // (2) A rows ready
            // -- U^T = e_t (S0 q_t) + K^T A^T; Us = f_t^2 U -> rows in LDS
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int t = 16 * tb + r;
                f32x4 ak = zero4;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (2 * ks <= tb) {
                        const int rb = 32 * ks + 8 * g;
                        const bf16x8 kt = tr8<LDW>(sm.K, rb, rb + 4, 16 * w, r);
                        ak = mfma(kt, ld8<LDN>(sm.Ah, t, 32 * ks + 8 * g), ak);
                        ak = mfma(kt, ld8<LDN>(sm.Al, t, 32 * ks + 8 * g), ak);
                    }
                }
                const float e = gp(static_cast<float>(t + 1));
                const float f2 = t < Lc ? gp(static_cast<float>(2 * (Lc - 1 - t))) : 0.0f;
                const f32x4 us = f2 * (e * us_[tb] + ak);
                bf16x4 h, mid, lo;
                split3(us, h, mid, lo);
                st4<LDW>(sm.Uh, t, 16 * w + 4 * g, h);
                st4<LDW>(sm.Ul, t, 16 * w + 4 * g, mid);
                st4<LDW>(sm.Ux, t, 16 * w + 4 * g, lo);
            }
            __syncthreads();  // (3) Us rows ready; A reads done
            if constexpr (OUT) {
                // -- P^T tiles -> P rows (hi/lo) in LDS (over the A rows)
                for (int idx = w; idx < 12; idx += 8) {
                    int tb, sb;
                    tri_tile(idx, tb, sb);
                    f32x4 pt = zero4;
                    if (idx < 10) {
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) {
                            const bf16x8 qv = ld8<LDW>(sm.Q, 16 * tb + r, 32 * kb + 8 * g);
                            pt = mfma(ld8<LDW>(sm.Uh, 16 * sb + r, 32 * kb + 8 * g), qv, pt);
                            pt = mfma(ld8<LDW>(sm.Ul, 16 * sb + r, 32 * kb + 8 * g), qv, pt);
                            pt = mfma(ld8<LDW>(sm.Ux, 16 * sb + r, 32 * kb + 8 * g), qv, pt);
                        }
                        const int t = 16 * tb + r;
                        const float inv_f2 = t < Lc ? gp(static_cast<float>(-2 * (Lc - 1 - t))) : 0.0f;
#pragma unroll
                        for (int c = 0; c < 4; ++c) pt[c] = 16 * sb + 4 * g + c <= t ? inv_f2 * pt[c] : 0.0f;
                    }
                    bf16x4 h, lo;
                    split4(pt, h, lo);
                    st4<LDN>(sm.Ah, 16 * tb + r, 16 * sb + 4 * g, h);
                    st4<LDN>(sm.Al, 16 * tb + r, 16 * sb + 4 * g, lo);
                }
                // -- the X0 part of num^T (rows j = 16w.., all t), from the X registers
                f32x4 qx[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) qx[tb] = zero4;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    bf16x8 xh, xl;
                    pair_operand(xacc[2 * kk], xacc[2 * kk + 1], xh, xl);
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) {
                        const bf16x8 qp = ld44<LDW>(sm.Q, 16 * tb + r, 32 * kk + 4 * g, 32 * kk + 16 + 4 * g);
                        qx[tb] = mfma(xh, qp, qx[tb]);
                        qx[tb] = mfma(xl, qp, qx[tb]);
                    }
                }
                __syncthreads();  // (4) P rows ready
                // -- num^T = V^T P^T + e_t^2 X0^T q_t; store
                const size_t tok0 = head_tok + static_cast<size_t>(c0 + jc) * W;
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const int t = 16 * tb + r;
                    f32x4 pv = zero4;
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        if (2 * ks <= tb) {
                            const int rb = 32 * ks + 8 * g;
                            const bf16x8 vt = tr8<LDW>(sm.V, rb, rb + 4, 16 * w, r);
                            pv = mfma(vt, ld8<LDN>(sm.Ah, t, 32 * ks + 8 * g), pv);
                            pv = mfma(vt, ld8<LDN>(sm.Al, t, 32 * ks + 8 * g), pv);
                        }
                    }
                    const float e = gp(static_cast<float>(t + 1));
                    const f32x4 o = pv + (e * e) * qx[tb];
                    if (t < Lc)
                        *reinterpret_cast<float4 *>(a.out + (tok0 + t) * D + 16 * w + 4 * g) =
                            make_float4(o[0], o[1], o[2], o[3]);
                }
            }
            // -- S <- g^L S + K^T diag(f) K   (columns b = 16w..)
            {
                const float rho = gp(static_cast<float>(Lc));
#pragma unroll
                for (int ab = 0; ab < 8; ++ab) sacc[ab] *= rho;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int rb = 32 * ks + 8 * g;
                    const bf16x8 kb = tr8<LDW>(sm.K, rb, rb + 4, 16 * w, r);
                    bf16x8 kh = kb, kl;
                    if (DECAY)
                        scaled_split(kb, rb, [&](int s) { return gp(static_cast<float>(Lc - 1 - s)); }, kh, kl);
#pragma unroll
                    for (int ab = 0; ab < 8; ++ab) {
                        const bf16x8 ka = tr8<LDW>(sm.K, rb, rb + 4, 16 * ab, r);
                        sacc[ab] = mfma(ka, kh, sacc[ab]);
                        if (DECAY) sacc[ab] = mfma(ka, kl, sacc[ab]);
                    }
                }
            }
            // -- X <- g^2L X + Us^T V   (columns j = 16w..)
            {
                const float rho2 = gp(static_cast<float>(2 * Lc));
#pragma unroll
                for (int ab = 0; ab < 8; ++ab) xacc[ab] *= rho2;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int rb = 32 * ks + 8 * g;
                    const bf16x8 vt = tr8<LDW>(sm.V, rb, rb + 4, 16 * w, r);
#pragma unroll
                    for (int ab = 0; ab < 8; ++ab) {
                        xacc[ab] = mfma(tr8<LDW>(sm.Uh, rb, rb + 4, 16 * ab, r), vt, xacc[ab]);
                        xacc[ab] = mfma(tr8<LDW>(sm.Ul, rb, rb + 4, 16 * ab, r), vt, xacc[ab]);
                    }
                }
            }
            if constexpr (!OUT && !STATE) {
                // -- Ct <- g^2L Ct + Q^T diag(g^(pos + 2L - 1 - s)) V   (columns j = 16w..)
                const float rho2 = gp(static_cast<float>(2 * Lc));
#pragma unroll
                for (int ab = 0; ab < 8; ++ab) cacc[ab] *= rho2;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int rb = 32 * ks + 8 * g;
                    const bf16x8 vt = tr8<LDW>(sm.V, rb, rb + 4, 16 * w, r);
                    bf16x8 vh = vt, vl;
                    if (DECAY)
                        scaled_split(vt, rb, [&](int s) { return gp(static_cast<float>(pos + 2 * Lc - 1 - s)); }, vh,
                                     vl);
#pragma unroll
                    for (int ab = 0; ab < 8; ++ab) {
                        const bf16x8 qa = tr8<LDW>(sm.Q, rb, rb + 4, 16 * ab, r);
                        cacc[ab] = mfma(qa, vh, cacc[ab]);
                        if (DECAY) cacc[ab] = mfma(qa, vl, cacc[ab]);
                    }
                }
            }
            if constexpr (!OUT && STATE) {
                // -- C_seg <- g^L C_seg + Q^T diag(g^(L - 1 - s)) V, m_seg <- g^L m_seg +
                // Q^T g^(L - 1 - s), ly <- g^2L ly + Us^T 1   (columns j, entries 16w..)
                const float rho = gp(static_cast<float>(Lc)), rho2 = rho * rho;
#pragma unroll
                for (int ab = 0; ab < 8; ++ab) cacc[ab] *= rho;
                macc *= rho;
                lyacc *= rho2;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int rb = 32 * ks + 8 * g;
                    auto wdec = [&](int s) { return gp(static_cast<float>(Lc - 1 - s)); };
                    const bf16x8 vt = tr8<LDW>(sm.V, rb, rb + 4, 16 * w, r);
                    bf16x8 vh = vt, vl;
                    if (DECAY) scaled_split(vt, rb, wdec, vh, vl);
#pragma unroll
                    for (int ab = 0; ab < 8; ++ab) {
                        const bf16x8 qa = tr8<LDW>(sm.Q, rb, rb + 4, 16 * ab, r);
                        cacc[ab] = mfma(qa, vh, cacc[ab]);
                        if (DECAY) cacc[ab] = mfma(qa, vl, cacc[ab]);
                    }
                    const bf16x8 qw = tr8<LDW>(sm.Q, rb, rb + 4, 16 * w, r);
                    bf16x8 qh = qw, ql;
                    if (DECAY) scaled_split(qw, rb, wdec, qh, ql);
                    macc = mfma(ones, qh, macc);
                    if (DECAY) macc = mfma(ones, ql, macc);
                    lyacc = mfma(ones, tr8<LDW>(sm.Uh, rb, rb + 4, 16 * w, r), lyacc);
                    lyacc = mfma(ones, tr8<LDW>(sm.Ul, rb, rb + 4, 16 * w, r), lyacc);
                    lyacc = mfma(ones, tr8<LDW>(sm.Ux, rb, rb + 4, 16 * w, r), lyacc);
                }
            }
            pos += Lc;
        }
    };

    // the initial state's part `kind` (0 S, 1 X, 2 C), scaled, added to acc
    auto add_init = [&](f32x4 (&acc)[8], int kind, float sc) {
        if constexpr (STATE) {
            if (a.iagg != nullptr)
                add_slots(acc, a.iagg, 3 * bh + kind, 1, tid, [&](int) { return sc; });
        }
    };
    if (a.P > 1 || fin_seg) {  // (one segment with a final state: pass 1 for C, m and y)
        if (tid == 0) sm.bad = 0u;  // read only after the barriers below
        walk(std::integral_constant<bool, false>{});
        const int spin_set = static_cast<int>(__hip_atomic_load(&a.ctrl[kSpinWord], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        // -1: give up without polling (a host-forced failure); n > 0: n polls
        const int spin = spin_set < 0 ? 0 : (spin_set > 0 ? spin_set : kSpinLimit);
        if (a.P > 1) {
            // ---- round 1: publish the segment's key moment; S carry from the earlier segments
            put32(a.aggS + (slot0 + p) * kSlot, tid, sacc);
            wait_stores();
            __syncthreads();
            if (tid == 0) __hip_atomic_store(&a.flags[2 * (slot0 + p)], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int pp = tid; pp < p; pp += kThreads)
                if (!wait_flag(&a.flags[2 * (slot0 + pp)], epoch, spin)) {
                    __hip_atomic_fetch_add(&a.ctrl[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    sm.bad = 1u;
                }
            __syncthreads();
            sum_slots(sacc, a.aggS, static_cast<int>(slot0), p, tid,
                      [&](int pp) { return gp(static_cast<float>((p - 1 - pp) * seg_tokens)); });
        } else {
#pragma unroll
            for (int b = 0; b < 8; ++b) sacc[b] = zero4;
        }
        add_init(sacc, 0, gp(static_cast<float>(p * seg_tokens)));
        if (sm.bad) poison(sacc);
        if (a.P > 1) {
            // ---- Z = S0 Ct + Lz: S0 -> LDS rows (hi/lo); lane holds S0[a][b = 16w+r] = S0[b][a]
            __bf16 *S0h = sm.K, *S0l = sm.K + 2 * kTile128;  // 128-row tiles over K, V and Q, Uh
#pragma unroll
            for (int ab = 0; ab < 8; ++ab) {
                bf16x4 h, lo;
                split4(sacc[ab], h, lo);
                st4<LDW>(S0h, 16 * w + r, 16 * ab + 4 * g, h);
                st4<LDW>(S0l, 16 * w + r, 16 * ab + 4 * g, lo);
            }
            __syncthreads();
            const float gT = STATE ? gp(static_cast<float>(T)) : 1.0f;  // STATE: Ct = g^T C_seg
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8 ch, cl2;
                if constexpr (STATE) pair_operand(gT * cacc[2 * kk], gT * cacc[2 * kk + 1], ch, cl2);
                else pair_operand(cacc[2 * kk], cacc[2 * kk + 1], ch, cl2);
#pragma unroll
                for (int ab = 0; ab < 8; ++ab) {
                    const int row = 16 * ab + r;
                    const bf16x8 s0h = ld44<LDW>(S0h, row, 32 * kk + 4 * g, 32 * kk + 16 + 4 * g);
                    const bf16x8 s0l = ld44<LDW>(S0l, row, 32 * kk + 4 * g, 32 * kk + 16 + 4 * g);
                    xacc[ab] = mfma(s0h, ch, xacc[ab]);
                    xacc[ab] = mfma(s0h, cl2, xacc[ab]);
                    xacc[ab] = mfma(s0l, ch, xacc[ab]);
                }
            }
        }
        // STATE: y_seg = S0 (g^T m_seg) + ly, entry b = 16w+r in lanes 0-15 (S0 symmetric)
        float yseg = 0.0f;
        if constexpr (STATE) {
            __syncthreads();  // (S0 tile reads done; sm.vec free)
            if (g == 0) sm.vec[16 * w + r] = macc[0];
            __syncthreads();
            float part = 0.0f;
#pragma unroll
            for (int ab = 0; ab < 8; ++ab)
#pragma unroll
                for (int e = 0; e < 4; ++e) part += sacc[ab][e] * sm.vec[16 * ab + 4 * g + e];
            part += __shfl_xor(part, 16);
            part += __shfl_xor(part, 32);
            yseg = gp(static_cast<float>(T)) * part + lyacc[0];
            __syncthreads();  // sm.vec reads done
        }
        if (a.P > 1) {
            // ---- round 2: publish Z (STATE: and C_seg, y_seg, m_seg); X carry from the earlier segments
            put32(a.aggZ + (slot0 + p) * kSlot, tid, xacc);
            if constexpr (STATE) {
                if (want_fin) {
                    put32(a.aggC + (slot0 + p) * kSlot, tid, cacc);
                    if (g == 0) {
                        put_vec(a.aggV + (slot0 + p) * 2 * D, 16 * w + r, yseg);
                        put_vec(a.aggV + (slot0 + p) * 2 * D, D + 16 * w + r, macc[0]);
                    }
                }
            }
            wait_stores();
            __syncthreads();
            if (tid == 0)
                __hip_atomic_store(&a.flags[2 * (slot0 + p) + 1], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int pp = tid; pp < p; pp += kThreads)
                if (!wait_flag(&a.flags[2 * (slot0 + pp) + 1], epoch, spin)) {
                    __hip_atomic_fetch_add(&a.ctrl[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    sm.bad = 1u;
                }
            __syncthreads();
            sum_slots(xacc, a.aggZ, static_cast<int>(slot0), p, tid,
                      [&](int pp) { return gp(static_cast<float>(2 * (p - 1 - pp) * seg_tokens)); });
        } else {
#pragma unroll
            for (int b = 0; b < 8; ++b) xacc[b] = zero4;
        }
        add_init(xacc, 1, gp(static_cast<float>(2 * p * seg_tokens)));
        if (sm.bad) poison(xacc);
        if constexpr (STATE) {
            if (fin_seg) {
                // C, m and y at the sequence end: this segment's own sums plus the
                // earlier segments' (decayed over the tokens after each) and the
                // initial state's; C to fin.C, m to fin.m and sm.vec, y to sm.vec
                auto after = [&](int pp) { return static_cast<float>(a.n - (pp + 1) * seg_tokens); };
                add_slots(cacc, a.aggC, static_cast<int>(slot0), p, tid, [&](int pp) { return gp(after(pp)); });
                add_init(cacc, 2, gp(static_cast<float>(a.n)));
                if (sm.bad) poison(cacc);
                float *C = a.fin.C + static_cast<size_t>(bh) * D * D;
#pragma unroll
                for (int ab = 0; ab < 8; ++ab)
#pragma unroll
                    for (int e = 0; e < 4; ++e) C[(16 * ab + 4 * g + e) * D + 16 * w + r] = cacc[ab][e];
                if (g == 0) {
                    float mv = macc[0], yv = yseg;
                    for (int pp = 0; pp < p; ++pp) {
                        const float *vs = a.aggV + (slot0 + pp) * 2 * D;
                        const float d1 = gp(after(pp));
                        yv += d1 * d1 * get_vec(vs, 16 * w + r);
                        mv += d1 * get_vec(vs, D + 16 * w + r);
                    }
                    if (a.iaggV != nullptr) {
                        const float dn = gp(static_cast<float>(a.n));
                        yv += dn * dn * a.iaggV[static_cast<size_t>(bh) * 2 * D + 16 * w + r];
                        mv += dn * a.iaggV[static_cast<size_t>(bh) * 2 * D + D + 16 * w + r];
                    }
                    if (sm.bad) mv = yv = __builtin_nanf("");
                    a.fin.m[static_cast<size_t>(bh) * D + 16 * w + r] = mv;
                    sm.vec[16 * w + r] = mv;
                    sm.vec[D + 16 * w + r] = yv;
                }
            }
        }
    } else if constexpr (STATE) {  // one segment, no final state: the carries are the initial state
        add_init(sacc, 0, 1.0f);
        add_init(xacc, 1, 1.0f);
    }
    walk(std::integral_constant<bool, true>{});

    __syncthreads();  // this segment's LDS reads are done before the next one is staged
    if constexpr (STATE) {
        if (fin_seg) {
            // ---- the final state: sacc, xacc hold S and X at the sequence end.
            // S is made exactly symmetric (the mean of the two triangles, through
            // fin.S), then h = S m - y, and G = S C - X with C reloaded from fin.C
            // (the product as for Z: S tiles in LDS, C from registers)
            float *S = a.fin.S + static_cast<size_t>(bh) * D * D;
#pragma unroll
            for (int ab = 0; ab < 8; ++ab)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[(16 * ab + 4 * g + e) * D + 16 * w + r] = sacc[ab][e];
            __syncthreads();
#pragma unroll
            for (int ab = 0; ab < 8; ++ab)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sacc[ab][e] = 0.5f * (sacc[ab][e] + S[(16 * w + r) * D + 16 * ab + 4 * g + e]);
            __syncthreads();
#pragma unroll
            for (int ab = 0; ab < 8; ++ab)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[(16 * ab + 4 * g + e) * D + 16 * w + r] = sacc[ab][e];
            float part = 0.0f;
#pragma unroll
            for (int ab = 0; ab < 8; ++ab)
#pragma unroll
                for (int e = 0; e < 4; ++e) part += sacc[ab][e] * sm.vec[16 * ab + 4 * g + e];
            part += __shfl_xor(part, 16);
            part += __shfl_xor(part, 32);
            if (g == 0) a.fin.h[static_cast<size_t>(bh) * D + 16 * w + r] = part - sm.vec[D + 16 * w + r];
            const float *C = a.fin.C + static_cast<size_t>(bh) * D * D;
#pragma unroll
            for (int ab = 0; ab < 8; ++ab) {
                xacc[ab] = -xacc[ab];
#pragma unroll
                for (int e = 0; e < 4; ++e) cacc[ab][e] = C[(16 * ab + 4 * g + e) * D + 16 * w + r];
            }
            __bf16 *S0h = sm.K, *S0l = sm.K + 2 * kTile128;
#pragma unroll
            for (int ab = 0; ab < 8; ++ab) {
                bf16x4 h, lo;
                split4(sacc[ab], h, lo);
                st4<LDW>(S0h, 16 * w + r, 16 * ab + 4 * g, h);
                st4<LDW>(S0l, 16 * w + r, 16 * ab + 4 * g, lo);
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8 ch, cl2;
                pair_operand(cacc[2 * kk], cacc[2 * kk + 1], ch, cl2);
#pragma unroll
                for (int ab = 0; ab < 8; ++ab) {
                    const int row = 16 * ab + r;
                    const bf16x8 s0h = ld44<LDW>(S0h, row, 32 * kk + 4 * g, 32 * kk + 16 + 4 * g);
                    const bf16x8 s0l = ld44<LDW>(S0l, row, 32 * kk + 4 * g, 32 * kk + 16 + 4 * g);
                    xacc[ab] = mfma(s0h, ch, xacc[ab]);
                    xacc[ab] = mfma(s0h, cl2, xacc[ab]);
                    xacc[ab] = mfma(s0l, ch, xacc[ab]);
                }
            }
            float *G = a.fin.G + static_cast<size_t>(bh) * D * D;
#pragma unroll
            for (int ab = 0; ab < 8; ++ab)
#pragma unroll
                for (int e = 0; e < 4; ++e) G[(16 * ab + 4 * g + e) * D + 16 * w + r] = xacc[ab][e];
            if (tid == 0 && a.fin.rho != nullptr)
                a.fin.rho[bh] = (a.irho != nullptr ? a.irho[bh] : 1.0f) * gp(static_cast<float>(a.n));
            __syncthreads();  // LDS reads done before the next segment is staged
        }
    }
    };
    // (a loop around the body costs registers even when it runs once, so the
    // one-segment-per-workgroup launch calls it straight)
    // the next segment: a ticket when segments wait on each other
    auto take = [&]() -> int {
        if (tid == 0)
            sm.ticket = static_cast<int>(
                __hip_atomic_fetch_add(&a.ctrl[kTicketWord], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        __syncthreads();
        const int t = __builtin_amdgcn_readfirstlane(sm.ticket);
        __syncthreads();  // every wave has read it before it is overwritten
        return t;
    };
    if constexpr (LOOP) {
        for (int seg = take(); seg < a.segs; seg = take()) seg_body(seg);
    } else {
        const int seg = a.P > 1 ? take() : static_cast<int>(blockIdx.x);
        if (seg < a.segs) seg_body(seg);
        else if (tid == 0)  // a ticket out of range: the control block was not zero before first use
            __hip_atomic_fetch_add(&a.ctrl[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- the last workgroup to finish resets the counters and advances the epoch
    if (tid == 0) {
        const uint32_t done = __hip_atomic_fetch_add(&a.ctrl[kLine], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            __hip_atomic_store(&a.ctrl[kLine], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.ctrl[kTicketWord], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.ctrl[kLine + 1], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(&a.ctrl[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// The initial state in the slot layout of the kernel's registers: thread tid
// = 64 w + 16 g + r holds, at floats 32 tid + 4 ab + e of a slot, element
// (16 ab + 4 g + e, 16 w + r) of S, of X = S C - G and of C; then y = S m - h
// and m as one vector pair.  Grid (BH, 8): workgroup (bh, y) forms rows
// 16y..16y+15; each thread a 1 x 8 block of X (fp32, all of C staged in LDS).
__global__ __launch_bounds__(256) void k_fused128_init(hla_state in, float *iagg, float *iaggV) {
    __shared__ float Cs[D * D], Ss[16 * D], ms[D];
    const int bh = blockIdx.x, r0 = 16 * blockIdx.y, tid = threadIdx.x;
    const size_t mo = static_cast<size_t>(bh) * D * D;
    for (int i = tid; i < D * D / 4; i += 256)
        reinterpret_cast<float4 *>(Cs)[i] = reinterpret_cast<const float4 *>(in.C + mo)[i];
    for (int i = tid; i < 16 * D / 4; i += 256)
        reinterpret_cast<float4 *>(Ss)[i] = reinterpret_cast<const float4 *>(in.S + mo + r0 * D)[i];
    if (tid < D / 2) {
        ms[2 * tid] = in.m[static_cast<size_t>(bh) * D + 2 * tid];
        ms[2 * tid + 1] = in.m[static_cast<size_t>(bh) * D + 2 * tid + 1];
    }
    __syncthreads();
    auto sidx = [](int ra, int c) {
        const int ab = ra >> 4, g = (ra >> 2) & 3, e = ra & 3, w = c >> 4, r = c & 15;
        return 32 * (64 * w + 16 * g + r) + 4 * ab + e;
    };
    float *dst = iagg + static_cast<size_t>(bh) * 3 * kSlot;
    const int lr = tid >> 4, c0 = 8 * (tid & 15), ra = r0 + lr;
    float x[8] = {};
    for (int b = 0; b < D; ++b) {
        const float sv = Ss[lr * D + b];
        const float4 u = *reinterpret_cast<const float4 *>(Cs + b * D + c0);
        const float4 v = *reinterpret_cast<const float4 *>(Cs + b * D + c0 + 4);
        x[0] = fmaf(sv, u.x, x[0]); x[1] = fmaf(sv, u.y, x[1]); x[2] = fmaf(sv, u.z, x[2]); x[3] = fmaf(sv, u.w, x[3]);
        x[4] = fmaf(sv, v.x, x[4]); x[5] = fmaf(sv, v.y, x[5]); x[6] = fmaf(sv, v.z, x[6]); x[7] = fmaf(sv, v.w, x[7]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int cj = c0 + u;
        const int at = sidx(ra, cj);
        dst[at] = Ss[lr * D + cj];                           // S[ra][cj]
        dst[kSlot + at] = x[u] - in.G[mo + ra * D + cj];     // X[ra][cj]
        dst[2 * kSlot + at] = Cs[ra * D + cj];               // C[ra][cj]
    }
    if (tid < 16) {
        float y = 0.0f;
        for (int b = 0; b < D; ++b) y = fmaf(Ss[tid * D + b], ms[b], y);
        iaggV[static_cast<size_t>(bh) * 2 * D + r0 + tid] = y - in.h[static_cast<size_t>(bh) * D + r0 + tid];
        iaggV[static_cast<size_t>(bh) * 2 * D + D + r0 + tid] = ms[r0 + tid];
    }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

void geometry(int BH, int nc, int *P, int *L) {
    // about one workgroup per CU: P segments per head of L chunks each
    int p = (256 + BH - 1) / BH;
    if (p > nc) p = nc;
    if (p < 1) p = 1;
    *L = (nc + p - 1) / p;
    *P = (nc + *L - 1) / *L;
}

// The data region (the flags live in a region of their own, which holds
// nothing but launch epochs: flag_bytes)
struct Layout128 {
    size_t aggS, aggZ, aggC, aggV, iagg, iaggV, total;
};

size_t flag_bytes(int BH, int P) { return align256(2 * static_cast<size_t>(BH) * P * sizeof(uint32_t)); }

Layout128 layout(int BH, int P) {
    Layout128 L{};
    const size_t slots = static_cast<size_t>(BH) * P;
    const size_t pub = P > 1 ? slots * kSlot * sizeof(float) : 0;  // one published 128 x 128 slot per segment
    L.aggS = 0;
    L.aggZ = L.aggS + pub;
    L.aggC = L.aggZ + pub;
    L.aggV = L.aggC + pub;
    L.iagg = L.aggV + align256(P > 1 ? slots * 2 * D * sizeof(float) : 0);
    L.iaggV = L.iagg + static_cast<size_t>(BH) * 3 * kSlot * sizeof(float);
    L.total = L.iaggV + static_cast<size_t>(BH) * 2 * D * sizeof(float);
    return L;
}

}  // namespace

bool fused128_supported(const FwdProblem &p) {
    if (!(p.dtype == HLA_BF16 && p.d == 128 && p.dv == 128 && p.ridge == 0.0f && !p.normalize &&
          p.den == nullptr && p.n > 0))
        return false;
    if (p.init.S != nullptr || p.fin.S != nullptr) {
        // with a state, the looped body (segments beyond one per CU) spills
        // heavily: those calls take the generic path
        if (p.B < 1 || p.H < 1) return false;
        int P, L;
        geometry(p.B * p.H, (p.n + W - 1) / W, &P, &L);
        if (P > 1 && static_cast<long>(p.B) * p.H * P > kStateMaxSegs) return false;
    }
    const int nh = p.gam.per_head ? p.H : 1;
    for (int h = 0; h < nh; ++h)
        if (p.gam.g[h] < kMinGamma) return false;
    return true;
}

size_t fused128_flag_bytes(int BH, int n) {
    const int nc = (n + W - 1) / W;
    int P, L;
    geometry(BH, nc, &P, &L);
    return flag_bytes(BH, P);
}

size_t fused128_data_bytes(int BH, int n) {
    const int nc = (n + W - 1) / W;
    int P, L;
    geometry(BH, nc, &P, &L);
    return layout(BH, P).total;
}

hipError_t fused128_forward(const FwdProblem &p, uint32_t *ctrl, uint32_t *flags, void *data, hipStream_t st) {
    Args128 a{};
    a.H = p.H; a.n = p.n; a.BH = p.B * p.H;
    a.nc = (p.n + W - 1) / W;
    geometry(a.BH, a.nc, &a.P, &a.L);
    a.segs = a.BH * a.P;
    a.q = static_cast<const uint16_t *>(p.q);
    a.k = static_cast<const uint16_t *>(p.k);
    a.v = static_cast<const uint16_t *>(p.v);
    a.out = p.out;
    a.ctrl = ctrl;
    const Layout128 L = layout(a.BH, a.P);
    char *base = static_cast<char *>(data);
    a.flags = flags;
    a.aggS = reinterpret_cast<float *>(base + L.aggS);
    a.aggZ = reinterpret_cast<float *>(base + L.aggZ);
    a.aggC = reinterpret_cast<float *>(base + L.aggC);
    a.aggV = reinterpret_cast<float *>(base + L.aggV);
    a.gam = p.gam;
    const bool state = p.init.S != nullptr || p.fin.S != nullptr;
    if (p.init.S != nullptr) {
        float *iagg = reinterpret_cast<float *>(base + L.iagg), *iaggV = reinterpret_cast<float *>(base + L.iaggV);
        a.iagg = iagg;
        a.iaggV = iaggV;
        a.irho = p.init.rho;
        hipLaunchKernelGGL(k_fused128_init, dim3(a.BH, 8), dim3(256), 0, st, p.init, iagg, iaggV);
        const hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) return e0;
    }
    a.fin = p.fin;
    const int nh = p.gam.per_head ? p.H : 1;
    bool decay = false;
    for (int h = 0; h < nh; ++h) decay = decay || p.gam.g[h] != 1.0f;
    // when segments of a head wait on each other, workgroups take them by
    // ticket, at most one workgroup per CU (its LDS fills the CU)
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    // with one segment per head no workgroup waits on another, so the grid need
    // not be resident: one workgroup per segment, without the looped body
    const bool loop = a.segs > cus && a.P > 1;
    const dim3 grid(static_cast<unsigned>(loop ? cus : a.segs));
    const dim3 block(kThreads);
    if (state) {
        if (decay) {
            if (loop) hipLaunchKernelGGL((k_fused128<true, true, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((k_fused128<true, false, true>), grid, block, 0, st, a);
        } else {
            if (loop) hipLaunchKernelGGL((k_fused128<false, true, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((k_fused128<false, false, true>), grid, block, 0, st, a);
        }
    } else if (decay) {
        if (loop) hipLaunchKernelGGL((k_fused128<true, true, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_fused128<true, false, false>), grid, block, 0, st, a);
    } else {
        if (loop) hipLaunchKernelGGL((k_fused128<false, true, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_fused128<false, false, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace hla
