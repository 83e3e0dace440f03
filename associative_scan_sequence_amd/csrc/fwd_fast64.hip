// fwd_fast64.hip -- one-launch masked second-order HLA forward for
// d = dv = 64, chunk w = 64, bf16 q/k/v, on gfx950 MFMA: the numerator
// q_t^T ((S_t + lambda I) C_t - G_t), optionally the denominator and the
// ratio (no state input or output).
//
// Method (Higher-order Linear Attention, paperlayer.ai summary sec. 4 and 5)
// and per-chunk algebra: with the corrected carry X = S C - G, per chunk
// (e_t = g^(t+1), f_s = g^(L-1-s))
//   A = (Q K^T) o D_g o L,  U = diag(e) Q S0 + A K,  Us = diag(f^2) U,
//   P = (Q Us^T) o L / f_t^2,  out = P V + diag(e^2) Q X0,
//   S0 <- g^L S0 + K^T diag(f) K,  X0 <- g^2L X0 + Us^T V.
// The ridge adds first-order attention with the queries as keys, and the
// denominator is the same sum with every value equal to one (y = S m - h is
// carried like X, m like C):
//   R = (Q Q^T) o D_g o L,  P' = P + lambda R,
//   num = P' V + diag(e^2) Q X0 + lambda diag(e) Q C0,
//   den = P' 1 + diag(e^2) Q y0 + lambda diag(e) Q m0,   out = num or num / den,
//   C0 <- g^L C0 + Q^T diag(f) V,  m0 <- g^L m0 + Q^T f,  y0 <- g^2L y0 + Us^T 1.
// Precision: fp32 operands split into bf16 hi + lo, Us into three terms
// for the P product (q_t . Us_s cancels heavily when q_t is nearly
// orthogonal to S_s q_s; a two-term Us would leave ~2^-18 / cos(q, S q)).
// With the denominator, S0 in U and Us in y take three terms as well: the
// ratio magnifies the absolute error of den where |den| is small.
//
// Division of work.  A workgroup (eight waves) owns a segment of up to four
// consecutive chunks of one head.  Two roles per wave:
//  * slice role: wave v works on 32 tokens (two 16-token blocks) of chunk
//    v/2, so every operand it reads from LDS serves both blocks; the two
//    waves of a SIMD (v, v+4) take opposite halves of their chunks, pairing a
//    light and a heavy share of the triangular products: the scores, U, P
//    (and R), the local numerator, the denominator and the output;
//  * tile role: wave v owns tiles 2v, 2v+1 of a 64 x 64 moment (row block
//    v/2, column blocks 2(v%2), 2(v%2)+1), summed over every chunk of the
//    segment: the key moment S, the X increment (and C), and the carries
//    built from the aggregates other segments publish.  Waves 0-1 also own
//    the y vector, waves 2-3 the m vector (column sums taken on the MFMA
//    with a ones operand).  No partial sums are exchanged between waves,
//    and wave v of a segment reads only what wave v of its predecessors
//    wrote, so every wave publishes and waits on its own flags.
// Order per segment (LDS holds sixteen 64 x 64 bf16 tiles T, twenty with the
// ridge):
//   stage K_c -> T[c]; S_seg by tiles; publish S
//   carry-free A^T and Uloc^T = K^T A^T by slices (ridge: Q_c -> T[16+c]);
//   stage V_c -> T[4+c]
//   round 1: S0 of every chunk -> T[8+2c] (hi), T[9+2c] (lo) (with the
//   denominator a third term in T[c])
//   U, Us of every chunk -> Us hi, mid in T[8+2c], T[9+2c], lo in T[c]
//   Z_seg = sum_c decayed V_c^T Us_c by tiles (and C_seg, y_seg, m_seg);
//   publish
//   P (P') and the local numerator by slices, while round 2 travels
//   round 2: X0 of every chunk -> T[8+2c], T[9+2c] (C0 -> T[c], T[4+c],
//   y0 and m0 -> a vector area); out = num + e^2 Q X0 (+ the ridge and
//   denominator terms)
// Segment s = p * BH + head.  When a head has several segments, workgroups
// take segments from a ticket counter in increasing order, so a segment is
// only ever held by a running workgroup and waits only on smaller segments of
// its head, which were taken earlier by running workgroups that wait on
// smaller ones still: every wait ends, whatever other streams keep resident.
// Aggregates and flags are device-coherent (sc1) accesses.  A wait that still
// gives up (spin limit, or forced from the host) makes the carry it waited
// for NaN, so no output is ever a silently wrong number.
#include "fast64_common.h"

namespace hla {
namespace {

template <int V>
struct IC {  // an int as a type, to instantiate a lambda for each half
    static constexpr int value = V;
};

constexpr int kFThreads = 512;
constexpr int kFMaxL = 4;   // chunks per segment
constexpr int kWaves = 8;

constexpr int kVecSlot = 128;  // floats per published vector pair (y, m)

struct FastArgs {
    int H, n, nc, P, L, BH, segs;  // segs = BH * P
    const uint16_t *q, *k, *v;
    const uint16_t *vl;  // VS: the values' lo half (values = v + vl)
    float *out, *den;  // den may be null
    float ridge;
    uint32_t *ctrl;   // control block (epoch, done counter, ticket, counters)
    uint32_t *flags;  // [BH * P][2 rounds][8 waves] at kFlagStride words: publication epoch
    float *aggS, *aggX, *aggC;  // [BH * P][16 tiles][64 lanes][4]
    float *aggV;                // [BH * P][kVecSlot]: y increment, then m increment
    GammaTab gam;
    // STATE variants only:
    const float *iagg;   // [BH][3][4096] the initial state's S, X = S C - G and C in the slot
                         // layout of the aggregates, or null (zero initial state)
    const float *iaggV;  // [BH][kVecSlot] its y = S m - h, then m
    const float *irho;   // initial rho [BH] or null (read as 1)
    hla_state fin;       // final state; fin.S null: not requested
};

template <int NT>
struct FastSmem {
    __bf16 T[NT][kTileElems];
};

// wave v's two tiles <-> a 16 KB slot: tile i at tile index 2v+i, lane l's
// 16 bytes at byte ((2v+i) * 64 + l) * 16 (device-coherent stores)
__device__ __forceinline__ void put_tiles(const float *slot, int v, int l, const f32x4 (&x)[2]) {
    const __amdgpu_buffer_rsrc_t rs = slot_rsrc(slot);
#pragma unroll
    for (int i = 0; i < 2; ++i) __builtin_amdgcn_raw_buffer_store_b128(x[i], rs, ((2 * v + i) * 64 + l) * 16, 0, kSc1);
}

// acc += sum over n slots of scale[s] * (wave v's tiles of slot s); all
// loads (device-coherent) are issued before the first add
template <int NB>
__device__ __forceinline__ void add_tiles(f32x4 (&acc)[2], const float *const (&slots)[NB],
                                          const float (&scale)[NB], int n, int v, int l) {
    f32x4 x[NB][2];
#pragma unroll
    for (int s = 0; s < NB; ++s)
        if (s < n) {
            const __amdgpu_buffer_rsrc_t rs = slot_rsrc(slots[s]);
#pragma unroll
            for (int i = 0; i < 2; ++i) x[s][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, ((2 * v + i) * 64 + l) * 16, 0, kSc1);
        }
#pragma unroll
    for (int s = 0; s < NB; ++s)
        if (s < n) {
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[i] += scale[s] * x[s][i];
        }
}

// one float per lane into / out of a published slot (device-coherent)
__device__ __forceinline__ void put_float(const float *slot, int idx, float x) {
    const __amdgpu_buffer_rsrc_t rs = slot_rsrc(slot);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, 4 * idx, 0, kSc1);
}

__device__ __forceinline__ float get_float(const float *slot, int idx) {
    const __amdgpu_buffer_rsrc_t rs = slot_rsrc(slot);
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * idx, 0, kSc1));
}

// RIDGE: lambda terms; DEN: the denominator (written to den when it is
// given); NORM: out = num / den.  STATE: an initial state enters every carry
// (a.iagg, prepared by k_fast64_init), and a final state is formed when
// a.fin.S is set.  A state has all of S, C, m, G, h, so the STATE variants
// carry C, m and y as the ridge and denominator variants do, whether or not
// the ridge and denominator themselves are asked for.  VS (plain numerator
// only): the values come as a bf16 pair v + vl (an fp32 intermediate split in
// two); products with the values take hi * x + lo * x_hi, the lo half staged
// in T[16+c].
template <bool DECAY, bool LOOP, bool RIDGE, bool DEN, bool NORM, bool STATE, bool VS = false>
__global__ __launch_bounds__(kFThreads, 1) void k_fast64(FastArgs a) {
    static_assert(!NORM || DEN, "the ratio needs the denominator");
    // the moments C and m (as the ridge needs them), and y (as the denominator does)
    constexpr bool CM = RIDGE || STATE, YV = DEN || STATE;
    static_assert(!VS || !(CM || YV), "value pairs only for the plain numerator");
    constexpr bool MV = RIDGE && DEN;  // the query mass m only enters the ridge part of den
    __shared__ FastSmem<(CM || VS) ? 20 : 16> sm;
    const int tid = threadIdx.x;
    // launch epoch, read by every wave: read now, first needed when the
    // segment sum is published
    uint32_t ep_raw = 0;
    if ((tid & 63) == 0) ep_raw = __hip_atomic_load(&a.ctrl[kLine + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t epoch = 0;
    const u32x4 z4 = u32x4{0u, 0u, 0u, 0u};
    const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
    float lg = 0.0f;
    auto gp = [&](float e) { return DECAY ? __builtin_amdgcn_exp2f(e * lg) : 1.0f; };  // g^e
    auto gpl = [&](float el) { return DECAY ? __builtin_amdgcn_exp2f(el) : 1.0f; };   // g^e from e log2(g)

    auto seg_body = [&](const int seg) __attribute__((always_inline)) {
        // lane indices, laundered per pass in the looped launch so that the
        // address arithmetic built on them is not hoisted out of the loop
        int tid_l = static_cast<int>(threadIdx.x);
        if constexpr (LOOP) asm volatile("" : "+v"(tid_l));
        const int wave = tid_l >> 6, l = tid_l & 63, r = l & 15, g = l >> 4;
        const int grp = wave >> 2, wt = tid_l & 255;  // staging: group grp stages chunks 2grp, 2grp+1
        // slice role: chunk sc, token blocks 2hh and 2hh+1 (the two waves of a
        // SIMD take opposite halves of the triangular work)
        const int sc = wave >> 1, hh = (wave ^ (wave >> 2)) & 1;
        const int t0 = 32 * hh + r;  // this lane's token in block 2hh; t0 + 16 in block 2hh+1
        const int tb = wave >> 1, cb = 2 * (wave & 1);  // tile role: row block, first column block

        // ---- global loads: keys now; queries once the key moment is published;
        // values once the queries are in.  The key moment and its flag are on
        // every segment's critical path, and the flag must wait for all of the
        // wave's outstanding memory operations, so nothing else is in flight
        // before it.  (With the ridge the queries come with the keys and the
        // values follow the flag: later query loads made those variants spill.)
        // Unconditional (rows past the chunk read the head's first row), masked
        // where used.
        u32x4 kx[2][2], qx[2][2], vx[2][2], vlx[2][2];
        auto chunk_rows = [&](int sg_, int jj, int &Lc_, size_t &tok0_, size_t &head_) {
            const int bh_ = sg_ % a.BH, p_ = sg_ / a.BH;
            head_ = static_cast<size_t>(bh_) * a.n;
            const int c0_ = p_ * a.L, Lseg_ = min(a.L, a.nc - c0_), j = 2 * grp + jj;
            Lc_ = j < Lseg_ ? min(W, a.n - (c0_ + j) * W) : 0;
            tok0_ = head_ + static_cast<size_t>(c0_ + j) * W;
        };
        auto issue_k = [&](int sg_) __attribute__((always_inline)) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                int Lc_;
                size_t tok0_, head_;
                chunk_rows(sg_, jj, Lc_, tok0_, head_);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int row = (wt + 256 * u) >> 3, cg = (wt + 256 * u) & 7;
                    const size_t src = row < Lc_ ? tok0_ + row : head_;
                    kx[jj][u] = *reinterpret_cast<const u32x4 *>(a.k + src * W + cg * 8);
                }
            }
        };
        auto issue_q = [&](int sg_) __attribute__((always_inline)) {
            {
                const int bh_ = sg_ % a.BH, p_ = sg_ / a.BH;
                const size_t head_ = static_cast<size_t>(bh_) * a.n;
                const int c0_ = p_ * a.L, Lseg_ = min(a.L, a.nc - c0_);
                const int Lc_ = sc < Lseg_ ? min(W, a.n - (c0_ + sc) * W) : 0;
                const size_t tok0_ = head_ + static_cast<size_t>(c0_ + sc) * W;
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const int tt = t0 + 16 * i;
                        const size_t src = tt < Lc_ ? tok0_ + tt : head_;
                        qx[i][ks] = *reinterpret_cast<const u32x4 *>(a.q + src * W + 32 * ks + 8 * g);
                    }
            }
        };
        auto issue_v = [&](int sg_) __attribute__((always_inline)) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                int Lc_;
                size_t tok0_, head_;
                chunk_rows(sg_, jj, Lc_, tok0_, head_);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int row = (wt + 256 * u) >> 3, cg = (wt + 256 * u) & 7;
                    const size_t src = row < Lc_ ? tok0_ + row : head_;
                    vx[jj][u] = *reinterpret_cast<const u32x4 *>(a.v + src * W + cg * 8);
                    if constexpr (VS) vlx[jj][u] = *reinterpret_cast<const u32x4 *>(a.vl + src * W + cg * 8);
                }
            }
        };
        issue_k(seg);
        if constexpr (RIDGE) issue_q(seg);
        const int bh = seg % a.BH, p = seg / a.BH;
        lg = DECAY ? log2f(head_gamma(a.gam, bh % a.H)) : 0.0f;
        // Per-element decay exponents are formed as fma(constant, log2 g, lane base):
        // in a masked 16 x 16 tile t - s = (block offset - e) + (r - 4g), and a
        // transposed operand's token is 32ks + 8g + e (+4).  The bases are formed
        // where they are used (kept from being merged into one long-lived value).
        auto lane_base = [&](int off) __attribute__((always_inline)) {
            if (!DECAY) return 0.0f;
            asm volatile("" : "+v"(off));
            return static_cast<float>(off) * lg;
        };
        const int c0 = p * a.L;
        const int Lseg = min(a.L, a.nc - c0);  // chunks in this segment (1..4)
        auto chunk_len = [&](int j) { return min(W, a.n - (c0 + j) * W); };
        int lc_of[2];  // tokens in staged chunk 2grp+jj (0 if none)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) lc_of[jj] = 2 * grp + jj < Lseg ? chunk_len(2 * grp + jj) : 0;
        const int Lcs = sc < Lseg ? chunk_len(sc) : 0;  // tokens in the slice chunk (0 if none)
        int lcc[kFMaxL];  // tokens per chunk of the segment, 0 past its end (absent
                          // chunks have zero key, value and Us tiles, so the tile
                          // sums below need no branch on them)
#pragma unroll
        for (int c = 0; c < kFMaxL; ++c) lcc[c] = c < Lseg ? chunk_len(c) : 0;
        const size_t slot = static_cast<size_t>(bh) * a.P + p;
        // the last segment of a head has no readers, unless a final state is formed from it
        const bool want_fin = STATE && a.fin.S != nullptr;
        const bool publish = p + 1 < a.P || want_fin;
        const bool fin_seg = want_fin && p + 1 == a.P;  // this workgroup writes the head's final state

        // ---- stage key rows
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int row = (wt + 256 * u) >> 3, cg = (wt + 256 * u) & 7;
                st16(sm.T[2 * grp + jj], row, cg * 8, row < lc_of[jj] ? kx[jj][u] : z4);
            }
        __syncthreads();

        // ================= phase A (tiles): key moments ===========================
        // spre[c] = moment of chunks 0..c-1 at chunk c's start; srun ends as S_seg.
        // Tile (a = 16tb+4g+e, b = 16(cb+i)+r) = sum_s K[s][a] f_s K[s][b].
        f32x4 spre[kFMaxL][2], srun[2] = {zero4, zero4};
#pragma unroll
        for (int c = 0; c < kFMaxL; ++c) {
#pragma unroll
            for (int i = 0; i < 2; ++i) spre[c][i] = srun[i];
            const int Lc = lcc[c];
            f32x4 acc[2] = {zero4, zero4};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int rb = 32 * ks + 8 * g;
                const bf16x8 ka = tr8(sm.T[c], rb, rb + 4, 16 * tb, r);
                bf16x8 kb[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) kb[i] = tr8(sm.T[c], rb, rb + 4, 16 * (cb + i), r);
                if (!DECAY) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) acc[i] = mfma(ka, kb[i], acc[i]);
                } else {
                    // f_s = g^(Lc - 1 - s) for the tokens s = 32ks + 8g + e (+4)
                    const float base = fmaf(static_cast<float>(Lc - 1), lg, lane_base(-8 * g));
                    f32x4 x0, x1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x0[e] = gpl(fmaf(static_cast<float>(-(32 * ks + e)), lg, base)) * static_cast<float>(ka[e]);
                        x1[e] = gpl(fmaf(static_cast<float>(-(32 * ks + 4 + e)), lg, base)) * static_cast<float>(ka[4 + e]);
                    }
                    bf16x8 h, lo;
                    pair_operand(x0, x1, h, lo);
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        acc[i] = mfma(h, kb[i], acc[i]);
                        acc[i] = mfma(lo, kb[i], acc[i]);
                    }
                }
            }
            const float rho = gp(static_cast<float>(Lc));
#pragma unroll
            for (int i = 0; i < 2; ++i) srun[i] = rho * srun[i] + acc[i];
        }
        auto flag_of = [&](size_t sl, int round) { return &a.flags[((sl * 2 + round) * kWaves + wave) * kFlagStride]; };
        if (publish) {
            put_tiles(a.aggS + slot * 4096, wave, l, srun);
            wait_stores();
            if (l == 0) set_flag(flag_of(slot, 0), epoch);
        }
        if constexpr (RIDGE) issue_v(seg);
        else issue_q(seg);

        bf16x8 qn[2][2];  // q of token t0 + 16i, features 32ks+8g..: B operand
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) qn[i][ks] = __builtin_bit_cast(bf16x8, t0 + 16 * i < Lcs ? qx[i][ks] : z4);
        if constexpr (!RIDGE) {
            // the value loads go out once the queries (first and last load) are in
            asm volatile("" : "+v"(qn[0][0]), "+v"(qn[1][1])::"memory");
            issue_v(seg);
        }
        if constexpr (CM) {  // query rows of the slice chunk (zero past its end), read after round 1
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    st16(sm.T[16 + sc], t0 + 16 * i, 32 * ks + 8 * g, __builtin_bit_cast(u32x4, qn[i][ks]));
        }

        // ================= carry-free slice work ====================================
        // A^T tiles (rows s, cols t) of both token blocks, then Uloc^T = K^T A^T
        // (rows b, cols t).  Block i (tokens 16(2hh+i)..) needs s-blocks <= 2hh+i;
        // operands read from LDS serve both blocks.
        f32x4 uloc[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) uloc[i][bb] = zero4;
        auto carry_free = [&](auto hc) __attribute__((always_inline)) {
            constexpr int HH = decltype(hc)::value;
            const float lg_rg = lane_base(r - 4 * g);
            f32x4 at[2][4];
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                at[0][ib] = at[1][ib] = zero4;
                if (ib <= 2 * HH + 1) {
                    const bf16x8 k0 = ld8(sm.T[sc], 16 * ib + r, 8 * g), k1 = ld8(sm.T[sc], 16 * ib + r, 32 + 8 * g);
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        if (ib <= 2 * HH + i) {
                            at[i][ib] = mfma(k1, qn[i][1], mfma(k0, qn[i][0], zero4));
                            // g^(t - s), t = 32HH + 16i + r, s = 16ib + 4g + e; s > t only in the diagonal tile
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float dec = gpl(fmaf(static_cast<float>(32 * HH + 16 * i - 16 * ib - e), lg, lg_rg));
                                if (ib == 2 * HH + i) at[i][ib][e] = 4 * g + e <= r ? dec * at[i][ib][e] : 0.0f;
                                else at[i][ib][e] *= dec;
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (2 * ks <= 2 * HH + 1) {
                    bf16x8 kt[4];
#pragma unroll
                    for (int bb = 0; bb < 4; ++bb) kt[bb] = tr8(sm.T[sc], 32 * ks + 4 * g, 32 * ks + 16 + 4 * g, 16 * bb, r);
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        if (2 * ks <= 2 * HH + i) {
                            bf16x8 ah, al;
                            pair_operand(at[i][2 * ks], at[i][2 * ks + 1], ah, al);
#pragma unroll
                            for (int bb = 0; bb < 4; ++bb) {
                                uloc[i][bb] = mfma(kt[bb], ah, uloc[i][bb]);
                                uloc[i][bb] = mfma(kt[bb], al, uloc[i][bb]);
                            }
                        }
                    }
                }
            }
        };
        if (Lcs > 0) {
            if (hh) carry_free(IC<1>{});
            else carry_free(IC<0>{});
        }
        // ---- value rows (read after the next barrier)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int row = (wt + 256 * u) >> 3, cg = (wt + 256 * u) & 7;
                st16(sm.T[4 + 2 * grp + jj], row, cg * 8, row < lc_of[jj] ? vx[jj][u] : z4);
                if constexpr (VS) st16(sm.T[16 + 2 * grp + jj], row, cg * 8, row < lc_of[jj] ? vlx[jj][u] : z4);
            }

        // ---- carry = sum over earlier segments pp of g^(pw * gap) * (wave's
        // tiles of agg[pp]), gap = tokens between; waits on this wave's flags only
        const int seg_tokens = a.L * W;
        // true when a wait of this wave gave up: the carry it sums is then
        // made NaN, so every output built on it is NaN (never a silently
        // wrong number), here and in the later segments that read it
        auto wait_round = [&](int round) -> bool {
            bool failed = false;
            for (int pp = l; pp < p; pp += 64)
                if (!wait_flag(flag_of(static_cast<size_t>(bh) * a.P + pp, round), epoch, a.ctrl + kSpinWord)) {
                    __hip_atomic_fetch_add(&a.ctrl[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    failed = true;
                }
            return __builtin_amdgcn_ballot_w64(failed) != 0;
        };
        auto poison = [&](f32x4 (&acc)[2]) {
            const float nan = __builtin_nanf("");
            acc[0] = acc[1] = f32x4{nan, nan, nan, nan};
        };
        // (STATE: plus the initial state's part `kind` (0 S, 1 X, 2 C), decayed
        // over the p * seg_tokens tokens before the segment)
        auto carry_tiles = [&](f32x4 (&acc)[2], const float *agg, int pw, int kind) {
            constexpr int NB = 8;
            acc[0] = acc[1] = zero4;
            for (int p0 = 0; p0 < p; p0 += NB) {
                const float *slots[NB];
                float scale[NB];
#pragma unroll
                for (int s2 = 0; s2 < NB; ++s2) {
                    const int pp = min(p0 + s2, p - 1);
                    slots[s2] = agg + (static_cast<size_t>(bh) * a.P + pp) * 4096;
                    scale[s2] = gp(static_cast<float>(pw * (p - 1 - pp) * seg_tokens));
                }
                const int cnt = min(NB, p - p0);
                add_tiles<NB>(acc, slots, scale, cnt, wave, l);
            }
            if constexpr (STATE) {
                if (a.iagg != nullptr) {
                    const float *slots[1] = {a.iagg + (static_cast<size_t>(bh) * 3 + kind) * 4096};
                    const float scale[1] = {gp(static_cast<float>(pw * p * seg_tokens))};
                    add_tiles<1>(acc, slots, scale, 1, wave, l);
                }
            }
            (void)kind;
        };
        // the same for entries off + 16(cb+i) + r of the published vectors
        auto carry_vec = [&](float (&acc)[2], int off, int pw) {
            constexpr int NB = 8;
            acc[0] = acc[1] = 0.0f;
            for (int p0 = 0; p0 < p; p0 += NB) {
                float x[NB][2];
#pragma unroll
                for (int s2 = 0; s2 < NB; ++s2) {
                    const float *vs = a.aggV + (static_cast<size_t>(bh) * a.P + min(p0 + s2, p - 1)) * kVecSlot;
#pragma unroll
                    for (int i = 0; i < 2; ++i) x[s2][i] = get_float(vs, off + 16 * (cb + i) + r);
                }
#pragma unroll
                for (int s2 = 0; s2 < NB; ++s2)
                    if (p0 + s2 < p) {
                        const float sc2 = gp(static_cast<float>(pw * (p - 1 - (p0 + s2)) * seg_tokens));
#pragma unroll
                        for (int i = 0; i < 2; ++i) acc[i] += sc2 * x[s2][i];
                    }
            }
            if constexpr (STATE) {
                if (a.iaggV != nullptr) {
                    const float *vs = a.iaggV + static_cast<size_t>(bh) * kVecSlot;
                    const float sc2 = gp(static_cast<float>(pw * p * seg_tokens));
#pragma unroll
                    for (int i = 0; i < 2; ++i) acc[i] += sc2 * get_float(vs, off + 16 * (cb + i) + r);
                }
            }
        };
        // STATE, the head's last segment: the state at the end of the sequence is
        // g^(pw len) * carry + this segment's own published aggregate (len = the
        // segment's tokens).  The own aggregate is loaded before the wait for the
        // carries, so that its latency overlaps theirs (after them in the ridge
        // variants, where the registers held across the wait would spill).
        constexpr bool kEarlyOwn = !RIDGE;
        auto own_tiles = [&](f32x4 (&x)[2], const float *agg) {
            const __amdgpu_buffer_rsrc_t rs = slot_rsrc(agg + slot * 4096);
#pragma unroll
            for (int i = 0; i < 2; ++i) x[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, ((2 * wave + i) * 64 + l) * 16, 0, kSc1);
        };
        const float dl1 = gp(static_cast<float>(a.n - p * seg_tokens));

        // ================= round 1: S0 of every chunk -> LDS ========================
        {
            f32x4 s0seg[2], own_s[2];
            if constexpr (STATE && kEarlyOwn) {
                if (fin_seg) own_tiles(own_s, a.aggS);
            }
            const bool bad = wait_round(0);
            carry_tiles(s0seg, a.aggS, 1, 0);
            if (bad) poison(s0seg);
            if constexpr (STATE) {
                if (fin_seg) {  // final S[a = 16tb+4g+e][b = 16(cb+i)+r]
                    if constexpr (!kEarlyOwn) own_tiles(own_s, a.aggS);
                    float *S = a.fin.S + static_cast<size_t>(bh) * W * W;
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const f32x4 sf = dl1 * s0seg[i] + own_s[i];
#pragma unroll
                        for (int e = 0; e < 4; ++e) S[(16 * tb + 4 * g + e) * W + 16 * (cb + i) + r] = sf[e];
                    }
                }
            }
            // With the denominator, S0 takes a third term (in the key tile: no
            // key is read after the carry-free stage).  The ratio amplifies the
            // absolute error of den where |den| is small, and a two-term S0 in U
            // is by far its largest source.
            if constexpr (DEN) __syncthreads();
#pragma unroll
            for (int c = 0; c < kFMaxL; ++c) {
                if (c < Lseg) {
                    const float d1 = gp(static_cast<float>(W * c));
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        // lane holds S0[a = 16tb+4g+e][b = 16(cb+i)+r]; tile rows b
                        if constexpr (DEN) {
                            bf16x4 h, mid, lo;
                            split3(d1 * s0seg[i] + spre[c][i], h, mid, lo);
                            st4(sm.T[8 + 2 * c], 16 * (cb + i) + r, 16 * tb + 4 * g, h);
                            st4(sm.T[9 + 2 * c], 16 * (cb + i) + r, 16 * tb + 4 * g, mid);
                            st4(sm.T[c], 16 * (cb + i) + r, 16 * tb + 4 * g, lo);
                        } else {
                            bf16x4 h, lo;
                            split4(d1 * s0seg[i] + spre[c][i], h, lo);
                            st4(sm.T[8 + 2 * c], 16 * (cb + i) + r, 16 * tb + 4 * g, h);
                            st4(sm.T[9 + 2 * c], 16 * (cb + i) + r, 16 * tb + 4 * g, lo);
                        }
                    }
                }
            }
        }
        __syncthreads();  // S0 and value tiles ready

        // ================= U and Us of the slice ===================================
        f32x4 usv[2][4];  // Us^T[b = 16bb+4g+e][t0 + 16i]
        if (Lcs > 0) {
            f32x4 acc[2][4];
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                acc[0][bb] = acc[1][bb] = zero4;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8 sh = ld8(sm.T[8 + 2 * sc], 16 * bb + r, 32 * ks + 8 * g);
                    const bf16x8 sl = ld8(sm.T[9 + 2 * sc], 16 * bb + r, 32 * ks + 8 * g);
                    bf16x8 sx;
                    if constexpr (DEN) sx = ld8(sm.T[sc], 16 * bb + r, 32 * ks + 8 * g);
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        acc[i][bb] = mfma(sh, qn[i][ks], acc[i][bb]);
                        acc[i][bb] = mfma(sl, qn[i][ks], acc[i][bb]);
                        if constexpr (DEN) acc[i][bb] = mfma(sx, qn[i][ks], acc[i][bb]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tt = t0 + 16 * i;
                const float e = gp(static_cast<float>(tt + 1));
                const float f2 = tt < Lcs ? gp(static_cast<float>(2 * (Lcs - 1 - tt))) : 0.0f;
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) usv[i][bb] = f2 * (e * acc[i][bb] + uloc[i][bb]);
            }
        }
        __syncthreads();  // S0 reads done: their tiles take Us
        if (Lcs > 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    bf16x4 h, mid, lo;
                    split3(usv[i][bb], h, mid, lo);
                    st4(sm.T[8 + 2 * sc], t0 + 16 * i, 16 * bb + 4 * g, h);
                    st4(sm.T[9 + 2 * sc], t0 + 16 * i, 16 * bb + 4 * g, mid);
                    st4(sm.T[sc], t0 + 16 * i, 16 * bb + 4 * g, lo);
                }
        } else {  // an absent chunk: zero Us hi, mid (its value tile is zero too)
            const bf16x4 z = __builtin_bit_cast(bf16x4, uint64_t{0});
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    st4(sm.T[8 + 2 * sc], t0 + 16 * i, 16 * bb + 4 * g, z);
                    st4(sm.T[9 + 2 * sc], t0 + 16 * i, 16 * bb + 4 * g, z);
                }
        }
        __syncthreads();  // every Us row ready

        // ================= Z_seg (tiles): the segment's X increment ================
        // xpre[c] = increment of chunks 0..c-1 at chunk c's start; xrun ends as Z.
        // Tile X^T (j = 16tb+4g+e, a = 16(cb+i)+r) = sum_s V[s][j] Us[s][a].
        // Ridge: C^T (same tiles) = sum_s V[s][j] f_s Q[s][a].  Vectors (row 0
        // of an accumulator, lanes 0-15, from a ones operand in row 0): waves
        // 0-1 y[a] = sum_s Us[s][a] (the three-term Us, lo in T[c]), waves 2-3
        // m[a] = sum_s f_s Q[s][a].
        const int tbu = __builtin_amdgcn_readfirstlane(tb);
        const bool yw = YV && tbu == 0, mw = (MV || STATE) && tbu == 1;
        const int voff = tbu == 0 ? 0 : 64;  // the vector's place in a published pair
        bf16x8 ones;
#pragma unroll
        for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(r == 0 ? 1.0f : 0.0f);
        f32x4 xpre[kFMaxL][2], xrun[2] = {zero4, zero4};
        f32x4 cpre[kFMaxL][2], crun[2] = {zero4, zero4};
        float vpre[kFMaxL][2];
        f32x4 vrun[2] = {zero4, zero4};
#pragma unroll
        for (int c = 0; c < kFMaxL; ++c) {
#pragma unroll
            for (int i = 0; i < 2; ++i) xpre[c][i] = xrun[i];
            const float rho = gp(static_cast<float>(lcc[c])), rho2 = gp(static_cast<float>(2 * lcc[c]));
#pragma unroll
            for (int i = 0; i < 2; ++i) xrun[i] *= rho2;
            if constexpr (CM) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    cpre[c][i] = crun[i];
                    crun[i] *= rho;
                }
            }
            if constexpr (YV) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    vpre[c][i] = vrun[i][0];
                    vrun[i] *= yw ? rho2 : rho;
                }
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int rb = 32 * ks + 8 * g;
                const bf16x8 vt = tr8(sm.T[4 + c], rb, rb + 4, 16 * tb, r);
                bf16x8 vtl;
                if constexpr (VS) vtl = tr8(sm.T[16 + c], rb, rb + 4, 16 * tb, r);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const bf16x8 uh = tr8(sm.T[8 + 2 * c], rb, rb + 4, 16 * (cb + i), r);
                    const bf16x8 um = tr8(sm.T[9 + 2 * c], rb, rb + 4, 16 * (cb + i), r);
                    xrun[i] = mfma(vt, uh, xrun[i]);
                    xrun[i] = mfma(vt, um, xrun[i]);
                    if constexpr (VS) xrun[i] = mfma(vtl, uh, xrun[i]);
                    if (yw) {  // all three terms: den cancels more than num near small values
                        vrun[i] = mfma(ones, uh, vrun[i]);
                        vrun[i] = mfma(ones, um, vrun[i]);
                        vrun[i] = mfma(ones, tr8(sm.T[c], rb, rb + 4, 16 * (cb + i), r), vrun[i]);
                    }
                }
                if constexpr (CM) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const bf16x8 qt = tr8(sm.T[16 + c], rb, rb + 4, 16 * (cb + i), r);
                        if (!DECAY) {
                            crun[i] = mfma(vt, qt, crun[i]);
                            if (mw) vrun[i] = mfma(ones, qt, vrun[i]);
                        } else {
                            const float base = fmaf(static_cast<float>(lcc[c] - 1), lg, lane_base(-8 * g));
                            f32x4 x0, x1;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                x0[e] = gpl(fmaf(static_cast<float>(-(32 * ks + e)), lg, base)) * static_cast<float>(qt[e]);
                                x1[e] = gpl(fmaf(static_cast<float>(-(32 * ks + 4 + e)), lg, base)) * static_cast<float>(qt[4 + e]);
                            }
                            bf16x8 h, lo;
                            pair_operand(x0, x1, h, lo);
                            crun[i] = mfma(vt, h, crun[i]);
                            crun[i] = mfma(vt, lo, crun[i]);
                            if (mw) {
                                vrun[i] = mfma(ones, h, vrun[i]);
                                vrun[i] = mfma(ones, lo, vrun[i]);
                            }
                        }
                    }
                }
            }
        }
        if (publish) {
            put_tiles(a.aggX + slot * 4096, wave, l, xrun);
            if constexpr (CM) put_tiles(a.aggC + slot * 4096, wave, l, crun);
            if ((yw || mw) && l < 16) {
#pragma unroll
                for (int i = 0; i < 2; ++i) put_float(a.aggV + slot * kVecSlot, voff + 16 * (cb + i) + r, vrun[i][0]);
            }
            wait_stores();
            if (l == 0) set_flag(flag_of(slot, 1), epoch);
        }

        // ================= P and the local numerator (slice) ======================
        // P^T[s][t] = (Us_s . q_t) / f_t^2 for s <= t (ridge: + lambda g^(t-s)
        // q_s . q_t);  num^T[j][t] = sum_s V[s][j] P[t][s]
        const float lam = a.ridge;
        f32x4 num[2][4];
        float dl[2] = {0.0f, 0.0f};  // this lane's part of sum_s P[t][s] (denominator)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) num[i][jb] = zero4;
        auto p_num = [&](auto hc) __attribute__((always_inline)) {
            constexpr int HH = decltype(hc)::value;
            const float lg_rg = RIDGE ? lane_base(r - 4 * g) : 0.0f;
            f32x4 pt[2][4], rt[2][4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                pt[0][sb] = pt[1][sb] = zero4;
                if constexpr (RIDGE) rt[0][sb] = rt[1][sb] = zero4;
                if (sb <= 2 * HH + 1) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        const bf16x8 u1 = ld8(sm.T[8 + 2 * sc], 16 * sb + r, 32 * kb + 8 * g);
                        const bf16x8 u2 = ld8(sm.T[9 + 2 * sc], 16 * sb + r, 32 * kb + 8 * g);
                        const bf16x8 u3 = ld8(sm.T[sc], 16 * sb + r, 32 * kb + 8 * g);
                        bf16x8 qs;
                        if constexpr (RIDGE) qs = ld8(sm.T[16 + sc], 16 * sb + r, 32 * kb + 8 * g);
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            if (sb <= 2 * HH + i) {
                                pt[i][sb] = mfma(u1, qn[i][kb], pt[i][sb]);
                                pt[i][sb] = mfma(u2, qn[i][kb], pt[i][sb]);
                                pt[i][sb] = mfma(u3, qn[i][kb], pt[i][sb]);
                                if constexpr (RIDGE) rt[i][sb] = mfma(qs, qn[i][kb], rt[i][sb]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tt = 32 * HH + 16 * i + r;
                const float inv_f2 = tt < Lcs ? gp(static_cast<float>(-2 * (Lcs - 1 - tt))) : 0.0f;
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) {
                    if (sb > 2 * HH + i) continue;  // tiles past the diagonal stay zero
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // s = 16sb + 4g + e; s > t only in the diagonal tile
                        float x = inv_f2 * pt[i][sb][e];
                        if constexpr (RIDGE)
                            x += lam * gpl(fmaf(static_cast<float>(32 * HH + 16 * i - 16 * sb - e), lg, lg_rg)) * rt[i][sb][e];
                        if (sb == 2 * HH + i) x = 4 * g + e <= r ? x : 0.0f;
                        pt[i][sb][e] = x;
                        if constexpr (DEN) dl[i] += x;
                    }
                }
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (2 * ks <= 2 * HH + 1) {
                    bf16x8 vt[4], vtl[4];
#pragma unroll
                    for (int jb = 0; jb < 4; ++jb) {
                        vt[jb] = tr8(sm.T[4 + sc], 32 * ks + 4 * g, 32 * ks + 16 + 4 * g, 16 * jb, r);
                        if constexpr (VS) vtl[jb] = tr8(sm.T[16 + sc], 32 * ks + 4 * g, 32 * ks + 16 + 4 * g, 16 * jb, r);
                    }
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        if (2 * ks <= 2 * HH + i) {
                            bf16x8 ph, pl;
                            pair_operand(pt[i][2 * ks], pt[i][2 * ks + 1], ph, pl);
#pragma unroll
                            for (int jb = 0; jb < 4; ++jb) {
                                num[i][jb] = mfma(vt[jb], ph, num[i][jb]);
                                num[i][jb] = mfma(vt[jb], pl, num[i][jb]);
                                if constexpr (VS) num[i][jb] = mfma(vtl[jb], ph, num[i][jb]);
                            }
                        }
                    }
                }
            }
        };
        if (Lcs > 0) {
            if (hh) p_num(IC<1>{});
            else p_num(IC<0>{});
        }

        // ================= round 2: X0 of every chunk -> LDS ========================
        // (ridge: C0 -> T[c] hi, T[4+c] lo; denominator: y0 and m0 of chunk c
        // at vec[c * kVecSlot], the m0 half at +64)
        f32x4 x0seg[2], c0seg[2];
        float v0seg[2];
        f32x4 own_x[2], own_c[2];
        float own_v[2];
        auto own_round2 = [&]() {
            own_tiles(own_x, a.aggX);
            own_tiles(own_c, a.aggC);
            if (yw || mw) {
#pragma unroll
                for (int i = 0; i < 2; ++i) own_v[i] = get_float(a.aggV + slot * kVecSlot, voff + 16 * (cb + i) + r);
            }
        };
        if constexpr (STATE && kEarlyOwn) {
            if (fin_seg) own_round2();
        }
        const bool bad2 = wait_round(1);
        carry_tiles(x0seg, a.aggX, 2, 1);
        if constexpr (CM) carry_tiles(c0seg, a.aggC, 1, 2);
        if (yw || mw) carry_vec(v0seg, voff, yw ? 2 : 1);
        if (bad2) {
            poison(x0seg);
            if constexpr (CM) poison(c0seg);
            v0seg[0] = v0seg[1] = __builtin_nanf("");
        }
        if constexpr (STATE) {
            // final X (into fin.G, which the finish step below turns into G =
            // S C - X) and C at [a = 16(cb+i)+r][j = 16tb+4g+e]; final y (into
            // fin.h, likewise) and m
            if (fin_seg) {
                if constexpr (!kEarlyOwn) own_round2();
                const size_t mo = static_cast<size_t>(bh) * W * W;
                const float dl2 = dl1 * dl1;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const f32x4 xf = dl2 * x0seg[i] + own_x[i], cf = dl1 * c0seg[i] + own_c[i];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const size_t at = mo + static_cast<size_t>(16 * (cb + i) + r) * W + 16 * tb + 4 * g + e;
                        a.fin.G[at] = xf[e];
                        a.fin.C[at] = cf[e];
                    }
                }
                if ((yw || mw) && l < 16) {
                    float *dst = (yw ? a.fin.h : a.fin.m) + static_cast<size_t>(bh) * W;
#pragma unroll
                    for (int i = 0; i < 2; ++i) dst[16 * (cb + i) + r] = (yw ? dl2 : dl1) * v0seg[i] + own_v[i];
                }
            }
        }
        float *const vec = reinterpret_cast<float *>(sm.T[RIDGE ? 16 : 0]);
        __syncthreads();  // every Us, value and query read done: the tiles take X0 (C0, vectors)
#pragma unroll
        for (int c = 0; c < kFMaxL; ++c) {
            if (c < Lseg) {
                const float d2 = gp(static_cast<float>(2 * W * c));
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    bf16x4 h, lo;
                    split4(d2 * x0seg[i] + xpre[c][i], h, lo);
                    // lane holds X0^T[j = 16tb+4g+e][a = 16(cb+i)+r]; tile rows a
                    st4(sm.T[8 + 2 * c], 16 * (cb + i) + r, 16 * tb + 4 * g, h);
                    st4(sm.T[9 + 2 * c], 16 * (cb + i) + r, 16 * tb + 4 * g, lo);
                }
                if constexpr (RIDGE) {
                    const float d1 = gp(static_cast<float>(W * c));
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        bf16x4 h, lo;
                        split4(d1 * c0seg[i] + cpre[c][i], h, lo);
                        st4(sm.T[c], 16 * (cb + i) + r, 16 * tb + 4 * g, h);
                        st4(sm.T[4 + c], 16 * (cb + i) + r, 16 * tb + 4 * g, lo);
                    }
                }
                if (DEN && (yw || mw) && l < 16) {
                    const float dv = gp(static_cast<float>((yw ? 2 : 1) * W * c));
#pragma unroll
                    for (int i = 0; i < 2; ++i) vec[c * kVecSlot + voff + 16 * (cb + i) + r] = dv * v0seg[i] + vpre[c][i];
                }
            }
        }
        __syncthreads();

        // ================= output: num + e^2 q_t^T X0 =============================
        if (Lcs > 0) {
            f32x4 acc[2][4];
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                acc[0][jb] = acc[1][jb] = zero4;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int rb = 32 * ks + 8 * g;
                    const bf16x8 xh = tr8(sm.T[8 + 2 * sc], rb, rb + 4, 16 * jb, r);
                    const bf16x8 xl = tr8(sm.T[9 + 2 * sc], rb, rb + 4, 16 * jb, r);
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        acc[i][jb] = mfma(xh, qn[i][ks], acc[i][jb]);
                        acc[i][jb] = mfma(xl, qn[i][ks], acc[i][jb]);
                    }
                }
            }
            f32x4 accc[2][4];  // ridge: C0^T q_t
            if constexpr (RIDGE) {
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) {
                    accc[0][jb] = accc[1][jb] = zero4;
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const int rb = 32 * ks + 8 * g;
                        const bf16x8 ch = tr8(sm.T[sc], rb, rb + 4, 16 * jb, r);
                        const bf16x8 cl = tr8(sm.T[4 + sc], rb, rb + 4, 16 * jb, r);
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            accc[i][jb] = mfma(ch, qn[i][ks], accc[i][jb]);
                            accc[i][jb] = mfma(cl, qn[i][ks], accc[i][jb]);
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tt = t0 + 16 * i;
                const float e = gp(static_cast<float>(tt + 1));
                const float e2 = e * e;
                // den_t = sum_s P[t][s] + q_t . (e^2 y0 + lambda e m0); this lane
                // holds features 32ks+8g.. of q_t, the other three quarters are
                // in lanes l^16, l^32, l^48
                float den = 0.0f;
                if constexpr (DEN) {
                    const float *y0 = vec + sc * kVecSlot;
                    float part = dl[i];
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const f32x4 ya = *reinterpret_cast<const f32x4 *>(y0 + 32 * ks + 8 * g);
                        const f32x4 yb = *reinterpret_cast<const f32x4 *>(y0 + 32 * ks + 8 * g + 4);
                        f32x4 ma = zero4, mb = zero4;
                        if constexpr (MV) {
                            ma = *reinterpret_cast<const f32x4 *>(y0 + 64 + 32 * ks + 8 * g);
                            mb = *reinterpret_cast<const f32x4 *>(y0 + 64 + 32 * ks + 8 * g + 4);
                        }
#pragma unroll
                        for (int e4 = 0; e4 < 4; ++e4) {
                            float wa = e2 * ya[e4], wb = e2 * yb[e4];
                            if constexpr (MV) {
                                wa += (lam * e) * ma[e4];
                                wb += (lam * e) * mb[e4];
                            }
                            part += static_cast<float>(qn[i][ks][e4]) * wa + static_cast<float>(qn[i][ks][4 + e4]) * wb;
                        }
                    }
                    part += __shfl_xor(part, 16);
                    den = part + __shfl_xor(part, 32);
                }
                if (tt < Lcs) {
                    const size_t tok = static_cast<size_t>(bh) * a.n + static_cast<size_t>(c0 + sc) * W + tt;
                    float *orow = a.out + tok * W;
                    const float rd = NORM ? 1.0f / den : 1.0f;
#pragma unroll
                    for (int jb = 0; jb < 4; ++jb) {
                        f32x4 o = num[i][jb] + e2 * acc[i][jb];
                        if constexpr (RIDGE) o += (lam * e) * accc[i][jb];
                        if constexpr (NORM) o *= rd;
                        // streamed past the caches: nothing is left to write back when the kernel ends
                        __builtin_nontemporal_store(o, reinterpret_cast<f32x4 *>(orow + 16 * jb + 4 * g));
                    }
                    if (DEN && a.den != nullptr && g == 0) a.den[tok] = den;
                }
            }
        }
        __syncthreads();  // this segment's LDS reads are done before the next one is staged
        if constexpr (STATE) {
            if (fin_seg) {
                // finish the final state: S made exactly symmetric (the mean of
                // the two triangles: the MFMA sums of the two triangles round
                // differently), then G = S C - X and h = S m - y (X and y were
                // left in G and h above), in fp32 (fp32 MFMA) from S and C staged
                // in LDS with padded rows (conflict-light operand reads)
                constexpr int SP = W + 4, CP = W + 16;
                float *Ss = reinterpret_cast<float *>(sm.T[0]);
                float *Cs = Ss + W * SP;
                float *ms = Cs + W * CP;
                const size_t mo = static_cast<size_t>(bh) * W * W;
                for (int idx = tid_l; idx < W * W; idx += kFThreads) {
                    Ss[(idx / W) * SP + idx % W] = a.fin.S[mo + idx];
                    Cs[(idx / W) * CP + idx % W] = a.fin.C[mo + idx];
                }
                if (tid_l < W) ms[tid_l] = a.fin.m[static_cast<size_t>(bh) * W + tid_l];
                __syncthreads();
                {
                    constexpr int PER = W * W / kFThreads;
                    float sym[PER];
#pragma unroll
                    for (int u = 0; u < PER; ++u) {
                        const int idx = tid_l + u * kFThreads, ra = idx / W, cj = idx % W;
                        sym[u] = 0.5f * (Ss[ra * SP + cj] + Ss[cj * SP + ra]);
                    }
                    __syncthreads();
#pragma unroll
                    for (int u = 0; u < PER; ++u) {
                        const int idx = tid_l + u * kFThreads;
                        Ss[(idx / W) * SP + idx % W] = sym[u];
                        a.fin.S[mo + idx] = sym[u];
                    }
                }
                __syncthreads();
                // wave v forms the 16 x 16 output tiles 2v and 2v+1 (row block t/4,
                // column block t%4): lane (g, r) takes S[m0 + r][k0 + g] and
                // C[k0 + g][n0 + r], and receives G[m0 + 4g + e][n0 + r]
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const int t = 2 * wave + tt, m0 = 16 * (t >> 2), n0 = 16 * (t & 3);
                    f32x4 acc = zero4;
#pragma unroll
                    for (int k0 = 0; k0 < W; k0 += 4)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Ss[(m0 + r) * SP + k0 + g], Cs[(k0 + g) * CP + n0 + r],
                                                                   acc, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float *G = a.fin.G + mo + static_cast<size_t>(m0 + 4 * g + e) * W + n0 + r;
                        *G = acc[e] - *G;
                    }
                }
                if (tid_l < W) {
                    float acc = 0.0f;
                    for (int b = 0; b < W; ++b) acc = fmaf(Ss[tid_l * SP + b], ms[b], acc);
                    float *h = a.fin.h + static_cast<size_t>(bh) * W + tid_l;
                    *h = acc - *h;
                }
                if (tid_l == 0 && a.fin.rho != nullptr)
                    a.fin.rho[bh] = (a.irho != nullptr ? a.irho[bh] : 1.0f) * gp(static_cast<float>(a.n));
                __syncthreads();  // LDS reads done before the next segment is staged
            }
        }
    };
    // A loop around the body costs registers even when it runs once, so the
    // one-segment launch calls the body straight.
    // The next segment: a ticket when segments wait on each other.  Thread 0
    // takes it and hands it to the other waves through the last key tile,
    // which is free at the start of every segment.  One-pass grid (one
    // segment per workgroup): head b mod BH, its segment index p from that
    // head's own counter (P workgroups per head contend for it; the one that
    // takes the last index resets it).  Looped grid: one counter over all
    // segments.  Either way a head's segments are taken in increasing order.
    auto take = [&]() -> int {
        int *slot = reinterpret_cast<int *>(sm.T[3]);
        if (tid == 0) {
            int t;
            if constexpr (LOOP) {
                t = static_cast<int>(
                    __hip_atomic_fetch_add(&a.ctrl[kTicketWord], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            } else {
                const int head = static_cast<int>(blockIdx.x) % a.BH;
                uint32_t *cnt = &a.ctrl[kHeadTicketWord + kHeadTicketStride * head];
                const int pp = static_cast<int>(__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                if (pp == a.P - 1) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                t = pp * a.BH + head;
            }
            *slot = t;
        }
        __syncthreads();
        const int t = __builtin_amdgcn_readfirstlane(*slot);
        __syncthreads();  // every wave has read it before the tile is staged
        return t;
    };
    const int seg0 = a.P > 1 ? take() : static_cast<int>(blockIdx.x);
    epoch = next_epoch(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(ep_raw))));
    if constexpr (LOOP) {  // (with one segment per head nothing waits: a plain stride)
        for (int seg = seg0; seg < a.segs; seg = a.P > 1 ? take() : seg + static_cast<int>(gridDim.x)) seg_body(seg);
    } else if (seg0 < a.segs) {
        seg_body(seg0);
    } else if (tid == 0) {  // a ticket out of range: the control block was not zero before first use
        __hip_atomic_fetch_add(&a.ctrl[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- the last workgroup to finish resets the counter and advances the epoch
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

// The initial state in the slot layout of the aggregates (put_tiles): S, X =
// S C - G and C as sixteen tiles of 64 lanes x 4 floats each, where tile 2v+i,
// lane 16g+r, entry e holds element (16tb+4g+e, 16(cb+i)+r), tb = v/2, cb =
// 2(v%2), of S, of X^T and of C^T; then y = S m - h and m as one vector pair.
// Grid (BH, 4): workgroup (bh, y) forms rows 16y..16y+15 of X, S, C, y; each
// thread a 1 x 4 block of X (fp32, all of C staged in LDS).
__global__ __launch_bounds__(256) void k_fast64_init(hla_state in, float *iagg, float *iaggV) {
    __shared__ float Cs[W * W], Ss[16 * W], ms[W];
    const int bh = blockIdx.x, r0 = 16 * blockIdx.y, tid = threadIdx.x;
    const size_t mo = static_cast<size_t>(bh) * W * W;
    for (int i = tid; i < W * W / 4; i += 256)
        reinterpret_cast<float4 *>(Cs)[i] = reinterpret_cast<const float4 *>(in.C + mo)[i];
    reinterpret_cast<float4 *>(Ss)[tid] = reinterpret_cast<const float4 *>(in.S + mo + r0 * W)[tid];
    if (tid < W) ms[tid] = in.m[static_cast<size_t>(bh) * W + tid];
    __syncthreads();
    // slot index of element (u, w): u the row index 16tb+4g+e, w the column index 16(cb+i)+r
    auto sidx = [](int u, int w) {
        const int tb = u >> 4, g = (u >> 2) & 3, e = u & 3, ci = w >> 4, r = w & 15;
        const int v = 2 * tb + (ci >> 1), i = ci & 1;
        return ((2 * v + i) * 64 + 16 * g + r) * 4 + e;
    };
    float *dst = iagg + static_cast<size_t>(bh) * 3 * 4096;
    const int lr = tid >> 4, c0 = 4 * (tid & 15), ra = r0 + lr;
    float x[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int b = 0; b < W; ++b) {
        const float s = Ss[lr * W + b];
        const float4 c = *reinterpret_cast<const float4 *>(Cs + b * W + c0);
        x[0] = fmaf(s, c.x, x[0]);
        x[1] = fmaf(s, c.y, x[1]);
        x[2] = fmaf(s, c.z, x[2]);
        x[3] = fmaf(s, c.w, x[3]);
    }
    const float4 gv = *reinterpret_cast<const float4 *>(in.G + mo + ra * W + c0);
    const float gg[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int cj = c0 + u;
        dst[sidx(ra, cj)] = Ss[lr * W + cj];                    // S[ra][cj]
        dst[4096 + sidx(cj, ra)] = x[u] - gg[u];                // X[ra][cj], transposed
        dst[2 * 4096 + sidx(cj, ra)] = Cs[ra * W + cj];         // C[ra][cj], transposed
    }
    if (tid < 16) {
        float y = 0.0f;
        for (int b = 0; b < W; ++b) y = fmaf(Ss[tid * W + b], ms[b], y);
        iaggV[static_cast<size_t>(bh) * kVecSlot + r0 + tid] = y - in.h[static_cast<size_t>(bh) * W + r0 + tid];
        iaggV[static_cast<size_t>(bh) * kVecSlot + 64 + r0 + tid] = ms[r0 + tid];
    }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// The data region (the flags live in a region of their own, which holds
// nothing but launch epochs: flag_bytes)
struct FastLayout {
    size_t aggS, aggX, aggC, aggV, iagg, iaggV, total;
};

size_t flag_bytes(int BH, int P) {
    return align256(static_cast<size_t>(BH) * P * 2 * kWaves * kFlagStride * sizeof(uint32_t));
}

FastLayout fast_layout(int BH, int P) {
    FastLayout L{};
    const size_t slots = static_cast<size_t>(BH) * P;
    L.aggS = 0;
    L.aggX = L.aggS + slots * 4096 * sizeof(float);
    L.aggC = L.aggX + slots * 4096 * sizeof(float);
    L.aggV = L.aggC + slots * 4096 * sizeof(float);
    L.iagg = L.aggV + align256(slots * kVecSlot * sizeof(float));
    L.iaggV = L.iagg + static_cast<size_t>(BH) * 3 * 4096 * sizeof(float);
    L.total = L.iaggV + static_cast<size_t>(BH) * kVecSlot * sizeof(float);
    return L;
}

template <bool DECAY, bool LOOP>
void launch_fast(const FastArgs &a, dim3 grid, hipStream_t st, bool ridge, bool den, bool norm, bool state) {
    const dim3 block(kFThreads);
    if (a.vl != nullptr) {  // values as a bf16 pair: the plain numerator only
        hipLaunchKernelGGL((k_fast64<DECAY, LOOP, false, false, false, false, true>), grid, block, 0, st, a);
        return;
    }
    if (state) {  // with an initial and/or a final state: the plain numerator, or every option
        if (norm) hipLaunchKernelGGL((k_fast64<DECAY, LOOP, true, true, true, true>), grid, block, 0, st, a);
        else if (ridge || den) hipLaunchKernelGGL((k_fast64<DECAY, LOOP, true, true, false, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_fast64<DECAY, LOOP, false, false, false, true>), grid, block, 0, st, a);
    } else if (ridge) {
        if (norm) hipLaunchKernelGGL((k_fast64<DECAY, LOOP, true, true, true, false>), grid, block, 0, st, a);
        else if (den) hipLaunchKernelGGL((k_fast64<DECAY, LOOP, true, true, false, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_fast64<DECAY, LOOP, true, false, false, false>), grid, block, 0, st, a);
    } else {
        if (norm) hipLaunchKernelGGL((k_fast64<DECAY, LOOP, false, true, true, false>), grid, block, 0, st, a);
        else if (den) hipLaunchKernelGGL((k_fast64<DECAY, LOOP, false, true, false, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_fast64<DECAY, LOOP, false, false, false, false>), grid, block, 0, st, a);
    }
}

void fast64_geometry(int BH, int nc, int *P, int *L) {
    // about one workgroup per CU; at most four chunks per workgroup
    const int target = (256 + BH - 1) / BH;
    int l = (nc + target - 1) / target;
    l = l < 1 ? 1 : (l > kFMaxL ? kFMaxL : l);
    *L = l;
    *P = (nc + l - 1) / l;
}

}  // namespace

bool fast64_supported(const FwdProblem &p) {
    if (!(p.dtype == HLA_BF16 && p.d == 64 && p.dv == 64 && p.w == 64 && p.n > 0)) return false;
    const int nh = p.gam.per_head ? p.H : 1;
    for (int h = 0; h < nh; ++h)
        if (p.gam.g[h] < kMinGamma) return false;
    return true;
}

size_t fast64_flag_bytes(int BH, int n) {
    const int nc = (n + W - 1) / W;
    int P, L;
    fast64_geometry(BH, nc, &P, &L);
    return flag_bytes(BH, P);
}

size_t fast64_data_bytes(int BH, int n) {
    const int nc = (n + W - 1) / W;
    int P, L;
    fast64_geometry(BH, nc, &P, &L);
    return fast_layout(BH, P).total;
}

hipError_t fast64_forward(const FwdProblem &p, uint32_t *ctrl, uint32_t *flags, void *data, hipStream_t st) {
    FastArgs a{};
    a.H = p.H; a.n = p.n; a.nc = p.nc; a.BH = p.B * p.H;
    fast64_geometry(a.BH, a.nc, &a.P, &a.L);
    a.segs = a.BH * a.P;
    a.q = static_cast<const uint16_t *>(p.q);
    a.k = static_cast<const uint16_t *>(p.k);
    a.v = static_cast<const uint16_t *>(p.v);
    a.vl = static_cast<const uint16_t *>(p.vl);
    a.out = p.out;
    a.den = p.den;
    a.ridge = p.ridge;
    a.ctrl = ctrl;
    const FastLayout L = fast_layout(a.BH, a.P);
    char *base = static_cast<char *>(data);
    a.flags = flags;
    a.aggS = reinterpret_cast<float *>(base + L.aggS);
    a.aggX = reinterpret_cast<float *>(base + L.aggX);
    a.aggC = reinterpret_cast<float *>(base + L.aggC);
    a.aggV = reinterpret_cast<float *>(base + L.aggV);
    a.gam = p.gam;
    const bool state = p.init.S != nullptr || p.fin.S != nullptr;
    if (p.init.S != nullptr) {
        a.iagg = reinterpret_cast<float *>(base + L.iagg);
        a.iaggV = reinterpret_cast<float *>(base + L.iaggV);
        a.irho = p.init.rho;
        hipLaunchKernelGGL(k_fast64_init, dim3(a.BH, 4), dim3(256), 0, st, p.init, const_cast<float *>(a.iagg),
                           const_cast<float *>(a.iaggV));
        const hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) return e0;
    }
    a.fin = p.fin;
    const int nh = p.gam.per_head ? p.H : 1;
    bool decay = false;
    for (int h = 0; h < nh; ++h) decay = decay || p.gam.g[h] != 1.0f;
    // one workgroup per CU at most (its LDS fills the CU); segments by ticket when they wait on each other
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const bool loop = a.segs > cus || (a.P > 1 && a.BH > kMaxTicketHeads);
    const dim3 grid(static_cast<unsigned>(loop ? cus : a.segs));
    const bool ridge = p.ridge != 0.0f, norm = p.normalize != 0, den = norm || p.den != nullptr;
    if (decay) {
        if (loop) launch_fast<true, true>(a, grid, st, ridge, den, norm, state);
        else launch_fast<true, false>(a, grid, st, ridge, den, norm, state);
    } else {
        if (loop) launch_fast<false, true>(a, grid, st, ridge, den, norm, state);
        else launch_fast<false, false>(a, grid, st, ridge, den, norm, state);
    }
    return hipGetLastError();
}

}  // namespace hla
