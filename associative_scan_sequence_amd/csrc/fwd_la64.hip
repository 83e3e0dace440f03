// fwd_la64.hip -- one-launch masked first-order (causal) linear attention
// for d = dv = 64, chunk 64, bf16 operands on gfx950 MFMA:
//   y_t = sum_{s <= t} g^(t - s) (q_t . k_s) v_s          (REV: s >= t, g^(s - t)).
// The asymmetric variant (AHLA) is this map applied twice, and masked third
// order is second-order HLA over values that this map has mixed (Higher-order
// Linear Attention, paperlayer.ai summary sec. 6 and 7; the decompositions
// are pinned on the CPU in tests/test_higher_oracle.py), so both are built
// from it where their inputs allow.  The gradient of the second-order
// numerator is a sum of such maps, forward and reverse in time (sec. 4: the
// reverse-mode scan; the identity is pinned in tests/test_backward_algebra.py),
// so the backward is built from it too (bwd_la64.hip).
//
// Per chunk (local t, s; L tokens; e_t = g^(t+1), f_s = g^(L-1-s)), with the
// carry C0 = sum over earlier tokens of g^(distance to the chunk start - 1) k v^T:
//   A = (Q K^T) o D_g o L,   y = A V + diag(e) Q C0,   C0 <- g^L C0 + K^T diag(f) V.
// The layout, segments, tickets and the device-coherent hand-off of the C
// aggregates are those of the second-order kernel (fwd_fast64.hip), with one
// exchange round instead of two:
//  * tile role: wave v sums tiles 2v, 2v+1 of the segment's C^T (rows j =
//    16tb+4g+e, columns a = 16(cb+i)+r) over its chunks, publishes them, and
//    sums the carry from the earlier segments' aggregates;
//  * slice role: wave v forms the masked A^T tiles of 32 tokens of chunk v/2
//    and the local part A V, then adds e_t C0^T q_t once the carry is in LDS.
// Output: fp32 (stored, or added to what out holds), or the result split into
// bf16 hi = bf16(y) and lo = bf16(y - hi), ready to be an operand of a later
// map.  Operand modes QM, KM, VM: 0 bf16; 1 such a pair (x = hi + lo, two
// bf16 arrays); 2 fp32, split into such a pair as it is staged.  Not keys and
// values both in pairs.  A product with a pair takes hi * y + lo * y_hi (the
// dropped lo * y_lo is about 2^-16 of the product).
// OUT2 >= 0: a second set of queries (mode Q2M) against the same keys, values
// and carries, with its own output (mode OUT2): its local part and output are
// formed after the first set's, while the carry tiles are still in LDS.
// REV: the map runs on the reversed sequence (token t read and written at
// n - 1 - t), which is the reverse-time map.
// SYM: the sum of the map and the map with keys and values exchanged,
//   y_t = sum g^|t-s| [(q_t . k_s) v_s + (q_t . v_s) k_s]   (d = dv),
// whose carry is C0 + C0^T: the C sums run as for the map alone, the output
// reads the carry tiles both ways, and the local part is formed twice with
// the key and value tiles exchanged.
// Precision: A is split into bf16 hi + lo (its entries are fp32 sums), as are
// the decayed key operand of the C sums and the carry C0.
// Carries: an initial carry M_in at position -1 adds r^(p+1) M_in^T q_p to
// the output at position p (its aggregate enters every segment's carry as a
// segment before the first), and the last segment can write the carry after
// the last token; a bias b adds r^(p+1) b.  Output mode kNone forms no
// output, only that final carry.
// k_la64 runs one map; k_la64_pair two maps that do not depend on each other
// in one grid, so that their launches do not wait on each other's tails.
#include "fast64_common.h"

namespace hla {
namespace {

template <int V>
struct IC {  // an int as a type, to instantiate a lambda for each half
    static constexpr int value = V;
};

constexpr int kLThreads = 512;
constexpr int kLMaxL = 4;  // chunks per segment
constexpr int kLWaves = 8;

constexpr int kStore = 0, kAccumulate = 1, kSplit = 2, kNone = 3;  // output modes (LaProblem::mode)

struct LaArgs {
    int H, n, nc, P, L, BH, segs;
    const uint16_t *q, *k, *v;
    const uint16_t *ql, *kl, *vl;  // the lo halves of paired operands (mode 1)
    const float *qf, *kf, *vf;     // fp32 operands (mode 2)
    const uint16_t *q2, *q2l;      // the second queries (OUT2 >= 0), bf16 or pair
    const float *q2f;              // or fp32
    float *out;             // kStore, kAccumulate
    uint16_t *oh, *ol;      // kSplit: bf16 hi and lo of the result
    float *out2;            // the second queries' output
    uint16_t *oh2, *ol2;
    const float *init;      // [BH][64 keys][64 values]: the carry at position -1 (null: zero)
    float *fin;             // [BH][64][64]: receives the carry after the last token (null: not formed)
    const float *bias;      // [BH][64]: y_t += r^(p+1) bias, p the position (null: none)
    uint32_t *ctrl;         // control block, as for the second-order kernel
    uint32_t *flags;        // [BH * P][8 waves] at kFlagStride words
    float *aggC;            // [BH * P][16 tiles][64 lanes][4]
    uint32_t *flags2;       // the chained map's second hand-off, laid out as flags and aggC
    float *aggC2;
    GammaTab gam;
    float gexp;             // the decay per token is g^gexp (1, or 2 for the squared decay)
};

template <int NT>
struct LaSmem {
    // K_c in T[c], V_c in T[4+c], C0 of chunk c in T[8+2c] (hi), T[9+2c] (lo);
    // KP or VP: the keys' or values' lo half in T[16+c]
    __bf16 T[NT][kTileElems];
};

__device__ __forceinline__ void put_tiles2(const float *slot, int v, int l, const f32x4 (&x)[2]) {
    const __amdgpu_buffer_rsrc_t rs = slot_rsrc(slot);
#pragma unroll
    for (int i = 0; i < 2; ++i) __builtin_amdgcn_raw_buffer_store_b128(x[i], rs, ((2 * v + i) * 64 + l) * 16, 0, kSc1);
}

// 8 consecutive values of a row (element e of the array) as raw registers:
// mode 0 raw[0] = 8 bf16; mode 1 raw[0], raw[1] = hi, lo; mode 2 raw[0],
// raw[1] = the 8 fp32 values (split later, so the load is not waited for here)
template <int M>
__device__ __forceinline__ void ld_op(const uint16_t *h, const uint16_t *lo, const float *f, size_t e,
                                      u32x4 (&raw)[2]) {
    if constexpr (M == 2) {
        raw[0] = *reinterpret_cast<const u32x4 *>(f + e);
        raw[1] = *reinterpret_cast<const u32x4 *>(f + e + 4);
    } else {
        raw[0] = *reinterpret_cast<const u32x4 *>(h + e);
        if constexpr (M == 1) raw[1] = *reinterpret_cast<const u32x4 *>(lo + e);
    }
}

// raw registers -> (hi, lo) bf16 (lo only for modes 1 and 2)
template <int M>
__device__ __forceinline__ void to_pair(const u32x4 (&raw)[2], u32x4 &hi, u32x4 &lo) {
    if constexpr (M == 2) {
        bf16x8 h, l;
        pair_operand(__builtin_bit_cast(f32x4, raw[0]), __builtin_bit_cast(f32x4, raw[1]), h, l);
        hi = __builtin_bit_cast(u32x4, h);
        lo = __builtin_bit_cast(u32x4, l);
    } else {
        hi = raw[0];
        if constexpr (M == 1) lo = raw[1];
    }
}

// One map: its segments are taken by nblocks workgroups, of which this is
// number block; its per-head ticket counters start at counter head_base.
// Returns the launch's epoch.
template <bool DECAY, bool LOOP, int OUT, int QM, int KM, int VM, bool REV, int OUT2 = -1, int Q2M = 0, bool SYM = false,
          bool CH = false>
struct LaMap {
    static constexpr int kTiles = (KM != 0 || VM != 0 || CH) ? 20 : 16;
    __device__ __forceinline__ static uint32_t run(const LaArgs &a, __bf16 (*T)[kTileElems], int block, int nblocks,
                                                   int head_base);
};

template <bool DECAY, bool LOOP, int OUT, int QM, int KM, int VM, bool REV, int OUT2, int Q2M, bool SYM, bool CH>
__device__ __forceinline__ uint32_t LaMap<DECAY, LOOP, OUT, QM, KM, VM, REV, OUT2, Q2M, SYM, CH>::run(
    const LaArgs &a, __bf16 (*T)[kTileElems], int block, int nblocks, int head_base) {
    constexpr bool KP = KM != 0, VP = VM != 0, Q2 = OUT2 >= 0;
    static_assert(!(KP && VP), "the lo halves of keys and values share four tiles");
    static_assert(!CH || (!KP && !VP && !SYM && !Q2 && OUT != kNone), "the chained map takes plain operands");
    const int tid = threadIdx.x;
    uint32_t ep_raw = 0;
    if ((tid & 63) == 0) ep_raw = __hip_atomic_load(&a.ctrl[kLine + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t epoch = 0;
    const u32x4 z4 = u32x4{0u, 0u, 0u, 0u};
    const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
    float lg = 0.0f;
    auto gp = [&](float e) { return DECAY ? __builtin_amdgcn_exp2f(e * lg) : 1.0f; };  // g^e
    auto gpl = [&](float el) { return DECAY ? __builtin_amdgcn_exp2f(el) : 1.0f; };   // g^e from e log2(g)

    auto seg_body = [&](const int seg) __attribute__((always_inline)) {
        int tid_l = static_cast<int>(threadIdx.x);
        if constexpr (LOOP) asm volatile("" : "+v"(tid_l));
        const int wave = tid_l >> 6, l = tid_l & 63, r = l & 15, g = l >> 4;
        const int grp = wave >> 2, wt = tid_l & 255;
        const int sc = wave >> 1, hh = (wave ^ (wave >> 2)) & 1;
        const int t0 = 32 * hh + r;
        const int tb = wave >> 1, cb = 2 * (wave & 1);
        const int bh = seg % a.BH, p = seg / a.BH;
        lg = DECAY ? a.gexp * log2f(head_gamma(a.gam, bh % a.H)) : 0.0f;
        const size_t head = static_cast<size_t>(bh) * a.n;
        // the head's token at position pos of the (possibly reversed) sequence
        auto at_pos = [&](int pos) { return head + static_cast<size_t>(REV ? a.n - 1 - pos : pos); };
        const int c0 = p * a.L;
        const int Lseg = min(a.L, a.nc - c0);
        auto chunk_len = [&](int j) { return min(W, a.n - (c0 + j) * W); };
        int lc_of[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) lc_of[jj] = 2 * grp + jj < Lseg ? chunk_len(2 * grp + jj) : 0;
        const int Lcs = sc < Lseg ? chunk_len(sc) : 0;
        int lcc[kLMaxL];
#pragma unroll
        for (int c = 0; c < kLMaxL; ++c) lcc[c] = c < Lseg ? chunk_len(c) : 0;
        const size_t slot = static_cast<size_t>(bh) * a.P + p;
        const bool publish = p + 1 < a.P;

        // ---- loads: keys and values of the segment's chunks (rows past a chunk
        // read the head's first row and are zeroed when staged), queries of the slice
        u32x4 kr[2][2][2], vr[2][2][2], qr[2][2][2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * grp + jj;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int row = (wt + 256 * u) >> 3, cg = (wt + 256 * u) & 7;
                const size_t src = row < lc_of[jj] ? at_pos((c0 + j) * W + row) : head;
                ld_op<KM>(a.k, a.kl, a.kf, src * W + cg * 8, kr[jj][u]);
                ld_op<VM>(a.v, a.vl, a.vf, src * W + cg * 8, vr[jj][u]);
            }
        }
        // queries of the slice: token t0 + 16i, features 32ks + 8g ..
        auto load_q = [&](auto mode, const uint16_t *h, const uint16_t *lo, const float *f, u32x4 (&raw)[2][2][2])
            __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int tt = t0 + 16 * i;
                    const size_t src = tt < Lcs ? at_pos((c0 + sc) * W + tt) : head;
                    ld_op<decltype(mode)::value>(h, lo, f, src * W + 32 * ks + 8 * g, raw[i][ks]);
                }
        };
        auto to_q = [&](auto mode, const u32x4 (&raw)[2][2][2], bf16x8 (&qh)[2][2], bf16x8 (&ql)[2][2])
            __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    u32x4 h, lo;
                    to_pair<decltype(mode)::value>(raw[i][ks], h, lo);
                    const bool in = t0 + 16 * i < Lcs;
                    qh[i][ks] = __builtin_bit_cast(bf16x8, in ? h : z4);
                    if constexpr (decltype(mode)::value != 0) ql[i][ks] = __builtin_bit_cast(bf16x8, in ? lo : z4);
                }
        };
        if constexpr (OUT != kNone) load_q(IC<QM>{}, a.q, a.ql, a.qf, qr);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int row = (wt + 256 * u) >> 3, cg = (wt + 256 * u) & 7;
                const bool in = row < lc_of[jj];
                u32x4 kh, kl_, vh, vl_;
                to_pair<KM>(kr[jj][u], kh, kl_);
                to_pair<VM>(vr[jj][u], vh, vl_);
                st16(T[2 * grp + jj], row, cg * 8, in ? kh : z4);
                st16(T[4 + 2 * grp + jj], row, cg * 8, in ? vh : z4);
                if constexpr (KP) st16(T[16 + 2 * grp + jj], row, cg * 8, in ? kl_ : z4);
                if constexpr (VP) st16(T[16 + 2 * grp + jj], row, cg * 8, in ? vl_ : z4);
            }
        bf16x8 qn[2][2], qnl[2][2];
        if constexpr (OUT != kNone) to_q(IC<QM>{}, qr, qn, qnl);
        __syncthreads();

        auto lane_base = [&](int off) __attribute__((always_inline)) {
            if (!DECAY) return 0.0f;
            asm volatile("" : "+v"(off));
            return static_cast<float>(off) * lg;
        };

        // ================= tiles: the segment's C^T ================================
        // cpre[c] = sum of chunks 0..c-1 at chunk c's start; crun ends as C_seg.
        // Tile (j = 16tb+4g+e, a = 16(cb+i)+r) = sum_s V[s][j] f_s K[s][a].
        // vpair: the values are a bf16 pair, hi in the value tiles and lo in T[16 + c]
        f32x4 cpre[kLMaxL][2], crun[2];
        auto csums = [&](auto vpair) __attribute__((always_inline)) {
        constexpr bool VPX = VP || decltype(vpair)::value != 0;
        crun[0] = crun[1] = zero4;
#pragma unroll
        for (int c = 0; c < kLMaxL; ++c) {
#pragma unroll
            for (int i = 0; i < 2; ++i) cpre[c][i] = crun[i];
            const int Lc = lcc[c];
            const float rho = gp(static_cast<float>(Lc));
#pragma unroll
            for (int i = 0; i < 2; ++i) crun[i] *= rho;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int rb = 32 * ks + 8 * g;
                const bf16x8 vt = tr8(T[4 + c], rb, rb + 4, 16 * tb, r);
                bf16x8 vtl;
                if constexpr (VPX) vtl = tr8(T[16 + c], rb, rb + 4, 16 * tb, r);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const bf16x8 kt = tr8(T[c], rb, rb + 4, 16 * (cb + i), r);
                    bf16x8 ktl;
                    if constexpr (KP) ktl = tr8(T[16 + c], rb, rb + 4, 16 * (cb + i), r);
                    if (!DECAY) {
                        crun[i] = mfma(vt, kt, crun[i]);
                        if constexpr (VPX) crun[i] = mfma(vtl, kt, crun[i]);
                        if constexpr (KP) crun[i] = mfma(vt, ktl, crun[i]);
                    } else {
                        // f_s = g^(Lc - 1 - s) for the tokens s = 32ks + 8g + e (+4)
                        const float base = fmaf(static_cast<float>(Lc - 1), lg, lane_base(-8 * g));
                        f32x4 x0, x1;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            x0[e] = gpl(fmaf(static_cast<float>(-(32 * ks + e)), lg, base)) * static_cast<float>(kt[e]);
                            x1[e] = gpl(fmaf(static_cast<float>(-(32 * ks + 4 + e)), lg, base)) * static_cast<float>(kt[4 + e]);
                        }
                        bf16x8 h, lo;
                        pair_operand(x0, x1, h, lo);
                        crun[i] = mfma(vt, h, crun[i]);
                        crun[i] = mfma(vt, lo, crun[i]);
                        if constexpr (VPX) crun[i] = mfma(vtl, h, crun[i]);
                        if constexpr (KP) {  // the decayed lo half, rounded once: its own lo is ~2^-16 of the product
                            f32x4 y0, y1;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                y0[e] = gpl(fmaf(static_cast<float>(-(32 * ks + e)), lg, base)) * static_cast<float>(ktl[e]);
                                y1[e] = gpl(fmaf(static_cast<float>(-(32 * ks + 4 + e)), lg, base)) * static_cast<float>(ktl[4 + e]);
                            }
                            bf16x8 hl, ll;
                            pair_operand(y0, y1, hl, ll);
                            crun[i] = mfma(vt, hl, crun[i]);
                        }
                    }
                }
            }
        }
        };
        auto flag_of = [&](uint32_t *flags, size_t sl) { return &flags[(sl * kLWaves + wave) * kFlagStride]; };
        auto publish_sums = [&](uint32_t *flags, float *aggC) __attribute__((always_inline)) {
            if (publish) {
                put_tiles2(aggC + slot * 4096, wave, l, crun);
                wait_stores();
                if (l == 0) set_flag(flag_of(flags, slot), epoch);
            }
        };

        // ================= slice: A^T and the local part A V =========================
        f32x4 num[2][4];
        auto local = [&](auto hc, auto qpair, auto swap, auto vpair, const bf16x8 (&qn)[2][2],
                         const bf16x8 (&qnl)[2][2]) __attribute__((always_inline)) {
            constexpr int HH = decltype(hc)::value;
            constexpr bool QP = decltype(qpair)::value != 0;
            // swap: the keys are read from the value tiles and the values from the key tiles
            constexpr bool SW = decltype(swap)::value != 0;
            constexpr bool VPX = VP || decltype(vpair)::value != 0;
            constexpr int KB = SW ? 4 : 0, VB = SW ? 0 : 4;
            constexpr bool LKP = SW ? VPX : KP, LVP = SW ? KP : VPX;
            const float lg_rg = lane_base(r - 4 * g);
            f32x4 at[2][4];
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                at[0][ib] = at[1][ib] = zero4;
                if (ib <= 2 * HH + 1) {
                    const bf16x8 k0 = ld8(T[KB + sc], 16 * ib + r, 8 * g), k1 = ld8(T[KB + sc], 16 * ib + r, 32 + 8 * g);
                    bf16x8 k0l, k1l;
                    if constexpr (LKP) {
                        k0l = ld8(T[16 + sc], 16 * ib + r, 8 * g);
                        k1l = ld8(T[16 + sc], 16 * ib + r, 32 + 8 * g);
                    }
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        if (ib <= 2 * HH + i) {
                            at[i][ib] = mfma(k1, qn[i][1], mfma(k0, qn[i][0], zero4));
                            if constexpr (QP) at[i][ib] = mfma(k1, qnl[i][1], mfma(k0, qnl[i][0], at[i][ib]));
                            if constexpr (LKP) at[i][ib] = mfma(k1l, qn[i][1], mfma(k0l, qn[i][0], at[i][ib]));
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
            // num^T[j][t] = sum_s V[s][j] A[t][s]
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (2 * ks <= 2 * HH + 1) {
                    bf16x8 vt[4], vtl[4];
#pragma unroll
                    for (int jb = 0; jb < 4; ++jb) {
                        vt[jb] = tr8(T[VB + sc], 32 * ks + 4 * g, 32 * ks + 16 + 4 * g, 16 * jb, r);
                        if constexpr (LVP) vtl[jb] = tr8(T[16 + sc], 32 * ks + 4 * g, 32 * ks + 16 + 4 * g, 16 * jb, r);
                    }
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        if (2 * ks <= 2 * HH + i) {
                            bf16x8 ah, al;
                            pair_operand(at[i][2 * ks], at[i][2 * ks + 1], ah, al);
#pragma unroll
                            for (int jb = 0; jb < 4; ++jb) {
                                num[i][jb] = mfma(vt[jb], ah, num[i][jb]);
                                num[i][jb] = mfma(vt[jb], al, num[i][jb]);
                                if constexpr (LVP) num[i][jb] = mfma(vtl[jb], ah, num[i][jb]);
                            }
                        }
                    }
                }
            }
        };
        auto local_part = [&](auto qpair, auto vpair, const bf16x8 (&qh)[2][2], const bf16x8 (&ql)[2][2])
            __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) num[i][jb] = zero4;
            if (Lcs > 0) {
                if (hh) local(IC<1>{}, qpair, IC<0>{}, vpair, qh, ql);
                else local(IC<0>{}, qpair, IC<0>{}, vpair, qh, ql);
                if constexpr (SYM) {
                    if (hh) local(IC<1>{}, qpair, IC<1>{}, vpair, qh, ql);
                    else local(IC<0>{}, qpair, IC<1>{}, vpair, qh, ql);
                }
            }
        };
        // ================= the carry: C0 of every chunk -> LDS =======================
        // from the earlier segments' sums behind flags / aggC (with the initial
        // carry and the final carry when states), then C0 of every chunk into
        // T[8 + 2c] (hi), T[9 + 2c] (lo) when tiles
        const int seg_tokens = a.L * W;
        const bool last = p == a.P - 1;
        auto carry = [&](uint32_t *flags, const float *aggC, bool states, bool tiles) __attribute__((always_inline)) {
            f32x4 c0seg[2] = {zero4, zero4};
            bool failed = false;
            for (int pp = l; pp < p; pp += 64)
                if (!wait_flag(flag_of(flags, static_cast<size_t>(bh) * a.P + pp), epoch, a.ctrl + kSpinWord)) {
                    __hip_atomic_fetch_add(&a.ctrl[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    failed = true;
                }
            const bool bad = __builtin_amdgcn_ballot_w64(failed) != 0;
            constexpr int NB = 8;
            for (int p0 = 0; p0 < p; p0 += NB) {
                f32x4 x[NB][2];
#pragma unroll
                for (int s2 = 0; s2 < NB; ++s2)
                    if (p0 + s2 < p) {
                        const __amdgpu_buffer_rsrc_t rs = slot_rsrc(aggC + (static_cast<size_t>(bh) * a.P + p0 + s2) * 4096);
#pragma unroll
                        for (int i = 0; i < 2; ++i)
                            x[s2][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, ((2 * wave + i) * 64 + l) * 16, 0, kSc1);
                    }
#pragma unroll
                for (int s2 = 0; s2 < NB; ++s2)
                    if (p0 + s2 < p) {
                        const float scl = gp(static_cast<float>((p - 1 - (p0 + s2)) * seg_tokens));
#pragma unroll
                        for (int i = 0; i < 2; ++i) c0seg[i] += scl * x[s2][i];
                    }
            }
            // this lane's elements of a [key a][value j] matrix of the head
            auto mat_at = [&](int i) {
                return static_cast<size_t>(bh) * 4096 + (16 * (cb + i) + r) * 64 + 16 * tb + 4 * g;
            };
            if (states && a.init != nullptr) {  // the carry at position -1, decayed to this segment's start
                const float scl = gp(static_cast<float>(p * seg_tokens));
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    c0seg[i] += scl * *reinterpret_cast<const f32x4 *>(a.init + mat_at(i));
            }
            if (bad) {  // a carry that could not be waited for: NaN, never a silently wrong number
                const float nan = __builtin_nanf("");
                c0seg[0] = c0seg[1] = f32x4{nan, nan, nan, nan};
            }
            if (states && a.fin != nullptr && last) {  // the carry after the last token
                const float scl = gp(static_cast<float>(a.n - c0 * W));
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    *reinterpret_cast<f32x4 *>(a.fin + mat_at(i)) = scl * c0seg[i] + crun[i];
            }
            if (!tiles) return;
#pragma unroll
            for (int c = 0; c < kLMaxL; ++c) {
                if (c < Lseg) {
                    const float d1 = gp(static_cast<float>(W * c));
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        bf16x4 h, lo;
                        split4(d1 * c0seg[i] + cpre[c][i], h, lo);
                        // lane holds C0^T[j = 16tb+4g+e][a = 16(cb+i)+r]; tile rows a
                        st4(T[8 + 2 * c], 16 * (cb + i) + r, 16 * tb + 4 * g, h);
                        st4(T[9 + 2 * c], 16 * (cb + i) + r, 16 * tb + 4 * g, lo);
                    }
                }
            }
            __syncthreads();
        };

        // ================= output: num + e_t C0^T q_t ==============================
        // acc[i][jb]: lane (g, r) holds (C0^T q_t)[16 jb + 4g + e] for t = t0 + 16 i
        auto carry_term = [&](auto qpair, const bf16x8 (&qn)[2][2], const bf16x8 (&qnl)[2][2], f32x4 (&acc)[2][4])
            __attribute__((always_inline)) {
            constexpr bool QP = decltype(qpair)::value != 0;
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                acc[0][jb] = acc[1][jb] = zero4;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int rb = 32 * ks + 8 * g;
                    const bf16x8 ch = tr8(T[8 + 2 * sc], rb, rb + 4, 16 * jb, r);
                    const bf16x8 cl = tr8(T[9 + 2 * sc], rb, rb + 4, 16 * jb, r);
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        acc[i][jb] = mfma(ch, qn[i][ks], acc[i][jb]);
                        acc[i][jb] = mfma(cl, qn[i][ks], acc[i][jb]);
                        if constexpr (QP) acc[i][jb] = mfma(ch, qnl[i][ks], acc[i][jb]);
                    }
                    if constexpr (SYM) {  // C0 read the other way: the same lanes and k slots, rows for columns
                        const bf16x8 th = ld8(T[8 + 2 * sc], 16 * jb + r, rb);
                        const bf16x8 tl = ld8(T[9 + 2 * sc], 16 * jb + r, rb);
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            acc[i][jb] = mfma(th, qn[i][ks], acc[i][jb]);
                            acc[i][jb] = mfma(tl, qn[i][ks], acc[i][jb]);
                            if constexpr (QP) acc[i][jb] = mfma(th, qnl[i][ks], acc[i][jb]);
                        }
                    }
                }
            }
        };
        auto output = [&](auto omode, auto qpair, const bf16x8 (&qn)[2][2], const bf16x8 (&qnl)[2][2], float *out,
                          uint16_t *oh, uint16_t *ol, const float *bias) __attribute__((always_inline)) {
            constexpr int OM = decltype(omode)::value;
            if (Lcs == 0) return;
            f32x4 acc[2][4];
            carry_term(qpair, qn, qnl, acc);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tt = t0 + 16 * i;
                if (tt < Lcs) {
                    const float e = gp(static_cast<float>(tt + 1));
                    const int pos = (c0 + sc) * W + tt;
                    const size_t tok = at_pos(pos);
                    const float eb = bias != nullptr ? gp(static_cast<float>(pos + 1)) : 0.0f;
#pragma unroll
                    for (int jb = 0; jb < 4; ++jb) {
                        f32x4 o = num[i][jb] + e * acc[i][jb];
                        if (bias != nullptr)
                            o += eb * *reinterpret_cast<const f32x4 *>(bias + static_cast<size_t>(bh) * W + 16 * jb + 4 * g);
                        const size_t at = tok * W + 16 * jb + 4 * g;
                        if constexpr (OM == kSplit) {
                            bf16x4 h, lo;
                            split4(o, h, lo);
                            *reinterpret_cast<bf16x4 *>(oh + at) = h;
                            *reinterpret_cast<bf16x4 *>(ol + at) = lo;
                        } else {
                            f32x4 *dst = reinterpret_cast<f32x4 *>(out + at);
                            if constexpr (OM == kAccumulate) o += *dst;
                            __builtin_nontemporal_store(o, dst);
                        }
                    }
                }
            }
        };
        // the chained map's first output, as the second one's values: the bf16
        // pair of every row of this slice (zero past the chunk) into the value
        // tiles, hi in T[4 + sc] and lo in T[16 + sc]
        auto output_values = [&](auto qpair, const bf16x8 (&qn)[2][2], const bf16x8 (&qnl)[2][2])
            __attribute__((always_inline)) {
            f32x4 acc[2][4];
            if (Lcs > 0) carry_term(qpair, qn, qnl, acc);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tt = t0 + 16 * i;
                const float e = gp(static_cast<float>(tt + 1));
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) {
                    const f32x4 o = tt < Lcs ? num[i][jb] + e * acc[i][jb] : zero4;
                    bf16x4 h, lo;
                    split4(o, h, lo);
                    st4(T[4 + sc], tt, 16 * jb + 4 * g, h);
                    st4(T[16 + sc], tt, 16 * jb + 4 * g, lo);
                }
            }
        };

        if constexpr (CH) {
            // the first map: its output stays in LDS as the second map's values
            csums(IC<0>{});
            publish_sums(a.flags, a.aggC);
            local_part(IC<QM>{}, IC<0>{}, qn, qnl);
            carry(a.flags, a.aggC, false, true);
            output_values(IC<QM>{}, qn, qnl);
            __syncthreads();
            // the second map over those values (a pair), with its own hand-off
            csums(IC<1>{});
            publish_sums(a.flags2, a.aggC2);
            local_part(IC<QM>{}, IC<1>{}, qn, qnl);
            carry(a.flags2, a.aggC2, true, true);
            output(IC<OUT>{}, IC<QM>{}, qn, qnl, a.out, a.oh, a.ol, a.bias);
        } else {
            csums(IC<0>{});
            publish_sums(a.flags, a.aggC);
            if constexpr (OUT != kNone) {
                local_part(IC<QM>{}, IC<0>{}, qn, qnl);
                carry(a.flags, a.aggC, true, true);
                if constexpr (Q2) {  // the second queries' loads go out now, used after the first output
                    u32x4 q2r[2][2][2];
                    load_q(IC<Q2M>{}, a.q2, a.q2l, a.q2f, q2r);
                    output(IC<OUT>{}, IC<QM>{}, qn, qnl, a.out, a.oh, a.ol, a.bias);
                    bf16x8 qn2[2][2], qnl2[2][2];
                    to_q(IC<Q2M>{}, q2r, qn2, qnl2);
                    local_part(IC<Q2M>{}, IC<0>{}, qn2, qnl2);
                    output(IC<OUT2>{}, IC<Q2M>{}, qn2, qnl2, a.out2, a.oh2, a.ol2, nullptr);
                } else {
                    output(IC<OUT>{}, IC<QM>{}, qn, qnl, a.out, a.oh, a.ol, a.bias);
                }
            } else if (a.fin != nullptr && last) {  // only the final carry
                carry(a.flags, a.aggC, true, false);
            }
        }
        __syncthreads();  // this segment's LDS reads are done before the next one is staged
    };
    // segments by ticket when they wait on each other (see fwd_fast64.hip)
    auto take = [&]() -> int {
        int *sl = reinterpret_cast<int *>(T[3]);
        if (tid == 0) {
            int t;
            if constexpr (LOOP) {
                t = static_cast<int>(
                    __hip_atomic_fetch_add(&a.ctrl[kTicketWord], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            } else {
                const int head = block % a.BH;
                uint32_t *cnt = &a.ctrl[kHeadTicketWord + kHeadTicketStride * (head_base + head)];
                const int pp = static_cast<int>(__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                if (pp == a.P - 1) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                t = pp * a.BH + head;
            }
            *sl = t;
        }
        __syncthreads();
        const int t = __builtin_amdgcn_readfirstlane(*sl);
        __syncthreads();
        return t;
    };
    const int seg0 = a.P > 1 ? take() : block;
    epoch = next_epoch(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(ep_raw))));
    if constexpr (LOOP) {
        for (int seg = seg0; seg < a.segs; seg = a.P > 1 ? take() : seg + nblocks) seg_body(seg);
    } else if (seg0 < a.segs) {
        seg_body(seg0);
    } else if (tid == 0) {  // a ticket out of range: the control block was not zero before first use
        __hip_atomic_fetch_add(&a.ctrl[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return epoch;
}

// The last workgroup of a launch to finish resets the looped grid's ticket
// and advances the epoch for the next launch.
__device__ __forceinline__ void la_done(uint32_t *ctrl, uint32_t epoch) {
    if (threadIdx.x == 0) {
        const uint32_t done = __hip_atomic_fetch_add(&ctrl[kLine], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            __hip_atomic_store(&ctrl[kLine], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&ctrl[kTicketWord], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&ctrl[kLine + 1], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(&ctrl[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <class M>
__global__ __launch_bounds__(kLThreads, 1) void k_la64(LaArgs a) {
    __shared__ LaSmem<M::kTiles> sm;
    const uint32_t epoch = M::run(a, sm.T, static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x), 0);
    la_done(a.ctrl, epoch);
}

// Two independent maps in one grid (one-pass): workgroups below a.segs take
// the first map's segments, the rest the second's, each by its own per-head
// tickets, flags and aggregates.  No wait crosses the maps.
template <class MA, class MB>
__global__ __launch_bounds__(kLThreads, 1) void k_la64_pair(LaArgs a, LaArgs b) {
    __shared__ LaSmem<(MA::kTiles > MB::kTiles ? MA::kTiles : MB::kTiles)> sm;
    const int blk = static_cast<int>(blockIdx.x);
    const uint32_t epoch = blk < a.segs ? MA::run(a, sm.T, blk, a.segs, 0) : MB::run(b, sm.T, blk - a.segs, b.segs, a.BH);
    la_done(a.ctrl, epoch);
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct LaLayout {
    size_t flags, aggC, total;
};

LaLayout la_layout(int BH, int P) {
    LaLayout L{};
    const size_t slots = static_cast<size_t>(BH) * P;
    L.flags = 0;
    L.aggC = align256(slots * kLWaves * kFlagStride * sizeof(uint32_t));
    L.total = L.aggC + slots * 4096 * sizeof(float);
    return L;
}

void la_geometry(int BH, int nc, int *P, int *L) {
    const int target = (256 + BH - 1) / BH;
    int l = (nc + target - 1) / target;
    l = l < 1 ? 1 : (l > kLMaxL ? kLMaxL : l);
    *L = l;
    *P = (nc + l - 1) / l;
}

// key of an operand/direction/output combination
constexpr int la_key(int qm, int km, int vm, bool rev, int mode, int mode2 = -1, int q2m = 0, bool sym = false,
                     bool ch = false) {
    return qm | (km << 2) | (vm << 4) | (rev ? 64 : 0) | (mode << 7) | (mode2 >= 0 ? ((1 + mode2) << 9) | (q2m << 11) : 0) |
           (sym ? 1 << 13 : 0) | (ch ? 1 << 14 : 0);
}

int la_key_of(const LaArgs &a, const LaProblem &p) {
    const int qm = a.qf ? 2 : (a.ql ? 1 : 0), km = a.kf ? 2 : (a.kl ? 1 : 0), vm = a.vf ? 2 : (a.vl ? 1 : 0);
    const int q2m = a.q2f ? 2 : (a.q2l ? 1 : 0);
    const bool two = a.q2 != nullptr || a.q2f != nullptr;
    return la_key(qm, km, vm, p.rev, p.mode, two ? p.mode2 : -1, two ? q2m : 0, p.sym, p.chain);
}

// the operand/direction/output combinations the library uses
template <bool DECAY, bool LOOP>
hipError_t launch_la(const LaArgs &a, dim3 grid, hipStream_t st, int key) {
    const dim3 block(kLThreads);
#define HLA_LA(QM_, KM_, VM_, REV_, OUT_, ...) \
    if (key == la_key(QM_, KM_, VM_, REV_, OUT_, ##__VA_ARGS__)) { \
        hipLaunchKernelGGL((k_la64<LaMap<DECAY, LOOP, OUT_, QM_, KM_, VM_, REV_, ##__VA_ARGS__>>), grid, block, 0, st, a); \
        return hipGetLastError(); \
    }
    HLA_LA(0, 0, 0, false, kSplit)                // first maps of AHLA and third order
    HLA_LA(0, 0, 0, false, kStore)                // a plain map
    HLA_LA(0, 0, 1, false, kStore)                // AHLA's second map (values as a pair)
    HLA_LA(0, 2, 0, true, kSplit)                 // backward: W = LA^rev (V, dO, Q; g^2)
    HLA_LA(0, 0, 0, false, kSplit, kStore, 1)     // backward: U = LA (Q, K, K; g) and LA (W, K, K; g)
    HLA_LA(2, 0, 1, false, kAccumulate)           // backward: + LA (dO, V, U; g^2)
    HLA_LA(0, 0, 1, true, kStore, -1, 0, true)    // backward: LA^rev (K, Q, W; g) + LA^rev (K, W, Q; g)
    HLA_LA(1, 0, 2, true, kStore)                 // backward: LA^rev (U, Q, dO; g^2)
    HLA_LA(1, 0, 0, false, kStore)                // backward with states: LA (W, K, K; g)
    HLA_LA(0, 0, 0, false, kNone)                 // backward with states: the final carry of (Q, V; g)
    HLA_LA(0, 0, 0, false, kStore, -1, 0, false, true)  // AHLA: LA (Q, K, LA (Q, K, V)) chained
#undef HLA_LA
    return hipErrorInvalidValue;
}

// the pairs of independent maps the backward launches together
template <bool D> using MapUdq = LaMap<D, false, kSplit, 0, 0, 0, false, kStore, 1>;
template <bool D> using MapDk = LaMap<D, false, kStore, 0, 0, 1, true, -1, 0, true>;
template <bool D> using MapDq2 = LaMap<D, false, kAccumulate, 2, 0, 1, false>;
template <bool D> using MapDv = LaMap<D, false, kStore, 1, 0, 2, true>;
template <bool D> using MapU = LaMap<D, false, kSplit, 0, 0, 0, false>;
template <bool D> using MapCfin = LaMap<D, false, kNone, 0, 0, 0, false>;
template <bool D> using MapDq1 = LaMap<D, false, kStore, 1, 0, 0, false>;

template <bool DECAY>
hipError_t launch_la_pair(const LaArgs &a, const LaArgs &b, hipStream_t st, int ka, int kb) {
    const dim3 block(kLThreads), grid(static_cast<unsigned>(a.segs + b.segs));
    if (ka == la_key(0, 0, 0, false, kSplit, kStore, 1) && kb == la_key(0, 0, 1, true, kStore, -1, 0, true)) {
        hipLaunchKernelGGL((k_la64_pair<MapUdq<DECAY>, MapDk<DECAY>>), grid, block, 0, st, a, b);
        return hipGetLastError();
    }
    if (ka == la_key(2, 0, 1, false, kAccumulate) && kb == la_key(1, 0, 2, true, kStore)) {
        hipLaunchKernelGGL((k_la64_pair<MapDq2<DECAY>, MapDv<DECAY>>), grid, block, 0, st, a, b);
        return hipGetLastError();
    }
    if (ka == la_key(0, 0, 0, false, kSplit) && kb == la_key(0, 0, 0, false, kNone)) {
        hipLaunchKernelGGL((k_la64_pair<MapU<DECAY>, MapCfin<DECAY>>), grid, block, 0, st, a, b);
        return hipGetLastError();
    }
    if (ka == la_key(1, 0, 0, false, kStore) && kb == la_key(0, 0, 1, true, kStore, -1, 0, true)) {
        hipLaunchKernelGGL((k_la64_pair<MapDq1<DECAY>, MapDk<DECAY>>), grid, block, 0, st, a, b);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

LaArgs la_args(const LaProblem &p, uint32_t *ctrl, LaSpace sp) {
    LaArgs a{};
    a.H = p.H; a.n = p.n; a.nc = (p.n + W - 1) / W; a.BH = p.B * p.H;
    la_geometry(a.BH, a.nc, &a.P, &a.L);
    a.segs = a.BH * a.P;
    a.q = static_cast<const uint16_t *>(p.q);
    a.k = static_cast<const uint16_t *>(p.k);
    a.v = static_cast<const uint16_t *>(p.v);
    a.ql = static_cast<const uint16_t *>(p.ql);
    a.kl = static_cast<const uint16_t *>(p.kl);
    a.vl = static_cast<const uint16_t *>(p.vl);
    a.qf = p.qf; a.kf = p.kf; a.vf = p.vf;
    a.q2 = static_cast<const uint16_t *>(p.q2);
    a.q2l = static_cast<const uint16_t *>(p.q2l);
    a.q2f = p.q2f;
    a.out2 = p.out2; a.oh2 = p.oh2; a.ol2 = p.ol2;
    a.out = p.out; a.oh = p.oh; a.ol = p.ol;
    a.init = p.init; a.fin = p.fin; a.bias = p.bias;
    a.ctrl = ctrl;
    a.flags = sp.flags;
    a.aggC = sp.aggC;
    a.gam = p.gam;
    a.gexp = p.gsq ? 2.0f : 1.0f;
    return a;
}

bool la_decay(const LaProblem &p) {
    const int nh = p.gam.per_head ? p.H : 1;
    bool decay = false;
    for (int h = 0; h < nh; ++h) decay = decay || p.gam.g[h] != 1.0f;
    return decay;
}

hipError_t cu_count(int *cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    return e;
}

}  // namespace

size_t la64_flag_bytes(int BH, int n) {
    int P, L;
    la_geometry(BH, (n + W - 1) / W, &P, &L);
    return la_layout(BH, P).aggC;
}

size_t la64_agg_bytes(int BH, int n) {
    int P, L;
    la_geometry(BH, (n + W - 1) / W, &P, &L);
    const LaLayout l = la_layout(BH, P);
    return l.total - l.aggC;
}

hipError_t la64_forward_in(const LaProblem &p, uint32_t *ctrl, LaSpace sp, hipStream_t st) {
    const LaArgs a = la_args(p, ctrl, sp);
    int cus = 0;
    const hipError_t e = cu_count(&cus);
    if (e != hipSuccess) return e;
    const bool loop = a.segs > cus || (a.P > 1 && a.BH > kMaxTicketHeads);
    const dim3 grid(static_cast<unsigned>(loop ? cus : a.segs));
    const int key = la_key_of(a, p);
    if (la_decay(p)) return loop ? launch_la<true, true>(a, grid, st, key) : launch_la<true, false>(a, grid, st, key);
    return loop ? launch_la<false, true>(a, grid, st, key) : launch_la<false, false>(a, grid, st, key);
}

hipError_t la64_chain(const LaProblem &p, uint32_t *ctrl, LaSpace s1, LaSpace s2, hipStream_t st) {
    LaProblem q = p;
    q.chain = true;
    LaArgs a = la_args(q, ctrl, s1);
    a.flags2 = s2.flags;
    a.aggC2 = s2.aggC;
    int cus = 0;
    const hipError_t e = cu_count(&cus);
    if (e != hipSuccess) return e;
    const bool loop = a.segs > cus || (a.P > 1 && a.BH > kMaxTicketHeads);
    const dim3 grid(static_cast<unsigned>(loop ? cus : a.segs));
    const int key = la_key_of(a, q);
    if (la_decay(q)) return loop ? launch_la<true, true>(a, grid, st, key) : launch_la<true, false>(a, grid, st, key);
    return loop ? launch_la<false, true>(a, grid, st, key) : launch_la<false, false>(a, grid, st, key);
}

hipError_t la64_forward_pair(const LaProblem &pa, LaSpace sa, const LaProblem &pb, LaSpace sb, uint32_t *ctrl,
                             hipStream_t st) {
    const LaArgs a = la_args(pa, ctrl, sa), b = la_args(pb, ctrl, sb);
    int cus = 0;
    hipError_t e = cu_count(&cus);
    if (e != hipSuccess) return e;
    // one grid when each map alone would take the one-pass grid and the
    // per-head ticket counters of both fit the control block
    const bool one = a.segs <= cus && b.segs <= cus && a.BH + b.BH <= kMaxTicketHeads && la_decay(pa) == la_decay(pb);
    if (one) {
        const int ka = la_key_of(a, pa), kb = la_key_of(b, pb);
        e = la_decay(pa) ? launch_la_pair<true>(a, b, st, ka, kb) : launch_la_pair<false>(a, b, st, ka, kb);
        if (e != hipErrorInvalidValue) return e;
        (void)hipGetLastError();
    }
    if ((e = la64_forward_in(pa, ctrl, sa, st)) != hipSuccess) return e;
    return la64_forward_in(pb, ctrl, sb, st);
}

}  // namespace hla
