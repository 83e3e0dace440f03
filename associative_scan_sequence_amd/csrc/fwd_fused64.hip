// fwd_fused64.hip -- one-launch masked second-order HLA forward for
// d = dv = 64, chunk w = 64, bf16 q/k/v, on gfx950 MFMA.
//
// Method (Higher-order Linear Attention, paperlayer.ai summary sec. 4 and 5):
// inside each chunk the token-level exclusive scan is evaluated as masked
// w x w products, and chunk summaries are scanned to give carry-ins.  The
// carry is held in the corrected form (S, X = S C - G), for which
//   X_t = g^2 X_{t-1} + S_t q_t v_t^T,   num_t = q_t^T X_t,
// so both S and X are *linear* scans once S is known (fwd_generic.hip gives
// the per-chunk formulas).  Per chunk (local token indices t, s; length L;
// e_t = g^(t+1), f_s = g^(L-1-s)):
//   A   = (Q K^T) o D_g o L                       masked scores
//   U   = diag(e) Q S0 + A K                      row s = S_s q_s
//   P   = (Q U^T) o D_{g^2} o L
//   num = P V + diag(e^2) Q X0
//   S0 <- g^L S0 + K^T diag(f) K,   X0 <- g^2L X0 + U^T diag(f^2) V
// With ridge lambda and the denominator (y = S m - h is carried like X with
// v = 1; C and m are plain decayed sums):
//   R   = (Q Q^T) o D_g o L,   P' = P + lambda R
//   num = P' V + diag(e^2) Q X0 + lambda diag(e) Q C0
//   den = P' 1 + diag(e^2) Q y0 + lambda diag(e) Q m0,   out = num or num / den
//   C0 <- g^L C0 + Q^T diag(f) V,  m0 <- g^L m0 + Q^T f,  y0 <- g^2L y0 + Us^T 1
// U is kept scaled as Us = diag(f^2) U.  Then the X update needs no further
// scaling, and since g^(2(t-s)) / f_s^2 = 1 / f_t^2 the masked P is
// (Q Us^T) o L scaled by 1 / f_t^2 per row.  (The kernel is used for
// g >= 0.75, so f^2 >= 0.75^126 and no scaled value leaves the normal range.)
//
// Parallel structure.  One workgroup owns a segment of up to four
// consecutive chunks of one head and runs two groups of four waves; group 0
// walks the segment's first two chunks and group 1 the last two, at the same
// time.  Group 1 starts from the key moment and X increment that group 0
// accumulates, handed over through LDS.  Two device-wide rounds:
//   A: the segment's key moment sum S_seg (both chunks, from zero); publish.
//      While the predecessors' sums travel, compute the carry-free parts of
//      every chunk: the masked scores A and A K.
//      Round 1: sum the decayed S_seg of every earlier segment -> S carry.
//   B: per chunk, U with the true S carry, P, the local part of num (kept in
//      registers) and the segment's X increment Z_seg; publish.
//      Round 2: sum the decayed Z_seg of every earlier segment -> X carry.
//   C: add diag(e^2) Q X0 (and the ridge and denominator carry terms) for
//      every chunk, divide if normalising, and store.
// C and m need no S carry; they travel with X in round 2.
// Both rounds are plain decayed sums of published aggregates (no serial
// chain between segments).  Segment s = p * BH + head.  The grid never
// exceeds the CU count and a workgroup fills a CU, so every workgroup of the
// launch is resident at once; workgroup b takes segments b, b + grid, ... in
// increasing order and waits only on smaller segments of the same head, so
// every wait is on work that is running or done and no wait can close a
// cycle.  Flags carry the launch epoch, so stale or foreign words in the flag
// area are never mistaken for a publication; the last workgroup to finish
// advances the epoch.
//
// Precision.  q, k, v are exact in bf16.  Every operand formed in fp32 (A,
// Us, P, S0, X0, and f-scaled K) is split as x = hi + lo with hi = bf16(x),
// lo = bf16(x - hi); each such product is two bf16 MFMAs with fp32
// accumulation, leaving ~2^-17 relative operand error.  Us enters P with a
// third term (x = hi + mid + lo to ~2^-26), held in the S0-hi tile once the
// S0 reads are done: q_t . Us_s cancels heavily when q_t is nearly
// orthogonal to S_s q_s (at t = s = 0 the value is (q.k)^2), where a
// two-term Us would leave an error of ~2^-18 / cos(q, S q).
//
// MFMA v_mfma_f32_16x16x32_bf16: lane l = 16 g + r supplies row r of the A
// operand and column r of the B operand at k = 8g .. 8g+7, and receives
// accumulator rows 4g .. 4g+3 of column r.  Two consequences are used:
//  * an accumulator pair (row blocks 2j, 2j+1) is directly a k-block operand
//    for a contraction over its row index, with k slot 8g+e holding row
//    32j+4g+e (e < 4) or 32j+16+4g+(e-4); the other operand is read with the
//    same slot order;
//  * operands whose k index runs down the rows of a row-major LDS tile (K,
//    V, Us read as transposes) are fetched with ds_read_b64_tr_b16: within
//    each 16-lane group, lane i receives element i&3 of the 8-byte pieces
//    addressed by lanes (i>>2)+4e, e = 0..3.
// Each wave owns a 16-token slice of its group's chunk; group 1 takes the
// slices in reverse order, so every SIMD pairs a light and a heavy slice of
// the masked (triangular) products.
#include "fused64_common.h"

namespace hla {
namespace {

constexpr int kLay = kPadded;  // LDS tile layout (this kernel is short of registers)
constexpr int kThreads = 512;  // two groups of four waves
constexpr int kPerGroup = 2;   // chunks per wave group
constexpr int kMaxL = 4;       // chunks per workgroup

struct FusedArgs {
    int H, n, nc, P, L, BH, segs;  // segs = BH * P
    const uint16_t *q, *k, *v;
    float *out, *den;   // den may be null
    float ridge;
    uint32_t *ctrl;     // line 0: [2] launch count, [3] wait-timeout count;
                        // line 1: [0] finished workgroups, [1] launch epoch;
                        // from word kTabWord: [workgroup] (epoch << 32) | XCD id
    uint32_t *flags;    // [BH * P][2] at kFlagStride words: epoch when the S sum /
                        // X increment was published
    float *aggS, *aggX, *aggC;  // [BH * P][4096], in accumulator order
    float *aggV;        // [BH * P][128]: y then m
    GammaTab gam;
};

// A group's 16 floats per thread (4 accumulator tiles) <-> a 16 KB slot; the
// thread's 64 bytes sit at byte offset 64 * xi, xi = its tile position.
// (local: plain stores, which the XCD's L2 holds; else written through)
__device__ __forceinline__ void put16(const float *slot, int xi, const f32x4 (&x)[4], bool local) {
    const __amdgpu_buffer_rsrc_t rs = slot_rsrc(slot);
    if (local) {
#pragma unroll
        for (int b = 0; b < 4; ++b) __builtin_amdgcn_raw_buffer_store_b128(x[b], rs, 64 * xi + 16 * b, 0, 0);
    } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) __builtin_amdgcn_raw_buffer_store_b128(x[b], rs, 64 * xi + 16 * b, 0, kSc1);
    }
}

// acc += sum over n slots of scale[i] * slot_i; all loads of a batch are
// issued before the first add.
template <int NB, int POL>
__device__ __forceinline__ void add_slots(f32x4 (&acc)[4], const float *const (&slots)[NB],
                                          const float (&scale)[NB], int n, int xi) {
    f32x4 v[NB][4];
#pragma unroll
    for (int s = 0; s < NB; ++s)
        if (s < n) {
            const __amdgpu_buffer_rsrc_t rs = slot_rsrc(slots[s]);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                v[s][b] = __builtin_amdgcn_raw_buffer_load_b128(rs, 64 * xi + 16 * b, 0, POL);
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
    __bf16 K[kPerGroup][kTileElems<kLay>];  // key rows [s][a] of the group's chunks
    __bf16 V[kPerGroup][kTileElems<kLay>];  // value rows [s][j]
    __bf16 Uh[kTileElems<kLay>];            // Us rows [s][b], hi and lo
    __bf16 Ul[kTileElems<kLay>];
    __bf16 Sh[kTileElems<kLay>];            // S0 (symmetric) of the chunk; in phase C X0 as [a][j]
    __bf16 Sl[kTileElems<kLay>];
};

struct Smem {
    GroupLds grp[2];
    float vpart[2][2][4][64];  // [group][y, m][wave]: per-wave sums of one chunk
    float vec[2][8][64];       // [group]: y, y after chunk 0, m, m after chunk 0,
                               //          chunk y0, chunk m0, group start y, m
    float vcar[2][64];         // y and m carries of the segment
    uint32_t epoch;
    int local;
};

// LOOP = false: one segment per workgroup (segs <= grid); true: workgroup b
// takes segments b, b + grid, ... (grid = CU count < segs).
template <bool DECAY, bool RIDGE, bool DEN, bool NORM, bool LOOP>
__global__ __launch_bounds__(kThreads, 1) void k_fused64(FusedArgs a) {
    static_assert(!NORM || DEN, "the ratio needs the denominator");
    constexpr bool MV = RIDGE && DEN;  // the query mass m is only read by the ridge denominator term
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    // ---- launch epoch: read now, first needed when the segment sum is published
    uint32_t ep_raw = 0;
    if (tid == 0) ep_raw = __hip_atomic_load(&a.ctrl[kLine + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    uint32_t epoch = 0;
    const u32x4 z4 = u32x4{0u, 0u, 0u, 0u};
    const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
    float lg = 0.0f;
    auto gp = [&](float e) { return DECAY ? __builtin_amdgcn_exp2f(e * lg) : 1.0f; };  // g^e
    auto seg_body = [&](const int seg) __attribute__((always_inline)) {
        // lane indices, laundered per pass in the looped launch so that the
        // address arithmetic built on them is not hoisted out of the loop
        int tid_l = static_cast<int>(threadIdx.x);
        if constexpr (LOOP) asm volatile("" : "+v"(tid_l));
        const int grp = tid_l >> 8, wt = tid_l & 255;
        const int wv = wt >> 6, l = wt & 63, r = l & 15, g = l >> 4;
        const int w = grp == 0 ? wv : 3 - wv;  // this wave's 16-token slice
        const int xi = 64 * w + l;  // position of this thread's tiles in exchanges and aggregate slots
        const int t = 16 * w + r;   // this lane's token (column of the B operand)
        GroupLds &G = sm.grp[grp];
        const int jbase = kPerGroup * grp;
        // ---- global loads of this group's chunks: keys and queries now, values
        // once the segment's key moment is published (the publishing stores must
        // not wait behind them, and phase B is the first to read them).  The
        // loads are unconditional (rows past the chunk read the head's first row)
        // and are masked to zero only where they are used, so each use waits for
        // its own loads alone.
        u32x4 kx[kPerGroup][2], vx[kPerGroup][2], qx[kPerGroup][2];
        auto issue_loads = [&](int sg_) __attribute__((always_inline)) {
            const int bh_ = sg_ % a.BH, p_ = sg_ / a.BH;
            const size_t head_tok_ = static_cast<size_t>(bh_) * a.n;
            const int c0_ = p_ * a.L;
            const int Lseg_ = min(a.L, a.nc - c0_);
            int Lcs[kPerGroup];
            size_t tok0s[kPerGroup];
#pragma unroll
            for (int jj = 0; jj < kPerGroup; ++jj) {
                const int j = kPerGroup * grp + jj;
                Lcs[jj] = j < Lseg_ ? min(W, a.n - (c0_ + j) * W) : 0;
                tok0s[jj] = head_tok_ + static_cast<size_t>(c0_ + j) * W;
            }
#pragma unroll
            for (int jj = 0; jj < kPerGroup; ++jj)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int idx = wt + 256 * u, row = idx >> 3, cg = idx & 7;
                    const size_t src = row < Lcs[jj] ? tok0s[jj] + row : head_tok_;
                    kx[jj][u] = *reinterpret_cast<const u32x4 *>(a.k + src * W + cg * 8);
                }
#pragma unroll
            for (int jj = 0; jj < kPerGroup; ++jj)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const size_t src = t < Lcs[jj] ? tok0s[jj] + t : head_tok_;
                    qx[jj][ks] = *reinterpret_cast<const u32x4 *>(a.q + src * W + 32 * ks + 8 * g);
                }
        };
        auto issue_v_loads = [&](int sg_) __attribute__((always_inline)) {
            const int bh_ = sg_ % a.BH, p_ = sg_ / a.BH;
            const size_t head_tok_ = static_cast<size_t>(bh_) * a.n;
            const int c0_ = p_ * a.L;
            const int Lseg_ = min(a.L, a.nc - c0_);
#pragma unroll
            for (int jj = 0; jj < kPerGroup; ++jj) {
                const int j = kPerGroup * grp + jj;
                const int Lc = j < Lseg_ ? min(W, a.n - (c0_ + j) * W) : 0;
                const size_t tok0 = head_tok_ + static_cast<size_t>(c0_ + j) * W;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int idx = wt + 256 * u, row = idx >> 3, cg = idx & 7;
                    const size_t src = row < Lc ? tok0 + row : head_tok_;
                    vx[jj][u] = *reinterpret_cast<const u32x4 *>(a.v + src * W + cg * 8);
                }
            }
        };
        issue_loads(seg);
        const bool first = seg == static_cast<int>(blockIdx.x);
        uint64_t *const xtab = reinterpret_cast<uint64_t *>(a.ctrl + kTabWord);
        const bool tab_ok = static_cast<int>(gridDim.x) <= kTabCap;
        if (tid == 0 && first && tab_ok)  // this workgroup's XCD, tagged with the launch epoch
            __hip_atomic_store(xtab + blockIdx.x, (static_cast<uint64_t>(next_epoch(ep_raw)) << 32) | 0x100u | xcd_id(),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int bh = seg % a.BH, p = seg / a.BH;
        const size_t head_tok = static_cast<size_t>(bh) * a.n;
        lg = DECAY ? log2f(head_gamma(a.gam, bh % a.H)) : 0.0f;
        const int c0 = p * a.L;
        const int Lseg = min(a.L, a.nc - c0);  // chunks in this segment (>= 1)
        const int nmine = max(0, min(kPerGroup, Lseg - jbase));
        auto chunk_len = [&](int j) { return min(W, a.n - (c0 + j) * W); };
        int lenA = 0, lenB = 0;  // tokens covered by group 0 and group 1
        for (int j = 0; j < Lseg; ++j) (j < kPerGroup ? lenA : lenB) += chunk_len(j);
        const int len0 = nmine > 0 ? chunk_len(jbase) : 0;  // this group's first chunk
        int lc_of[kPerGroup];  // tokens in this group's chunk jj (0 if none)
#pragma unroll
        for (int jj = 0; jj < kPerGroup; ++jj) lc_of[jj] = jj < nmine ? chunk_len(jbase + jj) : 0;
        f32x4 sc0[4], sg[4];  // first chunk's key moment, group sum

        // ---- stage key rows (values follow once phase A and the carry-free work are issued)
#pragma unroll
        for (int jj = 0; jj < kPerGroup; ++jj)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int idx = wt + 256 * u, row = idx >> 3, cg = idx & 7;
                st16<kLay>(G.K[jj], row, cg * 8, row < lc_of[jj] ? kx[jj][u] : z4);
            }
        __syncthreads();
        // ---- wave 0 fetches the XCD entries of the workgroups that hold this
        // head's segments (segment s runs on workgroup s mod grid); they were
        // written at the start, and are checked after phase A
        uint64_t tabv = 0;
        if (tid < 64 && tid < a.P && tab_ok)
            tabv = __hip_atomic_load(xtab + (tid * a.BH + bh) % static_cast<int>(gridDim.x), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);

        // ================= phase A: the segment's key moment sum ==================
        // acc (rows a = 16w+4g+c, cols b = 16bb+r) = K^T diag(f) K of one chunk
    #pragma unroll
        for (int bb = 0; bb < 4; ++bb) sc0[bb] = sg[bb] = zero4;
    #pragma unroll
        for (int jj = 0; jj < kPerGroup; ++jj) {
            if (jj < nmine) {
                const int Lc = chunk_len(jbase + jj);
                f32x4 acc[4];
    #pragma unroll
                for (int bb = 0; bb < 4; ++bb) acc[bb] = zero4;
    #pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int rb = 32 * ks + 8 * g;
                    const bf16x8 ka = tr8<kLay>(G.K[jj], rb, rb + 4, 16 * w, r);
                    bf16x8 kb[4];
    #pragma unroll
                    for (int bb = 0; bb < 4; ++bb) kb[bb] = tr8<kLay>(G.K[jj], rb, rb + 4, 16 * bb, r);
                    if (!DECAY) {
    #pragma unroll
                        for (int bb = 0; bb < 4; ++bb) acc[bb] = mfma(ka, kb[bb], acc[bb]);
                    } else {
                        f32x4 x0, x1;
    #pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            x0[e] = gp(static_cast<float>(Lc - 1 - (rb + e))) * static_cast<float>(ka[e]);
                            x1[e] = gp(static_cast<float>(Lc - 1 - (rb + 4 + e))) * static_cast<float>(ka[4 + e]);
                        }
                        bf16x8 h, lo;
                        pair_operand(x0, x1, h, lo);
    #pragma unroll
                        for (int bb = 0; bb < 4; ++bb) acc[bb] = mfma(h, kb[bb], acc[bb]);
    #pragma unroll
                        for (int bb = 0; bb < 4; ++bb) acc[bb] = mfma(lo, kb[bb], acc[bb]);
                    }
                }
                const float rho = gp(static_cast<float>(Lc));
    #pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    if (jj == 0) sc0[bb] = acc[bb];
                    sg[bb] = rho * sg[bb] + acc[bb];
                }
            }
        }

        // ---- the exchange with other segments of this head goes through the
        // XCD's L2 when every one of them runs on this XCD, else device-coherently;
        // all of them read the same entries, so they all take the same choice
        if (tid < 64) {
            const uint32_t ep_now = first ? next_epoch(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(ep_raw))))
                                          : epoch;
            const bool all = head_on_one_xcd(xtab, tab_ok, a.P, a.BH, bh, ep_now, tabv);
            if (tid == 0) sm.local = all ? 1 : 0;
        }
        // group 0 hands its sum to group 1, which publishes the segment sum
        float *xch = reinterpret_cast<float *>(sm.grp[1].Uh);  // 16 KB inside group 1's U tiles
        if (grp == 0) {
#pragma unroll
            for (int b = 0; b < 4; ++b) *reinterpret_cast<f32x4 *>(xch + xi * 16 + 4 * b) = sg[b];
        }
        // the launch epoch (read at the start; its load has long returned)
        if (tid == 0 && first) sm.epoch = ep_raw;
        __syncthreads();
        if (first)
            epoch = next_epoch(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(sm.epoch))));
        const bool local = __builtin_amdgcn_readfirstlane(sm.local) != 0;
        const size_t slot = static_cast<size_t>(bh) * a.P + p;
        f32x4 partA[4];  // group 0's sum (group 1 only)
        if (grp == 1) {
#pragma unroll
            for (int b = 0; b < 4; ++b) partA[b] = *reinterpret_cast<const f32x4 *>(xch + xi * 16 + 4 * b);
            f32x4 agg[4];
            const float rhoB = gp(static_cast<float>(lenB));
#pragma unroll
            for (int b = 0; b < 4; ++b) agg[b] = rhoB * partA[b] + sg[b];
            put16(a.aggS + slot * 4096, xi, agg, local);
            wait_stores();
        }
        __syncthreads();
        if (tid == 0) set_flag(&a.flags[2 * slot * kFlagStride], epoch, local);
        issue_v_loads(seg);

        bf16x8 qn[kPerGroup][2];  // q of token 16w+r, features 32ks+8g..: B operand
#pragma unroll
        for (int jj = 0; jj < kPerGroup; ++jj)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) qn[jj][ks] = __builtin_bit_cast(bf16x8, t < lc_of[jj] ? qx[jj][ks] : z4);

        // ---- carry-free work while the predecessors' sums travel:
        // A^T tiles of this wave's tokens, then Uloc^T = K^T A^T (rows b, cols t)
        f32x4 uloc[kPerGroup][4];
#pragma unroll
        for (int jj = 0; jj < kPerGroup; ++jj) {
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) uloc[jj][bb] = zero4;
            if (jj < nmine) {
                f32x4 at[4];  // A^T[i = 16ib+4g+c][t], masked and decayed
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    at[ib] = zero4;
                    if (ib <= w) {
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) at[ib] = mfma(ld8<kLay>(G.K[jj], 16 * ib + r, 32 * ks + 8 * g), qn[jj][ks], at[ib]);
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int i = 16 * ib + 4 * g + c;
                            at[ib][c] = i <= t ? gp(static_cast<float>(t - i)) * at[ib][c] : 0.0f;
                        }
                    }
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (2 * ks <= w) {
                        bf16x8 ah, al;
                        pair_operand(at[2 * ks], at[2 * ks + 1], ah, al);
#pragma unroll
                        for (int bb = 0; bb < 4; ++bb) {
                            const bf16x8 kt = tr8<kLay>(G.K[jj], 32 * ks + 4 * g, 32 * ks + 16 + 4 * g, 16 * bb, r);
                            uloc[jj][bb] = mfma(kt, ah, uloc[jj][bb]);
                            uloc[jj][bb] = mfma(kt, al, uloc[jj][bb]);
                        }
                    }
                }
            }
        }

        // ---- carry = sum over earlier segments pp of g^(pw * gap) * agg[pp] (gap =
        // tokens between); the groups each load every other predecessor and swap
        // their partial sums through LDS (the U tiles, unused here).
        const int seg_tokens = a.L * W;
        auto sum_earlier = [&](f32x4 (&acc)[4], const float *agg, int pw) {
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
                    scale[s2] = gp(static_cast<float>(pw * (p - 1 - pp) * seg_tokens));
                }
                if (local) add_slots<NB, 0>(acc, slots, scale, cnt, xi);
                else add_slots<NB, kSc1>(acc, slots, scale, cnt, xi);
            }
            float *mine = reinterpret_cast<float *>(sm.grp[grp].Uh);
            const float *other = reinterpret_cast<const float *>(sm.grp[grp ^ 1].Uh);
            __syncthreads();  // both U areas free
#pragma unroll
            for (int b = 0; b < 4; ++b) *reinterpret_cast<f32x4 *>(mine + xi * 16 + 4 * b) = acc[b];
            __syncthreads();
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[b] += *reinterpret_cast<const f32x4 *>(other + xi * 16 + 4 * b);
            __syncthreads();  // U areas may be written again
        };
        auto wait_round = [&](int which) {
            for (int pp = tid; pp < p; pp += kThreads)
                if (!wait_flag(&a.flags[(2 * (static_cast<size_t>(bh) * a.P + pp) + which) * kFlagStride], epoch, local))
                    __hip_atomic_fetch_add(&a.ctrl[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
        };

        // ---- value rows (read from phase B on; the next barrier publishes them)
#pragma unroll
        for (int jj = 0; jj < kPerGroup; ++jj)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int idx = wt + 256 * u, row = idx >> 3, cg = idx & 7;
                st16<kLay>(G.V[jj], row, cg * 8, row < lc_of[jj] ? vx[jj][u] : z4);
            }
        // ---- round 1: the S carry at this group's first chunk
        wait_round(0);
        f32x4 s0[4];
        {
            f32x4 carry[4];
            sum_earlier(carry, a.aggS, 1);
            const float rhoA = gp(static_cast<float>(lenA));
#pragma unroll
            for (int b = 0; b < 4; ++b) s0[b] = grp == 0 ? carry[b] : rhoA * carry[b] + partA[b];
        }

        // ================= phase B: each group walks its chunks ===================
        const float lam = a.ridge;
        f32x4 num[kPerGroup][4];
        f32x4 xacc[4], xsave[4];  // X^T increment, rows j = 16w+4g+c, cols a = 16ab+r
        f32x4 cacc[4], csave[4];  // C^T increment (ridge), same layout
        float dl[kPerGroup];      // this lane's part of sum_s P'[t][s] (denominator)
#pragma unroll
        for (int b = 0; b < 4; ++b) xacc[b] = xsave[b] = cacc[b] = csave[b] = zero4;
#pragma unroll
        for (int jj = 0; jj < kPerGroup; ++jj) dl[jj] = 0.0f;
        if (RIDGE) {  // the key tiles are no longer read: they now hold the query rows
#pragma unroll
            for (int jj = 0; jj < kPerGroup; ++jj)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    st16<kLay>(G.K[jj], t, 32 * ks + 8 * g, __builtin_bit_cast(u32x4, qn[jj][ks]));
        }
        if (DEN && wt < 64) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.vec[grp][i][wt] = 0.0f;
        }
#pragma unroll
        for (int jj = 0; jj < kPerGroup; ++jj) {
            const bool valid = jj < nmine;
            const int Lc = valid ? chunk_len(jbase + jj) : 0;
            // S0 -> LDS as hi/lo; lane holds S0[a = 16w+4g+c][b = 16bb+r] = S0[b][a]
            if (valid) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    bf16x4 h, lo;
                    split4(s0[bb], h, lo);
                    st4<kLay>(G.Sh, 16 * bb + r, 16 * w + 4 * g, h);
                    st4<kLay>(G.Sl, 16 * bb + r, 16 * w + 4 * g, lo);
                }
            }
            __syncthreads();  // (1) S0 ready; previous chunk's Us reads done
            f32x4 usv[4];  // Us^T[b = 16bb+4g+c][t] of this wave's tokens
            if (valid) {
                // U^T[b][t] = e_t (S0 q_t)[b] + Uloc^T[b][t]; stored as Us = f_t^2 U rows
                const float e = gp(static_cast<float>(t + 1));
                const float f2 = t < Lc ? gp(static_cast<float>(2 * (Lc - 1 - t))) : 0.0f;
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    f32x4 acc = zero4;
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        acc = mfma(ld8<kLay>(G.Sh, 16 * bb + r, 32 * ks + 8 * g), qn[jj][ks], acc);
                        acc = mfma(ld8<kLay>(G.Sl, 16 * bb + r, 32 * ks + 8 * g), qn[jj][ks], acc);
                    }
                    usv[bb] = f2 * (e * acc + uloc[jj][bb]);
                }
            }
            // Us's third term goes to the key tile (free in phase B) or, with the
            // ridge (query rows there), to the S0-hi tile once its reads are done
            __bf16 *Ux = RIDGE ? G.Sh : G.K[jj];
            if (RIDGE) __syncthreads();  // (1b)
            if (valid) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const f32x4 us = usv[bb];
                    bf16x4 h, mid, lo;
                    split3(us, h, mid, lo);
                    st4<kLay>(G.Uh, t, 16 * bb + 4 * g, h);
                    st4<kLay>(G.Ul, t, 16 * bb + 4 * g, mid);
                    st4<kLay>(Ux, t, 16 * bb + 4 * g, lo);
                    if (DEN) {  // y increment: sum over this wave's tokens of Us rows
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const float sum = row_sum16(us[c]);
                            if (r == 0) sm.vpart[grp][0][w][16 * bb + 4 * g + c] = sum;
                        }
                    }
                }
                if (MV) {  // m increment: sum over this wave's tokens of f_t q_t
                    const float f = t < Lc ? gp(static_cast<float>(Lc - 1 - t)) : 0.0f;
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                        for (int e8 = 0; e8 < 8; ++e8) {
                            const float sum = row_sum16(f * static_cast<float>(qn[jj][ks][e8]));
                            if (r == 0) sm.vpart[grp][1][w][32 * ks + 8 * g + e8] = sum;
                        }
                }
            }
            __syncthreads();  // (2) every Us row ready
            if (DEN && valid && wt < 64) {  // fold the per-wave sums in a fixed order
                const float (*vp)[4][64] = sm.vpart[grp];
                const float yinc = (vp[0][0][wt] + vp[0][1][wt]) + (vp[0][2][wt] + vp[0][3][wt]);
                float *v = &sm.vec[grp][0][0];
                v[wt] = gp(static_cast<float>(2 * Lc)) * v[wt] + yinc;
                if (jj == 0) v[64 + wt] = v[wt];
                if (MV) {
                    const float minc = (vp[1][0][wt] + vp[1][1][wt]) + (vp[1][2][wt] + vp[1][3][wt]);
                    v[128 + wt] = gp(static_cast<float>(Lc)) * v[128 + wt] + minc;
                    if (jj == 0) v[192 + wt] = v[128 + wt];
                }
            }
            if (valid) {
                // P'^T[s][t] = (Us_s . q_t) / f_t^2 + lambda g^(t-s) (q_s . q_t) for s <= t
                const float inv_f2 = t < Lc ? gp(static_cast<float>(-2 * (Lc - 1 - t))) : 0.0f;
                f32x4 pt[4];
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) {
                    pt[sb] = zero4;
                    if (sb <= w) {
                        f32x4 rt = zero4;
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) {
                            pt[sb] = mfma(ld8<kLay>(G.Uh, 16 * sb + r, 32 * kb + 8 * g), qn[jj][kb], pt[sb]);
                            pt[sb] = mfma(ld8<kLay>(G.Ul, 16 * sb + r, 32 * kb + 8 * g), qn[jj][kb], pt[sb]);
                            pt[sb] = mfma(ld8<kLay>(Ux, 16 * sb + r, 32 * kb + 8 * g), qn[jj][kb], pt[sb]);
                            if (RIDGE) rt = mfma(ld8<kLay>(G.K[jj], 16 * sb + r, 32 * kb + 8 * g), qn[jj][kb], rt);
                        }
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int sidx = 16 * sb + 4 * g + c;
                            float x = inv_f2 * pt[sb][c];
                            if (RIDGE) x += lam * gp(static_cast<float>(t - sidx)) * rt[c];
                            pt[sb][c] = sidx <= t ? x : 0.0f;
                        }
                        if (DEN) dl[jj] += (pt[sb][0] + pt[sb][1]) + (pt[sb][2] + pt[sb][3]);
                    }
                }
                // num^T[j][t] = sum_s V^T[j][s] P[t][s]
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) num[jj][jb] = zero4;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (2 * ks <= w) {
                        bf16x8 ph, pl;
                        pair_operand(pt[2 * ks], pt[2 * ks + 1], ph, pl);
#pragma unroll
                        for (int jb = 0; jb < 4; ++jb) {
                            const bf16x8 vt = tr8<kLay>(G.V[jj], 32 * ks + 4 * g, 32 * ks + 16 + 4 * g, 16 * jb, r);
                            num[jj][jb] = mfma(vt, ph, num[jj][jb]);
                            num[jj][jb] = mfma(vt, pl, num[jj][jb]);
                        }
                    }
                }
                // X^T <- g^2L X^T + V^T Us  (rows j = 16w.., all a)
                const float rho2 = gp(static_cast<float>(2 * Lc));
#pragma unroll
                for (int ab = 0; ab < 4; ++ab) xacc[ab] *= rho2;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int rb = 32 * ks + 8 * g;
                    const bf16x8 vt = tr8<kLay>(G.V[jj], rb, rb + 4, 16 * w, r);
#pragma unroll
                    for (int ab = 0; ab < 4; ++ab) {
                        xacc[ab] = mfma(vt, tr8<kLay>(G.Uh, rb, rb + 4, 16 * ab, r), xacc[ab]);
                        xacc[ab] = mfma(vt, tr8<kLay>(G.Ul, rb, rb + 4, 16 * ab, r), xacc[ab]);
                    }
                }
                if (jj == 0) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) xsave[b] = xacc[b];
                }
                if (RIDGE) {  // C^T <- g^L C^T + (diag(f) V)^T Q  (rows j = 16w.., all a)
                    const float rho = gp(static_cast<float>(Lc));
#pragma unroll
                    for (int ab = 0; ab < 4; ++ab) cacc[ab] *= rho;
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const int rb = 32 * ks + 8 * g;
                        const bf16x8 vt = tr8<kLay>(G.V[jj], rb, rb + 4, 16 * w, r);
                        bf16x8 vh = vt, vl;
                        if (DECAY) {
                            f32x4 x0, x1;
#pragma unroll
                            for (int e4 = 0; e4 < 4; ++e4) {
                                x0[e4] = gp(static_cast<float>(Lc - 1 - (rb + e4))) * static_cast<float>(vt[e4]);
                                x1[e4] = gp(static_cast<float>(Lc - 1 - (rb + 4 + e4))) * static_cast<float>(vt[4 + e4]);
                            }
                            pair_operand(x0, x1, vh, vl);
                        }
#pragma unroll
                        for (int ab = 0; ab < 4; ++ab) {
                            const bf16x8 qt = tr8<kLay>(G.K[jj], rb, rb + 4, 16 * ab, r);
                            cacc[ab] = mfma(vh, qt, cacc[ab]);
                            if (DECAY) cacc[ab] = mfma(vl, qt, cacc[ab]);
                        }
                    }
                    if (jj == 0) {
#pragma unroll
                        for (int b = 0; b < 4; ++b) csave[b] = cacc[b];
                    }
                }
                // S0 of the next chunk
                const float rho = gp(static_cast<float>(Lc));
#pragma unroll
                for (int b = 0; b < 4; ++b) s0[b] = rho * s0[b] + sc0[b];
            } else {
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) num[jj][jb] = zero4;
            }
            if (RIDGE) __syncthreads();  // (2b) the third Us term in the S0-hi tile is read
        }
        __syncthreads();  // U tiles free for the exchange

        // ---- group 1 adds group 0's increments, publishes the segment's X (and
        // C, y, m) increments; round 2
        float *xch2 = reinterpret_cast<float *>(sm.grp[1].Sh);  // 16 KB inside group 1's S tiles
        if (grp == 0) {
#pragma unroll
            for (int b = 0; b < 4; ++b) *reinterpret_cast<f32x4 *>(xch + xi * 16 + 4 * b) = xacc[b];
            if (RIDGE) {
#pragma unroll
                for (int b = 0; b < 4; ++b) *reinterpret_cast<f32x4 *>(xch2 + xi * 16 + 4 * b) = cacc[b];
            }
        }
        __syncthreads();
        f32x4 partC[4];  // group 0's C increment (group 1 only)
        if (grp == 1) {
#pragma unroll
            for (int b = 0; b < 4; ++b) partA[b] = *reinterpret_cast<const f32x4 *>(xch + xi * 16 + 4 * b);
            f32x4 agg[4];
            const float rhoB2 = gp(static_cast<float>(2 * lenB));
#pragma unroll
            for (int b = 0; b < 4; ++b) agg[b] = rhoB2 * partA[b] + xacc[b];
            put16(a.aggX + slot * 4096, xi, agg, local);
            if (RIDGE) {
                const float rhoB = gp(static_cast<float>(lenB));
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    partC[b] = *reinterpret_cast<const f32x4 *>(xch2 + xi * 16 + 4 * b);
                    agg[b] = rhoB * partC[b] + cacc[b];
                }
                put16(a.aggC + slot * 4096, xi, agg, local);
            }
            if (DEN && wt < 64) {
                const float ys = gp(static_cast<float>(2 * lenB)) * sm.vec[0][0][wt] + sm.vec[1][0][wt];
                if (local) __hip_atomic_store(&a.aggV[slot * 128 + wt], ys, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                else __hip_atomic_store(&a.aggV[slot * 128 + wt], ys, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (MV) {
                    const float ms = gp(static_cast<float>(lenB)) * sm.vec[0][2][wt] + sm.vec[1][2][wt];
                    if (local) __hip_atomic_store(&a.aggV[slot * 128 + 64 + wt], ms, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    else __hip_atomic_store(&a.aggV[slot * 128 + 64 + wt], ms, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            wait_stores();
        }
        __syncthreads();
        if (tid == 0) set_flag(&a.flags[(2 * slot + 1) * kFlagStride], epoch, local);
        wait_round(1);
        f32x4 xstart[4], cstart[4];
        {
            f32x4 carry[4];
            sum_earlier(carry, a.aggX, 2);
            const float rhoA2 = gp(static_cast<float>(2 * lenA));
#pragma unroll
            for (int b = 0; b < 4; ++b) xstart[b] = grp == 0 ? carry[b] : rhoA2 * carry[b] + partA[b];
            if (RIDGE) {
                sum_earlier(carry, a.aggC, 1);
                const float rhoA = gp(static_cast<float>(lenA));
#pragma unroll
                for (int b = 0; b < 4; ++b) cstart[b] = grp == 0 ? carry[b] : rhoA * carry[b] + partC[b];
            }
        }
        if (DEN) {
            // vector carries: group 0 sums y, group 1 sums m over earlier segments
            if (wt < 64 && (grp == 0 || MV)) {
                float acc = 0.0f;
                for (int pp = 0; pp < p; ++pp) {
                    float *src = &a.aggV[(static_cast<size_t>(bh) * a.P + pp) * 128 + 64 * grp + wt];
                    const float x = local ? __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
                                          : __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    acc += gp(static_cast<float>((2 - grp) * (p - 1 - pp) * seg_tokens)) * x;
                }
                sm.vcar[grp][wt] = acc;
            }
            __syncthreads();
            if (wt < 64) {  // this group's start: the carry, or (group 1) carried over group 0 plus its sums
                float *v = &sm.vec[grp][0][0];
                v[6 * 64 + wt] = grp == 0 ? sm.vcar[0][wt]
                                          : gp(static_cast<float>(2 * lenA)) * sm.vcar[0][wt] + sm.vec[0][0][wt];
                if (MV)
                    v[7 * 64 + wt] = grp == 0 ? sm.vcar[1][wt]
                                              : gp(static_cast<float>(lenA)) * sm.vcar[1][wt] + sm.vec[0][2][wt];
            }
        }

        // ================= phase C: carry terms of both chunks, ratio, store ======
        // Carries of chunk jj = decayed group start + (local sums before chunk jj).
        // Tiles: chunk 0 X0 in the S tiles, C0 in the U tiles; chunk 1 X0 in the
        // value tiles, C0 in the key tiles (all free once phase B is done).  The
        // lane holds X0^T[j = 16w+4g+c][a = 16ab+r] -> LDS X0[a][j] (C0 likewise).
        if (DEN) __syncthreads();  // group starts read before the chunk vectors are written
        auto xt = [&](int jj, int hl) -> __bf16 * { return jj == 0 ? (hl ? G.Sl : G.Sh) : G.V[hl]; };
        auto ct = [&](int jj, int hl) -> __bf16 * { return jj == 0 ? (hl ? G.Ul : G.Uh) : G.K[hl]; };
#pragma unroll
        for (int jj = 0; jj < kPerGroup; ++jj) {
            if (jj < nmine) {
                const float d2 = jj == 0 ? 1.0f : gp(static_cast<float>(2 * len0));
#pragma unroll
                for (int ab = 0; ab < 4; ++ab) {
                    const f32x4 x0 = d2 * xstart[ab] + (jj == 0 ? zero4 : xsave[ab]);
                    bf16x4 h, lo;
                    split4(x0, h, lo);
                    st4<kLay>(xt(jj, 0), 16 * ab + r, 16 * w + 4 * g, h);
                    st4<kLay>(xt(jj, 1), 16 * ab + r, 16 * w + 4 * g, lo);
                }
                if (RIDGE) {
                    const float d1 = jj == 0 ? 1.0f : gp(static_cast<float>(len0));
#pragma unroll
                    for (int ab = 0; ab < 4; ++ab) {
                        const f32x4 c0v = d1 * cstart[ab] + (jj == 0 ? zero4 : csave[ab]);
                        bf16x4 h, lo;
                        split4(c0v, h, lo);
                        st4<kLay>(ct(jj, 0), 16 * ab + r, 16 * w + 4 * g, h);
                        st4<kLay>(ct(jj, 1), 16 * ab + r, 16 * w + 4 * g, lo);
                    }
                }
                if (DEN && wt < 64) {
                    // chunk 0: y0, m0 in rows 4, 5; chunk 1 in rows 0, 2 (free by now)
                    float *v = &sm.vec[grp][0][0];
                    const int ry = jj == 0 ? 4 : 0, rm = jj == 0 ? 5 : 2;
                    v[ry * 64 + wt] = jj == 0 ? v[6 * 64 + wt] : d2 * v[6 * 64 + wt] + v[64 + wt];
                    if (MV)
                        v[rm * 64 + wt] = jj == 0 ? v[7 * 64 + wt]
                                                  : gp(static_cast<float>(len0)) * v[7 * 64 + wt] + v[3 * 64 + wt];
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int jj = 0; jj < kPerGroup; ++jj) {
            if (jj < nmine) {
                const int Lc = chunk_len(jbase + jj);
                const float e = gp(static_cast<float>(t + 1));
                const float e2 = e * e;
                const size_t trow = head_tok + static_cast<size_t>(c0 + jbase + jj) * W + t;
                float *orow = a.out + trow * W;
                f32x4 acc[4], accc[4];
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) acc[jb] = accc[jb] = zero4;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int rb = 32 * ks + 8 * g;
#pragma unroll
                    for (int jb = 0; jb < 4; ++jb) {
                        acc[jb] = mfma(tr8<kLay>(xt(jj, 0), rb, rb + 4, 16 * jb, r), qn[jj][ks], acc[jb]);
                        acc[jb] = mfma(tr8<kLay>(xt(jj, 1), rb, rb + 4, 16 * jb, r), qn[jj][ks], acc[jb]);
                        if (RIDGE) {
                            accc[jb] = mfma(tr8<kLay>(ct(jj, 0), rb, rb + 4, 16 * jb, r), qn[jj][ks], accc[jb]);
                            accc[jb] = mfma(tr8<kLay>(ct(jj, 1), rb, rb + 4, 16 * jb, r), qn[jj][ks], accc[jb]);
                        }
                    }
                }
                float den = 0.0f;
                if (DEN) {
                    // den_t = sum_s P'[t][s] + e^2 q_t . y0 + lambda e q_t . m0, summed over the 4 lane rows
                    const float *y0 = sm.vec[grp][jj == 0 ? 4 : 0];
                    const float *m0 = sm.vec[grp][jj == 0 ? 5 : 2];
                    float part = dl[jj];
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                        for (int e8 = 0; e8 < 8; ++e8) {
                            const int ai = 32 * ks + 8 * g + e8;
                            float coef = e2 * y0[ai];
                            if (MV) coef += lam * e * m0[ai];
                            part += coef * static_cast<float>(qn[jj][ks][e8]);
                        }
                    part += __shfl_xor(part, 16);
                    den = part + __shfl_xor(part, 32);
                }
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) {
                    f32x4 o = num[jj][jb] + e2 * acc[jb];
                    if (RIDGE) o += (lam * e) * accc[jb];
                    if (NORM) o = o / den;
                    if (t < Lc) *reinterpret_cast<float4 *>(orow + 16 * jb + 4 * g) = make_float4(o[0], o[1], o[2], o[3]);
                }
                if (DEN && a.den != nullptr && g == 0 && t < Lc) a.den[trow] = den;
            }
        }
        __syncthreads();  // this segment's LDS reads are done before the next one is staged
    };
    // A loop around the body costs registers even when it runs once (lane
    // addresses get hoisted out of it), so the one-segment launch calls the
    // body straight; the looped one launders the thread index per pass.
    if constexpr (LOOP) {
        for (int seg = static_cast<int>(blockIdx.x); seg < a.segs; seg += static_cast<int>(gridDim.x)) seg_body(seg);
    } else {
        seg_body(static_cast<int>(blockIdx.x));
    }

    // ---- the last workgroup to finish resets the counter and advances the epoch
    if (tid == 0) {
        // kernel completion publishes these to the next launch on the stream
        const uint32_t done = __hip_atomic_fetch_add(&a.ctrl[kLine], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            __hip_atomic_store(&a.ctrl[kLine], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.ctrl[kLine + 1], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(&a.ctrl[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Layout {
    size_t flags, aggS, aggX, aggC, aggV, total;
};

Layout layout(int BH, int P) {
    Layout L{};
    const size_t slots = static_cast<size_t>(BH) * P;
    L.flags = 0;
    L.aggS = L.flags + align256(2 * slots * kFlagStride * sizeof(uint32_t));
    L.aggX = L.aggS + slots * 4096 * sizeof(float);
    L.aggC = L.aggX + slots * 4096 * sizeof(float);
    L.aggV = L.aggC + slots * 4096 * sizeof(float);
    L.total = L.aggV + slots * 128 * sizeof(float);
    return L;
}

template <bool D, bool R, bool Dn, bool N>
void launch(const FusedArgs &a, dim3 grid, hipStream_t st, bool loop) {
    if (loop)
        hipLaunchKernelGGL((k_fused64<D, R, Dn, N, true>), grid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((k_fused64<D, R, Dn, N, false>), grid, dim3(kThreads), 0, st, a);
}

template <bool D>
void launch_opts(const FusedArgs &a, dim3 grid, hipStream_t st, bool ridge, bool den, bool norm, bool loop) {
    if (ridge) {
        if (norm) launch<D, true, true, true>(a, grid, st, loop);
        else if (den) launch<D, true, true, false>(a, grid, st, loop);
        else launch<D, true, false, false>(a, grid, st, loop);
    } else {
        if (norm) launch<D, false, true, true>(a, grid, st, loop);
        else if (den) launch<D, false, true, false>(a, grid, st, loop);
        else launch<D, false, false, false>(a, grid, st, loop);
    }
}

}  // namespace

bool fused64_supported(const FwdProblem &p) {
    if (!(p.dtype == HLA_BF16 && p.d == 64 && p.dv == 64 && p.w == 64 && p.init.S == nullptr &&
          p.fin.S == nullptr && p.n > 0))
        return false;
    const int nh = p.gam.per_head ? p.H : 1;
    for (int h = 0; h < nh; ++h)
        if (p.gam.g[h] < kMinGamma) return false;
    return true;
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
    return layout(BH, P).total;
}

hipError_t fused64_forward(const FwdProblem &p, uint32_t *ctrl, void *data, hipStream_t st) {
    FusedArgs a{};
    a.H = p.H; a.n = p.n; a.nc = p.nc; a.BH = p.B * p.H;
    fused64_geometry(a.BH, a.nc, &a.P, &a.L);
    a.segs = a.BH * a.P;
    a.q = static_cast<const uint16_t *>(p.q);
    a.k = static_cast<const uint16_t *>(p.k);
    a.v = static_cast<const uint16_t *>(p.v);
    a.out = p.out;
    a.den = p.den;
    a.ridge = p.ridge;
    a.ctrl = ctrl;
    const Layout L = layout(a.BH, a.P);
    char *base = static_cast<char *>(data);
    a.flags = reinterpret_cast<uint32_t *>(base + L.flags);
    a.aggS = reinterpret_cast<float *>(base + L.aggS);
    a.aggX = reinterpret_cast<float *>(base + L.aggX);
    a.aggC = reinterpret_cast<float *>(base + L.aggC);
    a.aggV = reinterpret_cast<float *>(base + L.aggV);
    a.gam = p.gam;
    const int nh = p.gam.per_head ? p.H : 1;
    bool decay = false;
    for (int h = 0; h < nh; ++h) decay = decay || p.gam.g[h] != 1.0f;
    const bool ridge = p.ridge != 0.0f, norm = p.normalize != 0, den = norm || p.den != nullptr;
    // one workgroup per CU at most (its LDS fills the CU), so the whole grid is resident
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const bool loop = a.segs > cus;
    const dim3 grid(static_cast<unsigned>(loop ? cus : a.segs));
    if (decay)
        launch_opts<true>(a, grid, st, ridge, den, norm, loop);
    else
        launch_opts<false>(a, grid, st, ridge, den, norm, loop);
    return hipGetLastError();
}

}  // namespace hla
