// hla_internal.h -- declarations shared by the host dispatch (hla_api.cpp)
// and the HIP kernel files of the library.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hla.h"

namespace hla {

// Per-head decays travel by value in kernel arguments.
constexpr int kMaxGammaHeads = 256;

struct GammaTab {
    float g[kMaxGammaHeads];
    int per_head;  // 0: g[0] applies to every head
};

__host__ __device__ inline float head_gamma(const GammaTab &t, int h) {
    return t.g[t.per_head ? h : 0];
}

// Everything a forward launch needs, validated by the host.
struct FwdProblem {
    int B, H, n, d, dv, w, nc;
    hla_dtype dtype;
    float ridge;
    int normalize;
    const void *q, *k, *v;
    const void *vl;    // one-launch d = 64 kernel, plain numerator only: the values are v + vl (a bf16 pair)
    float *out, *den;  // den may be null
    hla_state init;    // init.S == nullptr: zero state
    hla_state fin;     // fin.S == nullptr: not requested
    GammaTab gam;
    void *ws;
    size_t ws_bytes;
    int carries_only;  // generic path: stop after the carries and U (no out, den or final state)
    int own_prefix;    // generic path: the slots need not hold prefixes afterwards (a forward call)
};

// Every forward workspace starts with a control block of kCtrlBytes: words
// that the one-launch kernels keep valid across calls (a finished-workgroup
// counter and the launch epoch, a launch count, a wait give-up count and the
// spin limit, and the segment tickets: one over all segments, one per head).
// It must be zero before the first call; no kernel writes it except through
// those words.  Path data follows it.
constexpr size_t kCtrlBytes = 8192;

// Generic chunked forward: any d, dv, w in {16,32,64,128}, fp32 or bf16,
// several kernels over a per-chunk workspace.
size_t generic_workspace_bytes(int BH, int n, int d, int dv, int w);
hipError_t generic_forward(const FwdProblem &p, hipStream_t s);

// Where the generic forward keeps its per-chunk products inside p.ws: slots
// [BH][nc+1] of S, C, m, X = S C - G, y = S m - h (slot c = the state before
// chunk c) and U [BH][nc][w][d] (row s = S_s q_s).  The backward reads them.
struct GenericSlots {
    float *S, *C, *m, *X, *y, *U;
};
GenericSlots generic_slots(const FwdProblem &p);

// Chunked backward: gradients of sum(out * dout) with respect to q, k, v, from
// the zero state or a given initial state held constant; any d, dv, w in
// {16,32,64,128}, fp32 or bf16.
struct BwdProblem {
    FwdProblem f;        // the forward call (fin and den unused); f.ws = backward data area
    const float *dout;   // [B,H,n,dv]
    float *dq, *dk, *dv; // [B,H,n,d], [B,H,n,d], [B,H,n,dv]
    hla_state dinit;     // gradient with respect to the initial state; dinit.S null: not formed
    hla_state dfinal;    // gradient flowing into the final state; dfinal.S null: none
};
size_t generic_backward_workspace_bytes(int BH, int n, int d, int dv, int w);
hipError_t generic_backward(const BwdProblem &p, hipStream_t s);
// The plain-numerator backward as first-order maps (bwd_la64.hip): bf16,
// d = dv = w = 64, no ridge, ratio or states, every decay >= 0.75.
bool la_backward_eligible(const BwdProblem &p);
size_t la_backward_workspace_bytes(int BH, int n);
hipError_t la_backward(const BwdProblem &p, hipStream_t s);
// Workspace bytes of hla_backward_chunked: the larger of the two paths' needs
// when both can serve these widths.
size_t backward_workspace_bytes(int BH, int n, int d, int dv, int w);
// Writes zeros into every part of s that is set (the initial-state gradient
// of an empty sequence).
hipError_t zero_state_grad(const hla_state &s, int BH, int d, int dv, hipStream_t st);

// The body of the forward entry points (hla_api.cpp): validation, then the
// kernels.  scratch_name == nullptr: `workspace` is the caller's and must
// hold hla_forward_workspace_size(p) bytes.  Otherwise `workspace` is
// ignored: the static scratch (workspace_bytes of it, named scratch_name in
// errors) must hold what the path of this call needs, and its address is
// looked up only once every argument has passed validation.
hla_status forward_impl(const hla_params *p, const void *q, const void *k, const void *v, float *out,
                        float *den, const hla_state *init, hla_state *final_state, void *workspace,
                        size_t workspace_bytes, hipStream_t stream, const char *scratch_name);

// The current device's address of the static scratch behind
// hla_forward_chunked_noalloc (noalloc.hip; looked up once per device).
hla_status noalloc_scratch(void **ptr);
constexpr size_t kNoallocBytes = HLA_NOALLOC_SCRATCH_BYTES;
// The scratch's flag region, fixed so that calls with any params find every
// flag outside every other call's data: the largest one-launch call whose data
// fits the rest of the scratch needs about 2.6 MB of flags.
constexpr size_t kNoallocFlagBytes = static_cast<size_t>(4) << 20;

// Records msg as this thread's last error (hla_last_error) and returns s.
hla_status set_error(hla_status s, const char *msg);

// The one-launch forwards take three regions: the control block, their
// flags and their data.  A flag holds the epoch of the launch that last set
// it, and a wait compares it with the running launch's epoch; so a flag
// region must hold nothing but epochs (or the zeros it started as): every
// workspace keeps the flags in a region of their own, after the control
// block, that no path's data overlaps.  Flags of different one-launch kernels
// may share that region, as every epoch comes from the one sequence in the
// control block.

// One-launch MFMA forward for bf16, d = dv = w = 64, decays >= 0.75, any
// ridge, denominator, normalisation, initial and final state.
bool fast64_supported(const FwdProblem &p);
size_t fast64_flag_bytes(int BH, int n);
size_t fast64_data_bytes(int BH, int n);
hipError_t fast64_forward(const FwdProblem &p, uint32_t *ctrl, uint32_t *flags, void *data, hipStream_t s);

// One-launch MFMA forward for bf16, d = dv = 128 (any chunk setting; the
// kernel works in 64-token chunks), decays >= 0.75, no ridge, denominator or
// normalisation; an initial or final state while the segments fit one pass.
bool fused128_supported(const FwdProblem &p);
size_t fused128_flag_bytes(int BH, int n);
size_t fused128_data_bytes(int BH, int n);
hipError_t fused128_forward(const FwdProblem &p, uint32_t *ctrl, uint32_t *flags, void *data, hipStream_t s);

// Two-launch forward for short sequences (fwd_small.hip): n <= 256, d and dv
// in {16, 32}, fp32 or bf16, any decays, no ridge, denominator,
// normalisation or states (any chunk setting: the result does not depend on
// it).  Its data is the fp32 map U, [BH][n][d].
bool small_supported(const FwdProblem &p);
size_t small_data_bytes(int BH, int n, int d);
hipError_t small_forward(const FwdProblem &p, void *data, hipStream_t s);

struct DecodeProblem {
    int B, H, d, dv;
    hla_dtype dtype;
    float ridge;
    int normalize;
    const void *q, *k, *v;
    hla_state st;
    float *out, *den;
    GammaTab gam;
};
hipError_t decode_step(const DecodeProblem &p, hipStream_t s);

// Decode with the key moment packed and shared by the query heads of a group
// (decode_mq.hip); H query heads, kv_heads groups, H % kv_heads == 0.
struct DecodeMqProblem {
    int B, H, kv_heads, d, dv;
    hla_dtype dtype;
    float ridge;
    int normalize;
    const void *q, *k, *v;
    hla_mq_state st;
    float *out, *den;
    GammaTab gam;
};
hipError_t decode_step_mq(const DecodeMqProblem &p, hipStream_t s);
// count symmetric d x d matrices: full -> packed (pack) or packed -> full
hipError_t key_moment_pack(int count, int d, const float *src, float *dst, bool pack, hipStream_t s);

// The asymmetric variant (AHLA) and third order (fwd_higher.hip,
// decode_higher.hip).  A state: AHLA (X1, v1, X2, v2) = (P, m, E, n) and rho;
// third order S and (X1, v1, X2, v2) = (P, m, F, Fd).
struct HiState {
    float *S, *X1, *v1, *X2, *v2, *rho;
};
struct HiProblem {
    int B, H, n, d, dv, w;
    hla_dtype dtype;
    int normalize;
    bool third;
    const void *q, *k, *v;
    float *out, *den;
    HiState init, fin;  // init.X1 == nullptr: zero state; fin.X1 == nullptr: not returned
    GammaTab gam;
    void *ws;
};
size_t higher_workspace_bytes(int BH, int n, int d, int dv, int w, bool third);
hipError_t higher_forward(const HiProblem &p, hipStream_t s);
struct HiDecodeProblem {
    int B, H, d, dv;
    hla_dtype dtype;
    int normalize;
    bool third;
    const void *q, *k, *v;
    HiState st;
    float *out, *den;
    GammaTab gam;
};
hipError_t higher_decode(const HiDecodeProblem &p, hipStream_t s);

// One-launch masked first-order linear attention, bf16 q, k, v with d = dv =
// 64 (chunk 64, every decay >= 0.75): y_t = sum_{s<=t} g^(t-s) (q_t.k_s) v_s,
// or with rev the reverse-time map (s >= t, g^(s-t)).  mode 0: out = y; 1:
// out += y; 2: oh, ol = bf16 hi and lo of y.  ql, kl, vl set: that operand is
// the bf16 pair (x, xl); qf, kf, vf set: it is fp32 (and q, k, v unused).
// q2 (or q2 + q2l, or q2f) set: a second set of queries against the same
// keys and values, written to out2 (or oh2, ol2) with mode2.  sym: plus the
// map with keys and values exchanged.  mode 3: no output (only fin).  r is
// the decay per token (g, or g^2 with gsq); p the position in the direction
// of the map.  Only the combinations listed in
// fwd_la64.hip are built (hipErrorInvalidValue otherwise).  ctrl is the
// one-launch kernels' control block (zero before first use).
struct LaProblem {
    int B, H, n;
    const void *q, *k, *v;
    const void *ql, *kl, *vl;
    const float *qf, *kf, *vf;
    const void *q2, *q2l;
    const float *q2f;
    float *out;
    uint16_t *oh, *ol;
    float *out2;
    uint16_t *oh2, *ol2;
    int mode, mode2;
    bool rev;
    bool gsq;      // the decay per token is g^2 (g from gam)
    bool sym;      // plus the map with keys and values exchanged (d = dv; values bf16 or a pair, keys bf16)
    const float *init;  // [BH][64 keys][64 values] fp32: the carry at position -1 (null: zero)
    float *fin;         // [BH][64][64]: receives the carry after the last token (null: not formed)
    const float *bias;  // [BH][64]: out_p += r^(p+1) bias (null: none; first output only)
    bool chain;         // set by la64_chain
    GammaTab gam;
};
// A map's flags (zero before their first use) and its segment aggregates.
struct LaSpace {
    uint32_t *flags;
    float *aggC;
};
size_t la64_flag_bytes(int BH, int n);
size_t la64_agg_bytes(int BH, int n);
hipError_t la64_forward_in(const LaProblem &p, uint32_t *ctrl, LaSpace sp, hipStream_t s);
// The map applied twice in one launch, out = LA (Q, K, LA (Q, K, V)): the
// first map's output stays in LDS as the second's values (a bf16 pair); each
// map hands its segment sums over through its own space.  q, k, v bf16;
// mode store.
hipError_t la64_chain(const LaProblem &p, uint32_t *ctrl, LaSpace s1, LaSpace s2, hipStream_t s);
// Two maps that do not depend on each other, in one grid where the
// combination is built and both fit a one-pass grid, else one after the other.
hipError_t la64_forward_pair(const LaProblem &a, LaSpace sa, const LaProblem &b, LaSpace sb, uint32_t *ctrl,
                             hipStream_t s);

hipError_t state_compose(int count, int d, int dv, const hla_state &a, const hla_state &b,
                         const hla_state &r, hipStream_t s);

}  // namespace hla
