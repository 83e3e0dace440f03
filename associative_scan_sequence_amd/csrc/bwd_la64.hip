// bwd_la64.hip -- the backward of the plain second-order numerator as
// masked first-order maps, on the one-launch kernel of fwd_la64.hip.
//
// With L = sum_t <out_t, dout_t> and out_t = q_t^T (S_t C_t - G_t), the
// gradients are (Higher-order Linear Attention, paperlayer.ai summary sec. 4:
// the reverse-mode scan; the identity below is pinned against the oracle's
// autograd gradients on the CPU, tests/test_backward_algebra.py):
//   u_j = S_j q_j                 = LA (Q, K, K; g)
//   w_j = sum_{t>=j} g^(2(t-j)) q_t (dout_t . v_j)
//                                 = LA^rev (V, dO, Q; g^2)
//   dq  = LA (dO, V, U; g^2) + LA (W, K, K; g)
//   dk  = LA^rev (K, Q, W; g) + LA^rev (K, W, Q; g)
//   dv  = LA^rev (U, Q, dO; g^2)
// where LA (A, B, C; r)_t = sum_{s<=t} r^(t-s) (a_t . b_s) c_s and LA^rev the
// same over s >= t with r^(s-t).  dO, U and W are fp32; they enter the maps
// as bf16 pairs (hi = bf16(x), lo = bf16(x - hi)): dO split as it is staged,
// U and W written as pairs by the maps that form them.  U and the second part
// of dq share their keys, values and decay, so they are one launch with two
// sets of queries, and the two maps of dk are one launch whose carry is
// symmetric.  After W, the maps fall into two pairs that do not depend on
// each other, each pair one grid: three launches in all.
//
// Workspace: the first kCtrlBytes are the one-launch kernels' control block,
// then the flags of two maps, their aggregates, and the pairs of U and W.  The call clears
// the control block and the flags itself (a fill kernel), so the backward
// workspace needs no initialisation, as for the chunked path.
#include "device_common.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kBw = 64;  // d = dv = chunk

__global__ __launch_bounds__(256) void k_zero_words(uint32_t *p, size_t n) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<size_t>(gridDim.x) * 256)
        p[i] = 0u;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct BwdLaLayout {
    size_t flags, agg, uh, ul, wh, wl, total;
};

BwdLaLayout bwd_la_layout(int BH, int n) {
    const size_t pair = static_cast<size_t>(BH) * n * kBw * sizeof(uint16_t);
    BwdLaLayout L{};
    L.flags = kCtrlBytes;  // two maps' flags, then their aggregates
    L.agg = L.flags + 2 * la64_flag_bytes(BH, n);
    L.uh = align256(L.agg + 2 * la64_agg_bytes(BH, n));
    L.ul = align256(L.uh + pair);
    L.wh = align256(L.ul + pair);
    L.wl = align256(L.wh + pair);
    L.total = L.wl + pair;
    return L;
}

}  // namespace

bool la_backward_eligible(const BwdProblem &p) {
    const FwdProblem &f = p.f;
    if (!(f.dtype == HLA_BF16 && f.d == kBw && f.dv == kBw && f.w == kBw && f.n > 0 && f.ridge == 0.0f &&
          !f.normalize && f.init.S == nullptr && p.dinit.S == nullptr && p.dfinal.S == nullptr))
        return false;
    const int nh = f.gam.per_head ? f.H : 1;
    for (int h = 0; h < nh; ++h)
        if (f.gam.g[h] < 0.75f) return false;
    return true;
}

size_t la_backward_workspace_bytes(int BH, int n) { return bwd_la_layout(BH, n).total; }

size_t backward_workspace_bytes(int BH, int n, int d, int dv, int w) {
    const size_t gen = generic_backward_workspace_bytes(BH, n, d, dv, w);
    if (!(d == kBw && dv == kBw && w == kBw && n > 0)) return gen;
    const size_t la = la_backward_workspace_bytes(BH, n);
    return gen > la ? gen : la;
}

hipError_t la_backward(const BwdProblem &p, hipStream_t st) {
    const FwdProblem &f = p.f;
    const int BH = f.B * f.H;
    const BwdLaLayout L = bwd_la_layout(BH, f.n);
    char *base = static_cast<char *>(f.ws);
    uint32_t *ctrl = reinterpret_cast<uint32_t *>(base);
    const size_t fb = la64_flag_bytes(BH, f.n), ab = la64_agg_bytes(BH, f.n);
    const LaSpace sa{reinterpret_cast<uint32_t *>(base + L.flags), reinterpret_cast<float *>(base + L.agg)};
    const LaSpace sb{reinterpret_cast<uint32_t *>(base + L.flags + fb), reinterpret_cast<float *>(base + L.agg + ab)};
    auto pair = [&](size_t off) { return reinterpret_cast<uint16_t *>(base + off); };
    uint16_t *uh = pair(L.uh), *ul = pair(L.ul), *wh = pair(L.wh), *wl = pair(L.wl);
    // the control block and both maps' flags start clear (every launch below
    // then leaves them valid for the next)
    const size_t words = (kCtrlBytes + 2 * fb) / sizeof(uint32_t);
    hipLaunchKernelGGL(k_zero_words, dim3(static_cast<unsigned>((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024)),
                       dim3(256), 0, st, ctrl, words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    auto map = [&](bool rev, bool gsq) {
        LaProblem m{};
        m.B = f.B; m.H = f.H; m.n = f.n; m.gam = f.gam;
        m.rev = rev; m.gsq = gsq;
        return m;
    };
    // W = LA^rev (V, dO, Q; g^2), as a pair
    LaProblem w = map(true, true);
    w.q = f.v; w.kf = p.dout; w.v = f.q; w.mode = 2; w.oh = wh; w.ol = wl;
    if ((e = la64_forward_in(w, ctrl, sa, st)) != hipSuccess) return e;
    // U = LA (Q, K, K; g), as a pair, and dq = LA (W, K, K; g): two sets of queries;
    // with dk = LA^rev (K, Q, W; g) + LA^rev (K, W, Q; g), the symmetric carry
    LaProblem u = map(false, false), dk = map(true, false);
    u.q = f.q; u.k = f.k; u.v = f.k; u.mode = 2; u.oh = uh; u.ol = ul;
    u.q2 = wh; u.q2l = wl; u.mode2 = 0; u.out2 = p.dq;
    dk.q = f.k; dk.k = f.q; dk.v = wh; dk.vl = wl; dk.mode = 0; dk.sym = true; dk.out = p.dk;
    if ((e = la64_forward_pair(u, sa, dk, sb, ctrl, st)) != hipSuccess) return e;
    // dq += LA (dO, V, U; g^2), with dv = LA^rev (U, Q, dO; g^2)
    LaProblem dq = map(false, true), dv = map(true, true);
    dq.qf = p.dout; dq.k = f.v; dq.v = uh; dq.vl = ul; dq.mode = 1; dq.out = p.dq;
    dv.q = uh; dv.ql = ul; dv.k = f.q; dv.vf = p.dout; dv.mode = 0; dv.out = p.dv;
    return la64_forward_pair(dq, sa, dv, sb, ctrl, st);
}

}  // namespace hla
