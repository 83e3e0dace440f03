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
// symmetric: five launches in all.
//
// Workspace: the first kCtrlBytes are the one-launch kernels' control block,
// then their flags and aggregates, then the pairs of U and W.  The call clears
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
    size_t data, uh, ul, wh, wl, total;
};

BwdLaLayout bwd_la_layout(int BH, int n) {
    const size_t pair = static_cast<size_t>(BH) * n * kBw * sizeof(uint16_t);
    BwdLaLayout L{};
    L.data = kCtrlBytes;
    L.uh = align256(L.data + la64_workspace_bytes(BH, n));
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
    void *data = base + L.data;
    auto pair = [&](size_t off) { return reinterpret_cast<uint16_t *>(base + off); };
    uint16_t *uh = pair(L.uh), *ul = pair(L.ul), *wh = pair(L.wh), *wl = pair(L.wl);
    // the control block and the flags start clear (every launch below then
    // leaves them valid for the next)
    const size_t words = (kCtrlBytes + la64_flag_bytes(BH, f.n)) / sizeof(uint32_t);
    hipLaunchKernelGGL(k_zero_words, dim3(static_cast<unsigned>((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024)),
                       dim3(256), 0, st, ctrl, words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    auto map = [&](LaProblem m, bool rev, bool gsq) {
        m.B = f.B; m.H = f.H; m.n = f.n; m.gam = f.gam;
        m.rev = rev; m.gsq = gsq;
        return la64_forward(m, ctrl, data, st);
    };
    LaProblem m{};
    // W = LA^rev (V, dO, Q; g^2), as a pair
    m = LaProblem{}; m.q = f.v; m.kf = p.dout; m.v = f.q; m.mode = 2; m.oh = wh; m.ol = wl;
    if ((e = map(m, true, true)) != hipSuccess) return e;
    // U = LA (Q, K, K; g), as a pair, and dq = LA (W, K, K; g): one launch, two sets of queries
    m = LaProblem{}; m.q = f.q; m.k = f.k; m.v = f.k; m.mode = 2; m.oh = uh; m.ol = ul;
    m.q2 = wh; m.q2l = wl; m.mode2 = 0; m.out2 = p.dq;
    if ((e = map(m, false, false)) != hipSuccess) return e;
    // dq += LA (dO, V, U; g^2)
    m = LaProblem{}; m.qf = p.dout; m.k = f.v; m.v = uh; m.vl = ul; m.mode = 1; m.out = p.dq;
    if ((e = map(m, false, true)) != hipSuccess) return e;
    // dk = LA^rev (K, Q, W; g) + LA^rev (K, W, Q; g): one launch, the symmetric carry
    m = LaProblem{}; m.q = f.k; m.k = f.q; m.v = wh; m.vl = wl; m.mode = 0; m.sym = true; m.out = p.dk;
    if ((e = map(m, true, false)) != hipSuccess) return e;
    // dv = LA^rev (U, Q, dO; g^2)
    m = LaProblem{}; m.q = uh; m.ql = ul; m.k = f.q; m.vf = p.dout; m.mode = 0; m.out = p.dv;
    return map(m, true, true);
}

}  // namespace hla
