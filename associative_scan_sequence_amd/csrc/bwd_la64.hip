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
// as bf16 pairs (hi = bf16(x), lo = bf16(x - hi)).
//
// Workspace: the first kCtrlBytes are the one-launch kernels' control block,
// then their flags and aggregates, then the pairs of dO, U and W.  The call
// clears the control block and the flags itself (a fill kernel), so the
// backward workspace needs no initialisation, as for the chunked path.
#include "bf16_split.h"
#include "device_common.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kBw = 64;  // d = dv = chunk

__global__ __launch_bounds__(256) void k_zero_words(uint32_t *p, size_t n) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<size_t>(gridDim.x) * 256)
        p[i] = 0u;
}

// x (fp32) -> the bf16 pair (hi, lo), four values per thread
__global__ __launch_bounds__(256) void k_split_pair(const float *x, uint16_t *hi, uint16_t *lo, size_t n4) {
    const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n4) return;
    const float4 v = reinterpret_cast<const float4 *>(x)[i];
    bf16x4 h, l;
    split4(f32x4{v.x, v.y, v.z, v.w}, h, l);
    reinterpret_cast<bf16x4 *>(hi)[i] = h;
    reinterpret_cast<bf16x4 *>(lo)[i] = l;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct BwdLaLayout {
    size_t data, doh, dol, uh, ul, wh, wl, total;
};

BwdLaLayout bwd_la_layout(int BH, int n) {
    const size_t pair = static_cast<size_t>(BH) * n * kBw * sizeof(uint16_t);
    BwdLaLayout L{};
    L.data = kCtrlBytes;
    L.doh = align256(L.data + la64_workspace_bytes(BH, n));
    L.dol = align256(L.doh + pair);
    L.uh = align256(L.dol + pair);
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
    uint16_t *doh = pair(L.doh), *dol = pair(L.dol), *uh = pair(L.uh), *ul = pair(L.ul), *wh = pair(L.wh),
             *wl = pair(L.wl);
    // the control block and the flags start clear (every launch below then
    // leaves them valid for the next)
    const size_t words = (kCtrlBytes + la64_flag_bytes(BH, f.n)) / sizeof(uint32_t);
    hipLaunchKernelGGL(k_zero_words, dim3(static_cast<unsigned>((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024)),
                       dim3(256), 0, st, ctrl, words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t n4 = static_cast<size_t>(BH) * f.n * kBw / 4;
    hipLaunchKernelGGL(k_split_pair, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, st, p.dout, doh, dol,
                       n4);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    auto la = [&](const void *q, const void *ql, const void *k, const void *kl, const void *v, const void *vl,
                  bool rev, bool gsq, int mode, float *out, uint16_t *oh, uint16_t *ol) {
        LaProblem m{};
        m.B = f.B; m.H = f.H; m.n = f.n; m.gam = f.gam;
        m.q = q; m.ql = ql; m.k = k; m.kl = kl; m.v = v; m.vl = vl;
        m.rev = rev; m.gsq = gsq; m.mode = mode; m.out = out; m.oh = oh; m.ol = ol;
        return la64_forward(m, ctrl, data, st);
    };
    // U = LA (Q, K, K; g), W = LA^rev (V, dO, Q; g^2), both as pairs
    if ((e = la(f.q, nullptr, f.k, nullptr, f.k, nullptr, false, false, 2, nullptr, uh, ul)) != hipSuccess) return e;
    if ((e = la(f.v, nullptr, doh, dol, f.q, nullptr, true, true, 2, nullptr, wh, wl)) != hipSuccess) return e;
    // dq = LA (dO, V, U; g^2) + LA (W, K, K; g)
    if ((e = la(doh, dol, f.v, nullptr, uh, ul, false, true, 0, p.dq, nullptr, nullptr)) != hipSuccess) return e;
    if ((e = la(wh, wl, f.k, nullptr, f.k, nullptr, false, false, 1, p.dq, nullptr, nullptr)) != hipSuccess) return e;
    // dk = LA^rev (K, Q, W; g) + LA^rev (K, W, Q; g)
    if ((e = la(f.k, nullptr, f.q, nullptr, wh, wl, true, false, 0, p.dk, nullptr, nullptr)) != hipSuccess) return e;
    if ((e = la(f.k, nullptr, wh, wl, f.q, nullptr, true, false, 1, p.dk, nullptr, nullptr)) != hipSuccess) return e;
    // dv = LA^rev (U, Q, dO; g^2)
    return la(uh, ul, f.q, nullptr, doh, dol, true, true, 0, p.dv, nullptr, nullptr);
}

}  // namespace hla
