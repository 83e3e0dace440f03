// hla_api.cpp -- the extern "C" entry points declared in include/hla.h:
// host-only validation (nothing is enqueued on a bad argument), then dispatch
// to the HIP kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "hla_internal.h"

namespace {

thread_local std::string g_last_error;

hla_status fail(hla_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

hla_status ok() {
    g_last_error.clear();
    return HLA_OK;
}

bool width_ok(int x) { return x == 16 || x == 32 || x == 64 || x == 128; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    std::string name;
    uintptr_t lo, hi;  // [lo, hi)
};

Span span(const std::string &name, const void *p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{name, lo, lo + bytes};
}

bool overlaps(const Span &a, const Span &b) {
    if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// Every span in `outs` must be disjoint from every other span in `outs` and
// from every span in `ins`.
bool first_overlap(const std::vector<Span> &outs, const std::vector<Span> &ins,
                   std::string *detail) {
    for (size_t i = 0; i < outs.size(); ++i) {
        for (size_t j = i + 1; j < outs.size(); ++j)
            if (overlaps(outs[i], outs[j])) {
                *detail = outs[i].name + " overlaps " + outs[j].name;
                return true;
            }
        for (const Span &in : ins)
            if (overlaps(outs[i], in)) {
                *detail = outs[i].name + " overlaps " + in.name;
                return true;
            }
    }
    return false;
}

hla_status check_state(const hla_state *s, const char *what) {
    const float *ptrs[5] = {s->S, s->C, s->m, s->G, s->h};
    const char *names[5] = {"S", "C", "m", "G", "h"};
    for (int i = 0; i < 5; ++i) {
        if (!ptrs[i]) return fail(HLA_ERR_INVALID_ARGUMENT, "%s->%s is NULL", what, names[i]);
        if (!aligned16(ptrs[i]))
            return fail(HLA_ERR_ALIGNMENT, "%s->%s is not 16-byte aligned", what, names[i]);
    }
    if (s->rho && (reinterpret_cast<uintptr_t>(s->rho) & 3u))
        return fail(HLA_ERR_ALIGNMENT, "%s->rho is not 4-byte aligned", what);
    return HLA_OK;
}

void state_spans(const hla_state *s, const char *prefix, size_t N, int d, int dv,
                 std::vector<Span> *out) {
    const char *tags[6] = {"S", "C", "m", "G", "h", "rho"};
    const float *ptrs[6] = {s->S, s->C, s->m, s->G, s->h, s->rho};
    const size_t sizes[6] = {N * d * d, N * d * dv, N * d, N * d * dv, N * d, N};
    for (int i = 0; i < 6; ++i)
        if (ptrs[i]) out->push_back(span(std::string(prefix) + "." + tags[i], ptrs[i], sizes[i] * sizeof(float)));
}

// The dtype field as the integer the caller stored: an out-of-range value is
// read without ever holding it in the enum type.
static_assert(sizeof(hla_dtype) == sizeof(int32_t), "hla_dtype is a 32-bit int in the C ABI");
int dtype_code(const hla_params *p) {
    int32_t x;
    std::memcpy(&x, &p->dtype, sizeof(x));
    return x;
}

bool dtype_ok(const hla_params *p) { return dtype_code(p) == HLA_F32 || dtype_code(p) == HLA_BF16; }

hla_status check_common(int H, int d, int dv, int dtype, const float *gamma, float ridge,
                        int normalize, hla::GammaTab *tab) {
    if (!width_ok(d) || !width_ok(dv))
        return fail(HLA_ERR_UNSUPPORTED, "d=%d, dv=%d: each must be 16, 32, 64 or 128", d, dv);
    if (dtype != HLA_F32 && dtype != HLA_BF16) return fail(HLA_ERR_INVALID_ARGUMENT, "bad dtype %d", dtype);
    if (!std::isfinite(ridge) || ridge < 0.0f)
        return fail(HLA_ERR_INVALID_ARGUMENT, "ridge must be finite and >= 0");
    if (normalize != 0 && normalize != 1) return fail(HLA_ERR_INVALID_ARGUMENT, "normalize must be 0 or 1");
    tab->per_head = 0;
    tab->g[0] = 1.0f;
    if (gamma) {
        if (H > hla::kMaxGammaHeads)
            return fail(HLA_ERR_UNSUPPORTED, "per-head gamma supports at most %d heads (H=%d)",
                        hla::kMaxGammaHeads, H);
        for (int h = 0; h < H; ++h) {
            const float g = gamma[h];
            if (!std::isfinite(g) || !(g > 0.0f) || g > 1.0f)
                return fail(HLA_ERR_INVALID_ARGUMENT, "gamma[%d] = %g is not in (0, 1]", h, double(g));
            tab->g[h] = g;
        }
        tab->per_head = 1;
    }
    return HLA_OK;
}

// the chunk algebra costs O(w^2 d + w d^2) per chunk of w tokens, O(w d + d^2) per token: w = d
int default_chunk(int d) { return d <= 16 ? 16 : (d <= 32 ? 32 : (d <= 64 ? 64 : 128)); }

// Kernel path for a forward call.  init/fin/den only matter for the choice.
enum class FwdPath { Generic, Fast64, Fused128, Small };


struct Geometry {
    int w, nc;
};

hla_status forward_geometry(const hla_params *p, Geometry *geo) {
    if (!p) return fail(HLA_ERR_INVALID_ARGUMENT, "params is NULL");
    if (p->B < 1 || p->H < 1) return fail(HLA_ERR_INVALID_ARGUMENT, "B=%d, H=%d must be >= 1", p->B, p->H);
    if (p->n < 0) return fail(HLA_ERR_INVALID_ARGUMENT, "n=%d must be >= 0", p->n);
    const int w = p->chunk == 0 ? default_chunk(p->d) : p->chunk;
    if (!width_ok(w)) return fail(HLA_ERR_UNSUPPORTED, "chunk=%d must be 0, 16, 32, 64 or 128", p->chunk);
    const uint64_t BH = static_cast<uint64_t>(p->B) * p->H;
    if (BH > 65535) return fail(HLA_ERR_UNSUPPORTED, "B*H=%llu exceeds 65535", (unsigned long long)BH);
    const uint64_t wide = p->d > p->dv ? p->d : p->dv;
    if (BH * static_cast<uint64_t>(p->n) * wide > 0x7fffffffull)
        return fail(HLA_ERR_UNSUPPORTED, "B*H*n*max(d,dv) exceeds 2^31-1 elements");
    geo->w = w;
    geo->nc = (p->n + w - 1) / w;
    return HLA_OK;
}

FwdPath choose_path(const hla_params *p, const Geometry &geo, const hla_state *init,
                    const hla_state *fin, const float *den, const hla::GammaTab &gam) {
    hla::FwdProblem fp{};
    fp.dtype = p->dtype; fp.d = p->d; fp.dv = p->dv; fp.w = geo.w; fp.n = p->n; fp.B = p->B; fp.H = p->H;
    fp.gam = gam;
    fp.ridge = p->ridge; fp.normalize = p->normalize; fp.den = const_cast<float *>(den);
    if (init) fp.init = *init;
    if (fin) fp.fin = *fin;
    if (hla::fast64_supported(fp)) return FwdPath::Fast64;
    if (hla::fused128_supported(fp)) return FwdPath::Fused128;
    if (hla::small_supported(fp)) return FwdPath::Small;
    return FwdPath::Generic;
}

// A caller's workspace is the control block, a flag region, then the data
// of whichever path a call takes.  The flag region holds the flags of the
// one-launch kernel that calls with these params may take (none where no such
// kernel applies) and nothing else; its size depends on the params alone, so
// calls with the same params, whatever their states and den, find every flag
// outside every path's data.
size_t flag_area(const hla_params *p, const Geometry &geo) {
    const int BH = p->B * p->H;
    if (p->dtype == HLA_BF16 && p->d == 64 && p->dv == 64 && geo.w == 64 && p->n > 0)
        return hla::fast64_flag_bytes(BH, p->n);
    if (p->dtype == HLA_BF16 && p->d == 128 && p->dv == 128 && p->n > 0) return hla::fused128_flag_bytes(BH, p->n);
    return 0;
}

// Workspace bytes for any call with these params: the largest of the
// candidate paths' data (states and den are not known to the size query).
size_t workspace_need(const hla_params *p, const Geometry &geo) {
    const int BH = p->B * p->H;
    const size_t gen = hla::generic_workspace_bytes(BH, p->n, p->d, p->dv, geo.w);
    size_t fused = 0;
    if (p->dtype == HLA_BF16 && p->d == 64 && p->dv == 64 && geo.w == 64 && p->n > 0)
        fused = hla::fast64_data_bytes(BH, p->n);
    if (p->dtype == HLA_BF16 && p->d == 128 && p->dv == 128 && p->n > 0) fused = hla::fused128_data_bytes(BH, p->n);
    const size_t small = hla::small_data_bytes(BH, p->n, p->d);  // never above gen; kept for clarity
    if (small > fused) fused = small;
    return hla::kCtrlBytes + flag_area(p, geo) + (gen > fused ? gen : fused);
}

// Flag and data bytes of the one path a call takes.
struct PathNeed {
    size_t flags, data;
};

PathNeed path_need(const hla_params *p, const Geometry &geo, FwdPath path) {
    const int BH = p->B * p->H;
    if (path == FwdPath::Fast64) return PathNeed{hla::fast64_flag_bytes(BH, p->n), hla::fast64_data_bytes(BH, p->n)};
    if (path == FwdPath::Fused128)
        return PathNeed{hla::fused128_flag_bytes(BH, p->n), hla::fused128_data_bytes(BH, p->n)};
    if (path == FwdPath::Small) return PathNeed{0, hla::small_data_bytes(BH, p->n, p->d)};
    return PathNeed{0, hla::generic_workspace_bytes(BH, p->n, p->d, p->dv, geo.w)};
}

}  // namespace

extern "C" {

const char *hla_status_string(hla_status s) {
    switch (s) {
        case HLA_OK: return "HLA_OK";
        case HLA_ERR_INVALID_ARGUMENT: return "HLA_ERR_INVALID_ARGUMENT";
        case HLA_ERR_UNSUPPORTED: return "HLA_ERR_UNSUPPORTED";
        case HLA_ERR_ALIGNMENT: return "HLA_ERR_ALIGNMENT";
        case HLA_ERR_WORKSPACE: return "HLA_ERR_WORKSPACE";
        case HLA_ERR_DEVICE: return "HLA_ERR_DEVICE";
    }
    return "HLA_UNKNOWN_STATUS";
}

const char *hla_last_error(void) { return g_last_error.c_str(); }

size_t hla_forward_workspace_size(const hla_params *p) {
    Geometry geo{};
    if (forward_geometry(p, &geo) != HLA_OK) return 0;
    if (!width_ok(p->d) || !width_ok(p->dv) || !dtype_ok(p)) return 0;
    return workspace_need(p, geo);
}

hla_status hla_forward_chunked(const hla_params *p, const void *q, const void *k, const void *v,
                               float *out, float *den, const hla_state *init,
                               hla_state *final_state, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    return hla::forward_impl(p, q, k, v, out, den, init, final_state, workspace, workspace_bytes, stream,
                             nullptr);
}

hla_status hla_forward_chunked_noalloc(const hla_params *p, const void *q, const void *k, const void *v,
                                       float *out, float *den, const hla_state *init, hla_state *final_state,
                                       hipStream_t stream) {
    // validation first (host only); the static scratch (noalloc.hip) is looked up after it
    return hla::forward_impl(p, q, k, v, out, den, init, final_state, nullptr, hla::kNoallocBytes, stream,
                             "the library's static scratch");
}

}  // extern "C"

namespace hla {

hla_status set_error(hla_status s, const char *msg) { return fail(s, "%s", msg); }

// The forward entry points' common body.  scratch_name == nullptr: the
// caller's workspace, which must hold hla_forward_workspace_size(p) bytes
// (the largest path's need).  Otherwise a fixed buffer of workspace_bytes
// (so named in errors) that must hold only what the path this call takes
// needs.
hla_status forward_impl(const hla_params *p, const void *q, const void *k, const void *v, float *out,
                        float *den, const hla_state *init, hla_state *final_state, void *workspace,
                        size_t workspace_bytes, hipStream_t stream, const char *scratch_name) {
    Geometry geo{};
    hla_status s = forward_geometry(p, &geo);
    if (s != HLA_OK) return s;
    hla::FwdProblem fp{};
    s = check_common(p->H, p->d, p->dv, dtype_code(p), p->gamma, p->ridge, p->normalize, &fp.gam);
    if (s != HLA_OK) return s;
    const size_t BH = static_cast<size_t>(p->B) * p->H, n = static_cast<size_t>(p->n);
    const size_t esz = p->dtype == HLA_BF16 ? 2 : 4;
    if (n > 0) {
        const void *req[4] = {q, k, v, out};
        const char *nm[4] = {"q", "k", "v", "out"};
        for (int i = 0; i < 4; ++i) {
            if (!req[i]) return fail(HLA_ERR_INVALID_ARGUMENT, "%s is NULL", nm[i]);
            if (!aligned16(req[i])) return fail(HLA_ERR_ALIGNMENT, "%s is not 16-byte aligned", nm[i]);
        }
        if (den && !aligned16(den)) return fail(HLA_ERR_ALIGNMENT, "den is not 16-byte aligned");
    }
    if (init && (s = check_state(init, "init")) != HLA_OK) return s;
    if (final_state && (s = check_state(final_state, "final_state")) != HLA_OK) return s;
    // the static scratch keeps a flag region of fixed size, so that calls with
    // any params find every flag outside every other call's data
    const PathNeed pn = path_need(p, geo, choose_path(p, geo, init, final_state, den, fp.gam));
    const size_t area = scratch_name ? hla::kNoallocFlagBytes : flag_area(p, geo);
    const size_t need = scratch_name ? hla::kCtrlBytes + area + pn.data : workspace_need(p, geo);
    if (scratch_name && (pn.flags > area || need > workspace_bytes))
        return fail(HLA_ERR_WORKSPACE,
                    "this call needs %zu bytes of flags and %zu of data; %s holds %zu bytes: %zu for flags, %zu for data",
                    pn.flags, pn.data, scratch_name, workspace_bytes, area, workspace_bytes - hla::kCtrlBytes - area);
    if (!scratch_name && need > 0) {
        if (!workspace) return fail(HLA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
        if (workspace_bytes < need)
            return fail(HLA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(HLA_ERR_ALIGNMENT, "workspace is not 256-byte aligned");
    }
    // aliasing: outputs must be disjoint from each other and from the inputs
    std::vector<Span> outs, ins;
    if (n > 0) {
        outs.push_back(span("out", out, BH * n * p->dv * 4));
        if (den) outs.push_back(span("den", den, BH * n * 4));
        ins.push_back(span("q", q, BH * n * p->d * esz));
        ins.push_back(span("k", k, BH * n * p->d * esz));
        ins.push_back(span("v", v, BH * n * p->dv * esz));
    }
    if (need > 0) outs.push_back(span("workspace", workspace, need));
    if (final_state) state_spans(final_state, "final_state", BH, p->d, p->dv, &outs);
    if (init) state_spans(init, "init", BH, p->d, p->dv, &ins);
    std::string detail;
    if (first_overlap(outs, ins, &detail))
        return fail(HLA_ERR_INVALID_ARGUMENT, "aliasing: %s", detail.c_str());

    fp.B = p->B; fp.H = p->H; fp.n = p->n; fp.d = p->d; fp.dv = p->dv;
    fp.w = geo.w; fp.nc = geo.nc;
    fp.dtype = p->dtype; fp.ridge = p->ridge; fp.normalize = p->normalize;
    fp.q = q; fp.k = k; fp.v = v; fp.out = out; fp.den = den;
    if (init) fp.init = *init;
    if (final_state) fp.fin = *final_state;
    fp.ws = workspace; fp.ws_bytes = workspace_bytes;
    if (n == 0 && !final_state) return ok();
    if (scratch_name) {  // the static scratch: its address, once every argument has passed
        const hla_status ss = noalloc_scratch(&workspace);
        if (ss != HLA_OK) return ss;
        fp.ws = workspace;
    }
    char *ws = static_cast<char *>(workspace);
    uint32_t *ctrl = reinterpret_cast<uint32_t *>(ws), *flags = reinterpret_cast<uint32_t *>(ws + hla::kCtrlBytes);
    char *data = ws + hla::kCtrlBytes + area;
    hipError_t e;
    const FwdPath path = choose_path(p, geo, init, final_state, den, fp.gam);
    if (path == FwdPath::Fast64) {
        e = hla::fast64_forward(fp, ctrl, flags, data, stream);
    } else if (path == FwdPath::Fused128) {
        e = hla::fused128_forward(fp, ctrl, flags, data, stream);
    } else if (path == FwdPath::Small) {
        e = hla::small_forward(fp, data, stream);
    } else {
        fp.ws = data;
        fp.ws_bytes = workspace_bytes - hla::kCtrlBytes - area;
        fp.own_prefix = 1;  // nothing reads the slots after this call
        e = hla::generic_forward(fp, stream);
    }
    if (e != hipSuccess) return fail(HLA_ERR_DEVICE, "forward launch: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace hla

extern "C" {

size_t hla_backward_workspace_size(const hla_params *p) {
    Geometry geo{};
    if (forward_geometry(p, &geo) != HLA_OK) return 0;
    if (!width_ok(p->d) || !width_ok(p->dv) || !dtype_ok(p)) return 0;
    if (p->n == 0) return 0;
    return hla::backward_workspace_bytes(p->B * p->H, p->n, p->d, p->dv, geo.w);
}

hla_status hla_backward_chunked(const hla_params *p, const void *q, const void *k, const void *v,
                                const hla_state *init, const float *dout, float *dq, float *dk, float *dv,
                                const hla_state *dfinal, hla_state *dinit, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    Geometry geo{};
    hla_status s = forward_geometry(p, &geo);
    if (s != HLA_OK) return s;
    hla::BwdProblem bp{};
    hla::FwdProblem &fp = bp.f;
    s = check_common(p->H, p->d, p->dv, dtype_code(p), p->gamma, p->ridge, p->normalize, &fp.gam);
    if (s != HLA_OK) return s;
    const size_t BH = static_cast<size_t>(p->B) * p->H, n = static_cast<size_t>(p->n);
    if (init && (s = check_state(init, "init")) != HLA_OK) return s;
    if (dinit && (s = check_state(dinit, "dinit")) != HLA_OK) return s;
    if (dfinal && (s = check_state(dfinal, "dfinal")) != HLA_OK) return s;
    if (dfinal && p->gamma) {  // the seeds at position n divide by g^2
        for (int h = 0; h < p->H; ++h)
            if (!(p->gamma[h] >= 1e-6f))
                return fail(HLA_ERR_UNSUPPORTED, "gamma[%d]=%g: a final-state gradient needs gamma >= 1e-6", h,
                            double(p->gamma[h]));
    }
    if (dinit) {  // disjoint from each other and from the initial state and dfinal
        std::vector<Span> douts, dins;
        state_spans(dinit, "dinit", BH, p->d, p->dv, &douts);
        if (init) state_spans(init, "init", BH, p->d, p->dv, &dins);
        if (dfinal) state_spans(dfinal, "dfinal", BH, p->d, p->dv, &dins);
        std::string detail;
        if (first_overlap(douts, dins, &detail))
            return fail(HLA_ERR_INVALID_ARGUMENT, "aliasing: %s", detail.c_str());
    }
    if (n == 0) {  // the final state is the initial one: dinit = dfinal (zero without it)
        if (!dinit) return ok();
        hipError_t e = hla::zero_state_grad(*dinit, int(BH), p->d, p->dv, stream);
        if (e == hipSuccess && dfinal) {
            const float *src[5] = {dfinal->S, dfinal->C, dfinal->m, dfinal->G, dfinal->h};
            float *dst[5] = {dinit->S, dinit->C, dinit->m, dinit->G, dinit->h};
            const size_t cnt[5] = {BH * p->d * p->d, BH * p->d * p->dv, BH * p->d, BH * p->d * p->dv, BH * p->d};
            for (int i = 0; i < 5 && e == hipSuccess; ++i)
                e = hipMemcpyAsync(dst[i], src[i], cnt[i] * sizeof(float), hipMemcpyDeviceToDevice, stream);
        }
        if (e != hipSuccess) return fail(HLA_ERR_DEVICE, "backward launch: %s", hipGetErrorString(e));
        return ok();
    }
    const size_t esz = p->dtype == HLA_BF16 ? 2 : 4;
    const void *req[7] = {q, k, v, dout, dq, dk, dv};
    const char *nm[7] = {"q", "k", "v", "dout", "dq", "dk", "dv"};
    for (int i = 0; i < 7; ++i) {
        if (!req[i]) return fail(HLA_ERR_INVALID_ARGUMENT, "%s is NULL", nm[i]);
        if (!aligned16(req[i])) return fail(HLA_ERR_ALIGNMENT, "%s is not 16-byte aligned", nm[i]);
    }
    const size_t need = hla::backward_workspace_bytes(int(BH), p->n, p->d, p->dv, geo.w);
    if (!workspace) return fail(HLA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
        return fail(HLA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(HLA_ERR_ALIGNMENT, "workspace is not 256-byte aligned");
    std::vector<Span> outs, ins;
    outs.push_back(span("dq", dq, BH * n * p->d * 4));
    outs.push_back(span("dk", dk, BH * n * p->d * 4));
    outs.push_back(span("dv", dv, BH * n * p->dv * 4));
    outs.push_back(span("workspace", workspace, need));
    ins.push_back(span("q", q, BH * n * p->d * esz));
    ins.push_back(span("k", k, BH * n * p->d * esz));
    ins.push_back(span("v", v, BH * n * p->dv * esz));
    ins.push_back(span("dout", dout, BH * n * p->dv * 4));
    if (init) state_spans(init, "init", BH, p->d, p->dv, &ins);
    if (dinit) state_spans(dinit, "dinit", BH, p->d, p->dv, &outs);
    if (dfinal) state_spans(dfinal, "dfinal", BH, p->d, p->dv, &ins);
    std::string detail;
    if (first_overlap(outs, ins, &detail))
        return fail(HLA_ERR_INVALID_ARGUMENT, "aliasing: %s", detail.c_str());
    fp.B = p->B; fp.H = p->H; fp.n = p->n; fp.d = p->d; fp.dv = p->dv;
    fp.w = geo.w; fp.nc = geo.nc;
    fp.dtype = p->dtype; fp.ridge = p->ridge; fp.normalize = p->normalize;
    fp.q = q; fp.k = k; fp.v = v;
    if (init) fp.init = *init;
    fp.ws = workspace; fp.ws_bytes = workspace_bytes;
    bp.dout = dout; bp.dq = dq; bp.dk = dk; bp.dv = dv;
    if (dinit) bp.dinit = *dinit;
    if (dfinal) bp.dfinal = *dfinal;
    const hipError_t e = hla::la_backward_eligible(bp) ? hla::la_backward(bp, stream) : hla::generic_backward(bp, stream);
    if (e != hipSuccess) return fail(HLA_ERR_DEVICE, "backward launch: %s", hipGetErrorString(e));
    return ok();
}

hla_status hla_decode_step(const hla_params *p, const void *q, const void *k, const void *v,
                           hla_state *state, float *out, float *den, hipStream_t stream) {
    if (!p) return fail(HLA_ERR_INVALID_ARGUMENT, "params is NULL");
    if (p->B < 1 || p->H < 1) return fail(HLA_ERR_INVALID_ARGUMENT, "B=%d, H=%d must be >= 1", p->B, p->H);
    if (p->n != 1) return fail(HLA_ERR_INVALID_ARGUMENT, "decode needs n = 1 (got %d)", p->n);
    hla::DecodeProblem dp{};
    hla_status s = check_common(p->H, p->d, p->dv, dtype_code(p), p->gamma, p->ridge, p->normalize, &dp.gam);
    if (s != HLA_OK) return s;
    const uint64_t N = static_cast<uint64_t>(p->B) * p->H;
    if (N > 0x7fffffffull / (128ull * 128ull))
        return fail(HLA_ERR_UNSUPPORTED, "B*H=%llu too large", (unsigned long long)N);
    const void *req[4] = {q, k, v, out};
    const char *nm[4] = {"q", "k", "v", "out"};
    for (int i = 0; i < 4; ++i) {
        if (!req[i]) return fail(HLA_ERR_INVALID_ARGUMENT, "%s is NULL", nm[i]);
        if (!aligned16(req[i])) return fail(HLA_ERR_ALIGNMENT, "%s is not 16-byte aligned", nm[i]);
    }
    if (den && !aligned16(den)) return fail(HLA_ERR_ALIGNMENT, "den is not 16-byte aligned");
    if (!state) return fail(HLA_ERR_INVALID_ARGUMENT, "state is NULL");
    if ((s = check_state(state, "state")) != HLA_OK) return s;
    const size_t esz = p->dtype == HLA_BF16 ? 2 : 4;
    std::vector<Span> outs, ins;
    outs.push_back(span("out", out, N * p->dv * 4));
    if (den) outs.push_back(span("den", den, N * 4));
    state_spans(state, "state", N, p->d, p->dv, &outs);
    ins.push_back(span("q", q, N * p->d * esz));
    ins.push_back(span("k", k, N * p->d * esz));
    ins.push_back(span("v", v, N * p->dv * esz));
    std::string detail;
    if (first_overlap(outs, ins, &detail))
        return fail(HLA_ERR_INVALID_ARGUMENT, "aliasing: %s", detail.c_str());
    dp.B = p->B; dp.H = p->H; dp.d = p->d; dp.dv = p->dv; dp.dtype = p->dtype;
    dp.ridge = p->ridge; dp.normalize = p->normalize;
    dp.q = q; dp.k = k; dp.v = v; dp.st = *state; dp.out = out; dp.den = den;
    const hipError_t e = hla::decode_step(dp, stream);
    if (e != hipSuccess) return fail(HLA_ERR_DEVICE, "decode launch: %s", hipGetErrorString(e));
    return ok();
}

hla_status hla_decode_step_mq(const hla_params *p, int32_t kv_heads, const void *q, const void *k,
                              const void *v, hla_mq_state *state, float *out, float *den,
                              hipStream_t stream) {
    if (!p) return fail(HLA_ERR_INVALID_ARGUMENT, "params is NULL");
    if (p->B < 1 || p->H < 1) return fail(HLA_ERR_INVALID_ARGUMENT, "B=%d, H=%d must be >= 1", p->B, p->H);
    if (p->n != 1) return fail(HLA_ERR_INVALID_ARGUMENT, "decode needs n = 1 (got %d)", p->n);
    if (kv_heads < 1 || p->H % kv_heads != 0)
        return fail(HLA_ERR_INVALID_ARGUMENT, "kv_heads=%d must be >= 1 and divide H=%d", kv_heads, p->H);
    if (p->d != 32 && p->d != 64 && p->d != 128)
        return fail(HLA_ERR_UNSUPPORTED, "d=%d: the packed key moment needs d = 32, 64 or 128", p->d);
    hla::DecodeMqProblem dp{};
    hla_status s = check_common(p->H, p->d, p->dv, dtype_code(p), p->gamma, p->ridge, p->normalize, &dp.gam);
    if (s != HLA_OK) return s;
    const int R = p->H / kv_heads;
    if (p->gamma) {  // one decay per group: the group's S is decayed once
        for (int h = 0; h < p->H; ++h)
            if (p->gamma[h] != p->gamma[(h / R) * R])
                return fail(HLA_ERR_INVALID_ARGUMENT, "gamma[%d] differs from the first decay of its group", h);
    }
    const uint64_t N = static_cast<uint64_t>(p->B) * p->H, NG = static_cast<uint64_t>(p->B) * kv_heads;
    if (N > 0x7fffffffull / (128ull * 128ull))
        return fail(HLA_ERR_UNSUPPORTED, "B*H=%llu too large", (unsigned long long)N);
    const void *req[4] = {q, k, v, out};
    const char *nm[4] = {"q", "k", "v", "out"};
    for (int i = 0; i < 4; ++i) {
        if (!req[i]) return fail(HLA_ERR_INVALID_ARGUMENT, "%s is NULL", nm[i]);
        if (!aligned16(req[i])) return fail(HLA_ERR_ALIGNMENT, "%s is not 16-byte aligned", nm[i]);
    }
    if (den && !aligned16(den)) return fail(HLA_ERR_ALIGNMENT, "den is not 16-byte aligned");
    if (!state) return fail(HLA_ERR_INVALID_ARGUMENT, "state is NULL");
    {
        const hla_state as{state->S, state->C, state->m, state->G, state->h, state->rho};
        if ((s = check_state(&as, "state")) != HLA_OK) return s;
    }
    const size_t esz = p->dtype == HLA_BF16 ? 2 : 4, d = p->d, dv = p->dv;
    std::vector<Span> outs, ins;
    outs.push_back(span("out", out, N * dv * 4));
    if (den) outs.push_back(span("den", den, N * 4));
    outs.push_back(span("state.S", state->S, NG * (d * (d + 1) / 2) * 4));
    outs.push_back(span("state.C", state->C, N * d * dv * 4));
    outs.push_back(span("state.m", state->m, N * d * 4));
    outs.push_back(span("state.G", state->G, N * d * dv * 4));
    outs.push_back(span("state.h", state->h, N * d * 4));
    if (state->rho) outs.push_back(span("state.rho", state->rho, NG * 4));
    ins.push_back(span("q", q, N * d * esz));
    ins.push_back(span("k", k, NG * d * esz));
    ins.push_back(span("v", v, NG * dv * esz));
    std::string detail;
    if (first_overlap(outs, ins, &detail))
        return fail(HLA_ERR_INVALID_ARGUMENT, "aliasing: %s", detail.c_str());
    dp.B = p->B; dp.H = p->H; dp.kv_heads = kv_heads; dp.d = p->d; dp.dv = p->dv; dp.dtype = p->dtype;
    dp.ridge = p->ridge; dp.normalize = p->normalize;
    dp.q = q; dp.k = k; dp.v = v; dp.st = *state; dp.out = out; dp.den = den;
    const hipError_t e = hla::decode_step_mq(dp, stream);
    if (e != hipSuccess) return fail(HLA_ERR_DEVICE, "decode launch: %s", hipGetErrorString(e));
    return ok();
}

static hla_status pack_common(int32_t count, int32_t d, const float *src, float *dst, bool pack,
                              hipStream_t stream) {
    if (count < 0) return fail(HLA_ERR_INVALID_ARGUMENT, "count=%d must be >= 0", count);
    if (d != 32 && d != 64 && d != 128)
        return fail(HLA_ERR_UNSUPPORTED, "d=%d: the packed key moment needs d = 32, 64 or 128", d);
    if (count == 0) return ok();
    if (static_cast<uint64_t>(count) * 128ull * 128ull > 0x7fffffffull)
        return fail(HLA_ERR_UNSUPPORTED, "count=%d too large", count);
    if (!src || !dst) return fail(HLA_ERR_INVALID_ARGUMENT, "a pointer is NULL");
    if (!aligned16(src) || !aligned16(dst)) return fail(HLA_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const size_t full = static_cast<size_t>(count) * d * d * 4, packed = static_cast<size_t>(count) * (d * (d + 1) / 2) * 4;
    std::string detail;
    if (first_overlap({span("dst", dst, pack ? packed : full)}, {span("src", src, pack ? full : packed)}, &detail))
        return fail(HLA_ERR_INVALID_ARGUMENT, "aliasing: %s", detail.c_str());
    const hipError_t e = hla::key_moment_pack(count, d, src, dst, pack, stream);
    if (e != hipSuccess) return fail(HLA_ERR_DEVICE, "pack launch: %s", hipGetErrorString(e));
    return ok();
}

hla_status hla_key_moment_pack(int32_t count, int32_t d, const float *S_full, float *S_packed,
                               hipStream_t stream) {
    return pack_common(count, d, S_full, S_packed, true, stream);
}

hla_status hla_key_moment_unpack(int32_t count, int32_t d, const float *S_packed, float *S_full,
                                 hipStream_t stream) {
    return pack_common(count, d, S_packed, S_full, false, stream);
}

// ---- AHLA and third order: shared validation and dispatch

static hla_status higher_common(const hla_params *p, bool third, hla::GammaTab *gam) {
    hla_status s = check_common(p->H, p->d, p->dv, dtype_code(p), p->gamma, p->ridge, p->normalize, gam);
    if (s != HLA_OK) return s;
    if (p->ridge != 0.0f) return fail(HLA_ERR_UNSUPPORTED, "ridge must be 0 for this operator");
    if (third && p->gamma)
        for (int h = 0; h < p->H; ++h)
            if (p->gamma[h] != 1.0f)
                return fail(HLA_ERR_UNSUPPORTED, "third order takes no decay (gamma[%d] = %g)", h, double(p->gamma[h]));
    return HLA_OK;
}

static hla_status check_hi_state(const hla::HiState &st, bool third, const char *what) {
    const float *ptrs[5] = {st.X1, st.v1, st.X2, st.v2, st.S};
    const char *names[2][5] = {{"P", "m", "E", "n", "S"}, {"P", "m", "F", "Fd", "S"}};
    for (int i = 0; i < (third ? 5 : 4); ++i) {
        if (!ptrs[i]) return fail(HLA_ERR_INVALID_ARGUMENT, "%s->%s is NULL", what, names[third][i]);
        if (!aligned16(ptrs[i]))
            return fail(HLA_ERR_ALIGNMENT, "%s->%s is not 16-byte aligned", what, names[third][i]);
    }
    if (st.rho && (reinterpret_cast<uintptr_t>(st.rho) & 3u))
        return fail(HLA_ERR_ALIGNMENT, "%s->rho is not 4-byte aligned", what);
    return HLA_OK;
}

static void hi_spans(const hla::HiState &st, bool third, const char *prefix, size_t N, int d, int dv,
                     std::vector<Span> *out) {
    const char *tags[6] = {"P", "m", third ? "F" : "E", third ? "Fd" : "n", "S", "rho"};  // the header's names
    const float *ptrs[6] = {st.X1, st.v1, st.X2, st.v2, third ? st.S : nullptr, third ? nullptr : st.rho};
    const size_t sizes[6] = {N * d * dv, N * d, N * d * dv, N * d, N * d * d, N};
    for (int i = 0; i < 6; ++i)
        if (ptrs[i]) out->push_back(span(std::string(prefix) + "." + tags[i], ptrs[i], sizes[i] * sizeof(float)));
}

static size_t higher_need(const hla_params *p, bool third) {
    Geometry geo{};
    if (forward_geometry(p, &geo) != HLA_OK || !width_ok(p->d) || !width_ok(p->dv) || !dtype_ok(p)) return 0;
    return hla::higher_workspace_bytes(p->B * p->H, p->n, p->d, p->dv, geo.w, third);
}

static hla_status higher_forward_impl(const hla_params *p, bool third, const void *q, const void *k,
                                      const void *v, float *out, float *den, const hla::HiState *init,
                                      hla::HiState *fin, void *workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
    Geometry geo{};
    hla_status s = forward_geometry(p, &geo);
    if (s != HLA_OK) return s;
    hla::HiProblem hp{};
    if ((s = higher_common(p, third, &hp.gam)) != HLA_OK) return s;
    const size_t BH = static_cast<size_t>(p->B) * p->H, n = static_cast<size_t>(p->n);
    const size_t esz = p->dtype == HLA_BF16 ? 2 : 4;
    if (n > 0) {
        const void *req[4] = {q, k, v, out};
        const char *nm[4] = {"q", "k", "v", "out"};
        for (int i = 0; i < 4; ++i) {
            if (!req[i]) return fail(HLA_ERR_INVALID_ARGUMENT, "%s is NULL", nm[i]);
            if (!aligned16(req[i])) return fail(HLA_ERR_ALIGNMENT, "%s is not 16-byte aligned", nm[i]);
        }
        if (den && !aligned16(den)) return fail(HLA_ERR_ALIGNMENT, "den is not 16-byte aligned");
    }
    if (init && (s = check_hi_state(*init, third, "init")) != HLA_OK) return s;
    if (fin && (s = check_hi_state(*fin, third, "final_state")) != HLA_OK) return s;
    const size_t need = hla::higher_workspace_bytes(int(BH), p->n, p->d, p->dv, geo.w, third);
    if (need > 0) {
        if (!workspace) return fail(HLA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
        if (workspace_bytes < need)
            return fail(HLA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(HLA_ERR_ALIGNMENT, "workspace is not 256-byte aligned");
    }
    std::vector<Span> outs, ins;
    if (n > 0) {
        outs.push_back(span("out", out, BH * n * p->dv * 4));
        if (den) outs.push_back(span("den", den, BH * n * 4));
        ins.push_back(span("q", q, BH * n * p->d * esz));
        ins.push_back(span("k", k, BH * n * p->d * esz));
        ins.push_back(span("v", v, BH * n * p->dv * esz));
    }
    if (need > 0) outs.push_back(span("workspace", workspace, need));
    if (fin) hi_spans(*fin, third, "final_state", BH, p->d, p->dv, &outs);
    if (init) hi_spans(*init, third, "init", BH, p->d, p->dv, &ins);
    std::string detail;
    if (first_overlap(outs, ins, &detail))
        return fail(HLA_ERR_INVALID_ARGUMENT, "aliasing: %s", detail.c_str());
    if (n == 0 && !fin) return ok();
    hp.B = p->B; hp.H = p->H; hp.n = p->n; hp.d = p->d; hp.dv = p->dv; hp.w = geo.w;
    hp.dtype = p->dtype; hp.normalize = p->normalize; hp.third = third;
    hp.q = q; hp.k = k; hp.v = v; hp.out = out; hp.den = den;
    if (init) hp.init = *init;
    if (fin) hp.fin = *fin;
    hp.ws = workspace;
    const hipError_t e = hla::higher_forward(hp, stream);
    if (e != hipSuccess) return fail(HLA_ERR_DEVICE, "forward launch: %s", hipGetErrorString(e));
    return ok();
}

static hla_status higher_decode_impl(const hla_params *p, bool third, const void *q, const void *k,
                                     const void *v, hla::HiState *state, float *out, float *den,
                                     hipStream_t stream) {
    if (!p) return fail(HLA_ERR_INVALID_ARGUMENT, "params is NULL");
    if (p->B < 1 || p->H < 1) return fail(HLA_ERR_INVALID_ARGUMENT, "B=%d, H=%d must be >= 1", p->B, p->H);
    if (p->n != 1) return fail(HLA_ERR_INVALID_ARGUMENT, "decode needs n = 1 (got %d)", p->n);
    hla::HiDecodeProblem dp{};
    hla_status s = higher_common(p, third, &dp.gam);
    if (s != HLA_OK) return s;
    const uint64_t N = static_cast<uint64_t>(p->B) * p->H;
    if (N > 0x7fffffffull / (128ull * 128ull))
        return fail(HLA_ERR_UNSUPPORTED, "B*H=%llu too large", (unsigned long long)N);
    const void *req[4] = {q, k, v, out};
    const char *nm[4] = {"q", "k", "v", "out"};
    for (int i = 0; i < 4; ++i) {
        if (!req[i]) return fail(HLA_ERR_INVALID_ARGUMENT, "%s is NULL", nm[i]);
        if (!aligned16(req[i])) return fail(HLA_ERR_ALIGNMENT, "%s is not 16-byte aligned", nm[i]);
    }
    if (den && !aligned16(den)) return fail(HLA_ERR_ALIGNMENT, "den is not 16-byte aligned");
    if ((s = check_hi_state(*state, third, "state")) != HLA_OK) return s;
    const size_t esz = p->dtype == HLA_BF16 ? 2 : 4;
    std::vector<Span> outs, ins;
    outs.push_back(span("out", out, N * p->dv * 4));
    if (den) outs.push_back(span("den", den, N * 4));
    hi_spans(*state, third, "state", N, p->d, p->dv, &outs);
    ins.push_back(span("q", q, N * p->d * esz));
    ins.push_back(span("k", k, N * p->d * esz));
    ins.push_back(span("v", v, N * p->dv * esz));
    std::string detail;
    if (first_overlap(outs, ins, &detail))
        return fail(HLA_ERR_INVALID_ARGUMENT, "aliasing: %s", detail.c_str());
    dp.B = p->B; dp.H = p->H; dp.d = p->d; dp.dv = p->dv; dp.dtype = p->dtype; dp.normalize = p->normalize;
    dp.third = third; dp.q = q; dp.k = k; dp.v = v; dp.st = *state; dp.out = out; dp.den = den;
    const hipError_t e = hla::higher_decode(dp, stream);
    if (e != hipSuccess) return fail(HLA_ERR_DEVICE, "decode launch: %s", hipGetErrorString(e));
    return ok();
}

static hla::HiState from_ahla(const hla_ahla_state *s) {
    hla::HiState h{};
    if (s) h = hla::HiState{nullptr, s->P, s->m, s->E, s->n, s->rho};
    return h;
}

static hla::HiState from_third(const hla_third_state *s) {
    hla::HiState h{};
    if (s) h = hla::HiState{s->S, s->P, s->m, s->F, s->Fd, nullptr};
    return h;
}

size_t hla_ahla_workspace_size(const hla_params *p) { return p ? higher_need(p, false) : 0; }
size_t hla_third_workspace_size(const hla_params *p) { return p ? higher_need(p, true) : 0; }

hla_status hla_ahla_forward(const hla_params *p, const void *q, const void *k, const void *v, float *out,
                            float *den, const hla_ahla_state *init, hla_ahla_state *final_state,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!p) return fail(HLA_ERR_INVALID_ARGUMENT, "params is NULL");
    hla::HiState i = from_ahla(init), f = from_ahla(final_state);
    return higher_forward_impl(p, false, q, k, v, out, den, init ? &i : nullptr, final_state ? &f : nullptr,
                               workspace, workspace_bytes, stream);
}

hla_status hla_third_forward(const hla_params *p, const void *q, const void *k, const void *v, float *out,
                             float *den, const hla_third_state *init, hla_third_state *final_state,
                             void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!p) return fail(HLA_ERR_INVALID_ARGUMENT, "params is NULL");
    hla::HiState i = from_third(init), f = from_third(final_state);
    return higher_forward_impl(p, true, q, k, v, out, den, init ? &i : nullptr, final_state ? &f : nullptr,
                               workspace, workspace_bytes, stream);
}

hla_status hla_ahla_decode_step(const hla_params *p, const void *q, const void *k, const void *v,
                                hla_ahla_state *state, float *out, float *den, hipStream_t stream) {
    if (!state) return fail(HLA_ERR_INVALID_ARGUMENT, "state is NULL");
    hla::HiState s = from_ahla(state);
    return higher_decode_impl(p, false, q, k, v, &s, out, den, stream);
}

hla_status hla_third_decode_step(const hla_params *p, const void *q, const void *k, const void *v,
                                 hla_third_state *state, float *out, float *den, hipStream_t stream) {
    if (!state) return fail(HLA_ERR_INVALID_ARGUMENT, "state is NULL");
    hla::HiState s = from_third(state);
    return higher_decode_impl(p, true, q, k, v, &s, out, den, stream);
}

hla_status hla_state_compose(int32_t count, int32_t d, int32_t dv, const hla_state *earlier,
                             const hla_state *later, hla_state *result, hipStream_t stream) {
    if (count < 0) return fail(HLA_ERR_INVALID_ARGUMENT, "count=%d must be >= 0", count);
    if (!width_ok(d) || !width_ok(dv))
        return fail(HLA_ERR_UNSUPPORTED, "d=%d, dv=%d: each must be 16, 32, 64 or 128", d, dv);
    if (!earlier || !later || !result) return fail(HLA_ERR_INVALID_ARGUMENT, "a state pointer is NULL");
    if (count == 0) return ok();
    if (static_cast<uint64_t>(count) * 128ull * 128ull > 0x7fffffffull)
        return fail(HLA_ERR_UNSUPPORTED, "count=%d too large", count);
    hla_status s;
    if ((s = check_state(earlier, "earlier")) != HLA_OK) return s;
    if ((s = check_state(later, "later")) != HLA_OK) return s;
    if ((s = check_state(result, "result")) != HLA_OK) return s;
    std::vector<Span> outs, ins;
    state_spans(result, "result", size_t(count), d, dv, &outs);
    state_spans(earlier, "earlier", size_t(count), d, dv, &ins);
    state_spans(later, "later", size_t(count), d, dv, &ins);
    std::string detail;
    if (first_overlap(outs, ins, &detail))
        return fail(HLA_ERR_INVALID_ARGUMENT, "aliasing: %s", detail.c_str());
    const hipError_t e = hla::state_compose(count, d, dv, *earlier, *later, *result, stream);
    if (e != hipSuccess) return fail(HLA_ERR_DEVICE, "compose launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
