// device_stubs.cpp -- stand-ins for the device side of the library, so that
// the host entry points (argument validation, workspace sizing, error text)
// can be built with g++ and AddressSanitizer/UndefinedBehaviorSanitizer and
// run on a machine without a GPU.
//
// Nothing here computes.  Every launcher aborts: a call that reaches one has
// passed validation, and the sanitizer runs only make calls that must not.
// The workspace sizes are simple fixed formulas (not the library's), which is
// all that the validation of a workspace argument needs: it compares the
// caller's size with the size these functions report.
#include <cstdio>
#include <cstdlib>

#include "hla_internal.h"

namespace {
[[noreturn]] void reached(const char *what) {
    std::fprintf(stderr, "device stub reached: %s (a call passed validation)\n", what);
    std::abort();
}
size_t fixed_size(int BH, int n, int d, int dv) {
    return 8192 + static_cast<size_t>(BH) * (static_cast<size_t>(n) + 1) * (d + dv) * 16;
}
}  // namespace

namespace hla {

size_t generic_workspace_bytes(int BH, int n, int d, int dv, int) { return fixed_size(BH, n, d, dv); }
hipError_t generic_forward(const FwdProblem &, hipStream_t) { reached("generic_forward"); }
size_t generic_backward_workspace_bytes(int BH, int n, int d, int dv, int) { return 2 * fixed_size(BH, n, d, dv); }
hipError_t generic_backward(const BwdProblem &, hipStream_t) { reached("generic_backward"); }
hipError_t zero_state_grad(const hla_state &, int, int, int, hipStream_t) { reached("zero_state_grad"); }
bool la_backward_eligible(const BwdProblem &) { return false; }
size_t la_backward_workspace_bytes(int BH, int n) { return fixed_size(BH, n, 64, 64); }
hipError_t la_backward(const BwdProblem &, hipStream_t) { reached("la_backward"); }
size_t backward_workspace_bytes(int BH, int n, int d, int dv, int w) { return generic_backward_workspace_bytes(BH, n, d, dv, w); }
hla_status noalloc_scratch(void **) { reached("noalloc_scratch"); }
bool fast64_supported(const FwdProblem &) { return false; }
size_t fast64_flag_bytes(int BH, int n) { return fixed_size(BH, n, 1, 1); }
size_t fast64_data_bytes(int BH, int n) { return fixed_size(BH, n, 64, 64); }
hipError_t fast64_forward(const FwdProblem &, uint32_t *, uint32_t *, void *, hipStream_t) { reached("fast64_forward"); }
bool fused128_supported(const FwdProblem &) { return false; }
size_t fused128_flag_bytes(int BH, int n) { return fixed_size(BH, n, 1, 1); }
size_t fused128_data_bytes(int BH, int n) { return fixed_size(BH, n, 128, 128); }
hipError_t fused128_forward(const FwdProblem &, uint32_t *, uint32_t *, void *, hipStream_t) { reached("fused128_forward"); }
bool small_supported(const FwdProblem &) { return false; }
size_t small_data_bytes(int BH, int n, int d) { return fixed_size(BH, n, d, 1); }
hipError_t small_forward(const FwdProblem &, void *, hipStream_t) { reached("small_forward"); }
hipError_t decode_step(const DecodeProblem &, hipStream_t) { reached("decode_step"); }
hipError_t decode_step_mq(const DecodeMqProblem &, hipStream_t) { reached("decode_step_mq"); }
hipError_t key_moment_pack(int, int, const float *, float *, bool, hipStream_t) { reached("key_moment_pack"); }
size_t higher_workspace_bytes(int BH, int n, int d, int dv, int, bool third) {
    return (third ? 3 : 2) * fixed_size(BH, n, d, dv);
}
hipError_t higher_forward(const HiProblem &, hipStream_t) { reached("higher_forward"); }
hipError_t higher_decode(const HiDecodeProblem &, hipStream_t) { reached("higher_decode"); }
hipError_t state_compose(int, int, int, const hla_state &, const hla_state &, const hla_state &, hipStream_t) {
    reached("state_compose");
}

}  // namespace hla

// the two HIP runtime calls the host entry points make
extern "C" const char *hipGetErrorString(hipError_t) { return "hip runtime stand-in"; }
extern "C" hipError_t hipMemcpyAsync(void *, const void *, size_t, hipMemcpyKind, hipStream_t) {
    reached("hipMemcpyAsync");
}
