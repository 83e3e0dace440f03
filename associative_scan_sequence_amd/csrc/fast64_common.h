// fast64_common.h -- device helpers of the one-launch d = 64 forward
// (k_fast64): bf16 MFMA operand plumbing on swizzled 64 x 64 LDS tiles,
// operand splits, and the cross-workgroup hand-off.
#pragma once

#include "bf16_split.h"
#include "device_common.h"
#include "hla_internal.h"

namespace hla {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int W = 64;          // chunk width = d = dv
constexpr int kTileElems = W * W;  // one LDS tile: 64 rows of 64 bf16, see tile_off
constexpr int kSpinLimit = 1 << 22;
constexpr int kSpinWord = 4;   // control word: spin limit of the bounded waits (0: kSpinLimit)
constexpr int kLine = 64;      // words per 256-byte control line
constexpr int kTicketWord = kLine + 2;  // control word: next segment ticket (looped grids)
constexpr int kHeadTicketWord = 2 * kLine;  // per-head segment tickets, 8 words apart (one-pass grids)
constexpr int kHeadTicketStride = 8;
constexpr int kMaxTicketHeads = (static_cast<int>(kCtrlBytes / 4) - kHeadTicketWord) / kHeadTicketStride;
constexpr int kFlagStride = 32;  // words between flags (one 128-byte line each)
constexpr float kMinGamma = 0.75f;
static_assert(kCtrlBytes >= 2 * kLine * 4, "control block too small");

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS tile layout: 64 rows of 64 bf16, unpadded; the 8-byte pieces of a row
// are permuted by an XOR of their index with a function of the row, chosen so
// that every access pattern used on tiles (16-byte row reads of 16 rows x 4
// column groups, transposed 8-byte reads of 4+4 or 8 consecutive rows, 8-byte
// row writes, 16-byte staging writes) touches each of the 64 LDS banks at
// most once per cycle.  Pieces keep their pairs (XOR on index bits 1-3), so
// 16-byte accesses at 8-element columns stay contiguous and aligned.  (Rows
// padded to 72 elements would cost 2x on 16-byte row reads and ~1.75x on
// transposed reads.)
__device__ __forceinline__ int tile_off(int row, int col) {
    const int b1 = (row >> 1) & 1, b2 = (row >> 2) & 1, b3 = (row >> 3) & 1;
    const int h = b3 | ((b1 ^ b3) << 1) | ((b2 ^ b3) << 2);
    return row * W + ((((col >> 2) ^ (h << 1))) << 2) + (col & 3);
}

// 8 consecutive bf16 of one tile row (col a multiple of 8)
__device__ __forceinline__ bf16x8 ld8(const __bf16 *base, int row, int col) {
    return *reinterpret_cast<const bf16x8 *>(base + tile_off(row, col));
}

// 8 consecutive bf16 (16 bytes) written to one tile row (col a multiple of 8)
__device__ __forceinline__ void st16(__bf16 *base, int row, int col, const u32x4 &v) {
    *reinterpret_cast<u32x4 *>(base + tile_off(row, col)) = v;
}

// Transposed operand: lane (g, r) receives M[rb1 + e][col0 + r] (k slots 8g+e,
// e < 4) and M[rb2 + e][col0 + r] (slots 8g+4+e); rb1, rb2 may depend on g.
__device__ __forceinline__ bf16x8 tr8(const __bf16 *M, int rb1, int rb2, int col0, int r) {
    const int col = col0 + 4 * (r & 3);
    const __bf16 *p1 = M + tile_off(rb1 + (r >> 2), col);
    const __bf16 *p2 = M + tile_off(rb2 + (r >> 2), col);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p1));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p2));
    bf16x8 x;
    const bf16x4 ab = __builtin_bit_cast(bf16x4, a), bb = __builtin_bit_cast(bf16x4, b);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = ab[i];
        x[4 + i] = bb[i];
    }
    return x;
}

__device__ __forceinline__ void st4(__bf16 *base, int row, int col, const bf16x4 &v) {
    *reinterpret_cast<bf16x4 *>(base + tile_off(row, col)) = v;
}

template <int CTL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTL, 0xF, 0xF, true));
}

// sum over the 16 lanes of a DPP row; every lane of the row receives it
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    return v;
}

// Cross-workgroup hand-off without cache maintenance: aggregates and flags
// are written and read as device-coherent (sc1) accesses, so no L2
// write-back or invalidate is needed.  The writer waits for its stores to
// complete (vmcnt 0) before the flag store; readers poll the flag and only
// then load the aggregate.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ }

__device__ __forceinline__ uint32_t next_epoch(uint32_t e) { return e * 1664525u + 1013904223u; }

// The spin limit is kSpinLimit polls, or the control word *spin_word when it
// is nonzero; the word is read only once the first poll has failed.
__device__ __forceinline__ int spin_limit(const uint32_t *spin_word) {
    const int s = static_cast<int>(__hip_atomic_load(spin_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    return s > 0 ? s : (s < 0 ? 1 : kSpinLimit);  // -1: give up after the first poll
}

__device__ bool wait_flag(uint32_t *f, uint32_t want, const uint32_t *spin_word) {
    int spin = kSpinLimit;
    for (int it = 0; it < spin; ++it) {
        if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want) return true;
        if (it == 0) spin = spin_limit(spin_word);
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

__device__ __forceinline__ void set_flag(uint32_t *f, uint32_t v) {
    __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kSc1 = 16;  // buffer cache policy: sc1 (device scope)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const float *slot) {
    // slot addresses are uniform across the wave; say so, so the descriptor is scalar
    const uint64_t addr = reinterpret_cast<uint64_t>(slot);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(addr)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(addr >> 32)));
    float *base = reinterpret_cast<float *>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, 16384, 0x00020000);
}

}  // namespace
}  // namespace hla
