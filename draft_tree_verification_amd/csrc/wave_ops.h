// wave_ops.h -- wavefront-level reductions and scans for gfx950 (64 lanes).
//
// In-row steps use DPP lane permutes (quad_perm / row_mirror / row_shr), which
// are VALU operands with a few cycles of latency, instead of LDS-routed
// shuffles.  The four 16-lane rows are then combined through v_readlane into
// uniform values.  Every reduction combines values in one fixed order, so the
// results are bit-reproducible run to run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tev {
namespace wave {

// DPP control codes (GCN/CDNA encoding).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowShr = 0x110;        // row_shr:n = kRowShr + n

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
    const int2 v = __builtin_bit_cast(int2, x);
    const int lo = __builtin_amdgcn_mov_dpp(v.x, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(v.y, CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, int2{lo, hi});
}
// row_shr with zero fill for lanes whose source lies before the row start
template <int N>
__device__ __forceinline__ double shr_d(double x) {
    const int2 v = __builtin_bit_cast(int2, x);
    const int lo = __builtin_amdgcn_mov_dpp(v.x, kRowShr + N, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_mov_dpp(v.y, kRowShr + N, 0xF, 0xF, true);
    return __builtin_bit_cast(double, int2{lo, hi});
}

__device__ __forceinline__ float readlane_f(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ double readlane_d(double x, int l) {
    const int2 v = __builtin_bit_cast(int2, x);
    return __builtin_bit_cast(double, int2{__builtin_amdgcn_readlane(v.x, l),
                                           __builtin_amdgcn_readlane(v.y, l)});
}

// ---- reductions: every lane receives the result ----
__device__ __forceinline__ float max_f32(float x) {
    x = fmaxf(x, dpp_f<kQuadXor1>(x));
    x = fmaxf(x, dpp_f<kQuadXor2>(x));
    x = fmaxf(x, dpp_f<kRowHalfMirror>(x));
    x = fmaxf(x, dpp_f<kRowMirror>(x));
    return fmaxf(fmaxf(readlane_f(x, 0), readlane_f(x, 16)), fmaxf(readlane_f(x, 32), readlane_f(x, 48)));
}
__device__ __forceinline__ float sum_f32(float x) {
    x += dpp_f<kQuadXor1>(x);
    x += dpp_f<kQuadXor2>(x);
    x += dpp_f<kRowHalfMirror>(x);
    x += dpp_f<kRowMirror>(x);
    return (readlane_f(x, 0) + readlane_f(x, 16)) + (readlane_f(x, 32) + readlane_f(x, 48));
}
__device__ __forceinline__ double sum_f64(double x) {
    x += dpp_d<kQuadXor1>(x);
    x += dpp_d<kQuadXor2>(x);
    x += dpp_d<kRowHalfMirror>(x);
    x += dpp_d<kRowMirror>(x);
    return (readlane_d(x, 0) + readlane_d(x, 16)) + (readlane_d(x, 32) + readlane_d(x, 48));
}
__device__ __forceinline__ int sum_i32(int x) {
    x += dpp_i<kQuadXor1>(x);
    x += dpp_i<kQuadXor2>(x);
    x += dpp_i<kRowHalfMirror>(x);
    x += dpp_i<kRowMirror>(x);
    return (__builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16)) +
           (__builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48));
}
__device__ __forceinline__ int max_i32(int x) {
    x = max(x, dpp_i<kQuadXor1>(x));
    x = max(x, dpp_i<kQuadXor2>(x));
    x = max(x, dpp_i<kRowHalfMirror>(x));
    x = max(x, dpp_i<kRowMirror>(x));
    return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
               max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
__device__ __forceinline__ unsigned or_u32(unsigned x) {
    int y = (int)x;
    y |= dpp_i<kQuadXor1>(y);
    y |= dpp_i<kQuadXor2>(y);
    y |= dpp_i<kRowHalfMirror>(y);
    y |= dpp_i<kRowMirror>(y);
    return (unsigned)((__builtin_amdgcn_readlane(y, 0) | __builtin_amdgcn_readlane(y, 16)) |
                      (__builtin_amdgcn_readlane(y, 32) | __builtin_amdgcn_readlane(y, 48)));
}

// ---- inclusive scan over the 64 lanes in lane order (fp64) ----
// In-row Hillis-Steele with row_shr 1, 2, 4, 8, then the totals of the
// preceding rows are added (read back as uniform values).
__device__ __forceinline__ double incl_scan_f64(double x, int lane) {
    x += shr_d<1>(x);
    x += shr_d<2>(x);
    x += shr_d<4>(x);
    x += shr_d<8>(x);
    const double r0 = readlane_d(x, 15), r1 = readlane_d(x, 31), r2 = readlane_d(x, 47);
    const int row = lane >> 4;
    const double carry = row == 0 ? 0.0 : row == 1 ? r0 : row == 2 ? r0 + r1 : (r0 + r1) + r2;
    return carry + x;
}

// Total of the wave after incl_scan_f64 (lane 63's value).
__device__ __forceinline__ double last_lane_d(double x) { return readlane_d(x, 63); }

// Orders this wave's LDS traffic: the LDS executes one wave's instructions in
// program order, so only the compiler has to be kept from reordering.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

}  // namespace wave
}  // namespace tev
