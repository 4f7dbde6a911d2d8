// Cross-lane helpers of the gfx950 quantizers: DPP row operations and the
// ds_swizzle crossbar (no LDS memory, no VALU slot).
#pragma once

#include <hip/hip_runtime.h>

namespace kvq {

// DPP controls (gfx9 encoding)
constexpr int DPP_QUAD_XOR1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int DPP_ROR4 = 0x124;      // lane i <- lane (i - 4) mod 16
constexpr int DPP_ROR8 = 0x128;      // lane i <- lane (i - 8) mod 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Partner value across lanes, lane ^ M within 32-lane groups (ds_swizzle bit mode).
template <int M>
__device__ __forceinline__ float swz_xor(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (M << 10) | 0x1F));
}

// Sum / min / max over the 16 lanes of a DPP row; every lane gets the same bits.
__device__ __forceinline__ float row_sum16(float s) {
    s += dpp<DPP_ROR8>(s);
    s += dpp<DPP_ROR4>(s);
    s += dpp<DPP_QUAD_XOR2>(s);
    s += dpp<DPP_QUAD_XOR1>(s);
    return s;
}
__device__ __forceinline__ float row_min16(float s) {
    s = fminf(s, dpp<DPP_ROR8>(s));
    s = fminf(s, dpp<DPP_ROR4>(s));
    s = fminf(s, dpp<DPP_QUAD_XOR2>(s));
    return fminf(s, dpp<DPP_QUAD_XOR1>(s));
}
__device__ __forceinline__ float row_max16(float s) {
    s = fmaxf(s, dpp<DPP_ROR8>(s));
    s = fmaxf(s, dpp<DPP_ROR4>(s));
    s = fmaxf(s, dpp<DPP_QUAD_XOR2>(s));
    return fmaxf(s, dpp<DPP_QUAD_XOR1>(s));
}

}  // namespace kvq
