// wave_ops.h -- wave-level reductions and scans (64-lane waves, gfx950).
// Every routine adds in a fixed order, so results do not depend on timing.
#pragma once

#include <hip/hip_runtime.h>

namespace twell {

// Sum over the 64 lanes with DPP row shifts and row broadcasts (an inclusive
// scan whose last lane holds the total), returned as a wave-uniform value.
__device__ __forceinline__ float wave_sum(float v)
{
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));  // row_shr:1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));  // row_shr:2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));  // row_shr:4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));  // row_shr:8
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));  // row_bcast:15
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Integer sum over the 64 lanes (butterfly), the same value in every lane.
__device__ __forceinline__ int wave_isum(int v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, 64);
    return v;
}

// Inclusive scan over the 64 lanes (lane = this lane's index).
__device__ __forceinline__ int wave_incl_scan(int v, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o)
            v += u;
    }
    return v;
}

// Exclusive scan over the 64 lanes; `total` gets the sum of all lanes.
__device__ __forceinline__ int wave_excl_scan(int v, int lane, int &total)
{
    const int incl = wave_incl_scan(v, lane);
    total = __shfl(incl, 63, 64);
    return incl - v;
}

// Inclusive scan over the 64 lanes with DPP (row shifts, row broadcasts).
__device__ __forceinline__ int wave_incl_scan_dpp(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
    return v;
}

// Inclusive scan of v over segments of L lanes (L a power of two, <= 64; gl =
// lane within its segment): DPP row shifts inside 16-lane rows (masked at
// segment starts when L < 16), then row broadcasts across rows.
__device__ __forceinline__ int seg_incl_scan(int v, int gl, int L)
{
    int y = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += gl >= 1 ? y : 0;
    if (L > 2) {
        y = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
        v += gl >= 2 ? y : 0;
    }
    if (L > 4) {
        y = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
        v += gl >= 4 ? y : 0;
    }
    if (L > 8) {
        y = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
        v += gl >= 8 ? y : 0;
    }
    if (L > 16)
        v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    if (L > 32)
        v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
    return v;
}

}  // namespace twell
