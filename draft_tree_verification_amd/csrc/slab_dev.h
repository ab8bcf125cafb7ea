// slab_dev.h -- one slab of a logit row held in registers by a workgroup.
// Shared by the exit-guided loss and the tree builder.
#pragma once

#include "exit_law_dev.h"

namespace tev {
namespace {

// Slab ownership: thread t holds elements k*(THREADS*VW) + t*VW + j, k < EPT/VW,
// j < VW (VW = elements per 16 bytes).  Elements at or past len read a
// clamped valid address and become -inf; loads are unconditional.
template <typename T, bool VEC, int THREADS, int EPT>
__device__ __forceinline__ void load_slab(const T *p, int len, int tid, float *x) {
    constexpr int VW = 16 / (int)sizeof(T);
    constexpr int SPAN = THREADS * VW;
#pragma unroll
    for (int k = 0; k < EPT / VW; k++) {
        const int idx = k * SPAN + tid * VW;
        if (VEC) {
            // len is a multiple of VW (16-byte rows), so len - VW is a whole vector
            load16(p + min(idx, len - VW), &x[k * VW]);
#pragma unroll
            for (int j = 0; j < VW; j++) x[k * VW + j] = (idx < len) ? x[k * VW + j] : -kInf;
        } else {
#pragma unroll
            for (int j = 0; j < VW; j++) {
                const float t = to_f32<T>(p[min(idx + j, len - 1)]);
                x[k * VW + j] = (idx + j < len) ? t : -kInf;
            }
        }
    }
}

}  // namespace
}  // namespace tev
