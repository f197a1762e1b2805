// rmsn_fwd.hip -- instances of the forward and fused add+RMSNorm kernels.
#include "rmsn_kernels.hpp"

namespace rmsn {
namespace {

template <typename T, int NV, bool FUSED>
const void* pick_fwd(int k) {
    switch (k) {
        case -1: return reinterpret_cast<const void*>(&rows_looped<T, NV, FUSED ? 1 : 0>);
        case 1: return reinterpret_cast<const void*>(&fwd_rows<T, NV, 1, FUSED>);
        case 2: return reinterpret_cast<const void*>(&fwd_rows<T, NV, 2, FUSED>);
        case 4: return reinterpret_cast<const void*>(&fwd_rows<T, NV, 4, FUSED>);
        case 8: return reinterpret_cast<const void*>(&fwd_rows<T, NV, 8, FUSED>);
        default: return nullptr;
    }
}

template <typename T, bool FUSED>
const void* pick_fwd_nv(int nv, int k) {
    switch (nv) {
        case 1: return pick_fwd<T, 1, FUSED>(k);
        case 2: return pick_fwd<T, 2, FUSED>(k);
        case 4: return pick_fwd<T, 4, FUSED>(k);
        case 8:
            if constexpr (sizeof(T) == 2) return pick_fwd<T, 8, FUSED>(k);
            return nullptr;
        default: return nullptr;
    }
}

template <bool FUSED>
const void* pick_fwd_dt(int dt, int nv, int k) {
    switch (dt) {
        case kF32: return pick_fwd_nv<float, FUSED>(nv, k);
        case kF16: return pick_fwd_nv<_Float16, FUSED>(nv, k);
        case kBF16: return pick_fwd_nv<__bf16, FUSED>(nv, k);
        default: return nullptr;
    }
}

}  // namespace

const void* fwd_kernel(int dt, int nv, int k, bool fused) {
    return fused ? pick_fwd_dt<true>(dt, nv, k) : pick_fwd_dt<false>(dt, nv, k);
}

}  // namespace rmsn
