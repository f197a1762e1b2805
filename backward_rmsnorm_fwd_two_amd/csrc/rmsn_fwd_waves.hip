// rmsn_fwd_waves.hip -- forward and fused add + RMSNorm forward row kernels
// for rows of a whole number of waves that is not a power of two: lanes =
// 64 W, W = 3, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15, one or two 16-byte vectors
// per lane.
// Such rows (D = 3072, 5120, 6144, 7168 ... in 16-bit storage) then tile
// exactly instead of leaving part of a power-of-two lane group masked.  A
// separate translation unit, so that it compiles in parallel with the other
// instances.
#include "rmsn_kernels.hpp"

namespace rmsn {
namespace {

template <typename T, int K, bool FUSED>
const void* pick_waves(int lanes) {
    constexpr int NV = 16 / static_cast<int>(sizeof(T));
    switch (lanes) {
        case 192: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 192>);
        case 320: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 320>);
        case 384: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 384>);
        case 448: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 448>);
        case 576: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 576>);
        case 640: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 640>);
        case 704: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 704>);
        case 768: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 768>);
        case 832: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 832>);
        case 896: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 896>);
        case 960: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 960>);
        default: return nullptr;
    }
}

template <typename T, bool FUSED>
const void* pick_k(int nv, int k, int lanes) {
    if (nv != 16 / static_cast<int>(sizeof(T))) return nullptr;
    switch (k) {
        case 1: return pick_waves<T, 1, FUSED>(lanes);
        case 2: return pick_waves<T, 2, FUSED>(lanes);
        default: return nullptr;
    }
}

template <bool FUSED>
const void* pick_dt(int dt, int nv, int k, int lanes) {
    switch (dt) {
        case kF32: return pick_k<float, FUSED>(nv, k, lanes);
        case kF16: return pick_k<_Float16, FUSED>(nv, k, lanes);
        case kBF16: return pick_k<__bf16, FUSED>(nv, k, lanes);
        default: return nullptr;
    }
}

}  // namespace

const void* fwd_kernel_wave_rows(int dt, int nv, int k, bool fused, int lanes) {
    return fused ? pick_dt<true>(dt, nv, k, lanes) : pick_dt<false>(dt, nv, k, lanes);
}

}  // namespace rmsn
