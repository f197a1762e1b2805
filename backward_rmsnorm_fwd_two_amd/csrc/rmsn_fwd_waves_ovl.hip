// rmsn_fwd_waves_ovl.hip -- forward and fused add + RMSNorm forward row
// kernels on a whole number of waves (lanes = 64 W, W = 3, 5, 6, 7, 9 ... 15,
// one or two 16-byte vectors per lane) for rows that are not a whole number
// of 16-byte vectors: ceil(D / NV) vectors, the last one shifted back to end
// at the row's end, the slots past it masked.  Such rows (D = 2049, 4097,
// 6001 ... in 16-bit storage) would otherwise take a power-of-two lane
// count at about half fill.  A separate translation unit, so that it
// compiles in parallel with the other instances.
#include "rmsn_kernels.hpp"

namespace rmsn {
namespace {

template <typename T, int K, bool FUSED>
const void* pick_waves(int lanes) {
    constexpr int NV = 16 / static_cast<int>(sizeof(T));
    switch (lanes) {
        case 192: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 192, true>);
        case 320: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 320, true>);
        case 384: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 384, true>);
        case 448: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 448, true>);
        case 576: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 576, true>);
        case 640: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 640, true>);
        case 704: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 704, true>);
        case 768: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 768, true>);
        case 832: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 832, true>);
        case 896: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 896, true>);
        case 960: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 960, true>);
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

const void* fwd_kernel_wave_rows_ovl(int dt, int nv, int k, bool fused, int lanes) {
    return fused ? pick_dt<true>(dt, nv, k, lanes) : pick_dt<false>(dt, nv, k, lanes);
}

}  // namespace rmsn
