// rmsn_ovl.hip -- instances of the forward and plain-loop backward kernels
// for rows that are not a whole number of 16-byte vectors: ceil(D / NV)
// vectors per row, the last one shifted back to end at the row's end, its
// overlapped leading elements kept out of the sums and of dw (Cols in
// rmsn_kernels.hpp).
#include "rmsn_kernels.hpp"

namespace rmsn {
namespace {

template <typename T, bool FUSED>
const void* pick_fwd_ovl(int k) {
    constexpr int NV = 16 / static_cast<int>(sizeof(T));
    switch (k) {
        case 1: return reinterpret_cast<const void*>(&fwd_rows<T, NV, 1, FUSED, 0, true>);
        case 2: return reinterpret_cast<const void*>(&fwd_rows<T, NV, 2, FUSED, 0, true>);
        case 4: return reinterpret_cast<const void*>(&fwd_rows<T, NV, 4, FUSED, 0, true>);
        case 8: return reinterpret_cast<const void*>(&fwd_rows<T, NV, 8, FUSED, 0, true>);
        default: return nullptr;
    }
}

template <typename T, int MODE>
const void* pick_vjp_ovl(int k) {
    constexpr int NV = 16 / static_cast<int>(sizeof(T));
    switch (k) {
        case 1: return reinterpret_cast<const void*>(&vjp_rows<T, NV, 1, MODE, false, 0, PartialRowOut, true>);
        case 2: return reinterpret_cast<const void*>(&vjp_rows<T, NV, 2, MODE, false, 0, PartialRowOut, true>);
        case 4: return reinterpret_cast<const void*>(&vjp_rows<T, NV, 4, MODE, false, 0, PartialRowOut, true>);
        case 8: return reinterpret_cast<const void*>(&vjp_rows<T, NV, 8, MODE, false, 0, PartialRowOut, true>);
        default: return nullptr;
    }
}

template <typename T>
const void* pick_vjp_ovl_mode(int k, int mode) {
    switch (mode) {
        case kVjp: return pick_vjp_ovl<T, kVjp>(k);
        case kGrad: return pick_vjp_ovl<T, kGrad>(k);
        case kResGrad: return pick_vjp_ovl<T, kResGrad>(k);
        default: return nullptr;
    }
}

}  // namespace

const void* fwd_kernel_ovl(int dt, int k, bool fused) {
    switch (dt) {
        case kF32: return fused ? pick_fwd_ovl<float, true>(k) : pick_fwd_ovl<float, false>(k);
        case kF16: return fused ? pick_fwd_ovl<_Float16, true>(k) : pick_fwd_ovl<_Float16, false>(k);
        case kBF16: return fused ? pick_fwd_ovl<__bf16, true>(k) : pick_fwd_ovl<__bf16, false>(k);
        default: return nullptr;
    }
}

const void* vjp_kernel_ovl(int dt, int k, int mode) {
    switch (dt) {
        case kF32: return pick_vjp_ovl_mode<float>(k, mode);
        case kF16: return pick_vjp_ovl_mode<_Float16>(k, mode);
        case kBF16: return pick_vjp_ovl_mode<__bf16>(k, mode);
        default: return nullptr;
    }
}

}  // namespace rmsn
