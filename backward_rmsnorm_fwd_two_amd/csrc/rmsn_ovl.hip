// rmsn_ovl.hip -- instances of the forward and plain-loop backward kernels
// for rows that are not a whole number of 16-byte vectors: ceil(D / NV)
// vectors per row, the last one shifted back to end at the row's end, its
// overlapped leading elements kept out of the sums and of dw (Cols in
// rmsn_kernels.hpp).  The forward forms also come with the lanes fixed at
// compile time for the short rows the plan lays out on 16..128 lanes x 2 or
// 4 (the small-axis band, D = 257..1023 in 16-bit storage): the row
// reduction compiles without branches on the row width (16384 rows fp16, D
// = 257 / 500 / 511 on 32 lanes x 2: 8.8 -> 7.9 us; 513 on 64 x 2: 11.2 ->
// 10.5 us).
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

template <typename T, bool FUSED, int K>
const void* pick_fwd_ovl_lanes(int lanes) {
    constexpr int NV = 16 / static_cast<int>(sizeof(T));
    switch (lanes) {
        case 16: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 16, true>);
        case 32: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 32, true>);
        case 64: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 64, true>);
        case 128: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 128, true>);
        default: return nullptr;
    }
}

template <typename T, bool FUSED>
const void* pick_fwd_ovl_fixed(int k, int lanes) {
    switch (k) {
        case 2: return pick_fwd_ovl_lanes<T, FUSED, 2>(lanes);
        case 4: return pick_fwd_ovl_lanes<T, FUSED, 4>(lanes);
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

const void* fwd_kernel_ovl_fixed(int dt, int k, bool fused, int lanes) {
    switch (dt) {
        case kF32: return fused ? pick_fwd_ovl_fixed<float, true>(k, lanes) : pick_fwd_ovl_fixed<float, false>(k, lanes);
        case kF16:
            return fused ? pick_fwd_ovl_fixed<_Float16, true>(k, lanes) : pick_fwd_ovl_fixed<_Float16, false>(k, lanes);
        case kBF16: return fused ? pick_fwd_ovl_fixed<__bf16, true>(k, lanes) : pick_fwd_ovl_fixed<__bf16, false>(k, lanes);
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
