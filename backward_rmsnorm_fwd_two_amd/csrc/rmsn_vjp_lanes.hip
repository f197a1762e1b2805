// rmsn_vjp_lanes.hip -- pipelined VJP, grad-call and fused-backward row
// kernels with the lanes per row fixed at compile time, for the common
// geometries: 16-byte loads, one or
// two vectors per lane, 32 to 256 lanes per row (D = 256 .. 4096 in 16-bit
// storage, 128 .. 2048 in fp32, with whole row groups).  With the row width
// known, the per-row reductions compile without branches on it; everything
// else is the generic pipelined kernel.  A separate translation unit, so
// that it compiles in parallel with the other instances.
#include "rmsn_kernels.hpp"

namespace rmsn {
namespace {

template <typename T, int K, int MODE>
const void* pick_lanes(int lanes) {
    constexpr int NV = 16 / static_cast<int>(sizeof(T));
    switch (lanes) {
        case 32: return reinterpret_cast<const void*>(&vjp_rows<T, NV, K, MODE, true, 32>);
        case 64: return reinterpret_cast<const void*>(&vjp_rows<T, NV, K, MODE, true, 64>);
        case 128: return reinterpret_cast<const void*>(&vjp_rows<T, NV, K, MODE, true, 128>);
        case 256: return reinterpret_cast<const void*>(&vjp_rows<T, NV, K, MODE, true, 256>);
        case 512: return reinterpret_cast<const void*>(&vjp_rows<T, NV, K, MODE, true, 512>);
        case 1024:
            if constexpr (K == 1) return reinterpret_cast<const void*>(&vjp_rows<T, NV, K, MODE, true, 1024>);
            return nullptr;
        default: return nullptr;
    }
}

template <typename T, int MODE>
const void* pick_k(int nv, int k, int lanes) {
    if (nv != 16 / static_cast<int>(sizeof(T))) return nullptr;
    switch (k) {
        case 1: return pick_lanes<T, 1, MODE>(lanes);
        case 2: return pick_lanes<T, 2, MODE>(lanes);
        default: return nullptr;
    }
}

template <int MODE>
const void* pick_dt(int dt, int nv, int k, int lanes) {
    switch (dt) {
        case kF32: return pick_k<float, MODE>(nv, k, lanes);
        case kF16: return pick_k<_Float16, MODE>(nv, k, lanes);
        case kBF16: return pick_k<__bf16, MODE>(nv, k, lanes);
        default: return nullptr;
    }
}

}  // namespace

const void* vjp_kernel_fixed_lanes(int dt, int nv, int k, int mode, int lanes) {
    if (wave_rows(lanes) || k == 4) return vjp_kernel_wave_rows(dt, nv, k, mode, lanes);
    switch (mode) {
        case kVjp: return pick_dt<kVjp>(dt, nv, k, lanes);
        case kGrad: return pick_dt<kGrad>(dt, nv, k, lanes);
        case kResGrad: return pick_dt<kResGrad>(dt, nv, k, lanes);
        default: return nullptr;
    }
}

}  // namespace rmsn
