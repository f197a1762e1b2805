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

// 16-byte loads, one or two vectors per lane: the instance with the lanes
// fixed at compile time, 32 to 1024 lanes per row (measured on cold data:
// forward 0.8-3 % faster at every width, e.g. 8192 x 4096 fp16 24.4 vs 25.3
// us; fused forward 4 % faster up to 256 lanes; at 512 and 1024 lanes the
// fused forward takes it only on few rows, where it is faster, and the
// runtime-width kernel on many -- the plan decides)
template <typename T, int K, bool FUSED>
const void* pick_fixed(int lanes) {
    constexpr int NV = 16 / static_cast<int>(sizeof(T));
    if constexpr (FUSED) {
        switch (lanes) {
            case 32: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 32>);
            case 64: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 64>);
            case 128: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 128>);
            case 256: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 256>);
            case 512: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 512>);
            case 1024: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 1024>);
            default: return nullptr;
        }
    }
    switch (lanes) {
        case 32: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 32>);
        case 64: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 64>);
        case 128: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 128>);
        case 256: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 256>);
        case 512: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 512>);
        case 1024: return reinterpret_cast<const void*>(&fwd_rows<T, NV, K, FUSED, 1024>);
        default: return nullptr;
    }
}

template <typename T, bool FUSED>
const void* pick_fixed_k(int nv, int k, int lanes) {
    if (nv != 16 / static_cast<int>(sizeof(T))) return nullptr;
    switch (k) {
        case 1: return pick_fixed<T, 1, FUSED>(lanes);
        case 2: return pick_fixed<T, 2, FUSED>(lanes);
        default: return nullptr;
    }
}

template <bool FUSED>
const void* pick_fixed_dt(int dt, int nv, int k, int lanes) {
    switch (dt) {
        case kF32: return pick_fixed_k<float, FUSED>(nv, k, lanes);
        case kF16: return pick_fixed_k<_Float16, FUSED>(nv, k, lanes);
        case kBF16: return pick_fixed_k<__bf16, FUSED>(nv, k, lanes);
        default: return nullptr;
    }
}

}  // namespace

const void* fwd_kernel(int dt, int nv, int k, bool fused) {
    return fused ? pick_fwd_dt<true>(dt, nv, k) : pick_fwd_dt<false>(dt, nv, k);
}

const void* fwd_kernel_fixed_lanes(int dt, int nv, int k, bool fused, int lanes) {
    if (wave_rows(lanes)) return fwd_kernel_wave_rows(dt, nv, k, fused, lanes);
    return fused ? pick_fixed_dt<true>(dt, nv, k, lanes) : pick_fixed_dt<false>(dt, nv, k, lanes);
}

}  // namespace rmsn
