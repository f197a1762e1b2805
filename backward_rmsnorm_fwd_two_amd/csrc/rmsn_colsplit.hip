// rmsn_colsplit.hip -- instances of the column-split backward forms (few
// rows of a wide D): the statistics kernel and the apply kernel per mode.
#include "rmsn_kernels.hpp"

namespace rmsn {
namespace {

template <typename T, int NV>
void pick_cs_nv(int mode, const void** stats_fn, const void** apply_fn) {
    *stats_fn = reinterpret_cast<const void*>(&vjp_cs_stats<T, NV>);
    switch (mode) {
        case kVjp: *apply_fn = reinterpret_cast<const void*>(&vjp_cs_apply<T, NV, kVjp>); break;
        case kGrad: *apply_fn = reinterpret_cast<const void*>(&vjp_cs_apply<T, NV, kGrad>); break;
        case kResGrad: *apply_fn = reinterpret_cast<const void*>(&vjp_cs_apply<T, NV, kResGrad>); break;
        default: *stats_fn = nullptr; *apply_fn = nullptr; break;
    }
}

template <typename T>
void pick_cs(int nv, int mode, const void** stats_fn, const void** apply_fn) {
    switch (nv) {
        case 1: pick_cs_nv<T, 1>(mode, stats_fn, apply_fn); break;
        case 2: pick_cs_nv<T, 2>(mode, stats_fn, apply_fn); break;
        case 4: pick_cs_nv<T, 4>(mode, stats_fn, apply_fn); break;
        case 8:
            if constexpr (sizeof(T) == 2) pick_cs_nv<T, 8>(mode, stats_fn, apply_fn);
            break;
        default: break;
    }
}

}  // namespace

bool vjp_cs_kernels(int dt, int nv, int mode, const void** stats_fn, const void** apply_fn) {
    *stats_fn = nullptr;
    *apply_fn = nullptr;
    switch (dt) {
        case kF32: pick_cs<float>(nv, mode, stats_fn, apply_fn); break;
        case kF16: pick_cs<_Float16>(nv, mode, stats_fn, apply_fn); break;
        case kBF16: pick_cs<__bf16>(nv, mode, stats_fn, apply_fn); break;
        default: break;
    }
    return *stats_fn != nullptr && *apply_fn != nullptr;
}

}  // namespace rmsn
