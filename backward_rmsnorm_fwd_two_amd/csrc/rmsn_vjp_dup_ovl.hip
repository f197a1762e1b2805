// rmsn_vjp_dup_ovl.hip -- the duplicate-slot VJP, grad-call and
// fused-backward row kernels (rmsn_vjp_dup.hip) for rows that are not a
// whole number of 16-byte vectors: ceil(D / NV) vectors, the last one
// shifted back to end at the row's end (its overlapped leading elements
// left out of the sums and dw), on the smallest whole number of waves that
// holds them, the slots past the row's end duplicating slots inside it.
// The plan takes them where the row fills at least three quarters of the
// slots (D = 500, 511, 2049, 4097, 6001, 8191 ... in 16-bit storage), in
// place of the masked plain loop.  A separate translation unit, so that it
// compiles in parallel with the other instances.
#include "rmsn_kernels.hpp"

namespace rmsn {
namespace {

template <typename T, int K, int MODE, int LANES>
const void* one() {
    constexpr int NV = 16 / static_cast<int>(sizeof(T));
    if constexpr (vjp_dup_ovl_fit(LANES, K, sizeof(T), MODE))
        return reinterpret_cast<const void*>(&vjp_rows<T, NV, K, MODE, true, LANES, PartialRowOut, true, true>);
    return nullptr;
}

template <typename T, int K, int MODE>
const void* pick_lanes(int lanes) {
    switch (lanes) {
        case 64: return one<T, K, MODE, 64>();
        case 128: return one<T, K, MODE, 128>();
        case 192: return one<T, K, MODE, 192>();
        case 256: return one<T, K, MODE, 256>();
        case 320: return one<T, K, MODE, 320>();
        case 384: return one<T, K, MODE, 384>();
        case 448: return one<T, K, MODE, 448>();
        case 512: return one<T, K, MODE, 512>();
        case 576: return one<T, K, MODE, 576>();
        case 640: return one<T, K, MODE, 640>();
        case 704: return one<T, K, MODE, 704>();
        case 768: return one<T, K, MODE, 768>();
        case 832: return one<T, K, MODE, 832>();
        case 896: return one<T, K, MODE, 896>();
        case 960: return one<T, K, MODE, 960>();
        case 1024: return one<T, K, MODE, 1024>();
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

const void* vjp_kernel_dup_ovl(int dt, int nv, int k, int mode, int lanes) {
    switch (mode) {
        case kVjp: return pick_dt<kVjp>(dt, nv, k, lanes);
        case kGrad: return pick_dt<kGrad>(dt, nv, k, lanes);
        case kResGrad: return pick_dt<kResGrad>(dt, nv, k, lanes);
        default: return nullptr;
    }
}

}  // namespace rmsn
