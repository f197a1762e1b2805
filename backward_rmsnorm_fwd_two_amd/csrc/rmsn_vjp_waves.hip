// rmsn_vjp_waves.hip -- pipelined VJP, grad-call and fused-backward row
// kernels for rows of a whole number of waves that is not a power of two:
// lanes = 64 W, W = 3, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15, one or two 16-byte
// vectors per lane, where the row is exactly lanes * K vectors (D = 1536 ..
// 12288 in 16-bit storage, 768 .. 7680 in fp32; 16-bit rows of 13 to 15 waves
// with two vectors per lane would spill registers); wide 16-bit rows with four
// vectors per lane, one row per block, on 384, 448 or 512 lanes for the VJP
// and 448 or 512 for the grad call and the fused backward (D = 12288, 14336,
// 16384); fp32 rows of 512 lanes x 4 vectors (D = 8192).  The table of which
// exist is vjp_wave_rows_fit.
// A power-of-two lane count would mask a quarter to a half of such a row and
// fall back to the plain loop.  A separate translation unit, so that it
// compiles in parallel with the other instances.
#include "rmsn_kernels.hpp"

namespace rmsn {
namespace {

template <typename T, int K, int MODE, int LANES>
const void* one() {
    constexpr int NV = 16 / static_cast<int>(sizeof(T));
    if constexpr (vjp_wave_rows_fit(LANES, K, sizeof(T), MODE))
        return reinterpret_cast<const void*>(&vjp_rows<T, NV, K, MODE, true, LANES>);
    return nullptr;
}

template <typename T, int K, int MODE>
const void* pick_waves(int lanes) {
    switch (lanes) {
        case 192: return one<T, K, MODE, 192>();
        case 320: return one<T, K, MODE, 320>();
        case 384: return one<T, K, MODE, 384>();
        case 448: return one<T, K, MODE, 448>();
        case 576: return one<T, K, MODE, 576>();
        case 640: return one<T, K, MODE, 640>();
        case 704: return one<T, K, MODE, 704>();
        case 768: return one<T, K, MODE, 768>();
        case 832: return one<T, K, MODE, 832>();
        case 896: return one<T, K, MODE, 896>();
        case 960: return one<T, K, MODE, 960>();
        default: return nullptr;
    }
}

// four vectors per lane, one row per block: wide 16-bit rows and fp32 rows of
// 512 lanes (D = 8192)
template <typename T, int MODE>
const void* pick_wide(int lanes) {
    if constexpr (sizeof(T) == 2) {
        switch (lanes) {
            case 384: return one<T, 4, MODE, 384>();
            case 448: return one<T, 4, MODE, 448>();
            case 512: return one<T, 4, MODE, 512>();
            default: return nullptr;
        }
    } else {
        // fp32 raw data takes twice the registers of 16-bit: only a whole
        // 512-lane row per block (256 VGPRs) holds every form unspilled
        if (lanes == 512) return one<T, 4, MODE, 512>();
        return nullptr;
    }
}

template <typename T, int MODE>
const void* pick_k(int nv, int k, int lanes) {
    if (nv != 16 / static_cast<int>(sizeof(T))) return nullptr;
    switch (k) {
        case 1: return pick_waves<T, 1, MODE>(lanes);
        case 2: return pick_waves<T, 2, MODE>(lanes);
        case 4: return pick_wide<T, MODE>(lanes);
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

const void* vjp_kernel_wave_rows(int dt, int nv, int k, int mode, int lanes) {
    switch (mode) {
        case kVjp: return pick_dt<kVjp>(dt, nv, k, lanes);
        case kGrad: return pick_dt<kGrad>(dt, nv, k, lanes);
        case kResGrad: return pick_dt<kResGrad>(dt, nv, k, lanes);
        default: return nullptr;
    }
}

}  // namespace rmsn
