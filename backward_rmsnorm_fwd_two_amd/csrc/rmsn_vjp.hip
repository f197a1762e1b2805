// rmsn_vjp.hip -- instances of the VJP kernels and the dw combine.
#include "rmsn_kernels.hpp"

namespace rmsn {

// dw[j] = sum_b partial[b, j] for b = 0 .. nb-1, in a fixed order, stored
// as TO (fp32, or the weight dtype rounded once).  Block: 256 threads = 4
// column quads (16 columns) x 64 row groups.  Row group g sums rows g,
// g + 64, g + 128, ... (loads issued 8 at a time, added in row order); the
// 16 row groups of a wave are joined with DPP row rotations, a swizzle and a
// bpermute, and the four wave sums through LDS behind one barrier.
constexpr int kCombineGroups = 64;
constexpr int kCombineBatch = 8;

template <typename TO>
__global__ __launch_bounds__(256) void dw_combine(const float* __restrict__ partial,
                                                  TO* __restrict__ dw, int nb, int D) {
    __shared__ float buf[4][16];
    const int cq = threadIdx.x & 3;
    const int rg = threadIdx.x >> 2;
    const int wave = threadIdx.x >> 6;
    const int col0 = blockIdx.x * 16 + cq * 4;
    const bool vec = (D & 3) == 0;
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int b0 = rg; b0 < nb; b0 += kCombineGroups * kCombineBatch) {
        float v[kCombineBatch][4];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
            const int b = b0 + u * kCombineGroups;
            const float* row = partial + (int64_t)b * D;
            if (vec) {
                if (b < nb && col0 < D) {
                    const float4 q = *reinterpret_cast<const float4*>(row + col0);
                    v[u][0] = q.x; v[u][1] = q.y; v[u][2] = q.z; v[u][3] = q.w;
                } else {
                    v[u][0] = v[u][1] = v[u][2] = v[u][3] = 0.0f;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[u][e] = (b < nb && col0 + e < D) ? row[col0 + e] : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[e] += v[u][e];
    }
    // the wave's 16 row groups: lanes l, l+4, l+8, l+12 of each 16-lane row
    // (DPP rotations), then the four rows of the wave
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        s[e] += dpp_move<kDppRowRor4>(s[e]);
        s[e] += dpp_move<kDppRowRor8>(s[e]);
        s[e] = xor16_add(s[e]);
        s[e] = xor32_add(s[e]);
    }
    if ((threadIdx.x & 63) < 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) buf[wave][cq * 4 + e] = s[e];
    }
    __syncthreads();
    if (threadIdx.x < 16) {
        const int col = blockIdx.x * 16 + threadIdx.x;
        const float t = (buf[0][threadIdx.x] + buf[1][threadIdx.x]) + (buf[2][threadIdx.x] + buf[3][threadIdx.x]);
        if (col < D) dw[col] = from_f32<TO>(t);
    }
}

template <typename TO>
__global__ __launch_bounds__(256) void zero_fill(TO* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = from_f32<TO>(0.0f);
}

namespace {

template <typename T, int NV, int MODE>
const void* pick_looped(int jreg) {
    constexpr int OP = 2 + (MODE == kGrad ? 1 : MODE == kResGrad ? 2 : 0);
    switch (jreg) {
        case 0: return reinterpret_cast<const void*>(&rows_batched_vjp<T, NV, OP, RMSN_VJP_BATCH>);
        case 1: return reinterpret_cast<const void*>(&rows_looped<T, NV, OP, 1>);
        case 2: return reinterpret_cast<const void*>(&rows_looped<T, NV, OP, 2>);
        case 4: return reinterpret_cast<const void*>(&rows_looped<T, NV, OP, 4>);
        case 8:
            // at most 32 dw floats per thread (128 VGPRs at 1024 threads)
            if constexpr (NV <= 4) return reinterpret_cast<const void*>(&rows_looped<T, NV, OP, 8>);
            return nullptr;
        default: return nullptr;
    }
}

template <typename T, int NV, int K, int MODE>
const void* pick_rows(bool pipe) {
    if constexpr (K * NV <= kVjpPipeElems && MODE != kGrad) {
        if (pipe) return reinterpret_cast<const void*>(&vjp_rows<T, NV, K, MODE, true>);
    } else {
        if (pipe) return nullptr;
    }
    return reinterpret_cast<const void*>(&vjp_rows<T, NV, K, MODE, false>);
}

template <typename T, int NV, int MODE>
const void* pick_vjp(int k, int jreg, bool pipe) {
    switch (k) {
        case -1: return pipe ? nullptr : pick_looped<T, NV, MODE>(jreg);
        case 1: return pick_rows<T, NV, 1, MODE>(pipe);
        case 2: return pick_rows<T, NV, 2, MODE>(pipe);
        case 4: return pick_rows<T, NV, 4, MODE>(pipe);
        case 8: return pick_rows<T, NV, 8, MODE>(pipe);
        default: return nullptr;
    }
}

template <typename T, int MODE>
const void* pick_vjp_nv(int nv, int k, int jreg, bool pipe) {
    switch (nv) {
        case 1: return pick_vjp<T, 1, MODE>(k, jreg, pipe);
        case 2: return pick_vjp<T, 2, MODE>(k, jreg, pipe);
        case 4: return pick_vjp<T, 4, MODE>(k, jreg, pipe);
        case 8:
            if constexpr (sizeof(T) == 2) return pick_vjp<T, 8, MODE>(k, jreg, pipe);
            return nullptr;
        default: return nullptr;
    }
}

template <int MODE>
const void* pick_vjp_dt(int dt, int nv, int k, int jreg, bool pipe) {
    switch (dt) {
        case kF32: return pick_vjp_nv<float, MODE>(nv, k, jreg, pipe);
        case kF16: return pick_vjp_nv<_Float16, MODE>(nv, k, jreg, pipe);
        case kBF16: return pick_vjp_nv<__bf16, MODE>(nv, k, jreg, pipe);
        default: return nullptr;
    }
}

}  // namespace

const void* vjp_kernel(int dt, int nv, int k, int mode, int jreg, bool pipe) {
    switch (mode) {
        case kVjp: return pick_vjp_dt<kVjp>(dt, nv, k, jreg, pipe);
        case kGrad: return pick_vjp_dt<kGrad>(dt, nv, k, jreg, pipe);
        case kResGrad: return pick_vjp_dt<kResGrad>(dt, nv, k, jreg, pipe);
        default: return nullptr;
    }
}

const void* dw_combine_kernel(int dw_dt) {
    switch (dw_dt) {
        case kF32: return reinterpret_cast<const void*>(&dw_combine<float>);
        case kF16: return reinterpret_cast<const void*>(&dw_combine<_Float16>);
        case kBF16: return reinterpret_cast<const void*>(&dw_combine<__bf16>);
        default: return nullptr;
    }
}

const void* zero_kernel(int dw_dt) {
    switch (dw_dt) {
        case kF32: return reinterpret_cast<const void*>(&zero_fill<float>);
        case kF16: return reinterpret_cast<const void*>(&zero_fill<_Float16>);
        case kBF16: return reinterpret_cast<const void*>(&zero_fill<__bf16>);
        default: return nullptr;
    }
}

}  // namespace rmsn
