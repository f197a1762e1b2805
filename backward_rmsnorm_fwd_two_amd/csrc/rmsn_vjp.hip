// rmsn_vjp.hip -- instances of the VJP kernels and the dw combine.
#include "rmsn_kernels.hpp"

namespace rmsn {

// dw[j] = sum_b partial[b, j] for b = 0 .. nb-1, in a fixed order: 16 row
// groups each sum a strided subset, then a fixed LDS tree joins them.
// Block: 256 threads = 16 columns x 16 row groups.
__global__ __launch_bounds__(256) void dw_combine(const float* __restrict__ partial,
                                                  float* __restrict__ dw, int nb, int D) {
    __shared__ float buf[16][17];
    const int cx = threadIdx.x & 15;
    const int ry = threadIdx.x >> 4;
    const int col = blockIdx.x * 16 + cx;
    float s = 0.0f;
    if (col < D) {
        for (int b = ry; b < nb; b += 16) s += partial[(int64_t)b * D + col];
    }
    buf[ry][cx] = s;
    __syncthreads();
    for (int st = 8; st >= 1; st >>= 1) {
        if (ry < st) buf[ry][cx] += buf[ry + st][cx];
        __syncthreads();
    }
    if (ry == 0 && col < D) dw[col] = buf[0][cx];
}

__global__ __launch_bounds__(256) void zero_f32(float* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.0f;
}

namespace {

template <typename T, int NV>
const void* pick_vjp(int k) {
    switch (k) {
        case -1: return reinterpret_cast<const void*>(&rows_looped<T, NV, 2>);
        case 1: return reinterpret_cast<const void*>(&vjp_rows<T, NV, 1>);
        case 2: return reinterpret_cast<const void*>(&vjp_rows<T, NV, 2>);
        case 4: return reinterpret_cast<const void*>(&vjp_rows<T, NV, 4>);
        case 8: return reinterpret_cast<const void*>(&vjp_rows<T, NV, 8>);
        default: return nullptr;
    }
}

template <typename T>
const void* pick_vjp_nv(int nv, int k) {
    switch (nv) {
        case 1: return pick_vjp<T, 1>(k);
        case 2: return pick_vjp<T, 2>(k);
        case 4: return pick_vjp<T, 4>(k);
        case 8:
            if constexpr (sizeof(T) == 2) return pick_vjp<T, 8>(k);
            return nullptr;
        default: return nullptr;
    }
}

}  // namespace

const void* vjp_kernel(int dt, int nv, int k) {
    switch (dt) {
        case kF32: return pick_vjp_nv<float>(nv, k);
        case kF16: return pick_vjp_nv<_Float16>(nv, k);
        case kBF16: return pick_vjp_nv<__bf16>(nv, k);
        default: return nullptr;
    }
}

const void* dw_combine_kernel() { return reinterpret_cast<const void*>(&dw_combine); }
const void* zero_kernel() { return reinterpret_cast<const void*>(&zero_f32); }

}  // namespace rmsn
