// rmsn_gate.hip -- the gated activation of the mlxcel issue "Fused
// residual-add RMSNorm and fused RoPE + KV-append decode kernels" (its
// candidate-fusion list): for x = [rows, 2d], y[r, j] = silu(x[r, j]) *
// x[r, d + j], silu(a) = a / (1 + e^-a), in fp32 with one rounding on store.
//
// Pure streaming work (two reads, one write per output vector), so the
// kernel is laid out for HBM: the output is treated as one flat array of
// `total` vectors of NV elements, each block takes chunks of blockDim * U
// consecutive output vectors (fully coalesced in y, and in both halves of x
// within each row), and every thread issues all of its 2U loads before its
// first use.  Locating a vector's row needs no integer division per vector:
// a chunk's first row comes from one fp64 estimate (corrected to exact),
// and the row offset inside a chunk is either 0/1 (rows at least a chunk
// long) or a multiply-high by a reciprocal that is exact for the small
// numbers involved.
#include "rmsn_device.hpp"
#include "rmsn_launch.hpp"

namespace rmsn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// silu(a) * b: e^-a as 2^(-a log2 e) (v_exp_f32), the reciprocal with
// v_rcp_f32.  Large positive a gives e = 0 and silu(a) = a exactly; below
// a = -88.7 e overflows to inf and silu(a) is a signed zero (the true value
// is smaller than 6e-37 in magnitude); a = -inf gives NaN (as -inf / inf).
__device__ __forceinline__ float silu_mul(float a, float b) {
    const float e = __builtin_amdgcn_exp2f(-a * kLog2e);
    return (a * __builtin_amdgcn_rcpf(1.0f + e)) * b;
}

// total  = rows * nvec output vectors; nvec = d / NV vectors per half row;
// recip  = ceil(2^32 / nvec) when nvec > 1 (0 when nvec == 1);
// inv    = 1 / nvec in fp64; nchunks = ceil(total / (blockDim * U)).
template <typename T, int NV, int U>
__global__ __launch_bounds__(1024) void silu_gate_kernel(const T* __restrict__ x, T* __restrict__ y,
                                                        int64_t total, int64_t nvec, uint32_t recip,
                                                        double inv, int64_t nchunks) {
    const uint32_t bs = blockDim.x;
    const int64_t chunk = static_cast<int64_t>(bs) * U;
    const bool wide = nvec >= chunk;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t base = c * chunk;
        // first row of the chunk: fp64 estimate, then one correction step
        // (the estimate is off by at most one while base < 2^52)
        int64_t row0 = static_cast<int64_t>(static_cast<double>(base) * inv);
        int64_t rel = base - row0 * nvec;
        if (rel < 0) { --row0; rel += nvec; }
        if (rel >= nvec) { ++row0; rel -= nvec; }
        const uint32_t rel0 = static_cast<uint32_t>(rel);

        Raw<T, NV> a[U], b[U];
        int64_t g[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            g[k] = base + threadIdx.x + static_cast<int64_t>(k) * bs;
            // past the end: load the last vector (in bounds), store nothing
            const int64_t gc = g[k] < total ? g[k] : total - 1;
            const uint32_t loc = rel0 + static_cast<uint32_t>(gc - base);
            // rows below the chunk's first: loc / nvec, with loc < 2 * chunk
            // when nvec < chunk, else loc < 2 * nvec
            const uint32_t dr = wide ? static_cast<uint32_t>(loc >= nvec)
                                     : (recip ? __umulhi(loc, recip) : loc);
            // x offset of the first half: output index + row * nvec vectors
            const int64_t ax = (gc + (row0 + dr) * nvec) * NV;
            a[k] = load_raw<T, NV>(x + ax);
            b[k] = load_raw<T, NV>(x + ax + nvec * NV);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            if (g[k] < total) {
                float o[NV];
#pragma unroll
                for (int e = 0; e < NV; ++e) o[e] = silu_mul(elem(a[k], e), elem(b[k], e));
                store_f32<T, NV>(y + g[k] * NV, o);
            }
        }
    }
}

template <typename T, int NV>
const void* pick_u(int u) {
    switch (u) {
        case 1: return reinterpret_cast<const void*>(&silu_gate_kernel<T, NV, 1>);
        case 2: return reinterpret_cast<const void*>(&silu_gate_kernel<T, NV, 2>);
        case 4: return reinterpret_cast<const void*>(&silu_gate_kernel<T, NV, 4>);
        case 8: return reinterpret_cast<const void*>(&silu_gate_kernel<T, NV, 8>);
        default: return nullptr;
    }
}

template <typename T>
const void* pick_nv(int nv, int u) {
    switch (nv) {
        case 1: return pick_u<T, 1>(u);
        case 2: return pick_u<T, 2>(u);
        case 4: return pick_u<T, 4>(u);
        case 8:
            if constexpr (sizeof(T) == 2) return pick_u<T, 8>(u);
            return nullptr;
        default: return nullptr;
    }
}

}  // namespace

const void* gate_kernel(int dt, int nv, int u) {
    switch (dt) {
        case kF32: return pick_nv<float>(nv, u);
        case kF16: return pick_nv<_Float16>(nv, u);
        case kBF16: return pick_nv<__bf16>(nv, u);
        default: return nullptr;
    }
}

}  // namespace rmsn
