// rmsn_gate.hip -- the gated activation of the mlxcel issue "Fused
// residual-add RMSNorm and fused RoPE + KV-append decode kernels" (its
// candidate-fusion list): for x = [rows, 2d], y[r, j] = silu(x[r, j]) *
// x[r, d + j], silu(a) = a / (1 + e^-a), in fp32 with one rounding on store.
//
// The backward (silu_gate_vjp_kernel) maps the same vectors: for dy of y's
// shape it writes dx = [da | db] of x's shape, with s = sigmoid(a),
// db = dy * a * s and da = dy * b * s * (1 + a * (1 - s)).
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

// Row-locating arithmetic shared by both kernels.  A chunk's first row
// comes from an fp64 estimate and one correction step (the estimate is off
// by at most one while base < 2^52).
__device__ __forceinline__ void gate_chunk_row(int64_t base, double inv, int64_t nvec, int64_t& row0,
                                               uint32_t& rel0) {
    row0 = static_cast<int64_t>(static_cast<double>(base) * inv);
    int64_t rel = base - row0 * nvec;
    if (rel < 0) { --row0; rel += nvec; }
    if (rel >= nvec) { ++row0; rel -= nvec; }
    rel0 = static_cast<uint32_t>(rel);
}

// The x offset (in elements) of the first half for output vector gc of a
// chunk starting at `base`.  Rows below the chunk's first: loc / nvec, with
// loc < 2 * chunk when nvec < chunk (exact multiply-high), else loc < 2 * nvec
// (a 0/1 compare).  Output index + row * nvec vectors gives the first half.
__device__ __forceinline__ int64_t gate_x_offset(int64_t gc, int64_t base, int64_t row0, uint32_t rel0,
                                                 int64_t nvec, uint32_t recip, bool wide, int nv) {
    const uint32_t loc = rel0 + static_cast<uint32_t>(gc - base);
    const uint32_t dr = wide ? static_cast<uint32_t>(loc >= nvec) : (recip ? __umulhi(loc, recip) : loc);
    return (gc + (row0 + dr) * nvec) * nv;
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
        int64_t row0;
        uint32_t rel0;
        gate_chunk_row(base, inv, nvec, row0, rel0);

        Raw<T, NV> a[U], b[U];
        int64_t g[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            g[k] = base + threadIdx.x + static_cast<int64_t>(k) * bs;
            // past the end: load the last vector (in bounds), store nothing
            const int64_t gc = g[k] < total ? g[k] : total - 1;
            const int64_t ax = gate_x_offset(gc, base, row0, rel0, nvec, recip, wide, NV);
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

// Backward.  dy [rows, d] is indexed like y (flat output vector g); dx
// [rows, 2d] like x.  dx may be x itself: each thread reads a, b and dy of
// its vectors before writing da and db to the same places (so x and dx are
// not __restrict__).
template <typename T, int NV, int U>
__global__ __launch_bounds__(1024) void silu_gate_vjp_kernel(const T* x, const T* __restrict__ dy, T* dx,
                                                            int64_t total, int64_t nvec, uint32_t recip,
                                                            double inv, int64_t nchunks) {
    const uint32_t bs = blockDim.x;
    const int64_t chunk = static_cast<int64_t>(bs) * U;
    const bool wide = nvec >= chunk;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t base = c * chunk;
        int64_t row0;
        uint32_t rel0;
        gate_chunk_row(base, inv, nvec, row0, rel0);
        Raw<T, NV> a[U], b[U], g[U];
        int64_t ax[U], gi[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            gi[k] = base + threadIdx.x + static_cast<int64_t>(k) * bs;
            const int64_t gc = gi[k] < total ? gi[k] : total - 1;
            ax[k] = gate_x_offset(gc, base, row0, rel0, nvec, recip, wide, NV);
            a[k] = load_raw<T, NV>(x + ax[k]);
            b[k] = load_raw<T, NV>(x + ax[k] + nvec * NV);
            g[k] = load_raw<T, NV>(dy + gc * NV);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            if (gi[k] < total) {
                float da[NV], db[NV];
#pragma unroll
                for (int e = 0; e < NV; ++e) {
                    const float av = elem(a[k], e), bv = elem(b[k], e), gv = elem(g[k], e);
                    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-av * kLog2e));
                    db[e] = (gv * av) * sg;
                    da[e] = ((gv * bv) * sg) * __builtin_fmaf(av, 1.0f - sg, 1.0f);
                }
                store_f32<T, NV>(dx + ax[k], da);
                store_f32<T, NV>(dx + ax[k] + nvec * NV, db);
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

namespace {

template <typename T, int NV>
const void* pick_vjp_u(int u) {
    switch (u) {
        case 1: return reinterpret_cast<const void*>(&silu_gate_vjp_kernel<T, NV, 1>);
        case 2: return reinterpret_cast<const void*>(&silu_gate_vjp_kernel<T, NV, 2>);
        case 4: return reinterpret_cast<const void*>(&silu_gate_vjp_kernel<T, NV, 4>);
        case 8: return reinterpret_cast<const void*>(&silu_gate_vjp_kernel<T, NV, 8>);
        default: return nullptr;
    }
}

template <typename T>
const void* pick_vjp_nv(int nv, int u) {
    switch (nv) {
        case 1: return pick_vjp_u<T, 1>(u);
        case 2: return pick_vjp_u<T, 2>(u);
        case 4: return pick_vjp_u<T, 4>(u);
        case 8:
            if constexpr (sizeof(T) == 2) return pick_vjp_u<T, 8>(u);
            return nullptr;
        default: return nullptr;
    }
}

}  // namespace

const void* gate_vjp_kernel(int dt, int nv, int u) {
    switch (dt) {
        case kF32: return pick_vjp_nv<float>(nv, u);
        case kF16: return pick_vjp_nv<_Float16>(nv, u);
        case kBF16: return pick_vjp_nv<__bf16>(nv, u);
        default: return nullptr;
    }
}

}  // namespace rmsn
