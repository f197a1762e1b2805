// rmsn_device.hpp -- gfx950 device helpers shared by the RMSNorm kernels:
// storage-type conversion, vector loads/stores, wave64 DPP / swizzle / bpermute
// reductions and the LDS-only workgroup barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmsn {

// ----------------------------------------------------------------- dtypes
// fp16 / bf16 widen exactly to fp32; narrowing uses the hardware's
// round-to-nearest-even conversions (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32).
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(_Float16 v) { return static_cast<float>(v); }
__device__ __forceinline__ float to_f32(__bf16 v) { return static_cast<float>(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v) { return static_cast<T>(v); }

// fp16: the value is first pinned as an fp32 register (an empty asm operand,
// no instruction), so the compiler cannot fold the fma that produced it and
// this conversion into one mixed-precision instruction that rounds to fp16
// once (v_fma_mixlo_f16 / v_fma_mixhi_f16).  It did so in some instances and
// not in others, and their outputs then differed by one ulp; pinned, every
// kernel rounds the same fp32 value to nearest even.
template <>
__device__ __forceinline__ _Float16 from_f32<_Float16>(float v) {
    __asm__("" : "+v"(v));
    return static_cast<_Float16>(v);
}

// Raw row data as 32-bit words: NV elements moved by one load instruction
// (NV * sizeof(T) bytes; 16 selects global_load_dwordx4).  Keeping the
// words packed (rather than as 16-bit scalars) lets prefetched data stay in
// flight until it is used.
template <typename T, int NV>
struct Raw {
    static constexpr int kBytes = NV * static_cast<int>(sizeof(T));
    static constexpr int kWords = kBytes >= 4 ? kBytes / 4 : 1;
    uint32_t w[kWords];
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Cache policy of the streamed row traffic.  Row tensors are touched once
// per call, so their loads and stores are non-temporal (the "nt" bit: the
// lines are not kept in the caches); only the weight, which every block
// re-reads, keeps the default policy.  On cold data this runs 3-4 % faster
// than the default policy on 64 MiB tensors and 8-12 % faster on tensors
// larger than the last-level cache, with identical outputs.  Setting
// RMSN_NT_ROWS to 0 selects the default policy everywhere.
#ifndef RMSN_NT_ROWS
#define RMSN_NT_ROWS 1
#endif

// STREAM: a row tensor read once; otherwise data that every block re-reads.
// A: the alignment the address is known to have, the element size of the
// tensor.  A row vector may start at any element (a base pointer that is not
// 16-byte aligned, or a row pitch that is not a multiple of 16 bytes); gfx950
// reads and writes 8 and 16 bytes of global memory at any such address with
// the same instructions as at an aligned one.
template <typename V, bool STREAM, int A>
__device__ __forceinline__ V ld_stream(const void* p) {
    typedef V VA __attribute__((aligned(A)));
    const VA* q = static_cast<const VA*>(p);
#if RMSN_NT_ROWS
    if constexpr (STREAM) return __builtin_nontemporal_load(q);
#endif
    return *q;
}

template <typename V, int A>
__device__ __forceinline__ void st_stream(void* p, V v) {
    typedef V VA __attribute__((aligned(A)));
    VA* q = static_cast<VA*>(p);
#if RMSN_NT_ROWS
    __builtin_nontemporal_store(v, q);
#else
    *q = v;
#endif
}

template <typename T, int NV, bool STREAM = true>
__device__ __forceinline__ Raw<T, NV> load_raw(const T* p) {
    constexpr int A = static_cast<int>(sizeof(T));
    Raw<T, NV> r;
    constexpr int B = Raw<T, NV>::kBytes;
    if constexpr (B == 16) {
        const u32x4 v = ld_stream<u32x4, STREAM, A>(p);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else if constexpr (B == 8) {
        const u32x2 v = ld_stream<u32x2, STREAM, A>(p);
        r.w[0] = v.x; r.w[1] = v.y;
    } else if constexpr (B == 4) {
        r.w[0] = ld_stream<uint32_t, STREAM, A>(p);
    } else {
        static_assert(B == 2, "unsupported vector width");
        r.w[0] = ld_stream<uint16_t, STREAM, 2>(p);
    }
    return r;
}

// The weight vector: read by every block, so loaded with the default policy.
template <typename T, int NV>
__device__ __forceinline__ Raw<T, NV> load_w(const T* p) {
    return load_raw<T, NV, false>(p);
}

template <typename T, int NV>
__device__ __forceinline__ void zero_raw(Raw<T, NV>& r) {
#pragma unroll
    for (int i = 0; i < Raw<T, NV>::kWords; ++i) r.w[i] = 0u;
}

// Element e of a raw vector, widened exactly to fp32.
template <typename T, int NV>
__device__ __forceinline__ float elem(const Raw<T, NV>& r, int e) {
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(float, r.w[e]);
    } else {
        const uint32_t word = r.w[e >> 1];
        if constexpr (__is_same(T, _Float16)) {
            const uint16_t h = (e & 1) ? static_cast<uint16_t>(word >> 16)
                                       : static_cast<uint16_t>(word & 0xFFFFu);
            return static_cast<float>(__builtin_bit_cast(_Float16, h));
        } else {
            return __builtin_bit_cast(float, (e & 1) ? (word & 0xFFFF0000u) : (word << 16));
        }
    }
}

// Store N fp32 values as T (round to nearest even) with one instruction;
// used for the streamed outputs (y, normed, new_residual, dx).
template <typename T, int N>
struct alignas(sizeof(T) * N) Pack {
    T v[N];
};

template <typename T, int N>
__device__ __forceinline__ void store_f32(T* p, const float (&v)[N]) {
    constexpr int A = static_cast<int>(sizeof(T));
    Pack<T, N> pk;
#pragma unroll
    for (int i = 0; i < N; ++i) pk.v[i] = from_f32<T>(v[i]);
    constexpr int B = N * static_cast<int>(sizeof(T));
    if constexpr (B == 16) {
        st_stream<u32x4, A>(p, __builtin_bit_cast(u32x4, pk));
    } else if constexpr (B == 8) {
        st_stream<u32x2, A>(p, __builtin_bit_cast(u32x2, pk));
    } else if constexpr (B == 4) {
        st_stream<uint32_t, A>(p, __builtin_bit_cast(uint32_t, pk));
    } else {
        static_assert(B == 2, "unsupported vector width");
        st_stream<uint16_t, 2>(p, __builtin_bit_cast(uint16_t, pk));
    }
}

// Plain (cached) store of N floats; used for the dw partial rows, which the
// combine kernel reads back right away.
template <int N>
__device__ __forceinline__ void store_floats(float* p, const float (&v)[N]) {
    Pack<float, N> pk;
#pragma unroll
    for (int i = 0; i < N; ++i) pk.v[i] = v[i];
    *reinterpret_cast<Pack<float, N>*>(p) = pk;
}

// ------------------------------------------------------- wave reductions
// All-reduce (sum) over aligned groups of `lanes` consecutive lanes of a
// wave64 (lanes = 1, 2, 4, ..., 64, wave-uniform).  Butterfly steps: DPP
// quad permutations for distance 1 and 2, half-row and row mirrors for the
// 8- and 16-lane groups, a ds_swizzle (bit mode, xor 16) to join the two
// rows of each 32-lane half and a ds_bpermute (lane ^ 32) to join the
// halves.  Each step adds the partner's value to the lane's own, so every
// lane of a group ends with the bit-identical sum (fp32 addition commutes)
// in a fixed order.  Every lane of the wave must execute this.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// ds_swizzle offset, bit mode: and_mask 0x1F, or_mask 0, xor_mask 0x10.
constexpr int kSwizzleXor16 = (0x10 << 10) | 0x1F;

__device__ __forceinline__ float xor16_add(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                     kSwizzleXor16));
}

__device__ __forceinline__ float xor32_add(float v) {
    const int src = static_cast<int>((__lane_id() ^ 32u) << 2);
    return v + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v)));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16
constexpr int kDppRowRor4 = 0x124;    // rotate right by 4 within 16
constexpr int kDppRowRor8 = 0x128;    // rotate right by 8 within 16

__device__ __forceinline__ float wave_sum(float v);

__device__ __forceinline__ float group_sum(float v, int lanes) {
    if (lanes >= 64) return wave_sum(v);
    if (lanes > 1) v += dpp_move<kDppXor1>(v);
    if (lanes > 2) v += dpp_move<kDppXor2>(v);
    if (lanes > 4) v += dpp_move<kDppHalfMirror>(v);
    if (lanes > 8) v += dpp_move<kDppMirror>(v);
    if (lanes > 16) v = xor16_add(v);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_move<kDppXor1>(v);
    v += dpp_move<kDppXor2>(v);
    v += dpp_move<kDppHalfMirror>(v);
    v += dpp_move<kDppMirror>(v);
    v = xor16_add(v);
    return xor32_add(v);
}

// Workgroup barrier that orders LDS traffic only: global loads issued
// before it stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum NV values across the `waves` consecutive waves that share one row
// (waves = lanes_per_row / 64 > 1).  Each value must already be a wave
// total.  `red` is LDS of 2 * 16 * NV floats used in alternation (parity),
// so one barrier per call suffices: a wave cannot rewrite a buffer before
// every wave has passed the barrier that follows the reads of it.  FIRST0:
// the block holds one row, whose first wave is wave 0.
template <int NV, bool FIRST0 = false>
__device__ __forceinline__ void cross_wave_sum(float (&v)[NV], int waves, float* red, int parity) {
    const int wave = threadIdx.x >> 6;
    float* buf = red + parity * (16 * NV);
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int n = 0; n < NV; ++n) buf[wave * NV + n] = v[n];
    }
    lds_barrier();
    const int first = FIRST0 ? 0 : (wave / waves) * waves;
#pragma unroll
    for (int n = 0; n < NV; ++n) {
        float s = buf[first * NV + n];
        for (int i = 1; i < waves; ++i) s += buf[(first + i) * NV + n];
        v[n] = s;
    }
}

// Kernel arguments shared by every row kernel (passed by value).
struct RowArgs {
    const void* x;
    const void* res;
    const void* w;
    const void* dy;
    void* y;        // y / normed
    void* newres;   // new_residual
    void* dx;
    float* partial; // [gridDim.x, D] fp32 dw partials (VJP, gridDim.x > 1)
    float* dw;      // [D] fp32
    int64_t rows;
    int32_t D;
    int32_t nvec;   // vectors per row: D / NV (ceil(D / NV), the last overlapped)
    int32_t lanes;  // lanes per row: a power of two, or 64 W for wave rows (lanes fixed at compile time)
    int32_t lshift; // log2(lanes) when lanes is a power of two
    float eps;
    float wb;
};

}  // namespace rmsn
