// rmsn_kernels.hpp -- RMSNorm forward, fused add+RMSNorm and VJP kernels
// for gfx950 (wave64, CDNA4).  All arithmetic is fp32; storage is fp32, fp16
// or bf16, rounded to nearest-even once on store.
//
// Row geometry (register-resident kernels): `lanes` consecutive threads own
// one row; lane l holds vectors v = k * lanes + l (k < K) of NV elements,
// i.e. columns [v * NV, v * NV + NV).  A block of blockDim.x threads works on
// blockDim.x / lanes rows at a time and strides over row groups with the
// grid.  Row sums reduce within the lane group by DPP / swizzle / bpermute; when
// a row spans several waves (lanes > 64) the wave totals meet in LDS.
//
// The streaming kernel (rows_looped) serves any D: one block per row, two
// passes over the row (sums, then outputs), re-reading the row.
//
// In place: an output may be the very buffer of a row input (y over x, dx
// over dy, new_residual over residual, ...).  Every kernel reads all inputs
// of an element before it writes that element's outputs, from the same
// thread, and the first pass of rows_looped writes nothing; row pointers
// are therefore not declared __restrict__.
#pragma once

#include "rmsn_device.hpp"
#include "rmsn_launch.hpp"

// Row groups whose loads are issued together per loop iteration (more
// bytes in flight per wave without loop-carried registers).
#ifndef RMSN_UNROLL
#define RMSN_UNROLL 1
#endif

namespace rmsn {

// Per-lane column bookkeeping shared by the register-resident kernels.
// A lane's vector k covers columns [v * NV, v * NV + NV), v = k * lanes +
// lane; vectors at or past nvec are masked.  Loads are issued
// unconditionally from a clamped (always valid) offset so that every load
// of a row is in flight at once; masked data is zeroed after arrival.
//
// Overlapped last vector (second constructor): a row of D elements that is
// not a whole number of NV-element vectors is covered by nvec = ceil(D / NV)
// vectors, the last one shifted back to end at the row's end (columns
// [D - NV, D)).  Its first skip elements are also the previous vector's
// last ones: they take no part in the row sums or in dw, and the outputs
// stored for them are the very values the previous vector stores (same
// inputs, same arithmetic).  skip is 0 everywhere else, and a compile-time 0
// with the first constructor.
template <int K>
struct Cols {
    int64_t off[K];
    bool ok[K];
    int skip[K];
    __device__ __forceinline__ Cols(int lanes, int lane, int nvec, int nv) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int v = k * lanes + lane;
            ok[k] = v < nvec;
            off[k] = ok[k] ? (int64_t)v * nv : 0;
            skip[k] = 0;
        }
    }
    __device__ __forceinline__ Cols(int lanes, int lane, int nvec, int nv, int64_t D) {
        const int64_t last = D - nv;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int v = k * lanes + lane;
            const int64_t o = (int64_t)v * nv;
            ok[k] = v < nvec;
            off[k] = ok[k] ? (o < last ? o : last) : 0;
            skip[k] = ok[k] && o > last ? static_cast<int>(o - last) : 0;
        }
    }
};

// The column bookkeeping of a kernel: OVL selects the overlapped last vector.
template <int K, bool OVL>
__device__ __forceinline__ Cols<K> make_cols(int lanes, int lane, int nvec, int nv, int64_t D) {
    if constexpr (OVL) return Cols<K>(lanes, lane, nvec, nv, D);
    return Cols<K>(lanes, lane, nvec, nv);
}

// Duplicate slots: a vector slot past the row's end (v >= nvec; the plan
// keeps lanes * K <= 2 nvec) takes the columns of vector v - nvec, which
// another slot owns (with OVL, the last vector's shifted columns).  It loads
// the same data and the same gain, and stores the very values the owner
// stores; only the row sums and dw leave it out (ok[k] false).  Past 2 nvec
// slots (never planned) it would take the row's last vector, still inside
// the row.
template <int K, bool OVL>
__device__ __forceinline__ Cols<K> make_dup_cols(int lanes, int lane, int nvec, int nv, int64_t D) {
    Cols<K> c = make_cols<K, OVL>(lanes, lane, nvec, nv, D);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int v = k * lanes + lane;
        const int owner = v - nvec < nvec ? v - nvec : nvec - 1;
        int64_t o = (int64_t)owner * nv;
        if (OVL && o > D - nv) o = D - nv;
        if (!c.ok[k]) c.off[k] = o;
    }
    return c;
}

// A finished dw vector into the block's partial row: an overlapped last
// vector stores only its own columns (the previous vector's lane stores the
// others).
template <class DwOut, int NV>
__device__ __forceinline__ void store_dw(float* out, const float (&v)[NV], bool vec_ok, int skip) {
    if (skip > 0) {
#pragma unroll
        for (int e = 0; e < NV; ++e)
            if (e >= skip) out[e] = v[e];
    } else {
        DwOut::template store<NV>(out, v, vec_ok);
    }
}

template <typename T, int NV, int K>
__device__ __forceinline__ void issue_row(const T* p, int64_t base, const Cols<K>& c,
                                          Raw<T, NV> (&dst)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) dst[k] = load_raw<T, NV>(p + base + c.off[k]);
}

template <typename T, int NV, int K>
__device__ __forceinline__ void issue_w(const T* w, const Cols<K>& c, Raw<T, NV> (&dst)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) dst[k] = load_w<T, NV>(w + c.off[k]);
}

template <typename T, int NV, int K>
__device__ __forceinline__ void mask_cols(const Cols<K>& c, Raw<T, NV> (&d)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int i = 0; i < Raw<T, NV>::kWords; ++i) d[k].w[i] = c.ok[k] ? d[k].w[i] : 0u;
}

// A thread's row slot in its block and its lane in the row.  Power-of-two
// lane counts split threadIdx.x with a mask and a shift (lshift = log2 of
// the lanes, from the arguments when LANES is 0); a wave-row instance
// (LANES = 64 W, W not a power of two) divides by the constant LANES.
struct RowSlot {
    int lane;
    int slot;
    int nslots;
};

template <int LANES>
__device__ __forceinline__ RowSlot row_slot(int lshift_arg) {
    RowSlot r;
    if constexpr (wave_rows(LANES)) {
        r.slot = static_cast<int>(threadIdx.x) / LANES;
        r.lane = static_cast<int>(threadIdx.x) - r.slot * LANES;
        r.nslots = static_cast<int>(blockDim.x) / LANES;
    } else {
        constexpr int kShift = LANES >= 1024 ? 10 : LANES >= 512 ? 9 : LANES >= 256 ? 8 : LANES >= 128 ? 7
                             : LANES >= 64 ? 6 : LANES >= 32 ? 5 : LANES >= 16 ? 4 : LANES >= 8 ? 3
                             : LANES >= 4 ? 2 : LANES >= 2 ? 1 : 0;
        const int lshift = LANES > 0 ? kShift : lshift_arg;
        r.lane = static_cast<int>(threadIdx.x) & ((1 << lshift) - 1);
        r.slot = static_cast<int>(threadIdx.x) >> lshift;
        r.nslots = static_cast<int>(blockDim.x) >> lshift;
    }
    return r;
}

// ------------------------------------------------------------ forward
// y = x * rsqrt(mean(x^2) + eps) * (wb + w)   (FUSED: x := x + residual,
// which is also stored rounded as new_residual; the unrounded fp32 sum is
// what is normalised).  Every load of a row group is issued before the
// first use; latency is hidden by the other waves resident on the CU.
template <typename T, int NV, int K, bool FUSED>
struct FwdRow {
    Raw<T, NV> x[K];
    Raw<T, NV> r[K];
};

template <typename T, int NV, int K, bool FUSED>
__device__ __forceinline__ void fwd_issue(const RowArgs& a, int64_t row0, int slot, const Cols<K>& c,
                                          FwdRow<T, NV, K, FUSED>& d) {
    const int64_t row = row0 + slot;
    const int64_t base = row < a.rows ? row * a.D : 0;
    issue_row<T, NV, K>(static_cast<const T*>(a.x), base, c, d.x);
    if constexpr (FUSED) issue_row<T, NV, K>(static_cast<const T*>(a.res), base, c, d.r);
}

template <typename T, int NV, int K, bool FUSED, bool OVL = false>
__device__ __forceinline__ void fwd_process(const RowArgs& a, int64_t row0, int slot, int lanes,
                                            const Cols<K>& c, const float (&g)[K][NV],
                                            FwdRow<T, NV, K, FUSED>& d, float* red, int& parity) {
    const int64_t row = row0 + slot;
    const bool rok = row < a.rows;
    const int64_t base = row * a.D;
    mask_cols<T, NV, K>(c, d.x);
    if constexpr (FUSED) mask_cols<T, NV, K>(c, d.r);

    float h[K][NV];
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
#pragma unroll
        for (int e = 0; e < NV; ++e) {
            float hv = elem(d.x[k], e);
            if constexpr (FUSED) hv += elem(d.r[k], e);
            h[k][e] = hv;
            const float hs = !OVL || e >= c.skip[k] ? hv : 0.0f;
            ss = __builtin_fmaf(hs, hs, ss);
        }
    }
    // new_residual goes out before the row reduction -- except with an
    // overlapped last vector: there two lanes, possibly in different waves,
    // read the overlapped elements, and new_residual may be stored over x or
    // residual, so it waits until the reduction has seen every wave's loads
    // complete
    T* newres = static_cast<T*>(a.newres);
    if constexpr (FUSED && !OVL) {
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (rok && c.ok[k]) store_f32<T, NV>(newres + base + c.off[k], h[k]);
    }

    ss = group_sum(ss, lanes < 64 ? lanes : 64);
    if (lanes > 64) {
        float t[1] = {ss};
        cross_wave_sum<1>(t, lanes >> 6, red, parity);
        ss = t[0];
        parity ^= 1;
    }
    const float r = rsqrtf(ss / static_cast<float>(a.D) + a.eps);
    if constexpr (FUSED && OVL) {
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (rok && c.ok[k]) store_f32<T, NV>(newres + base + c.off[k], h[k]);
    }

    T* y = static_cast<T*>(a.y);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (rok && c.ok[k]) {
            float o[NV];
#pragma unroll
            for (int e = 0; e < NV; ++e) o[e] = h[k][e] * r * g[k][e];
            store_f32<T, NV>(y + base + c.off[k], o);
        }
    }
}

// LANES > 0: the lanes per row fixed at compile time (instances for the
// common geometries), so the row reduction compiles without branches on the
// row width; 0: taken from the arguments.
// OVL: rows that are not a whole number of vectors, the last vector
// overlapped.
template <typename T, int NV, int K, bool FUSED, int LANES = 0, bool OVL = false>
__global__ __launch_bounds__(max_block_threads(FUSED ? 1 : 0, K, NV, sizeof(T))) void fwd_rows(RowArgs a) {
    static_assert(LANES == 0 || ((LANES & (LANES - 1)) == 0 && LANES <= 1024) || wave_rows_supported(LANES),
                  "lanes: a power of two or a supported whole number of waves");
    __shared__ float red[2 * 16];
    const int lanes = LANES > 0 ? LANES : a.lanes;
    const RowSlot rs = row_slot<LANES>(a.lshift);
    const int lane = rs.lane;
    const int slot = rs.slot;
    const int nslots = rs.nslots;
    const Cols<K> c = make_cols<K, OVL>(lanes, lane, a.nvec, NV, a.D);
    const int64_t step = (int64_t)gridDim.x * nslots;
    int64_t row0 = (int64_t)blockIdx.x * nslots;
    if (row0 >= a.rows) return;  // whole block

    // First iteration: the row loads go out before the gain's, so the two
    // latencies overlap.  Row groups past the end load a clamped (valid)
    // group and are not processed.
    constexpr int U = RMSN_UNROLL;
    int parity = 0;
    float g[K][NV];
    {
        FwdRow<T, NV, K, FUSED> d[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = row0 + u * step;
            fwd_issue<T, NV, K, FUSED>(a, r < a.rows ? r : row0, slot, c, d[u]);
        }
        Raw<T, NV> pw[K];
        issue_w<T, NV, K>(static_cast<const T*>(a.w), c, pw);
        mask_cols<T, NV, K>(c, pw);
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int e = 0; e < NV; ++e) g[k][e] = a.wb + elem(pw[k], e);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (row0 + u * step < a.rows)
                fwd_process<T, NV, K, FUSED, OVL>(a, row0 + u * step, slot, lanes, c, g, d[u], red, parity);
    }
    for (row0 += U * step; row0 < a.rows; row0 += U * step) {
        FwdRow<T, NV, K, FUSED> d[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = row0 + u * step;
            fwd_issue<T, NV, K, FUSED>(a, r < a.rows ? r : row0, slot, c, d[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (row0 + u * step < a.rows)
                fwd_process<T, NV, K, FUSED, OVL>(a, row0 + u * step, slot, lanes, c, g, d[u], red, parity);
    }
}

// ---------------------------------------------------------------- VJP
// dx = r g dy - x r^3 S / D,  S = sum(dy g x)  (kGrad: also y = x r g, the
// grad call's forward output from the same pass; kResGrad: dx plus the
// residual-stream gradient, the backward of the fused add form);  the dw partial over this
// block's rows is accumulated in registers, combined over the block's row
// slots in LDS (fixed tree order), and written to partial[blockIdx.x, :]
// (or to dw when the grid is a single block).  `dyn` LDS: blockDim.x * NV
// floats when the block holds more than one row slot.  The blocks are
// persistent (a bounded grid strides over the row groups, so that dw has a
// bounded number of partial rows); PIPE instances overlap each group's
// loads with the processing of the previous group.
// VJP row kernel modes.
constexpr int kVjp = 0;       // dx, dw
constexpr int kGrad = 1;      // also y = x r g (grad call)
constexpr int kResGrad = 2;   // dx + d_new_residual (backward of the fused add form)

template <typename T, int NV, int K>
struct VjpRow {
    Raw<T, NV> x[K];
    Raw<T, NV> dy[K];
    Raw<T, NV> dr[K];   // d_new_residual (kResGrad only)
};

// WITH_DR: also the d_new_residual row (kResGrad) into d.dr; instances that
// keep one d_new_residual buffer of their own load it with vjp_issue_dr.
template <typename T, int NV, int K, int MODE, bool WITH_DR = true>
__device__ __forceinline__ void vjp_issue(const RowArgs& a, int64_t row0, int slot, const Cols<K>& c,
                                          VjpRow<T, NV, K>& d) {
    const int64_t row = row0 + slot;
    const int64_t base = row < a.rows ? row * a.D : 0;
    issue_row<T, NV, K>(static_cast<const T*>(a.x), base, c, d.x);
    issue_row<T, NV, K>(static_cast<const T*>(a.dy), base, c, d.dy);
    if constexpr (MODE == kResGrad && WITH_DR) issue_row<T, NV, K>(static_cast<const T*>(a.res), base, c, d.dr);
}

template <typename T, int NV, int K>
__device__ __forceinline__ void vjp_issue_dr(const RowArgs& a, int64_t row0, int slot, const Cols<K>& c,
                                             Raw<T, NV> (&dr)[K]) {
    const int64_t row = row0 + slot;
    issue_row<T, NV, K>(static_cast<const T*>(a.res), row < a.rows ? row * a.D : 0, c, dr);
}

// FULL: every vector of the row is in range and every processed row exists
// (the plan selects the pipelined kernel only for rows of exactly lanes * K
// vectors, and its loop passes FULL for every row group but a ragged last
// one), so no element is masked and every store is unconditional -- which
// also keeps the wave's count of outstanding memory operations the same on
// every path (a store skipped on some paths would make later waits for loads
// wait for everything).
// OVL: the row's last vector may be overlapped (Cols).
template <typename T, int NV, int K, int MODE, bool FULL = false, bool ONE_ROW = false, bool OVL = false,
          bool DUP = false>
__device__ __forceinline__ void vjp_process(const RowArgs& a, int64_t row0, int slot, int lanes,
                                            const Cols<K>& c, const float (&g)[K][NV],
                                            float (&acc)[K][NV], VjpRow<T, NV, K>& d,
                                            const Raw<T, NV> (&dr)[K], float* red, int& parity) {
    const int64_t row = row0 + slot;
    const bool rok = FULL || row < a.rows;
    const int64_t base = row * a.D;
    if constexpr (!FULL) {
        mask_cols<T, NV, K>(c, d.x);
        mask_cols<T, NV, K>(c, d.dy);
    }

    float s2[2] = {0.0f, 0.0f};  // sum x^2, sum dy g x
#pragma unroll
    for (int k = 0; k < K; ++k) {
#pragma unroll
        for (int e = 0; e < NV; ++e) {
            if constexpr (DUP) {
                // a duplicate slot adds nothing, nor does an overlapped element
                const bool live = c.ok[k] && (!OVL || e >= c.skip[k]);
                const float xv = live ? elem(d.x[k], e) : 0.0f;
                const float dv = elem(d.dy[k], e);
                s2[0] = __builtin_fmaf(xv, xv, s2[0]);
                s2[1] = __builtin_fmaf(dv * g[k][e], xv, s2[1]);
            } else if constexpr (OVL) {
                const bool live = e >= c.skip[k];  // not an overlapped element
                const float xv = live ? elem(d.x[k], e) : 0.0f;
                const float dg = live ? elem(d.dy[k], e) * g[k][e] : 0.0f;
                s2[0] = __builtin_fmaf(xv, xv, s2[0]);
                s2[1] = __builtin_fmaf(dg, xv, s2[1]);
            } else {
                const float xv = elem(d.x[k], e);
                const float dv = elem(d.dy[k], e);
                s2[0] = __builtin_fmaf(xv, xv, s2[0]);
                s2[1] = __builtin_fmaf(dv * g[k][e], xv, s2[1]);
            }
        }
    }
    if constexpr (K * NV > kVjpPipeElems) {
        // Wide rows (32 elements per lane): the row's raw 16-bit words are
        // pinned (an empty asm operand, no instruction) so that the fp32
        // values widened for the sums above are not kept alive across the
        // row reduction for the output loop below, which widens the words
        // again: that frees the registers the two-buffer pipeline needs.
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int i = 0; i < Raw<T, NV>::kWords; ++i) __asm__("" : "+v"(d.x[k].w[i]), "+v"(d.dy[k].w[i]));
    }
    const int gl = lanes < 64 ? lanes : 64;
    s2[0] = group_sum(s2[0], gl);
    s2[1] = group_sum(s2[1], gl);
    if (lanes > 64) {
        cross_wave_sum<2, ONE_ROW>(s2, lanes >> 6, red, parity);
        parity ^= 1;
    }
    const float inv_d = 1.0f / static_cast<float>(a.D);
    // explicit fma: every instance (VJP, grad call, fused backward, pipelined
    // or not) rounds the row statistic identically, whatever the compiler
    // would contract
    const float r = rsqrtf(__builtin_fmaf(s2[0], inv_d, a.eps));
    const float cc = r * r * r * s2[1] * inv_d;

    if (rok) {
        T* dx = static_cast<T*>(a.dx);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float o[NV];
#pragma unroll
            for (int e = 0; e < NV; ++e) {
                const float xv = elem(d.x[k], e);
                const float dv = elem(d.dy[k], e);
                // fixed evaluation order (explicit fma), so every instance
                // that computes dx rounds it identically
                o[e] = __builtin_fmaf(-xv, cc, (r * g[k][e]) * dv);
                if constexpr (MODE == kResGrad) o[e] += elem(dr[k], e);
                if (!OVL || e >= c.skip[k]) acc[k][e] = __builtin_fmaf(dv * xv, r, acc[k][e]);
            }
            if (FULL || c.ok[k]) store_f32<T, NV>(dx + base + c.off[k], o);
        }
        if constexpr (MODE == kGrad) {
            // grad call: the forward output from the same pass over x
            T* y = static_cast<T*>(a.y);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float o[NV];
#pragma unroll
                for (int e = 0; e < NV; ++e) o[e] = elem(d.x[k], e) * r * g[k][e];
                if (FULL || c.ok[k]) store_f32<T, NV>(y + base + c.off[k], o);
            }
        }
    }
}

// What a VJP block does with its finished dw partial.  The library's policy
// stores it as the block's row of the [gridDim.x, D] partial buffer (or as
// dw itself for a one-block grid) for the separate combine pass; begin and
// end do nothing.  The hook lets a measurement program run the very same
// row kernel with other ways of finishing the reduction (its store serves
// blocks of one row slot; blocks of several slots store their joined row
// directly).
struct PartialRowOut {
    __device__ __forceinline__ static void begin(const RowArgs&) {}
    template <int NV>
    __device__ __forceinline__ static void store(float* out, const float (&v)[NV], bool vec_ok) {
        if (vec_ok) {
            store_floats<NV>(out, v);
        } else {
#pragma unroll
            for (int e = 0; e < NV; ++e) out[e] = v[e];
        }
    }
    __device__ __forceinline__ static void end(const RowArgs&) {}
};

// LANES > 0: the lanes per row are a compile-time constant (pipelined
// instances for the common geometries), so the row reductions compile
// without branches on the row width; 0: taken from the arguments.  OVL:
// rows that are not a whole number of vectors, the last vector overlapped
// (the plain row loop only).  DUP: rows of fewer vectors than lanes x K
// (at least half of them), pipelined and unmasked through duplicate slots
// (make_dup_cols): the slots past the row's end load, compute and store
// the columns another slot owns, and only the row sums leave them out.
template <typename T, int NV, int K, int MODE, bool PIPE = false, int LANES = 0, class DwOut = PartialRowOut,
          bool OVL = false, bool DUP = false>
__global__ __launch_bounds__(!PIPE ? (OVL ? max_block_threads_ovl(2, K, NV, sizeof(T)) : max_block_threads(2, K, NV, sizeof(T)))
                             : wave_rows(LANES) ? wave_rows_block_max(LANES, K * NV)
                             : (LANES > kVjpPipeBlock ? LANES : kVjpPipeBlock)) void vjp_rows(RowArgs a) {
    static_assert(!PIPE || K * NV <= kVjpPipeElems ||
                      (K * NV <= kVjpPipeElemsWide && LANES > 0 && LANES <= kVjpPipeFixedMax),
                  "pipelined instances hold two row groups");
    static_assert(LANES == 0 || (PIPE && (((LANES & (LANES - 1)) == 0 &&
                                           (LANES <= kVjpPipeFixedMax || (LANES == 1024 && K == 1))) ||
                                          wave_rows_supported(LANES))),
                  "fixed lane counts are pipelined: powers of two or supported whole numbers of waves");
    static_assert(!OVL || (!PIPE && LANES == 0) || DUP,
                  "overlapped rows run in the plain row loop or in the duplicate-slot instances");
    static_assert(!DUP || (PIPE && LANES > 0), "duplicate slots run in the pipelined fixed-width instances");
    extern __shared__ float dyn[];
    __shared__ float red[2 * 16 * 2];
    // Instances whose blocks hold exactly one row (the lane count fixes it)
    // never see a ragged group and compile without the masked copy of the
    // processing, which would cost the tightest of them registers, nor with
    // the join of several row slots' dw.
    constexpr bool kOneRow =
        LANES > 0 && (wave_rows(LANES) ? wave_rows_block_max(LANES, K * NV) == LANES : LANES >= kVjpPipeBlock);
    DwOut::begin(a);
    const int lanes = LANES > 0 ? LANES : a.lanes;
    const RowSlot rs = row_slot<LANES>(a.lshift);
    const int lane = rs.lane;
    const int slot = rs.slot;
    const int nslots = rs.nslots;
    const Cols<K> c =
        DUP ? make_dup_cols<K, OVL>(lanes, lane, a.nvec, NV, a.D) : make_cols<K, OVL>(lanes, lane, a.nvec, NV, a.D);
    const int64_t step = (int64_t)gridDim.x * nslots;
    int64_t row0 = (int64_t)blockIdx.x * nslots;

    float acc[K][NV];
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int e = 0; e < NV; ++e) acc[k][e] = 0.0f;

    if (row0 < a.rows) {  // block-uniform
        int parity = 0;
        float g[K][NV];
        if constexpr (PIPE) {
            // Software pipeline over the block's row groups: the loads of
            // group i + 1 are issued before group i is processed, so every
            // wave keeps one group's loads in flight while it reduces,
            // computes and stores the previous one (a persistent block
            // otherwise pays one full memory round trip per row group).  Two
            // register buffers alternate (the loop is unrolled twice): a copy
            // of loaded data would make the wave wait for the prefetch at the
            // end of every iteration.  The gain's loads go out first, so that
            // none of them is still pending when the loop starts.  Every
            // vector slot of a row is in range here (the plan selects this
            // kernel only then) or, in DUP instances, a duplicate of one that
            // is, and every row group but a block's last is full, so the
            // loop's processing masks nothing and stores unconditionally; a
            // ragged last group (rows not a multiple of the row slots) is
            // processed masked on the loop's exit path, after which the
            // block only joins its dw.
            // kDrOwn (the fused backward on rows of 9, 11 or 12 waves x 2 16-bit
            // vectors, a VGPR or two short otherwise, and on the wide rows of
            // four vectors per lane): one d_new_residual buffer, loaded for
            // the next group right after the current group has used it --
            // behind the next group's x / dy loads, so the in-order wait
            // counts need not drain those to reach it.
            constexpr bool kDrOwn =
                MODE == kResGrad &&
                (((LANES == 576 || LANES == 704 || LANES == 768) && K * NV == kVjpPipeElems) ||
                 K * NV > kVjpPipeElems);
            Raw<T, NV> pw[K];
            issue_w<T, NV, K>(static_cast<const T*>(a.w), c, pw);
            VjpRow<T, NV, K> ra, rb;
            Raw<T, NV> drs[K];
            vjp_issue<T, NV, K, MODE, !kDrOwn>(a, row0, slot, c, ra);
            if constexpr (kDrOwn) vjp_issue_dr<T, NV, K>(a, row0, slot, c, drs);
            if constexpr (!DUP) mask_cols<T, NV, K>(c, pw);
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int e = 0; e < NV; ++e) g[k][e] = a.wb + elem(pw[k], e);
            int64_t next = row0 + step;
            for (;;) {  // ra holds group row0
                if (next >= a.rows) {  // the block's last group, possibly ragged
                    if (kOneRow || row0 + nslots <= a.rows)
                        vjp_process<T, NV, K, MODE, true, kOneRow, OVL, DUP>(a, row0, slot, lanes, c, g, acc,
                                                                               ra, kDrOwn ? drs : ra.dr, red, parity);
                    else if constexpr (!kOneRow)
                        vjp_process<T, NV, K, MODE, false, false, OVL, DUP>(a, row0, slot, lanes, c, g, acc, ra,
                                                           kDrOwn ? drs : ra.dr, red, parity);
                    break;
                }
                vjp_issue<T, NV, K, MODE, !kDrOwn>(a, next, slot, c, rb);
                vjp_process<T, NV, K, MODE, true, kOneRow, OVL, DUP>(a, row0, slot, lanes, c, g, acc, ra,
                                                                       kDrOwn ? drs : ra.dr, red, parity);
                if constexpr (kDrOwn) vjp_issue_dr<T, NV, K>(a, next, slot, c, drs);
                row0 = next;
                next += step;
                // rb holds group row0
                if (next >= a.rows) {  // the block's last group, possibly ragged
                    if (kOneRow || row0 + nslots <= a.rows)
                        vjp_process<T, NV, K, MODE, true, kOneRow, OVL, DUP>(a, row0, slot, lanes, c, g, acc,
                                                                               rb, kDrOwn ? drs : rb.dr, red, parity);
                    else if constexpr (!kOneRow)
                        vjp_process<T, NV, K, MODE, false, false, OVL, DUP>(a, row0, slot, lanes, c, g, acc, rb,
                                                           kDrOwn ? drs : rb.dr, red, parity);
                    break;
                }
                vjp_issue<T, NV, K, MODE, !kDrOwn>(a, next, slot, c, ra);
                vjp_process<T, NV, K, MODE, true, kOneRow, OVL, DUP>(a, row0, slot, lanes, c, g, acc, rb,
                                                                       kDrOwn ? drs : rb.dr, red, parity);
                if constexpr (kDrOwn) vjp_issue_dr<T, NV, K>(a, next, slot, c, drs);
                row0 = next;
                next += step;
            }
        } else {
            // one row group in flight: its loads, then (first group only) the
            // gain's, then the group is processed
            {
                VjpRow<T, NV, K> d;
                vjp_issue<T, NV, K, MODE>(a, row0, slot, c, d);
                Raw<T, NV> pw[K];
                issue_w<T, NV, K>(static_cast<const T*>(a.w), c, pw);
                mask_cols<T, NV, K>(c, pw);
#pragma unroll
                for (int k = 0; k < K; ++k)
#pragma unroll
                    for (int e = 0; e < NV; ++e) g[k][e] = a.wb + elem(pw[k], e);
                vjp_process<T, NV, K, MODE, false, false, OVL>(a, row0, slot, lanes, c, g, acc, d, d.dr, red, parity);
            }
            for (row0 += step; row0 < a.rows; row0 += step) {
                VjpRow<T, NV, K> d;
                vjp_issue<T, NV, K, MODE>(a, row0, slot, c, d);
                vjp_process<T, NV, K, MODE, false, false, OVL>(a, row0, slot, lanes, c, g, acc, d, d.dr, red, parity);
            }
        }
    }

    // Join the row slots' accumulators and write this block's dw row (a
    // block without rows writes zeros).  One slot: the lanes store their
    // vectors (through DwOut).  Several: every slot's accumulators go to LDS,
    // then thread t adds columns t, t + blockDim.x, ... of the vector group
    // over the slots in slot order and stores them -- two barriers per
    // vector group whatever the slot count (a pairwise tree took log2(slots)
    // + 2: five rounds at 32 one-vector-group rows per block).
    float* dst = (gridDim.x == 1) ? a.dw : a.partial + (int64_t)blockIdx.x * a.D;
    const bool vec_ok = (reinterpret_cast<uintptr_t>(dst) % (NV * sizeof(float))) == 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (!kOneRow && nslots > 1) {
            float* mine = dyn + (int64_t)threadIdx.x * NV;  // slot * lanes + lane
#pragma unroll
            for (int e = 0; e < NV; ++e) mine[e] = acc[k][e];
            lds_barrier();
            const int cols = lanes * NV;
            for (int j = threadIdx.x; j < cols; j += blockDim.x) {
                float sum = dyn[j];
                for (int sl = 1; sl < nslots; ++sl) sum += dyn[(int64_t)sl * cols + j];
                const int l = j / NV;
                const int e = j - l * NV;
                const int v = k * lanes + l;
                if (v < a.nvec) {
                    const int64_t o = (int64_t)v * NV;
                    if constexpr (OVL) {
                        // the overlapped last vector stores only its own columns
                        const int64_t last = static_cast<int64_t>(a.D) - NV;
                        if (o <= last)
                            dst[o + e] = sum;
                        else if (e >= o - last)
                            dst[last + e] = sum;
                    } else {
                        dst[o + e] = sum;
                    }
                }
            }
            lds_barrier();  // before the next vector group reuses the LDS
        } else if (c.ok[k]) {
            store_dw<DwOut, NV>(dst + c.off[k], acc[k], vec_ok, c.skip[k]);
        }
    }
    DwOut::end(a);
}

// ---------------------------------------------------- streaming kernel
// Any D.  One row per block iteration, threads stride over the row's
// vectors.  OP 0: forward, 1: fused add + forward, 2: VJP, 3: VJP that also
// writes the forward output y (grad call), 4: VJP plus the residual-stream
// gradient (fused backward).  dw (OP >= 2): every thread owns at most J
// vectors of columns (v = threadIdx.x + j * blockDim.x) and sums their dw in
// registers over the block's rows, in row order, writing this block's
// partial row once at the end (rows wider than that take rows_batched_vjp).
// First-pass loads of the two-pass streaming kernels keep the default cache
// policy: the second pass re-reads the row and finds it in L2 / the
// last-level cache (non-temporal first-pass loads measured 15-30 % slower
// at D = 16392..65536: the re-read went back to HBM).
constexpr bool kPass1Stream = false;

// The streaming forward keeps this many vectors per thread in flight: each
// iteration issues the loads of kStreamUnroll vectors (v, v + blockDim.x,
// ...; a lane skips those past the row's end), then consumes them.  With one
// load per iteration a 1024-thread block holds 16 KiB in flight, and a few
// rows of a very wide D (one block per row) ran at 2.8 TB/s.
constexpr int kStreamUnroll = 4;

// Pass 1 of the streaming forward: this thread's share of a row's sum of
// h^2 (h = x, or x + residual for OP 1) in s2[0].
template <typename T, int NV, int OP>
__device__ __forceinline__ void stream_row_sums(const RowArgs& a, int64_t base, float (&s2)[2]) {
    static_assert(OP == 0 || OP == 1, "forward forms");
    const T* x = static_cast<const T*>(a.x);
    const T* res = static_cast<const T*>(a.res);
    constexpr int U = kStreamUnroll;
    const int bd = static_cast<int>(blockDim.x);
    for (int v0 = threadIdx.x; v0 < a.nvec; v0 += U * bd) {
        Raw<T, NV> px[U], pr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * bd;
            if (v < a.nvec) {
                const int64_t off = base + (int64_t)v * NV;
                px[u] = load_raw<T, NV, kPass1Stream>(x + off);
                if constexpr (OP == 1) pr[u] = load_raw<T, NV, kPass1Stream>(res + off);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (v0 + u * bd < a.nvec) {
#pragma unroll
                for (int e = 0; e < NV; ++e) {
                    float hv = elem(px[u], e);
                    if constexpr (OP == 1) hv += elem(pr[u], e);
                    s2[0] = __builtin_fmaf(hv, hv, s2[0]);
                }
            }
        }
    }
}

template <int NV>
__device__ __forceinline__ void block_sum(float (&v)[NV], float* red, int& parity) {
#pragma unroll
    for (int n = 0; n < NV; ++n) v[n] = wave_sum(v[n]);
    if (blockDim.x > 64) {
        cross_wave_sum<NV>(v, blockDim.x >> 6, red, parity);
        parity ^= 1;
    }
}

template <typename T, int NV, int OP, int J = 0>
__global__ __launch_bounds__(1024) void rows_looped(RowArgs a) {
    static_assert(OP < 2 || J > 0, "the streaming VJP keeps dw in registers");
    __shared__ float red[2 * 16 * 2];
    const T* x = static_cast<const T*>(a.x);
    const T* res = static_cast<const T*>(a.res);
    const T* w = static_cast<const T*>(a.w);
    const T* dy = static_cast<const T*>(a.dy);
    T* y = static_cast<T*>(a.y);
    T* newres = static_cast<T*>(a.newres);
    T* dx = static_cast<T*>(a.dx);
    const float inv_d = 1.0f / static_cast<float>(a.D);
    int parity = 0;
    constexpr int JA = J > 0 ? J : 1;
    float acc[JA][NV];
#pragma unroll
    for (int j = 0; j < JA; ++j)
#pragma unroll
        for (int e = 0; e < NV; ++e) acc[j][e] = 0.0f;

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const int64_t base = row * a.D;
        float s2[2] = {0.0f, 0.0f};
        if constexpr (OP >= 2) {
            for (int v = threadIdx.x; v < a.nvec; v += blockDim.x) {
                const int64_t off = base + (int64_t)v * NV;
                const Raw<T, NV> px = load_raw<T, NV, kPass1Stream>(x + off);
                const Raw<T, NV> pd = load_raw<T, NV, kPass1Stream>(dy + off);
                const Raw<T, NV> pw = load_w<T, NV>(w + (int64_t)v * NV);
#pragma unroll
                for (int e = 0; e < NV; ++e) {
                    const float xv = elem(px, e);
                    s2[0] = __builtin_fmaf(xv, xv, s2[0]);
                    s2[1] = __builtin_fmaf(elem(pd, e) * (a.wb + elem(pw, e)), xv, s2[1]);
                }
            }
        } else {
            stream_row_sums<T, NV, OP>(a, base, s2);
        }
        if constexpr (OP >= 2) {
            block_sum<2>(s2, red, parity);
        } else {
            float t[1] = {s2[0]};
            block_sum<1>(t, red, parity);
            s2[0] = t[0];
        }
        const float r = rsqrtf(__builtin_fmaf(s2[0], inv_d, a.eps));
        const float c = r * r * r * s2[1] * inv_d;

        if constexpr (OP >= 2) {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int v = threadIdx.x + j * static_cast<int>(blockDim.x);
                if (v < a.nvec) {
                    const int64_t off = base + (int64_t)v * NV;
                    const Raw<T, NV> px = load_raw<T, NV>(x + off);
                    const Raw<T, NV> pw = load_w<T, NV>(w + (int64_t)v * NV);
                    const Raw<T, NV> pd = load_raw<T, NV>(dy + off);
                    float o[NV];
#pragma unroll
                    for (int e = 0; e < NV; ++e) {
                        const float xv = elem(px, e);
                        const float dv = elem(pd, e);
                        o[e] = __builtin_fmaf(-xv, c, (r * (a.wb + elem(pw, e))) * dv);
                        acc[j][e] += dv * xv * r;
                    }
                    if constexpr (OP == 4) {
                        const Raw<T, NV> pr = load_raw<T, NV>(res + off);
#pragma unroll
                        for (int e = 0; e < NV; ++e) o[e] += elem(pr, e);
                    }
                    store_f32<T, NV>(dx + off, o);
                    if constexpr (OP == 3) {
#pragma unroll
                        for (int e = 0; e < NV; ++e) o[e] = elem(px, e) * r * (a.wb + elem(pw, e));
                        store_f32<T, NV>(y + off, o);
                    }
                }
            }
        } else {
            constexpr int U = kStreamUnroll;
            const int bd = static_cast<int>(blockDim.x);
            for (int v0 = threadIdx.x; v0 < a.nvec; v0 += U * bd) {
                Raw<T, NV> px[U], pr[U], pw[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int v = v0 + u * bd;
                    if (v < a.nvec) {
                        const int64_t off = base + (int64_t)v * NV;
                        px[u] = load_raw<T, NV>(x + off);
                        pw[u] = load_w<T, NV>(w + (int64_t)v * NV);
                        if constexpr (OP == 1) pr[u] = load_raw<T, NV>(res + off);
                    }
                }
                // every output after every load of the iteration: x or
                // residual may be overwritten
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int v = v0 + u * bd;
                    if (v < a.nvec) {
                        const int64_t off = base + (int64_t)v * NV;
                        float h[NV], o[NV];
#pragma unroll
                        for (int e = 0; e < NV; ++e) {
                            h[e] = elem(px[u], e);
                            if constexpr (OP == 1) h[e] += elem(pr[u], e);
                            o[e] = h[e] * r * (a.wb + elem(pw[u], e));
                        }
                        if constexpr (OP == 1) store_f32<T, NV>(newres + off, h);
                        store_f32<T, NV>(y + off, o);
                    }
                }
            }
        }
    }
    if constexpr (OP >= 2) {
        // this block's dw partial row (zeros for a block without rows)
        float* dst = (gridDim.x == 1) ? a.dw : a.partial + (int64_t)blockIdx.x * a.D;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int v = threadIdx.x + j * static_cast<int>(blockDim.x);
            if (v < a.nvec) {
#pragma unroll
                for (int e = 0; e < NV; ++e) dst[(int64_t)v * NV + e] = acc[j][e];
            }
        }
    }
}

// Streaming VJP for rows wider than the register dw (more than 32 columns
// per thread).  Rows are taken RB at a time (rows row0, row0 + gridDim.x,
// ...): the first pass computes each row's statistics (one block-wide
// reduction per row), the second walks the block's columns once for all RB
// rows, so the block's dw partial row is read-modify-written once per RB
// rows instead of once per row.  OP: 2 VJP, 3 grad call, 4 fused backward.
#ifndef RMSN_VJP_BATCH
#define RMSN_VJP_BATCH 8
#endif

template <typename T, int NV, int OP, int RB>
__global__ __launch_bounds__(1024) void rows_batched_vjp(RowArgs a) {
    static_assert(OP >= 2 && OP <= 4, "backward ops only");
    __shared__ float red[2 * 16 * 2];
    const T* x = static_cast<const T*>(a.x);
    const T* res = static_cast<const T*>(a.res);
    const T* w = static_cast<const T*>(a.w);
    const T* dy = static_cast<const T*>(a.dy);
    T* y = static_cast<T*>(a.y);
    T* dx = static_cast<T*>(a.dx);
    float* dst = (gridDim.x == 1) ? a.dw : a.partial + (int64_t)blockIdx.x * a.D;
    const float inv_d = 1.0f / static_cast<float>(a.D);
    const int64_t stride = gridDim.x;
    int parity = 0;
    bool first = true;

    for (int64_t row0 = blockIdx.x; row0 < a.rows; row0 += RB * stride) {
        float rr[RB], cc[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            const int64_t row = row0 + b * stride;
            rr[b] = 0.0f;
            cc[b] = 0.0f;
            if (row < a.rows) {  // block-uniform
                const int64_t base = row * a.D;
                float s2[2] = {0.0f, 0.0f};
                for (int v = threadIdx.x; v < a.nvec; v += blockDim.x) {
                    const int64_t off = base + (int64_t)v * NV;
                    const Raw<T, NV> px = load_raw<T, NV, kPass1Stream>(x + off);
                    const Raw<T, NV> pd = load_raw<T, NV, kPass1Stream>(dy + off);
                    const Raw<T, NV> pw = load_w<T, NV>(w + (int64_t)v * NV);
#pragma unroll
                    for (int e = 0; e < NV; ++e) {
                        const float xv = elem(px, e);
                        s2[0] = __builtin_fmaf(xv, xv, s2[0]);
                        s2[1] = __builtin_fmaf(elem(pd, e) * (a.wb + elem(pw, e)), xv, s2[1]);
                    }
                }
                block_sum<2>(s2, red, parity);
                rr[b] = rsqrtf(__builtin_fmaf(s2[0], inv_d, a.eps));
                cc[b] = rr[b] * rr[b] * rr[b] * s2[1] * inv_d;
            }
        }
        for (int v = threadIdx.x; v < a.nvec; v += blockDim.x) {
            const Raw<T, NV> pw = load_w<T, NV>(w + (int64_t)v * NV);
            float acc[NV];
#pragma unroll
            for (int e = 0; e < NV; ++e) acc[e] = 0.0f;
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const int64_t row = row0 + b * stride;
                if (row < a.rows) {
                    const int64_t off = row * a.D + (int64_t)v * NV;
                    const Raw<T, NV> px = load_raw<T, NV>(x + off);
                    const Raw<T, NV> pd = load_raw<T, NV>(dy + off);
                    float o[NV];
#pragma unroll
                    for (int e = 0; e < NV; ++e) {
                        const float xv = elem(px, e);
                        const float dv = elem(pd, e);
                        o[e] = __builtin_fmaf(-xv, cc[b], (rr[b] * (a.wb + elem(pw, e))) * dv);
                        acc[e] += dv * xv * rr[b];
                    }
                    if constexpr (OP == 4) {
                        const Raw<T, NV> pr = load_raw<T, NV>(res + off);
#pragma unroll
                        for (int e = 0; e < NV; ++e) o[e] += elem(pr, e);
                    }
                    store_f32<T, NV>(dx + off, o);
                    if constexpr (OP == 3) {
#pragma unroll
                        for (int e = 0; e < NV; ++e) o[e] = elem(px, e) * rr[b] * (a.wb + elem(pw, e));
                        store_f32<T, NV>(y + off, o);
                    }
                }
            }
            float* dcol = dst + (int64_t)v * NV;
#pragma unroll
            for (int e = 0; e < NV; ++e) dcol[e] = first ? acc[e] : dcol[e] + acc[e];
        }
        first = false;
    }
}

}  // namespace rmsn

namespace rmsn {

// ------------------------------------------- column-split backward forms
// For few rows of a wide D, where one block per row (or per pair of rows)
// leaves CUs idle.  Two kernels:
//   vjp_cs_stats  one block per (column slice, row): the slice's partial
//                 sums (sum x^2, sum dy g x) into stats[row, slice, 2];
//   vjp_cs_apply  one block per (column tile, row chunk): every row's r and
//                 c from its slices' partials (added in a fixed order, so
//                 every block derives the same values), then the tile's
//                 columns walked over the chunk's rows -- dx (y, the
//                 residual-stream gradient) stored, dw summed in registers in
//                 row order and written once per chunk (to dw itself when the
//                 rows form one chunk).
// x and dy are read twice (a slice of a row is 16 KiB, gone from the caches
// by the time the apply pass comes back to it): 5 row passes for the VJP
// against 3, traded for every CU at work.
// (kCsThreads, kCsStatVecs and kCsMaxChunk: rmsn_launch.hpp)
constexpr int kCsRowUnroll = 4;   // rows whose loads the apply pass issues together

template <typename T, int NV>
__global__ __launch_bounds__(kCsThreads) void vjp_cs_stats(RowArgs a, float* stats, int slices) {
    __shared__ float red[2 * 16 * 2];
    const T* x = static_cast<const T*>(a.x);
    const T* dy = static_cast<const T*>(a.dy);
    const T* w = static_cast<const T*>(a.w);
    const int64_t row = blockIdx.y;
    const int v0 = static_cast<int>(blockIdx.x) * (kCsThreads * kCsStatVecs) + static_cast<int>(threadIdx.x);
    const int64_t base = row * a.D;
    Raw<T, NV> px[kCsStatVecs], pd[kCsStatVecs], pw[kCsStatVecs];
#pragma unroll
    for (int u = 0; u < kCsStatVecs; ++u) {
        const int v = v0 + u * kCsThreads;
        if (v < a.nvec) {
            px[u] = load_raw<T, NV, kPass1Stream>(x + base + (int64_t)v * NV);
            pd[u] = load_raw<T, NV, kPass1Stream>(dy + base + (int64_t)v * NV);
            pw[u] = load_w<T, NV>(w + (int64_t)v * NV);
        }
    }
    float s2[2] = {0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < kCsStatVecs; ++u) {
        if (v0 + u * kCsThreads < a.nvec) {
#pragma unroll
            for (int e = 0; e < NV; ++e) {
                const float xv = elem(px[u], e);
                s2[0] = __builtin_fmaf(xv, xv, s2[0]);
                s2[1] = __builtin_fmaf(elem(pd[u], e) * (a.wb + elem(pw[u], e)), xv, s2[1]);
            }
        }
    }
    int parity = 0;
    block_sum<2>(s2, red, parity);
    if (threadIdx.x == 0) {
        float* dst = stats + (row * slices + blockIdx.x) * 2;
        dst[0] = s2[0];
        dst[1] = s2[1];
    }
}

template <typename T, int NV, int MODE>
__global__ __launch_bounds__(kCsThreads) void vjp_cs_apply(RowArgs a, const float* stats, int slices,
                                                           int chunk_rows) {
    __shared__ float rc[2 * kCsMaxChunk];
    const T* x = static_cast<const T*>(a.x);
    const T* dy = static_cast<const T*>(a.dy);
    const T* dr = static_cast<const T*>(a.res);
    const T* w = static_cast<const T*>(a.w);
    T* dx = static_cast<T*>(a.dx);
    T* y = static_cast<T*>(a.y);
    const int64_t r0 = (int64_t)blockIdx.y * chunk_rows;
    const int nrows = static_cast<int>(a.rows - r0 < chunk_rows ? a.rows - r0 : chunk_rows);
    const float inv_d = 1.0f / static_cast<float>(a.D);

    // r and c of the chunk's rows: wave i takes rows i, i + 4, ...; lane l
    // adds slices l, l + 64, ... in order, then the wave's fixed tree
    const int wave = static_cast<int>(threadIdx.x) >> 6;
    const int lane = static_cast<int>(threadIdx.x) & 63;
    for (int i = wave; i < nrows; i += kCsThreads / 64) {
        const float* st = stats + (r0 + i) * slices * 2;
        float s0 = 0.0f, s1 = 0.0f;
        for (int sl = lane; sl < slices; sl += 64) {
            s0 += st[2 * sl];
            s1 += st[2 * sl + 1];
        }
        s0 = wave_sum(s0);
        s1 = wave_sum(s1);
        if (lane == 0) {
            // explicit fma: the same rounding as the other backward kernels
            const float r = rsqrtf(__builtin_fmaf(s0, inv_d, a.eps));
            rc[2 * i] = r;
            rc[2 * i + 1] = r * r * r * s1 * inv_d;
        }
    }
    lds_barrier();

    const int v = static_cast<int>(blockIdx.x) * kCsThreads + static_cast<int>(threadIdx.x);
    if (v >= a.nvec) return;  // no barrier follows
    const int64_t col = (int64_t)v * NV;
    const Raw<T, NV> pw = load_w<T, NV>(w + col);
    float g[NV], acc[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) {
        g[e] = a.wb + elem(pw, e);
        acc[e] = 0.0f;
    }
    for (int i0 = 0; i0 < nrows; i0 += kCsRowUnroll) {
        // the loads of kCsRowUnroll rows before their first store (an
        // output may be the very buffer of an input); rows past the chunk
        // are skipped (uniform across the block)
        Raw<T, NV> px[kCsRowUnroll], pd[kCsRowUnroll], pr[kCsRowUnroll];
#pragma unroll
        for (int u = 0; u < kCsRowUnroll; ++u) {
            if (i0 + u < nrows) {
                const int64_t off = (r0 + i0 + u) * a.D + col;
                px[u] = load_raw<T, NV>(x + off);
                pd[u] = load_raw<T, NV>(dy + off);
                if constexpr (MODE == kResGrad) pr[u] = load_raw<T, NV>(dr + off);
            }
        }
#pragma unroll
        for (int u = 0; u < kCsRowUnroll; ++u) {
            const int i = i0 + u;
            if (i < nrows) {
                const float r = rc[2 * i];
                const float cc = rc[2 * i + 1];
                const int64_t off = (r0 + i) * a.D + col;
                float o[NV];
#pragma unroll
                for (int e = 0; e < NV; ++e) {
                    const float xv = elem(px[u], e);
                    const float dv = elem(pd[u], e);
                    o[e] = __builtin_fmaf(-xv, cc, (r * g[e]) * dv);
                    if constexpr (MODE == kResGrad) o[e] += elem(pr[u], e);
                    acc[e] = __builtin_fmaf(dv * xv, r, acc[e]);
                }
                store_f32<T, NV>(dx + off, o);
                if constexpr (MODE == kGrad) {
#pragma unroll
                    for (int e = 0; e < NV; ++e) o[e] = elem(px[u], e) * r * g[e];
                    store_f32<T, NV>(y + off, o);
                }
            }
        }
    }
    float* dst = (gridDim.y == 1 ? a.dw : a.partial + (int64_t)blockIdx.y * a.D) + col;
#pragma unroll
    for (int e = 0; e < NV; ++e) dst[e] = acc[e];
}

}  // namespace rmsn
