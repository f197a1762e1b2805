// rmsn_launch.hpp -- host-side view of the kernel set: which instances
// exist, how large a block each may take, and the launch helpers that the
// C-ABI layer calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rmsn {

struct RowArgs;

enum Op : int { kOpFwd = 0, kOpFused = 1, kOpVjp = 2, kOpGrad = 3, kOpFusedVjp = 4 };
enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Largest block a register-resident instance may run with.  Per-thread
// state grows with the elements of one row a lane holds (E = K * NV: gain,
// dw accumulators and fp32 temporaries per element, raw row words, and a
// 64-bit offset per vector), so the wide instances are compiled for fewer
// threads and more VGPRs per thread (1024 threads: 128 VGPRs, 512: 256,
// 256: 512).  The thresholds keep every instance's VGPR count (ISA
// metadata) within its budget.  op: 0 forward, 1 fused forward, 2 any VJP
// form.
constexpr int max_block_threads(int op, int k, int nv, int itemsize) {
    (void)itemsize;
    const int elems = k * nv;
    const int lim1024 = op == 0 ? 32 : op == 1 ? (k > 4 ? 16 : 32) : (k > 4 ? 8 : 16);
    return elems <= lim1024 ? 1024 : (elems <= 2 * lim1024 ? 512 : 256);
}

// The instances for rows with an overlapped last vector also hold a skip
// count per vector and the masks built from it: their backward forms are
// compiled for at most 512 threads (256 VGPRs; at 1024 threads the fp32
// fused backward with 16 elements per lane would spill).
constexpr int max_block_threads_ovl(int op, int k, int nv, int itemsize) {
    return op == 2 && max_block_threads(op, k, nv, itemsize) > 512 ? 512 : max_block_threads(op, k, nv, itemsize);
}

// The VJP row kernel also comes software-pipelined (the next row group's
// loads in flight while the current one is processed; two groups of raw data
// live), for instances with at most this many elements per lane; the
// generic (runtime-width) pipelined kernel runs in blocks of at most
// kVjpPipeBlock threads, the fixed-width instances below also in wider
// blocks of one row.  The pipelined kernel serves rows that are exactly
// lanes * K vectors and masks nothing but a block's ragged last row group.
constexpr int kVjpPipeElems = 16;
constexpr int kVjpPipeBlock = 256;
// Instances with the lanes per row fixed at compile time also exist for rows
// of up to this many lanes (a 512-lane row runs pipelined in a 512-thread
// block, one block per CU).
constexpr int kVjpPipeFixedMax = 512;

// Rows of a whole number of waves that is not a power of two (lanes = 64 W,
// W = 3, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15): D = 3072, 4608, 5120, 6144,
// 6656, 7168 ... in 16-bit storage tile such rows exactly, where a
// power-of-two lane count would leave a quarter to a half of its vectors
// masked.  Instances exist with the lanes fixed at compile time, in blocks of
// one or two rows.
constexpr bool wave_rows(int lanes) { return lanes > 64 && (lanes & (lanes - 1)) != 0; }
constexpr bool wave_rows_supported(int lanes) {
    return lanes == 192 || lanes == 320 || lanes == 384 || lanes == 448 || lanes == 576 || lanes == 640 ||
           lanes == 704 || lanes == 768 || lanes == 832 || lanes == 896 || lanes == 960;
}
// Wide 16-bit rows (D = 12288, 14336, 16384) also come pipelined with four
// vectors per lane on 384, 448 or 512 lanes, one row per block: up to this
// many elements per lane, where a block of at most 512 threads leaves the 256
// VGPRs the two register buffers need.
constexpr int kVjpPipeElemsWide = 32;
// Largest block of a pipelined VJP wave-row instance (elems = K * NV): up to
// four rows while they fit 768 threads (the two register buffers need about
// 90-170 VGPRs; 768 threads leave 170, larger blocks would cap below that);
// one row for the wide instances.
constexpr int wave_rows_block_max(int lanes, int elems) {
    return elems > kVjpPipeElems ? lanes : 4 * lanes <= 768 ? 4 * lanes : 2 * lanes <= 768 ? 2 * lanes : lanes;
}
// Pipelined VJP instances of the wave-row family: 16-bit rows with two
// vectors per lane need up to 168 VGPRs, which rows of up to 12 waves leave
// (170) and rows of 13 to 15 waves do not (128); fp32 rows with four vectors
// per lane fit only as one 512-lane row
// per block.  The wide instances exist for 384, 448 and 512 lanes for the
// VJP (mode 0, 243-255 VGPRs, no spills) and for 448 and 512 lanes for the
// grad call (mode 1: 254 VGPRs at 512 lanes, three spilled to scratch at
// 448) and the fused backward (mode 2, one d_new_residual buffer: 9-15
// VGPRs spilled to scratch).  Even spilling, these run D = 14336 and 16384
// 16-bit rows 2-21 % faster than the plain loop on 256 lanes x 8.
constexpr bool vjp_wave_rows_fit(int lanes, int k, int itemsize, int mode) {
    return k * (16 / itemsize) > kVjpPipeElems ? (mode == 0 ? (lanes == 384 || lanes == 448 || lanes == 512)
                                                            : (lanes == 448 || lanes == 512))
           : itemsize == 4 && k == 4                ? lanes == 512
           : k * (16 / itemsize) == kVjpPipeElems && lanes > 640 ? (lanes == 704 || lanes == 768)
                                                    : true;
}

// Duplicate-slot instances (rows that lanes x K does not tile exactly): one
// or two 16-byte vectors per lane on 64 W lanes, W = 1..15, wherever the
// exact instance of that geometry fits its registers.
constexpr bool vjp_dup_fit(int lanes, int k, int itemsize, int mode) {
    return (k == 1 || k == 2) && lanes % 64 == 0 && lanes >= 64 && lanes <= 960 &&
           vjp_wave_rows_fit(lanes, k, itemsize, mode);
}
// The same for rows whose last vector is overlapped (the skip counts and
// their selects take registers): the grad call and the fused backward hold
// 16-bit rows of one vector per lane only, and the fp32 fused backward rows
// of at most 13 waves with two, where the exact instances' budget holds
// them without spills.  So that 16-bit rows of 961..1024 vectors (D = 7681
// .. 8191) need not fall back to the plain loop for those two forms, they
// also come with one vector per lane on 1024 lanes (one row per block, the
// same 128-VGPR budget as the 960-lane instances).
constexpr bool vjp_dup_ovl_fit(int lanes, int k, int itemsize, int mode) {
    return (vjp_dup_fit(lanes, k, itemsize, mode) && (mode == 0 || k * (16 / itemsize) < kVjpPipeElems) &&
            !(itemsize == 4 && mode == 2 && k == 2 && lanes > 832)) ||
           (lanes == 1024 && k == 1 && itemsize == 2 && mode != 0);
}
// Largest block of a pipelined instance with the lanes fixed at compile
// time (its launch bound): wave rows as above; power-of-two lanes one row of
// 256 lanes or more, or up to 256 threads of shorter rows.
constexpr int vjp_pipe_block_max(int lanes, int elems) {
    return wave_rows(lanes) ? wave_rows_block_max(lanes, elems) : (lanes > kVjpPipeBlock ? lanes : kVjpPipeBlock);
}

inline int dtype_size(int dt) { return dt == kF32 ? 4 : 2; }

// Kernel entry for (op, dtype, NV, K); K == -1 is the streaming kernel.
// Returns nullptr for a combination that is not compiled.
const void* fwd_kernel(int dt, int nv, int k, bool fused);
// The register forward kernel with `lanes` fixed at compile time, or nullptr
// where no such instance exists (then fwd_kernel serves).
const void* fwd_kernel_fixed_lanes(int dt, int nv, int k, bool fused, int lanes);
// mode: 0 VJP, 1 grad call (also writes y), 2 fused backward (adds the
// residual-stream gradient).  jreg (streaming kernel only): vectors of dw
// columns each thread keeps in registers (1, 2, 4, 8), or 0 for rows wider
// than that (the row-batched streaming VJP).
// pipe: the software-pipelined register kernel (k > 0, k * nv <=
// kVjpPipeElems, block <= kVjpPipeBlock).
const void* vjp_kernel(int dt, int nv, int k, int mode, int jreg, bool pipe);
// The pipelined VJP kernel with `lanes` fixed at compile time, or nullptr
// where no such instance exists (then vjp_kernel(..., pipe = true) serves).
const void* vjp_kernel_fixed_lanes(int dt, int nv, int k, int mode, int lanes);
// The wave-row instances (lanes = 64 W, W not a power of two), or nullptr.
const void* fwd_kernel_wave_rows(int dt, int nv, int k, bool fused, int lanes);
const void* vjp_kernel_wave_rows(int dt, int nv, int k, int mode, int lanes);
// The duplicate-slot instances (vjp_dup_fit), or nullptr; _ovl: for rows
// whose last vector is overlapped.
const void* vjp_kernel_dup(int dt, int nv, int k, int mode, int lanes);
const void* vjp_kernel_dup_ovl(int dt, int nv, int k, int mode, int lanes);
// Rows that are not a whole number of 16-byte vectors, the last vector
// overlapped (forward, and the backward forms' plain row loop), or nullptr.
const void* fwd_kernel_ovl(int dt, int k, bool fused);
const void* fwd_kernel_ovl_fixed(int dt, int k, bool fused, int lanes);
const void* fwd_kernel_wave_rows_ovl(int dt, int nv, int k, bool fused, int lanes);
const void* vjp_kernel_ovl(int dt, int k, int mode);
// Column-split backward forms: threads per block (both kernels), vectors per
// thread in a statistics slice, rows per chunk of the apply kernel (their r
// and c live in LDS).
constexpr int kCsThreads = 256;
constexpr int kCsStatVecs = 4;
constexpr int kCsMaxChunk = 512;

// The column-split backward forms (few rows of a wide D): the statistics
// and apply kernels for (dt, nv, mode); false where not compiled.
bool vjp_cs_kernels(int dt, int nv, int mode, const void** stats_fn, const void** apply_fn);
// dw_dt: dtype of dw (fp32, or the weight dtype).
const void* dw_combine_kernel(int dw_dt);
// Gated activation silu(x[:, :d]) * x[:, d:2d]: NV elements per load, U
// output vectors per thread per chunk.
const void* gate_kernel(int dt, int nv, int u);
// Its backward (dx = [da | db] for dy of y's shape), same geometry.
const void* gate_vjp_kernel(int dt, int nv, int u);
const void* zero_kernel(int dw_dt);

}  // namespace rmsn
