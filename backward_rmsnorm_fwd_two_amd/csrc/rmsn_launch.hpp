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
// 256: 512).  The thresholds keep every instance's measured VGPR count
// (ISA metadata) within its budget without spills.
constexpr int max_block_threads(int op, int k, int nv, int itemsize) {
    (void)itemsize;
    const int elems = k * nv;
    // per-element state: forward < fused forward < VJP (two row tensors, the
    // dw accumulators); many-vector instances add per-vector offsets
    const int lim1024 = op == 0 ? 32 : op == 1 ? (k > 4 ? 16 : 32) : (k > 4 ? 8 : 16);
    return elems <= lim1024 ? 1024 : (elems <= 2 * lim1024 ? 512 : 256);
}

inline int dtype_size(int dt) { return dt == kF32 ? 4 : 2; }

// Kernel entry for (op, dtype, NV, K); K == -1 is the streaming kernel.
// Returns nullptr for a combination that is not compiled.
const void* fwd_kernel(int dt, int nv, int k, bool fused);
// mode: 0 VJP, 1 grad call (also writes y), 2 fused backward (adds the
// residual-stream gradient).  jreg (streaming kernel only): vectors of dw
// columns each thread keeps in registers (1, 2, 4, 8), or 0 for rows wider
// than that (the row-batched streaming VJP).
const void* vjp_kernel(int dt, int nv, int k, int mode, int jreg);
// dw_dt: dtype of dw (fp32, or the weight dtype).
const void* dw_combine_kernel(int dw_dt);
// Gated activation silu(x[:, :d]) * x[:, d:2d]: NV elements per load, U
// output vectors per thread per chunk.
const void* gate_kernel(int dt, int nv, int u);
// Its backward (dx = [da | db] for dy of y's shape), same geometry.
const void* gate_vjp_kernel(int dt, int nv, int u);
const void* zero_kernel(int dw_dt);

}  // namespace rmsn
