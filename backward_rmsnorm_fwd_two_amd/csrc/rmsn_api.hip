// rmsn_api.hip -- the C ABI declared in include/rmsnorm_mi355x.h: argument
// checks, the per-shape kernel plan (load width, threads per row, vectors
// per thread, block, grid) and the launches.  Host code only; the kernels
// live in rmsn_fwd.hip / rmsn_vjp.hip / rmsn_gate.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "rmsn_device.hpp"
#include "rmsn_launch.hpp"
#include "rmsnorm_mi355x.h"

namespace {

using rmsn::RowArgs;

constexpr int kMaxDevices = 64;
constexpr int kMaxPartialRows = 2048;   // bound on dw partial rows (workspace)
// Row data a CU should hold in flight in the wave-row VJP, in units of one
// wave's 16-byte vector of one row tensor (see make_plan).
constexpr int kWaveRowsInFlight = 15;
std::atomic<int> g_cu_count[kMaxDevices];

// Scratch of rmsnorm_vjp_noalloc: its dw partial rows live in this
// file-scope device array (one copy per GPU, held until the process ends)
// instead of a caller workspace.  Host code never passes the array's name to
// a kernel (on the host it is a stand-in, not a device address): the first
// call on a device resolves the device address once, with that device
// current, and every launch takes that pointer.
static __device__ __align__(256) unsigned char scratch[RMSN_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (resolved once per device).
int scratch_ptr(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RMSN_E_HIP;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RMSN_E_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return RMSN_OK;
}

// Compute units of the current device (cached per device; the cache is the
// library's only global state).
int cu_count(int* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return RMSN_E_HIP;
    if (dev < 0 || dev >= kMaxDevices) return RMSN_E_HIP;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return RMSN_E_HIP;
        g_cu_count[dev].store(n, std::memory_order_relaxed);
    }
    *out = n;
    return RMSN_OK;
}

int itemsize(int dt) { return dt == RMSN_F32 ? 4 : 2; }

int next_pow2(int64_t v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

int log2i(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Persistent grid of a backward launch: at most `cap` blocks, and whenever
// there are at least two row groups every block owns at least two, so the dw
// partial rows number at most half the row groups -- never one partial row
// per row, the [rows, D] temporary the MLX pull request "RMSNormVJP backward
// writes a full {n_rows, D} gw_temp intermediate" removes (Proposed changes).
int64_t vjp_grid(int64_t groups, int64_t cap) {
    int64_t g = std::min(groups, cap);
    if (groups > 1) g = std::min(g, (groups + 1) / 2);
    return std::max<int64_t>(g, 1);
}

struct Plan {
    int nv = 1;       // elements per load
    int nvec = 1;     // D / nv
    int k = 1;        // vectors per lane; -1 = streaming kernel
    int lanes = 1;    // threads per row
    int jreg = 0;     // streaming VJP: dw vectors per thread in registers (0: in memory)
    int block = 256;
    int64_t grid = 1;
    size_t shmem = 0;
    bool pipe = false;        // backward forms: the software-pipelined row kernel
    bool fixed_lanes = false; // ... in an instance with the lanes fixed at compile time
    bool ovl = false;         // rows of ceil(D / nv) vectors, the last one overlapped
    bool fwd_generic = false; // forward forms: the runtime-width kernel although a fixed-width one exists
    bool dup = false;         // backward forms: the duplicate-slot instance (lanes * k > nvec)
    // column-split backward (k == -2): statistics slices per row, column
    // tiles, rows per chunk (grid = chunks), workspace bytes of the row
    // statistics (ahead of the dw partial rows)
    int cs_slices = 0;
    int cs_tiles = 0;
    int cs_chunk = 0;
    size_t cs_stats_bytes = 0;
};

// The column-split backward forms for `rows` rows of p->nvec vectors (p->nv
// set): statistics slices of 256 threads x 4 vectors, apply tiles of 256
// vectors, and row chunks -- enough (tiles x chunks) blocks for two per CU,
// unless `chunks` asks for a number.
int plan_colsplit(int64_t rows, int cus, int64_t chunks, Plan* p) {
    if (rows > 65535) return RMSN_E_CONFIG;
    const int64_t per_slice = (int64_t)rmsn::kCsThreads * rmsn::kCsStatVecs;
    const int64_t slices = (p->nvec + per_slice - 1) / per_slice;
    const int64_t tiles = (p->nvec + rmsn::kCsThreads - 1) / rmsn::kCsThreads;
    int64_t rc = chunks;
    if (rc == 0) rc = std::max<int64_t>(1, (2 * (int64_t)cus + tiles - 1) / tiles);
    // at least two rows per chunk whenever there are two: the chunks' dw
    // rows never number one per row (as vjp_grid for the persistent grids)
    rc = std::min(rc, rows > 1 ? (rows + 1) / 2 : rows);
    int64_t chunk = (rows + rc - 1) / rc;
    if (chunk > rmsn::kCsMaxChunk) {
        if (chunks != 0) return RMSN_E_CONFIG;
        chunk = rmsn::kCsMaxChunk;
    }
    rc = (rows + chunk - 1) / chunk;  // every chunk holds at least one row
    if (rc < 1 || rc > 1024) return RMSN_E_CONFIG;
    p->k = -2;
    p->lanes = 0;
    p->block = rmsn::kCsThreads;
    p->grid = rc;
    p->shmem = 0;
    p->pipe = p->fixed_lanes = p->ovl = false;
    p->cs_slices = static_cast<int>(slices);
    p->cs_tiles = static_cast<int>(tiles);
    p->cs_chunk = static_cast<int>(chunk);
    p->cs_stats_bytes = ((static_cast<size_t>(rows) * static_cast<size_t>(slices) * 2 * sizeof(float)) + 255) &
                        ~static_cast<size_t>(255);
    return RMSN_OK;
}

// The kernel plan for one call.  The load width depends on the row length
// only: row vectors are read and written at element alignment, so a base
// pointer that is not 16-byte aligned still gets the widest loads.
// op: RMSN_OP_FWD, RMSN_OP_FUSED, or one of the backward forms RMSN_OP_VJP,
// RMSN_OP_GRAD, RMSN_OP_FUSED_VJP (all planned alike).  ovl_ok: rows that are
// not a whole number of 16-byte vectors may take 16-byte vectors with the
// last one overlapped (register kernels); otherwise narrower loads.
int make_plan(int op, int64_t rows, int64_t D, int dt, const rmsn_config_t* cfg, Plan* p,
              bool ovl_ok = true) {
    const bool vjp = op == RMSN_OP_VJP || op == RMSN_OP_GRAD || op == RMSN_OP_FUSED_VJP;
    const int budget_op = vjp ? 2 : op;
    const int s = itemsize(dt);
    int cus = 0;
    int st = cu_count(&cus);
    if (st != RMSN_OK) return st;

    // load width
    int vb = 0;
    bool ovl = false;
    if (cfg && cfg->vecs_per_lane == -2) {
        if (!vjp || cfg->lanes_per_row != 0 || (cfg->block_threads != 0 && cfg->block_threads != rmsn::kCsThreads))
            return RMSN_E_CONFIG;
        ovl_ok = false;  // whole vectors only
    }
    if (cfg && cfg->vec_bytes) {
        vb = cfg->vec_bytes;
        if (vb < s || vb > 16 || !is_pow2(vb)) return RMSN_E_CONFIG;
        if ((D * s) % vb != 0) {
            // 16-byte vectors on a row that is not a whole number of them:
            // the last vector overlapped
            if (vb != 16 || D * s < 16 || !ovl_ok) return RMSN_E_CONFIG;
            ovl = true;
        }
    } else {
        for (int c = 16; c >= s; c >>= 1) {
            if ((D * s) % c == 0) { vb = c; break; }
        }
        if (vb == 0) vb = s;
        // A row that is not a whole number of 16-byte vectors (D = 257, 500,
        // 511, 513 in 16-bit storage) takes 16-byte vectors with the last
        // one shifted back to end at the row's end, rather than loads of the
        // largest width dividing the row (2 bytes for an odd D).
        if (vb < 16 && ovl_ok && D * s > 16) {
            vb = 16;
            ovl = true;
        }
    }
    p->nv = vb / s;
    p->nvec = static_cast<int>(ovl ? (D + p->nv - 1) / p->nv : D / p->nv);
    p->ovl = ovl;

    const int req_k = cfg ? cfg->vecs_per_lane : 0;
    const int req_l = cfg ? cfg->lanes_per_row : 0;
    const int req_b = cfg ? cfg->block_threads : 0;
    if (req_k == -2) return plan_colsplit(rows, cus, cfg->num_blocks, p);
    // Few rows (no more than the CUs) of 64..768 whole 16-byte vectors, a
    // multiple of 64 (D = 512..6144 in 16-bit storage; decode batches): the
    // forward forms take one vector per lane on as many lanes as the row has
    // vectors (a fixed-width power-of-two or wave-row instance), one row per
    // block.  There latency, not bandwidth, decides: 32 calls chained
    // through a residual stream and replayed from one graph, bf16, 1..256
    // rows, per call: forward D = 2560 2.47 -> 1.96 us, 3584 2.57 -> 1.99,
    // 4608 2.51 -> 2.08, 6144 2.22 -> 2.14; fused forward D = 2048 at 8 rows
    // 2.71 -> 2.21, 4096 2.31 -> 2.12, 4608 2.38 -> 2.24, 6144 2.43 -> 2.31.
    // At 1024 vectors the two layouts ran alike, and at 512..4096 rows too
    // (warm).  Only when the whole geometry is automatic: a requested block
    // size keeps the bandwidth layouts it fits.
    const bool few_rows_k1 = !vjp && req_k == 0 && req_l == 0 && req_b == 0 && vb == 16 && !ovl && rows <= cus &&
                             p->nvec >= 64 && p->nvec <= 768 && p->nvec % 64 == 0;
    // The backward forms on few rows (rows x D x itemsize <= 32 KiB, at most
    // 1024 16-byte vectors per row in 16-bit storage and 512 in fp32 or
    // with the last one overlapped, whose instances are built for 512
    // threads): one
    // block, which loops over the rows, so no combine launch follows; one
    // vector per lane; a block of lanes x min(next_pow2(rows), cap / lanes)
    // threads, at least 64 -- cap 512 for rows of 16 lanes or fewer (D = 128
    // in 16-bit storage), 256 above.  The default plan put such rows in
    // 256-thread blocks of up to 32 row slots, the empty slots still part of
    // the dw join, and on more than one block it adds the combine launch.
    // fp16, 32 calls replayed from one graph, per call (VJP; the grad call
    // and the fused backward alike): one row: D = 128 3.83 -> 2.45 us, 512
    // 3.16 -> 1.84, 1024 3.32 -> 2.10, 2048 3.59 -> 2.24, 4096 3.94 -> 2.49;
    // D = 128 x 128 rows 7.02 -> 5.05, 256 x 64 6.95 -> 4.72, 512 x 32 6.25
    // -> 5.23, 1024 x 16 6.48 -> 5.94, 2048 x 8 6.67 -> 5.65, 4096 x 4 7.14
    // -> 4.39 (at 64 KiB the combine was ahead again: 2048 x 16 6.78
    // against 7.82 us in one block).  Rows of 513..1024 16-bit vectors take
    // their exact wave-row instance (D = 5120 / 6144 / 7168: 4.56 / 4.90 /
    // 5.48 -> 2.74 / 2.74 / 3.01 us at one row) or 1024 lanes (D = 8192:
    // 6.04 -> 3.98); fp32 rows of 1024 vectors keep 512 x 2 (3.14 against
    // 3.34 us on 1024 lanes).
    const bool few_rows_vjp = vjp && req_k == 0 && req_l == 0 && req_b == 0 && vb == 16 && rows >= 1 &&
                              rows <= 32768 && p->nvec <= (s == 2 && !ovl ? 1024 : 512) && rows * D * s <= 32768;
    // slots of the few-rows backward block for a row of `l` lanes
    auto few_rows_slots = [&](int l) {
        const int cap = l <= 16 ? 512 : 256;
        return std::min<int64_t>(next_pow2(std::min<int64_t>(rows, 1024)), std::max(1, cap / l));
    };
    bool looped = req_k == -1 || (req_k == 0 && req_l == 0 && p->nvec > 1024 * 8);
    int loop_block = 1024;  // streaming kernel's default block

    if (!looped) {
        int lanes = req_l;
        int k = req_k;
        // Rows of a whole number of waves that is not a power of two (lanes
        // = 64 W with one or two 16-byte vectors per lane: D = 3072, 5120,
        // 6144, 7168 ... in 16-bit storage) are tiled exactly by an instance
        // with the lanes fixed at compile time -- pipelined and unmasked for
        // the backward forms -- instead of masking part of a power-of-two
        // lane group.
        // Four vectors per lane, one row per block, for the backward forms:
        // wide 16-bit rows (D = 12288, 14336, 16384 on 384, 448 or 512 lanes
        // for the VJP, 448 or 512 for the grad call and the fused backward)
        // and fp32 rows of 512 lanes (D = 8192).
        const bool wide_ok = vjp;
        const int vmode = op == RMSN_OP_GRAD ? 1 : op == RMSN_OP_FUSED_VJP ? 2 : 0;
        // (rows whose last vector is overlapped enter only for the
        // backward forms' duplicate-slot layouts and the forward forms'
        // masked whole-wave layouts below, the latter also on request)
        const bool ovl_dup_only = ovl && vjp && lanes == 0 && k == 0;
        const bool ovl_fwd_req = ovl && !vjp && lanes != 0 && rmsn::wave_rows(lanes);
        const bool ovl_fwd_waves = ovl && !vjp && ((lanes == 0 && k == 0 && !few_rows_k1) || ovl_fwd_req);
        if (vb == 16 && (!ovl || ovl_dup_only || ovl_fwd_waves) &&
            (lanes == 0 ? k == 0 : (rmsn::wave_rows(lanes) || (wide_ok && k == 4 && lanes == 512)))) {
            // the first of 2, 1, 4 vectors per lane that tiles the row and
            // has an instance
            int wl = 0, wk = 0;
            const void* fn = nullptr;
            for (int kk : {2, 1, 4}) {
                if (fn || ovl || (k != 0 && kk != k) || p->nvec % kk != 0 || (kk == 4 && !wide_ok)) continue;
                if ((few_rows_k1 || few_rows_vjp) && kk != 1) continue;
                // The backward forms of 16-bit rows of 10 to 15 whole waves of
                // vectors (D = 5120 ... 7680) take one vector per lane, one row
                // per block, rather than two on half the lanes (bf16 / fp16,
                // 64 MiB tensors, VJP / grad call / fused backward: D = 5120
                // 42.2 / 52.7 / 52.8 -> 40.1 / 51.5 / 51.1 us, 6144 42.5 /
                // 54.5 / 53.3 -> 39.9 / 52.9 / 52.1, 7168 44.2 / 55.3 / 53.3
                // -> 41.3 / 53.3 / 52.3; at 3072 the two ran within 3 %).
                if (vjp && lanes == 0 && k == 0 && kk == 2 && s == 2 && p->nvec >= 640 && p->nvec <= 960 &&
                    p->nvec % 64 == 0)
                    continue;
                const int l = p->nvec / kk;
                const bool tiles = (rmsn::wave_rows(l) && rmsn::wave_rows_supported(l)) || (kk == 4 && l == 512);
                if ((lanes != 0 && l != lanes) || !tiles) continue;
                // The automatic forward takes wave rows with two vectors per
                // lane on rows of at most 1024 vectors; with one vector per
                // lane the masked power-of-two layout measured as fast or
                // faster (cold 64 MiB tensors: D = 5120 bf16 24.5 vs 25.8 us;
                // D = 3584 bf16 25.0 vs 24.2 us), and longer rows of the
                // plain forward take 256 lanes x 8 (below); the fused
                // forward keeps wave rows up to 768 lanes.
                if (lanes == 0 && !vjp && !few_rows_k1 &&
                    (kk != 2 || l > 768 || (op == RMSN_OP_FWD && p->nvec > 1024)))
                    continue;
                fn = vjp ? rmsn::vjp_kernel_fixed_lanes(dt, p->nv, kk, vmode, l)
                         : rmsn::fwd_kernel_fixed_lanes(dt, p->nv, kk, op == RMSN_OP_FUSED, l);
                if (fn) {
                    wl = l;
                    wk = kk;
                }
            }
            // Backward rows of whole 16-byte vectors that no instance tiles
            // (D = 1152, 2304, 3840, 5376 ... in 16-bit storage) take the
            // smallest whole number of waves holding the row with one or two
            // vectors per lane, where the row fills at least three quarters
            // of the slots (equal fill: two vectors), in the duplicate-slot
            // instances: the slots past the row's end redo columns inside
            // it, so the pipelined loop masks nothing.  The masked plain loop
            // ran these rows 25-45 % slower (bf16, 64 MiB tensors, VJP /
            // grad call / fused backward: D = 1152 57.2 / 63.1 / 70.6 ->
            // 41.4 / 54.0 / 50.0 us; 2304 60.8 / 66.1 / 73.7 -> 40.3 / 52.4 /
            // 49.6; 5376 51.2 / 59.2 / 60.7 -> 40.7 / 52.7 / 50.6).  A
            // requested wave-row lane count with more slots than the row's
            // vectors (at most twice as many) takes them too.  Rows whose
            // last vector is overlapped (D = 500, 511, 2049, 4097, 8191 ...)
            // take them as well, with as many slots as vectors included,
            // instead of the masked plain loop (fp16 / bf16, 64 MiB tensors,
            // VJP / grad call / fused backward: D = 2049 58.8 / 66.8 / 75.8
            // -> 49.5 / 60.7 / 68.1 us; 4097 73.7 / 88.1 / 96.8 -> 54.7 /
            // 67.6 / 65.0; 6001 67.4 / 86.1 / 84.3 -> 53.2 / 64.1 / 62.7;
            // the grad call and the fused backward on 1024 lanes x 1: 8191
            // 79.0 / 78.9 -> 64.3 / 62.9).
            // On rows of at most 128 vectors (one wave x 2) the grad call
            // keeps the plain loop (D = 768 5.15 against 4.87 TB/s,
            // overlapped D = 500 57.3 against 70.0 us), and so does the VJP
            // on overlapped ones (42.5 against 44.2 us); the fused backward
            // gains there too (500: 62.4 -> 52.4 us).
            bool dup = false;
            const bool one_wave_keeps_plain =
                lanes == 0 && p->nvec <= 128 && (op == RMSN_OP_GRAD || (ovl && op == RMSN_OP_VJP));
            if (!fn && vjp && !few_rows_vjp && !one_wave_keeps_plain) {
                double best = lanes == 0 ? 0.75 : 0.5;
                for (int kk : {2, 1}) {
                    if (k != 0 && kk != k) continue;
                    const int l = lanes != 0 ? lanes : 64 * static_cast<int>((p->nvec + 64 * kk - 1) / (64 * kk));
                    const int64_t nslot = (int64_t)l * kk;
                    if (nslot < p->nvec || (nslot == p->nvec && !ovl) || nslot > 2 * (int64_t)p->nvec) continue;
                    const double fill = static_cast<double>(p->nvec) / static_cast<double>(nslot);
                    if (fill < best || (dup && fill == best)) continue;
                    const void* f = ovl ? rmsn::vjp_kernel_dup_ovl(dt, p->nv, kk, vmode, l)
                                        : rmsn::vjp_kernel_dup(dt, p->nv, kk, vmode, l);
                    if (!f) continue;
                    fn = f;
                    wl = l;
                    wk = kk;
                    best = fill;
                    dup = true;
                }
            }
            // Forward forms on rows whose last vector is overlapped: a whole
            // number of waves (not a power of two) with one or two vectors
            // per lane, the slots past the row's end masked, where it fills
            // at least three quarters of its slots and more than the
            // power-of-two layout below would (about half at D = 2049,
            // 4097).  Rows of more than 512 vectors only where that layout
            // (8 vectors per lane) fills under 65 % of its slots; below, the
            // forward on rows of more than 256 vectors and the fused forward
            // on rows of at most 256 (fp16, 64 MiB tensors, forward / fused
            // forward: D = 4500 30.6 / 52.7 -> 28.1 / 49.3 us on 576 lanes;
            // 3001 28.9 -> 27.3 and 2049 35.0 -> 33.5 forward; 1500 50.1 ->
            // 47.5 fused; but D = 7001 28.7 / 53.0 -> 31.7 / 57.9 on 448 x 2
            // against 128 x 8 at 85 % fill, 6001 bf16 -4 %, the fused
            // forward of 2049 57.5 -> 59.1, and the forward of 1300 27.5 ->
            // 29.6 on 192 x 1 against 64 x 4).
            const int64_t pk = p->nvec > 512 ? 8 : p->nvec > 256 ? 4 : 2;
            const int64_t pl = std::min<int64_t>(1024, next_pow2((p->nvec + pk - 1) / pk));
            const double pfill = static_cast<double>(p->nvec) /
                                 static_cast<double>(pl * next_pow2((p->nvec + pl - 1) / pl));
            const bool waves_pay = p->nvec > 512 ? pfill < 0.65 : (op == RMSN_OP_FWD) == (p->nvec > 256);
            // A requested whole-wave lane count (and vectors per lane, or
            // the fewest that hold the row) is taken as asked.
            if (!fn && ovl_fwd_waves && p->nvec <= 1024 && (waves_pay || ovl_fwd_req)) {
                double best = ovl_fwd_req ? 0.0 : std::max(0.75, pfill + 0.05);
                static constexpr int kAsked[2] = {1, 2}, kAuto[2] = {2, 1};
                for (int i = 0; i < 2; ++i) {
                    const int kk = (ovl_fwd_req ? kAsked : kAuto)[i];
                    if (ovl_fwd_req && (fn || (k != 0 && kk != k) || (int64_t)lanes * kk < p->nvec)) continue;
                    const int l = ovl_fwd_req ? lanes : 64 * static_cast<int>((p->nvec + 64 * kk - 1) / (64 * kk));
                    if (!rmsn::wave_rows(l) || !rmsn::wave_rows_supported(l)) continue;
                    const double fill = static_cast<double>(p->nvec) / (static_cast<double>(l) * kk);
                    if (fill < best || (fn && fill == best)) continue;
                    const void* f = rmsn::fwd_kernel_wave_rows_ovl(dt, p->nv, kk, op == RMSN_OP_FUSED, l);
                    if (!f) continue;
                    fn = f;
                    wl = l;
                    wk = kk;
                    best = fill;
                }
            }
            // one, two or four rows per block, as the registers allow
            const int most = vjp ? rmsn::vjp_pipe_block_max(wl, wk * p->nv)
                                 : (4 * wl <= 1024 ? 4 * wl : 2 * wl <= 1024 ? 2 * wl : wl);
            const int maxb = fn ? std::min(rmsn::max_block_threads(budget_op, wk, p->nv, s), most) : 0;
            // Rows per block and the persistent grid of the backward forms:
            // each CU needs enough row data in flight, counted as waves per
            // row x vectors per lane x row tensors loaded (2; 3 for the fused
            // backward) x rows per block.  Rows per block double until that
            // reaches kWaveRowsInFlight (as the registers allow); if it still
            // falls short, two blocks per CU.  Cold 64 MiB tensors, VJP: D =
            // 1536 bf16 (3 waves, one vector) 39.4 us at four rows per block
            // vs 63.3 at one; 2560 fp16 39.4 vs 48.0 at two; 3072 fp16 40.0
            // vs 44.6 at two; 5120 fp16 40.7 at one vs 42.3 at two; 3584
            // bf16 41.1 at two blocks per CU vs 42.2.  Fused backward: 1536
            // bf16 47.1 at two rows vs 63.1 at one, 3072 fp16 48.1 at one vs
            // 51.6 at two.  The forward (not persistent) runs two three-wave
            // rows per block (D = 3072 fp16 24.0 vs 24.6 us).
            const int w_units = wl / 64 * wk * (op == RMSN_OP_FUSED_VJP ? 3 : 2);
            int block = req_b;
            if (fn && !block) {
                int slots = 1;
                if (few_rows_vjp) {
                    slots = static_cast<int>(few_rows_slots(wl));  // 1 here: wl >= 192
                } else if (vjp) {
                    while (slots < 4 && w_units * slots < kWaveRowsInFlight && 2 * slots * wl <= maxb)
                        slots *= 2;
                } else if (wl == 192 && 2 * wl <= maxb && !few_rows_k1) {
                    slots = 2;
                }
                block = slots * wl;
            }
            const bool block_ok = fn && wl <= maxb && (block == wl || block == 2 * wl || block == 4 * wl) &&
                                  block <= maxb;
            if (block_ok) {
                const int nslots = block / wl;
                const int64_t groups = (rows + nslots - 1) / nslots;
                int64_t grid;
                if (cfg && cfg->num_blocks) {
                    grid = cfg->num_blocks;
                } else if (few_rows_vjp) {
                    grid = 1;
                } else if (vjp) {
                    // persistent: one block per CU, two where the blocks hold
                    // too little row data -- except the grad call, whose two
                    // stored outputs keep the CU busy (D = 3584 bf16, 7 waves
                    // x 1: 51.0 us at one block per CU vs 54.2 at two) -- and
                    // two for the VJP on duplicate-slot rows of one or two
                    // waves (bf16, 64 MiB: D = 768 / 896 / 1600 4.45 / 4.76 /
                    // 4.30 -> 4.90 / 5.03 / 4.76 TB/s; the grad call and the
                    // fused backward ran 4-10 % slower that way)
                    const bool two = (w_units * nslots < kWaveRowsInFlight && op != RMSN_OP_GRAD) ||
                                     (dup && op == RMSN_OP_VJP && wl <= 128);
                    const int per_cu = two ? 2 : 1;
                    grid = vjp_grid(groups, std::min<int64_t>(kMaxPartialRows, (int64_t)per_cu * cus));
                } else {
                    grid = std::min<int64_t>(groups, (int64_t)1 << 20);
                }
                if (grid < 1 || grid > ((int64_t)1 << 30)) return RMSN_E_CONFIG;
                if (vjp && grid > kMaxPartialRows) return RMSN_E_CONFIG;
                p->lanes = wl;
                p->k = wk;
                p->block = block;
                p->pipe = vjp;
                p->fixed_lanes = true;
                p->dup = dup;
                p->grid = grid;
                p->shmem = (vjp && nslots > 1) ? (size_t)block * p->nv * sizeof(float) : 0;
                return RMSN_OK;
            }
            // requested wave rows that do not apply; a requested power of two
            // (512 lanes x 4 in a block this path does not serve) continues
            // to the power-of-two kernels below
            if (lanes != 0 && rmsn::wave_rows(lanes)) return RMSN_E_CONFIG;
        }
        if (lanes == 0 && k == 0) {
            // About 32 bytes of each row tensor per lane: 2 vectors of 16
            // bytes, up to 8 of a narrower width (narrow loads on fewer
            // lanes keep more rows in flight per wave; measured 1.4-2.5x
            // faster than 2 narrow vectors per lane at D = 257..513 fp16)
            int kt = std::min(8, std::max(1, 32 / vb));
            // The plain forward of rows of 1025..2048 16-byte vectors (D =
            // 8200..16384 in 16-bit storage, 4100..8192 in fp32): 256 lanes
            // x 8 vectors in 256-thread blocks, half-empty or full, ran
            // faster than wave rows, 1024 lanes x 2 and the streaming kernel
            // on cold data (bf16, 64 MiB tensors: D = 10240 25.6 vs 28.3-29.1
            // us, 8200 27.9 vs 30.1-31.7, 16384 25.9 vs 26.7-28.7; 256 MiB:
            // D = 10240 87.1 vs 96.9-102.6 us; fp32 D = 4100 26.6 vs 29.0).
            if (op == RMSN_OP_FWD && vb == 16 && p->nvec > 1024 && p->nvec <= 2048) kt = 8;
            // Forward forms on overlapped rows (their vector counts rarely
            // fill a power of two): 8 vectors per lane on rows of 513..1024
            // vectors, 4 from 257 -- fp16, 64 MiB tensors: forward D = 6001
            // 33.0 -> 29.9 us, 8191 31.3 -> 28.5, 4097 39.8 -> 34.8; fused
            // forward D = 2049 71.6 -> 58.9, 3001 60.9 -> 51.6, 6001 63.7 ->
            // 54.9, 8191 57.5 -> 50.8 (D = 4500 ran 8 % slower that way).
            // On rows of 129..256 vectors the forward keeps 2 (128 lanes;
            // against 4 on 64: D = 1025 33.9 -> 33.1, 1201 31.6 -> 29.6,
            // 1450 bf16 27.9 -> 25.9, 1500 27.1 -> 26.0, 1601 28.9 -> 27.4;
            // 1100 28.1 -> 28.7), unlike rows of whole vectors (below).
            if (ovl && !vjp && p->nvec <= 1024) {
                if (p->nvec > 512)
                    kt = 8;
                else if (p->nvec > 256)
                    kt = 4;
            }
            if (few_rows_k1 || few_rows_vjp) kt = 1;
            // The backward forms of 16-bit rows of exactly 512 or 1024
            // vectors (D = 4096, 8192) take one vector per lane on as many
            // lanes, one row per block, pipelined (twice the waves per SIMD
            // of 256 x 2 / 512 x 2): 8192 x 4096 fp16 VJP / grad call /
            // fused backward 42.2 / 53.0 / 50.5 -> 40.7 / 51.1 / 49.4 us,
            // 16384 x 4096 bf16 76.0 / 95.2 / 92.6 -> 73.0 / 93.2 / 91.2;
            // 4096 x 8192 bf16 44.7 / 55.6 / 54.2 -> 41.9 / 53.6 / 52.2,
            // 8192 x 8192 fp16 75.2 / 98.9 / 96.5 -> 73.5 / 96.4 / 93.6,
            // 32768 x 8192 bf16 265.1 / 369.9 / 352.1 -> 261.3 / 363.2 /
            // 355.5.  fp32 rows of 1024 vectors ran alike and keep 512 x 2;
            // rows of 256 vectors ran 7-21 % slower on 256 x 1 (D = 2048
            // fp16) and keep 128 x 2.
            if (vjp && !few_rows_vjp && !ovl && s == 2 && vb == 16 && (p->nvec == 512 || p->nvec == 1024)) kt = 1;
            lanes = std::min(1024, next_pow2((p->nvec + kt - 1) / kt));
            k = next_pow2((p->nvec + lanes - 1) / lanes);
            // The plain forward of a row of 129..1024 vectors that this
            // layout leaves under 90 % full (and that wave rows did not
            // take): 4 vectors per lane on half the lanes, same fill, ran
            // faster cold (bf16 64 MiB: D = 4608 25.3 vs 29.1 us, 2560 24.8
            // vs 27.0, 1536 23.7 vs 24.9, 3584 24.8 vs 25.0; full rows keep 2
            // vectors).
            if (op == RMSN_OP_FWD && vb == 16 && !ovl && kt == 2 && p->nvec > 128 && p->nvec <= 1024 &&
                (int64_t)p->nvec * 10 < (int64_t)lanes * k * 9) {
                kt = 4;
                lanes = std::min(1024, next_pow2((p->nvec + kt - 1) / kt));
                k = next_pow2((p->nvec + lanes - 1) / lanes);
            }
        } else if (lanes == 0) {
            lanes = std::min(1024, next_pow2((p->nvec + k - 1) / k));
        } else if (k == 0) {
            k = next_pow2((p->nvec + lanes - 1) / lanes);
            if (k > 8) return RMSN_E_CONFIG;
        }
        if (!is_pow2(lanes) || lanes > 1024) return RMSN_E_CONFIG;
        if (k != 1 && k != 2 && k != 4 && k != 8) return RMSN_E_CONFIG;
        if ((int64_t)lanes * k < p->nvec) return RMSN_E_CONFIG;
        auto block_max = [&](int kk) {
            return ovl ? rmsn::max_block_threads_ovl(budget_op, kk, p->nv, s)
                       : rmsn::max_block_threads(budget_op, kk, p->nv, s);
        };
        int maxb = block_max(k);
        // automatic choice: more vectors per lane on fewer lanes while the
        // row does not fit the budget's block
        while (!req_l && !req_k && lanes > maxb && k < 8 && lanes > 64) {
            k <<= 1;
            lanes >>= 1;
            maxb = block_max(k);
        }
        const bool automatic = !req_l && !req_k;
        if (lanes > maxb) {
            if (!automatic) return RMSN_E_CONFIG;
            looped = true;  // automatic choice: fall back to the streaming kernel
        } else if (automatic && op == RMSN_OP_FWD && lanes == 1024 &&
                   (int64_t)p->nvec * 10 < (int64_t)lanes * k * 7 && !(k == 4 && p->nv == 4)) {
            // A forward row that needs 1024 lanes but fills under 70 % of
            // their vectors streams faster, in 512-thread blocks (rows of
            // more than 2048 vectors: D = 16392..22936 bf16, 8196..11468
            // fp32; measured 12-35 % faster on cold 256 MiB tensors; the
            // 4-vector fp32 instance measured 4 % faster in registers)
            looped = true;
            loop_block = 512;
        } else {
            int block = req_b;
            if (block == 0) {
                // Small blocks: a block-wide barrier per row group holds fewer
                // waves in lock step (measured fastest for both kernels) --
                // except the persistent VJP on narrow loads, whose 512-block
                // grid then needs 512-thread blocks to keep enough waves
                // resident (measured 10-25 % faster at D = 257..513), and on
                // overlapped rows that fill under 90 % of their vector slots,
                // on row tensors of 24 MiB or more (fp16, 64 MiB tensors: D =
                // 513 64.9 -> 58.9 us, 1025 75.7 -> 64.0, 2049 79.0 -> 62.7,
                // 257 64.6 -> 60.2; but at 16384 rows, 8-16 MiB, and on
                // nearly full rows such as D = 500 and 511, 256 threads ran
                // 4-20 % faster).
                const bool ovl_sparse_big = ovl && (int64_t)p->nvec * 10 < (int64_t)lanes * k * 9 &&
                                            rows * D * s >= ((int64_t)24 << 20);
                const int cap = (vjp && (vb <= 4 || ovl_sparse_big)) ? 512 : 256;
                block = few_rows_k1    ? std::max(lanes, 64)
                        : few_rows_vjp ? std::max<int>(64, lanes * static_cast<int>(few_rows_slots(lanes)))
                                       : std::max(std::max(lanes, 64), std::min(cap, maxb));
            }
            if (block < 64 || block > maxb || block % 64 != 0 || block % lanes != 0 || !is_pow2(block))
                return RMSN_E_CONFIG;
            // A 16-bit backward row of 1536..2048 vectors (at least 3/4 of
            // the 2048 slots) that no pipelined instance serves would run the
            // plain loop on 1024 lanes x 2; on 256 lanes x 8 vectors, one
            // 256-thread block per CU, it ran 5-12 % faster on cold data
            // (bf16 64 MiB: D = 14336 grad call 67.7-70.9 vs 73.2-75.2 us,
            // fused backward 68.1-68.5 vs 76.3-77.1 us; D = 16384 fused
            // backward 65.9-66.0 vs 75.2-75.3 us; D = 13312 VJP 58.7 vs 62.1
            // us).  Sparser rows measured slower that way (D = 8200 VJP 70.8
            // vs 67.4 us), and where a pipelined instance exists (chosen
            // above) it stays ahead (D = 10240 VJP 43.2 vs 61.7 us); no
            // pipelined instance has 1024 lanes.
            bool eight_wide = false;
            if (vjp && automatic && !req_b && s == 2 && vb == 16 && lanes == 1024 && k == 2 && p->nvec >= 1536) {
                lanes = 256;
                k = 8;
                block = 256;
                eight_wide = true;
                if (block > block_max(k)) return RMSN_E_CONFIG;
            }
            p->lanes = lanes;
            p->k = k;
            p->block = block;
            // The fused forward on rows of 512 or 1024 lanes takes the instance
            // with the lanes fixed at compile time on no more rows than CUs
            // (bf16, per call: D = 8192 at 1..8 rows 2.92-3.08 -> 2.52-2.69 us;
            // D = 16384 at 8..256 rows 2-8 % faster) and the runtime-width
            // kernel beyond (D = 16384 at 1024 / 4096 rows 0.9 / 2.9 us slower
            // fixed; 32768 x 8192 355 vs 351 us).
            p->fwd_generic = op == RMSN_OP_FUSED && lanes >= 512 && rows > cus;
            const int nslots = block / lanes;
            const int64_t groups = (rows + nslots - 1) / nslots;
            // Backward forms: the software-pipelined kernel stores
            // unconditionally (a block's ragged last row group aside), so it
            // serves rows that are exactly lanes * k vectors.  The grad
            // call runs pipelined only in an instance with the lanes fixed
            // (8192 x 4096 fp16: 50.6 us against 53.5 in the plain loop; the
            // generic pipelined kernel measured slower than the plain one).
            // Blocks wider than kVjpPipeBlock are pipelined only as a whole
            // 512-lane row in an instance with the lanes fixed (the generic
            // pipelined kernel needs more registers than two such blocks per
            // CU leave; with the width fixed, one block per CU runs faster).
            const bool whole_wide_row = (lanes == rmsn::kVjpPipeFixedMax || (lanes == 1024 && k == 1)) && block == lanes;
            p->pipe = vjp && !ovl && k * p->nv <= rmsn::kVjpPipeElems &&
                      (block <= rmsn::kVjpPipeBlock || whole_wide_row) && (int64_t)lanes * k == p->nvec;
            p->fixed_lanes = p->pipe && rmsn::vjp_kernel_fixed_lanes(dt, p->nv, k, vmode, lanes) != nullptr;
            // the grad call runs pipelined only with the lanes fixed
            if (p->pipe && !p->fixed_lanes && (block > rmsn::kVjpPipeBlock || op == RMSN_OP_GRAD)) p->pipe = false;
            int64_t grid;
            if (cfg && cfg->num_blocks) {
                grid = cfg->num_blocks;
            } else if (few_rows_vjp) {
                grid = 1;  // the block loops over the rows; dw written directly
            } else if (eight_wide) {
                grid = vjp_grid(groups, std::min<int64_t>(kMaxPartialRows, cus));
            } else if (p->fixed_lanes) {
                // one persistent block per CU: with the row width fixed at
                // compile time the pipelined kernel keeps HBM busy with four
                // (or eight) waves per CU, and half the partial rows make the
                // combine cheaper (8192 x 4096 fp16: VJP 39.2 us vs 40.9 at
                // two blocks per CU; 32768 x 8192 bf16: 260 us vs 266 for the
                // plain loop)
                grid = vjp_grid(groups, std::min<int64_t>(kMaxPartialRows, cus));
            } else if (vjp) {
                // Two persistent blocks per CU: every extra partial row costs
                // D * 4 bytes written and re-read by the combine.
                grid = vjp_grid(groups, std::min<int64_t>(kMaxPartialRows, 2 * cus));
            } else {
                grid = std::min<int64_t>(groups, (int64_t)1 << 20);
            }
            if (grid < 1 || grid > ((int64_t)1 << 30)) return RMSN_E_CONFIG;
            if (vjp && grid > kMaxPartialRows) return RMSN_E_CONFIG;
            p->grid = grid;
            p->shmem = (vjp && nslots > 1) ? (size_t)block * p->nv * sizeof(float) : 0;
            return RMSN_OK;
        }
    }

    // streaming kernel: one block per row, whole vectors only
    if (ovl) {
        if (cfg && cfg->vec_bytes) return RMSN_E_CONFIG;
        *p = Plan();
        return make_plan(op, rows, D, dt, cfg, p, false);
    }
    // Backward forms: the column split where the streaming kernel would
    // leave CUs idle (fewer rows than two per CU: at most one persistent
    // block per two rows) or its second pass would miss the caches (long
    // rows; from enough rows on, its single pass over dy and dx wins back).
    // bf16, three rotating sets, VJP: 128 x 2^20 1145 -> 244 us; 511 x
    // 262144 464 -> 250; 1024 x 65536 168 -> 126; 4096 x 65536 522 -> 496;
    // 1024 x 32768 69.1 -> 61.7 (2048 rows: 112.8 against 124.8 split); 256
    // x 16392 21.0 -> 18.6 (1024 rows: 37.2 against 39.8 split).
    if (vjp && !cfg) {
        const int64_t per_cu = (rows + cus - 1) / cus;
        if (rows < 2 * (int64_t)cus || (p->nvec >= 8192 && per_cu <= 16) || (p->nvec >= 4096 && per_cu <= 4))
            return plan_colsplit(rows, cus, 0, p);
    }
    int block = req_b ? req_b : loop_block;
    if (block < 64 || block > 1024 || block % 64 != 0) return RMSN_E_CONFIG;
    p->k = -1;
    p->lanes = block;
    p->block = block;
    // streaming VJP: dw in registers when every thread owns at most 32
    // columns (j vectors of nv), else a partial row in memory
    p->jreg = 0;
    for (int j = 1; j <= 8 && j * p->nv <= 32; j <<= 1) {
        if ((int64_t)j * block >= p->nvec) { p->jreg = j; break; }
    }
    int64_t grid;
    if (cfg && cfg->num_blocks) {
        grid = cfg->num_blocks;
        if (grid > rows && rows > 0) return RMSN_E_CONFIG;  // every block must own a row
    } else if (vjp) {
        // Persistent: at most as many blocks per CU as the kernel's
        // registers let reside at once.  Blocks past that run in a second
        // round, which adds dw partial rows (D * 4 bytes each, written and
        // re-read) but no parallelism: the instances that keep 4 vectors of
        // dw per thread (D = 16392..32768 in 16-bit storage) hold 88-98
        // VGPRs, one 1024-thread block per CU, and on 64 MiB tensors ran
        // 63.5 us at 256 blocks against 80.0 at 512 (D = 32768 bf16; D =
        // 16392 60.5 vs 69.9 us).  Rows past the register dw (row-batched
        // kernel): one block per CU, since every partial row there is D * 4
        // bytes written and re-read (measured best from 40000 to 262144
        // columns).
        int per_cu = 1;
        if (p->jreg != 0) {
            per_cu = std::max(1, 2048 / block);
            const int mode = op == RMSN_OP_GRAD ? 1 : op == RMSN_OP_FUSED_VJP ? 2 : 0;
            const void* fn = rmsn::vjp_kernel(dt, p->nv, -1, mode, p->jreg, false);
            int resident = 0;
            if (fn && hipOccupancyMaxActiveBlocksPerMultiprocessor(&resident, fn, block, 0) == hipSuccess &&
                resident > 0)
                per_cu = std::min(per_cu, resident);
        }
        grid = vjp_grid(rows, std::min<int64_t>(kMaxPartialRows, (int64_t)cus * per_cu));
    } else {
        grid = std::min<int64_t>(rows, (int64_t)1 << 20);
    }
    if (grid < 1) grid = 1;
    if (vjp && grid > kMaxPartialRows) return RMSN_E_CONFIG;
    p->grid = grid;
    p->shmem = 0;
    return RMSN_OK;
}

struct Range {
    uintptr_t lo, hi;
};

Range range_of(const void* p, int64_t bytes) {
    const uintptr_t u = reinterpret_cast<uintptr_t>(p);
    return Range{u, u + static_cast<uintptr_t>(bytes)};
}

bool overlaps(Range a, Range b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

// A row output may be the very buffer of a row input (in place: same start,
// same extent); any other overlap is refused.
bool bad_alias(Range out, Range in) {
    return overlaps(out, in) && !(out.lo == in.lo && out.hi == in.hi);
}

int check_common(int64_t rows, int64_t D, int dt) {
    if (dt != RMSN_F32 && dt != RMSN_F16 && dt != RMSN_BF16) return RMSN_E_DTYPE;
    if (rows < 0 || D < 1 || D > RMSN_MAX_D) return RMSN_E_SHAPE;
    const int64_t s = itemsize(dt);
    if (rows > 0 && rows > INT64_MAX / (D * s)) return RMSN_E_SHAPE;
    return RMSN_OK;
}

bool elem_aligned(const void* p, int s) {
    return reinterpret_cast<uintptr_t>(p) % static_cast<uintptr_t>(s) == 0;
}

int launch(const void* fn, const Plan& p, RowArgs& a, hipStream_t stream) {
    a.lanes = p.lanes;
    a.lshift = log2i(p.lanes);
    a.nvec = p.nvec;
    void* args[] = {&a};
    if (hipLaunchKernel(fn, dim3(static_cast<unsigned>(p.grid)), dim3(p.block), args, p.shmem, stream) !=
        hipSuccess)
        return RMSN_E_HIP;
    return RMSN_OK;
}

int fwd_impl(bool fused, const void* x, const void* res, const void* w, void* y, void* newres,
             int64_t rows, int64_t D, int dt, float eps, float wb, const rmsn_config_t* cfg,
             void* stream) {
    int st = check_common(rows, D, dt);
    if (st != RMSN_OK) return st;
    if (rows == 0) return RMSN_OK;
    if (!x || !w || !y || (fused && (!res || !newres))) return RMSN_E_NULLPTR;
    const int s = itemsize(dt);
    if (!elem_aligned(x, s) || !elem_aligned(w, s) || !elem_aligned(y, s) ||
        (fused && (!elem_aligned(res, s) || !elem_aligned(newres, s))))
        return RMSN_E_ALIGN;
    const int64_t tb = rows * D * s;
    const Range rx = range_of(x, tb), rw = range_of(w, D * s), ry = range_of(y, tb);
    if (fused) {
        const Range rr = range_of(res, tb), rn = range_of(newres, tb);
        const Range outs[2] = {ry, rn};
        for (const Range& o : outs)
            if (bad_alias(o, rx) || bad_alias(o, rr) || overlaps(o, rw)) return RMSN_E_OVERLAP;
        if (overlaps(ry, rn)) return RMSN_E_OVERLAP;
    } else {
        if (bad_alias(ry, rx) || overlaps(ry, rw)) return RMSN_E_OVERLAP;
    }

    Plan p;
    st = make_plan(fused ? RMSN_OP_FUSED : RMSN_OP_FWD, rows, D, dt, cfg, &p);
    if (st != RMSN_OK) return st;
    const void* fn = nullptr;
    if (p.ovl) {
        fn = rmsn::wave_rows(p.lanes) ? rmsn::fwd_kernel_wave_rows_ovl(dt, p.nv, p.k, fused, p.lanes)
                                      : rmsn::fwd_kernel_ovl_fixed(dt, p.k, fused, p.lanes);
        if (!fn && !rmsn::wave_rows(p.lanes)) fn = rmsn::fwd_kernel_ovl(dt, p.k, fused);
    } else {
        fn = p.k > 0 && !p.fwd_generic ? rmsn::fwd_kernel_fixed_lanes(dt, p.nv, p.k, fused, p.lanes) : nullptr;
        if (!fn && !(p.k > 0 && rmsn::wave_rows(p.lanes))) fn = rmsn::fwd_kernel(dt, p.nv, p.k, fused);
    }
    if (!fn) return RMSN_E_CONFIG;

    RowArgs a;
    std::memset(&a, 0, sizeof(a));
    a.x = x;
    a.res = res;
    a.w = w;
    a.y = y;
    a.newres = newres;
    a.rows = rows;
    a.D = static_cast<int32_t>(D);
    a.eps = eps;
    a.wb = wb;
    return launch(fn, p, a, static_cast<hipStream_t>(stream));
}

// Workspace bytes for a plan: fp32 partial rows when the grid has > 1
// block; with dw in the weight dtype also for a one-block grid (the fp32
// sum is staged there and rounded by the combine).
size_t ws_bytes(const Plan& p, int64_t D, bool typed_dw = false) {
    const int64_t nrows = p.grid > 1 ? p.grid : (typed_dw ? 1 : 0);
    return p.cs_stats_bytes + static_cast<size_t>(nrows) * static_cast<size_t>(D) * sizeof(float);
}

// The column-split backward forms: statistics, apply, and (for more than one
// row chunk, or dw in the weight dtype) the combine of the chunks' dw rows.
// Workspace: the row statistics [rows, slices, 2] fp32, then the partial
// rows [chunks, D] fp32.
int colsplit_launch(const Plan& p, const void* x, const void* w, const void* dy, void* y, const void* dres,
                    void* dx, void* dw, int dw_dt, void* ws, int64_t rows, int64_t D, int dt, float eps, float wb,
                    hipStream_t hs) {
    const int mode = y ? 1 : dres ? 2 : 0;
    const void* sfn = nullptr;
    const void* afn = nullptr;
    if (!rmsn::vjp_cs_kernels(dt, p.nv, mode, &sfn, &afn)) return RMSN_E_CONFIG;
    const bool typed_dw = dw_dt != RMSN_F32;
    float* stats = static_cast<float*>(ws);
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.cs_stats_bytes);
    RowArgs a;
    std::memset(&a, 0, sizeof(a));
    a.x = x;
    a.w = w;
    a.dy = dy;
    a.y = y;
    a.res = dres;
    a.dx = dx;
    a.partial = part;
    a.dw = (p.grid == 1 && !typed_dw) ? static_cast<float*>(dw) : part;
    a.rows = rows;
    a.D = static_cast<int32_t>(D);
    a.nvec = p.nvec;
    a.eps = eps;
    a.wb = wb;
    int slices = p.cs_slices;
    void* sargs[] = {&a, &stats, &slices};
    if (hipLaunchKernel(sfn, dim3(static_cast<unsigned>(slices), static_cast<unsigned>(rows)), dim3(p.block),
                        sargs, 0, hs) != hipSuccess)
        return RMSN_E_HIP;
    const float* cstats = stats;
    int chunk = p.cs_chunk;
    void* aargs[] = {&a, &cstats, &slices, &chunk};
    if (hipLaunchKernel(afn, dim3(static_cast<unsigned>(p.cs_tiles), static_cast<unsigned>(p.grid)),
                        dim3(p.block), aargs, 0, hs) != hipSuccess)
        return RMSN_E_HIP;
    if (p.grid == 1 && !typed_dw) return RMSN_OK;
    const float* cpart = part;
    int nb = static_cast<int>(p.grid);
    int d32 = static_cast<int>(D);
    void* cargs[] = {&cpart, &dw, &nb, &d32};
    const unsigned cg = static_cast<unsigned>((D + 15) / 16);
    if (hipLaunchKernel(rmsn::dw_combine_kernel(dw_dt), dim3(cg), dim3(256), cargs, 0, hs) != hipSuccess)
        return RMSN_E_HIP;
    return RMSN_OK;
}

// y != nullptr: the grad call (forward output too); dres != nullptr: the
// fused backward (dx += d_new_residual); neither: the VJP.  dw has dtype
// dw_dt: fp32, or dt (rounded once from the fp32 sum).
int vjp_impl(const void* x, const void* w, const void* dy, void* y, const void* dres, void* dx,
             void* dw, int dw_dt, void* ws, size_t ws_size, int64_t rows, int64_t D, int dt,
             float eps, float wb, const rmsn_config_t* cfg, void* stream) {
    int st = check_common(rows, D, dt);
    if (st != RMSN_OK) return st;
    if (dw_dt != RMSN_F32 && dw_dt != dt) return RMSN_E_DTYPE;
    const bool typed_dw = dw_dt != RMSN_F32;
    const int dws = itemsize(dw_dt);
    if (!dw) return RMSN_E_NULLPTR;
    if (!elem_aligned(dw, dws)) return RMSN_E_ALIGN;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (rows == 0) {
        void* args[] = {&dw, &D};
        const unsigned g = static_cast<unsigned>(std::min<int64_t>((D + 255) / 256, 1024));
        if (hipLaunchKernel(rmsn::zero_kernel(dw_dt), dim3(g), dim3(256), args, 0, hs) != hipSuccess)
            return RMSN_E_HIP;
        return RMSN_OK;
    }
    if (!x || !w || !dy || !dx) return RMSN_E_NULLPTR;
    const bool grad = y != nullptr;
    const bool resgrad = dres != nullptr;
    const int s = itemsize(dt);
    if (!elem_aligned(x, s) || !elem_aligned(w, s) || !elem_aligned(dy, s) || !elem_aligned(dx, s) ||
        (grad && !elem_aligned(y, s)) || (resgrad && !elem_aligned(dres, s)))
        return RMSN_E_ALIGN;
    const int64_t tb = rows * D * s;
    const Range rx = range_of(x, tb), rw = range_of(w, D * s), rd = range_of(dy, tb),
                rdx = range_of(dx, tb), rdw = range_of(dw, D * dws),
                ry = grad ? range_of(y, tb) : Range{0, 0},
                rr = resgrad ? range_of(dres, tb) : Range{0, 0};
    {
        // dx and y may each be exactly one of the row inputs (x, dy,
        // d_new_residual); dw overlaps nothing
        const Range row_ins[3] = {rx, rd, rr};
        for (const Range& i : row_ins)
            if (bad_alias(rdx, i) || bad_alias(ry, i) || overlaps(rdw, i)) return RMSN_E_OVERLAP;
        if (overlaps(rdx, rw) || overlaps(ry, rw) || overlaps(rdw, rw)) return RMSN_E_OVERLAP;
        if (overlaps(rdx, rdw) || overlaps(ry, rdx) || overlaps(ry, rdw)) return RMSN_E_OVERLAP;
    }
    Plan p;
    st = make_plan(resgrad ? RMSN_OP_FUSED_VJP : (grad ? RMSN_OP_GRAD : RMSN_OP_VJP), rows, D, dt, cfg, &p);
    if (st != RMSN_OK) return st;
    const size_t need = ws_bytes(p, D, typed_dw);
    if (need > 0) {
        if (!ws || ws_size < need) return RMSN_E_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(ws) % 16 != 0) return RMSN_E_ALIGN;
        const Range rws = range_of(ws, static_cast<int64_t>(need));
        const Range all[7] = {rx, rw, rd, rdx, rdw, ry, rr};
        for (const Range& o : all)
            if (overlaps(rws, o)) return RMSN_E_OVERLAP;
    }
    const int mode = grad ? 1 : resgrad ? 2 : 0;
    if (p.k == -2) return colsplit_launch(p, x, w, dy, y, dres, dx, dw, dw_dt, ws, rows, D, dt, eps, wb, hs);
    const void* fn = nullptr;
    if (p.dup && p.ovl) {
        fn = rmsn::vjp_kernel_dup_ovl(dt, p.nv, p.k, mode, p.lanes);
    } else if (p.ovl) {
        fn = rmsn::vjp_kernel_ovl(dt, p.k, mode);
    } else {
        fn = p.dup           ? rmsn::vjp_kernel_dup(dt, p.nv, p.k, mode, p.lanes)
             : p.fixed_lanes ? rmsn::vjp_kernel_fixed_lanes(dt, p.nv, p.k, mode, p.lanes)
                             : nullptr;
        if (!fn && !p.dup && !(p.k > 0 && rmsn::wave_rows(p.lanes)))
            fn = rmsn::vjp_kernel(dt, p.nv, p.k, mode, p.jreg, p.pipe);
    }
    if (!fn) return RMSN_E_CONFIG;

    RowArgs a;
    std::memset(&a, 0, sizeof(a));
    a.x = x;
    a.w = w;
    a.dy = dy;
    a.y = y;
    a.res = dres;
    a.dx = dx;
    a.partial = static_cast<float*>(ws);
    // a one-block grid writes the fp32 sum straight to dw, or, for a dw in
    // the weight dtype, to the workspace for the combine to round
    a.dw = typed_dw ? static_cast<float*>(ws) : static_cast<float*>(dw);
    a.rows = rows;
    a.D = static_cast<int32_t>(D);
    a.eps = eps;
    a.wb = wb;
    st = launch(fn, p, a, hs);
    if (st != RMSN_OK || (p.grid == 1 && !typed_dw)) return st;

    const float* partial = static_cast<const float*>(ws);
    int nb = static_cast<int>(p.grid);
    int d32 = static_cast<int>(D);
    void* cargs[] = {&partial, &dw, &nb, &d32};
    const unsigned cg = static_cast<unsigned>((D + 15) / 16);
    if (hipLaunchKernel(rmsn::dw_combine_kernel(dw_dt), dim3(cg), dim3(256), cargs, 0, hs) != hipSuccess)
        return RMSN_E_HIP;
    return RMSN_OK;
}

// ------------------------------------------------------ gated activation

struct GatePlan {
    int nv = 1;        // elements per load
    int64_t nvec = 1;  // d / nv
    int u = 1;         // output vectors per thread per chunk
    int block = 256;
    int64_t nchunks = 1;
    int64_t grid = 1;
};

int check_gate(int64_t rows, int64_t d, int dt) {
    if (dt != RMSN_F32 && dt != RMSN_F16 && dt != RMSN_BF16) return RMSN_E_DTYPE;
    if (rows < 0 || d < 1 || d > RMSN_MAX_GATE_D) return RMSN_E_SHAPE;
    if (rows > 0 && rows > INT64_MAX / (2 * d * itemsize(dt))) return RMSN_E_SHAPE;
    return RMSN_OK;
}

int make_gate_plan(int64_t rows, int64_t d, int dt, const rmsn_config_t* cfg,
                   GatePlan* p) {
    const int s = itemsize(dt);
    if (cfg && (cfg->lanes_per_row != 0 || cfg->vecs_per_lane < 0)) return RMSN_E_CONFIG;
    int vb = 0;
    if (cfg && cfg->vec_bytes) {
        vb = cfg->vec_bytes;
        if (vb < s || vb > 16 || !is_pow2(vb) || (d * s) % vb != 0)
            return RMSN_E_CONFIG;
    } else {
        for (int c = 16; c >= s; c >>= 1) {
            if ((d * s) % c == 0) { vb = c; break; }
        }
        if (vb == 0) vb = s;
    }
    p->nv = vb / s;
    p->nvec = d / p->nv;
    // Default: one-wave blocks, 16 bytes of each half of x per thread in
    // flight (measured fastest on the prefill-scale MLP shape: many small
    // blocks keep every CU's wave slots refilled as soon as a wave retires).
    int u = cfg && cfg->vecs_per_lane ? cfg->vecs_per_lane : std::min(8, std::max(1, 16 / vb));
    if (u != 1 && u != 2 && u != 4 && u != 8) return RMSN_E_CONFIG;
    const int block = cfg && cfg->block_threads ? cfg->block_threads : 64;
    if (block < 64 || block > 1024 || block % 64 != 0) return RMSN_E_CONFIG;
    p->u = u;
    p->block = block;
    const int64_t chunk = static_cast<int64_t>(block) * u;
    const int64_t total = rows * p->nvec;
    p->nchunks = (total + chunk - 1) / chunk;
    // the kernel locates rows with an fp64 estimate that needs chunk starts < 2^52
    if (p->nchunks > ((int64_t)1 << 52) / chunk) return RMSN_E_SHAPE;
    const int64_t max_grid = ((int64_t)1 << 32) / block - 1;  // work-items per dimension < 2^32
    int64_t grid = cfg && cfg->num_blocks ? cfg->num_blocks : std::min<int64_t>(p->nchunks, (int64_t)1 << 20);
    if (grid < 1 || grid > max_grid) return RMSN_E_CONFIG;
    p->grid = grid;
    return RMSN_OK;
}

// Forward (dy == nullptr): out = y [rows, d].  Backward: out = dx [rows, 2d]
// for the upstream gradient dy [rows, d]; dx may be x itself.
int gate_impl(bool vjp, const void* x, const void* dy, void* out, int64_t rows, int64_t d, int dt,
              const rmsn_config_t* cfg, void* stream) {
    int st = check_gate(rows, d, dt);
    if (st != RMSN_OK) return st;
    if (rows == 0) return RMSN_OK;
    if (!x || !out || (vjp && !dy)) return RMSN_E_NULLPTR;
    const int s = itemsize(dt);
    if (!elem_aligned(x, s) || !elem_aligned(out, s) || (vjp && !elem_aligned(dy, s))) return RMSN_E_ALIGN;
    const Range rx = range_of(x, rows * 2 * d * s);
    if (vjp) {
        const Range rdx = range_of(out, rows * 2 * d * s), rdy = range_of(dy, rows * d * s);
        if (bad_alias(rdx, rx) || overlaps(rdx, rdy)) return RMSN_E_OVERLAP;
    } else if (overlaps(range_of(out, rows * d * s), rx)) {
        return RMSN_E_OVERLAP;
    }
    GatePlan p;
    st = make_gate_plan(rows, d, dt, cfg, &p);
    if (st != RMSN_OK) return st;
    const void* fn = vjp ? rmsn::gate_vjp_kernel(dt, p.nv, p.u) : rmsn::gate_kernel(dt, p.nv, p.u);
    if (!fn) return RMSN_E_CONFIG;
    int64_t total = rows * p.nvec;
    int64_t nvec = p.nvec;
    // ceil(2^32 / nvec); exact row offsets for the small quotients inside a chunk
    uint32_t recip = nvec > 1 ? static_cast<uint32_t>((((uint64_t)1 << 32) + nvec - 1) / nvec) : 0u;
    double inv = 1.0 / static_cast<double>(nvec);
    int64_t nchunks = p.nchunks;
    void* fargs[] = {&x, &out, &total, &nvec, &recip, &inv, &nchunks};
    void* bargs[] = {&x, &dy, &out, &total, &nvec, &recip, &inv, &nchunks};
    if (hipLaunchKernel(fn, dim3(static_cast<unsigned>(p.grid)), dim3(p.block), vjp ? bargs : fargs, 0,
                        static_cast<hipStream_t>(stream)) != hipSuccess)
        return RMSN_E_HIP;
    return RMSN_OK;
}

}  // namespace

extern "C" {

int silu_gate(const void* x, void* y, int64_t rows, int64_t d, int dt, void* hip_stream) {
    return gate_impl(false, x, nullptr, y, rows, d, dt, nullptr, hip_stream);
}

int silu_gate_cfg(const void* x, void* y, int64_t rows, int64_t d, int dt, const rmsn_config_t* cfg,
                  void* hip_stream) {
    return gate_impl(false, x, nullptr, y, rows, d, dt, cfg, hip_stream);
}

int silu_gate_vjp(const void* x, const void* dy, void* dx, int64_t rows, int64_t d, int dt,
                  void* hip_stream) {
    return gate_impl(true, x, dy, dx, rows, d, dt, nullptr, hip_stream);
}

int silu_gate_vjp_cfg(const void* x, const void* dy, void* dx, int64_t rows, int64_t d, int dt,
                      const rmsn_config_t* cfg, void* hip_stream) {
    return gate_impl(true, x, dy, dx, rows, d, dt, cfg, hip_stream);
}

int rmsnorm_fwd(const void* x, const void* w, void* y, int64_t rows, int64_t D, int dt, float eps,
                float weight_bias, void* hip_stream) {
    return fwd_impl(false, x, nullptr, w, y, nullptr, rows, D, dt, eps, weight_bias, nullptr,
                    hip_stream);
}

int rmsnorm_fwd_cfg(const void* x, const void* w, void* y, int64_t rows, int64_t D, int dt,
                    float eps, float weight_bias, const rmsn_config_t* cfg, void* hip_stream) {
    return fwd_impl(false, x, nullptr, w, y, nullptr, rows, D, dt, eps, weight_bias, cfg,
                    hip_stream);
}

int fused_add_rmsnorm_fwd(const void* x, const void* residual, const void* w, void* normed,
                          void* new_residual, int64_t rows, int64_t D, int dt, float eps,
                          float weight_bias, void* hip_stream) {
    return fwd_impl(true, x, residual, w, normed, new_residual, rows, D, dt, eps, weight_bias,
                    nullptr, hip_stream);
}

int fused_add_rmsnorm_fwd_cfg(const void* x, const void* residual, const void* w, void* normed,
                              void* new_residual, int64_t rows, int64_t D, int dt, float eps,
                              float weight_bias, const rmsn_config_t* cfg, void* hip_stream) {
    return fwd_impl(true, x, residual, w, normed, new_residual, rows, D, dt, eps, weight_bias, cfg,
                    hip_stream);
}

size_t rmsnorm_vjp_workspace_bytes(int64_t rows, int64_t D, int dt) {
    if (check_common(rows, D, dt) != RMSN_OK) return 0;
    size_t best = 0;
    if (rows > 0) {
        for (int op : {RMSN_OP_VJP, RMSN_OP_GRAD, RMSN_OP_FUSED_VJP}) {
            Plan p;
            if (make_plan(op, rows, D, dt, nullptr, &p) != RMSN_OK) return 0;
            best = std::max(best, ws_bytes(p, D, /*typed_dw=*/true));
        }
    }
    return std::max<size_t>(best, 256);
}

int rmsnorm_vjp(const void* x, const void* w, const void* dy, void* dx, float* dw, void* workspace,
                size_t workspace_bytes, int64_t rows, int64_t D, int dt, float eps, float weight_bias,
                void* hip_stream) {
    return vjp_impl(x, w, dy, nullptr, nullptr, dx, dw, RMSN_F32, workspace, workspace_bytes, rows, D, dt, eps,
                    weight_bias, nullptr, hip_stream);
}

int rmsnorm_vjp_noalloc(const void* x, const void* w, const void* dy, void* dx, float* dw, int64_t rows,
                        int64_t D, int dt, float eps, float weight_bias, void* hip_stream) {
    // argument errors first, so that they do not depend on the device
    int st = check_common(rows, D, dt);
    if (st != RMSN_OK) return st;
    void* ws = nullptr;
    if (rows > 0) {
        st = scratch_ptr(&ws);
        if (st != RMSN_OK) return st;
    }
    // vjp_impl plans the launch and returns RMSN_E_WORKSPACE when the plan's
    // partial rows need more than the scratch holds
    return vjp_impl(x, w, dy, nullptr, nullptr, dx, dw, RMSN_F32, ws, RMSN_NOALLOC_SCRATCH_BYTES, rows, D, dt, eps,
                    weight_bias, nullptr, hip_stream);
}

int rmsnorm_fwd_vjp(const void* x, const void* w, const void* dy, void* y, void* dx, float* dw,
                    void* workspace, size_t workspace_bytes, int64_t rows, int64_t D, int dt,
                    float eps, float weight_bias, void* hip_stream) {
    if (rows > 0 && !y) return RMSN_E_NULLPTR;
    return vjp_impl(x, w, dy, rows > 0 ? y : nullptr, nullptr, dx, dw, RMSN_F32, workspace, workspace_bytes, rows, D,
                    dt, eps, weight_bias, nullptr, hip_stream);
}

int rmsnorm_fwd_vjp_cfg(const void* x, const void* w, const void* dy, void* y, void* dx, float* dw,
                        void* workspace, size_t workspace_bytes, int64_t rows, int64_t D, int dt,
                        float eps, float weight_bias, const rmsn_config_t* cfg, void* hip_stream) {
    if (rows > 0 && !y) return RMSN_E_NULLPTR;
    return vjp_impl(x, w, dy, rows > 0 ? y : nullptr, nullptr, dx, dw, RMSN_F32, workspace, workspace_bytes, rows, D,
                    dt, eps, weight_bias, cfg, hip_stream);
}

int rmsnorm_vjp_cfg(const void* x, const void* w, const void* dy, void* dx, float* dw,
                    void* workspace, size_t workspace_bytes, int64_t rows, int64_t D, int dt,
                    float eps, float weight_bias, const rmsn_config_t* cfg, void* hip_stream) {
    return vjp_impl(x, w, dy, nullptr, nullptr, dx, dw, RMSN_F32, workspace, workspace_bytes, rows, D, dt, eps,
                    weight_bias, cfg, hip_stream);
}

int fused_add_rmsnorm_vjp(const void* h, const void* w, const void* dy, const void* d_new_residual,
                          void* dh, float* dw, void* workspace, size_t workspace_bytes, int64_t rows,
                          int64_t D, int dt, float eps, float weight_bias, void* hip_stream) {
    if (rows > 0 && !d_new_residual) return RMSN_E_NULLPTR;
    return vjp_impl(h, w, dy, nullptr, rows > 0 ? d_new_residual : nullptr, dh, dw, RMSN_F32, workspace,
                    workspace_bytes, rows, D, dt, eps, weight_bias, nullptr, hip_stream);
}

int fused_add_rmsnorm_vjp_cfg(const void* h, const void* w, const void* dy,
                              const void* d_new_residual, void* dh, float* dw, void* workspace,
                              size_t workspace_bytes, int64_t rows, int64_t D, int dt, float eps,
                              float weight_bias, const rmsn_config_t* cfg, void* hip_stream) {
    if (rows > 0 && !d_new_residual) return RMSN_E_NULLPTR;
    return vjp_impl(h, w, dy, nullptr, rows > 0 ? d_new_residual : nullptr, dh, dw, RMSN_F32, workspace,
                    workspace_bytes, rows, D, dt, eps, weight_bias, cfg, hip_stream);
}

int rmsnorm_backward(const void* x, const void* w, const void* dy, const void* d_new_residual,
                     void* y, void* dx, void* dw, int dw_dt, void* workspace,
                     size_t workspace_bytes, int64_t rows, int64_t D, int dt, float eps,
                     float weight_bias, const rmsn_config_t* cfg, void* hip_stream) {
    if (y && d_new_residual) return RMSN_E_CONFIG;  // no kernel computes both
    return vjp_impl(x, w, dy, rows > 0 ? y : nullptr, rows > 0 ? d_new_residual : nullptr, dx, dw,
                    dw_dt, workspace, workspace_bytes, rows, D, dt, eps, weight_bias, cfg, hip_stream);
}

int rmsn_query_config(int op, int64_t rows, int64_t D, int dt, int align_bytes, rmsn_config_t* out) {
    if (!out) return RMSN_E_NULLPTR;
    if (op == RMSN_OP_GATE) {
        int st = check_gate(rows, D, dt);
        if (st != RMSN_OK) return st;
        if (align_bytes <= 0 || !is_pow2(align_bytes)) return RMSN_E_ALIGN;
        GatePlan g;
        st = make_gate_plan(std::max<int64_t>(rows, 1), D, dt, nullptr, &g);
        if (st != RMSN_OK) return st;
        out->lanes_per_row = 0;
        out->vecs_per_lane = g.u;
        out->vec_bytes = g.nv * itemsize(dt);
        out->block_threads = g.block;
        out->num_blocks = static_cast<int32_t>(g.grid);
        return RMSN_OK;
    }
    if (op < RMSN_OP_FWD || op > RMSN_OP_FUSED_VJP) return RMSN_E_CONFIG;
    int st = check_common(rows, D, dt);
    if (st != RMSN_OK) return st;
    if (align_bytes <= 0 || !is_pow2(align_bytes)) return RMSN_E_ALIGN;
    Plan p;
    st = make_plan(op, std::max<int64_t>(rows, 1), D, dt, nullptr, &p);
    if (st != RMSN_OK) return st;
    out->lanes_per_row = p.k < 0 ? 0 : p.lanes;
    out->vecs_per_lane = p.k;
    out->vec_bytes = p.nv * itemsize(dt);
    out->block_threads = p.block;
    out->num_blocks = static_cast<int32_t>(p.grid);
    return RMSN_OK;
}

const char* rmsn_status_str(int status) {
    switch (status) {
        case RMSN_OK: return "ok";
        case RMSN_E_NULLPTR: return "a required pointer is NULL";
        case RMSN_E_SHAPE: return "invalid shape (rows < 0, D < 1, D too large or sizes overflow)";
        case RMSN_E_DTYPE: return "unknown dtype, or a dw dtype other than fp32 and the storage dtype";
        case RMSN_E_WORKSPACE: return "workspace missing or too small";
        case RMSN_E_OVERLAP: return "an output overlaps another argument";
        case RMSN_E_HIP: return "HIP runtime error";
        case RMSN_E_ALIGN: return "pointer not aligned to its element size";
        case RMSN_E_CONFIG: return "kernel configuration cannot serve this shape";
        default: return "unknown status";
    }
}

}  // extern "C"
