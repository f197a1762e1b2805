// dw_reduction.hip -- measurement program (not part of the library): where
// the time goes when the VJP's weight-gradient reduction is finished in
// different ways, at the [8192, 4096] fp16 shape of the MLX pull request's
// POC (x, w, dy ~ U(0,1), eps 1e-5).
//
// The MLX pull request "RMSNormVJP backward writes a full {n_rows, D}
// gw_temp intermediate" (Proposed changes) sums the rows of gw inside the
// kernel.  On MI355X the library's VJP accumulates dw per block in registers
// and writes one fp32 partial row per block; a second, tiny launch adds the
// rows in a fixed order.  This program runs the library's own pipelined row
// kernel (vjp_rows, 256 lanes x 2 vectors, one persistent block per CU) with
// other ways of finishing, through the kernel's dw output hook:
//
//   rows_only         the partial rows are stored and nothing adds them (a
//                     floor: dw is not formed);
//   ticket_fence      a deterministic two-level last-arrival reduction in the
//                     same launch: each block stores its partial row, makes an
//                     agent-scope release, and one lane takes a ticket with a
//                     vector atomic on its group's counter (groups of G
//                     consecutive blocks); the last arrival of a group adds
//                     the group's rows in block order into the group's first
//                     row, then takes a ticket on the top counter; the last
//                     group adds the group rows in order into dw.  Counters are
//                     reset by the arrival that completes them.  No block
//                     waits for another;
//   ticket_wt         the same tree, with the partial rows written and read
//                     by agent-scope relaxed atomic stores and loads (write-
//                     through, so no L2 write-back fence is needed) and the
//                     ticket taken once every store of the thread is
//                     acknowledged.
//
// Reported: back-to-back times (HIP events) of the library's fwd + VJP step,
// of its VJP, of each variant, of an empty kernel (the per-launch floor), and
// per-block timestamps (the 100 MHz constant clock) of one launch of each
// variant: when the blocks finish their rows, take their tickets, finish the
// group sums and write dw.  dw of each variant is checked against the
// library's (relative difference) and for bitwise repeatability.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "rmsn_kernels.hpp"
#include "rmsnorm_mi355x.h"

namespace probe {

using rmsn::RowArgs;

constexpr int kMaxBlocks = 4096;
constexpr int kStages = 6;  // block start, rows done, group ticket, group sum, top ticket, dw written
__device__ unsigned long long g_ts[kStages][kMaxBlocks];
__device__ unsigned g_cnt[1024];  // ticket counters: zero before the first launch, left zero by each

__device__ __forceinline__ void stamp(int i) {
    if (threadIdx.x == 0 && blockIdx.x < kMaxBlocks) g_ts[i][blockIdx.x] = __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// dst[c] = sum over r < n of src[r * stride + c], rows added in order r = 0,
// 1, ...; AGENT: agent-scope atomic loads and stores (fp32 words), else
// float4 loads and stores (D % 4 == 0).  dst may be src's first row.
template <bool AGENT>
__device__ void sum_rows(const float* src, int n, int64_t stride, int D, float* dst) {
    constexpr int U = 16;  // rows in flight per batch
    if constexpr (AGENT) {
        for (int c0 = threadIdx.x; c0 < D; c0 += 4 * blockDim.x) {
            float s[4] = {0.f, 0.f, 0.f, 0.f};
            for (int r = 0; r < n; r += U) {
                float v[U][4];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int rr = r + u < n ? r + u : r;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int c = c0 + j * static_cast<int>(blockDim.x);
                        v[u][j] = c < D ? ld_agent(src + rr * stride + c) : 0.f;
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (r + u < n)
#pragma unroll
                        for (int j = 0; j < 4; ++j) s[j] += v[u][j];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = c0 + j * static_cast<int>(blockDim.x);
                if (c < D) st_agent(dst + c, s[j]);
            }
        }
    } else {
        const int nq = D >> 2;
        for (int q = threadIdx.x; q < nq; q += blockDim.x) {
            float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int r = 0; r < n; r += U) {
                float4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int rr = r + u < n ? r + u : r;
                    v[u] = *reinterpret_cast<const float4*>(src + rr * stride + 4 * q);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (r + u < n) {
                        s.x += v[u].x;
                        s.y += v[u].y;
                        s.z += v[u].z;
                        s.w += v[u].w;
                    }
                }
            }
            *reinterpret_cast<float4*>(dst + 4 * q) = s;
        }
    }
}

// The two-level last-arrival reduction (every thread of the block calls it
// after its partial row stores).
template <int G, bool AGENT>
__device__ void ticket_tree(const RowArgs& a) {
    __shared__ unsigned s_ticket;
    if constexpr (AGENT) {
        __builtin_amdgcn_s_waitcnt(0);  // this thread's write-through stores acknowledged
    } else {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    }
    __syncthreads();
    const int nb = gridDim.x, b = blockIdx.x, D = a.D;
    const int ng = (nb + G - 1) / G, g = b / G, g0 = g * G, gs = min(G, nb - g0);
    if (threadIdx.x == 0)
        s_ticket = __hip_atomic_fetch_add(&g_cnt[1 + g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    stamp(2);
    if (s_ticket != static_cast<unsigned>(gs - 1)) return;
    if constexpr (!AGENT) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (threadIdx.x == 0) __hip_atomic_store(&g_cnt[1 + g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float* gdst = ng == 1 ? a.dw : a.partial + (int64_t)g0 * D;
    sum_rows<AGENT>(a.partial + (int64_t)g0 * D, gs, D, D, gdst);
    stamp(3);
    if (ng == 1) return;
    if constexpr (AGENT) {
        __builtin_amdgcn_s_waitcnt(0);
    } else {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    }
    __syncthreads();
    if (threadIdx.x == 0)
        s_ticket = __hip_atomic_fetch_add(&g_cnt[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    stamp(4);
    if (s_ticket != static_cast<unsigned>(ng - 1)) return;
    if constexpr (!AGENT) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (threadIdx.x == 0) __hip_atomic_store(&g_cnt[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sum_rows<AGENT>(a.partial, ng, (int64_t)G * D, D, a.dw);
    stamp(5);
}

// dw output policies for rmsn::vjp_rows
struct RowsOnly {
    __device__ static void begin(const RowArgs&) { stamp(0); }
    template <int NV>
    __device__ static void store(float* out, const float (&v)[NV], bool vec_ok) {
        rmsn::PartialRowOut::store<NV>(out, v, vec_ok);
    }
    __device__ static void end(const RowArgs&) {
        __syncthreads();
        stamp(1);
    }
};

template <int G>
struct TicketFence {
    __device__ static void begin(const RowArgs&) { stamp(0); }
    template <int NV>
    __device__ static void store(float* out, const float (&v)[NV], bool vec_ok) {
        rmsn::PartialRowOut::store<NV>(out, v, vec_ok);
    }
    __device__ static void end(const RowArgs& a) {
        __syncthreads();
        stamp(1);
        if (gridDim.x > 1) ticket_tree<G, false>(a);
    }
};

template <int G>
struct TicketWriteThrough {
    __device__ static void begin(const RowArgs&) { stamp(0); }
    template <int NV>
    __device__ static void store(float* out, const float (&v)[NV], bool) {
#pragma unroll
        for (int e = 0; e < NV; ++e) st_agent(out + e, v[e]);
    }
    __device__ static void end(const RowArgs& a) {
        __syncthreads();
        stamp(1);
        if (gridDim.x > 1) ticket_tree<G, true>(a);
    }
};

// Partial rows stored non-temporally (the row tensors' cache policy).
struct NtPartial {
    __device__ static void begin(const RowArgs&) {}
    template <int NV>
    __device__ static void store(float* out, const float (&v)[NV], bool) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int e = 0; e < NV; e += 4) {
            const f32x4 q = {v[e], v[e + 1], v[e + 2], v[e + 3]};
            __builtin_nontemporal_store(q, reinterpret_cast<f32x4*>(out + e));
        }
    }
    __device__ static void end(const RowArgs&) {}
};

// Combine layouts: a block adds COLS columns over all nb partial rows.  COLS
// / 4 threads cover one row's columns with float4 loads (COLS = 32: one
// 128-byte line per row), RG = THREADS * 4 / COLS row groups; thread (rg, q)
// adds rows rg, rg + RG, ... in order, then the RG sums of each column are
// added in row-group order from LDS.  D % COLS == 0, nb % RG == 0.
template <int COLS, int THREADS>
__global__ __launch_bounds__(THREADS) void combine_cols(const float* __restrict__ partial, float* __restrict__ dw,
                                                        int nb, int D) {
    constexpr int TPR = COLS / 4;
    constexpr int RG = THREADS / TPR;
    __shared__ float4 buf[RG][TPR];
    const int q = threadIdx.x % TPR, rg = threadIdx.x / TPR;
    const int col = blockIdx.x * COLS + 4 * q;
    const int per = nb / RG;  // rows per thread
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r0 = 0; r0 < per; r0 += 8) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int r = r0 + u < per ? r0 + u : r0;
            v[u] = *reinterpret_cast<const float4*>(partial + (int64_t)(rg + r * RG) * D + col);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (r0 + u < per) {
                s.x += v[u].x;
                s.y += v[u].y;
                s.z += v[u].z;
                s.w += v[u].w;
            }
        }
    }
    buf[rg][q] = s;
    __syncthreads();
    if (threadIdx.x < COLS) {
        const int qq = threadIdx.x / 4, e = threadIdx.x % 4;
        float t = 0.f;
        for (int g = 0; g < RG; ++g) {
            const float4 b = buf[g][qq];
            t += e == 0 ? b.x : e == 1 ? b.y : e == 2 ? b.z : b.w;
        }
        dw[blockIdx.x * COLS + threadIdx.x] = t;
    }
}

__global__ void empty_kernel() {}

__global__ void init_u01(_Float16* p, size_t n, unsigned seed) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        unsigned h = static_cast<unsigned>(i) * 2654435761u ^ seed;
        h ^= h >> 15;
        h *= 2246822519u;
        h ^= h >> 13;
        p[i] = static_cast<_Float16>((h >> 8) * (1.0f / 16777216.0f));
    }
}

}  // namespace probe

#define CK(x)                                                                             \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)
#define RS(x)                                                                    \
    do {                                                                         \
        int s_ = (x);                                                            \
        if (s_ != 0) {                                                           \
            fprintf(stderr, "library status %d at line %d\n", s_, __LINE__);     \
            exit(1);                                                             \
        }                                                                        \
    } while (0)

namespace {

template <class OUT>
const void* row_kernel() {
    return reinterpret_cast<const void*>(&rmsn::vjp_rows<_Float16, 8, 2, rmsn::kVjp, true, 256, OUT>);
}

struct Times {
    double lo = 1e30, hi = 0;
    int n = 0;
};

Times stage(const std::vector<unsigned long long>& ts, int k, int nb, unsigned long long base) {
    Times t;
    for (int b = 0; b < nb; ++b) {
        const unsigned long long v = ts[(size_t)k * probe::kMaxBlocks + b];
        if (!v) continue;
        const double us = (static_cast<double>(v) - static_cast<double>(base)) * 0.01;
        t.lo = std::min(t.lo, us);
        t.hi = std::max(t.hi, us);
        ++t.n;
    }
    return t;
}

}  // namespace

int main() {
    const int64_t R = 8192, D = 4096;
    const size_t n = static_cast<size_t>(R * D);
    const int NS = 5;  // rotating buffer sets: a set is touched again after >= 1 GiB of other traffic
    const int N = 300;
    int cus = 0;
    CK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    const int nb = std::min<int>(cus, probe::kMaxBlocks);

    _Float16 *x[NS], *dy[NS], *y[NS], *dx[NS], *w;
    float *dw, *partial;
    for (int s = 0; s < NS; ++s) {
        CK(hipMalloc(&x[s], n * 2));
        CK(hipMalloc(&dy[s], n * 2));
        CK(hipMalloc(&y[s], n * 2));
        CK(hipMalloc(&dx[s], n * 2));
        probe::init_u01<<<1024, 256>>>(x[s], n, 11 + s);
        probe::init_u01<<<1024, 256>>>(dy[s], n, 101 + s);
    }
    CK(hipMalloc(&w, D * 2));
    probe::init_u01<<<16, 256>>>(w, D, 7);
    CK(hipMalloc(&dw, D * 4));
    const size_t wsb = std::max(rmsnorm_vjp_workspace_bytes(R, D, RMSN_F16), (size_t)nb * D * 4);
    CK(hipMalloc(&partial, wsb));
    {
        static unsigned zero[1024];
        CK(hipMemcpyToSymbol(HIP_SYMBOL(probe::g_cnt), zero, sizeof(zero)));
    }
    hipStream_t st;
    CK(hipStreamCreate(&st));
    CK(hipDeviceSynchronize());

    auto fwd = [&](int s) { RS(rmsnorm_fwd(x[s], w, y[s], R, D, RMSN_F16, 1e-5f, 0.f, st)); };
    auto vjp = [&](int s) { RS(rmsnorm_vjp(x[s], w, dy[s], dx[s], dw, partial, wsb, R, D, RMSN_F16, 1e-5f, 0.f, st)); };
    auto launch = [&](const void* fn, int s) {
        rmsn::RowArgs a;
        std::memset(&a, 0, sizeof(a));
        a.x = x[s];
        a.w = w;
        a.dy = dy[s];
        a.dx = dx[s];
        a.partial = partial;
        a.dw = dw;
        a.rows = R;
        a.D = static_cast<int32_t>(D);
        a.nvec = static_cast<int32_t>(D / 8);
        a.lanes = 256;
        a.lshift = 8;
        a.eps = 1e-5f;
        a.wb = 0.f;
        void* args[] = {&a};
        CK(hipLaunchKernel(fn, dim3(nb), dim3(256), args, 0, st));
    };
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    auto timed = [&](auto fn) {
        for (int i = 0; i < 10; ++i) fn(i % NS);
        CK(hipStreamSynchronize(st));
        CK(hipEventRecord(e0, st));
        for (int i = 0; i < N; ++i) fn(i % NS);
        CK(hipEventRecord(e1, st));
        CK(hipEventSynchronize(e1));
        float ms = 0;
        CK(hipEventElapsedTime(&ms, e0, e1));
        return ms * 1e3 / N;
    };
    std::vector<float> dw_lib(D), dw_a(D), dw_b(D);
    std::vector<unsigned long long> ts((size_t)probe::kStages * probe::kMaxBlocks);
    auto timeline = [&](const void* fn) {  // one fwd + variant step after a clear
        std::vector<unsigned long long> z(ts.size(), 0ull);
        CK(hipStreamSynchronize(st));
        CK(hipMemcpyToSymbol(HIP_SYMBOL(probe::g_ts), z.data(), z.size() * sizeof(z[0])));
        fwd(0);
        launch(fn, 0);
        CK(hipStreamSynchronize(st));
        CK(hipMemcpyFromSymbol(ts.data(), HIP_SYMBOL(probe::g_ts), ts.size() * sizeof(ts[0])));
    };

    const double t_empty = timed([&](int) { probe::empty_kernel<<<1, 64, 0, st>>>(); });
    const double t_step_lib = timed([&](int s) { fwd(s); vjp(s); });
    const double t_vjp_lib = timed([&](int s) { vjp(s); });
    const double t_fwd_lib = timed([&](int s) { fwd(s); });
    vjp(0);
    CK(hipStreamSynchronize(st));
    CK(hipMemcpy(dw_lib.data(), dw, D * 4, hipMemcpyDeviceToHost));
    double dwmax = 0;
    for (float v : dw_lib) dwmax = std::max(dwmax, (double)std::fabs(v));

    struct Variant {
        const char* name;
        const void* fn;
        bool forms_dw;
    };
    const Variant variants[] = {
        {"rows_only", row_kernel<probe::RowsOnly>(), false},
        {"ticket_fence_g16", row_kernel<probe::TicketFence<16>>(), true},
        {"ticket_fence_g8", row_kernel<probe::TicketFence<8>>(), true},
        {"ticket_fence_g32", row_kernel<probe::TicketFence<32>>(), true},
        {"ticket_wt_g16", row_kernel<probe::TicketWriteThrough<16>>(), true},
        {"ticket_wt_g8", row_kernel<probe::TicketWriteThrough<8>>(), true},
        {"ticket_wt_g32", row_kernel<probe::TicketWriteThrough<32>>(), true},
    };
    printf("{\"shape\": \"8192x4096 fp16\", \"blocks\": %d, \"empty_kernel_us\": %.3f, "
           "\"library\": {\"step_us\": %.3f, \"vjp_us\": %.3f, \"fwd_us\": %.3f}, \"variants\": [",
           nb, t_empty, t_step_lib, t_vjp_lib, t_fwd_lib);
    bool first = true;
    for (const Variant& v : variants) {
        const double t_vjp = timed([&](int s) { launch(v.fn, s); });
        const double t_step = timed([&](int s) {
            fwd(s);
            launch(v.fn, s);
        });
        double rel = -1;
        int repeat = -1;
        unsigned nonzero = 0;
        if (v.forms_dw) {
            launch(v.fn, 0);
            CK(hipStreamSynchronize(st));
            CK(hipMemcpy(dw_a.data(), dw, D * 4, hipMemcpyDeviceToHost));
            launch(v.fn, 0);
            CK(hipStreamSynchronize(st));
            CK(hipMemcpy(dw_b.data(), dw, D * 4, hipMemcpyDeviceToHost));
            double md = 0;
            for (int j = 0; j < D; ++j) md = std::max(md, (double)std::fabs(dw_a[j] - dw_lib[j]));
            rel = md / dwmax;
            repeat = std::memcmp(dw_a.data(), dw_b.data(), D * 4) == 0;
            unsigned cnt[1024];
            CK(hipMemcpyFromSymbol(cnt, HIP_SYMBOL(probe::g_cnt), sizeof(cnt)));
            for (unsigned c : cnt) nonzero += c != 0;
        }
        timeline(v.fn);
        unsigned long long base = ~0ull;
        for (int b = 0; b < nb; ++b) base = std::min(base, ts[b]);
        const char* names[probe::kStages] = {"start", "rows_done", "group_ticket", "group_sum", "top_ticket",
                                             "dw_written"};
        printf("%s{\"name\": \"%s\", \"vjp_us\": %.3f, \"step_us\": %.3f, \"step_GBps\": %.1f, "
               "\"dw_rel_diff_vs_library\": %.3g, \"dw_bitwise_repeat\": %d, \"counters_left_nonzero\": %u, "
               "\"timeline_us\": {",
               first ? "" : ", ", v.name, t_vjp, t_step, 335577088.0 / (t_step * 1e-6) / 1e9, rel, repeat, nonzero);
        first = false;
        for (int k = 0; k < probe::kStages; ++k) {
            const Times t = stage(ts, k, nb, base);
            printf("%s\"%s\": {\"blocks\": %d, \"first\": %.2f, \"last\": %.2f}", k ? ", " : "", names[k], t.n,
                   t.n ? t.lo : 0.0, t.n ? t.hi : 0.0);
        }
        printf("}}");
        fflush(stdout);
    }
    printf("], \"combine_layouts\": [");
    // rows (library policy or non-temporal partial stores) + a combine layout
    struct Comb {
        const char* name;
        const void* rows;
        const void* comb;
        int cols, threads;
    };
    const void* lib_rows = row_kernel<rmsn::PartialRowOut>();
    const void* nt_rows = row_kernel<probe::NtPartial>();
    const Comb combs[] = {
        {"cols16_t256", lib_rows, reinterpret_cast<const void*>(&probe::combine_cols<16, 256>), 16, 256},
        {"cols32_t256", lib_rows, reinterpret_cast<const void*>(&probe::combine_cols<32, 256>), 32, 256},
        {"cols64_t256", lib_rows, reinterpret_cast<const void*>(&probe::combine_cols<64, 256>), 64, 256},
        {"cols128_t256", lib_rows, reinterpret_cast<const void*>(&probe::combine_cols<128, 256>), 128, 256},
        {"cols32_t512", lib_rows, reinterpret_cast<const void*>(&probe::combine_cols<32, 512>), 32, 512},
        {"cols32_t1024", lib_rows, reinterpret_cast<const void*>(&probe::combine_cols<32, 1024>), 32, 1024},
        {"cols64_t1024", lib_rows, reinterpret_cast<const void*>(&probe::combine_cols<64, 1024>), 64, 1024},
        {"nt_rows_cols32_t256", nt_rows, reinterpret_cast<const void*>(&probe::combine_cols<32, 256>), 32, 256},
        {"nt_rows_cols64_t1024", nt_rows, reinterpret_cast<const void*>(&probe::combine_cols<64, 1024>), 64, 1024},
    };
    first = true;
    for (const Comb& cb : combs) {
        auto vjp2 = [&](int s) {
            launch(cb.rows, s);
            const float* pp = partial;
            float* dd = dw;
            int nbv = nb, dv = static_cast<int>(D);
            void* args[] = {&pp, &dd, &nbv, &dv};
            CK(hipLaunchKernel(cb.comb, dim3(static_cast<unsigned>(D / cb.cols)), dim3(cb.threads), args, 0, st));
        };
        const double t_vjp = timed(vjp2);
        const double t_step = timed([&](int s) {
            fwd(s);
            vjp2(s);
        });
        vjp2(0);
        CK(hipStreamSynchronize(st));
        CK(hipMemcpy(dw_a.data(), dw, D * 4, hipMemcpyDeviceToHost));
        double md = 0;
        for (int j = 0; j < D; ++j) md = std::max(md, (double)std::fabs(dw_a[j] - dw_lib[j]));
        printf("%s{\"name\": \"%s\", \"vjp_us\": %.3f, \"step_us\": %.3f, \"step_GBps\": %.1f, "
               "\"dw_rel_diff_vs_library\": %.3g}",
               first ? "" : ", ", cb.name, t_vjp, t_step, 335577088.0 / (t_step * 1e-6) / 1e9, md / dwmax);
        first = false;
        fflush(stdout);
    }
    printf("]}\n");
    return 0;
}
