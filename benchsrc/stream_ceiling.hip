// stream_ceiling.hip -- measurement tool (not part of the library): the HBM
// throughput trivial streaming kernels reach on this GPU for the traffic
// mixes of the RMSNorm kernels, on buffers far larger than the last-level
// cache:  1 read + 1 write (forward), 2 reads + 1 write (VJP), 2 reads +
// 2 writes (fused forward, grad call), 3 reads + 1 write (fused backward).
// Each stream is `bytes` long; streams are consecutive `bytes`-sized chunks
// of a 4 GiB pool, and each launch moves on to the next chunks, so a chunk is
// touched again only after >= 1 GiB of other traffic (nothing is served from
// the 256 MB last-level cache).  Prints one line per (mix, cache policy,
// stream size, block, grid): best and median of 14 timed launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// NT: non-temporal loads and stores (the "nt" cache-policy bit), as the
// library's kernels use for row traffic; otherwise the default policy.
template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
}
template <bool NT>
__device__ __forceinline__ void st(u32x4* p, u32x4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <bool NT>
__global__ void k11(const u32x4* __restrict__ a, u32x4* __restrict__ c, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        st<NT>(c + i, ld<NT>(a + i));
}
template <bool NT>
__global__ void k21(const u32x4* __restrict__ a, const u32x4* __restrict__ b, u32x4* __restrict__ c, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        st<NT>(c + i, ld<NT>(a + i) ^ ld<NT>(b + i));
}
template <bool NT>
__global__ void k22(const u32x4* __restrict__ a, const u32x4* __restrict__ b, u32x4* __restrict__ c,
                    u32x4* __restrict__ d, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const u32x4 x = ld<NT>(a + i), y = ld<NT>(b + i);
        st<NT>(c + i, x ^ y);
        st<NT>(d + i, x + y);
    }
}
template <bool NT>
__global__ void k31(const u32x4* __restrict__ a, const u32x4* __restrict__ b, const u32x4* __restrict__ e,
                    u32x4* __restrict__ c, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        st<NT>(c + i, ld<NT>(a + i) ^ ld<NT>(b + i) ^ ld<NT>(e + i));
}

template <bool NT>
void launch(int mix, int g, int bs, u32x4* const (&p)[4], int64_t n) {
    if (mix == 0) hipLaunchKernelGGL(k11<NT>, dim3(g), dim3(bs), 0, 0, p[0], p[1], n);
    if (mix == 1) hipLaunchKernelGGL(k21<NT>, dim3(g), dim3(bs), 0, 0, p[0], p[1], p[2], n);
    if (mix == 2) hipLaunchKernelGGL(k22<NT>, dim3(g), dim3(bs), 0, 0, p[0], p[1], p[2], p[3], n);
    if (mix == 3) hipLaunchKernelGGL(k31<NT>, dim3(g), dim3(bs), 0, 0, p[0], p[1], p[2], p[3], n);
}

#define CHECK(x)                                                                   \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));   \
            return 1;                                                              \
        }                                                                          \
    } while (0)

int main() {
    const int64_t kPool = 4LL << 30;
    char* pool = nullptr;
    CHECK(hipMalloc(&pool, kPool));
    CHECK(hipMemset(pool, 1, kPool));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    const char* names[4] = {"1R1W", "2R1W", "2R2W", "3R1W"};
    const int streams[4] = {2, 3, 4, 4};
    for (int64_t bytes : {64LL << 20, 512LL << 20}) {
        const int64_t n = bytes / 16;
        const int64_t chunks = kPool / bytes;
        // (block, grid): grid 0 = one 16-byte element per thread
        const int shapes[5][2] = {{256, 2048}, {256, 8192}, {256, 0}, {64, 0}, {1024, 0}};
        for (const auto& sh : shapes)
        for (int nt = 0; nt < 2; ++nt) {
            const int bs = sh[0], grid = sh[1];
            const int g = grid ? grid : (int)((n + bs - 1) / bs);
            for (int mix = 0; mix < 4; ++mix) {
                std::vector<float> t;
                for (int r = 0; r < 16; ++r) {
                    u32x4* p[4];
                    for (int q = 0; q < 4; ++q) p[q] = (u32x4*)(pool + ((r * 4 + q) % chunks) * bytes);
                    CHECK(hipEventRecord(e0));
                    if (nt) launch<true>(mix, g, bs, p, n);
                    else launch<false>(mix, g, bs, p, n);
                    CHECK(hipGetLastError());
                    CHECK(hipEventRecord(e1));
                    CHECK(hipEventSynchronize(e1));
                    float ms = 0.0f;
                    CHECK(hipEventElapsedTime(&ms, e0, e1));
                    if (r >= 2) t.push_back(ms);
                }
                std::sort(t.begin(), t.end());
                const double best = t.front(), med = t[t.size() / 2];
                std::printf("mix=%s policy=%s stream_MiB=%lld block=%d grid=%d best_us=%.2f med_us=%.2f GBps=%.0f "
                            "GBps_med=%.0f\n",
                            names[mix], nt ? "nt" : "default", (long long)(bytes >> 20), bs, g, best * 1e3, med * 1e3,
                            streams[mix] * (double)bytes / (best * 1e-3) / 1e9,
                            streams[mix] * (double)bytes / (med * 1e-3) / 1e9);
            }
        }
    }
    CHECK(hipFree(pool));
    return 0;
}
