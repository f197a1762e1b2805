// stream_ceiling.hip -- measurement tool (not part of the library): the HBM
// throughput trivial streaming kernels reach on this GPU for the traffic
// mixes of the RMSNorm kernels, on buffers far larger than the last-level
// cache:  1 read + 1 write (forward), 2 reads + 1 write (VJP), 2 reads +
// 2 writes (fused forward, grad call), 3 reads + 1 write (fused backward).
// Each stream is `bytes` long; streams are consecutive `bytes`-sized chunks
// of a 4 GiB pool, and each launch moves on to the next chunks, so a chunk is
// touched again only after >= 1 GiB of other traffic (nothing is served from
// the 256 MB last-level cache).  Prints one line per (mix, stream size,
// block, grid): best and median of 14 timed launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void k11(const u32x4* __restrict__ a, u32x4* __restrict__ c, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        c[i] = a[i];
}
__global__ void k21(const u32x4* __restrict__ a, const u32x4* __restrict__ b, u32x4* __restrict__ c, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        c[i] = a[i] ^ b[i];
}
__global__ void k22(const u32x4* __restrict__ a, const u32x4* __restrict__ b, u32x4* __restrict__ c,
                    u32x4* __restrict__ d, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const u32x4 x = a[i], y = b[i];
        c[i] = x ^ y;
        d[i] = x + y;
    }
}
__global__ void k31(const u32x4* __restrict__ a, const u32x4* __restrict__ b, const u32x4* __restrict__ e,
                    u32x4* __restrict__ c, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        c[i] = a[i] ^ b[i] ^ e[i];
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
        for (const auto& sh : shapes) {
            const int bs = sh[0], grid = sh[1];
            const int g = grid ? grid : (int)((n + bs - 1) / bs);
            for (int mix = 0; mix < 4; ++mix) {
                std::vector<float> t;
                for (int r = 0; r < 16; ++r) {
                    u32x4* p[4];
                    for (int q = 0; q < 4; ++q) p[q] = (u32x4*)(pool + ((r * 4 + q) % chunks) * bytes);
                    CHECK(hipEventRecord(e0));
                    if (mix == 0) hipLaunchKernelGGL(k11, dim3(g), dim3(bs), 0, 0, p[0], p[1], n);
                    if (mix == 1) hipLaunchKernelGGL(k21, dim3(g), dim3(bs), 0, 0, p[0], p[1], p[2], n);
                    if (mix == 2) hipLaunchKernelGGL(k22, dim3(g), dim3(bs), 0, 0, p[0], p[1], p[2], p[3], n);
                    if (mix == 3) hipLaunchKernelGGL(k31, dim3(g), dim3(bs), 0, 0, p[0], p[1], p[2], p[3], n);
                    CHECK(hipGetLastError());
                    CHECK(hipEventRecord(e1));
                    CHECK(hipEventSynchronize(e1));
                    float ms = 0.0f;
                    CHECK(hipEventElapsedTime(&ms, e0, e1));
                    if (r >= 2) t.push_back(ms);
                }
                std::sort(t.begin(), t.end());
                const double best = t.front(), med = t[t.size() / 2];
                std::printf("mix=%s stream_MiB=%lld block=%d grid=%d best_us=%.2f med_us=%.2f GBps=%.0f GBps_med=%.0f\n",
                            names[mix], (long long)(bytes >> 20), bs, g, best * 1e3, med * 1e3,
                            streams[mix] * (double)bytes / (best * 1e-3) / 1e9,
                            streams[mix] * (double)bytes / (med * 1e-3) / 1e9);
            }
        }
    }
    CHECK(hipFree(pool));
    return 0;
}
