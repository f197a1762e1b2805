// fetch_calibration.hip -- measurement program (not part of the library):
// kernels that move a known number of bytes in the access shapes the RMSNorm
// kernels use, so that rocprofv3's FETCH_SIZE and WRITE_SIZE (per dispatch)
// can be scaled to bytes per access shape:
//
//   read_lines      every byte of 64 MiB read once with 16-byte loads,
//                   consecutive lanes on consecutive vectors (whole 128-byte
//                   lines: the row kernels' loads);
//   read_halves     the first 64 bytes of every 128-byte line of 128 MiB (64
//                   MiB read, in 64-byte pieces, the other half never);
//   read_split      every byte of 64 MiB read once in 64-byte pieces, the two
//                   halves of each line by two different blocks (the dw
//                   combine's pattern: a block reads 16 columns of fp32);
//   write_lines     every byte of 64 MiB written once with 16-byte stores
//                   (whole lines: the row kernels' stores).
//
// Each kernel is launched 4 times on fresh regions of a 1 GiB pool (nothing
// is served from a cache); run under
//   rocprofv3 --pmc FETCH_SIZE -- benchsrc/bin/fetch_calibration
//   rocprofv3 --pmc WRITE_SIZE -- benchsrc/bin/fetch_calibration
// and divide the bytes printed per kernel by the counter's value per dispatch.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define CK(x)                                                                             \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

// The xor of everything read lands in sink only under a condition the data
// never meets, so the loads cannot be removed and nothing extra is written.
__device__ __forceinline__ void keep(u32x4 acc, u32x4* sink) {
    if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) sink[threadIdx.x] = acc;
}

// n16: 16-byte vectors in the region; grid-stride over them.
__global__ void read_lines(const u32x4* __restrict__ src, size_t n16, u32x4* sink) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        acc ^= src[i];
    keep(acc, sink);
}

// nlines: 128-byte lines in the region; 4 lanes read the first 64 bytes of
// one line.
__global__ void read_halves(const u32x4* __restrict__ src, size_t nlines, u32x4* sink) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    const size_t n = nlines * 4;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        acc ^= src[(i / 4) * 8 + (i % 4)];
    keep(acc, sink);
}

// nlines: 128-byte lines; block pair (2p, 2p + 1) covers the same lines, the
// even block the first half of each, the odd block the second.
__global__ void read_split(const u32x4* __restrict__ src, size_t nlines, u32x4* sink) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    const size_t half = blockIdx.x & 1;
    const size_t pairs = gridDim.x / 2;
    const size_t n = nlines * 4;
    for (size_t i = (blockIdx.x / 2) * (size_t)blockDim.x + threadIdx.x; i < n; i += pairs * blockDim.x)
        acc ^= src[(i / 4) * 8 + half * 4 + (i % 4)];
    keep(acc, sink);
}

__global__ void write_lines(u32x4* __restrict__ dst, size_t n16) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        dst[i] = u32x4{static_cast<uint32_t>(i), 1u, 2u, 3u};
}

int main() {
    const size_t pool = size_t(1) << 30, mib64 = size_t(64) << 20;
    u32x4 *buf, *sink;
    // one chunk of slack: a region of two chunks may start at the last chunk
    CK(hipMalloc(&buf, pool + mib64));
    CK(hipMalloc(&sink, 1024 * sizeof(u32x4)));
    CK(hipMemset(buf, 1, pool + mib64));
    CK(hipDeviceSynchronize());
    const dim3 grid(8192), block(256);
    // regions: 16 chunks of 64 MiB; each launch takes new chunks
    size_t chunk = 0;
    auto at = [&](size_t chunks) {
        u32x4* p = buf + (chunk % 16) * (mib64 / 16);
        chunk += chunks;
        return p;
    };
    for (int rep = 0; rep < 4; ++rep) {
        read_lines<<<grid, block>>>(at(1), mib64 / 16, sink);
        read_halves<<<grid, block>>>(at(2), (2 * mib64) / 128, sink);
        read_split<<<grid, block>>>(at(1), mib64 / 128, sink);
        write_lines<<<grid, block>>>(at(1), mib64 / 16);
    }
    CK(hipDeviceSynchronize());
    printf("read_lines bytes_read=%zu\n", mib64);
    printf("read_halves bytes_read=%zu\n", mib64);
    printf("read_split bytes_read=%zu\n", mib64);
    printf("write_lines bytes_written=%zu\n", mib64);
    return 0;
}
