// stream_read -- the device's practical streaming-read rate, the yardstick
// beside the published HBM peak for the bandwidth-bound decode kernel.
//
// Every thread reads 16-byte words grid-stride (eight loads in flight per
// unrolled step), folds them with XOR and writes one word, so the only
// traffic is the read itself.  For each byte count given on the command line
// (default: 56 MiB, 256 MiB, 1 GiB, 4 GiB) and each grid size it prints one
// JSON line with the mean launch time over repeated back-to-back launches
// (HIP events around them, launch gaps included).  Consecutive launches read
// disjoint regions of a pool of at least 2 GiB (and at least four regions),
// so no launch finds its bytes in the 256 MB last-level cache: the rate is
// the HBM streaming rate.  Not part of the library: built beside it, run by
// profiling.py and bench.py.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

__global__ __launch_bounds__(256) void stream_read(const uint4* __restrict__ p, size_t n16,
                                                   uint32_t* __restrict__ out) {
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * 256;
    uint32_t acc = 0;
#pragma unroll 8
    for (; i < n16; i += stride) {
        const uint4 w = p[i];
        acc ^= w.x ^ w.y ^ w.z ^ w.w;
    }
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

bool ok(hipError_t e, const char* what) {
    if (e == hipSuccess) return true;
    std::fprintf(stderr, "stream_read: %s: %s\n", what, hipGetErrorString(e));
    return false;
}

}  // namespace

int main(int argc, char** argv) {
    std::vector<size_t> sizes;
    for (int i = 1; i < argc; ++i) {
        const size_t sz = (size_t)std::strtoull(argv[i], nullptr, 10) & ~(size_t)15;
        if (sz >= 16) sizes.push_back(sz);  // at least one 16-byte word
    }
    if (sizes.empty()) sizes = {(size_t)56 << 20, (size_t)256 << 20, (size_t)1 << 30, (size_t)4 << 30};
    constexpr size_t kMinPool = (size_t)2 << 30;  // far above the 256 MB last-level cache
    size_t pool = kMinPool;
    for (size_t s : sizes) pool = 4 * s > pool ? 4 * s : pool;
    const int grids[] = {1024, 2048, 4096, 8192};
    uint4* p = nullptr;
    uint32_t* out = nullptr;
    if (!ok(hipMalloc(&p, pool), "hipMalloc") || !ok(hipMalloc(&out, (size_t)8192 * 256 * 4), "hipMalloc") ||
        !ok(hipMemset(p, 1, pool), "hipMemset"))
        return 1;
    hipEvent_t a, b;
    if (!ok(hipEventCreate(&a), "event") || !ok(hipEventCreate(&b), "event")) return 1;
    for (size_t sz : sizes) {
        // launch r reads region r mod n_reg of the pool (regions of sz bytes,
        // 16-byte aligned: sz is a multiple of 16)
        const size_t n_reg = pool / sz;
        auto region = [&](int r) { return p + (size_t)(r % (int)n_reg) * (sz / 16); };
        for (int g : grids) {
            const size_t n16 = sz / 16;
            for (int w = 0; w < 3; ++w) hipLaunchKernelGGL(stream_read, dim3(g), dim3(256), 0, 0, region(w), n16, out);
            const int reps = sz >= ((size_t)1 << 30) ? 10 : 50;
            if (!ok(hipEventRecord(a), "record")) return 1;
            for (int r = 0; r < reps; ++r)
                hipLaunchKernelGGL(stream_read, dim3(g), dim3(256), 0, 0, region(r + 3), n16, out);
            if (!ok(hipEventRecord(b), "record") || !ok(hipEventSynchronize(b), "sync")) return 1;
            float ms = 0.f;
            if (!ok(hipEventElapsedTime(&ms, a, b), "elapsed")) return 1;
            const double us = ms * 1e3 / reps;
            std::printf("{\"bytes\": %zu, \"grid\": %d, \"us\": %.2f, \"TBps\": %.3f, \"pool_bytes\": %zu, "
                        "\"regions\": %zu}\n",
                        sz, g, us, sz / us * 1e-6, pool, n_reg);
            std::fflush(stdout);
        }
    }
    return ok(hipGetLastError(), "launch") ? 0 : 1;
}
