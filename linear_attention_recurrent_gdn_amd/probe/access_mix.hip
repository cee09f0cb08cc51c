// access_mix -- the device's rate for the decode step's memory mix, the
// second yardstick beside stream_read (which only reads).
//
// One workgroup of 256 threads per unit, the accesses a decode step makes for
// a unit with an empty window at d = 128, 4 compensator lines and two value
// heads per key head, and nothing else: a 16 KiB tile read by the whole
// workgroup; five 512-byte vectors (q, k, v, scales, smoothing), 2 KiB of
// compensator lines and two 256-byte window rows read by one wavefront; and,
// in the modes that write, the 512-byte writes (the appended value, the
// appended key for every other unit, the output) and three 4-byte writes.
// Modes: 0 reads only; 1 reads and writes; 2 as 1 with the 512-byte writes
// non-temporal.  Consecutive launches use disjoint copies of every array
// (more than 1 GiB in all), so no launch finds its data in the 256 MB
// last-level cache.  For each mode it prints one JSON line: mean launch time
// over back-to-back launches (HIP events, launch gaps included), bytes read
// and written per launch, and the rate.  Not part of the library: built
// beside it, run by profiling.py and bench.py.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

struct Arrays {
    const uint4* tile;   // [U][1024]
    const float* side;   // [5][U][128]
    const float* comp;   // [U][4][128]
    const float* win;    // [2][U][64]
    float* wbuf;         // [2][U][128]
    float* wsmall;       // [3][U]
    float* out;          // [U][128]
    uint32_t* sink;      // [256]
    int U;
};

template <int MODE>
__global__ __launch_bounds__(256) void unit_mix(Arrays p) {
    const int u = blockIdx.x, t = threadIdx.x, w = t / 64, l = t % 64;
    uint32_t acc = 0;
    const uint4* tl = p.tile + (size_t)u * 1024;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 x = tl[i * 256 + t];
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
    float f = 0.f;
    if (w == 0) {
#pragma unroll
        for (int s = 0; s < 5; ++s) {
            const float2 x = *reinterpret_cast<const float2*>(p.side + ((size_t)s * p.U + u) * 128 + 2 * l);
            f += x.x + x.y;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float2 x = *reinterpret_cast<const float2*>(p.comp + ((size_t)u * 4 + c) * 128 + 2 * l);
            f += x.x + x.y;
        }
        f += p.win[(size_t)u * 64 + l] + p.win[((size_t)p.U + u) * 64 + l];
        if constexpr (MODE >= 1) {
            float* dst[3] = {p.wbuf + (size_t)u * 128 + 2 * l, p.wbuf + ((size_t)p.U + u) * 128 + 2 * l,
                             p.out + (size_t)u * 128 + 2 * l};
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                if (i == 1 && (u & 1)) continue;  // the key: once per two value heads
                if constexpr (MODE == 2) {
                    __builtin_nontemporal_store(f, dst[i]);
                    __builtin_nontemporal_store(f, dst[i] + 1);
                } else {
                    *reinterpret_cast<float2*>(dst[i]) = make_float2(f, f);
                }
            }
            if (l == 0) {
                p.wsmall[u] = f;
                p.wsmall[p.U + u] = f;
                p.wsmall[2 * p.U + u] = f;
            }
        }
    }
    if (acc == 0x9e3779b9u && f == 1.25f) p.sink[t] = acc;  // keeps the loads
}

bool ok(hipError_t e, const char* what) {
    if (e == hipSuccess) return true;
    std::fprintf(stderr, "access_mix: %s: %s\n", what, hipGetErrorString(e));
    return false;
}

}  // namespace

int main(int argc, char** argv) {
    const int U = argc > 1 ? std::atoi(argv[1]) : 8192;
    if (U < 1 || U > (1 << 20)) {
        std::fprintf(stderr, "access_mix: unit count out of range\n");
        return 2;
    }
    const size_t tileB = (size_t)U * 16384, sideB = (size_t)5 * U * 512, compB = (size_t)U * 2048,
                 winB = (size_t)2 * U * 256, wbufB = (size_t)2 * U * 512, wsB = (size_t)3 * U * 4,
                 outB = (size_t)U * 512;
    const size_t per_copy = tileB + sideB + compB + winB + wbufB + wsB + outB;
    const int R = (int)((((size_t)1 << 30) + per_copy - 1) / per_copy) + 1;  // > 1 GiB in all
    uint32_t* sink = nullptr;
    if (!ok(hipMalloc(&sink, 256 * 4), "hipMalloc")) return 1;
    std::vector<Arrays> cp(R);
    for (int r = 0; r < R; ++r) {
        char* b = nullptr;
        if (!ok(hipMalloc(&b, per_copy + 7 * 256), "hipMalloc") || !ok(hipMemset(b, 1, per_copy + 7 * 256), "hipMemset"))
            return 1;
        size_t off = 0;
        auto take = [&](size_t n) { char* q = b + off; off += (n + 255) / 256 * 256; return q; };
        cp[r] = Arrays{(const uint4*)take(tileB), (const float*)take(sideB), (const float*)take(compB),
                       (const float*)take(winB), (float*)take(wbufB), (float*)take(wsB), (float*)take(outB),
                       sink, U};
    }
    hipEvent_t a, e;
    if (!ok(hipEventCreate(&a), "event") || !ok(hipEventCreate(&e), "event")) return 1;
    const double rd = (double)tileB + sideB + compB + winB;
    for (int mode = 0; mode < 3; ++mode) {
        const double wr = mode == 0 ? 0.0 : (double)U * 512 * 2 + (double)((U + 1) / 2) * 512 + 12.0 * U;
        auto launch = [&](int r) {
            if (mode == 0) hipLaunchKernelGGL(unit_mix<0>, dim3(U), dim3(256), 0, 0, cp[r % R]);
            else if (mode == 1) hipLaunchKernelGGL(unit_mix<1>, dim3(U), dim3(256), 0, 0, cp[r % R]);
            else hipLaunchKernelGGL(unit_mix<2>, dim3(U), dim3(256), 0, 0, cp[r % R]);
        };
        for (int r = 0; r < R; ++r) launch(r);
        const int reps = 40;
        if (!ok(hipEventRecord(a), "record")) return 1;
        for (int r = 0; r < reps; ++r) launch(r);
        if (!ok(hipEventRecord(e), "record") || !ok(hipEventSynchronize(e), "sync")) return 1;
        float ms = 0.f;
        if (!ok(hipEventElapsedTime(&ms, a, e), "elapsed")) return 1;
        const double us = ms * 1e3 / reps;
        std::printf("{\"mode\": %d, \"units\": %d, \"us\": %.2f, \"read_bytes\": %.0f, \"write_bytes\": %.0f, "
                    "\"TBps\": %.3f, \"copies\": %d}\n",
                    mode, U, us, rd, wr, (rd + wr) / us * 1e-6, R);
        std::fflush(stdout);
    }
    return ok(hipGetLastError(), "launch") ? 0 : 1;
}
