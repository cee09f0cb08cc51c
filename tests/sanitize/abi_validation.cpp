// Host-only build of liblq's C ABI layer (lq_api.hip) with its kernel
// launchers and the two HIP runtime calls it makes replaced by counting stubs,
// so every entry point's argument checks and the blob layout run under
// AddressSanitizer and UndefinedBehaviorSanitizer on the CPU.  Test
// infrastructure: built and run by tests/test_sanitizers.py.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "lq_internal.h"

namespace lq {
int g_launches = 0;
hipError_t launch_decode_q8(const DecodeArgs&, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode_fp32(const Fp32DecodeArgs&, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_materialize(const MatArgs&, int, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_clear_status(uint32_t*, hipStream_t) { ++g_launches; return hipSuccess; }
alignas(256) int32_t g_scratch[16];
hipError_t scratch_work_list(int32_t** out) { *out = g_scratch; return hipSuccess; }
}  // namespace lq

// the runtime calls of lq_read_status: the device address is never touched
hipError_t hipMemcpyAsync(void* dst, const void*, size_t n, hipMemcpyKind, hipStream_t) {
    std::memset(dst, 0, n);
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

static int g_fail = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
            ++g_fail;                                                       \
        }                                                                   \
    } while (0)

static lq_config base() {
    lq_config c{};
    c.n_seq = 3; c.n_v_heads = 4; c.n_k_heads = 2; c.d_k = 128; c.d_v = 128;
    c.window = 64; c.n_comp = 4; c.gate_kind = LQ_GATE_SCALAR;
    c.code_format = LQ_CODE_INT8; c.buffer_format = LQ_BUFFER_FP32;
    return c;
}

static void check_layout(const lq_config& c) {
    lq_layout L{};
    EXPECT(lq_state_layout(&c, &L) == LQ_OK);
    const size_t off[] = {L.status, L.fill, L.codes, L.sigma, L.smooth, L.comp_idx, L.comp_vec,
                          L.buf_k, L.buf_v, L.buf_beta, L.buf_gate, L.work, L.total_bytes};
    for (size_t i = 0; i + 1 < sizeof(off) / sizeof(off[0]); ++i) {
        EXPECT(off[i] % 256 == 0);
        EXPECT(off[i] <= off[i + 1]);
    }
    const size_t U = (size_t)c.n_seq * c.n_v_heads;
    EXPECT(L.codes - L.fill >= U * 4);
    EXPECT(L.sigma - L.codes >= U * c.d_v * c.d_k);
    EXPECT(L.total_bytes - L.work >= (U + 1) * 4);
    size_t b = 0;
    EXPECT(lq_state_bytes(&c, &b) == LQ_OK && b == L.total_bytes);
}

int main() {
    alignas(256) static unsigned char blob[1 << 12];
    alignas(16) static float buf[64];
    void* st = blob;
    const float* f = buf;
    float* o = buf;
    uint32_t flags = 7;

    // configurations: every field's limits, and inconsistent ones
    lq_config c = base();
    EXPECT(lq_state_bytes(nullptr, nullptr) == LQ_EINVAL);
    int variants = 0;
    for (int d : {64, 128})
        for (int gk : {0, 1})
            for (int fmt : {0, 1})
                for (int bf : {0, 1})
                    for (int W : {1, 17, 128, 256})
                        for (int nc : {0, 1, 16}) {
                            lq_config x = base();
                            x.d_k = x.d_v = d; x.gate_kind = gk; x.code_format = fmt;
                            x.buffer_format = bf; x.window = W; x.n_comp = nc;
                            check_layout(x);
                            ++variants;
                        }
    lq_config x = base(); x.d_k = 96; x.d_v = 96; EXPECT(lq_state_bytes(&x, nullptr) == LQ_EUNSUPPORTED || lq_state_bytes(&x, nullptr) == LQ_EINVAL);
    size_t nb = 0;
    x = base(); x.d_k = 64; EXPECT(lq_state_bytes(&x, &nb) == LQ_EUNSUPPORTED);
    x = base(); x.window = 0; EXPECT(lq_state_bytes(&x, &nb) == LQ_EINVAL);
    x = base(); x.window = 257; EXPECT(lq_state_bytes(&x, &nb) == LQ_EUNSUPPORTED);
    x = base(); x.n_comp = -1; EXPECT(lq_state_bytes(&x, &nb) == LQ_EINVAL);
    x = base(); x.n_comp = 17; EXPECT(lq_state_bytes(&x, &nb) == LQ_EUNSUPPORTED);
    x = base(); x.n_k_heads = 3; EXPECT(lq_state_bytes(&x, &nb) == LQ_EINVAL);
    x = base(); x.gate_kind = 2; EXPECT(lq_state_bytes(&x, &nb) == LQ_EINVAL);
    x = base(); x.code_format = -1; EXPECT(lq_state_bytes(&x, &nb) == LQ_EINVAL);
    x = base(); x.buffer_format = 9; EXPECT(lq_state_bytes(&x, &nb) == LQ_EINVAL);
    x = base(); x.flush_cus = -1; EXPECT(lq_state_bytes(&x, &nb) == LQ_EINVAL);
    x = base(); x.flush_cus = 100000; EXPECT(lq_state_bytes(&x, &nb) == LQ_OK);
    x = base(); x.n_seq = 0; EXPECT(lq_state_bytes(&x, &nb) == LQ_EINVAL);
    x = base(); x.n_seq = 1 << 30; x.n_v_heads = 4; x.n_k_heads = 4; EXPECT(lq_state_bytes(&x, &nb) == LQ_EUNSUPPORTED);
    x = base(); x.n_seq = (1 << 20); x.n_v_heads = 2047; x.n_k_heads = 1;  // just under 2^31 units
    check_layout(x);

    // entry points: nulls and misalignment are rejected before any launch
    lq::g_launches = 0;
    const float* mis = buf + 1;  // 4-byte aligned only
    void* st_mis = blob + 16;
    EXPECT(lq_state_init(&c, nullptr, f, nullptr) == LQ_EINVAL);
    EXPECT(lq_state_init(&c, st_mis, f, nullptr) == LQ_EINVAL);
    EXPECT(lq_state_init(&c, st, mis, nullptr) == LQ_EINVAL);
    EXPECT(lq_decode_step(&c, st, nullptr, f, f, f, f, o, nullptr) == LQ_EINVAL);
    EXPECT(lq_decode_step(&c, st, mis, f, f, f, f, o, nullptr) == LQ_EINVAL);
    EXPECT(lq_decode_step(&c, st, f, f, f, f, f, nullptr, nullptr) == LQ_EINVAL);
    EXPECT(lq_fp32_decode_step(&c, nullptr, f, f, f, f, f, o, nullptr) == LQ_EINVAL);
    EXPECT(lq_window_flush(&c, st_mis, nullptr, nullptr) == LQ_EINVAL);
    EXPECT(lq_dequant_state(&c, st, nullptr, 1, nullptr) == LQ_EINVAL);
    EXPECT(lq_prefill(&c, st, nullptr, -1, f, f, f, f, f, o, nullptr) == LQ_EINVAL);
    EXPECT(lq_prefill(&c, st, nullptr, 5, nullptr, f, f, f, f, o, nullptr) == LQ_EINVAL);
    EXPECT(lq_read_status(&c, st, nullptr, nullptr) == LQ_EINVAL);
    EXPECT(lq_clear_status(&c, st_mis, nullptr) == LQ_EINVAL);
    EXPECT(lq_decode_step(nullptr, st, f, f, f, f, f, o, nullptr) == LQ_EINVAL);
    EXPECT(lq::g_launches == 0);

    // valid calls reach their launchers
    EXPECT(lq_state_init(&c, st, nullptr, nullptr) == LQ_OK);
    EXPECT(lq_state_init(&c, st, f, nullptr) == LQ_OK);
    EXPECT(lq_decode_step(&c, st, f, f, f, f, f, o, nullptr) == LQ_OK);
    EXPECT(lq_fp32_decode_step(&c, o, f, f, f, f, f, o, nullptr) == LQ_OK);
    EXPECT(lq_window_flush(&c, st, nullptr, nullptr) == LQ_OK);
    EXPECT(lq_dequant_state(&c, st, o, 0, nullptr) == LQ_OK);
    EXPECT(lq_prefill(&c, st, nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == LQ_OK);
    EXPECT(lq_prefill(&c, st, f, 7, f, f, f, f, f, o, nullptr) == LQ_OK);
    EXPECT(lq_clear_status(&c, st, nullptr) == LQ_OK);
    EXPECT(lq_read_status(&c, st, &flags, nullptr) == LQ_OK && flags == 0);
    EXPECT(lq_window_flush_noalloc(&c, st, nullptr, nullptr) == LQ_OK);
    EXPECT(lq::g_launches == 10);
    // the allocation-free call: its unit limit and its argument checks launch nothing
    lq_config big = base();
    big.n_seq = LQ_NOALLOC_MAX_UNITS / 4 + 1;  // 4 value heads: one unit over the limit
    EXPECT(lq_window_flush_noalloc(&big, st, nullptr, nullptr) == LQ_ESCRATCH);
    big.n_seq = LQ_NOALLOC_MAX_UNITS / 4;
    EXPECT(lq_window_flush_noalloc(&big, st, nullptr, nullptr) == LQ_OK);
    EXPECT(lq_window_flush_noalloc(&c, nullptr, nullptr, nullptr) == LQ_EINVAL);
    EXPECT(lq_window_flush_noalloc(&c, st_mis, nullptr, nullptr) == LQ_EINVAL);
    EXPECT(lq::g_launches == 11);
    for (int code : {0, -1, -2, -3, -4, 5, -100}) EXPECT(std::strlen(lq_strerror(code)) > 0);

    if (g_fail) return 1;
    std::printf("abi validation: %d layouts, all checks passed\n", variants);
    return 0;
}
