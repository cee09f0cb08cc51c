// lq_api.hip -- the extern "C" entry points of liblq.so: argument checks,
// blob layout, kernel launches.  Every check runs on the host before any HIP
// call, so a rejected call launches nothing (and needs no GPU).

#include <hip/hip_runtime.h>

#include "lq_internal.h"

using namespace lq;

namespace {

int32_t check_config(const lq_config* c) {
    if (c == nullptr) return LQ_EINVAL;
    if (c->n_seq < 1 || c->n_v_heads < 1 || c->n_k_heads < 1 || c->d_k < 1 || c->d_v < 1 ||
        c->window < 1 || c->n_comp < 0)
        return LQ_EINVAL;
    if (c->n_v_heads % c->n_k_heads != 0) return LQ_EINVAL;
    if (c->gate_kind != LQ_GATE_SCALAR && c->gate_kind != LQ_GATE_CHANNEL) return LQ_EINVAL;
    if (c->code_format != LQ_CODE_INT8 && c->code_format != LQ_CODE_E4M3) return LQ_EINVAL;
    if (c->buffer_format != LQ_BUFFER_FP32 && c->buffer_format != LQ_BUFFER_FP16 &&
        c->buffer_format != LQ_BUFFER_NFORM)
        return LQ_EINVAL;
    if (c->flush_cus < 0) return LQ_EINVAL;
    if (c->load_policy != LQ_LOADS_AUTO && c->load_policy != LQ_LOADS_STREAM && c->load_policy != LQ_LOADS_CACHED)
        return LQ_EINVAL;
    if ((int64_t)c->n_seq * c->n_v_heads >= ((int64_t)1 << 31)) return LQ_EUNSUPPORTED;
    if (c->d_k != c->d_v || (c->d_k != 64 && c->d_k != 128)) return LQ_EUNSUPPORTED;
    if (c->window > 256 || c->n_comp > 16) return LQ_EUNSUPPORTED;
    if (c->buffer_format == LQ_BUFFER_NFORM && (c->gate_kind != LQ_GATE_SCALAR || c->d_k != 128))
        return LQ_EUNSUPPORTED;
    return LQ_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

Dims dims_of(const lq_config* c) {
    Dims d;
    d.n_units = c->n_seq * c->n_v_heads;
    d.n_v_heads = c->n_v_heads;
    d.n_k_heads = c->n_k_heads;
    d.group = c->n_v_heads / c->n_k_heads;
    d.window = c->window;
    d.n_comp = c->n_comp;
    d.code_format = c->code_format;
    d.buffer_format = c->buffer_format;
    d.max_cus = c->flush_cus;
    d.load_policy = c->load_policy;
    return d;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? LQ_OK : LQ_EHIP; }

}  // namespace

extern "C" {

int32_t lq_state_bytes(const lq_config* cfg, size_t* bytes) {
    int32_t rc = check_config(cfg);
    if (rc != LQ_OK) return rc;
    if (bytes == nullptr) return LQ_EINVAL;
    lq_layout L;
    compute_layout(*cfg, L);
    *bytes = L.total_bytes;
    return LQ_OK;
}

int32_t lq_state_layout(const lq_config* cfg, lq_layout* layout) {
    int32_t rc = check_config(cfg);
    if (rc != LQ_OK) return rc;
    if (layout == nullptr) return LQ_EINVAL;
    compute_layout(*cfg, *layout);
    return LQ_OK;
}

int32_t lq_state_init(const lq_config* cfg, void* state, const float* S0, hipStream_t stream) {
    int32_t rc = check_config(cfg);
    if (rc != LQ_OK) return rc;
    if (state == nullptr || !aligned(state, kSectionAlign)) return LQ_EINVAL;
    if (S0 != nullptr && !aligned(S0, 16)) return LQ_EINVAL;
    lq_layout L;
    compute_layout(*cfg, L);
    MatArgs a{};
    a.blob = blob_ptrs(state, L);
    a.dm = dims_of(cfg);
    a.S0 = S0;
    return hip_status(launch_materialize(a, kModeInit, cfg->d_k, cfg->gate_kind, stream));
}

int32_t lq_prefill(const lq_config* cfg, void* state, const float* S0, int32_t n_tok, const float* q,
                   const float* k, const float* v, const float* beta, const float* gate, float* o,
                   hipStream_t stream) {
    int32_t rc = check_config(cfg);
    if (rc != LQ_OK) return rc;
    if (state == nullptr || n_tok < 0) return LQ_EINVAL;
    // offsets inside a 16-token chunk of the prompt are 32-bit element counts
    if ((uint64_t)16 * cfg->n_seq * cfg->n_v_heads * cfg->d_k > 0xFFFFFFFFull) return LQ_EUNSUPPORTED;
    if (!aligned(state, kSectionAlign) || (S0 != nullptr && !aligned(S0, 16))) return LQ_EINVAL;
    if (n_tok > 0) {
        if (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || gate == nullptr)
            return LQ_EINVAL;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(beta, 4) ||
            !aligned(gate, cfg->gate_kind == LQ_GATE_CHANNEL ? 16 : 4) || (o != nullptr && !aligned(o, 16)))
            return LQ_EINVAL;
    }
    lq_layout L;
    compute_layout(*cfg, L);
    MatArgs a{};
    a.blob = blob_ptrs(state, L);
    a.dm = dims_of(cfg);
    a.S0 = S0;
    a.n_tok = n_tok;
    a.pq = q;
    a.pk = k;
    a.pv = v;
    a.pbeta = beta;
    a.pgate = gate;
    a.po = n_tok > 0 ? o : nullptr;
    return hip_status(launch_materialize(a, kModePrefill, cfg->d_k, cfg->gate_kind, stream));
}

int32_t lq_decode_step(const lq_config* cfg, void* state, const float* q, const float* k,
                       const float* v, const float* beta, const float* gate, float* o,
                       hipStream_t stream) {
    int32_t rc = check_config(cfg);
    if (rc != LQ_OK) return rc;
    if (state == nullptr || q == nullptr || k == nullptr || v == nullptr || beta == nullptr ||
        gate == nullptr || o == nullptr)
        return LQ_EINVAL;
    if (!aligned(state, kSectionAlign) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
        !aligned(beta, 4) || !aligned(gate, cfg->gate_kind == LQ_GATE_CHANNEL ? 16 : 4) ||
        !aligned(o, 16))
        return LQ_EINVAL;
    lq_layout L;
    compute_layout(*cfg, L);
    DecodeArgs a{};
    a.blob = blob_ptrs(state, L);
    a.dm = dims_of(cfg);
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.gate = gate;
    a.o = o;
    return hip_status(launch_decode_q8(a, cfg->d_k, cfg->gate_kind, stream));
}

int32_t lq_window_flush(const lq_config* cfg, void* state, const uint8_t* force_mask,
                        hipStream_t stream) {
    int32_t rc = check_config(cfg);
    if (rc != LQ_OK) return rc;
    if (state == nullptr || !aligned(state, kSectionAlign)) return LQ_EINVAL;
    lq_layout L;
    compute_layout(*cfg, L);
    MatArgs a{};
    a.blob = blob_ptrs(state, L);
    a.dm = dims_of(cfg);
    a.force = force_mask;
    return hip_status(launch_materialize(a, kModeFlush, cfg->d_k, cfg->gate_kind, stream));
}

int32_t lq_window_flush_noalloc(const lq_config* cfg, void* state, const uint8_t* force_mask,
                                hipStream_t stream) {
    int32_t rc = check_config(cfg);
    if (rc != LQ_OK) return rc;
    if (state == nullptr || !aligned(state, kSectionAlign)) return LQ_EINVAL;
    if ((int64_t)cfg->n_seq * cfg->n_v_heads > kScratchMaxUnits) return LQ_ESCRATCH;
    lq_layout L;
    compute_layout(*cfg, L);
    MatArgs a{};
    a.blob = blob_ptrs(state, L);
    a.dm = dims_of(cfg);
    a.force = force_mask;
    int32_t* work = nullptr;
    if (scratch_work_list(&work) != hipSuccess) return LQ_EHIP;
    a.blob.work = work;  // the library's array instead of the blob's work section
    return hip_status(launch_materialize(a, kModeFlush, cfg->d_k, cfg->gate_kind, stream));
}

int32_t lq_dequant_state(const lq_config* cfg, const void* state, float* S_out,
                         int32_t include_buffer, hipStream_t stream) {
    int32_t rc = check_config(cfg);
    if (rc != LQ_OK) return rc;
    if (state == nullptr || S_out == nullptr || !aligned(state, kSectionAlign) || !aligned(S_out, 16))
        return LQ_EINVAL;
    lq_layout L;
    compute_layout(*cfg, L);
    MatArgs a{};
    a.blob = blob_ptrs(const_cast<void*>(state), L);
    a.dm = dims_of(cfg);
    a.S_out = S_out;
    a.include_buffer = include_buffer != 0;
    return hip_status(launch_materialize(a, kModeDequant, cfg->d_k, cfg->gate_kind, stream));
}

int32_t lq_fp32_decode_step(const lq_config* cfg, float* S, const float* q, const float* k,
                            const float* v, const float* beta, const float* gate, float* o,
                            hipStream_t stream) {
    int32_t rc = check_config(cfg);
    if (rc != LQ_OK) return rc;
    if (S == nullptr || q == nullptr || k == nullptr || v == nullptr || beta == nullptr ||
        gate == nullptr || o == nullptr)
        return LQ_EINVAL;
    if (!aligned(S, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(beta, 4) ||
        !aligned(gate, cfg->gate_kind == LQ_GATE_CHANNEL ? 16 : 4) || !aligned(o, 4))
        return LQ_EINVAL;
    Fp32DecodeArgs a{};
    a.dm = dims_of(cfg);
    a.S = S;
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.gate = gate;
    a.o = o;
    return hip_status(launch_decode_fp32(a, cfg->d_k, cfg->gate_kind, stream));
}

int32_t lq_read_status(const lq_config* cfg, const void* state, uint32_t* flags, hipStream_t stream) {
    int32_t rc = check_config(cfg);
    if (rc != LQ_OK) return rc;
    if (state == nullptr || flags == nullptr || !aligned(state, kSectionAlign)) return LQ_EINVAL;
    lq_layout L;
    compute_layout(*cfg, L);
    const uint32_t* dev = (const uint32_t*)((const char*)state + L.status);
    if (hipMemcpyAsync(flags, dev, sizeof(uint32_t), hipMemcpyDeviceToHost, stream) != hipSuccess)
        return LQ_EHIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return LQ_EHIP;
    return LQ_OK;
}

int32_t lq_clear_status(const lq_config* cfg, void* state, hipStream_t stream) {
    int32_t rc = check_config(cfg);
    if (rc != LQ_OK) return rc;
    if (state == nullptr || !aligned(state, kSectionAlign)) return LQ_EINVAL;
    lq_layout L;
    compute_layout(*cfg, L);
    return hip_status(launch_clear_status((uint32_t*)((char*)state + L.status), stream));
}

const char* lq_strerror(int32_t code) {
    switch (code) {
        case LQ_OK: return "ok";
        case LQ_EINVAL: return "invalid argument (null or misaligned pointer, or inconsistent sizes)";
        case LQ_EUNSUPPORTED: return "unsupported configuration";
        case LQ_EHIP: return "HIP runtime error";
        case LQ_ESCRATCH: return "more units than the allocation-free call's scratch holds (262144)";
        default: return "unknown lq status code";
    }
}

}  // extern "C"
