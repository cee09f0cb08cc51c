// lq_internal.h -- internal declarations of liblq.so: blob layout, kernel
// argument blocks, and wavefront (DPP) reduction helpers for gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lq.h"

namespace lq {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr size_t kSectionAlign = 256;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Blob layout: the sections listed with lq_layout, each 256-byte aligned.
inline void compute_layout(const lq_config& c, lq_layout& L) {
    const size_t U = (size_t)c.n_seq * c.n_v_heads;
    const size_t KH = (size_t)c.n_seq * c.n_k_heads;
    const size_t D = (size_t)(c.d_k > c.d_v ? c.d_k : c.d_v);
    const size_t W = (size_t)c.window;
    const size_t nc = (size_t)c.n_comp;
    const size_t esz = c.buffer_format == LQ_BUFFER_FP16 ? 2 : 4;  // k, v element bytes
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + bytes, kSectionAlign);
        return o;
    };
    L.status = take(sizeof(uint32_t));
    L.fill = take(U * sizeof(int32_t));
    L.codes = take(U * c.d_v * c.d_k);
    L.sigma = take(U * c.d_v * sizeof(float));
    L.smooth = take(U * c.d_k * sizeof(float));
    L.comp_idx = take(U * nc * sizeof(int32_t));
    L.comp_vec = take(U * nc * D * sizeof(float));
    L.buf_k = take(KH * W * c.d_k * esz);
    L.buf_v = take(U * W * c.d_v * esz);
    L.buf_beta = take(U * W * sizeof(float));
    L.buf_gate = take(U * W * (c.gate_kind == LQ_GATE_CHANNEL ? c.d_k : 1) * sizeof(float));
    L.work = take((U + 1) * sizeof(int32_t));
    L.total_bytes = off;
}

// Device view of one blob.
struct BlobPtrs {
    uint32_t* status;
    int32_t* fill;
    int8_t* codes;
    float* sigma;
    float* smooth;
    int32_t* comp_idx;
    float* comp_vec;
    void* buf_k;  // float or _Float16 elements (Dims::buffer_format)
    void* buf_v;
    float* buf_beta;
    float* buf_gate;
    int32_t* work;  // [0] = count, [1..] = units due at the window boundary
};

inline BlobPtrs blob_ptrs(void* base, const lq_layout& L) {
    char* b = (char*)base;
    BlobPtrs p;
    p.status = (uint32_t*)(b + L.status);
    p.fill = (int32_t*)(b + L.fill);
    p.codes = (int8_t*)(b + L.codes);
    p.sigma = (float*)(b + L.sigma);
    p.smooth = (float*)(b + L.smooth);
    p.comp_idx = (int32_t*)(b + L.comp_idx);
    p.comp_vec = (float*)(b + L.comp_vec);
    p.buf_k = (void*)(b + L.buf_k);
    p.buf_v = (void*)(b + L.buf_v);
    p.buf_beta = (float*)(b + L.buf_beta);
    p.buf_gate = (float*)(b + L.buf_gate);
    p.work = (int32_t*)(b + L.work);
    return p;
}

// Sizes every kernel needs.
struct Dims {
    int n_units;    // n_seq * n_v_heads
    int n_v_heads;
    int n_k_heads;
    int group;      // n_v_heads / n_k_heads
    int window;
    int n_comp;
    int code_format;    // LQ_CODE_INT8 or LQ_CODE_E4M3
    int buffer_format;  // LQ_BUFFER_FP32 or LQ_BUFFER_FP16 (k and v of the window buffer)
    int max_cus;        // CUs the persistent (materialize) grid may occupy; 0: all
    int load_policy;    // LQ_LOADS_*: streaming loads in the decode step
};

struct DecodeArgs {
    BlobPtrs blob;
    Dims dm;
    const float* q;
    const float* k;
    const float* v;
    const float* beta;
    const float* gate;
    float* o;
};

struct Fp32DecodeArgs {
    Dims dm;
    float* S;
    const float* q;
    const float* k;
    const float* v;
    const float* beta;
    const float* gate;
    float* o;
};

enum MatMode : int { kModeInit = 0, kModeFlush = 1, kModeDequant = 2, kModePrefill = 3 };

struct MatArgs {
    BlobPtrs blob;
    Dims dm;
    const float* S0;          // init: fp32 start state or nullptr (zero)
    const uint8_t* force;     // flush: per-sequence force mask or nullptr
    float* S_out;             // dequant: fp32 output
    int include_buffer;       // dequant: replay the buffered tokens
    // prefill: the prompt, token-major (layouts as for one decode step, per token)
    int n_tok;
    const float* pq;
    const float* pk;
    const float* pv;
    const float* pbeta;
    const float* pgate;
    float* po;                // outputs [n_tok][units][d_v], or nullptr
};

// Host launchers (lq_decode.hip / lq_flush.hip).  Return hipSuccess or the
// launch error.
hipError_t launch_decode_q8(const DecodeArgs& a, int d, int gate_kind, hipStream_t st);
hipError_t launch_decode_fp32(const Fp32DecodeArgs& a, int d, int gate_kind, hipStream_t st);
hipError_t launch_materialize(const MatArgs& a, int mode, int d, int gate_kind, hipStream_t st);
hipError_t launch_clear_status(uint32_t* status, hipStream_t st);

// Units the allocation-free boundary call can list: its work list lives in a
// file-scope device array of 1 + kScratchMaxUnits int32 (lq_flush.hip).
constexpr int kScratchMaxUnits = LQ_NOALLOC_MAX_UNITS;
// Device address of that array on the current device (looked up once per device).
hipError_t scratch_work_list(int32_t** out);

}  // namespace lq

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
#if defined(__HIPCC__)
namespace lq {

// DPP control codes (GFX9 encoding, valid on gfx950).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xF,
                                           false));
}

// Sum over groups of 8 consecutive lanes, result in every lane of the group.
__device__ __forceinline__ float sum8(float x) {
    x += dpp_f32<kDppRowHalfMirror>(x);
    x += dpp_f32<kDppQuadXor2>(x);
    x += dpp_f32<kDppQuadXor1>(x);
    return x;
}

// Sum over groups of 4 consecutive lanes.
__device__ __forceinline__ float sum4(float x) {
    x += dpp_f32<kDppQuadXor2>(x);
    x += dpp_f32<kDppQuadXor1>(x);
    return x;
}

// Sum over groups of 16 consecutive lanes (one DPP row).
__device__ __forceinline__ float sum16(float x) {
    x += dpp_f32<kDppRowHalfMirror>(x);
    x += dpp_f32<kDppRowMirror>(x);
    x += dpp_f32<kDppQuadXor2>(x);
    x += dpp_f32<kDppQuadXor1>(x);
    return x;
}

// Sum over the whole wavefront; the result is uniform (read from lane 63).
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_f32<kDppQuadXor1>(x);
    x += dpp_f32<kDppQuadXor2>(x);
    x += dpp_f32<kDppRowHalfMirror>(x);
    x += dpp_f32<kDppRowMirror>(x);
    x += dpp_f32<kDppRowBcast15, 0xA>(x);
    x += dpp_f32<kDppRowBcast31, 0xC>(x);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Sum over the whole wavefront, left in every lane (no scalar round trip):
// four DPP stages inside each 16-lane row, then the gfx950 row swaps
// (v_permlane16_swap, v_permlane32_swap) add the rows pairwise.
__device__ __forceinline__ float wave_sum_all(float x) {
    x += dpp_f32<kDppQuadXor1>(x);
    x += dpp_f32<kDppQuadXor2>(x);
    x += dpp_f32<kDppRowHalfMirror>(x);
    x += dpp_f32<kDppRowMirror>(x);
    const int b = __builtin_bit_cast(int, x);
    const auto p16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    x = __builtin_bit_cast(float, (int)p16[0]) + __builtin_bit_cast(float, (int)p16[1]);
    const int c = __builtin_bit_cast(int, x);
    const auto p32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
    return __builtin_bit_cast(float, (int)p32[0]) + __builtin_bit_cast(float, (int)p32[1]);
}

// N independent sums over the whole wavefront, each left in every lane: the
// stages of wave_sum_all applied to all N values in turn, so the N chains
// overlap and cost about the latency of one.
template <int N>
__device__ __forceinline__ void wave_sum_all_n(float (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f32<kDppQuadXor1>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f32<kDppQuadXor2>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f32<kDppRowHalfMirror>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f32<kDppRowMirror>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int b = __builtin_bit_cast(int, x[i]);
        const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
        x[i] = __builtin_bit_cast(float, (int)p[0]) + __builtin_bit_cast(float, (int)p[1]);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int b = __builtin_bit_cast(int, x[i]);
        const auto p = __builtin_amdgcn_permlane32_swap(b, b, false, false);
        x[i] = __builtin_bit_cast(float, (int)p[0]) + __builtin_bit_cast(float, (int)p[1]);
    }
}

// Exclusive prefix sum over the lanes of the wavefront (lane 0 gets 0):
// shifts of 1, 2, 4 and 8 lanes inside each 16-lane row, the row ends
// carried with row_bcast, then the whole result moved up one lane.  Each
// partial sum covers a run of lanes starting at lane 0 of the scan.
__device__ __forceinline__ float wave_prefix_sum_excl(float x) {
    x += dpp_f32<0x111>(x);  // row_shr:1
    x += dpp_f32<0x112>(x);  // row_shr:2
    x += dpp_f32<0x114>(x);  // row_shr:4
    x += dpp_f32<0x118>(x);  // row_shr:8
    x += dpp_f32<kDppRowBcast15, 0xA>(x);
    x += dpp_f32<kDppRowBcast31, 0xC>(x);
    return dpp_f32<0x138>(x);  // wave_shr:1
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, i.e. waits for every outstanding store of the wave to be
// acknowledged, which costs microseconds when the wave has just written the
// window buffer; exchanges through LDS do not need that.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace lq
#endif
