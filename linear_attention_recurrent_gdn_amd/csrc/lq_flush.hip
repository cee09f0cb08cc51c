// lq_flush.hip -- window-boundary materialization and requantization, state
// init and dequantization for gfx950.
//
// The arXiv 2609.38166 abstract ("Abstract (arXiv)" section, mlsanity.com
// paper page): the state is quantized only once, at the end of a window; the
// largest outliers are kept as a few high-precision Compensator Tokens; the
// remaining residual is smoothed, then quantized to 8 bits.  The
// bedrocknews.com review: the biggest outlier rows and columns are pulled out
// and kept in FP16/FP32, and the state goes from FP32 to INT8.
//
// Work list: a one-workgroup scan writes the units whose window is due (full,
// or forced and non-empty) into the blob's work list; the materialize kernel
// then runs on a fixed grid that walks that list, so a boundary that concerns
// a few units does not launch a workgroup per unit.
//
// Materialize: one workgroup of D/16 wavefronts per unit at a time.  The
// FP64 state lives in the accumulator layout of the FP64 matrix instruction
// v_mfma_f64_16x16x4f64 (lane l, register r of a 16x16 result holds row
// 4r + l/16, column l%16): wavefront w owns rows n = 16w + (l % 16) and lane
// l holds, for every 16-column block b, the 4 consecutive columns
// 16b + 4(l/16) .. +3 of its row, as the 16x16 block b of S^T.
//   A  load: S = Diag(sigma) Q Diag(s) + compensator lines (flush, dequant) or
//      the caller's FP32 start state (init);
//   B  forward replay of the buffered tokens in FP64 (FP64 so that the
//      rounding decisions below match an FP64 reference), 16 tokens per
//      chunk, in a rescaled form (scalar gate S = g T, channel gate
//      S = T Diag(G); g and G are folded into T at a chunk start before they
//      can underflow, gates are floored at 2^-45).  With kf_e, kb_e the
//      token's key scaled forward and back (k, k for the scalar gate;
//      G_e k, k / G_e for the channel gate) and v'_e = v_e / g_e (scalar) or
//      v_e, the token-by-token replay
//          d_e = T kf_e;  T += beta_e (v'_e - d_e) kb_e^T
//      is, for a whole chunk,
//          A = T Kf^T;  C = (v' - A) Diag(beta) M^T;  T += C Kb
//      with L_ee' = kf_e . kb_e' (e' < e) and M = (I + Diag(beta) L)^-1,
//      a unit lower-triangular 16x16 matrix shared by all rows.  Both
//      d_v x d_k x 16 products and C run on the FP64 matrix cores; L is
//      assembled from per-wavefront partial products over column slices, and
//      M^T is solved by back substitution in one wavefront (all 64 lanes, each
//      holding four entries in the accumulator layout, finished rows broadcast
//      across row groups with the gfx950 permlane swaps) while the others form A;
//   C  quantizer, in the same workgroup (readings; the pages print no
//      formula): line scores = squared L2 norms of rows and columns; the
//      n_comp best lines (ties to the lower candidate index, rows before
//      columns) go to fp32 compensator slots, rows taken whole, columns with
//      the selected rows' entries zeroed; the residual R has those lines
//      zeroed; s_j = sqrt(max_i |R_ij|) (1 if zero), sigma_i =
//      max_j |R_ij / s_j| / qmax, both fp32; codes of x = R_ij /
//      (sigma_i s_j): INT8 clamp(rne(x), -127, 127) with qmax = 127, or
//      the nearest E4M3 8-bit float (ties to even) with qmax = 448.
// Row reductions combine the four lanes that share a row (permlane swaps);
// column reductions reduce-scatter over the 16 lanes of a row group, then
// combine the wavefronts through LDS in a fixed order, so results are
// deterministic.

#include <atomic>

#include "lq_internal.h"

namespace lq {

// Work list of the allocation-free boundary call (lq_window_flush_noalloc):
// [0] = count, [1..] = units due.  Every call on a device shares that device's
// copy and leaves the last call's list in it; the due-unit scan rewrites the
// count and every entry it uses, so nothing needs clearing.  In host code the
// name is a stand-in, not a device address: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) int32_t scratch[1 + kScratchMaxUnits];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int32_t*> g_scratch_addr[kMaxDevices];  // per device, set on first use
}  // namespace

hipError_t scratch_work_list(int32_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int32_t* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void* q = nullptr;
        e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        p = static_cast<int32_t*>(q);
        g_scratch_addr[dev].store(p, std::memory_order_release);  // a racing thread stores the same address
    }
    *out = p;
    return hipSuccess;
}

namespace {

typedef double v4d __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr double kRescaleBelow = 0x1p-200;  // fold the gate product into T below this
constexpr double kMinGate = 0x1p-45;        // per-token gate floor inside the flush
constexpr int kDppRowRor8 = 0x128;          // row_ror:8
constexpr int kDppRowShr1 = 0x111;          // row_shr:n = 0x110 + n
constexpr int kDppRowNewBcast0 = 0x150;     // row_newbcast:n = 0x150 + n (lane n of each row to the row)

// The value lane L of each 16-lane row holds, in every lane of that row.
template <int L>
__device__ __forceinline__ double row_bcast(double x) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)b, kDppRowNewBcast0 + L, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), kDppRowNewBcast0 + L, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Steps E2, E2 - 1, .., 1 of a row-wise back substitution: lane e of a row
// holds y[e], and step e2 folds the (final) y[e2] into every lane,
// y[e] -= n[e2] y[e2], where lane e's n[e2] is zero for e >= e2.
template <int E2, int N>
__device__ __forceinline__ void back_substitute(double& y, const double (&n)[N]) {
    if constexpr (E2 >= 1) {
        y = __builtin_fma(-n[E2], row_bcast<E2>(y), y);
        back_substitute<E2 - 1>(y, n);
    }
}

// x * (the value of lane l - SH of the same 16-lane row, or 1 where that
// lane lies before the row)
template <int SH>
__device__ __forceinline__ double times_row_shr(double x) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, kDppRowShr1 - 1 + SH, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0x3FF00000, (int)(uint32_t)(b >> 32), kDppRowShr1 - 1 + SH, 0xF, 0xF,
                                               false);
    return x * __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Inclusive prefix product over each 16-lane row: lane l gets the product of
// lanes row_start .. l (four row_shr steps).
__device__ __forceinline__ double row_prefix_product(double x) {
    x = times_row_shr<1>(x);
    x = times_row_shr<2>(x);
    x = times_row_shr<4>(x);
    return times_row_shr<8>(x);
}

__device__ __forceinline__ v4d mfma(double a, double b, v4d c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Combine the four lanes that share a row (lanes m, m+16, m+32, m+48).
template <bool MAX>
__device__ __forceinline__ double across_rows(double x) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const uint64_t b = __builtin_bit_cast(uint64_t, x);
        const int lo = (int)(uint32_t)b, hi = (int)(uint32_t)(b >> 32);
        int l0, l1, h0, h1;
        if (s == 0) {
            const auto pl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
            const auto ph = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
            l0 = pl[0]; l1 = pl[1]; h0 = ph[0]; h1 = ph[1];
        } else {
            const auto pl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
            const auto ph = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
            l0 = pl[0]; l1 = pl[1]; h0 = ph[0]; h1 = ph[1];
        }
        const double a = __builtin_bit_cast(double, ((uint64_t)(uint32_t)h0 << 32) | (uint32_t)l0);
        const double c = __builtin_bit_cast(double, ((uint64_t)(uint32_t)h1 << 32) | (uint32_t)l1);
        x = MAX ? fmax(a, c) : a + c;
    }
    return x;
}

// One reduce-scatter stage over the first N entries of v among the 16 lanes
// of a row group: the lane and its DPP partner keep one half each (the upper
// half where `up`) and combine the partner's copy of it.
template <int N, int CTRL, bool MAX, int M>
__device__ __forceinline__ void rs_stage(double (&v)[M], bool up) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        const double send = up ? v[i] : v[i + N / 2];
        const double keep = up ? v[i + N / 2] : v[i];
        const double got = dpp_f64<CTRL>(send);
        v[i] = MAX ? fmax(keep, got) : keep + got;
    }
}

// Column reduction of NV = 4 * NB values (value 4b + r = column 16b + 4q + r)
// over the 16 lanes of a row group.  Afterwards lane m holds NV / 16 totals in
// v[0..), for the values returned + i; every value is held by exactly one lane.
template <int NV, bool MAX>
__device__ __forceinline__ int reduce_columns(double (&v)[NV], int m) {
    static_assert(NV == 32 || NV == 16, "4 or 8 column blocks");
    // stage 1: every lane holds every value, so any pairing works (mirror in 8)
    rs_stage<NV, kDppRowHalfMirror, MAX>(v, (m & 4) != 0);
    rs_stage<NV / 2, kDppQuadXor1, MAX>(v, (m & 1) != 0);
    rs_stage<NV / 4, kDppQuadXor2, MAX>(v, (m & 2) != 0);
    if constexpr (NV == 32) {
        rs_stage<4, kDppRowRor8, MAX>(v, (m & 8) != 0);
        return 16 * ((m >> 2) & 1) + 8 * (m & 1) + 4 * ((m >> 1) & 1) + 2 * ((m >> 3) & 1);
    } else {
        // 2 values left per lane after three stages: the ror:8 pair splits them
        rs_stage<2, kDppRowRor8, MAX>(v, (m & 8) != 0);
        return 8 * ((m >> 2) & 1) + 4 * (m & 1) + 2 * ((m >> 1) & 1) + ((m >> 3) & 1);
    }
}

// Wavefront maximum of a 32-bit unsigned value, in every lane (DPP inside
// each 16-lane row, then the row swaps).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppQuadXor1, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppQuadXor2, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppRowHalfMirror, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppRowMirror, 0xF, 0xF, false));
    const auto p16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max((uint32_t)p16[0], (uint32_t)p16[1]);
    const auto p32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max((uint32_t)p32[0], (uint32_t)p32[1]);
}

// E4M3 byte of x (FP64): the nearest value of the 8-bit float format with
// 4 exponent bits (bias 7) and 3 mantissa bits, ties to the even mantissa,
// magnitudes above the largest finite 448 taken as 448, zero as the byte 0.
// Around a magnitude a the values are spaced 2^(E-3), E = max(floor(log2 a),
// -6); a / 2^(E-3) rounds to k = m (subnormal), 8 + m, or 16 (next binade).
// Both scalings are exact powers of two built from the exponent bits.
__device__ __forceinline__ uint32_t e4m3_code(double x) {
    const double ax = fmin(fabs(x), 448.0);
    const int E = max((int)((__builtin_bit_cast(uint64_t, ax) >> 52) & 0x7FF) - 1023, -6);
    const double up = __builtin_bit_cast(double, (uint64_t)(1023 + 3 - E) << 52);  // 2^(3-E)
    const int k = (int)rint(ax * up);
    if (k == 0) return 0u;
    uint32_t e, m;
    if (k < 8) {
        e = 0u;
        m = (uint32_t)k;
    } else if (k == 16) {
        e = (uint32_t)(E + 8);
        m = 0u;
    } else {
        e = (uint32_t)(E + 7);
        m = (uint32_t)(k - 8);
    }
    return (x < 0.0 ? 0x80u : 0u) | (e << 3) | m;
}

__device__ __forceinline__ bool finite4(const float4& f) {
    return __builtin_isfinite(f.x) && __builtin_isfinite(f.y) && __builtin_isfinite(f.z) &&
           __builtin_isfinite(f.w);
}

// Raise LQ_DEV_NONFINITE_INPUT when any lane of the wavefront saw a NaN or
// Inf (rare: a uniform branch around one atomic).
__device__ __forceinline__ void flag_nonfinite(uint32_t* status, bool bad) {
    if (__builtin_expect(__any(bad), 0)) {
        // lane 0, its index recomputed here from an opaque mask (not kept live)
        uint32_t all = ~0u;
        asm volatile("" : "+s"(all));
        if (__builtin_amdgcn_mbcnt_hi(all, __builtin_amdgcn_mbcnt_lo(all, 0u)) == 0)
            atomicOr(status, (uint32_t)LQ_DEV_NONFINITE_INPUT);
    }
}

__device__ __forceinline__ float pick4(const float4& f, int i) {
    return i == 0 ? f.x : i == 1 ? f.y : i == 2 ? f.z : f.w;
}

// One chunk of buffered tokens as fetched by one thread: four of the
// chunk's keys and values as stored (four fp32, or four binary16 in the first
// two words; token-major, D elements per token), four channel gates, and, for
// the first 16 threads, one beta and scalar gate.  The conversion waits for
// the data, so it happens when the chunk is staged, not when it is fetched.
template <bool KDA>
struct Stage {
    uint4 k, v;
    float4 g;
    float b, al;
};

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Four consecutive buffer elements as stored.  A 32-bit element offset from a
// uniform base keeps the address in the scalar-base form (no 64-bit per-lane
// address registers).
template <bool H16>
__device__ __forceinline__ uint4 load4_buf(const void* base, uint32_t off) {
    if constexpr (H16) {
        const uint2 h = *reinterpret_cast<const uint2*>(reinterpret_cast<const _Float16*>(base) + off);
        uint4 r;  // the last two words stay unset (unread): no write that must wait for an earlier load
        r.x = h.x;
        r.y = h.y;
        return r;
    } else {
        return *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(base) + off);
    }
}

// The four elements of load4_buf as fp32 (binary16 converts exactly).
__device__ __forceinline__ float4 unpack4(const uint4& r, bool h16) {
    if (h16) {
        const f16x4 h = __builtin_bit_cast(f16x4, make_uint2(r.x, r.y));
        return make_float4((float)h.x, (float)h.y, (float)h.z, (float)h.w);
    }
    return __builtin_bit_cast(float4, r);
}

// Token strides (elements) of the replayed tokens: the window buffer holds
// them entry-major per unit (k, v: D; beta: 1; gate: 1 or D); a prompt is
// token-major over all units.
struct TokStrides {
    size_t k, v, b, g;
};

template <int D, int NT, bool KDA, bool H16>
__device__ __forceinline__ Stage<KDA> fetch_stage(const void* bk, const void* bv, const float* bb,
                                                    const float* bg, TokStrides ts, int i0, int n_replay, int tid) {
    constexpr int EB = 16;
    Stage<KDA> st;
    const int ne = (n_replay - i0) < EB ? (n_replay - i0) : EB;
    const int x = 4 * tid;
    const uint32_t e = (uint32_t)min(x / D, ne - 1), c = (uint32_t)(x % D);
    // uniform chunk bases, then 32-bit offsets inside the chunk (16 token strides)
    constexpr size_t esz = H16 ? 2 : 4;
    const char* k0 = (const char*)bk + (size_t)i0 * ts.k * esz;
    const char* v0 = (const char*)bv + (size_t)i0 * ts.v * esz;
    const float* g0 = bg + (size_t)i0 * ts.g;
    const float* b0 = bb + (size_t)i0 * ts.b;
    // every thread loads a (clamped) token's beta and scalar gate; the first
    // 16 use them.  No constant is written to these registers: such a write
    // would have to wait for every load in flight, this chunk's too.  For the
    // same reason every address is formed before the first load is issued.
    const uint32_t t = (uint32_t)min(tid, ne - 1);
    const uint32_t ok = e * (uint32_t)ts.k + c, ov = e * (uint32_t)ts.v + c, og = e * (uint32_t)ts.g + c;
    const uint32_t ob = t * (uint32_t)ts.b, oa = t * (uint32_t)ts.g;
    __builtin_amdgcn_sched_barrier(0);
    st.k = load4_buf<H16>(k0, ok);
    st.v = load4_buf<H16>(v0, ov);
    if constexpr (KDA) st.g = *reinterpret_cast<const float4*>(g0 + og);
    st.b = b0[ob];
    if constexpr (!KDA) st.al = g0[oa];
    __builtin_amdgcn_sched_barrier(0);
    return st;
}

// The chunk's queries, four consecutive fp32 per thread of token-major
// [16][D] (like the keys), fetched into registers a stage ahead.  (A copy
// straight into LDS would make every barrier after it wait for the copy.)
template <int D>
__device__ __forceinline__ float4 fetch_q(const float* bq, size_t stride, int i0, int n_replay, int tid) {
    constexpr int EB = 16;
    const int ne = (n_replay - i0) < EB ? (n_replay - i0) : EB;
    const int x = 4 * tid;
    const uint32_t e = (uint32_t)min(x / D, ne - 1), c = (uint32_t)(x % D);
    const float* q0 = bq + (size_t)i0 * stride;
    return *reinterpret_cast<const float4*>(q0 + (e * (uint32_t)stride + c));
}

}  // namespace


// x from the lane the DPP control names; 1.0 where that lane lies outside
// the row (or the wavefront) or the row is masked off.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64_or1(double x) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0x3FF00000, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Exclusive prefix product over the lanes of the wavefront (lane 0 gets 1):
// shifts of 1, 2, 4, 8 lanes inside each 16-lane row, the row ends carried
// with row_bcast, then the result moved up one lane.
__device__ __forceinline__ double wave_prefix_prod_excl(double x) {
    x *= dpp_f64_or1<0x111>(x);  // row_shr:1
    x *= dpp_f64_or1<0x112>(x);  // row_shr:2
    x *= dpp_f64_or1<0x114>(x);  // row_shr:4
    x *= dpp_f64_or1<0x118>(x);  // row_shr:8
    x *= dpp_f64_or1<0x142, 0xA>(x);  // row_bcast:15
    x *= dpp_f64_or1<0x143, 0xC>(x);  // row_bcast:31
    return dpp_f64_or1<0x138>(x);  // wave_shr:1
}

__device__ __forceinline__ double lane_value_f64(double x, int l) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// H16: the window buffer holds binary16 keys and values (a flush or dequant
// that replays it; fp32 otherwise).  NF: the buffer is in the chain-free form
// (entries k_i, gate alpha_i and n_i; scalar gate): the window-end state is
// S = g S_hat + sum_i (g / g_i) n_i k_i^T, one product instead of the replay.
template <int D, bool KDA, int MODE, bool H16, bool NF = false>
__global__ __launch_bounds__(kWave * D / 16) void materialize_kernel(MatArgs a) {
    static_assert(!H16 || MODE == kModeFlush || MODE == kModeDequant, "binary16 applies to the window buffer");
    static_assert(!NF || (!KDA && !H16 && (MODE == kModeFlush || MODE == kModeDequant)),
                  "the chain-free buffer: scalar gate, fp32, boundary and dequantization");
    constexpr int NW = D / 16;          // wavefronts = 16-row groups
    constexpr int NT = kWave * NW;      // threads
    constexpr int NB = D / 16;          // 16-column blocks
    constexpr int NV = 4 * NB;          // state values per lane
    constexpr int EB = 16;              // buffered tokens per chunk
    constexpr int KP = D + 2;           // padded FP64 length of a staged key
    constexpr int CPL = 2 * D / kWave;  // selection candidates per lane
    constexpr bool PF = MODE == kModePrefill;

    // keys of the chunk: forward-scaled (kf), back-scaled (kb, channel gate);
    // the keys the update of T reads are double-buffered by chunk parity
    __shared__ double lds_kf[KDA ? 1 : 2][EB][KP];
    __shared__ double lds_kb[KDA ? 2 : 1][KDA ? EB : 1][KDA ? KP : 1];
    __shared__ float lds_v[EB][D];                          // values as fetched
    __shared__ float lds_kraw[KDA ? EB : 1][KDA ? D : 1];  // channel gate: keys as fetched
    __shared__ float lds_graw[KDA ? EB : 1][KDA ? D : 1];  // channel gate: gates as fetched
    __shared__ float lds_b[EB];
    __shared__ double lds_ig[EB];                           // scalar gate: 1 / g_e
    __shared__ double lds_gs[2];                            // scalar gate: fold factor, new g
    __shared__ double lds_G[2][KDA ? D : 1];                // channel gate: running G per column (by chunk parity)
    __shared__ double lds_fold[KDA ? D : 1];                // channel gate: fold factor per column
    __shared__ int lds_anyfold;                             // channel gate: some column folded
    // small [16][16] matrices padded to 17 columns: a column read across the
    // 16 rows (a matrix-pipe operand) would otherwise hit one LDS bank
    __shared__ double lds_gram[NW][EB][EB + 1];             // partial kf . kb over column slices
    __shared__ double lds_N[EB][EB];                        // Diag(beta) L (strictly lower)
    __shared__ double lds_M[EB][EB + 1];                    // (I + N)^-1
    // prefill outputs: queries as fetched and scaled, qf . kb, its future part
    __shared__ float lds_qraw[PF ? EB : 1][PF ? D : 1];
    __shared__ double lds_qf[PF ? EB : 1][PF ? KP : 1];
    __shared__ double lds_gq[PF ? EB : 1];                  // scalar gate: g_e
    __shared__ double lds_gramq[PF ? NW : 1][PF ? EB : 1][PF ? EB + 1 : 1];
    __shared__ double lds_P[PF ? EB : 1][PF ? EB + 1 : 1];  // (e' <= e) qf_e . kb_e'
    __shared__ double lds_score[2 * D];
    __shared__ double lds_part[NW][D];
    __shared__ float lds_smooth[D];
    __shared__ double lds_ismooth[D];
    __shared__ int lds_slot[2 * D];  // slot + 1 of each selected candidate, 0 otherwise
    __shared__ int lds_chosen[16];

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int q = lane >> 4;        // column quad inside a 16-column block
    const int m = lane & 15;        // row inside the wavefront's 16 rows
    const int n = 16 * wave + m;    // state row of this lane
    const int W = a.dm.window;
    const int nc = a.dm.n_comp;

    const int n_work = (MODE == kModeFlush) ? a.blob.work[0] : a.dm.n_units;
    constexpr bool kFromCodes = !(MODE == kModeInit || PF);  // the start state is the quantized one
    // The unit of this workgroup's work item k.  A flush reads the work list
    // 64 items at a time into a register (lane j: item 64 i + j), so that a
    // unit is a register read rather than a wait for memory (a wait for one
    // load is a wait for every load and store requested before it).  Called
    // with k increasing, every multiple of 64 included.
    int wl_units = 0;
    auto work_unit = [&](int k) -> int {
        if constexpr (MODE == kModeFlush) {
            if ((k & 63) == 0) {
                // the lane index recomputed here (from an opaque mask), not kept live across the unit
                uint32_t all = ~0u;
                asm volatile("" : "+s"(all));
                const int l = (int)__builtin_amdgcn_mbcnt_hi(all, __builtin_amdgcn_mbcnt_lo(all, 0u));
                const int idx = (int)blockIdx.x + (k + l) * (int)gridDim.x;
                wl_units = idx < n_work ? a.blob.work[1 + idx] : 0;
            }
            return __builtin_amdgcn_readlane(wl_units, k & 63);
        } else {
            return (int)blockIdx.x + k * (int)gridDim.x;
        }
    };
    int u_next = (int)blockIdx.x < n_work ? work_unit(0) : 0;
    // tokens replayed from a unit's window buffer
    auto replay_count = [&](int fill) {
        return (MODE == kModeFlush || (MODE == kModeDequant && a.include_buffer)) ? (fill < W ? fill : W) : 0;
    };
    // window buffer of unit uu: keys (per key head), values, betas, gates
    auto unit_buffers = [&](int uu, const void*& bk, const void*& bv, const float*& bb, const float*& bg) {
        const int s = uu / a.dm.n_v_heads;
        const int h = uu - s * a.dm.n_v_heads;
        const size_t kvec = (size_t)s * a.dm.n_k_heads + h / a.dm.group;
        constexpr size_t esz = H16 ? 2 : 4;
        bk = (const char*)a.blob.buf_k + kvec * (size_t)W * D * esz;
        bv = (const char*)a.blob.buf_v + (size_t)uu * W * D * esz;
        bb = a.blob.buf_beta + (size_t)uu * W;
        bg = a.blob.buf_gate + (size_t)uu * W * (KDA ? D : 1);
    };
    // Starting from the codes, what a unit's start reads (codes, row scale,
    // smoothing, compensator lines, window count, then the first chunk of its
    // buffer) is requested one unit ahead, while the previous unit is
    // quantized: hw, hsg (this lane's row), hsm (channel tid), hcv, hcil, hfill.
    uint32_t hw[NB];
    float hsg = 0.f, hsm = 1.f;
    float4 hcv = make_float4(0.f, 0.f, 0.f, 0.f);
    int hcil = 0, hfill = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) hw[b] = 0u;
    Stage<KDA> pf{};  // the chunk being fetched (registers until it is staged)
    auto head_fetch = [&](int uu) {
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));  // indices recomputed here, not kept live
        const int rq = (t % kWave) >> 4, rn = 16 * (t / kWave) + (t & 15);
        hsg = a.blob.sigma[(size_t)uu * D + rn];
#pragma unroll
        for (int b = 0; b < NB; ++b)
            hw[b] = *reinterpret_cast<const uint32_t*>(a.blob.codes + ((size_t)uu * D + rn) * D + 16 * b + 4 * rq);
        hsm = a.blob.smooth[(size_t)uu * D + min(t, D - 1)];
        if (nc > 0) {
            static_assert(NT * 4 >= 16 * D, "one float4 per thread covers 16 lines");
            hcv = *reinterpret_cast<const float4*>(a.blob.comp_vec + (size_t)uu * nc * D + min(4 * t, nc * D - 4));
            hcil = a.blob.comp_idx[(size_t)uu * nc + min(t % kWave, nc - 1)];
        }
        // a vector load, counted with the ones above (a scalar load would hold
        // up the next wait on LDS)
        const int* fp = a.blob.fill + uu;
        asm volatile("" : "+v"(fp));
        hfill = *fp;
    };
    int nr_next = 0;  // tokens the fetched unit replays (uniform)
    // the head is in by the time this runs: a wait for it here, before the
    // first chunk's loads (on every path, fetched or not), keeps the wait at
    // the unit's start from covering those loads as well
    auto head_settle = [&]() {
#pragma unroll
        for (int b = 0; b < NB; ++b) asm volatile("" ::"v"(hw[b]));
        asm volatile("" ::"v"(hsg), "v"(hsm), "v"(hcv.x), "v"(hcv.y), "v"(hcv.z), "v"(hcv.w), "v"(hcil), "v"(hfill));
    };
    auto chunk0_fetch = [&](int uu) {
        const int nr = replay_count(__builtin_amdgcn_readfirstlane(hfill));
        nr_next = nr;
        if (!NF && nr > 0) {
            const void *bk, *bv;
            const float *bb, *bg;
            unit_buffers(uu, bk, bv, bb, bg);
            int t = threadIdx.x;
            asm volatile("" : "+v"(t));
            pf = fetch_stage<D, NT, KDA, H16>(bk, bv, bb, bg, TokStrides{(size_t)D, (size_t)D, 1, KDA ? (size_t)D : 1},
                                              0, nr, t);
        }
    };
    if constexpr (kFromCodes) {
        if ((int)blockIdx.x < n_work) head_fetch(u_next);
        head_settle();
        if ((int)blockIdx.x < n_work) chunk0_fetch(u_next);
    }
    for (int wi = blockIdx.x, k = 0; wi < n_work; wi += gridDim.x, ++k) {
        const int u = u_next;
        const bool ahead = wi + (int)gridDim.x < n_work;  // uniform: this workgroup has a next item
        if constexpr (!kFromCodes) {
            if (ahead) u_next = work_unit(k + 1);
        }
        const int s = u / a.dm.n_v_heads;
        const int h = u - s * a.dm.n_v_heads;
        const int kh = h / a.dm.group;
        const size_t kvec = (size_t)s * a.dm.n_k_heads + kh;

        // ---------------- A: the window-start state; T[b][r] = S[n][16b + 4q + r]
        //
        // From a start state (init, prefill): its loads depend on the unit
        // alone and are requested first, the first chunk of replayed tokens
        // after them, so the conversion waits for none of those (vector loads
        // complete in order).  From the codes: everything was requested while
        // the previous unit was quantized (or before the first).
        float4 sv[NB];  // start state S0 (init, prefill)
        if constexpr (!kFromCodes) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                sv[b] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (a.S0 != nullptr)
                    sv[b] = *reinterpret_cast<const float4*>(a.S0 + ((size_t)u * D + n) * D + 16 * b + 4 * q);
            }
        }

        int n_replay = 0;
        if constexpr (kFromCodes) n_replay = nr_next;
        if constexpr (PF) n_replay = a.n_tok;

        // the replayed tokens (window buffer, or the prompt)
        constexpr size_t esz = H16 ? 2 : 4;
        const void* bk = (const char*)a.blob.buf_k + kvec * (size_t)W * D * esz;
        const void* bv = (const char*)a.blob.buf_v + (size_t)u * W * D * esz;
        const float* bb = a.blob.buf_beta + (size_t)u * W;
        const float* bg = a.blob.buf_gate + (size_t)u * W * (KDA ? D : 1);
        const float* bq = nullptr;
        TokStrides ts{(size_t)D, (size_t)D, 1, KDA ? (size_t)D : 1};
        if constexpr (PF) {
            const size_t U = (size_t)a.dm.n_units;
            const size_t KU = U / a.dm.n_v_heads * a.dm.n_k_heads;  // key-head rows per token
            bk = a.pk + kvec * D;
            bq = a.pq + kvec * D;
            bv = a.pv + (size_t)u * D;
            bb = a.pbeta + u;
            bg = a.pgate + (size_t)u * (KDA ? D : 1);
            ts = TokStrides{KU * D, U * D, U, U * (KDA ? D : 1)};
        }
        double gam = 1.0;  // scalar gate: g of the last replayed token (uniform)
        if constexpr (KDA) {
            if (tid < D) lds_G[0][tid] = 1.0;
        }
        float4 pfq = make_float4(0.f, 0.f, 0.f, 0.f);  // prefill: the staged chunk's queries
        if (!kFromCodes && n_replay > 0) {
            pf = fetch_stage<D, NT, KDA, H16>(bk, bv, bb, bg, ts, 0, n_replay, tid);
            if constexpr (PF) pfq = fetch_q<D>(bq, ts.k, 0, n_replay, tid);
        }

        v4d T[NB];
        if constexpr (!kFromCodes) {
            bool bad = false;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                T[b] = v4d{(double)sv[b].x, (double)sv[b].y, (double)sv[b].z, (double)sv[b].w};
                bad = bad || !finite4(sv[b]);
            }
            flag_nonfinite(a.blob.status, bad);  // a NaN or Inf in the caller's start state
        } else {
            // the smoothing factors and the unit's compensator lines (at most
            // 16 d floats, in the partial-gram space that the replay only uses
            // later) pass through LDS
            float* lds_cv = reinterpret_cast<float*>(&lds_gram[0][0][0]);
            static_assert(sizeof(lds_gram) >= 16 * D * sizeof(float), "room for 16 lines");
            if (tid < D) lds_ismooth[tid] = (double)hsm;  // the smoothing factors, in FP64 here
            if (nc > 0) *reinterpret_cast<float4*>(lds_cv + 4 * tid) = hcv;
            // slot + 1 of each row (x < D) and column (x - D) that is a line, 0 otherwise
            static_assert(NT >= 2 * D, "one thread per candidate line");
            if (tid < 2 * D) {
                int sl = 0;
                for (int c = 0; c < nc; ++c)
                    if (__builtin_amdgcn_readlane(hcil, c) == tid) sl = c + 1;
                lds_slot[tid] = sl;
            }
            __syncthreads();
            const double sgr = (double)hsg;
            const bool e4m3 = a.dm.code_format == LQ_CODE_E4M3;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                double cd[4];  // the codes' values (exact in FP64)
                if (e4m3) {
                    // exact: every E4M3 value is an fp32 value
                    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(hw[b], false);
                    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(hw[b], true);
                    cd[0] = (double)lo.x;
                    cd[1] = (double)lo.y;
                    cd[2] = (double)hi.x;
                    cd[3] = (double)hi.y;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) cd[r] = (double)((int)(hw[b] << (24 - 8 * r)) >> 24);
                }
                const double2 s01 = *reinterpret_cast<const double2*>(&lds_ismooth[16 * b + 4 * q]);
                const double2 s23 = *reinterpret_cast<const double2*>(&lds_ismooth[16 * b + 4 * q + 2]);
                T[b][0] = sgr * cd[0] * s01.x;
                T[b][1] = sgr * cd[1] * s01.y;
                T[b][2] = sgr * cd[2] * s23.x;
                T[b][3] = sgr * cd[3] * s23.y;
            }
            // compensator lines: a row slot adds its line to the four lanes of
            // that row, a column slot adds one value per row.  The per-lane
            // slot reads come from the table above; a wavefront with no lane
            // concerned skips each step.
            if (nc > 0) {
                const int rs = lds_slot[n];
                if (__any(rs > 0)) {
                    const float* rv = lds_cv + max(rs - 1, 0) * D;
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        const float4 x = *reinterpret_cast<const float4*>(rv + 16 * b + 4 * q);
                        if (rs > 0) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) T[b][r] += (double)pick4(x, r);
                        }
                    }
                }
                // value positions (4 b + r) that some column line meets in some
                // row quad: the same for every wavefront, a scalar mask
                uint32_t pos = 0u;
                for (int c = 0; c < nc; ++c) {
                    const int col = __builtin_amdgcn_readlane(hcil, c) - D;
                    if (col >= 0) pos |= 1u << (4 * (col >> 4) + (col & 3));
                }
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (pos & (1u << (4 * b + r))) {
                            const int cs = lds_slot[D + 16 * b + 4 * q + r];
                            if (cs > 0) T[b][r] += (double)lds_cv[(cs - 1) * D + n];
                        }
                    }
            }
        }

        // ---------------- B (chain-free buffer): S = g S_hat + sum_i (g / g_i) n_i k_i^T
        if constexpr (NF) {
            if (n_replay > 0) {
                // g / g_i for every entry (exclusive suffix products of the
                // gates, floored at 2^-126 as in the decode, FP64), into LDS;
                // g into gam
                double* lds_ratio = &lds_part[0][0];
                static_assert(sizeof(lds_part) >= 256 * sizeof(double), "room for a window of ratios");
                if (wave == 0) {
                    double carry = 1.0;
#pragma unroll 1
                    for (int w = 0; w * kWave < n_replay; ++w) {  // uniform
                        const int idx = n_replay - 1 - (lane + w * kWave);
                        const double g = idx >= 0 ? fmax((double)bg[max(idx, 0)], 0x1p-126) : 1.0;
                        const double ex = wave_prefix_prod_excl(g);
                        if (idx >= 0) lds_ratio[idx] = carry * ex;
                        carry *= lane_value_f64(ex, kWave - 1) * lane_value_f64(g, kWave - 1);
                    }
                    if (lane == 0) lds_gs[1] = carry;
                }
                __syncthreads();
                gam = lds_gs[1];
#pragma unroll
                for (int b = 0; b < NB; ++b) T[b] *= gam;
                const int colm = 4 * (m & 3) + (m >> 2);  // column of block b held by result row m
                const float* bkf = reinterpret_cast<const float*>(bk);
                const float* bvf = reinterpret_cast<const float*>(bv);
#pragma unroll 1
                for (int c = 0; c * EB < n_replay; ++c) {  // uniform
                    const int i0 = c * EB;
                    const int ne = (n_replay - i0) < EB ? (n_replay - i0) : EB;
                    const int par = c & 1;
                    {
                        // the chunk's keys into LDS as FP64 (zero past the last entry)
                        int t = threadIdx.x;
                        asm volatile("" : "+v"(t));
                        const int x = 4 * t;
                        const int e = x / D, col = x % D;
                        float4 kx = make_float4(0.f, 0.f, 0.f, 0.f);
                        if (e < ne) kx = *reinterpret_cast<const float4*>(bkf + (size_t)(i0 + e) * D + col);
                        double* kd = &lds_kf[par][e][col];
                        kd[0] = (double)kx.x;
                        kd[1] = (double)kx.y;
                        kd[2] = (double)kx.z;
                        kd[3] = (double)kx.w;
                    }
                    // this lane's n for tokens 4r + q of the chunk, times g / g_i
                    double nb[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int e = 4 * r + q;
                        nb[r] = e < ne ? (double)bvf[(size_t)(i0 + e) * D + n] * lds_ratio[i0 + e] : 0.0;
                    }
                    __syncthreads();
                    const double(*kf)[KP] = (const double(*)[KP])lds_kf[par];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        double kv[NB];
#pragma unroll
                        for (int b = 0; b < NB; ++b) kv[b] = kf[4 * r + q][16 * b + colm];
#pragma unroll
                        for (int b = 0; b < NB; ++b) T[b] = mfma(kv[b], nb[r], T[b]);
                    }
                }
                gam = 1.0;  // g is in T
                __syncthreads();  // the ratios' LDS is the quantizer's
            }
        } else {
        // ---------------- B: forward replay of the buffered tokens (or the prompt), 16 per chunk
        //
        // Software-pipelined over chunks.  Chunk c+1 is staged while chunk c
        // finishes, so the products the next chunk needs first (its partial
        // grams) enter the matrix pipe ahead of chunk c's update of T, and the
        // reduction to N runs while that update executes:
        //   gemm_a(c) with M(c) | R(c), C(c) | barrier | stage(c+1) | grams(c+1)
        //   | T += C Kb for chunk c, with the gram write, a barrier, the
        //     reduction to N(c+1) and a barrier between its four token groups
        // The keys T += C Kb reads (kb, which is kf with a scalar gate) are
        // double-buffered by chunk parity; everything else a chunk stages is
        // read before the barrier that precedes the next stage.
        const int n_chunks = (n_replay + EB - 1) / EB;
        auto kf_of = [&](int par) -> const double(*)[KP] {
            return (const double(*)[KP])lds_kf[KDA ? 0 : par];
        };
        auto kb_of = [&](int par) -> const double(*)[KP] {
            if constexpr (KDA) return (const double(*)[KP])lds_kb[par];
            else return (const double(*)[KP])lds_kf[par];
        };
        // stage chunk c from the fetched registers into LDS, then request chunk
        // c + 1; ends with a barrier after which the chunk's data is readable
        // (with live false: only the caller's work and a barrier)
        auto stage = [&](int c, bool live, auto&& mid) {
            if (!live) {
                mid();
                __syncthreads();
                return;
            }
            // the thread index through an opaque copy: the address arithmetic
            // below is redone at each call instead of being kept live across the
            // replay (registers are short)
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const int i0 = c * EB;
            const int ne = (n_replay - i0) < EB ? (n_replay - i0) : EB;
            const int qb = c & 1;  // chunk parity: keys, queries (prefill), running gate (channel)
            if constexpr (PF) {
                // a NaN or Inf in the prompt
                bool bad = !finite4(unpack4(pf.k, false)) || !finite4(unpack4(pf.v, false)) || !finite4(pfq) ||
                           !__builtin_isfinite(pf.b) || !__builtin_isfinite(pf.al);
                if constexpr (KDA) bad = bad || !finite4(pf.g);
                flag_nonfinite(a.blob.status, bad);
            }
            {
                const int x = 4 * tid;
                const int e = x / D, col = x % D;
                const bool live = e < ne;  // padding tokens: zero key, zero beta
                const float4 kx = unpack4(pf.k, H16), vx = unpack4(pf.v, H16);
                *reinterpret_cast<float4*>(&lds_v[e][col]) = vx;
                if constexpr (PF) *reinterpret_cast<float4*>(&lds_qraw[e][col]) = pfq;
                if constexpr (KDA) {
                    *reinterpret_cast<float4*>(&lds_kraw[e][col]) = kx;
                    *reinterpret_cast<float4*>(&lds_graw[e][col]) = pf.g;
                } else {
                    double* kd = &lds_kf[qb][e][col];
                    kd[0] = live ? (double)kx.x : 0.0;
                    kd[1] = live ? (double)kx.y : 0.0;
                    kd[2] = live ? (double)kx.z : 0.0;
                    kd[3] = live ? (double)kx.w : 0.0;
                }
                if (tid < EB) {
                    lds_b[tid] = tid < ne ? pf.b : 0.f;
                }
                if (KDA && tid == 0) lds_anyfold = 0;
                if constexpr (!KDA) {
                    // the running gate product g_e = g * prod_{l <= e} alpha_l and its
                    // reciprocal, one token per lane of wavefront 0 (lane e holds
                    // alpha_e as fetched; padding tokens count 1) by a prefix
                    // product across the lanes; the chunk folds g into T first
                    // when its product could fall below the threshold
                    if (wave == 0) {
                        const double al = lane < ne ? fmax((double)pf.al, kMinGate) : 1.0;
                        const double pre = row_prefix_product(al);
                        const double P = __builtin_bit_cast(
                            double, ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(
                                         (int)(__builtin_bit_cast(uint64_t, pre) >> 32), EB - 1) << 32) |
                                        (uint32_t)__builtin_amdgcn_readlane(
                                            (int)(uint32_t)__builtin_bit_cast(uint64_t, pre), EB - 1));
                        const bool fold = gam * P < kRescaleBelow;
                        const double g = (fold ? 1.0 : gam) * pre;
                        if (lane < EB) lds_ig[lane] = lane < ne ? 1.0 / g : 0.0;
                        if (PF && lane < EB) lds_gq[lane] = lane < ne ? g : 0.0;
                        if (lane == 0) {
                            lds_gs[0] = fold ? gam : 1.0;
                            lds_gs[1] = (fold ? 1.0 : gam) * P;
                        }
                    }
                }
            }
            mid();  // work of the caller that overlaps the stage (no LDS it writes)
            __syncthreads();
            if constexpr (KDA) {
                // four threads per column, four tokens each: fold G into T if the
                // chunk could take it below the threshold, then the keys (and
                // queries) scaled by the running gate product, both ways
                static_assert(NT == 4 * D, "four threads per column");
                {
                    const int col = tid % D, seg = tid / D;
                    double pre = 1.0, P = 1.0;  // product before this thread's tokens, whole chunk
#pragma unroll
                    for (int e = 0; e < EB; ++e) {
                        const double al = e < ne ? fmax((double)lds_graw[e][col], kMinGate) : 1.0;
                        if (e < 4 * seg) pre *= al;
                        P *= al;
                    }
                    // read this chunk's G, write the next chunk's: no thread of
                    // the column overwrites what another still has to read
                    const double G0 = lds_G[qb][col];
                    const bool fold = G0 * P < kRescaleBelow;  // the same in the column's four threads
                    if (seg == 0) {
                        lds_fold[col] = fold ? G0 : 1.0;
                        if (fold) lds_anyfold = 1;  // every writer stores the same value
                    }
                    double G = (fold ? 1.0 : G0) * pre;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int e = 4 * seg + i;
                        double kfv = 0.0, kbv = 0.0, qfv = 0.0;
                        if (e < ne) {
                            G *= fmax((double)lds_graw[e][col], kMinGate);
                            const double kc = (double)lds_kraw[e][col];
                            kfv = G * kc;
                            kbv = kc / G;
                            if constexpr (PF) qfv = G * (double)lds_qraw[e][col];
                        }
                        lds_kf[0][e][col] = kfv;
                        lds_kb[qb][e][col] = kbv;
                        if constexpr (PF) lds_qf[e][col] = qfv;
                    }
                    if (seg == 3) lds_G[qb ^ 1][col] = (fold ? 1.0 : G0) * P;
                }
            }
            if constexpr (PF && !KDA) {
                // queries scaled by the running gate: qf_e = g_e q_e
                const int x = 4 * tid;
                const int e = x / D, col = x % D;
#pragma unroll
                for (int i = 0; i < 4; ++i) lds_qf[e][col + i] = lds_gq[e] * (double)lds_qraw[e][col + i];
            }
            // the next chunk, in flight until the next stage
            if (i0 + EB < n_replay) {
                pf = fetch_stage<D, NT, KDA, H16>(bk, bv, bb, bg, ts, i0 + EB, n_replay, tid);
                if constexpr (PF) pfq = fetch_q<D>(bq, ts.k, i0 + EB, n_replay, tid);
            }
            if constexpr (KDA || PF) __syncthreads();
        };
        // partial L of chunk c over this wavefront's 16-column slice: lane (q, m),
        // register r -> sum_k kf[4r + q][k] kb[m][k]; prefill also qf . kb
        // (one accumulator each: the matrix pipe forwards a dependent accumulator)
        v4d gr, grq;
        auto gram_issue = [&](int c) {
            const double(*kf)[KP] = kf_of(c & 1);
            const double(*kb)[KP] = kb_of(c & 1);
            gr = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int k = 16 * wave + 4 * t + q;
                gr = mfma(kf[m][k], kb[m][k], gr);
            }
            if constexpr (PF) {
                // partial qf . kb: lane (q, m), register r -> qf[4r + q] . kb[m]
                grq = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int k = 16 * wave + 4 * t + q;
                    grq = mfma(lds_qf[m][k], kb[m][k], grq);
                }
            }
        };
        auto gram_write = [&]() {
#pragma unroll
            for (int r = 0; r < 4; ++r) lds_gram[wave][4 * r + q][m] = gr[r];
            if constexpr (PF) {
#pragma unroll
                for (int r = 0; r < 4; ++r) lds_gramq[wave][4 * r + q][m] = grq[r];
            }
        };
        // N = Diag(beta) L (strictly lower), and for the prefill P, each
        // element summed over the slices in a fixed order, shared out over the
        // whole block
        auto n_reduce = [&]() {
            constexpr int NEL = (PF ? 2 : 1) * EB * EB;
#pragma unroll
            for (int t = 0; t < (NEL + NT - 1) / NT; ++t) {
                const int idx = tid + NT * t;
                if (NEL % NT != 0 && idx >= NEL) break;
                const int j = idx % (EB * EB);
                const int e = j / EB, e2 = j % EB;
                double sum = 0.0;
                if (!PF || idx < EB * EB) {
#pragma unroll
                    for (int w = 0; w < NW; ++w) sum += lds_gram[w][e][e2];
                    lds_N[e][e2] = e2 < e ? (double)lds_b[e] * sum : 0.0;
                } else if constexpr (PF) {
#pragma unroll
                    for (int w = 0; w < NW; ++w) sum += lds_gramq[w][e][e2];
                    lds_P[e][e2] = e2 <= e ? sum : 0.0;
                }
            }
        };
        if (n_chunks > 0) {
            stage(0, true, [] {});
            gram_issue(0);
            gram_write();
            __syncthreads();
            n_reduce();
            __syncthreads();
        }
        for (int c = 0; c < n_chunks; ++c) {
            const int i0 = c * EB;
            const int ne = (n_replay - i0) < EB ? (n_replay - i0) : EB;
            const bool more = c + 1 < n_chunks;  // uniform
            // folds into T (decided when the chunk was staged)
            if constexpr (KDA) {
                if (lds_anyfold) {  // uniform, rare
#pragma unroll
                    for (int b = 0; b < NB; ++b)
#pragma unroll
                        for (int r = 0; r < 4; ++r) T[b][r] *= lds_fold[16 * b + 4 * q + r];
                }
            } else {
                const double f = lds_gs[0];
                if (f != 1.0) {
#pragma unroll
                    for (int b = 0; b < NB; ++b) T[b] *= f;
                }
                gam = lds_gs[1];
            }
            // every wavefront: A = T Kf^T (prefill: also Aq = T Qf^T, register r:
            // token 4r + q, row n) on the matrix pipe, one accumulator each (the
            // pipe forwards a dependent accumulator to the next product).  The
            // keys of block b + 1 are requested before the products of block b;
            // the scheduling barriers keep that order.
            v4d Aq4 = {0.0, 0.0, 0.0, 0.0};
            v4d A4;
            {
                const double(*kf)[KP] = kf_of(c & 1);
                v4d acc = {0.0, 0.0, 0.0, 0.0};
                double kc[2][4], qc[4];
                auto load_keys = [&](int b, double* kd) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) kd[r] = kf[m][16 * b + 4 * q + r];
                };
                // (prefill, short of registers: the keys of block b with its queries)
                if constexpr (!PF) load_keys(0, kc[0]);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int cur = PF ? 0 : b & 1;
                    if (PF) load_keys(b, kc[0]);
                    else if (b + 1 < NB) load_keys(b + 1, kc[cur ^ 1]);
                    if constexpr (PF) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) qc[r] = lds_qf[m][16 * b + 4 * q + r];
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc = mfma(kc[cur][r], T[b][r], acc);
                    if constexpr (PF) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) Aq4 = mfma(qc[r], T[b][r], Aq4);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                A4 = acc;  // register r: A[token 4r + q][row n]
            }
            // R = (v' - A) Diag(beta): register r -> token 4r + q, row n
            v4d R4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = 4 * r + q;
                const double vp = KDA ? (double)lds_v[e][n] : (double)lds_v[e][n] * lds_ig[e];
                R4[r] = (double)lds_b[e] * (vp - A4[r]);
            }
            // M = (I + N)^-1 while the next chunk is staged, into LDS, on the
            // last four wavefronts (the first computes the scalar gates), one row
            // of M per row group: lane (g, e) of solver wavefront w holds
            // Y = M[m][e], m = 4 w + g.  M (I + N) = I with N strictly lower
            // gives M[m][e] = [m == e] - sum_{e2 > e} M[m][e2] N[e2][e]: from
            // e2 = 15 down, M[m][e2] is final, is broadcast across its row group
            // (DPP row_newbcast) and folds into every e < e2 (N[e2][e] is zero
            // for e >= e2, so every lane takes the same step).  Each step waits
            // on one FMA and one broadcast; lane e's column of N is requested
            // before the first.  (As vector ALU work beside the products it
            // slowed the matrix pipe.)
            auto solve_m = [&]() {
                if (wave < NW - 4) return;
                const int e = lane & 15;
                const int mrow = 4 * (wave - (NW - 4)) + (lane >> 4);
                double ncol[EB];  // ncol[e2] = N[e2][e]
#pragma unroll
                for (int e2 = 1; e2 < EB; ++e2) ncol[e2] = lds_N[e2][e];
                double Y = e == mrow ? 1.0 : 0.0;
                back_substitute<EB - 1>(Y, ncol);
                lds_M[mrow][e] = Y;
            };
            if (more) __syncthreads();  // chunk c's staged data, keys aside, is read
            stage(c + 1, more, solve_m);
            // C = M R (per row): register r -> token 4r + q, row n
            v4d C4 = {0.0, 0.0, 0.0, 0.0};
            C4 = mfma(lds_M[m][q], R4[0], C4);
            C4 = mfma(lds_M[m][4 + q], R4[1], C4);
            C4 = mfma(lds_M[m][8 + q], R4[2], C4);
            C4 = mfma(lds_M[m][12 + q], R4[3], C4);
            // prefill outputs of the chunk's tokens: o_e = T qf_e + sum_{e' <= e} C_e' (kb_e' . qf_e)
            const bool outs = PF && a.po != nullptr;
            if constexpr (PF) {
                if (outs) {
                    Aq4 = mfma(lds_P[m][q], C4[0], Aq4);
                    Aq4 = mfma(lds_P[m][4 + q], C4[1], Aq4);
                    Aq4 = mfma(lds_P[m][8 + q], C4[2], Aq4);
                    Aq4 = mfma(lds_P[m][12 + q], C4[3], Aq4);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int e = 4 * rr + q;
                        float* o0 = a.po + ((size_t)i0 * a.dm.n_units + u) * D;  // uniform
                        if (e < ne) o0[(uint32_t)e * (uint32_t)a.dm.n_units * D + n] = (float)Aq4[rr];
                    }
                }
            }
            // T += C Kb: block b of S^T, token group r; the keys of token group
            // r + 1 are requested before the products of group r.  Between the
            // groups (when `tasks`): chunk c+1's partial grams to LDS, a
            // barrier, its N, a barrier
            auto t_update = [&](bool tasks) {
                const double(*kb)[KP] = kb_of(c & 1);
                const int colm = 4 * (m & 3) + (m >> 2);  // column of block b held by result row m
                double kv[2][NB];
                auto load_kb = [&](int r, double* dst) {
#pragma unroll
                    for (int b = 0; b < NB; ++b) dst[b] = kb[4 * r + q][16 * b + colm];
                };
                load_kb(0, kv[0]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int cur = r & 1;
                    if (r + 1 < 4) load_kb(r + 1, kv[cur ^ 1]);
#pragma unroll
                    for (int b = 0; b < NB; ++b) T[b] = mfma(kv[cur][b], C4[r], T[b]);
                    if (tasks) {
                        if (r == 0) gram_write();
                        if (r == 1) __syncthreads();
                        if (r == 2) n_reduce();
                        if (r == 3) __syncthreads();
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            if (more) gram_issue(c + 1);
            t_update(more);
        }
        }  // chain-free or token buffer
        // the next unit's head, requested while this one finishes (from the codes)
        if (kFromCodes && MODE != kModeDequant && ahead) {
            u_next = work_unit(k + 1);
            head_fetch(u_next);
        }
        // back to S
        if constexpr (KDA) {
            __syncthreads();
            if (n_replay > 0) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r) T[b][r] *= lds_G[((n_replay + EB - 1) / EB) & 1][16 * b + 4 * q + r];
            }
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b) T[b] *= gam;
        }

        // the next unit's start, requested a unit ahead (from the codes)
        if constexpr (MODE == kModeDequant) {
            if (ahead) {
                u_next = work_unit(k + 1);
                head_fetch(u_next);
            }
            head_settle();
            if (ahead) chunk0_fetch(u_next);
#pragma unroll
            for (int b = 0; b < NB; ++b)
                *reinterpret_cast<float4*>(a.S_out + ((size_t)u * D + n) * D + 16 * b + 4 * q) =
                    make_float4((float)T[b][0], (float)T[b][1], (float)T[b][2], (float)T[b][3]);
            __syncthreads();  // LDS is reused by the next unit
            continue;
        }

        {
        // the lane's coordinates again through an opaque copy of the thread
        // index: recomputed here rather than kept live across the replay
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int wave = tid / kWave;
        const int lane = tid % kWave;
        const int q = lane >> 4;
        const int m = lane & 15;
        const int n = 16 * wave + m;
        // ---------------- C1: line scores
        {
            double rs = 0.0;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) rs = __builtin_fma(T[b][r], T[b][r], rs);
            rs = across_rows<false>(rs);
            if (q == 0) lds_score[n] = rs;
            double sq[NV];
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) sq[4 * b + r] = T[b][r] * T[b][r];
            const int v0 = reduce_columns<NV, false>(sq, m);
#pragma unroll
            for (int i = 0; i < NV / 16; ++i) {
                const int v = v0 + i;
                lds_part[wave][16 * (v / 4) + 4 * q + (v % 4)] = sq[i];
            }
            __syncthreads();
            if (tid < D) {
                double t = 0.0;
                for (int w = 0; w < NW; ++w) t += lds_part[w][tid];
                lds_score[D + tid] = t;
            }
            __syncthreads();
        }

        // (the next unit's first chunk, once its head is in: before the stores
        // below, which a wait for the head would otherwise also wait for)
        if constexpr (kFromCodes) {
            head_settle();
            if (ahead) chunk0_fetch(u_next);
        }
        // ---------------- C2: top-n_comp selection (wavefront 0)
        if (wave == 0) {
            // Candidates are ranked by a 64-bit key: 2 + the bits of the score
            // (scores are >= 0, and the bit patterns of non-negative doubles
            // order as their values), 1 for a NaN score (non-finite input:
            // below every real one), 0 once taken.  Each lane sorts its own
            // candidates once (key descending, the lower index first on equal
            // keys); a round takes the wavefront maximum of the lanes' first
            // keys (high words, then the low words of the lanes that tie) and
            // the first lane offering it, whose candidates precede those of
            // later lanes: equal scores go to the lower candidate index.  The
            // winning lane then drops its first candidate.
            uint64_t key[CPL];
            int idx[CPL];
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const double sc = lds_score[lane * CPL + i] + 0.0;  // (a -0.0 as +0.0)
                key[i] = __builtin_isnan(sc) ? 1ull : 2ull + __builtin_bit_cast(uint64_t, sc);
                idx[i] = i;
            }
            auto order = [&](int x, int y) {  // positions x < y: y first if it ranks higher
                const bool sw = key[y] > key[x] || (key[y] == key[x] && idx[y] < idx[x]);
                const uint64_t kx = key[x], ky = key[y];
                const int ix = idx[x], iy = idx[y];
                key[x] = sw ? ky : kx;
                key[y] = sw ? kx : ky;
                idx[x] = sw ? iy : ix;
                idx[y] = sw ? ix : iy;
            };
            static_assert(CPL == 2 || CPL == 4, "two or four candidates per lane");
            if constexpr (CPL == 4) {
                order(0, 1);
                order(2, 3);
                order(0, 2);
                order(1, 3);
                order(1, 2);
            } else {
                order(0, 1);
            }
            int mine = 0;  // lane r: the candidate chosen in round r
            for (int r = 0; r < nc; ++r) {
                const uint32_t hi = (uint32_t)(key[0] >> 32), lo = (uint32_t)key[0];
                const uint32_t mh = wave_max_u32(hi);
                uint64_t win = __ballot(hi == mh);
                if (__builtin_popcountll(win) > 1) {  // uniform: the high words tie
                    const uint32_t ml = wave_max_u32(hi == mh ? lo : 0u);
                    win = __ballot(hi == mh && lo == ml);
                }
                const int L = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(win));
                const int pick = __builtin_amdgcn_readlane(idx[0], L);
                const int best = L * CPL + pick;
                if (lane == L) {
#pragma unroll
                    for (int i = 0; i + 1 < CPL; ++i) {
                        key[i] = key[i + 1];
                        idx[i] = idx[i + 1];
                    }
                    key[CPL - 1] = 0ull;
                }
                if (lane == r) mine = best;
                if (lane == 0) lds_chosen[r] = best;
            }
            // slots in ascending candidate order (rows, then columns)
            for (int x = lane; x < 2 * D; x += kWave) lds_slot[x] = 0;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (lane < nc) {
                int rank = 0;
                for (int q2 = 0; q2 < nc; ++q2) rank += __builtin_amdgcn_readlane(mine, q2) < mine;
                lds_slot[mine] = rank + 1;
                a.blob.comp_idx[(size_t)u * nc + rank] = mine;
            }
        }
        __syncthreads();

        // ---------------- C3: extract compensator lines, zero them in the residual
        {
            float* cvb = a.blob.comp_vec + (size_t)u * nc * D;
            const int rslot = lds_slot[n];
            if (rslot) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    *reinterpret_cast<float4*>(cvb + (size_t)(rslot - 1) * D + 16 * b + 4 * q) =
                        make_float4((float)T[b][0], (float)T[b][1], (float)T[b][2], (float)T[b][3]);
            }
            // column lines: the value positions (4 b + r) that a chosen column
            // meets in some row quad form a scalar mask (the same for every
            // wavefront); at such a position a lane whose column is chosen
            // (its slot from the table) writes the line's value for its row
            // and zeroes it.  Where a row line crosses it, the row line keeps
            // the value.
            const int chl = lds_chosen[max(min(lane, nc - 1), 0)];
            uint32_t pos = 0u;
            for (int c = 0; c < nc; ++c) {
                const int col = __builtin_amdgcn_readlane(chl, c) - D;
                if (col >= 0) pos |= 1u << (4 * (col >> 4) + (col & 3));
            }
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (pos & (1u << (4 * b + r))) {
                        const int cs = lds_slot[D + 16 * b + 4 * q + r];
                        if (cs > 0) {
                            cvb[(size_t)(cs - 1) * D + n] = rslot ? 0.0f : (float)T[b][r];
                            T[b][r] = 0.0;
                        }
                    }
                }
            if (rslot) {
#pragma unroll
                for (int b = 0; b < NB; ++b) T[b] = v4d{0.0, 0.0, 0.0, 0.0};
            }
        }

        // (the next unit's first chunk, once its window count is in)
        // ---------------- C4: smoothing per key channel
        {
            double am[NV];
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) am[4 * b + r] = fabs(T[b][r]);
            const int v0 = reduce_columns<NV, true>(am, m);
#pragma unroll
            for (int i = 0; i < NV / 16; ++i) {
                const int v = v0 + i;
                lds_part[wave][16 * (v / 4) + 4 * q + (v % 4)] = am[i];
            }
            __syncthreads();
            if (tid < D) {
                double mx = 0.0;
                for (int w = 0; w < NW; ++w) mx = fmax(mx, lds_part[w][tid]);
                const float sj = mx > 0.0 ? (float)sqrt(mx) : 1.0f;
                lds_smooth[tid] = sj;
                lds_ismooth[tid] = 1.0 / (double)sj;
                a.blob.smooth[(size_t)u * D + tid] = sj;
            }
            __syncthreads();
        }

        // ---------------- C5: per-row scale and codes
        {
            // divisions by s_j, then by sigma_i, as products with FP64
            // reciprocals (a few ulps of FP64 off the quotient; the codes round
            // at 2^-10 of a tie or closer only by chance either way).  T is
            // divided in place: it is not needed after the codes.
            double mx = 0.0;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    T[b][r] *= lds_ismooth[16 * b + 4 * q + r];
                    mx = fmax(mx, fabs(T[b][r]));
                }
            mx = across_rows<true>(mx);
            const bool e4m3 = a.dm.code_format == LQ_CODE_E4M3;
            const float sg = (float)(mx / (e4m3 ? 448.0 : 127.0));
            if (q == 0) a.blob.sigma[(size_t)u * D + n] = sg;
            // an all-zero row (sigma 0) gets 1/sigma = 0, so every x below is 0
            // and takes code 0
            const double isg = sg != 0.0f ? 1.0 / (double)sg : 0.0;
            uint32_t* crow = reinterpret_cast<uint32_t*>(a.blob.codes + ((size_t)u * D + n) * D + 4 * q);
            if (e4m3) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    uint32_t packed = 0u;
#pragma unroll
                    for (int r = 0; r < 4; ++r) packed |= e4m3_code(T[b][r] * isg) << (8 * r);
                    crow[4 * b] = packed;
                }
            } else {
#pragma unroll
                // |x| <= 127 (1 + 2^-23) here, so rint gives a code in [-127, 127]
                // (the integer clamp only guards a non-finite state); the four
                // low bytes are packed by byte permutes
                for (int b = 0; b < NB; ++b) {
                    int k[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) k[r] = min(max((int)rint(T[b][r] * isg), -127), 127);
                    const uint32_t lo = __builtin_amdgcn_perm((uint32_t)k[1], (uint32_t)k[0], 0x0c0c0400u);
                    const uint32_t hi = __builtin_amdgcn_perm((uint32_t)k[3], (uint32_t)k[2], 0x0c0c0400u);
                    crow[4 * b] = lo | (hi << 16);
                }
            }
        }
        }
        if (tid == 0) a.blob.fill[u] = 0;
        __syncthreads();  // LDS is reused by the next unit
    }
}

// Units whose window is due, in ascending order, into the blob's work list.
// A pass covers 16 blocks of 1,024 units: every thread requests all of its
// fill counts and sequence flags before it uses any (one memory trip per pass,
// not one per block), the per-wavefront counts of the pass are scanned once,
// and each due unit is written at its offset.
__global__ __launch_bounds__(1024) void due_scan_kernel(MatArgs a) {
    constexpr int P = 16;      // 1,024-unit blocks per pass
    constexpr int NWV = 16;    // wavefronts
    __shared__ int cnt[P * NWV];  // due units per (block, wavefront), then their offsets
    __shared__ int base;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = lane_id();
    const int n = a.dm.n_units;
    if (tid == 0) base = 0;
    for (int p0 = 0; p0 < n; p0 += P * 1024) {
        int fill[P], forced[P];
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int u = p0 + i * 1024 + tid;
            const bool in = u < n;
            fill[i] = in ? a.blob.fill[u] : 0;
            forced[i] = (in && a.force != nullptr) ? (int)a.force[u / a.dm.n_v_heads] : 0;
        }
        uint64_t mask[P];
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const bool due = fill[i] >= a.dm.window || (forced[i] != 0 && fill[i] > 0);
            mask[i] = __ballot(due);
            if (lane == 0) cnt[i * NWV + wave] = __popcll(mask[i]);
        }
        __syncthreads();
        if (wave == 0) {
            // exclusive offsets in (block, wavefront) order: four counts per
            // lane, then an inclusive scan of the lane sums
            static_assert(P * NWV == 4 * kWave, "four counts per lane");
            int c[4], sum = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[j] = cnt[4 * lane + j];
                sum += c[j];
            }
            int incl = sum;
#pragma unroll
            for (int d = 1; d < kWave; d *= 2) {
                const int y = __shfl_up(incl, d, kWave);
                if (lane >= d) incl += y;
            }
            int off = base + incl - sum;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                cnt[4 * lane + j] = off;
                off += c[j];
            }
            const int total = __shfl(incl, kWave - 1, kWave);
            if (lane == 0) base += total;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const uint64_t m = mask[i];
            if ((m >> lane) & 1u) {
                const int before =
                    __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
                a.blob.work[1 + cnt[i * NWV + wave] + before] = p0 + i * 1024 + tid;
            }
        }
        __syncthreads();  // the offsets are rewritten by the next pass
    }
    if (tid == 0) a.blob.work[0] = base;
}

__global__ void clear_status_kernel(uint32_t* status) { *status = 0u; }

// Workgroups of `kernel` that the CUs available to it hold at once: the size
// of a persistent grid, asked of the runtime at every launch (the library
// keeps no state between calls).  The CUs are the device's, at most max_cus
// of them when max_cus > 0 (the caller's share for a boundary that runs
// beside other kernels; the grid stays within it wherever the dispatcher
// places it, because the d = 128 workgroup needs a whole CU).  0 when the
// runtime cannot say (the caller then falls back to a fixed size).
template <typename K>
int resident_blocks(K kernel, int block, int max_cus) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, block, 0) != hipSuccess) return 0;
    const int n = (max_cus > 0 && max_cus < cus) ? max_cus : cus;
    return n * (per > 0 ? per : 1);
}

hipError_t launch_materialize(const MatArgs& a, int mode, int d, int gate_kind, hipStream_t st) {
    // a persistent grid, as many workgroups as the device holds at once, walks
    // the units (init, dequant, prefill) or the work list (flush): idle
    // workgroups would otherwise wait for a free CU only to find no work
    const int block_threads = kWave * d / 16;
    const dim3 block(block_threads);
    const bool kda = gate_kind == LQ_GATE_CHANNEL;
    if (mode == kModeInit || mode == kModePrefill) {
        // a new state starts with no flags; cleared before any unit can raise one
        hipError_t e = launch_clear_status(a.blob.status, st);
        if (e != hipSuccess) return e;
    }
    if (mode == kModeFlush) {
        hipLaunchKernelGGL(due_scan_kernel, dim3(1), dim3(1024), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    auto grid_for = [&](auto kernel) {
        int g = resident_blocks(kernel, block_threads, a.dm.max_cus);
        if (g <= 0) g = 2048;
        return dim3(a.dm.n_units < g ? a.dm.n_units : g);
    };
    const bool h16 = a.dm.buffer_format == LQ_BUFFER_FP16;
    const bool nf = a.dm.buffer_format == LQ_BUFFER_NFORM;
#define LQ_MAT(D_, K_, M_, H_)                                                                  \
    hipLaunchKernelGGL((materialize_kernel<D_, K_, M_, H_>), grid_for(materialize_kernel<D_, K_, M_, H_>), \
                       block, 0, st, a)
#define LQ_MAT_NF(D_, M_)                                                                        \
    hipLaunchKernelGGL((materialize_kernel<D_, false, M_, false, true>),                         \
                       grid_for(materialize_kernel<D_, false, M_, false, true>), block, 0, st, a)
#define LQ_MAT_MODE(D_, K_)                                                            \
    do {                                                                               \
        if (mode == kModeInit) LQ_MAT(D_, K_, kModeInit, false);                       \
        else if (nf && !K_ && D_ == 128 && mode == kModeFlush) LQ_MAT_NF(128, kModeFlush);     \
        else if (nf && !K_ && D_ == 128 && mode == kModeDequant) LQ_MAT_NF(128, kModeDequant); \
        else if (mode == kModePrefill) LQ_MAT(D_, K_, kModePrefill, false);            \
        else if (mode == kModeFlush && h16) LQ_MAT(D_, K_, kModeFlush, true);          \
        else if (mode == kModeFlush) LQ_MAT(D_, K_, kModeFlush, false);                \
        else if (h16) LQ_MAT(D_, K_, kModeDequant, true);                              \
        else LQ_MAT(D_, K_, kModeDequant, false);                                      \
    } while (0)
    if (d == 128) {
        if (kda) LQ_MAT_MODE(128, true);
        else LQ_MAT_MODE(128, false);
    } else {
        if (kda) LQ_MAT_MODE(64, true);
        else LQ_MAT_MODE(64, false);
    }
#undef LQ_MAT_MODE
#undef LQ_MAT_NF
#undef LQ_MAT
    return hipGetLastError();
}

hipError_t launch_clear_status(uint32_t* status, hipStream_t st) {
    hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(1), 0, st, status);
    return hipGetLastError();
}

}  // namespace lq
