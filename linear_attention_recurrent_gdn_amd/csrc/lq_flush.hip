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
// One workgroup per unit, four threads per state row, each thread holding a
// quarter row in FP64 registers:
//   A  load: S = Diag(sigma) Q Diag(s) + compensator lines (flush, dequant) or
//      the caller's FP32 start state (init);
//   B  forward replay of the buffered tokens, row form
//        x = g * S[i,:];  S[i,:] = x + beta (v_i - x.k) k
//      in FP64 with the buffer staged through LDS a batch at a time (FP64 so
//      that the rounding decisions below match an FP64 reference);
//   C  quantizer, in the same pass (readings; the pages print no formula):
//        line scores = squared L2 norms of rows and columns; the n_comp best
//        lines (ties to the lower candidate index, rows before columns) go to
//        fp32 compensator slots, rows taken whole, columns with the selected
//        rows' entries zeroed; the residual R has those lines zeroed;
//        s_j = sqrt(max_i |R_ij|) (1 if zero), sigma_i = max_j |R_ij/s_j|/127,
//        both fp32; codes = clamp(rne(R_ij / (sigma_i s_j)), -127, 127).
// Column reductions go lane-to-lane inside a wave (reduce-scatter over the
// 16 rows a wave holds), then across waves through LDS in a fixed order, so
// results are deterministic.

#include "lq_internal.h"

namespace lq {

namespace {

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ double sum4_f64(double x) {
    x += dpp_f64<kDppQuadXor1>(x);
    x += dpp_f64<kDppQuadXor2>(x);
    return x;
}

__device__ __forceinline__ double max4_f64(double x) {
    x = fmax(x, dpp_f64<kDppQuadXor1>(x));
    x = fmax(x, dpp_f64<kDppQuadXor2>(x));
    return x;
}

__device__ __forceinline__ double shfl_xor_f64(double x, int m) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const int lane = lane_id();
    const int src = (lane ^ m) << 2;
    const int lo = __builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)b);
    const int hi = __builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(b >> 32));
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Reduce-scatter of a thread's CPT column values over the 16 lanes of a wave
// that share its column quarter (lane bits 2..5).  Afterwards each lane holds
// CPT/16 reduced values in v[0 .. CPT/16); their columns are
// c0 + colbase + {0 .. CPT/16 - 1}, colbase returned.
template <int CPT, int N, bool MAX>
__device__ __forceinline__ void rs_stage(double (&v)[CPT], int lane, int m, int& colbase) {
    constexpr int HALF = N / 2;
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
        const double keep = upper ? v[HALF + i] : v[i];
        const double send = upper ? v[i] : v[HALF + i];
        const double got = shfl_xor_f64(send, m);
        v[i] = MAX ? fmax(keep, got) : keep + got;
    }
    if (upper) colbase += HALF;
}

template <int CPT, bool MAX>
__device__ __forceinline__ int reduce_scatter_cols(double (&v)[CPT]) {
    const int lane = lane_id();
    int colbase = 0;
    rs_stage<CPT, CPT, MAX>(v, lane, 4, colbase);
    rs_stage<CPT, CPT / 2, MAX>(v, lane, 8, colbase);
    rs_stage<CPT, CPT / 4, MAX>(v, lane, 16, colbase);
    rs_stage<CPT, CPT / 8, MAX>(v, lane, 32, colbase);
    return colbase;
}

}  // namespace

template <int D, bool KDA, int MODE>
__global__ __launch_bounds__(4 * D) void materialize_kernel(MatArgs a) {
    constexpr int NT = 4 * D;
    constexpr int CPT = D / 4;     // columns per thread
    constexpr int NW = NT / kWave; // waves per workgroup
    constexpr int EB = 16;         // buffered tokens staged per batch
    constexpr int CPL = 2 * D / kWave;  // selection candidates per lane
    static_assert(CPT % 16 == 0, "reduce-scatter needs 16 | CPT");

    __shared__ double lds_k[EB][D];
    __shared__ float lds_v[EB][D];
    __shared__ float lds_g[KDA ? EB : 1][KDA ? D : 1];
    __shared__ float lds_b[EB];
    __shared__ float lds_a[EB];
    __shared__ double lds_score[2 * D];
    __shared__ double lds_part[NW][D];
    __shared__ float lds_smooth[D];
    __shared__ int lds_slot[2 * D];  // slot + 1 of each selected candidate, 0 otherwise
    __shared__ int lds_chosen[16];

    const int u = blockIdx.x;
    const int tid = threadIdx.x;
    const int row = tid >> 2;
    const int qd = tid & 3;
    const int c0 = qd * CPT;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int W = a.dm.window;
    const int nc = a.dm.n_comp;
    const int s = u / a.dm.n_v_heads;
    const int h = u - s * a.dm.n_v_heads;
    const int kh = h / a.dm.group;
    const size_t kvec = (size_t)s * a.dm.n_k_heads + kh;

    int n_replay = 0;
    if constexpr (MODE == kModeFlush) {
        const int fill = a.blob.fill[u];
        const bool forced = a.force != nullptr && a.force[s] != 0 && fill > 0;
        if (!(fill >= W || forced)) return;  // not due: untouched (uniform per workgroup)
        n_replay = fill < W ? fill : W;
    } else if constexpr (MODE == kModeDequant) {
        if (a.include_buffer) {
            const int fill = a.blob.fill[u];
            n_replay = fill < W ? fill : W;
        }
    }

    // ---------------- A: load the window-start state
    double S[CPT];
    if constexpr (MODE == kModeInit) {
        if (a.S0 != nullptr) {
            const float4* src = reinterpret_cast<const float4*>(a.S0 + ((size_t)u * D + row) * D + c0);
#pragma unroll
            for (int t = 0; t < CPT / 4; ++t) {
                const float4 f = src[t];
                S[4 * t + 0] = f.x;
                S[4 * t + 1] = f.y;
                S[4 * t + 2] = f.z;
                S[4 * t + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int c = 0; c < CPT; ++c) S[c] = 0.0;
        }
    } else {
        const double sgr = (double)a.blob.sigma[(size_t)u * D + row];
        const uint4* cp = reinterpret_cast<const uint4*>(a.blob.codes + ((size_t)u * D + row) * D + c0);
        const float4* sp = reinterpret_cast<const float4*>(a.blob.smooth + (size_t)u * D + c0);
#pragma unroll
        for (int t = 0; t < CPT / 16; ++t) {
            const uint4 w = cp[t];
            const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int b = 0; b < 16; ++b) {
                const int code = (int)(wd[b / 4] << (24 - 8 * (b % 4))) >> 24;
                const float4 s4 = sp[(16 * t + b) / 4];
                const float sj = ((b % 4) == 0) ? s4.x : ((b % 4) == 1) ? s4.y : ((b % 4) == 2) ? s4.z : s4.w;
                S[16 * t + b] = sgr * (double)code * (double)sj;
            }
        }
        for (int sl = 0; sl < nc; ++sl) {
            const int idx = a.blob.comp_idx[(size_t)u * nc + sl];
            const float* vec = a.blob.comp_vec + ((size_t)u * nc + sl) * D;
            if (idx < D) {
                if (idx == row) {
#pragma unroll
                    for (int c = 0; c < CPT; ++c) S[c] += (double)vec[c0 + c];
                }
            } else {
                const int col = idx - D;
                if (col >= c0 && col < c0 + CPT) {
                    const double add = (double)vec[row];
#pragma unroll
                    for (int c = 0; c < CPT; ++c)
                        if (c0 + c == col) S[c] += add;
                }
            }
        }
    }

    // ---------------- B: forward replay of the buffered tokens (FP64)
    const float* bk = a.blob.buf_k + kvec * (size_t)W * D;
    const float* bv = a.blob.buf_v + (size_t)u * W * D;
    const float* bb = a.blob.buf_beta + (size_t)u * W;
    const float* bg = a.blob.buf_gate + (size_t)u * W * (KDA ? D : 1);
    for (int i0 = 0; i0 < n_replay; i0 += EB) {
        const int ne = (n_replay - i0) < EB ? (n_replay - i0) : EB;
        __syncthreads();
        for (int x = tid; x < ne * D; x += NT) {
            const int e = x / D, c = x - e * D;
            lds_k[e][c] = (double)bk[(size_t)(i0 + e) * D + c];
            lds_v[e][c] = bv[(size_t)(i0 + e) * D + c];
            if constexpr (KDA) lds_g[e][c] = bg[(size_t)(i0 + e) * D + c];
        }
        if (tid < ne) {
            lds_b[tid] = bb[i0 + tid];
            if constexpr (!KDA) lds_a[tid] = bg[i0 + tid];
        }
        __syncthreads();
        for (int e = 0; e < ne; ++e) {
            double d = 0.0;
            if constexpr (KDA) {
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    S[c] *= (double)lds_g[e][c0 + c];
                    d = __builtin_fma(S[c], lds_k[e][c0 + c], d);
                }
            } else {
                const double al = (double)lds_a[e];
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    S[c] *= al;
                    d = __builtin_fma(S[c], lds_k[e][c0 + c], d);
                }
            }
            d = sum4_f64(d);
            const double coef = (double)lds_b[e] * ((double)lds_v[e][row] - d);
#pragma unroll
            for (int c = 0; c < CPT; ++c) S[c] = __builtin_fma(coef, lds_k[e][c0 + c], S[c]);
        }
    }

    if constexpr (MODE == kModeDequant) {
        float4* dst = reinterpret_cast<float4*>(a.S_out + ((size_t)u * D + row) * D + c0);
#pragma unroll
        for (int t = 0; t < CPT / 4; ++t)
            dst[t] = make_float4((float)S[4 * t], (float)S[4 * t + 1], (float)S[4 * t + 2], (float)S[4 * t + 3]);
        return;
    }

    // ---------------- C1: line scores
    {
        double rs = 0.0;
#pragma unroll
        for (int c = 0; c < CPT; ++c) rs = __builtin_fma(S[c], S[c], rs);
        rs = sum4_f64(rs);
        if (qd == 0) lds_score[row] = rs;
        double sq[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) sq[c] = S[c] * S[c];
        const int cb = reduce_scatter_cols<CPT, false>(sq);
#pragma unroll
        for (int i = 0; i < CPT / 16; ++i) lds_part[wave][c0 + cb + i] = sq[i];
        __syncthreads();
        if (tid < D) {
            double t = 0.0;
            for (int w = 0; w < NW; ++w) t += lds_part[w][tid];
            lds_score[D + tid] = t;
        }
        __syncthreads();
    }

    // ---------------- C2: top-n_comp selection (wave 0)
    if (wave == 0) {
        // scores are >= 0; a NaN score (non-finite input) ranks below every
        // real one, and a lane with nothing left offers (-1, INT_MAX), which
        // always loses, so every round picks one untaken candidate
        double val[CPL];
        bool taken[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const double sc = lds_score[lane * CPL + i];
            val[i] = __builtin_isnan(sc) ? -0.5 : sc;
            taken[i] = false;
        }
        for (int r = 0; r < nc; ++r) {
            double bv_ = -1.0;
            int bi = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                if (!taken[i] && val[i] > bv_) {
                    bv_ = val[i];
                    bi = lane * CPL + i;
                }
            for (int m = 1; m < kWave; m <<= 1) {
                const double ov = shfl_xor_f64(bv_, m);
                const int oi = __shfl_xor(bi, m);
                if (ov > bv_ || (ov == bv_ && oi < bi)) {
                    bv_ = ov;
                    bi = oi;
                }
            }
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                if (bi == lane * CPL + i) taken[i] = true;
            if (lane == 0) lds_chosen[r] = bi;
        }
        // slots in ascending candidate order (rows, then columns)
        for (int x = lane; x < 2 * D; x += kWave) lds_slot[x] = 0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < nc) {
            const int me = lds_chosen[lane];
            int rank = 0;
            for (int q2 = 0; q2 < nc; ++q2) rank += lds_chosen[q2] < me;
            lds_slot[me] = rank + 1;
            a.blob.comp_idx[(size_t)u * nc + rank] = me;
        }
    }
    __syncthreads();

    // ---------------- C3: extract compensator lines, zero them in the residual
    {
        const int rslot = lds_slot[row];
        float* cvb = a.blob.comp_vec + (size_t)u * nc * D;
        if (rslot) {
#pragma unroll
            for (int c = 0; c < CPT; ++c) cvb[(size_t)(rslot - 1) * D + c0 + c] = (float)S[c];
        }
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int cs = lds_slot[D + c0 + c];
            if (cs) {
                cvb[(size_t)(cs - 1) * D + row] = rslot ? 0.0f : (float)S[c];
                S[c] = 0.0;
            }
            if (rslot) S[c] = 0.0;
        }
    }

    // ---------------- C4: smoothing per key channel
    {
        double am[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) am[c] = fabs(S[c]);
        const int cb = reduce_scatter_cols<CPT, true>(am);
#pragma unroll
        for (int i = 0; i < CPT / 16; ++i) lds_part[wave][c0 + cb + i] = am[i];
        __syncthreads();
        if (tid < D) {
            double m = 0.0;
            for (int w = 0; w < NW; ++w) m = fmax(m, lds_part[w][tid]);
            const float sj = m > 0.0 ? (float)sqrt(m) : 1.0f;
            lds_smooth[tid] = sj;
            a.blob.smooth[(size_t)u * D + tid] = sj;
        }
        __syncthreads();
    }

    // ---------------- C5: per-row scale and codes
    {
        double sj[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) sj[c] = (double)lds_smooth[c0 + c];
        double m = 0.0;
#pragma unroll
        for (int c = 0; c < CPT; ++c) m = fmax(m, fabs(S[c] / sj[c]));
        m = max4_f64(m);
        const float sg = (float)(m / 127.0);
        if (qd == 0) a.blob.sigma[(size_t)u * D + row] = sg;
        uint32_t packed[CPT / 4];
#pragma unroll
        for (int w = 0; w < CPT / 4; ++w) packed[w] = 0;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            int code = 0;
            if (sg != 0.0f) {
                double x = rint(S[c] / ((double)sg * sj[c]));
                x = fmin(fmax(x, -127.0), 127.0);
                code = (int)x;
            }
            packed[c / 4] |= ((uint32_t)code & 0xFFu) << (8 * (c % 4));
        }
        uint4* dst = reinterpret_cast<uint4*>(a.blob.codes + ((size_t)u * D + row) * D + c0);
#pragma unroll
        for (int t = 0; t < CPT / 16; ++t)
            dst[t] = make_uint4(packed[4 * t], packed[4 * t + 1], packed[4 * t + 2], packed[4 * t + 3]);
    }
    if (tid == 0) {
        a.blob.fill[u] = 0;
        if (MODE == kModeInit && u == 0) *a.blob.status = 0u;
    }
}

__global__ void clear_status_kernel(uint32_t* status) { *status = 0u; }

hipError_t launch_materialize(const MatArgs& a, int mode, int d, int gate_kind, hipStream_t st) {
    const dim3 grid(a.dm.n_units), block(4 * d);
    const bool kda = gate_kind == LQ_GATE_CHANNEL;
#define LQ_MAT(D_, K_, M_) hipLaunchKernelGGL((materialize_kernel<D_, K_, M_>), grid, block, 0, st, a)
#define LQ_MAT_MODE(D_, K_)                              \
    do {                                                 \
        if (mode == kModeInit) LQ_MAT(D_, K_, kModeInit);       \
        else if (mode == kModeFlush) LQ_MAT(D_, K_, kModeFlush); \
        else LQ_MAT(D_, K_, kModeDequant);                \
    } while (0)
    if (d == 128) {
        if (kda) LQ_MAT_MODE(128, true);
        else LQ_MAT_MODE(128, false);
    } else {
        if (kda) LQ_MAT_MODE(64, true);
        else LQ_MAT_MODE(64, false);
    }
#undef LQ_MAT_MODE
#undef LQ_MAT
    return hipGetLastError();
}

hipError_t launch_clear_status(uint32_t* status, hipStream_t st) {
    hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(1), 0, st, status);
    return hipGetLastError();
}

}  // namespace lq
