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
// Materialize: one workgroup per unit at a time, each thread holding 2 rows x
// 16 columns of the state in FP64 registers (a row is split over D/16
// consecutive lanes):
//   A  load: S = Diag(sigma) Q Diag(s) + compensator lines (flush, dequant) or
//      the caller's FP32 start state (init);
//   B  forward replay of the buffered tokens in FP64 (FP64 so that the
//      rounding decisions below match an FP64 reference), in a rescaled form
//      that costs two FMAs per element and token:
//        scalar gate  S = g T:  g' = g alpha;  d = T[i,:].k;
//                     T[i,:] += beta (v_i - g' d) / g' * k
//        channel gate S = T Diag(G):  G' = G * a;  d = T[i,:].(G' * k);
//                     T[i,:] += beta (v_i - d) * (k / G')
//      (a token-by-token restatement of x = g * S[i,:]; S[i,:] = x + beta
//      (v_i - x.k) k).  g and G are folded into T before they can
//      underflow.  The key (and for the channel gate its two scaled forms) is
//      staged through LDS as FP64, a batch of tokens at a time, with a padded
//      layout so the D/16 column chunks that a wavefront reads at once fall in
//      different LDS banks;
//   C  quantizer, in the same workgroup (readings; the pages print no
//      formula): line scores = squared L2 norms of rows and columns; the
//      n_comp best lines (ties to the lower candidate index, rows before
//      columns) go to fp32 compensator slots, rows taken whole, columns with
//      the selected rows' entries zeroed; the residual R has those lines
//      zeroed; s_j = sqrt(max_i |R_ij|) (1 if zero), sigma_i =
//      max_j |R_ij / s_j| / 127, both fp32; codes = clamp(rne(R_ij /
//      (sigma_i s_j)), -127, 127).
// Column reductions go lane-to-lane inside a wavefront (reduce-scatter over
// its row pairs), then across wavefronts through LDS in a fixed order, so
// results are deterministic.

#include "lq_internal.h"

namespace lq {

namespace {

constexpr double kRescaleBelow = 0x1p-200;   // fold the gate product into T below this
constexpr double kMinChannelGate = 0x1p-45;  // per-token channel gate floor inside the flush

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Sum / max over groups of N consecutive lanes (N = 4 or 8), result in every lane.
template <int N>
__device__ __forceinline__ double group_sum(double x) {
    if constexpr (N == 8) x += dpp_f64<kDppRowHalfMirror>(x);
    x += dpp_f64<kDppQuadXor2>(x);
    x += dpp_f64<kDppQuadXor1>(x);
    return x;
}
template <int N>
__device__ __forceinline__ double group_max(double x) {
    if constexpr (N == 8) x = fmax(x, dpp_f64<kDppRowHalfMirror>(x));
    x = fmax(x, dpp_f64<kDppQuadXor2>(x));
    x = fmax(x, dpp_f64<kDppQuadXor1>(x));
    return x;
}

__device__ __forceinline__ double shfl_xor_f64(double x, int m) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const int src = (lane_id() ^ m) << 2;
    const int lo = __builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)b);
    const int hi = __builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(b >> 32));
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// One reduce-scatter stage over lane bit m: keep half of the N values, add
// (or max) the partner's copy of that half.
template <int N, bool MAX>
__device__ __forceinline__ void rs_stage(double (&v)[16], int m, int& colbase) {
    constexpr int HALF = N / 2;
    const bool upper = (lane_id() & m) != 0;
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
        const double keep = upper ? v[HALF + i] : v[i];
        const double send = upper ? v[i] : v[HALF + i];
        const double got = shfl_xor_f64(send, m);
        v[i] = MAX ? fmax(keep, got) : keep + got;
    }
    if (upper) colbase += HALF;
}

// Reduce each of a thread's 16 column values over the row pairs of its
// wavefront (the lanes that share its column chunk).  Afterwards each lane
// holds 16 / (64 / CPR) reduced values in v[0..); their columns are
// c0 + colbase + i.
template <int CPR, bool MAX>
__device__ __forceinline__ int reduce_rows_in_wave(double (&v)[16]) {
    int colbase = 0;
    if constexpr (CPR == 8) {  // row pairs on lane bits 3..5
        rs_stage<16, MAX>(v, 8, colbase);
        rs_stage<8, MAX>(v, 16, colbase);
        rs_stage<4, MAX>(v, 32, colbase);
    } else {  // CPR == 4: row pairs on lane bits 2..5
        rs_stage<16, MAX>(v, 4, colbase);
        rs_stage<8, MAX>(v, 8, colbase);
        rs_stage<4, MAX>(v, 16, colbase);
        rs_stage<2, MAX>(v, 32, colbase);
    }
    return colbase;
}

__device__ __forceinline__ float pick4(const float4& f, int i) {
    return i == 0 ? f.x : i == 1 ? f.y : i == 2 ? f.z : f.w;
}

// One batch of buffered tokens as fetched by one thread of the materialize
// kernel: F4 float4 of the batch's keys, values and channel gates (token-major,
// D floats per token), and, for the first threads, one beta and scalar gate.
template <int F4, bool KDA>
struct Stage {
    float4 k[F4], v[F4], g[KDA ? F4 : 1];
    float b, al;
};

template <int D, int EB, int NT, int F4, bool KDA>
__device__ __forceinline__ Stage<F4, KDA> fetch_stage(const float* bk, const float* bv, const float* bb,
                                                     const float* bg, int i0, int n_replay, int tid) {
    Stage<F4, KDA> st;
    const int ne = (n_replay - i0) < EB ? (n_replay - i0) : EB;
#pragma unroll
    for (int f = 0; f < F4; ++f) {
        const int x = 4 * (tid + f * NT);
        const int e = min(x / D, ne - 1), c = x % D;
        st.k[f] = *reinterpret_cast<const float4*>(bk + (size_t)(i0 + e) * D + c);
        st.v[f] = *reinterpret_cast<const float4*>(bv + (size_t)(i0 + e) * D + c);
        if constexpr (KDA) st.g[f] = *reinterpret_cast<const float4*>(bg + (size_t)(i0 + e) * D + c);
    }
    st.b = 0.f;
    st.al = 1.f;
    if (tid < EB) {
        st.b = bb[i0 + min(tid, ne - 1)];
        if constexpr (!KDA) st.al = bg[i0 + min(tid, ne - 1)];
    }
    return st;
}

}  // namespace

// Units whose window is due, in ascending order, into the blob's work list.
__global__ __launch_bounds__(1024) void due_scan_kernel(MatArgs a) {
    __shared__ int wave_cnt[16];
    __shared__ int base;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = lane_id();
    if (tid == 0) base = 0;
    __syncthreads();
    for (int c0 = 0; c0 < a.dm.n_units; c0 += 1024) {
        const int u = c0 + tid;
        bool due = false;
        if (u < a.dm.n_units) {
            const int fill = a.blob.fill[u];
            const int s = u / a.dm.n_v_heads;
            due = fill >= a.dm.window || (a.force != nullptr && a.force[s] != 0 && fill > 0);
        }
        const uint64_t m = __ballot(due);
        const int before =
            __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (lane == 0) wave_cnt[wave] = __popcll(m);
        __syncthreads();
        int off = base;
        for (int w = 0; w < wave; ++w) off += wave_cnt[w];
        if (due) a.blob.work[1 + off + before] = u;
        __syncthreads();
        if (tid == 0) {
            int t = 0;
            for (int w = 0; w < 16; ++w) t += wave_cnt[w];
            base += t;
        }
        __syncthreads();
    }
    if (tid == 0) a.blob.work[0] = base;
}

template <int D, bool KDA, int MODE>
__global__ __launch_bounds__(D * D / 32) void materialize_kernel(MatArgs a) {
    constexpr int CPR = D / 16;         // column chunks per row = threads per row pair
    constexpr int NT = D * D / 32;      // threads
    constexpr int NW = NT / kWave;      // wavefronts
    constexpr int EB = D == 128 ? 16 : 8;  // buffered tokens staged per batch (one float4 per thread)
    constexpr int KS = CPR * 18;        // padded FP64 length of one staged key (18 per 16-chunk)
    constexpr int CPL = 2 * D / kWave;  // selection candidates per lane
    constexpr int RPW = 64 / CPR;       // row pairs per wavefront
    constexpr int NVAL = 16 / RPW;      // reduced column values per lane after reduce_rows_in_wave
    constexpr int F4 = EB * D / (4 * NT);  // float4 of a staged batch per thread

    __shared__ double lds_k[EB][KS];                        // key (scalar gate) or G' * key (channel gate)
    __shared__ double lds_kd[KDA ? EB : 1][KDA ? KS : 1];  // key / G' (channel gate)
    __shared__ float lds_v[EB][D];
    __shared__ float lds_kraw[KDA ? EB : 1][KDA ? D : 1];  // channel gate: keys as fetched
    __shared__ float lds_graw[KDA ? EB : 1][KDA ? D : 1];  // channel gate: gates as fetched
    __shared__ float lds_al[KDA ? 1 : EB];                  // scalar gate: gates as fetched
    __shared__ double lds_coef[EB][2];  // scalar gate: g', 1 / g'
    __shared__ float lds_b[EB];
    __shared__ int lds_resc[EB];        // scalar gate: fold g into T before this token
    __shared__ double lds_G[KDA ? D : 1];     // channel gate: running G per column
    __shared__ double lds_fold[KDA ? D : 1];  // channel gate: per-column fold factor of a batch
    __shared__ double lds_score[2 * D];
    __shared__ double lds_part[NW][D];
    __shared__ float lds_smooth[D];
    __shared__ double lds_ismooth[D];
    __shared__ int lds_slot[2 * D];  // slot + 1 of each selected candidate, 0 otherwise
    __shared__ int lds_chosen[16];

    const int tid = threadIdx.x;
    const int rp = tid / CPR;  // row pair
    const int ch = tid % CPR;  // column chunk
    const int r0 = 2 * rp;
    const int c0 = ch * 16;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int W = a.dm.window;
    const int nc = a.dm.n_comp;

    const int n_work = (MODE == kModeFlush) ? a.blob.work[0] : a.dm.n_units;
    for (int wi = blockIdx.x; wi < n_work; wi += gridDim.x) {
        const int u = (MODE == kModeFlush) ? a.blob.work[1 + wi] : wi;
        const int s = u / a.dm.n_v_heads;
        const int h = u - s * a.dm.n_v_heads;
        const int kh = h / a.dm.group;
        const size_t kvec = (size_t)s * a.dm.n_k_heads + kh;

        int n_replay = 0;
        if (MODE == kModeFlush || (MODE == kModeDequant && a.include_buffer)) {
            const int fill = a.blob.fill[u];
            n_replay = fill < W ? fill : W;
        }

        // ---------------- A: the window-start state, 2 rows x 16 columns per thread
        double T[2][16];
        if constexpr (MODE == kModeInit) {
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                if (a.S0 != nullptr) {
                    const float4* src =
                        reinterpret_cast<const float4*>(a.S0 + ((size_t)u * D + r0 + rr) * D + c0);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float4 f = src[t];
                        T[rr][4 * t + 0] = f.x;
                        T[rr][4 * t + 1] = f.y;
                        T[rr][4 * t + 2] = f.z;
                        T[rr][4 * t + 3] = f.w;
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < 16; ++c) T[rr][c] = 0.0;
                }
            }
        } else {
            const float4* sp = reinterpret_cast<const float4*>(a.blob.smooth + (size_t)u * D + c0);
            float4 s4[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) s4[t] = sp[t];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const double sgr = (double)a.blob.sigma[(size_t)u * D + r0 + rr];
                const uint4 w = *reinterpret_cast<const uint4*>(a.blob.codes + ((size_t)u * D + r0 + rr) * D + c0);
                const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int b = 0; b < 16; ++b) {
                    const int code = (int)(wd[b / 4] << (24 - 8 * (b % 4))) >> 24;
                    T[rr][b] = sgr * (double)code * (double)pick4(s4[b / 4], b % 4);
                }
            }
            // compensator lines, four slots at a time: every load of a group is
            // issued before any is used (row slots use the 16 columns of this
            // thread, column slots the entries of its two rows)
            for (int sl0 = 0; sl0 < nc; sl0 += 4) {
                int idx[4];
                float4 rowv[4][4];
                float colv[4][2];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int sl = min(sl0 + q, nc - 1);
                    idx[q] = a.blob.comp_idx[(size_t)u * nc + sl];
                    const float* vec = a.blob.comp_vec + ((size_t)u * nc + sl) * D;
#pragma unroll
                    for (int t = 0; t < 4; ++t) rowv[q][t] = reinterpret_cast<const float4*>(vec + c0)[t];
                    colv[q][0] = vec[r0];
                    colv[q][1] = vec[r0 + 1];
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (sl0 + q >= nc) break;
                    if (idx[q] < D) {
#pragma unroll
                        for (int rr = 0; rr < 2; ++rr)
                            if (idx[q] == r0 + rr) {
#pragma unroll
                                for (int c = 0; c < 16; ++c) T[rr][c] += (double)pick4(rowv[q][c / 4], c % 4);
                            }
                    } else {
                        const int col = idx[q] - D;
#pragma unroll
                        for (int c = 0; c < 16; ++c)
                            if (c0 + c == col) {
                                T[0][c] += (double)colv[q][0];
                                T[1][c] += (double)colv[q][1];
                            }
                    }
                }
            }
        }

        // ---------------- B: forward replay of the buffered tokens (FP64, rescaled)
        const float* bk = a.blob.buf_k + kvec * (size_t)W * D;
        const float* bv = a.blob.buf_v + (size_t)u * W * D;
        const float* bb = a.blob.buf_beta + (size_t)u * W;
        const float* bg = a.blob.buf_gate + (size_t)u * W * (KDA ? D : 1);
        double gam = 1.0;  // scalar gate: running product g (uniform)
        if constexpr (KDA) {
            if (tid < D) lds_G[tid] = 1.0;
        }
        // A batch's keys, values (and channel gates) are fetched into registers
        // one batch ahead, F4 float4 per thread, every load independent of the
        // others; tokens past the end of the window repeat the last one and are
        // never used.
        Stage<F4, KDA> pf{};
        if (n_replay > 0) pf = fetch_stage<D, EB, NT, F4, KDA>(bk, bv, bb, bg, 0, n_replay, tid);
        for (int i0 = 0; i0 < n_replay; i0 += EB) {
            const int ne = (n_replay - i0) < EB ? (n_replay - i0) : EB;
            __syncthreads();  // the previous batch is done with LDS
#pragma unroll
            for (int f = 0; f < F4; ++f) {
                const int x = 4 * (tid + f * NT);
                const int e = x / D, c = x % D;
                *reinterpret_cast<float4*>(&lds_v[e][c]) = pf.v[f];
                if constexpr (KDA) {
                    *reinterpret_cast<float4*>(&lds_kraw[e][c]) = pf.k[f];
                    *reinterpret_cast<float4*>(&lds_graw[e][c]) = pf.g[f];
                } else {
                    double* dk = &lds_k[e][(c / 16) * 18 + (c % 16)];
                    dk[0] = pf.k[f].x;
                    dk[1] = pf.k[f].y;
                    dk[2] = pf.k[f].z;
                    dk[3] = pf.k[f].w;
                }
            }
            if (tid < EB) {
                lds_b[tid] = pf.b;
                if constexpr (!KDA) lds_al[tid] = pf.al;
            }
            __syncthreads();
            if (i0 + EB < n_replay)  // in flight during this batch
                pf = fetch_stage<D, EB, NT, F4, KDA>(bk, bv, bb, bg, i0 + EB, n_replay, tid);
            if constexpr (KDA) {
                // one thread per column walks the batch: fold G into T if it got
                // small, then G' = G a and the key scaled both ways
                if (tid < D) {
                    const int c = tid;
                    double G = lds_G[c];
                    lds_fold[c] = (G < kRescaleBelow) ? G : 1.0;
                    if (G < kRescaleBelow) G = 1.0;
                    const int slot = (c / 16) * 18 + (c % 16);
                    for (int e = 0; e < ne; ++e) {
                        const double ag = fmax((double)lds_graw[e][c], kMinChannelGate);
                        G *= ag;
                        const double kc = (double)lds_kraw[e][c];
                        lds_k[e][slot] = G * kc;
                        lds_kd[e][slot] = kc / G;
                    }
                    lds_G[c] = G;
                }
            } else {
                // the running gate product, token by token (thread 0), then its
                // reciprocals in parallel (wavefront 0)
                if (tid == 0) {
                    double g = gam;
                    for (int e = 0; e < ne; ++e) {
                        const double al = (double)lds_al[e];
                        const bool fold = g * al < kRescaleBelow;
                        lds_resc[e] = fold ? 1 : 0;
                        if (fold) g = 1.0;  // T takes the old product first
                        g *= al;
                        lds_coef[e][0] = g;
                    }
                }
                if (wave == 0) {
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    if (lane < ne) lds_coef[lane][1] = 1.0 / lds_coef[lane][0];
                }
            }
            __syncthreads();
            if constexpr (KDA) {
                // fold this batch's per-column factors into T (rare)
                bool any = false;
#pragma unroll
                for (int c = 0; c < 16; ++c) any = any || (lds_fold[c0 + c] != 1.0);
                if (any) {
#pragma unroll
                    for (int c = 0; c < 16; ++c) {
                        const double f = lds_fold[c0 + c];
                        T[0][c] *= f;
                        T[1][c] *= f;
                    }
                }
            }
            for (int e = 0; e < ne; ++e) {
                double kk[16];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const double2 k2 = *reinterpret_cast<const double2*>(&lds_k[e][ch * 18 + 2 * t]);
                    kk[2 * t] = k2.x;
                    kk[2 * t + 1] = k2.y;
                }
                if constexpr (!KDA) {
                    if (lds_resc[e]) {  // uniform: fold the gate product into T
#pragma unroll
                        for (int c = 0; c < 16; ++c) {
                            T[0][c] *= gam;
                            T[1][c] *= gam;
                        }
                    }
                }
                double d0a = 0.0, d0b = 0.0, d1a = 0.0, d1b = 0.0;
#pragma unroll
                for (int c = 0; c < 16; c += 2) {
                    d0a = __builtin_fma(T[0][c], kk[c], d0a);
                    d0b = __builtin_fma(T[0][c + 1], kk[c + 1], d0b);
                    d1a = __builtin_fma(T[1][c], kk[c], d1a);
                    d1b = __builtin_fma(T[1][c + 1], kk[c + 1], d1b);
                }
                const double d0 = group_sum<CPR>(d0a + d0b);
                const double d1 = group_sum<CPR>(d1a + d1b);
                const double be = (double)lds_b[e];
                double k0, k1;
                if constexpr (KDA) {
                    k0 = be * ((double)lds_v[e][r0] - d0);
                    k1 = be * ((double)lds_v[e][r0 + 1] - d1);
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const double2 k2 = *reinterpret_cast<const double2*>(&lds_kd[e][ch * 18 + 2 * t]);
                        kk[2 * t] = k2.x;
                        kk[2 * t + 1] = k2.y;
                    }
                } else {
                    const double g = lds_coef[e][0], ig = lds_coef[e][1];
                    gam = g;
                    k0 = be * ((double)lds_v[e][r0] - g * d0) * ig;
                    k1 = be * ((double)lds_v[e][r0 + 1] - g * d1) * ig;
                }
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    T[0][c] = __builtin_fma(k0, kk[c], T[0][c]);
                    T[1][c] = __builtin_fma(k1, kk[c], T[1][c]);
                }
            }
        }
        // back to S
        if constexpr (KDA) {
            __syncthreads();
            if (n_replay > 0) {
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const double G = lds_G[c0 + c];
                    T[0][c] *= G;
                    T[1][c] *= G;
                }
            }
        } else {
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                T[0][c] *= gam;
                T[1][c] *= gam;
            }
        }

        if constexpr (MODE == kModeDequant) {
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                float4* dst = reinterpret_cast<float4*>(a.S_out + ((size_t)u * D + r0 + rr) * D + c0);
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    dst[t] = make_float4((float)T[rr][4 * t], (float)T[rr][4 * t + 1], (float)T[rr][4 * t + 2],
                                         (float)T[rr][4 * t + 3]);
            }
            __syncthreads();  // LDS is reused by the next unit
            continue;
        }

        // ---------------- C1: line scores
        {
            double rs0 = 0.0, rs1 = 0.0;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                rs0 = __builtin_fma(T[0][c], T[0][c], rs0);
                rs1 = __builtin_fma(T[1][c], T[1][c], rs1);
            }
            rs0 = group_sum<CPR>(rs0);
            rs1 = group_sum<CPR>(rs1);
            if (ch == 0) {
                lds_score[r0] = rs0;
                lds_score[r0 + 1] = rs1;
            }
            double sq[16];
#pragma unroll
            for (int c = 0; c < 16; ++c) sq[c] = T[0][c] * T[0][c] + T[1][c] * T[1][c];
            const int cb = reduce_rows_in_wave<CPR, false>(sq);
#pragma unroll
            for (int i = 0; i < NVAL; ++i) lds_part[wave][c0 + cb + i] = sq[i];
            __syncthreads();
            if (tid < D) {
                double t = 0.0;
                for (int w = 0; w < NW; ++w) t += lds_part[w][tid];
                lds_score[D + tid] = t;
            }
            __syncthreads();
        }

        // ---------------- C2: top-n_comp selection (wavefront 0)
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
            float* cvb = a.blob.comp_vec + (size_t)u * nc * D;
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int rslot = lds_slot[r0 + rr];
                if (rslot) {
                    float4* dst = reinterpret_cast<float4*>(cvb + (size_t)(rslot - 1) * D + c0);
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        dst[t] = make_float4((float)T[rr][4 * t], (float)T[rr][4 * t + 1], (float)T[rr][4 * t + 2],
                                             (float)T[rr][4 * t + 3]);
                }
            }
            const int rs0 = lds_slot[r0], rs1 = lds_slot[r0 + 1];
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const int cs = lds_slot[D + c0 + c];
                if (cs) {
                    cvb[(size_t)(cs - 1) * D + r0] = rs0 ? 0.0f : (float)T[0][c];
                    cvb[(size_t)(cs - 1) * D + r0 + 1] = rs1 ? 0.0f : (float)T[1][c];
                    T[0][c] = 0.0;
                    T[1][c] = 0.0;
                }
                if (rs0) T[0][c] = 0.0;
                if (rs1) T[1][c] = 0.0;
            }
        }

        // ---------------- C4: smoothing per key channel
        {
            double am[16];
#pragma unroll
            for (int c = 0; c < 16; ++c) am[c] = fmax(fabs(T[0][c]), fabs(T[1][c]));
            const int cb = reduce_rows_in_wave<CPR, true>(am);
#pragma unroll
            for (int i = 0; i < NVAL; ++i) lds_part[wave][c0 + cb + i] = am[i];
            __syncthreads();
            if (tid < D) {
                double m = 0.0;
                for (int w = 0; w < NW; ++w) m = fmax(m, lds_part[w][tid]);
                const float sj = m > 0.0 ? (float)sqrt(m) : 1.0f;
                lds_smooth[tid] = sj;
                lds_ismooth[tid] = 1.0 / (double)sj;
                a.blob.smooth[(size_t)u * D + tid] = sj;
            }
            __syncthreads();
        }

        // ---------------- C5: per-row scale and codes
        {
            // divisions by s_j and sigma_i s_j as products with FP64 reciprocals
            // (a few ulps of FP64 off the quotient; the codes round at 2^-10 of
            // a tie or closer only by chance either way)
            double isj[16];
#pragma unroll
            for (int c = 0; c < 16; ++c) isj[c] = lds_ismooth[c0 + c];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                double m = 0.0;
#pragma unroll
                for (int c = 0; c < 16; ++c) m = fmax(m, fabs(T[rr][c] * isj[c]));
                m = group_max<CPR>(m);
                const float sg = (float)(m / 127.0);
                if (ch == 0) a.blob.sigma[(size_t)u * D + r0 + rr] = sg;
                const double isg = sg != 0.0f ? 1.0 / (double)sg : 0.0;
                uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    int code = 0;
                    if (sg != 0.0f) {
                        double x = rint(T[rr][c] * (isg * isj[c]));
                        x = fmin(fmax(x, -127.0), 127.0);
                        code = (int)x;
                    }
                    packed[c / 4] |= ((uint32_t)code & 0xFFu) << (8 * (c % 4));
                }
                *reinterpret_cast<uint4*>(a.blob.codes + ((size_t)u * D + r0 + rr) * D + c0) =
                    make_uint4(packed[0], packed[1], packed[2], packed[3]);
            }
        }
        if (tid == 0) {
            a.blob.fill[u] = 0;
            if (MODE == kModeInit && u == 0) *a.blob.status = 0u;
        }
        __syncthreads();  // LDS is reused by the next unit
    }
}

__global__ void clear_status_kernel(uint32_t* status) { *status = 0u; }

hipError_t launch_materialize(const MatArgs& a, int mode, int d, int gate_kind, hipStream_t st) {
    // a fixed grid walks the units (init, dequant) or the work list (flush)
    const int grid_cap = 2048;
    const dim3 grid(a.dm.n_units < grid_cap ? a.dm.n_units : grid_cap), block(d * d / 32);
    const bool kda = gate_kind == LQ_GATE_CHANNEL;
    if (mode == kModeFlush) {
        hipLaunchKernelGGL(due_scan_kernel, dim3(1), dim3(1024), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
#define LQ_MAT(D_, K_, M_) hipLaunchKernelGGL((materialize_kernel<D_, K_, M_>), grid, block, 0, st, a)
#define LQ_MAT_MODE(D_, K_)                                      \
    do {                                                         \
        if (mode == kModeInit) LQ_MAT(D_, K_, kModeInit);        \
        else if (mode == kModeFlush) LQ_MAT(D_, K_, kModeFlush); \
        else LQ_MAT(D_, K_, kModeDequant);                       \
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
