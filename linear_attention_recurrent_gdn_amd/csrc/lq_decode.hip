// lq_decode.hip -- per-token decode kernels for gfx950.
//
// decode_q8_kernel: one token of the windowed 8-bit scheme (INT8 codes, or
// E4M3 8-bit floats: the review says INT8, the abstract only "8-bit").  The arXiv
// 2609.38166 abstract ("Abstract (arXiv)" section, mlsanity.com paper page):
// a token inside a window takes its output from the 8-bit state, unchanged
// since the window began, and the window's full-precision tokens.  The bedrocknews.com review: the cost
// is recomputing the buffered tokens' contributions, traded for far less
// state traffic.  Per unit (sequence x value head), with the window-start
// state S_hat = Diag(sigma) Q Diag(s) + sum_c v_c k_c^T and buffered tokens
// 1..n (the current token is n):
//     r = q;  acc = 0
//     for i = n..1:  c = k_i . r;  acc += beta_i c v_i;  r = g_i * (r - beta_i c k_i)
//     o = sigma * (Q (s * r)) + sum_c v_c (k_c . r) + acc
// so r = A_1..A_n q and acc = sum_i beta_i v_i k_i^T A_{i+1}..A_n q, and o is
// S_n q.  The 8-bit tile, sigma, s and compensators are only read.  Q holds
// the code values: the integers themselves, or the E4M3 values, which the
// gfx950 conversion v_cvt_pk_f32_fp8 produces exactly (two per instruction).
// The buffer keeps each token's k and v in fp32 or in binary16 (rounded as the
// token enters the window, then used in that rounded form everywhere), which
// halves the replay's bytes.
//
// Mapping: one workgroup of four wavefronts per unit.  Each wavefront
// requests its quarter of the 8-bit tile (4 KiB at d = 128) with 16-byte
// coalesced loads at kernel start.  Wavefront 0 runs the reverse pass: the
// buffered tokens stream through a register ring refilled a fixed number of
// tokens ahead (so the wait counts are exact and memory latency is paid once
// per ring, not per token), the d-length dot products reduce with DPP, and
// with a scalar gate the running gate product stays off the dependent chain.
// Wavefronts 1-3 convert their codes to floats while the reverse pass runs
// (wavefront 0 converts its own after it).  After one barrier every
// wavefront multiplies its tile rows by s*r (read from LDS, each lane covering
// 16 columns, rows reduced over 8 lanes with DPP) and writes its rows of o:
// only the products are left there, where the four units that share a CU
// reach it together.  The kernel is HBM-bound (about one flop per byte):
// no MFMA.
//
// decode_fp32_kernel: the FP32-state step the pages compare against (the
// bedrocknews.com review: the comparison keeps a 32-bit float state).  The row form
// x = g * S[i,:];  S[i,:] = x + beta (v_i - x.k) k;  o_i = x.q + beta (v_i - x.k)(k.q)
// reads and writes each 512-byte row once.

#include "lq_internal.h"


namespace lq {

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int EPL>
struct Vec {
    float e[EPL];
};

template <int EPL>
__device__ __forceinline__ Vec<EPL> load_vec(const float* p) {
    Vec<EPL> r;
    if constexpr (EPL == 2) {
        float2 t = *reinterpret_cast<const float2*>(p);
        r.e[0] = t.x;
        r.e[1] = t.y;
    } else {
        r.e[0] = p[0];
    }
    return r;
}

// The same, as streaming (non-temporal) loads where STREAM: for data that a
// launch reads exactly once (a unit's 8-bit tile, scales, compensator lines,
// buffered values), so that it does not displace in the caches what is read
// again (the keys that the value heads of one key head share, the lines that
// the stores write).  A state small enough to stay in the last-level cache
// from one token to the next (1,024 units of d = 128 on their own) is read
// faster with ordinary loads: lq_config.load_policy chooses.
template <int EPL, bool STREAM>
__device__ __forceinline__ Vec<EPL> load_vec_as(const float* p) {
    if constexpr (!STREAM) return load_vec<EPL>(p);
    Vec<EPL> r;
    if constexpr (EPL == 2) {
        const f32x2 t = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
        r.e[0] = t[0];
        r.e[1] = t[1];
    } else {
        r.e[0] = __builtin_nontemporal_load(p);
    }
    return r;
}

template <bool STREAM>
__device__ __forceinline__ uint4 load_tile_as(const uint4* p) {
    if constexpr (!STREAM) return *p;
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
}

template <int EPL>
__device__ __forceinline__ void store_vec(float* p, const Vec<EPL>& v) {
    if constexpr (EPL == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(v.e[0], v.e[1]);
    } else {
        p[0] = v.e[0];
    }
}

__device__ __forceinline__ bool finite(float x) { return __builtin_isfinite(x); }

// A zero the compiler cannot see through: an index built from it is taken as
// varying across lanes, so the load is a vector load.
__device__ __forceinline__ int vgpr_zero() {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

// Unit of a workgroup.  The dispatcher hands workgroup b to XCD b % 8, and
// each XCD has its own L2.  With grouped heads (G value heads per key head)
// the G units that read the same key vectors (the buffered k and the token's
// q, k) are given workgroups b, b + 8, ..., on one XCD and next to each other
// in dispatch order, so the shared keys come from that XCD's L2 after the
// first read.  Needs the unit count to be a multiple of 8 G; otherwise
// workgroup b runs unit b.
__device__ __forceinline__ int unit_of_block(int b, const Dims& dm) {
    constexpr int kXcds = 8;
    const int G = dm.group;
    if (G <= 1 || dm.n_units % (kXcds * G) != 0) return b;
    const int slot = b / kXcds;
    const int kvec = (slot / G) * kXcds + b % kXcds;
    return kvec * G + slot % G;
}

// A wavefront-uniform pair held in scalar registers (frees two vector
// registers per ring slot).
__device__ __forceinline__ float2 uniform2(float2 x) {
    return make_float2(__builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x.x))),
                       __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x.y))));
}

__device__ __forceinline__ float lane_value(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Stores values that are already binary16-representable when H16; NT: as
// non-temporal stores.
template <int EPL, bool H16, bool NT = false>
__device__ __forceinline__ void store_buf(void* base, size_t off, const Vec<EPL>& v) {
    if constexpr (H16) {
        _Float16* p = reinterpret_cast<_Float16*>(base) + off;
        if constexpr (EPL == 2) {
            const f16x2 h = f16x2{(_Float16)v.e[0], (_Float16)v.e[1]};
            if constexpr (NT) __builtin_nontemporal_store(h, reinterpret_cast<f16x2*>(p));
            else *reinterpret_cast<f16x2*>(p) = h;
        } else {
            if constexpr (NT) __builtin_nontemporal_store((_Float16)v.e[0], p);
            else p[0] = (_Float16)v.e[0];
        }
    } else {
        float* p = reinterpret_cast<float*>(base) + off;
        if constexpr (EPL == 2) {
            const f32x2 f = f32x2{v.e[0], v.e[1]};
            if constexpr (NT) __builtin_nontemporal_store(f, reinterpret_cast<f32x2*>(p));
            else *reinterpret_cast<f32x2*>(p) = f;
        } else {
            if constexpr (NT) __builtin_nontemporal_store(v.e[0], p);
            else p[0] = v.e[0];
        }
    }
}

// A value as the binary16 buffer holds it: nearest-even (the default rounding
// mode of v_cvt_f16_f32), magnitudes above 65504 stored as 65504 (sat set),
// NaN kept.
__device__ __forceinline__ float to_f16_buffer(float x, bool& sat) {
    if (__builtin_fabsf(x) > 65504.f) {
        sat = true;
        x = __builtin_copysignf(65504.f, x);
    }
    return (float)(_Float16)x;
}

// One buffered token as held in registers during the reverse pass.
template <int EPL, int GE>
struct Entry {
    Vec<EPL> k, v;
    Vec<GE> g;
    float beta;
};

// A buffered token in the register ring.  With the binary16 buffer, k and v
// stay packed (one 32-bit word holds this lane's EPL <= 2 halves) until the
// token is used, so a ring entry costs half the registers.
template <int EPL, int GE, bool H16>
struct RingEntry {
    Vec<EPL> k, v;
    Vec<GE> g;
    float2 ba;  // beta, scalar gate (uniform)
};

template <int EPL, int GE>
struct RingEntry<EPL, GE, true> {
    uint32_t k, v;
    Vec<GE> g;
    float2 ba;
};

constexpr int kBufferFlags = 0x00020000;  // raw 32-bit buffer resource word 3 (gfx9 family)
// cache-policy operand of a buffer load: 0 ordinary, kStream the non-temporal
// (streaming) bit of gfx950's buffer instructions
constexpr int kStream = 2;

// EPL consecutive fp32 (or packed binary16 when H16) of a buffer resource at
// a per-lane byte offset plus a uniform (scalar) byte offset.
template <int EPL, int POL = 0>
__device__ __forceinline__ Vec<EPL> buf_load_f32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    Vec<EPL> x;
    if constexpr (EPL == 2) {
        // the builtin returns a two-element vector of its own (GCC vector) type
        const auto w = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, POL);
        x.e[0] = __builtin_bit_cast(float, (unsigned int)w[0]);
        x.e[1] = __builtin_bit_cast(float, (unsigned int)w[1]);
    } else {
        x.e[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, POL));
    }
    return x;
}

template <int EPL, int POL = 0>
__device__ __forceinline__ uint32_t buf_load_halves(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    if constexpr (EPL == 2) return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, POL);
    else return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, POL);
}

// beta and scalar gate of the whole window as loaded, NWB per lane (token i
// in lane i % 64 of register i / 64)
template <int NWB>
struct WindowRegs {
    float b[NWB], a[NWB];
};

template <int EPL>
__device__ __forceinline__ Vec<EPL> unpack_halves(uint32_t w) {
    Vec<EPL> r;
    const f16x2 h = __builtin_bit_cast(f16x2, w);
    r.e[0] = (float)h.x;
    if constexpr (EPL == 2) r.e[1] = (float)h.y;
    return r;
}

// The 16 codes of one 16-byte tile load as floats, in column order (exact:
// an INT8 code or an E4M3 value is an fp32 value).
template <int FMT>
__device__ __forceinline__ void codes_to_float(const uint4& w4, float (&cf)[16]) {
    const uint32_t wd[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
        if constexpr (FMT == LQ_CODE_E4M3) {
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(wd[wi], false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(wd[wi], true);
            cf[4 * wi + 0] = lo.x;
            cf[4 * wi + 1] = lo.y;
            cf[4 * wi + 2] = hi.x;
            cf[4 * wi + 3] = hi.y;
        } else {
#pragma unroll
            for (int by = 0; by < 4; ++by) cf[4 * wi + by] = (float)((int)(wd[wi] << (24 - 8 * by)) >> 24);
        }
    }
}

}  // namespace

// LARGE selects the form for launches of many units per CU: no early code
// conversion, four compensator slots in registers for the scalar gate and
// the ring's beta and gate in scalar registers (72 registers, seven
// wavefronts per SIMD: with many units per CU occupancy is worth more than
// the conversion saved at the barrier), and the 512-byte writes (the
// appended entry, the outputs) as non-temporal stores (about 1 us less per
// launch on the hybrid stack; the 4-byte writes stay ordinary stores, as
// non-temporal they cost more).  The other form (one round of workgroups)
// keeps the codes converted early and eight slots in registers.  STREAM
// (lq_config.load_policy) reads the unit's once-read bytes with streaming
// loads, and makes the 512-byte writes non-temporal in either form.
template <int D, bool KDA, int P, int NWB, int FMT, bool H16, bool LARGE, bool STREAM>
__global__ __launch_bounds__(256) void decode_q8_kernel(DecodeArgs a) {
    constexpr int EPL = D / kWave;   // state elements per lane in the chain wave
    constexpr int GE = KDA ? EPL : 1;
    constexpr int RW = D / 4;        // tile rows per wave
    constexpr int LPR = D / 16;      // lanes per code row (16 codes per 16-byte load)
    constexpr int RPL = kWave / LPR; // code rows per wave-wide 16-byte load
    constexpr int NLW = RW / RPL;    // 16-byte tile loads per lane
    // compensator slots held in registers through the reverse pass (the rest
    // are loaded after it)
    constexpr int NCP = (KDA || !LARGE) ? 8 : 4;

    __shared__ float lds_x[D];       // s * r, r = A_1..A_n q (all waves read it)
    __shared__ float lds_add[D];     // buffered-token and compensator terms of o
    __shared__ float2 lds_ba[256];   // wavefront 0: beta and scalar gate of each window slot

    if ((int)blockIdx.x >= a.dm.n_units) return;
    const int u = unit_of_block(blockIdx.x, a.dm);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = lane_id();
    const int W = a.dm.window;
    const int nc = a.dm.n_comp;
    const int s = u / a.dm.n_v_heads;
    const int h = u - s * a.dm.n_v_heads;
    const int kh = h / a.dm.group;
    const size_t kvec = ((size_t)s * a.dm.n_k_heads + kh);  // key-head row of q, k

    // ---- every wave owns a quarter of the 8-bit tile (RW rows) and writes those rows of o
    const int cg = lane % LPR;  // this lane's 16-column group
    const int row0 = wave * RW;
    const uint4* tile = reinterpret_cast<const uint4*>(a.blob.codes + ((size_t)u * D + row0) * D);
    const int my_row = row0 + min(cg, NLW - 1) * RPL + lane / LPR;  // row this lane writes (cg < NLW)
    uint4 tw[NLW];
    // The tile quarter as floats, converted before the barrier.  Not with the
    // binary16 buffer: there the extra registers cost a wavefront per SIMD of
    // occupancy, more than the conversion saves.
    constexpr bool kEarlyCodes = !H16 && !LARGE;
    // the 512-byte writes (the appended entry, the outputs) as non-temporal
    // stores: in the large form, and wherever the loads stream
    constexpr bool NTST = LARGE || STREAM;
    float cf[NLW][16];
    float sg_row;

    // tokens already in the window (uniform: every branch below is scalar).
    // Only the window's own entries need it: every other load is requested
    // before the wait for it, so the count and those loads share one trip.  A
    // full window (no flush since W tokens) runs as an empty one with no
    // stores to the window and NaN outputs; there is no early return, which
    // would let the compiler move the loads below the wait.
    const int j_ld = a.blob.fill[u];
    int j;

    if (wave != 0) {
#pragma unroll
        for (int t = 0; t < NLW; ++t) tw[t] = load_tile_as<STREAM>(&tile[t * kWave + lane]);
        sg_row = a.blob.sigma[(size_t)u * D + my_row];
        j = __builtin_amdgcn_readfirstlane(j_ld);
        // the codes to floats while wavefront 0 runs the reverse pass, so
        // that only the products remain after the barrier
        if constexpr (kEarlyCodes) {
#pragma unroll
            for (int t = 0; t < NLW; ++t) codes_to_float<FMT>(tw[t], cf[t]);
        }
    } else {
        const size_t kb0 = kvec * (size_t)W * D;  // element offsets of this unit's k and v entries
        const size_t vb0 = (size_t)u * W * D;
        float* bb = a.blob.buf_beta + (size_t)u * W;
        float* bg = a.blob.buf_gate + (size_t)u * W * (KDA ? D : 1);

        // loads in the order they are consumed (vector loads return in order):
        // the current token, beta and the scalar gate of the whole window (NWB
        // per lane, window <= 64 NWB), this wave's tile quarter, smoothing and
        // compensators; then, once the count is in, the newest P buffered
        // tokens (a ring refilled P tokens ahead of use)
        const Vec<EPL> qv = load_vec<EPL>(a.q + kvec * D + lane * EPL);
        Entry<EPL, GE> cur;
        cur.k = load_vec<EPL>(a.k + kvec * D + lane * EPL);
        cur.v = load_vec<EPL>(a.v + (size_t)u * D + lane * EPL);
        // beta and the scalar gate through the vector path, in order with the
        // token's other loads (a scalar load would be issued, and waited for,
        // on its own)
        const float bgv = (KDA || lane == 0 ? a.beta : a.gate)[u + vgpr_zero()];
        cur.beta = lane_value(bgv, 0);
        if constexpr (KDA) {
            cur.g = load_vec<GE>(a.gate + (size_t)u * D + lane * EPL);
        } else {
            cur.g.e[0] = lane_value(bgv, 1);
        }
        WindowRegs<NWB> win;
#pragma unroll
        for (int w = 0; w < NWB; ++w) {
            win.b[w] = bb[min(lane + w * kWave, W - 1)];
            win.a[w] = KDA ? 0.f : bg[min(lane + w * kWave, W - 1)];
        }
#pragma unroll
        for (int t = 0; t < NLW; ++t) tw[t] = load_tile_as<STREAM>(&tile[t * kWave + lane]);
        sg_row = a.blob.sigma[(size_t)u * D + my_row];
        const Vec<EPL> sm = load_vec_as<EPL, STREAM>(a.blob.smooth + (size_t)u * D + lane * EPL);
        const int cidx = a.blob.comp_idx[(size_t)u * nc + min(lane, max(nc - 1, 0))];
        Vec<EPL> cvec[NCP];
#pragma unroll
        for (int c = 0; c < NCP; ++c)
            cvec[c] = load_vec_as<EPL, STREAM>(a.blob.comp_vec + ((size_t)u * nc + min(c, max(nc - 1, 0))) * D + lane * EPL);

        j = __builtin_amdgcn_readfirstlane(j_ld);
        const bool over = j >= W;
        const int jr = over ? 0 : j;  // entries replayed
        // the window's entries through buffer resources: a constant per-lane
        // offset and a scalar per-entry offset, no per-lane address arithmetic.
        // Ring slots with no entry left (index below 0) load through a
        // resource of zero size: out of range, the load returns zeros without
        // a memory access.  So every slot is loaded unconditionally (the
        // compiler's wait counts stay exact) and the unused loads cost no
        // memory trip to wait for.
        constexpr int ESZ = H16 ? 2 : 4;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (char*)a.blob.buf_k + kb0 * ESZ, (short)0, W * D * ESZ, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (char*)a.blob.buf_v + vb0 * ESZ, (short)0, W * D * ESZ, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
            bg, (short)0, KDA ? W * D * 4 : 4, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rnone =
            __builtin_amdgcn_make_buffer_rsrc((char*)a.blob.buf_k, (short)0, 0, kBufferFlags);
        const int voff = lane * EPL * ESZ;
        // values are read once per launch and streamed; so are the keys with
        // the channel gate, whose entries carry a gate vector as well (with a
        // scalar gate, streamed keys and gates were slower: measured)
        constexpr int KPOL = (STREAM && KDA) ? kStream : 0;
        constexpr int VPOL = STREAM ? kStream : 0;
        auto load_entry = [&](int i, RingEntry<EPL, GE, H16>& en) {
            const bool live = i >= 0;  // uniform
            const int ie = live ? i : 0;
            if constexpr (H16) {
                en.k = buf_load_halves<EPL, KPOL>(live ? rk : rnone, voff, ie * D * ESZ);
                en.v = buf_load_halves<EPL, VPOL>(live ? rv : rnone, voff, ie * D * ESZ);
            } else {
                en.k = buf_load_f32<EPL, KPOL>(live ? rk : rnone, voff, ie * D * ESZ);
                en.v = buf_load_f32<EPL, VPOL>(live ? rv : rnone, voff, ie * D * ESZ);
            }
            if constexpr (KDA) en.g = buf_load_f32<GE>(live ? rg : rnone, lane * EPL * 4, ie * D * 4);
        };
        RingEntry<EPL, GE, H16> ring[P];
#pragma unroll
        for (int p = 0; p < P; ++p) load_entry(jr - 1 - p, ring[p]);

        // check the current token and append it to the window buffer
        bool ok = finite(cur.beta);
        for (int e = 0; e < EPL; ++e) ok = ok && finite(qv.e[e]) && finite(cur.k.e[e]) && finite(cur.v.e[e]);
        for (int e = 0; e < GE; ++e) ok = ok && finite(cur.g.e[e]);
        if (__any(!ok) && lane == 0) atomicOr(a.blob.status, (uint32_t)LQ_DEV_NONFINITE_INPUT);
        if constexpr (H16) {
            // the token enters the window as the buffer holds it, and is used so
            bool sat = false;
            for (int e = 0; e < EPL; ++e) {
                cur.k.e[e] = to_f16_buffer(cur.k.e[e], sat);
                cur.v.e[e] = to_f16_buffer(cur.v.e[e], sat);
            }
            if (__any(sat) && lane == 0) atomicOr(a.blob.status, (uint32_t)LQ_DEV_BUFFER_SATURATED);
        }
        if (!over) {
            if (h % a.dm.group == 0) store_buf<EPL, H16, NTST>(a.blob.buf_k, kb0 + (size_t)j * D + lane * EPL, cur.k);
            store_buf<EPL, H16, NTST>(a.blob.buf_v, vb0 + (size_t)j * D + lane * EPL, cur.v);
        }
        // beta and scalar gate of every buffered slot into LDS, then the ring's
        // first entries take theirs (uniform reads; later refills read ahead)
#pragma unroll
        for (int w = 0; w < NWB; ++w)
            if (lane + w * kWave < W) lds_ba[lane + w * kWave] = make_float2(win.b[w], win.a[w]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const float2 ba = lds_ba[max(jr - 1 - p, 0)];
            ring[p].ba = LARGE ? uniform2(ba) : ba;
        }
        if (!over) {
            if constexpr (KDA) {
                store_vec(bg + (size_t)j * D + lane * EPL, cur.g);
            } else {
                if (lane == 0) bg[j] = cur.g.e[0];
            }
            if (lane == 0) bb[j] = cur.beta;
        }

        // reverse pass over the window, newest token first.  With a scalar
        // gate the running gate product sc stays off the dependent chain:
        // r_true = sc * r, so r -= (beta (k.r)) k and acc += beta sc (k.r) v.
        // the reverse pass is the workgroup's dependent chain: it takes issue
        // priority over the other wavefronts on its SIMD (other workgroups'
        // tile products and prologues) until its results are in LDS
        __builtin_amdgcn_s_setprio(3);
        Vec<EPL> r = qv;
        Vec<EPL> acc;
        for (int e = 0; e < EPL; ++e) acc.e[e] = 0.f;
        float sc = 1.0f;
        auto step = [&](const Vec<EPL>& ek, const Vec<EPL>& ev, const Vec<GE>& eg, float beta, float alpha) {
            float p = 0.f;
            for (int e = 0; e < EPL; ++e) p = __builtin_fmaf(ek.e[e], r.e[e], p);
            const float red = wave_sum_all(p);
            const float cr = beta * red;
            if constexpr (KDA) {
                for (int e = 0; e < EPL; ++e) {
                    r.e[e] = eg.e[e] * __builtin_fmaf(-cr, ek.e[e], r.e[e]);
                    acc.e[e] = __builtin_fmaf(cr, ev.e[e], acc.e[e]);
                }
            } else {
                for (int e = 0; e < EPL; ++e) r.e[e] = __builtin_fmaf(-cr, ek.e[e], r.e[e]);
                const float w = cr * sc;
                for (int e = 0; e < EPL; ++e) acc.e[e] = __builtin_fmaf(w, ev.e[e], acc.e[e]);
                sc *= alpha;
            }
        };
        step(cur.k, cur.v, cur.g, cur.beta, cur.g.e[0]);
        // k and v of ring entry p as fp32
        auto ring_k = [&](int p) {
            if constexpr (H16) return unpack_halves<EPL>(ring[p].k);
            else return ring[p].k;
        };
        auto ring_v = [&](int p) {
            if constexpr (H16) return unpack_halves<EPL>(ring[p].v);
            else return ring[p].v;
        };
        // whole ring cycles, then the last partial one (no refills needed
        // there)
        int s0 = 0;
        for (; s0 + P <= jr; s0 += P) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int i = jr - 1 - (s0 + p);
                step(ring_k(p), ring_v(p), ring[p].g, ring[p].ba.x, ring[p].ba.y);
                load_entry(i - P, ring[p]);
                const float2 ba = lds_ba[max(i - P, 0)];
                ring[p].ba = LARGE ? uniform2(ba) : ba;
            }
        }
#pragma unroll
        for (int p = 0; p < P; ++p)
            if (s0 + p < jr) step(ring_k(p), ring_v(p), ring[p].g, ring[p].ba.x, ring[p].ba.y);
        if constexpr (!KDA)
            for (int e = 0; e < EPL; ++e) r.e[e] *= sc;

        // compensator tokens: rows add (k_c . r) at their row, columns add v_c r[col]
        auto comp = [&](int idx, const Vec<EPL>& w) {
            if (idx < D) {
                float p = 0.f;
                for (int e = 0; e < EPL; ++e) p = __builtin_fmaf(w.e[e], r.e[e], p);
                const float dot = wave_sum(p);
                // a select per element: an indexed update here would make the
                // compiler move acc to LDS addressed by the flat thread id, which
                // costs every workgroup a read of the dispatch packet
                for (int e = 0; e < EPL; ++e) acc.e[e] += (lane * EPL + e == idx) ? dot : 0.f;
            } else {
                const int col = idx - D;
                // read each element from the owning lane, then choose: selecting
                // r.e[col % EPL] first would index a private array dynamically
                float rc = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r.e[0]), col / EPL));
                if constexpr (EPL == 2) {
                    const float rc1 = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r.e[1]), col / EPL));
                    rc = (col & 1) ? rc1 : rc;
                }
                for (int e = 0; e < EPL; ++e) acc.e[e] = __builtin_fmaf(w.e[e], rc, acc.e[e]);
            }
        };
#pragma unroll
        for (int c = 0; c < NCP; ++c)
            if (c < nc) comp(__builtin_amdgcn_readlane(cidx, c), cvec[c]);
        for (int c = NCP; c < nc; ++c)
            comp(__builtin_amdgcn_readlane(cidx, c),
                 load_vec_as<EPL, STREAM>(a.blob.comp_vec + ((size_t)u * nc + c) * D + lane * EPL));

        for (int e = 0; e < EPL; ++e) {
            lds_x[lane * EPL + e] = sm.e[e] * r.e[e];
            lds_add[lane * EPL + e] = acc.e[e];
        }
        if constexpr (kEarlyCodes) {
#pragma unroll
            for (int t = 0; t < NLW; ++t) codes_to_float<FMT>(tw[t], cf[t]);
        }
        __builtin_amdgcn_s_setprio(0);
    }
    lds_barrier();

    // ---- every wave: its rows of Q (s * r), then o = sigma * that + the rest
    float xs[16];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float4 x4 = *reinterpret_cast<const float4*>(&lds_x[cg * 16 + 4 * t]);
        xs[4 * t + 0] = x4.x;
        xs[4 * t + 1] = x4.y;
        xs[4 * t + 2] = x4.z;
        xs[4 * t + 3] = x4.w;
    }
    float mine = 0.f;
#pragma unroll
    for (int t = 0; t < NLW; ++t) {
        if constexpr (!kEarlyCodes) codes_to_float<FMT>(tw[t], cf[t]);
        // even columns into p0, odd into p1, each in column order
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int c = 0; c < 16; c += 2) {
            p0 = __builtin_fmaf(cf[t][c], xs[c], p0);
            p1 = __builtin_fmaf(cf[t][c + 1], xs[c + 1], p1);
        }
        float p = p0 + p1;
        if constexpr (LPR == 8) p = sum8(p);
        else p = sum4(p);
        if (t == cg) mine = p;
    }
    const bool over = j >= W;
    if (cg < NLW)
    {
        const float ov = over ? __builtin_nanf("") : __builtin_fmaf(sg_row, mine, lds_add[my_row]);
        if constexpr (NTST) __builtin_nontemporal_store(ov, a.o + (size_t)u * D + my_row);
        else a.o[(size_t)u * D + my_row] = ov;
    }
    if (wave == 0 && lane == 0) {
        if (over) atomicOr(a.blob.status, (uint32_t)LQ_DEV_WINDOW_OVERFLOW);
        else a.blob.fill[u] = j + 1;
    }
}


// The chain-free form of the window buffer (LQ_BUFFER_NFORM, scalar gate).
// Within a window the gated delta rule's state is, by the WY form of a
// product of (I - beta k k^T) factors (the compact-WY representation that
// the works the pages cite use for chunked training),
//     S_t = g_t S_hat + sum_{i <= t} (g_t / g_i) n_i k_i^T,
//     n_t = beta_t (v_t - g_t S_hat k_t - sum_{i < t} (g_t / g_i) n_i (k_i . k_t)),
// with g_t the product of the window's gates up to token t.  A buffer entry
// keeps k_i (per key head, as in the token form), n_i in place of v_i, and
// the token's gate; beta is inside n_i.  The ratios g_t / g_i are 2 to the
// sum of log2 of the gates of the tokens after i, a gate floored at 2^-126
// (a gate of 0 makes the earlier ratios underflow to 0): the sums are taken
// newest entry first, so each one is a short sum of the gates that matter,
// not a difference of two long ones.  The output o_t = S_t q_t needs the dot products of every buffered
// key with k_t and with q_t, which are independent of each other: the four
// wavefronts of the workgroup take every fourth entry, with no dependent
// chain across entries.
template <int D, int FMT, bool STREAM>
__global__ __launch_bounds__(256) void decode_nform_kernel(DecodeArgs a) {
    constexpr int EPL = D / kWave;    // vector elements per lane
    constexpr int RW = D / 4;         // tile rows per wave
    constexpr int LPR = D / 16;       // lanes per code row
    constexpr int RPL = kWave / LPR;  // code rows per wave-wide 16-byte load
    constexpr int NLW = RW / RPL;     // 16-byte tile loads per lane
    constexpr int P = 4;              // entries requested ahead, per wavefront
    constexpr int NCP = 8;            // compensator slots held in registers
    constexpr float kLogFloor = -126.f;

    __shared__ float lds_x[2][D];        // s * k_t, s * q_t
    __shared__ float lds_add[2][D];      // compensator terms of S_hat k_t, S_hat q_t per row
    __shared__ float lds_part[4][2][D];  // per wavefront: sum over its entries of ratio (k_i . x) n_i
    __shared__ float lds_scal[2];        // g_t, k_t . q_t

    if ((int)blockIdx.x >= a.dm.n_units) return;
    const int u = unit_of_block(blockIdx.x, a.dm);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = lane_id();
    const int W = a.dm.window;
    const int nc = a.dm.n_comp;
    const int s = u / a.dm.n_v_heads;
    const int h = u - s * a.dm.n_v_heads;
    const int kh = h / a.dm.group;
    const size_t kvec = ((size_t)s * a.dm.n_k_heads + kh);

    const int cg = lane % LPR;
    const int row0 = wave * RW;
    const uint4* tile = reinterpret_cast<const uint4*>(a.blob.codes + ((size_t)u * D + row0) * D);
    const int my_row = row0 + min(cg, NLW - 1) * RPL + lane / LPR;
    uint4 tw[NLW];
#pragma unroll
    for (int t = 0; t < NLW; ++t) tw[t] = load_tile_as<STREAM>(&tile[t * kWave + lane]);
    const float sg_row = a.blob.sigma[(size_t)u * D + my_row];
    const float v_row = a.v[(size_t)u * D + my_row];

    // every wavefront: the current token's k and q (its dot products need them)
    const Vec<EPL> kt = load_vec<EPL>(a.k + kvec * D + lane * EPL);
    const Vec<EPL> qt = load_vec<EPL>(a.q + kvec * D + lane * EPL);
    const float beta = a.beta[u];
    const float alpha = a.gate[u];
    float* bg = a.blob.buf_gate + (size_t)u * W;  // gates of the window's entries
    const int j_ld = a.blob.fill[u];
    const int j = __builtin_amdgcn_readfirstlane(j_ld);
    const bool over = j >= W;
    const int jr = over ? 0 : j;
    // log2 of the entries' gates, newest first: lane l of register w holds
    // entry jr - 1 - (l + 64 w) (0 past the oldest); its ratio exponent is the
    // sum over the newer entries (an exclusive prefix sum across the lanes,
    // earlier registers carried) plus the current token's
    const float lt = fmaxf(__builtin_log2f(alpha), kLogFloor);
    float rexp[4];
    float carry = lt;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int idx = jr - 1 - (lane + w * kWave);
        const float g = bg[max(idx, 0)];
        const float lg = idx >= 0 ? fmaxf(__builtin_log2f(g), kLogFloor) : 0.f;
        const float ex = wave_prefix_sum_excl(lg);
        rexp[w] = carry + ex;
        carry += lane_value(ex, kWave - 1) + lane_value(lg, kWave - 1);
    }
    const float gt = __builtin_exp2f(carry);  // g_t: every buffered gate and the current one
    auto entry_ratio = [&](int i) {  // g_t / g_i for buffered entry i (uniform)
        const int r = jr - 1 - i;
        const int w = r >> 6;
        const float x = w == 0 ? rexp[0] : w == 1 ? rexp[1] : w == 2 ? rexp[2] : rexp[3];
        return __builtin_exp2f(lane_value(x, r & 63));
    };

    // entries i = wave, wave + 4, ... (< jr), through buffer resources; slots
    // past the end load through a zero-size resource (zeros, no memory access)
    const size_t kb0 = kvec * (size_t)W * D;
    const size_t vb0 = (size_t)u * W * D;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (char*)a.blob.buf_k + kb0 * 4, (short)0, W * D * 4, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rn = __builtin_amdgcn_make_buffer_rsrc(
        (char*)a.blob.buf_v + vb0 * 4, (short)0, W * D * 4, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rnone =
        __builtin_amdgcn_make_buffer_rsrc((char*)a.blob.buf_k, (short)0, 0, kBufferFlags);
    const int voff = lane * EPL * 4;
    Vec<EPL> ek[P], en[P];
    auto load_entry = [&](int i, int p) {
        const bool live = i < jr;  // uniform
        const int ie = live ? i : 0;
        ek[p] = buf_load_f32<EPL>(live ? rk : rnone, voff, ie * D * 4);
        en[p] = buf_load_f32<EPL, STREAM ? kStream : 0>(live ? rn : rnone, voff, ie * D * 4);
    };
#pragma unroll
    for (int p = 0; p < P; ++p) load_entry(wave + 4 * p, p);

    // compensator lines (wavefront 0)
    int cidx = 0;
    Vec<EPL> cvec[NCP];
    Vec<EPL> sm;
    if (wave == 0) {
        sm = load_vec_as<EPL, STREAM>(a.blob.smooth + (size_t)u * D + lane * EPL);
        cidx = a.blob.comp_idx[(size_t)u * nc + min(lane, max(nc - 1, 0))];
#pragma unroll
        for (int c = 0; c < NCP; ++c)
            cvec[c] = load_vec_as<EPL, STREAM>(a.blob.comp_vec + ((size_t)u * nc + min(c, max(nc - 1, 0))) * D + lane * EPL);
    }

    // the entries: A1 = sum ratio_i (k_i . k_t) n_i, A2 = sum ratio_i (k_i . q_t) n_i
    Vec<EPL> A1, A2;
    for (int e = 0; e < EPL; ++e) A1.e[e] = A2.e[e] = 0.f;
    for (int s0 = 0; wave + 4 * s0 < jr; s0 += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int i = wave + 4 * (s0 + p);
            if (i < jr) {  // uniform
                float pr[2] = {0.f, 0.f};
                for (int e = 0; e < EPL; ++e) {
                    pr[0] = __builtin_fmaf(ek[p].e[e], kt.e[e], pr[0]);
                    pr[1] = __builtin_fmaf(ek[p].e[e], qt.e[e], pr[1]);
                }
                wave_sum_all_n<2>(pr);
                const float ratio = entry_ratio(i);
                const float w1 = ratio * pr[0], w2 = ratio * pr[1];
                for (int e = 0; e < EPL; ++e) {
                    A1.e[e] = __builtin_fmaf(w1, en[p].e[e], A1.e[e]);
                    A2.e[e] = __builtin_fmaf(w2, en[p].e[e], A2.e[e]);
                }
            }
            load_entry(i + 4 * P, p);
        }
    }
    for (int e = 0; e < EPL; ++e) {
        lds_part[wave][0][lane * EPL + e] = A1.e[e];
        lds_part[wave][1][lane * EPL + e] = A2.e[e];
    }

    if (wave == 0) {
        // check the token, then S_hat's compensator terms for x = k_t and q_t
        bool ok = finite(beta) && finite(alpha);
        for (int e = 0; e < EPL; ++e) ok = ok && finite(qt.e[e]) && finite(kt.e[e]);
        if (__any(!ok) && lane == 0) atomicOr(a.blob.status, (uint32_t)LQ_DEV_NONFINITE_INPUT);
        Vec<EPL> c1, c2;
        for (int e = 0; e < EPL; ++e) c1.e[e] = c2.e[e] = 0.f;
        auto comp = [&](int idx, const Vec<EPL>& w) {
            if (idx < D) {
                float pr[2] = {0.f, 0.f};
                for (int e = 0; e < EPL; ++e) {
                    pr[0] = __builtin_fmaf(w.e[e], kt.e[e], pr[0]);
                    pr[1] = __builtin_fmaf(w.e[e], qt.e[e], pr[1]);
                }
                wave_sum_all_n<2>(pr);
                for (int e = 0; e < EPL; ++e) {
                    c1.e[e] += (lane * EPL + e == idx) ? pr[0] : 0.f;
                    c2.e[e] += (lane * EPL + e == idx) ? pr[1] : 0.f;
                }
            } else {
                const int col = idx - D;
                float x1 = lane_value(kt.e[0], col / EPL), x2 = lane_value(qt.e[0], col / EPL);
                if constexpr (EPL == 2) {
                    const float y1 = lane_value(kt.e[1], col / EPL), y2 = lane_value(qt.e[1], col / EPL);
                    x1 = (col & 1) ? y1 : x1;
                    x2 = (col & 1) ? y2 : x2;
                }
                for (int e = 0; e < EPL; ++e) {
                    c1.e[e] = __builtin_fmaf(w.e[e], x1, c1.e[e]);
                    c2.e[e] = __builtin_fmaf(w.e[e], x2, c2.e[e]);
                }
            }
        };
#pragma unroll
        for (int c = 0; c < NCP; ++c)
            if (c < nc) comp(__builtin_amdgcn_readlane(cidx, c), cvec[c]);
        for (int c = NCP; c < nc; ++c)
            comp(__builtin_amdgcn_readlane(cidx, c),
                 load_vec_as<EPL, STREAM>(a.blob.comp_vec + ((size_t)u * nc + c) * D + lane * EPL));
        float kq = 0.f;
        for (int e = 0; e < EPL; ++e) {
            lds_x[0][lane * EPL + e] = sm.e[e] * kt.e[e];
            lds_x[1][lane * EPL + e] = sm.e[e] * qt.e[e];
            lds_add[0][lane * EPL + e] = c1.e[e];
            lds_add[1][lane * EPL + e] = c2.e[e];
            kq = __builtin_fmaf(kt.e[e], qt.e[e], kq);
        }
        kq = wave_sum_all(kq);
        if (lane == 0) lds_scal[1] = kq;
        // append k_t and L_t (the n entry is written per row below)
        if (!over) {
            if (h % a.dm.group == 0) store_vec(reinterpret_cast<float*>(a.blob.buf_k) + kb0 + (size_t)j * D + lane * EPL, kt);
            if (lane == 0) bg[j] = alpha;
        }
    }
    lds_barrier();

    // every wave: its rows of Q (s * k_t) and Q (s * q_t)
    float xs1[16], xs2[16];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float4 a1 = *reinterpret_cast<const float4*>(&lds_x[0][cg * 16 + 4 * t]);
        const float4 a2 = *reinterpret_cast<const float4*>(&lds_x[1][cg * 16 + 4 * t]);
        xs1[4 * t + 0] = a1.x; xs1[4 * t + 1] = a1.y; xs1[4 * t + 2] = a1.z; xs1[4 * t + 3] = a1.w;
        xs2[4 * t + 0] = a2.x; xs2[4 * t + 1] = a2.y; xs2[4 * t + 2] = a2.z; xs2[4 * t + 3] = a2.w;
    }
    float mine1 = 0.f, mine2 = 0.f;
#pragma unroll
    for (int t = 0; t < NLW; ++t) {
        float cf[16];
        codes_to_float<FMT>(tw[t], cf);
        float p1 = 0.f, p2 = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            p1 = __builtin_fmaf(cf[c], xs1[c], p1);
            p2 = __builtin_fmaf(cf[c], xs2[c], p2);
        }
        if constexpr (LPR == 8) {
            p1 = sum8(p1);
            p2 = sum8(p2);
        } else {
            p1 = sum4(p1);
            p2 = sum4(p2);
        }
        if (t == cg) {
            mine1 = p1;
            mine2 = p2;
        }
    }
    if (cg < NLW) {
        const float kq = lds_scal[1];
        const float y1 = __builtin_fmaf(sg_row, mine1, lds_add[0][my_row]);
        const float y2 = __builtin_fmaf(sg_row, mine2, lds_add[1][my_row]);
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            s1 += lds_part[w][0][my_row];
            s2 += lds_part[w][1][my_row];
        }
        // n_t = beta (v - g_t S_hat k_t - sum ratio n_i (k_i . k_t));
        // o = g_t S_hat q_t + sum_{i < t} ratio n_i (k_i . q_t) + n_t (k_t . q_t)
        const float nt = beta * (v_row - __builtin_fmaf(gt, y1, s1));
        const float ov = over ? __builtin_nanf("") : __builtin_fmaf(nt, kq, __builtin_fmaf(gt, y2, s2));
        a.o[(size_t)u * D + my_row] = ov;
        if (!over) reinterpret_cast<float*>(a.blob.buf_v)[vb0 + (size_t)j * D + my_row] = nt;
    }
    if (wave == 0 && lane == 0) {
        if (over) atomicOr(a.blob.status, (uint32_t)LQ_DEV_WINDOW_OVERFLOW);
        else a.blob.fill[u] = j + 1;
    }
}

template <int D, bool KDA>
__global__ __launch_bounds__(256) void decode_fp32_kernel(Fp32DecodeArgs a) {
    constexpr int LPR = D / 8;        // lanes per state row, 8 floats per lane
    constexpr int RPP = kWave / LPR;  // rows per wave pass
    constexpr int ROWS = D / 4;       // rows per wave (four waves per unit)
    constexpr int NP = ROWS / RPP;    // passes

    if ((int)blockIdx.x >= a.dm.n_units) return;
    const int u = unit_of_block(blockIdx.x, a.dm);
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int cg = lane % LPR;
    const int rsub = lane / LPR;
    const int s = u / a.dm.n_v_heads;
    const int h = u - s * a.dm.n_v_heads;
    const int kh = h / a.dm.group;
    const size_t kvec = ((size_t)s * a.dm.n_k_heads + kh);

    float* S = a.S + (size_t)u * D * D;
    float4 sv[NP][2];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int row = wave * ROWS + p * RPP + rsub;
        const float4* src = reinterpret_cast<const float4*>(S + (size_t)row * D + cg * 8);
        sv[p][0] = src[0];
        sv[p][1] = src[1];
    }
    auto ld8 = [&](const float* p, float (&x)[8]) {
        float4 a0 = reinterpret_cast<const float4*>(p)[0];
        float4 a1 = reinterpret_cast<const float4*>(p)[1];
        x[0] = a0.x; x[1] = a0.y; x[2] = a0.z; x[3] = a0.w;
        x[4] = a1.x; x[5] = a1.y; x[6] = a1.z; x[7] = a1.w;
    };
    float kk[8], qq[8], gg[8];
    ld8(a.k + kvec * D + cg * 8, kk);
    ld8(a.q + kvec * D + cg * 8, qq);
    if constexpr (KDA) {
        ld8(a.gate + (size_t)u * D + cg * 8, gg);
    } else {
        const float al = a.gate[u];
        for (int e = 0; e < 8; ++e) gg[e] = al;
    }
    const float beta = a.beta[u];
    float vrow[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) vrow[p] = a.v[(size_t)u * D + wave * ROWS + p * RPP + rsub];

    float kq = 0.f;
    for (int e = 0; e < 8; ++e) kq = __builtin_fmaf(kk[e], qq[e], kq);
    kq = (LPR == 16) ? sum16(kq) : sum8(kq);

#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int row = wave * ROWS + p * RPP + rsub;
        float x[8] = {sv[p][0].x, sv[p][0].y, sv[p][0].z, sv[p][0].w,
                      sv[p][1].x, sv[p][1].y, sv[p][1].z, sv[p][1].w};
        float dk = 0.f, dq = 0.f;
        for (int e = 0; e < 8; ++e) {
            x[e] *= gg[e];
            dk = __builtin_fmaf(x[e], kk[e], dk);
            dq = __builtin_fmaf(x[e], qq[e], dq);
        }
        if constexpr (LPR == 16) {
            dk = sum16(dk);
            dq = sum16(dq);
        } else {
            dk = sum8(dk);
            dq = sum8(dq);
        }
        const float c = beta * (vrow[p] - dk);
        for (int e = 0; e < 8; ++e) x[e] = __builtin_fmaf(c, kk[e], x[e]);
        float4* dst = reinterpret_cast<float4*>(S + (size_t)row * D + cg * 8);
        dst[0] = make_float4(x[0], x[1], x[2], x[3]);
        dst[1] = make_float4(x[4], x[5], x[6], x[7]);
        if (cg == 0) a.o[(size_t)u * D + row] = __builtin_fmaf(c, kq, dq);
    }
}

// register-ring depths (buffered tokens in flight per unit), from sweeps on
// the decode workloads
#ifndef LQ_RING_GDN
#define LQ_RING_GDN 6
#endif
// the small form with streaming loads (states read from HBM at 1,024 units:
// 12.1 -> 11.9 us per launch against 6 entries, 12.8 with 4)
// the large form with the binary16 buffer and streaming loads (hybrid stack:
// 2.59 -> 2.52 ms per step with the boundary beside the decode)
#ifndef LQ_RING_GDN_H16_LARGE
#define LQ_RING_GDN_H16_LARGE 8
#endif
#ifndef LQ_RING_GDN_SMALL_STREAM
#define LQ_RING_GDN_SMALL_STREAM 8
#endif
#ifndef LQ_RING_KDA
#define LQ_RING_KDA 8
#endif
#ifndef LQ_RING_GDN_H16
#define LQ_RING_GDN_H16 6
#endif
#ifndef LQ_RING_KDA_H16
#define LQ_RING_KDA_H16 4
#endif

// Launches of more units than this take the LARGE form (many workgroups per
// CU); the smaller ones (the GDN decode workload's 1,024 units: four
// workgroups per CU, one round) keep the early code conversion.
#ifndef LQ_LARGE_UNITS_MIN
#define LQ_LARGE_UNITS_MIN 2048
#endif

// streaming loads for this launch (lq_config.load_policy; automatic: the
// large form)
static bool stream_loads(const Dims& dm) {
    if (dm.load_policy == LQ_LOADS_STREAM) return true;
    if (dm.load_policy == LQ_LOADS_CACHED) return false;
    return dm.n_units > LQ_LARGE_UNITS_MIN;
}

template <int NWB, int FMT, bool H16, bool LARGE, bool STREAM>
void launch_decode_q8_w(const DecodeArgs& a, int d, int gate_kind, hipStream_t st) {
    const dim3 grid(a.dm.n_units), block(256);
    if (d == 128) {
        constexpr int PK = H16 ? LQ_RING_KDA_H16 : LQ_RING_KDA;
        constexpr int PG = H16 ? (LARGE ? LQ_RING_GDN_H16_LARGE : LQ_RING_GDN_H16)
                               : (!LARGE && STREAM) ? LQ_RING_GDN_SMALL_STREAM : LQ_RING_GDN;
        if (gate_kind == LQ_GATE_CHANNEL)
            hipLaunchKernelGGL((decode_q8_kernel<128, true, PK, NWB, FMT, H16, LARGE, STREAM>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((decode_q8_kernel<128, false, PG, NWB, FMT, H16, LARGE, STREAM>), grid, block, 0, st, a);
    } else {
        if (gate_kind == LQ_GATE_CHANNEL)
            hipLaunchKernelGGL((decode_q8_kernel<64, true, 16, NWB, FMT, H16, LARGE, STREAM>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((decode_q8_kernel<64, false, 16, NWB, FMT, H16, LARGE, STREAM>), grid, block, 0, st, a);
    }
}

template <int NWB, int FMT, bool H16>
void launch_decode_q8_s(const DecodeArgs& a, int d, int gate_kind, hipStream_t st) {
    const bool large = a.dm.n_units > LQ_LARGE_UNITS_MIN;
    const bool stream = stream_loads(a.dm);
    if (large) {
        if (stream) launch_decode_q8_w<NWB, FMT, H16, true, true>(a, d, gate_kind, st);
        else launch_decode_q8_w<NWB, FMT, H16, true, false>(a, d, gate_kind, st);
    } else {
        if (stream) launch_decode_q8_w<NWB, FMT, H16, false, true>(a, d, gate_kind, st);
        else launch_decode_q8_w<NWB, FMT, H16, false, false>(a, d, gate_kind, st);
    }
}

template <int FMT, bool H16>
void launch_decode_q8_f(const DecodeArgs& a, int d, int gate_kind, hipStream_t st) {
    if (a.dm.window <= 2 * kWave) launch_decode_q8_s<2, FMT, H16>(a, d, gate_kind, st);
    else launch_decode_q8_s<4, FMT, H16>(a, d, gate_kind, st);
}

template <bool H16>
void launch_decode_q8_b(const DecodeArgs& a, int d, int gate_kind, hipStream_t st) {
    if (a.dm.code_format == LQ_CODE_E4M3) launch_decode_q8_f<LQ_CODE_E4M3, H16>(a, d, gate_kind, st);
    else launch_decode_q8_f<LQ_CODE_INT8, H16>(a, d, gate_kind, st);
}

hipError_t launch_decode_q8(const DecodeArgs& a, int d, int gate_kind, hipStream_t st) {
    if (a.dm.buffer_format == LQ_BUFFER_NFORM) {  // scalar gate only (checked by the caller)
        const dim3 grid(a.dm.n_units), block(256);
        const bool e4m3 = a.dm.code_format == LQ_CODE_E4M3;
        (void)d;  // d = 128 only (checked by the caller)
        const bool stream = stream_loads(a.dm);
        if (e4m3) {
            if (stream) hipLaunchKernelGGL((decode_nform_kernel<128, LQ_CODE_E4M3, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((decode_nform_kernel<128, LQ_CODE_E4M3, false>), grid, block, 0, st, a);
        } else {
            if (stream) hipLaunchKernelGGL((decode_nform_kernel<128, LQ_CODE_INT8, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((decode_nform_kernel<128, LQ_CODE_INT8, false>), grid, block, 0, st, a);
        }
        return hipGetLastError();
    }
    if (a.dm.buffer_format == LQ_BUFFER_FP16) launch_decode_q8_b<true>(a, d, gate_kind, st);
    else launch_decode_q8_b<false>(a, d, gate_kind, st);
    return hipGetLastError();
}

hipError_t launch_decode_fp32(const Fp32DecodeArgs& a, int d, int gate_kind, hipStream_t st) {
    const dim3 grid(a.dm.n_units), block(256);
    if (d == 128) {
        if (gate_kind == LQ_GATE_CHANNEL) hipLaunchKernelGGL((decode_fp32_kernel<128, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((decode_fp32_kernel<128, false>), grid, block, 0, st, a);
    } else {
        if (gate_kind == LQ_GATE_CHANNEL) hipLaunchKernelGGL((decode_fp32_kernel<64, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((decode_fp32_kernel<64, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace lq
