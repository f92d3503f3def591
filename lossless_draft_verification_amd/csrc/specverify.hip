// specverify.hip -- verify/accept kernels for block speculative decoding on
// MI355X (gfx950, CDNA4, wave64) and the C-ABI entry points of
// include/specverify.h.
//
// The path (one decode cycle, per sequence): a target logit block [K+1, V]
// (row 0 = p_1 from the anchor step, rows 1..K = p_2..p_{K+1} from one verify
// forward, row K = bonus position; "dspark-mlx 0.1.0" wheel diff,
// dspark_mlx/adapter.py, "Logit conventions") and, for the sampling rule, a
// draft block [K, V] with K draft tokens.
//
// Kernels (all HBM-bound streaming reductions; no MFMA -- nothing here is a
// dense contraction):
//   row_stats_greedy  one wave per 16 KiB row segment: per-lane max and first
//                     argmax over 16 coalesced 16-byte loads, wave butterfly
//                     merge (larger value, then lower index).
//   row_stats_sample  same segment walk over every target and draft row:
//                     per-lane max, per-lane fp32 sum of exp2((z-m)*log2e/T),
//                     lane sums merged in double at the wave's max.
//   scan_greedy       one wave per sequence: fixed-order merge of the segment
//                     partials, accept-prefix scan, outputs.
//   scan_sample       one wave per sequence: fixed-order double merge to the
//                     log-normalisers, gather of z[x_i], Philox uniforms,
//                     ratio test, outputs, and the draw plan for slot n.
//   residual_mass     one wave per segment of the rejected row pair:
//                     sum of max(0, p - q) over the segment.
//   draw_token        one 256-thread block per sequence: prefix over segment
//                     masses, re-read of the one segment holding t, block
//                     prefix sum in double, inverse-CDF search.
//
// Every merge runs in a fixed order with no floating-point atomics, so two
// calls on the same bytes give the same bits.

#include <hip/hip_runtime.h>

#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "specverify.h"

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kVecPerLane = 16;                      // 16-byte loads per lane per segment
constexpr int kSegVec = kWave * kVecPerLane;         // 1024 vectors = 16 KiB per wave

enum : int32_t { kModeNone = 0, kModeResidual = 1, kModeTarget = 2 };

struct GreedyPartial {
    float m;        // largest raw logit of the segment
    int32_t idx;    // its lowest index; -1 when the segment holds NaN or +inf
};

struct SamplePartial {
    float m;        // largest raw logit of the segment (-FLT_MAX if none finite)
    int32_t pad;
    double S;       // sum over the segment of exp((z - m) / T)
};

// Draw plan for one sequence, written by scan_sample.
struct DrawPlan {
    int32_t mode;       // kModeNone / kModeResidual / kModeTarget
    int32_t slot;       // n: the slot whose token is drawn
    double u2;          // U(seed, s, n, 1)
    float Mt, Md;       // raw row maxima of target row n and draft row n
    float Lt_hi, Lt_lo; // log2 of the target row's sum at Mt, split hi + lo
    float Ld_hi, Ld_lo; // same for the draft row
    double St;          // target row sum at Mt
};

__host__ __device__ constexpr int elems_per_vec(int dtype) { return dtype == SPEC_BF16 ? 8 : 4; }
__host__ __device__ constexpr int elem_bytes(int dtype) { return dtype == SPEC_BF16 ? 2 : 4; }
__host__ __device__ inline int64_t seg_elems(int dtype) { return (int64_t)kSegVec * elems_per_vec(dtype); }

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
// Element access.

template <int DT>
__device__ inline float elem_at(const void *rowp, int64_t v) {
    if constexpr (DT == SPEC_BF16) {
        uint32_t h = ((const uint16_t *)rowp)[v];
        return __uint_as_float(h << 16);
    } else {
        return ((const float *)rowp)[v];
    }
}

// Element k of a 16-byte vector (8 bf16 or 4 fp32), ascending memory order.
template <int DT>
__device__ inline float vec_elem(const uint4 &d, int k) {
    if constexpr (DT == SPEC_BF16) {
        uint32_t w = (k >> 1) == 0 ? d.x : (k >> 1) == 1 ? d.y : (k >> 1) == 2 ? d.z : d.w;
        return (k & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
    } else {
        uint32_t w = k == 0 ? d.x : k == 1 ? d.y : k == 2 ? d.z : d.w;
        return __uint_as_float(w);
    }
}

// Pairwise fp32 sum of N values (N = 4 or 8), a fixed tree.
template <int N>
__device__ inline float pairwise_sum(const float (&e)[N]) {
    if constexpr (N == 8) return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    else return (e[0] + e[1]) + (e[2] + e[3]);
}

// Vector vi of a row, or -inf padding past the end (element-wise for the one
// vector that straddles V).
template <int DT>
__device__ inline uint4 load_vec_tail(const void *rowp, int64_t vi, int V) {
    const int epv = elems_per_vec(DT);
    uint32_t w[4];
    if constexpr (DT == SPEC_BF16) {
        const uint16_t *p = (const uint16_t *)rowp;
        uint16_t h[8];
        for (int k = 0; k < 8; ++k) {
            int64_t e = vi * epv + k;
            h[k] = e < V ? p[e] : (uint16_t)0xFF80u;   // bf16 -inf
        }
        for (int k = 0; k < 4; ++k) w[k] = (uint32_t)h[2 * k] | ((uint32_t)h[2 * k + 1] << 16);
    } else {
        const uint32_t *p = (const uint32_t *)rowp;
        for (int k = 0; k < 4; ++k) {
            int64_t e = vi * epv + k;
            w[k] = e < V ? p[e] : 0xFF800000u;         // fp32 -inf
        }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// The 16 vectors a lane owns in segment `seg`: vector seg*1024 + u*64 + lane.
template <int DT>
__device__ inline void load_segment(const void *rowp, int seg, int lane, int V, uint4 (&d)[kVecPerLane]) {
    const int epv = elems_per_vec(DT);
    const int64_t nfull = (int64_t)V / epv;
    const int64_t v0 = (int64_t)seg * kSegVec;
    const uint4 *vp = (const uint4 *)rowp;
    if (v0 + kSegVec <= nfull) {
#pragma unroll
        for (int u = 0; u < kVecPerLane; ++u) d[u] = vp[v0 + u * kWave + lane];
    } else {
#pragma unroll
        for (int u = 0; u < kVecPerLane; ++u) {
            int64_t vi = v0 + u * kWave + lane;
            d[u] = vi < nfull ? vp[vi] : load_vec_tail<DT>(rowp, vi, V);
        }
    }
}

// ---------------------------------------------------------------------------
// Wave-level merges (butterfly: every lane ends with the same bits).

__device__ inline float wave_max(float x) {
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
    return x;
}

__device__ inline double wave_sum(double x) {
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

__device__ inline void wave_argmax(float &m, int32_t &idx) {
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) {
        float om = __shfl_xor(m, off, kWave);
        int32_t oi = __shfl_xor(idx, off, kWave);
        if (om > m || (om == m && oi < idx)) {
            m = om;
            idx = oi;
        }
    }
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror & Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies by the round multipliers with the high halves xored
// into the other counter words and the round key; the key advances by the two
// Weyl increments between rounds.

__device__ inline double philox_uniform(uint64_t seed, uint32_t row, uint32_t pos, uint32_t tag) {
    uint32_t x0 = pos, x1 = row, x2 = tag, x3 = 0u;
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t a = 0xD2511F53u, c = 0xCD9E8D57u;
        uint32_t hi_a = __umulhi(a, x0), lo_a = a * x0;
        uint32_t hi_c = __umulhi(c, x2), lo_c = c * x2;
        uint32_t y0 = hi_c ^ x1 ^ k0;
        uint32_t y2 = hi_a ^ x3 ^ k1;
        x0 = y0;
        x1 = lo_c;
        x2 = y2;
        x3 = lo_a;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return (double)(x0 >> 8) * (1.0 / 16777216.0);
}

// ---------------------------------------------------------------------------
// Row addressing.  `row` enumerates (sequence, row-in-block) pairs.

template <int DT>
__device__ inline const void *row_ptr(const void *base, int64_t bstride, int64_t rstride, int s, int i) {
    return (const char *)base + ((int64_t)s * bstride + (int64_t)i * rstride) * (int64_t)elem_bytes(DT);
}

// ---------------------------------------------------------------------------
// Greedy row pass.

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void row_stats_greedy(
    const void *__restrict__ target, int64_t bs, int64_t rs, int K1, int V, int nseg,
    int seg_blocks, GreedyPartial *__restrict__ part) {
    const int lane = threadIdx.x & (kWave - 1);
    const int row = blockIdx.x / seg_blocks;
    const int seg = (blockIdx.x - row * seg_blocks) * kWavesPerBlock + (threadIdx.x >> 6);
    if (seg >= nseg) return;
    const int s = row / K1, i = row - s * K1;
    const void *rowp = row_ptr<DT>(target, bs, rs, s, i);

    float mx = -INFINITY;
    int32_t ix = INT_MAX;
    bool bad = false;
    if constexpr (VEC) {
        uint4 d[kVecPerLane];
        load_segment<DT>(rowp, seg, lane, V, d);
        const int epv = elems_per_vec(DT);
#pragma unroll
        for (int u = 0; u < kVecPerLane; ++u) {
            const int32_t e0 = (int32_t)(((int64_t)seg * kSegVec + u * kWave + lane) * epv);
#pragma unroll
            for (int k = 0; k < elems_per_vec(DT); ++k) {
                float f = vec_elem<DT>(d[u], k);
                bad |= !(f < INFINITY);
                if (f > mx) {
                    mx = f;
                    ix = e0 + k;
                }
            }
        }
    } else {
        const int64_t e_begin = (int64_t)seg * seg_elems(DT);
        const int64_t e_end = min((int64_t)V, e_begin + seg_elems(DT));
        for (int64_t e = e_begin + lane; e < e_end; e += kWave) {
            float f = elem_at<DT>(rowp, e);
            bad |= !(f < INFINITY);
            if (f > mx) {
                mx = f;
                ix = (int32_t)e;
            }
        }
    }
    wave_argmax(mx, ix);
    const bool any_bad = __ballot(bad) != 0ull;
    if (lane == 0) {
        GreedyPartial p;
        p.m = mx;
        p.idx = any_bad ? -1 : ix;
        part[(int64_t)row * nseg + seg] = p;
    }
}

// ---------------------------------------------------------------------------
// Sampling row pass.  c_hi + c_lo = log2(e) / T with c_hi rounded down and
// c_lo >= FLT_MIN, so that z = -inf gives exp2(-inf) = 0 and never NaN.

template <int DT>
__device__ inline float scaled_exp2(float dz, float c_hi, float c_lo) {
    return __builtin_amdgcn_exp2f(fmaf(dz, c_hi, dz * c_lo));
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void row_stats_sample(
    const void *__restrict__ target, const void *__restrict__ draft,
    int64_t tbs, int64_t trs, int64_t dbs, int64_t drs, int K, int V, int nseg,
    int seg_blocks, float c_hi, float c_lo, double c64, SamplePartial *__restrict__ part) {
    const int lane = threadIdx.x & (kWave - 1);
    const int row = blockIdx.x / seg_blocks;
    const int seg = (blockIdx.x - row * seg_blocks) * kWavesPerBlock + (threadIdx.x >> 6);
    if (seg >= nseg) return;
    const int R = 2 * K + 1;
    const int s = row / R, i = row - s * R;
    const void *rowp = i <= K ? row_ptr<DT>(target, tbs, trs, s, i)
                              : row_ptr<DT>(draft, dbs, drs, s, i - K - 1);

    // Per lane: max, then the sum of exp2 at that max -- pairwise in fp32
    // inside each 16-byte vector, in double across vectors.
    float ml = -FLT_MAX;
    double sl = 0.0;
    if constexpr (VEC) {
        uint4 d[kVecPerLane];
        load_segment<DT>(rowp, seg, lane, V, d);
#pragma unroll
        for (int u = 0; u < kVecPerLane; ++u)
#pragma unroll
            for (int k = 0; k < elems_per_vec(DT); ++k) ml = fmaxf(ml, vec_elem<DT>(d[u], k));
#pragma unroll
        for (int u = 0; u < kVecPerLane; ++u) {
            float e[elems_per_vec(DT)];
#pragma unroll
            for (int k = 0; k < elems_per_vec(DT); ++k)
                e[k] = scaled_exp2<DT>(vec_elem<DT>(d[u], k) - ml, c_hi, c_lo);
            sl += (double)pairwise_sum<elems_per_vec(DT)>(e);
        }
    } else {
        const int64_t e_begin = (int64_t)seg * seg_elems(DT);
        const int64_t e_end = min((int64_t)V, e_begin + seg_elems(DT));
        for (int64_t e = e_begin + lane; e < e_end; e += kWave) ml = fmaxf(ml, elem_at<DT>(rowp, e));
        for (int64_t e = e_begin + lane; e < e_end; e += kWave)
            sl += (double)scaled_exp2<DT>(elem_at<DT>(rowp, e) - ml, c_hi, c_lo);
    }
    const float mw = wave_max(ml);
    const double contrib = sl * exp2(((double)ml - (double)mw) * c64);
    const double Sw = wave_sum(contrib);
    if (lane == 0) {
        SamplePartial p;
        p.m = mw;
        p.pad = 0;
        p.S = Sw;
        part[(int64_t)row * nseg + seg] = p;
    }
}

// ---------------------------------------------------------------------------
// Greedy accept-prefix scan: one wave per sequence.

__global__ __launch_bounds__(kWave) void scan_greedy(
    const GreedyPartial *__restrict__ part, int nseg, int K, int V,
    const int32_t *__restrict__ draft_tokens, int32_t *__restrict__ n_out,
    int32_t *__restrict__ tokens, int32_t *__restrict__ argmax_out) {
    const int s = blockIdx.x;
    const int lane = threadIdx.x;
    const int K1 = K + 1;
    __shared__ int32_t sA[SPEC_MAX_K + 1];
    __shared__ int32_t sBad;
    if (lane == 0) sBad = 0;
    __syncthreads();
    for (int i = 0; i < K1; ++i) {
        const GreedyPartial *pr = part + ((int64_t)s * K1 + i) * nseg;
        float m = -INFINITY;
        int32_t idx = INT_MAX;
        bool bad = false;
        for (int j = lane; j < nseg; j += kWave) {   // ascending segments: ties keep the lower index
            GreedyPartial p = pr[j];
            if (p.idx < 0) bad = true;
            else if (p.m > m) {
                m = p.m;
                idx = p.idx;
            }
        }
        wave_argmax(m, idx);
        const bool any_bad = __ballot(bad) != 0ull;
        if (lane == 0) {
            sA[i] = idx;
            if (any_bad || !(m > -INFINITY)) sBad = 1;
        }
    }
    __syncthreads();
    bool tok_bad = false;
    if (lane < K) {
        int32_t x = draft_tokens[(int64_t)s * K + lane];
        tok_bad = x < 0 || x >= V;
    }
    const bool invalid = sBad || (__ballot(tok_bad) != 0ull);
    int32_t *tok = tokens + (int64_t)s * K1;
    if (invalid) {
        if (lane < K1) {
            tok[lane] = -1;
            if (argmax_out) argmax_out[(int64_t)s * K1 + lane] = -1;
        }
        if (lane == 0) n_out[s] = -1;
        return;
    }
    bool mismatch = false;
    if (lane < K) mismatch = draft_tokens[(int64_t)s * K + lane] != sA[lane];
    const unsigned long long mm = __ballot(mismatch);
    const int n = mm ? (int)__ffsll((long long)mm) - 1 : K;
    if (lane < K1) {
        int32_t t = lane < n ? draft_tokens[(int64_t)s * K + lane] : lane == n ? sA[n] : -1;
        tok[lane] = t;
        if (argmax_out) argmax_out[(int64_t)s * K1 + lane] = sA[lane];
    }
    if (lane == 0) n_out[s] = n;
}

// ---------------------------------------------------------------------------
// Sampling accept scan: one wave per sequence.

template <int DT>
__global__ __launch_bounds__(kWave) void scan_sample(
    const SamplePartial *__restrict__ part, int nseg, int K, int V, double T, double c64,
    const void *__restrict__ target, const void *__restrict__ draft,
    int64_t tbs, int64_t trs, int64_t dbs, int64_t drs,
    const int32_t *__restrict__ draft_tokens, const uint64_t *__restrict__ seeds,
    int32_t *__restrict__ n_out, int32_t *__restrict__ tokens,
    float *__restrict__ p_out, float *__restrict__ q_out, DrawPlan *__restrict__ plan) {
    const int s = blockIdx.x;
    const int lane = threadIdx.x;
    const int R = 2 * K + 1;
    __shared__ float sM[2 * SPEC_MAX_K + 1];
    __shared__ double sS[2 * SPEC_MAX_K + 1];

    bool row_bad = false;
    for (int r = 0; r < R; ++r) {
        const SamplePartial *pr = part + ((int64_t)s * R + r) * nseg;
        float m = -FLT_MAX;
        for (int j = lane; j < nseg; j += kWave) m = fmaxf(m, pr[j].m);
        const float M = wave_max(m);
        double acc = 0.0;
        for (int j = lane; j < nseg; j += kWave) {
            SamplePartial p = pr[j];
            acc += p.S * exp2(((double)p.m - (double)M) * c64);
        }
        const double S = wave_sum(acc);
        if (lane == 0) {
            sM[r] = M;
            sS[r] = S;
        }
        if (!(S > 0.0) || !(S < INFINITY)) row_bad = true;   // NaN/+inf seen, or no finite entry
    }
    __syncthreads();

    const uint64_t seed = seeds[s];
    int32_t x = 0;
    bool tok_bad = false;
    if (lane < K) {
        x = draft_tokens[(int64_t)s * K + lane];
        tok_bad = x < 0 || x >= V;
    }
    const bool invalid = row_bad || (__ballot(tok_bad) != 0ull);
    int32_t *tok = tokens + (int64_t)s * (K + 1);
    if (invalid) {
        if (lane <= K) tok[lane] = -1;
        if (lane < K) {
            if (p_out) p_out[(int64_t)s * K + lane] = NAN;
            if (q_out) q_out[(int64_t)s * K + lane] = NAN;
        }
        if (lane == 0) {
            n_out[s] = -1;
            DrawPlan pl = {};
            pl.mode = kModeNone;
            plan[s] = pl;
        }
        return;
    }

    bool reject = false;
    if (lane < K) {
        const float zt = elem_at<DT>(row_ptr<DT>(target, tbs, trs, s, lane), x);
        const float zd = elem_at<DT>(row_ptr<DT>(draft, dbs, drs, s, lane), x);
        const double lp = ((double)zt - (double)sM[lane]) / T - log(sS[lane]);
        const double lq = ((double)zd - (double)sM[K + 1 + lane]) / T - log(sS[K + 1 + lane]);
        double r;
        if (zt == -INFINITY) r = 0.0;                 // p(x) = 0: never accepted
        else if (zd == -INFINITY) r = INFINITY;       // q(x) = 0 < p(x): always accepted
        else r = exp(lp - lq);
        const double u = philox_uniform(seed, (uint32_t)s, (uint32_t)lane, 0u);
        reject = !(u < r);                            // u < 1, so u < r == u < min(1, r)
        if (p_out) p_out[(int64_t)s * K + lane] = (float)exp(lp);
        if (q_out) q_out[(int64_t)s * K + lane] = (float)exp(lq);
    }
    const unsigned long long rj = __ballot(reject);
    const int n = rj ? (int)__ffsll((long long)rj) - 1 : K;
    if (lane <= K) tok[lane] = lane < n ? x : -1;    // slot n is filled by draw_token
    if (lane == 0) {
        n_out[s] = n;
        DrawPlan pl;
        pl.mode = n < K ? kModeResidual : kModeTarget;
        pl.slot = n;
        pl.u2 = philox_uniform(seed, (uint32_t)s, (uint32_t)n, 1u);
        const double St = sS[n];
        const double Lt = log2(St);
        pl.Mt = sM[n];
        pl.St = St;
        pl.Lt_hi = (float)Lt;
        pl.Lt_lo = (float)(Lt - (double)pl.Lt_hi);
        if (n < K) {
            const double Ld = log2(sS[K + 1 + n]);
            pl.Md = sM[K + 1 + n];
            pl.Ld_hi = (float)Ld;
            pl.Ld_lo = (float)(Ld - (double)pl.Ld_hi);
        } else {
            pl.Md = 0.0f;
            pl.Ld_hi = 0.0f;
            pl.Ld_lo = 0.0f;
        }
        plan[s] = pl;
    }
}

// ---------------------------------------------------------------------------
// Draw weights.  p(v) = exp2((z - M) * log2(e)/T - log2 S), evaluated as
// fma(dz, c_hi, -L_hi) + fma(dz, c_lo, -L_lo) so the large terms cancel inside
// one rounding.  residual_mass and draw_token call the same function on the
// same constants, so a weight has the same bits in both.

__device__ inline float target_weight(float zt, const DrawPlan &pl, float c_hi, float c_lo) {
    const float dz = fmaxf(zt - pl.Mt, -3.0e38f);
    return __builtin_amdgcn_exp2f(fmaf(dz, c_hi, -pl.Lt_hi) + fmaf(dz, c_lo, -pl.Lt_lo));
}

__device__ inline float residual_weight(float zt, float zd, const DrawPlan &pl, float c_hi, float c_lo) {
    const float dzd = fmaxf(zd - pl.Md, -3.0e38f);
    const float q = __builtin_amdgcn_exp2f(fmaf(dzd, c_hi, -pl.Ld_hi) + fmaf(dzd, c_lo, -pl.Ld_lo));
    const float w = target_weight(zt, pl, c_hi, c_lo) - q;
    return w > 0.0f ? w : 0.0f;
}

// Segment masses of max(0, p_n - q_n) for sequences that rejected a slot.
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void residual_mass(
    const void *__restrict__ target, const void *__restrict__ draft,
    int64_t tbs, int64_t trs, int64_t dbs, int64_t drs, int V, int nseg, int seg_blocks,
    float c_hi, float c_lo, const DrawPlan *__restrict__ plan, double *__restrict__ rmass) {
    const int lane = threadIdx.x & (kWave - 1);
    const int s = blockIdx.x / seg_blocks;
    const int seg = (blockIdx.x - s * seg_blocks) * kWavesPerBlock + (threadIdx.x >> 6);
    if (seg >= nseg) return;
    const DrawPlan pl = plan[s];
    if (pl.mode != kModeResidual) return;
    const void *tp = row_ptr<DT>(target, tbs, trs, s, pl.slot);
    const void *dp = row_ptr<DT>(draft, dbs, drs, s, pl.slot);
    double acc = 0.0;
    if constexpr (VEC) {
        uint4 a[kVecPerLane], b[kVecPerLane];
        load_segment<DT>(tp, seg, lane, V, a);
        load_segment<DT>(dp, seg, lane, V, b);
#pragma unroll
        for (int u = 0; u < kVecPerLane; ++u) {
            float w[elems_per_vec(DT)];
#pragma unroll
            for (int k = 0; k < elems_per_vec(DT); ++k)
                w[k] = residual_weight(vec_elem<DT>(a[u], k), vec_elem<DT>(b[u], k), pl, c_hi, c_lo);
            acc += (double)pairwise_sum<elems_per_vec(DT)>(w);
        }
    } else {
        const int64_t e_begin = (int64_t)seg * seg_elems(DT);
        const int64_t e_end = min((int64_t)V, e_begin + seg_elems(DT));
        for (int64_t e = e_begin + lane; e < e_end; e += kWave)
            acc += (double)residual_weight(elem_at<DT>(tp, e), elem_at<DT>(dp, e), pl, c_hi, c_lo);
    }
    const double Sw = wave_sum(acc);
    if (lane == 0) rmass[(int64_t)s * nseg + seg] = Sw;
}

// Block-wide exclusive prefix over one double per thread, in thread order
// (thread 0 adds them up sequentially: the order never changes).
__device__ inline double block_exclusive_prefix(double v, double *sbuf, double &total) {
    sbuf[threadIdx.x] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        double run = 0.0;
        for (int t = 0; t < kBlock; ++t) {
            double x = sbuf[t];
            sbuf[t] = run;
            run += x;
        }
        sbuf[kBlock] = run;
    }
    __syncthreads();
    const double pre = sbuf[threadIdx.x];
    total = sbuf[kBlock];
    __syncthreads();
    return pre;
}

// Draw the token of slot n: inverse CDF over ascending vocabulary index of
// the residual (mode residual) or of p_n (mode target: the bonus, or a
// rejected slot whose residual mass is zero).
template <int DT>
__global__ __launch_bounds__(kBlock) void draw_token(
    const void *__restrict__ target, const void *__restrict__ draft,
    int64_t tbs, int64_t trs, int64_t dbs, int64_t drs, int K, int V, int nseg,
    float c_hi, float c_lo, double c64, const SamplePartial *__restrict__ spart,
    const double *__restrict__ rmass, const DrawPlan *__restrict__ plan,
    int32_t *__restrict__ tokens) {
    const int s = blockIdx.x;
    const int t = threadIdx.x;
    __shared__ double sbuf[kBlock + 1];
    __shared__ int32_t sSeg;
    __shared__ double sOff;
    __shared__ int32_t sY;

    const DrawPlan pl = plan[s];
    if (pl.mode == kModeNone) return;
    int mode = pl.mode;
    const int R = 2 * K + 1;
    const SamplePartial *tpart = spart + ((int64_t)s * R + pl.slot) * nseg;
    const double *rm = rmass + (int64_t)s * nseg;

    // Segment masses, summed per thread over a contiguous range of segments
    // (sequentially from zero), then an exclusive prefix over threads.
    auto seg_mass = [&](int j, int md) -> double {
        return md == kModeResidual ? rm[j]
                                   : tpart[j].S * exp2(((double)tpart[j].m - (double)pl.Mt) * c64) / pl.St;
    };
    const int per = (nseg + kBlock - 1) / kBlock;
    const int j0 = min(nseg, t * per), j1 = min(nseg, j0 + per);
    double local = 0.0, total = 0.0, pre = 0.0;
    for (int pass = 0; pass < 2; ++pass) {
        local = 0.0;
        for (int j = j0; j < j1; ++j) local += seg_mass(j, mode);
        pre = block_exclusive_prefix(local, sbuf, total);
        if (mode == kModeResidual && !(total > 0.0)) {
            mode = kModeTarget;            // zero residual mass: draw from p_n
            continue;
        }
        break;
    }
    const double tt = pl.u2 * total;       // u2 < 1, so tt < total when total > 0
    if (t == 0) {
        sSeg = -1;
        sY = -1;
    }
    __syncthreads();
    // The first segment whose running mass exceeds tt.  The thread holding it
    // re-accumulates its own range exactly as `local` was formed, so the scan
    // is certain to stop inside the range.
    if (pre <= tt && pre + local > tt) {
        double run = 0.0;
        for (int j = j0; j < j1; ++j) {
            const double before = run;
            run += seg_mass(j, mode);
            if (pre + run > tt || j == j1 - 1) {
                sSeg = j;
                sOff = pre + before;
                break;
            }
        }
    }
    __syncthreads();
    if (sSeg < 0 && t == 0) {
        // total == 0 (no mass anywhere): take the first segment.
        sSeg = 0;
        sOff = 0.0;
    }
    __syncthreads();
    const int seg = sSeg;
    const double tl = tt - sOff;

    // Re-read segment `seg`: thread t owns a contiguous run of elements.
    const void *tp = row_ptr<DT>(target, tbs, trs, s, pl.slot);
    const void *dp = row_ptr<DT>(draft, dbs, drs, s, mode == kModeResidual ? pl.slot : 0);
    const int64_t E = seg_elems(DT) / kBlock;
    const int64_t e0 = (int64_t)seg * seg_elems(DT) + (int64_t)t * E;
    const int64_t e1 = min((int64_t)V, e0 + E);
    auto weight = [&](int64_t e) -> float {
        return mode == kModeResidual ? residual_weight(elem_at<DT>(tp, e), elem_at<DT>(dp, e), pl, c_hi, c_lo)
                                     : target_weight(elem_at<DT>(tp, e), pl, c_hi, c_lo);
    };
    double wsum = 0.0;
    for (int64_t e = e0; e < e1; ++e) wsum += (double)weight(e);
    double segtotal = 0.0;
    const double wpre = block_exclusive_prefix(wsum, sbuf, segtotal);
    if (!(tl < segtotal)) {
        // tl at or past this segment's recomputed total by rounding: the
        // last positive weight of the segment is the one reached.
        int64_t last_pos = -1;
        for (int64_t e = e0; e < e1; ++e)
            if (weight(e) > 0.0f) last_pos = e;
        if (last_pos >= 0) atomicMax(&sY, (int32_t)last_pos);
    } else if (wpre <= tl && wpre + wsum > tl) {
        // Exactly one thread gets here; re-accumulating from zero in the same
        // order reproduces wsum, so the scan stops inside the range.
        double run = 0.0;
        for (int64_t e = e0; e < e1; ++e) {
            run += (double)weight(e);
            if (wpre + run > tl) {
                sY = (int32_t)e;
                break;
            }
        }
    }
    __syncthreads();
    if (t == 0) {
        int32_t y = sY;
        if (y < 0) y = (int32_t)min((int64_t)V - 1, (int64_t)seg * seg_elems(DT));
        tokens[(int64_t)s * (K + 1) + pl.slot] = y;
    }
}

// ---------------------------------------------------------------------------
// Streaming copy used to calibrate byte counters.

__global__ __launch_bounds__(kBlock) void stream_copy_kernel(uint4 *__restrict__ dst, const uint4 *__restrict__ src,
                                                              int64_t nvec) {
    const int64_t base = (int64_t)blockIdx.x * (kBlock * kVecPerLane);
    uint4 d[kVecPerLane];
#pragma unroll
    for (int u = 0; u < kVecPerLane; ++u) {
        int64_t vi = base + u * kBlock + threadIdx.x;
        if (vi < nvec) d[u] = src[vi];
    }
#pragma unroll
    for (int u = 0; u < kVecPerLane; ++u) {
        int64_t vi = base + u * kBlock + threadIdx.x;
        if (vi < nvec) dst[vi] = d[u];
    }
}

// ---------------------------------------------------------------------------
// Host side.

thread_local hipEvent_t *t_stage_events = nullptr;
thread_local int t_stage_n = 0;

inline void stage_mark(int k, int nkernels, hipStream_t st) {
    if (t_stage_events && t_stage_n >= nkernels + 1) (void)hipEventRecord(t_stage_events[k], st);
}

struct Layout {
    int nseg;
    size_t part_off, part_bytes;
    size_t plan_off, plan_bytes;
    size_t rmass_off, rmass_bytes;
    size_t total;
};

bool make_layout(int b, int K, int V, int dtype, int sampling, Layout &L) {
    if (b < 1 || K < 1 || K > SPEC_MAX_K || V < 1) return false;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return false;
    const int64_t se = seg_elems(dtype);
    L.nseg = (int)(((int64_t)V + se - 1) / se);
    const int64_t rows = sampling ? (int64_t)b * (2 * K + 1) : (int64_t)b * (K + 1);
    const size_t psize = sampling ? sizeof(SamplePartial) : sizeof(GreedyPartial);
    L.part_off = 0;
    L.part_bytes = align256((size_t)rows * (size_t)L.nseg * psize);
    L.plan_off = L.part_off + L.part_bytes;
    L.plan_bytes = sampling ? align256((size_t)b * sizeof(DrawPlan)) : 0;
    L.rmass_off = L.plan_off + L.plan_bytes;
    L.rmass_bytes = sampling ? align256((size_t)b * (size_t)L.nseg * sizeof(double)) : 0;
    L.total = L.rmass_off + L.rmass_bytes;
    return true;
}

bool rows_vector_aligned(const void *p, int es, int64_t bs, int64_t rs) {
    return ((uintptr_t)p % 16 == 0) && ((bs * es) % 16 == 0) && ((rs * es) % 16 == 0);
}

// log2(e)/T as hi + lo with hi rounded down and lo >= FLT_MIN.
void split_scale(double T, float &c_hi, float &c_lo, double &c64) {
    c64 = 1.4426950408889634 / T;
    float hi = (float)c64;
    if ((double)hi > c64) hi = nextafterf(hi, 0.0f);
    double lo = c64 - (double)hi;
    c_hi = hi;
    c_lo = (float)lo < FLT_MIN ? FLT_MIN : (float)lo;
}

template <int DT, bool VEC>
int launch_greedy(const void *target, int64_t bs, int64_t rs, const int32_t *x, int b, int K, int V,
                  int32_t *n_out, int32_t *tok, int32_t *am, char *ws, const Layout &L, hipStream_t st) {
    const int seg_blocks = (L.nseg + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t grid = (int64_t)b * (K + 1) * seg_blocks;
    if (grid > INT_MAX) return SPEC_EINVAL;
    GreedyPartial *part = (GreedyPartial *)(ws + L.part_off);
    stage_mark(0, 2, st);
    hipLaunchKernelGGL((row_stats_greedy<DT, VEC>), dim3((unsigned)grid), dim3(kBlock), 0, st,
                       target, bs, rs, K + 1, V, L.nseg, seg_blocks, part);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(1, 2, st);
    hipLaunchKernelGGL(scan_greedy, dim3((unsigned)b), dim3(kWave), 0, st, part, L.nseg, K, V, x, n_out, tok, am);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(2, 2, st);
    return SPEC_OK;
}

template <int DT, bool VEC>
int launch_sample(const void *target, const void *draft, int64_t tbs, int64_t trs, int64_t dbs, int64_t drs,
                  const int32_t *x, int b, int K, int V, double T, const uint64_t *seeds, int32_t *n_out,
                  int32_t *tok, float *p_out, float *q_out, char *ws, const Layout &L, hipStream_t st) {
    const int seg_blocks = (L.nseg + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t grid1 = (int64_t)b * (2 * K + 1) * seg_blocks;
    const int64_t grid3 = (int64_t)b * seg_blocks;
    if (grid1 > INT_MAX) return SPEC_EINVAL;
    float c_hi, c_lo;
    double c64;
    split_scale(T, c_hi, c_lo, c64);
    SamplePartial *part = (SamplePartial *)(ws + L.part_off);
    DrawPlan *plan = (DrawPlan *)(ws + L.plan_off);
    double *rmass = (double *)(ws + L.rmass_off);
    stage_mark(0, 4, st);
    hipLaunchKernelGGL((row_stats_sample<DT, VEC>), dim3((unsigned)grid1), dim3(kBlock), 0, st,
                       target, draft, tbs, trs, dbs, drs, K, V, L.nseg, seg_blocks, c_hi, c_lo, c64, part);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(1, 4, st);
    hipLaunchKernelGGL((scan_sample<DT>), dim3((unsigned)b), dim3(kWave), 0, st, part, L.nseg, K, V, T, c64,
                       target, draft, tbs, trs, dbs, drs, x, seeds, n_out, tok, p_out, q_out, plan);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(2, 4, st);
    hipLaunchKernelGGL((residual_mass<DT, VEC>), dim3((unsigned)grid3), dim3(kBlock), 0, st,
                       target, draft, tbs, trs, dbs, drs, V, L.nseg, seg_blocks, c_hi, c_lo, plan, rmass);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(3, 4, st);
    hipLaunchKernelGGL((draw_token<DT>), dim3((unsigned)b), dim3(kBlock), 0, st, target, draft, tbs, trs, dbs,
                       drs, K, V, L.nseg, c_hi, c_lo, c64, part, rmass, plan, tok);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(4, 4, st);
    return SPEC_OK;
}

}  // namespace

extern "C" {

size_t spec_workspace_bytes(int b, int K, int V, int dtype, int sampling) {
    Layout L;
    if (!make_layout(b, K, V, dtype, sampling, L)) return 0;
    return L.total;
}

const char *spec_status_string(int status) {
    switch (status) {
        case SPEC_OK: return "ok";
        case SPEC_EINVAL: return "invalid argument (size, stride, temperature, null pointer or workspace)";
        case SPEC_EDTYPE: return "unknown dtype";
        case SPEC_EALIGN: return "logit pointer not aligned to its element size";
        case SPEC_ELAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

int spec_set_stage_events(void *const *events, int n_events) {
    t_stage_events = (events && n_events > 0) ? (hipEvent_t *)events : nullptr;
    t_stage_n = t_stage_events ? n_events : 0;
    return SPEC_OK;
}

int spec_greedy_accept(const void *target, int dtype, int64_t t_batch_stride, int64_t t_row_stride,
                       const int32_t *draft_tokens, int b, int K, int V, int32_t *n_accepted,
                       int32_t *tokens, int32_t *target_argmax, void *workspace, size_t workspace_bytes,
                       void *hip_stream) {
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EDTYPE;
    Layout L;
    if (!make_layout(b, K, V, dtype, 0, L)) return SPEC_EINVAL;
    if (!target || !draft_tokens || !n_accepted || !tokens || !workspace) return SPEC_EINVAL;
    if (t_row_stride < V || t_batch_stride < 0) return SPEC_EINVAL;
    if (workspace_bytes < L.total) return SPEC_EINVAL;
    const int es = elem_bytes(dtype);
    if ((uintptr_t)target % es != 0) return SPEC_EALIGN;
    hipStream_t st = (hipStream_t)hip_stream;
    const bool vec = rows_vector_aligned(target, es, t_batch_stride, t_row_stride);
    char *ws = (char *)workspace;
    if (dtype == SPEC_BF16)
        return vec ? launch_greedy<SPEC_BF16, true>(target, t_batch_stride, t_row_stride, draft_tokens, b, K, V,
                                                     n_accepted, tokens, target_argmax, ws, L, st)
                   : launch_greedy<SPEC_BF16, false>(target, t_batch_stride, t_row_stride, draft_tokens, b, K, V,
                                                      n_accepted, tokens, target_argmax, ws, L, st);
    return vec ? launch_greedy<SPEC_F32, true>(target, t_batch_stride, t_row_stride, draft_tokens, b, K, V,
                                                n_accepted, tokens, target_argmax, ws, L, st)
               : launch_greedy<SPEC_F32, false>(target, t_batch_stride, t_row_stride, draft_tokens, b, K, V,
                                                 n_accepted, tokens, target_argmax, ws, L, st);
}

int spec_sample_accept(const void *target, const void *draft, int dtype, int64_t t_batch_stride,
                       int64_t t_row_stride, int64_t d_batch_stride, int64_t d_row_stride,
                       const int32_t *draft_tokens, int b, int K, int V, double temperature,
                       const uint64_t *seeds, int32_t *n_accepted, int32_t *tokens, float *p_draft,
                       float *q_draft, void *workspace, size_t workspace_bytes, void *hip_stream) {
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EDTYPE;
    Layout L;
    if (!make_layout(b, K, V, dtype, 1, L)) return SPEC_EINVAL;
    if (!target || !draft || !draft_tokens || !seeds || !n_accepted || !tokens || !workspace) return SPEC_EINVAL;
    if (!(temperature > 0.0) || !(temperature < INFINITY)) return SPEC_EINVAL;
    if (t_row_stride < V || t_batch_stride < 0 || d_row_stride < V || d_batch_stride < 0) return SPEC_EINVAL;
    if (workspace_bytes < L.total) return SPEC_EINVAL;
    const int es = elem_bytes(dtype);
    if ((uintptr_t)target % es != 0 || (uintptr_t)draft % es != 0) return SPEC_EALIGN;
    hipStream_t st = (hipStream_t)hip_stream;
    const bool vec = rows_vector_aligned(target, es, t_batch_stride, t_row_stride) &&
                     rows_vector_aligned(draft, es, d_batch_stride, d_row_stride);
    char *ws = (char *)workspace;
    if (dtype == SPEC_BF16)
        return vec ? launch_sample<SPEC_BF16, true>(target, draft, t_batch_stride, t_row_stride, d_batch_stride,
                                                     d_row_stride, draft_tokens, b, K, V, temperature, seeds,
                                                     n_accepted, tokens, p_draft, q_draft, ws, L, st)
                   : launch_sample<SPEC_BF16, false>(target, draft, t_batch_stride, t_row_stride, d_batch_stride,
                                                      d_row_stride, draft_tokens, b, K, V, temperature, seeds,
                                                      n_accepted, tokens, p_draft, q_draft, ws, L, st);
    return vec ? launch_sample<SPEC_F32, true>(target, draft, t_batch_stride, t_row_stride, d_batch_stride,
                                                d_row_stride, draft_tokens, b, K, V, temperature, seeds, n_accepted,
                                                tokens, p_draft, q_draft, ws, L, st)
               : launch_sample<SPEC_F32, false>(target, draft, t_batch_stride, t_row_stride, d_batch_stride,
                                                 d_row_stride, draft_tokens, b, K, V, temperature, seeds, n_accepted,
                                                 tokens, p_draft, q_draft, ws, L, st);
}

int spec_stream_copy(void *dst, const void *src, size_t nbytes, void *hip_stream) {
    if (!dst || !src || nbytes % 16 != 0 || (uintptr_t)dst % 16 || (uintptr_t)src % 16) return SPEC_EINVAL;
    if (nbytes == 0) return SPEC_OK;
    const int64_t nvec = (int64_t)(nbytes / 16);
    const int64_t per_block = (int64_t)kBlock * kVecPerLane;
    const int64_t grid = (nvec + per_block - 1) / per_block;
    if (grid > INT_MAX) return SPEC_EINVAL;
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)grid), dim3(kBlock), 0, (hipStream_t)hip_stream,
                       (uint4 *)dst, (const uint4 *)src, nvec);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

}  // extern "C"
