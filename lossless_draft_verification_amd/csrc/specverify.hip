// specverify.hip -- verify/accept kernels for block speculative decoding on
// MI355X (gfx950, CDNA4, wave64) and the C-ABI entry points of
// include/specverify.h.
//
// The path (one decode cycle, per sequence): a target logit block [K+1, V]
// (row 0 = p_1 from the anchor step, rows 1..K = p_2..p_{K+1} from one verify
// forward, row K = bonus position; "dspark-mlx 0.1.0" wheel diff,
// dspark_mlx/adapter.py, "Logit conventions") and, for the sampling rule, a
// draft block [K, V] with K draft tokens.  Each sequence follows the greedy
// rule (temperature 0) or the speculative-sampling rule (temperature T > 0).
//
// Verify kernels (HBM-bound streaming reductions; no MFMA -- nothing in the
// verify itself is a dense contraction):
//   row_pass       one single-wave workgroup per 16 KiB segment of a logit
//                  row: 16 coalesced nontemporal 16-byte loads per lane,
//                  then per lane either max + first argmax (greedy rows) or
//                  max + sum of
//                  exp2((z - max) * log2(e)/T) (sampling rows), merged across
//                  the wave by a butterfly (sums in double).  Calls with
//                  per-sequence draft lengths (up to 256 sequences) take
//                  row_pass_listed, which streams only rows inside the blocks.
//   scan           one 1024-thread block per sequence, one wave per row:
//                  fixed-order merge of the segment partials (double for the
//                  log-normalisers), then the accept-prefix scan (greedy
//                  compare, or gather of z[x_i], Philox uniforms and ratio
//                  test), the outputs and the draw plan for slot n; a
//                  rejecting sequence appends a residual work item.
//   residual_mass  one single-wave workgroup per 4 KiB segment of each
//                  rejected row pair (the work items the scans appended):
//                  sum of max(0, p - q) over the segment.
//   draw_token     one 256-thread block per sampling sequence: block scan over
//                  the segment masses, re-read of the one segment holding t
//                  into registers, block scan in double, inverse-CDF search.
//
// The fused verify (lm_head_fused.inc) and the draft-side Markov decode
// (markov_draft.inc) add the one dense contraction on the path, the lm_head /
// Markov-table GEMM, on the matrix cores; the vocabulary-sharded verify
// (vocab_sharded.inc) runs the verify kernels per shard.
//
// Every merge and scan runs in a fixed order with no floating-point atomics,
// so two calls on the same bytes give the same bits (the one integer atomic,
// a slot in the residual work list, decides only which workgroup computes a
// segment).  Kernel boundaries are the only cross-workgroup synchronisation:
// a device-scope release fence per workgroup (an L2 write-back on this
// multi-XCD part) costs far more than a launch.

#include <hip/hip_runtime.h>

#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "specverify.h"

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kScanBlock = 1024;                     // scan: one wave per row
constexpr int kVecPerLane = 16;                      // row pass: 16-byte loads per lane
constexpr int kSegVec = kWave * kVecPerLane;         // 1024 vectors = 16 KiB per wave segment
constexpr int kResVecPerLane = 4;                    // residual pass: 4 vectors per lane per row
constexpr int kResSegVec = kWave * kResVecPerLane;   // 256 vectors = 4 KiB per row per wave

enum : int32_t { kModeNone = 0, kModeResidual = 1, kModeTarget = 2 };
enum : int { kRuleInvalid = 0, kRuleGreedy = 1, kRuleSample = 2 };

// Per-segment statistics of one row.  Greedy rows: m = largest raw logit,
// idx = its lowest index (-1 if the segment holds NaN or +inf).  Sampling
// rows: m = largest raw logit (-FLT_MAX if none is finite), S = sum over the
// segment of exp((z - m) / T).
struct Partial {
    float m;
    int32_t idx;
    double S;
};

// Draw plan for one sampling sequence, written by scan.
struct DrawPlan {
    int32_t mode;       // kModeNone / kModeResidual / kModeTarget
    int32_t slot;       // n: the slot whose token is drawn
    double u2;          // U(seed, s, n, 1)
    double T;           // the sequence's temperature
    float Mt, Md;       // raw row maxima of target row n and draft row n
    float Lt_hi, Lt_lo; // log2 of the target row's sum at Mt, split hi + lo
    float Ld_hi, Ld_lo; // same for the draft row
    double St;          // target row sum at Mt
    int32_t shard;      // vocabulary-sharded call: the shard that draws
    double t_local;     // and the draw's target mass inside that shard
};

__host__ __device__ constexpr int elems_per_vec(int dtype) { return dtype == SPEC_BF16 ? 8 : 4; }
__host__ __device__ constexpr int elem_bytes(int dtype) { return dtype == SPEC_BF16 ? 2 : 4; }
__host__ __device__ constexpr int64_t seg_elems(int dtype) { return (int64_t)kSegVec * elems_per_vec(dtype); }
__host__ __device__ constexpr int64_t rseg_elems(int dtype) { return (int64_t)kResSegVec * elems_per_vec(dtype); }

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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load of streamed data: nontemporal, so it does not displace
// anything from the caches.
__device__ inline uint4 load_stream(const uint4 *p) {
    u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
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

// N vectors of a row for one lane: vector vbase + u*64 + lane, u < N, with
// -inf past the end of the row.  Vectors wholly inside the row are loaded
// with streaming 16-byte loads.
template <int DT, int N>
__device__ inline void load_vecs(const void *rowp, int64_t vbase, int lane, int V, uint4 (&d)[N]) {
    const int64_t nfull = (int64_t)V / elems_per_vec(DT);
    const uint4 *vp = (const uint4 *)rowp;
    if (vbase + (int64_t)N * kWave <= nfull) {
#pragma unroll
        for (int u = 0; u < N; ++u) d[u] = load_stream(vp + vbase + u * kWave + lane);
    } else {
#pragma unroll
        for (int u = 0; u < N; ++u) {
            int64_t vi = vbase + u * kWave + lane;
            d[u] = vi < nfull ? load_stream(vp + vi) : load_vec_tail<DT>(rowp, vi, V);
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

// Block-wide scan of one double per thread (256 threads): inclusive scan in
// each wave, then wave offsets added in wave order.  `excl` of thread t is,
// bit for bit, `incl` of thread t-1 (0 for thread 0), and `total` is `incl`
// of the last thread, so the intervals [excl, incl) tile [0, total) exactly.
// Every thread of the block must call it.
__device__ inline void block_scan(double v, double &excl, double &incl, double &total, double *sw) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x >> 6;
    double x = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    if (lane == kWave - 1) sw[w] = x;
    __syncthreads();
    double woff = 0.0;
    for (int k = 0; k < w; ++k) woff += sw[k];
    double tot = 0.0;
    for (int k = 0; k < kWavesPerBlock; ++k) tot += sw[k];
    __syncthreads();
    incl = woff + x;
    const double prev = __shfl_up(incl, 1, kWave);
    excl = lane == 0 ? woff : prev;
    total = tot;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror & Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies by the round multipliers with the high halves xored
// into the other counter words and the round key; the key advances by the two
// Weyl increments between rounds.  U = top 24 bits of output word 0 * 2^-24.

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
// Rules and scales.

// Temperature 0 is the greedy rule, a finite positive temperature the
// sampling rule; anything else makes the sequence invalid.
__device__ inline int rule_of(double T) {
    if (T == 0.0) return kRuleGreedy;
    if (T > 0.0 && T < INFINITY) return kRuleSample;
    return kRuleInvalid;
}

// log2(e)/T as c_hi + c_lo: c_hi rounded down, c_lo >= FLT_MIN, so both
// products of a -inf logit difference stay -inf (never -inf + inf = NaN).
__device__ inline void split_scale(double T, float &c_hi, float &c_lo, double &c64) {
    c64 = 1.4426950408889634 / T;
    c_hi = __double2float_rd(c64);
    const float lo = (float)(c64 - (double)c_hi);
    c_lo = lo < FLT_MIN ? FLT_MIN : lo;
}

// exp2(d * log2(e)/T) for a non-positive max difference d = m - M (floats),
// in fp32 with the split scale, as the elements' own weights are taken.
__device__ inline double rescale_exp2(float d, float c_hi, float c_lo) {
    return (double)__builtin_amdgcn_exp2f(fmaf(d, c_hi, d * c_lo));
}

template <int DT>
__device__ inline const void *row_ptr(const void *base, int64_t bstride, int64_t rstride, int s, int i) {
    return (const char *)base + ((int64_t)s * bstride + (int64_t)i * rstride) * (int64_t)elem_bytes(DT);
}

// ---------------------------------------------------------------------------
// Per-call parameters shared by every device role.

struct Ctx {
    const void *target, *draft;
    int64_t tbs, trs, dbs, drs;        // element strides
    int K, V, nseg, nres, rps;         // rps: partial rows per sequence (K+1 or 2K+1)
    const double *temps;               // per-sequence temperatures, or NULL
    double T_uniform;                  // the call's temperature when temps is NULL
    const int32_t *klen;               // per-sequence draft lengths [b], or NULL (all K)
    int row_lo, rpl;                   // row pass: partial rows row_lo .. row_lo+rpl-1 of each sequence
    int shard_id;                      // vocabulary-sharded call: this launch's shard, else -1
    int32_t col0;                      // first vocabulary column of the shard (0 unsharded)
    const float *zx;                   // sharded scan: gathered [b, K, 2] z_t(x_i), z_d(x_i), or NULL
    const int32_t *x;                  // draft tokens [b, K]
    const uint64_t *seeds;             // [b]
    int32_t *n_out, *tok;              // [b], [b, K+1]
    float *p_out, *q_out;              // [b, K] or NULL
    int32_t *am;                       // [b, K+1] or NULL
    Partial *part;                     // [b, rps, nseg]
    DrawPlan *plan;                    // [b] or NULL (greedy-only calls)
    double *rmass;                     // [b, nres] or NULL
    int32_t *rlist;                    // residual work list, or NULL: [0] the count, then the items
    uint32_t nres_m, nres_l;           // nres as a multiply-high divisor (fast_div)
};

// n / d for 0 <= n < 2^31 and d >= 1 by a multiply-high and a shift, all in
// scalar registers for wave-uniform n (the hardware has no integer divide):
// with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
// n / d = (mulhi(n, m) + n) >> l (the round-up method of Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994;
// mulhi(n, m) <= n, so the sum stays below 2^32).
inline void fast_div(uint32_t d, uint32_t &m, uint32_t &l) {
    l = 0;
    while (l < 32 && (uint64_t(1) << l) < d) ++l;
    m = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
}

__device__ inline uint32_t fdiv(uint32_t n, uint32_t m, uint32_t l) { return (__umulhi(n, m) + n) >> l; }

inline void set_nres(Ctx &c, int nres) {
    c.nres = nres;
    fast_div((uint32_t)(nres > 0 ? nres : 1), c.nres_m, c.nres_l);
}

// The residual work list: the row pass clears the count, each scan whose
// sequence rejects a slot appends a work item (ResItem, from int32 kListOff
// on), and the residual pass maps its workgroups onto the listed items only.
constexpr int kListOff = 64;

__device__ inline double seq_temperature(const Ctx &c, int s) { return c.temps ? c.temps[s] : c.T_uniform; }

// Draft length Ks of sequence s: its block is target rows 0..Ks (row Ks the
// bonus position) and draft rows 0..Ks-1.  A length outside [0, K] makes the
// sequence invalid.
__device__ inline int seq_len(const Ctx &c, int s) { return c.klen ? c.klen[s] : c.K; }

__device__ inline int seq_rule(const Ctx &c, double T, int Ks) {
    return (Ks < 0 || Ks > c.K) ? kRuleInvalid : rule_of(T);
}

// Whether partial row r (target rows 0..K, then draft rows K+1..2K) is part
// of the block of a sequence with draft length Ks.
__device__ inline bool row_in_block(int r, int K, int Ks) { return r <= K ? r <= Ks : r - (K + 1) < Ks; }

// ---------------------------------------------------------------------------
// Row pass, one wave: segment `seg` of row i of sequence s.  Greedy rows keep
// max + first argmax; sampling rows keep max + sum of exp2((z - max) c).

template <int DT, bool VEC>
__device__ inline void row_wave(const Ctx &c, int s, int i, int seg, int lane, int rule, double T) {
    const int K = c.K, V = c.V;
    const void *rowp = i <= K ? row_ptr<DT>(c.target, c.tbs, c.trs, s, i)
                              : row_ptr<DT>(c.draft, c.dbs, c.drs, s, i - K - 1);
    Partial out;
    if (rule == kRuleGreedy) {
        float mx = -INFINITY;
        int32_t ix = INT_MAX;
        bool bad = false;
        if constexpr (VEC) {
            uint4 d[kVecPerLane];
            load_vecs<DT, kVecPerLane>(rowp, (int64_t)seg * kSegVec, lane, V, d);
#pragma unroll
            for (int u = 0; u < kVecPerLane; ++u) {
                const int32_t e0 = (int32_t)(((int64_t)seg * kSegVec + u * kWave + lane) * elems_per_vec(DT));
#pragma unroll
                for (int k = 0; k < elems_per_vec(DT); ++k) {
                    const float f = vec_elem<DT>(d[u], k);
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
                const float f = elem_at<DT>(rowp, e);
                bad |= !(f < INFINITY);
                if (f > mx) {
                    mx = f;
                    ix = (int32_t)e;
                }
            }
        }
        wave_argmax(mx, ix);
        const bool any_bad = __ballot(bad) != 0ull;
        out.m = mx;
        out.idx = any_bad ? -1 : ix;
        out.S = 0.0;
    } else {
        float c_hi, c_lo;
        double c64;
        split_scale(T, c_hi, c_lo, c64);
        // Per lane: max, then the sum of exp2 at that max -- pairwise in fp32
        // inside each 16-byte vector, in double across vectors.  The lane
        // sums meet at the wave's max, rescaled by exp2 of the (non-positive)
        // max difference in fp32 with the split scale, as the elements are.
        float ml = -FLT_MAX;
        double sl = 0.0;
        if constexpr (VEC) {
            uint4 d[kVecPerLane];
            load_vecs<DT, kVecPerLane>(rowp, (int64_t)seg * kSegVec, lane, V, d);
#pragma unroll
            for (int u = 0; u < kVecPerLane; ++u)
#pragma unroll
                for (int k = 0; k < elems_per_vec(DT); ++k) ml = fmaxf(ml, vec_elem<DT>(d[u], k));
#pragma unroll
            for (int u = 0; u < kVecPerLane; ++u) {
                float e[elems_per_vec(DT)];
#pragma unroll
                for (int k = 0; k < elems_per_vec(DT); ++k) {
                    const float dz = vec_elem<DT>(d[u], k) - ml;
                    e[k] = __builtin_amdgcn_exp2f(fmaf(dz, c_hi, dz * c_lo));
                }
                sl += (double)pairwise_sum<elems_per_vec(DT)>(e);
            }
        } else {
            const int64_t e_begin = (int64_t)seg * seg_elems(DT);
            const int64_t e_end = min((int64_t)V, e_begin + seg_elems(DT));
            for (int64_t e = e_begin + lane; e < e_end; e += kWave) ml = fmaxf(ml, elem_at<DT>(rowp, e));
            for (int64_t e = e_begin + lane; e < e_end; e += kWave) {
                const float dz = elem_at<DT>(rowp, e) - ml;
                sl += (double)__builtin_amdgcn_exp2f(fmaf(dz, c_hi, dz * c_lo));
            }
        }
        const float mw = wave_max(ml);
        const float dm = ml - mw;
        out.m = mw;
        out.idx = 0;
        out.S = wave_sum(sl * rescale_exp2(dm, c_hi, c_lo));
    }
    if (lane == 0) c.part[((int64_t)s * c.rps + i) * c.nseg + seg] = out;
}

// ---------------------------------------------------------------------------
// Draw weight constants.  A draw weight is exp2 of an exponent formed from
// c = log2(e)/T (split hi + lo), an offset subtracted first and a constant,
// per row (the weights and the two forms of their exponent are defined with
// the draw, below).  DrawExp holds the offset (M, or 0 in the folded form)
// and the constant (L, or B), split hi + lo.  z - 0 is z, bit for bit, so the
// general evaluation (FOLDED = false) gives the folded form's bits too: the
// draw takes it for either form, and only the residual pass, where the two
// operations per element count, instantiates the folded one.
struct DrawExp {
    float c_hi, c_lo;
    float Mt, Et_hi, Et_lo;     // target row: offset (M, or 0 folded) and L or B, split hi + lo
    float Md, Ed_hi, Ed_lo;     // draft row (residual draws), the same
    bool fold;                  // the folded form for both rows
};

__device__ inline bool fold_split(float M, float L_hi, float L_lo, double c64, float &B_hi, float &B_lo) {
    const double B = (double)M * c64 + ((double)L_hi + (double)L_lo);
    B_hi = (float)B;
    B_lo = (float)(B - (double)B_hi);
    return fabs(B) <= 1048576.0;                    // false for NaN
}

__device__ inline DrawExp draw_exp(const DrawPlan &pl, float c_hi, float c_lo, double c64) {
    DrawExp x;
    x.c_hi = c_hi;
    x.c_lo = c_lo;
    x.fold = fold_split(pl.Mt, pl.Lt_hi, pl.Lt_lo, c64, x.Et_hi, x.Et_lo) &&
             fold_split(pl.Md, pl.Ld_hi, pl.Ld_lo, c64, x.Ed_hi, x.Ed_lo);
    if (x.fold) {
        x.Mt = 0.0f;
        x.Md = 0.0f;
    } else {
        x.Mt = pl.Mt;
        x.Md = pl.Md;
        x.Et_hi = pl.Lt_hi;
        x.Et_lo = pl.Lt_lo;
        x.Ed_hi = pl.Ld_hi;
        x.Ed_lo = pl.Ld_lo;
    }
    return x;
}

// One residual work item, written by the scan of a rejecting sequence: the
// sequence, its rejected slot and the weight constants the draw will use
// (draw_exp of its plan), as 32-bit words, so a residual wave needs one round
// trip (the count and its item, loaded together) before its row loads.
struct ResItem {
    int32_t s, slot;
    float c_hi, c_lo, Mt, Et_hi, Et_lo, Md, Ed_hi, Ed_lo;
    int32_t fold, pad;
};

__device__ inline ResItem res_item(int s, int slot, const DrawExp &x) {
    ResItem it;
    it.s = s;
    it.slot = slot;
    it.c_hi = x.c_hi;
    it.c_lo = x.c_lo;
    it.Mt = x.Mt;
    it.Et_hi = x.Et_hi;
    it.Et_lo = x.Et_lo;
    it.Md = x.Md;
    it.Ed_hi = x.Ed_hi;
    it.Ed_lo = x.Ed_lo;
    it.fold = x.fold ? 1 : 0;
    it.pad = 0;
    return it;
}

__device__ inline DrawExp res_item_exp(const ResItem &it) {
    DrawExp x;
    x.c_hi = it.c_hi;
    x.c_lo = it.c_lo;
    x.Mt = it.Mt;
    x.Et_hi = it.Et_hi;
    x.Et_lo = it.Et_lo;
    x.Md = it.Md;
    x.Ed_hi = it.Ed_hi;
    x.Ed_lo = it.Ed_lo;
    x.fold = it.fold != 0;
    return x;
}

// Every word of the item in a register before the code that follows, so the
// compiler cannot move the item's loads below the exit test (and wait for
// them in a second round trip).
__device__ __forceinline__ void res_item_ready(const ResItem &it) {
    asm volatile("" ::"s"(it.s), "s"(it.slot), "s"(it.c_hi), "s"(it.c_lo), "s"(it.Mt), "s"(it.Et_hi),
                 "s"(it.Et_lo), "s"(it.Md), "s"(it.Ed_hi), "s"(it.Ed_lo), "s"(it.fold));
}

__device__ inline const ResItem *res_items(const Ctx &c) { return (const ResItem *)(c.rlist + kListOff); }

// exp(l) of a log-probability l (double, <= 0 or -inf) as a float, in fp32
// hardware arithmetic: with a = l log2(e) = a_hi + a_lo (a_hi its float
// rounding, |a_lo| <= 2^-24 |a|), exp2(a_hi) (1 + a_lo ln 2) is within a few
// float ulps of exp(l) (the dropped term is of order a_lo^2).  Below
// 2^-200 the float is 0 either way; NaN stays NaN.
__device__ inline float exp_to_float(double l) {
    const double a = l * 1.4426950408889634;
    if (a < -200.0) return 0.0f;
    const float a_hi = (float)a;
    const float a_lo = (float)(a - (double)a_hi);
    return __builtin_amdgcn_exp2f(a_hi) * fmaf(a_lo, 0.69314718f, 1.0f);
}

// ---------------------------------------------------------------------------
// Accept scan of one sequence by one block of NW waves.  Wave w merges rows
// w, w + NW, ... (each wave's first kPre row loads issued together, before
// the temperature decides the rule); wave 0 then runs the scan.

constexpr int kPre = 4;

template <int DT, int NW>
__device__ inline void scan_seq(const Ctx &c, int s) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int K = c.K, V = c.V, nseg = c.nseg, rps = c.rps;
    const int K1 = K + 1;
    __shared__ float sM[2 * SPEC_MAX_K + 1];
    __shared__ double sS[2 * SPEC_MAX_K + 1];
    __shared__ double sL[2 * SPEC_MAX_K + 1];     // log2 S (the draw's normaliser)
    __shared__ double sLn[2 * SPEC_MAX_K + 1];    // ln S (p(x), q(x) and the accept ratio)
    __shared__ int32_t sA[SPEC_MAX_K + 1];
    __shared__ int32_t sBad;

    Partial pre[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
        pre[k].m = -FLT_MAX;
        pre[k].idx = INT_MAX;
        pre[k].S = 0.0;
        const int r = wave + k * NW;
        if (r < rps && lane < nseg) pre[k] = c.part[((int64_t)s * rps + r) * nseg + lane];
    }
    const double T = seq_temperature(c, s);
    const int Ks = seq_len(c, s);
    const int rule = seq_rule(c, T, Ks);
    int32_t *tok = c.tok + (int64_t)s * K1;

    if (rule == kRuleInvalid) {
        if (wave != 0) return;
        if (lane < K1) {
            tok[lane] = -1;
            if (c.am) c.am[(int64_t)s * K1 + lane] = -1;
        }
        if (lane < K) {
            if (c.p_out) c.p_out[(int64_t)s * K + lane] = NAN;
            if (c.q_out) c.q_out[(int64_t)s * K + lane] = NAN;
        }
        if (lane == 0) {
            c.n_out[s] = -1;
            if (c.plan) {
                DrawPlan pl = {};
                pl.mode = kModeNone;
                c.plan[s] = pl;
            }
        }
        return;
    }

    if (threadIdx.x == 0) sBad = 0;
    __syncthreads();

    // Wave 0 reads the draft tokens (and, sampling, gathers z[x_i]) while the
    // other waves merge.
    int32_t x = 0;
    bool tok_bad = false;
    float zt = 0.0f, zd = 0.0f;
    if (wave == 0 && lane < Ks) {
        x = c.x[(int64_t)s * K + lane];
        tok_bad = x < 0 || x >= V;
        if (rule == kRuleSample && !tok_bad) {
            if (c.zx) {
                zt = c.zx[((int64_t)s * K + lane) * 2];
                zd = c.zx[((int64_t)s * K + lane) * 2 + 1];
            } else {
                zt = elem_at<DT>(row_ptr<DT>(c.target, c.tbs, c.trs, s, lane), x);
                zd = elem_at<DT>(row_ptr<DT>(c.draft, c.dbs, c.drs, s, lane), x);
            }
        }
    }

    if (rule == kRuleGreedy) {
        // Row i: (max, lowest argmax) over ascending segments, the first
        // segment of this lane from `first` when it was preloaded.
        auto merge_row = [&](int i, const Partial *first) {
            const Partial *pr = c.part + ((int64_t)s * rps + i) * nseg;
            float m = -INFINITY;
            int32_t idx = INT_MAX;
            bool bad = false;
            auto take = [&](const Partial &p) {
                if (p.idx < 0) bad = true;
                else if (p.m > m) {
                    m = p.m;
                    idx = p.idx;
                }
            };
            int j = lane;
            if (first) {
                if (j < nseg) take(*first);
                j += kWave;
            }
            for (; j < nseg; j += kWave) take(pr[j]);
            wave_argmax(m, idx);
            const bool any_bad = __ballot(bad) != 0ull;
            if (lane == 0) {
                sA[i] = idx;
                if (any_bad || !(m > -INFINITY)) sBad = 1;
            }
        };
#pragma unroll
        for (int k = 0; k < kPre; ++k)
            if (wave + k * NW <= Ks) merge_row(wave + k * NW, &pre[k]);
        for (int i = wave + kPre * NW; i <= Ks; i += NW) merge_row(i, nullptr);
        __syncthreads();
        if (wave != 0) return;
        const bool invalid = sBad || (__ballot(tok_bad) != 0ull);
        if (lane < K) {
            if (c.p_out) c.p_out[(int64_t)s * K + lane] = NAN;
            if (c.q_out) c.q_out[(int64_t)s * K + lane] = NAN;
        }
        if (lane == 0 && c.plan) {
            DrawPlan pl = {};
            pl.mode = kModeNone;
            c.plan[s] = pl;
        }
        if (invalid) {
            if (lane < K1) {
                tok[lane] = -1;
                if (c.am) c.am[(int64_t)s * K1 + lane] = -1;
            }
            if (lane == 0) c.n_out[s] = -1;
            return;
        }
        const bool mismatch = lane < Ks && x != sA[lane];
        const unsigned long long mm = __ballot(mismatch);
        const int n = mm ? (int)__ffsll((long long)mm) - 1 : Ks;
        if (lane < K1) {
            tok[lane] = lane < n ? x : lane == n ? sA[n] : -1;
            if (c.am) c.am[(int64_t)s * K1 + lane] = lane <= Ks ? sA[lane] : -1;
        }
        if (lane == 0) c.n_out[s] = n;
        return;
    }

    // Sampling.  Wave 0 draws the uniforms first, while the segment records
    // are still in flight: lane i holds U(seed, s, i, 0), the accept test of
    // slot i, and U(seed, s, i, 1), the draw if slot i is the one drawn.
    // 1/T too, so that after the barrier the log-probabilities take products.
    double u_acc = 0.0, u_draw = 0.0, inv_T = 0.0;
    if (wave == 0 && lane < K1) {
        const uint64_t seed = c.seeds[s];
        u_acc = philox_uniform(seed, (uint32_t)s, (uint32_t)lane, 0u);
        u_draw = philox_uniform(seed, (uint32_t)s, (uint32_t)lane, 1u);
        inv_T = 1.0 / T;
    }

    // Log-normalisers of the 2K+1 rows.
    const int R = 2 * K + 1;
    float c_hi, c_lo;
    double c64;
    split_scale(T, c_hi, c_lo, c64);
    // Row r: M = max of the segment maxima, S = sum of the segment sums
    // rescaled to M (double), the first segment of this lane from `first`.
    auto merge_row = [&](int r, const Partial *first) {
        const Partial *pr = c.part + ((int64_t)s * rps + r) * nseg;
        float m = -FLT_MAX;
        int j = lane;
        if (first) {
            if (j < nseg) m = fmaxf(m, first->m);
            j += kWave;
        }
        for (; j < nseg; j += kWave) m = fmaxf(m, pr[j].m);
        const float M = wave_max(m);
        double acc = 0.0;
        j = lane;
        if (first) {
            if (j < nseg) acc += first->S * rescale_exp2(first->m - M, c_hi, c_lo);
            j += kWave;
        }
        for (; j < nseg; j += kWave) {
            const Partial p = pr[j];
            acc += p.S * rescale_exp2(p.m - M, c_hi, c_lo);
        }
        const double S = wave_sum(acc);                 // the same bits in every lane
        if (lane == 0) {
            sM[r] = M;
            sS[r] = S;
            sL[r] = log2(S);
            if (!(S > 0.0) || !(S < INFINITY)) sBad = 1;   // NaN/+inf seen, or no finite entry
        } else if (lane == 1) {
            sLn[r] = log(S);
        }
    };
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
        const int r = wave + k * NW;
        if (r < R && row_in_block(r, K, Ks)) merge_row(r, &pre[k]);
    }
    for (int r = wave + kPre * NW; r < R; r += NW)
        if (row_in_block(r, K, Ks)) merge_row(r, nullptr);
    __syncthreads();
    if (wave != 0) return;

    if (c.am && lane < K1) c.am[(int64_t)s * K1 + lane] = -1;
    const bool invalid = sBad || (__ballot(tok_bad) != 0ull);
    if (invalid) {
        if (lane < K1) tok[lane] = -1;
        if (lane < K) {
            if (c.p_out) c.p_out[(int64_t)s * K + lane] = NAN;
            if (c.q_out) c.q_out[(int64_t)s * K + lane] = NAN;
        }
        if (lane == 0) {
            DrawPlan pl = {};
            pl.mode = kModeNone;
            c.plan[s] = pl;
            c.n_out[s] = -1;
        }
        return;
    }
    bool reject = false;
    if (lane < Ks) {
        const double lp = ((double)zt - (double)sM[lane]) * inv_T - sLn[lane];
        const double lq = ((double)zd - (double)sM[K1 + lane]) * inv_T - sLn[K1 + lane];
        double r;
        if (zt == -INFINITY) r = 0.0;                 // p(x) = 0: never accepted
        else if (zd == -INFINITY) r = INFINITY;       // q(x) = 0 < p(x): always accepted
        else r = exp(lp - lq);
        reject = !(u_acc < r);                        // u < 1, so u < r == u < min(1, r)
        if (c.p_out) c.p_out[(int64_t)s * K + lane] = exp_to_float(lp);
        if (c.q_out) c.q_out[(int64_t)s * K + lane] = exp_to_float(lq);
    } else if (lane < K) {                            // slots past the block
        if (c.p_out) c.p_out[(int64_t)s * K + lane] = NAN;
        if (c.q_out) c.q_out[(int64_t)s * K + lane] = NAN;
    }
    const unsigned long long rj = __ballot(reject);
    const int n = rj ? (int)__ffsll((long long)rj) - 1 : Ks;
    // A rejecting sequence takes its place in the residual work list now, so
    // the atomic's round trip overlaps the rest.
    int listed = -1;
    if (lane == 0 && n < Ks && c.rlist) listed = atomicAdd(c.rlist, 1);
    const double u2 = __shfl(u_draw, n, kWave);
    if (lane < K1) tok[lane] = lane < n ? x : -1;     // slot n is filled by the draw
    if (lane == 0) {
        c.n_out[s] = n;
        DrawPlan pl;
        pl.mode = n < Ks ? kModeResidual : kModeTarget;
        pl.slot = n;
        pl.u2 = u2;
        pl.T = T;
        const double St = sS[n];
        const double Lt = sL[n];
        pl.Mt = sM[n];
        pl.St = St;
        pl.Lt_hi = (float)Lt;
        pl.Lt_lo = (float)(Lt - (double)pl.Lt_hi);
        if (n < Ks) {
            const double Ld = sL[K1 + n];
            pl.Md = sM[K1 + n];
            pl.Ld_hi = (float)Ld;
            pl.Ld_lo = (float)(Ld - (double)pl.Ld_hi);
        } else {
            pl.Md = 0.0f;
            pl.Ld_hi = 0.0f;
            pl.Ld_lo = 0.0f;
        }
        c.plan[s] = pl;
        if (listed >= 0)   // the draw's own constants, bit for bit
            ((ResItem *)(c.rlist + kListOff))[listed] = res_item(s, n, draw_exp(pl, c_hi, c_lo, c64));
    }
}

// ---------------------------------------------------------------------------
// Draw weights.  p(v) = exp2((z - M) * c - L) with c = log2(e)/T and
// L = log2 S.  With B = M*c + L the exponent is z*c - B, evaluated as
// fma(z, c_hi, -B_hi) + fma(z, c_lo, -B_lo) (B split hi + lo like c): each
// product is exact inside its fma and the large terms cancel inside one
// rounding, so the exponent carries the error of its last two roundings, as
// with the difference z - M formed first, in two fewer operations per
// element.  The low parts' own rounding is 2^-48 |B| absolute, so this
// folded form is taken while |B| <= 2^20 (below 2^-28); past that (tiny T or
// huge logits) the exponent is fma(z - M, c_hi, -L_hi) + fma(z - M, c_lo,
// -L_lo).  A -inf logit gives -inf in both products (c_hi, c_lo > 0), hence
// weight 0.  The residual pass and the draw build the constants from the same
// plan with the same code (draw_exp), so a weight has the same bits in both.

// FOLDED = true only where x.fold holds.
template <bool FOLDED>
__device__ inline float target_weight(float zt, const DrawExp &x) {
    const float z = FOLDED ? zt : zt - x.Mt;
    return __builtin_amdgcn_exp2f(fmaf(z, x.c_hi, -x.Et_hi) + fmaf(z, x.c_lo, -x.Et_lo));
}

template <bool FOLDED>
__device__ inline float residual_weight(float zt, float zd, const DrawExp &x) {
    const float z = FOLDED ? zd : zd - x.Md;
    const float q = __builtin_amdgcn_exp2f(fmaf(z, x.c_hi, -x.Ed_hi) + fmaf(z, x.c_lo, -x.Ed_lo));
    const float w = target_weight<FOLDED>(zt, x) - q;
    return w > 0.0f ? w : 0.0f;
}

// Sum of the residual weights of one 4 KiB-per-row segment, this lane's share.
template <int DT, bool VEC, bool FOLDED>
__device__ inline double residual_lane_sum(const void *tp, const void *dp, int seg, int V, const DrawExp &x,
                                           int lane) {
    double acc = 0.0;
    const int64_t vbase = (int64_t)seg * kResSegVec;
    if (VEC && vbase + kResSegVec <= (int64_t)V / elems_per_vec(DT)) {
        // The whole segment lies inside the row (the same for every lane).
        // Loads and arithmetic sit in one block, so the arithmetic on vector u
        // waits only for the loads of vector u.  Plain (temporal) loads here:
        // with non-temporal ones the next row pass measured about 3 us
        // slower, against 0.7 us more for this pass.
        const uint4 *ta = (const uint4 *)tp + vbase + lane, *db = (const uint4 *)dp + vbase + lane;
        uint4 a[kResVecPerLane], b[kResVecPerLane];
#pragma unroll
        for (int u = 0; u < kResVecPerLane; ++u) {
            a[u] = ta[u * kWave];
            b[u] = db[u * kWave];
        }
#pragma unroll
        for (int u = 0; u < kResVecPerLane; ++u) {
            float w[elems_per_vec(DT)];
#pragma unroll
            for (int k = 0; k < elems_per_vec(DT); ++k)
                w[k] = residual_weight<FOLDED>(vec_elem<DT>(a[u], k), vec_elem<DT>(b[u], k), x);
            acc += (double)pairwise_sum<elems_per_vec(DT)>(w);
        }
    } else {
        // The row's last segment when it is partial, or rows not on 16-byte
        // boundaries: element by element.
        const int64_t e_begin = (int64_t)seg * rseg_elems(DT);
        const int64_t e_end = min((int64_t)V, e_begin + rseg_elems(DT));
        for (int64_t e = e_begin + lane; e < e_end; e += kWave)
            acc += (double)residual_weight<FOLDED>(elem_at<DT>(tp, e), elem_at<DT>(dp, e), x);
    }
    return acc;
}

// Residual mass of segment `seg` of sequence s's rejected row pair (slot),
// one wave.
template <int DT, bool VEC>
__device__ inline void residual_seg(const Ctx &c, int s, int slot, const DrawExp &x, int seg, int lane) {
    const void *tp = row_ptr<DT>(c.target, c.tbs, c.trs, s, slot);
    const void *dp = row_ptr<DT>(c.draft, c.dbs, c.drs, s, slot);
    const double acc = x.fold ? residual_lane_sum<DT, VEC, true>(tp, dp, seg, c.V, x, lane)
                              : residual_lane_sum<DT, VEC, false>(tp, dp, seg, c.V, x, lane);
    const double Sw = wave_sum(acc);
    if (lane == 0) c.rmass[(int64_t)s * c.nres + seg] = Sw;
}

// The same from sequence s's plan (the vocabulary-sharded residual pass).
template <int DT, bool VEC>
__device__ inline void residual_wave(const Ctx &c, int s, int seg, int lane) {
    const DrawPlan pl = c.plan[s];
    if (pl.mode != kModeResidual) return;
    float c_hi, c_lo;
    double c64;
    split_scale(pl.T, c_hi, c_lo, c64);
    residual_seg<DT, VEC>(c, s, pl.slot, draw_exp(pl, c_hi, c_lo, c64), seg, lane);
}

// Inverse-CDF search inside one segment [e_seg0, e_seg0 + 256*E) of the
// drawn row: thread t holds elements e_seg0 + t*E .. + E - 1 in registers.
// Writes the drawn index to *sY (or the segment's last positive weight to
// *sLastPos when tl sits at or past the segment's recomputed total).
template <int DT, bool VEC, int E, bool RESID>
__device__ inline void search_segment(const void *tp, const void *dp, int64_t e_seg0, int V, const DrawExp &x,
                                      double tl, double *sw, int32_t *sY, int32_t *sLastPos) {
    constexpr int EPV = elems_per_vec(DT);
    const int64_t e0 = e_seg0 + (int64_t)threadIdx.x * E;
    float w[E];
    if (VEC && E % EPV == 0 && e0 + E <= V) {
        constexpr int NV = E / EPV;
        uint4 a[NV];
#pragma unroll
        for (int u = 0; u < NV; ++u) a[u] = ((const uint4 *)tp)[e0 / EPV + u];
        if constexpr (RESID) {
            uint4 b[NV];
#pragma unroll
            for (int u = 0; u < NV; ++u) b[u] = ((const uint4 *)dp)[e0 / EPV + u];
#pragma unroll
            for (int u = 0; u < NV; ++u)
#pragma unroll
                for (int k = 0; k < EPV; ++k)
                    w[u * EPV + k] = residual_weight<false>(vec_elem<DT>(a[u], k), vec_elem<DT>(b[u], k), x);
        } else {
#pragma unroll
            for (int u = 0; u < NV; ++u)
#pragma unroll
                for (int k = 0; k < EPV; ++k) w[u * EPV + k] = target_weight<false>(vec_elem<DT>(a[u], k), x);
        }
    } else {
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int64_t e = e0 + k;
            float wk = 0.0f;
            if (e < V) {
                if constexpr (RESID) wk = residual_weight<false>(elem_at<DT>(tp, e), elem_at<DT>(dp, e), x);
                else wk = target_weight<false>(elem_at<DT>(tp, e), x);
            }
            w[k] = wk;
        }
    }
    double tsum = 0.0;
    int32_t lastpos = -1;
#pragma unroll
    for (int k = 0; k < E; ++k) {
        tsum += (double)w[k];
        if (w[k] > 0.0f) lastpos = (int32_t)(e0 + k);
    }
    double wex, win, segtotal;
    block_scan(tsum, wex, win, segtotal, sw);
    if (!(tl < segtotal)) {
        if (lastpos >= 0) atomicMax(sLastPos, lastpos);
    } else if (wex <= tl && tl < win) {
        double run = wex;
        int32_t y = lastpos;                           // rounding fallback
#pragma unroll
        for (int k = 0; k < E; ++k) {
            run += (double)w[k];
            if (run > tl) {
                y = (int32_t)(e0 + k);
                break;
            }
        }
        *sY = y;
    }
}

// Draw the token of slot n of sequence s (one 256-thread block): inverse CDF
// over ascending vocabulary index of the residual (mode residual, residual
// segments) or of p_n (mode target, row-pass segments: the bonus, or a
// rejected slot whose residual mass is zero).  `pl` is the sequence's plan,
// `tpart` the segment records of its slot n (global memory or LDS), `rm` its
// residual masses with this thread's first one preloaded in `rm_first` (both
// unused without a residual draw).
template <int DT, bool VEC>
__device__ inline void draw_core(const Ctx &c, int s, const DrawPlan &pl, const Partial *tpart, const double *rm,
                                 double rm_first) {
    const int t = threadIdx.x;
    const int K = c.K, V = c.V, nseg = c.nseg, nres = c.nres;
    __shared__ double sw[kWavesPerBlock];
    __shared__ int32_t sSeg;
    __shared__ double sOff;
    __shared__ int32_t sY;
    __shared__ int32_t sLastPos;

    const int rper = (nres + kBlock - 1) / kBlock;
    const int r0 = min(nres, t * rper);
    if (pl.mode == kModeNone) return;
    const bool sharded = c.shard_id >= 0;
    if (sharded && pl.shard != c.shard_id) return;
    float c_hi, c_lo;
    double c64;
    split_scale(pl.T, c_hi, c_lo, c64);
    bool resid = pl.mode == kModeResidual;

    // (a) segment masses: thread t sums a contiguous range of segments.
    auto seg_mass = [&](int j) -> double {
        return resid ? rm[j] : tpart[j].S * rescale_exp2(tpart[j].m - pl.Mt, c_hi, c_lo) / pl.St;
    };
    int nsg = resid ? nres : nseg;
    int per = (nsg + kBlock - 1) / kBlock;
    int j0 = min(nsg, t * per), j1 = min(nsg, j0 + per);
    // The thread's first mass is kept for (b), so the common case (one
    // segment per thread) reads no mass twice.
    double local = 0.0, m_first = 0.0, excl, incl, total;
    for (int j = j0; j < j1; ++j) {
        const double mj = (resid && j == r0) ? rm_first : seg_mass(j);
        if (j == j0) m_first = mj;
        local += mj;
    }
    block_scan(local, excl, incl, total, sw);
    if (!sharded && resid && !(total > 0.0)) {         // zero residual mass: draw from p_n
        resid = false;
        nsg = nseg;
        per = (nsg + kBlock - 1) / kBlock;
        j0 = min(nsg, t * per);
        j1 = min(nsg, j0 + per);
        local = 0.0;
        for (int j = j0; j < j1; ++j) {
            const double mj = seg_mass(j);
            if (j == j0) m_first = mj;
            local += mj;
        }
        block_scan(local, excl, incl, total, sw);
    }
    // u2 < 1: tt < total when total > 0.  A shard draws at the mass the shard
    // selection left inside it, kept below this shard's own total.
    const double tt = sharded ? fmin(pl.t_local, nextafter(total, 0.0)) : pl.u2 * total;
    if (t == 0) {
        sSeg = 0;
        sOff = 0.0;
        sY = -1;
        sLastPos = -1;
    }
    __syncthreads();
    // (b) the segment holding tt: exactly one thread has excl <= tt < incl.
    if (excl <= tt && tt < incl) {
        double run = excl;
        int sel = -1, last = -1;
        double sel_off = 0.0, last_off = 0.0;
        for (int j = j0; j < j1; ++j) {
            const double mj = j == j0 ? m_first : seg_mass(j);
            if (mj > 0.0) {
                last = j;
                last_off = run;
            }
            if (run + mj > tt) {
                sel = j;
                sel_off = run;
                break;
            }
            run += mj;
        }
        if (sel < 0) {                                 // rounding: the range's last mass
            sel = last < 0 ? j0 : last;
            sel_off = last_off;
        }
        sSeg = sel;
        sOff = sel_off;
    }
    __syncthreads();
    const int seg = sSeg;
    const double tl = fmax(0.0, tt - sOff);

    // (c) re-read the segment and search it.
    const void *tp = row_ptr<DT>(c.target, c.tbs, c.trs, s, pl.slot);
    const DrawExp x = draw_exp(pl, c_hi, c_lo, c64);
    if (resid) {
        const void *dp = row_ptr<DT>(c.draft, c.dbs, c.drs, s, pl.slot);
        search_segment<DT, VEC, (int)(rseg_elems(DT) / kBlock), true>(
            tp, dp, (int64_t)seg * rseg_elems(DT), V, x, tl, sw, &sY, &sLastPos);
    } else {
        search_segment<DT, VEC, (int)(seg_elems(DT) / kBlock), false>(
            tp, tp, (int64_t)seg * seg_elems(DT), V, x, tl, sw, &sY, &sLastPos);
    }
    __syncthreads();
    if (t == 0) {
        int32_t y = sY >= 0 ? sY : sLastPos;
        if (y < 0) y = (int32_t)min((int64_t)V - 1, (int64_t)seg * (resid ? rseg_elems(DT) : seg_elems(DT)));
        c.tok[(int64_t)s * (K + 1) + pl.slot] = y + c.col0;
    }
}

// Every field of a plan in registers before the code that follows, so the
// compiler cannot load the fields after the early-exit tests on the mode and
// the shard (three dependent round trips instead of one).
__device__ __forceinline__ void plan_ready(const DrawPlan &pl) {
    asm volatile("" ::"s"(pl.mode), "s"(pl.slot), "s"(pl.u2), "s"(pl.T), "s"(pl.Mt), "s"(pl.Md), "s"(pl.Lt_hi),
                 "s"(pl.Lt_lo), "s"(pl.Ld_hi), "s"(pl.Ld_lo), "s"(pl.St), "s"(pl.shard), "s"(pl.t_local));
}

// The draw of sequence s from the plan and records in the workspace.
template <int DT, bool VEC>
__device__ inline void draw_seq(const Ctx &c, int s) {
    // The residual masses of this thread's range are loaded together with the
    // plan (their address does not depend on it); unused when the plan says
    // otherwise.
    const int nres = c.nres;
    const double *rm = c.rmass + (int64_t)s * nres;
    const int rper = (nres + kBlock - 1) / kBlock;
    const int r0 = min(nres, (int)threadIdx.x * rper);
    const double rm_first = r0 < min(nres, r0 + rper) ? rm[r0] : 0.0;
    const DrawPlan pl = c.plan[s];
    plan_ready(pl);
    draw_core<DT, VEC>(c, s, pl, c.part + ((int64_t)s * c.rps + pl.slot) * c.nseg, rm, rm_first);
}

// ---------------------------------------------------------------------------
// Kernels.

// Row pass: one single-wave workgroup per (row of the call, segment), rows
// taken sequence by sequence, rps per sequence.  Draft rows of greedy
// sequences, rows past a sequence's draft length and rows of invalid
// sequences are skipped.  (Single-wave
// workgroups stream measurably faster on this part than 4-wave ones: a wave
// starts as soon as one wave's resources free up.)
template <int DT, bool VEC>
__device__ inline void row_pass_block(const Ctx &c, int blk, int lane) {
    // (the same in every lane: scalar loads and pointer arithmetic follow)
    const int row = __builtin_amdgcn_readfirstlane(blk / c.nseg);
    const int seg = blk - row * c.nseg;
    const int s = __builtin_amdgcn_readfirstlane(row / c.rpl), i = c.row_lo + (row - s * c.rpl);
    const double T = seq_temperature(c, s);
    const int Ks = seq_len(c, s);
    const int rule = seq_rule(c, T, Ks);
    if (rule == kRuleInvalid || (rule == kRuleGreedy && i > c.K) || !row_in_block(i, c.K, Ks)) return;
    row_wave<DT, VEC>(c, s, i, seg, lane, rule, T);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kWave) void row_pass(Ctx c) {
    if (c.rlist && blockIdx.x == 0 && threadIdx.x == 0) c.rlist[0] = 0;
    row_pass_block<DT, VEC>(c, (int)blockIdx.x, (int)threadIdx.x);
}

// Row pass of a call with per-sequence draft lengths, over the rows that are
// part of their sequence's block only (a row past the block costs nothing,
// where the plain row pass spends a workgroup on it): a fixed grid of waves,
// wave w taking work items w, w + grid, ...  The rows are
// listed sequence by sequence (target rows 0..Ks, then, sampling, draft rows
// 0..Ks-1); item k is segment k % nseg of listed row k / nseg.  Lane l holds
// the first listed row of sequences l + 64 j, so a wave finds an item's
// sequence with ballots; the sequences' lengths, rules and temperatures sit
// in LDS.  Three waves per SIMD, as the plain row pass runs.
constexpr int kListedSeqPerLane = 4;
constexpr int kListedMaxB = kWave * kListedSeqPerLane;

template <int DT, bool VEC>
__global__ __launch_bounds__(kWave, 3) void row_pass_listed(Ctx c, int b) {
    __shared__ int32_t sFirst[kListedMaxB], sKs[kListedMaxB], sRule[kListedMaxB];
    __shared__ double sT[kListedMaxB];
    const int lane = threadIdx.x;
    if (c.rlist && blockIdx.x == 0 && lane == 0) c.rlist[0] = 0;
    int first[kListedSeqPerLane];
    int total = 0;
#pragma unroll
    for (int j = 0; j < kListedSeqPerLane; ++j) {
        const int s = lane + j * kWave;
        int rows = 0;
        if (s < b) {
            const double T = seq_temperature(c, s);
            const int Ks = seq_len(c, s);
            const int rule = seq_rule(c, T, Ks);
            rows = rule == kRuleInvalid ? 0 : rule == kRuleGreedy ? Ks + 1 : 2 * Ks + 1;
            sT[s] = T;
            sKs[s] = Ks;
            sRule[s] = rule;
        }
        int incl = rows;                                // inclusive prefix over the lanes
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int y = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += y;
        }
        first[j] = total + incl - rows;
        if (s < b) sFirst[s] = first[j];
        total += __shfl(incl, kWave - 1, kWave);
    }
    __syncthreads();
    const int nseg = c.nseg;
    const int items = total * nseg;                    // at most the full grid, checked on the host
    for (int k = (int)blockIdx.x; k < items; k += (int)gridDim.x) {
        const int r = __builtin_amdgcn_readfirstlane(k / nseg);
        const int seg = k - r * nseg;
        // the item's sequence: the last one whose first listed row is <= r
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < kListedSeqPerLane; ++j)
            cnt += __popcll(__ballot(lane + j * kWave < b && first[j] <= r));
        const int s = cnt - 1;
        // LDS reads land in vector registers; the values are the same in
        // every lane, and saying so keeps the rule's branch uniform.
        const int Ks = __builtin_amdgcn_readfirstlane(sKs[s]);
        const int rule = __builtin_amdgcn_readfirstlane(sRule[s]);
        const int li = r - __builtin_amdgcn_readfirstlane(sFirst[s]);   // listed row of the sequence
        const int i = __builtin_amdgcn_readfirstlane(li <= Ks ? li : c.K + 1 + (li - Ks - 1));
        const uint64_t tb = (uint64_t)__double_as_longlong(sT[s]);
        const double T = __longlong_as_double((long long)(
            (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)tb) |
            ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(tb >> 32)) << 32)));
        row_wave<DT, VEC>(c, s, i, seg, lane, rule, T);
    }
}

// Scan of every sequence of the call: one 1024-thread block per sequence.
template <int DT>
__global__ __launch_bounds__(kScanBlock) void scan_kernel(Ctx c) {
    scan_seq<DT, kScanBlock / kWave>(c, blockIdx.x);
}

// Residual pass: one single-wave workgroup per (work item, residual
// segment).  The grid covers every sequence; workgroups past the listed
// items come last and return at once.
template <int DT, bool VEC>
__global__ __launch_bounds__(kWave) void residual_kernel(Ctx c) {
    const int item = (int)fdiv(blockIdx.x, c.nres_m, c.nres_l);
    // The count and the item are read together (item < b: inside the list;
    // past the count it holds stale bytes, never used).
    const int count = c.rlist[0];
    const ResItem it = res_items(c)[item];
    res_item_ready(it);
    if (item >= count) return;
    residual_seg<DT, VEC>(c, it.s, it.slot, res_item_exp(it), (int)blockIdx.x - item * c.nres, threadIdx.x);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void draw_kernel(Ctx c) {
    draw_seq<DT, VEC>(c, blockIdx.x);
}

// ---------------------------------------------------------------------------
// The uniforms of the accept and draw steps on a grid of counters, for
// checking the device Philox against an independent one:
// out[r * npos + p] = U(seed, row0 + r, pos0 + p, tag), counters wrapping mod 2^32.

__global__ __launch_bounds__(kBlock) void philox_grid_kernel(uint64_t seed, uint32_t row0, int nrow, uint32_t pos0,
                                                             int npos, uint32_t tag, double *out) {
    const int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (k >= (int64_t)nrow * npos) return;
    const int r = (int)(k / npos), p = (int)(k - (int64_t)r * npos);
    out[k] = philox_uniform(seed, row0 + (uint32_t)r, pos0 + (uint32_t)p, tag);
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
        if (vi < nvec) d[u] = load_stream(src + vi);
    }
#pragma unroll
    for (int u = 0; u < kVecPerLane; ++u) {
        int64_t vi = base + u * kBlock + threadIdx.x;
        if (vi < nvec) dst[vi] = d[u];
    }
}

// Read-only stream with the row pass's shape (one wave per 16 KiB, 16
// nontemporal 16-byte loads per lane issued together): the achievable read
// bandwidth.  The loaded words are folded together and written only if they
// equal a value no real data gives, so the loads cannot be dropped.
__global__ __launch_bounds__(kWave) void stream_read_kernel(const uint4 *__restrict__ src, int64_t nvec,
                                                            uint32_t *sink) {
    const int64_t base = (int64_t)blockIdx.x * kSegVec;
    uint4 d[kVecPerLane];
#pragma unroll
    for (int u = 0; u < kVecPerLane; ++u) {
        const int64_t vi = base + u * kWave + threadIdx.x;
        d[u] = vi < nvec ? load_stream(src + vi) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t x = 0u;
#pragma unroll
    for (int u = 0; u < kVecPerLane; ++u) x ^= d[u].x ^ d[u].y ^ d[u].z ^ d[u].w;
    if (x == 0x9E3779B9u && threadIdx.x == 63) sink[0] = x;
}

// ---------------------------------------------------------------------------
// Host side.

thread_local hipEvent_t *t_stage_events = nullptr;
thread_local int t_stage_n = 0;

// Profiling marks never fail a call: an event-record error is cleared here so
// it cannot surface at the next launch check.
inline void stage_mark(int k, hipStream_t st) {
    if (t_stage_events && k < t_stage_n) {
        if (hipEventRecord(t_stage_events[k], st) != hipSuccess) (void)hipGetLastError();
    }
}

enum : int { kCallGreedy = 0, kCallSample = 1, kCallMixed = 2 };

struct Layout {
    int nseg, nres, rps;
    size_t part_off, plan_off, rmass_off, rlist_off, total;
};

bool make_layout(int b, int K, int V, int dtype, int kind, Layout &L) {
    if (b < 1 || K < 1 || K > SPEC_MAX_K || V < 1 || V > INT_MAX - 65536) return false;
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return false;
    if (kind != kCallGreedy && kind != kCallSample && kind != kCallMixed) return false;
    L.nseg = (int)(((int64_t)V + seg_elems(dtype) - 1) / seg_elems(dtype));
    L.nres = (int)(((int64_t)V + rseg_elems(dtype) - 1) / rseg_elems(dtype));
    L.rps = kind == kCallGreedy ? K + 1 : 2 * K + 1;
    const bool draws = kind != kCallGreedy;
    L.part_off = 0;
    L.plan_off = L.part_off + align256((size_t)b * L.rps * (size_t)L.nseg * sizeof(Partial));
    L.rmass_off = L.plan_off + (draws ? align256((size_t)b * sizeof(DrawPlan)) : 0);
    L.rlist_off = L.rmass_off + (draws ? align256((size_t)b * (size_t)L.nres * sizeof(double)) : 0);
    L.total = L.rlist_off + (draws ? align256(kListOff * sizeof(int32_t) + (size_t)b * sizeof(ResItem)) : 0);
    return true;
}

bool rows_vector_aligned(const void *p, int es, int64_t bs, int64_t rs) {
    return ((uintptr_t)p % 16 == 0) && ((bs * es) % 16 == 0) && ((rs * es) % 16 == 0);
}

#include "lm_head_fused.inc"

int device_cu_count();

// Grid of row_pass_listed<DT, VEC>: four times the waves the device holds at
// once, so each wave takes a few items (measured fastest against one and two
// times, where waves live longer, and eight, where each wave's table is built
// for about one item); 0 if unknown.  Read once per device.
template <int DT, bool VEC>
int listed_grid() {
    static std::atomic<int> cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        const int g = cached[dev].load(std::memory_order_relaxed);
        if (g > 0) return g;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, row_pass_listed<DT, VEC>, kWave, 0) != hipSuccess)
        return 0;
    const int g = 4 * per_cu * device_cu_count();
    if (g > 0 && dev < 64) cached[dev].store(g, std::memory_order_relaxed);
    return g;
}

template <int DT, bool VEC>
int launch(const Ctx &c, int b, int kind, const Layout &L, hipStream_t st) {
    const int64_t grid_rows = (int64_t)b * c.rpl * L.nseg;
    const int64_t grid_res = (int64_t)b * L.nres;
    if (grid_rows > INT_MAX || grid_res > INT_MAX) return SPEC_EINVAL;
    stage_mark(0, st);
    int listed = (c.klen && b <= kListedMaxB) ? listed_grid<DT, VEC>() : 0;
    if (grid_rows > (int64_t)INT_MAX - listed) listed = 0;    // the item loop counts in int
    if (listed > 0)
        hipLaunchKernelGGL((row_pass_listed<DT, VEC>), dim3((unsigned)min((int64_t)listed, grid_rows)), dim3(kWave),
                           0, st, c, b);
    else
        hipLaunchKernelGGL((row_pass<DT, VEC>), dim3((unsigned)grid_rows), dim3(kWave), 0, st, c);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(1, st);
    hipLaunchKernelGGL((scan_kernel<DT>), dim3((unsigned)b), dim3(kScanBlock), 0, st, c);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(2, st);
    if (kind == kCallGreedy) return SPEC_OK;
    hipLaunchKernelGGL((residual_kernel<DT, VEC>), dim3((unsigned)grid_res), dim3(kWave), 0, st, c);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(3, st);
    hipLaunchKernelGGL((draw_kernel<DT, VEC>), dim3((unsigned)b), dim3(kBlock), 0, st, c);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(4, st);
    return SPEC_OK;
}

// Fills the workspace pointers of `c` and launches the call's kernels.
int dispatch(Ctx c, int b, void *workspace, int dtype, int kind, const Layout &L, hipStream_t st) {
    char *ws = (char *)workspace;
    c.nseg = L.nseg;
    set_nres(c, L.nres);
    c.rps = L.rps;
    c.row_lo = 0;
    c.rpl = L.rps;
    c.shard_id = -1;
    c.col0 = 0;
    c.zx = nullptr;
    c.part = (Partial *)(ws + L.part_off);
    const bool draws = kind != kCallGreedy;
    c.plan = draws ? (DrawPlan *)(ws + L.plan_off) : nullptr;
    c.rmass = draws ? (double *)(ws + L.rmass_off) : nullptr;
    c.rlist = draws ? (int32_t *)(ws + L.rlist_off) : nullptr;
    const int es = elem_bytes(dtype);
    bool vec = rows_vector_aligned(c.target, es, c.tbs, c.trs);
    if (kind != kCallGreedy) vec = vec && rows_vector_aligned(c.draft, es, c.dbs, c.drs);
    if (dtype == SPEC_BF16)
        return vec ? launch<SPEC_BF16, true>(c, b, kind, L, st) : launch<SPEC_BF16, false>(c, b, kind, L, st);
    return vec ? launch<SPEC_F32, true>(c, b, kind, L, st) : launch<SPEC_F32, false>(c, b, kind, L, st);
}

// ---------------------------------------------------------------------------
// Fused verify: workspace layout and launch sequence.

struct FusedLayout {
    Layout L;                 // the fp32 mixed-call layout (partials, plans, residual masses)
    int ntiles, tiles_h;
    int64_t lrs;              // logits row stride (elements, a multiple of 64)
    size_t tpart_off, logits_off, total;
};

bool make_fused_layout(int b, int K, int V, int D, FusedLayout &F) {
    if (D < kLmBK || D % kLmBK != 0) return false;
    if (!make_layout(b, K, V, SPEC_F32, kCallMixed, F.L)) return false;
    const int64_t M = (int64_t)b * (K + 1);
    F.ntiles = (int)(((int64_t)V + kLmBV - 1) / kLmBV);
    const int64_t th = (M + kLmBH - 1) / kLmBH;
    if (th > INT_MAX || (int64_t)F.ntiles * th > INT_MAX) return false;
    F.tiles_h = (int)th;
    F.lrs = ((int64_t)V + 63) / 64 * 64;
    F.tpart_off = F.L.total;
    F.logits_off = F.tpart_off + align256((size_t)M * (size_t)F.ntiles * sizeof(Partial));
    F.total = F.logits_off + align256((size_t)M * (size_t)F.lrs * sizeof(float));
    return true;
}

template <bool VEC>
int launch_fused(Ctx c, const LmArgs &la, int b, const FusedLayout &F, hipStream_t st) {
    const Layout &L = F.L;
    stage_mark(0, st);
    launch_lm_head<kEpiVerify>(la, (unsigned)(F.ntiles * F.tiles_h), st);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(1, st);
    const int64_t nmerge = (int64_t)b * (c.K + 1) * L.nseg * kLmTilesPerSeg;
    hipLaunchKernelGGL(tile_merge_kernel, dim3((unsigned)((nmerge + kBlock - 1) / kBlock)), dim3(kBlock), 0, st, c,
                       (const Partial *)la.tpart, F.ntiles, c.K + 1, b, 0, kLmTilesPerSeg);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(2, st);
    // draft rows only (partial rows K+1 .. 2K)
    c.row_lo = c.K + 1;
    c.rpl = c.K;
    const int64_t grid_draft = (int64_t)b * c.K * L.nseg;
    const int64_t grid_res = (int64_t)b * L.nres;
    if (grid_draft > INT_MAX || grid_res > INT_MAX) return SPEC_EINVAL;
    hipLaunchKernelGGL((row_pass<SPEC_F32, VEC>), dim3((unsigned)grid_draft), dim3(kWave), 0, st, c);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(3, st);
    hipLaunchKernelGGL((scan_kernel<SPEC_F32>), dim3((unsigned)b), dim3(kScanBlock), 0, st, c);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(4, st);
    hipLaunchKernelGGL((residual_kernel<SPEC_F32, VEC>), dim3((unsigned)grid_res), dim3(kWave), 0, st, c);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(5, st);
    hipLaunchKernelGGL((draw_kernel<SPEC_F32, VEC>), dim3((unsigned)b), dim3(kBlock), 0, st, c);
    if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    stage_mark(6, st);
    return SPEC_OK;
}

#include "vocab_sharded.inc"
#include "markov_draft.inc"

// Compute units of the current device (0 if it cannot be read), read once
// per device; callers on several host threads may race to fill the cache
// with the same value.
int device_cu_count() {
    static std::atomic<int> cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

bool bf16_operand_ok(const void *p, int64_t stride, int D) {
    return p && (uintptr_t)p % 16 == 0 && stride >= D && stride % 8 == 0;
}

}  // namespace

// ---------------------------------------------------------------------------
// Fixed device scratch for callers that cannot allocate (code under graph
// capture, tight serving loops): spec_mixed_accept_noalloc runs the mixed
// call's kernels with this array as their workspace.  Every GPU the library
// runs on holds its own copy until the process ends.  In host code the name
// `scratch` is only a host-side stand-in: kernels get the device address
// that hipGetSymbolAddress returns for the current device.

static __device__ __align__(256) unsigned char scratch[SPEC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxScratchDevices] = {};
std::mutex g_scratch_mu;

// The copy of `scratch` on the GPU that `st` runs on (the current device for
// the null stream), looked up once per device with that device current and
// kept.  SPEC_ELAUNCH if the runtime cannot give it.
int scratch_address(hipStream_t st, void **out) {
    int dev = 0;
    const hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
        (void)hipGetLastError();
        return SPEC_ELAUNCH;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            int cur = -1;
            if (hipGetDevice(&cur) != hipSuccess || (cur != dev && hipSetDevice(dev) != hipSuccess)) {
                (void)hipGetLastError();
                return SPEC_ELAUNCH;
            }
            const hipError_t se = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (cur != dev) (void)hipSetDevice(cur);
            if (se != hipSuccess || !p) {
                (void)hipGetLastError();
                return SPEC_ELAUNCH;
            }
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SPEC_OK;
}

}  // namespace

extern "C" {

size_t spec_workspace_bytes(int b, int K, int V, int dtype, int sampling) {
    Layout L;
    if (!make_layout(b, K, V, dtype, sampling ? kCallSample : kCallGreedy, L)) return 0;
    return L.total;
}

size_t spec_mixed_workspace_bytes(int b, int K, int V, int dtype) {
    Layout L;
    if (!make_layout(b, K, V, dtype, kCallMixed, L)) return 0;
    return L.total;
}

const char *spec_status_string(int status) {
    switch (status) {
        case SPEC_OK: return "ok";
        case SPEC_EINVAL: return "invalid argument (size, stride, temperature, null pointer or workspace)";
        case SPEC_EDTYPE: return "unknown dtype";
        case SPEC_EALIGN: return "logit pointer not aligned to its element size";
        case SPEC_ELAUNCH: return "kernel launch failed";
        case SPEC_ESCRATCH: return "the call needs more than the SPEC_SCRATCH_BYTES of fixed device scratch";
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
    if (!make_layout(b, K, V, dtype, kCallGreedy, L)) return SPEC_EINVAL;
    if (!target || !draft_tokens || !n_accepted || !tokens || !workspace) return SPEC_EINVAL;
    if (t_row_stride < V || t_batch_stride < 0) return SPEC_EINVAL;
    if (workspace_bytes < L.total || (uintptr_t)workspace % 256 != 0) return SPEC_EINVAL;
    if ((uintptr_t)target % elem_bytes(dtype) != 0) return SPEC_EALIGN;
    Ctx c = {};
    c.target = target;
    c.tbs = t_batch_stride;
    c.trs = t_row_stride;
    c.K = K;
    c.V = V;
    c.T_uniform = 0.0;
    c.x = draft_tokens;
    c.n_out = n_accepted;
    c.tok = tokens;
    c.am = target_argmax;
    return dispatch(c, b, workspace, dtype, kCallGreedy, L, (hipStream_t)hip_stream);
}

int spec_sample_accept(const void *target, const void *draft, int dtype, int64_t t_batch_stride,
                       int64_t t_row_stride, int64_t d_batch_stride, int64_t d_row_stride,
                       const int32_t *draft_tokens, int b, int K, int V, double temperature,
                       const uint64_t *seeds, int32_t *n_accepted, int32_t *tokens, float *p_draft,
                       float *q_draft, void *workspace, size_t workspace_bytes, void *hip_stream) {
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EDTYPE;
    Layout L;
    if (!make_layout(b, K, V, dtype, kCallSample, L)) return SPEC_EINVAL;
    if (!target || !draft || !draft_tokens || !seeds || !n_accepted || !tokens || !workspace) return SPEC_EINVAL;
    if (!(temperature > 0.0) || !(temperature < INFINITY)) return SPEC_EINVAL;
    if (t_row_stride < V || t_batch_stride < 0 || d_row_stride < V || d_batch_stride < 0) return SPEC_EINVAL;
    if (workspace_bytes < L.total || (uintptr_t)workspace % 256 != 0) return SPEC_EINVAL;
    const int es = elem_bytes(dtype);
    if ((uintptr_t)target % es != 0 || (uintptr_t)draft % es != 0) return SPEC_EALIGN;
    Ctx c = {};
    c.target = target;
    c.draft = draft;
    c.tbs = t_batch_stride;
    c.trs = t_row_stride;
    c.dbs = d_batch_stride;
    c.drs = d_row_stride;
    c.K = K;
    c.V = V;
    c.T_uniform = temperature;
    c.x = draft_tokens;
    c.seeds = seeds;
    c.n_out = n_accepted;
    c.tok = tokens;
    c.p_out = p_draft;
    c.q_out = q_draft;
    return dispatch(c, b, workspace, dtype, kCallSample, L, (hipStream_t)hip_stream);
}

// Argument checks of the mixed call, shared by its two entry points (the
// workspace is checked by each).
static int mixed_check(const void *target, const void *draft, int dtype, int64_t t_batch_stride,
                       int64_t t_row_stride, int64_t d_batch_stride, int64_t d_row_stride,
                       const int32_t *draft_tokens, int b, int K, int V, const double *temperatures,
                       const uint64_t *seeds, int32_t *n_accepted, int32_t *tokens, Layout &L) {
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EDTYPE;
    if (!make_layout(b, K, V, dtype, kCallMixed, L)) return SPEC_EINVAL;
    if (!target || !draft || !draft_tokens || !temperatures || !seeds || !n_accepted || !tokens)
        return SPEC_EINVAL;
    if (t_row_stride < V || t_batch_stride < 0 || d_row_stride < V || d_batch_stride < 0) return SPEC_EINVAL;
    return SPEC_OK;
}

static int mixed_run(const void *target, const void *draft, int dtype, int64_t t_batch_stride,
                     int64_t t_row_stride, int64_t d_batch_stride, int64_t d_row_stride,
                     const int32_t *draft_tokens, int b, int K, int V, const double *temperatures,
                     const int32_t *draft_lengths, const uint64_t *seeds, int32_t *n_accepted, int32_t *tokens,
                     float *p_draft, float *q_draft, int32_t *target_argmax, void *workspace, const Layout &L,
                     void *hip_stream) {
    const int es = elem_bytes(dtype);
    if ((uintptr_t)target % es != 0 || (uintptr_t)draft % es != 0) return SPEC_EALIGN;
    Ctx c = {};
    c.target = target;
    c.draft = draft;
    c.tbs = t_batch_stride;
    c.trs = t_row_stride;
    c.dbs = d_batch_stride;
    c.drs = d_row_stride;
    c.K = K;
    c.V = V;
    c.temps = temperatures;
    c.klen = draft_lengths;
    c.x = draft_tokens;
    c.seeds = seeds;
    c.n_out = n_accepted;
    c.tok = tokens;
    c.p_out = p_draft;
    c.q_out = q_draft;
    c.am = target_argmax;
    return dispatch(c, b, workspace, dtype, kCallMixed, L, (hipStream_t)hip_stream);
}

int spec_mixed_accept(const void *target, const void *draft, int dtype, int64_t t_batch_stride,
                      int64_t t_row_stride, int64_t d_batch_stride, int64_t d_row_stride,
                      const int32_t *draft_tokens, int b, int K, int V, const double *temperatures,
                      const int32_t *draft_lengths, const uint64_t *seeds, int32_t *n_accepted, int32_t *tokens, float *p_draft,
                      float *q_draft, int32_t *target_argmax, void *workspace, size_t workspace_bytes,
                      void *hip_stream) {
    Layout L;
    int rc = mixed_check(target, draft, dtype, t_batch_stride, t_row_stride, d_batch_stride, d_row_stride,
                         draft_tokens, b, K, V, temperatures, seeds, n_accepted, tokens, L);
    if (rc != SPEC_OK) return rc;
    if (!workspace || workspace_bytes < L.total || (uintptr_t)workspace % 256 != 0) return SPEC_EINVAL;
    return mixed_run(target, draft, dtype, t_batch_stride, t_row_stride, d_batch_stride, d_row_stride, draft_tokens,
                     b, K, V, temperatures, draft_lengths, seeds, n_accepted, tokens, p_draft, q_draft,
                     target_argmax, workspace, L, hip_stream);
}

int spec_mixed_accept_noalloc(const void *target, const void *draft, int dtype, int64_t t_batch_stride,
                              int64_t t_row_stride, int64_t d_batch_stride, int64_t d_row_stride,
                              const int32_t *draft_tokens, int b, int K, int V, const double *temperatures,
                              const int32_t *draft_lengths, const uint64_t *seeds, int32_t *n_accepted,
                              int32_t *tokens, float *p_draft, float *q_draft, int32_t *target_argmax,
                              void *hip_stream) {
    Layout L;
    int rc = mixed_check(target, draft, dtype, t_batch_stride, t_row_stride, d_batch_stride, d_row_stride,
                         draft_tokens, b, K, V, temperatures, seeds, n_accepted, tokens, L);
    if (rc != SPEC_OK) return rc;
    if (L.total > (size_t)SPEC_SCRATCH_BYTES) return SPEC_ESCRATCH;
    void *ws = nullptr;
    rc = scratch_address((hipStream_t)hip_stream, &ws);
    if (rc != SPEC_OK) return rc;
    // The mixed kernels need no cleared workspace: every record they read in a
    // call is written earlier in the same call.
    return mixed_run(target, draft, dtype, t_batch_stride, t_row_stride, d_batch_stride, d_row_stride, draft_tokens,
                     b, K, V, temperatures, draft_lengths, seeds, n_accepted, tokens, p_draft, q_draft,
                     target_argmax, ws, L, hip_stream);
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

int spec_philox_uniforms(uint64_t seed, uint32_t row0, int nrow, uint32_t pos0, int npos, uint32_t tag,
                         double *out, void *hip_stream) {
    if (!out || nrow < 0 || npos < 0 || (uintptr_t)out % 8 != 0) return SPEC_EINVAL;
    const int64_t n = (int64_t)nrow * npos;
    if (n == 0) return SPEC_OK;
    const int64_t grid = (n + kBlock - 1) / kBlock;
    if (grid > INT_MAX) return SPEC_EINVAL;
    hipLaunchKernelGGL(philox_grid_kernel, dim3((unsigned)grid), dim3(kBlock), 0, (hipStream_t)hip_stream, seed,
                       row0, nrow, pos0, npos, tag, out);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

int spec_stream_read(const void *src, size_t nbytes, uint32_t *sink, void *hip_stream) {
    if (!src || !sink || nbytes % 16 != 0 || (uintptr_t)src % 16 || (uintptr_t)sink % 4) return SPEC_EINVAL;
    if (nbytes == 0) return SPEC_OK;
    const int64_t nvec = (int64_t)(nbytes / 16);
    const int64_t grid = (nvec + kSegVec - 1) / kSegVec;
    if (grid > INT_MAX) return SPEC_EINVAL;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kWave), 0, (hipStream_t)hip_stream,
                       (const uint4 *)src, nvec, sink);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

size_t spec_fused_workspace_bytes(int b, int K, int V, int D) {
    FusedLayout F;
    if (!make_fused_layout(b, K, V, D, F)) return 0;
    return F.total;
}

int spec_fused_mixed_accept(const void *hidden, int64_t h_batch_stride, int64_t h_row_stride, const void *weight,
                            int64_t w_row_stride, int D, float softcap, const float *draft, int64_t d_batch_stride,
                            int64_t d_row_stride, const int32_t *draft_tokens, int b, int K, int V,
                            const double *temperatures, const int32_t *draft_lengths, const uint64_t *seeds,
                            int32_t *n_accepted, int32_t *tokens, float *p_draft, float *q_draft,
                            int32_t *target_argmax, void *workspace, size_t workspace_bytes, void *hip_stream) {
    FusedLayout F;
    if (!make_fused_layout(b, K, V, D, F)) return SPEC_EINVAL;
    if (!draft || !draft_tokens || !temperatures || !seeds || !n_accepted || !tokens || !workspace)
        return SPEC_EINVAL;
    if (!hidden || !weight) return SPEC_EINVAL;
    if (!(softcap >= 0.0f) || !(softcap < INFINITY)) return SPEC_EINVAL;
    if (d_row_stride < V || d_batch_stride < 0 || h_batch_stride < 0) return SPEC_EINVAL;
    if (workspace_bytes < F.total || (uintptr_t)workspace % 256 != 0) return SPEC_EINVAL;
    if (!bf16_operand_ok(hidden, h_row_stride, D) || !bf16_operand_ok(weight, w_row_stride, D) ||
        h_batch_stride % 8 != 0)
        return SPEC_EALIGN;
    if ((uintptr_t)draft % 4 != 0) return SPEC_EALIGN;
    // the GEMM addresses hidden and one weight tile with 32-bit byte offsets
    const int64_t hspan = (int64_t)(b - 1) * h_batch_stride + (int64_t)K * h_row_stride + D;
    if (hspan > (int64_t)INT_MAX || (int64_t)kLmBV * w_row_stride * 2 > (int64_t)INT_MAX) return SPEC_EINVAL;
    char *ws = (char *)workspace;
    float *logits = (float *)(ws + F.logits_off);
    LmArgs la = {};
    la.hidden = (const uint16_t *)hidden;
    la.hbs = h_batch_stride;
    la.hrs = h_row_stride;
    la.hspan_bytes = (uint32_t)(hspan * 2);
    la.weight = (const uint16_t *)weight;
    la.wrs = w_row_stride;
    la.b = b;
    la.K1 = K + 1;
    la.V = V;
    la.D = D;
    la.M = b * (K + 1);
    la.cap = softcap;
    la.inv_cap = softcap > 0.0f ? 1.0f / softcap : 0.0f;
    la.temps = temperatures;
    la.klen = draft_lengths;
    la.K = K;
    la.logits = logits;
    la.lrs = F.lrs;
    la.lbs = (int64_t)(K + 1) * F.lrs;
    la.tpart = (Partial *)(ws + F.tpart_off);
    la.ntiles = F.ntiles;
    la.tiles_h = F.tiles_h;
    Ctx c = {};
    c.target = logits;
    c.draft = draft;
    c.tbs = la.lbs;
    c.trs = la.lrs;
    c.dbs = d_batch_stride;
    c.drs = d_row_stride;
    c.K = K;
    c.V = V;
    c.temps = temperatures;
    c.klen = draft_lengths;
    c.x = draft_tokens;
    c.seeds = seeds;
    c.n_out = n_accepted;
    c.tok = tokens;
    c.p_out = p_draft;
    c.q_out = q_draft;
    c.am = target_argmax;
    const Layout &L = F.L;
    c.nseg = L.nseg;
    set_nres(c, L.nres);
    c.rps = L.rps;
    c.row_lo = 0;
    c.rpl = L.rps;
    c.shard_id = -1;
    c.col0 = 0;
    c.zx = nullptr;
    c.part = (Partial *)(ws + L.part_off);
    c.plan = (DrawPlan *)(ws + L.plan_off);
    c.rmass = (double *)(ws + L.rmass_off);
    c.rlist = (int32_t *)(ws + L.rlist_off);
    const bool vec = rows_vector_aligned(draft, 4, d_batch_stride, d_row_stride);
    return vec ? launch_fused<true>(c, la, b, F, (hipStream_t)hip_stream)
               : launch_fused<false>(c, la, b, F, (hipStream_t)hip_stream);
}

int spec_lm_head_logits(const void *hidden, int64_t h_row_stride, int rows, const void *weight,
                        int64_t w_row_stride, int V, int D, float softcap, float *logits, int64_t l_row_stride,
                        void *hip_stream) {
    if (rows < 1 || V < 1 || V > INT_MAX - 65536 || D < kLmBK || D % kLmBK != 0) return SPEC_EINVAL;
    if (!hidden || !weight || !logits) return SPEC_EINVAL;
    if (!(softcap >= 0.0f) || !(softcap < INFINITY)) return SPEC_EINVAL;
    if (l_row_stride < V) return SPEC_EINVAL;
    if (!bf16_operand_ok(hidden, h_row_stride, D) || !bf16_operand_ok(weight, w_row_stride, D)) return SPEC_EALIGN;
    if ((uintptr_t)logits % 16 != 0 || l_row_stride % 4 != 0) return SPEC_EALIGN;
    const int64_t hspan = (int64_t)(rows - 1) * h_row_stride + D;
    if (hspan > (int64_t)INT_MAX || (int64_t)kLmBV * w_row_stride * 2 > (int64_t)INT_MAX) return SPEC_EINVAL;
    const int64_t ntiles = ((int64_t)V + kLmBV - 1) / kLmBV;
    const int64_t th = ((int64_t)rows + kLmBH - 1) / kLmBH;
    if (ntiles * th > INT_MAX) return SPEC_EINVAL;
    LmArgs la = {};
    la.hidden = (const uint16_t *)hidden;
    la.hbs = h_row_stride;
    la.hrs = 0;
    la.hspan_bytes = (uint32_t)(hspan * 2);
    la.weight = (const uint16_t *)weight;
    la.wrs = w_row_stride;
    la.b = rows;
    la.K1 = 1;
    la.V = V;
    la.D = D;
    la.M = rows;
    la.cap = softcap;
    la.inv_cap = softcap > 0.0f ? 1.0f / softcap : 0.0f;
    la.logits = logits;
    la.lbs = l_row_stride;
    la.lrs = 0;
    la.ntiles = (int)ntiles;
    la.tiles_h = (int)th;
    launch_lm_head<kEpiLogits>(la, (unsigned)(ntiles * th), (hipStream_t)hip_stream);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

size_t spec_sharded_workspace_bytes(int G, const int *shard_V, int b, int K, int dtype) {
    ShardedLayout S;
    if (!make_sharded_layout(G, shard_V, b, K, dtype, S)) return 0;
    return S.total;
}

int spec_sharded_mixed_accept(int G, const void *const *target_shards, const void *const *draft_shards,
                              const int *shard_V, const int64_t *t_strides, const int64_t *d_strides, int dtype,
                              const int32_t *draft_tokens, int b, int K, const double *temperatures,
                              const int32_t *draft_lengths, const uint64_t *seeds, int32_t *n_accepted,
                              int32_t *tokens, float *p_draft, float *q_draft, int32_t *target_argmax,
                              void *workspace, size_t workspace_bytes, void *hip_stream) {
    if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EDTYPE;
    ShardedLayout S;
    if (!make_sharded_layout(G, shard_V, b, K, dtype, S)) return SPEC_EINVAL;
    if (!target_shards || !draft_shards || !t_strides || !d_strides) return SPEC_EINVAL;
    if (!draft_tokens || !temperatures || !seeds || !n_accepted || !tokens || !workspace) return SPEC_EINVAL;
    if (workspace_bytes < S.total || (uintptr_t)workspace % 256 != 0) return SPEC_EINVAL;
    const int es = elem_bytes(dtype);
    char *ws = (char *)workspace;
    Ctx cg[kMaxShards];
    bool vec[kMaxShards];
    int32_t col0 = 0;
    for (int g = 0; g < G; ++g) {
        const void *tp = target_shards[g], *dp = draft_shards[g];
        const int64_t tbs = t_strides[2 * g], trs = t_strides[2 * g + 1];
        const int64_t dbs = d_strides[2 * g], drs = d_strides[2 * g + 1];
        if (!tp || !dp) return SPEC_EINVAL;
        if (trs < shard_V[g] || tbs < 0 || drs < shard_V[g] || dbs < 0) return SPEC_EINVAL;
        if ((uintptr_t)tp % es != 0 || (uintptr_t)dp % es != 0) return SPEC_EALIGN;
        Ctx c = {};
        c.target = tp;
        c.draft = dp;
        c.tbs = tbs;
        c.trs = trs;
        c.dbs = dbs;
        c.drs = drs;
        c.K = K;
        c.V = shard_V[g];
        c.nseg = S.nseg[g];
        set_nres(c, S.nres[g]);
        c.rps = S.rps;
        c.row_lo = 0;
        c.rpl = S.rps;
        c.temps = temperatures;
        c.klen = draft_lengths;
        c.x = draft_tokens;
        c.seeds = seeds;
        c.n_out = n_accepted;
        c.tok = tokens;
        c.part = (Partial *)(ws + S.part_off[g]);
        c.rmass = (double *)(ws + S.rmass_off[g]);
        c.plan = (DrawPlan *)(ws + S.plan_off);
        c.shard_id = g;
        c.col0 = col0;
        c.zx = nullptr;
        cg[g] = c;
        vec[g] = rows_vector_aligned(tp, es, tbs, trs) && rows_vector_aligned(dp, es, dbs, drs);
        col0 += shard_V[g];
    }
    // The scan's view: one record per shard in place of segments, the gathered
    // draft-token logits, the whole vocabulary for the token range check.
    Ctx call = cg[0];
    call.V = col0;
    call.nseg = G;
    call.part = (Partial *)(ws + S.rec_off);
    call.zx = (const float *)(ws + S.zx_off);
    call.shard_id = -1;
    call.col0 = 0;
    call.p_out = p_draft;
    call.q_out = q_draft;
    call.am = target_argmax;
    hipStream_t st = (hipStream_t)hip_stream;
    bool all_vec = true;
    for (int g = 0; g < G; ++g) all_vec = all_vec && vec[g];
    if (dtype == SPEC_BF16)
        return all_vec ? launch_sharded<SPEC_BF16, true>(cg, call, b, S, ws, st)
                       : launch_sharded<SPEC_BF16, false>(cg, call, b, S, ws, st);
    return all_vec ? launch_sharded<SPEC_F32, true>(cg, call, b, S, ws, st)
                   : launch_sharded<SPEC_F32, false>(cg, call, b, S, ws, st);
}

size_t spec_markov_workspace_bytes(int b, int K, int V, int r) {
    MarkovLayout L;
    if (!make_markov_layout(b, K, V, r, L)) return 0;
    return L.total;
}

int spec_markov_block_decode(const float *base, int64_t base_batch_stride, int64_t base_row_stride,
                             const int32_t *anchors, const void *w1, int64_t w1_row_stride, const void *w2,
                             int64_t w2_row_stride, int r, int b, int K, int V, const double *temperatures,
                             const uint64_t *seeds, const void *hidden, int64_t h_batch_stride,
                             int64_t h_row_stride, int D, const void *conf_w, float conf_b, float threshold,
                             int32_t *tokens, float *draft_logits, int64_t q_batch_stride, int64_t q_row_stride,
                             float *confidence, int32_t *lengths, void *workspace, size_t workspace_bytes,
                             void *hip_stream) {
    MarkovLayout L;
    if (!make_markov_layout(b, K, V, r, L)) return SPEC_EINVAL;
    if (!base || !anchors || !w1 || !w2 || !temperatures || !seeds || !tokens || !draft_logits || !workspace)
        return SPEC_EINVAL;
    if (workspace_bytes < L.total || (uintptr_t)workspace % 256 != 0) return SPEC_EINVAL;
    if (base_row_stride < V || base_batch_stride < 0 || q_row_stride < V || q_batch_stride < 0) return SPEC_EINVAL;
    if (!(threshold == threshold) || !(conf_b == conf_b)) return SPEC_EINVAL;
    // The confidence head runs when either of its outputs is asked for, and
    // then needs its inputs.
    const bool want_conf = confidence != nullptr || lengths != nullptr;
    if (want_conf && (!hidden || !conf_w || D < 1 || h_row_stride < D || h_batch_stride < 0)) return SPEC_EINVAL;
    if ((uintptr_t)base % 4) return SPEC_EALIGN;
    if ((uintptr_t)draft_logits % 16 || q_row_stride % 4 || q_batch_stride % 4) return SPEC_EALIGN;
    if (!bf16_operand_ok(w1, w1_row_stride, r) || !bf16_operand_ok(w2, w2_row_stride, r)) return SPEC_EALIGN;
    if (want_conf && ((uintptr_t)hidden % 2 || (uintptr_t)conf_w % 2)) return SPEC_EALIGN;
    const int64_t w1span = (int64_t)(V - 1) * w1_row_stride + r;
    if (w1span > (int64_t)INT_MAX || (int64_t)MqS::kBV * w2_row_stride * 2 > (int64_t)INT_MAX) return SPEC_EINVAL;
    hipStream_t st = (hipStream_t)hip_stream;
    char *ws = (char *)workspace;

    Ctx c = {};
    c.target = draft_logits;
    c.draft = draft_logits;
    c.tbs = q_batch_stride;
    c.trs = q_row_stride;
    c.dbs = q_batch_stride;
    c.drs = q_row_stride;
    c.K = K - 1;                         // q has K rows per sequence, tokens [b, K]
    c.V = V;
    c.nseg = L.nseg;
    set_nres(c, 0);
    c.rps = K;
    c.row_lo = 0;
    c.rpl = K;
    c.temps = temperatures;
    c.seeds = seeds;
    c.tok = tokens;
    c.part = (Partial *)(ws + L.part_off);
    c.plan = (DrawPlan *)(ws + L.plan_off);
    c.rmass = (double *)(ws + L.part_off);   // unused: no residual draws here
    c.shard_id = -1;

    MqArgs ma = {};
    ma.w1 = (const uint16_t *)w1;
    ma.w1rs = w1_row_stride;
    ma.w1span = (uint32_t)(w1span * 2);
    ma.w2 = (const uint16_t *)w2;
    ma.w2rs = w2_row_stride;
    ma.base = base;
    ma.bbs = base_batch_stride;
    ma.brs = base_row_stride;
    ma.q = draft_logits;
    ma.qbs = q_batch_stride;
    ma.qrs = q_row_stride;
    ma.temps = temperatures;
    ma.b = b;
    ma.V = V;
    ma.r = r;
    ma.ntiles = L.ntiles;
    ma.tiles_h = L.tiles_h;
    ma.tpart = (Partial *)(ws + L.tpart_off);
    const unsigned grid_q = (unsigned)(L.ntiles * L.tiles_h);
    static_assert(kMsBV == MqS::kBV, "both position kernels write 128-entry tile records");

    // Ranks up to 256 (multiples of 64) with 16-byte aligned base rows whose
    // 128-sequence span fits a 31-bit offset: the persistent streaming kernel,
    // one workgroup per CU.
    static_assert(kMsMaxR == 256, "one streaming instance per r / 64 in 1..4");
    const bool streaming = r <= kMsMaxR && (uintptr_t)base % 16 == 0 && base_batch_stride % 4 == 0 &&
                           base_row_stride % 4 == 0 && (int64_t)(kMsBH - 1) * base_batch_stride * 4 + 128 < INT_MAX;
    MsArgs sa = {};
    unsigned grid_s = 0;
    if (streaming) {
        const int ncu = device_cu_count();
        if (ncu < 1) return SPEC_ELAUNCH;
        sa.w1 = ma.w1;
        sa.w1rs = w1_row_stride;
        sa.w2 = ma.w2;
        sa.w2rs = w2_row_stride;
        sa.base = base;
        sa.bbs = base_batch_stride;
        sa.brs = base_row_stride;
        sa.base_end = (int64_t)(b - 1) * base_batch_stride + (int64_t)(K - 1) * base_row_stride + V;
        sa.q = draft_logits;
        sa.qbs = q_batch_stride;
        sa.qrs = q_row_stride;
        sa.temps = temperatures;
        sa.b = b;
        sa.V = V;
        sa.r = r;
        sa.ntiles = L.ntiles;
        sa.P = min(L.ntiles, max(1, ncu / L.tiles_h));     // every workgroup gets at least one tile
        const int stage = kMsChunkRows * r * 2 + kMsBaseB;    // a chunk's W2 rows and base logits
        const int icp = stage / 1024 / kMsPW;                 // loads per chunk per producer wave
        sa.ahead = min((63 - kMsZp) / icp - 1, 15);           // (ahead + 1) * icp loads and kMsZp stores in flight
        sa.nst = sa.ahead + 2;
        while (sa.nst * stage > kMsRingB) {
            --sa.nst;
            sa.ahead = sa.nst - 2;
        }
        sa.tpart = ma.tpart;
        if ((int64_t)sa.P * L.tiles_h > INT_MAX) return SPEC_EINVAL;
        grid_s = (unsigned)(sa.P * L.tiles_h);
    }
    stage_mark(0, st);
    for (int i = 0; i < K; ++i) {
        const int32_t *prev = i == 0 ? anchors : tokens + (i - 1);
        const int64_t pstride = i == 0 ? 1 : K;
        if (streaming) {
            sa.prev = prev;
            sa.pstride = pstride;
            sa.step = i;
            switch (r / 64) {
            case 1: hipLaunchKernelGGL(markov_stream_kernel<2>, dim3(grid_s), dim3(kMsThreads), 0, st, sa); break;
            case 2: hipLaunchKernelGGL(markov_stream_kernel<4>, dim3(grid_s), dim3(kMsThreads), 0, st, sa); break;
            case 3: hipLaunchKernelGGL(markov_stream_kernel<6>, dim3(grid_s), dim3(kMsThreads), 0, st, sa); break;
            default: hipLaunchKernelGGL(markov_stream_kernel<8>, dim3(grid_s), dim3(kMsThreads), 0, st, sa); break;
            }
        } else {
            ma.prev = prev;
            ma.pstride = pstride;
            ma.step = i;
            hipLaunchKernelGGL((markov_q_kernel<MqS::kBV, MqS::kBH, MqS::kNW, MqS::kNST>), dim3(grid_q),
                               dim3(MqS::kThreads), 0, st, ma);
        }
        if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
        hipLaunchKernelGGL(draft_select_kernel, dim3((unsigned)b), dim3(kBlock), 0, st, c, i,
                           (const Partial *)ma.tpart, L.ntiles, prev, pstride);
        if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    }
    stage_mark(1, st);
    if (want_conf) {
        const int vec = (uintptr_t)hidden % 16 == 0 && h_row_stride % 8 == 0 && h_batch_stride % 8 == 0 &&
                        (uintptr_t)conf_w % 16 == 0;
        hipLaunchKernelGGL(confidence_length_kernel, dim3((unsigned)b), dim3(kConfWaves * kWave), 0, st,
                           (const uint16_t *)hidden, h_batch_stride, h_row_stride, D, (const uint16_t *)w1,
                           w1_row_stride, r, (const uint16_t *)conf_w, conf_b, anchors, (const int32_t *)tokens, K, V,
                           vec, confidence, threshold, lengths);
        if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
    }
    stage_mark(2, st);
    return SPEC_OK;
}

}  // extern "C"
