// Device code of the routing stage shared by route.hip (the routing launches)
// and layer_persistent.hip (the one-launch decode layer): router logits of
// one (token, expert group) per block, top-k + softmax per wavefront and the
// stable counting sort of the pairs by expert.  Not part of the C ABI.
#pragma once

#include "moe_internal.h"

#include <climits>

namespace {

constexpr int kSelThreads = 512;         // 8 waves per token
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelTokens = 4;            // tokens per block of the prefill logits + selection
constexpr int kGrpThreads = 1024;        // 16 waves for the grouping
constexpr int kGrpWaves = kGrpThreads / 64;
constexpr int kMaxH = 4096;
constexpr int kSplit = 30;               // products with shift < kSplit go to the low integer limb

constexpr int ilog2_ceil(int n) { return n <= 1 ? 0 : 1 + ilog2_ceil((n + 1) / 2); }

// FP16 bits -> signed integer significand m and exponent field q, value = m * 2^(q-25).
__device__ inline void dec16(uint32_t b, int &m, int &q)
{
    const int e = (b >> 10) & 31;
    const int mag = (b & 0x3ff) | (e ? 0x400 : 0);
    m = (b & 0x8000) ? -mag : mag;
    q = e ? e : 1;
}

__device__ inline double h2d(uint16_t b) { return (double)(float)__builtin_bit_cast(_Float16, b); }

// Correctly rounded FP32 of (hi * 2^kSplit + lo) * 2^-48, ties to even.
__device__ float rn32_limbs(long long hi, long long lo)
{
    // 128-bit two's complement value = hi * 2^30 + lo, as (vh, vl).
    unsigned long long al = (unsigned long long)hi << kSplit;
    long long ah = hi >> (64 - kSplit);
    unsigned long long bl = (unsigned long long)lo;
    long long bh = lo >> 63;
    unsigned long long vl = al + bl;
    long long vh = ah + bh + (vl < al ? 1 : 0);
    if (vh == 0 && vl == 0) return 0.0f;
    const bool neg = vh < 0;
    if (neg) {                               // magnitude
        vl = ~vl + 1ull;
        vh = ~vh + (vl == 0 ? 1 : 0);
    }
    unsigned long long uh = (unsigned long long)vh;
    const int L = uh ? 128 - __builtin_clzll(uh) : 64 - __builtin_clzll(vl);   // bit length
    unsigned int mant;
    int sh = 0;
    if (L <= 24) {
        mant = (unsigned int)vl;
    } else {
        sh = L - 24;
        unsigned long long m = sh >= 64 ? (uh >> (sh - 64)) : ((vl >> sh) | (sh ? (uh << (64 - sh)) : 0ull));
        mant = (unsigned int)m;
        const int rb = sh - 1;               // round bit position
        const unsigned long long round = rb >= 64 ? (uh >> (rb - 64)) & 1ull : (vl >> rb) & 1ull;
        bool sticky;
        if (rb >= 64) sticky = vl != 0 || (rb > 64 && (uh & ((1ull << (rb - 64)) - 1ull)) != 0);
        else sticky = rb > 0 && (vl & ((1ull << rb) - 1ull)) != 0;
        if (round && (sticky || (mant & 1u))) mant += 1u;
    }
    const float r = ldexpf((float)mant, sh - 48);
    return neg ? -r : r;
}

// True when every real number within err of v rounds (to nearest, ties to
// even) to the same FP32 value as v does: no FP32 rounding midpoint lies in
// [v - err, v + err].
__device__ inline bool rn32_certain(double v, double err)
{
    const float f = (float)v;
    const unsigned int b = __builtin_bit_cast(unsigned int, f);
    float up, dn;
    if (f == 0.0f) {
        up = __builtin_bit_cast(float, 1u);
        dn = -up;
    } else if (f > 0.0f) {
        up = __builtin_bit_cast(float, b + 1u);
        dn = __builtin_bit_cast(float, b - 1u);
    } else {
        up = __builtin_bit_cast(float, b - 1u);
        dn = __builtin_bit_cast(float, b + 1u);
    }
    const double mid_up = 0.5 * ((double)f + (double)up);      // exact in fp64
    const double mid_dn = 0.5 * ((double)f + (double)dn);
    return (v - err > mid_dn) && (v + err < mid_up);
}

struct RouteArgs {
    const uint16_t *x;      // [T][H]
    const uint16_t *wr;     // [H][E]
    const float *bias;      // [E] or null
    int T, H, E, k;
    float *logits;          // [T][E] or null
    int32_t *ids;           // [T][k]
    float *w;               // [T][k]
    int32_t *offsets;       // [E+1]
    int32_t *sorted_pairs;  // [T*k]
    int32_t *pair_pos;      // [T*k]
    int32_t *active;        // [E]
    int32_t *n_active;      // [1]
    int force_exact;        // recompute every logit with the integer path
    float *lbuf;            // [T][E] logits handed from the logits kernel to the grouping kernel
};

// Exact logit of one expert, computed by the whole block: integer limbs of
// the products x[h] * wr[h][e], summed in two 64-bit accumulators (each holds
// fewer than 2^12 terms below 2^51, so neither overflows), then reduced
// across the block and rounded once.
// x[t, :] is read from sx, the block's row of FP16 values held as doubles
// (exact); the limb sums are integers, so their order does not matter.  The
// result is valid in thread 0.
template <typename XT>
__device__ float exact_logit(const RouteArgs &a, const XT *sx, int e, long long (*red)[2])
{
    const int tid = threadIdx.x;
    long long hi = 0, lo = 0;
    for (int h = tid; h < a.H; h += kSelThreads) {
        int mx, qx, mw, qw;
        dec16(__builtin_bit_cast(uint16_t, (_Float16)sx[h]), mx, qx);
        dec16(a.wr[(size_t)h * a.E + e], mw, qw);
        const long long prod = (long long)(mx * mw);               // |prod| < 2^22
        const int sh = qx + qw - 2;                                // product = prod * 2^(sh-48), sh in [0, 58]
        if (sh < kSplit) lo += (long long)((unsigned long long)prod << sh);
        else hi += (long long)((unsigned long long)prod << (sh - kSplit));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        hi += __shfl_xor(hi, off);
        lo += __shfl_xor(lo, off);
    }
    if ((tid & 63) == 0) {
        red[tid >> 6][0] = hi;
        red[tid >> 6][1] = lo;
    }
    __syncthreads();
    float r = 0.0f;
    if (tid == 0) {
        long long H2 = 0, L2 = 0;
        for (int w = 0; w < kSelWaves; ++w) {
            H2 += red[w][0];
            L2 += red[w][1];
        }
        r = rn32_limbs(H2, L2);
    }
    __syncthreads();                                               // red is reused by the next call
    return r;
}

// Maximum of an int over the 64 lanes of a wavefront, in every lane: DPP
// shifts build per-row prefix maxima (lane 15 of each row of 16 holds the
// row's maximum), two row broadcasts fold the rows into lane 63, and a
// readlane hands it to every lane.
template <int CTRL, int ROW_MASK>
__device__ inline int dpp_max_step(int v)
{
    return max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, CTRL, ROW_MASK, 0xf, false));
}

__device__ inline int wave_max(int v)
{
    v = dpp_max_step<0x111, 0xf>(v);         // row_shr:1
    v = dpp_max_step<0x112, 0xf>(v);         // row_shr:2
    v = dpp_max_step<0x114, 0xf>(v);         // row_shr:4
    v = dpp_max_step<0x118, 0xf>(v);         // row_shr:8
    v = dpp_max_step<0x142, 0xa>(v);         // row_bcast:15 into rows 1 and 3
    v = dpp_max_step<0x143, 0xc>(v);         // row_bcast:31 into rows 2 and 3
    return __builtin_amdgcn_readlane(v, 63);
}

// An int with the order of the finite float f (-0 and +0 map to one key).
__device__ inline int order_key(float f)
{
    const int b = __builtin_bit_cast(int, f + 0.0f);
    return b ^ ((b >> 31) & 0x7FFFFFFF);
}

using moe::add_partner;
using moe::add_row_ror;
using moe::sum_phases;

// Top-k (ties to the lower expert index, slots in descending order) and
// softmax over the k selected logits, for NTOK tokens at once (independent
// chains, so their latencies overlap); one full wavefront, lane = expert,
// lv[i] = that expert's final logit (bias included) for token tok[i] (tokens
// >= a.T are skipped).  k rounds of a wavefront maximum; the lowest lane
// holding it wins the slot and drops out.  Lane j < k keeps slot j.  The
// softmax denominator is summed in a fixed order (DPP prefix over lanes 0..7).
// Writes ids and w (at device scope when DEV), and the ids also to s_ids (if not null).
template <int NTOK, bool DEV = false>
__device__ void topk_softmax_wave(const RouteArgs &a, const int (&tok)[NTOK], int lane, const float (&lv)[NTOK],
                                  int *s_ids)
{
    const int E = a.E, k = a.k;
    int key[NTOK];
    float my_l[NTOK], m0[NTOK];
    int my_id[NTOK];
#pragma unroll
    for (int i = 0; i < NTOK; ++i) {
        key[i] = lane < E ? order_key(lv[i]) : INT_MIN;  // missing experts never outrank a real one
        my_id[i] = 0;
        my_l[i] = 0.0f;
        m0[i] = 0.0f;
    }
    for (int j = 0; j < k; ++j) {
        int m[NTOK];
#pragma unroll
        for (int i = 0; i < NTOK; ++i) m[i] = wave_max(key[i]);
#pragma unroll
        for (int i = 0; i < NTOK; ++i) {
            const int win = (int)__builtin_ctzll(__ballot(key[i] == m[i]));
            const float l = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lv[i]), win));
            if (lane == win) key[i] = INT_MIN;
            if (lane == j) {
                my_id[i] = win;
                my_l[i] = l;
            }
            if (j == 0) m0[i] = l;
        }
    }
#pragma unroll
    for (int i = 0; i < NTOK; ++i) {
        if (tok[i] >= a.T) continue;
        const float ex = lane < k ? expf(my_l[i] - m0[i]) : 0.0f;
        float den = ex;                       // lanes 0..7 of row 0 hold the k values
        den += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, den), 0x111, 0xf, 0xf, false));
        den += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, den), 0x112, 0xf, 0xf, false));
        den += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, den), 0x114, 0xf, 0xf, false));
        den = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, den), 7));
        if (lane < k) {
            const size_t p = (size_t)tok[i] * k + lane;
            moe::put<DEV>(&a.ids[p], (int32_t)my_id[i]);
            moe::put<DEV>(&a.w[p], ex / den);
            if (s_ids) s_ids[p] = my_id[i];
        }
    }
}

// Loads VEC consecutive FP16 router weights (experts e0 .. e0+VEC-1 of row h).
template <int VEC>
struct WLoad;
template <>
struct WLoad<8> {
    typedef unsigned int T __attribute__((ext_vector_type(4)));
    static __device__ inline T ld(const uint16_t *p) { return *reinterpret_cast<const T *>(p); }
    static __device__ inline uint16_t get(const T &v, int j) { return (uint16_t)(v[j >> 1] >> (16 * (j & 1))); }
};
template <>
struct WLoad<4> {
    typedef unsigned int T __attribute__((ext_vector_type(2)));
    static __device__ inline T ld(const uint16_t *p) { return *reinterpret_cast<const T *>(p); }
    static __device__ inline uint16_t get(const T &v, int j) { return (uint16_t)(v[j >> 1] >> (16 * (j & 1))); }
};
template <>
struct WLoad<2> {
    typedef unsigned int T;
    static __device__ inline T ld(const uint16_t *p) { return *reinterpret_cast<const T *>(p); }
    static __device__ inline uint16_t get(const T &v, int j) { return (uint16_t)(v >> (16 * j)); }
};
template <>
struct WLoad<1> {
    typedef uint16_t T;
    static __device__ inline T ld(const uint16_t *p) { return *p; }
    static __device__ inline uint16_t get(const T &v, int) { return v; }
};

constexpr int kGroupE = 16;                // experts per block in the decode kernel

// Lanes of the wave holding the same value e (0 <= e < 64) as this lane;
// lanes with e < 0 match nothing.
__device__ inline unsigned long long same_expert_lanes(int e)
{
    unsigned long long m = __ballot(e >= 0);
#pragma unroll
    for (int b = 0; b < 6; ++b) {
        const bool bit = (e >> b) & 1;
        const unsigned long long v = __ballot(bit);
        m &= bit ? v : ~v;
    }
    return e >= 0 ? m : 0ull;
}

constexpr int kGrpLdsIds = 4096;           // pairs whose ids the grouping keeps in LDS
constexpr int kTopkBatch = 2;              // tokens a wave routes together
constexpr int kTopkChunk = 8;              // tokens whose logits a wave requests together

template <int NW, bool TOPK>
struct GroupLds {
    int cnt[NW][MOE_MAX_EXPERTS];
    int base[NW][MOE_MAX_EXPERTS];
    int ids[TOPK ? kGrpLdsIds : 1];
};

// Run by one block of NW wavefronts (DEV: the logits are read and the results
// written at device scope, for blocks of the same launch).  With TOPK, first the top-k + softmax of
// every token from the logits in a.lbuf (one wave per token, lane = expert);
// then the stable counting sort of the T*k pairs by expert.  Wave w owns the
// contiguous pair range [w*n/NW, (w+1)*n/NW): per-wave counts (LDS atomics),
// a prefix over experts and waves gives each wave its starting position per
// expert, then each wave walks its range 64 pairs at a time; a pair's rank
// among equal experts of its chunk comes from a ballot.
template <int NW, bool TOPK, bool DEV = false>
__device__ void group_phase(const RouteArgs &a, GroupLds<NW, TOPK> &S)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = a.T * a.k, E = a.E;
    if (TOPK) {
        // A wave routes tokens wave, wave + NW, ...: the logit rows of kTopkChunk of
        // them are requested together (one memory round trip per chunk, not one
        // per pair of tokens), then routed kTopkBatch at a time.
        for (int c0 = wave; c0 < a.T; c0 += NW * kTopkChunk) {
            int tok[kTopkChunk];
            float lv[kTopkChunk];
#pragma unroll
            for (int i = 0; i < kTopkChunk; ++i) {
                tok[i] = c0 + i * NW;
                // clamped (always valid) addresses: the loads issue back to back
                const float *src = a.lbuf + (size_t)min(tok[i], a.T - 1) * E + min(lane, E - 1);
                lv[i] = DEV ? moe::load_dev(src) : *src;
            }
            if (a.logits && a.logits != a.lbuf && lane < E) {
#pragma unroll
                for (int i = 0; i < kTopkChunk; ++i)
                    if (tok[i] < a.T) a.logits[(size_t)tok[i] * E + lane] = lv[i];
            }
#pragma unroll
            for (int i = 0; i < kTopkChunk; i += kTopkBatch) {
                if (tok[i] >= a.T) break;                   // the rest of the chunk is past the batch
                int tb[kTopkBatch];
                float lb[kTopkBatch];
#pragma unroll
                for (int j = 0; j < kTopkBatch; ++j) {
                    tb[j] = tok[i + j];
                    lb[j] = lv[i + j];
                }
                topk_softmax_wave<kTopkBatch, DEV>(a, tb, lane, lb, S.ids);
            }
        }
        __syncthreads();
    }
    // ids of pair p: from LDS when this block just produced them, else from memory
    auto id_of = [&](int p) { return TOPK ? S.ids[p] : a.ids[p]; };
    const int p0 = (int)((long long)n * wave / NW), p1 = (int)((long long)n * (wave + 1) / NW);
    S.cnt[wave][lane] = 0;
    __syncthreads();
    for (int p = p0 + lane; p < p1; p += 64) {
        const int e = id_of(p);
        if (e >= 0 && e < E) atomicAdd(&S.cnt[wave][e], 1);
    }
    __syncthreads();
    if (wave == 0) {
        // per expert (lane): total count, exclusive prefix over experts, per-wave starts
        int c = 0;
        for (int w = 0; w < NW; ++w) c += (lane < E) ? S.cnt[w][lane] : 0;
        const int incl = moe::wave_inclusive_sum(c);
        const int excl = incl - c;
        int run = excl;
        for (int w = 0; w < NW; ++w) {
            S.base[w][lane] = run;
            run += (lane < E) ? S.cnt[w][lane] : 0;
        }
        const unsigned long long act = __ballot(lane < E && c > 0);
        const int na = __popcll(act);
        const unsigned long long below = (1ull << lane) - 1ull;
        if (lane < E) {
            moe::put<DEV>(&a.offsets[lane], (int32_t)excl);
            if (c > 0) moe::put<DEV>(&a.active[__popcll(act & below)], (int32_t)lane);
            if (lane >= na) moe::put<DEV>(&a.active[lane], (int32_t)-1);
            if (lane == E - 1) moe::put<DEV>(&a.offsets[E], (int32_t)incl);
        }
        if (lane == 0) moe::put<DEV>(&a.n_active[0], (int32_t)na);
    }
    __syncthreads();
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int c0 = p0; c0 < p1; c0 += 64) {
        const int p = c0 + lane;
        int e = p < p1 ? id_of(p) : -1;
        if (e >= E) e = -1;
        const unsigned long long peers = same_expert_lanes(e);
        if (e >= 0) {
            const int rank = __popcll(peers & below);
            const int pos = S.base[wave][e] + rank;
            moe::put<DEV>(&a.sorted_pairs[pos], (int32_t)p);
            moe::put<DEV>(&a.pair_pos[p], (int32_t)pos);
            if (rank == 0) S.base[wave][e] = pos + __popcll(peers);   // one leader per expert and chunk
        }
    }
}

// Small batches: block = (token t, group g of kGroupE experts) computes those
// logits (+ bias) into a.lbuf; route_group_kernel<true> then routes and
// groups.  fp64 pass: lane = EQ*hp + eq, EQ = kGroupE/VEC lanes per
// row, loads VEC experts of a row; rows h = RPW*(kSelWaves*i + wave) + hp,
// RPW = 64/EQ rows per wave step.  The first batch of router rows is loaded
// before the activation row is staged, so the two memory latencies overlap.
struct LogitsLds {
    double x[kMaxH];
    double acc[kSelWaves][kGroupE];
    float bnd[kSelWaves][kGroupE];
    long long red[kSelWaves][2];
    float logit[kGroupE];
    unsigned long long redo;
};

// DEV: the logits go to a.lbuf at device scope (read by another block of the
// same launch).
template <int VEC, bool DEV = false>
__device__ void logits_block(const RouteArgs &a, LogitsLds &S, int t, int g)
{
    constexpr int EQ = kGroupE / VEC;
    constexpr int RPW = 64 / EQ;
    // rows in flight per thread: 16 (two batches for H = 2048; 32 in one
    // batch measured no faster and needs 152 VGPRs instead of 96, too many
    // for a routing block to share a CU with another kernel's block)
    constexpr int U = VEC >= 8 ? 8 : 16;
    typedef WLoad<VEC> L;
    constexpr int kPath = kMaxH / (RPW * kSelWaves) + ilog2_ceil(RPW) + kSelWaves;
    constexpr int kErrExp = ilog2_ceil(kPath) + 1 - 53;
    static_assert(kErrExp <= -44, "summation paths of at most 256 additions");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.E, H = a.H;
    double *s_x = S.x;
    auto &s_acc = S.acc;
    auto &s_bnd = S.bnd;
    auto &s_red = S.red;
    float *s_logit = S.logit;
    unsigned long long &s_redo = S.redo;

    const int eq = lane % EQ, hp = lane / EQ;
    const int e0 = g * kGroupE + VEC * eq;          // first expert of this lane
    const uint16_t *wcol = a.wr + (e0 < E ? e0 : 0);
    const int step = RPW * kSelWaves;
    int h0 = RPW * wave + hp;
    typename L::T wv[U];
    // rows past H load a clamped (valid) row and use x = 0
    auto load_rows = [&](int hb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const unsigned int h = (unsigned int)min(hb + u * step, H - 1);
            wv[u] = L::ld(wcol + h * (unsigned int)E);
        }
    };
    // the x row first (it is needed first), then the router rows
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    u32x2 v[kMaxH / 4 / kSelThreads];
    {
        const u32x2 *src = reinterpret_cast<const u32x2 *>(a.x + (size_t)t * H);
#pragma unroll
        for (int r = 0; r < kMaxH / 4 / kSelThreads; ++r) v[r] = src[min(tid + r * kSelThreads, H / 4 - 1)];
    }
    __builtin_amdgcn_sched_barrier(0);     // keep the x loads ahead of the router loads
    load_rows(h0);

    {   // x row -> fp64 in LDS
#pragma unroll
        for (int r = 0; r < kMaxH / 4 / kSelThreads; ++r) {
            const int i = tid + r * kSelThreads;
            if (i < H / 4) {
#pragma unroll
                for (int j = 0; j < 4; ++j) s_x[4 * i + j] = h2d((uint16_t)(v[r][j >> 1] >> (16 * (j & 1))));
            }
        }
    }
    __syncthreads();

    double acc[VEC];
    float bnd[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) { acc[j] = 0.0; bnd[j] = 0.0f; }
    for (; h0 < H; h0 += U * step) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int h = h0 + u * step;
            const double xv = (h < H && e0 < E) ? s_x[h] : 0.0;
            const float xa = fabsf((float)xv);
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const float wf = (float)__builtin_bit_cast(_Float16, L::get(wv[u], j));
                acc[j] = fma(xv, (double)wf, acc[j]);              // exact product, fp64 sum
                bnd[j] = fmaf(xa, fabsf(wf), bnd[j]);              // sum |x*w| (for the error bound)
            }
        }
        if (h0 + U * step < H) load_rows(h0 + U * step);
    }
    // sum the RPW row phases within the wave (lanes eq, eq+EQ, ...)
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
        acc[j] = sum_phases<EQ>(acc[j]);
        bnd[j] = sum_phases<EQ>(bnd[j]);
    }
    if (hp == 0) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            s_acc[wave][VEC * eq + j] = acc[j];
            s_bnd[wave][VEC * eq + j] = bnd[j];
        }
    }
    __syncthreads();
    if (wave == 0) {
        const int e = g * kGroupE + lane;
        double v = 0.0;
        float B = 0.0f;
        if (lane < kGroupE) {
            for (int r = 0; r < kSelWaves; ++r) {
                v += s_acc[r][lane];
                B += s_bnd[r][lane];
            }
        }
        // Any summation path above has at most n = H/(RPW*kSelWaves) +
        // log2(RPW) + kSelWaves fp64 additions (kPath, H <= kMaxH), so
        // |v - exact| <= n * 2^-53 * sum|x*w| * (1 + n 2^-53); B (FP32, at
        // most n roundings) is within a factor 1 + 2^-16 of the true sum|x*w|.
        // Hence err = 2^(ceil(log2 n) + 1 - 53) * B covers it.
        const double err = ldexp((double)B, kErrExp);
        const bool certain = lane >= kGroupE || e >= E || (!a.force_exact && rn32_certain(v, err));
        if (lane < kGroupE) s_logit[lane] = (float)v;
        const unsigned long long m = __ballot(!certain);
        if (lane == 0) s_redo = m;
    }
    __syncthreads();
    unsigned long long redo = s_redo;
    while (redo) {                                   // rare: exact recomputation by the whole block
        const int j = __builtin_ctzll(redo);
        redo &= redo - 1ull;
        const float l = exact_logit(a, s_x, g * kGroupE + j, s_red);
        if (tid == 0) s_logit[j] = l;
    }
    __syncthreads();
    if (tid < kGroupE) {
        const int e = g * kGroupE + tid;
        if (e < E) {
            float lv = s_logit[tid];
            if (a.bias) lv = lv + a.bias[e];
            if (DEV) moe::store_dev(&a.lbuf[(size_t)t * E + e], lv);
            else a.lbuf[(size_t)t * E + e] = lv;
        }
    }
}

// Small batches in one launch: every logits task (token, expert group) is
// computed as route_logits_kernel does and stored at device scope; once it
// is complete its block counts itself in `done`, and the block that counts
// last (no block ever waits for another) runs the top-k and the grouping over
// all logits, read at device scope, and resets the counter for the next call.
union FusedRouteLds {
    LogitsLds lg;
    GroupLds<kSelWaves, true> gr;
};

// Logits task `task` of `ntask` (token task / G, expert group task % G, G
// groups of kGroupE experts).
template <int VEC>
__device__ inline void fused_route_task(const RouteArgs &a, FusedRouteLds &S, int &s_last, unsigned int *done, int task,
                                        int ntask)
{
    const int G = (a.E + kGroupE - 1) / kGroupE;
    logits_block<VEC, true>(a, S.lg, task / G, task % G);
    moe::wait_stores();                                     // this wave's logits are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned int before = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = before == (unsigned int)ntask - 1;
    }
    __syncthreads();
    if (!s_last) return;
    group_phase<kSelWaves, true, true>(a, S.gr);
    if (threadIdx.x == 0) *done = 0u;
}

}  // namespace
