// Routing for the W4A16 routed-expert layer: router logits, top-k softmax and
// token-to-expert grouping in one launch.
//
// Routing selects the experts of each token at every routed layer
// ("horizonrunmap.com/en", section "06 / Follow a token", step "Select
// experts"); the router keeps FP16 weights outside INT4 (section "08 /
// Precision & quality", paragraph "Other components").  The pages give no
// router formula; the logit is the correctly rounded FP32 value of the exact
// FP16 dot product, so expert selection is independent of summation order.
//
// Launch shape: one block per (token, slice of H).  Each block accumulates
// its slice of every logit of its token exactly, as integers, and stores the
// partial sums in its own workspace slot (plain stores: no two blocks write
// the same address, so nothing contends).  A per-token ticket (one atomic per
// block, released after the stores) finds the block that completes a token;
// that block acquires, adds the slices exactly, rounds the logits to FP32 and
// runs top-k and softmax in one wavefront (lane = expert).  The block that
// completes the last token runs the counting sort for all T*k pairs.  No
// block ever waits for another, so every block exits.
#include "moe_internal.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kSubs = kThreads / 64;     // H sub-slices per block (one wave each)
constexpr int kSplit = 30;               // products with shift < kSplit go to the low limb
constexpr int kMaxSlice = 256;           // router rows staged in LDS per block
constexpr int kMaxSlices = 32;           // H slices per token (sizes the partial-sum workspace)

// Agent-scope loads/stores for data handed between blocks of one launch.
template <typename T>
__device__ inline T ld_agent(const T *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename T>
__device__ inline void st_agent(T *p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// FP16 bits -> signed integer significand m and exponent field q, value = m * 2^(q-25).
__device__ inline void dec16(uint32_t b, int &m, int &q)
{
    const int e = (b >> 10) & 31;
    const int mag = (b & 0x3ff) | (e ? 0x400 : 0);
    m = (b & 0x8000) ? -mag : mag;
    q = e ? e : 1;
}

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

struct RouteArgs {
    const uint16_t *x;      // [T][H]
    const uint16_t *wr;     // [H][E]
    const float *bias;      // [E] or null
    int T, H, E, k, HS;     // HS = H slices per token
    long long *part;        // [T][HS][E][2] exact partial limbs (hi, lo) per slice
    unsigned int *tok_ticket;   // [T]
    unsigned int *glob_ticket;  // [1]
    float *logits;          // [T][E] or null
    int32_t *ids;           // [T][k]
    float *w;               // [T][k]
    int32_t *offsets;       // [E+1]
    int32_t *sorted_pairs;  // [T*k]
    int32_t *pair_pos;      // [T*k]
    int32_t *active;        // [E]
    int32_t *n_active;      // [1]
};

// Top-k + softmax of token t, executed by one full wavefront; lane = expert,
// (hi, lo) = the exact logit limbs of that expert.
__device__ void finalize_token(const RouteArgs &a, int t, int lane, long long hi, long long lo)
{
    const int E = a.E, k = a.k;
    float v = 0.0f;
    if (lane < E) {
        v = rn32_limbs(hi, lo);
        if (a.bias) v = v + a.bias[lane];
        if (a.logits) a.logits[(size_t)t * E + lane] = v;
    }
    bool live = lane < E;
    float selv[MOE_MAX_TOPK];
    int seli[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        selv[j] = 0.0f;
        seli[j] = 0;
        if (j >= k) continue;
        float bv = v;
        int bi = live ? lane : 64;                       // 64 = no candidate
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            // order: a candidate beats none; larger value; on equal value, lower index
            const bool take = oi < 64 && (bi == 64 || ov > bv || (ov == bv && oi < bi));
            if (take) { bv = ov; bi = oi; }
        }
        selv[j] = bv;
        seli[j] = bi;
        if (lane == bi) live = false;
    }
    // softmax over the k selected logits (loops fully unrolled: the arrays stay in registers)
    float ex[MOE_MAX_TOPK];
    float den = 0.0f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        ex[j] = 0.0f;
        if (j < k) {
            ex[j] = expf(selv[j] - selv[0]);
            den += ex[j];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK; ++j) {
            if (j < k) {
                st_agent(&a.ids[(size_t)t * k + j], (int32_t)seli[j]);
                a.w[(size_t)t * k + j] = ex[j] / den;
            }
        }
    }
}

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

// Stable counting sort of all pairs by expert; run by the last block.
// Counts: LDS atomics over all threads.  Offsets and the active list: one
// wave, prefix sum by shuffles.  Scatter: wave 0 walks the pairs in order, 64
// at a time; a pair's place among equal experts of its chunk comes from a
// ballot, and each expert's running base advances by its chunk count.
__device__ void group_pairs(const RouteArgs &a)
{
    __shared__ int cnt[MOE_MAX_EXPERTS];
    __shared__ int base[MOE_MAX_EXPERTS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int n = a.T * a.k, E = a.E;
    if (tid < MOE_MAX_EXPERTS) cnt[tid] = 0;
    __syncthreads();
    for (int p = tid; p < n; p += kThreads) {
        const int e = ld_agent(&a.ids[p]);
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (tid >= 64) return;                  // wave 0 only from here
    const int c = lane < E ? cnt[lane] : 0;
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    const int excl = incl - c;
    const unsigned long long act = __ballot(c > 0);
    const int na = __popcll(act);
    const unsigned long long below = (1ull << lane) - 1ull;
    if (lane < E) {
        a.offsets[lane] = excl;
        base[lane] = excl;
        if (c > 0) a.active[__popcll(act & below)] = lane;
        if (lane >= na) a.active[lane] = -1;
        if (lane == E - 1) a.offsets[E] = incl;
    }
    if (lane == 0) a.n_active[0] = na;
    for (int c0 = 0; c0 < n; c0 += 64) {
        const int p = c0 + lane;
        int e = p < n ? ld_agent(&a.ids[p]) : -1;
        if (e >= E) e = -1;
        const unsigned long long peers = same_expert_lanes(e);
        if (e >= 0) {
            const int rank = __popcll(peers & below);
            const int pos = base[e] + rank;
            a.sorted_pairs[pos] = p;
            a.pair_pos[p] = pos;
            if (rank == 0) base[e] = pos + __popcll(peers);     // one leader per expert and chunk
        }
    }
}

__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a)
{
    const int t = blockIdx.x / a.HS;
    const int c = blockIdx.x % a.HS;
    const int tid = threadIdx.x, lane = tid & 63, sub = tid >> 6;
    const int E = a.E;
    const int slice = a.H / a.HS;            // multiple of 32, at most kMaxSlice
    const int per = slice / kSubs;           // multiple of 8
    const int h0 = c * slice;

    // Stage the router rows h0 .. h0+slice-1 (contiguous, 16-byte aligned) and
    // the token's decoded activations in LDS.
    __shared__ u32x4 s_w[kMaxSlice * MOE_MAX_EXPERTS * 2 / 16];
    __shared__ int2 s_x[kMaxSlice];
    {
        // all loads first (one memory latency), then the LDS writes
        const u32x4 *src = reinterpret_cast<const u32x4 *>(a.wr + (size_t)h0 * E);
        const int n16 = slice * E * 2 / 16;
        constexpr int kPer = kMaxSlice * MOE_MAX_EXPERTS * 2 / 16 / kThreads;
        u32x4 v[kPer];
#pragma unroll
        for (int r = 0; r < kPer; ++r) {                 // unconditional: indices clamped into the slice
            const int i = min(tid + r * kThreads, n16 - 1);
            v[r] = src[i];
        }
        uint16_t xb = 0;
        if (tid < slice) xb = a.x[(size_t)t * a.H + h0 + tid];
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int i = tid + r * kThreads;
            if (i < n16) s_w[i] = v[r];
        }
        if (tid < slice) {
            int m, q;
            dec16(xb, m, q);
            s_x[tid] = make_int2(m, q - 2);
        }
    }
    __syncthreads();
    const uint16_t *sw = reinterpret_cast<const uint16_t *>(s_w);

    // exact partial sums of this thread's h range for expert `lane`
    long long hi = 0, lo = 0;
    if (lane < E) {
#pragma unroll 8
        for (int i = sub * per; i < sub * per + per; ++i) {
            const int2 xv = s_x[i];
            int mw, qw;
            dec16(sw[i * E + lane], mw, qw);
            const long long prod = (long long)(xv.x * mw);     // |prod| < 2^22
            const int sh = xv.y + qw;                          // product = prod * 2^(sh-48), sh in [0, 58]
            if (sh < kSplit) lo += (long long)((unsigned long long)prod << sh);
            else hi += (long long)((unsigned long long)prod << (sh - kSplit));
        }
    }
    __shared__ long long red[kSubs][64][2];
    red[sub][lane][0] = hi;
    red[sub][lane][1] = lo;
    __syncthreads();
    if (sub == 0 && lane < E) {
        long long shi = 0, slo = 0;
        for (int s = 0; s < kSubs; ++s) { shi += red[s][lane][0]; slo += red[s][lane][1]; }
        // write-through (agent-scope) stores: nothing is left dirty in this
        // XCD's L2 for the release below to write back
        long long *p = a.part + (((size_t)t * a.HS + c) * E + lane) * 2;
        st_agent(p, shi);
        st_agent(p + 1, slo);
    }
    // Completion: the ticket increment is a release by wave 0, which stored
    // the partial sums; only the block that takes the last ticket acquires.
    // (A full fence in every block would write back and invalidate the L2 of
    // its XCD each time.)
    __shared__ int last_slice, last_token;
    if (tid == 0) {
        const unsigned int prev =
            __hip_atomic_fetch_add(&a.tok_ticket[t], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        last_slice = (prev == (unsigned int)a.HS - 1u);
    }
    __syncthreads();
    if (!last_slice) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // exact sum of the token's slices: wave `sub` adds slices sub, sub+4, ...
    hi = 0;
    lo = 0;
    if (lane < E) {
#pragma unroll
        for (int r = 0; r < kMaxSlices / kSubs; ++r) {
            const int cc = sub + r * kSubs;
            if (cc < a.HS) {
                const long long *p = a.part + (((size_t)t * a.HS + cc) * E + lane) * 2;
                hi += ld_agent(p);
                lo += ld_agent(p + 1);
            }
        }
    }
    __syncthreads();                    // everyone is done with red from the block reduction
    red[sub][lane][0] = hi;
    red[sub][lane][1] = lo;
    __syncthreads();
    if (sub == 0) {
        long long shi = 0, slo = 0;
        for (int s = 0; s < kSubs; ++s) { shi += red[s][lane][0]; slo += red[s][lane][1]; }
        finalize_token(a, t, lane, shi, slo);
        if (lane == 0) st_agent(&a.tok_ticket[t], 0u);
    }
    if (tid == 0) {
        const unsigned int prev = __hip_atomic_fetch_add(a.glob_ticket, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        last_token = (prev == (unsigned int)a.T - 1u);
    }
    __syncthreads();
    if (!last_token) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    group_pairs(a);
    if (tid == 0) st_agent(a.glob_ticket, 0u);
}

size_t align_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

struct WsLayout {
    size_t part, tok, glob, total;
};

// Workspace: tickets first (they must start at zero and are left at zero),
// then the partial sums (fully written before they are read).
WsLayout ws_layout(int T, int HS, int E)
{
    WsLayout L;
    L.tok = 0;
    L.glob = align_up((size_t)T * sizeof(unsigned int), 256);
    L.part = L.glob + 256;
    L.total = L.part + align_up((size_t)T * HS * E * 2 * sizeof(long long), 256);
    return L;
}

// Number of H slices per token: a divisor of H/32 (slices hold a multiple of
// 32 rows) with slices of 128 .. kMaxSlice rows where H allows, at most
// kMaxSlices, chosen to give a small batch about 256 blocks.
int pick_slices(int T, int H)
{
    const int units = H / 32;
    const int min_hs = (H + kMaxSlice - 1) / kMaxSlice;
    int max_hs = H / 128 > min_hs ? H / 128 : min_hs;
    if (max_hs > kMaxSlices) max_hs = kMaxSlices;
    const int target = 256 / (T > 0 ? T : 1);
    int best = -1;
    for (int d = 1; d <= units; ++d) {
        if (units % d || d < min_hs || d > max_hs) continue;
        if (best < 0) best = d;                 // smallest admissible
        if (d <= target) best = d;              // largest admissible not above the target
    }
    return best;
}

}  // namespace

extern "C" {

size_t moe_route_workspace_size(int T, int H, int E)
{
    if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || H <= 0 || H % 128 || H > 4096) return 0;
    const int HS = pick_slices(T, H);
    if (HS < 1) return 0;
    return ws_layout(T, HS, E).total;
}

int moe_route(const void *x_dev, const void *w_router_dev, const float *bias_dev,
              int T, int H, int E, int k,
              float *logits_dev, int32_t *topk_ids_dev, float *topk_w_dev,
              int32_t *expert_offsets_dev, int32_t *sorted_pairs_dev, int32_t *pair_pos_dev,
              int32_t *active_list_dev, int32_t *n_active_dev,
              void *ws_dev, size_t ws_bytes, void *stream)
{
    moe::clear_error();
    int rc = moe::check_shape(T, H, 0, E, k, false);
    if (rc) return rc;
    if (H > 4096) return moe::fail(MOE_ERR_UNSUPPORTED, "moe_route: H=%d > 4096", H);
    if (T == 0) return MOE_OK;
    if (!x_dev || !w_router_dev || !topk_ids_dev || !topk_w_dev || !expert_offsets_dev || !sorted_pairs_dev ||
        !pair_pos_dev || !active_list_dev || !n_active_dev)
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_route: null pointer argument");
    if (!moe::aligned(x_dev, 2) || !moe::aligned(w_router_dev, 16))
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_route: x must be 2-byte and w_router 16-byte aligned");
    const int HS = pick_slices(T, H);
    if (HS < 1) return moe::fail(MOE_ERR_UNSUPPORTED, "moe_route: no slicing of H=%d", H);
    const WsLayout L = ws_layout(T, HS, E);
    if (!ws_dev || ws_bytes < L.total || !moe::aligned(ws_dev, 256))
        return moe::fail(MOE_ERR_WORKSPACE, "moe_route: workspace needs %zu bytes, 256-byte aligned", L.total);

    RouteArgs a;
    a.x = (const uint16_t *)x_dev;
    a.wr = (const uint16_t *)w_router_dev;
    a.bias = bias_dev;
    a.T = T; a.H = H; a.E = E; a.k = k;
    a.HS = HS;
    char *ws = (char *)ws_dev;
    a.part = (long long *)(ws + L.part);
    a.tok_ticket = (unsigned int *)(ws + L.tok);
    a.glob_ticket = (unsigned int *)(ws + L.glob);
    a.logits = logits_dev;
    a.ids = topk_ids_dev;
    a.w = topk_w_dev;
    a.offsets = expert_offsets_dev;
    a.sorted_pairs = sorted_pairs_dev;
    a.pair_pos = pair_pos_dev;
    a.active = active_list_dev;
    a.n_active = n_active_dev;
    const unsigned int blocks = (unsigned int)T * (unsigned int)a.HS;
    hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, a);
    return moe::check_launch("moe_route");
}

}  // extern "C"
