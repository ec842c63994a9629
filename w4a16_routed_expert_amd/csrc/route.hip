// Routing for the W4A16 routed-expert layer: router logits, top-k softmax and
// token-to-expert grouping.
//
// Routing selects the experts of each token at every routed layer
// ("horizonrunmap.com/en", section "06 / Follow a token", step "Select
// experts"); the router keeps FP16 weights outside INT4 (section "08 /
// Precision & quality", paragraph "Other components").  The pages give no
// router formula; the logit is the correctly rounded FP32 value of the exact
// FP16 dot product, so expert selection is independent of summation order.
//
// Logits: every FP16 x FP16 product is exact in fp64; a block sums them in
// fp64 and, alongside, sum |x*w| in FP32.  A standard bound on the fp64
// summation error (at most n roundings of relative size 2^-53 along any
// summation path) then tells whether the fp64 sum and the exact sum round to
// the same FP32 value: true unless the exact value lies within that bound of
// an FP32 rounding midpoint.  Logits that fail the test (exact ties at a
// midpoint among them) are recomputed exactly with 64-bit integer limbs by
// the whole block.
//   Small batches (decode): route_logits_kernel, one block per (token, group
//   of 16 experts), spreads the logits over many CUs; route_group_kernel (one
//   block) then runs top-k + softmax per token (one wavefront per token, lane
//   = expert) and the stable counting sort of the T*k pairs.
//   Large batches (prefill): route_select_kernel, one block per 4 tokens
//   (every router row loaded serves the 4), does logits, top-k and softmax;
//   route_count_kernel and route_scatter_kernel sort on many blocks.
#include "moe_internal.h"

#include <climits>
#include <mutex>

#include "route_dev.h"

namespace {

// One block per token.  fp64 pass: lane = (64/VEC)*hp + eq handles experts
// VEC*eq .. VEC*eq+VEC-1 (one vector load per row) and rows
// h = PH*(kSelWaves*i + wave) + hp, PH = 64*VEC/64 row phases per wave.
// Prefill: TB tokens per block share every router row loaded (the router is
// read once per TB tokens); x rows stay FP16 in LDS (small enough for two
// blocks per CU).
template <int VEC, int TB>
__global__ __launch_bounds__(kSelThreads) void route_select_kernel(RouteArgs a)
{
    constexpr int EQ = 64 / VEC;             // lanes sharing one row
    constexpr int PH = VEC;                  // rows per wave step (64 / EQ)
    constexpr int U = 4;                     // rows in flight per thread
    constexpr int kPath = kMaxH / (PH * kSelWaves) + ilog2_ceil(PH) + kSelWaves;
    constexpr int kErrExp = ilog2_ceil(kPath) + 1 - 53;
    static_assert(TB <= kSelWaves, "one wavefront per token for the selection");
    typedef WLoad<VEC> L;
    const int t0 = blockIdx.x * TB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.E, H = a.H, T = a.T;
    __shared__ _Float16 s_x[TB][kMaxH];
    __shared__ double s_acc[kSelWaves][TB][64];
    __shared__ float s_wsq[kSelWaves][64];
    __shared__ float s_xsq[TB];
    __shared__ long long s_red[kSelWaves][2];
    __shared__ float s_logit[TB][64];
    __shared__ unsigned long long s_redo[TB];

    {   // x rows -> FP32 in LDS, 4 values per thread per step, all loads first
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        constexpr int R = TB * kMaxH / 4 / kSelThreads;
        const int q4 = H / 4;
        u32x2 v[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = tid + r * kSelThreads;          // (token i / q4, quad i % q4)
            const int tt = i / q4, qq = i - tt * q4;
            const bool ok = tt < TB && t0 + tt < T;
            v[r] = ok ? reinterpret_cast<const u32x2 *>(a.x + (size_t)(t0 + tt) * H)[qq] : u32x2{0u, 0u};
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = tid + r * kSelThreads;
            const int tt = i / q4, qq = i - tt * q4;
            if (tt < TB) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    s_x[tt][4 * qq + j] = __builtin_bit_cast(_Float16, (uint16_t)(v[r][j >> 1] >> (16 * (j & 1))));
            }
        }
    }
    __syncthreads();
    if (wave < TB) {
        // sum of x^2 of token `wave` (squares exact in FP32)
        float q = 0.0f;
        for (int h = lane; h < H; h += 64) {
            const float xf = (float)s_x[wave][h];
            q = fmaf(xf, xf, q);
        }
        q = sum_phases<1>(q);
        if (lane == 0) s_xsq[wave] = q;
    }
    const int eq = lane % EQ, hp = lane / EQ;
    const int e0 = VEC * eq;
    double acc[TB][VEC];
    float wsq[VEC];                           // sum of w^2 per expert (the error bound)
#pragma unroll
    for (int j = 0; j < VEC; ++j) wsq[j] = 0.0f;
#pragma unroll
    for (int tt = 0; tt < TB; ++tt)
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc[tt][j] = 0.0;
    if (e0 < E) {
        const uint16_t *wcol = a.wr + e0;
        const int step = PH * kSelWaves;
        // branch-free body: rows past H load a clamped (valid) row and use x = 0
        for (int h0 = PH * wave + hp; h0 < H; h0 += U * step) {
            typename L::T wv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const unsigned int h = (unsigned int)min(h0 + u * step, H - 1);
                wv[u] = L::ld(wcol + h * (unsigned int)E);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int h = h0 + u * step;
                float wf[VEC];
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    wf[j] = h < H ? (float)__builtin_bit_cast(_Float16, L::get(wv[u], j)) : 0.0f;
                    wsq[j] = fmaf(wf[j], wf[j], wsq[j]);
                }
#pragma unroll
                for (int tt = 0; tt < TB; ++tt) {
                    const double xv = (double)(float)s_x[tt][min(h, H - 1)];
#pragma unroll
                    for (int j = 0; j < VEC; ++j) acc[tt][j] = fma(xv, (double)wf[j], acc[tt][j]);   // exact product, fp64 sum
                }
            }
        }
    }
    // sum the PH row phases of each expert within the wave (lanes eq, eq+EQ, ...)
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) acc[tt][j] = sum_phases<EQ>(acc[tt][j]);
        wsq[j] = sum_phases<EQ>(wsq[j]);
    }
    if (hp == 0) {
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
#pragma unroll
            for (int tt = 0; tt < TB; ++tt) s_acc[wave][tt][e0 + j] = acc[tt][j];
            s_wsq[wave][e0 + j] = wsq[j];
        }
    }
    __syncthreads();
    if (wave < TB) {
        const int tt = wave;
        double v = 0.0;
        float W = 0.0f;
        for (int r = 0; r < kSelWaves; ++r) {
            v += s_acc[r][tt][lane];
            W += s_wsq[r][lane];
        }
        // Any summation path above has at most n = H/(PH*kSelWaves) +
        // log2(PH) + kSelWaves fp64 additions (kPath, H <= kMaxH), so
        // |v - exact| <= n * 2^-53 * sum|x*w| * (1 + n 2^-53).  By
        // Cauchy-Schwarz sum|x*w| <= sqrt(sum x^2 * sum w^2); both FP32 sums of
        // exact squares (at most H roundings, H <= 4096) are within a factor
        // 1 + 2^-11 of their true values, so B = sqrt(X W) (1 + 2^-10) bounds
        // sum|x*w|, and err = 2^(ceil(log2 n) + 1 - 53) * B covers the error.
        const double B = sqrt((double)s_xsq[tt] * (double)W) * (1.0 + 0x1p-10);
        const double err = ldexp(B, kErrExp);
        const bool certain = lane >= E || t0 + tt >= T || (!a.force_exact && rn32_certain(v, err));
        s_logit[tt][lane] = (float)v;
        const unsigned long long m = __ballot(!certain);
        if (lane == 0) s_redo[tt] = m;
    }
    __syncthreads();
    for (int tt = 0; tt < TB; ++tt) {
        unsigned long long redo = s_redo[tt];
        while (redo) {                               // rare: exact recomputation by the whole block
            const int e = __builtin_ctzll(redo);
            redo &= redo - 1ull;
            const float l = exact_logit(a, &s_x[tt][0], e, s_red);
            if (tid == 0) s_logit[tt][e] = l;
        }
    }
    __syncthreads();
    if (wave >= TB || t0 + wave >= T) return;

    // logits (+ bias), then top-k and softmax, lane = expert
    const int t = t0 + wave;
    float lv = 0.0f;
    if (lane < E) {
        lv = s_logit[wave][lane];
        if (a.bias) lv = lv + a.bias[lane];
        if (a.logits) a.logits[(size_t)t * E + lane] = lv;
    }
    const int tok[1] = {t};
    const float l1[1] = {lv};
    topk_softmax_wave<1>(a, tok, lane, l1, nullptr);
}

template <int VEC>
__global__ __launch_bounds__(kSelThreads) void route_logits_kernel(RouteArgs a)
{
    __shared__ LogitsLds S;
    const int G = (a.E + kGroupE - 1) / kGroupE;
    logits_block<VEC>(a, S, blockIdx.x / G, blockIdx.x % G);
}

// One block: top-k + softmax of every token from a.lbuf (TOPK), then the
// grouping.
template <bool TOPK>
__global__ __launch_bounds__(kGrpThreads) void route_group_kernel(RouteArgs a)
{
    __shared__ GroupLds<kGrpWaves, TOPK> s_grp;
    group_phase<kGrpWaves, TOPK>(a, s_grp);
}

// Small batches in one launch (the fused layer, moe_layer_forward): block b
// runs logits task b (fused_route_task in route_dev.h).
template <int VEC>
__global__ __launch_bounds__(kSelThreads) void route_fused_kernel(RouteArgs a, unsigned int *done)
{
    __shared__ FusedRouteLds S;
    __shared__ int s_last;
    fused_route_task<VEC>(a, S, s_last, done, blockIdx.x, gridDim.x);
}

// Large batches: the stable counting sort runs on many blocks (one single
// block would send every scattered store through one CU).  Segment g holds
// pairs [g kSeg, (g + 1) kSeg); route_count_kernel writes its per-expert
// counts to the workspace; route_scatter_kernel then gives each segment its
// starting position per expert (all earlier segments' counts plus the
// expert's offset) and places the segment's pairs in order.
constexpr int kSeg = 256;

__global__ __launch_bounds__(kSeg) void route_count_kernel(RouteArgs a)
{
    __shared__ int cnt[MOE_MAX_EXPERTS];
    const int g = blockIdx.x, n = a.T * a.k, E = a.E;
    if (threadIdx.x < MOE_MAX_EXPERTS) cnt[threadIdx.x] = 0;
    __syncthreads();
    const int p = g * kSeg + (int)threadIdx.x;
    if (p < n) {
        const int e = a.ids[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if ((int)threadIdx.x < E) reinterpret_cast<int *>(a.lbuf)[(size_t)g * E + threadIdx.x] = cnt[threadIdx.x];
}

__global__ __launch_bounds__(kSeg) void route_scatter_kernel(RouteArgs a, int G)
{
    constexpr int NWV = kSeg / 64;
    __shared__ int s_tot[NWV][64], s_pre[NWV][64];
    __shared__ int s_base[64];
    const int g = blockIdx.x, n = a.T * a.k, E = a.E;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int *cnt = reinterpret_cast<const int *>(a.lbuf);
    // expert `lane`: total count and the count of segments before this one
    // (wavefront w sums the segments g' = w mod NWV)
    int tot = 0, pre = 0;
    if (lane < E) {
#pragma unroll 8
        for (int q = wave; q < G; q += NWV) {
            const int c = cnt[(size_t)q * E + lane];
            tot += c;
            if (q < g) pre += c;
        }
    }
    s_tot[wave][lane] = tot;
    s_pre[wave][lane] = pre;
    __syncthreads();
    if (wave != 0) return;
    int c = 0, pr = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
        c += s_tot[w][lane];
        pr += s_pre[w][lane];
    }
    const int incl = moe::wave_inclusive_sum(c);
    const int excl = incl - c;
    s_base[lane] = excl + pr;
    if (g == 0) {
        const unsigned long long act = __ballot(lane < E && c > 0);
        const int na = __popcll(act);
        const unsigned long long below = (1ull << lane) - 1ull;
        if (lane < E) {
            a.offsets[lane] = excl;
            if (c > 0) a.active[__popcll(act & below)] = lane;
            if (lane >= na) a.active[lane] = -1;
            if (lane == E - 1) a.offsets[E] = incl;
        }
        if (lane == 0) a.n_active[0] = na;
    }
    // the segment's pairs 64 at a time, in order; a pair's rank among equal
    // experts of its chunk comes from a ballot
    const int b0 = g * kSeg, b1 = min(n, b0 + kSeg);
    int ids[kSeg / 64];
#pragma unroll
    for (int i = 0; i < kSeg / 64; ++i) {
        const int p = b0 + 64 * i + lane;
        ids[i] = p < b1 ? a.ids[p] : -1;
    }
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < kSeg / 64; ++i) {
        const int p = b0 + 64 * i + lane;
        int e = ids[i];
        if (e >= E) e = -1;
        const unsigned long long peers = same_expert_lanes(e);
        if (e >= 0) {
            const int rank = __popcll(peers & below);
            const int pos = s_base[e] + rank;
            a.sorted_pairs[pos] = p;
            a.pair_pos[p] = pos;
            if (rank == 0) s_base[e] = pos + __popcll(peers);   // one leader per expert and chunk
        }
    }
}

constexpr int kSmallBatch = 256;           // largest T routed with the split logits kernel

// Workspace: the logits [T][E] handed from the logit blocks to the grouping block.
size_t route_ws_bytes(int T, int E) { return ((size_t)T * E * sizeof(float) + 255) / 256 * 256; }

int route_launch(const void *x_dev, const void *w_router_dev, const float *bias_dev, int T, int H, int E, int k,
                 float *logits_dev, int32_t *topk_ids_dev, float *topk_w_dev, int32_t *expert_offsets_dev,
                 int32_t *sorted_pairs_dev, int32_t *pair_pos_dev, int32_t *active_list_dev, int32_t *n_active_dev,
                 void *ws_dev, size_t ws_bytes, int force_exact, void *stream)
{
    moe::clear_error();
    int rc = moe::check_shape(T, H, 0, E, k, false);
    if (rc) return rc;
    if (H > kMaxH) return moe::fail(MOE_ERR_UNSUPPORTED, "moe_route: H=%d > %d", H, kMaxH);
    if (T == 0) return MOE_OK;
    if (!x_dev || !w_router_dev || !topk_ids_dev || !topk_w_dev || !expert_offsets_dev || !sorted_pairs_dev ||
        !pair_pos_dev || !active_list_dev || !n_active_dev)
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_route: null pointer argument");
    if (!moe::aligned(x_dev, 8) || !moe::aligned(w_router_dev, 2))
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_route: x must be 8-byte and w_router 2-byte aligned");
    const bool small = T <= kSmallBatch;
    if (!ws_dev || ws_bytes < route_ws_bytes(T, E) || !moe::aligned(ws_dev, 256))
        return moe::fail(MOE_ERR_WORKSPACE, "moe_route: the workspace needs %zu bytes, 256-byte aligned",
                         route_ws_bytes(T, E));
    float *lbuf = (float *)ws_dev;

    RouteArgs a;
    a.x = (const uint16_t *)x_dev;
    a.wr = (const uint16_t *)w_router_dev;
    a.bias = bias_dev;
    a.T = T; a.H = H; a.E = E; a.k = k;
    a.logits = logits_dev;
    a.ids = topk_ids_dev;
    a.w = topk_w_dev;
    a.offsets = expert_offsets_dev;
    a.sorted_pairs = sorted_pairs_dev;
    a.pair_pos = pair_pos_dev;
    a.active = active_list_dev;
    a.n_active = n_active_dev;
    a.force_exact = force_exact;
    a.lbuf = lbuf;
    hipStream_t s = (hipStream_t)stream;
    // widest router-row load the layout allows for the prefill kernel: 4 experts per lane, else 1
    const bool v4 = E % 4 == 0 && moe::aligned(w_router_dev, 8);
    if (small) {
        const unsigned int blocks = (unsigned int)T * (unsigned int)((E + kGroupE - 1) / kGroupE);
        // two experts per lane: short cross-lane sums, 4-byte router loads
        if (E % 2 == 0 && moe::aligned(w_router_dev, 4))
            hipLaunchKernelGGL(route_logits_kernel<2>, dim3(blocks), dim3(kSelThreads), 0, s, a);
        else hipLaunchKernelGGL(route_logits_kernel<1>, dim3(blocks), dim3(kSelThreads), 0, s, a);
        rc = moe::check_launch("moe_route (logits)");
        if (rc) return rc;
        hipLaunchKernelGGL(route_group_kernel<true>, dim3(1), dim3(kGrpThreads), 0, s, a);
        return moe::check_launch("moe_route (top-k, group)");
    }
    const unsigned int sel_blocks = (unsigned int)((T + kSelTokens - 1) / kSelTokens);
    // four experts per lane: with 4 tokens, 8 per lane would not fit the registers
    if (v4) hipLaunchKernelGGL((route_select_kernel<4, kSelTokens>), dim3(sel_blocks), dim3(kSelThreads), 0, s, a);
    else hipLaunchKernelGGL((route_select_kernel<1, kSelTokens>), dim3(sel_blocks), dim3(kSelThreads), 0, s, a);
    rc = moe::check_launch("moe_route (select)");
    if (rc) return rc;
    // segment counts fit the logits workspace: G <= T (kSeg >= k)
    const int G = (T * k + kSeg - 1) / kSeg;
    hipLaunchKernelGGL(route_count_kernel, dim3((unsigned int)G), dim3(kSeg), 0, s, a);
    rc = moe::check_launch("moe_route (count)");
    if (rc) return rc;
    hipLaunchKernelGGL(route_scatter_kernel, dim3((unsigned int)G), dim3(kSeg), 0, s, a, G);
    return moe::check_launch("moe_route (scatter)");
}

}  // namespace

int moe::route_fused(const void *x_dev, const void *w_router_dev, const float *bias_dev, int T, int H, int E, int k,
                     float *logits_dev, int32_t *topk_ids_dev, float *topk_w_dev, int32_t *expert_offsets_dev,
                     int32_t *sorted_pairs_dev, int32_t *pair_pos_dev, int32_t *active_list_dev,
                     int32_t *n_active_dev, float *lbuf, unsigned int *done, hipStream_t s)
{
    if (T < 1 || T > kSmallBatch) return moe::fail(MOE_ERR_UNSUPPORTED, "fused routing: T=%d outside [1, %d]", T,
                                                   kSmallBatch);
    if (H > kMaxH) return moe::fail(MOE_ERR_UNSUPPORTED, "fused routing: H=%d > %d", H, kMaxH);
    if (!moe::aligned(x_dev, 8) || !moe::aligned(w_router_dev, 2))
        return moe::fail(MOE_ERR_INVALID_ARG, "fused routing: x must be 8-byte and w_router 2-byte aligned");
    RouteArgs a;
    a.x = (const uint16_t *)x_dev;
    a.wr = (const uint16_t *)w_router_dev;
    a.bias = bias_dev;
    a.T = T; a.H = H; a.E = E; a.k = k;
    a.logits = logits_dev;
    a.ids = topk_ids_dev;
    a.w = topk_w_dev;
    a.offsets = expert_offsets_dev;
    a.sorted_pairs = sorted_pairs_dev;
    a.pair_pos = pair_pos_dev;
    a.active = active_list_dev;
    a.n_active = n_active_dev;
    a.force_exact = 0;
    a.lbuf = lbuf;
    const unsigned int blocks = (unsigned int)T * (unsigned int)((E + kGroupE - 1) / kGroupE);
    if (E % 2 == 0 && moe::aligned(w_router_dev, 4))
        hipLaunchKernelGGL(route_fused_kernel<2>, dim3(blocks), dim3(kSelThreads), 0, s, a, done);
    else hipLaunchKernelGGL(route_fused_kernel<1>, dim3(blocks), dim3(kSelThreads), 0, s, a, done);
    return moe::check_launch("moe_layer_forward (routing)");
}

size_t moe::route_logits_bytes(int T, int E) { return route_ws_bytes(T, E); }

extern "C" {

size_t moe_route_workspace_size(int T, int H, int E)
{
    (void)H;
    if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS) return 0;
    return route_ws_bytes(T, E);
}

int moe_route(const void *x_dev, const void *w_router_dev, const float *bias_dev,
              int T, int H, int E, int k,
              float *logits_dev, int32_t *topk_ids_dev, float *topk_w_dev,
              int32_t *expert_offsets_dev, int32_t *sorted_pairs_dev, int32_t *pair_pos_dev,
              int32_t *active_list_dev, int32_t *n_active_dev,
              void *ws_dev, size_t ws_bytes, void *stream)
{
    return route_launch(x_dev, w_router_dev, bias_dev, T, H, E, k, logits_dev, topk_ids_dev, topk_w_dev,
                        expert_offsets_dev, sorted_pairs_dev, pair_pos_dev, active_list_dev, n_active_dev, ws_dev,
                        ws_bytes, 0, stream);
}

int moe_route_exact(const void *x_dev, const void *w_router_dev, const float *bias_dev,
                    int T, int H, int E, int k,
                    float *logits_dev, int32_t *topk_ids_dev, float *topk_w_dev,
                    int32_t *expert_offsets_dev, int32_t *sorted_pairs_dev, int32_t *pair_pos_dev,
                    int32_t *active_list_dev, int32_t *n_active_dev, void *ws_dev, size_t ws_bytes, void *stream)
{
    return route_launch(x_dev, w_router_dev, bias_dev, T, H, E, k, logits_dev, topk_ids_dev, topk_w_dev,
                        expert_offsets_dev, sorted_pairs_dev, pair_pos_dev, active_list_dev, n_active_dev, ws_dev,
                        ws_bytes, 1, stream);
}

}  // extern "C"

// ------------------------------------------------------------ allocation-free routing
// moe_route_static: moe_route with its workspace in a fixed device array of
// this library instead of a caller buffer, for callers that cannot allocate.
namespace {

constexpr size_t kStaticScratchBytes = (size_t)1 << 20;     // logits of 4096 tokens x 64 experts
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_dev[64];             // device address of `scratch`, per device ordinal

// Device address of `scratch` on the current device, looked up on the first
// call there (host code must not use the array's name as an address).
int scratch_address(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return moe::fail(MOE_ERR_HIP, "moe_route_static: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return moe::fail(MOE_ERR_UNSUPPORTED, "moe_route_static: device ordinal %d", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return moe::fail(MOE_ERR_HIP, "moe_route_static: hipGetSymbolAddress: %s", hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_route_static_max_bytes(void) { return kStaticScratchBytes; }

int moe_route_static(const void *x_dev, const void *w_router_dev, const float *bias_dev,
                     int T, int H, int E, int k,
                     float *logits_dev, int32_t *topk_ids_dev, float *topk_w_dev,
                     int32_t *expert_offsets_dev, int32_t *sorted_pairs_dev, int32_t *pair_pos_dev,
                     int32_t *active_list_dev, int32_t *n_active_dev, void *stream)
{
    moe::clear_error();
    int rc = moe::check_shape(T, H, 0, E, k, false);
    if (rc) return rc;
    const size_t need = route_ws_bytes(T, E);
    if (need > kStaticScratchBytes)
        return moe::fail(MOE_ERR_WORKSPACE, "moe_route_static: T=%d, E=%d need %zu bytes of scratch; the fixed "
                         "array holds %zu (use moe_route with a workspace)", T, E, need, kStaticScratchBytes);
    void *ws = nullptr;
    rc = scratch_address(&ws);
    if (rc) return rc;
    return route_launch(x_dev, w_router_dev, bias_dev, T, H, E, k, logits_dev, topk_ids_dev, topk_w_dev,
                        expert_offsets_dev, sorted_pairs_dev, pair_pos_dev, active_list_dev, n_active_dev, ws,
                        kStaticScratchBytes, 0, stream);
}

}  // extern "C"
