// The routed-expert layer of a decode batch in ONE launch: routing (logits,
// top-k + softmax, grouping), the W4A16 gate/up projection with SiLU(gate) *
// up, the W4A16 down projection and the weighted combine, with the same
// operation, rounding points and summation orders as the separate launches
// (the outputs are bit-identical to moe_route + the streaming FFN launches +
// moe_combine).  The pages' "top4-fused-v1" executor is prior art for running
// the layer as one executor ("Horizon RunMap - architecture", section
// "Regimes and executor boundaries"); its kernels are not published.
//
// Design (gfx950).  The grid is exactly the blocks that fit on the device at
// once (compute units x resident blocks per unit), and each block runs the
// four phases in order:
//   1. logits of (token, group of 16 experts) tasks, task i on block
//      i mod grid; each finished task counts itself in a device-scope
//      counter and the block that completes the count runs the top-k and
//      the grouping, then raises the routing flag;
//   2. after the flag, the block's share of the gate/up work items (the
//      streaming FFN's items: a token tile x 8 row groups), signalling per
//      expert how many of its items are done;
//   3. its share of the down items: the weight tiles of the first unit are
//      requested first, then the block waits until every gate/up item of
//      the unit's expert is done (its h rows complete) and stages them;
//   4. the combine of its tokens (token t on block t mod grid), after the
//      down items of the token's k experts are done.
// No block waits for a block that is still in an earlier phase of its own
// work, and all blocks are resident together, so every wait ends; each wait
// is nevertheless bounded (about 2^18 polls) and gives up with
// MOE_ERR_TIMEOUT in the status word rather than hang.  Data handed between
// blocks (logits, routing results, h, pair outputs) is stored and loaded at
// device scope (the sc1 cache policy: coherent across the XCDs' L2 caches);
// a block's stores are complete (s_waitcnt vmcnt(0)) before the counter
// update that publishes them.  The last block to leave resets every counter,
// so the control block is zero before and after each call.
#include "ffn_stream.h"
#include "route_dev.h"

namespace {

using namespace ffn;

// Control words (uint32) at the start of the layer workspace.
constexpr int kCtlLogits = 0;                 // finished logits tasks
constexpr int kCtlRouted = 1;                 // routing results published
constexpr int kCtlExit = 2;                   // blocks that left
constexpr int kCtlGu = 64;                    // [E]: finished gate/up items per expert
constexpr int kCtlDn = 64 + MOE_MAX_EXPERTS;  // [E]: finished down items per expert
constexpr int kCtlWords = 64 + 2 * MOE_MAX_EXPERTS;
constexpr int kSpinLimit = 1 << 18;

struct PArgs {
    RouteArgs r;
    FfnArgs f;                 // status word in f.status
    const float *topk_w;
    const int32_t *pair_pos;
    const float *shared_out, *shared_gate;
    uint16_t *y;
    uint32_t *ctl;
};

// One thread waits until *c >= target; false after kSpinLimit polls.
__device__ inline bool wait_at_least(const uint32_t *c, uint32_t target)
{
    for (int i = 0; i < kSpinLimit; ++i) {
        if (moe::load_dev(c) >= target) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// Thread 0 only.  After a timeout the block waits no more (ok = false) and
// runs to its end with whatever the buffers hold.
__device__ inline void wait_or_fail(const PArgs &p, const uint32_t *c, uint32_t target, bool &ok)
{
    if (!ok) return;
    if (!wait_at_least(c, target)) {
        ok = false;
        if (p.f.status) *p.f.status = MOE_ERR_TIMEOUT;
    }
}

// Wave 0: every lane with `active` waits until *c >= target (its own counter
// and target), all lanes polling together; false after kSpinLimit polls.
__device__ inline bool wave_wait_at_least(const uint32_t *c, uint32_t target, bool active)
{
    for (int i = 0; i < kSpinLimit; ++i) {
        const bool done = !active || moe::load_dev(c) >= target;
        if (__ballot(!done) == 0ull) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// The slot table's inputs (routing results of this launch) at device scope.
__device__ inline TableIn table_loads_dev(const FfnArgs &a)
{
    const int lane = threadIdx.x;          // wave 0 only
    TableIn t;
    const bool in = lane < a.E;
    t.e = in ? moe::load_dev(&a.active[lane]) : -1;
    t.o0 = in ? moe::load_dev(&a.offsets[lane]) : 0;
    t.o1 = in ? moe::load_dev(&a.offsets[lane + 1]) : 0;
    t.sl = in ? (a.slot_map ? a.slot_map[lane] : lane) : -1;
    return t;
}

template <int NTG, int SG, int NTD, int SD>
union PLds {
    LogitsLds lg;
    GroupLds<kSelWaves, true> gr;
    typename Ffn<true, NTG, SG, false, true>::Lds gu;
    typename Ffn<false, NTD, SD, false, true>::Lds dn;
};

// Publishes `n` finished items of expert e (kCtlGu or kCtlDn): every wave's
// stores complete, then one device-scope add.
__device__ inline void signal_items(uint32_t *ctl, int base, int e, int n)
{
    moe::wait_stores();
    lds_barrier();
    if (threadIdx.x == 0 && e >= 0 && n > 0)
        __hip_atomic_fetch_add(&ctl[base + e], (uint32_t)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One phase of the streaming FFN over this block's contiguous share of the
// work items (the item split of the separate launch, which has the same
// grid).  Items of one expert are consecutive; their count is published when
// the block moves to another expert and at the end.  DOWN: before staging the
// h rows of an expert, wait until all its gate/up items (cg per token tile)
// are done.
template <bool GATEUP, int NT, int S>
__device__ void ffn_phase(const PArgs &p, typename Ffn<GATEUP, NT, S, false, true>::Lds &L, const TableIn &tin,
                          int nact, int cg, bool &ok)
{
    using F = Ffn<GATEUP, NT, S, false, true>;
    const F f(p.f, L, nact);
    if (threadIdx.x < 64) build_table(L.tb, p.f, tin, nact, 16, f.CH);
    __syncthreads();
    const long long N = L.tb.first[nact];
    const int it0 = (int)(N * blockIdx.x / gridDim.x), it1 = (int)(N * (blockIdx.x + 1) / gridDim.x);
    if (it0 >= it1) return;
    const int base = GATEUP ? kCtlGu : kCtlDn;
    auto ready = [&](const Unit &u) {
        if (GATEUP || threadIdx.x != 0) return;
        const int n = L.tb.n[u.slot];
        wait_or_fail(p, &p.ctl[kCtlGu + L.tb.e[u.slot]], (uint32_t)(((n + 15) / 16) * cg), ok);
    };
    u32x4 wq[F::D][F::NMAT][F::QW];
    _Float16 ws[F::D][F::NMAT];
    Unit cur = f.unit(it0, 0);
#pragma unroll
    for (int j = 0; j < F::D; ++j)
#pragma unroll
        for (int mat = 0; mat < F::NMAT; ++mat) {
            f.load_tile(wq[j][mat], cur.row, cur.nrec, cur.rg, mat, j);
            ws[j][mat] = f.load_s(cur.row, cur.nrec, cur.rg, mat, j);
        }
    ready(cur);
    f.stage(cur);
    int done = 0;
    for (int it = it0; it < it1; ++it) {
        const Unit nxt = (it + 1 < it1) ? f.unit(it + 1, cur.slot) : f.none();
        f.run(cur, nxt, wq, ws);
        ++done;
        if (nxt.slot != cur.slot) {
            signal_items(p.ctl, base, L.tb.e[cur.slot], done);
            done = 0;
        }
        if (nxt.slot >= 0 && (nxt.slot != cur.slot || nxt.mt != cur.mt)) {
            if (nxt.slot != cur.slot) ready(nxt);
            f.stage(nxt);
        }
        cur = nxt;
    }
}

template <int NTG, int SG, int NTD, int SD>
__global__ __launch_bounds__(kSelThreads) void layer_persistent_kernel(PArgs p)
{
    __shared__ PLds<NTG, SG, NTD, SD> L;
    __shared__ int s_last;
    const int tid = threadIdx.x;
    const RouteArgs &ra = p.r;
    const FfnArgs &fa = p.f;
    const int T = fa.T, E = fa.E, k = fa.k;
    bool ok = true;                       // meaningful in thread 0

    // 1. routing
    const int G = (E + kGroupE - 1) / kGroupE;
    const int ntask = T * G;
    for (int task = blockIdx.x; task < ntask; task += gridDim.x) {
        logits_block<2, true>(ra, L.lg, task / G, task % G);
        moe::wait_stores();
        __syncthreads();
        if (tid == 0) {
            const uint32_t before = __hip_atomic_fetch_add(&p.ctl[kCtlLogits], 1u, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
            s_last = before == (uint32_t)ntask - 1;
        }
        __syncthreads();
        if (s_last) {
            group_phase<kSelWaves, true, true>(ra, L.gr);
            moe::wait_stores();
            __syncthreads();
            if (tid == 0) moe::store_dev(&p.ctl[kCtlRouted], 1u);
        }
        __syncthreads();
    }
    if (tid == 0) wait_or_fail(p, &p.ctl[kCtlRouted], 1u, ok);
    __syncthreads();

    // 2, 3. expert FFN
    TableIn tin{};
    if (tid < 64) tin = table_loads_dev(fa);
    int nact = moe::load_dev(fa.n_active);
    if (nact > E) nact = E;
    if (nact > 0) {
        using FG = Ffn<true, NTG, SG, false, true>;
        const int cg = FG(fa, L.gu, nact).CH;       // gate/up items per token tile
        ffn_phase<true, NTG, SG>(p, L.gu, tin, nact, cg, ok);
        __syncthreads();
        ffn_phase<false, NTD, SD>(p, L.dn, tin, nact, cg, ok);
    }
    moe::wait_stores();
    __syncthreads();

    // 4. combine: token t waits for the down items of its k experts
    using FD = Ffn<false, NTD, SD, false, true>;
    const int cd = nact > 0 ? FD(fa, L.dn, nact).CH : 0;  // down items per token tile
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
        if (tid < 64) {
            // lane j < k: expert of slot j, its down-item count, and the wait for it (all lanes together)
            int e = tid < k ? moe::load_dev(&ra.ids[(size_t)t * k + tid]) : -1;
            if (e >= E) e = -1;
            const int n = e >= 0 ? moe::load_dev(&fa.offsets[e + 1]) - moe::load_dev(&fa.offsets[e]) : 0;
            const bool wok = __builtin_amdgcn_readfirstlane((int)ok) != 0;    // thread 0's: no timeout yet
            const bool waited = !wok || wave_wait_at_least(&p.ctl[kCtlDn + (e >= 0 ? e : 0)],
                                                           (uint32_t)(((n + 15) / 16) * cd), e >= 0);
            if (!waited && tid == 0) {
                ok = false;
                if (p.f.status) *p.f.status = MOE_ERR_TIMEOUT;
            }
        }
        __syncthreads();
        for (int c4 = tid; c4 < fa.H / 4; c4 += kSelThreads) {
            int pos[MOE_MAX_TOPK];
            float w[MOE_MAX_TOPK];
#pragma unroll
            for (int j = 0; j < MOE_MAX_TOPK; ++j) {
                pos[j] = j < k ? moe::load_dev(&p.pair_pos[(size_t)t * k + j]) : -1;
                w[j] = j < k ? moe::load_dev(&p.topk_w[(size_t)t * k + j]) : 0.0f;
            }
            const __amdgpu_buffer_rsrc_t ro = rsrc(fa.out, T * k * fa.H * 4);
            f32x4 v[MOE_MAX_TOPK];
#pragma unroll
            for (int j = 0; j < MOE_MAX_TOPK; ++j)
                v[j] = (j < k && pos[j] >= 0)
                           ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                           ro, (pos[j] * fa.H + 4 * c4) * 4, 0, moe::kDevScope))
                           : f32x4{0.f, 0.f, 0.f, 0.f};
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < MOE_MAX_TOPK; ++j)
                if (j < k)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[c] += w[j] * v[j][c];
            if (p.shared_out) {
                const float sg = p.shared_gate[t];
                const f32x4 so = *reinterpret_cast<const f32x4 *>(&p.shared_out[(size_t)t * fa.H + 4 * c4]);
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] += sg * so[c];
            }
            uint16_t *yo = p.y + (size_t)t * fa.H + 4 * c4;
            const uint32_t lo = (uint32_t)float_to_half_bits(acc[0]) | ((uint32_t)float_to_half_bits(acc[1]) << 16);
            const uint32_t hi = (uint32_t)float_to_half_bits(acc[2]) | ((uint32_t)float_to_half_bits(acc[3]) << 16);
            *reinterpret_cast<uint2 *>(yo) = make_uint2(lo, hi);
        }
        __syncthreads();
    }

    // leave: the last block resets the control words for the next call
    if (tid == 0) {
        const uint32_t before = __hip_atomic_fetch_add(&p.ctl[kCtlExit], 1u, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
        if (before == gridDim.x - 1) {
            for (int i = 0; i < kCtlWords; ++i) moe::store_dev(&p.ctl[i], 0u);
        }
    }
}

template <int NTG, int SG, int NTD, int SD>
int launch(const PArgs &p, hipStream_t s)
{
    auto kern = layer_persistent_kernel<NTG, SG, NTD, SD>;
    static int occ_cache[64];
    const int occ = moe::blocks_per_cu(kern, kSelThreads, occ_cache);
    const unsigned int grid = (unsigned int)(cu_count() * occ);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kSelThreads), 0, s, p);
    return moe::check_launch("moe_layer_forward (one launch)");
}

// The shapes and splits built into the one-launch layer: (H/128, I/128) in
// {(2, 4), (16, 8), (16, 11)} with the splits the separate launches choose.
int dispatch(const PArgs &p, int SG, int SD, hipStream_t s)
{
    const int NTG = p.f.H / 128, NTD = p.f.I / 128;
    if (NTG == 2 && NTD == 4) {
        if (SG == 1 && SD == 1) return launch<2, 1, 4, 1>(p, s);
        if (SG == 1 && SD == 2) return launch<2, 1, 4, 2>(p, s);
    }
    if (NTG == 16 && NTD == 8) {
        if (SG == 1 && SD == 1) return launch<16, 1, 8, 1>(p, s);
        if (SG == 2 && SD == 2) return launch<16, 2, 8, 2>(p, s);
        if (SG == 4 && SD == 4) return launch<16, 4, 8, 4>(p, s);
        if (SG == 2 && SD == 1) return launch<16, 2, 8, 1>(p, s);
        if (SG == 4 && SD == 2) return launch<16, 4, 8, 2>(p, s);
        if (SG == 8 && SD == 4) return launch<16, 8, 8, 4>(p, s);
    }
    if (NTG == 16 && NTD == 11) {
        if (SD == 1) {
            if (SG == 1) return launch<16, 1, 11, 1>(p, s);
            if (SG == 2) return launch<16, 2, 11, 1>(p, s);
            if (SG == 4) return launch<16, 4, 11, 1>(p, s);
            if (SG == 8) return launch<16, 8, 11, 1>(p, s);
        }
    }
    return -1;
}

}  // namespace

size_t moe::layer_persistent_ctl_bytes() { return kCtlWords * sizeof(uint32_t); }

bool moe::layer_persistent_supported(int T, int H, int I, int E, int k)
{
    if (T < 1 || T > kPersistentMaxT || E % 2 != 0 || (long long)T * k >= 64LL * E) return false;
    const int NTG = H / 128, NTD = I / 128;
    if (H % 128 || I % 128) return false;
    const int SG = ffn::stream_split(true, T, H, I, E, k), SD = ffn::stream_split(false, T, H, I, E, k);
    if (NTG == 2 && NTD == 4) return SG == 1 && SD <= 2;
    if (NTG == 16 && NTD == 8)
        return (SG == SD && SG <= 4) || (SG == 2 * SD && SD <= 4);
    if (NTG == 16 && NTD == 11) return SD == 1;
    return false;
}

int moe::layer_persistent(const void *x_dev, const void *w_router_dev, const float *bias_dev, int T, int H, int I,
                          int E, int k, const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                          const float *shared_out_dev, const float *shared_gate_dev, void *y_dev,
                          const moe_layer_buffers *b, float *lbuf, uint32_t *ctl, hipStream_t s)
{
    const char *who = "moe_layer_forward (one launch)";
    if (!layer_persistent_supported(T, H, I, E, k))
        return moe::fail(MOE_ERR_UNSUPPORTED, "%s: shape T=%d H=%d I=%d E=%d k=%d not built into the one-launch "
                         "layer", who, T, H, I, E, k);
    if (!moe::aligned(x_dev, 8) || !moe::aligned(w_router_dev, 4))
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: x must be 8-byte and w_router 4-byte aligned", who);
    PArgs p;
    int rc = ffn::make_ffn_args(p.f, x_dev, T, H, I, E, k, rows_dev, row_stride, slot_map_dev, b->expert_offsets,
                                b->sorted_pairs, b->active_list, b->n_active, b->h, b->pair_out, b->status, who);
    if (rc) return rc < 0 ? MOE_OK : rc;
    RouteArgs &a = p.r;
    a.x = (const uint16_t *)x_dev;
    a.wr = (const uint16_t *)w_router_dev;
    a.bias = bias_dev;
    a.T = T; a.H = H; a.E = E; a.k = k;
    a.logits = b->logits;
    a.ids = b->topk_ids;
    a.w = b->topk_w;
    a.offsets = b->expert_offsets;
    a.sorted_pairs = b->sorted_pairs;
    a.pair_pos = b->pair_pos;
    a.active = b->active_list;
    a.n_active = b->n_active;
    a.force_exact = 0;
    a.lbuf = lbuf;
    p.topk_w = b->topk_w;
    p.pair_pos = b->pair_pos;
    p.shared_out = shared_out_dev;
    p.shared_gate = shared_gate_dev;
    p.y = (uint16_t *)y_dev;
    p.ctl = ctl;
    const int SG = ffn::stream_split(true, T, H, I, E, k), SD = ffn::stream_split(false, T, H, I, E, k);
    rc = dispatch(p, SG, SD, s);
    if (rc < 0) return moe::fail(MOE_ERR_UNSUPPORTED, "%s: split (%d, %d) not built", who, SG, SD);
    return rc;
}
