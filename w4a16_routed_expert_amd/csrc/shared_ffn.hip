// FP16 shared expert launches (the device code is in shared_dev.h):
// os = Wsd * fp16(silu(Wsg x) * (Wsu x)) and the per-token sigmoid gate
// sigma = sigmoid(wgate . x); see shared_dev.h for the weight layout and the
// kernel design.
#include "shared_dev.h"

namespace ffn {
int cu_count();   // compute units of the current device (expert_ffn.hip)
}

namespace {

using namespace shx;

template <bool GATEUP, int MT, int NTW, int RU>
__global__ __launch_bounds__(kThreads) void fp16_stream_kernel(SArgs a, int nkc, int n_main, float *dst)
{
    __shared__ StreamLds<GATEUP, MT> red;
    fp16_stream_block<GATEUP, MT, NTW, RU>(a, nkc, n_main, dst, blockIdx.x, gridDim.x, red);
}

// hs = RN16(silu(sum_kc g) * sum_kc u), chunks in order, 4 columns per thread.
__global__ __launch_bounds__(kThreads) void shared_gateup_finish(SArgs a, int nkc)
{
    const int n4 = a.Is / 4;
    const long long total = (long long)a.T * n4;
    const size_t stride = (size_t)a.T * 2 * a.Is;
    for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < total; i += (long long)gridDim.x * kThreads) {
        const int t = (int)(i / n4), c = (int)(i % n4) * 4;
        const float *pg = a.part + (size_t)t * 2 * a.Is + c;
        f32x4 g = *reinterpret_cast<const f32x4 *>(pg), u = *reinterpret_cast<const f32x4 *>(pg + a.Is);
        for (int kc = 1; kc < nkc; ++kc) {
            g += *reinterpret_cast<const f32x4 *>(pg + kc * stride);
            u += *reinterpret_cast<const f32x4 *>(pg + kc * stride + a.Is);
        }
        uint32_t h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = float_to_half_bits(g[q] / (1.0f + expf(-g[q])) * u[q]);
        *reinterpret_cast<u32x2 *>(a.hs + (size_t)t * a.Is + c) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    }
}

// shared_out = sum_kc of the down projection's partial sums, chunks in order.
__global__ __launch_bounds__(kThreads) void shared_down_finish(SArgs a, int nkc)
{
    const int n4 = a.H / 4;
    const long long total = (long long)a.T * n4;
    const size_t stride = (size_t)a.T * a.H;
    for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < total; i += (long long)gridDim.x * kThreads) {
        const int t = (int)(i / n4), c = (int)(i % n4) * 4;
        const float *pp = a.part + (size_t)t * a.H + c;
        f32x4 v = *reinterpret_cast<const f32x4 *>(pp);
        for (int kc = 1; kc < nkc; ++kc) v += *reinterpret_cast<const f32x4 *>(pp + kc * stride);
        *reinterpret_cast<f32x4 *>(a.out + (size_t)t * a.H + c) = v;
    }
}

// tile8 packing: one thread per 16-byte chunk of the packed matrix (8
// consecutive FP16 values of one row), read from the row-major source.
__global__ __launch_bounds__(256) void pack_tile8_kernel(const uint16_t *src, uint16_t *dst, int R, int K)
{
    const int NT = K / 128;
    const long long chunks = (long long)R * K / 8;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < chunks; i += (long long)gridDim.x * 256) {
        const long long tile = i >> 7;                    // 128 chunks per 2048-byte tile
        const int j = (int)(i & 127);
        const int s = j >> 5, g = (j >> 3) & 3, r = j & 7;
        const long long r8 = tile / NT;
        const int kt = (int)(tile - r8 * NT);
        const long long row = 8 * r8 + r;
        const long long col = 128LL * kt + 32 * s + 8 * g;
        *reinterpret_cast<u32x4 *>(dst + 8 * i) = *reinterpret_cast<const u32x4 *>(src + row * K + col);
    }
}

// How one projection is cut: rows per unit (RU), chunks of the reduction
// axis (NKC), token tiles per pass (MT) and tiles per wavefront per unit (NTW).
struct Plan {
    int ru, nkc, mt, ntw;
};

// Token tiles per pass: one tile for T <= 16, two for T <= 32, else four.
int plan_mt(int T) { return T <= 16 ? 1 : (T <= 32 ? 2 : 4); }

// Largest NTW the registers allow for the ring of one wave (8-row units
// only run with one token tile).
int max_ntw(bool gateup, int ru) { return ru == 8 ? (gateup ? 4 : 6) : 2; }

// Small batches (one token tile): units of 8 rows over the whole reduction
// axis when a wave's share of it fits the ring, which needs no partial sums
// (twice the units of 16-row groups spread the bytes evenly over the CUs).
// Otherwise 16-row units and the chunk count (at least NT / 16) whose units
// fill 256 blocks best, a unit's efficiency being the share of the 8 NTW
// tile slots it uses; ties go to fewer chunks (less partial-sum traffic).
Plan plan_of(bool gateup, int T, int R, int K)
{
    const int NT = K / 128;
    const int mt = plan_mt(T);
    if (mt == 1 && (NT + 7) / 8 <= max_ntw(gateup, 8)) return Plan{8, 1, 1, (NT + 7) / 8};
    const int RG = R / 16;
    const long long passes = (T + 16 * mt - 1) / (16 * mt);
    const int kmax = max_ntw(gateup, 16);
    int best = (NT + 8 * kmax - 1) / (8 * kmax);
    double best_eff = -1.0;
    for (int nkc = best; nkc <= NT; ++nkc) {
        const int ntw = ((NT + nkc - 1) / nkc + 7) / 8;
        if (ntw > kmax) continue;
        const long long units = passes * RG * nkc;
        const long long rounds = (units + kPlanBlocks - 1) / kPlanBlocks;
        const double eff = (double)units / (double)(rounds * kPlanBlocks) * ((double)NT / nkc) / (8.0 * ntw);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best = nkc;
        }
    }
    return Plan{16, best, mt, ((NT + best - 1) / best + 7) / 8};
}

// Blocks of one pass: one per CU, as the unit plan assumes (measured: a
// second resident block per CU leaves the CUs with uneven unit counts and is
// slower), a multiple of the chunk count; gate/up also one wave per token for
// the sigmoid gate.
void grid_of_pass(const SArgs &a, bool gateup, long long units, int nkc, long long *g_out, long long *gsig_out)
{
    long long g = (long long)ffn::cu_count();
    if (g > units) g = units;
    if (g >= nkc) g -= g % nkc;          // each block keeps one chunk
    const long long nsig = (a.T + kWaves - 1) / kWaves;
    *g_out = g;
    *gsig_out = gateup ? (nsig < ffn::cu_count() ? nsig : ffn::cu_count()) : 0;
}

template <bool GATEUP, int MT, int NTW, int RU>
int launch_stream(const SArgs &a, const Plan &pl, float *dst, hipStream_t s, const char *who)
{
    const int R = GATEUP ? a.Is : a.H;
    const long long passes = (a.T + 16 * MT - 1) / (16 * MT);
    const long long units = passes * (R / RU) * pl.nkc;
    auto kern = fp16_stream_kernel<GATEUP, MT, NTW, RU>;
    long long g, gsig;
    grid_of_pass(a, GATEUP, units, pl.nkc, &g, &gsig);
    hipLaunchKernelGGL(kern, dim3((unsigned int)(g + gsig)), dim3(kThreads), 0, s, a, pl.nkc, (int)g, dst);
    return moe::check_launch(who);
}

template <bool GATEUP, int RU, int MT, int N>
int launch_ntw(const SArgs &a, const Plan &pl, float *dst, hipStream_t s, const char *who)
{
    if constexpr (N > 1) {
        if (pl.ntw < N) return launch_ntw<GATEUP, RU, MT, N - 1>(a, pl, dst, s, who);
    }
    return launch_stream<GATEUP, MT, N, RU>(a, pl, dst, s, who);
}

template <bool GATEUP>
int launch_proj(const SArgs &a, const Plan &pl, float *dst, hipStream_t s, const char *who)
{
    if (pl.ru == 8) return launch_ntw<GATEUP, 8, 1, GATEUP ? 4 : 6>(a, pl, dst, s, who);
    if (pl.mt == 1) return launch_ntw<GATEUP, 16, 1, 2>(a, pl, dst, s, who);
    if (pl.mt == 2) return launch_ntw<GATEUP, 16, 2, 2>(a, pl, dst, s, who);
    return launch_ntw<GATEUP, 16, 4, 2>(a, pl, dst, s, who);
}

// Workspace: hs (FP16 [T][Is]), then the partial sums of whichever
// projection needs more (the down projection's are written after the
// gate/up ones are consumed).
size_t hs_bytes(int T, int Is) { return ((size_t)T * Is * 2 + 255) / 256 * 256; }

size_t part_bytes(int T, int H, int Is)
{
    const int nkg = plan_of(true, T, Is, H).nkc, nkd = plan_of(false, T, H, Is).nkc;
    const size_t gu = nkg > 1 ? (size_t)nkg * T * 2 * Is : 0;
    const size_t dn = nkd > 1 ? (size_t)nkd * T * H : 0;
    return (gu > dn ? gu : dn) * 4;
}

size_t ws_bytes(int T, int H, int Is) { return hs_bytes(T, Is) + part_bytes(T, H, Is); }

unsigned int finish_grid(long long n4)
{
    const long long g = (n4 + kThreads - 1) / kThreads;
    return (unsigned int)(g < 4LL * ffn::cu_count() ? g : 4LL * ffn::cu_count());
}

}  // namespace

int shx::make_args(SArgs &a, const void *x_dev, const void *w_gate_dev, const void *w_up_dev, const void *w_down_dev,
                   const void *w_sgate_dev, int T, int H, int Is, float *shared_out_dev, float *shared_gate_dev,
                   void *ws_dev, size_t ws_bytes_, const char *who)
{
    if (T < 0 || T > 65536) return moe::fail(MOE_ERR_UNSUPPORTED, "%s: T=%d outside [0, 65536]", who, T);
    if (H <= 0 || H % 128 || Is <= 0 || Is % 128)
        return moe::fail(MOE_ERR_UNSUPPORTED, "%s: H=%d and Is=%d must be positive multiples of 128", who, H, Is);
    if ((long long)H * Is * 2 >= (1ll << 31) || (long long)T * (H > Is ? H : Is) * 2 >= (1ll << 31))
        return moe::fail(MOE_ERR_UNSUPPORTED, "%s: a matrix over 2 GiB", who);
    if (T == 0) return -1;
    if (!x_dev || !w_gate_dev || !w_up_dev || !w_down_dev || !w_sgate_dev || !shared_out_dev || !shared_gate_dev)
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: null pointer argument", who);
    if (!moe::aligned(x_dev, 16) || !moe::aligned(w_gate_dev, 16) || !moe::aligned(w_up_dev, 16) ||
        !moe::aligned(w_down_dev, 16) || !moe::aligned(w_sgate_dev, 16) || !moe::aligned(shared_out_dev, 16))
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: x, weights and shared_out must be 16-byte aligned", who);
    const size_t need = ws_bytes(T, H, Is);
    if (!ws_dev || ws_bytes_ < need || !moe::aligned(ws_dev, 256))
        return moe::fail(MOE_ERR_WORKSPACE, "%s: the shared-expert workspace needs %zu bytes, 256-byte aligned", who,
                         need);
    a.x = (const uint16_t *)x_dev;
    a.wg = (const uint16_t *)w_gate_dev;
    a.wu = (const uint16_t *)w_up_dev;
    a.wd = (const uint16_t *)w_down_dev;
    a.wgate = (const uint16_t *)w_sgate_dev;
    a.T = T; a.H = H; a.Is = Is;
    a.hs = (uint16_t *)ws_dev;
    a.part = reinterpret_cast<float *>((uint8_t *)ws_dev + hs_bytes(T, Is));
    a.out = shared_out_dev;
    a.sigma = shared_gate_dev;
    return MOE_OK;
}

shx::GateupPlan shx::gateup_plan(int T, int H, int Is)
{
    const Plan pg = plan_of(true, T, Is, H);
    return GateupPlan{pg.ru, pg.mt, pg.ntw, pg.nkc};
}

void shx::gateup_blocks(const SArgs &a, int *n_main, int *n_sig)
{
    const Plan pg = plan_of(true, a.T, a.Is, a.H);
    const long long units = (long long)((a.T + 16 * pg.mt - 1) / (16 * pg.mt)) * (a.Is / pg.ru) * pg.nkc;
    long long g, gsig;
    grid_of_pass(a, true, units, pg.nkc, &g, &gsig);
    *n_main = (int)g;
    *n_sig = (int)gsig;
}

int shx::launch_rest(const SArgs &a, hipStream_t s, const char *who)
{
    const Plan pg = plan_of(true, a.T, a.Is, a.H);
    if (pg.nkc > 1) {
        // SwiGLU of the summed chunks, about 4 columns per thread
        hipLaunchKernelGGL(shared_gateup_finish, dim3(finish_grid((long long)a.T * (a.Is / 4))), dim3(kThreads), 0,
                           s, a, pg.nkc);
        const int rc = moe::check_launch(who);
        if (rc) return rc;
    }
    const Plan pd = plan_of(false, a.T, a.H, a.Is);
    int rc = launch_proj<false>(a, pd, pd.nkc > 1 ? a.part : a.out, s, who);
    if (rc || pd.nkc == 1) return rc;
    hipLaunchKernelGGL(shared_down_finish, dim3(finish_grid((long long)a.T * (a.H / 4))), dim3(kThreads), 0, s, a,
                       pd.nkc);
    return moe::check_launch(who);
}

extern "C" {

size_t moe_shared_ffn_workspace_size(int T, int H, int Is)
{
    if (T < 0 || T > 65536 || H <= 0 || Is <= 0 || H % 128 || Is % 128) return 0;
    return ws_bytes(T, H, Is);
}

int moe_shared_ffn(const void *x_dev, const void *w_gate_dev, const void *w_up_dev, const void *w_down_dev,
                   const void *w_sgate_dev, int T, int H, int Is, float *shared_out_dev, float *shared_gate_dev,
                   void *ws_dev, size_t ws_bytes_, void *stream)
{
    moe::clear_error();
    SArgs a;
    int rc = shx::make_args(a, x_dev, w_gate_dev, w_up_dev, w_down_dev, w_sgate_dev, T, H, Is, shared_out_dev,
                            shared_gate_dev, ws_dev, ws_bytes_, "moe_shared_ffn");
    if (rc) return rc < 0 ? MOE_OK : rc;
    hipStream_t s = (hipStream_t)stream;
    const Plan pg = plan_of(true, T, Is, H);
    rc = launch_proj<true>(a, pg, a.part, s, "moe_shared_ffn (gate/up)");
    if (rc) return rc;
    return shx::launch_rest(a, s, "moe_shared_ffn");
}

int moe_pack_fp16_tile8(const void *src_dev, void *dst_dev, int R, int K, void *stream)
{
    moe::clear_error();
    if (R <= 0 || K <= 0 || R % 8 || K % 128)
        return moe::fail(MOE_ERR_UNSUPPORTED, "moe_pack_fp16_tile8: R=%d must be a positive multiple of 8 and "
                         "K=%d of 128", R, K);
    if ((long long)R * K * 2 >= (1ll << 31)) return moe::fail(MOE_ERR_UNSUPPORTED, "moe_pack_fp16_tile8: over 2 GiB");
    if (!src_dev || !dst_dev) return moe::fail(MOE_ERR_INVALID_ARG, "moe_pack_fp16_tile8: null pointer argument");
    if (!moe::aligned(src_dev, 16) || !moe::aligned(dst_dev, 16))
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_pack_fp16_tile8: src and dst must be 16-byte aligned");
    const uintptr_t a0 = (uintptr_t)src_dev, b0 = (uintptr_t)dst_dev, n = (uintptr_t)R * K * 2;
    if (a0 < b0 + n && b0 < a0 + n)
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_pack_fp16_tile8: src and dst overlap");
    const long long chunks = (long long)R * K / 8;
    long long g = (chunks + 255) / 256;
    if (g > 8LL * ffn::cu_count()) g = 8LL * ffn::cu_count();
    hipLaunchKernelGGL(pack_tile8_kernel, dim3((unsigned int)g), dim3(256), 0, (hipStream_t)stream,
                       (const uint16_t *)src_dev, (uint16_t *)dst_dev, R, K);
    return moe::check_launch("moe_pack_fp16_tile8");
}

}  // extern "C"
