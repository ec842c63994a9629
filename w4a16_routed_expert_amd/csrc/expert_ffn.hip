// W4A16 expert FFN launches for small batches (the streaming kernels of
// ffn_stream.h: gate/up projection with the fused SiLU(gate) * up epilogue,
// and the down projection, read straight from qpacked INT4 expert rows) and
// the choice between them and the grouped GEMM of expert_gemm.hip.
#include "ffn_stream.h"

namespace {

template <bool GATEUP, int NT, int S, bool F16W = false>
__global__ __launch_bounds__(kThreads) void w4a16_ffn_kernel(FfnArgs a, const int32_t *__restrict__ active,
                                                             const int32_t *__restrict__ offsets,
                                                             const int32_t *__restrict__ slot_map,
                                                             const int32_t *__restrict__ n_active)
{
    using F = Ffn<GATEUP, NT, S, F16W>;
    __shared__ typename F::Lds L;
    // the slot table's inputs first: their loads do not wait for n_active
    TableIn tin{};
    if (threadIdx.x < 64) tin = table_loads(a, active, offsets, slot_map);
    int nact = *n_active;
    if (nact > a.E) nact = a.E;
    if (nact <= 0) return;
    const F f(a, L, nact);
    if (threadIdx.x < 64) build_table(L.tb, a, tin, nact, 16, f.CH);
    __syncthreads();
    const long long N = L.tb.first[nact];
    const int it0 = (int)(N * blockIdx.x / gridDim.x), it1 = (int)(N * (blockIdx.x + 1) / gridDim.x);
    if (it0 >= it1) return;

    u32x4 wq[F::D][F::NMAT][F::QW];
    _Float16 ws[F::D][F::NMAT];
    Unit cur = f.unit(it0, 0);
    // A wavefront's loads return in order, so the activation gather of the
    // staging waits behind every weight tile requested before it.  With a
    // split reduction axis (few units per CU, a short launch) only the first
    // ring slot goes out before the staging (measured at OLMoE T = 1: gate/up
    // 8.98 -> 8.63 us, down 5.96 -> 5.60); otherwise the whole ring does
    // (requesting it after the staging was slower: T = 32 gate/up 28.3 -> 30.6).
    constexpr int J0 = S > 1 ? 1 : F::D;
    auto fill = [&](int j) {
#pragma unroll
        for (int mat = 0; mat < F::NMAT; ++mat) {
            f.load_tile(wq[j][mat], cur.row, cur.nrec, cur.rg, mat, j);
            if constexpr (!F16W) ws[j][mat] = f.load_s(cur.row, cur.nrec, cur.rg, mat, j);
        }
    };
#pragma unroll
    for (int j = 0; j < J0; ++j) fill(j);
    f.stage(cur);
#pragma unroll
    for (int j = J0; j < F::D; ++j) fill(j);
    // The body is the same for every item, so the ring registers need no
    // copies on the loop's back edge.
    for (int it = it0; it < it1; ++it) {
        const Unit nxt = (it + 1 < it1) ? f.unit(it + 1, cur.slot) : f.none();
        f.run(cur, nxt, wq, ws);
        if (nxt.slot >= 0 && (nxt.slot != cur.slot || nxt.mt != cur.mt)) f.stage(nxt);
        cur = nxt;
    }
}

}  // namespace

int ffn::cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    static int ncu[64];
    if (dev >= 0 && dev < 64) {
        int v = __atomic_load_n(&ncu[dev], __ATOMIC_RELAXED);
        if (v == 0) {
            if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
            __atomic_store_n(&ncu[dev], v, __ATOMIC_RELAXED);
        }
        return v;
    }
    return 256;
}

namespace {

template <bool GATEUP, int NT, int S, bool F16W>
int launch_one(const FfnArgs &a, hipStream_t s, long long max_items, const char *who)
{
    auto kern = w4a16_ffn_kernel<GATEUP, NT, S, F16W>;
    static int occ_cache[64];
    const int occ = moe::blocks_per_cu(kern, kThreads, occ_cache);
    long long g = (long long)cu_count() * occ;
    if (g > max_items) g = max_items;
    if (g < 1) g = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned int)g), dim3(kThreads), 0, s, a, a.active, a.offsets, a.slot_map,
                       a.n_active);
    return moe::check_launch(who);
}

// Split of the reduction axis: the smallest S that gives about 8 wavefronts
// per CU of work (one block of 8 per CU is what the kernel's LDS and
// registers leave resident; measured, more splitting costs more in staging
// and partial sums than it gains), from the expected number of routed
// experts of a uniform router (a launch-shape choice only: any S gives the
// same sums in the same order per slice).
int choose_split(int NT, int RG, int T, int k, int E)
{
    const double P = (double)T * k;
    double miss = 1.0;
    for (int i = 0; i < T && miss > 1e-9; ++i) miss *= 1.0 - (double)k / E;
    const double slots = E * (1.0 - miss) + P / 16.0;
    const double waves = 8.0 * cu_count();
    int S = 1;
    while (S < 8 && slots * RG * S < waves) {
        const int n = S * 2;
        if (NT % n || (NT / n) % 2) break;
        S = n;
    }
    return S;
}

template <bool GATEUP, int NT, bool F16W>
int launch_nt(const FfnArgs &a, hipStream_t s, int S, long long max_items, const char *who)
{
    if constexpr (NT % 4 == 0) {
        if (S == 2) return launch_one<GATEUP, NT, 2, F16W>(a, s, max_items * 2, who);
    }
    if constexpr (NT % 8 == 0) {
        if (S == 4) return launch_one<GATEUP, NT, 4, F16W>(a, s, max_items * 4, who);
    }
    if constexpr (NT % 16 == 0) {
        if (S == 8) return launch_one<GATEUP, NT, 8, F16W>(a, s, max_items * 8, who);
    }
    return launch_one<GATEUP, NT, 1, F16W>(a, s, max_items, who);
}

// The grouped GEMM once experts average 64 routed pairs or more: then the
// layer is bound by the matrix cores and the streaming kernel, built to keep
// HBM busy at a few pairs per expert, would convert every weight tile once
// per 16 pairs.  `mode` (MOE_FFN_PATH_*) forces either family.
bool use_gemm(const FfnArgs &a, int mode)
{
    if (mode == MOE_FFN_PATH_STREAM) return false;
    if (mode == MOE_FFN_PATH_GEMM) return true;
    return (long long)a.T * a.k >= 64LL * a.E;
}

template <bool GATEUP, bool F16W = false>
int launch_ffn(const FfnArgs &a, int mode, hipStream_t s, const char *who)
{
    if (!F16W && use_gemm(a, mode)) return GATEUP ? launch_gemm_gateup(a, s) : launch_gemm_down(a, s);
    const int K = GATEUP ? a.H : a.I;
    const int R = GATEUP ? a.I : a.H;
    // row slots of wavefronts: gate/up one row group each, down two when the
    // reduction axis has an even number of tiles
    const int NT = K / 128;
    const int RG = R / 16 / ((GATEUP || NT % 2) ? 1 : 2);
    const long long pairs = (long long)a.T * a.k;
    const long long max_slots = pairs < a.E ? pairs : a.E;
    const long long max_items = (max_slots + pairs / 16) * ((RG + kWaves - 1) / kWaves);
    const int S = choose_split(NT, RG, a.T, a.k, a.E);
    switch (NT) {
    case 1: return launch_nt<GATEUP, 1, F16W>(a, s, S, max_items, who);
    case 2: return launch_nt<GATEUP, 2, F16W>(a, s, S, max_items, who);
    case 3: return launch_nt<GATEUP, 3, F16W>(a, s, S, max_items, who);
    case 4: return launch_nt<GATEUP, 4, F16W>(a, s, S, max_items, who);
    case 5: return launch_nt<GATEUP, 5, F16W>(a, s, S, max_items, who);
    case 6: return launch_nt<GATEUP, 6, F16W>(a, s, S, max_items, who);
    case 7: return launch_nt<GATEUP, 7, F16W>(a, s, S, max_items, who);
    case 8: return launch_nt<GATEUP, 8, F16W>(a, s, S, max_items, who);
    case 9: return launch_nt<GATEUP, 9, F16W>(a, s, S, max_items, who);
    case 10: return launch_nt<GATEUP, 10, F16W>(a, s, S, max_items, who);
    case 11: return launch_nt<GATEUP, 11, F16W>(a, s, S, max_items, who);
    case 12: return launch_nt<GATEUP, 12, F16W>(a, s, S, max_items, who);
    case 13: return launch_nt<GATEUP, 13, F16W>(a, s, S, max_items, who);
    case 14: return launch_nt<GATEUP, 14, F16W>(a, s, S, max_items, who);
    case 15: return launch_nt<GATEUP, 15, F16W>(a, s, S, max_items, who);
    case 16: return launch_nt<GATEUP, 16, F16W>(a, s, S, max_items, who);
    default: return moe::fail(MOE_ERR_UNSUPPORTED, "%s: reduction length %d > %d", who, K, kMaxNT * 128);
    }
}

int make_args(FfnArgs &a, const void *x_dev, int T, int H, int I, int E, int k, const void *rows_dev,
              size_t row_stride, const int32_t *slot_map_dev, const int32_t *expert_offsets_dev,
              const int32_t *sorted_pairs_dev, const int32_t *active_list_dev, const int32_t *n_active_dev,
              void *h_dev, float *pair_out_dev, int32_t *status_dev, int mode, const char *who, bool f16 = false)
{
    int rc = moe::check_shape(T, H, I, E, k, true);
    if (rc) return rc;
    if (mode != MOE_FFN_PATH_AUTO && mode != MOE_FFN_PATH_STREAM && mode != MOE_FFN_PATH_GEMM)
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: unknown mode %d", who, mode);
    if (T == 0) return -1;          // nothing to do; callers return MOE_OK
    if (H > kMaxNT * 128 || I > kMaxNT * 128)
        return moe::fail(MOE_ERR_UNSUPPORTED, "%s: H and I must be <= %d", who, kMaxNT * 128);
    size_t off[6];
    const size_t rb = f16 ? moe::row_bytes_fp16(H, I, off) : moe::row_bytes(H, I, off);
    if (!rows_dev || !expert_offsets_dev || !active_list_dev || !n_active_dev || !h_dev)
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: null pointer argument", who);
    if (!moe::aligned(rows_dev, 256) || row_stride < rb || row_stride % 256)
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: rows must be 256-byte aligned with stride >= %zu, multiple of 256",
                         who, rb);
    if (!moe::aligned(h_dev, 16) || (x_dev && !moe::aligned(x_dev, 16)) ||
        (pair_out_dev && !moe::aligned(pair_out_dev, 16)))
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: x, h and pair_out must be 16-byte aligned", who);
    a.x = (const uint16_t *)x_dev;
    a.T = T; a.H = H; a.I = I; a.E = E; a.k = k;
    a.rows = (const uint8_t *)rows_dev;
    a.stride = row_stride;
    a.slot_map = slot_map_dev;
    a.offsets = expert_offsets_dev;
    a.sorted_pairs = sorted_pairs_dev;
    a.active = active_list_dev;
    a.n_active = n_active_dev;
    a.h = (uint16_t *)h_dev;
    a.out = pair_out_dev;
    a.status = status_dev;
    a.row_bytes = (int)rb;          // < 2^31 for H, I <= 2048
    for (int i = 0; i < 3; ++i) {
        a.off_q[i] = (int)off[i];
        a.off_s[i] = (int)off[3 + i];
    }
    return MOE_OK;
}

int launch_gateup(const FfnArgs &a, int mode, hipStream_t s) { return launch_ffn<true>(a, mode, s, "moe_w4a16_gateup"); }

int launch_down(const FfnArgs &a, int mode, hipStream_t s) { return launch_ffn<false>(a, mode, s, "moe_w4a16_down"); }

}  // namespace

int ffn::stream_split(bool gateup, int T, int H, int I, int E, int k)
{
    const int K = gateup ? H : I, R = gateup ? I : H;
    const int NT = K / 128;
    const int RG = R / 16 / ((gateup || NT % 2) ? 1 : 2);
    return choose_split(NT, RG, T, k, E);
}

int ffn::make_ffn_args(FfnArgs &a, const void *x_dev, int T, int H, int I, int E, int k, const void *rows_dev,
                       size_t row_stride, const int32_t *slot_map_dev, const int32_t *expert_offsets_dev,
                       const int32_t *sorted_pairs_dev, const int32_t *active_list_dev, const int32_t *n_active_dev,
                       void *h_dev, float *pair_out_dev, int32_t *status_dev, const char *who)
{
    return make_args(a, x_dev, T, H, I, E, k, rows_dev, row_stride, slot_map_dev, expert_offsets_dev,
                     sorted_pairs_dev, active_list_dev, n_active_dev, h_dev, pair_out_dev, status_dev,
                     MOE_FFN_PATH_STREAM, who);
}

int moe::ffn_ksplit_width(int T, int H, int I, int E, int k) { return ffn::ksplit_width(T, H, I, E, k); }

int moe::ffn_ksplit(const void *x_dev, int T, int H, int I, int E, int k, const void *rows_dev, size_t row_stride,
                    const int32_t *slot_map_dev, const int32_t *expert_offsets_dev, const int32_t *sorted_pairs_dev,
                    const int32_t *active_list_dev, const int32_t *n_active_dev, void *h_dev, int32_t *status_dev,
                    float *planes, int width, hipStream_t s)
{
    const char *who = "moe_layer_forward (expert FFN)";
    if (width <= 0 || width != ffn::ksplit_width(T, H, I, E, k) || !planes || !sorted_pairs_dev || !x_dev)
        return moe::fail(MOE_ERR_INVALID_ARG, "%s: K-split launch arguments", who);
    FfnArgs a;
    const int rc = make_args(a, x_dev, T, H, I, E, k, rows_dev, row_stride, slot_map_dev, expert_offsets_dev,
                             sorted_pairs_dev, active_list_dev, n_active_dev, h_dev, planes, status_dev,
                             MOE_FFN_PATH_STREAM, who);
    if (rc == -1) return MOE_OK;
    if (rc) return rc;
    return ffn::launch_ksplit(a, planes, width, s, who);
}

extern "C" {

int moe_w4a16_gateup(const void *x_dev, int T, int H, int I, int E, int k,
                     const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                     const int32_t *expert_offsets_dev, const int32_t *sorted_pairs_dev,
                     const int32_t *active_list_dev, const int32_t *n_active_dev,
                     void *h_dev, int32_t *status_dev, int mode, void *stream)
{
    moe::clear_error();
    FfnArgs a;
    int rc = make_args(a, x_dev, T, H, I, E, k, rows_dev, row_stride, slot_map_dev, expert_offsets_dev,
                       sorted_pairs_dev, active_list_dev, n_active_dev, h_dev, nullptr, status_dev, mode,
                       "moe_w4a16_gateup");
    if (rc) return rc < 0 ? MOE_OK : rc;
    if (!x_dev || !sorted_pairs_dev) return moe::fail(MOE_ERR_INVALID_ARG, "moe_w4a16_gateup: null pointer argument");
    return launch_gateup(a, mode, (hipStream_t)stream);
}

int moe_w4a16_down(int T, int H, int I, int E, int k,
                   const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                   const int32_t *expert_offsets_dev, const int32_t *active_list_dev,
                   const int32_t *n_active_dev, const void *h_dev, float *pair_out_dev,
                   int32_t *status_dev, int mode, void *stream)
{
    moe::clear_error();
    FfnArgs a;
    int rc = make_args(a, nullptr, T, H, I, E, k, rows_dev, row_stride, slot_map_dev, expert_offsets_dev,
                       nullptr, active_list_dev, n_active_dev, const_cast<void *>(h_dev), pair_out_dev, status_dev,
                       mode, "moe_w4a16_down");
    if (rc) return rc < 0 ? MOE_OK : rc;
    if (!pair_out_dev) return moe::fail(MOE_ERR_INVALID_ARG, "moe_w4a16_down: null pointer argument");
    return launch_down(a, mode, (hipStream_t)stream);
}

int moe_w4a16_expert_ffn(const void *x_dev, int T, int H, int I, int E, int k,
                         const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                         const int32_t *expert_offsets_dev, const int32_t *sorted_pairs_dev,
                         const int32_t *active_list_dev, const int32_t *n_active_dev,
                         void *h_dev, float *pair_out_dev, int32_t *status_dev, int mode, void *stream)
{
    moe::clear_error();
    FfnArgs a;
    int rc = make_args(a, x_dev, T, H, I, E, k, rows_dev, row_stride, slot_map_dev, expert_offsets_dev,
                       sorted_pairs_dev, active_list_dev, n_active_dev, h_dev, pair_out_dev, status_dev, mode,
                       "moe_w4a16_expert_ffn");
    if (rc) return rc < 0 ? MOE_OK : rc;
    if (!x_dev || !sorted_pairs_dev || !pair_out_dev)
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_w4a16_expert_ffn: null pointer argument");
    rc = launch_gateup(a, mode, (hipStream_t)stream);
    if (rc) return rc;
    return launch_down(a, mode, (hipStream_t)stream);
}

// ------------------------------------------------------------ FP16 execution slots
// The offload-qpacked profile ("Horizon RunMap - architecture", section
// "Historical contracts remain distinct"; "Horizon technical notes —
// publication edition v1", section "Precision is profile-specific"): the
// low-bit source is dequantized into FP16 execution slots, which the FFN then
// reads instead of the compact rows.

int moe_fp16_expert_ffn(const void *x_dev, int T, int H, int I, int E, int k,
                        const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                        const int32_t *expert_offsets_dev, const int32_t *sorted_pairs_dev,
                        const int32_t *active_list_dev, const int32_t *n_active_dev,
                        void *h_dev, float *pair_out_dev, int32_t *status_dev, void *stream)
{
    moe::clear_error();
    const char *who = "moe_fp16_expert_ffn";
    FfnArgs a;
    int rc = make_args(a, x_dev, T, H, I, E, k, rows_dev, row_stride, slot_map_dev, expert_offsets_dev,
                       sorted_pairs_dev, active_list_dev, n_active_dev, h_dev, pair_out_dev, status_dev,
                       MOE_FFN_PATH_STREAM, who, true);
    if (rc) return rc < 0 ? MOE_OK : rc;
    if (!x_dev || !sorted_pairs_dev || !pair_out_dev) return moe::fail(MOE_ERR_INVALID_ARG, "%s: null pointer argument", who);
    rc = launch_ffn<true, true>(a, MOE_FFN_PATH_STREAM, (hipStream_t)stream, who);
    if (rc) return rc;
    return launch_ffn<false, true>(a, MOE_FFN_PATH_STREAM, (hipStream_t)stream, who);
}

}  // extern "C"
