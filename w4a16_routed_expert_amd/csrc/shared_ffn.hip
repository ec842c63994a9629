// FP16 shared expert: os = Wsd * fp16(silu(Wsg x) * (Wsu x)) and the per-token
// sigmoid gate sigma = sigmoid(wgate . x).
//
// Non-routed weights stay FP16 ("horizonrunmap.com/en", section "08 /
// Precision & quality", paragraph "Other components"); the layer adds the
// shared expert's output, scaled by a sigmoid gate, to the routed experts'
// weighted sum.  Rounding points are those of a routed expert: FP32 sums, the
// SwiGLU activation rounded to FP16 before the down projection, FP32 outputs.
//
// Kernel design (gfx950, wave64).  Decode batches make this a skinny GEMM,
// bound by HBM (69 MB of FP16 weights for the Qwen shape):
//   * The weights are plain row-major [R][K] FP16.  A work unit is 16 output
//     rows x a 1/S slice of the reduction axis x MT token tiles of 16 tokens
//     (up to 64 tokens share each weight load); the S waves of a row group
//     reduce their FP32 partials in LDS in a fixed order.  A block holds 8/S
//     row groups of one pass over MT token tiles.
//   * Per 128-column tile a lane loads four 16-byte pieces of its row (columns
//     32s + 8g .. +7, s = 0..3): each is one MFMA B operand as stored, and the
//     A operand is the same columns of a token's activation row, read straight
//     from memory (L2-resident; no permutation is needed for FP16 weights).
//   * A ring of D tiles per wave stays in flight; tiles past the slice and
//     rows past the matrix use zero-byte buffer resources or out-of-range
//     offsets, so their loads return zeros without memory traffic.
#include "moe_internal.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRsrcWord3 = 0x00020000;    // raw buffer, 32-bit data format (gfx9 family)
constexpr int kOob = 0x7FFFFFF0;          // lane offset past any buffer: the load returns zeros

struct SArgs {
    const uint16_t *x;      // [T][H]
    const uint16_t *wg;     // [Is][H]
    const uint16_t *wu;     // [Is][H]
    const uint16_t *wd;     // [H][Is]
    const uint16_t *wgate;  // [H]
    int T, H, Is;
    uint16_t *hs;           // [T][Is] FP16 activations between the two kernels
    float *out;             // [T][H]
    float *sigma;           // [T]
};

__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *base, int nbytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, nbytes, kRsrcWord3);
}

__device__ inline u32x4 bload(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

__device__ inline f32x4 mfma(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0,
                                                  0);
}

__device__ inline void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ inline uint16_t float_to_half_bits(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

// Block = 8/S row groups of one token tile; wave = (row group, slice of the
// reduction axis).  GATEUP: the gate and up projections of x and the SwiGLU
// epilogue into hs; else the down projection of hs into out.  Blocks past the
// last item compute sigma (GATEUP only).
template <bool GATEUP, int S, int D, int MT>
__global__ __launch_bounds__(kThreads) void fp16_ffn_kernel(SArgs a, int n_items)
{
    constexpr int NMAT = GATEUP ? 2 : 1;
    constexpr int RGB = kWaves / S;
    constexpr int NACC = NMAT * MT;
    __shared__ float red[S > 1 ? S - 1 : 1][S > 1 ? RGB : 1][S > 1 ? NACC : 1][S > 1 ? 4 : 1][S > 1 ? 64 : 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    const int g4 = lane >> 4, n16 = lane & 15;
    const int K = GATEUP ? a.H : a.Is, R = GATEUP ? a.Is : a.H;
    const int RG = R / 16, NT = K / 128;
    const int CH = (RG + RGB - 1) / RGB;

    if (GATEUP && (int)blockIdx.x >= n_items) {
        // sigma[t] = sigmoid(wgate . x_t): one wave per token, FP32 sums
        for (int t = (blockIdx.x - n_items) * kWaves + wave; t < a.T; t += (gridDim.x - n_items) * kWaves) {
            float z = 0.0f;
            for (int c = lane; c < a.H; c += 64)
                z += (float)__builtin_bit_cast(_Float16, a.wgate[c]) *
                     (float)__builtin_bit_cast(_Float16, a.x[(size_t)t * a.H + c]);
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
            if (lane == 0) a.sigma[t] = 1.0f / (1.0f + expf(-z));
        }
        return;
    }

    const int pass = blockIdx.x / CH, c = blockIdx.x % CH;
    const int rgl = wave / S, ks = wave % S;
    const int rg = c * RGB + rgl;
    const bool row_ok = rg < RG;
    const int t0 = ks * NT / S, t1 = (ks + 1) * NT / S;      // this wave's tiles
    const int NR = (t1 - t0 + D - 1) / D;                    // rounds of D tiles (the last may be partial)

    // weights: lane (g4, n16) reads row 16 rg + n16, columns 32s + 8 g4 of each tile
    const uint16_t *wm[NMAT];
    if (GATEUP) {
        wm[0] = a.wg;
        wm[NMAT - 1] = a.wu;
    } else {
        wm[0] = a.wd;
    }
    const int wbytes = R * K * 2;                            // < 2^31 (checked on the host)
    const int wvoff = row_ok ? ((rg * 16 + n16) * K + 8 * g4) * 2 : kOob;
    // activations: lane (g4, n16) of token tile m reads token 16 (MT pass + m) + n16, same columns
    const uint16_t *am = GATEUP ? a.x : a.hs;
    const int abytes = a.T * K * 2;
    int avoff[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int tok = (pass * MT + m) * 16 + n16;
        avoff[m] = tok < a.T ? (tok * K + 8 * g4) * 2 : kOob;
    }

    u32x4 wb[D][NMAT][4], ab[D][MT][4];
    auto issue = [&](int d, int t) {
        const bool ok = t < t1;
        const int soff = (ok ? t : 0) * 256;
#pragma unroll
        for (int mat = 0; mat < NMAT; ++mat) {
            const __amdgpu_buffer_rsrc_t wr = rsrc(wm[mat], ok ? wbytes : 0);
#pragma unroll
            for (int s = 0; s < 4; ++s) wb[d][mat][s] = bload(wr, wvoff, soff + 64 * s);
        }
        const __amdgpu_buffer_rsrc_t arr = rsrc(am, ok ? abytes : 0);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int s = 0; s < 4; ++s) ab[d][m][s] = bload(arr, avoff[m], soff + 64 * s);
    };
    // the same load order as the refills in the loop, so the wait before each
    // slot's first use counts only the loads issued after it
#pragma unroll
    for (int d = 0; d < D; ++d) {
        __builtin_amdgcn_sched_barrier(0);
        issue(d, t0 + d);
    }
    __builtin_amdgcn_sched_barrier(0);

    f32x4 acc[NMAT][MT];
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[mat][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                    for (int m = 0; m < MT; ++m) acc[mat][m] = mfma(ab[d][m][s], wb[d][mat][s], acc[mat][m]);
            // every read of this slot happens above: reload it in place
            __builtin_amdgcn_sched_barrier(0);
            issue(d, t0 + (r + 1) * D + d);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    if (S > 1) {
        if (ks > 0) {
#pragma unroll
            for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int q = 0; q < 4; ++q) red[ks - 1][rgl][mat * MT + m][q][lane] = acc[mat][m][q];
        }
        lds_barrier();
        if (ks != 0) return;
#pragma unroll
        for (int k2 = 1; k2 < S; ++k2)
#pragma unroll
            for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[mat][m][q] += red[k2 - 1][rgl][mat * MT + m][q][lane];
    }
    if (!row_ok) return;
    // lane (g4, n16) holds tokens 16 (MT pass + m) + 4 g4 + q of row 16 rg + n16
    const int col = rg * 16 + n16;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = (pass * MT + m) * 16 + 4 * g4 + q;
            if (t < a.T) {
                if constexpr (GATEUP) {
                    const float g = acc[0][m][q], u = acc[NMAT - 1][m][q];
                    a.hs[(size_t)t * a.Is + col] = float_to_half_bits(g / (1.0f + expf(-g)) * u);
                } else {
                    a.out[(size_t)t * a.H + col] = acc[0][m][q];
                }
            }
        }
}

constexpr int kSplit = 8;

// MT token tiles share every weight load; a pass covers 16*MT tokens.
template <bool GATEUP, int D, int MT>
int launch_mt(const SArgs &a, hipStream_t s, const char *who)
{
    const int R = GATEUP ? a.Is : a.H;
    const int RG = R / 16, RGB = kWaves / kSplit;
    const int CH = (RG + RGB - 1) / RGB;
    const int passes = (a.T + 16 * MT - 1) / (16 * MT);
    const int n_items = CH * passes;
    const int sig_blocks = GATEUP ? (a.T + kWaves - 1) / kWaves : 0;
    hipLaunchKernelGGL((fp16_ffn_kernel<GATEUP, kSplit, D, MT>), dim3((unsigned int)(n_items + sig_blocks)),
                       dim3(kThreads), 0, s, a, n_items);
    return moe::check_launch(who);
}

template <bool GATEUP>
int launch(const SArgs &a, hipStream_t s, const char *who)
{
    // (gate/up holds two weight matrices per tile, so its register budget
    // allows two token tiles per pass)
    const int tiles = (a.T + 15) / 16;
    if (tiles <= 1) return launch_mt<GATEUP, GATEUP ? 2 : 3, 1>(a, s, who);
    if (GATEUP || tiles == 2) return launch_mt<GATEUP, GATEUP ? 1 : 2, 2>(a, s, who);
    return launch_mt<false, 1, 4>(a, s, who);
}

size_t ws_bytes(int T, int Is) { return ((size_t)T * Is * 2 + 255) / 256 * 256; }

}  // namespace

extern "C" {

size_t moe_shared_ffn_workspace_size(int T, int H, int Is)
{
    if (T < 0 || H <= 0 || Is <= 0 || H % 128 || Is % 128) return 0;
    return ws_bytes(T, Is);
}

int moe_shared_ffn(const void *x_dev, const void *w_gate_dev, const void *w_up_dev, const void *w_down_dev,
                   const void *w_sgate_dev, int T, int H, int Is, float *shared_out_dev, float *shared_gate_dev,
                   void *ws_dev, size_t ws_bytes_, void *stream)
{
    moe::clear_error();
    if (T < 0 || T > 65536) return moe::fail(MOE_ERR_UNSUPPORTED, "moe_shared_ffn: T=%d outside [0, 65536]", T);
    if (H <= 0 || H % 128 || Is <= 0 || Is % 128)
        return moe::fail(MOE_ERR_UNSUPPORTED, "moe_shared_ffn: H=%d and Is=%d must be positive multiples of 128", H,
                         Is);
    if ((long long)H * Is * 2 >= (1ll << 31) || (long long)T * (H > Is ? H : Is) * 2 >= (1ll << 31))
        return moe::fail(MOE_ERR_UNSUPPORTED, "moe_shared_ffn: a matrix over 2 GiB");
    if (T == 0) return MOE_OK;
    if (!x_dev || !w_gate_dev || !w_up_dev || !w_down_dev || !w_sgate_dev || !shared_out_dev || !shared_gate_dev)
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_shared_ffn: null pointer argument");
    if (!moe::aligned(x_dev, 16) || !moe::aligned(w_gate_dev, 16) || !moe::aligned(w_up_dev, 16) ||
        !moe::aligned(w_down_dev, 16) || !moe::aligned(shared_out_dev, 16))
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_shared_ffn: x, weights and shared_out must be 16-byte aligned");
    if (!ws_dev || ws_bytes_ < ws_bytes(T, Is) || !moe::aligned(ws_dev, 256))
        return moe::fail(MOE_ERR_WORKSPACE, "moe_shared_ffn: the workspace needs %zu bytes, 256-byte aligned",
                         ws_bytes(T, Is));
    SArgs a;
    a.x = (const uint16_t *)x_dev;
    a.wg = (const uint16_t *)w_gate_dev;
    a.wu = (const uint16_t *)w_up_dev;
    a.wd = (const uint16_t *)w_down_dev;
    a.wgate = (const uint16_t *)w_sgate_dev;
    a.T = T; a.H = H; a.Is = Is;
    a.hs = (uint16_t *)ws_dev;
    a.out = shared_out_dev;
    a.sigma = shared_gate_dev;
    hipStream_t s = (hipStream_t)stream;
    int rc = launch<true>(a, s, "moe_shared_ffn (gate/up)");
    if (rc) return rc;
    return launch<false>(a, s, "moe_shared_ffn (down)");
}

}  // extern "C"
