// FP16 shared expert: os = Wsd * fp16(silu(Wsg x) * (Wsu x)) and the per-token
// sigmoid gate sigma = sigmoid(wgate . x).
//
// Non-routed weights stay FP16 ("horizonrunmap.com/en", section "08 /
// Precision & quality", paragraph "Other components"); the layer adds the
// shared expert's output, scaled by a sigmoid gate, to the routed experts'
// weighted sum.  Rounding points are those of a routed expert: FP32 sums, the
// SwiGLU activation rounded to FP16 before the down projection, FP32 outputs.
//
// Weight layout ("tile8", written by moe_pack_fp16_tile8 from row-major
// [R][K]): tile (r8, kt) = rows 8 r8 .. 8 r8 + 7 x columns 128 kt .. 128 kt +
// 127, 2048 bytes at element (r8 * K/128 + kt) * 1024; its piece s (512 bytes
// at element s * 256) holds, at element (8 g + r) * 8, row 8 r8 + r, columns
// 128 kt + 32 s + 8 g .. +7.  One MFMA B operand of 8 rows (32 columns) is
// then one contiguous 512-byte run: row-major weights would give each
// instruction sixteen 64-byte runs, which stream from HBM about a fifth
// slower (measured on the MI355X with a read-pattern probe).
//
// Kernel design (gfx950, wave64).  Decode batches make this a skinny GEMM,
// bound by HBM (69 MB of FP16 weights for the Qwen shape), and a CU only
// streams at its share of HBM bandwidth when it holds an equal share of the
// bytes, so the work is cut into many equal units:
//   * The weights are in the tile8 layout above.  A unit is 16 output rows
//     (gate/up: the same 16 rows of both matrices) x one chunk of the
//     reduction axis x one pass of up to 16 MT tokens.  The chunk count NKC
//     is planned on the host so that the units spread evenly over 256 blocks
//     and the 8 wavefronts of a block share a chunk's 128-column tiles
//     (wave w takes tiles w, w + 8 of the chunk, NTW <= 2 per wave).
//   * Per 128-column tile a lane loads four 16-byte pieces of its row
//     (columns 32s + 8g .. +7, one from each 512-byte piece of its 8-row
//     tile): each is one MFMA B operand as stored, and the A operand is the
//     same columns of a token's activation row, read straight from memory
//     (L2-resident).  Every wave keeps its NTW tiles of the next unit in
//     flight while it computes the current one.
//   * The 8 partial sums of a unit meet in LDS and are added in wave order;
//     the unit's FP32 result goes to partial sums [NKC][T][NMAT R], which a
//     second kernel adds in chunk order (gate/up: then the SwiGLU into hs,
//     and the sigmoid gate; down: into shared_out, or written there directly
//     when NKC = 1).  Summation order is fixed, so results are run-to-run
//     identical.
//   * Tiles past a chunk, tokens past the batch and units past the last use
//     zero-byte buffer resources or out-of-range offsets, so their loads
//     return zeros without memory traffic.
#include "moe_internal.h"

namespace ffn {
int cu_count();   // compute units of the current device (expert_ffn.hip)
}

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRsrcWord3 = 0x00020000;    // raw buffer, 32-bit data format (gfx9 family)
constexpr int kOob = 0x7FFFFFF0;          // lane offset past any buffer: the load returns zeros
constexpr int kPlanBlocks = 256;          // blocks the chunking is planned for (one per CU)

struct SArgs {
    const uint16_t *x;      // [T][H]
    const uint16_t *wg;     // [Is][H], tile8 layout
    const uint16_t *wu;     // [Is][H], tile8 layout
    const uint16_t *wd;     // [H][Is], tile8 layout
    const uint16_t *wgate;  // [H]
    int T, H, Is;
    uint16_t *hs;           // [T][Is] FP16 activations between the projections
    float *part;            // partial sums [NKC][T][NMAT R]
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

// Sigmoid gate sigma[t] = sigmoid(wgate . x_t) of tokens t = first, first +
// stride, ...: one wave per token, FP32 sums; lane l takes columns 512 i +
// 8 l .. +7, four such steps loaded together (columns past H read as zeros).
__device__ void sigmoid_gate(const SArgs &a, int first, int stride)
{
    const int lane = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t rg = rsrc(a.wgate, a.H * 2);
    for (int t = first; t < a.T; t += stride) {
        const __amdgpu_buffer_rsrc_t rx = rsrc(a.x + (size_t)t * a.H, a.H * 2);
        float z = 0.0f;
        for (int c0 = 0; c0 < a.H; c0 += 4 * 512) {
            u32x4 wv[4], xv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                wv[i] = bload(rg, lane * 16, (c0 + 512 * i) * 2);
                xv[i] = bload(rx, lane * 16, (c0 + 512 * i) * 2);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half8 w8 = __builtin_bit_cast(half8, wv[i]), x8 = __builtin_bit_cast(half8, xv[i]);
#pragma unroll
                for (int j = 0; j < 8; ++j) z += (float)w8[j] * (float)x8[j];
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
        if (lane == 0) a.sigma[t] = 1.0f / (1.0f + expf(-z));
    }
}

// One projection's streaming pass.  GATEUP: g and u of x (K = H, R = Is);
// else the down projection of hs (K = Is, R = H).  Unit u = (pass p, group
// rg of RU rows, chunk kc), kc fastest; blocks b < n_main take units b,
// b + n_main, ...; with RU = 8 the lanes of rows 8..15 of the MFMA tile load
// nothing.  With nkc = 1 the result is final: gate/up applies the SwiGLU and
// writes hs, down writes dst = shared_out.  Otherwise dst receives partial
// sums [nkc][T][NMAT R].  GATEUP blocks from n_main on compute the sigmoid gate.
template <bool GATEUP, int MT, int NTW, int RU>
__global__ __launch_bounds__(kThreads) void fp16_stream_kernel(SArgs a, int nkc, int n_main, float *dst)
{
    constexpr int NMAT = GATEUP ? 2 : 1;
    constexpr int NE = NMAT * MT;                    // accumulator tiles of a wave
    static_assert(RU == 8 || RU == 16, "row groups of 8 or 16 rows");
    __shared__ f32x4 red[kWaves][NE][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    const int g4 = lane >> 4, n16 = lane & 15;
    if (GATEUP && (int)blockIdx.x >= n_main) {
        sigmoid_gate(a, (blockIdx.x - n_main) * kWaves + wave, (gridDim.x - n_main) * kWaves);
        return;
    }
    const int K = GATEUP ? a.H : a.Is, R = GATEUP ? a.Is : a.H;
    const int RG = R / RU, NT = K / 128;
    const int passes = (a.T + 16 * MT - 1) / (16 * MT);
    const int units = passes * RG * nkc;
    if ((int)blockIdx.x >= units) return;

    const uint16_t *wm[NMAT];
    if (GATEUP) {
        wm[0] = a.wg;
        wm[NMAT - 1] = a.wu;
    } else {
        wm[0] = a.wd;
    }
    const int wbytes = R * K * 2;                    // < 2^31 (checked on the host)
    const uint16_t *am = GATEUP ? a.x : a.hs;
    const int abytes = a.T * K * 2;

    // Loads of this wave's tile j of unit u (zeros past the chunk or the last unit).
    struct Src {
        int wvoff, kt0, kt1;
        int avoff[MT];
    };
    auto src_of = [&](int u) {
        Src q;
        const bool any = u < units;
        const int uu = any ? u : 0;
        const int kc = uu % nkc, rest = uu / nkc;
        const int rg = rest % RG, p = rest / RG;
        q.kt0 = kc * NT / nkc;
        q.kt1 = any ? (kc + 1) * NT / nkc : q.kt0;
        // row rg RU + n16: 8-row tile r8, row r within it; pieces start at
        // the tile's byte (r8 NT) 2048 plus kt 2048 + s 512 (soffset)
        const int row = rg * RU + n16;
        q.wvoff = n16 < RU ? (((row >> 3) * NT) * 1024 + (8 * g4 + (row & 7)) * 8) * 2 : kOob;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int tok = (p * MT + m) * 16 + n16;
            q.avoff[m] = tok < a.T ? (tok * K + 8 * g4) * 2 : kOob;
        }
        return q;
    };
    // With one token pass and a block stride that is a multiple of nkc, every
    // unit of a block has the same chunk (kc = u mod nkc), so a wave's tiles
    // and activation fragments are the same in each: loaded once and kept.
    const bool act_fixed = passes == 1 && n_main % nkc == 0;
    u32x4 wb[NTW][NMAT][4], ab[NTW][MT][4];
    auto issue_act = [&](const Src &q, int j, bool ok, int kt) {
        const __amdgpu_buffer_rsrc_t arr = rsrc(am, ok ? abytes : 0);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int s = 0; s < 4; ++s) ab[j][m][s] = bload(arr, q.avoff[m], kt * 256 + 64 * s);
    };
    auto issue = [&](const Src &q, int j, bool with_act) {
        const int kt0 = q.kt0 + wave + 8 * j;
        const bool ok = kt0 < q.kt1;
        const int kt = ok ? kt0 : 0;
#pragma unroll
        for (int mat = 0; mat < NMAT; ++mat) {
            const __amdgpu_buffer_rsrc_t wr = rsrc(wm[mat], ok ? wbytes : 0);
#pragma unroll
            for (int s = 0; s < 4; ++s) wb[j][mat][s] = bload(wr, q.wvoff, kt * 2048 + 512 * s);
        }
        if (with_act) issue_act(q, j, ok, kt);
    };

    int u = blockIdx.x;
    Src cur = src_of(u);
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        issue(cur, j, true);
    }
    __builtin_amdgcn_sched_barrier(0);
    for (; u < units; u += n_main) {
        const Src nxt = src_of(u + n_main);
        f32x4 acc[NMAT][MT];
#pragma unroll
        for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[mat][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                    for (int m = 0; m < MT; ++m) acc[mat][m] = mfma(ab[j][m][s], wb[j][mat][s], acc[mat][m]);
            // every read of this slot happens above: refill it with the next unit's tile
            __builtin_amdgcn_sched_barrier(0);
            issue(nxt, j, !act_fixed);
            __builtin_amdgcn_sched_barrier(0);
        }
        // the unit's 8 partial sums, added in wave order; lane (g4, n16) of
        // tile (mat, m) holds tokens 16 (MT p + m) + 4 g4 + q of row RU rg + n16
#pragma unroll
        for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
            for (int m = 0; m < MT; ++m) red[wave][mat * MT + m][lane] = acc[mat][m];
        lds_barrier();
        {
            const int kc = u % nkc, rest = u / nkc;
            const int rg = rest % RG, p = rest / RG;
            for (int i = tid; i < MT * 64; i += kThreads) {
                const int m = i >> 6, l = i & 63;
                if ((l & 15) >= RU) continue;
                f32x4 v[NMAT];
#pragma unroll
                for (int mat = 0; mat < NMAT; ++mat) {
                    v[mat] = red[0][mat * MT + m][l];
#pragma unroll
                    for (int w = 1; w < kWaves; ++w) v[mat] += red[w][mat * MT + m][l];
                }
                const int col = rg * RU + (l & 15);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int t = (p * MT + m) * 16 + 4 * (l >> 4) + q;
                    if (t >= a.T) continue;
                    if (GATEUP && nkc == 1) {
                        const float g = v[0][q], uv = v[NMAT - 1][q];
                        a.hs[(size_t)t * a.Is + col] = float_to_half_bits(g / (1.0f + expf(-g)) * uv);
                    } else {
#pragma unroll
                        for (int mat = 0; mat < NMAT; ++mat)
                            dst[((size_t)kc * a.T + t) * (size_t)(NMAT * R) + mat * R + col] = v[mat][q];
                    }
                }
            }
        }
        lds_barrier();
        cur = nxt;
    }
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

template <bool GATEUP, int MT, int NTW, int RU>
int launch_stream(const SArgs &a, const Plan &pl, float *dst, hipStream_t s, const char *who)
{
    const int R = GATEUP ? a.Is : a.H;
    const long long passes = (a.T + 16 * MT - 1) / (16 * MT);
    const long long units = passes * (R / RU) * pl.nkc;
    auto kern = fp16_stream_kernel<GATEUP, MT, NTW, RU>;
    // one block per CU, as the unit plan assumes (measured: a second resident
    // block per CU leaves the CUs with uneven unit counts and is slower)
    long long g = (long long)ffn::cu_count();
    if (g > units) g = units;
    if (g >= pl.nkc) g -= g % pl.nkc;    // each block keeps one chunk
    // gate/up: one more wave per token for the sigmoid gate
    const long long gsig = GATEUP ? ((a.T + kWaves - 1) / kWaves < ffn::cu_count() ? (a.T + kWaves - 1) / kWaves
                                                                                 : ffn::cu_count())
                                  : 0;
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

}  // namespace

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
        !moe::aligned(w_down_dev, 16) || !moe::aligned(w_sgate_dev, 16) || !moe::aligned(shared_out_dev, 16))
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_shared_ffn: x, weights and shared_out must be 16-byte aligned");
    const size_t need = ws_bytes(T, H, Is);
    if (!ws_dev || ws_bytes_ < need || !moe::aligned(ws_dev, 256))
        return moe::fail(MOE_ERR_WORKSPACE, "moe_shared_ffn: the workspace needs %zu bytes, 256-byte aligned", need);
    SArgs a;
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
    hipStream_t s = (hipStream_t)stream;
    const Plan pg = plan_of(true, T, Is, H), pd = plan_of(false, T, H, Is);
    int rc = launch_proj<true>(a, pg, a.part, s, "moe_shared_ffn (gate/up)");
    if (rc) return rc;
    auto grid_of = [](long long n4) {
        long long g = (n4 + kThreads - 1) / kThreads;
        return (unsigned int)(g < 4LL * ffn::cu_count() ? g : 4LL * ffn::cu_count());
    };
    if (pg.nkc > 1) {
        // SwiGLU of the summed chunks, about 4 columns per thread
        hipLaunchKernelGGL(shared_gateup_finish, dim3(grid_of((long long)T * (Is / 4))), dim3(kThreads), 0, s, a,
                           pg.nkc);
        rc = moe::check_launch("moe_shared_ffn (SwiGLU)");
        if (rc) return rc;
    }
    rc = launch_proj<false>(a, pd, pd.nkc > 1 ? a.part : a.out, s, "moe_shared_ffn (down)");
    if (rc || pd.nkc == 1) return rc;
    hipLaunchKernelGGL(shared_down_finish, dim3(grid_of((long long)T * (H / 4))), dim3(kThreads), 0, s, a, pd.nkc);
    return moe::check_launch("moe_shared_ffn (down sums)");
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
