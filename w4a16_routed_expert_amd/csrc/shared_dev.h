// Device code of the FP16 shared expert, shared by shared_ffn.hip (its launches)
// and layer_shared.hip (the decode layer whose routing launch also runs the
// shared expert's gate/up).  Not part of the C ABI.
//
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
#pragma once

#include "moe_internal.h"

namespace shx {

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
__device__ inline void sigmoid_gate(const SArgs &a, int first, int stride)
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
template <bool GATEUP, int MT>
using StreamLds = f32x4[kWaves][(GATEUP ? 2 : 1) * MT][64];

// The pass as run by block `bid` of `nblk` (the launch's blocks, or a share
// of a launch that also does other work), with its LDS passed in.
template <bool GATEUP, int MT, int NTW, int RU>
__device__ void fp16_stream_block(const SArgs &a, int nkc, int n_main, float *dst, int bid, int nblk,
                                  StreamLds<GATEUP, MT> &red)
{
    constexpr int NMAT = GATEUP ? 2 : 1;
    static_assert(RU == 8 || RU == 16, "row groups of 8 or 16 rows");
    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    const int g4 = lane >> 4, n16 = lane & 15;
    if (GATEUP && bid >= n_main) {
        sigmoid_gate(a, (bid - n_main) * kWaves + wave, (nblk - n_main) * kWaves);
        return;
    }
    const int K = GATEUP ? a.H : a.Is, R = GATEUP ? a.Is : a.H;
    const int RG = R / RU, NT = K / 128;
    const int passes = (a.T + 16 * MT - 1) / (16 * MT);
    const int units = passes * RG * nkc;
    if (bid >= units) return;

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

    int u = bid;
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


// Host side (shared_ffn.hip).  make_args: the checks and set-up of
// moe_shared_ffn (MOE_OK, an error code, or -1 for T = 0: nothing to do).
// gateup_plan: how the gate/up pass of a batch is cut (rows per unit, token
// tiles per pass, tiles per wavefront per unit, chunks of the reduction axis;
// with more than one chunk the pass writes FP32 partial sums to the
// workspace).  gateup_blocks: the blocks of that pass (without the
// sigmoid-gate blocks), and the sigmoid-gate blocks.  launch_rest:
// everything of the shared expert after that pass (the SwiGLU of the summed
// chunks if any, the down projection, its chunk sums if any).
struct GateupPlan {
    int ru, mt, ntw, nkc;
};
int make_args(SArgs &a, const void *x_dev, const void *w_gate_dev, const void *w_up_dev, const void *w_down_dev,
              const void *w_sgate_dev, int T, int H, int Is, float *shared_out_dev, float *shared_gate_dev,
              void *ws_dev, size_t ws_bytes, const char *who);
GateupPlan gateup_plan(int T, int H, int Is);
void gateup_blocks(const SArgs &a, int *n_main, int *n_sig);
int launch_rest(const SArgs &a, hipStream_t s, const char *who);

}  // namespace shx
