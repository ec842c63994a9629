// W4A16 expert FFN: gate/up projection with the fused SiLU(gate) * up epilogue,
// and the down projection, read straight from qpacked INT4 expert rows.
//
// Routed experts stay compact INT4 (256-value blocks, FP16 scales) in GPU
// memory and the kernels convert the values they need during the operation,
// without an expanded expert copy ("Horizon RunMap - architecture", table
// "Representation and computation"; "horizonrunmap.com/en", section "08 /
// Precision & quality", paragraphs "Store" and "Compute": FP16 activations,
// FP32 accumulation stages, explicit rounding).
//
// Kernel design (gfx950, wave64).  Decode batches are bandwidth-bound: the
// kernels exist to keep HBM busy with qpacked bytes.
//   * Work item = (active expert, RGW groups of 16 weight rows).  Blocks are
//     persistent: block b walks the contiguous item range
//     [b*N/G, (b+1)*N/G), so consecutive items usually share the expert and
//     its activations stay in registers.
//   * A block is 4 wavefronts; wave w owns 128-column tiles
//     [w*NT/4, (w+1)*NT/4) of the reduction axis.  Partial sums meet in LDS
//     (double-buffered, one barrier per item).
//   * Prefetch without extra registers: as soon as a tile of item i has been
//     converted to FP16, its registers are reloaded with the same tile of
//     item i+1, so the next item's loads are in flight while item i finishes.
//   * A 1024-byte qpacked tile is read by one 16-byte load per lane (fully
//     coalesced).  Lane 16g + r gets row r, columns 32g .. 32g+31 of the tile:
//     four 32-bit words, each the 8-value B operand of one
//     v_mfma_f32_16x16x32_f16 after an exact INT4 -> FP16 conversion in
//     registers (OR the nibble into the exponent of 1024.0, subtract).
//   * The A operand is the FP16 activation of up to 16 routed tokens of the
//     expert (missing tokens are zero), its elements permuted to the order
//     the conversion produces.  More than 16 tokens take several passes over
//     the same weight registers.
//   * The FP16 block scale multiplies the FP32 partial of each tile (scales
//     are per 256-column block and tiles never straddle a block), so weights
//     are never rounded after scaling.
#include "moe_internal.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

struct FfnArgs {
    const uint16_t *x;          // [T][H] FP16
    int T, H, I, E, k;
    const uint8_t *rows;
    size_t stride;
    const int32_t *slot_map;    // [E] or null
    const int32_t *offsets;     // [E+1]
    const int32_t *sorted_pairs;
    const int32_t *active;      // [E], -1 past the active count
    const int32_t *n_active;    // [1]
    uint16_t *h;                // [T*k][I] FP16
    float *out;                 // [T*k][H] FP32
    int32_t *status;
    size_t off_gq, off_uq, off_dq, off_gs, off_us, off_ds;
};

__device__ inline u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// 8 INT4 codes of one 32-bit word (columns c..c+7; column c+2i in the low
// nibble of byte i, c+2i+1 in the high nibble) -> FP16 (code - 8), exact, in
// the order (c, c+4, c+1, c+5, c+2, c+6, c+3, c+7).
__device__ inline half8 dequant8(uint32_t w)
{
    const uint32_t s = w >> 8;
    const uint32_t p0 = (w & 0x000F000Fu) | 0x64006400u;   // 1024 + code        (c,   c+4)
    const uint32_t p1 = (w & 0x00F000F0u) | 0x64006400u;   // 1024 + 16 * code   (c+1, c+5)
    const uint32_t p2 = (s & 0x000F000Fu) | 0x64006400u;   //                    (c+2, c+6)
    const uint32_t p3 = (s & 0x00F000F0u) | 0x64006400u;   //                    (c+3, c+7)
    const half2v k1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2v k1_16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const half2v k72 = {(_Float16)72.0f, (_Float16)72.0f};
    const half2v h0 = __builtin_bit_cast(half2v, p0) - k1032;
    const half2v h1 = __builtin_bit_cast(half2v, p1) * k1_16 - k72;
    const half2v h2 = __builtin_bit_cast(half2v, p2) - k1032;
    const half2v h3 = __builtin_bit_cast(half2v, p3) * k1_16 - k72;
    half8 r;
    r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
    r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
    return r;
}

// 8 consecutive FP16 activations (x0..x7 in 4 dwords) -> the order of dequant8.
__device__ inline half8 act8(u32x4 d)
{
    u32x4 p;
    p[0] = (d[0] & 0xFFFFu) | (d[2] << 16);           // x0, x4
    p[1] = (d[0] >> 16) | (d[2] & 0xFFFF0000u);       // x1, x5
    p[2] = (d[1] & 0xFFFFu) | (d[3] << 16);           // x2, x6
    p[3] = (d[1] >> 16) | (d[3] & 0xFFFF0000u);       // x3, x7
    return __builtin_bit_cast(half8, p);
}

__device__ inline f32x4 mfma(half8 a, half8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline uint16_t float_to_half_bits(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

// Barrier that orders LDS only: prefetched global loads stay in flight across it
// (__syncthreads() would also wait for every outstanding global load).
__device__ inline void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// FP16 scale bits (low half of a register) -> float, as an explicit conversion
// at this point of the program (the compiler would otherwise fold it into a
// later mixed-precision FMA and keep the half register alive past its refill).
__device__ inline float scale_f32(uint32_t bits)
{
    float f;
    asm volatile("v_cvt_f32_f16 %0, %1" : "=v"(f) : "v"(bits));
    return f;
}

// Per-block table of the active slots, built once in LDS: expert, first
// grouped pair, pair count, device slot and the first work item of the slot.
struct SlotTable {
    int e[MOE_MAX_EXPERTS];
    int p0[MOE_MAX_EXPERTS];
    int n[MOE_MAX_EXPERTS];
    int sl[MOE_MAX_EXPERTS];
    int first[MOE_MAX_EXPERTS + 1];
};

// Built by wave 0, one lane per slot.  Routing metadata outside its valid
// range (a workspace that was not zero-filled, say) marks the status word and
// the slot gets no work.
__device__ void build_table(SlotTable &tb, const FfnArgs &a, const int32_t *__restrict__ active,
                            const int32_t *__restrict__ offsets, const int32_t *__restrict__ slot_map,
                            int nact, int items_per_tile)
{
    const int lane = threadIdx.x;          // wave 0 only
    int e = -1, p0 = 0, n = 0, sl = -1;
    if (lane < nact) {
        e = active[lane];
        if (e >= 0 && e < a.E) {
            const int q0 = offsets[e], q1 = offsets[e + 1];
            if (q0 >= 0 && q1 >= q0 && (long long)q1 <= (long long)a.T * a.k) {
                p0 = q0;
                n = q1 - q0;
                sl = slot_map ? slot_map[e] : e;
            } else {
                if (a.status) *a.status = MOE_ERR_INVALID_ARG;
                e = -1;
            }
        } else {
            e = -1;
        }
    }
    int cnt = (e >= 0) ? ((n + 15) / 16) * items_per_tile : 0;
    // inclusive scan of the item counts across the wave
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane < MOE_MAX_EXPERTS) {
        tb.e[lane] = e;
        tb.p0[lane] = p0;
        tb.n[lane] = n;
        tb.sl[lane] = sl;
        tb.first[lane + 1] = incl;
    }
    if (lane == 0) tb.first[0] = 0;
}

// One work item: 16 tokens (tile mt) of one active slot x RGW row groups.
struct Item {
    int slot, mt, rg0;
    int e, p0, n, sl;
    const uint8_t *row;     // expert row; for an absent expert, slot 0's row (read but never used)
};

// Per-item register buffer: weights and scales of NMAT matrices x RGW row groups x MAXT tiles.
template <int NMAT, int RGW, int MAXT>
struct WBuf {
    u32x4 w[NMAT][RGW][MAXT];
    uint32_t s[NMAT][RGW][MAXT];      // FP16 scale bits, one register each (no packing on refill)
};

template <int NMAT, int RGW, int MAXT, bool GATEUP>
struct Stream {
    const FfnArgs &a;
    int K, R, NT, NB, RGI;          // reduction length, rows per matrix, tiles, blocks, items per token tile
    int kb, ke;                     // this wave's tile range
    int lane, wave, r16, g4;
    size_t offq[NMAT], offs[NMAT];

    __device__ Stream(const FfnArgs &args) : a(args)
    {
        K = GATEUP ? a.H : a.I;
        R = GATEUP ? a.I : a.H;
        NT = K / 128;
        NB = (K + 255) / 256;
        RGI = R / 16 / RGW;
        const int tid = threadIdx.x;
        lane = tid & 63;
        wave = uni(tid >> 6);           // wave-uniform: tile ranges and addresses stay scalar
        r16 = lane & 15;
        g4 = lane >> 4;
        kb = wave * NT / kWaves;
        ke = (wave + 1) * NT / kWaves;
        if (GATEUP) {
            offq[0] = a.off_gq; offs[0] = a.off_gs;
            offq[NMAT - 1] = a.off_uq; offs[NMAT - 1] = a.off_us;
        } else {
            offq[0] = a.off_dq; offs[0] = a.off_ds;
        }
    }

    // Work item `it` of the block-wide enumeration (slot-major, then token tile, then row groups).
    __device__ Item item(const SlotTable &tb, int nact, int it, int slot_hint) const
    {
        int s = slot_hint;
        while (s + 1 < nact && tb.first[s + 1] <= it) ++s;
        s = uni(s);
        Item m;
        m.slot = s;
        const int local = uni(it - tb.first[s]);
        m.mt = local / RGI;
        m.rg0 = (local % RGI) * RGW;
        m.e = uni(tb.e[s]);
        m.p0 = uni(tb.p0[s]);
        m.n = uni(tb.n[s]);
        m.sl = uni(tb.sl[s]);
        m.row = a.rows + (size_t)(m.sl >= 0 ? m.sl : 0) * a.stride;
        return m;
    }

    // Loads tile j of row group rg0 + r, matrix mat: scalar row base + scalar
    // tile offset + per-lane offset.
    __device__ void load_tile(WBuf<NMAT, RGW, MAXT> &b, const Item &m, int mat, int r, int j) const
    {
        const uint8_t *qbase = m.row + offq[mat] + ((size_t)(m.rg0 + r) * NT + kb + j) * 1024;
        const uint16_t *sbase = reinterpret_cast<const uint16_t *>(m.row + offs[mat]) +
                                ((size_t)(m.rg0 + r) * NB + ((kb + j) >> 1)) * 16;
        b.w[mat][r][j] = ld16(qbase + lane * 16);
        b.s[mat][r][j] = sbase[r16];
    }

    __device__ void issue(WBuf<NMAT, RGW, MAXT> &b, const Item &m) const
    {
#pragma unroll
        for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
            for (int r = 0; r < RGW; ++r)
#pragma unroll
                for (int j = 0; j < MAXT; ++j)
                    if (kb + j < ke) load_tile(b, m, mat, r, j);
    }

    // A-operand fragments of the item's 16 tokens, in the element order of dequant8.
    __device__ void load_x(half8 (&X)[MAXT][4], const Item &m) const
    {
        const uint16_t *src = nullptr;
        const int pi = m.mt * 16 + r16;
        if (pi < m.n) {
            if (GATEUP) {
                const int tok = a.sorted_pairs[m.p0 + pi] / a.k;
                if (tok >= 0 && tok < a.T) src = a.x + (size_t)tok * a.H + 32 * g4;
            } else {
                src = a.h + (size_t)(m.p0 + pi) * a.I + 32 * g4;
            }
        }
#pragma unroll
        for (int j = 0; j < MAXT; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                X[j][q] = act8((src && kb + j < ke) ? ld16(src + 128 * (kb + j) + 8 * q) : u32x4{0u, 0u, 0u, 0u});
    }

    // Computes item m from the weights in b.  If nxt is given, each tile's
    // registers are reloaded with the same tile of item nxt right after the
    // tile has been converted.  Ends with the LDS reduction and the epilogue.
    __device__ void compute(const Item &m, WBuf<NMAT, RGW, MAXT> &b, const half8 (&X)[MAXT][4], const Item *nxt,
                            float (*red)[kWaves][NMAT * RGW][4][64], int &rbuf) const
    {
        f32x4 acc[NMAT][RGW];
#pragma unroll
        for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
            for (int r = 0; r < RGW; ++r) acc[mat][r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < MAXT; ++j) {
            if (kb + j < ke) {
#pragma unroll
                for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                    for (int r = 0; r < RGW; ++r) {
                        half8 d[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) d[q] = dequant8(b.w[mat][r][j][q]);
                        const float sc = scale_f32(b.s[mat][r][j]);
                        if (nxt) {
                            // every read of this tile's registers happens before they are
                            // reloaded, so the refill reuses them (no copies, no early wait)
                            __builtin_amdgcn_sched_barrier(0);
                            load_tile(b, *nxt, mat, r, j);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int q = 0; q < 4; ++q) p = mfma(X[j][q], d[q], p);
                        acc[mat][r] += sc * p;
                    }
            }
        }
        float (*rd)[NMAT * RGW][4][64] = red[rbuf];
#pragma unroll
        for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
            for (int r = 0; r < RGW; ++r)
#pragma unroll
                for (int v = 0; v < 4; ++v) rd[wave][mat * RGW + r][v][lane] = acc[mat][r][v];
        lds_barrier();
        // waves 0..3: wave v finishes token mt*16 + 4*g4 + v, row r16 of each row group.
        // An absent expert (no device row) gets zeros and flags the status word.
        const bool gone = m.sl < 0;
        if (gone && threadIdx.x == 0 && a.status) *a.status = MOE_ERR_ABSENT_EXPERT;
        if (wave < 4) {
            const int v = wave;
            const int i = m.mt * 16 + 4 * g4 + v;
            if (i < m.n) {
                const size_t p = (size_t)(m.p0 + i);
                if (GATEUP) {
                    float g = 0.f, u = 0.f;
#pragma unroll
                    for (int w = 0; w < kWaves; ++w) { g += rd[w][0][v][lane]; u += rd[w][1][v][lane]; }
                    a.h[p * a.I + m.rg0 * 16 + r16] = gone ? (uint16_t)0 : float_to_half_bits(g / (1.0f + expf(-g)) * u);
                } else {
#pragma unroll
                    for (int r = 0; r < RGW; ++r) {
                        float o = 0.f;
#pragma unroll
                        for (int w = 0; w < kWaves; ++w) o += rd[w][r][v][lane];
                        a.out[p * a.H + (m.rg0 + r) * 16 + r16] = gone ? 0.0f : o;
                    }
                }
            }
        }
        rbuf ^= 1;              // the next item writes the other buffer: one barrier per item
    }
};

template <int NMAT, int RGW, int MAXT, bool GATEUP>
__global__ __launch_bounds__(kThreads) void w4a16_stream_kernel(FfnArgs a, const int32_t *__restrict__ active,
                                                                const int32_t *__restrict__ offsets,
                                                                const int32_t *__restrict__ slot_map,
                                                                const int32_t *__restrict__ n_active)
{
    static_assert(!GATEUP || (NMAT == 2 && RGW == 1), "gate/up items are one row group of both matrices");
    __shared__ float red[2][kWaves][NMAT * RGW][4][64];
    __shared__ SlotTable tb;
    const Stream<NMAT, RGW, MAXT, GATEUP> S(a);
    int nact = *n_active;
    if (nact > a.E) nact = a.E;
    if (nact <= 0) return;
    if (threadIdx.x < 64) build_table(tb, a, active, offsets, slot_map, nact, S.RGI);
    __syncthreads();
    const long long N = tb.first[nact];
    const int it0 = (int)(N * blockIdx.x / gridDim.x), it1 = (int)(N * (blockIdx.x + 1) / gridDim.x);
    if (it0 >= it1) return;

    WBuf<NMAT, RGW, MAXT> w;
    half8 X[MAXT][4];
    int rbuf = 0;
    Item cur = S.item(tb, nact, it0, 0);
    S.issue(w, cur);
    S.load_x(X, cur);
    // Every item but the last refills the weight registers with the next
    // item's tiles while it is computed; the body is the same for every item
    // so the refilled registers need no copies on the loop's back edge.
    for (int it = it0; it + 1 < it1; ++it) {
        const Item nxt = S.item(tb, nact, it + 1, cur.slot);
        S.compute(cur, w, X, &nxt, red, rbuf);
        if (nxt.slot != cur.slot || nxt.mt != cur.mt) S.load_x(X, nxt);
        cur = nxt;
    }
    S.compute(cur, w, X, nullptr, red, rbuf);
}

constexpr int kDownRGW = 2;

int cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    static int ncu[64];
    if (dev >= 0 && dev < 64) {
        if (ncu[dev] == 0) {
            int v = 0;
            if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
            ncu[dev] = v;
        }
        return ncu[dev];
    }
    return 256;
}

// Launch: the number of 128-column tiles per wave selects the template
// instance; the grid is one wave of resident blocks (CUs x occupancy), capped
// by an upper bound of the number of work items.
template <int NMAT, int RGW, bool GATEUP>
int launch_stream(const FfnArgs &a, hipStream_t s, const char *who)
{
    const int K = GATEUP ? a.H : a.I;
    const int R = GATEUP ? a.I : a.H;
    const int maxt = (K / 128 + kWaves - 1) / kWaves;
    const long long pairs = (long long)a.T * a.k;
    const long long max_slots = pairs < a.E ? pairs : a.E;
    const long long max_items = (max_slots + pairs / 16) * (R / 16 / RGW);
    const int cus = cu_count();
    auto go = [&](auto kern) {
        int occ = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kThreads, 0) != hipSuccess || occ <= 0) occ = 1;
        long long g = (long long)cus * occ;
        if (g > max_items) g = max_items;
        if (g < 1) g = 1;
        hipLaunchKernelGGL(kern, dim3((unsigned int)g), dim3(kThreads), 0, s, a, a.active, a.offsets, a.slot_map,
                           a.n_active);
        return moe::check_launch(who);
    };
    switch (maxt) {
    case 1: return go(w4a16_stream_kernel<NMAT, RGW, 1, GATEUP>);
    case 2: return go(w4a16_stream_kernel<NMAT, RGW, 2, GATEUP>);
    default: return moe::fail(MOE_ERR_UNSUPPORTED, "%s: reduction length %d > 2048", who, K);
    }
}

int make_args(FfnArgs &a, const void *x_dev, int T, int H, int I, int E, int k, const void *rows_dev,
              size_t row_stride, const int32_t *slot_map_dev, const int32_t *expert_offsets_dev,
              const int32_t *sorted_pairs_dev, const int32_t *active_list_dev, const int32_t *n_active_dev,
              void *h_dev, float *pair_out_dev, int32_t *status_dev, const char *who)
{
    int rc = moe::check_shape(T, H, I, E, k, true);
    if (rc) return rc;
    if (T == 0) return -1;          // nothing to do; callers return MOE_OK
    if (H > 2048 || I > 2048) return moe::fail(MOE_ERR_UNSUPPORTED, "%s: H and I must be <= 2048", who);
    size_t off[6];
    const size_t rb = moe::row_bytes(H, I, off);
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
    a.off_gq = off[0]; a.off_uq = off[1]; a.off_dq = off[2];
    a.off_gs = off[3]; a.off_us = off[4]; a.off_ds = off[5];
    return MOE_OK;
}

int launch_gateup(const FfnArgs &a, hipStream_t s)
{
    return launch_stream<2, 1, true>(a, s, "moe_w4a16_gateup");
}

int launch_down(const FfnArgs &a, hipStream_t s)
{
    return launch_stream<1, kDownRGW, false>(a, s, "moe_w4a16_down");
}

}  // namespace

extern "C" {

int moe_w4a16_gateup(const void *x_dev, int T, int H, int I, int E, int k,
                     const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                     const int32_t *expert_offsets_dev, const int32_t *sorted_pairs_dev,
                     const int32_t *active_list_dev, const int32_t *n_active_dev,
                     void *h_dev, int32_t *status_dev, void *stream)
{
    moe::clear_error();
    FfnArgs a;
    int rc = make_args(a, x_dev, T, H, I, E, k, rows_dev, row_stride, slot_map_dev, expert_offsets_dev,
                       sorted_pairs_dev, active_list_dev, n_active_dev, h_dev, nullptr, status_dev,
                       "moe_w4a16_gateup");
    if (rc) return rc < 0 ? MOE_OK : rc;
    if (!x_dev || !sorted_pairs_dev) return moe::fail(MOE_ERR_INVALID_ARG, "moe_w4a16_gateup: null pointer argument");
    return launch_gateup(a, (hipStream_t)stream);
}

int moe_w4a16_down(int T, int H, int I, int E, int k,
                   const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                   const int32_t *expert_offsets_dev, const int32_t *active_list_dev,
                   const int32_t *n_active_dev, const void *h_dev, float *pair_out_dev,
                   int32_t *status_dev, void *stream)
{
    moe::clear_error();
    FfnArgs a;
    int rc = make_args(a, nullptr, T, H, I, E, k, rows_dev, row_stride, slot_map_dev, expert_offsets_dev,
                       nullptr, active_list_dev, n_active_dev, const_cast<void *>(h_dev), pair_out_dev, status_dev,
                       "moe_w4a16_down");
    if (rc) return rc < 0 ? MOE_OK : rc;
    if (!pair_out_dev) return moe::fail(MOE_ERR_INVALID_ARG, "moe_w4a16_down: null pointer argument");
    return launch_down(a, (hipStream_t)stream);
}

int moe_w4a16_expert_ffn(const void *x_dev, int T, int H, int I, int E, int k,
                         const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                         const int32_t *expert_offsets_dev, const int32_t *sorted_pairs_dev,
                         const int32_t *active_list_dev, const int32_t *n_active_dev,
                         void *h_dev, float *pair_out_dev, int32_t *status_dev, void *stream)
{
    moe::clear_error();
    FfnArgs a;
    int rc = make_args(a, x_dev, T, H, I, E, k, rows_dev, row_stride, slot_map_dev, expert_offsets_dev,
                       sorted_pairs_dev, active_list_dev, n_active_dev, h_dev, pair_out_dev, status_dev,
                       "moe_w4a16_expert_ffn");
    if (rc) return rc < 0 ? MOE_OK : rc;
    if (!x_dev || !sorted_pairs_dev || !pair_out_dev)
        return moe::fail(MOE_ERR_INVALID_ARG, "moe_w4a16_expert_ffn: null pointer argument");
    rc = launch_gateup(a, (hipStream_t)stream);
    if (rc) return rc;
    return launch_down(a, (hipStream_t)stream);
}

}  // extern "C"
