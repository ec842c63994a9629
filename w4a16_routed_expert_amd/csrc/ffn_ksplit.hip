// W4A16 expert FFN of small decode batches in one launch, with no block
// waiting for another: the work is cut along the expert's intermediate axis.
//
// Operation and rounding points are those of the streaming kernels
// (expert_ffn.hip): qpacked INT4 weights converted inside the kernel ("Horizon
// RunMap - architecture", section "Representation and computation"), FP16
// activations, FP32 accumulation, h = RN16(silu(g) * u) ("horizonrunmap.com/
// en", section "08 / Precision & quality").  What differs is the split:
//   * A work item is (active expert, slice j of W consecutive columns of the
//     intermediate axis I).  Its block computes g and u for the slice's W
//     rows of the gate and up matrices over all of H, rounds h for those W
//     columns into LDS, and multiplies them with the matching W columns of
//     the down matrix for all H output rows.  The result is a partial pair
//     output (the down projection's sum over the slice's columns only),
//     written to plane j of the partial-output planes [I/W][T*k][H]; the
//     combine adds the planes of a pair in plane order.  h never leaves the
//     block, so gate/up and down need no second launch and no exchange
//     between blocks (the L2 caches of the XCDs are not coherent with each
//     other within a launch).
//   * Used for batches of at most 16 tokens, where every expert has one token
//     tile: the launch start and the planes' traffic (T*k*H*4 bytes per
//     plane) are then small against two launches of the streaming kernels.
//   * Gate/up: the slice's W/16 row groups times the waves' shares of the
//     reduction axis (8 waves: W/16 row groups x 128/W quarters of H);
//     partial sums meet in LDS in wave order.  Weights: one 16-byte load per
//     lane per 1 KB tile (row n16, columns 32 g4 .. +31); activations: the
//     same 32 columns of the lane's token, loaded from memory; a ring of up
//     to 4 tiles in flight.  Each word of 8 codes becomes one MFMA operand in
//     natural column order with the zero point folded in: the nibble in bits
//     4-7 of a half is the subnormal code * 2^-20, and adding -8 * 2^-20
//     (a packed FP16 add) gives (code - 8) * 2^-20 exactly.  Per scale block
//     acc += scale * P in FP32; results are acc * 2^20.
//   * Down: every wave takes H/128 row groups; for each, the slice's W
//     columns are W/32 dword loads per lane (lane (g4, n16): word g4 of the
//     32-column group of row n16, 256 contiguous bytes per instruction), one
//     scale per row (a slice never straddles a 256-column scale block), and
//     the h slice from LDS as the other MFMA operand.
#include "ffn_common.h"

namespace {

using namespace ffn;

constexpr int kKWaves = 8;
constexpr int kKThreads = 64 * kKWaves;
constexpr uint32_t kNone = 0x40000000u;     // lane offset past every buffer used here: the load returns zeros

template <int W>
struct KsLds {
    static constexpr int RGW = W / 16;
    static constexpr int KQ = kKWaves / RGW;
    float red[KQ > 1 ? KQ - 1 : 1][RGW][2][4][64];   // gate/up partial sums of waves kq >= 1
    uint16_t hs[16][W + 8];                          // h slice: token m, column c (FP16 bits); padded rows
    SlotTable tb;
};

template <int NTH, int W>
__global__ __launch_bounds__(kKThreads) void w4a16_ffn_ksplit_kernel(FfnArgs a, float *planes,
                                                                     const int32_t *__restrict__ active,
                                                                     const int32_t *__restrict__ offsets,
                                                                     const int32_t *__restrict__ slot_map,
                                                                     const int32_t *__restrict__ n_active)
{
    constexpr int RGW = W / 16;           // gate/up row groups of a slice
    constexpr int KQ = kKWaves / RGW;      // waves per row group (shares of H)
    constexpr int NTW = NTH / KQ;          // gate/up tiles per wave
    constexpr int D = NTW % 4 == 0 ? 4 : 2;   // tiles in flight (divides NTW, which is even)
    constexpr int GC = W / 32;             // 32-column groups of the down slice
    constexpr int NB = (NTH + 1) / 2;      // scale blocks of H
    constexpr int DB = GC >= 4 ? 8 : 16;   // down row groups in flight per wave
    static_assert(KQ * RGW == kKWaves, "8 waves cover the slice");
    static_assert(NTH % KQ == 0 && NTW % 2 == 0 && NTW % D == 0, "whole scale blocks per wave");
    __shared__ KsLds<W> L;

    TableIn tin{};
    if (threadIdx.x < 64) tin = table_loads(a, active, offsets, slot_map);
    int nact = *n_active;
    if (nact > a.E) nact = a.E;
    if (nact <= 0) return;
    const int S = a.I / W;                 // slices (= planes)
    if (threadIdx.x < 64) build_table(L.tb, a, tin, nact, 16, S);
    __syncthreads();
    const int N = L.tb.first[nact];

    const int lane = threadIdx.x & 63, wave = uni(threadIdx.x >> 6);
    const int g4 = lane >> 4, n16 = lane & 15;
    const int rgl = wave / KQ, kq = wave % KQ;
    const int NTI = a.I / 128, NBI = (a.I + 255) / 256;
    const int DPW = a.H / 128;             // down row groups per wave
    const size_t plane = (size_t)a.T * a.k * a.H;
    const _Float16 zs = (_Float16)kZeroPoint;
    const half8 zp = {zs, zs, zs, zs, zs, zs, zs, zs};
    const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, a.T * a.H * 2);

    int hint = 0;
    for (int it = blockIdx.x; it < N; it += gridDim.x) {
        int s = hint;
        while (s + 1 < nact && L.tb.first[s + 1] <= it) ++s;
        s = uni(s);
        hint = s;
        const int j = uni(it - L.tb.first[s]);            // slice (one token tile per slot)
        const int p0 = uni(L.tb.p0[s]);
        const int n = uni(min(16, L.tb.n[s]));
        const int sl = uni(L.tb.sl[s]);
        const bool absent = sl < 0;
        const uint8_t *row = a.rows + (absent ? 0 : (size_t)sl * a.stride);
        const __amdgpu_buffer_rsrc_t rw = rsrc(row, absent ? 0 : a.row_bytes);
        if (absent && threadIdx.x == 0 && a.status) *a.status = MOE_ERR_ABSENT_EXPERT;
        // this lane's token (lane n16 of the MFMA activation operand)
        uint32_t xoff = kNone;
        if (n16 < n) {
            const int tok = a.sorted_pairs[p0 + n16] / a.k;
            if (tok >= 0 && tok < a.T) xoff = (uint32_t)tok * (uint32_t)(a.H * 2) + 64u * g4;
        }

        // ---- gate/up: row group rg of the slice, tiles kt0 .. kt0 + NTW - 1 of H
        const int rg = j * RGW + rgl;
        const int kt0 = kq * NTW;
        u32x4 wq[D][2], xq[D][4];
        _Float16 ws[D][2];
        auto issue = [&](int d, int t) {
            const int kt = kt0 + t;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                wq[d][m] = __builtin_amdgcn_raw_buffer_load_b128(rw, lane * 16, a.off_q[m] + (rg * NTH + kt) * 1024, 0);
                ws[d][m] = __builtin_bit_cast(_Float16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(
                                                            rw, n16 * 2, a.off_s[m] + (rg * NB + kt / 2) * 32, 0));
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) xq[d][q] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff, kt * 256 + 16 * q, 0);
        };
#pragma unroll
        for (int d = 0; d < D; ++d) issue(d, d);
        f32x4 acc[2], P[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) acc[m] = P[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int r0 = 0; r0 < NTW; r0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int t = r0 + d;
                half8 xa[4], b[2][4];
                float sc[2];
#pragma unroll
                for (int q = 0; q < 4; ++q) xa[q] = __builtin_bit_cast(half8, xq[d][q]);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) b[m][q] = codes_to_signed_natural(wq[d][m][q], zp);
                    sc[m] = scale_f32(ws[d][m]);
                }
                // every read of ring slot d is above: refill it with the tile D ahead
                __builtin_amdgcn_sched_barrier(0);
                if (t + D < NTW) issue(d, t + D);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int q = 0; q < 4; ++q) P[m] = mfma(xa[q], b[m][q], P[m]);
                if (t % 2 == 1) {
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[m][r] += sc[m] * P[m][r];
                        P[m] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                }
            }
        }

        // ---- down loads of this wave, the first DB of them issued before the
        // h slice is complete: row groups wave + 8 i, the slice's GC 32-column
        // groups and one scale per row
        uint32_t dq[DB][GC];
        _Float16 dsc[DB];
        auto issue_down = [&](int slot, int i) {
            const int rgd = wave + 8 * i;
#pragma unroll
            for (int gc = 0; gc < GC; ++gc) {
                // uniform part (tile, 32-column group) as the scalar offset,
                // the lane's part (row n16, word g4) as the vector offset
                const int c0 = j * W + 32 * gc;
                const int off = a.off_q[2] + (rgd * NTI + (c0 >> 7)) * 1024 + ((c0 >> 5) & 3) * 256;
                dq[slot][gc] = __builtin_amdgcn_raw_buffer_load_b32(rw, n16 * 16 + 4 * g4, off, 0);
            }
            dsc[slot] = __builtin_bit_cast(_Float16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(
                                                         rw, n16 * 2, a.off_s[2] + (rgd * NBI + (j * W) / 256) * 32, 0));
        };
#pragma unroll
        for (int i = 0; i < DB; ++i)
            if (i < DPW) issue_down(i, i);

        // ---- the wave's gate/up sums meet in LDS (wave order); h of the slice
        if (kq > 0) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) L.red[kq - 1][rgl][m][r][lane] = acc[m][r];
        }
        lds_barrier();
        if (kq == 0) {
#pragma unroll
            for (int q = 1; q < KQ; ++q)
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[m][r] += L.red[q - 1][rgl][m][r][lane];
            // lane (g4, n16): tokens 4 g4 + r of row n16 of row group rg
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * g4 + r;
                const float g = acc[0][r] * kUnit, u = acc[1][r] * kUnit;
                const uint16_t hb = (m < n && !absent) ? float_to_half_bits(g / (1.0f + expf(-g)) * u) : (uint16_t)0;
                L.hs[m][rgl * 16 + n16] = hb;
                if (m < n) a.h[(size_t)(p0 + m) * a.I + rg * 16 + n16] = hb;
            }
        }
        lds_barrier();

        // ---- down: partial outputs of the slice for every output row
        half8 ha[GC];
#pragma unroll
        for (int gc = 0; gc < GC; ++gc) ha[gc] = *reinterpret_cast<const half8 *>(&L.hs[n16][32 * gc + 8 * g4]);
        float *pl = planes + (size_t)j * plane;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i < DPW) {
                const int rgd = wave + 8 * i;
                const int slot = i % DB;          // a constant once the loop is unrolled
                half8 bq[GC];
#pragma unroll
                for (int gc = 0; gc < GC; ++gc) bq[gc] = codes_to_signed_natural(dq[slot][gc], zp);
                const float sc = scale_f32(dsc[slot]) * kUnit;
                // the slot is free again: it loads the row group DB further on
                __builtin_amdgcn_sched_barrier(0);
                if (i + DB < DPW) issue_down(slot, i + DB);
                __builtin_amdgcn_sched_barrier(0);
                f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int gc = 0; gc < GC; ++gc) p = mfma(ha[gc], bq[gc], p);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 4 * g4 + r;
                    if (m < n) pl[(size_t)(p0 + m) * a.H + rgd * 16 + n16] = absent ? 0.0f : sc * p[r];
                }
            }
        }
        // the next item overwrites the h slice: every wave is done reading it
        lds_barrier();
    }
}

template <int NTH, int W>
int launch_w(const FfnArgs &a, float *planes, hipStream_t s, const char *who)
{
    auto kern = w4a16_ffn_ksplit_kernel<NTH, W>;
    static int occ_cache[64];
    const int occ = moe::blocks_per_cu(kern, kKThreads, occ_cache);
    const long long pairs = (long long)a.T * a.k;
    const long long items = (pairs < a.E ? pairs : a.E) * (a.I / W);
    long long g = (long long)cu_count() * occ;
    if (g > items) g = items;
    if (g < 1) g = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned int)g), dim3(kKThreads), 0, s, a, planes, a.active, a.offsets, a.slot_map,
                       a.n_active);
    return moe::check_launch(who);
}

template <int NTH>
int launch_nth(const FfnArgs &a, float *planes, int W, hipStream_t s, const char *who)
{
    if constexpr (NTH % 8 == 0) {
        if (W == 32) return launch_w<NTH, 32>(a, planes, s, who);
    }
    if constexpr (NTH % 4 == 0) {
        if (W == 64) return launch_w<NTH, 64>(a, planes, s, who);
    }
    if (W == 128) return launch_w<NTH, 128>(a, planes, s, who);
    return moe::fail(MOE_ERR_UNSUPPORTED, "%s: slice width %d with H = %d", who, W, NTH * 128);
}

}  // namespace

// Slice width for a batch: the widest of 128, 64, 32 columns (fewer planes
// to write and add) that still gives about one item per CU for the number
// of experts a uniform router activates on average, else the narrowest the
// shape allows; 0 when the kernel does not apply (more than 16 tokens, H or
// I over 2048, or H/128 odd).  A launch-shape choice: every width computes
// the same sums, only their grouping into planes differs.
int ffn::ksplit_width(int T, int H, int I, int E, int k)
{
    if (T < 1 || T > 16 || H > 2048 || I > 2048 || I % 128 || H % 256) return 0;
    const int NTH = H / 128;
    double miss = 1.0;
    for (int i = 0; i < T; ++i) miss *= 1.0 - (double)k / E;
    const double active = E * (1.0 - miss);
    const int widths[3] = {128, 64, 32};
    int best = 0;
    for (int w : widths) {
        const int kq = kKWaves / (w / 16);
        if (NTH % kq || (NTH / kq) % 2) continue;
        best = w;
        if (active * (I / w) >= 0.99 * cu_count()) break;
    }
    return best;
}

int ffn::launch_ksplit(const FfnArgs &a, float *planes, int W, hipStream_t s, const char *who)
{
    switch (a.H / 128) {
    case 2: return launch_nth<2>(a, planes, W, s, who);
    case 4: return launch_nth<4>(a, planes, W, s, who);
    case 6: return launch_nth<6>(a, planes, W, s, who);
    case 8: return launch_nth<8>(a, planes, W, s, who);
    case 10: return launch_nth<10>(a, planes, W, s, who);
    case 12: return launch_nth<12>(a, planes, W, s, who);
    case 14: return launch_nth<14>(a, planes, W, s, who);
    case 16: return launch_nth<16>(a, planes, W, s, who);
    default: return moe::fail(MOE_ERR_UNSUPPORTED, "%s: H = %d", who, a.H);
    }
}
