// The streaming W4A16 expert FFN of small batches as a device-side building
// block: expert_ffn.hip launches it per projection, layer_persistent.hip runs
// both projections inside the one-launch decode layer.  Not part of the C ABI.
//
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
// Kernel design (gfx950, wave64).  Decode batches are bound by HBM: the
// kernels exist to keep it busy with qpacked bytes while spending as few
// vector instructions per byte as possible.
//   * Work unit of a wavefront = one token tile (up to 16 routed tokens of an
//     expert) x one group of 16 weight rows x the whole reduction axis (or a
//     1/S slice of it for small batches, S in {2, 4, 8}, reduced in LDS).
//     The 8 wavefronts of a block take 8/S consecutive row groups of the
//     same token tile; blocks are persistent and walk a contiguous range of
//     such items, so the activations of a token tile are staged in LDS once
//     and shared by every row group of the block.
//   * Weights: one 16-byte buffer load per lane per 1024-byte tile (fully
//     coalesced, scalar tile offset + fixed lane offset).  A ring of D tiles
//     per matrix stays in flight; when a tile has been converted its
//     registers are reloaded with the tile D steps ahead, which at the end of
//     a unit is the first tile of the wavefront's next unit.  A unit that
//     reads no weights (nothing left, rows past the matrix, absent expert)
//     uses a buffer resource of 0 bytes: its loads return zeros and move no
//     memory.
//   * INT4 -> FP16 without arithmetic: a nibble moved to bits 4-7 of an FP16
//     half and masked out is the subnormal 16 * code * 2^-24 = code * 2^-20.
//     From a 32-bit word (8 codes, column 2i in the low nibble of byte i)
//     w & 0x00F000F0 gives columns (1, 5), (w << 4) & .. columns (0, 4),
//     (w >> 8) & .. columns (3, 7) and (w >> 4) & .. columns (2, 6): 7 vector
//     instructions per 8 weights, one MFMA B operand.  The activation
//     fragments in LDS are permuted to the same column order.  The matrix
//     cores take these subnormals without loss: measured against an exact
//     sum, code * 2^-20 operands err like FP32 rounding (2^-25 of the sum of
//     |terms|), while code * 2^-24 (the nibble left at bits 0-3) loses bits
//     (2^-19.6), so every nibble is moved up.
//   * The zero point: sum x * (code - 8) = sum x * code - 8 * sum x.  The
//     second term is per token and scale block, computed once while staging
//     the activations, and enters as the initial accumulator of the block's
//     MFMA chain.
//   * Per scale block: acc += scale * P in FP32 (the FP16 scale multiplies the
//     FP32 partial, weights are never rounded after scaling); the result is
//     acc * 2^20.
#pragma once

#include "ffn_common.h"

namespace {

using namespace ffn;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxNT = 16;                       // reduction axis <= 2048 columns

// Tiles kept in flight per matrix: the whole unit when it is short, else the
// largest divisor of the unit's tile count with at most maxw tiles of weights
// (an even one when there is one, so scale blocks never straddle rounds).
constexpr int ring_depth(int ntw, int nmat, int maxw)
{
    if (ntw * nmat <= 12) return ntw;
    int best = 1, best_even = 0;
    for (int d = 1; d * nmat <= maxw; ++d)
        if (ntw % d == 0) {
            best = d;
            if (d % 2 == 0) best_even = d;
        }
    return best_even ? best_even : best;
}

template <int NT, int S, int NMAT>
struct Shared {
    static constexpr int RS = S > 1 ? 1 : 0;
    u32x4 xl[NT * 4 * 64];            // activation fragments [tile][kind][lane]
    float sx[(NT + 1) / 2][16];       // -8 * 2^-20 * (sum of a token's activations over a scale block)
    float sxp[NT][4][16];             // staging partial sums [tile][32-column group][token]
    float red[RS ? S - 1 : 1][RS ? kWaves / S : 1][RS ? NMAT : 1][RS ? 4 : 1][RS ? 64 : 1];
    SlotTable tb;
};

// What one wavefront computes in one item.
struct Unit {
    const uint8_t *row;   // expert row (the rows base when nothing is read)
    int nrec;             // bytes the loads may read; 0: loads return zeros
    int slot;             // index into the slot table, -1 = no item
    int mt;               // token tile of the slot
    int rg;               // row group (valid when < RG)
    int p0;               // first grouped pair of the token tile
    int nval;             // tokens in the tile (1..16)
    bool write;           // the unit has rows to write
    bool absent;          // the expert has no device row
};

// F16W: the weights are FP16 values in the expanded slot layout (the
// offload-qpacked profile) instead of qpacked INT4: a 4096-byte tile covers
// the same 16 rows x 128 columns and is read as four coalesced 1024-byte
// pieces, piece q giving each lane one MFMA operand (row n16, columns
// 32*g4 + 8q .. +7 of the tile, natural order); no conversion, no zero
// point, no scale.
// DEV: the routing metadata and h are read, and h and the pair outputs
// written, at device scope (the one-launch layer hands them between blocks of
// the same launch).
template <bool GATEUP, int NT, int S, bool F16W = false, bool DEV = false>
struct Ffn {
    // Weight streams per wavefront: gate/up the gate and up rows of one row
    // group; down two adjacent row groups (each activation fragment then
    // feeds two MFMAs, and a unit streams twice the bytes per overhead) when
    // the reduction axis has an even number of tiles, else one (measured:
    // with an odd count the two-stream ring cannot be deep enough).
    static constexpr int NMAT = (GATEUP || NT % 2 == 0) ? 2 : 1;
    static constexpr int RPW = GATEUP ? 1 : NMAT;  // output row groups per wavefront
    static constexpr int NTW = NT / S;          // tiles of one wavefront
    static constexpr int RGB = kWaves / S;      // wavefront row slots per item
    static constexpr int NB = (NT + 1) / 2;     // scale blocks of the reduction axis
    static constexpr int QW = F16W ? 4 : 1;    // 16-byte loads per lane per tile
    // 8 tiles of weights in flight per wavefront; 16 in the one-launch layer
    // (DEV), which runs one block per CU instead of two (its routing stage
    // needs the registers), so a CU keeps the same bytes in flight.
    static constexpr int D = ring_depth(NTW, NMAT * QW, DEV ? 16 : 8);
    static constexpr float kOut = F16W ? 1.0f : kUnit;
    static_assert(NT >= 1 && NT <= kMaxNT, "reduction axis of 128 .. 2048 columns");
    static_assert(NT % S == 0 && (S == 1 || NTW % 2 == 0), "split slices cover whole scale blocks");
    static_assert(NTW % D == 0, "ring depth divides the unit");

    using Lds = Shared<NT, S, NMAT>;

    const FfnArgs &a;
    Lds &L;
    int lane, wave, g4, n16, ks, rgl, t0;
    int RG, CH;               // row groups of the output, items per token tile
    int nact;

    __device__ Ffn(const FfnArgs &args, Lds &lds, int nact_) : a(args), L(lds), nact(nact_)
    {
        const int tid = threadIdx.x;
        lane = tid & 63;
        wave = uni(tid >> 6);
        g4 = lane >> 4;
        n16 = lane & 15;
        ks = wave % S;
        rgl = wave / S;
        t0 = ks * NTW;
        RG = (GATEUP ? a.I : a.H) / 16;
        CH = (RG + RGB * RPW - 1) / (RGB * RPW);
    }

    // Unit of this wavefront in item `it` (slot search starts at `hint`).
    __device__ Unit unit(int it, int hint) const
    {
        int s = hint;
        while (s + 1 < nact && L.tb.first[s + 1] <= it) ++s;
        s = uni(s);
        Unit u;
        u.slot = s;
        const int local = uni(it - L.tb.first[s]);
        u.mt = local / CH;
        const int c = local - u.mt * CH;
        const int n = uni(L.tb.n[s]);
        const int sl = uni(L.tb.sl[s]);
        u.p0 = uni(L.tb.p0[s]) + 16 * u.mt;
        u.nval = min(16, n - 16 * u.mt);
        u.rg = (c * RGB + rgl) * RPW;
        u.absent = sl < 0;
        u.write = u.rg < RG;
        const bool reads = u.write && !u.absent;
        u.row = a.rows + (reads ? (size_t)sl * a.stride : 0);
        u.nrec = reads ? a.row_bytes : 0;
        if (!u.write) u.rg = 0;
        return u;
    }

    __device__ Unit none() const
    {
        Unit u;
        u.row = a.rows;
        u.nrec = 0;
        u.slot = -1;
        u.mt = 0;
        u.rg = 0;
        u.p0 = 0;
        u.nval = 0;
        u.write = false;
        u.absent = false;
        return u;
    }

    // Tile j of a unit (row base, readable bytes, row group) of stream mat:
    // gate/up matrix mat of row group rg, down row group rg + mat.
    __device__ u32x4 load_q(const uint8_t *row, int nrec, int rg, int mat, int j) const
    {
        const int qm = GATEUP ? a.off_q[mat] : a.off_q[2];
        const int r = GATEUP ? rg : rg + mat;
        return __builtin_amdgcn_raw_buffer_load_b128(rsrc(row, nrec), lane * 16, qm + ((r * NT) + t0 + j) * 1024, 0);
    }

    // All QW loads of tile j into w (the qpacked tile, or the four FP16 pieces).
    __device__ void load_tile(u32x4 (&w)[QW], const uint8_t *row, int nrec, int rg, int mat, int j) const
    {
        if constexpr (F16W) {
            const int qm = GATEUP ? a.off_q[mat] : a.off_q[2];
            const int r = GATEUP ? rg : rg + mat;
            const int base = qm + ((r * NT) + t0 + j) * 4096;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                w[q] = __builtin_amdgcn_raw_buffer_load_b128(rsrc(row, nrec), lane * 16, base + q * 1024, 0);
        } else {
            w[0] = load_q(row, nrec, rg, mat, j);
        }
    }

    // FP16 scale of the block of tile j, row n16 of the row group.
    __device__ _Float16 load_s(const uint8_t *row, int nrec, int rg, int mat, int j) const
    {
        const int sm = GATEUP ? a.off_s[mat] : a.off_s[2];
        const int r = GATEUP ? rg : rg + mat;
        const uint16_t b = __builtin_amdgcn_raw_buffer_load_b16(rsrc(row, nrec), n16 * 2,
                                                                 sm + (r * NB + (t0 + j) / 2) * 32, 0);
        return __builtin_bit_cast(_Float16, b);
    }

    // Activations of a token tile -> LDS fragments (permuted to the column
    // order of the weight conversion) and per-block sums for the zero point.
    __device__ void stage(const Unit &u) const
    {
        lds_barrier();                     // every wave is done with the previous tile
        const int nval = u.nval;
        for (int task = threadIdx.x; task < 16 * NT * 4; task += kThreads) {
            const int m = task & 15, tg = task >> 4;
            const int t = tg >> 2, g = tg & 3;
            u32x4 d0 = {0u, 0u, 0u, 0u}, d1 = d0, d2 = d0, d3 = d0;
            if (m < nval) {
                const uint16_t *src = nullptr;
                if (GATEUP) {
                    const int tok = moe::get<DEV>(&a.sorted_pairs[u.p0 + m]) / a.k;
                    if (tok >= 0 && tok < a.T) src = a.x + (size_t)tok * a.H;
                } else {
                    src = a.h + (size_t)(u.p0 + m) * a.I;
                }
                if (src && (GATEUP || !DEV)) {
                    src += 128 * t + 32 * g;
                    d0 = ld16(src);
                    d1 = ld16(src + 8);
                    d2 = ld16(src + 16);
                    d3 = ld16(src + 24);
                } else if (src) {
                    // h of this launch: 16-byte loads at device scope
                    const __amdgpu_buffer_rsrc_t r = rsrc(a.h, a.T * a.k * a.I * 2);
                    const int o = ((u.p0 + m) * a.I + 128 * t + 32 * g) * 2;
                    d0 = __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, moe::kDevScope);
                    d1 = __builtin_amdgcn_raw_buffer_load_b128(r, o + 16, 0, moe::kDevScope);
                    d2 = __builtin_amdgcn_raw_buffer_load_b128(r, o + 32, 0, moe::kDevScope);
                    d3 = __builtin_amdgcn_raw_buffer_load_b128(r, o + 48, 0, moe::kDevScope);
                }
            }
            u32x4 *dst = &L.xl[(t * 4) * 64 + g * 16 + m];
            // kind q holds columns 8q + (1, 5, 0, 4, 3, 7, 2, 6) of the group,
            // the order in which the weight conversion yields them
            if constexpr (F16W) {
                dst[0] = d0;
                dst[64] = d1;
                dst[128] = d2;
                dst[192] = d3;
                continue;
            }
            dst[0] = permute_activations(d0);
            dst[64] = permute_activations(d1);
            dst[128] = permute_activations(d2);
            dst[192] = permute_activations(d3);
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s += half_bits_to_float(d0[i]) + half_bits_to_float(d0[i] >> 16);
                s += half_bits_to_float(d1[i]) + half_bits_to_float(d1[i] >> 16);
                s += half_bits_to_float(d2[i]) + half_bits_to_float(d2[i] >> 16);
                s += half_bits_to_float(d3[i]) + half_bits_to_float(d3[i] >> 16);
            }
            L.sxp[t][g][m] = s;
        }
        lds_barrier();
        if constexpr (F16W) return;
        for (int i = threadIdx.x; i < NB * 16; i += kThreads) {
            const int b = i >> 4, m = i & 15;
            float s = 0.f;
            for (int t = 2 * b; t < 2 * b + 2 && t < NT; ++t)
#pragma unroll
                for (int g = 0; g < 4; ++g) s += L.sxp[t][g][m];
            L.sx[b][m] = s * kZeroPoint;
        }
        lds_barrier();
    }

    // One unit: stream the weight tiles through the ring, refilling each slot
    // with the tile D steps ahead (from unit `nxt` past the end), then write
    // the unit's outputs.  Rounds of D tiles run as a loop, so the ring slot
    // of every tile is fixed and the loop carries the ring in place.
    __device__ void run(const Unit &cur, const Unit &nxt, u32x4 (&wq)[D][NMAT][QW], _Float16 (&ws)[D][NMAT]) const
    {
        constexpr int NR = NTW / D;
        const u32x4 *xl = &L.xl[t0 * 4 * 64 + lane];
        const f32x4 *sx = reinterpret_cast<const f32x4 *>(&L.sx[t0 / 2][4 * g4]);
        f32x4 acc[NMAT], p[NMAT];
#pragma unroll
        for (int mat = 0; mat < NMAT; ++mat) acc[mat] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int jo = 0; jo < NR; ++jo) {
            // the refills of this round: the next round of this unit, or the
            // first round of the next unit
            const bool last = jo == NR - 1;
            const uint8_t *rrow = last ? nxt.row : cur.row;
            const int rnrec = last ? nxt.nrec : cur.nrec;
            const int rrg = last ? nxt.rg : cur.rg;
            const int rj0 = last ? 0 : (jo + 1) * D;
#pragma unroll
            for (int jd = 0; jd < D; ++jd) {
                const int j = jo * D + jd;
                if (!F16W && j % 2 == 0) {
                    const f32x4 z = sx[(j / 2) * 4];      // zero-point term of this scale block
#pragma unroll
                    for (int mat = 0; mat < NMAT; ++mat) p[mat] = z;
                }
                half8 xa[4];
#pragma unroll
                for (int kd = 0; kd < 4; ++kd) xa[kd] = __builtin_bit_cast(half8, xl[(j * 4 + kd) * 64]);
                const bool merge = (j % 2 == 1) || (j == NTW - 1);
                float sc[NMAT];
#pragma unroll
                for (int mat = 0; mat < NMAT; ++mat) {
                    if constexpr (F16W) {
                        half8 b[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) b[q] = __builtin_bit_cast(half8, wq[jd][mat][q]);
                        __builtin_amdgcn_sched_barrier(0);
                        load_tile(wq[jd][mat], rrow, rnrec, rrg, mat, rj0 + jd);
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[mat] = mfma(xa[q], b[q], acc[mat]);
                        continue;
                    }
                    const u32x4 w = wq[jd][mat][0];
                    half8 b[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) b[q] = codes_to_operand(w[q]);
                    sc[mat] = scale_f32(ws[jd][mat]);
                    // every read of this slot happens above: reload it in place
                    __builtin_amdgcn_sched_barrier(0);
                    wq[jd][mat][0] = load_q(rrow, rnrec, rrg, mat, rj0 + jd);
                    ws[jd][mat] = load_s(rrow, rnrec, rrg, mat, rj0 + jd);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int q = 0; q < 4; ++q) p[mat] = mfma(xa[q], b[q], p[mat]);
                }
                if (!F16W && merge) {
#pragma unroll
                    for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[mat][r] += sc[mat] * p[mat][r];
                }
            }
        }
        if (S > 1) {
            // K slices 1..S-1 hand their partials to slice 0 of the same row group
            if (ks > 0) {
#pragma unroll
                for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                    for (int r = 0; r < 4; ++r) L.red[ks - 1][rgl][mat][r][lane] = acc[mat][r];
            }
            lds_barrier();
            if (ks == 0) {
#pragma unroll
                for (int q = 1; q < S; ++q)
#pragma unroll
                    for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[mat][r] += L.red[q - 1][rgl][mat][r][lane];
            }
            lds_barrier();
            if (ks != 0) return;
        }
        if (!cur.write) return;
        if (cur.absent && lane == 0 && a.status) *a.status = MOE_ERR_ABSENT_EXPERT;
        // lane (g4, n16) holds tokens 4*g4 + r of row n16 of the row group
        // (down: of row groups rg and rg + 1, both present: H % 128 == 0)
        const int col = cur.rg * 16 + n16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * g4 + r;
            if (m < cur.nval) {
                const size_t pr = (size_t)(cur.p0 + m);
                if constexpr (GATEUP) {
                    const float g = acc[0][r] * kOut, u = acc[NMAT - 1][r] * kOut;
                    const uint16_t hv = cur.absent ? (uint16_t)0 : float_to_half_bits(g / (1.0f + expf(-g)) * u);
                    if constexpr (DEV)
                        __builtin_amdgcn_raw_buffer_store_b16(hv, rsrc(a.h, a.T * a.k * a.I * 2),
                                                              (int)((pr * a.I + col) * 2), 0, moe::kDevScope);
                    else
                        a.h[pr * a.I + col] = hv;
                } else {
#pragma unroll
                    for (int mat = 0; mat < NMAT; ++mat)
                        moe::put<DEV>(&a.out[pr * a.H + col + 16 * mat], cur.absent ? 0.0f : acc[mat][r] * kOut);
                }
            }
        }
    }
};

}  // namespace
