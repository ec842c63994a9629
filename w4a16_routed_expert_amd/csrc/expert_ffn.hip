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
#include "ffn_common.h"

namespace {

using namespace ffn;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxNT = 16;                       // reduction axis <= 2048 columns

// Tiles kept in flight per matrix: the whole unit when it is short, else the
// largest divisor of the unit's tile count with at most 8 tiles of weights
// (an even one when there is one, so scale blocks never straddle rounds).
constexpr int ring_depth(int ntw, int nmat)
{
    if (ntw * nmat <= 12) return ntw;
    int best = 1, best_even = 0;
    for (int d = 1; d * nmat <= 8; ++d)
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
template <bool GATEUP, int NT, int S, bool F16W = false>
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
    static constexpr int D = ring_depth(NTW, NMAT * QW);
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
                    const int tok = a.sorted_pairs[u.p0 + m] / a.k;
                    if (tok >= 0 && tok < a.T) src = a.x + (size_t)tok * a.H;
                } else {
                    src = a.h + (size_t)(u.p0 + m) * a.I;
                }
                if (src) {
                    src += 128 * t + 32 * g;
                    d0 = ld16(src);
                    d1 = ld16(src + 8);
                    d2 = ld16(src + 16);
                    d3 = ld16(src + 24);
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
                    a.h[pr * a.I + col] = cur.absent ? (uint16_t)0 : float_to_half_bits(g / (1.0f + expf(-g)) * u);
                } else {
#pragma unroll
                    for (int mat = 0; mat < NMAT; ++mat)
                        a.out[pr * a.H + col + 16 * mat] = cur.absent ? 0.0f : acc[mat][r] * kOut;
                }
            }
        }
    }
};

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
#pragma unroll
    for (int j = 0; j < F::D; ++j)
#pragma unroll
        for (int mat = 0; mat < F::NMAT; ++mat) {
            f.load_tile(wq[j][mat], cur.row, cur.nrec, cur.rg, mat, j);
            if constexpr (!F16W) ws[j][mat] = f.load_s(cur.row, cur.nrec, cur.rg, mat, j);
        }
    f.stage(cur);
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
