// W4A16 expert FFN for large batches: a grouped GEMM over the routed pairs of
// each active expert, read straight from qpacked INT4 expert rows (same
// operation and rounding points as the streaming kernel of expert_ffn.hip:
// routed experts stay compact INT4 with FP16 block scales and are converted
// inside the kernel, "Horizon RunMap - architecture", table "Representation
// and computation"; FP16 activations and FP32 accumulation stages,
// "horizonrunmap.com/en", section "08 / Precision & quality").
//
// With hundreds of pairs per expert the layer is bound by the matrix cores,
// not by HBM, so the design maximises MFMA work per converted weight and per
// LDS byte and keeps every global load off the instruction stream:
//   * v_mfma_f32_32x32x16_f16 (8 passes: the same rate per FLOP as the
//     16x16x32 form, half the instructions).
//   * Work item = 128 grouped pairs of one expert x one block of output rows
//     (gate/up: 128 rows of I for both matrices; down: 256 rows of H).  A
//     block of 8 wavefronts takes one item; every wavefront owns all 128
//     pairs (4 m-tiles of 32) x one 32-row n-tile: for gate/up 16 rows of the
//     gate matrix and the same 16 rows of the up matrix, for down 32 rows of
//     H.  Each converted weight operand feeds 4 MFMAs.  The weights are the
//     first MFMA operand, so a lane of the result holds one pair and 4
//     consecutive output rows per register quad: gate and up of an output
//     meet in the same lane, and the outputs leave as 8- and 16-byte stores.
//   * Activations staged with direct global-to-LDS loads (no registers, no
//     VALU): the item's 128 activation rows (gathered through sorted_pairs
//     for gate/up) per K-tile of 128 columns, two K-tiles (one scale block)
//     at a time with each wavefront's 32 row scales of that block, in a ring
//     of two such pairs: each K-tile of a pair stages its counterpart of the
//     next pair (the second also the scales), and one barrier per pair,
//     preceded by a wait that counts the loads issued since, publishes it
//     (one barrier per K-tile, or the whole next pair staged by the first
//     K-tile, measured slower).  Each wavefront's weights are its
//     own: they go straight into registers (two 16-byte loads per lane per
//     K-tile, issued one K-tile ahead) - staging them through LDS as well
//     was measured 3% slower.
//     Activation layout: 64-byte granules, granule (row / 4, piece ^ (row / 4
//     % 4)) holds the 16-byte piece of 4 consecutive rows, so one direct load
//     instruction fills a whole 1 KB granule run and the MFMA operand reads
//     (32 rows x 2 pieces per instruction) are free of bank conflicts.  The
//     operand reads run several MFMAs ahead of their use.
//   * Weights: K-step s of a lane uses word s % 4 of chunk s / 4 of its row
//     (lanes 0-31 columns 32 h2 + 64 (s / 4) + 8 (s % 4).., lanes 32-63 the
//     columns 32 further on) and the activation reads the same columns.  Each
//     8-code word becomes one operand in natural column order (7 VALU + 4
//     packed adds).
//   * Zero point in the operand: the converted subnormal code * 2^-20 minus
//     8 * 2^-20 (one packed FP16 add per dword) is (code - 8) * 2^-20 exactly,
//     so no activation sums are needed.  Per scale block the 8 K-steps
//     accumulate P = sum x * (code - 8) * 2^-20 on the matrix cores, then
//     acc += scale * P in FP32 (weights never rounded after scaling); the
//     result is acc * 2^20.
//   * An odd number of K-tiles is padded with one K-tile whose weight
//     operands are exactly zero, so every scale block has two ring slots.
#include "ffn_common.h"

#include <type_traits>

namespace {

using namespace ffn;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kBM = 128;              // grouped pairs per item
constexpr int kStageBytes = kBM * 256;  // one staged K-tile
constexpr int kStages = 4;            // staged K-tiles: two pairs
constexpr int kMT = 4;                // m-tiles (32 pairs) per wavefront: all 128 pairs of the item
constexpr int kPD = 4;                // operand reads in flight ahead of the MFMAs
// Buffer offset of a row (or lane) that reads nothing: past every resource
// used here (at most 256 MiB) and positive as a signed 32-bit value, so the
// range check of the buffer load turns it into zeros.
constexpr uint32_t kNone = 0x40000000u;

struct GLds {
    uint8_t xa[kStages][kStageBytes];    // staged activations (layout: see stage_addr); pair slot q: stages 2q, 2q + 1
    uint8_t sc[2][kGWaves][256];         // each wavefront's 32 row scales of a pair's scale block (64 bytes used)
    uint32_t src[2][kBM];                // byte offset of each pair's activation row (kNone: none), two items
    SlotTable tb;
};

// One work item as every lane of the block sees it (all fields uniform).
struct GItem {
    const uint8_t *row;   // expert row (the rows base when nothing is read)
    int nrec;             // readable bytes of the row; 0 = read nothing
    int p0;               // first grouped pair of the item
    int nval;             // valid pairs, 0..128 (0: no item)
    int rg0;              // first row group of the item
    int absent;           // the expert has no device row
};

// Byte offset of 16-byte piece c (columns 8c .. 8c+7 of the K-tile) of
// staged row r: granule (r / 4) * 16 + (c ^ (r / 4 % 4)) of 64 bytes, slot r % 4.
__device__ inline int stage_addr(int r, int c) { return (((r >> 2) << 4) + (c ^ ((r >> 2) & 3))) * 64 + (r & 3) * 16; }

__device__ inline f32x16 mfma32(half8 a, half8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <bool GATEUP>
struct Gemm {
    static constexpr int RGW = GATEUP ? 1 : 2;   // row groups of 16 per wavefront (gate/up: in both matrices)
    static constexpr int RGB = kGWaves * RGW;    // row groups per item

    const FfnArgs &a;
    GLds &L;
    int nact;
    int lane, wave, j32, h2;
    int K, NT, NTP, NBK, RG, NBLK;
    int aq[4];                           // stage_addr of this lane's operand pieces, m-tile 0, K-steps q (+ 4n)

    __device__ Gemm(const FfnArgs &args, GLds &lds, int nact_) : a(args), L(lds), nact(nact_)
    {
        const int tid = threadIdx.x;
        lane = tid & 63;
        wave = uni(tid >> 6);
        j32 = lane & 31;                 // MFMA column (output row) of the lane
        h2 = lane >> 5;                  // which 8 of the 16 K values the lane feeds
        K = GATEUP ? a.H : a.I;
        NT = K / 128;
        NTP = NT + (NT & 1);
        NBK = (NT + 1) / 2;
        RG = (GATEUP ? a.I : a.H) / 16;
        NBLK = (RG + RGB - 1) / RGB;
        for (int q = 0; q < 4; ++q) aq[q] = stage_addr(j32, 4 * h2 + q);
    }

    __device__ GItem none() const
    {
        GItem it;
        it.row = a.rows;
        it.nrec = 0;
        it.p0 = 0;
        it.nval = 0;
        it.rg0 = 0;
        it.absent = 0;
        return it;
    }

    // Item number `it` (slot search starts at `hint`, which is advanced).
    __device__ GItem item(int it, int end, int &hint) const
    {
        if (it >= end) return none();
        int s = hint;
        while (s + 1 < nact && L.tb.first[s + 1] <= it) ++s;
        s = uni(s);
        hint = s;
        const int local = uni(it - L.tb.first[s]);
        const int mb = local / NBLK, nb = local - mb * NBLK;
        const int n = uni(L.tb.n[s]);
        const int sl = uni(L.tb.sl[s]);
        GItem g;
        g.p0 = uni(L.tb.p0[s]) + kBM * mb;
        g.nval = min(kBM, n - kBM * mb);
        g.rg0 = nb * RGB;
        g.absent = sl < 0;
        g.row = a.rows + (sl >= 0 ? (size_t)sl * a.stride : 0);
        g.nrec = sl >= 0 ? a.row_bytes : 0;
        return g;
    }

    // Staging source of K-tile kt of the item (rows past its pairs, and the
    // padding tile kt == NT, read as zeros).
    __device__ __amdgpu_buffer_rsrc_t src_rsrc(const GItem &it, int kt) const
    {
        const bool ok = it.nval > 0 && kt < NT;
        if (GATEUP) return rsrc(a.x, ok ? a.T * a.H * 2 : 0);
        return rsrc(a.h + (size_t)it.p0 * a.I, ok ? it.nval * a.I * 2 : 0);
    }

    // The routed pair behind grouped pair threadIdx % 128 of the item, as
    // loaded (gate/up only).  Every thread issues exactly one load (a buffer
    // load that reads nothing past the item's pairs), which the wait counts
    // rely on.
    __device__ uint32_t pair_of(const GItem &it) const
    {
        if constexpr (!GATEUP) return 0;
        const int r = threadIdx.x & (kBM - 1);
        return __builtin_amdgcn_raw_buffer_load_b32(rsrc(a.sorted_pairs + it.p0, it.nval * 4), (uint32_t)r * 4u, 0, 0);
    }

    // Row offset of that pair's activation row (kNone: none).
    __device__ uint32_t src_of(const GItem &it, uint32_t pair) const
    {
        const int r = threadIdx.x & (kBM - 1);
        if constexpr (GATEUP) {
            const int tok = (int)pair / a.k;
            return (r < it.nval && tok >= 0 && tok < a.T) ? (uint32_t)tok * (uint32_t)(a.H * 2) : kNone;
        } else {
            return r < it.nval ? (uint32_t)r * (uint32_t)(a.I * 2) : kNone;
        }
    }

    __device__ void put_src(int par, uint32_t o) const
    {
        if (threadIdx.x < kBM) L.src[par][threadIdx.x] = o;
    }

    // Byte offset in the expert row of tile t (0, 1) of this wavefront for
    // K-tile kt: the qpacked tile of row group rg0 + wave (gate/up: t = the
    // matrix) or rg0 + 2 wave + t (down); kNone for a K-tile or row group
    // that does not exist.
    __device__ uint32_t wtile_off(const GItem &it, int kt, int t) const
    {
        const int rg = it.rg0 + (GATEUP ? wave : 2 * wave + t);
        const int sec = GATEUP ? (t ? a.off_q[1] : a.off_q[0]) : a.off_q[2];
        return (kt < NT && rg < RG) ? (uint32_t)(sec + (rg * NT + kt) * 1024) : kNone;
    }

    // Byte offset of this lane's first 16-byte piece of the wavefront's
    // weights of K-tile kt (the second is 512 bytes on): tile j32 / 16 of its
    // two, piece 16 h2 + j32 % 16 (row j32 % 16, columns 32 h2 .. +31 of the
    // tile's first chunk; the second piece: of its second chunk); past the
    // row (zeros) when nothing is read.
    __device__ uint32_t wpiece_off(const GItem &it, int kt) const
    {
        return wtile_off(it, kt, j32 >> 4) + 16 * (16 * h2 + (j32 & 15));
    }

    // Byte offset, for lane l < 16, of 4 bytes of the wavefront's row scales
    // of scale block b: lanes 0-7 the 16 scales of its first tile's row group
    // (gate, or the first down row group), lanes 8-15 those of the second
    // (up, or the second down row group); kNone for other lanes and for a
    // row group that does not exist.
    __device__ uint32_t scale_off(const GItem &it, int b) const
    {
        const int t = (lane >> 3) & 1;
        const int rg = it.rg0 + (GATEUP ? wave : 2 * wave + t);
        const int sec = GATEUP ? (t ? a.off_s[1] : a.off_s[0]) : a.off_s[2];
        return (lane < 16 && rg < RG) ? (uint32_t)(sec + (rg * NBK + b) * 32 + 4 * (lane & 7)) : kNone;
    }
};

// f(std::integral_constant<int, I>) for I = B .. E-1, as straight-line code
// (the step index is a constant expression inside f).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// End of a K-tile: this wavefront's direct-to-LDS loads older than its
// newest N vector-memory operations are complete (N counted by the caller),
// its LDS operations too, then the block barrier.  Written as one asm
// statement so that no memory fence asks for every outstanding load.
template <int N>
__device__ inline void stage_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// SiLU(g) * u in FP32 with the hardware exponential and reciprocal (about
// 2 ulp of FP32, far below the FP16 rounding of the result).
__device__ inline float silu_mul(float g, float u)
{
    const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
    return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

template <bool GATEUP>
__global__ __launch_bounds__(kGThreads) void w4a16_gemm_kernel(FfnArgs a, const int32_t *__restrict__ active,
                                                               const int32_t *__restrict__ offsets,
                                                               const int32_t *__restrict__ slot_map,
                                                               const int32_t *__restrict__ n_active)
{
    using G = Gemm<GATEUP>;
    __shared__ GLds L;
    // the slot table's inputs first: their loads do not wait for n_active
    TableIn tin{};
    if (threadIdx.x < 64) tin = table_loads(a, active, offsets, slot_map);
    int nact = *n_active;
    if (nact > a.E) nact = a.E;
    if (nact <= 0) return;
    const G f(a, L, nact);
    if (threadIdx.x < 64) build_table(L.tb, a, tin, nact, kBM, f.NBLK);
    // Stages start as zeros: rows that no load fills then hold finite values.
    for (int i = threadIdx.x; i < kStages * kStageBytes / 16; i += kGThreads)
        reinterpret_cast<u32x4 *>(&L.xa[0][0])[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    // Items are numbered slot by slot (m-block major, row block minor).  The
    // block runs on die (XCD) blockIdx % 8; each die takes a contiguous
    // eighth of the items and its blocks interleave through it, so at any
    // time the compute units of a die work on neighbouring items of the same
    // expert and share its activations and weights in that die's L2.
    const long long N = L.tb.first[nact];
    const int NX = (gridDim.x % 8 == 0) ? 8 : 1;
    const int xcd = blockIdx.x % NX, W = gridDim.x / NX, w = blockIdx.x / NX;
    const int c0 = (int)(N * xcd / NX), c1 = (int)(N * (xcd + 1) / NX);
    if (c0 + w >= c1) return;
    const int nk = (c1 - c0 - w + W - 1) / W;        // items of this block: c0 + w + k W, k < nk
    auto item_no = [&](int k) { return k < nk ? c0 + w + k * W : c1; };

    const int NTP = f.NTP;
    int hint = 0;
    int ci = 0;                            // item of the current K-tile, counted from the block's first
    GItem cur = f.item(item_no(0), c1, hint);
    GItem nxt = f.item(item_no(1), c1, hint);
    f.put_src(0, f.src_of(cur, f.pair_of(cur)));
    f.put_src(1, f.src_of(nxt, f.pair_of(nxt)));
    uint32_t pend = 0;                     // pair_of the next item, loaded at the last item end
    bool pend_put = true;
    if (cur.absent && threadIdx.x == 0 && a.status) *a.status = MOE_ERR_ABSENT_EXPERT;

    f32x16 acc[kMT], P[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        acc[mt] = f32x16{};
        P[mt] = acc[mt];
    }
    // K-tile 2 pr + H of item `it` (row offsets in L.src[par]) loaded
    // straight into stage 2 q + H: one instruction per row quad g = wave +
    // 8 j fills the 1 KB granule run of rows 4g .. 4g+3, lane l taking row
    // 4g + l % 4, piece (l / 4) ^ (g % 4), which lands at stage_addr of that
    // row and piece.  A row that reads nothing has offset kNone, which stays
    // out of range with the column added (the lane stores zeros or nothing;
    // such rows only feed outputs that are never written).  With H = 1 also
    // the wavefront's row scales of scale block pr.  Four (H = 0) or five
    // vector-memory operations per wavefront.
    auto stage_half = [&](auto h_c, const GItem &it, int par, int pr, int q) {
        constexpr int H = decltype(h_c)::value;
        const int kt = 2 * pr + H;
        // the four row offsets first, so their LDS reads overlap
        uint32_t so[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) so[j] = L.src[par][4 * (f.wave + 8 * j) + (f.lane & 3)];
        const __amdgpu_buffer_rsrc_t r = f.src_rsrc(it, kt);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int g = f.wave + 8 * j;
            const uint32_t off = so[j] + kt * 256 + 16 * ((f.lane >> 2) ^ (g & 3));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)&L.xa[2 * q + H][1024 * g], 16,
                                                     off, 0, 0, 0);
        }
        if constexpr (H == 1) {
            const __amdgpu_buffer_rsrc_t rw = rsrc(it.row, it.nrec);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void *)&L.sc[q][f.wave][0], 4,
                                                     f.scale_off(it, pr), 0, 0, 0);
        }
    };
    // This lane's weights of K-tile kt of item `it`: two 16-byte loads into
    // registers (zeros past the row).
    struct WTile {
        u32x4 v[2];
    };
    auto wload = [&](const GItem &it, int kt) {
        const __amdgpu_buffer_rsrc_t rw = rsrc(it.row, it.nrec);
        const uint32_t o = f.wpiece_off(it, kt);
        WTile t;
        t.v[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, o, 0, 0));
        t.v[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, o + 512, 0, 0));
        return t;
    };

    WTile wA, wB;                          // weights of the pair's first and second K-tile
    __syncthreads();
    wA = wload(cur, 0);
    stage_half(std::integral_constant<int, 0>{}, cur, 0, 0, 0);
    stage_half(std::integral_constant<int, 1>{}, cur, 0, 0, 0);
    stage_barrier<0>();

    const int total = nk * NTP;
    const int NPR = NTP / 2;               // pairs (scale blocks) per item
    int pr = 0;                            // pair of the current item
    for (int g = 0; g < total; g += 2) {
        const int rq = (g >> 1) & 1;       // ring slot of this pair
        static_for<0, 2>([&](auto slot_c) {
            constexpr int SLOT = decltype(slot_c)::value;
            const int kt = 2 * pr + SLOT;
            // 32 steps (K-step s of 16 columns, m-tile mt), one MFMA each;
            // the operand reads from LDS run kPD steps ahead of their use.
            // K-step s uses word s % 4 of chunk s / 4: lanes h2 = 0 take
            // piece 8 (s / 4) + s % 4, lanes h2 = 1 the piece 4 further on.
            const uint8_t *xs = &L.xa[2 * rq + SLOT][0];
            // stage_addr(32 mt + j32, 8 (s / 4) + 4 h2 + s % 4) = aq[s % 4] + 8192 mt + 512 (s / 4)
            auto rd = [&](int st) {
                const int s = st >> 2, mt = st & 3;
                return *reinterpret_cast<const half8 *>(xs + f.aq[s & 3] + 8192 * mt + 512 * (s >> 2));
            };
            // The first operand reads go out before the loads below, so their
            // latency overlaps the address arithmetic of those loads.
            half8 xr[kPD + 1];
#pragma unroll
            for (int st = 0; st < kPD; ++st) xr[st] = rd(st);
            const WTile wq = SLOT == 0 ? wA : wB;
            // The vector-memory operations of a pair, in this order (the wait
            // before the pair's barrier counts on it): SLOT 0's two weight
            // loads and four staging loads, SLOT 1's five staging loads and
            // two weight loads.  Staged: this K-tile's counterpart in the
            // next pair (after an item's last pair: the next item's first),
            // into the other ring slot.  Weights: the next K-tile's (after an
            // item's last K-tile: the next item's first).
            {
                const bool anx = pr + 1 >= NPR;
                const GItem &ait = anx ? nxt : cur;
                const int apar = (ci + anx) & 1, apr = anx ? 0 : pr + 1;
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (SLOT == 0) {
                    wB = wload(cur, kt + 1);
                    __builtin_amdgcn_sched_barrier(0);
                    stage_half(std::integral_constant<int, 0>{}, ait, apar, apr, rq ^ 1);
                } else {
                    stage_half(std::integral_constant<int, 1>{}, ait, apar, apr, rq ^ 1);
                    __builtin_amdgcn_sched_barrier(0);
                    wA = wload(anx ? nxt : cur, anx ? 0 : kt + 1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            {
                half8 bq;
                // a padding K-tile's operand is exactly zero (its stage may hold stale codes)
                const bool real = kt < f.NT;
                const _Float16 zs = real ? (_Float16)(-8.0f / 1048576.0f) : (_Float16)0.0f;
                const half8 zp = {zs, zs, zs, zs, zs, zs, zs, zs};
                const uint32_t wmask = real ? 0xFFFFFFFFu : 0u;
                static_for<0, 32>([&](auto c) {
                    constexpr int st = decltype(c)::value;
                    constexpr int s = st >> 2, mt = st & 3;
                    constexpr bool pre = st + kPD < 32;
                    if constexpr (pre) xr[(st + kPD) % (kPD + 1)] = rd(st + kPD);
                    if constexpr (mt == 0) bq = codes_to_signed_natural(wq.v[s >> 2][s & 3] & wmask, zp);
                    const half8 xf = xr[st % (kPD + 1)];
                    // weights as the first operand: lane l of the result then
                    // holds pair l % 32 of the m-tile (see the epilogue)
                    if constexpr (SLOT == 0 && s == 0) {
                        P[mt] = mfma32(bq, xf, f32x16{});
                    } else {
                        P[mt] = mfma32(bq, xf, P[mt]);
                    }
                    // keep the schedule in step order: the read kPD steps
                    // ahead, this step's MFMA, a share of the other work
                    __builtin_amdgcn_sched_group_barrier(0x100, pre ? 1 : 0, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
                });
            }

            if (SLOT == 1) {
                // The scale block ends: acc += scale * P.  Register r of lane
                // l holds output row n = 8 (r / 4) + 4 h2 + r % 4 of the
                // wavefront's 32 (tile n / 16, row n % 16), pair l % 32 of the
                // m-tile; the scales of rows 8 q + 4 h2 .. +3 are 8 bytes at
                // 16 q + 8 h2 of the wavefront's scale stage.
                const uint8_t *sp = &L.sc[rq][f.wave][8 * f.h2];
                _Float16 scl[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x2 v = *reinterpret_cast<const u32x2 *>(sp + 16 * q);
                    scl[4 * q + 0] = __builtin_bit_cast(_Float16, (uint16_t)(v[0] & 0xFFFFu));
                    scl[4 * q + 1] = __builtin_bit_cast(_Float16, (uint16_t)(v[0] >> 16));
                    scl[4 * q + 2] = __builtin_bit_cast(_Float16, (uint16_t)(v[1] & 0xFFFFu));
                    scl[4 * q + 3] = __builtin_bit_cast(_Float16, (uint16_t)(v[1] >> 16));
                }
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mt][r] += (float)scl[r] * P[mt][r];
            }
            if (SLOT == 1 && kt == NTP - 1) {
                // Item done: write its outputs with buffer stores whose range
                // ends at the item's last pair (pairs past it are dropped).
                // Gate/up: rows n < 16 are gate rows, n + 16 the up rows of
                // the same outputs, so lane l holds g and u of outputs
                // 4 h2 + 0..3 and 8 + 4 h2 + 0..3 of its row group: two
                // 8-byte stores per m-tile.  Down: outputs 8 q + 4 h2 + 0..3
                // of the wavefront's 32 rows of H, four 16-byte stores.
                if constexpr (GATEUP) {
                    const int rg = cur.rg0 + f.wave;
                    {
                        const __amdgpu_buffer_rsrc_t ro = rsrc(a.h + (size_t)cur.p0 * a.I, cur.nval * a.I * 2);
#pragma unroll
                        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                            for (int q = 0; q < 2; ++q) {
                                uint32_t w[2];
#pragma unroll
                                for (int e = 0; e < 2; ++e) {
                                    const int r0 = 4 * q + 2 * e;
                                    const float h0 = silu_mul(acc[mt][r0] * kUnit, acc[mt][r0 + 8] * kUnit);
                                    const float h1 = silu_mul(acc[mt][r0 + 1] * kUnit, acc[mt][r0 + 9] * kUnit);
                                    w[e] = cur.absent ? 0u : (uint32_t)float_to_half_bits(h0) | ((uint32_t)float_to_half_bits(h1) << 16);
                                }
                                const uint32_t off = rg < f.RG ? (uint32_t)(((32 * mt + f.j32) * a.I + rg * 16 + 8 * q + 4 * f.h2) * 2) : kNone;
                                __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, ro, off, 0, 0);
                            }
                    }
                } else {
                    const int rg = cur.rg0 + 2 * f.wave;
                    {
                        const __amdgpu_buffer_rsrc_t ro = rsrc(a.out + (size_t)cur.p0 * a.H, cur.nval * a.H * 4);
#pragma unroll
                        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                f32x4 v;
#pragma unroll
                                for (int e = 0; e < 4; ++e) v[e] = cur.absent ? 0.0f : acc[mt][4 * q + e] * kUnit;
                                const uint32_t off = rg < f.RG ? (uint32_t)(((32 * mt + f.j32) * a.H + rg * 16 + 8 * q + 4 * f.h2) * 4) : kNone;
                                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro, off, 0, 0);
                            }
                    }
                }
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt) acc[mt] = f32x16{};
                ++ci;
                cur = nxt;
                nxt = f.item(item_no(ci + 1), c1, hint);
                // The next item's row offsets: loaded now, written to LDS at
                // the end of its first pair (the first direct loads that read
                // them come with this item's last pair; with one pair per
                // item, at once).
                pend = f.pair_of(nxt);
                pend_put = NPR == 1;
                if (pend_put) f.put_src((ci + 1) & 1, f.src_of(nxt, pend));
                if (cur.absent && threadIdx.x == 0 && a.status) *a.status = MOE_ERR_ABSENT_EXPERT;
                pr = 0;
                // Issued after the staging loads of the pair read next: SLOT
                // 1's two weight loads, the output stores (gate/up 8, down 16)
                // and the offset load.
                stage_barrier<GATEUP ? 2 + 8 + 1 : 2 + 16>();
            } else if (SLOT == 1) {
                if (!pend_put) {
                    f.put_src((ci + 1) & 1, f.src_of(nxt, pend));
                    pend_put = true;
                }
                ++pr;
                // Issued after the staging loads of the pair read next: SLOT
                // 1's two weight loads.
                stage_barrier<2>();
            }
        });
    }
}

template <bool GATEUP>
int launch_gemm(const FfnArgs &a, hipStream_t s, const char *who)
{
    const int RGB = Gemm<GATEUP>::RGB;
    const int RG = (GATEUP ? a.I : a.H) / 16;
    const long long nblk = (RG + RGB - 1) / RGB;
    const long long pairs = (long long)a.T * a.k;
    const long long max_slots = pairs < a.E ? pairs : a.E;
    const long long max_items = (max_slots + pairs / kBM) * nblk;
    auto kern = w4a16_gemm_kernel<GATEUP>;
    static int occ_cache[64];
    const int occ = moe::blocks_per_cu(kern, kGThreads, occ_cache);
    long long g = (long long)cu_count() * occ;
    if (g > max_items) g = max_items;
    if (g < 1) g = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned int)g), dim3(kGThreads), 0, s, a, a.active, a.offsets, a.slot_map,
                       a.n_active);
    return moe::check_launch(who);
}

}  // namespace

int ffn::launch_gemm_gateup(const FfnArgs &a, hipStream_t s) { return launch_gemm<true>(a, s, "moe_w4a16_gateup"); }

int ffn::launch_gemm_down(const FfnArgs &a, hipStream_t s) { return launch_gemm<false>(a, s, "moe_w4a16_down"); }
