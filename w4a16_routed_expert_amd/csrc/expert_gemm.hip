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
// LDS byte:
//   * v_mfma_f32_32x32x16_f16: on the MI355X it sustains about 2 PFLOP/s,
//     the 16x16x32 form about 1.1 (measured with register-only chains).
//   * Work item = 128 grouped pairs of one expert x one block of output rows
//     (gate/up: 128 rows of I for both matrices; down: 256 rows of H).  A
//     block of 8 wavefronts takes one item; every wavefront owns all 128
//     pairs (4 m-tiles of 32) x one 32-column n-tile: for gate/up 16 rows of
//     the gate matrix and the same 16 rows of the up matrix (lane l and lane
//     l ^ 16 then hold g and u of one output, so SiLU(g) * u needs one lane
//     swap), for down 32 rows of H.  Each converted weight operand feeds 4
//     MFMAs.
//   * Activations: each K-tile (128 columns) of the item's 128 pairs is
//     staged once in LDS (each wavefront instruction loads 4 whole pair rows
//     of 256 bytes, rows gathered through sorted_pairs for gate/up), already
//     permuted to the column order of the INT4 conversion; a ring of 3
//     K-tiles, staged two K-tiles ahead, so one barrier per K-tile suffices.
//     LDS layout: 64-byte granules, granule (row / 4, piece ^ (row / 4 % 4))
//     holds the 16-byte piece of 4 consecutive rows, so the MFMA operand
//     reads (32 rows x 2 pieces per instruction) and the staging writes are
//     both free of bank conflicts.  The operand reads run several MFMAs ahead
//     of their use.
//   * Weights: per K-tile every lane loads two 16-byte chunks of qpacked
//     tiles (two K-tiles ahead), chosen so that word w of a lane is the
//     B operand of one MFMA: lanes 0-31 take columns 8w.., lanes 32-63 the
//     columns 32 further on, and the activation operand reads the same
//     columns.  Each 8-code word becomes one operand (7 VALU + 4 packed adds).
//   * Zero point in the operand: the converted subnormal code * 2^-20 minus
//     8 * 2^-20 (one packed FP16 add per dword) is (code - 8) * 2^-20 exactly,
//     so no activation sums are needed.  Per scale block the 8 K-steps
//     accumulate P = sum x * (code - 8) * 2^-20 on the matrix cores, then
//     acc += scale * P in FP32 (weights never rounded after scaling); the
//     result is acc * 2^20.
//   * An odd number of K-tiles is padded with one K-tile that reads nothing
//     and computes nothing, so every scale block has two ring slots.
#include "ffn_common.h"

#include <type_traits>

namespace {

using namespace ffn;

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kBM = 128;              // grouped pairs per item
constexpr int kStageBytes = kBM * 256;  // one staged K-tile
constexpr int kStages = 3;            // staged K-tiles
constexpr int kMT = 4;                // m-tiles (32 pairs) per wavefront: all 128 pairs of the item
constexpr int kPD = 4;                // operand reads in flight ahead of the MFMAs
// Buffer offset of a row (or lane) that reads nothing: past every resource
// used here (at most 256 MiB) and positive as a signed 32-bit value, so the
// range check of the buffer load turns it into zeros.
constexpr uint32_t kNone = 0x40000000u;

struct GLds {
    uint8_t xa[kStages][kStageBytes];    // staged activations (layout: see stage_addr)
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
    int lane, wave, j32, h2, sc, sr0;
    int K, NT, NTP, NBK, RG, NBLK;
    int lrg, lmat;                       // this lane's n-tile column: row group offset and matrix
    int qsec, ssec;                      // byte offsets of that matrix's codes and scales in a row
    int aq[4];                           // stage_addr of this lane's operand pieces, m-tile 0, K-steps q (+ 4n)

    __device__ Gemm(const FfnArgs &args, GLds &lds, int nact_) : a(args), L(lds), nact(nact_)
    {
        const int tid = threadIdx.x;
        lane = tid & 63;
        wave = uni(tid >> 6);
        j32 = lane & 31;                 // MFMA column (output row) of the lane
        h2 = lane >> 5;                  // which 8 of the 16 K values the lane feeds
        sc = lane >> 2;                  // staging: 16-byte piece of a K-tile row
        sr0 = 4 * wave + (lane & 3);     // staging: rows sr0 + 32 j (4 whole rows per instruction)
        K = GATEUP ? a.H : a.I;
        NT = K / 128;
        NTP = NT + (NT & 1);
        NBK = (NT + 1) / 2;
        RG = (GATEUP ? a.I : a.H) / 16;
        NBLK = (RG + RGB - 1) / RGB;
        lrg = GATEUP ? wave : 2 * wave + (j32 >> 4);
        lmat = GATEUP ? (j32 >> 4) : 2;
        // selected from uniform values: indexing the argument arrays with the
        // per-lane matrix would read them with vector loads
        qsec = GATEUP ? (lmat ? a.off_q[1] : a.off_q[0]) : a.off_q[2];
        ssec = GATEUP ? (lmat ? a.off_s[1] : a.off_s[0]) : a.off_s[2];
        for (int q = 0; q < 4; ++q) aq[q] = stage_addr_(j32, 4 * h2 + q);
    }

    // same as stage_addr below (needed here before its definition)
    static __device__ int stage_addr_(int r, int c) { return (((r >> 2) << 4) + (c ^ ((r >> 2) & 3))) * 64 + (r & 3) * 16; }

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

    // Row offsets of the item's pairs into L.src[par] (threads 0..127).
    __device__ void write_src(const GItem &it, int par) const
    {
        const int r = threadIdx.x;
        if (r >= kBM) return;
        uint32_t o = kNone;
        if (r < it.nval) {
            if (GATEUP) {
                const int tok = a.sorted_pairs[it.p0 + r] / a.k;
                if (tok >= 0 && tok < a.T) o = (uint32_t)tok * (uint32_t)(a.H * 2);
            } else {
                o = (uint32_t)r * (uint32_t)(a.I * 2);
            }
        }
        L.src[par][r] = o;
    }

    // Chunk `half` (0, 1) of this lane's weights for K-tile kt: 16 bytes of
    // row j32 % 16 of its row group, columns 32 (h2 + 2 half) .. +31 of the
    // K-tile; zeros for a K-tile or row group that does not exist.
    __device__ u32x4 load_q(const GItem &it, int kt, int half) const
    {
        const int rg = it.rg0 + lrg;
        const bool ok = kt < NT && rg < RG;
        const uint32_t off = ok ? (uint32_t)(qsec + (rg * NT + kt) * 1024 + (16 * (h2 + 2 * half) + (j32 & 15)) * 16)
                                : kNone;
        return __builtin_amdgcn_raw_buffer_load_b128(rsrc(it.row, it.nrec), off, 0, 0);
    }

    // FP16 scale of scale block b of this lane's output row.
    __device__ _Float16 load_s(const GItem &it, int b) const
    {
        const int rg = it.rg0 + lrg;
        const uint32_t off = rg < RG ? (uint32_t)(ssec + ((rg * NBK + b) * 16 + (j32 & 15)) * 2) : kNone;
        const uint16_t v = __builtin_amdgcn_raw_buffer_load_b16(rsrc(it.row, it.nrec), off, 0, 0);
        return __builtin_bit_cast(_Float16, v);
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

// Byte offset of 16-byte piece c (columns 8c .. 8c+7 of the K-tile) of
// staged row r: granule (r / 4) * 16 + (c ^ (r / 4 % 4)) of 64 bytes, slot r % 4.
__device__ inline int stage_addr(int r, int c) { return (((r >> 2) << 4) + (c ^ ((r >> 2) & 3))) * 64 + (r & 3) * 16; }

// permute_activations with one byte permute per dword.
__device__ inline u32x4 permute_pieces(u32x4 d)
{
    return u32x4{__builtin_amdgcn_perm(d[2], d[0], 0x07060302u), __builtin_amdgcn_perm(d[2], d[0], 0x05040100u),
                 __builtin_amdgcn_perm(d[3], d[1], 0x07060302u), __builtin_amdgcn_perm(d[3], d[1], 0x05040100u)};
}

// codes_to_operand minus 8 * 2^-20 in every half: (code - 8) * 2^-20, exact
// (FP16 subnormals are kept, and the difference is a multiple of 2^-24).
__device__ inline half8 codes_to_signed_operand(uint32_t w)
{
    const _Float16 m8 = (_Float16)(-8.0f / 1048576.0f);
    const half8 z = {m8, m8, m8, m8, m8, m8, m8, m8};
    return codes_to_operand(w) + z;
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
    int nact = *n_active;
    if (nact > a.E) nact = a.E;
    if (nact <= 0) return;
    const G f(a, L, nact);
    if (threadIdx.x < 64) build_table(L.tb, a, active, offsets, slot_map, nact, kBM, f.NBLK);
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
    f.write_src(cur, 0);
    f.write_src(nxt, 1);
    if (cur.absent && threadIdx.x == 0 && a.status) *a.status = MOE_ERR_ABSENT_EXPERT;

    f32x16 acc[kMT], P[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        acc[mt] = f32x16{};
        P[mt] = acc[mt];
    }
    u32x4 wq[2][2];                        // [ring slot][chunk]
    wq[0][0] = f.load_q(cur, 0, 0);
    wq[0][1] = f.load_q(cur, 0, 1);
    wq[1][0] = f.load_q(cur, 1, 0);
    wq[1][1] = f.load_q(cur, 1, 1);
    _Float16 ws = f.load_s(cur, 0);       // scale of the block being accumulated
    float wprev = 0.f;                     // scale of the block being merged

    // Global loads of K-tile kt of item `it` (row offsets in L.src[par]);
    // a row that reads nothing has offset kNone, which stays out of range
    // with the column added.
    auto fetch = [&](const GItem &it, int par, int kt, u32x4 (&d)[4]) {
        const __amdgpu_buffer_rsrc_t r = f.src_rsrc(it, kt);
        const uint32_t col = kt * 256 + 16 * f.sc;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            d[j] = __builtin_amdgcn_raw_buffer_load_b128(r, L.src[par][f.sr0 + 32 * j] + col, 0, 0);
    };
    // Staged K-tile into stage `st`.
    auto stage = [&](int st, const u32x4 (&d)[4]) {
        uint8_t *dst = &L.xa[st][0];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<u32x4 *>(dst + stage_addr(f.sr0 + 32 * j, f.sc)) = permute_pieces(d[j]);
    };

    __syncthreads();
    {
        u32x4 d[4];
        fetch(cur, 0, 0, d);
        stage(0, d);
        fetch(cur, 0, 1, d);
        stage(1, d);
    }
    lds_barrier();

    const int total = nk * NTP;
    int kt = 0;
    for (int g = 0; g < total; g += 2) {
        static_for<0, 2>([&](auto slot_c) {
            constexpr int SLOT = decltype(slot_c)::value;
            const int gg = g + SLOT;
            // K-tile two ahead: staged and its weights loaded during this one
            const bool anx = kt + 2 >= NTP;
            const int akt = anx ? kt + 2 - NTP : kt + 2;
            const GItem &ait = anx ? nxt : cur;
            const int sst = (gg + 2) % kStages;
            u32x4 d[4];
            fetch(ait, (ci + anx) & 1, akt, d);
            if (SLOT == 1) {
                // this block's scale for the merge at its end; the next block's loaded
                wprev = scale_f32(ws);
                ws = f.load_s(ait, akt / 2);
            }
            {
                // 32 steps (K-step s of 16 columns, m-tile mt), one MFMA each;
                // the operand reads from LDS run kPD steps ahead of their use.
                // K-step s uses word s % 4 of chunk s / 4: lanes h2 = 0 take
                // piece 8 (s / 4) + s % 4, lanes h2 = 1 the piece 4 further on.
                // Interleaved with the MFMAs: the reloads of the weight chunks
                // as soon as they are converted, and the staging writes.
                const uint8_t *xs = &L.xa[gg % kStages][0];
                // stage_addr(32 mt + j32, 8 (s / 4) + 4 h2 + s % 4) = aq[s % 4] + 8192 mt + 512 (s / 4)
                auto rd = [&](int st) {
                    const int s = st >> 2, mt = st & 3;
                    return *reinterpret_cast<const half8 *>(xs + f.aq[s & 3] + 8192 * mt + 512 * (s >> 2));
                };
                half8 xr[kPD + 1];
#pragma unroll
                for (int st = 0; st < kPD; ++st) xr[st] = rd(st);
                half8 bq;
                static_for<0, 32>([&](auto c) {
                    constexpr int st = decltype(c)::value;
                    constexpr int s = st >> 2, mt = st & 3;
                    constexpr bool pre = st + kPD < 32;
                    if constexpr (pre) xr[(st + kPD) % (kPD + 1)] = rd(st + kPD);
                    if constexpr (mt == 0) bq = codes_to_signed_operand(wq[SLOT][s >> 2][s & 3]);
                    if constexpr (st == 13) wq[SLOT][0] = f.load_q(ait, akt, 0);
                    if constexpr (st == 29) wq[SLOT][1] = f.load_q(ait, akt, 1);
                    const half8 xf = xr[st % (kPD + 1)];
                    if constexpr (SLOT == 0 && s == 0) {
                        P[mt] = mfma32(xf, bq, f32x16{});
                    } else {
                        P[mt] = mfma32(xf, bq, P[mt]);
                    }
                    if constexpr (st == 20) stage(sst, d);
                    // keep the schedule in step order: the read kPD steps
                    // ahead, this step's MFMA, a share of the other work
                    __builtin_amdgcn_sched_group_barrier(0x100, pre ? 1 : 0, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
                });
            }

            if (SLOT == 1) {
                // the scale block ends: acc += scale * P
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mt][r] += wprev * P[mt][r];
            }
            if (SLOT == 1 && kt == NTP - 1) {
                // item done: write its outputs.  Lane l holds column j32 for
                // rows 8 (r / 4) + 4 h2 + r % 4 of each 32-pair m-tile.
                const int rg = cur.rg0 + f.lrg;
                const bool rows_ok = rg < f.RG;
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int lp = 32 * mt + 8 * (r >> 2) + 4 * f.h2 + (r & 3);
                        const float v = acc[mt][r] * kUnit;
                        if constexpr (GATEUP) {
                            // lanes with j32 < 16 hold g, lanes j32 + 16 the u of the same row
                            const float u = __builtin_bit_cast(float, moe::partner_u32<true>(__builtin_bit_cast(uint32_t, v)));
                            if (f.j32 < 16 && rows_ok && lp < cur.nval) {
                                const size_t pr = (size_t)(cur.p0 + lp);
                                a.h[pr * a.I + rg * 16 + f.j32] = cur.absent ? (uint16_t)0 : float_to_half_bits(silu_mul(v, u));
                            }
                        } else {
                            if (rows_ok && lp < cur.nval) {
                                const size_t pr = (size_t)(cur.p0 + lp);
                                a.out[pr * a.H + rg * 16 + (f.j32 & 15)] = cur.absent ? 0.0f : v;
                            }
                        }
                    }
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt) acc[mt] = f32x16{};
                ++ci;
                cur = nxt;
                nxt = f.item(item_no(ci + 1), c1, hint);
                f.write_src(nxt, (ci + 1) & 1);
                if (cur.absent && threadIdx.x == 0 && a.status) *a.status = MOE_ERR_ABSENT_EXPERT;
                kt = 0;
            } else {
                ++kt;
            }
            lds_barrier();
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
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kGThreads, 0) != hipSuccess || occ <= 0) occ = 1;
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
