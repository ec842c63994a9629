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
//   * Work item = 128 grouped pairs of one expert x one block of output rows
//     (gate/up: 128 rows of I for both matrices; down: 256 rows of H).  A
//     block of 8 wavefronts takes one item; wavefront (wm, wn) owns 64 pairs
//     (4 MFMA m-tiles) x 4 n-tiles of 16 rows (gate/up: 2 row groups x
//     {gate, up}, so SiLU(g) * u happens in registers; down: 4 row groups).
//   * Activations: each K-tile (128 columns) of the item's 128 pairs is
//     staged once in LDS (coalesced 16-byte loads, 16 lanes per pair row,
//     rows gathered through sorted_pairs for gate/up), already permuted to the
//     column order of the INT4 conversion; a ring of 3 K-tiles, staged two
//     K-tiles ahead, so one barrier per K-tile suffices.  The per-pair sums of
//     each 256-column scale block (for the zero point) are reduced across the
//     16 lanes of a row while staging.
//   * Weights: every wavefront loads its own 4 qpacked tiles per K-tile
//     (one 16-byte buffer load per lane each) two K-tiles ahead, converts each
//     8-code word into one MFMA operand (7 VALU) and feeds it to 4 MFMAs.
//   * Per scale block: P = -8 * 2^-20 * sum(x) enters as the initial
//     accumulator, the 8 K-steps of the block accumulate code * 2^-20 * x on
//     the matrix cores, and acc += scale * P in FP32 (weights never rounded
//     after scaling); the result is acc * 2^20.
//   * An odd number of K-tiles is padded with one K-tile that reads nothing
//     and computes nothing, so every scale block has two ring slots.
#include "ffn_common.h"

namespace {

using namespace ffn;

constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kBM = 128;              // grouped pairs per item
constexpr int kRowH = 136;            // halves per staged LDS row: 128 + 8 of padding (conflict-free reads)
constexpr int kStages = 3;            // staged K-tiles
constexpr int kMT = 4;                // m-tiles (16 pairs) per wavefront
constexpr int kNTL = 4;               // n-tiles (16 rows of one matrix) per wavefront
// Buffer offset of a row that reads nothing: past every staging resource
// (at most 256 MiB) and positive as a signed 32-bit value, so the range check
// of the buffer load turns it into zeros.  Used as the whole offset, never
// added to.
constexpr uint32_t kNone = 0x40000000u;

struct GLds {
    uint16_t xa[kStages][kBM * kRowH];   // staged activations [stage][pair][column]
    float sx[kStages][kBM];              // -8 * 2^-20 * (sum of a pair's activations over a scale block)
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

template <bool GATEUP>
struct Gemm {
    static constexpr int NMAT = GATEUP ? 2 : 1;
    static constexpr int RGW = kNTL / NMAT;      // row groups per wavefront
    static constexpr int RGB = 4 * RGW;          // row groups per item

    const FfnArgs &a;
    GLds &L;
    int nact;
    int lane, wave, g4, n16, wm, wn, sc, sr0;
    int K, NT, NTP, NBK, RG, NBLK;

    __device__ Gemm(const FfnArgs &args, GLds &lds, int nact_) : a(args), L(lds), nact(nact_)
    {
        const int tid = threadIdx.x;
        lane = tid & 63;
        wave = uni(tid >> 6);
        g4 = lane >> 4;
        n16 = lane & 15;
        wm = wave >> 2;
        wn = wave & 3;
        sc = tid & 15;           // staging: 16-byte column chunk of a K-tile
        sr0 = tid >> 4;          // staging: rows sr0 + 32 j
        K = GATEUP ? a.H : a.I;
        NT = K / 128;
        NTP = NT + (NT & 1);
        NBK = (NT + 1) / 2;
        RG = (GATEUP ? a.I : a.H) / 16;
        NBLK = (RG + RGB - 1) / RGB;
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

    // Staging source of the item (rows past its pairs read as zeros).
    __device__ __amdgpu_buffer_rsrc_t src_rsrc(const GItem &it) const
    {
        if (GATEUP) return rsrc(a.x, it.nval ? a.T * a.H * 2 : 0);
        return rsrc(a.h + (size_t)it.p0 * a.I, it.nval * a.I * 2);
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

    // Weight tile (K-tile kt) of n-tile nt; zeros when the tile does not exist.
    __device__ u32x4 load_q(const GItem &it, int nt, int kt) const
    {
        const int rg = it.rg0 + wn * RGW + nt / NMAT;
        const int mat = GATEUP ? nt % NMAT : 2;
        const bool ok = kt < NT && rg < RG;
        return __builtin_amdgcn_raw_buffer_load_b128(rsrc(it.row, ok ? it.nrec : 0), lane * 16,
                                                     a.off_q[mat] + (rg * NT + kt) * 1024, 0);
    }

    // FP16 scale of scale block b, row n16 of n-tile nt.
    __device__ _Float16 load_s(const GItem &it, int nt, int b) const
    {
        const int rg = it.rg0 + wn * RGW + nt / NMAT;
        const int mat = GATEUP ? nt % NMAT : 2;
        const bool ok = rg < RG;
        const uint16_t v = __builtin_amdgcn_raw_buffer_load_b16(rsrc(it.row, ok ? it.nrec : 0), n16 * 2,
                                                                a.off_s[mat] + (rg * NBK + b) * 32, 0);
        return __builtin_bit_cast(_Float16, v);
    }
};

typedef _Float16 half2 __attribute__((ext_vector_type(2)));

// Two FP16 values of a dword.  A value parameter on purpose: bit-casting a
// vector subscript inline (d[j][i]) has been compiled as a cast of element 0.
__device__ inline half2 as_half2(uint32_t w) { return __builtin_bit_cast(half2, w); }

template <int N>
__device__ inline float add_row_ror(float v)
{
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + N, 0xf,
                                                                     0xf, false));
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
    const long long N = L.tb.first[nact];
    const int it0 = (int)(N * blockIdx.x / gridDim.x), it1 = (int)(N * (blockIdx.x + 1) / gridDim.x);
    if (it0 >= it1) return;

    const int NT = f.NT, NTP = f.NTP;
    int hint = 0;
    int ci = 0;                            // item of the current K-tile, counted from it0
    GItem cur = f.item(it0, it1, hint);
    GItem nxt = f.item(it0 + 1, it1, hint);
    f.write_src(cur, 0);
    f.write_src(nxt, 1);
    if (cur.absent && threadIdx.x == 0 && a.status) *a.status = MOE_ERR_ABSENT_EXPERT;

    f32x4 acc[kMT][kNTL], P[kMT][kNTL];
    u32x4 wq[2][kNTL];
    _Float16 ws[kNTL];
    float part[4];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < kNTL; ++nt) {
            acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            P[mt][nt] = acc[mt][nt];
        }
#pragma unroll
    for (int nt = 0; nt < kNTL; ++nt) {
        wq[0][nt] = f.load_q(cur, nt, 0);
        wq[1][nt] = f.load_q(cur, nt, 1);
        ws[nt] = f.load_s(cur, nt, 0);
    }

    // Global loads of K-tile kt of item `it` (row offsets in L.src[par]).
    auto fetch = [&](const GItem &it, int par, int kt, u32x4 (&d)[4]) {
        const __amdgpu_buffer_rsrc_t r = f.src_rsrc(it);
        const uint32_t col = kt * 256 + 16 * f.sc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t o = L.src[par][f.sr0 + 32 * j];
            d[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (o == kNone || kt >= NT) ? kNone : o + col, 0, 0);
        }
    };
    // Staged K-tile into stage `st`; a scale block ends (pair sums written to
    // sx[sb]) when `last`.
    auto stage = [&](int st, bool first, bool last, int sb, const u32x4 (&d)[4]) {
        uint16_t *dst = &L.xa[st][0];
        const half2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = f.sr0 + 32 * j;
            *reinterpret_cast<u32x4 *>(dst + r * kRowH + 8 * f.sc) = permute_activations(d[j]);
            float s = first ? 0.f : part[j];
#pragma unroll
            for (int i = 0; i < 4; ++i) s = __builtin_amdgcn_fdot2(as_half2(d[j][i]), ones, s, false);
            part[j] = s;
        }
        if (last) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float t = part[j];
                t = add_row_ror<8>(t);
                t = add_row_ror<4>(t);
                t = add_row_ror<2>(t);
                t = add_row_ror<1>(t);
                if (f.sc == 0) L.sx[sb][f.sr0 + 32 * j] = t * kZeroPoint;
            }
        }
    };

    __syncthreads();
    {
        u32x4 d[4];
        fetch(cur, 0, 0, d);
        stage(0, true, false, 0, d);
        fetch(cur, 0, 1, d);
        stage(1, false, true, 0, d);
    }
    lds_barrier();

    const int total = (it1 - it0) * NTP;
    int kt = 0;
    for (int g = 0; g < total; g += 2) {
#pragma unroll
        for (int SLOT = 0; SLOT < 2; ++SLOT) {
            const int gg = g + SLOT;
            // K-tile two ahead: staged and its weights loaded during this one
            const bool anx = kt + 2 >= NTP;
            const int akt = anx ? kt + 2 - NTP : kt + 2;
            const GItem &ait = anx ? nxt : cur;
            u32x4 d[4];
            fetch(ait, (ci + anx) & 1, akt, d);
            if (kt < NT) {
                const uint16_t *xs = &L.xa[gg % kStages][(f.wm * 64 + f.n16) * kRowH + 32 * f.g4];
                const float *zs = &L.sx[(gg / 2) % kStages][f.wm * 64 + 4 * f.g4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    half8 xf[kMT];
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt)
                        xf[mt] = *reinterpret_cast<const half8 *>(xs + mt * 16 * kRowH + 8 * q);
#pragma unroll
                    for (int nt = 0; nt < kNTL; ++nt) {
                        const half8 b = codes_to_operand(wq[SLOT][nt][q]);
#pragma unroll
                        for (int mt = 0; mt < kMT; ++mt) {
                            if (SLOT == 0 && q == 0)
                                P[mt][nt] = mfma(xf[mt], b, *reinterpret_cast<const f32x4 *>(zs + mt * 16));
                            else
                                P[mt][nt] = mfma(xf[mt], b, P[mt][nt]);
                        }
                    }
                }
            }
#pragma unroll
            for (int nt = 0; nt < kNTL; ++nt) wq[SLOT][nt] = f.load_q(ait, nt, akt);
            if (SLOT == 1) {
#pragma unroll
                for (int nt = 0; nt < kNTL; ++nt) {
                    const float sc = scale_f32(ws[nt]);
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[mt][nt][r] += sc * P[mt][nt][r];
                }
#pragma unroll
                for (int nt = 0; nt < kNTL; ++nt) ws[nt] = f.load_s(ait, nt, akt / 2);
            }
            stage((gg + 2) % kStages, SLOT == 0, SLOT == 1, ((gg + 2) / 2) % kStages, d);

            if (SLOT == 1 && kt == NTP - 1) {
                // item done: write its outputs
                const int RG = f.RG;
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                    for (int rw = 0; rw < G::RGW; ++rw) {
                        const int rg = cur.rg0 + f.wn * G::RGW + rw;
                        const int col = rg * 16 + f.n16;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int lp = f.wm * 64 + mt * 16 + 4 * f.g4 + r;
                            if (rg < RG && lp < cur.nval) {
                                const size_t pr = (size_t)(cur.p0 + lp);
                                if constexpr (GATEUP) {
                                    const float gv = acc[mt][2 * rw][r] * kUnit, uv = acc[mt][2 * rw + 1][r] * kUnit;
                                    a.h[pr * a.I + col] =
                                        cur.absent ? (uint16_t)0 : float_to_half_bits(gv / (1.0f + expf(-gv)) * uv);
                                } else {
                                    a.out[pr * a.H + col] = cur.absent ? 0.0f : acc[mt][rw][r] * kUnit;
                                }
                            }
                        }
                    }
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < kNTL; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                ++ci;
                cur = nxt;
                nxt = f.item(it0 + ci + 1, it1, hint);
                f.write_src(nxt, (ci + 1) & 1);
                if (cur.absent && threadIdx.x == 0 && a.status) *a.status = MOE_ERR_ABSENT_EXPERT;
                kt = 0;
            } else {
                ++kt;
            }
            lds_barrier();
        }
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
