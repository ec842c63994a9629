// Pieces shared by the two W4A16 expert FFN kernels (the streaming kernel of
// expert_ffn.hip for small batches, the grouped GEMM of expert_gemm.hip for
// large ones): launch arguments, buffer resources, the INT4 -> FP16 operand
// conversion and the per-block table of active experts.  Not part of the C ABI.
#pragma once

#include "moe_internal.h"

namespace ffn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;            // raw buffer, 32-bit data format (gfx9 family)
constexpr float kUnit = 1048576.0f;               // 2^20: a code c enters the MFMA as c * 2^-20
constexpr float kZeroPoint = -8.0f / 1048576.0f;  // -8 * 2^-20
constexpr uint32_t kNib = 0x00F000F0u;            // bits 4-7 of each half

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
    int row_bytes;
    int off_q[3], off_s[3];     // gate, up, down sections of a row
};

__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ inline u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *base, int nbytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, nbytes, kRsrcWord3);
}

__device__ inline f32x4 mfma(half8 a, half8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline uint16_t float_to_half_bits(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

__device__ inline float half_bits_to_float(uint32_t b)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(b & 0xFFFFu));
}

// FP16 scale -> float, converted at this point of the program so the
// register that held it can be reloaded at once (left to itself the compiler
// folds the conversion into a later mixed-precision FMA, which keeps the old
// value alive past the reload and costs a copy and an early wait).
__device__ inline float scale_f32(_Float16 h)
{
    float f;
    asm volatile("v_cvt_f32_f16 %0, %1" : "=v"(f) : "v"(h));
    return f;
}

// Barrier that orders LDS only: prefetched global loads stay in flight across it
// (__syncthreads() would also wait for every outstanding global load).
__device__ inline void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Two FP16 values from the low (lo) or high (hi) halves of two dwords.
__device__ inline uint32_t lo2(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ inline uint32_t hi2(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// One MFMA B operand from a word of 8 codes (column 2i in the low nibble of
// byte i): each nibble moved to bits 4-7 of an FP16 half is the subnormal
// code * 2^-20.  Halves come out as columns (1, 5), (0, 4), (3, 7), (2, 6).
__device__ inline half8 codes_to_operand(uint32_t w)
{
    return __builtin_bit_cast(half8, u32x4{w & kNib, (w << 4) & kNib, (w >> 8) & kNib, (w >> 4) & kNib});
}

// Eight FP16 activations (columns 0..7 in natural order) rearranged to the
// column order of codes_to_operand.
__device__ inline u32x4 permute_activations(u32x4 d)
{
    return u32x4{hi2(d[0], d[2]), lo2(d[0], d[2]), hi2(d[1], d[3]), lo2(d[1], d[3])};
}

// One MFMA operand from a word of 8 codes (column 2i in the low nibble of
// byte i) with the columns in natural order: half j is code j moved to bits
// 4-7, the FP16 subnormal code * 2^-20, plus the zero point zp (-8 * 2^-20,
// which makes (code - 8) * 2^-20 exactly; 0 for a padding K-tile, whose
// operand is then exactly zero).  Byte j of lo holds code 2j in its high
// nibble, byte j of hi code 2j + 1; one byte permute per dword places them.
__device__ inline half8 codes_to_signed_natural(uint32_t w, half8 zp)
{
    const uint32_t lo = (w << 4) & 0xF0F0F0F0u, hi = w & 0xF0F0F0F0u;
    const u32x4 d = {__builtin_amdgcn_perm(hi, lo, 0x0C040C00u), __builtin_amdgcn_perm(hi, lo, 0x0C050C01u),
                     __builtin_amdgcn_perm(hi, lo, 0x0C060C02u), __builtin_amdgcn_perm(hi, lo, 0x0C070C03u)};
    return __builtin_bit_cast(half8, d) + zp;
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

// What the slot table needs, loaded by wave 0 in one round trip: lane l
// holds active[l] and, by expert index l, offsets[l], offsets[l + 1] and the
// device slot of expert l (so no load waits for another).
struct TableIn {
    int e, o0, o1, sl;
};

__device__ inline TableIn table_loads(const FfnArgs &a, const int32_t *__restrict__ active,
                                      const int32_t *__restrict__ offsets, const int32_t *__restrict__ slot_map)
{
    const int lane = threadIdx.x;          // wave 0 only
    TableIn t;
    const bool in = lane < a.E;
    t.e = in ? active[lane] : -1;
    t.o0 = in ? offsets[lane] : 0;
    t.o1 = in ? offsets[lane + 1] : 0;
    t.sl = in ? (slot_map ? slot_map[lane] : lane) : -1;
    return t;
}

// Built by wave 0, one lane per slot (lane s takes expert active[s] and its
// per-expert values from lane active[s]); a slot of n pairs has
// ceil(n / tile) * items_per_tile work items.  Routing metadata outside its
// valid range (a workspace that was not zero-filled, say) marks the status
// word and the slot gets no work.
__device__ inline void build_table(SlotTable &tb, const FfnArgs &a, const TableIn &in, int nact, int tile,
                                   int items_per_tile)
{
    const int lane = threadIdx.x;          // wave 0 only
    int e = lane < nact ? in.e : -1;
    const bool eok = e >= 0 && e < a.E;
    const int src = eok ? e : 0;
    const int q0 = __shfl(in.o0, src), q1 = __shfl(in.o1, src), sle = __shfl(in.sl, src);
    int p0 = 0, n = 0, sl = -1;
    if (eok) {
        if (q0 >= 0 && q1 >= q0 && (long long)q1 <= (long long)a.T * a.k) {
            p0 = q0;
            n = q1 - q0;
            sl = sle;
        } else {
            if (a.status) *a.status = MOE_ERR_INVALID_ARG;
            e = -1;
        }
    } else {
        e = -1;
    }
    const int cnt = (e >= 0) ? ((n + tile - 1) / tile) * items_per_tile : 0;
    const int incl = moe::wave_inclusive_sum(cnt);
    if (lane < MOE_MAX_EXPERTS) {
        tb.e[lane] = e;
        tb.p0[lane] = p0;
        tb.n[lane] = n;
        tb.sl[lane] = sl;
        tb.first[lane + 1] = incl;
    }
    if (lane == 0) tb.first[0] = 0;
}

// Compute units of the current device (cached per device).
int cu_count();

// Split of the reduction axis the streaming launches choose for a batch
// (expert_ffn.hip), and the argument checks and set-up of those launches
// (returns -1 for T = 0: nothing to do).
int stream_split(bool gateup, int T, int H, int I, int E, int k);
int make_ffn_args(FfnArgs &a, const void *x_dev, int T, int H, int I, int E, int k, const void *rows_dev,
                  size_t row_stride, const int32_t *slot_map_dev, const int32_t *expert_offsets_dev,
                  const int32_t *sorted_pairs_dev, const int32_t *active_list_dev, const int32_t *n_active_dev,
                  void *h_dev, float *pair_out_dev, int32_t *status_dev, const char *who);

// Grouped-GEMM launches for large batches (expert_gemm.hip).
int launch_gemm_gateup(const FfnArgs &a, hipStream_t s);
int launch_gemm_down(const FfnArgs &a, hipStream_t s);

// The K-split FFN of batches of at most 16 tokens (ffn_ksplit.hip): slice
// width W (0: not applicable to the shape), and the launch writing h and the
// I/W planes of partial pair outputs [I/W][T*k][H] (FP32).
int ksplit_width(int T, int H, int I, int E, int k);
int launch_ksplit(const FfnArgs &a, float *planes, int W, hipStream_t s, const char *who);

}  // namespace ffn
