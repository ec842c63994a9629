/*
 * moe_w4a16.h -- C ABI of the W4A16 routed-expert MoE layer for one MI355X (gfx950).
 *
 * The layer (Horizon RunMap pages):
 *   - routed experts stored as INT4 "qpacked" weights, 256-value blocks with
 *     one FP16 scale each; FP16 activations; no persistent expanded FP16/BF16
 *     expert ("Horizon RunMap - architecture", table "Representation and
 *     computation"; "horizonrunmap.com/en", section "08 / Precision &
 *     quality": weights are converted inside the kernel as computation needs
 *     them, with FP32 accumulation stages and explicit rounding);
 *   - routing chooses the experts of each token at each routed layer
 *     ("horizonrunmap.com/en", section "06 / Follow a token", step "Select
 *     experts"); routing and other non-routed parts stay outside INT4, with
 *     FP16 weights (section "08", paragraph "Other components");
 *   - a resident expert is not necessarily routed, and a missing expert row
 *     is copied host-to-device only ("Horizon RunMap - architecture",
 *     sections "Immutable authority and miss lifecycle" and "Regimes and
 *     executor boundaries").
 * The pages give no formula for the router or the expert FFN.  This library
 * implements: top-k softmax routing over FP16 router logits, a SwiGLU expert
 * (gate, up, SiLU(gate) * up, down) and the weighted sum of the k expert
 * outputs.
 *
 * Conventions for every call
 *   - Pointers named *_dev are device pointers (hipMalloc'd or torch CUDA
 *     tensors); the caller owns them.  FP16 tensors are passed as void*.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Compute calls
 *     only enqueue kernels on it: they are asynchronous, never synchronize,
 *     and never allocate.
 *   - Return value: MOE_OK or an MOE_ERR_* code.  Arguments are validated on
 *     the host before anything is enqueued; on error nothing is enqueued and
 *     moe_last_error() returns a message (thread-local).
 *   - Shapes: E <= 64 experts, 1 <= k <= min(E, 8), H and I multiples of 128,
 *     T >= 0 (T = 0 enqueues nothing and returns MOE_OK).
 *
 * qpacked v1 weight layout of one matrix with R rows (output features) and K
 * columns (reduction index), R % 16 == 0, K % 128 == 0.  A weight is
 * (code - 8) * scale; the pages fix no zero point, so codes 0..15 stand for
 * -8..7.
 *   nibble plane (R*K/2 bytes): 1024-byte tiles.  Tile (rg, kt) holds rows
 *     16rg .. 16rg+15, columns 128kt .. 128kt+127, at byte
 *     (rg*(K/128) + kt)*1024.  Within a tile, the 16-byte chunk number
 *     16g + r holds row 16rg + r, columns 128kt + 32g .. 128kt + 32g + 31;
 *     byte i of the chunk holds column 2i in bits 0-3 and column 2i+1 in
 *     bits 4-7 (relative to the chunk's first column).
 *   scale plane (R*ceil(K/256) FP16): the scale of row 16rg + r for block b
 *     (columns 256b .. min(256b+256, K)-1; the last block of a row may hold
 *     only 128 columns) is element (rg*ceil(K/256) + b)*16 + r.
 * Expert row: the unit that lives in one device slot and is uploaded on a
 *   miss.  Sections, each starting on a 256-byte boundary, in this order:
 *   gate nibbles [I][H], up nibbles [I][H], down nibbles [H][I], gate
 *   scales, up scales, down scales.
 *
 * Pair numbering: token t's j-th selected expert (j = 0..k-1, descending
 * logit) is pair p = t*k + j.  Grouping sorts pairs by expert (stable: within
 * an expert, ascending p); pos = pair_pos[p] is a pair's place in that order
 * and sorted_pairs[pos] = p.
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,     /* null pointer, bad shape, misaligned pointer */
    MOE_ERR_UNSUPPORTED = 2,     /* shape outside the supported envelope */
    MOE_ERR_WORKSPACE = 3,       /* workspace missing or too small */
    MOE_ERR_CAPACITY = 4,        /* expert table: not enough spare rows / staging at create */
    MOE_ERR_HIP = 5,             /* a HIP runtime call or kernel launch failed */
    MOE_ERR_FAULTED = 6,         /* expert table faulted by a failure after publication */
    MOE_ERR_ABSENT_EXPERT = 7,   /* a routed expert has no published device row */
    MOE_ERR_SOURCE = 8,          /* expert table: host source failed its identity or layout check */
    MOE_ERR_TIMEOUT = 9,         /* one-launch layer: a wait between its blocks gave up (status word) */
};

#define MOE_MAX_EXPERTS 64
#define MOE_MAX_TOPK 8

/* Library version (major*10000 + minor*100 + patch). */
int moe_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char *moe_last_error(void);

/* Size in bytes of one qpacked v1 expert row for hidden size H and expert
 * intermediate size I (0 if H or I is not a positive multiple of 128).
 * off6, if not NULL, receives the byte offsets of the six sections
 * (gate_q, up_q, down_q, gate_s, up_s, down_s). */
size_t moe_expert_row_bytes(int H, int I, size_t *off6);

/* ------------------------------------------------------------ routing
 * moe_route: router logits, top-k softmax and token-to-expert grouping (two
 * kernel launches: for T <= 256 logits spread over many blocks, then one
 * block for top-k and the grouping; for larger T per-token logits and top-k,
 * then the grouping).
 *   logit[t][e] = RN32( exact sum_h x[t][h] * w_router[h][e] ) (+ bias[e])
 *     The correctly rounded FP32 value of the exact dot product of FP16
 *     values, so the selected experts do not depend on summation order.  The
 *     kernel sums the (exact) products in fp64 and recomputes a logit with
 *     integer arithmetic only when an error bound cannot exclude that the
 *     exact value rounds differently.  bias, if given, is added in FP32.
 *   topk_ids[t][j]: the k largest logits, descending, ties to the lower
 *     expert index.  topk_w[t][j] = softmax over those k logits (FP32; the
 *     weights of a token sum to 1).
 *   expert_offsets[E+1]: exclusive prefix sum of the per-expert pair counts.
 *   sorted_pairs[T*k], pair_pos[T*k]: the stable grouping described above.
 *   active_list[E]: experts with at least one pair, ascending; entries past
 *     *n_active_dev are set to -1.  n_active_dev[0]: their number.
 *   logits_dev: FP32 [T][E] copy of the logits (bias included), or NULL.
 * Inputs:  x_dev FP16 [T][H] row-major; w_router_dev FP16 [H][E] row-major;
 *          bias_dev FP32 [E] or NULL.
 * ws_dev / ws_bytes: workspace of moe_route_workspace_size(T, H, E) bytes,
 *   256-byte aligned, required; it holds what passes between the call's
 *   kernels (the logits for T <= 256, per-segment expert counts above) and
 *   needs no initialization.  One workspace must not be used by two calls
 *   that can overlap; a workspace sized for T serves any T' <= T.
 * Limits: T <= 65536, H <= 4096 (bounds the exact integer accumulators);
 *   x_dev 8-byte aligned. */
size_t moe_route_workspace_size(int T, int H, int E);
int moe_route(const void *x_dev, const void *w_router_dev, const float *bias_dev,
              int T, int H, int E, int k,
              float *logits_dev, int32_t *topk_ids_dev, float *topk_w_dev,
              int32_t *expert_offsets_dev, int32_t *sorted_pairs_dev, int32_t *pair_pos_dev,
              int32_t *active_list_dev, int32_t *n_active_dev,
              void *ws_dev, size_t ws_bytes, void *stream);

/* moe_route_exact: same outputs as moe_route, every logit computed with the
 * integer path (slow; for checking the fast path and for callers that want
 * no floating-point shortcut at all).  Results are bit-identical to
 * moe_route's. */
int moe_route_exact(const void *x_dev, const void *w_router_dev, const float *bias_dev,
                    int T, int H, int E, int k,
                    float *logits_dev, int32_t *topk_ids_dev, float *topk_w_dev,
                    int32_t *expert_offsets_dev, int32_t *sorted_pairs_dev, int32_t *pair_pos_dev,
                    int32_t *active_list_dev, int32_t *n_active_dev,
                    void *ws_dev, size_t ws_bytes, void *stream);

/* moe_route_static: moe_route without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The workspace is a fixed array of
 * moe_route_static_max_bytes() bytes (1 MiB) inside this library, one per
 * device, held until the process ends; the call itself allocates nothing.
 * Shapes whose workspace would exceed it (moe_route_workspace_size(T, H, E)
 * > the maximum, e.g. T > 4096 at E = 64) return MOE_ERR_WORKSPACE.  Every
 * call on a device shares that device's array: calls that can overlap on one
 * GPU (other streams, other threads) race and must not be issued.  Results
 * are bit-identical to moe_route's. */
size_t moe_route_static_max_bytes(void);
int moe_route_static(const void *x_dev, const void *w_router_dev, const float *bias_dev,
                     int T, int H, int E, int k,
                     float *logits_dev, int32_t *topk_ids_dev, float *topk_w_dev,
                     int32_t *expert_offsets_dev, int32_t *sorted_pairs_dev, int32_t *pair_pos_dev,
                     int32_t *active_list_dev, int32_t *n_active_dev, void *stream);

/* ------------------------------------------------------------ expert FFN
 * Expert rows are addressed as rows_dev + slot_map_dev[e] * row_stride
 * (slot_map_dev NULL means slot e for expert e).  row_stride >=
 * moe_expert_row_bytes(H, I) and a multiple of 256; rows_dev 256-byte
 * aligned.  A routed expert whose slot is negative is an absent expert: its
 * pairs get zero output and *status_dev (if not NULL) is set to
 * MOE_ERR_ABSENT_EXPERT (the library never clears it; the caller zeroes it).
 * expert_offsets / sorted_pairs / active_list / n_active are moe_route's
 * outputs for the same T, E, k.
 *
 * moe_w4a16_gateup: for every pair p = (t, j) routed to expert e, in grouped
 *   order pos = pair_pos[p]:
 *     g = Wg[e] x[t], u = Wu[e] x[t]            (FP32 accumulation)
 *     h[pos][i] = RN16( silu(g_i) * u_i ),  silu(g) = g / (1 + exp(-g))
 *   h_dev: FP16 [T*k][I] workspace (16-byte aligned).
 * moe_w4a16_down: pair_out[pos][r] = sum_i Wd[e][r][i] * h[pos][i] (FP32).
 *   pair_out_dev: FP32 [T*k][H].
 * moe_w4a16_expert_ffn: gateup then down on the same stream.
 * Weights are read as INT4 codes and converted to FP16 in registers; the
 * per-block FP16 scale is applied to the FP32 partial sum of each block, so
 * no expanded weight matrix is ever stored. */

/* mode: kernel family of the call (a per-call choice; it never changes the
 * result beyond FP32 summation order).  Both families compute the same sums
 * per scale block in FP32 and round at the same points.
 *   MOE_FFN_PATH_STREAM: one wavefront per 16 pairs x 16 rows of an expert,
 *     streaming each weight tile once per 16 pairs (built for decode batches,
 *     bound by HBM);
 *   MOE_FFN_PATH_GEMM: a grouped GEMM over 128-pair tiles of each expert
 *     (built for prefill batches, bound by the matrix cores);
 *   MOE_FFN_PATH_AUTO: the GEMM when T*k >= 64*E, else the streaming kernels.
 * Any other value returns MOE_ERR_INVALID_ARG. */
enum moe_ffn_path {
    MOE_FFN_PATH_AUTO = 0,
    MOE_FFN_PATH_STREAM = 1,
    MOE_FFN_PATH_GEMM = 2,
    MOE_FFN_PATH_KSPLIT = 3,
    MOE_FFN_PATH_ONE_LAUNCH = 4
};
/* MOE_FFN_PATH_KSPLIT and MOE_FFN_PATH_ONE_LAUNCH: moe_layer_forward only (the
 * FFN calls reject them); see there. */

int moe_w4a16_gateup(const void *x_dev, int T, int H, int I, int E, int k,
                     const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                     const int32_t *expert_offsets_dev, const int32_t *sorted_pairs_dev,
                     const int32_t *active_list_dev, const int32_t *n_active_dev,
                     void *h_dev, int32_t *status_dev, int mode, void *stream);
int moe_w4a16_down(int T, int H, int I, int E, int k,
                   const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                   const int32_t *expert_offsets_dev, const int32_t *active_list_dev,
                   const int32_t *n_active_dev, const void *h_dev, float *pair_out_dev,
                   int32_t *status_dev, int mode, void *stream);
int moe_w4a16_expert_ffn(const void *x_dev, int T, int H, int I, int E, int k,
                         const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                         const int32_t *expert_offsets_dev, const int32_t *sorted_pairs_dev,
                         const int32_t *active_list_dev, const int32_t *n_active_dev,
                         void *h_dev, float *pair_out_dev, int32_t *status_dev, int mode, void *stream);

/* ------------------------------------------------------------ whole layer
 * moe_layer_forward: route -> gate/up + SiLU*up -> down -> combine in one call,
 * with the results of moe_route, the FFN calls and moe_combine (the pages'
 * "top4-fused-v1" executor is prior art for fusing the layer: "Horizon
 * RunMap - architecture", section "Regimes and executor boundaries").
 * Decode batches (the streaming kernels: mode STREAM or KSPLIT, or AUTO with
 * T*k < 64*E, and T <= 256) route in one launch instead of two: the block
 * that finishes its logits last runs the top-k and the grouping (no block
 * waits for another).  Then
 *   - mode KSPLIT (T <= 16, H <= 2048 with H/128 even, I <= 2048; AUTO
 *     does not choose it: measured slower than the streaming kernels at
 *     every batch so far): ONE expert-FFN launch for gate/up and down.  Its work items are (active expert, slice of W columns of I);
 *     the block of an item keeps that slice of h in LDS and multiplies it
 *     with the same columns of the down matrix, writing partial pair outputs
 *     to I/W planes in the workspace; the combine adds each pair's planes in
 *     plane order (and writes that sum to pair_out).  Same operation and
 *     rounding points; only the FP32 summation order of the down projection
 *     differs from the streaming kernels.  Three launches in all.
 *   - mode ONE_LAUNCH (1 <= T <= 64, T*k < 64*E, E even, (H/128, I/128) in
 *     {(2, 4), (16, 8), (16, 11)}; AUTO does not choose it: measured slower
 *     than the four launches, OLMoE shape T = 1 29.4 against 26.7 us per
 *     step, T = 32 74.8 against 59.8 us): the routing AND the expert FFN AND the
 *     combine in ONE launch.  Its grid is exactly the blocks resident at once;
 *     blocks hand the routing results, h and the pair outputs to each other
 *     through device-scope counters in the workspace (published by the
 *     writer after its stores complete, polled by the reader).  y, h,
 *     pair_out and the routing results are bit-identical to the separate
 *     calls.  Every wait is bounded: a wait that gives up writes
 *     MOE_ERR_TIMEOUT to the status word (the call's outputs are then
 *     undefined) - which needs every block of the launch to be resident,
 *     so calls that can overlap on one GPU must not share it with other
 *     long-running kernels.  shared_ready_event is waited for before the
 *     launch (the shared expert then does not overlap the routed work);
 *   - otherwise the streaming gate/up and down launches and the combine (y
 *     then bit-identical to the separate calls).
 * Other batches run moe_route, moe_w4a16_expert_ffn and moe_combine in order.
 * Buffers (device, caller-owned, sized for T): the routing outputs and the
 * FFN intermediates of moe_route / moe_w4a16_expert_ffn (h and pair_out are
 * written on every path), plus
 *   ws / ws_bytes: moe_layer_workspace_size(T, H, I, E, k) bytes, 256-byte
 *     aligned, ZERO-FILLED BEFORE ITS FIRST USE; every call leaves its counter
 *     zero again (a workspace sized for T serves any T' <= T); not shared by
 *     calls that can overlap.
 * Workspace control words: the first moe_layer_workspace_size bytes hold,
 * at their start, the counters of the routing launch and of the one-launch
 * layer (1 KB); every call leaves them zero.
 * shared_out / shared_gate: the shared-expert terms (moe_shared_ffn) or both
 * NULL; shared_ready_event: a hipEvent_t recorded after the shared expert (on
 * another stream), waited for before the combine, or NULL when the shared
 * terms are already ordered before the call on `stream`.
 * mode: MOE_FFN_PATH_* as for the FFN calls. */
typedef struct {
    float *logits;                     /* FP32 [T][E] or NULL */
    int32_t *topk_ids;                 /* [T][k] */
    float *topk_w;                     /* [T][k] */
    int32_t *expert_offsets;           /* [E+1] */
    int32_t *sorted_pairs, *pair_pos;  /* [T*k] */
    int32_t *active_list;              /* [E] */
    int32_t *n_active;                 /* [1] */
    void *h;                           /* FP16 [T*k][I], 16-byte aligned */
    float *pair_out;                   /* FP32 [T*k][H], 16-byte aligned */
    int32_t *status;                   /* [1] or NULL, as for the FFN calls */
    void *ws;
    size_t ws_bytes;
} moe_layer_buffers;

size_t moe_layer_workspace_size(int T, int H, int I, int E, int k);
int moe_layer_forward(const void *x_dev, const void *w_router_dev, const float *bias_dev, int T, int H, int I,
                      int E, int k, const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                      const float *shared_out_dev, const float *shared_gate_dev, void *shared_ready_event,
                      void *y_dev, const moe_layer_buffers *buffers, int mode, void *stream);

/* moe_layer_forward_shared: the layer with its FP16 shared expert in one call
 * (moe_shared_ffn, then moe_layer_forward with the shared terms, and the same
 * results bit for bit).  For decode batches whose shared gate/up is one pass
 * of 8-row units over the whole reduction axis (T <= 16 at H = 2048) and that
 * take the streaming kernels (mode STREAM, or AUTO with T*k < 64*E; E even,
 * w_router 4-byte aligned), the routing launch also runs the shared expert's
 * gate/up pass and sigmoid gate as extra blocks (the routing is bound by
 * latency and leaves HBM idle; a second stream does not overlap the two on
 * this GPU because each launch's grid takes every CU), then the routed expert
 * FFN, the shared down projection and the combine follow on `stream`.  Other
 * batches and modes run moe_shared_ffn and moe_layer_forward in order.
 * Arguments: those of moe_layer_forward (without shared_ready_event) and of
 * moe_shared_ffn (shared weights in the tile8 layout, shared_out, shared_gate,
 * and its workspace of moe_shared_ffn_workspace_size(T, H, Is) bytes).
 * Errors: both calls' argument checks (shapes, nulls, alignment, both
 * workspaces, the mode) run before anything is launched; only a shape that
 * mode KSPLIT or ONE_LAUNCH does not take is reported after the shared expert
 * has run (by the moe_layer_forward it then calls). */
int moe_layer_forward_shared(const void *x_dev, const void *w_router_dev, const float *bias_dev, int T, int H, int I,
                             int E, int k, const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                             const void *w_sgate_proj_dev, const void *w_sup_dev, const void *w_sdown_dev,
                             const void *w_sgate_dev, int Is, float *shared_out_dev, float *shared_gate_dev,
                             void *shared_ws_dev, size_t shared_ws_bytes, void *y_dev,
                             const moe_layer_buffers *buffers, int mode, void *stream);

/* ------------------------------------------------------------ shared expert
 * moe_shared_ffn: the FP16 shared expert of a layer that has one (non-routed
 * weights stay FP16: "horizonrunmap.com/en", section "08 / Precision &
 * quality", paragraph "Other components"), with the rounding points of a
 * routed expert:
 *   g = Wsg x_t, u = Wsu x_t (FP32 sums of FP16 products),
 *   hs = RN16(silu(g) * u),  shared_out[t] = Wsd hs (FP32),
 *   shared_gate[t] = 1 / (1 + exp(-(w_sgate . x_t)))  (FP32).
 * The layer output then adds shared_gate[t] * shared_out[t] (moe_combine).
 * Inputs:  x_dev FP16 [T][H] row-major; w_gate_dev, w_up_dev FP16 [Is][H] and
 *          w_down_dev FP16 [H][Is] in the tile8 layout (moe_pack_fp16_tile8);
 *          w_sgate_dev FP16 [H]; all 16-byte aligned.  H and Is positive
 *          multiples of 128, each matrix under 2 GiB, 0 <= T <= 65536.
 * Outputs: shared_out_dev FP32 [T][H] (16-byte aligned), shared_gate_dev FP32 [T].
 * ws_dev / ws_bytes: workspace of moe_shared_ffn_workspace_size(T, H, Is)
 *   bytes (256-byte aligned) holding hs and, for shapes whose reduction axis
 *   is cut into chunks, the FP32 partial sums of the chunks; no
 *   initialization; not shared by overlapping calls.
 * Two to four kernel launches on `stream` (chunk sums are added in a fixed
 * order: results do not depend on scheduling); T = 0 enqueues nothing. */
size_t moe_shared_ffn_workspace_size(int T, int H, int Is);
/* tile8 layout of an FP16 matrix W [R][K] (R a multiple of 8, K of 128): tile
 * (r8, kt) = rows 8 r8 .. 8 r8 + 7 x columns 128 kt .. 128 kt + 127 is 1024
 * values at element (r8 * K/128 + kt) * 1024; its piece s (0..3, 256 values
 * at element s * 256) holds, at element (8 g + r) * 8 + c (g 0..3, r 0..7,
 * c 0..7), W[8 r8 + r][128 kt + 32 s + 8 g + c].  Each 512-byte piece is the
 * weight operand of one matrix instruction over 8 rows, read as one
 * contiguous run.
 * moe_pack_fp16_tile8: dst_dev (R*K FP16) = tile8 of the row-major src_dev;
 * both device, 16-byte aligned, not overlapping; one kernel on `stream`. */
int moe_pack_fp16_tile8(const void *src_dev, void *dst_dev, int R, int K, void *stream);
int moe_shared_ffn(const void *x_dev, const void *w_gate_dev, const void *w_up_dev, const void *w_down_dev,
                   const void *w_sgate_dev, int T, int H, int Is, float *shared_out_dev, float *shared_gate_dev,
                   void *ws_dev, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------ resident expert table
 * Which experts have a published device row, and the miss path that brings a
 * missing row to the GPU ("Horizon RunMap - architecture", section
 * "Immutable authority and miss lifecycle"; "Horizon technical notes —
 * publication edition v1", section "Immutable cache — the scope of ADR
 * 0009"):
 *   - the host source holds every expert's qpacked row; it belongs to the
 *     caller, must stay unchanged and outlive the table, and is only read.
 *     When the whole source is page-locked host memory (hipHostMalloc, a
 *     pinned torch tensor), misses are copied straight from it and the
 *     staging buffers are not used (counter direct_copies); pageable sources
 *     go through the staging buffers as below.
 *     Creation takes a 64-bit digest of every row (its identity; compared
 *     with desc->row_digests when given) and checks that every FP16 scale is
 *     finite (its layout); moe_table_verify_source re-checks the digests;
 *   - the table owns capacity + spare_rows device rows (one allocation,
 *     row_stride = row bytes rounded up to 256), a ring of 4 device maps
 *     (int32 [E]: slot of each expert, -1 = no row; one per recent
 *     generation), staging_rows pinned staging buffers of one row, a copy
 *     stream (default priority) and a fixed pool of events; nothing else is
 *     allocated after moe_table_create;
 *   - a generation is one complete published map.  A consumer captures the
 *     current generation with moe_table_acquire (a lease: that generation's
 *     map and the rows it names stay untouched) and ends it with
 *     moe_table_release on the stream of its last reading kernel;
 *   - moe_upload_expert_rows is one miss transaction (transactions are
 *     serialized: a table is used by one host thread at a time).  Each miss
 *     goes host source -> pinned staging (a host memcpy, after that staging
 *     buffer's previous copy has retired) -> a spare row (hipMemcpyAsync on
 *     the copy stream); a spare row is one that neither the current
 *     generation nor any generation with an open lease names, and the copy
 *     stream first waits for the released consumers of every generation that
 *     last named it.  After the copies the next generation's map is written
 *     (same stream) and becomes current: kernels ordered after it see the new
 *     rows, never a partly written one, while readers of older generations
 *     keep theirs;
 *   - the next generation keeps at most `capacity` experts published: least
 *     recently used experts outside the current step lose their device copy
 *     (ties go to the lower expert id);
 *   - no expert bytes ever move device -> host and the host source is never
 *     written (counter expert_d2h_bytes stays 0; host_writes counts rows that
 *     moe_table_verify_source found changed).
 * Failures: before publication (a copy, a wait, the map write) the call
 * returns MOE_ERR_HIP and the previous generation stays current and intact;
 * an ambiguous failure after publication faults the table (every later call
 * returns MOE_ERR_FAULTED).  MOE_ERR_CAPACITY from an upload means the spare
 * rows are held by open leases (or the step exceeds max_tokens).
 * Use per step: bring the active expert list to the host, moe_table_misses,
 * moe_upload_expert_rows(misses, stream), moe_table_acquire(stream), the FFN
 * calls with the lease's rows and map, moe_table_release(lease, stream). */
typedef struct moe_table moe_table;

typedef struct {
    int E, H, I;                       /* experts, hidden size, expert intermediate size */
    int capacity;                      /* experts published between steps (1..E) */
    int spare_rows;                    /* extra device rows that receive misses (see below) */
    int staging_rows;                  /* pinned staging buffers of one row each (1..16) */
    int top_k;                         /* experts per token of the layer (1..min(E, 8)) */
    int max_tokens;                    /* largest step (tokens) the table serves (1..65536) */
    const void *host_source;           /* host: expert e's row at host_source + e*host_row_stride */
    size_t host_row_stride;            /* >= moe_expert_row_bytes(H, I) */
    const int32_t *initial_resident;   /* host: `capacity` distinct expert ids, or NULL for 0..capacity-1 */
    const uint64_t *row_digests;       /* host: E expected moe_row_digest values, or NULL */
    int slot_format;                   /* MOE_SLOT_QPACKED: device rows are qpacked copies (the
                                          resident-qpacked cache); MOE_SLOT_FP16: FP16 execution slots
                                          (offload-qpacked: each miss is copied qpacked, then
                                          dequantized on the GPU into its slot; the FFN reads the slots
                                          with moe_fp16_expert_ffn) */
} moe_table_desc;
enum moe_slot_format { MOE_SLOT_QPACKED = 0, MOE_SLOT_FP16 = 1 };
/* Creation rejects (MOE_ERR_CAPACITY) spare_rows below
 * min(E - capacity, A + max(0, A - capacity)) with A = min(E, max_tokens *
 * top_k): after a step at most max(capacity, A) experts stay published, and
 * the next step's A misses must find rows outside that set. */

typedef struct {
    uint64_t steps;                    /* moe_table_misses calls */
    uint64_t hits, misses;             /* active experts found published / not */
    uint64_t evictions;                /* device copies dropped */
    uint64_t h2d_bytes;                /* expert bytes copied host -> device after creation */
    uint64_t staging_waits;            /* copies that waited for a staging buffer */
    uint64_t expert_d2h_bytes;         /* always 0 */
    uint64_t host_writes;              /* host rows found changed by moe_table_verify_source */
    uint64_t generation;               /* current generation (1 after creation) */
    uint64_t open_leases;              /* leases acquired and not released */
    uint64_t failed_uploads;           /* transactions that failed before publication */
    uint64_t prefetched;               /* rows uploaded by moe_table_prefetch */
    uint64_t prefetch_hits;            /* prefetched experts that a later step routed */
    uint64_t prefetch_unused;          /* prefetched experts evicted before any step routed them */
    uint64_t direct_copies;            /* rows copied straight from a page-locked host source (no staging) */
} moe_table_counters;

typedef struct {
    uint64_t generation;               /* the captured generation */
    const void *rows_dev;              /* device rows (slot s at rows_dev + s*row_stride) */
    size_t row_stride;
    const int32_t *slot_map_dev;       /* that generation's device map, int32 [E] */
} moe_table_lease;

/* Digest of n host bytes (the identity moe_table_create checks). */
uint64_t moe_row_digest(const void *p, size_t n);
/* Creates the table, validates the host source, uploads the initial
 * residents and publishes generation 1 (waits for it).  *out receives the
 * table.  `stream` is unused (the table has its own copy stream). */
int moe_table_create(moe_table **out, const moe_table_desc *desc, void *stream);
/* Waits for the table's copies and for the consumers of released leases,
 * then frees it (NULL is a no-op).  Leases must have been released. */
void moe_table_destroy(moe_table *table);
/* Device rows, their stride and the current generation's map (no lease). */
int moe_table_device(const moe_table *table, const void **rows_dev, size_t *row_stride,
                     const int32_t **slot_map_dev);
/* Starts a step: records the active experts (host array of n ids; duplicates
 * count once) as used now and writes those without a published row to
 * miss_out (capacity n), their number to *n_miss. */
int moe_table_misses(moe_table *table, const int32_t *active_host, int n, int32_t *miss_out, int *n_miss);
/* One miss transaction for the n experts (none may be published already);
 * `stream` (NULL = the default stream) is ordered after the publication.
 * n = 0 publishes nothing. */
int moe_upload_expert_rows(moe_table *table, const int32_t *expert_ids, int n, void *stream);
/* Speculative load of n experts a later step is expected to route (e.g. the
 * next layer's experts predicted from the current activations): starts a
 * step whose active set is these ids (the transaction's eviction keeps them)
 * and uploads those without a published row as one transaction that no
 * stream waits for, so the copies overlap whatever the GPU is running; the
 * next moe_table_acquire orders its consumer after the publication.  Counted
 * in prefetched / prefetch_hits / prefetch_unused, not as misses.  (The pages
 * list speculative next-layer loading among related systems' staging
 * semantics: "Horizon RunMap - Architecture, Experimental Evidence and
 * Scope", "Architecture comparison matrix", row "Publication/staging
 * semantics".) */
int moe_table_prefetch(moe_table *table, const int32_t *expert_ids, int n);
/* Captures the current generation; `stream` is ordered after its publication. */
int moe_table_acquire(moe_table *table, void *stream, moe_table_lease *lease);
/* Ends a lease; its consumers are the work enqueued on `stream` so far. */
int moe_table_release(moe_table *table, const moe_table_lease *lease, void *stream);
/* Re-checks every host row against its digest from creation
 * (MOE_ERR_SOURCE if any changed). */
int moe_table_verify_source(moe_table *table);
int moe_table_stats(const moe_table *table, moe_table_counters *out);
/* Host copy of the current generation's map (E entries, slot or -1). */
int moe_table_published(const moe_table *table, int32_t *slot_map_host);

/* ------------------------------------------------------------ combine
 * y[t][c] = RN16( sum_{j=0..k-1} topk_w[t][j] * pair_out[pair_pos[t*k+j]][c]
 *                 (+ shared_gate[t] * shared_out[t][c]) ), FP32, j ascending.
 * shared_out_dev (FP32 [T][H]) and shared_gate_dev (FP32 [T]) are both NULL
 * or both given.  y_dev: FP16 [T][H]. */
int moe_combine(const float *pair_out_dev, const int32_t *pair_pos_dev, const float *topk_w_dev,
                const float *shared_out_dev, const float *shared_gate_dev,
                int T, int H, int k, void *y_dev, void *stream);

/* ------------------------------------------------------------ FP16 execution slots
 * The offload-qpacked profile ("Horizon RunMap - architecture", section
 * "Historical contracts remain distinct"; "Horizon technical notes —
 * publication edition v1", section "Precision is profile-specific"): a
 * low-bit source dequantized into bounded FP16 execution slots.  Each weight
 * of a slot is the FP16 value nearest (code - 8) * scale (rounded once; this
 * profile's numbers differ from the exact W4A16 layer by that rounding).
 * Slot row: gate [I][H], up [I][H], down [H][I] FP16, each matrix in
 * 4096-byte tiles: tile (rg, kt) = rows 16rg..16rg+15 x columns
 * 128kt..128kt+127 at byte (rg*K/128 + kt)*4096; its piece q (1024 bytes at
 * q*1024) holds, at byte (16g + r)*16, row 16rg + r, columns
 * 128kt + 32g + 8q .. +7 in order.  moe_expert_row_bytes_fp16(H, I) =
 * 3*I*H*2 bytes.
 * moe_dequant_expert_rows: n qpacked rows (stride q_stride) -> n slot rows
 *   (stride f_stride); both 256-byte aligned, strides multiples of 256.
 * moe_fp16_expert_ffn: moe_w4a16_expert_ffn over slot rows (same routing
 *   inputs, rounding points, outputs and status; the streaming kernels). */
size_t moe_expert_row_bytes_fp16(int H, int I);
int moe_dequant_expert_rows(const void *q_rows_dev, size_t q_stride, void *f_rows_dev, size_t f_stride, int n, int H,
                            int I, void *stream);
int moe_fp16_expert_ffn(const void *x_dev, int T, int H, int I, int E, int k,
                        const void *rows_dev, size_t row_stride, const int32_t *slot_map_dev,
                        const int32_t *expert_offsets_dev, const int32_t *sorted_pairs_dev,
                        const int32_t *active_list_dev, const int32_t *n_active_dev,
                        void *h_dev, float *pair_out_dev, int32_t *status_dev, void *stream);

/* ------------------------------------------------------------ residual stream
 * out[i] = RN16(a[i] + b[i]) for FP16 a, b (n elements; out may alias a or
 * b): the residual connection that chains layers of a stack, x_{l+1} = x_l +
 * y_l (the sum of two FP16 values is exact in fp64 and rounded once). */
int moe_residual_add(const void *a_dev, const void *b_dev, void *out_dev, long long n, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_W4A16_H */
