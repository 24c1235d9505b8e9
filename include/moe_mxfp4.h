/*
 * moe_mxfp4.h - C ABI of the MI355X (gfx950) MXFP4 grouped-expert MoE layer.
 *
 * The layer is the gpt-oss mixture-of-experts block that the SimpleLLM
 * write-up ("A 297-line kernel file that decodes faster than vLLM") profiles
 * as "Router + top-k", "MoE gate/up + SwiGLU" and "MoE down + combine"
 * (section "Where the time went"), with the expert weights kept in MXFP4 and
 * routed through a per-expert tile table (section "Optimizations": "MXFP4 MoE
 * on tensor cores", "Per-expert routing tile table", "MoE token tile follows
 * tokens per expert").  The triton-kernels README's fused MoE dispatch
 * (section "Quick Start") names the same pipeline: router with softmax
 * gating and top-k, permute, expert FFN, unpermute.
 *
 * One layer call is three entry points, all enqueued on one stream:
 *   moe_route        router logits -> top-k -> softmax (or sigmoid) over
 *                    the k selected
 *   moe_build_tiles  per-expert counts, offsets, stable sort, tile table
 *   moe_forward      grouped gate/up GEMM + SwiGLU, grouped down GEMM,
 *                    weighted combine back to token order
 * with fewer launches for small batches: moe_route_tiles (the first two in
 * one launch, up to 64 tokens), moe_layer_one_token (all of it in one
 * launch, one token) and moe_layer_small_batch (all of it in one launch,
 * 2 to 4 tokens).  moe_repack_weights prepares, once at load, the
 * blocked layout of the packed codes that every expert kernel streams
 * fastest.
 *
 * Conventions shared by every entry point:
 *   - Every array argument is a DEVICE pointer on the current HIP device,
 *     allocated and owned by the caller.  The library allocates nothing,
 *     keeps no state across calls (beyond a per-device architecture check),
 *     never synchronises the host, and enqueues all work on `stream`
 *     (NULL = the default stream).
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     non-OK return nothing was enqueued and nothing was written.  A launch
 *     that fails returns MOE_ERR_HIP.
 *   - T == 0 is a no-op that returns MOE_OK.
 *   - Device pointers to arrays read with 128-bit loads (x, w_router, the
 *     packed weights, workspaces) must be 16-byte aligned (MOE_ERR_ALIGN).
 *   - Only gfx950 devices are accepted (MOE_ERR_DEVICE).
 *   - Calls on one stream are ordered; calls that share output or workspace
 *     buffers on different streams race.
 *
 * Data layouts (row-major, C order):
 *   x             bf16 bits, uint16 [T][H]
 *   w_router      fp32 [E][H];  bias fp32 [E] or NULL
 *   w13_q         uint8 [E][2I][H/2]  MXFP4 e2m1 codes, two per byte, the
 *                 even K element in the low nibble; rows [0, I) are the gate
 *                 projection W1, rows [I, 2I) the up projection W3
 *   w13_s         uint8 [E][2I][H/32] E8M0 scales, one per 32 consecutive K
 *                 elements of a row: value 2^(s-127), s = 255 is NaN
 *   w2_q, w2_s    uint8 [E][H][I/2], uint8 [E][H][I/32]  down projection
 *   topk_ids      int32 [T][k];  topk_weights fp32 [T][k]
 *   expert_offsets int32 [E+1];  sorted_ids int32 [T*k]
 *   tiles         int32 [tiles_max][3] rows (expert, row_start, rows)
 *   num_tiles     int32 [1]
 *   out           bf16 bits, uint16 [T][H]
 * The packed codes w13_q and w2_q may instead be in the blocked layout
 * (MOE_LAYOUT_BLOCKED below, made by moe_repack_weights); the entry points
 * that read them take a `layout` argument.  Scales are always as above.
 *
 * Numerics: router logits are accumulated in fp64 (bf16 x fp32 products are
 * exact in fp64), so the top-k choice matches an exact evaluation whenever
 * logits differ by more than ~1e-13.  Expert weights are decoded exactly to
 * bf16 (exact for scale bytes 2..252) and multiplied on bf16 MFMA with fp32
 * accumulation; h = silu(g)*u is rounded to bf16, y kept in fp32, and the
 * combine accumulates in fp32 in slot order and rounds once to bf16.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* hipStream_t is `struct ihipStream_t*` */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,      /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,     /* a size is out of the supported range */
  MOE_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = 4, /* workspace smaller than the *_workspace_bytes query */
  MOE_ERR_DEVICE = 5,    /* current device is not gfx950 or cannot be queried */
  MOE_ERR_HIP = 6,       /* a kernel launch failed */
  MOE_ERR_OVERLAP = 7    /* an output buffer overlaps an input it must not */
} moe_status;

/* Static description of a status code (host). */
const char* moe_status_string(int status);

/* Library version string, e.g. "0.1.0" (host). */
const char* moe_version(void);

/* ------------------------------------------------------------------ limits */
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 8
#define MOE_MAX_DIM 65536 /* largest H or I */

/* Gating of the k selected logits (the `gating` argument of the routing
 * entry points).  The triton-kernels README ("Project Structure",
 * moe/router.py) names softmax and sigmoid gating beside top-k; the
 * selection is the same top-k of the logits for both.
 *   MOE_GATING_SOFTMAX  w_j = exp(L_j - max) / sum over the k of the same
 *   MOE_GATING_SIGMOID  w_j = s_j / sum over the k of s, s = 1/(1+exp(-L_j))
 * Both are evaluated in fp64, the sum taken in ascending slot order, and the
 * weights rounded to fp32 once.  Any other value gives MOE_ERR_SHAPE. */
#define MOE_GATING_SOFTMAX 0
#define MOE_GATING_SIGMOID 1

/* Byte layout of the packed codes w13_q / w2_q (the `layout` argument of the
 * entry points that read them; any other value gives MOE_ERR_SHAPE).
 *   MOE_LAYOUT_CANONICAL  row-major [rows][K/2] as described above.
 *   MOE_LAYOUT_BLOCKED    the same bytes regrouped within each run of 16
 *                         consecutive rows (rows 16g .. 16g+15 of the
 *                         flattened [E*rows][K/2] matrix): byte i (0..15) of
 *                         MX block b of row 16g + r sits at byte
 *                         16g*(K/2) + 256b + 16r + i.
 * The blocked layout gives every wave of the expert kernels one contiguous
 * kilobyte per load instruction.  Results are bit-identical between the two
 * layouts. */
#define MOE_LAYOUT_CANONICAL 0
#define MOE_LAYOUT_BLOCKED 1

/* ------------------------------------------------------ moe_repack_weights
 * Reorders a packed code matrix from MOE_LAYOUT_CANONICAL to
 * MOE_LAYOUT_BLOCKED, once, when weights are loaded.  The SimpleLLM write-up
 * permutes its MXFP4 weights at load into the order its kernel reads
 * ("Optimizations": "MXFP4 MoE on tensor cores"; "Dead ends": fixing the
 * layout inside the kernel was slower) and re-quantizes nothing
 * ("Correctness"); here too only bytes move.
 *   q          device, uint8 [rows][K/2] canonical (w13_q: rows = E*2I,
 *              K = H; w2_q: rows = E*H, K = I), 16-byte aligned, read only
 *   rows       > 0, a multiple of 16;  K: > 0, a multiple of 32, <= 65536
 *   q_blocked  device, uint8 [rows][K/2], 16-byte aligned, written; must not
 *              overlap q (MOE_ERR_OVERLAP)
 * Scales are not touched.  Errors: MOE_ERR_SHAPE (sizes), MOE_ERR_NULL,
 * MOE_ERR_ALIGN, MOE_ERR_OVERLAP, MOE_ERR_DEVICE, MOE_ERR_HIP; on error
 * nothing is written. */
moe_status moe_repack_weights(const uint8_t* q, int64_t rows, int K, uint8_t* q_blocked,
                              struct ihipStream_t* stream);

/* Token tile for the tile table (host, pure function).  The SimpleLLM
 * write-up pins the tile rather than autotuning it ("Fixed decode tiles")
 * and grows the token tile with tokens per expert ("MoE token tile follows
 * tokens per expert"), so that an expert's weights are unpacked once rather
 * than once per small tile.  An expert receives at most one slot per token,
 * so BM >= T keeps every expert in one tile.  Rule: the smallest of
 * 16, 32, 64, 128 that is >= T (128 when T > 64).  The kernels process a
 * tile's rows in passes of at most 16 while its weights stay in registers,
 * so a large BM costs nothing at small T.  Returns 16 for T <= 16. */
int moe_pick_bm(int T, int k, int E);

/* Upper bound on num_tiles for any routing (host, pure function):
 * min(T*k, ceil(T*k/BM) + min(E, T*k)).  The tiles array passed to
 * moe_build_tiles / moe_forward must hold this many rows of 3 int32. */
int64_t moe_tiles_max(int T, int k, int E, int BM);

/* Workspace bytes moe_route needs (host, pure function; 0 when T == 0). */
size_t moe_route_workspace_bytes(int T, int H, int E);

/* Workspace bytes moe_forward needs (host, pure function): h bf16 [T*k][I]
 * and y fp32 [T*k][H], each rounded up to 256 bytes. */
size_t moe_forward_workspace_bytes(int T, int H, int I, int k);

/* ------------------------------------------------------------- moe_route
 * Router logits L[t][e] = sum_h x[t][h]*w_router[e][h] (+ bias[e]) in fp64,
 * then per token the k largest logits in descending order (exact ties go to
 * the lower expert index) and the gating (softmax, or normalised sigmoid:
 * MOE_GATING_*) over those k logits.
 * ("Where the time went": "Router + top-k"; the triton-kernels README,
 * section "Project Structure", lists a router module that pairs top-k with
 * softmax or sigmoid gating.)
 *
 *   x           [T][H] bf16 bits, 16-byte aligned
 *   w_router    [E][H] fp32, 16-byte aligned
 *   bias        [E] fp32 or NULL; added before top-k and gating
 *   T >= 0, 0 < H <= 65536, H % 32 == 0, 1 <= E <= 256, 1 <= k <= min(E, 8),
 *   T*E < 2^31, gating MOE_GATING_SOFTMAX or MOE_GATING_SIGMOID
 *   topk_ids    out [T][k] int32
 *   topk_weights out [T][k] fp32 (each row sums to 1 within 1e-6)
 *   logits      out [T][E] fp64, or NULL if not wanted
 *   workspace   >= moe_route_workspace_bytes(T, H, E), 16-byte aligned
 * NaN logits make the choice unspecified (but in range).
 */
moe_status moe_route(const uint16_t* x, const float* w_router, const float* bias,
                     int T, int H, int E, int k, int gating,
                     int32_t* topk_ids, float* topk_weights, double* logits,
                     void* workspace, size_t workspace_bytes,
                     struct ihipStream_t* stream);

/* ------------------------------------------------------- moe_build_tiles
 * Per-expert tile table ("Optimizations": "Per-expert routing tile table" -
 * each expert writes its own tiles instead of the GEMM searching a
 * tiles x experts grid; "MoE token tile follows tokens per expert").
 * Bit-exact and deterministic:
 *   counts c_e = #{p : topk_ids[p] == e}, p = t*k + j the flat slot id
 *   expert_offsets[0] = 0, expert_offsets[e+1] = expert_offsets[e] + c_e
 *   sorted_ids = the slot ids ordered by expert, ascending p within an
 *                expert (a stable counting sort)
 *   tiles: for e ascending, for i in 0..ceil(c_e/BM)-1:
 *          (e, expert_offsets[e] + i*BM, min(BM, c_e - i*BM))
 *   num_tiles[0] = sum_e ceil(c_e/BM)
 *
 *   topk_ids    [T][k] int32; ids outside [0, E) are dropped from counts and
 *               tiles (they are placed after expert_offsets[E] in
 *               sorted_ids so every slot id still appears exactly once)
 *   T >= 0, 1 <= k <= 8, 1 <= E <= 256, T*k < 2^31, BM in {16,32,64,128}
 *   expert_offsets out [E+1]; sorted_ids out [T*k];
 *   tiles out [moe_tiles_max(T,k,E,BM)][3] (rows past num_tiles untouched);
 *   num_tiles out [1]
 */
moe_status moe_build_tiles(const int32_t* topk_ids, int T, int k, int E, int BM,
                           int32_t* expert_offsets, int32_t* sorted_ids,
                           int32_t* tiles, int32_t* num_tiles,
                           struct ihipStream_t* stream);

/* ----------------------------------------------------------- moe_forward
 * For every tile (e, row_start, rows) and each slot p = sorted_ids[r],
 * r in [row_start, row_start+rows), token t = p / k:
 *   g = x[t] W1_e^T, u = x[t] W3_e^T, h[r] = silu(g) * u       (gate/up)
 *   y[p] = h[r] W2_e^T                                          (down)
 * then out[t] = sum_{j<k} topk_weights[t][j] * y[t*k + j]       (combine)
 * with MXFP4 weights W = e2m1(code) * 2^(s-127).  ("MXFP4 MoE on tensor
 * cores", "MoE gate/up + SwiGLU", "MoE down + combine"; the README's fused
 * SwiGLU is silu(gate) * up.)  The combine uses no atomics; results are
 * bit-identical from run to run.
 *
 *   x             [T][H] bf16 bits, 16-byte aligned
 *   w13_q, w13_s, w2_q, w2_s   MXFP4 weights (layouts above), 16-byte aligned
 *   layout        MOE_LAYOUT_CANONICAL or MOE_LAYOUT_BLOCKED, for w13_q and w2_q
 *   topk_weights  [T][k] fp32 (from moe_route)
 *   sorted_ids, tiles, num_tiles  from moe_build_tiles with the same T, k,
 *                 E and BM; every slot id must appear once in sorted_ids
 *   T >= 0, 0 < H, I <= 65536, H % 32 == 0, I % 32 == 0, 1 <= E <= 256,
 *   1 <= k <= min(E, 8), BM in {16,32,64,128}, T*k < 2^31, E*2I < 2^31
 *   workspace     >= moe_forward_workspace_bytes(T, H, I, k), 16-byte aligned
 *   out           out [T][H] bf16 bits
 * If topk_ids held ids outside [0, E) the output is unspecified, but every
 * memory access stays inside the buffers described here.
 */
moe_status moe_forward(const uint16_t* x,
                       const uint8_t* w13_q, const uint8_t* w13_s,
                       const uint8_t* w2_q, const uint8_t* w2_s,
                       const float* topk_weights, const int32_t* sorted_ids,
                       const int32_t* tiles, const int32_t* num_tiles,
                       int T, int H, int I, int E, int k, int BM, int layout,
                       void* workspace, size_t workspace_bytes,
                       uint16_t* out, struct ihipStream_t* stream);

/* ---------------------------------------------------- moe_forward_gptoss
 * moe_forward with the expert form of the released gpt-oss models, whose
 * MXFP4 checkpoints the SimpleLLM write-up runs unchanged ("Correctness")
 * without spelling out their expert arithmetic; its definition here is the
 * released model's own (not on the pages):
 *   z = x[t] W13_e^T + b13[e]
 *   g = min(z_gate, limit), u = clip(z_up, -limit, limit)
 *   h = g * sigmoid(alpha * g) * (u + 1)                    (rounded to bf16)
 *   y[p] = h W2_e^T + b2[e]
 * then the same combine.  The released models use alpha = 1.702, limit = 7.
 *
 *   arguments as for moe_forward, plus
 *   w13_q, w13_s  gate rows [0, I) and up rows [I, 2I) of each expert: a
 *                 checkpoint's interleaved rows (gate of output i at row 2i,
 *                 up at 2i + 1) go through moe_deinterleave_rows first (and
 *                 then moe_repack_weights for the blocked layout)
 *   b13           [E][2I] fp32 in the same row order as w13 (so also
 *                 de-interleaved), or NULL for zero biases
 *   b2            [E][H] fp32, or NULL
 *   alpha         finite;  limit > 0 (INFINITY: no clamp), else MOE_ERR_SHAPE
 * Only the separate-launch path has this form (moe_layer_one_token keeps the
 * plain SwiGLU). */
moe_status moe_forward_gptoss(const uint16_t* x,
                              const uint8_t* w13_q, const uint8_t* w13_s,
                              const uint8_t* w2_q, const uint8_t* w2_s,
                              const float* b13, const float* b2, float alpha, float limit,
                              const float* topk_weights, const int32_t* sorted_ids,
                              const int32_t* tiles, const int32_t* num_tiles,
                              int T, int H, int I, int E, int k, int BM, int layout,
                              void* workspace, size_t workspace_bytes,
                              uint16_t* out, struct ihipStream_t* stream);

/* ------------------------------------------------- moe_deinterleave_rows
 * Load-time row permutation for checkpoints that keep each output's gate and
 * up rows adjacent: within each of E blocks of 2I rows, destination row i
 * takes source row 2i and destination row I + i takes source row 2i + 1.
 * Bytes move unchanged ("Correctness": nothing is re-quantised).
 *   src, dst   device, E * 2I rows of row_bytes bytes each (w13_q: row_bytes
 *              = H/2; w13_s: H/32; b13 as fp32: 4); must not overlap
 *              (MOE_ERR_OVERLAP)
 *   E >= 1, I >= 1, row_bytes >= 1, total bytes < 2^40, else MOE_ERR_SHAPE
 */
moe_status moe_deinterleave_rows(const void* src, int E, int I, int row_bytes, void* dst,
                                 struct ihipStream_t* stream);

/* ------------------------------------------ moe_forward_static_workspace
 * moe_forward for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  The h and y intermediates live in a workspace the library
 * holds itself, a device array of MOE_STATIC_WORKSPACE_BYTES bytes on each
 * GPU it runs on (created with the library's code object and kept until the
 * process ends); the call allocates nothing and frees nothing.
 *
 *   arguments as for moe_forward, without workspace and workspace_bytes
 *   MOE_ERR_WORKSPACE when moe_forward_workspace_bytes(T, H, I, k) exceeds
 *   MOE_STATIC_WORKSPACE_BYTES (about 970 slots of 2880 x 2880: T <= 242 at
 *   k = 4), checked on the host before anything is enqueued.
 * Every call on one GPU uses that GPU's one array: the array is fully
 * written before it is read within a call (nothing in it needs to start at
 * zero), and calls in one process on one GPU that overlap in time (on
 * different streams or host threads) race and give unspecified outputs.
 * Results are bit-identical to moe_forward. */
#define MOE_STATIC_WORKSPACE_BYTES (16u << 20)

moe_status moe_forward_static_workspace(const uint16_t* x,
                                        const uint8_t* w13_q, const uint8_t* w13_s,
                                        const uint8_t* w2_q, const uint8_t* w2_s,
                                        const float* topk_weights, const int32_t* sorted_ids,
                                        const int32_t* tiles, const int32_t* num_tiles,
                                        int T, int H, int I, int E, int k, int BM, int layout,
                                        uint16_t* out, struct ihipStream_t* stream);

/* ------------------------------------------------------- moe_route_tiles
 * moe_route followed by moe_build_tiles in a single launch, for decode-sized
 * batches (T <= 64; otherwise MOE_ERR_SHAPE).  The write-up counts launch
 * and host gaps as their own cost of a decode step ("Where the time went":
 * "Launch and host gaps"), and at decode sizes the routing work is too small
 * to hide them.  The workgroups computing partial logits take tickets from
 * counters in the workspace: up to 16 tokens the last one sums the partials
 * in a fixed order and runs top-k, softmax and the tile table; from 17 to 64
 * tokens the last one of each 4-token block runs that block's top-k and
 * gating, and the last block builds the table.  Outputs are bit-identical to
 * moe_route + moe_build_tiles with the same arguments.  (On MI355X the two
 * separate launches measured faster from 17 tokens on: 11.5 against 13.5 us
 * at 64 tokens, 2880 hidden, 32 experts; the one launch saves a host
 * enqueue.)
 *
 *   arguments as for moe_route and moe_build_tiles
 *   workspace   >= moe_route_tiles_workspace_bytes(T, H, E), 16-byte aligned.
 *               Its first 256 bytes hold the ticket counters: they must be
 *               zero before the first call, and every call leaves them zero
 *               (a workspace sized for the largest T serves every smaller
 *               one).  Calls that share a workspace must not overlap in time.
 */
size_t moe_route_tiles_workspace_bytes(int T, int H, int E);

moe_status moe_route_tiles(const uint16_t* x, const float* w_router, const float* bias,
                           int T, int H, int E, int k, int gating, int BM,
                           int32_t* topk_ids, float* topk_weights, double* logits,
                           int32_t* expert_offsets, int32_t* sorted_ids,
                           int32_t* tiles, int32_t* num_tiles,
                           void* workspace, size_t workspace_bytes,
                           struct ihipStream_t* stream);

/* --------------------------------------------------- moe_layer_one_token
 * The whole layer for a single token (T = 1) in one launch: moe_route_tiles
 * followed by moe_forward.  The write-up books launch and host gaps as their
 * own cost of a decode step ("Where the time went": "Launch and host gaps");
 * with one token, five dependent launches leave the GPU waiting between
 * steps.  Here the routing, gate/up and down workgroups share one grid: each
 * waits (by polling words in the workspace) only for workgroups with a
 * lower index; up to 32 routing workgroups each compute the top-k from the
 * published partial logits and publish the plan, so the GEMM workgroups
 * learn their experts without a single serial tail; the last down
 * workgroup of each 16-row block combines its k slots.  Every output is
 * bit-identical to moe_route_tiles + moe_forward with the same arguments
 * (BM any valid value: one token gives k one-row tiles).
 *
 *   arguments as for moe_route_tiles and moe_forward with T = 1 (layout
 *   included: it follows gating); logits may
 *   be NULL; bias may be NULL.  Also requires H <= 3072 and I <= 3072 (one
 *   register chunk of weights per lane), else MOE_ERR_SHAPE.
 *   workspace   >= moe_layer_one_token_workspace_bytes(H, I, E, k) (0 means
 *               the shape is not accepted), 16-byte aligned.  Its first
 *               moe_layer_one_token_sync_bytes(H) bytes are counters and
 *               flags: zero before the first call; each call leaves them
 *               consistent for the next (zeroing the whole region between
 *               calls is also allowed, zeroing part of it is not).  The int
 *               at byte 4 counts completed calls.  Calls that share a
 *               workspace must not overlap in time.  If a wait ever gave up
 *               (a GPU too busy to run the grid for about a second), the
 *               int at byte 8 is set and the outputs are unspecified until
 *               the region is zeroed.  The int at byte 12 bounds the
 *               polls: zero (as zeroed) keeps the default of 2^20 re-polls
 *               per wait; a value n > 0, written by the caller between
 *               calls, lowers it to n - 1 re-polls (a test of the give-up
 *               path writes 1).  It is read on the device at every call, so
 *               a captured graph follows the current value.
 */
size_t moe_layer_one_token_workspace_bytes(int H, int I, int E, int k);
size_t moe_layer_one_token_sync_bytes(int H);

moe_status moe_layer_one_token(const uint16_t* x, const float* w_router, const float* bias,
                               const uint8_t* w13_q, const uint8_t* w13_s,
                               const uint8_t* w2_q, const uint8_t* w2_s,
                               int H, int I, int E, int k, int gating, int layout,
                               int32_t* topk_ids, float* topk_weights, double* logits,
                               int32_t* expert_offsets, int32_t* sorted_ids,
                               int32_t* tiles, int32_t* num_tiles,
                               void* workspace, size_t workspace_bytes,
                               uint16_t* out, struct ihipStream_t* stream);

/* ------------------------------------------------- moe_layer_small_batch
 * The whole layer for a small batch (2 <= T <= 4, T * k <= 16) in one
 * launch: moe_route_tiles followed by moe_forward, with the scheme of
 * moe_layer_one_token ("Where the time went": "Launch and host gaps") and
 * tiles of several rows: each publisher's wave t routes token t and one
 * wave builds the table, whose plan words carry each tile's expert, rows
 * and slots; a gate/up job covers all rows of its tile, a down job reads
 * the tile's h rows as they arrive, and the last tile's down job of each
 * 16-column block combines every token of the block.  Every output is
 * bit-identical to moe_route_tiles + moe_forward with the same arguments
 * (BM any valid value: at most T <= 4 rows per expert give one tile each).
 * (On MI355X it does not beat the separate launches at the gpt-oss-20b
 * shape: 35.4 against 35.3 us at 2 tokens (32.6 against 34.4 under a skewed
 * router), 59.4 against 52.7 at 4; it saves the host three enqueues per
 * call.)
 *
 *   arguments as for moe_route_tiles and moe_forward; logits may be NULL;
 *   bias may be NULL.  Also requires layout == MOE_LAYOUT_BLOCKED, H <= 3072
 *   and I <= 3072, else MOE_ERR_SHAPE.
 *   workspace   >= moe_layer_small_batch_workspace_bytes(T, H, I, E, k) (0
 *               means the shape is not accepted), 16-byte aligned.  Its
 *               first moe_layer_small_batch_sync_bytes() bytes are counters,
 *               flags and published words with the same contract as
 *               moe_layer_one_token's sync bytes (zero before the first
 *               call, left consistent by each call; the int at byte 8 set if
 *               a wait gave up; the int at byte 12 bounds the polls).  Calls
 *               that share a workspace must not overlap in time.
 */
size_t moe_layer_small_batch_workspace_bytes(int T, int H, int I, int E, int k);
size_t moe_layer_small_batch_sync_bytes(void);

moe_status moe_layer_small_batch(const uint16_t* x, const float* w_router, const float* bias,
                                 const uint8_t* w13_q, const uint8_t* w13_s,
                                 const uint8_t* w2_q, const uint8_t* w2_s,
                                 int T, int H, int I, int E, int k, int gating, int layout,
                                 int32_t* topk_ids, float* topk_weights, double* logits,
                                 int32_t* expert_offsets, int32_t* sorted_ids,
                                 int32_t* tiles, int32_t* num_tiles,
                                 void* workspace, size_t workspace_bytes,
                                 uint16_t* out, struct ihipStream_t* stream);

/* --------------------------------------------- the three steps of moe_forward
 * moe_forward is exactly these three calls in order; they are exported so a
 * caller can time or overlap them separately.  Arguments and constraints are
 * those of moe_forward; h and y are caller buffers (device):
 *   h  bf16 bits [T*k][I], row r = position r in sorted_ids
 *   y  fp32 [T*k][H], row p = flat slot id p = t*k + j
 */

/* Grouped gate/up GEMM with fused SwiGLU ("Where the time went": "MoE
 * gate/up + SwiGLU"; triton-kernels README "Fused SwiGLU": silu(gate) * up):
 * h[r] = bf16(silu(x[t] W1_e^T) * (x[t] W3_e^T)) for every tiled row r. */
moe_status moe_gateup_swiglu(const uint16_t* x, const uint8_t* w13_q, const uint8_t* w13_s,
                             const int32_t* sorted_ids, const int32_t* tiles,
                             const int32_t* num_tiles, int T, int H, int I, int E, int k, int BM,
                             int layout, uint16_t* h, struct ihipStream_t* stream);

/* Grouped down GEMM ("MoE down + combine"): y[sorted_ids[r]] = h[r] W2_e^T. */
moe_status moe_down(const uint16_t* h, const uint8_t* w2_q, const uint8_t* w2_s,
                    const int32_t* sorted_ids, const int32_t* tiles, const int32_t* num_tiles,
                    int T, int H, int I, int E, int k, int BM, int layout, float* y,
                    struct ihipStream_t* stream);

/* Weighted combine ("MoE down + combine"; the README's unpermute):
 * out[t] = bf16(sum_{j<k} topk_weights[t][j] * y[t*k + j]), fp32 in
 * ascending j.  y must be 16-byte aligned. */
moe_status moe_combine(const float* y, const float* topk_weights, int T, int H, int k,
                       uint16_t* out, struct ihipStream_t* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
