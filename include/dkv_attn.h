/*
 * dkv_attn.h -- C ABI of libdkv_attn: DKV decode attention over a compressed
 * KV cache on AMD Instinct MI355X (gfx950).
 *
 * The method is the one described on the pages "DKV: Anchor + Low-Rank
 * Differential KV-Cache Compression for Scalable Long-Context Inference"
 * (Zenodo record, abstract) and the Differential-KV README ("Core Architecture
 * & Paper Overview", "Decode & Prefill Innovations", "Key Environment Knobs").
 *
 * Storage of one 256-token block, per layer and KV head:
 *   anchor (a_k, a_v)   the block's first token, exact                 fp16 [d] each
 *   U                   joint K|V delta coefficients of tokens 1..255  fp16 [255][r]
 *   V_K, V_V            right bases of the delta                       fp16 [r][d] each
 *   residual rows       exact K, V rows                                fp16 [R][d] each
 *   residual positions  in-block position (1..255) of each residual    uint8 [R]
 *   route key           c = a_k + mean_i(U_i) V_K                      fp32 [d]
 * Token i (1..255) of a block is k_i = a_k + U_{i-1} V_K, v_i = a_v + U_{i-1} V_V,
 * except that a residual row replaces the token at its recorded position.
 *
 * Decode output for query head g of sequence b is exact softmax attention
 * over: the 256 rows of each routed block (anchor, reconstructed rows that are
 * not residual positions, residual rows) and the first win_len[b] rows of the
 * dense recency window, with scores z = scale * q_g . k.  The library never
 * materialises reconstructed K or V; scores of reconstructed rows are taken
 * in the rank-r space, q.a_k + U_i.(V_K q), and their values gathered as
 * (sum p) a_v + (p^T U) V_V.  Pools that hold keys from before the rotary
 * embedding (dkv_pool.rope_freq) rotate every key to its absolute position
 * at read: their kernels rebuild each block's keys 16 at a time in registers
 * (a_k + U_i V_K on matrix cores), rotate them and score them; values are the
 * same.  Such pools may also share bases between blocks (dkv_pool.basis_of).
 *
 * Conventions shared by every entry point
 *   - head_dim d = 128 and block size 256 are fixed (DKV_ERR_UNSUPPORTED
 *     otherwise); 1 <= r <= 64; 0 <= R <= 255; G = Hq / Hkv <= 16.
 *   - All pointers in dkv_pool / dkv_batch and every array argument are DEVICE
 *     pointers, owned by the caller.  The library allocates nothing, frees
 *     nothing and keeps no pointer after a call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work and return; results are valid after the stream is
 *     synchronised.  Device-side faults surface at that synchronisation.
 *   - Scalar arguments, pointer presence and alignment are validated on the
 *     host before anything is enqueued; on failure the call returns an error
 *     code, enqueues nothing, and dkv_last_error() describes the problem.
 *   - Contents of device arrays are preconditions and are not checked on the
 *     hot path: residual positions distinct in 1..255 (in any order), finite
 *     values.  Block table entries outside [0, n_slots) and idx entries
 *     outside [0, n_blocks[b]) are treated as empty blocks (no rows), never
 *     read.
 *   - Alignment: every fp16 / fp32 array base and every slot / head stride
 *     (in bytes) must be a multiple of 16, except `u` (a multiple of 8 bytes
 *     when r is a multiple of 4, else of 2) and `resid_pos` (any alignment);
 *     quantised residual codes and their scale/bias arrays also take 16.
 *   - Deterministic: identical inputs give bit-identical outputs (fixed
 *     reduction orders, no floating-point atomics).
 *   - lse values are natural logarithms of sums of exp of SCALED scores.
 *     A part or a sequence with no rows has o = 0 and lse = -inf.
 *   - fp16 outputs are rounded from fp32 to nearest even.
 */
#ifndef DKV_ATTN_H
#define DKV_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DKV_ABI_VERSION 5
#define DKV_HEAD_DIM 128
#define DKV_BLOCK_SIZE 256
#define DKV_MAX_RANK 64
#define DKV_MAX_RESID 255
#define DKV_MAX_GROUP 16
#define DKV_MAX_ROUTE_BLOCKS 12288
#define DKV_MAX_SLOTS ((1 << 24) - 3)  /* blocks a pool may hold */

/* Storage format of the residual rows (README "Physical 4-Bit Group-Quantized
 * Residual Buffers" and its "Tunable Quantization Dials"): fp16 rows, or
 * asymmetric group quantisation in groups of 64 of the 128 dimensions with an
 * fp16 scale and bias per group: x[d] = scale_g * code[d] + bias_g, g = d / 64,
 * unsigned codes (0..255 or 0..15).  4-bit codes are packed two per byte,
 * dimension 2j in the low nibble of byte j (the little-endian order of the
 * pages' packed uint32 words). */
#define DKV_RESID_FP16 0
#define DKV_RESID_INT8 1
#define DKV_RESID_INT4 2

typedef int32_t dkv_status;
#define DKV_OK 0
#define DKV_ERR_INVALID_ARG 1  /* null pointer, negative size, bad combination */
#define DKV_ERR_UNSUPPORTED 2  /* d != 128, block != 256, r > 64, R > 255, G > 16, n_slots > DKV_MAX_SLOTS, misalignment */
#define DKV_ERR_WORKSPACE 3    /* workspace missing or smaller than dkv_decode_workspace_size() */
#define DKV_ERR_HIP 4          /* a HIP launch failed; see dkv_last_error() */

/* A strided view of one per-(slot, KV head) array of the block pool: the entry of
 * (slot s, head h) starts at element  ptr + s * slot_stride + h * head_stride
 * (strides in ELEMENTS of the array's type); inside an entry rows are packed. */
typedef struct dkv_view {
  const void* ptr;
  int64_t slot_stride;
  int64_t head_stride;
} dkv_view;

/* One layer's block pool (README "Core Architecture & Paper Overview", items 1-3). */
typedef struct dkv_pool {
  int32_t head_dim;    /* d, must be 128 */
  int32_t block_size;  /* must be 256 */
  int32_t rank;        /* r, 1..64 */
  int32_t n_resid;     /* R, 0..255: residual rows stored in every block */
  int32_t n_kv_heads;  /* Hkv >= 1 */
  int32_t n_slots;     /* number of blocks the pool holds */
  dkv_view anchor_k;   /* fp16 [d]      */
  dkv_view anchor_v;   /* fp16 [d]      */
  dkv_view u;          /* fp16 [255][r] */
  dkv_view vk;         /* fp16 [r][d]   */
  dkv_view vv;         /* fp16 [r][d]   */
  dkv_view resid_k;    /* fp16 [R][d]; or uint8 codes [R][d] (INT8) / [R][d/2] (INT4) */
  dkv_view resid_v;    /* same as resid_k */
  dkv_view resid_pos;  /* uint8 [R], distinct values in 1..255 */
  dkv_view route_key;  /* fp32 [d]; written by dkv_route_keys, read by routing */
  int32_t resid_format;   /* DKV_RESID_FP16 (0, what zero-initialised structs hold), _INT8 or _INT4 */
  int32_t reserved0;
  dkv_view resid_k_sb;    /* quantised formats only: fp16 [R][2][2], (scale, bias) of dims 0..63, 64..127 */
  dkv_view resid_v_sb;    /* same for the V rows */
  /* Un-rotated pools (README "Key Environment Knobs", DKV_ROTATED_POOL = 0, and
   * the preset ladder's "keys stored" column): the anchors, V_K and residual
   * keys hold keys from before the rotary position embedding, and every read
   * rotates a key to its absolute position: the anchor of the block in slot s
   * to slot_pos[s], low-rank row i to slot_pos[s] + i, a residual row to
   * slot_pos[s] + its resid_pos.  Rotation pairs dimension j with j + 64 and
   * turns the pair by the angle position * theta_j:
   *   x'_j = x_j cos - x_{j+64} sin,   x'_{j+64} = x_{j+64} cos + x_j sin.
   * Values, the queries and the dense window are never rotated by the library
   * (the queries and window keys arrive rotated).  NULL rope_freq: the pool
   * holds rotated keys (the default).  Residual rows may be fp16 or quantised.
   *   rope_freq: fp32 [2][64] device, theta_j / (2 pi) as an unevaluated sum
   *              row0[j] + row1[j] of two floats (dkv_rope_freqs fills it);
   *   slot_pos:  int32 [n_slots] device, positions in [0, 2^24 - 256]. */
  const float* rope_freq;
  const int32_t* slot_pos;
  /* Shared basis (README "Key Environment Knobs", DKV_SHARED_BASIS and
   * DKV_SHARED_BASIS_FRAC; "3. Shared Low-Rank Bases"): several blocks may
   * use one stored V_K, V_V pair, so the basis store can hold fewer entries
   * than the pool has slots.
   * NULL, or int32 [n_slots] device: the block in slot s reads its V_K and V_V
   * from entry basis_of[s] of vk and vv (entry e at vk.ptr + e * vk.slot_stride
   * + h * vk.head_stride: the basis store may be an array of its own, n_basis
   * entries); its anchors, U and residual rows stay in slot s.  Needs an
   * un-rotated pool (the pages refuse sharing with rotated keys).  A block
   * whose entry lies outside [0, n_basis) contributes no rows and its routing
   * key is not written. */
  const int32_t* basis_of;
  int32_t n_basis;
  int32_t reserved2;
} dkv_pool;

/* One decode step's batch: one new query token per sequence. */
typedef struct dkv_batch {
  int32_t batch;             /* B >= 0 sequences */
  int32_t n_q_heads;         /* Hq, a multiple of n_kv_heads with Hq / Hkv <= 16 */
  int32_t window;            /* W: window rows allocated per (sequence, KV head) */
  int32_t max_blocks;        /* columns of block_table */
  const int32_t* block_table;/* int32 [B][max_blocks]: pool slot of logical block j */
  const int32_t* n_blocks;   /* int32 [B]: compressed blocks of each sequence (<= max_blocks) */
  const int32_t* win_len;    /* int32 [B]: valid window rows (<= W), or NULL for W everywhere */
  const void* q;             /* fp16 [B][Hq][d]: the decode queries (post-RoPE) */
  const void* win_k;         /* fp16 [B][Hkv][W][d]: exact recency window keys */
  const void* win_v;         /* fp16 [B][Hkv][W][d]: exact recency window values */
  const float* route_keys;   /* fp32 [B][Hkv][max_blocks][d]: routing key of logical block j
                                of each sequence (a copy of pool->route_key in block-table
                                order, see dkv_gather_route_keys), 16-byte aligned; or NULL to
                                read pool->route_key through block_table.  Routing then reads
                                each sequence's keys as one contiguous run, with no wait for
                                the block table.  Entries of invalid table slots are ignored. */
} dkv_batch;

/* Human-readable name of a status code (static string). */
const char* dkv_status_string(dkv_status status);

/* Detail of the last failing call on this thread (static thread-local buffer). */
const char* dkv_last_error(void);

/* DKV_ABI_VERSION of the built library. */
int32_t dkv_abi_version(void);

/* The rotary frequency table of an un-rotated pool, on the host: for
 * j < head_dim / 2, theta_j = base^(-2 j / head_dim) (the rotary embedding's
 * frequencies, computed in double precision) and f_j = theta_j / (2 pi), stored
 * as out[j] = (float) f_j and out[head_dim / 2 + j] = (float) (f_j - out[j]).
 * The caller copies the 2 * 64 floats to device memory for pool->rope_freq.
 *   base > 1; head_dim must be 128.  out: host float [2][head_dim / 2]. */
dkv_status dkv_rope_freqs(double base, int32_t head_dim, float* out);

/* Routing-key precompute, once per sealed block (off the per-query path).
 * Computes c = a_k + (1/255) sum_{i=1..255} U_i V_K in fp32 for every KV head of
 * the listed slots and stores it through pool->route_key (which must point to
 * writable memory).  The routing key is the block's centroid key, the mean of
 * its anchor-relative reconstructed rows 1..255 (all of them, residual
 * positions included); the pages keep such per-block router metadata (README,
 * "Per-Block Memory Breakdown", the decode-router row).  In an un-rotated
 * pool the key is the mean of those rows each rotated to its own position,
 * c = (1/255) sum_{i=1..255} rot(a_k + U_i V_K, slot_pos[s] + i).
 *   slots:   int32 [n_list] pool slots to process, or NULL for every slot
 *            (then n_list is ignored).  Out-of-range slots are skipped. */
dkv_status dkv_route_keys(const dkv_pool* pool, const int32_t* slots, int32_t n_list,
                          void* stream);

/* Per-sequence routing-key table for dkv_batch.route_keys:
 * out[b][h][j] = pool->route_key[block_table[b][j]][h] for j < n_blocks[b] and a
 * valid slot, zero otherwise.  Refresh a sequence's rows when its block table
 * changes (once per sealed block), like the block table itself.
 *   out: fp32 [B][Hkv][max_blocks][d], 16-byte aligned, caller-owned. */
dkv_status dkv_gather_route_keys(const dkv_pool* pool, const dkv_batch* batch, float* out,
                                 void* stream);

/* Top-K block routing (README "Key Environment Knobs": DKV_TOPK_BLOCKS,
 * DKV_CB_GQA_ROUTE head averaging, DKV_CB_ROUTE_ALL scoring of every block).
 * For each (sequence b, KV head h): q_bar = mean of the group's G query heads
 * (fp32), s_j = q_bar . c_j over all n_blocks[b] logical blocks, and the
 * K_eff = min(top_k, n_blocks[b]) largest scores are kept, ties going to the
 * lower logical block index.
 *   idx:    int32 [B][Hkv][top_k] out: chosen logical block indices, ascending,
 *           entries beyond K_eff set to -1.
 *   scores: fp32 [B][Hkv][top_k] out, or NULL: score of each chosen block in idx
 *           order (-inf for padding).
 * top_k >= 1; max_blocks <= DKV_MAX_ROUTE_BLOCKS. */
dkv_status dkv_route_topk(const dkv_pool* pool, const dkv_batch* batch, int32_t top_k,
                          int32_t* idx, float* scores, void* stream);

/* Partials layout shared by the attention entry points and dkv_lse_merge:
 * row r = b * Hq + head, part p:
 *   part_o  [n_rows][n_parts][d]  fp32, normalised (sum p v / sum p)
 *   part_lse[n_rows][n_parts]     fp32, log sum exp of the part's scaled scores
 * An entry point writes parts part_offset .. part_offset + (its count) - 1. */

/* Low-rank part of each routed block (README "Decode & Prefill Innovations":
 * low-rank space query scoring).  For routed block k of (b, h) it attends the
 * anchor row and the 255 reconstructed rows minus the residual positions:
 *   z_0 = scale q.a_k,  z_i = scale (q.a_k + U_i.(V_K q)),
 *   o = ((sum p) a_v + (p^T U) V_V) / sum p.
 * Writes top_k parts (k = 0..top_k-1); idx entries of -1 give empty parts.
 *   idx: int32 [B][Hkv][top_k] logical block indices (as from dkv_route_topk). */
dkv_status dkv_lowrank_attn(const dkv_pool* pool, const dkv_batch* batch, const int32_t* idx,
                            int32_t top_k, float scale, float* part_o, float* part_lse,
                            int32_t n_parts, int32_t part_offset, void* stream);

/* Exact attention (Zenodo abstract: residuals and the dense recency window are
 * attended exactly).  Writes top_k parts holding the R residual rows of routed
 * block k (only when idx != NULL; with idx == NULL top_k must be 0), then
 * window_splits parts: part s covers window rows [s c, min((s+1) c, win_len[b]))
 * with c = ceil(W / window_splits). */
dkv_status dkv_exact_attn(const dkv_pool* pool, const dkv_batch* batch, const int32_t* idx,
                          int32_t top_k, int32_t window_splits, float scale, float* part_o,
                          float* part_lse, int32_t n_parts, int32_t part_offset, void* stream);

/* Flash-style log-sum-exp combine (README "Decode & Prefill Innovations"):
 * for each of n_rows rows, M = max_p lse_p, lse = M + log sum_p exp(lse_p - M),
 * o = sum_p exp(lse_p - lse) o_p, summed in part order.
 *   out:     fp16 [n_rows][d] out;  out_lse: fp32 [n_rows] out.
 * head_dim must be 128. */
dkv_status dkv_lse_merge(const float* part_o, const float* part_lse, int32_t n_parts,
                         int32_t n_rows, int32_t head_dim, void* out, float* out_lse,
                         void* stream);

/* Bytes of workspace dkv_decode needs for this pool, batch and top_k (>= 0). */
size_t dkv_decode_workspace_size(const dkv_pool* pool, const dkv_batch* batch, int32_t top_k);

/* Prepare a dkv_decode workspace for first use: zeroes its control area (at
 * its start: 4 KB, plus 256 bytes per (sequence, KV head) unit, 4 bytes per
 * unit and routed block, and, when top_k > 0, 8 bytes per unit and
 * block-table entry) with a kernel on `stream` (no memset, so it may be captured
 * in a graph).  Not needed for memory that is already zero-filled.  Every
 * dkv_decode leaves the control area zeroed again, so a workspace is prepared
 * once and may then be reused by any number of calls (one at a time). */
dkv_status dkv_decode_workspace_init(const dkv_pool* pool, const dkv_batch* batch, int32_t top_k,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* One decode step of one layer in a single kernel launch: routing, low-rank +
 * residual attention of every routed block, window attention and the LSE
 * combine (the Zenodo abstract's decode path).  top_k = 0 attends the window
 * only.  Every (sequence, KV head) unit has its work items: score items, each
 * scoring 64 of its blocks against the GQA-mean query and writing (slot,
 * score) words to the workspace; then its parts, each of which attends its
 * share of the window, waits until all of the unit's words are written, ranks
 * the blocks itself (top_k by score, the lower block index first among equal
 * scores; the same ranking dkv_route_topk gives) and attends the routed block
 * at its own position; then one merge per query row, which waits until the
 * unit's parts are stored.  Workgroup w takes a fixed item: the units u with
 * u % 8 == x form list x (their score items, parts, merges, in that order) and
 * workgroup x + 8 i runs item i of list x, so every wait is on a workgroup of
 * a smaller index.  The last merge clears the words once every score item is
 * counted.
 *   workspace: device memory of >= dkv_decode_workspace_size() bytes, 256-byte
 *              aligned, owned by the caller, whose control area is zero (fresh
 *              zero-filled memory, dkv_decode_workspace_init, or a previous
 *              dkv_decode with the same or a larger-or-equal shape).  Calls
 *              that share a workspace must not overlap.  Word 2 of the
 *              workspace (uint32 at byte 8) is a sticky flag set if a part
 *              ever gave up waiting for its unit's scores, or the last merge
 *              for the score items (never in a correct run); word 3 counts
 *              launches.
 *   out:     fp16 [B][Hq][d] out;  out_lse: fp32 [B][Hq] out.
 *   out_idx: int32 [B][Hkv][top_k] out (the routed blocks), or NULL. */
dkv_status dkv_decode(const dkv_pool* pool, const dkv_batch* batch, int32_t top_k, float scale,
                      void* workspace, size_t workspace_bytes, void* out, float* out_lse,
                      int32_t* out_idx, void* stream);

/* dkv_decode with timing (the pages' DKV_PROFILE_CB knob, README "Key
 * Environment Knobs": GPU-kernel latency profiling).  Identical results;
 * additionally records the two caller-created hipEvent_t handles in `events`
 * on `stream`, [0] right before and [1] right after the decode kernel. */
dkv_status dkv_decode_profiled(const dkv_pool* pool, const dkv_batch* batch, int32_t top_k,
                               float scale, void* workspace, size_t workspace_bytes, void* out,
                               float* out_lse, int32_t* out_idx, void* const* events,
                               void* stream);

/* dkv_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same decode, with its workspace in a fixed device array of
 * dkv_decode_noalloc_max_bytes() bytes (16 MiB) that the library holds on
 * each GPU it runs on until the process ends.  The call allocates and frees
 * nothing; it clears the array's control area with a small kernel on
 * `stream`, then runs dkv_decode on it.  A decode whose
 * dkv_decode_workspace_size() exceeds the array returns DKV_ERR_WORKSPACE and
 * enqueues nothing.  All calls on one GPU share that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and must not be
 * made; consecutive calls on one stream are fine.  Arguments and results as
 * dkv_decode. */
dkv_status dkv_decode_noalloc(const dkv_pool* pool, const dkv_batch* batch, int32_t top_k, float scale,
                              void* out, float* out_lse, int32_t* out_idx, void* stream);
size_t dkv_decode_noalloc_max_bytes(void);

/* ---- Layer-batched decode -------------------------------------------------
 * The fused decode step (dkv_decode) of n_layers independent layers at once,
 * so that the layers' work shares the chip and the step streams the cache at
 * full bandwidth.  Use it when several layers' queries are at hand at once:
 * micro-batches in flight at different layers, or a model's layers evaluated
 * on given queries (a single token's layers depend on each other and cannot).
 * All layers share head_dim, block size, n_kv_heads and the batch shape
 * (batch, n_q_heads, window, max_blocks) and top_k; pools may differ in rank,
 * residual count and slot count.  The routed blocks are those of n_layers
 * dkv_decode calls; outputs equal dkv_decode's up to the rounding of another
 * split of the rows into partials, and repeat bit for bit from step to step.
 *
 * When every layer's pool qualifies (rotated keys, fp16 residual rows, rank a
 * multiple of 8 up to 56, residual count a multiple of 4, 16-byte aligned
 * arrays; plan->stream = 1), a step is three launches: the routings; the
 * streams, one-wave workgroups each running a contiguous segment of the step's
 * work (window rows, the low-rank parts and the residual rows of the routed
 * blocks; segments of about equal cost, fixed at prepare) through its own LDS
 * ring; and the log-sum-exp merges of each unit's partials.  Otherwise a step
 * is one launch whose routing, block-attention and merge items come from
 * per-XCD queues (the window in parts of its own; plan->group merge items per
 * unit).
 *
 * dkv_decode_layers_prepare (once; synchronous, not capturable in a graph)
 * validates every layer, writes the per-layer argument table into `table`
 * (device memory of dkv_decode_layers_table_size bytes, caller-owned), zeroes
 * the control words of `workspace` (device memory of
 * dkv_decode_layers_workspace_size bytes, 256-byte aligned, caller-owned),
 * writes the streams' schedule into it, and fills *plan.  dkv_decode_layers
 * (any number of times; asynchronous, may be captured) runs one step.  The
 * pools, batches, outputs, table and workspace given to prepare must keep
 * their addresses; their contents (e.g. the queries, window lengths, block
 * tables) may change between calls.  Calls sharing a workspace must not
 * overlap.  Word 2 of the workspace is the sticky wait-timeout flag (one
 * launch only).
 *   outs[l]: fp16 [B][Hq][d]; out_lses[l]: fp32 [B][Hq];
 *   out_idxs: NULL, or per layer int32 [B][Hkv][top_k] or NULL. */
typedef struct dkv_layers_plan {
  int32_t n_layers;
  int32_t n_units;        /* (sequence, KV head) units per layer */
  int32_t routes;         /* routing items per unit (0 or 1) */
  int32_t parts;          /* routed-block parts per unit */
  int32_t win_parts;      /* window parts per unit */
  int32_t group;          /* merge items per unit (1: one per unit) */
  int32_t n_items;        /* work items of one launch */
  int32_t lds_bytes;      /* dynamic LDS per workgroup */
  int32_t max_tiles;      /* largest 16-column low-rank tile count of the layers */
  int32_t quantised;      /* 1 if any layer's residual rows are quantised */
  int32_t unrotated;      /* 1 if the layers' pools are un-rotated (all of them or none) */
  int32_t stream;         /* 1: the streaming launches (every layer qualifies): the routings, then one
                             stream of window rows and routed blocks per wave, then the merges */
  int32_t stream_top_k;   /* streaming launches: routed blocks per unit */
  int32_t stream_items;   /* streaming launches: work items of the streams' schedule */
  int32_t stream_waves;   /* streaming launches: streams (one-wave workgroups) */
  int32_t stream_sched;   /* streaming launches: 32-bit word offset of the schedule in the workspace */
  const void* table;
  void* workspace;
} dkv_layers_plan;

size_t dkv_decode_layers_table_size(int32_t n_layers);
size_t dkv_decode_layers_workspace_size(const dkv_pool* pools, const dkv_batch* batches, int32_t n_layers,
                                        int32_t top_k);
dkv_status dkv_decode_layers_prepare(const dkv_pool* pools, const dkv_batch* batches, int32_t n_layers,
                                     int32_t top_k, float scale, void* const* outs, float* const* out_lses,
                                     int32_t* const* out_idxs, void* table, size_t table_bytes,
                                     void* workspace, size_t workspace_bytes, dkv_layers_plan* plan);
dkv_status dkv_decode_layers(const dkv_layers_plan* plan, void* stream);

/* dkv_decode_layers with timing (the pages' DKV_PROFILE_CB knob, README "Key
 * Environment Knobs": GPU-kernel latency profiling).  Identical results;
 * additionally records the four caller-created hipEvent_t handles in `events`
 * on `stream`: [0] before the step, [1] after the routings, [2] after the
 * streams, [3] after the merges (a one-launch step: [1] and [2] right before
 * [3], after its launch). */
dkv_status dkv_decode_layers_profiled(const dkv_layers_plan* plan, void* const* events, void* stream);

/* The streams' read ceiling: the loads dkv_decode_layers streams with (16-byte
 * buffer loads straight into a four-page LDS ring, one ring per one-wave
 * workgroup) over a plain array, as a measure of the box's streaming-read
 * bandwidth for them.  n_waves workgroups each read a contiguous 1/n_waves of
 * `src` (device memory, `bytes` a multiple of 4096 * n_waves, 16-byte
 * aligned) in pages of 4096 bytes, and write the 32-bit wrapping sum of their
 * share's 32-bit words to sink[w] (uint32, device memory).  Asynchronous on
 * `stream`.  DKV_ERR_INVALID_ARG for a size, alignment or count it cannot
 * take. */
dkv_status dkv_stream_read_probe(const void* src, size_t bytes, int32_t n_waves, uint32_t* sink, void* stream);

/* Block sealing, the write side of the cache (README "Core Architecture &
 * Paper Overview", items 1-3; "Content-Aware / Rarity-Aware Residual
 * Selection", the plain L2 selection; "Key Environment Knobs", DKV_SVD_SEED:
 * the SVD is randomised and seeded).
 * Block b (0 <= b < n_blocks), KV head h: its 256 keys and values, fp16 rows of
 * 128 (row stride 128), start at src_k.ptr + b * src_k.slot_stride +
 * h * src_k.head_stride (elements), likewise src_v.  The block is written into
 * pool slot slots[b] (device array; a slot outside [0, n_slots) skips it):
 *   anchor_k, anchor_v  row 0, exact;
 *   u, vk, vv           rank-r factors of A = [K[1:] - K[0] | V[1:] - V[0]]
 *                       (255 x 256): U = Q E_r S_r (singular values folded
 *                       in), [V_K | V_V] = W_r^T, fp16 (round to nearest even),
 *                       from the randomised subspace iteration Y = A omega,
 *                       Q = orth(Y), power_iters times Z = orth(A^T Q),
 *                       Q = orth(A Z), and the exact SVD B = Q^T A = E S W^T;
 *   resid_pos/k/v       the n_resid positions in 1..255 whose key is worst
 *                       reconstructed, |k_i - (a_k + U_{i-1} V_K)| from the
 *                       stored fp16 factors (fp32 arithmetic; equal errors to
 *                       the lower position), ascending, and their exact rows:
 *                       fp16, or in the pool's 8- / 4-bit format (README
 *                       "2. Physical 4-Bit Group-Quantized Residual Buffers
 *                       (INT4)", "Tunable Quantization Dials"): per row and
 *                       group of 64 dims, bias = the smallest value, scale =
 *                       (largest - smallest) / L in fp32 rounded up to fp16,
 *                       code = round((x - bias) / scale) in fp32, ties to
 *                       even, clamped to [0, L] (L = 255 or 15; 0 for a zero
 *                       scale), into resid_k / resid_v and resid_k_sb /
 *                       resid_v_sb;
 *   route_key           as dkv_route_keys, if pool->route_key.ptr is set.
 *   omega: fp32 [256][width], the Gaussian test matrix (the caller's seeded
 *          draw); rank <= width <= 80 (DKV_ERR_UNSUPPORTED above 80);
 *   power_iters: 0..8.
 * Sources: 16-byte aligned pointers and strides; residual rows likewise.
 * Source rows and the pool slots written must not overlap, nor two entries of
 * slots name the same slot.  Asynchronous on `stream`. */
dkv_status dkv_seal_blocks(const dkv_pool* pool, dkv_view src_k, dkv_view src_v, const int32_t* slots,
                           int32_t n_blocks, const float* omega, int32_t width, int32_t power_iters,
                           void* stream);

/* Join blocks to a shared basis: the write side of DKV_SHARED_BASIS (README
 * "Key Environment Knobs" and "3. Shared Low-Rank Bases": a joined block reads
 * the group's basis, keeping the part of its delta the group's subspace can
 * express; joins are judged by the retained energy).  For item i, block slot
 * s = slots[i] (current basis entry cur = basis_of[s], or s without sharing)
 * and target entry g = entries[i], per KV head h, with V = [V_K | V_V]:
 *   M = V_cur V_g^T,  U' = U M (V_g V_g^T)^-1  (the least-squares solution of
 *   U' V_g = U V_cur; U M when the rows of V_g are orthonormal, as the sealer
 *   writes them),  energy[i * n_kv_heads + h] = |U' V_g|^2 / |U V_cur|^2,
 * fp32 from the fp16 arrays; V_g V_g^T is factored by Cholesky, and a pivot
 * below 1e-6 of its largest diagonal drops that direction (rows of V_g are
 * meant to be linearly independent).  write != 0 stores U' into slot s's U
 * (fp16, round to nearest even); write = 0 only scores the candidate.  The
 * caller then sets basis_of[s] = g (its own array) and recomputes the routing
 * key (dkv_route_keys).  Entries index vk / vv: [0, n_basis) with basis_of set,
 * else [0, n_slots).  An item with a slot or entry out of range writes energy
 * -1 and changes nothing.  With write != 0, slots of one call must be
 * distinct (scoring one slot against several entries may repeat it).
 *   slots, entries: int32 [n] device;  energy: fp32 [n][n_kv_heads] device out. */
dkv_status dkv_join_basis(const dkv_pool* pool, const int32_t* slots, const int32_t* entries, int32_t n,
                          int32_t write, float* energy, void* stream);

/* Shared bases under a budget (README "Key Environment Knobs", DKV_SHARED_BASIS
 * and DKV_SHARED_BASIS_FRAC: a basis store of a capacity fixed as a fraction
 * of the block slots; "3. Shared Low-Rank Bases": voluntary joins when the
 * retained energy is high enough, forced joins once the store is full).
 * `pool` holds each block's own basis (basis_of NULL), e.g. as dkv_seal_blocks
 * wrote it.  The blocks in slots[0 .. n) (host array, distinct slots) are taken
 * in that order; block i is scored (dkv_join_basis) against the basis of the
 * block that opened each entry so far, its energy for an entry being the mean
 * over the KV heads, and with the best entry (largest energy, ties to the
 * lower entry):
 *   - energy >= threshold: a voluntary join (kind 1);
 *   - else, while fewer than `capacity` entries are open: block i opens a new
 *     entry with its own basis (kind 0, energy 1);
 *   - else: a forced join to the best entry (kind 2).
 * A join writes U' into the block's U (dkv_join_basis, write = 1).  At the
 * end entry j of the store (store_vk, store_vv: device views like pool's vk,
 * vv, at least min(capacity, n) entries) holds the basis of the block that
 * opened it.  Host outputs: entry[n] (the store entry each block reads),
 * opener[min(capacity, n)] (the slot that opened each entry), energy[n],
 * kind[n], *n_entries.  The caller then reads the blocks through the store:
 * basis_of[slots[i]] = entry[i], vk / vv = the store, n_basis = *n_entries, and
 * recomputes their routing keys (dkv_route_keys).  Synchronous on `stream`
 * (energies come back to the host after each block; the decisions are made
 * on the host in fp32); allocates a little device memory for the call. */
dkv_status dkv_share_bases(const dkv_pool* pool, const int32_t* slots, int32_t n, int32_t capacity, float threshold,
                           dkv_view store_vk, dkv_view store_vv, int32_t* entry, int32_t* opener, float* energy,
                           int32_t* kind, int32_t* n_entries, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DKV_ATTN_H */
