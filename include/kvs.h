/*
 * kvs.h - host-streamed, paged flash-attention over a Q8_0-K / Q4_0-V (or Q8_0-V) cache
 *         (C ABI of libkvs.so, built for AMD MI355X / gfx950).
 *
 * The method (three pages on "Adaptive KV Streaming" for llama.cpp):
 *   - The authoritative KV history lives in pinned host memory; the device holds
 *     a bounded working set of resident pages plus one transfer ring shared by
 *     all layers, and flash-attention consumes both (page 1, "Summary"; page 2,
 *     opening paragraph).
 *   - The unit of residency and transfer is a 256-token page of one layer
 *     (page 2, "Dynamic draft eject": thresholds counted in 256-token pages).
 *   - The cache types are Q8_0 for K and Q4_0 for V (page 1, "What it is useful
 *     for"; page 2, "TLDR": the q8_0-q4_0 kernel pair), or Q8_0 for both
 *     (page 3, "1. Correctness - PPL parity" runs -ctk q8_0 -ctv q8_0).
 *   - A byte budget sizes the device region; the smallest useful budget is one
 *     page (page 3, "Diagnostic log": minimum_stage_bytes).
 *   - Unsupported K/V type pairs and over-wide batches fail with an explicit
 *     error instead of silently doing something else (page 1, "How engineers
 *     can use it": explicit capability errors; page 2, "Phase arena:
 *     speculative verify batches": batches wider than
 *     max(n_seq_max, 1 + n_max_spec_draft) are rejected).
 *
 * Conventions for every call:
 *   - Return 0 (KVS_OK) on success or a negative KVS_ERR_* code. Nothing
 *     throws across this boundary. On error the pool's state is unchanged and
 *     kvs_last_error() describes the failure (thread-local string).
 *   - Device pointers are plain HIP device addresses; host pointers are plain
 *     process addresses; streams are hipStream_t handles passed as void*.
 *   - The caller owns every buffer it passes: the device arena, the pinned host
 *     page records, q, out, lse and the compute streams. The library owns only
 *     its metadata, its HIP events and its own streams (a prefetch stream and
 *     three compute lanes, created at the default priority), and never frees
 *     caller memory.
 *   - Calls on one pool may use different streams: each call that launches
 *     work first makes its stream wait for the pool's previous work (the
 *     split-K workspace and ring are shared by every layer).
 *     Inside a HIP graph capture that wait is skipped, so a captured sequence
 *     must issue all of its calls on the capture stream.
 *   - A HIP runtime failure after a call has started device work marks the
 *     pool unusable: that call and every later one return KVS_ERR_HIP.
 *   - A pool is bound to the HIP device that is current when it is created;
 *     later calls must be made with that device current.
 *
 * Page record format (one record per layer and page, page_bytes long):
 *   [ K: for kv head g = 0..Hkv-1, token row r = 0..255, block b = 0..d/32-1:
 *        a Q8_0 block of 34 bytes ]
 *   [ V: same order, Q4_0 blocks of 18 bytes (type_v KVS_TYPE_Q4_0) or Q8_0
 *        blocks of 34 bytes (type_v KVS_TYPE_Q8_0) ]
 *   Q8_0 block: little-endian binary16 scale d, then 32 int8 codes q;
 *               element i = d * q[i].
 *   Q4_0 block: little-endian binary16 scale d, then 16 bytes; byte j holds
 *               element j in its low nibble and element j + 16 in its high
 *               nibble; element i = d * (nibble - 8).
 *   Token t of a layer lives in page t / 256, row t % 256. Each kv head's K tile
 *   (256 x d/32 x 34 bytes) and V tile (256 x d/32 x 18 or 34 bytes) is
 *   contiguous, so one workgroup reads one head of one page as two line-aligned
 *   streams. For Hkv = 4, d = 128: K row 136 B per head, page_bytes = 212992
 *   (Q4_0 V) or 278528 (Q8_0 V).
 *   Rows at or beyond the layer's token count may hold any bytes (even NaN
 *   scales); they are never read into a result.
 */
#ifndef KVS_H
#define KVS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Block types, numbered as in ggml's type enumeration. */
#define KVS_TYPE_F16  1
#define KVS_TYPE_Q4_0 2
#define KVS_TYPE_Q8_0 8

/* Query element types for kvs_attend. */
#define KVS_Q_F32 0
#define KVS_Q_F16 1

/* Error codes. */
#define KVS_OK                  0
#define KVS_ERR_INVALID_ARG    -1  /* null pointer, out-of-range size or index        */
#define KVS_ERR_UNSUPPORTED    -2  /* type pair, head_dim, page size, unpinned memory */
#define KVS_ERR_BUDGET         -3  /* budget below kvs_min_budget_bytes               */
#define KVS_ERR_NO_SLOTS       -4  /* more resident pages than free device slots      */
#define KVS_ERR_BATCH_TOO_WIDE -5  /* n_q above max_q_tokens                          */
#define KVS_ERR_NOT_READY      -6  /* host pages or page table of the layer unset     */
#define KVS_ERR_STATE          -7  /* ring already lent to another layer's prefetch   */
#define KVS_ERR_NOT_RESIDENT   -8  /* kvs_debug_read_page on a streamed page          */
#define KVS_ERR_HIP            -9  /* a HIP runtime call failed                       */

/* kvs_config.flags */
#define KVS_FLAG_POISON_RING 1u    /* debug: fill each ring chunk with 0xA5 after its
                                      kernel, before the slot is reused             */
#define KVS_FLAG_ZERO_COPY   2u    /* streamed pages are read in place from their pinned
                                      host records by the attention kernels (mapped
                                      host memory over the link, no ring copies): the
                                      A/B against the ring. The ring is unused,
                                      kvs_stream_enqueue is a no-op, and a streamed
                                      layer may be captured in a HIP graph. Outputs
                                      equal the ring's bit for bit. */

typedef struct kvs_config {
    int32_t n_layers;      /* layers sharing the pool and the ring (>= 1)                 */
    int32_t n_kv_heads;    /* Hkv (1..64)                                                 */
    int32_t n_q_heads;     /* Hq, a multiple of Hkv; query head h reads kv head h/(Hq/Hkv) */
    int32_t head_dim;      /* d; 128 is the only supported value                          */
    int32_t page_tokens;   /* 256 is the only supported value                             */
    int32_t type_k;        /* KVS_TYPE_Q8_0                                                */
    int32_t type_v;        /* KVS_TYPE_Q4_0 or KVS_TYPE_Q8_0                               */
    int32_t max_pages;     /* most pages any layer will hold (sizes tables and workspace) */
    int32_t max_q_tokens;  /* widest query block kvs_attend admits: 1 for decode,
                              1 + n_draft for a speculative verify, the ubatch for prefill */
    int32_t ring_pages;    /* device ring capacity in pages (>= 1)                        */
    int32_t chunk_pages;   /* pages per ring chunk (1..16), a divisor of ring_pages: one
                              launch computes a chunk while its copy workgroups pull a
                              later chunk from host memory into a free chunk slot. A
                              chunk holds whole split-K groups when group_pages <=
                              chunk_pages (so it may carry fewer pages); only then can
                              two chunk launches run concurrently                      */
    int32_t group_pages;   /* pages per split-K partial (>= 1). Partials are keyed by this
                              logical grouping only, so results do not depend on which
                              pages are resident, nor on ring or chunk sizes.              */
    uint32_t flags;        /* KVS_FLAG_*                                                   */
} kvs_config;

typedef struct kvs_status_info {
    int64_t page_bytes;          /* bytes of one page record                         */
    int64_t slot_count;          /* resident page slots carved from the arena        */
    int64_t slots_used;          /* slots holding a resident page                    */
    int64_t ring_pages;          /* ring capacity in pages                           */
    int64_t workspace_bytes;     /* split-K partial workspace carved from the arena  */
    int64_t bytes_h2d;           /* bytes copied host->device through the ring       */
    int64_t pages_streamed;      /* pages copied through the ring                    */
    int64_t copies_issued;       /* ring chunk refills issued (each carried by a launch's
                                    copy workgroups, or a prefetch's copy-only launch) */
    int64_t kernels_launched;    /* kernel launches issued by kvs_attend/debug calls */
    int64_t resident_upload_bytes; /* bytes copied into resident slots              */
    int64_t pinned_slots;        /* slots held by pinned regions (kvs_pool_pin_layer) */
} kvs_status_info;

typedef struct kvs_pool kvs_pool;

/* 1 if the K/V block type pair has a kernel (Q8_0 K with Q4_0 or Q8_0 V), else 0.
 * Pure: no HIP call. The pages compile flash-attention per K/V type pair and
 * reject unqualified pairs (page 2, "TLDR"; page 1, "How engineers can use it"). */
int kvs_type_pair_supported(int32_t type_k, int32_t type_v);

/* Validate a configuration without touching the GPU. Returns KVS_OK,
 * KVS_ERR_INVALID_ARG or KVS_ERR_UNSUPPORTED. Pure. */
int kvs_config_validate(const kvs_config* cfg);

/* Bytes of one page record for cfg. Pure; 0 on an invalid config. */
uint64_t kvs_page_bytes(const kvs_config* cfg);

/* Smallest budget kvs_pool_create accepts for cfg, written to *out: the ring,
 * the split-K workspace (max_q_tokens x n_q_heads rows per page group) and
 * the per-layer tables, each rounded up to 256 bytes. Pure. */
int kvs_min_budget_bytes(const kvs_config* cfg, uint64_t* out);

/* Number of resident page slots a budget yields for cfg (0 if below the
 * minimum), at most 2^23 - 1 (slot indices travel in 24 bits of the launch
 * plan). A pool created with the same budget has this many slots. Pure. */
int64_t kvs_slots_for_budget(const kvs_config* cfg, uint64_t budget_bytes);

/* Pool policy: automatic sizing and the newest-page residency rule.
 *
 * The pages size the device stage from the context alone when asked for
 * "auto" (page 3, description: 10 % of the context resident per layer, a
 * 2048-token floor and an 8192 MiB ceiling; its diagnostic logs print the
 * resident tokens per layer and the stage for 64 Ki and 256 Ki contexts).
 *
 * kvs_auto_resident_pages: resident pages per layer for a context of n_ctx
 *   tokens: ceil(0.1 n_ctx) rounded up to whole 256-token pages (10 % of
 *   65536 gives 26 pages = 6656 tokens, of 262144 gives 103 = 26368, as
 *   logged), at least 2048 tokens (8 pages), at most the context's own pages.
 *   0 for n_ctx <= 0. Pure.
 * kvs_auto_stage_bytes: the pages' stage size for n_layers streamed layers of
 *   bytes_per_token bytes per token and layer: n_layers x (resident pages + 4)
 *   x 256 x bytes_per_token, capped at 8192 MiB (reproduces the logged 255 MiB
 *   at 64 Ki and 910 MiB at 256 Ki for 2176 B q8_0/q8_0 tokens). Pure; 0 on
 *   non-positive arguments.
 * kvs_auto_budget_bytes: this pool's budget for the same residency: the
 *   minimum budget of cfg plus n_layers x resident pages x page_bytes, capped
 *   at 8192 MiB (never below the minimum). Written to *out. Pure. */
int32_t kvs_auto_resident_pages(int64_t n_ctx);
uint64_t kvs_auto_stage_bytes(int32_t n_layers, int64_t n_ctx, uint64_t bytes_per_token);
int kvs_auto_budget_bytes(const kvs_config* cfg, int64_t n_ctx, uint64_t* out);

/* Residency as a context grows: the device window follows the newest tokens
 * (page 2, "Dynamic draft eject": the draft's KV slides to follow the
 * target's decode window). Given the current mask of
 * n_cur pages and a layer that now has n_new >= n_cur pages, write the mask
 * of n_new pages to out. Each new page, in order, becomes resident; then,
 * while more than max_resident pages are resident, the oldest resident page
 * is streamed (max_resident = 0: new pages stay streamed). Pages that were
 * streamed stay streamed; n_new == n_cur copies the mask. out may alias cur.
 * Pure. */
int kvs_residency_promote_newest(const uint8_t* cur, int32_t n_cur, int32_t n_new, int32_t max_resident,
                                 uint8_t* out);

/* The launch plan kvs_page_table_set would build for one layer of n_pages
 * pages with the given residency (resident[i] != 0: page i resident). Pure
 * host computation, no device needed; for inspection and tests.
 *
 * Split-K groups are runs of group_pages logical pages (page 2, "Phase arena:
 * speculative verify batches": a verify batch attends the whole cache; the
 * grouping is this library's, fixed by page index so results do not depend on
 * residency). Groups with no streamed page form the resident launch; the
 * streamed pages, in ascending order, are cut into ring chunks of at most
 * chunk_pages pages, each chunk launch also computing the resident pages of
 * the groups it finishes.
 *
 * Outputs: *info (required); if segs is not NULL, segment i is written to
 * segs[4i .. 4i+3] = {group, first page, pages, flags (1 = starts its group)},
 * resident launch first; if chunks is not NULL, chunk c is written to
 * chunks[4c .. 4c+3] = {first streamed rank, pages, first segment, segments}.
 * KVS_ERR_INVALID_ARG if a capacity is too small or an argument is invalid. */
typedef struct kvs_plan_info {
    int32_t n_groups;         /* split-K groups of the layer                       */
    int32_t n_streamed;       /* pages not resident                                */
    int32_t n_segs;           /* segments over all launches                        */
    int32_t n_resident_segs;  /* segments of the resident launch                   */
    int32_t n_chunks;         /* ring chunk launches                               */
    int32_t whole_groups;     /* 1 if no group spans two launches (then chunk
                                 launches may run on two streams at once)          */
} kvs_plan_info;
int kvs_plan_layer(const kvs_config* cfg, int32_t n_pages, const uint8_t* resident, kvs_plan_info* info,
                   int32_t* segs, int32_t seg_cap, int32_t* chunks, int32_t chunk_cap);

/* Create a pool that carves [ring | workspace | tables | resident slots] out
 * of the caller's device arena of budget_bytes bytes (256-byte aligned): one
 * bounded device region holds the resident pages and the one
 * transfer ring all layers share (page 1, "Summary"; page 2, opening
 * paragraph), sized by a byte budget whose least useful value is one page
 * (page 3, "Diagnostic log": minimum_stage_bytes). KVS_ERR_BUDGET below
 * kvs_min_budget_bytes. The library never allocates device memory; the arena
 * must outlive the pool. Creates the pool's streams and events on the current
 * device. */
int kvs_pool_create(const kvs_config* cfg, void* dev_arena, uint64_t budget_bytes,
                    kvs_pool** out_pool);

/* Wait for every copy the pool issued, then release its events, streams and
 * metadata. Never frees caller memory. Safe on NULL. */
void kvs_pool_destroy(kvs_pool* pool);

/* Register the authoritative host records of a layer: n_pages records of
 * page_bytes each, contiguous, in pinned host memory (hipHostMalloc or an
 * equivalent page-locked allocation; anything else is KVS_ERR_UNSUPPORTED).
 * The library writes them only through kvs_append; they must stay valid, and
 * the caller must not change them, while work that reads them is in flight. */
int kvs_host_pages_set(kvs_pool* pool, int32_t layer, const void* pinned_records,
                       int32_t n_pages);

/* Set which pages of a layer are resident (resident[p] = 1) for a layer of
 * n_pages pages (n_pages <= max_pages and <= the registered host pages): the
 * page table mapping each logical page to a device slot or to its host record
 * (the pages' working set of resident pages; page 3's review notes its
 * variant had no such table). Builds the layer's launch plan (resident
 * groups, ring chunks, copy runs), uploads the plan and the records of newly
 * resident pages on `stream` (after the pool's earlier work), and waits for
 * that stream. Pages that stay resident keep their slot and its contents
 * (kvs_append keeps slots and records in step); after kvs_host_pages_set
 * registers the layer's records again, every resident page is uploaded.
 * A growing layer calls this with its new page count, typically with
 * kvs_residency_promote_newest's mask. A pinned layer (kvs_pool_pin_layer)
 * takes slots from its own region only. KVS_ERR_NO_SLOTS if too few slots are
 * free; every validation error leaves the pool unchanged. */
int kvs_page_table_set(kvs_pool* pool, int32_t layer, int32_t n_pages,
                       const uint8_t* resident, void* stream);

/* Start copying the first ring chunk of `layer` over the host link on the
 * pool's prefetch stream (after the previous ring reader finished), so it
 * overlaps whatever the caller runs before kvs_attend(layer): the pages
 * overlap transfers of non-resident pages with compute (page 1, "Summary";
 * page 2, opening paragraph). The ring serves one layer at a time,
 * in call order: KVS_ERR_STATE if another layer's prefetch has not been
 * consumed yet. A layer with no streamed pages is a no-op. Without a prefetch,
 * kvs_attend copies the first chunk itself. */
int kvs_stream_enqueue(kvs_pool* pool, int32_t layer);

/* Attention of n_q query tokens against the layer's cache of n_kv tokens:
 * flash-attention over the resident pages and, through the ring, the
 * streamed ones (page 1, "Summary"), for a decode token, a speculative-verify
 * block of 1 + draft tokens (page 2, "Phase arena: speculative verify
 * batches") or a prefill ubatch (page 2, "TLDR - recommended setup"). The
 * result is the plain softmax attention of the dequantized cache, whichever
 * pages are resident (page 3, "KLD": streaming runs the same math).
 *   q:    device, [n_q, n_q_heads, head_dim], f32 or f16 (q_dtype), contiguous.
 *   out:  device, [n_q, n_q_heads, head_dim] f32; lse: device [n_q, n_q_heads]
 *         f32 natural-log sum-exp of the scaled scores, or NULL.
 *   Query i sits at position q_pos0 + i and reads keys t < n_kv, and with
 *   causal != 0 only t <= q_pos0 + i (then q_pos0 >= 0 and q_pos0 + n_q <= n_kv
 *   are required). n_kv must satisfy ceil(n_kv / 256) == the layer's n_pages.
 *   Scores are scale * q.k. A row without any allowed key gets out = 0 and
 *   lse = -inf.
 * Supported inputs and accuracy (outputs within 2e-3 of float64 attention,
 * normwise per row: max_c |o - r| / max_c |r|):
 *   - K blocks: any finite binary16 scale (subnormals, zero, negative, up to
 *     65504) and any codes (-128 included). Scores are float32 sums of exact
 *     products: the codes enter the matrix cores exactly and each block's
 *     scale multiplies its product in float32.
 *   - q: finite f32 or f16. Decode-width blocks (n_q x Hq / Hkv <= 6) hold
 *     each query row as 16-bit fixed point relative to its largest element;
 *     wider blocks hold it exactly as f16 limbs (two for f32) after a
 *     power-of-two scaling per row.
 *   - V blocks: any finite binary16 scale, nibbles 0..15 (Q4_0) or any codes
 *     (Q8_0, -128 included). Probabilities and V values pass through f16 with
 *     one rounding each; at widths above decode, a page (verify widths) or
 *     a 64-token sub-block (prefill widths, more than 64 rows per kv head)
 *     whose 32-channel V block holds a scale magnitude above 8188 (Q4_0) or
 *     511.75 (Q8_0) is taken divided by 8 (Q4_0) or 128 (Q8_0), so that no V
 *     operand overflows f16. Within one such range and one 32-channel block,
 *     V scale magnitudes should lie within a factor of 2^14 of the block's
 *     largest: the contribution of a token whose scale is smaller than that
 *     (relative to the largest, in the same quarter page at decode width)
 *     carries an absolute error up to 2^-24 of the largest scale.
 * Enqueues the resident-group launch, then one launch per ring chunk, then
 * the split-K combine on `stream`; with several ring chunks the chunk
 * launches go to up to three compute lanes (the pool's own streams, forked
 * from and joined back to `stream` by events). Each chunk launch computes on
 * a chunk an earlier launch of its lane copied into the ring, while its own
 * copy workgroups read a later chunk's pages from pinned host memory over the
 * host link into a ring slot of the same lane; kernel boundaries on a lane
 * order each copy before its reader and each reader before the slot is
 * refilled. Returns without waiting. KVS_ERR_BATCH_TOO_WIDE if n_q exceeds
 * max_q_tokens (the pages' "decode batch too wide").
 * A layer whose pages are all resident, or any layer of a zero-copy pool,
 * may be captured into a HIP graph (stream capture on `stream`) and
 * replayed; a layer that streams pages through the ring returns
 * KVS_ERR_UNSUPPORTED under capture, because its ring chunks are ordered by
 * events on the pool's lanes. */
int kvs_attend(kvs_pool* pool, int32_t layer, const void* q, int32_t q_dtype, int32_t n_q,
               int64_t q_pos0, int64_t n_kv, float scale, int32_t causal, float* out,
               float* lse, void* stream);

/* kvs_attend for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results (bit for bit), but the split-K partial records
 * live in a fixed array of KVS_NOALLOC_SCRATCH_BYTES in the library's own
 * device memory instead of the pool's workspace, and the call creates
 * nothing (no timing events either: kvs_profile_enable does not apply). It
 * needs n_groups x n_q x n_q_heads x 130 x 4 bytes of that array, where
 * n_groups = ceil(n_pages / group_pages) of the layer; a call needing more
 * returns KVS_ERR_INVALID_ARG before any device work. Every call on a GPU,
 * from any pool, shares that GPU's one array, which keeps the last call's
 * contents (nothing in it needs clearing: every group's first launch starts
 * its record afresh). Calls of one pool are ordered like kvs_attend's; calls
 * of different pools that overlap in time on one GPU race on the array. */
#define KVS_NOALLOC_SCRATCH_BYTES (4u << 20)
int kvs_attend_noalloc(kvs_pool* pool, int32_t layer, const void* q, int32_t q_dtype, int32_t n_q,
                       int64_t q_pos0, int64_t n_kv, float scale, int32_t causal, float* out, float* lse,
                       void* stream);

/* Append a step's new K and V rows to a layer: quantize them into Q8_0 (K)
 * and Q4_0 or Q8_0 (V, the pool's type_v) blocks and write them at tokens pos0 .. pos0 + n_tok - 1 of
 * the layer, into the authoritative host records and, for each resident page,
 * into its device slot. The pages keep the whole history in pinned host
 * memory and a working set on the device (page 1, "Summary"; page 2, opening
 * paragraph), so every new row reaches the host record; a streamed page is
 * read from there by the next ring copy.
 *   k_new, v_new: device, [n_tok, n_kv_heads, head_dim], f32 or f16 (dtype
 *     KVS_Q_F32 / KVS_Q_F16), contiguous, 16-byte aligned, finite; a block's
 *     largest magnitude is 0 or at least 2^-100.
 *   The tokens must lie in the layer's pages (pos0 >= 0, pos0 + n_tok <=
 *     256 * n_pages of its page table); grow the table with
 *     kvs_page_table_set before appending into a new page. n_tok = 0 is a
 *     no-op.
 *   Block rule (ggml's reference quantizers, float32, scale stored as the
 *     nearest binary16): Q8_0 d = max|x| / 127, code = x / d rounded half away
 *     from zero; Q4_0 d = (first element of largest magnitude) / -8,
 *     nibble = min(15, trunc(x / d + 8.5)).
 * Enqueues one kernel on `stream` and returns without waiting. Later
 * attention, gathers and prefetches of any layer wait for it. KVS_ERR_STATE
 * if a prefetch of this layer (kvs_stream_enqueue) is pending and a target
 * page is streamed: that prefetch may be reading the record. */
int kvs_append(kvs_pool* pool, int32_t layer, const void* k_new, const void* v_new, int32_t dtype,
               int64_t pos0, int32_t n_tok, void* stream);

/* Pinned region (page 2, "New arena and context API": a pinned region
 * bump-allocated from the top of the arena, the rest of the pool below it;
 * page 1, "Summary": the draft head's KV is one more logical attention layer
 * that borrows the same physical pool). kvs_pool_pin_layer reserves the
 * n_slots highest free slots below any earlier pinned region for `layer`
 * alone: its page table takes slots only from there (at most n_slots
 * resident pages, e.g. a newest-page window from
 * kvs_residency_promote_newest), and no other layer can take them. The
 * layer must hold no resident slot (set an empty page table first), and the
 * slots being reserved must be free: KVS_ERR_STATE or KVS_ERR_NO_SLOTS
 * otherwise. kvs_pool_reset_pinned returns every pinned region to the pool
 * (page 2's draft eject returns the draft's KV to the arena); each pinned
 * layer must first hold no resident page (KVS_ERR_STATE). Host-only. */
int kvs_pool_pin_layer(kvs_pool* pool, int32_t layer, int32_t n_slots);
int kvs_pool_reset_pinned(kvs_pool* pool);

/* Counters and sizes of the pool. */
int kvs_status(const kvs_pool* pool, kvs_status_info* info);

/* Dequantize tokens tok0 .. tok0 + n_tok - 1 of a layer into float32
 * k_out / v_out (device, [n_tok, n_kv_heads, head_dim]) through the same page
 * table, ring pipeline and block decode the attention kernels use. Streamed
 * pages travel through the ring. Dequantization is exact in float32. */
int kvs_debug_gather(kvs_pool* pool, int32_t layer, int64_t tok0, int64_t n_tok, float* k_out,
                     float* v_out, void* stream);

/* Copy the bytes of a resident page's device slot to dst_host (page_bytes).
 * Synchronous. KVS_ERR_NOT_RESIDENT for a streamed page. */
int kvs_debug_read_page(kvs_pool* pool, int32_t layer, int32_t page, void* dst_host);

/* Raw bytes of every page record of a layer as the attention kernels read
 * them, copied to dst (device, n_pages x page_bytes, 16-byte aligned): a
 * resident page from its slot, a streamed page from the ring chunk it was
 * copied into during this call's pass over the layer (or in place from its
 * pinned record in a zero-copy pool). Runs the layer's ring pipeline like
 * kvs_attend; enqueued on `stream`. */
int kvs_debug_export_pages(kvs_pool* pool, int32_t layer, void* dst, void* stream);

/* The matrix-core operands of every page of a layer, converted by the same
 * code the prefill kernel runs on each 64-token sub-block (query blocks wider
 * than 64 rows per kv head), written to dst (device, 256-byte aligned) as
 * n_pages x n_kv_heads tiles of KVS_STAGED_TILE_BYTES, tile (page, kv head)
 * at (page x n_kv_heads + head) x KVS_STAGED_TILE_BYTES. n_kv is the layer's
 * token count (rows at or past it are not cached). Streamed pages pass through
 * the ring. Enqueued on `stream`. Tile layout (binary16 little-endian):
 *   K operands, bytes [0, 65536): for token tile T = 0..15, block b = 0..3,
 *     lane = 0..63: 8 values; lane (n, j) = (lane % 16, lane / 16) holds the
 *     codes of token 16 T + n, elements 32 b + 8 j .. 32 b + 8 j + 7, exact.
 *   V^T operands, bytes [65536, 131072): for chunk c = 0..7, channel tile
 *     t = 0..7, lane = 0..63: 8 values; lane (n, j) holds channel
 *     16 t + n (element 16 (t % 2) + n of block t / 2: the low nibbles of a
 *     Q4_0 block for even t, its high nibbles for odd t) of tokens
 *     32 c + 4 j + s for slot s < 4 and 32 c + 12 + 4 j + s for s >= 4, each
 *     d x (nibble - 8) (Q4_0) or d x code (Q8_0), divided by 2^shift and
 *     rounded once to binary16 (0 for uncached rows), shift = the V shift of
 *     the token's 64-token sub-block (c / 2) and the channel's block.
 *   K scales, bytes [131072, 135168): token t's four block scales as
 *     float32 (exact) at 16 t.
 *   V shifts, bytes [135168, 135232): int32 at 4 (4 s + b) for sub-block
 *     s = 0..3 (tokens 64 s .. 64 s + 63) and block b: 0, or, if a cached row
 *     of the sub-block has a block b scale magnitude above 8188 (binary16 bits
 *     above 0x6FFF) for Q4_0 V or 511.75 (bits above 0x5FFF) for Q8_0 V, 3
 *     (Q4_0) or 7 (Q8_0). */
#define KVS_STAGED_TILE_BYTES 135424
int kvs_debug_stage(kvs_pool* pool, int32_t layer, int64_t n_kv, void* dst, void* stream);

/* Kernel timing. With enable != 0, kvs_attend brackets every attention kernel
 * launch (kind 0) and every split-K combine launch (kind 1) with a start/stop
 * event pair carried by the kernel's own dispatch (so the time is the
 * kernel's execution, not its queueing); launches under graph capture are not
 * timed. Attention launches on several compute lanes overlap, so their summed
 * time can exceed the wall time of a call. kvs_profile_read waits
 * for the recorded events and returns the number of timed launches of that
 * kind and their summed duration in milliseconds; reset != 0 clears the
 * record. At most 65536 launches per kind are kept (later ones are not timed). */
int kvs_profile_enable(kvs_pool* pool, int32_t enable);
int kvs_profile_read(kvs_pool* pool, int32_t kind, int64_t* launches, double* total_ms, int32_t reset);

/* Message of the last failing call on this thread ("" if none). */
const char* kvs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVS_H */
