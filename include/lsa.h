/*
 * lsa.h -- C interface of the Lookahead Sparse Attention (LSA) decode path,
 * hand-written HIP for AMD Instinct MI355X (gfx950).
 *
 * The method (pages on "FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long
 * Context via Lookahead Sparse Attention"; the zhichai.net explainer, section 2
 * "Core Idea of LSA", gives the loop as five steps):
 *   every tau = 64 decode steps a Query Encoder projects the current hidden
 *   state, three independent indexers score every 64-token KV block against
 *   frozen precomputed block keys (KIComp), blocks whose sigmoid score is above
 *   0.5 are selected, the three selections are OR-unioned, the selected blocks
 *   are moved from a host-memory cold pool into GPU memory, and the next 64
 *   decode steps attend over those blocks plus the recent local window.
 *
 * Three calls carry the loop:
 *   lsa_index_refresh   score, threshold, OR-union and compact (device, async)
 *   lsa_gather_blocks   make one request's hot pool hold a new selection
 *                       (host planning + one copy kernel, async); the _batch
 *                       form does it for the requests of one refresh at once
 *   lsa_sparse_decode   one decode step over window + loaded blocks (device, async)
 *
 * Conventions for every call:
 *   - All buffers belong to the caller.  "dev" = device memory (hipMalloc),
 *     "host" = ordinary host memory, "pinned" = page-locked host memory
 *     (hipHostMalloc).  The library allocates nothing on these paths.
 *   - Arguments are validated before anything is enqueued: on any non-OK
 *     status nothing was enqueued and no caller state was changed.  The
 *     message of the last failure on the calling thread is lsa_last_error().
 *   - Launch failures return LSA_ERR_HIP; faults inside kernels surface at the
 *     caller's next synchronisation, as for any asynchronous HIP work.
 *   - A workspace serves one call at a time: calls that overlap in time must
 *     use distinct workspaces.
 *   - bf16 tensors are raw bfloat16 bit patterns (uint16); f32 are IEEE floats.
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lsa_status;
#define LSA_OK 0
#define LSA_ERR_INVALID (-1)     /* a pointer, size or layout argument is wrong */
#define LSA_ERR_UNSUPPORTED (-2) /* a shape or dtype this build has no kernel for */
#define LSA_ERR_CAPACITY (-3)    /* the hot pool cannot hold the selection */
#define LSA_ERR_WORKSPACE (-4)   /* workspace missing or smaller than the query said */
#define LSA_ERR_HIP (-5)         /* a HIP runtime call failed (message has the HIP error) */

typedef enum { LSA_F32 = 0, LSA_BF16 = 1 } lsa_dtype;

#define LSA_BLOCK_TOKENS 64     /* tokens per KV block: the unit scored, selected and moved */
#define LSA_MAX_REFRESH_REQ 64  /* requests per lsa_index_refresh call */
#define LSA_MAX_DECODE_REQ 64   /* requests per lsa_sparse_decode call */
#define LSA_ABI_VERSION 14

/* Message of the last non-OK status returned on this thread ("" if none). */
const char* lsa_last_error(void);

/* LSA_ABI_VERSION of the built library. */
int32_t lsa_abi_version(void);

/* sizeof the argument structs below, so a binding can check its own layout:
 * which = 0 refresh args, 1 gather args, 2 decode args, 3 latent args, 4 denoise args,
 * 5 device gather args.
 * Returns 0 for others. */
size_t lsa_struct_size(int32_t which);

/* --------------------------------------------------------------------------------------
 * KV block format.
 *
 * A block holds the keys and values of 64 consecutive tokens (rows t = 0..63) of
 * the single KV head: 2*64*D elements = lsa_block_bytes(dtype, D) bytes (32 KiB for
 * bf16, D = 128), keys first, then values.  The cold pool, the hot pool and each
 * request's window ring are arrays of such blocks.  The window ring of capacity C
 * tokens (a multiple of 64) holds token p in ring block (p % C) / 64, row p % 64.
 *
 * bf16: matrix-core fragment order.  Both halves are runs of 16-byte pieces (8
 * elements); every 64 consecutive pieces (1 KiB) are the operand one 64-lane wave
 * loads with one instruction, piece u + 16 g going to lane u + 16 g.  With KS = D/32:
 *     key (t, d)    element ((((j*KS + ks)*4 + g)*16 + u)*8 + e)
 *                   j = 2*(t/32) + (t/4)%2,  u = 4*((t/8)%4) + t%4,
 *                   ks = d/32,  g = (d/8)%4,  e = d%8
 *     value (t, d)  element 64*D + ((((c*2 + kk)*4 + g)*16 + u)*8 + e)
 *                   c = d/16,  u = d%16,  kk = t/32,  g = (t/8)%4,  e = t%8
 * (a value piece holds 8 consecutive tokens of one dimension, a key piece 8
 * consecutive dimensions of one token).
 * f32: keys row-major K[64][D] (token t's key is D contiguous elements), then
 * values transposed Vt[D][64] (dimension d of every token contiguous).
 * ------------------------------------------------------------------------------------ */

/* Bytes of one block; 0 if dtype or head_dim is not supported (D in {64, 128}). */
size_t lsa_block_bytes(int32_t dtype, int32_t head_dim);

/* Host-side packing of token-major K and V into the block format above (used to
 * build the cold pool and the initial window ring).
 *   k_tok, v_tok  host [n_tokens][head_dim]: tokens pos0 .. pos0+n_tokens-1
 *   dst           host or pinned, n_dst_blocks blocks; token p goes to block
 *                 (p / 64) % n_dst_blocks, row p % 64
 * Rows of dst blocks that receive no token are left untouched.  n_threads <= 0
 * picks a thread count.  Pure host code: no HIP call. */
lsa_status lsa_pack_blocks(int32_t dtype, int32_t head_dim, const void* k_tok, const void* v_tok,
                           int64_t pos0, int64_t n_tokens, void* dst, int64_t n_dst_blocks,
                           int32_t n_threads);

/* --------------------------------------------------------------------------------------
 * (1) Index refresh.
 *
 * For request r with B_r blocks and indexers i < n_idx (zhichai.net explainer,
 * sections 2-4; 1kpapers report page, Summary):
 *   q[i]     = W_q[i] h                        Query Encoder, fp32 accumulation, kept in fp32
 *   z[i][b]  = q[i] . keys[i][b] + bias[i]      dual-encoder block logit, fp32 accumulation (bf16
 *                                              keys meet q as the sum of two bf16 parts, within
 *                                              2^-18 of q relative)
 *   s[i][b]  = z[i][b] > logit(level)           sigmoid(z) > level (0.5 by default: z > 0), decided on z
 *   u[b]     = OR_i s[i][b]                     OR-mode union
 *   sel_ids  = ascending b with u[b], sel_count = their number
 * ------------------------------------------------------------------------------------ */
typedef struct lsa_refresh_args {
    int32_t n_req;             /* requests in this call, 1..LSA_MAX_REFRESH_REQ */
    int32_t d_model;           /* hidden size: multiple of 256, <= 16384 */
    int32_t d_idx;             /* index dim: 128 or 256 */
    int32_t n_idx;             /* indexers: 1..4 (the method uses 3) */
    int32_t dtype;             /* lsa_dtype of hidden, w_q and keys */
    float select_level;        /* keep a block when sigmoid(z) > select_level, decided on the logit as
                                  z > log(level / (1 - level)) in fp32; 0 means the pages' 0.5
                                  (z > 0), else 0 < select_level < 1 (the explainer, section 7, calls
                                  0.5 a preliminary choice) */
    const void* hidden;        /* dev: request r, indexer i reads d_model elements at
                                  r*hidden_req_stride + i*hidden_idx_stride */
    int64_t hidden_req_stride; /* elements between requests (>= d_model) */
    int64_t hidden_idx_stride; /* elements between indexers; 0 = one shared hidden state */
    const void* w_q;           /* dev [n_idx][d_idx][d_model]; row j projects onto output j */
    const void* keys;          /* dev; request r's keys [n_idx][B_r][d_idx] start at element
                                  n_idx*d_idx*blk_off[r] */
    const int64_t* blk_off;    /* host [n_req+1]: blk_off[0] = 0, B_r = blk_off[r+1]-blk_off[r],
                                  1 <= B_r <= 2^24 */
    const float* bias;         /* dev [n_req][n_idx] */
    int32_t* sel_ids;          /* dev: request r's ascending ids written at sel_ids + blk_off[r]
                                  (capacity B_r); or NULL with masks: the refresh then writes the bit
                                  planes only and leaves the ordering of the selection to the
                                  caller (lsa_gather_plan_device ranks the blocks from the union
                                  plane itself), with no compaction step; table_out must be NULL */
    int32_t* sel_count;        /* dev [n_req]: the counts, -1 for a request whose waits gave up; with
                                  sel_ids NULL only the -1 is written (a count is left as it was) */
    uint64_t* masks;           /* dev or NULL.  Request r's n_idx+1 bit planes of W_r =
                                  ceil(B_r/64) words start at word (n_idx+1)*M_r, where M_r is
                                  the sum of W_r' over r' < r; plane i < n_idx holds s[i],
                                  plane n_idx holds u; block b is bit b%64 of word b/64 */
    void* workspace;           /* dev, 256-byte aligned, workspace_bytes >= lsa_index_refresh_workspace(),
                                  zero-filled before its first use and then left to the library:
                                  it holds q and per-word counts, tagged with a number unique to
                                  each call, so nothing is cleared between calls (a captured graph
                                  that replays one call is therefore not supported) */
    size_t workspace_bytes;
    hipEvent_t ev_begin;       /* optional, used only when both are set: they receive the start and */
    hipEvent_t ev_end;         /* end time of the refresh kernel's dispatch */
    int32_t* table_out;        /* dev or NULL: the decode block table for a pool that holds every
                                  block (a fully resident pool).  Request r's pairs start at pair
                                  blk_off[r] (capacity B_r): pair j = (sel_ids[j],
                                  table_slot_base[r] + sel_ids[j]), written with the ids, so
                                  lsa_sparse_decode can read them with n_sel_dev = sel_count and
                                  tbl_off[r] = blk_off[r], with no host round trip */
    const int32_t* table_slot_base; /* host [n_req]: slot of block 0 of request r in that pool
                                  (block b at slot base + b); required with table_out, base + B_r
                                  <= 2^31 - 1 */
    float* logits;             /* dev or NULL: the fp32 logits z[i][b] the threshold was applied to
                                  (bias included), request r's [n_idx][B_r] starting at element
                                  n_idx*blk_off[r]; 4-byte aligned.  For checking the fp32 logits
                                  against exact ones; NULL writes nothing (the default) */
} lsa_refresh_args;

lsa_status lsa_index_refresh_workspace(const lsa_refresh_args* a, size_t* bytes);
lsa_status lsa_index_refresh(const lsa_refresh_args* a, hipStream_t stream);

/* --------------------------------------------------------------------------------------
 * (1a) Low-rank query projection, first factor (zhichai.net explainer, section 4,
 * training tricks: the query projection is low-rank, r = 2048, through the
 * backbone's MLA/MQA bottleneck).  For request r and indexer i:
 *   c[r][i][k] = sum_m A[i][k][m] h[r][i][m]     fp32 accumulation, then stored in
 *                                                the input type (bf16: nearest,
 *                                                ties to even), like any activation
 * lsa_index_refresh then runs with hidden = c (hidden_req_stride = n_idx*rank,
 * hidden_idx_stride = rank), d_model = rank and w_q = B [n_idx][d_idx][rank]:
 * q_i = B_i c_i.  All asynchronous on `stream`; validation happens before any launch.
 * ------------------------------------------------------------------------------------ */
typedef struct lsa_latent_args {
    int32_t n_req;             /* 1..LSA_MAX_REFRESH_REQ */
    int32_t d_model;           /* hidden size: multiple of 256, <= 16384 */
    int32_t rank;              /* latent size r: multiple of 256, <= 16384 */
    int32_t n_idx;             /* indexers: 1..4 */
    int32_t dtype;             /* lsa_dtype of hidden, w_down and latent */
    int32_t reserved0;         /* must be 0 */
    const void* hidden;        /* dev: request r, indexer i reads d_model elements at
                                  r*hidden_req_stride + i*hidden_idx_stride (16-byte aligned) */
    int64_t hidden_req_stride; /* elements between requests (>= d_model unless n_req = 1) */
    int64_t hidden_idx_stride; /* elements between indexers; 0 = one shared hidden state */
    const void* w_down;        /* dev [n_idx][rank][d_model]: A (16-byte aligned) */
    void* latent;              /* dev [n_req][n_idx][rank] out (16-byte aligned) */
    hipEvent_t ev_begin;       /* optional, used only when both are set: they receive the start and */
    hipEvent_t ev_end;         /* end time of the kernel's dispatch */
} lsa_latent_args;

lsa_status lsa_query_latent(const lsa_latent_args* a, hipStream_t stream);

/* --------------------------------------------------------------------------------------
 * (2) Block gather: after a refresh, make the hot pool of ONE request hold exactly
 * its new selection (zhichai.net explainer, section 2 steps 3 and 5: the selected
 * blocks are moved from the CPU cold pool to the GPU and the loaded set is
 * refreshed).
 *
 * Host part: blocks that left the selection free their slots, blocks that
 * entered take free slots, blocks that stayed keep theirs.  Device part: one
 * kernel on `stream` copies the entering blocks cold -> hot and writes the
 * request's block table: n_sel entries (block id, slot), ascending by block id.
 *
 * Ordering contract (the caller's, with events):
 *   - before the call, `stream` must wait for the last decode step that read the
 *     previous selection (slots of leaving blocks are overwritten);
 *   - decode steps that use the new selection must wait for `stream`;
 *   - `stage` is read by the copy kernel: do not reuse it until `stream` has
 *     passed this call.
 * State (slot_of_block, free_slots, n_free) is updated only on LSA_OK.
 *
 * Several attention layers (the pages' indexers feed the block loads of the
 * whole model: 1kpapers report page, Summary, and the explainer's section 4 with
 * indexers at three layers): with n_layers = L > 1 the one plan and the one
 * table serve L layers, each with its own cold and hot pool at a fixed byte
 * stride from layer 0's, and every entering block is copied for every layer.
 * ------------------------------------------------------------------------------------ */
typedef struct lsa_gather_args {
    int64_t n_blocks;          /* blocks of this request */
    int32_t n_slots_total;     /* slots in the whole hot pool (bounds check of slot ids) */
    int32_t block_bytes;       /* lsa_block_bytes(dtype, D) */
    const void* cold;          /* pinned host or dev: [n_blocks][block_bytes] */
    void* hot;                 /* dev: [n_slots_total][block_bytes] */
    const int32_t* new_ids;    /* host [n_new], ascending, each < n_blocks */
    int32_t n_new;
    int32_t stage_ints;        /* capacity of `stage` in int32, >= 4*n_new */
    int32_t* slot_of_block;    /* host [n_blocks]: slot holding block b, or -1 (in/out) */
    int32_t* free_slots;       /* host [capacity]: stack of this request's free slots (in/out) */
    int32_t* n_free;           /* host: entries in free_slots (in/out) */
    int32_t capacity;          /* this request's slot count (free_slots capacity) */
    int32_t n_layers;          /* 0 or 1: one layer; L in 2..256: layers 0..L-1 (strides below) */
    int32_t* stage;            /* pinned: copy list (source block, slot) pairs, then the table */
    int32_t* table_dev;        /* dev [capacity][2]: (block id, slot) pairs, ascending */
    int32_t* n_copied;         /* host out: blocks copied (per layer) */
    int32_t* n_kept;           /* host out: blocks that stayed resident */
    int64_t cold_layer_bytes;  /* L > 1: layer l's cold pool at cold + l*cold_layer_bytes (one
                                  allocation; >= n_blocks*block_bytes, multiple of 16) */
    int64_t hot_layer_bytes;   /* L > 1: layer l's hot pool at hot + l*hot_layer_bytes
                                  (>= n_slots_total*block_bytes, multiple of 16) */
    hipEvent_t ev_begin;       /* optional (NULL): recorded with the start stamp of the copy kernel's
                                  dispatch (of the first one, in a batch); only a[0]'s are used by
                                  lsa_gather_blocks_batch.  With nothing to launch, recorded on the
                                  stream at the call. */
    hipEvent_t ev_end;         /* optional (NULL): the end stamp of the (last) copy kernel's dispatch.
                                  A launch that records stamps costs ~30 us of host time against ~3 us
                                  for a plain one, so leave both NULL outside measurement. */
} lsa_gather_args;

lsa_status lsa_gather_blocks(const lsa_gather_args* a, hipStream_t stream);

/* The gathers of n requests (1..LSA_MAX_REFRESH_REQ) after one refresh: the same as calling
 * lsa_gather_blocks on a[0..n-1] in turn, except that every request is validated and planned
 * before anything is enqueued (any failure: nothing enqueued, no state changed for any request)
 * and the copies of all of them go into one kernel launch per 16 requests.  The requests must
 * have distinct residency state and staging buffers and the same block_bytes; their hot slots must
 * not overlap. */
lsa_status lsa_gather_blocks_batch(const lsa_gather_args* a, int32_t n, hipStream_t stream);

/* --------------------------------------------------------------------------------------
 * (2b) The gather planned on the device (zhichai.net explainer, section 2 steps 3 and 5),
 * for requests 0..n_req-1 right after their refresh, with no host round trip: the refresh's
 * union bits (its masks, plane n_idx) are compared with the resident set kept in device
 * memory; the slots of blocks that left go onto the request's device free stack, blocks
 * that entered take slots from its top and are copied cold -> hot (every layer), and the
 * request's block table is rewritten in ascending block id.  lsa_sparse_decode then reads
 * the table with n_sel_dev = table_count, tbl_off[r] = slot_off[r] and n_sel[r] = the
 * request's slot count.  A selection that does not fit a request's slots changes nothing
 * for that request and sets its status to 1 (its table and count stay those of the last
 * refresh that fitted).  The state (resident, slot_of_block, free_slots, n_free) belongs
 * to the caller and is set up by lsa_residency_reset; calls that share it must be ordered
 * on one stream.  Two launches on `stream` (plan, copy); validation happens first.
 * ------------------------------------------------------------------------------------ */
typedef struct lsa_device_gather_args {
    int32_t n_req;             /* 1..LSA_MAX_REFRESH_REQ */
    int32_t n_idx;             /* indexers of the refresh whose masks are read: 1..4 */
    int32_t block_bytes;       /* lsa_block_bytes(dtype, D) */
    int32_t n_layers;          /* 1..256 */
    const int64_t* blk_off;    /* host [n_req+1], as for the refresh (B_r = blk_off[r+1]-blk_off[r]) */
    const int32_t* slot_off;   /* host [n_req+1]: request r owns hot slots slot_off[r] .. slot_off[r+1]-1 */
    const uint64_t* masks;     /* dev: the refresh's bit planes (lsa_refresh_args.masks layout) */
    int32_t* sel_count;        /* dev [n_req]: the refresh's counts; a negative count (a refresh that
                                  gave up) changes nothing for the request and sets its status to 2.
                                  The plan then writes each request's count of selected blocks
                                  there (0 after a refresh that gave up), so that a refresh that
                                  wrote no counts (sel_ids NULL) leaves a valid one behind */
    uint64_t* resident;        /* dev [sum_r ceil(B_r/64)] state: request r's words start at word
                                  sum_{r'<r} ceil(B_r'/64); bit b = block b resident */
    int32_t* slot_of_block;    /* dev [blk_off[n_req]] state: slot of each block, or -1 */
    int32_t* free_slots;       /* dev [slot_off[n_req]] state: request r's stack at slot_off[r] */
    int32_t* n_free;           /* dev [n_req] state: entries on each stack */
    const void* const* cold;   /* host [n_req]: request r's cold pool, device memory (HBM) or pinned
                                  host memory (then the copy reads it over the host link) */
    int64_t cold_layer_bytes;  /* n_layers > 1: layer l of request r's cold pool at cold[r] + l*this */
    void* hot;                 /* dev: hot pool of slot_off[n_req] slots (per layer) */
    int64_t hot_layer_bytes;   /* n_layers > 1: layer l's hot pool at hot + l*this */
    int32_t* table;            /* dev: request r's (block id, slot) pairs from pair slot_off[r] */
    int32_t* table_count;      /* dev [n_req] out: entries in r's table */
    int32_t* copied;           /* dev [n_req] out: blocks that entered (copied once per layer) */
    int32_t* status;           /* dev [n_req] out: 0; 1 when the selection did not fit; 2 after a
                                  refresh that gave up */
    int32_t* status_any;       /* dev [n_req] or NULL: OR-ed with every nonzero status of the request
                                  (sticky until the caller clears it), so one read after many calls
                                  shows whether any of them failed */
    void* workspace;           /* dev, workspace_bytes >= lsa_gather_plan_device_workspace() */
    size_t workspace_bytes;
    hipEvent_t ev_begin;       /* optional (NULL): the start stamp of the plan kernel's dispatch */
    hipEvent_t ev_end;         /* optional (NULL): the end stamp of the copy kernel's dispatch; each is
                                  used on its own, and a launch that records a stamp costs ~30 us of
                                  host time against ~3 us for a plain one */
} lsa_device_gather_args;

lsa_status lsa_gather_plan_device_workspace(const lsa_device_gather_args* a, size_t* bytes);
lsa_status lsa_gather_plan_device(const lsa_device_gather_args* a, hipStream_t stream);

/* Set up the device residency state of lsa_gather_plan_device: nothing resident, every
 * slot of request r free (free_slots at slot_off[r] holds slot_off[r+1]-1 .. slot_off[r],
 * so the lowest slot is on top), n_free = slot count, table_count = 0, status = 0. */
lsa_status lsa_residency_reset(const lsa_device_gather_args* a, hipStream_t stream);

/* --------------------------------------------------------------------------------------
 * (3) Sparse decode: one decode step for n_req requests (zhichai.net explainer,
 * section 2 step 4).  For request r with L = seq_len[r] tokens (the current token
 * is position L-1) and ws = max(0, L - window[r]):
 *   attended T = {p : ws <= p < L}  U  {p < ws : p/64 is in the request's table}
 *   out[r][h] = sum_{p in T} softmax_p(scale * q[r][h] . K[p]) V[p]
 * All n_heads query heads share the single KV head.  Window tokens come from the
 * ring, selected-block tokens from the hot pool via the table.  When k_new and
 * v_new are given, the current token's K/V are taken from them and also written
 * into the ring (slot (L-1) % win_cap), so the call both appends and attends.
 * Work is split over all compute units (split-K over tiles of 64 tokens) and the
 * partial softmax states are combined by log-sum-exp.
 * ------------------------------------------------------------------------------------ */
typedef struct lsa_decode_args {
    int32_t n_req;             /* 1..LSA_MAX_DECODE_REQ */
    int32_t n_heads;           /* query heads, 1..16, sharing one KV head */
    int32_t head_dim;          /* 64 or 128 */
    int32_t dtype;             /* lsa_dtype of q, k_new, v_new, ring and pool */
    int32_t win_cap;           /* ring capacity in tokens, multiple of 64, >= every window[r] */
    float scale;               /* softmax scale (usually 1/sqrt(head_dim)) */
    const void* q;             /* dev [n_req][n_heads][head_dim] */
    const void* k_new;         /* dev [n_req][head_dim] or NULL (ring already holds token L-1) */
    const void* v_new;         /* dev [n_req][head_dim] or NULL (both or neither) */
    void* ring;                /* dev: request r's ring of win_cap/64 blocks at byte
                                  r*(win_cap/64)*block_bytes */
    const void* pool;          /* dev: hot pool [n_slots_total][block_bytes] */
    int32_t n_slots_total;     /* slots in the hot pool */
    int32_t reserved0;         /* must be 0 */
    const int32_t* table;      /* dev: request r's (block id, slot) pairs start at pair tbl_off[r] */
    const int32_t* tbl_off;    /* host [n_req] */
    const int32_t* n_sel;      /* host [n_req]: entries in request r's table (ascending block id);
                                  the kernel itself leaves out the tokens of blocks at or past the
                                  window start, so the whole table is passed */
    const int32_t* seq_len;    /* host [n_req]: L, >= 1 */
    const int32_t* window;     /* host [n_req]: W, 1..win_cap */
    float* out;                /* dev [n_req][n_heads][head_dim] fp32 */
    void* workspace;           /* dev, workspace_bytes >= lsa_sparse_decode_workspace() */
    size_t workspace_bytes;
    int32_t max_groups;        /* 0 = all compute units; else cap on work-groups (tests) */
    int32_t reserved1;         /* must be 0 */
    hipEvent_t ev_attn_begin;  /* optional, used only when both are set: they receive the start and */
    hipEvent_t ev_attn_end;    /* end time of the attention kernel's dispatch (the merge is outside) */
    const int32_t* n_sel_dev;  /* dev [n_req] or NULL.  When set, request r's entry count is read on
                                  the device from n_sel_dev[r] (clamped to 0..n_sel[r]; a negative
                                  count, a failed refresh, attends no block), n_sel[r] is only its
                                  capacity, and the split of the work over the groups is computed
                                  by the kernels: the refresh's sel_count feeds the decode with no
                                  host round trip */
    const int32_t* req_rows;   /* host [n_req] or NULL (identity).  Request r of this call is row
                                  req_rows[r] of every device array indexed by request: q, k_new,
                                  v_new, ring, out and n_sel_dev (the host arrays above stay this
                                  call's own, indexed by r).  Rows must be distinct (each request
                                  writes its own ring row and output row).  A call over some of a
                                  batch's requests then needs no copies: two such calls over
                                  disjoint rows, with their own workspaces, may run on two streams
                                  at once */
} lsa_decode_args;

lsa_status lsa_sparse_decode_workspace(const lsa_decode_args* a, size_t* bytes);
lsa_status lsa_sparse_decode(const lsa_decode_args* a, hipStream_t stream);

/* lsa_sparse_decode without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The same
 * kernels and results as lsa_sparse_decode; a->workspace and a->workspace_bytes are ignored and the
 * split-K partials go to a static array of the library, one per device (3,195,392 bytes: up to
 * 320 work-groups plus LSA_MAX_DECODE_REQ requests at head_dim 128), held until the process ends.
 * A call that would need more returns LSA_ERR_WORKSPACE and enqueues nothing.  The call allocates
 * nothing (its first call on a device looks the array's device address up once).  Every call on
 * a device shares that device's array: calls that overlap in time on one device race, so order
 * them on one stream. */
lsa_status lsa_sparse_decode_noalloc(const lsa_decode_args* a, hipStream_t stream);

/* --------------------------------------------------------------------------------------
 * (4) Label denoising for the indexer's training labels (zhichai.net explainer,
 * section 3, the three-step pipeline).  For layer l and token window w with the raw
 * indexer logits x[b] of its B_w history blocks:
 *   p[b]      = softmax over the row's blocks
 *   S[l][w]   = the smallest set of blocks whose probabilities sum to >= top_p:
 *               blocks taken by decreasing logit (equal logits: increasing block id)
 *               until the running sum reaches top_p
 *   label[w]  = blocks kept by at least min_votes layers; naive[w] = kept by any layer
 * Arithmetic: exp(x - max) in fp64, held as fixed point with 48 fraction bits, so
 * every sum is exact and independent of order; "reaches top_p" is the integer test
 * sum >= ceil(top_p * total).  Three launches on `stream` (top-p, top-p for rows
 * whose boundary falls in a run of > 1,024 equal-valued logits, vote); validation
 * happens first.
 * Every output row has W = ceil(max_w B_w / 64) 64-bit words (block b of window w
 * is bit b % 64 of word w*W + b/64; bits at b >= B_w are 0).
 * ------------------------------------------------------------------------------------ */
typedef struct lsa_denoise_args {
    int32_t n_layers;          /* layers that vote (21 on the pages), 1..64 */
    int32_t n_windows;         /* token windows, 1..65536 */
    int32_t min_votes;         /* layers that must keep a block (3 on the pages), 1..n_layers */
    int32_t reserved0;         /* must be 0 */
    double top_p;              /* mass a layer's set reaches (0.6 on the pages), 0 < top_p <= 1 */
    const float* logits;       /* dev [n_layers][n_windows][logit_stride] fp32, finite; row (l, w)
                                  holds its B_w logits first (16-byte aligned) */
    int64_t logit_stride;      /* elements between rows, >= max B_w, multiple of 4 */
    const int32_t* n_blk;      /* host [n_windows]: B_w, 1..16384 */
    const int32_t* n_blk_dev;  /* dev copy of n_blk */
    uint64_t* layer_sets;      /* dev [n_layers][n_windows][W] or NULL (then kept in the workspace) */
    uint64_t* labels;          /* dev [n_windows][W] */
    int32_t* n_pos;            /* dev [n_windows]: labels per window */
    int32_t* n_naive;          /* dev [n_windows] or NULL: blocks any layer keeps */
    void* workspace;           /* dev, 8-byte aligned, workspace_bytes >= lsa_label_denoise_workspace()
                                  (always needed: per-row flags, plus the layer sets when
                                  layer_sets is NULL) */
    size_t workspace_bytes;
    hipEvent_t ev_begin;       /* optional, used only when both are set: they receive the start and */
    hipEvent_t ev_end;         /* end time of the top-p kernel's dispatch (the rarely busy second
                                  top-p pass for crowded rows and the vote are outside) */
} lsa_denoise_args;

lsa_status lsa_label_denoise_workspace(const lsa_denoise_args* a, size_t* bytes);
lsa_status lsa_label_denoise(const lsa_denoise_args* a, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LSA_H */
