/*
 * msa.h -- C ABI of libmsa, Multi-Segment Attention (MSA) for AMD MI355X (gfx950).
 *
 * What it computes.  For every query row r of sequence b and every query head h,
 * exact softmax attention (Eq. 1 of the AsymCache / Multi-Segment Attention
 * paper: A = QK^T / sqrt(d_k), O = softmax(A) V) over the keys of b's context.
 * The context is made of several disjoint segments of a block-paged KV pool
 * (section 4.1 of that paper: a cached prefix and a cached suffix, with evicted
 * blocks rebuilt on demand, handled by one kernel).  A key at absolute position
 * p is visible to row r iff p <= q_pos[r] when causal (always otherwise), so
 * the regions l1, q1, l2, q2 of Eq. 5 keep their places in the sequence
 * whatever the order of the descriptors.  The result equals attention over
 * the gathered contiguous context; it does not depend on how the context is
 * split into segments or in which order they are listed.
 *
 * Conventions shared by every entry point:
 *  - Return value: MSA_OK (0) or a negative MSA_ERR_* code; msa_last_error()
 *    then returns a message (thread-local, valid until the next call on the
 *    same thread).
 *  - "host" pointers are read during the call only; "device" pointers are HIP
 *    device memory on the pool's device and must stay valid until the work
 *    enqueued on `stream` has completed.
 *  - All argument checks happen before any HIP call: on an error nothing has
 *    been enqueued.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes --------------------------------------------------------- */
#define MSA_OK               0
#define MSA_ERR_INVALID_ARG (-1)  /* malformed descriptor, null pointer, bad size    */
#define MSA_ERR_UNSUPPORTED (-2)  /* head_dim, dtype, block size or GQA ratio       */
#define MSA_ERR_OOM         (-3)  /* a device or pinned allocation failed           */
#define MSA_ERR_WORKSPACE   (-4)  /* plan exceeds the library's size limits         */
#define MSA_ERR_HIP         (-5)  /* a HIP runtime call failed                      */

/* ---- element types -------------------------------------------------------- */
#define MSA_BF16 0                /* q, K, V, out in bfloat16; fp32 accumulation    */
#define MSA_FP32 1                /* q, K, V, out in float32; fp32 throughout       */

#define MSA_BLOCK_SIZE 16         /* tokens per KV block (the only size supported)  */
#define MSA_SEG_FRESH  1          /* segment flag bit 0: K/V written in this step
                                     (recomputed after eviction, or new tokens).
                                     Metadata only: it does not change the result. */

/* ---- pool ----------------------------------------------------------------- */
/* A block-paged KV pool: two device arrays K and V, each laid out
 * [num_blocks][num_kv_heads][MSA_BLOCK_SIZE][head_dim], row-major, of `dtype`.
 * One (block, kv head) tile is contiguous (4 KiB for bf16 and head_dim 128).
 * The pool also owns the library's per-call workspace (device plan buffer,
 * partial results of split work) and pinned, device-mapped host staging. */
typedef struct msa_pool msa_pool;

typedef struct {
  int32_t num_blocks;     /* > 0                                            */
  int32_t block_size;     /* must be MSA_BLOCK_SIZE                         */
  int32_t num_kv_heads;   /* > 0                                            */
  int32_t head_dim;       /* 64 or 128                                      */
  int32_t dtype;          /* MSA_BF16 or MSA_FP32                           */
  int32_t device;         /* HIP device ordinal holding K, V and workspace  */
} msa_pool_desc;

/* Create a pool.  If k_base and v_base are both NULL the library allocates K
 * and V (hipMalloc, contents undefined) and frees them in msa_destroy_pool;
 * otherwise both must be non-NULL device pointers to caller-owned arrays of the
 * layout above, which the pool only references.  No HIP call is made when the
 * caller supplies K and V; the workspace is allocated on first use.
 * Errors: INVALID_ARG (null desc/out, sizes <= 0, only one of k/v given),
 * UNSUPPORTED (block_size, head_dim, dtype), OOM, HIP. */
int msa_create_pool(const msa_pool_desc* desc, void* k_base, void* v_base, msa_pool** out);

/* Device addresses of K and V (for the caller to write blocks into). */
int msa_pool_kv_ptrs(const msa_pool* pool, void** k, void** v);

/* Free the pool, its workspace and, if it allocated them, K and V.  Waits for
 * the pool's outstanding work first.  NULL is accepted (no-op). */
int msa_destroy_pool(msa_pool* pool);

/* ---- segment descriptors -------------------------------------------------- */
/* One contiguous run of tokens of a sequence: token i (0 <= i < len) has
 * absolute position pos_start + i and is stored in pool block
 * block_table[bt_start + i / 16], slot i % 16.  A segment starts at slot 0 of
 * a block; its last block may be partially filled (slots >= the remainder are
 * never read, whatever they hold).  len may be 0 (the segment is ignored). */
typedef struct {
  int32_t pos_start;  /* >= 0                                                  */
  int32_t len;        /* >= 0; pos_start + len must not overflow int32          */
  int32_t bt_start;   /* >= 0; bt_start + ceil(len/16) <= block_table_len        */
  int32_t flags;      /* MSA_SEG_FRESH or 0                                     */
} msa_segment;

/* A batch of sequences.  All arrays are host memory, read during the call.
 * Sequence b owns query rows q_offsets[b] .. q_offsets[b+1]-1 and segments
 * seg_offsets[b] .. seg_offsets[b+1]-1.  Within one sequence the position
 * ranges of the segments must not overlap (they may be listed in any order
 * and may leave gaps).  A query row may have any position; a row that sees no
 * key gets out = 0 and lse = -inf. */
typedef struct {
  int32_t batch;               /* >= 0                                              */
  int32_t num_q_heads;         /* multiple of the pool's num_kv_heads; the group
                                  of q head h is kv head h / (num_q_heads/num_kv_heads);
                                  that ratio must be <= 128                         */
  const int32_t* q_offsets;    /* [batch+1], q_offsets[0] == 0, non-decreasing       */
  const int32_t* q_pos;        /* [q_offsets[batch]] absolute query positions        */
  const int32_t* seg_offsets;  /* [batch+1], seg_offsets[0] == 0, non-decreasing     */
  const msa_segment* segs;     /* [seg_offsets[batch]]                               */
  int32_t block_table_len;     /* entries in block_table                            */
  float scale;                 /* score scale, >= 0; 0 selects 1/sqrt(head_dim)      */
  int32_t causal;              /* 1: key visible iff k_pos <= q_pos; 0: all visible   */
} msa_seg_desc;

/* ---- attention -------------------------------------------------------------- */
/* out[r][h][:] = softmax over visible keys of (scale * q[r][h] . k) applied to V,
 * lse[r][h]    = natural log of sum over visible keys of exp(scale * q[r][h] . k).
 *
 *  q            device [total_q][num_q_heads][head_dim], pool dtype
 *  block_table  device int32 [block_table_len]; entries are pool block ids in
 *               [0, num_blocks), read on `stream`.  An id out of range is
 *               clamped into the pool on the device and not reported, unless
 *               MSA_OPT_CHECK_BLOCK_IDS is set (then the call fails with
 *               MSA_ERR_INVALID_ARG before any attention kernel)
 *  out          device [total_q][num_q_heads][head_dim], pool dtype
 *  lse          device float32 [total_q][num_q_heads], or NULL
 *  stream       hipStream_t to enqueue on (NULL = default stream)
 *
 * Work is enqueued asynchronously on `stream`; results are valid once it
 * completes.  Values: the q, K and V elements a call reads must be finite;
 * a NaN or infinity among them gives unspecified out and lse for the rows
 * that see it (the bf16 kernels are built without NaN-propagation guarantees
 * in their max and exponent arithmetic).  Pool slots outside the segments are
 * never read into the arithmetic, whatever they hold.  A pool serialises its workspace on one stream at a time: calls
 * on one pool must be issued from one host thread and, if they use different
 * streams, the caller must order those streams.  q, out and lse must not alias.
 * Errors: INVALID_ARG, UNSUPPORTED, OOM, WORKSPACE, HIP. */
int msa_forward(const void* q, const msa_seg_desc* desc, const int32_t* block_table,
                msa_pool* pool, void* out, float* lse, void* stream);

/* ---- attention without allocation --------------------------------------------- */
/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, arguments and checks as msa_forward, with the same kernels,
 * but the call's plan and the partial results of split work go to a fixed
 * scratch array that the library holds on each GPU it runs on (16 MiB per
 * GPU, kept until the process ends) instead of the pool's workspace.  The call
 * makes no hipMalloc, hipFree, pinned or other device allocation; its plan
 * goes from host memory of the calling thread into the scratch through
 * hipMemcpyAsync on `stream` (a copy from pageable memory, so the call waits
 * until the host side of that copy has been taken).  Host-side, the planner's
 * working lists and that per-thread buffer are ordinary heap memory that grows
 * to the largest call seen and is then reused.  No kernel timing is
 * recorded (MSA_OPT_TIMING is ignored); MSA_OPT_SPLIT_BLOCKS and
 * MSA_OPT_NUM_CUS apply.
 *
 * Limits: at most 2 MiB of packed plan (block list of 8 bytes per KV block,
 * 4 bytes per query row, 32 bytes per work item, each part rounded to 256
 * bytes) and 12 MiB of split partials ((head_dim + 1) * 4 bytes per partial
 * row); a call beyond either returns MSA_ERR_WORKSPACE before any HIP call.
 * The scratch is shared by every call on one GPU and keeps the last call's
 * contents (each call writes all it reads); calls on one GPU whose work can
 * overlap -- on different streams, or from different host threads -- race on
 * it, so the caller must order them.
 * Errors: as msa_forward, plus WORKSPACE for the limits above. */
int msa_forward_noalloc(const void* q, const msa_seg_desc* desc, const int32_t* block_table,
                        msa_pool* pool, void* out, float* lse, void* stream);

/* ---- KV write (recompute-scatter) ------------------------------------------- */
/* Place freshly computed K/V rows -- a prefill chunk's own tokens, or evicted
 * blocks rebuilt on demand (abstract and section 4.1 / Figure 5 of the
 * AsymCache / Multi-Segment Attention paper) -- into the pool blocks that
 * their segment descriptors name, so that msa_forward then reads them like
 * any other segment.  For segment s, token i < segs[s].len and every kv head h:
 *   K[block_table[segs[s].bt_start + i/16]][h][i%16][:] = k_src[src_rows[s] + i][h][:]
 * and the same for V.  pos_start and flags are not used.  Slots that no token
 * maps to (the tail of a partial last block, every other block) keep their
 * contents.  The copy is exact.
 *
 *  k_src, v_src  device [num_src_rows][num_kv_heads][head_dim], pool dtype (the
 *                row-major output of a K/V projection); must not overlap each
 *                other or the pool's K/V arrays (checked)
 *  segs          host [num_segs]; len 0 is allowed (nothing written)
 *  src_rows      host int32 [num_segs]: row of k_src/v_src holding token 0 of
 *                segment s; 0 <= src_rows[s], src_rows[s] + len <= num_src_rows
 *  block_table   device int32 [block_table_len], as for msa_forward; entries are
 *                clamped into [0, num_blocks) on the device, or checked with
 *                MSA_OPT_CHECK_BLOCK_IDS (then an out-of-range id fails the
 *                call with MSA_ERR_INVALID_ARG before the write kernel)
 *  stream        hipStream_t to enqueue on; ordered with msa_forward calls on
 *                the same pool and stream
 *
 * Two segments may not use the same block-table entry (checked).  Distinct
 * entries naming the same pool block are a caller error that is not checked
 * (which write lands is then unspecified).
 * Errors: INVALID_ARG, OOM, WORKSPACE (block_table_len above 2^28, or more
 * than 2^31 (block, kv head) tiles), HIP. */
int msa_write_kv(msa_pool* pool, const void* k_src, const void* v_src, int32_t num_src_rows,
                 const msa_segment* segs, const int32_t* src_rows, int32_t num_segs,
                 const int32_t* block_table, int32_t block_table_len, void* stream);

/* Message for the last error on this thread ("" if none). */
const char* msa_last_error(void);

/* ---- options and diagnostics ------------------------------------------------ */
#define MSA_OPT_TIMING       1  /* 1: record HIP events around every kernel launch   */
#define MSA_OPT_SPLIT_BLOCKS 2  /* >0: cap on KV blocks per work item (forces split
                                   KV work and the merge); 0: automatic            */
#define MSA_OPT_NUM_CUS      3  /* >0: compute-unit count the planner balances for;
                                   0: the device's                                  */
#define MSA_OPT_CHECK_BLOCK_IDS 4 /* 1: before any attention or write kernel, check on
                                   the device that every block-table entry the call
                                   reads names a pool block in [0, num_blocks); if
                                   one does not, the call returns MSA_ERR_INVALID_ARG
                                   (naming the first such block-table index) with
                                   only the plan copy into the library's own buffer
                                   enqueued.  Synchronises the stream on every call.
                                   0 (default): ids are clamped into the pool on
                                   the device, without a report                     */
#define MSA_OPT_CHUNK_WAVES 6   /* 4 or 8: work-group size (waves) of the bf16 chunk
                                   launch, 128- or 256-row tiles; 0 (default): the
                                   planner's choice (8 only for prefill-only batches
                                   with at least two 256-row tiles per compute unit
                                   and long contexts)                                */
#define MSA_OPT_PHASE_TRACE 5   /* measurement builds only (libmsa_trace.so, built
                                   with MSA_PHASE_TRACE): device address of a
                                   buffer of n_items x 8 x 8 uint64 (8 wave slots
                                   per work item of the chunk launch, zeroed by the
                                   caller) into which the
                                   chunk kernel writes, per work item and wave, the
                                   step count and the summed shader-clock time of
                                   each phase of its steps (see msa_prefill.hip);
                                   0 turns it off.  The caller owns the buffer.  A
                                   library built without tracing returns
                                   MSA_ERR_UNSUPPORTED for a non-zero value.        */

int msa_pool_set_option(msa_pool* pool, int32_t option, int64_t value);

/* Kernel kinds reported by msa_pool_kernel_time. */
#define MSA_KERNEL_PREFILL 0    /* bf16 MFMA chunk kernel                           */
#define MSA_KERNEL_DECODE  1    /* bf16 bandwidth-bound decode kernel               */
#define MSA_KERNEL_FP32    2    /* fp32 kernel                                      */
#define MSA_KERNEL_MERGE   3    /* log-sum-exp merge of split partials              */
#define MSA_KERNEL_UPLOAD  4    /* copy of the per-call plan into device memory     */
#define MSA_KERNEL_WRITE   5    /* KV write (msa_write_kv)                          */

/* With MSA_OPT_TIMING on: total device time (ms, from HIP events recorded on
 * the launch stream around each launch) and number of launches of `kind`
 * since the last reset.  Synchronises on the recorded events.  reset != 0
 * clears the counters after reading. */
int msa_pool_kernel_time(msa_pool* pool, int32_t kind, double* total_ms, int64_t* launches,
                         int32_t reset);

/* With MSA_OPT_TIMING on: the durations (ms) of the most recent launches of
 * `kind` since the last reset, oldest first, at most `max` of them, written
 * to out (host array); *n receives the count.  The pool keeps up to 65 536
 * durations per kind (older ones are dropped).  Synchronises like
 * msa_pool_kernel_time.  Errors: INVALID_ARG, HIP. */
int msa_pool_kernel_samples(msa_pool* pool, int32_t kind, double* out, int32_t max, int32_t* n);

/* One work item of a plan (as the kernels see it). */
typedef struct {
  int32_t kind;       /* MSA_KERNEL_PREFILL / DECODE / FP32: the work the item is  */
  int32_t seq;        /* sequence index                                          */
  int32_t kv_head;
  int32_t q_row0;     /* first query row                                         */
  int32_t n_q;        /* number of query rows                                    */
  int32_t blk_begin;  /* [blk_begin, blk_end): entries of the block list          */
  int32_t blk_end;
  int32_t part_row;   /* -1: writes out/lse directly; else first partial row      */
  int32_t launch;     /* kernel launch that runs it: as kind, except that a batch
                         of prefill chunks and decode tokens runs its decode
                         items in the MSA_KERNEL_PREFILL launch                 */
} msa_plan_item;

/* One entry of the position-ordered block list. */
typedef struct {
  int32_t bt_index;   /* index into block_table                                  */
  int32_t pos0;       /* position of slot 0                                      */
  int32_t valid;      /* slots in use, 1..16                                     */
} msa_plan_block;

/* Run the planner alone (host only, no HIP call) for a pool of the given shape
 * and `num_cus` compute units.  Writes at most max_items items and max_blocks
 * blocks, and the counts needed in *n_items and *n_blocks (a call with
 * max_* = 0 queries the sizes).  split_blocks as MSA_OPT_SPLIT_BLOCKS.
 * Errors: as msa_forward's argument checks. */
int msa_plan_debug(const msa_seg_desc* desc, int32_t num_kv_heads, int32_t head_dim,
                   int32_t dtype, int32_t num_cus, int32_t split_blocks,
                   msa_plan_item* items, int32_t max_items, int32_t* n_items,
                   msa_plan_block* blocks, int32_t max_blocks, int32_t* n_blocks);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
