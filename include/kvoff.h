/*
 * kvoff.h - C ABI of the MI355X sparse KV-cache offloading hot path.
 *
 * One decode step of one attention layer over a KV cache held mostly in
 * pinned host DRAM, after PulseInfer ("PulseInfer: I/O-Centric Sparse KV
 * Cache Offloading for Efficient Long-Context LLM Decoding", abstract: most
 * historical KV blocks are stored in CPU DRAM and only selected blocks are
 * recalled on demand; SoloHead selection and a gather-scatter I/O engine
 * coalesce the fragmented transfers that per-head selection causes):
 *
 *   kvoff_offload_blocks  build per-block key digests in HBM and write the
 *                         KV blocks to the pinned host store
 *   kvoff_select          score every block and take one top-k block set
 *                         per request (SoloHead) or per KV head (headwise)
 *   kvoff_recall          move the selected, non-resident blocks host->HBM
 *   kvoff_sparse_decode   GQA decode attention over the recalled blocks
 *   kvoff_step            select, recall and attend over a range of layers,
 *                         recall of layer l+1 overlapped with attention of l
 *
 * Block scoring.  The pages leave the per-(head, block) importance S(h, b)
 * undefined ("PulseInfer Guide: I/O-Centric Sparse KV Cache Offloading",
 * aiFetchly, section "SoloHead Sparse Selection").  The rule fixed here:
 *   digest D[b][g][j] = fp32 rounding of the mean, over the valid tokens of
 *                       block b, of key K[t][g][j] (fp64 sum, one division)
 *   score  S[b]       = sum over query heads h and dims j of
 *                       q[h][j] * D[b][floor(h/G)][j], in fp64
 *   headwise S_g[b]   = the same sum over the G heads of KV head g.
 * Selection keeps the min(k, nb) largest scores (ties: lower block id; -0.0
 * equals +0.0) and lists them in ascending block order.
 *
 * Conventions for every call.
 *   - Returns 0 (KVOFF_OK) or a negative KVOFF_E* status; no call throws.
 *     kvoff_last_error() gives a thread-local message for the last failure.
 *   - Device buffers are plain device pointers owned by the caller; no call
 *     allocates device memory after kvoff_create.  Streams are hipStream_t
 *     values passed as void* (NULL = the null stream).
 *   - Calls enqueue work and return; outputs are valid once the stream has
 *     synchronised.  Exceptions: kvoff_register_request and kvoff_create are
 *     synchronous; kvoff_recall with KVOFF_ENGINE_DMA or KVOFF_ENGINE_STAGED
 *     and any call given a non-NULL kvoff_stats synchronise the stream they
 *     run on.
 *   - A context belongs to the device that is current when kvoff_create
 *     runs.  Every call on it runs on that device and leaves the calling
 *     thread's current device as it found it.
 *   - Dtype of q, K, V: IEEE fp16 or bf16 (the context's dtype).
 *     head_dim must be 128; block_size 16 or 32 tokens.
 *   - Non-finite inputs give undefined results (not scanned).
 *   - A context may be used from one host thread at a time.
 */
#ifndef KVOFF_H
#define KVOFF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status
   Every call that returns int returns one of these; the detail of the last
   failure on the calling thread is in kvoff_last_error().  No C++ exception
   leaves the library: a failed host allocation inside a call is reported as
   KVOFF_ENOMEM, any other internal failure as KVOFF_ESTATE. */
enum {
  KVOFF_OK = 0,
  KVOFF_EINVAL = -1, /* invalid argument or shape                          */
  KVOFF_ENOMEM = -2, /* host (pinned) allocation failed                    */
  KVOFF_ENODEV = -3, /* no usable GPU                                      */
  KVOFF_EHIP = -4,   /* a HIP runtime call failed (message in last_error)  */
  KVOFF_ERANGE = -5, /* a capacity, batch or buffer size is exceeded       */
  KVOFF_ESTATE = -6  /* e.g. a (layer, request) read before it was offloaded */
};

enum { KVOFF_F16 = 1, KVOFF_BF16 = 2 };

/* selection modes */
enum {
  KVOFF_SOLOHEAD = 0,  /* one block set per request, shared by all heads     */
  KVOFF_HEADWISE = 1,  /* one block set per KV head (fragmentation baseline) */
  /* one shared set ranked by the guide's consensus rule ("SoloHead Sparse
     Selection", consensus equation, applied across KV heads as in its
     simulator's SoloHeadSelector): S[b] = max_g S_g[b] + lambda * mean_g
     S_g[b], S_g the per-KV-head score; lambda per context (default 0.5).
     Its selection, recall and attention use the SoloHead layouts, and
     kvoff_recall / kvoff_sparse_decode treat it as KVOFF_SOLOHEAD. */
  KVOFF_CONSENSUS = 2,
  /* the same consensus rule with the scope the guide's text gives: the query
     heads of one GQA group.  S_g[b] = max_{h in g} s_h[b] + lambda *
     mean_{h in g} s_h[b], s_h[b] = sum_j q[h][j] * D[b][g][j]; one set per
     KV head, so it uses the KVOFF_HEADWISE layouts, and kvoff_recall /
     kvoff_sparse_decode treat it as KVOFF_HEADWISE. */
  KVOFF_CONSENSUS_GROUP = 3
};

/* recall engines */
enum {
  /* one HIP kernel reads the mapped pinned store over the host link and
     writes the HBM slots; the plan stays on the GPU, no host round trip */
  KVOFF_ENGINE_ZEROCOPY = 0,
  /* the selection is copied to the host, which issues one hipMemcpyAsync per
     coalesced run (per (block, KV head) slice in headwise mode), round robin
     over the call's stream and up to three copy streams the context owns
     (created on first use, non-blocking, default priority); the call's
     stream then waits for all of them.  Synchronises that stream first */
  KVOFF_ENGINE_DMA = 1,
  /* the guide's three-phase engine ("The Gather-Scatter I/O Engine"): host
     worker threads gather the selected records into a pinned staging
     buffer, which bulk hipMemcpyAsync copies move to HBM: chunks of 1 MiB,
     3 MiB, then 16 MiB each, each issued as soon as it is filled (the stats
     count these copies as transfers).  Items are placed compactly: the n-th
     recalled item of the call (in request, [KV head,] rank order) goes to
     slot recall_base_slot + n (headwise: slice recall_base_slot*Hkv + n);
     the block table says where.  Synchronises the stream first and returns
     once every chunk is gathered and its copy enqueued.  The context keeps
     two sets of pinned staging buffers (grown on demand) and uses them by
     turns: a set is reused once the copies of the call that used it last
     have completed.  The context's worker threads (three fewer than the
     hardware threads the process may run on, at most 10) spin for 500 us
     after a call before they sleep. */
  KVOFF_ENGINE_STAGED = 2
};

/* what runs the QK^T contraction of the attention (the G query heads of a
   group against a block's keys) */
enum {
  KVOFF_QK_MFMA = 0, /* v_mfma_f32_16x16x32 on the matrix cores (default) */
  KVOFF_QK_VALU = 1  /* v_dot2 on the vector ALUs; G <= 8 only          */
};

/* kind of pinned host memory for the store */
enum {
  KVOFF_HOST_COHERENT = 0,   /* fine-grained (hipHostMallocCoherent)      */
  KVOFF_HOST_NONCOHERENT = 1 /* coarse-grained (hipHostMallocNonCoherent) */
};

/* largest batch one call accepts */
#define KVOFF_MAX_BATCH 128

typedef struct kvoff_ctx kvoff_ctx;

typedef struct kvoff_config {
  int32_t num_layers;           /* layers the store holds                        */
  int32_t num_q_heads;          /* Hq; a multiple of num_kv_heads                 */
  int32_t num_kv_heads;         /* Hkv; G = Hq/Hkv must be 1, 2, 4, 8 or 16      */
  int32_t head_dim;             /* d; must be 128                                 */
  int32_t block_size;           /* bs tokens per block: 16 or 32                  */
  int32_t dtype;                /* KVOFF_F16 or KVOFF_BF16                        */
  int32_t max_requests;         /* registrations the context accepts              */
  int32_t host_mem_kind;        /* KVOFF_HOST_COHERENT or KVOFF_HOST_NONCOHERENT  */
  int64_t host_capacity_blocks; /* block records the pinned store holds, summed
                                   over layers and requests                       */
} kvoff_config;

/* Transfer statistics of one recall (or of a whole kvoff_step). */
typedef struct kvoff_stats {
  int64_t selected;        /* selected (block) or (block, KV head) entries     */
  int64_t pool_hits;       /* of those, already resident in the HBM pool       */
  int64_t items_recalled;  /* records (slices in headwise mode) moved          */
  int64_t transfers;       /* coalesced transfers: maximal runs of consecutive
                              missing blocks (one per slice in headwise mode) */
  int64_t bytes;           /* bytes moved host -> HBM                          */
} kvoff_stats;

/* ------------------------------------------------------------- lifecycle */

/* Validates cfg, selects the current HIP device and allocates the pinned host
 * store (host_capacity_blocks records of 2*Hkv*bs*d*es bytes, the record size
 * of the guide's simulator, GatherScatterEngine) plus a small device request
 * table.  *out receives the context.  Errors: EINVAL, ENODEV, ENOMEM, EHIP. */
int kvoff_create(const kvoff_config* cfg, kvoff_ctx** out);

/* Frees the store and the context; waits for the device first.  NULL is a no-op. */
int kvoff_destroy(kvoff_ctx* ctx);

/* Bytes of one block record: 2 * Hkv * bs * d * es. */
int64_t kvoff_record_bytes(const kvoff_ctx* ctx);

/* Sets lambda of KVOFF_CONSENSUS (>= 0; the guide prints 0.5 in its formula
 * and simulator and 1 in its worked figure).  Errors: EINVAL. */
int kvoff_set_consensus_lambda(kvoff_ctx* ctx, double lambda);

/* Chooses what computes the attention's QK^T (KVOFF_QK_MFMA or
 * KVOFF_QK_VALU) for later kvoff_sparse_decode / kvoff_step calls on this
 * context.  Both give the same result within fp32 rounding.  Errors: EINVAL
 * (unknown value, or KVOFF_QK_VALU with G = Hq/Hkv > 8). */
int kvoff_set_attention_qk(kvoff_ctx* ctx, int32_t qk);

/* Reserves store capacity for a request of n_tokens tokens in every layer
 * (nb = ceil(n_tokens / bs) records per layer) and returns its id in
 * *req_id.  Synchronous.  Errors: EINVAL (n_tokens < 1), ERANGE (store or
 * request table full), EHIP. */
int kvoff_register_request(kvoff_ctx* ctx, int64_t n_tokens, int32_t* req_id);

/* Host address of the record of (layer, req_id, block) in the pinned store,
 * laid out as [Hkv][K,V][bs][d] elements.  For inspection and tests. */
int kvoff_host_record(kvoff_ctx* ctx, int32_t layer, int32_t req_id, int64_t block,
                      const void** ptr);

/* --------------------------------------------------------------- offload */

/* Digest and offload one (layer, request).
 *   k_dev, v_dev  [n_tokens][Hkv][d] keys and values in HBM (the request's
 *                 registered n_tokens), dtype of the context
 *   digest_dev    out: [nb][Hkv][d] fp32 digests in HBM
 * Writes every block record (K rows then V rows of each KV head; rows past
 * the context end are zero) into the pinned store through its mapped
 * address.  Errors: EINVAL, ERANGE (layer), ESTATE (unknown request), EHIP. */
int kvoff_offload_blocks(kvoff_ctx* ctx, int32_t layer, int32_t req_id, const void* k_dev,
                         const void* v_dev, float* digest_dev, void* stream);

/* ---------------------------------------------------------------- select */

/* Score and select for a batch of n_req requests (n_req <= KVOFF_MAX_BATCH).
 *   req_ids       host [n_req] registered request ids
 *   q_dev         [n_req][Hq][d] decode queries
 *   digest_dev    [n_req][digest_stride][Hkv][d] fp32: request r's digests
 *                 start at r * digest_stride blocks (digest_stride >= nb_r)
 *   topk          host [n_req] block budgets k_r >= 1 (k_r > nb_r takes all)
 *   mode          KVOFF_SOLOHEAD or KVOFF_HEADWISE
 *   scores_dev    out: fp64 scores, [n_req][digest_stride] (SoloHead) or
 *                 [n_req][Hkv][digest_stride] (headwise); entries past nb_r
 *                 are not written
 *   sel_idx_dev   out: [n_req][k_stride] (SoloHead) or [n_req][Hkv][k_stride]
 *                 int32 selected block ids, ascending; unused entries -1
 *   sel_cnt_dev   out: [n_req] int32 K_r = min(k_r, nb_r)
 *   k_stride      row stride of sel_idx; must be >= every K_r
 * Errors: EINVAL (k_r < 1, bad mode/sizes), ERANGE (k_stride < K_r,
 * n_req > KVOFF_MAX_BATCH), ESTATE (unregistered request), EHIP. */
int kvoff_select(kvoff_ctx* ctx, int32_t layer, int32_t n_req, const int32_t* req_ids,
                 const void* q_dev, const float* digest_dev, int64_t digest_stride,
                 const int32_t* topk, int32_t mode, double* scores_dev, int32_t* sel_idx_dev,
                 int32_t* sel_cnt_dev, int32_t k_stride, void* stream);

/* ---------------------------------------------------------------- recall */

/* Recall the selected blocks of one layer into the HBM slot pool.
 *   slot_pool_dev [n_slots] records of kvoff_record_bytes() each, in HBM
 *                 (the pool holds n_slots records; owned by the caller;
 *                 1 <= n_slots and n_slots * Hkv <= INT32_MAX)
 *   recall_base_slot  first slot of the recall region: the record of rank i
 *                 of request r goes to slot recall_base_slot + r*k_stride + i
 *                 (headwise: KV head g's slice of that slot), so consecutive
 *                 ranks land in consecutive slots and each coalesced run is
 *                 one contiguous copy on both sides
 *   pool_hit_dev  nullable [n_req][pool_stride] uint8: 1 where block b of
 *                 request r is already resident in the pool at slot
 *                 pool_slot_dev[r*pool_stride + b]; resident blocks are not
 *                 moved.  A hit whose slot lies outside [0, n_slots) (for
 *                 instance -1) gets the table entry -1, so kvoff_sparse_decode
 *                 never reads it, and is not counted in the stats.  The DMA
 *                 and staged engines, which read the maps on the host, then
 *                 return KVOFF_ESTATE once the call's work is enqueued; the
 *                 zero-copy engine counts such hits on the device and the next
 *                 call on the context that fills stats (this one, or a later
 *                 kvoff_recall or kvoff_step) returns KVOFF_ESTATE for them
 *   block_table_dev out: SoloHead [n_req][k_stride] slot of each rank;
 *                 headwise [n_req][Hkv][k_stride] slice index (slot*Hkv + g);
 *                 unused entries -1
 *   engine        KVOFF_ENGINE_ZEROCOPY, KVOFF_ENGINE_DMA or KVOFF_ENGINE_STAGED
 *   stats         nullable; when given, filled after synchronising the stream
 * Errors: EINVAL (including n_slots outside its range), ERANGE (recall
 * region past n_slots), ESTATE (layer of a request not offloaded, or pool
 * hits outside the pool as above), EHIP. */
int kvoff_recall(kvoff_ctx* ctx, int32_t layer, int32_t n_req, const int32_t* req_ids,
                 int32_t mode, const int32_t* sel_idx_dev, const int32_t* sel_cnt_dev,
                 int32_t k_stride, const uint8_t* pool_hit_dev, const int32_t* pool_slot_dev,
                 int64_t pool_stride, void* slot_pool_dev, int64_t n_slots,
                 int64_t recall_base_slot, int32_t* block_table_dev, int32_t engine,
                 kvoff_stats* stats, void* stream);

/* --------------------------------------------------------------- attention */

/* Sparse GQA decode attention over the recalled blocks.
 *   q_dev         [n_req][Hq][d]
 *   slot_pool_dev, n_slots: the slot pool kvoff_recall filled, n_slots
 *                 records of kvoff_record_bytes() (1 <= n_slots and
 *                 n_slots * Hkv <= INT32_MAX)
 *   block_table_dev, sel_idx_dev, sel_cnt_dev, k_stride: as produced by
 *                 kvoff_recall / kvoff_select (sel_idx gives each entry's
 *                 block id, so a request's partial last block is masked).
 *                 Entries that are not a block of the request or of the pool
 *                 are skipped: a block id outside the request, a negative
 *                 table entry, or one at or past n_slots (headwise: slice
 *                 index at or past n_slots * Hkv).
 *   scale         logit scale (1/sqrt(d) for standard attention)
 *   out_dev       out: [n_req][Hq][d] fp32
 *   ws_dev        scratch of at least kvoff_workspace_size(ctx,
 *                 KVOFF_CALL_SPARSE_DECODE, n_req, k_stride, mode) bytes
 * Head h reads KV head floor(h/G).  Errors: EINVAL, ERANGE (ws too small),
 * ESTATE, EHIP. */
int kvoff_sparse_decode(kvoff_ctx* ctx, int32_t n_req, const int32_t* req_ids, int32_t mode,
                        const void* q_dev, const void* slot_pool_dev, int64_t n_slots,
                        const int32_t* block_table_dev, const int32_t* sel_idx_dev,
                        const int32_t* sel_cnt_dev, int32_t k_stride, float scale,
                        float* out_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* kvoff_sparse_decode without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  The split partials go to a scratch
 * array of KVOFF_NOALLOC_SCRATCH_BYTES that the library holds in device
 * memory, one per GPU for the life of the process (its address is looked up
 * by kvoff_create); the call allocates nothing.  Arguments and results as
 * kvoff_sparse_decode.  Every call on one GPU uses that GPU's one array:
 * calls that overlap in time on the same GPU (two streams, or two host
 * threads, whatever the context) race and give wrong results; calls ordered
 * on one stream do not.  Nothing in the array needs to start at zero, and
 * it keeps the last call's partials.  Errors: as kvoff_sparse_decode, and
 * ERANGE when kvoff_workspace_size(ctx, KVOFF_CALL_SPARSE_DECODE, n_req,
 * k_stride, mode) exceeds KVOFF_NOALLOC_SCRATCH_BYTES (16 MiB: n_req * Hq *
 * splits <= 32,263 partial rows of 520 bytes). */
#define KVOFF_NOALLOC_SCRATCH_BYTES (16u << 20)
int kvoff_sparse_decode_noalloc(kvoff_ctx* ctx, int32_t n_req, const int32_t* req_ids,
                                int32_t mode, const void* q_dev, const void* slot_pool_dev,
                                int64_t n_slots, const int32_t* block_table_dev,
                                const int32_t* sel_idx_dev, const int32_t* sel_cnt_dev,
                                int32_t k_stride, float scale, float* out_dev, void* stream);

enum { KVOFF_CALL_SPARSE_DECODE = 1, KVOFF_CALL_STEP = 2 };

/* Scratch bytes a call needs for the given batch (0 if none). */
size_t kvoff_workspace_size(const kvoff_ctx* ctx, int32_t call, int32_t n_req,
                            int32_t k_stride, int32_t mode);

/* ------------------------------------------------------------------ step */

/* Select, recall and attend for layers [layer_begin, layer_end) of one batch.
 * Per-layer arrays are indexed by layer - layer_begin.  Two buffer sets
 * (index 0/1) alternate between consecutive layers: select of layer l+1 is
 * enqueued on the compute stream ahead of attention of layer l, recall runs
 * on the copy stream as soon as its selection is ready, so the host link
 * stays busy while attention trails one layer behind (the single-GPU form of
 * the guide's one-layer-ahead prefetch, section "The Fallacy of Naive
 * Offloading", and of its layer-wise scheduling).  With copy_stream equal to
 * compute_stream the layers run serially.  Outputs equal a serial run bit
 * for bit.
 * Errors are found before any work is enqueued (EINVAL, ERANGE, ESTATE for
 * an unregistered request or a layer not offloaded; overlapped layers,
 * L > 1 with copy_stream != compute_stream, need recall regions of n_req *
 * k_stride slots that share no slot, else EINVAL), except the pool-slot
 * report of kvoff_recall: with stats, a step whose pool hits named slots
 * outside the pool still runs every layer and then returns KVOFF_ESTATE.
 * A call can be captured into a HIP graph on its compute stream (stream
 * capture; the copy streams join it through the call's own events) when the
 * engine is KVOFF_ENGINE_ZEROCOPY and stats and timing are NULL: the
 * captured work then holds no host synchronisation and no memset.  Replays
 * reuse the pointers and host arguments of the captured call (the inputs at
 * those addresses may change between replays); one context's captured
 * steps must not overlap each other or its eager calls, since they share its
 * events and counters. */
typedef struct kvoff_step_args {
  int32_t layer_begin, layer_end;
  int32_t n_req;
  const int32_t* req_ids;            /* host [n_req]                          */
  const int32_t* topk;               /* host [n_req]                          */
  int32_t mode, engine, k_stride;
  const void* const* q_dev;          /* [layers] -> [n_req][Hq][d]            */
  const float* const* digest_dev;    /* [layers] -> digests (see kvoff_select) */
  int64_t digest_stride;
  const uint8_t* const* pool_hit_dev;  /* nullable; [layers] -> hit maps; a  */
  const int32_t* const* pool_slot_dev; /* layer's pair may be NULL (no pool) */
  int64_t pool_stride;
  void* slot_pool_dev;
  int64_t n_slots;
  int64_t recall_base_slot[2];       /* recall region of buffer set 0 / 1      */
  double* scores_dev[2];
  int32_t* sel_idx_dev[2];
  int32_t* sel_cnt_dev[2];
  int32_t* block_table_dev[2];
  float scale;
  float* const* out_dev;             /* [layers] -> [n_req][Hq][d] fp32        */
  void* ws_dev;                      /* kvoff_workspace_size(KVOFF_CALL_STEP)  */
  size_t ws_bytes;
  void* compute_stream;
  void* copy_stream;
  kvoff_stats* stats;                /* nullable: summed over layers; syncs    */
  /* 0: recall and attend each layer's whole batch at once.  n > 0: per-request
     interruptible scheduling (the guide's section "Interruptible Layer-Wise
     Scheduling"): the batch is cut into contiguous groups of n requests,
     each group's recall is followed on the compute stream by that group's
     attention as soon as its own recall has landed, so attention of early
     groups runs while later groups are still crossing the link.  Within a
     layer the groups go in ascending order of the blocks they must
     transfer: the selected blocks of their requests that kvoff_make_resident
     has not pinned for that layer (fewest first, ties in batch order).
     Outputs are identical to n = 0. */
  int32_t group_requests;
  /* nullable host pointer: when set, the step records timing events on the
     compute stream and, after synchronising it, fills *timing */
  struct kvoff_step_timing* timing;
  /* Recalls of odd layers run on a second copy stream, so the recall of
     layer l+1 is not queued behind the end of layer l's on one stream (each
     still waits, through events, for its selection and for the attention
     that last read its buffer set).  NULL: a stream the context creates on
     first use (non-blocking, default priority).  Unused when copy_stream ==
     compute_stream (the serial order). */
  void* copy_stream2;
} kvoff_step_args;

/* Where the time went in one kvoff_step, from HIP timing events
 * (milliseconds): the first four on the compute stream, recall_ms on the copy
 * streams around each recall call (one per layer, or per request group). */
typedef struct kvoff_step_timing {
  double step_ms;              /* first select launched -> last attention done */
  double compute_wait_ms;      /* compute stream idle, waiting for recalls      */
  double mean_request_done_ms; /* mean over requests of step start -> the end
                                  of that request's last-layer attention       */
  double max_request_done_ms;  /* the same, latest request                     */
  double recall_ms;            /* sum over the step's recall calls of their
                                  duration, from events on the copy streams   */
  int64_t recalls;             /* number of those recall calls                 */
} kvoff_step_timing;

int kvoff_step(kvoff_ctx* ctx, const kvoff_step_args* args);

/* ------------------------------------------------------------- diagnostics of the selection */

/* Attention mass a selection keeps ("PulseInfer Guide", aiFetchly, section
 * "SoloHead Sparse Selection", attention mass preservation).  For request
 * i and query head h (KV head g = floor(h/G)), with z_t = scale * <q_h,
 * K_t[g]> over every valid token t of layer `layer` of the request:
 *   mass_dev[i*Hq + h] = sum_{t in blocks selected for g} exp(z_t - max z)
 *                        / sum_{all t} exp(z_t - max z).
 * Logits in fp32, sums in fp64.  The keys are read from the pinned store
 * over the host link (half of every record of the layer), so the call costs
 * about as much as recalling the whole layer; it is a diagnostic, not part
 * of the decode step.  mode: the layout of sel_idx_dev as kvoff_select wrote
 * it (shared set for KVOFF_SOLOHEAD / KVOFF_CONSENSUS, one set per KV head
 * for KVOFF_HEADWISE / KVOFF_CONSENSUS_GROUP); ids ascending, sel_cnt_dev[i]
 * <= k_stride entries per set.  q_dev [n_req][Hq][d]; mass_dev [n_req][Hq]
 * fp64.  Enqueued on `stream`.  Errors: EINVAL, ERANGE, ESTATE (unknown
 * request, layer not offloaded), EHIP. */
int kvoff_attention_mass(kvoff_ctx* ctx, int32_t layer, int32_t n_req, const int32_t* req_ids,
                         int32_t mode, const void* q_dev, const int32_t* sel_idx_dev,
                         const int32_t* sel_cnt_dev, int32_t k_stride, float scale,
                         double* mass_dev, void* stream);

/* ------------------------------------------------------------- admission */

/* IO-adaptive offloading admission ("PulseInfer Guide", aiFetchly, section
 * "Interruptible Layer-Wise Scheduling & Adaptive Admission"; abstract:
 * IO-Adaptive Offloading Admission adapts offloading decisions): with the
 * host link lightly used the store takes up to max_offload of the layers;
 * near saturation the most active layers (the first and the last) are kept
 * in HBM.  Resident layers are recalled from HBM: their blocks are pool hits. */
typedef struct kvoff_admission_policy {
  double low;          /* utilisation below which layers are released (0.50)   */
  double high;         /* utilisation above which more layers are pinned (0.85) */
  double max_offload;  /* largest offloaded fraction of the layers (0.90)      */
  int32_t step_layers; /* layers pinned or released per decision (2)           */
  int32_t max_resident; /* most layers the HBM budget holds (INT32_MAX: no cap);
                           applied last, so it wins over the offload ceiling  */
} kvoff_admission_policy;

/* Fills *p with the defaults above. */
void kvoff_admission_defaults(kvoff_admission_policy* p);

/* One admission decision.  utilization = recalled bytes / (elapsed seconds *
 * link peak) over the last window.  resident [num_layers] is the current plan
 * on entry (1 = kept in HBM) and the new plan on return.  Layers are pinned
 * in the order 0, L-1, 1, L-2, ... and released in the reverse order; at
 * least ceil((1 - max_offload) * num_layers) stay resident, and at most
 * max_resident.  *n_resident receives the new count.  Pure host logic.
 * Errors: EINVAL. */
int kvoff_admission_plan(const kvoff_admission_policy* p, int32_t num_layers, double utilization,
                         uint8_t* resident, int32_t* n_resident);

/* Makes (layer, req_id) resident: one bulk hipMemcpyAsync of its nb records
 * from the pinned store into HBM slots [first_slot, first_slot + nb) of
 * slot_pool_dev, then sets pool_hit_dev[b] = 1 and pool_slot_dev[b] =
 * first_slot + b for b < nb (the request's row of the maps kvoff_recall
 * takes).  Enqueued on `stream`: the caller orders later recalls after it
 * (same stream or an event) and keeps the slots out of every recall region.
 * n_slots * Hkv must not exceed INT32_MAX.
 * Errors: EINVAL, ERANGE (slots past n_slots), ESTATE (layer not offloaded),
 * EHIP. */
int kvoff_make_resident(kvoff_ctx* ctx, int32_t layer, int32_t req_id, void* slot_pool_dev,
                        int64_t n_slots, int64_t first_slot, uint8_t* pool_hit_dev,
                        int32_t* pool_slot_dev, void* stream);

/* Releases (layer, req_id): clears pool_hit_dev[b] for b < nb, so the next
 * recall moves its blocks from the store again.  Errors: EINVAL, ESTATE. */
int kvoff_release_resident(kvoff_ctx* ctx, int32_t layer, int32_t req_id, uint8_t* pool_hit_dev,
                           void* stream);

/* ------------------------------------------------------------- diagnostics */

/* Mean per-kernel durations of the timed kvoff_select and kvoff_sparse_decode
 * calls (also those made inside kvoff_step) since timing was turned on, in
 * milliseconds, from start and stop events bound to each kernel's own
 * dispatch. */
typedef struct kvoff_kernel_times {
  double score_ms;       /* score kernel of kvoff_select                     */
  double topk_ms;        /* its top-k kernel                                  */
  double attend_ms;      /* attention kernel of kvoff_sparse_decode          */
  double combine_ms;     /* its split merge                                   */
  int64_t select_calls;  /* timed kvoff_select calls the first two average   */
  int64_t decode_calls;  /* timed kvoff_sparse_decode calls the last two average */
} kvoff_kernel_times;

/* Turns per-kernel timing on (on != 0) or off for later calls on this
 * context; either way the accumulated times are cleared.  While on, each
 * kernel of kvoff_select and kvoff_sparse_decode is launched with a start
 * and a stop event from a ring of 64 per kernel that the context owns
 * (created by the first call that turns timing on).  Calls do not wait for
 * their own events: the host waits only when the ring wraps, for the events
 * of the call 64 calls earlier.  A call captured into a HIP graph must not
 * hold these events: switch timing off before capturing.  Results are
 * unchanged.  Errors: EINVAL, EHIP. */
int kvoff_set_kernel_timing(kvoff_ctx* ctx, int32_t on);

/* Waits for the stop events of every timed call not yet accounted and fills
 * *t with the means since timing was turned on (zeros and zero counts when
 * no call was timed).  Errors: EINVAL, EHIP. */
int kvoff_get_kernel_times(kvoff_ctx* ctx, kvoff_kernel_times* t);

/* Reads n_bytes (a multiple of 4096) at ptr with a GPU kernel and writes an
 * XOR reduction to dev_sink (>= 4096 bytes).  ptr is device memory or pinned
 * host memory from hipHostMalloc (read over the host link through its mapped
 * address): a probe of the achievable read rate for the recall kernel (host)
 * and of HBM (device).  n_wg workgroups (0 = default). */
int kvoff_probe_read(const void* ptr, int64_t n_bytes, void* dev_sink, int32_t n_wg,
                     void* stream);

const char* kvoff_strerror(int status);
const char* kvoff_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
