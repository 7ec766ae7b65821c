/*
 * moe.h -- C ABI of libmoe, the MI355X (gfx950) routed-expert MoE decode
 * library: router logits -> top-k selection -> per-expert SwiGLU computed
 * directly on 3.00-bit residual-vector-quantised (RVQ) expert records ->
 * gate-weighted combine, fed from an HBM LRU expert-slot cache whose misses
 * are copied from pinned host memory on a side stream.
 *
 * Sources (pages on routed expert streaming; the pages give the method in
 * prose only):
 *  [WISP]  "WISP -- 실행될 수 없는 것을 스트리밍하다" (molayo1419.me):
 *          section "통찰" (the model's own router selects the experts of each
 *          token; lookups go to the fastest tier holding the expert; an LRU
 *          cache promotes frequently used experts), section "더블 버퍼 비동기
 *          파이프라인" (the next experts are loaded into pinned RAM while the
 *          GPU computes) and "Lesson 2" (the router is the scheduler).
 *  [WASTE] "2.78조 파라미터 모델을 노트북에서: NVMe 스트리밍 추론 엔진 WASTE"
 *          (ttj.ttj.kr): section "유휴 가중치는 메모리가 아니라 제때 닿기만
 *          하면 된다" (one 4 KiB-aligned record per expert with gate, up and
 *          down adjacent, so routing to an expert costs one read; RVQ at 3.00
 *          bits per weight, never expanded; a bounded expert cache) and
 *          section "병목은 산술이 아니라 저장장치와 램이다" (expert reads
 *          overlap arithmetic; reads still dominate a decode step).
 *  [WARP]  "WARP 소개" (discuss.pytorch.kr): section "WARP가 모델을 램에
 *          올리지 않는 방법" (look-ahead only changes timing, never results),
 *          section "WARP의 캐시 설정에서 드러나는 역설" (experts per token is a
 *          manifest field; the engine refuses to start below the model's
 *          floor) and section "WARP 빌드와 실행" (one public C header serves
 *          every front end).
 *
 * Conventions
 *  - Every function returns int status: MOE_OK (0) or a negative MOE_E_*
 *    code; moe_last_error() then describes the failure (thread-local text,
 *    valid until the next call on the same thread).  No C++ exception
 *    crosses the ABI and the library never aborts the process.
 *  - Pointers marked [dev] are device (HBM) pointers, [host] host pointers,
 *    [pinned] page-locked host memory.  Streams are hipStream_t passed as
 *    void* (NULL = the default stream).
 *  - Ownership: the caller owns every device buffer, workspace, slot pool,
 *    pinned pool and stream.  The library never allocates device memory; it
 *    owns only host-side cache metadata, the hipEvents it creates and, once
 *    a record is copied from pageable memory, the cache's four pinned bounce
 *    buffers (slot_bytes each) and host copy threads, all of which
 *    expert_cache_destroy() frees.
 *  - Expert records for the cache ([pinned] below) may also be in pageable
 *    host memory: such a record is copied by host threads into the next
 *    bounce buffer (after that buffer's previous transfer has completed,
 *    which the calling thread waits for) and transferred from there, since
 *    the runtime's own staging of pageable transfers runs well below the
 *    link rate.
 *  - Kernels are asynchronous: argument and launch errors are returned at
 *    once, execution errors surface at the caller's next synchronisation.
 *  - T = 0 is a no-op returning MOE_OK.
 *  - Dimensions: H and I must be positive multiples of 128; 1 <= k <= E,
 *    k <= MOE_MAX_K, E <= MOE_MAX_E.
 *
 * Expert record (one per routed expert, bytes; section offsets from
 * moe_rvq_record_layout):
 *   gate codes [I, H] | up codes [I, H] | down codes [H, I] |
 *   gate scales fp16 [I] | up scales fp16 [I] | down scales fp16 [H] |
 *   gate, up, down codebooks fp16 [4096][8]
 *  Each section starts on a 256-byte boundary; the record is padded to
 *  4 KiB.  Weight W[r, 8q+i] of a matrix = s_r * (C[a][i] + C[b][i]), with the
 *  24-bit code pair v = a | b << 12 of row r, group q.  Codes are stored in
 *  64-row x 128-column tiles of 3072 bytes, tile (t, j) at (t*(K/128)+j)*3072;
 *  inside a tile, byte p of row l's 48-byte strip is at
 *  (p/16)*1024 + l*16 + p%16, and strip byte 3g+m is byte m (little-endian)
 *  of group 16j+g's code pair.
 *  Numerics: products and sums are fp32; activations (x, and the SwiGLU
 *  intermediate h) are rounded to fp16 for the GEMVs only after a
 *  power-of-two scaling of their block, undone exactly after the fp32 sums,
 *  so any finite fp32 activation is accepted.  The table-lookup decode
 *  methods also store C[c] . x_q (8 terms) in fp16: codebook entries must be
 *  below 16 in magnitude (RVQ codebooks are unit-scale; the row scales carry
 *  the magnitude).
 * Shared expert (optional, always on, weight 1): dense bf16
 *   gate [I, H] | up [I, H] | down [H, I], row-major.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

#define MOE_OK 0
#define MOE_E_INVAL (-1)   /* bad argument: null pointer, bad dims, k, dtype  */
#define MOE_E_HIP (-2)     /* HIP runtime error (message has hipGetErrorString) */
#define MOE_E_SPACE (-3)   /* workspace, pool or trace buffer too small       */
#define MOE_E_STATE (-4)   /* cache misuse: duplicate insert, bad slot         */
#define MOE_E_NOMEM (-5)   /* host allocation failed                           */

#define MOE_SCORE_SOFTMAX 0
#define MOE_SCORE_SIGMOID 1
#define MOE_DTYPE_F32 0
#define MOE_DTYPE_BF16 1

#define MOE_MAX_K 32
#define MOE_MAX_E 1024
#define MOE_CODEBOOK_ROWS 4096
#define MOE_NO_KEY 0xFFFFFFFFu
#define MOE_HBM_READ_BLOCKS 2048   /* partial words moe_hbm_read writes        */

/* Section offsets and sizes (bytes) of an expert record; index order:
 * 0 gate codes, 1 up codes, 2 down codes, 3 gate scales, 4 up scales,
 * 5 down scales, 6 gate codebook, 7 up codebook, 8 down codebook. */
typedef struct moe_record_layout {
    int64_t offset[9];
    int64_t size[9];
    int64_t nbytes;   /* end of the last section */
    int64_t padded;   /* nbytes rounded up to 4 KiB */
} moe_record_layout;

/* Router of one layer (WISP "통찰"; WARP "WARP의 캐시 설정에서 드러나는
 * 역설": k is a per-model manifest value, overridable here). */
typedef struct moe_router {
    const float *weight;  /* [dev] [E, H] fp32, row-major                        */
    const float *bias;    /* [dev] [E] fp32 added to the logits, or NULL          */
    int32_t E;            /* experts in the layer                                 */
    int32_t k;            /* experts selected per token                           */
    int32_t score_fn;     /* MOE_SCORE_SOFTMAX or MOE_SCORE_SIGMOID               */
} moe_router;

/* One MoE layer with all routed experts resident in HBM. */
typedef struct moe_layer {
    int32_t H;                    /* hidden size                                  */
    int32_t I;                    /* expert intermediate size                     */
    moe_router router;
    const void *const *records;   /* [dev] array of E [dev] record pointers;      */
                                  /* may be NULL for moe_layer_forward_streamed   */
    const uint16_t *shared;       /* [dev] dense bf16 shared expert, or NULL      */
} moe_layer;

typedef struct moe_cache moe_cache;

/* One cache lookup of a streamed decode (expert_cache_trace). */
typedef struct moe_trace_rec {
    uint32_t key;       /* layer_id * E + expert                                  */
    int32_t hit;        /* 1 = hit, 0 = miss; look-ahead touches (not lookups):   */
                        /* 2 = inserted ahead, 3 = already present (moved to MRU) */
                        /* exclusive host tier: 4 = lookup found nothing (nothing */
                        /* inserted, slot -1), 5 = the HBM cache's evicted key    */
                        /* moved in                                               */
    int32_t slot;       /* slot holding the key after the lookup                  */
    uint32_t evicted;   /* key evicted by this miss, or MOE_NO_KEY                */
} moe_trace_rec;

/* Text of the last error on this thread ("" if none). */
const char *moe_last_error(void);

/* MOE_ABI_VERSION of the loaded library. */
int moe_abi_version(void);

/* Record layout for dims (H, I) (WASTE "유휴 가중치는 ...": gate, up and down
 * adjacent in one aligned record).  Host-only and pure.  MOE_E_INVAL if H or I
 * is not a positive multiple of 128 or out is NULL. */
int moe_rvq_record_layout(int32_t H, int32_t I, moe_record_layout *out);

/* Workspace bytes that moe_route_topk needs for T tokens of E experts. */
size_t moe_route_workspace_bytes(int32_t E, int32_t T);

/* Router: z = W x + b for each token, select the k largest logits (ties go
 * to the lower expert id), weights = softmax or sigmoid of the selected
 * logits renormalised to sum 1 (WISP "통찰", "Lesson 2").
 *   x      [dev] [T, H], fp32 (MOE_DTYPE_F32) or bf16 (MOE_DTYPE_BF16)
 *   idx    [dev] [T, k] int32 expert ids in selection order (logit desc)
 *   w      [dev] [T, k] fp32 gate weights, same order
 *   ws     [dev] workspace of >= moe_route_workspace_bytes(E, T) bytes */
int moe_route_topk(const moe_router *r, const void *x, int32_t x_dtype, int32_t T,
                   int32_t H, int32_t *idx, float *w, void *ws, size_t ws_bytes,
                   void *hip_stream);

/* Workspace bytes that moe_expert_ffn_rvq needs. */
size_t moe_expert_ffn_workspace_bytes(int32_t H, int32_t I, int32_t T);

/* One routed expert applied to T tokens directly on its RVQ codes (WASTE
 * "유휴 가중치는 ...": matrices never expanded):
 *   y_t = (accumulate ? y_t : 0) + g_t * W_d (SiLU(W_g x_t) * (W_u x_t))
 *   record  [dev] expert record (layout above), 256-byte aligned
 *   x       [dev] [T, H] fp32;  y [dev] [T, H] fp32
 *   gate_w  [dev] [T] fp32 per-token weight g_t, or NULL for 1
 *   ws      [dev] >= moe_expert_ffn_workspace_bytes(H, I, T) bytes */
int moe_expert_ffn_rvq(const void *record, int32_t H, int32_t I, const float *x, int32_t T,
                       const float *gate_w, float *y, int32_t accumulate, void *ws,
                       size_t ws_bytes, void *hip_stream);

/* Workspace bytes that moe_layer_forward needs for T tokens. */
size_t moe_layer_workspace_bytes(const moe_layer *L, int32_t T);

/* One MoE layer, all experts resident: route, run each token's k experts on
 * their RVQ codes, combine out_t = sum_j w_tj y_j(x_t) + shared(x_t) in fixed
 * rank order (no atomics: results are run-to-run identical).
 *   x        [dev] [T, H] fp32 or bf16;  out [dev] [T, H] fp32
 *   idx_out  [dev] [T, k] int32 or NULL;  w_out [dev] [T, k] fp32 or NULL
 *   ws       [dev] >= moe_layer_workspace_bytes(L, T) bytes */
int moe_layer_forward(const moe_layer *L, const void *x, int32_t x_dtype, int32_t T,
                      float *out, int32_t *idx_out, float *w_out, void *ws,
                      size_t ws_bytes, void *hip_stream);

/* Workspace bytes that moe_decode_forward needs. */
size_t moe_decode_workspace_bytes(const moe_layer *layers, int32_t n_layers);

/* Decode driver: T tokens one at a time, each through n_layers resident
 * layers in order (WISP "통찰": token -> router -> experts -> next layer).
 * Layer inputs are given per (token, layer); token t's layer L runs only
 * after its layer L-1 has finished.  All layers must share H, I, E and k.
 * Runs as one cooperative persistent kernel (one workgroup per CU) for up to
 * 40 layers; the combine order is fixed, so results are run-to-run
 * identical (they may differ in the last bits from moe_layer_forward, whose
 * partial sums are split differently).
 *   layers  [host] array of n_layers layers (all with the same H, I)
 *   x       [dev] [T, n_layers, H] fp32;  out [dev] [T, n_layers, H] fp32
 *   idx_out [dev] [T, n_layers, k] int32 or NULL (k of each layer must agree)
 *   ws      [dev] >= moe_decode_workspace_bytes(layers, n_layers) bytes */
int moe_decode_forward(const moe_layer *layers, int32_t n_layers, const float *x,
                       int32_t T, float *out, int32_t *idx_out, void *ws,
                       size_t ws_bytes, void *hip_stream);

/* Which gate/up method moe_decode_forward uses for these layers on the
 * current device: 0 = codebook-row gathers (two 16-byte LDS reads per group
 * of 8 weights), 1 = table lookup (a per-chunk table of codebook-row x group
 * dot products in LDS, two 2-byte reads per group).  Both compute the same
 * products of the RVQ weights (WASTE article, section "유휴 가중치는 메모리가
 * 아니라 제때 닿기만 하면 된다": weights never expanded); the kernel picks
 * table lookup where each table serves many rows (I >= 8192), and the
 * environment variable MOE_DECODE_LUT (0 gathers, 1 table lookup for gate/up
 * and down, 2 table lookup for gate/up only) overrides where the shape allows.
 * Host-only query; needs a device (reads its compute-unit count).
 *   layers [host] as for moe_decode_forward;  method: 0 or 1 */
int moe_decode_gate_up_method(const moe_layer *layers, int32_t n_layers, int32_t *method);

/* The same for the down projection (same source): 0 = codebook-row gathers,
 * 1 = table lookup, one table per (rank, 128-column chunk of I) built from
 * that chunk of the SwiGLU intermediate h and serving all H rows.  Chosen
 * with gate/up's table lookup by default (I >= 8192).
 *   layers [host] as for moe_decode_forward;  method: 0 or 1 */
int moe_decode_down_method(const moe_layer *layers, int32_t n_layers, int32_t *method);

/* Whether any moe_decode_forward on this workspace since the previous
 * moe_decode_status call (or since the workspace's first use) hit its
 * device-side wait limit (a dependency between workgroups did not resolve
 * within a few seconds; every wave of that launch then leaves the kernel and
 * the outputs of that call are invalid).  The status is sticky across
 * launches and is reset by this call once read.  Synchronises the device
 * (hipDeviceSynchronize), then reads one word.
 *   ws [dev] the workspace passed to moe_decode_forward, or NULL for the
 *            current device's scratch array of moe_decode_forward_noalloc;
 *   timed_out: 0 or 1 */
int moe_decode_status(const void *ws, int32_t *timed_out);

/* Bytes of the device scratch array that moe_decode_forward_noalloc uses
 * (one per device, held from the library's load until the process ends). */
#define MOE_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)

/* moe_decode_forward without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The decode's workspace (counters and the
 * step-tagged exchange buffers, cleared by a kernel at each launch) is a
 * file-scope device array of MOE_NOALLOC_SCRATCH_BYTES in the library, one
 * copy per device, whose address is looked up on the first call on each
 * device; nothing is allocated (no hipMalloc, hipFree or allocating library
 * call).  Outputs equal moe_decode_forward's bit for bit.  The caller still
 * passes x, out and idx_out as for moe_decode_forward.  Every call on a
 * device shares that device's array: calls that overlap on one device (on
 * different streams or host threads) race and give invalid results.  The
 * wait-limit status is read with moe_decode_status(NULL, ...).
 * MOE_E_SPACE if these layers need more workspace than
 * MOE_NOALLOC_SCRATCH_BYTES (moe_decode_workspace_bytes tells; the Mixtral-,
 * Kimi-Linear- and K3-shaped decodes need at most 12 MB); other errors as
 * for moe_decode_forward. */
int moe_decode_forward_noalloc(const moe_layer *layers, int32_t n_layers, const float *x, int32_t T,
                               float *out, int32_t *idx_out, void *hip_stream);

/* Workspace bytes that moe_layer_forward_grouped needs for T tokens. */
size_t moe_grouped_workspace_bytes(const moe_layer *L, int32_t T);

/* Batched layer (many tokens, WASTE "실무자에게 남는 질문은 ...": one image
 * is 256 prompt positions, each through every MoE layer): route all tokens,
 * group (token, rank) pairs per expert, then per expert and matrix a
 * bf16-input GEMM on matrix cores with fp32 accumulation whose weight
 * operand is the codebook rows the RVQ codes pick (the codebook in LDS, no
 * dequantised matrix), SiLU(gate) * up, the down GEMM, and a fixed-order
 * combine plus the shared expert.  x [dev] [T, H] bf16 (MOE_DTYPE_BF16) or fp32; out [T, H] fp32.
 * Accuracy: relative L2 <= 1e-2 against an fp64 evaluation. */
int moe_layer_forward_grouped(const moe_layer *L, const void *x, int32_t x_dtype,
                              int32_t T, float *out, int32_t *idx_out, float *w_out,
                              void *ws, size_t ws_bytes, void *hip_stream);

/* ---------------------------------------------------------------- cache --
 * HBM expert-slot cache (WISP "통찰": LRU promotion; WASTE "유휴 가중치는 ...":
 * a bounded cache).  One LRU over integer keys; slot s occupies bytes
 * [s * slot_bytes, (s+1) * slot_bytes) of the caller's device pool.  A
 * lookup hit moves the key to most-recently-used.  An insert takes the
 * lowest-numbered free slot, else evicts the least recently used key and
 * reuses its slot, and copies the host record into the slot on copy_stream.
 * The object is not thread-safe: one host thread drives it. */

/* capacity >= 1; slot_bytes > 0 and a multiple of 256; pool_dev [dev] holds
 * capacity * slot_bytes bytes (caller-owned).  Creates 2 events per slot. */
int expert_cache_create(int32_t capacity, uint64_t slot_bytes, void *pool_dev,
                        moe_cache **out);
void expert_cache_destroy(moe_cache *c);

/* slot = slot holding key (hit: moved to MRU, counted), or -1 (miss). */
int expert_cache_lookup(moe_cache *c, uint32_t key, int32_t *slot);

/* Insert a key that is not cached: pick its slot (evicting if full), make
 * copy_stream wait for the slot's last-use event (write-after-read guard),
 * enqueue the slot_bytes copy from host_src [pinned] and record the slot's
 * ready event.  MOE_E_STATE if the key is already cached.  On a copy error
 * the cache is left as it was.  evicted = evicted key or MOE_NO_KEY. */
int expert_cache_insert(moe_cache *c, uint32_t key, const void *host_src, void *copy_stream,
                        int32_t *slot, uint32_t *evicted);

/* Make compute_stream wait until the slot's latest copy has landed. */
int expert_cache_wait(moe_cache *c, int32_t slot, void *compute_stream);

/* Record the slot's last-use event on compute_stream after the work that
 * reads the slot has been enqueued (a later eviction's copy waits on it). */
int expert_cache_release(moe_cache *c, int32_t slot, void *compute_stream);

/* Device address of a slot. */
int expert_cache_slot_ptr(moe_cache *c, int32_t slot, void **ptr);

/* Copy up to cap trace records (oldest first) into buf [host]; n = records
 * available in total.  Every lookup and insert of the streamed path appends
 * one record; MOE_E_SPACE if cap < n (buf then holds the first cap). */
int expert_cache_trace(moe_cache *c, moe_trace_rec *buf, int64_t cap, int64_t *n);

/* Clear the trace (the cache contents stay). */
int expert_cache_trace_reset(moe_cache *c);

/* Look-ahead counters since creation: keys inserted ahead (copies), keys
 * found present, inserted keys later hit by a lookup, and inserted keys
 * evicted before any lookup (wasted copies).  Any pointer may be NULL. */
int expert_cache_stats_ahead(moe_cache *c, int64_t *inserted, int64_t *present, int64_t *used,
                             int64_t *wasted);

/* Counters since creation: lookups, hits, inserts (copies), evictions. */
int expert_cache_stats(moe_cache *c, int64_t *lookups, int64_t *hits, int64_t *inserts,
                       int64_t *evictions);

/* LRU stack distances of a reference string of cache keys (hit rate against
 * cache size, WARP "WARP의 캐시 설정에서 드러나는 역설", Table C), computed in
 * one pass by the stack algorithm of Mattson et al. (1970): dist[i] = number
 * of distinct keys referenced since the previous reference to keys[i] (0 =
 * it was the most recent), or -1 for its first reference.  The expert cache's
 * policy (hit -> MRU; miss -> insert at MRU, evict the LRU key when full) is
 * LRU over the key sequence of its trace, so a cache of capacity C started
 * empty hits exactly the references with 0 <= dist[i] < C: one pass gives
 * the hit count at every capacity.  Host-only, O(n log n) time, O(n) memory.
 *   keys [host] n keys;  dist [host] n int32 (caller-owned)
 * MOE_E_INVAL if n < 0, n > INT32_MAX, or keys/dist NULL with n > 0;
 * MOE_E_SPACE if host memory runs out. */
int moe_lru_stack_distances(const uint32_t *keys, int64_t n, int32_t *dist);

/* Workspace bytes that moe_layer_forward_streamed needs for T tokens. */
size_t moe_streamed_workspace_bytes(const moe_layer *L, int32_t T);

/* One layer fed from the cache (WISP "더블 버퍼 비동기 파이프라인"; WASTE
 * "병목은 ...": reads overlap arithmetic; WARP "WARP의 캐시 설정에서 드러나는
 * 역설": refuse to run below the floor).  T must be 1 (decode).  Routes on
 * compute_stream (the top-k kernel writes the k expert ids to page-locked
 * host memory; one sync), looks the keys layer_id * E + e up in ascending
 * expert id, inserts each miss (copied from experts_host[e], alternately on
 * copy_stream and on a second copy stream the cache owns; copy_stream then
 * waits for the second, so it completes after every copy of the call), runs
 * the hit experts at once and the miss experts (two per launch, one from
 * each copy stream) once their copies have landed, then combines in fixed
 * rank order with the shared expert.  Output equals moe_layer_forward's bit
 * for bit.  MOE_E_INVAL if the cache capacity is below k or its slot size
 * below the record size.
 *   experts_host [host] array of E [pinned] record pointers
 *   x [dev] [1, H] fp32;  out [dev] [1, H] fp32;  idx_out [dev] [1, k] or NULL */
int moe_layer_forward_streamed(const moe_layer *L, moe_cache *c, uint32_t layer_id,
                               const void *const *experts_host, const float *x, int32_t T,
                               float *out, int32_t *idx_out, void *ws, size_t ws_bytes,
                               void *compute_stream, void *copy_stream);

/* moe_layer_forward_streamed plus a look-ahead read (WARP "WARP가 모델을 램에
 * 올리지 않는 방법": a pre-read router guesses the next layer's experts so their
 * reads start early, while the real router still decides; WISP "더블 버퍼
 * 비동기 파이프라인": loads for the next step overlap this step's compute).
 * The next layer's router (next->router weights and bias, k_ahead experts) is
 * applied to this layer's input x on compute_stream, with this layer's own
 * routing and the same single host sync.  After this layer's work is queued
 * (and its slots released), the predicted keys next_layer_id * E_next + e are
 * touched in the cache in ascending e, like lookups that count as neither
 * hit nor miss (trace kinds 2 and 3): an absent key is inserted (evicting the
 * LRU key if full) and copied from next_experts_host[e] on copy_stream behind
 * this layer's miss copies; its copy waits for the victim slot's last
 * readers.  Outputs are those of moe_layer_forward_streamed bit for bit: the
 * prediction changes only which copies happen and when.  Only predictions
 * whose weight, the next router's score renormalised over its k_ahead
 * choices as the gate weights are, is at least min_weight are touched (a
 * confidence threshold: 0 touches all k_ahead; 1/k_ahead keeps those above
 * the mean).
 *   next [host] the next layer (its records are not read; H must match)
 *   next_experts_host [host] array of E_next [pinned] record pointers
 *   k_ahead in 1..min(E_next, MOE_MAX_K, capacity); min_weight in [0, 1]
 * MOE_E_INVAL on a NULL next or bad arguments, as well as the conditions of
 * moe_layer_forward_streamed.  ws: moe_streamed_workspace_bytes(L, T). */
int moe_layer_forward_streamed_ahead(const moe_layer *L, moe_cache *c, uint32_t layer_id,
                                     const void *const *experts_host, const float *x, int32_t T,
                                     float *out, int32_t *idx_out, void *ws, size_t ws_bytes,
                                     void *compute_stream, void *copy_stream, const moe_layer *next,
                                     uint32_t next_layer_id, const void *const *next_experts_host,
                                     int32_t k_ahead, float min_weight);

/* ---- third tier: expert records in a file ------------------------------- */
typedef struct moe_host_tier moe_host_tier;

/* A file of n_records records of record_bytes each (record i at byte
 * i * record_bytes), read with O_DIRECT (WASTE "유휴 가중치는 …": one aligned
 * read per expert, no OS page cache, so measured hit rates are real) into a
 * caller-owned pinned host pool of `slots` records kept as LRU (WISP "통찰":
 * VRAM, then RAM, then the disk).  io_threads host threads read the misses of
 * one layer call in parallel.  MOE_E_INVAL if record_bytes is not a multiple
 * of 4096, the pool is not 4096-aligned, the file cannot be opened with
 * O_DIRECT or is shorter than n_records records. */
int moe_host_tier_create(const char *path, uint64_t record_bytes, int64_t n_records, int32_t slots,
                         void *pinned_pool, int32_t io_threads, moe_host_tier **out);
/* The same file tier as an exclusive lower tier of the HBM cache (WISP
 * "통찰": each lookup goes to the fastest tier that holds the expert, read as
 * a hierarchy where a record sits in one tier at a time).  In
 * moe_layer_forward_streamed_tiered, per key of the layer in ascending expert
 * id: an HBM miss looks the key up here; a key found here leaves this tier
 * and its slot is the copy's source, else the record is read from the file
 * into a transit page; the key is inserted in the HBM cache, and the key the
 * HBM cache evicts (if its slot was filled) moves here, at the most recent
 * end, its bytes copied device-to-host from its HBM slot on the copy stream
 * before the slot is overwritten (this tier evicts its own least recently
 * used key if full).  The two tiers then hold the c1 + c2 most recently used
 * keys, as one LRU of their combined size would (the oracle's two_tier
 * model).  Keys are the HBM cache's keys (layer_id * E + e), so record0 must
 * equal layer_id * E.  The pool holds `slots` records: slots - MOE_MAX_K are
 * the LRU's capacity, MOE_MAX_K are transit pages for one layer call's
 * copies.  MOE_E_INVAL as moe_host_tier_create, or if slots <= MOE_MAX_K. */
int moe_host_tier_create_exclusive(const char *path, uint64_t record_bytes, int64_t n_records, int32_t slots,
                                   void *pinned_pool, int32_t io_threads, moe_host_tier **out);
/* Keys moved into an exclusive host tier from the HBM cache since creation. */
int moe_host_tier_demotions(moe_host_tier *t, int64_t *demotions);
/* Waits for the copies still reading the pool, closes the file. */
void moe_host_tier_destroy(moe_host_tier *t);
/* Counters since creation: lookups and hits of the host slots, records read
 * from the file, their bytes, and the wall time spent in reads (ns). */
int moe_host_tier_stats(moe_host_tier *t, int64_t *lookups, int64_t *hits, int64_t *reads,
                        int64_t *read_bytes, int64_t *read_ns);
/* The host tier's LRU trace (keys are record indices), as expert_cache_trace. */
int moe_host_tier_trace(moe_host_tier *t, moe_trace_rec *buf, int64_t cap, int64_t *n);

/* moe_layer_forward_streamed with the file tier behind the HBM cache: the
 * records of the HBM misses (expert e is file record record0 + e) come from
 * the host slots, the absent ones read from the file first (in parallel,
 * while the hit experts compute); each copy then goes to the device as in
 * moe_layer_forward_streamed.  Outputs are identical to it bit for bit.
 * MOE_E_INVAL if the host tier has fewer slots than k, besides the
 * conditions of moe_layer_forward_streamed. */
int moe_layer_forward_streamed_tiered(const moe_layer *L, moe_cache *c, uint32_t layer_id,
                                      moe_host_tier *tier, int64_t record0, const float *x, int32_t T,
                                      float *out, int32_t *idx_out, void *ws, size_t ws_bytes,
                                      void *compute_stream, void *copy_stream);

/* ---- measurement aid ---------------------------------------------------- */
/* The plain-read reference for expert-weight bandwidth: one pass of 16-byte
 * nontemporal loads over buf, with no arithmetic besides an XOR per load.
 * The expert bytes a decode streams are quoted as a fraction of this rate as
 * well as of the HBM peak.  sink [dev] receives MOE_HBM_READ_BLOCKS words
 * whose XOR equals the XOR of buf's 32-bit words (so the reads are checked
 * and never dead code).  Asynchronous on hip_stream.  MOE_E_INVAL if sink is
 * NULL, buf is NULL with bytes > 0, buf is not 16-byte aligned or bytes is
 * not a multiple of 16; bytes = 0 writes zero partials. */
int moe_hbm_read(const void *buf, uint64_t bytes, uint32_t *sink, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
