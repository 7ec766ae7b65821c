// Internal declarations shared by the HIP kernels and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kCbRows = MOE_CODEBOOK_ROWS;   // codebook rows (12-bit indices)
constexpr int kTileRows = 64;                // rows per code tile = lanes per wave
constexpr int kChunkCols = 128;              // columns per code tile (16 groups)
constexpr int kTileBytes = 3072;             // 64 rows x 48 bytes
constexpr int kTileVec = kTileBytes / 16;    // 16-byte words per tile

// How a work item finds its expert record.  A launch covers T tokens x
// n_local items per token; local item l of token t is global item t*k + rank,
// where rank = l (table mode) or rank[l] (list mode).  Global items index the
// SwiGLU intermediate and the down partial sums, so any grouping of ranks
// into launches produces the same bytes.
struct RecSrc {
    const void *const *table;      // [dev] record pointer per expert, or nullptr
    const int32_t *idx;            // [dev] expert id per global item (table mode)
    const void *list[MOE_MAX_K];   // list mode: record pointer of local item l
    int32_t rank[MOE_MAX_K];       // list mode: rank of local item l (32-bit: read by scalar loads)
    int32_t k;                     // ranks per token
    int32_t n_local;               // local items per token in this launch
};

// Section offsets of one record (bytes).
struct RecOffsets {
    int64_t codes[3];   // gate, up, down
    int64_t scales[3];
    int64_t cb[3];
};

// Workspace carving for one layer call.
struct LayerWs {
    float *z;          // [T, E] router logits
    int32_t *idx;      // [T, k]
    float *w;          // [T, k]
    uint32_t *xh;      // [T, H/2] x as fp16 pairs, scaled by 2^-xexp[t]
    int32_t *xexp;     // [T] range exponent of each token's x
    float *hh;         // [T*k, 2, I] gate and up outputs (fp32); the down kernel forms SiLU(g) * u
    float *ypart;      // [T*k, KS, H] down partial sums (scaled)
    float *hs;         // [T, I] shared-expert intermediate (fp32)
    float *ysh;        // [T, H] shared-expert output
    size_t bytes;
};

// ---- launchers (kernels.hip) ------------------------------------------------
hipError_t launch_route_logits(const float *W, const float *bias, int E, int H, const void *x,
                               int x_dtype, int T, float *z, hipStream_t s);
// idx_host / w_host (optional, page-locked host memory): the ids and weights
// are written there too, visible once the kernel has completed, or (token 0)
// as soon as seq appears in *flag_host (optional, page-locked host memory).
hipError_t launch_topk(const float *z, int E, int k, int score_fn, int T, int32_t *idx, float *w,
                       hipStream_t s, int32_t *idx_host = nullptr, float *w_host = nullptr,
                       uint32_t *flag_host = nullptr, uint32_t seq = 0);
// Many-token router logits: H-sliced partial sums (part: route_blocked_slices
// x T x E floats) reduced in slice order into z.  H % 64 == 0.
constexpr int kRouteMaxSlices = 64;
int route_blocked_slices(int E, int H, int T);
hipError_t launch_route_blocked(const float *W, const float *bias, int E, int H, const void *x, int x_dtype, int T,
                                float *part, float *z, hipStream_t s);
hipError_t launch_pack_x(const void *x, int x_dtype, int T, int H, int64_t x_stride, uint32_t *xh, int32_t *xexp,
                         hipStream_t s);
// n_local_total = T * src.n_local local items in the launch
hipError_t launch_rvq_gateup(const RecSrc &src, const RecOffsets &off, int H, int I, int n_local_total,
                             const uint32_t *xh, const int32_t *xexp, float *gu, hipStream_t s);
hipError_t launch_rvq_down(const RecSrc &src, const RecOffsets &off, int H, int I, int n_local_total,
                           int KS, const float *gu, float *ypart, hipStream_t s);
hipError_t launch_combine(const float *ypart, int k, int KS, int H, const float *w, const float *ysh,
                          float *out, int64_t out_stride, int T, int accumulate, hipStream_t s);
hipError_t launch_dense_gateup(const uint16_t *shared, int H, int I, const void *x, int x_dtype,
                               int64_t x_stride, int T, float *hs, hipStream_t s);
hipError_t launch_hbm_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s);
hipError_t launch_dense_down(const uint16_t *shared, int H, int I, const float *hs, int T,
                             float *ysh, hipStream_t s);

int down_splits(int H, int I, int n_items);

// ---- persistent decode (kernels_decode.hip) ----------------------------------
constexpr int kDecMaxLayers = 40;   // layer descriptors carried in one launch's arguments
// Optional per-(step, workgroup) wall-clock stamps of the decode kernel
// (profiling aid), in this order:
enum DecStamp {
    kStampStart,        // step begins
    kStampLayerWait,    // previous step's outputs all written
    kStampRouted,       // top-k known
    kStampGuStaged,     // gate/up codebooks and x in LDS, or its lookup table built (last segment)
    kStampGuLoop,       // gate/up streaming done (last segment)
    kStampGuDone,       // gate/up partials joined
    kStampSharedDown,   // shared-expert down rows done
    kStampDownStaged,   // h and the down codebook in LDS (last segment)
    kStampDownLoop,     // down streaming done (last segment)
    kStampDownDone,     // down partials and output tiles done
    kDecStamps
};

struct DecLayer {
    const float *W;
    const float *bias;
    const void *const *records;
    const uint16_t *shared;
    int32_t E, k, score_fn, pad;
};

// Phases of the decode kernel done by table lookup (bits of DecodeLaunch::lut).
constexpr int kLutGateUp = 1, kLutDown = 2;

struct DecodeLaunch {
    DecLayer layers[kDecMaxLayers];
    int nL, T, H, I, k, E_max, G, has_shared;
    const float *x;
    float *out;
    int32_t *idx_out;
    RecOffsets off;
    unsigned *sync;
    size_t clear_words;      // 32-bit words from sync on that are zeroed before the launch
                             // (the counters and every step-tagged buffer)
    DecLayer *layer_buf;     // [kDecMaxLayers] device copy of the descriptors
    uint64_t *z, *ysh, *part_gu, *part_d;   // step-tagged exchange buffers
    float *hh;               // [k][I] fp32 h (gather down)
    uint64_t *hq;            // tagged fp32 h (down by table lookup), zeroed before the launch
    float *hs;
    int slots_gu, slots_d;
    int slots_red_gu, slots_red_d;
    int lut;                 // kLutGateUp | kLutDown: phases by table lookup (decode_plan decides)
    unsigned long long *stamps;   // phase timestamps (profiling aid), or null
    int stamp_steps;
};

// Values of the decode workspace's sticky status word (32-bit word 1).
constexpr unsigned kDecodeStatusClean = 0x600D600Du, kDecodeStatusFailed = 0xBAD0BAD0u;

struct DecodePlanOut {
    int G;                        // persistent workgroups (one per CU)
    int slots_gu, slots_d;        // most contributors to one tile's partial sums
    int slots_red_gu, slots_red_d;   // most tiles one workgroup touches per phase
    int lut;                      // kLutGateUp | kLutDown: the phases done by table lookup
    size_t sync_words;
    bool lds_ok;
    bool units_ok;   // the unit spaces fit the kernel's 32-bit range arithmetic
};
// lut_mode: -1 = choose by shape, 0 = codebook gathers, 1 = table lookup
// for gate/up and down, 2 = table lookup for gate/up only (a phase whose
// shape does not allow it uses gathers).
hipError_t decode_plan(int H, int I, int k, int lut_mode, DecodePlanOut *o);
hipError_t launch_decode_persistent(const DecodeLaunch &d, hipStream_t s);

// The decode driver behind moe_decode_forward and moe_decode_forward_noalloc
// (moe_api.hip): argument checks (MOE_OK also for T = 0), the workspace size
// (with or without the optional profiling stamps), and the launches.
int decode_check_args(const moe_layer *layers, int32_t n_layers, const float *x, int32_t T, const float *out);
int decode_ws_bytes(const moe_layer *layers, int32_t n_layers, bool stamps, size_t *bytes);
int decode_forward_impl(const moe_layer *layers, int32_t n_layers, const float *x, int32_t T, float *out,
                        int32_t *idx_out, void *ws, size_t ws_bytes, bool stamps, hipStream_t s);
// Device address of the current device's no-alloc scratch array
// (decode_noalloc.hip).
int decode_noalloc_scratch(void **out);

// ---- batched path (kernels_grouped.hip) --------------------------------------
// idx: T * k expert ids, a token's k ids distinct (top-k)
hipError_t launch_group(const int32_t *idx, int n_pairs, int k, int E, int32_t *perm, int32_t *inv,
                        int32_t *counts, int32_t *offsets, hipStream_t s);
hipError_t launch_to_bf16(const void *x, int x_dtype, size_t n, uint16_t *xb, hipStream_t s);
hipError_t launch_grouped_rvq(const void *const *table, const RecOffsets &off, int E, int H, int I, int n_pairs,
                              const int32_t *counts, const int32_t *offsets, const int32_t *perm, int k,
                              const uint16_t *xb, uint16_t *hbuf, float *ybuf, hipStream_t s);
// Shared expert over all T tokens (dense bf16 GEMMs, K split into slices when
// few tokens leave the CUs idle): part holds dense_part_floats(H, I, T)
// floats; the down GEMM's *nsh slices of [T, H] partial sums stay in part for
// the combine to add.
int dense_splits(int N, int T, int K, int M);
size_t dense_part_floats(int H, int I, int T);
hipError_t launch_grouped_dense(const uint16_t *shared, int H, int I, int T, const uint16_t *xb, uint16_t *hs,
                                float *part, int *nsh, hipStream_t s);
hipError_t launch_grouped_combine(const float *ybuf, const int32_t *inv, const float *w, int k, int H, int T,
                                  const float *ysh, int nsh, float *out, hipStream_t s);

}  // namespace moe
