// C ABI of libmoe: argument validation, workspace carving and the launch
// sequences of the routed-expert MoE path.  Declarations and the meaning of
// every argument are in include/moe.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "expert_cache.h"
#include "host_tier.h"
#include "moe_internal.h"

using namespace moe;

namespace moe {
thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(MOE_E_HIP, "%s: %s", what, hipGetErrorString(e));
}
}  // namespace moe

#define HIPCHK(expr, what)                           \
    do {                                             \
        hipError_t e_ = (expr);                      \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

namespace {

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool dims_ok(int32_t H, int32_t I) { return H > 0 && I > 0 && H % 128 == 0 && I % 128 == 0; }

void layout_of(int32_t H, int32_t I, moe_record_layout *L) {
    const int64_t s[9] = {(int64_t)I * (H / 8) * 3, (int64_t)I * (H / 8) * 3, (int64_t)H * (I / 8) * 3,
                          2 * (int64_t)I, 2 * (int64_t)I, 2 * (int64_t)H,
                          (int64_t)kCbRows * 16, (int64_t)kCbRows * 16, (int64_t)kCbRows * 16};
    int64_t pos = 0;
    for (int i = 0; i < 9; i++) {
        pos = align_up(pos, 256);
        L->offset[i] = pos;
        L->size[i] = s[i];
        pos += s[i];
    }
    L->nbytes = pos;
    L->padded = align_up(pos, 4096);
}

RecOffsets offsets_of(int32_t H, int32_t I) {
    moe_record_layout L;
    layout_of(H, I, &L);
    RecOffsets o;
    for (int m = 0; m < 3; m++) {
        o.codes[m] = L.offset[m];
        o.scales[m] = L.offset[3 + m];
        o.cb[m] = L.offset[6 + m];
    }
    return o;
}

// Sequential carving of a workspace into 256-byte aligned pieces.
struct Carver {
    char *base;
    size_t pos = 0;
    explicit Carver(void *b) : base((char *)b) {}
    template <class T>
    T *take(size_t n) {
        pos = (size_t)align_up((int64_t)pos, 256);
        T *p = base ? (T *)(base + pos) : nullptr;
        pos += n * sizeof(T);
        return p;
    }
};

LayerWs carve_layer(void *ws, int H, int I, int E, int k, int T, bool shared) {
    Carver c(ws);
    LayerWs L;
    const int items = T * k;
    const int KS = down_splits(H, I, items);
    L.z = c.take<float>((size_t)T * E);
    L.idx = c.take<int32_t>((size_t)T * k);
    L.w = c.take<float>((size_t)T * k);
    L.xh = c.take<uint32_t>((size_t)T * H / 2);
    L.xexp = c.take<int32_t>((size_t)T);
    L.hh = c.take<float>((size_t)items * 2 * I);   // gate and up per item
    L.ypart = c.take<float>((size_t)items * KS * H);
    L.hs = shared ? c.take<float>((size_t)T * I) : nullptr;
    L.ysh = shared ? c.take<float>((size_t)T * H) : nullptr;
    L.bytes = (size_t)align_up((int64_t)c.pos, 256);
    return L;
}

struct GroupedWs {
    float *z, *zpart;
    int32_t *idx, *perm, *inv, *counts, *offsets;
    float *w;
    uint16_t *xb, *hbuf, *hs;
    float *ybuf, *ysh;
    size_t bytes;
};

GroupedWs carve_grouped(void *ws, int H, int I, int E, int k, int T, bool shared) {
    Carver c(ws);
    GroupedWs G;
    const size_t pairs = (size_t)T * k;
    G.z = c.take<float>((size_t)T * E);
    G.zpart = c.take<float>((size_t)route_blocked_slices(E, H, T) * T * E);
    G.idx = c.take<int32_t>(pairs);
    G.w = c.take<float>(pairs);
    G.perm = c.take<int32_t>(pairs);
    G.inv = c.take<int32_t>(pairs);
    G.counts = c.take<int32_t>((size_t)E);
    G.offsets = c.take<int32_t>((size_t)E + 1);
    G.xb = c.take<uint16_t>((size_t)T * H);
    G.hbuf = c.take<uint16_t>(pairs * I);
    G.ybuf = c.take<float>(pairs * std::max(H, 2 * I));   // y, or gate and up before it
    G.hs = shared ? c.take<uint16_t>((size_t)T * I) : nullptr;
    G.ysh = shared ? c.take<float>(dense_part_floats(H, I, T)) : nullptr;   // shared expert's partial sums
    G.bytes = (size_t)align_up((int64_t)c.pos, 256);
    return G;
}

int check_router(const moe_router *r, int32_t H) {
    if (!r) return fail(MOE_E_INVAL, "router is NULL");
    if (!r->weight) return fail(MOE_E_INVAL, "router weight is NULL");
    if (r->E < 1 || r->E > MOE_MAX_E) return fail(MOE_E_INVAL, "E=%d outside [1, %d]", r->E, MOE_MAX_E);
    if (r->k < 1 || r->k > r->E || r->k > MOE_MAX_K)
        return fail(MOE_E_INVAL, "k=%d outside [1, min(E=%d, %d)]", r->k, r->E, MOE_MAX_K);
    if (r->score_fn != MOE_SCORE_SOFTMAX && r->score_fn != MOE_SCORE_SIGMOID)
        return fail(MOE_E_INVAL, "unknown score_fn %d", r->score_fn);
    if (H <= 0 || H % 128) return fail(MOE_E_INVAL, "H=%d is not a positive multiple of 128", H);
    return MOE_OK;
}

int check_layer(const moe_layer *L, bool need_records) {
    if (!L) return fail(MOE_E_INVAL, "layer is NULL");
    if (!dims_ok(L->H, L->I))
        return fail(MOE_E_INVAL, "H=%d, I=%d must be positive multiples of 128", L->H, L->I);
    int rc = check_router(&L->router, L->H);
    if (rc) return rc;
    if (need_records && !L->records) return fail(MOE_E_INVAL, "records table is NULL");
    return MOE_OK;
}

bool dtype_ok(int32_t d) { return d == MOE_DTYPE_F32 || d == MOE_DTYPE_BF16; }

// route -> pack -> gate/up -> down (+ shared) -> combine for T tokens whose
// experts come from `src` (table mode: idx filled by the router).
int run_experts(const moe_layer *L, const LayerWs &ws, const RecSrc &src, const void *x, int32_t x_dtype,
                int32_t T, int k, const float *w, float *out, hipStream_t s) {
    const int H = L->H, I = L->I, items = T * k;
    const RecOffsets off = offsets_of(H, I);
    const int KS = down_splits(H, I, items);
    HIPCHK(launch_pack_x(x, x_dtype, T, H, H, ws.xh, ws.xexp, s), "pack_x launch");
    if (L->shared) HIPCHK(launch_dense_gateup(L->shared, H, I, x, x_dtype, H, T, ws.hs, s), "shared gate/up launch");
    HIPCHK(launch_rvq_gateup(src, off, H, I, items, ws.xh, ws.xexp, ws.hh, s), "rvq gate/up launch");
    HIPCHK(launch_rvq_down(src, off, H, I, items, KS, ws.hh, ws.ypart, s), "rvq down launch");
    if (L->shared) HIPCHK(launch_dense_down(L->shared, H, I, ws.hs, T, ws.ysh, s), "shared down launch");
    HIPCHK(launch_combine(ws.ypart, k, KS, H, w, L->shared ? ws.ysh : nullptr, out, H, T, 0, s), "combine launch");
    return MOE_OK;
}

}  // namespace

extern "C" {

const char *moe_last_error(void) { return g_err.c_str(); }

int moe_abi_version(void) { return MOE_ABI_VERSION; }

int moe_hbm_read(const void *buf, uint64_t bytes, uint32_t *sink, void *hip_stream) {
    if ((!buf && bytes) || !sink) return fail(MOE_E_INVAL, "buf (unless bytes = 0) and sink must be non-NULL");
    if ((uintptr_t)buf % 16 || bytes % 16)
        return fail(MOE_E_INVAL, "buf must be 16-byte aligned and bytes a multiple of 16 (bytes=%llu)",
                    (unsigned long long)bytes);
    HIPCHK(launch_hbm_read(buf, (size_t)bytes, sink, (hipStream_t)hip_stream), "hbm read launch");
    return MOE_OK;
}

int moe_rvq_record_layout(int32_t H, int32_t I, moe_record_layout *out) {
    if (!out) return fail(MOE_E_INVAL, "out is NULL");
    if (!dims_ok(H, I)) return fail(MOE_E_INVAL, "H=%d, I=%d must be positive multiples of 128", H, I);
    layout_of(H, I, out);
    return MOE_OK;
}

size_t moe_route_workspace_bytes(int32_t E, int32_t T) {
    if (E < 1 || T < 0) return 0;
    return (size_t)align_up((int64_t)E * T * 4, 256);
}

int moe_route_topk(const moe_router *r, const void *x, int32_t x_dtype, int32_t T, int32_t H, int32_t *idx,
                   float *w, void *ws, size_t ws_bytes, void *hip_stream) {
    int rc = check_router(r, H);
    if (rc) return rc;
    if (T < 0) return fail(MOE_E_INVAL, "T=%d < 0", T);
    if (!dtype_ok(x_dtype)) return fail(MOE_E_INVAL, "unknown x dtype %d", x_dtype);
    if (T == 0) return MOE_OK;
    if (!x || !idx || !w || !ws) return fail(MOE_E_INVAL, "x, idx, w and ws must be non-NULL");
    if (ws_bytes < moe_route_workspace_bytes(r->E, T))
        return fail(MOE_E_SPACE, "workspace %zu < %zu bytes", ws_bytes, moe_route_workspace_bytes(r->E, T));
    hipStream_t s = (hipStream_t)hip_stream;
    HIPCHK(launch_route_logits(r->weight, r->bias, r->E, H, x, x_dtype, T, (float *)ws, s), "route logits launch");
    HIPCHK(launch_topk((const float *)ws, r->E, r->k, r->score_fn, T, idx, w, s), "top-k launch");
    return MOE_OK;
}

size_t moe_expert_ffn_workspace_bytes(int32_t H, int32_t I, int32_t T) {
    if (!dims_ok(H, I) || T < 0) return 0;
    return carve_layer(nullptr, H, I, 1, 1, std::max(T, 1), false).bytes;
}

int moe_expert_ffn_rvq(const void *record, int32_t H, int32_t I, const float *x, int32_t T, const float *gate_w,
                       float *y, int32_t accumulate, void *ws, size_t ws_bytes, void *hip_stream) {
    if (!dims_ok(H, I)) return fail(MOE_E_INVAL, "H=%d, I=%d must be positive multiples of 128", H, I);
    if (T < 0) return fail(MOE_E_INVAL, "T=%d < 0", T);
    if (T == 0) return MOE_OK;
    if (!record || !x || !y || !ws) return fail(MOE_E_INVAL, "record, x, y and ws must be non-NULL");
    if ((uintptr_t)record % 256) return fail(MOE_E_INVAL, "record must be 256-byte aligned");
    const size_t need = moe_expert_ffn_workspace_bytes(H, I, T);
    if (ws_bytes < need) return fail(MOE_E_SPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    hipStream_t s = (hipStream_t)hip_stream;
    const LayerWs L = carve_layer(ws, H, I, 1, 1, T, false);
    RecSrc src{};
    src.list[0] = record;
    src.rank[0] = 0;
    src.k = 1;
    src.n_local = 1;
    const RecOffsets off = offsets_of(H, I);
    const int KS = down_splits(H, I, T);
    HIPCHK(launch_pack_x(x, MOE_DTYPE_F32, T, H, H, L.xh, L.xexp, s), "pack_x launch");
    HIPCHK(launch_rvq_gateup(src, off, H, I, T, L.xh, L.xexp, L.hh, s), "rvq gate/up launch");
    HIPCHK(launch_rvq_down(src, off, H, I, T, KS, L.hh, L.ypart, s), "rvq down launch");
    HIPCHK(launch_combine(L.ypart, 1, KS, H, gate_w, nullptr, y, H, T, accumulate, s), "combine launch");
    return MOE_OK;
}

size_t moe_layer_workspace_bytes(const moe_layer *L, int32_t T) {
    if (!L || !dims_ok(L->H, L->I) || L->router.E < 1 || L->router.k < 1 || T < 0) return 0;
    return carve_layer(nullptr, L->H, L->I, L->router.E, L->router.k, std::max(T, 1), L->shared != nullptr).bytes;
}

int moe_layer_forward(const moe_layer *L, const void *x, int32_t x_dtype, int32_t T, float *out, int32_t *idx_out,
                      float *w_out, void *ws, size_t ws_bytes, void *hip_stream) {
    int rc = check_layer(L, true);
    if (rc) return rc;
    if (T < 0) return fail(MOE_E_INVAL, "T=%d < 0", T);
    if (!dtype_ok(x_dtype)) return fail(MOE_E_INVAL, "unknown x dtype %d", x_dtype);
    if (T == 0) return MOE_OK;
    if (!x || !out || !ws) return fail(MOE_E_INVAL, "x, out and ws must be non-NULL");
    const size_t need = moe_layer_workspace_bytes(L, T);
    if (ws_bytes < need) return fail(MOE_E_SPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    hipStream_t s = (hipStream_t)hip_stream;
    const int E = L->router.E, k = L->router.k;
    const LayerWs W = carve_layer(ws, L->H, L->I, E, k, T, L->shared != nullptr);
    int32_t *idx = idx_out ? idx_out : W.idx;
    float *w = w_out ? w_out : W.w;
    HIPCHK(launch_route_logits(L->router.weight, L->router.bias, E, L->H, x, x_dtype, T, W.z, s),
           "route logits launch");
    HIPCHK(launch_topk(W.z, E, k, L->router.score_fn, T, idx, w, s), "top-k launch");
    RecSrc src{};
    src.table = L->records;
    src.idx = idx;
    src.k = k;
    src.n_local = k;
    return run_experts(L, W, src, x, x_dtype, T, k, w, out, s);
}

}  // extern "C"

namespace {
struct DecodeWs {
    unsigned *sync;
    DecLayer *layers;
    uint64_t *z, *ysh, *part_gu, *part_d;
    float *hh;
    uint64_t *hq;
    float *hs;
    unsigned long long *stamps;
    int stamp_steps;
    int G, slots_gu, slots_d, slots_red_gu, slots_red_d, lut;
    size_t sync_words, clear_words, bytes;
};

// Profiling aid: MOE_DECODE_STAMPS=<n> makes the decode workspace end with
// n steps x G workgroups x kDecStamps wall-clock stamps (see DecStamp).
int decode_stamp_steps() {
    const char *e = getenv("MOE_DECODE_STAMPS");
    return e ? std::max(0, atoi(e)) : 0;
}

// MOE_DECODE_LUT forces the decode kernel's methods: 0 codebook gathers, 1
// table lookup for gate/up and down, 2 table lookup for gate/up only; unset,
// the shape decides.
int decode_lut_mode() {
    const char *e = getenv("MOE_DECODE_LUT");
    if (!e || !*e) return -1;
    const int v = atoi(e);
    return v == 2 ? 2 : (v ? 1 : 0);
}

int carve_decode(void *ws, const moe_layer *layers, int32_t n_layers, DecodeWs *D, bool stamps = true) {
    const int H = layers[0].H, I = layers[0].I, k = layers[0].router.k;
    int E_max = 1;
    bool shared = false;
    for (int l = 0; l < n_layers; l++) {
        E_max = std::max(E_max, layers[l].router.E);
        shared = shared || layers[l].shared;
    }
    DecodePlanOut P;
    hipError_t e = decode_plan(H, I, k, decode_lut_mode(), &P);
    if (e != hipSuccess) return hip_fail(e, "decode plan");
    if (!P.lds_ok) return fail(MOE_E_INVAL, "decode kernel: H=%d, I=%d do not fit its LDS layout", H, I);
    if (!P.units_ok) return fail(MOE_E_INVAL, "decode kernel: k=%d, H=%d, I=%d exceed its work-range arithmetic", k, H, I);
    D->G = P.G;
    D->slots_gu = P.slots_gu;
    D->slots_d = P.slots_d;
    D->slots_red_gu = P.slots_red_gu;
    D->slots_red_d = P.slots_red_d;
    D->lut = P.lut;
    D->sync_words = P.sync_words;
    Carver c(ws);
    // zeroed before every launch: the counters (word 0 is the launch's
    // abort flag; word 1, the sticky status that moe_decode_status reads, is
    // kept), then the step-tagged buffers
    D->sync = c.take<unsigned>(D->sync_words);
    D->z = c.take<uint64_t>((size_t)E_max);
    D->ysh = c.take<uint64_t>((size_t)H);
    // table-lookup partials pack two rows per word: half the words per tile
    D->part_gu = c.take<uint64_t>((size_t)k * (I / 64) * D->slots_gu * ((D->lut & kLutGateUp) ? 64 : 128));
    D->part_d = c.take<uint64_t>((size_t)k * (H / 64) * D->slots_d * ((D->lut & kLutDown) ? 32 : 64));
    D->hq = (D->lut & kLutDown) ? c.take<uint64_t>((size_t)k * I) : nullptr;
    D->clear_words = c.pos / 4;
    D->layers = c.take<DecLayer>(kDecMaxLayers);
    D->hh = c.take<float>((size_t)k * I);
    D->hs = c.take<float>((size_t)I);
    D->stamp_steps = stamps ? decode_stamp_steps() : 0;
    D->stamps = D->stamp_steps ? c.take<unsigned long long>((size_t)D->stamp_steps * D->G * kDecStamps) : nullptr;
    D->bytes = (size_t)align_up((int64_t)c.pos, 256);
    (void)shared;
    return MOE_OK;
}
}  // namespace

namespace moe {
int decode_check_args(const moe_layer *layers, int32_t n_layers, const float *x, int32_t T, const float *out) {
    if (!layers || n_layers < 1) return fail(MOE_E_INVAL, "layers is NULL or n_layers < 1");
    for (int l = 0; l < n_layers; l++) {
        int rc = check_layer(&layers[l], true);
        if (rc) return rc;
        if (layers[l].H != layers[0].H || layers[l].I != layers[0].I || layers[l].router.k != layers[0].router.k ||
            layers[l].router.E != layers[0].router.E)
            return fail(MOE_E_INVAL, "layer %d differs from layer 0 in H, I, E or k", l);
    }
    if (T < 0) return fail(MOE_E_INVAL, "T=%d < 0", T);
    if (T == 0) return MOE_OK;
    if (!x || !out) return fail(MOE_E_INVAL, "x and out must be non-NULL");
    return MOE_OK;
}

int decode_ws_bytes(const moe_layer *layers, int32_t n_layers, bool stamps, size_t *bytes) {
    if (!layers || n_layers < 1 || !dims_ok(layers[0].H, layers[0].I) || layers[0].router.k < 1)
        return fail(MOE_E_INVAL, "decode workspace: invalid layers, n_layers or shapes");
    DecodeWs D;
    int rc = carve_decode(nullptr, layers, n_layers, &D, stamps);
    if (rc) return rc;
    *bytes = D.bytes;
    return MOE_OK;
}

int decode_forward_impl(const moe_layer *layers, int32_t n_layers, const float *x, int32_t T, float *out,
                        int32_t *idx_out, void *ws, size_t ws_bytes, bool stamps, hipStream_t s) {
    DecodeWs D;
    int rc = carve_decode(ws, layers, n_layers, &D, stamps);
    if (rc) return rc;
    if (ws_bytes < D.bytes) return fail(MOE_E_SPACE, "workspace %zu < %zu bytes", ws_bytes, D.bytes);
    const int H = layers[0].H, I = layers[0].I, k = layers[0].router.k;
    DecodeLaunch d{};
    d.H = H;
    d.I = I;
    d.k = k;
    d.E_max = layers[0].router.E;
    d.G = D.G;
    d.off = offsets_of(H, I);
    d.sync = D.sync;
    d.clear_words = D.clear_words;
    d.layer_buf = D.layers;
    d.z = D.z;
    d.hh = D.hh;
    d.hq = D.hq;
    d.hs = D.hs;
    d.ysh = D.ysh;
    d.part_gu = D.part_gu;
    d.part_d = D.part_d;
    d.slots_gu = D.slots_gu;
    d.slots_d = D.slots_d;
    d.slots_red_gu = D.slots_red_gu;
    d.slots_red_d = D.slots_red_d;
    d.lut = D.lut;
    d.stamps = D.stamps;
    d.stamp_steps = D.stamp_steps;
    auto set_layers = [&](int l0, int nl) {
        d.nL = nl;
        d.has_shared = 0;
        for (int l = 0; l < nl; l++) {
            const moe_layer &L = layers[l0 + l];
            d.layers[l] = DecLayer{L.router.weight, L.router.bias, L.records, L.shared, L.router.E, L.router.k,
                                   L.router.score_fn, 0};
            d.has_shared |= L.shared != nullptr;
        }
    };
    if (n_layers <= kDecMaxLayers) {
        // the whole decode in one launch
        set_layers(0, n_layers);
        d.T = T;
        d.x = x;
        d.out = out;
        d.idx_out = idx_out;
        HIPCHK(launch_decode_persistent(d, s), "persistent decode launch");
        return MOE_OK;
    }
    // more layers than one launch carries: one launch per (token, layer group)
    for (int t = 0; t < T; t++) {
        for (int l0 = 0; l0 < n_layers; l0 += kDecMaxLayers) {
            const int nl = std::min(kDecMaxLayers, n_layers - l0);
            set_layers(l0, nl);
            d.T = 1;
            d.x = x + ((size_t)t * n_layers + l0) * H;
            d.out = out + ((size_t)t * n_layers + l0) * H;
            d.idx_out = idx_out ? idx_out + ((size_t)t * n_layers + l0) * k : nullptr;
            HIPCHK(launch_decode_persistent(d, s), "persistent decode launch");
        }
    }
    return MOE_OK;
}
}  // namespace moe

extern "C" {

size_t moe_decode_workspace_bytes(const moe_layer *layers, int32_t n_layers) {
    size_t n = 0;
    return decode_ws_bytes(layers, n_layers, true, &n) == MOE_OK ? n : 0;
}

int moe_decode_forward(const moe_layer *layers, int32_t n_layers, const float *x, int32_t T, float *out,
                       int32_t *idx_out, void *ws, size_t ws_bytes, void *hip_stream) {
    int rc = decode_check_args(layers, n_layers, x, T, out);
    if (rc || T == 0) return rc;
    if (!ws) return fail(MOE_E_INVAL, "ws must be non-NULL");
    return decode_forward_impl(layers, n_layers, x, T, out, idx_out, ws, ws_bytes, true, (hipStream_t)hip_stream);
}

static int decode_method(const moe_layer *layers, int32_t n_layers, int32_t *method, int bit) {
    if (!layers || n_layers < 1 || !method) return fail(MOE_E_INVAL, "layers or method is NULL, or n_layers < 1");
    if (!dims_ok(layers[0].H, layers[0].I) || layers[0].router.k < 1)
        return fail(MOE_E_INVAL, "invalid layer shape");
    DecodeWs D;
    int rc = carve_decode(nullptr, layers, n_layers, &D);
    if (rc) return rc;
    *method = (D.lut & bit) ? 1 : 0;
    return MOE_OK;
}

int moe_decode_gate_up_method(const moe_layer *layers, int32_t n_layers, int32_t *method) {
    return decode_method(layers, n_layers, method, kLutGateUp);
}

int moe_decode_down_method(const moe_layer *layers, int32_t n_layers, int32_t *method) {
    return decode_method(layers, n_layers, method, kLutDown);
}

int moe_decode_status(const void *ws, int32_t *timed_out) {
    if (!timed_out) return fail(MOE_E_INVAL, "timed_out must be non-NULL");
    if (!ws) {
        // the current device's scratch array of moe_decode_forward_noalloc
        void *p = nullptr;
        int rc = decode_noalloc_scratch(&p);
        if (rc) return rc;
        ws = p;
    }
    // the sticky status is 32-bit word 1 of the workspace (the counters
    // come first); the device is idle once hipDeviceSynchronize returns
    unsigned *word = (unsigned *)ws + 1;
    unsigned v = 0;
    HIPCHK(hipDeviceSynchronize(), "synchronise before reading the decode status");
    HIPCHK(hipMemcpy(&v, word, sizeof v, hipMemcpyDeviceToHost), "read decode status");
    *timed_out = v == kDecodeStatusFailed;
    if (*timed_out) {
        const unsigned clean = kDecodeStatusClean;
        HIPCHK(hipMemcpy(word, &clean, sizeof clean, hipMemcpyHostToDevice), "reset decode status");
    }
    return MOE_OK;
}

// Look-ahead region after the layer's own workspace: the next layer's
// logits, predicted ids and (unused) weights.
constexpr size_t kAheadBytes = MOE_MAX_E * sizeof(float) + 256 + 2 * MOE_MAX_K * sizeof(float) + 256;

size_t moe_streamed_workspace_bytes(const moe_layer *L, int32_t T) {
    const size_t b = moe_layer_workspace_bytes(L, T);
    return b ? b + kAheadBytes : 0;
}

}  // extern "C"

namespace {
struct Ahead {
    const moe_layer *L = nullptr;          // next layer, or null: no look-ahead
    uint32_t layer_id = 0;
    const void *const *host = nullptr;
    int k = 0;
    float min_weight = 0.f;                // predictions with a smaller weight are not read ahead
};
struct Tier {
    moe_host_tier *t = nullptr;            // file tier, or null: records from experts_host
    int64_t record0 = 0;
};

int streamed_impl(const moe_layer *L, moe_cache *c, uint32_t layer_id, const void *const *experts_host,
                  const float *x, int32_t T, float *out, int32_t *idx_out, void *ws, size_t ws_bytes,
                  void *compute_stream, void *copy_stream, const Ahead &ah, const Tier &tier = Tier{}) {
    int rc = check_layer(L, false);
    if (rc) return rc;
    if (!c) return fail(MOE_E_INVAL, "cache is NULL");
    if (T < 0 || T > 1) return fail(MOE_E_INVAL, "streamed decode takes T = 1 token (got %d)", T);
    if (T == 0) return MOE_OK;
    if ((!experts_host && !tier.t) || !x || !out || !ws)
        return fail(MOE_E_INVAL, "experts_host (or a tier), x, out and ws must be non-NULL");
    const int H = L->H, I = L->I, E = L->router.E, k = L->router.k;
    if (c->core.capacity() < k)
        return fail(MOE_E_INVAL, "cache capacity %d is below k = %d: the layer cannot hold one token's experts",
                    c->core.capacity(), k);
    moe_record_layout lay;
    layout_of(H, I, &lay);
    if ((int64_t)c->slot_bytes < lay.nbytes)
        return fail(MOE_E_INVAL, "slot size %llu is below the record size %lld", (unsigned long long)c->slot_bytes,
                    (long long)lay.nbytes);
    if ((uint64_t)layer_id * (uint64_t)E + (uint64_t)E - 1 >= (uint64_t)MOE_NO_KEY)
        return fail(MOE_E_INVAL, "layer_id * E overflows the 32-bit key");
    const size_t need = moe_streamed_workspace_bytes(L, T);
    if (ws_bytes < need) return fail(MOE_E_SPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    if (ah.L) {
        rc = check_layer(ah.L, false);
        if (rc) return rc;
        if (ah.L->H != H) return fail(MOE_E_INVAL, "next layer H=%d differs from this layer's %d", ah.L->H, H);
        if (ah.k < 1 || ah.k > ah.L->router.E || ah.k > MOE_MAX_K || ah.k > c->core.capacity())
            return fail(MOE_E_INVAL, "look-ahead k=%d must be in 1..min(E, %d, capacity)", ah.k, MOE_MAX_K);
        if (!ah.host) return fail(MOE_E_INVAL, "next layer's experts_host is NULL");
        if ((uint64_t)ah.layer_id * (uint64_t)ah.L->router.E + (uint64_t)ah.L->router.E - 1 >= (uint64_t)MOE_NO_KEY)
            return fail(MOE_E_INVAL, "next layer_id * E overflows the 32-bit key");
        moe_record_layout nlay;
        layout_of(ah.L->H, ah.L->I, &nlay);
        if ((int64_t)c->slot_bytes < nlay.nbytes)
            return fail(MOE_E_INVAL, "slot size is below the next layer's record size");
    }
    hipStream_t cs = (hipStream_t)compute_stream, ps = (hipStream_t)copy_stream;
    const LayerWs W = carve_layer(ws, H, I, E, k, 1, L->shared != nullptr);
    float *za = nullptr, *wa = nullptr;
    int32_t *ia = nullptr;
    {
        Carver ca((char *)ws + moe_layer_workspace_bytes(L, T));
        za = ca.take<float>(MOE_MAX_E);
        ia = ca.take<int32_t>(MOE_MAX_K);
        wa = ca.take<float>(MOE_MAX_K);
    }
    int32_t *h_ahead = c->h_idx + MOE_MAX_K;
    float *h_ahead_w = (float *)(c->h_idx + 2 * MOE_MAX_K);
    int32_t *idx = idx_out ? idx_out : W.idx;
    const RecOffsets off = offsets_of(H, I);
    const int KS = down_splits(H, I, k);

    // route; the host waits only for the expert ids, while the work that does
    // not depend on the choice (x packing, the shared expert) runs on
    HIPCHK(launch_route_logits(L->router.weight, L->router.bias, E, H, x, MOE_DTYPE_F32, 1, W.z, cs), "route logits");
    // ids to the host too, with a sequence flag after them (1, 2, ..., skipping 0)
    const uint32_t seq = ++c->ids_seq ? c->ids_seq : ++c->ids_seq;
    uint32_t *ids_flag = (uint32_t *)(c->h_idx + kIdsFlag);
    HIPCHK(launch_topk(W.z, E, k, L->router.score_fn, 1, idx, W.w, cs, c->h_idx, nullptr, ids_flag, seq), "top-k");
    HIPCHK(hipEventRecord(c->idx_ev, cs), "ids written");
    if (ah.L) {
        // the next layer's router on this layer's input: a prediction only
        HIPCHK(launch_route_logits(ah.L->router.weight, ah.L->router.bias, ah.L->router.E, H, x, MOE_DTYPE_F32, 1, za,
                                   cs), "look-ahead logits");
        HIPCHK(launch_topk(za, ah.L->router.E, ah.k, ah.L->router.score_fn, 1, ia, wa, cs, h_ahead, h_ahead_w),
               "look-ahead top-k");
        HIPCHK(hipEventRecord(c->ahead_ev, cs), "look-ahead ids written");
    }
    HIPCHK(launch_pack_x(x, MOE_DTYPE_F32, 1, H, H, W.xh, W.xexp, cs), "pack_x");
    if (L->shared) {
        HIPCHK(launch_dense_gateup(L->shared, H, I, x, MOE_DTYPE_F32, H, 1, W.hs, cs), "shared gate/up");
        HIPCHK(launch_dense_down(L->shared, H, I, W.hs, 1, W.ysh, cs), "shared down");
    }
    // the ids are readable once the flag shows this call's sequence number
    // (written by the top-k after them, before its completion is signalled);
    // past a bound (the stream may still be busy with earlier work) the
    // event's wait takes over, which also reports a failed launch
    {
        const auto t0 = std::chrono::steady_clock::now();
        bool seen = false;
        for (int n = 0;; n++) {
            if (__atomic_load_n(ids_flag, __ATOMIC_ACQUIRE) == seq) { seen = true; break; }
            if ((n & 255) == 255 && std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(2)) break;
        }
        if (!seen) HIPCHK(hipEventSynchronize(c->idx_ev), "wait for the expert ids");
    }

    // cache bookkeeping in ascending expert id (get-or-insert, the LRU order
    // the trace records); the copies of misses are enqueued after the hit
    // experts have been launched, so those compute while the copies run (and
    // while the host is held by copies from pageable memory)
    int order[MOE_MAX_K];
    for (int j = 0; j < k; j++) {
        order[j] = j;
        if (c->h_idx[j] < 0 || c->h_idx[j] >= E) return fail(MOE_E_HIP, "router produced expert id %d", c->h_idx[j]);
        if (!tier.t && !experts_host[c->h_idx[j]]) return fail(MOE_E_INVAL, "experts_host[%d] is NULL", c->h_idx[j]);
    }
    std::sort(order, order + k, [&](int a, int b) { return c->h_idx[a] < c->h_idx[b]; });
    int32_t slot_of[MOE_MAX_K];
    bool hit[MOE_MAX_K];
    // exclusive host tier: per miss, the page its record comes from (-1: the
    // file) and the page the HBM cache's evicted key moves to (-1: none)
    moe_host_tier *X = tier.t && tier.t->exclusive ? tier.t : nullptr;
    int32_t spage[MOE_MAX_K], vpage[MOE_MAX_K];
    int32_t transit[MOE_MAX_K];
    int ntransit = 0;
    // pages in transit are free again when this call returns, on every path
    // (a page's event says when its last copy is done)
    struct TransitBack {
        moe_host_tier *X;
        const int32_t *pages;
        const int *n;
        ~TransitBack() {
            if (X)
                for (int q = 0; q < *n; q++) X->free_pages.push_back(pages[q]);
        }
    } transit_back{X, transit, &ntransit};
    for (int n = 0; n < k; n++) {
        const int j = order[n];
        const uint32_t key = layer_id * (uint32_t)E + (uint32_t)c->h_idx[j];
        int32_t s = c->core.lookup(key);
        hit[j] = s >= 0;
        spage[j] = vpage[j] = -1;
        if (s < 0) {
            if (X) {
                // the lower tier: a key found there leaves it (its page is in
                // transit until this call's copies are enqueued)
                const int32_t h = X->core.probe(key);
                if (h >= 0) {
                    spage[j] = transit[ntransit++] = X->page_of[h];
                    X->page_of[h] = -1;
                    X->core.drop_slot(h);
                }
            }
            uint32_t victim = kNoKey;
            s = c->core.plan_insert(key, &victim);
            const bool demote = X && victim != kNoKey && c->filled[s];
            c->core.commit_insert(key, s, victim);
            c->filled[s] = 0;                 // until its copy is enqueued below
            if (demote) {
                // the evicted key moves down, at the lower tier's most recent end
                uint32_t gone = kNoKey;
                const int32_t hv = X->core.insert_kind(victim, kTraceDemote, &gone);
                if (gone == kNoKey) {
                    rc = tier_take_page(X, false, X->down, &X->page_of[hv]);
                    if (rc) {
                        X->core.drop_slot(hv);      // no page: the key is not kept
                        return rc;
                    }
                }
                vpage[j] = X->page_of[hv];     // a key that left the tier leaves its page to this one
                X->demotions++;
            }
        }
        slot_of[j] = s;
    }

    // misses in copy order: records in page-locked memory first (ascending
    // id), then pageable ones (ascending id), so the host threads stage a
    // pageable record while the copy engine moves the page-locked ones.  (The
    // cache's operations were all done above, in ascending id; only the
    // copies' order differs.)
    int morder[MOE_MAX_K], nmiss = 0, nlocked = 0;
    for (int pass = 0; pass < 2; pass++)
        for (int n = 0; n < k; n++) {
            const int j = order[n];
            if (hit[j]) continue;
            const bool locked = tier.t || host_page_locked(experts_host[c->h_idx[j]]);
            if (locked == (pass == 0)) morder[nmiss++] = j;
            if (locked && pass == 0) nlocked++;
        }
    const char *src_of[MOE_MAX_K] = {};
    // an event not yet complete: stream st waits for it
    auto after = [&](hipStream_t st, hipEvent_t ev) {
        hipError_t q = hipEventQuery(ev);
        return q == hipErrorNotReady ? hipStreamWaitEvent(st, ev, 0) : q;
    };
    // a miss's copy into its slot on copy stream ps (or the cache's second
    // one), after the slot's previous copy (which may have been on the other
    // stream) and readers (and, with an exclusive host tier, after the slot's
    // old record has been copied down to its page)
    auto copy_miss = [&](int j, hipStream_t ps) -> int {
        const int32_t s = slot_of[j];
        HIPCHK(after(ps, c->ready[s]), "copy waits for the slot's previous copy");
        HIPCHK(cache_wait_readers(c, s, ps), "copy waits for slot readers");
        if (vpage[j] >= 0) {
            // the evicted record goes down on the tier's own stream (the link
            // carries it while the copy stream moves records up), after the
            // slot's record landed and the page's last copy; the copy up into
            // the slot waits for it
            const int32_t vp = vpage[j];
            HIPCHK(after(X->down, c->ready[s]), "demotion waits for the slot's record");
            if (X->pending[vp]) HIPCHK(after(X->down, X->copied[vp]), "demotion waits for the page");
            HIPCHK(hipMemcpyAsync(tier_page(X, vp), c->pool + (size_t)s * c->slot_bytes, c->slot_bytes,
                                  hipMemcpyDeviceToHost, X->down), "demotion copy");
            int r = tier_page_copied(X, vp, X->down);
            if (r) return r;
            HIPCHK(hipStreamWaitEvent(ps, X->copied[vp], 0), "copy up waits for the copy down");
        }
        if (X && X->pending[(int32_t)((src_of[j] - X->pool) / (ptrdiff_t)X->record_bytes)])
            HIPCHK(after(ps, X->copied[(int32_t)((src_of[j] - X->pool) / (ptrdiff_t)X->record_bytes)]),
                   "copy up waits for its page");
        const void *src = tier.t ? (const void *)src_of[j] : experts_host[c->h_idx[j]];
        bool enqueued = false;   // the key is committed either way: a failed copy drops its slot
        hipError_t e = tier.t ? hipMemcpyAsync(c->pool + (size_t)s * c->slot_bytes, src, c->slot_bytes,
                                               hipMemcpyHostToDevice, ps)
                              : cache_copy_in(c, s, src, ps, &enqueued);
        if (e == hipSuccess && tier.t) {
            const int trc = X ? tier_page_copied(X, (int32_t)((src_of[j] - X->pool) / (ptrdiff_t)X->record_bytes), ps)
                              : tier_copied(tier.t, src_of[j], ps);
            if (trc) {
                c->core.drop_slot(s);
                return trc;
            }
        }
        if (e == hipSuccess) e = hipEventRecord(c->ready[s], ps);
        if (e != hipSuccess) {
            c->core.drop_slot(s);             // the slot's contents are unknown now
            return hip_fail(e, "expert copy");
        }
        c->filled[s] = 1;
        return MOE_OK;
    };
    // misses' experts js[0..nj), once their copies have landed, in one launch
    // each for gate/up and down (an expert's result does not depend on which
    // others share the launch)
    auto run_misses = [&](const int *js, int nj) -> int {
        RecSrc src{};
        src.k = k;
        src.n_local = nj;
        for (int q = 0; q < nj; q++) {
            const int32_t s = slot_of[js[q]];
            int r = cache_wait(c, s, cs);
            if (r) return r;
            src.list[q] = c->pool + (size_t)s * c->slot_bytes;
            src.rank[q] = js[q];
        }
        HIPCHK(launch_rvq_gateup(src, off, H, I, nj, W.xh, W.xexp, W.hh, cs), "rvq gate/up (misses)");
        HIPCHK(launch_rvq_down(src, off, H, I, nj, KS, W.hh, W.ypart, cs), "rvq down (misses)");
        return MOE_OK;
    };
    // the hit experts, all at once
    auto run_hits = [&]() -> int {
        RecSrc hits{};
        hits.k = k;
        for (int n = 0; n < k; n++) {
            const int j = order[n];
            if (!hit[j]) continue;
            int r = cache_wait(c, slot_of[j], cs);
            if (r) return r;
            hits.list[hits.n_local] = c->pool + (size_t)slot_of[j] * c->slot_bytes;
            hits.rank[hits.n_local] = j;
            hits.n_local++;
        }
        if (hits.n_local) {
            HIPCHK(launch_rvq_gateup(hits, off, H, I, hits.n_local, W.xh, W.xexp, W.hh, cs), "rvq gate/up (hits)");
            HIPCHK(launch_rvq_down(hits, off, H, I, hits.n_local, KS, W.hh, W.ypart, cs), "rvq down (hits)");
        }
        return MOE_OK;
    };
    // The misses' copies alternate between the caller's copy stream and the
    // cache's own (copy n on the second when n is odd), so consecutive misses
    // n, n+1 land together and their experts run as one pair.  On every path
    // out of the miss loops (an error included) the caller's copy stream
    // waits for the second one once that one has a copy.
    struct Join {
        moe_cache *c;
        hipStream_t ps;
        bool used = false;
        hipError_t run() {
            if (!used) return hipSuccess;
            used = false;
            hipError_t e = hipEventRecord(c->ps2_done, c->ps2);
            return e == hipSuccess ? hipStreamWaitEvent(ps, c->ps2_done, 0) : e;
        }
        ~Join() { (void)run(); }
    } join{c, ps};
    auto copy_ps = [&](int n) {
        if (n % 2 == 0) return ps;
        join.used = true;
        return c->ps2;
    };
    // misses morder[0..nmiss) copied and run in pairs
    auto copy_run_pairs = [&]() -> int {
        for (int n = 0; n < nmiss; n += 2) {
            const int nj = std::min(2, nmiss - n);
            for (int q = 0; q < nj; q++) {
                const int r = copy_miss(morder[n + q], copy_ps(n + q));
                if (r) return r;
            }
            const int r = run_misses(morder + n, nj);
            if (r) return r;
        }
        return MOE_OK;
    };
    if (!tier.t) {
        // page-locked misses' copies first (the copy engine starts at once),
        // then the hit experts, then the misses' experts
        for (int n = 0; n < nlocked; n++)
            if ((rc = copy_miss(morder[n], copy_ps(n)))) return rc;
        if ((rc = run_hits())) return rc;
        for (int n = 0; n < nlocked; n += 2)
            if ((rc = run_misses(morder + n, std::min(2, nlocked - n)))) return rc;
        for (int n = nlocked; n < nmiss; n += 2) {
            const int nj = std::min(2, nmiss - n);
            for (int q = 0; q < nj; q++)
                if ((rc = copy_miss(morder[n + q], copy_ps(n + q)))) return rc;
            if ((rc = run_misses(morder + n, nj))) return rc;
        }
        HIPCHK(join.run(), "copy stream waits for the second");
    } else if (X) {
        // exclusive host tier: the hit experts run while the records found in
        // neither tier are read from the file into transit pages; then the
        // misses' copies (down, then up) in ascending id
        if ((rc = run_hits())) return rc;
        int64_t recs[MOE_MAX_K];
        int32_t pages[MOE_MAX_K];
        int nr = 0;
        for (int n = 0; n < nmiss; n++) {
            const int j = morder[n];
            if (spage[j] >= 0) continue;
            rc = tier_take_page(X, true, ps, &spage[j]);
            if (rc) return rc;
            transit[ntransit++] = spage[j];
            recs[nr] = tier.record0 + c->h_idx[j];
            pages[nr++] = spage[j];
        }
        rc = tier_read_pages(X, recs, pages, nr);
        if (rc) {
            for (int n = 0; n < nmiss; n++) c->core.drop_slot(slot_of[morder[n]]);   // never filled
            return rc;
        }
        for (int n = 0; n < nmiss; n++) src_of[morder[n]] = tier_page(X, spage[morder[n]]);
        if ((rc = copy_run_pairs())) return rc;
        HIPCHK(join.run(), "copy stream waits for the second");
    } else {
        // file tier: the hit experts run while the misses' records are read
        // into host slots
        if ((rc = run_hits())) return rc;
        int64_t recs[MOE_MAX_K];
        for (int n = 0; n < nmiss; n++) recs[n] = tier.record0 + c->h_idx[morder[n]];
        const char *ptrs[MOE_MAX_K];
        rc = tier_fetch(tier.t, recs, nmiss, ptrs);
        if (rc) {
            for (int n = 0; n < nmiss; n++) c->core.drop_slot(slot_of[morder[n]]);   // never filled
            return rc;
        }
        for (int n = 0; n < nmiss; n++) src_of[morder[n]] = ptrs[n];
        if ((rc = copy_run_pairs())) return rc;
        HIPCHK(join.run(), "copy stream waits for the second");
    }
    HIPCHK(launch_combine(W.ypart, k, KS, H, W.w, L->shared ? W.ysh : nullptr, out, H, 1, 0, cs), "combine");
    rc = cache_release_many(c, slot_of, k, cs);
    if (rc) return rc;
    if (!ah.L) return MOE_OK;
    // look-ahead: the predicted keys of the next layer (ascending id) are
    // touched in the LRU; the absent ones are copied now, behind this layer's
    // misses on the copy stream, so they land while this layer computes.  A
    // victim slot's copy still waits for that slot's last readers.
    HIPCHK(hipEventSynchronize(c->ahead_ev), "wait for the look-ahead ids");
    // the predictions whose weight (renormalised over the k_ahead predicted)
    // is at least min_weight, in ascending id
    int pred[MOE_MAX_K], np = 0;
    const int En = ah.L->router.E;
    for (int j = 0; j < ah.k; j++) {
        const int e = h_ahead[j];
        if (e < 0 || e >= En) return fail(MOE_E_HIP, "look-ahead router produced expert id %d", e);
        if (!(h_ahead_w[j] >= ah.min_weight)) continue;
        if (!ah.host[e]) return fail(MOE_E_INVAL, "next layer's experts_host[%d] is NULL", e);
        pred[np++] = e;
    }
    std::sort(pred, pred + np);
    for (int j = 0; j < np; j++) {
        const uint32_t key = ah.layer_id * (uint32_t)En + (uint32_t)pred[j];
        uint32_t victim = kNoKey;
        bool inserted = false;
        const int32_t s = c->core.touch_ahead(key, &victim, &inserted);
        if (!inserted) continue;
        c->filled[s] = 0;
        HIPCHK(cache_wait_readers(c, s, ps), "look-ahead copy waits for slot readers");
        bool enqueued = false;
        hipError_t e = cache_copy_in(c, s, ah.host[pred[j]], ps, &enqueued);
        if (e == hipSuccess) e = hipEventRecord(c->ready[s], ps);
        if (e != hipSuccess) {
            c->core.drop_slot(s);
            return hip_fail(e, "look-ahead copy");
        }
        c->filled[s] = 1;
    }
    return MOE_OK;
}
}  // namespace

extern "C" {

int moe_layer_forward_streamed(const moe_layer *L, moe_cache *c, uint32_t layer_id, const void *const *experts_host,
                               const float *x, int32_t T, float *out, int32_t *idx_out, void *ws, size_t ws_bytes,
                               void *compute_stream, void *copy_stream) {
    return streamed_impl(L, c, layer_id, experts_host, x, T, out, idx_out, ws, ws_bytes, compute_stream, copy_stream,
                         Ahead{});
}

int moe_layer_forward_streamed_tiered(const moe_layer *L, moe_cache *c, uint32_t layer_id, moe_host_tier *tier,
                                      int64_t record0, const float *x, int32_t T, float *out, int32_t *idx_out,
                                      void *ws, size_t ws_bytes, void *compute_stream, void *copy_stream) {
    if (!tier) return fail(MOE_E_INVAL, "host tier is NULL");
    if (c && tier->record_bytes < c->slot_bytes)
        return fail(MOE_E_INVAL, "host tier records (%llu bytes) are smaller than the cache slots (%llu)",
                    (unsigned long long)tier->record_bytes, (unsigned long long)c->slot_bytes);
    if (L && tier->core.capacity() < L->router.k)
        return fail(MOE_E_INVAL, "host tier has %d slots, below k = %d", tier->core.capacity(), L->router.k);
    if (record0 < 0) return fail(MOE_E_INVAL, "record0=%lld < 0", (long long)record0);
    if (tier->exclusive && L && (int64_t)layer_id * L->router.E != record0)
        return fail(MOE_E_INVAL, "an exclusive host tier keys records like the HBM cache: record0 must be "
                                 "layer_id * E = %lld (got %lld)", (long long)layer_id * L->router.E,
                    (long long)record0);
    Tier tr;
    tr.t = tier;
    tr.record0 = record0;
    return streamed_impl(L, c, layer_id, nullptr, x, T, out, idx_out, ws, ws_bytes, compute_stream, copy_stream,
                         Ahead{}, tr);
}

int moe_layer_forward_streamed_ahead(const moe_layer *L, moe_cache *c, uint32_t layer_id,
                                     const void *const *experts_host, const float *x, int32_t T, float *out,
                                     int32_t *idx_out, void *ws, size_t ws_bytes, void *compute_stream,
                                     void *copy_stream, const moe_layer *next, uint32_t next_layer_id,
                                     const void *const *next_experts_host, int32_t k_ahead, float min_weight) {
    if (!next) return fail(MOE_E_INVAL, "next layer is NULL (use moe_layer_forward_streamed)");
    if (!(min_weight >= 0.f && min_weight <= 1.f)) return fail(MOE_E_INVAL, "min_weight must be in [0, 1]");
    Ahead ah;
    ah.L = next;
    ah.layer_id = next_layer_id;
    ah.host = next_experts_host;
    ah.k = k_ahead;
    ah.min_weight = min_weight;
    return streamed_impl(L, c, layer_id, experts_host, x, T, out, idx_out, ws, ws_bytes, compute_stream, copy_stream,
                         ah);
}

size_t moe_grouped_workspace_bytes(const moe_layer *L, int32_t T) {
    if (!L || !dims_ok(L->H, L->I) || L->router.E < 1 || L->router.k < 1 || T < 0) return 0;
    return carve_grouped(nullptr, L->H, L->I, L->router.E, L->router.k, std::max(T, 1), L->shared != nullptr).bytes;
}

int moe_layer_forward_grouped(const moe_layer *L, const void *x, int32_t x_dtype, int32_t T, float *out,
                              int32_t *idx_out, float *w_out, void *ws, size_t ws_bytes, void *hip_stream) {
    int rc = check_layer(L, true);
    if (rc) return rc;
    if (T < 0) return fail(MOE_E_INVAL, "T=%d < 0", T);
    if (!dtype_ok(x_dtype)) return fail(MOE_E_INVAL, "unknown x dtype %d", x_dtype);
    if (T == 0) return MOE_OK;
    if (!x || !out || !ws) return fail(MOE_E_INVAL, "x, out and ws must be non-NULL");
    const size_t need = moe_grouped_workspace_bytes(L, T);
    if (ws_bytes < need) return fail(MOE_E_SPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    hipStream_t s = (hipStream_t)hip_stream;
    const int H = L->H, I = L->I, E = L->router.E, k = L->router.k;
    const GroupedWs W = carve_grouped(ws, H, I, E, k, T, L->shared != nullptr);
    int32_t *idx = idx_out ? idx_out : W.idx;
    float *w = w_out ? w_out : W.w;
    HIPCHK(launch_route_blocked(L->router.weight, L->router.bias, E, H, x, x_dtype, T, W.zpart, W.z, s),
           "route logits");
    HIPCHK(launch_topk(W.z, E, k, L->router.score_fn, T, idx, w, s), "top-k");
    HIPCHK(launch_group(idx, T * k, k, E, W.perm, W.inv, W.counts, W.offsets, s), "group");
    HIPCHK(launch_to_bf16(x, x_dtype, (size_t)T * H, W.xb, s), "x to bf16");
    int nsh = 0;
    if (L->shared) HIPCHK(launch_grouped_dense(L->shared, H, I, T, W.xb, W.hs, W.ysh, &nsh, s), "shared expert");
    HIPCHK(launch_grouped_rvq(L->records, offsets_of(H, I), E, H, I, T * k, W.counts, W.offsets, W.perm, k, W.xb, W.hbuf,
                              W.ybuf, s), "grouped RVQ GEMMs");
    HIPCHK(launch_grouped_combine(W.ybuf, W.inv, w, k, H, T, W.ysh, nsh, out, s), "combine");
    return MOE_OK;
}

}  // extern "C"
