// Persistent decode kernel: a whole decode (T tokens x n_layers resident MoE
// layers, token-major) in one cooperative launch, one workgroup per CU.
//
// Sources: WISP launch post, section "통찰" (token -> the model's router ->
// the selected experts -> next layer); WASTE article, section "유휴 가중치는
// 메모리가 아니라 제때 닿기만 하면 된다" (RVQ experts, 3.00 bits per weight,
// never expanded).
//
// Per (token, layer) step:
//   shared gate/up   rows split evenly over the workgroups (does not wait for
//                    routing); fp32 h of the shared expert
//   route            logit rows split over min(E, G) workgroups; then every
//                    workgroup recomputes the top-k itself from the logits
//   gate/up          the (rank, 64-row tile, 128-column chunk) space is split
//                    into G equal contiguous ranges; partial sums per
//                    (tile, contributor) are joined by the last contributor
//                    (per-tile counter), which writes fp16 SiLU(g) * u
//   shared down      rows split evenly; counted as contributions to the
//                    output tiles they touch
//   down             the (rank, 64-row tile of H, chunk) space likewise,
//                    after the rank's h is complete; the last contributor of
//                    an output tile combines sum_j w_j y_j + shared in fixed
//                    (rank, contributor) order and counts the tile as done.
//                    Where gate/up and down go by table lookup (many rows per
//                    codebook), down's space is (rank, chunk, tile), each
//                    segment waits only for its chunk of h (tagged words),
//                    and 16-row output slices over all workgroups combine
//                    the per-chunk partials
// The next step's routing starts when every output tile of this step is done.
// Counters only grow within a launch (targets are multiples of the step
// index), are zeroed before the launch, and every wait is bounded: on
// timeout the kernel sets an error flag and all waves leave.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "moe_internal.h"
#include "rvq_device.h"

namespace moe {
namespace {

constexpr int kPW = 8;                 // waves per workgroup
constexpr int kXcds = 8;               // accelerator complex dies (each with its own L2) of an MI355X
constexpr long kSpinLimit = 1L << 24;  // x ~0.1 us per poll: a few seconds
constexpr int kDecLdsBytes = 160 * 1024;

// Counter words, each on its own 256-byte line (pollers of one counter do
// not contend with adders of another): the error flag, up to kLayerCopiesMax
// layer-done counters (the kernel's LC of them: output unit u adds to copy
// u % LC; a waiter sums them), then h_ready[j] for j = 0..k (k: the shared expert).
// Word kErr is this launch's abort flag (zeroed before every launch, polled
// by every wait); word kStatus, on the same line, keeps kStatusFailed from a
// failed launch until the host reads and resets it, so a failure is seen
// even when later launches on the workspace succeed.
constexpr int kLine = 64;          // words per counter line
constexpr int kLayerCopiesMax = 16;
enum SyncIdx { kErr = 0, kStatus = 1, kLayerDone = kLine, kHReady = kLine * (1 + kLayerCopiesMax) };

// Mark this launch as failed: every wait then leaves, and the sticky status
// records it.
__device__ __forceinline__ void set_error(unsigned *sync) {
    __hip_atomic_store(sync + kStatus, (unsigned)kDecodeStatusFailed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(sync + kErr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Cross-workgroup data (logits, packed x, partial sums, h, shared-expert
// vectors) is written and read with agent-scope relaxed atomic accesses,
// which are coherent across the chip's XCDs without writing back or
// invalidating whole L2 caches.  A producer waits until its stores have
// completed (vmcnt 0), then bumps a counter; a consumer that has seen the
// counter reach its target issues its loads afterwards.
template <class T>
__device__ __forceinline__ void st_x(T *p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <class T>
__device__ __forceinline__ T ld_x(const T *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

__device__ __forceinline__ unsigned ld_cnt(const unsigned *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int AUX>
__device__ __forceinline__ void stage_lds(char *dst, const void *src, int nbytes, int wave, int lane) {
    stage_lds_waves<AUX, kPW>(dst, src, nbytes, wave, lane);
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// Wave-level coherent copy of one 64-float block (lane l: src[l]) into LDS at
// dst (wave-uniform), written by other workgroups in this launch.
__device__ __forceinline__ void dma_block(float *dst, const float *src, int lane) {
    __builtin_amdgcn_global_load_lds((gvoid *)(src + lane), (lvoid *)dst, 4, 0, kLdsCoherent);
}
// Wait until all but this wave's N most recent vector memory operations
// (and all its LDS operations) are done, then a plain workgroup barrier.
// For LDS data only: __syncthreads() would also wait for the N loads still
// in flight.  The asm's memory clobber keeps the compiler from moving memory
// accesses across the barrier.
template <int N>
__device__ __forceinline__ void wait_lds_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
// Workgroup barrier for LDS data: waits for this wave's LDS operations only,
// so stores and loads to global memory stay in flight across it
// (__syncthreads() would wait for all of them: a memory round trip).
__device__ __forceinline__ void lds_sync() {
    wait_lds_barrier<63>();
    lds_barrier();
}

// Workgroup-wide wait until the sum of the NC counters p[0], p[kLine], ...
// reaches target.  Returns false (error flag set) on timeout or if another
// workgroup already failed.
template <int NC = 1>
__device__ __forceinline__ bool wg_wait(unsigned *sync, const unsigned *p, unsigned target, int *bcast) {
    if (threadIdx.x == 0) {
        long spins = 0;
        int ok = 1;
        for (;;) {
            // all loads in flight together: one memory round trip per poll
            unsigned c = 0;
#pragma unroll
            for (int i = 0; i < NC; i++) c += ld_cnt(p + i * kLine);
            const unsigned err = ld_cnt(sync + kErr);
            if (c >= target) break;
            if (err) { ok = 0; break; }
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
                set_error(sync);
                ok = 0;
                break;
            }
        }
        *bcast = ok;
    }
    lds_sync();
    const bool ok = *bcast != 0;
    lds_sync();
    return ok;
}

// Values exchanged between workgroups inside a step carry the step: value
// in the low and (step + 1) in the high half of one 64-bit word, stored and
// loaded as a single atomic access.  A writer needs no wait and no counter;
// a reader polls until every word it needs carries the current step, and has
// the data in the same load.  (Buffers start zeroed, so tag 0 never matches;
// the layer-done barrier keeps the next step from rewriting a word that a
// reader of this step still polls.)
__device__ __forceinline__ void st_tagged(uint64_t *p, float v, unsigned tag) {
    __hip_atomic_store(p, (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tagged(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_ok(uint64_t v, unsigned tag) { return (unsigned)(v >> 32) == tag; }
__device__ __forceinline__ float tag_val(uint64_t v) { return __uint_as_float((unsigned)v); }

// Row-pair words of the table-lookup phases' partials: rows l and l + 32 of
// a tile in one 64-bit word, each as the top 24 bits of its fp32 value
// (rounded to nearest: 15 mantissa bits, relative error <= 2^-16), with a
// 16-bit step tag, (step mod 65535) + 1, in bits 48..63, so a tile's
// partial is 32 words where it was 64.  Every word of these buffers is
// rewritten each step, so consecutive steps' tags always differ.
__device__ __forceinline__ unsigned tag16(int s) { return (unsigned)(s % 65535) + 1u; }
__device__ __forceinline__ uint64_t f24(float v) { return (uint64_t)((__float_as_uint(v) + 0x80u) >> 8); }
// lane l < 32 stores rows l and l + 32 (the value of lane l + 32 comes across)
__device__ __forceinline__ void st_pair(uint64_t *p, float v, unsigned tag, int lane) {
    const float hi = __shfl_down(v, 32, 64);
    if (lane < 32) st_x(p + lane, f24(v) | (f24(hi) << 24) | ((uint64_t)tag << 48));
}
__device__ __forceinline__ bool pair_ok(uint64_t v, unsigned tag) { return (unsigned)(v >> 48) == tag; }
// the value of row lane (0..63) from the word of rows lane % 32, lane % 32 + 32
__device__ __forceinline__ float pair_val(uint64_t v, int lane) {
    return __uint_as_float((unsigned)(lane < 32 ? v : v >> 24) << 8);
}

// Wave-level bound on a poll loop: false (and the error flag set) after too
// many polls, or once another workgroup has failed.
__device__ __forceinline__ bool poll_more(unsigned *sync, long &spins) {
    if (++spins > kSpinLimit) {
        set_error(sync);
        return false;
    }
    if ((spins & 31) == 0 && ld_cnt(sync + kErr)) return false;
    __builtin_amdgcn_s_sleep(1);
    return true;
}

// Loads of weights and record fields through pointers held in memory (the
// layer table, record pointers) as global-memory loads: through a generic
// pointer they would be flat loads, which also count against the LDS wait
// counter and cannot be reordered with LDS accesses.
typedef float g_f32x4 __attribute__((ext_vector_type(4)));
template <class T>
__device__ __forceinline__ T gld(const T *p) {
    return *(__attribute__((address_space(1))) const T *)p;
}
__device__ __forceinline__ float4 gld4(const float *p) {
    const g_f32x4 v = *(__attribute__((address_space(1))) const g_f32x4 *)p;
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 gldu4(const void *p) {
    const u32x4 v = *(gu32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// A space of n units is split over Ga = min(G, n) active workgroups into
// contiguous, non-empty ranges [start(w), start(w+1)); workgroups w >= Ga get
// nothing.  Non-empty ranges keep the contributors of any unit interval
// contiguous in w.  32-bit arithmetic: every space here has n * (G + 1) <
// 2^31 (the plan checks it), so the products cannot overflow (a 64-bit
// division is a long instruction sequence, and these sit on phases' tails).
__device__ __forceinline__ int active_of(int n, int G) { return n < G ? n : G; }
__device__ __forceinline__ int range_start(int n, int G, int w) {
    const int Ga = active_of(n, G);
    return w >= Ga ? n : (int)((unsigned)(n * w) / (unsigned)Ga);
}
// workgroup owning unit u
__device__ __forceinline__ int range_owner(int n, int G, int u) {
    const int Ga = active_of(n, G);
    return (int)((unsigned)((u + 1) * Ga + n - 1) / (unsigned)n) - 1;
}

// One strip (64 rows x 128 columns, 16 groups of 8 columns) of codes against
// x pairs in LDS.  Each lane owns one row; a group costs two codebook-row
// gathers (codes a and b) and a broadcast read of the group's x pairs (a
// wave-uniform address).  Groups are processed in batches whose reads are
// software-pipelined: batch B+1's gathers are issued before batch B's dot
// products, so a wave always has LDS work queued while it computes.
// sched_barrier fences keep the compiler from hoisting further batches
// (which would hold every gathered row in registers at once).

// gate and up together, two groups per batch (8 gathers + 2 x reads)
struct GuBatch {
    u32x4 g0[2], g1[2], u0[2], u1[2], xq[2];
};
template <int B>
__device__ __forceinline__ void gu_read(GuBatch &d, const uint32_t (&dg)[12], const uint32_t (&du)[12], const char *cbg,
                                        const char *cbu, const uint32_t *xl) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
        uint32_t ga, gb, ua, ub;
        if (i == 0) { group_addr<2 * B>(dg, ga, gb); group_addr<2 * B>(du, ua, ub); }
        else { group_addr<2 * B + 1>(dg, ga, gb); group_addr<2 * B + 1>(du, ua, ub); }
        d.g0[i] = *(const u32x4 *)(cbg + ga);
        d.g1[i] = *(const u32x4 *)(cbg + gb);
        d.u0[i] = *(const u32x4 *)(cbu + ua);
        d.u1[i] = *(const u32x4 *)(cbu + ub);
        d.xq[i] = *(const u32x4 *)(xl + 4 * (2 * B + i));
    }
}
template <int B>
__device__ __forceinline__ void gu_dots(GuBatch &d, float (&ag)[4], float (&au)[4]) {
    // the batch's values are complete here (waits only for this batch)
    asm volatile("" : "+v"(d.g0[0]), "+v"(d.g0[1]), "+v"(d.g1[0]), "+v"(d.g1[1]), "+v"(d.u0[0]), "+v"(d.u0[1]),
                 "+v"(d.u1[0]), "+v"(d.u1[1]), "+v"(d.xq[0]), "+v"(d.xq[1]));
#pragma unroll
    for (int i = 0; i < 2; i++) {
        float a = ag[(2 * B + i) & 3], b = au[(2 * B + i) & 3];
        a = dot2(d.g0[i].x, d.xq[i].x, a); b = dot2(d.u0[i].x, d.xq[i].x, b);
        a = dot2(d.g0[i].y, d.xq[i].y, a); b = dot2(d.u0[i].y, d.xq[i].y, b);
        a = dot2(d.g0[i].z, d.xq[i].z, a); b = dot2(d.u0[i].z, d.xq[i].z, b);
        a = dot2(d.g0[i].w, d.xq[i].w, a); b = dot2(d.u0[i].w, d.xq[i].w, b);
        a = dot2(d.g1[i].x, d.xq[i].x, a); b = dot2(d.u1[i].x, d.xq[i].x, b);
        a = dot2(d.g1[i].y, d.xq[i].y, a); b = dot2(d.u1[i].y, d.xq[i].y, b);
        a = dot2(d.g1[i].z, d.xq[i].z, a); b = dot2(d.u1[i].z, d.xq[i].z, b);
        a = dot2(d.g1[i].w, d.xq[i].w, a); b = dot2(d.u1[i].w, d.xq[i].w, b);
        ag[(2 * B + i) & 3] = a;
        au[(2 * B + i) & 3] = b;
    }
}
template <int B>
__device__ __forceinline__ void gu_pipe(const uint32_t (&dg)[12], const uint32_t (&du)[12], const char *cbg,
                                        const char *cbu, const uint32_t *xl, GuBatch &cur, GuBatch &nxt,
                                        float (&ag)[4], float (&au)[4]) {
    if constexpr (B < 8) {
        if constexpr (B + 1 < 8) gu_read<B + 1>(nxt, dg, du, cbg, cbu, xl);
        __builtin_amdgcn_sched_barrier(0);
        gu_dots<B>(cur, ag, au);
        __builtin_amdgcn_sched_barrier(0);
        gu_pipe<B + 1>(dg, du, cbg, cbu, xl, nxt, cur, ag, au);
    }
}
__device__ __forceinline__ void strip_gateup(const uint32_t (&dg)[12], const uint32_t (&du)[12], const char *cbg,
                                             const char *cbu, const uint32_t *xl, float (&ag)[4], float (&au)[4]) {
    GuBatch p, q;
    gu_read<0>(p, dg, du, cbg, cbu, xl);
    gu_pipe<0>(dg, du, cbg, cbu, xl, p, q, ag, au);
}

// one matrix, four groups per batch (8 gathers + 4 x reads)
struct DBatch {
    u32x4 c0[4], c1[4], xq[4];
};
template <int B>
__device__ __forceinline__ void d_read(DBatch &d, const uint32_t (&c)[12], const char *cb, const uint32_t *xl) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t aa, ba;
        switch (i) {
            case 0: group_addr<4 * B + 0>(c, aa, ba); break;
            case 1: group_addr<4 * B + 1>(c, aa, ba); break;
            case 2: group_addr<4 * B + 2>(c, aa, ba); break;
            default: group_addr<4 * B + 3>(c, aa, ba); break;
        }
        d.c0[i] = *(const u32x4 *)(cb + aa);
        d.c1[i] = *(const u32x4 *)(cb + ba);
        d.xq[i] = *(const u32x4 *)(xl + 4 * (4 * B + i));
    }
}
__device__ __forceinline__ void d_dots(DBatch &d, float (&acc)[4]) {
    asm volatile("" : "+v"(d.c0[0]), "+v"(d.c0[1]), "+v"(d.c0[2]), "+v"(d.c0[3]), "+v"(d.c1[0]), "+v"(d.c1[1]),
                 "+v"(d.c1[2]), "+v"(d.c1[3]), "+v"(d.xq[0]), "+v"(d.xq[1]), "+v"(d.xq[2]), "+v"(d.xq[3]));
#pragma unroll
    for (int i = 0; i < 4; i++) {
        float a = acc[i];
        a = dot2(d.c0[i].x, d.xq[i].x, a);
        a = dot2(d.c0[i].y, d.xq[i].y, a);
        a = dot2(d.c0[i].z, d.xq[i].z, a);
        a = dot2(d.c0[i].w, d.xq[i].w, a);
        a = dot2(d.c1[i].x, d.xq[i].x, a);
        a = dot2(d.c1[i].y, d.xq[i].y, a);
        a = dot2(d.c1[i].z, d.xq[i].z, a);
        a = dot2(d.c1[i].w, d.xq[i].w, a);
        acc[i] = a;
    }
}
template <int B>
__device__ __forceinline__ void d_pipe(const uint32_t (&c)[12], const char *cb, const uint32_t *xl, DBatch &cur,
                                       DBatch &nxt, float (&acc)[4]) {
    if constexpr (B < 4) {
        if constexpr (B + 1 < 4) d_read<B + 1>(nxt, c, cb, xl);
        __builtin_amdgcn_sched_barrier(0);
        d_dots(cur, acc);
        __builtin_amdgcn_sched_barrier(0);
        d_pipe<B + 1>(c, cb, xl, nxt, cur, acc);
    }
}
__device__ __forceinline__ void strip_down(const uint32_t (&c)[12], const char *cb, const uint32_t *xl,
                                           float (&acc)[4]) {
    DBatch p, q;
    d_read<0>(p, c, cb, xl);
    d_pipe<0>(c, cb, xl, p, q, acc);
}

// The streaming GEMV loops are inlined into the kernel: as separate
// functions, the call convention makes each call save and restore most of
// the register file through scratch memory.  They address the kernel's
// dynamic LDS directly.
extern __shared__ __align__(16) char dec_lds[];

// LDS layout (bytes).  Gate/up: [gate cb 64K][up cb 64K][x pairs][sums];
// down: [down cb 64K][h pairs][sums]; a small tail holds routing results.
struct DecLds {
    int x_gu, red_gu, x_d, red_d;
};
__device__ __forceinline__ DecLds dec_lds_layout(int H, int I) {
    DecLds L;
    L.x_gu = 2 * kCbRows * 16;
    L.red_gu = L.x_gu + ((H * 2 + 255) & ~255);
    L.x_d = kCbRows * 16;
    L.red_d = L.x_d + ((I * 2 + 255) & ~255);
    return L;
}
constexpr int kDecTail = kDecLdsBytes - 1024;     // sidx, sw, broadcast words, router partials
constexpr int kDecRecs = kDecTail - 8 * MOE_MAX_E;   // the layer's record pointers, until top-k

constexpr int kDecCtr = kDecLdsBytes - 4;   // the lookup phase's tile counter (unused end of the tail)
constexpr int kRingGU = 3;      // code buffers per wave (2 units in flight ahead)
constexpr int kShRows = 8;      // shared-expert rows per load group (gate/up)
constexpr int kShDR = 3;        // shared-expert down rows per wave in flight
constexpr int kShCP = 4;        // 512-column passes of those rows in flight (I <= 2048 in one)
constexpr int kTopkScratch = 2048;   // LDS bytes (codebook area, free while routing): top-k staging
constexpr int kXStage = 16 * 1024;   // LDS bytes (codebook area, free while routing): fp32 x for the gathers
constexpr int kTopkGroups = 8;       // first-level groups of the top-k
// zkey [MOE_MAX_E], candidates [kTopkGroups * MOE_MAX_K] (slot group * k + local rank), logits in
// rank order [MOE_MAX_K]

// Order-preserving key of a float (larger float, larger key; -0 and +0 one
// key, as they compare equal) and back.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    u = u == 0x80000000u ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
constexpr int kRingD = 4;       // (3 ahead)

__device__ __forceinline__ void load_codes(gu32x4 *base, int u, int lane, uint32_t (&d)[12]) {
    load_strip((const u32x4 *)(base + (long)u * kTileVec), lane, d);
}

// A wave's position in its units: tile t, chunk c; it advances kPW units at
// a time.  Tile sums accumulate in registers and are flushed to the LDS slot
// (tile - t0) when the tile changes.
struct UnitPos {
    int t, c, cur_t;
    float rcp;    // 1 / cpr
};
// Branch-free advance (a loop here lets the compiler sink the unit's dot
// products past it, keeping every gathered row live): the float quotient of
// c < cpr + kPW by cpr is exact or one low, and one select corrects it.
__device__ __forceinline__ void next_unit(UnitPos &p, int cpr) {
    const int c = p.c + kPW;
    int q = (int)((float)c * p.rcp);
    int r = c - q * cpr;
    const bool hi = r >= cpr;
    q += hi ? 1 : 0;
    r -= hi ? cpr : 0;
    p.t += q;
    p.c = r;
}

__device__ __forceinline__ void gu_unit(const uint32_t (&dg)[12], const uint32_t (&du)[12], const char *cbg,
                                        const char *cbu, const uint32_t *xl, float *red, int t0, int cpr, int wave,
                                        int lane, UnitPos &p, float (&ag)[4], float (&au)[4]) {
    if (p.t != p.cur_t) {
        float *s = red + ((p.cur_t - t0) * kPW + wave) * 128;
        s[lane] = (ag[0] + ag[1]) + (ag[2] + ag[3]);
        s[64 + lane] = (au[0] + au[1]) + (au[2] + au[3]);
        ag[0] = ag[1] = ag[2] = ag[3] = 0.f;
        au[0] = au[1] = au[2] = au[3] = 0.f;
        p.cur_t = p.t;
    }
    strip_gateup(dg, du, cbg, cbu, xl + p.c * 64, ag, au);
    next_unit(p, cpr);
}

__device__ __forceinline__ void d_unit(const uint32_t (&d)[12], const char *cb, const uint32_t *xl, float *red, int t0,
                                       int cpr, int wave, int lane, UnitPos &p, float (&acc)[4]) {
    if (p.t != p.cur_t) {
        red[((p.cur_t - t0) * kPW + wave) * 64 + lane] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        acc[0] = acc[1] = acc[2] = acc[3] = 0.f;
        p.cur_t = p.t;
    }
    strip_down(d, cb, xl + p.c * 64, acc);
    next_unit(p, cpr);
}

// Gate and up of one expert: units [la, lb) (unit u = tile u / cpr, chunk
// u % cpr; its codes are 3072 bytes at base + u * 3072), against the x pairs
// already in LDS.  Wave v takes units la + v, la + v + kPW, ...; tile sums go
// to LDS slot (tile - t0).  The steady-state loop has no branches around its loads:
// loads past the wave's last unit re-read that unit (their buffers are never
// consumed), so every load of the ring stays in flight while older units are
// computed.
// count_at: if not null, this wave adds 1 there once the staging has waited
// for all of its memory operations (stores issued before the call included).
__device__ __forceinline__ void stream_gateup(const u32x4 *gsec, const u32x4 *usec, const u32x4 *cbg_src,
                                           const u32x4 *cbu_src, int H, int I,
                                           int cpr, int la, int lb, int t0, int nslots, int wave, int lane,
                                           unsigned long long *stamp, unsigned *count_at) {
    const DecLds L = dec_lds_layout(H, I);
    char *cbg = dec_lds, *cbu = dec_lds + kCbRows * 16;
    uint32_t *xl = (uint32_t *)(dec_lds + L.x_gu);
    float *red = (float *)(dec_lds + L.red_gu);
    gu32x4 *gb = (gu32x4 *)gsec, *ub = (gu32x4 *)usec;
    const int first = __builtin_amdgcn_readfirstlane(la + wave);
    const int n = __builtin_amdgcn_readfirstlane(first < lb ? (lb - first + kPW - 1) / kPW : 0);
    // stage the codebooks and clear this segment's sum slots
    stage_lds<kLdsPlain>(cbg, cbg_src, kCbRows * 16, wave, lane);
    stage_lds<kLdsPlain>(cbu, cbu_src, kCbRows * 16, wave, lane);
    uint32_t bg[kRingGU][12], bu[kRingGU][12];
    for (int i = threadIdx.x; i < nslots * kPW * 128; i += kPW * 64) red[i] = 0.f;
    wait_lds_barrier<0>();
    if (count_at && lane == 0) __hip_atomic_fetch_add(count_at, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lds_barrier();
    // first ring stages, issued after the codebooks have landed (issued
    // together, the chip-wide burst of code loads delays the codebooks); a
    // wave without units loads the segment's first unit (never consumed)
#pragma unroll
    for (int r = 0; r < kRingGU - 1; r++) {
        const int u = n ? first + min(r, n - 1) * kPW : la;
        load_codes(gb, u, lane, bg[r]);
        load_codes(ub, u, lane, bu[r]);
    }
    if (stamp && threadIdx.x == 0) stamp[kStampGuStaged] = wall_clock64();
    if (!n) return;
    float ag[4] = {0.f, 0.f, 0.f, 0.f}, au[4] = {0.f, 0.f, 0.f, 0.f};
    UnitPos p{first / cpr, first % cpr, first / cpr, 1.f / (float)cpr};
    int i = 0;
    for (; i + kRingGU <= n; i += kRingGU) {
#pragma unroll
        for (int r = 0; r < kRingGU; r++) {
            const int u = first + min(i + r + kRingGU - 1, n - 1) * kPW;
            load_codes(gb, u, lane, bg[(r + kRingGU - 1) % kRingGU]);
            load_codes(ub, u, lane, bu[(r + kRingGU - 1) % kRingGU]);
            gu_unit(bg[r], bu[r], cbg, cbu, xl, red, t0, cpr, wave, lane, p, ag, au);
        }
    }
    // the last n - i (< kRingGU) units are already in buffers 0, 1, ...
#pragma unroll
    for (int r = 0; r < kRingGU - 1; r++)
        if (i + r < n) gu_unit(bg[r], bu[r], cbg, cbu, xl, red, t0, cpr, wave, lane, p, ag, au);
    float *s = red + ((p.cur_t - t0) * kPW + wave) * 128;
    s[lane] = (ag[0] + ag[1]) + (ag[2] + ag[3]);
    s[64 + lane] = (au[0] + au[1]) + (au[2] + au[3]);
}

// Down of one expert: units [la, lb) over tiles of H, like stream_gateup.
// The first loads are issued before waiting for the expert's h (counter
// h_ready >= h_target) and staging it with the codebook.  Returns 0 if the
// wait failed.
__device__ __forceinline__ int stream_down(const u32x4 *dsec, const u32x4 *cbd_src, const float *h_src, unsigned *sync,
                                        const unsigned *h_ready, unsigned h_target, int *bcast, float *wmax, int &he,
                                        int H, int I, int cpr, int la, int lb, int t0, int nslots, int wave, int lane,
                                        unsigned long long *stamp) {
    const DecLds L = dec_lds_layout(H, I);
    char *cb = dec_lds;
    uint32_t *xl = (uint32_t *)(dec_lds + L.x_d);
    float *red = (float *)(dec_lds + L.red_d);
    gu32x4 *db = (gu32x4 *)dsec;
    const int first = __builtin_amdgcn_readfirstlane(la + wave);
    const int n = __builtin_amdgcn_readfirstlane(first < lb ? (lb - first + kPW - 1) / kPW : 0);
    uint32_t bd[kRingD][12];
#pragma unroll
    for (int r = 0; r < kRingD - 1; r++) load_codes(db, n ? first + min(r, n - 1) * kPW : la, lane, bd[r]);
    stage_lds<kLdsPlain>(cb, cbd_src, kCbRows * 16, wave, lane);
    for (int i = threadIdx.x; i < nslots * kPW * 64; i += kPW * 64) red[i] = 0.f;
    if (!wg_wait(sync, h_ready, h_target, bcast)) return 0;
    // h (fp32, written by other workgroups) into LDS as fp16 pairs scaled by
    // 2^-he (he from the largest |h|, the same in every workgroup); the
    // partial sums are scaled back by 2^he.  Up to 4 pairs per thread stay
    // in registers; a larger I reloads the rest for the conversion.
    {
        const uint64_t *hp = (const uint64_t *)h_src;
        const int np = I / 2;
        constexpr int kReg = 4, kStride = kPW * 64;
        uint64_t hv[kReg];
        float m = 0.f;
        auto mag = [](uint64_t v) {
            return fmaxf(fabsf(__uint_as_float((uint32_t)v)), fabsf(__uint_as_float((uint32_t)(v >> 32))));
        };
#pragma unroll
        for (int i = 0; i < kReg; i++) {
            const int p = threadIdx.x + i * kStride;
            hv[i] = p < np ? ld_x(hp + p) : 0;
            m = fmaxf(m, mag(hv[i]));
        }
        for (int p = threadIdx.x + kReg * kStride; p < np; p += kStride) m = fmaxf(m, mag(ld_x(hp + p)));
        m = wave_max(m);
        if (lane == 0) wmax[wave] = m;
        lds_sync();
        m = wmax[0];
#pragma unroll
        for (int v = 1; v < kPW; v++) m = fmaxf(m, wmax[v]);
        he = __builtin_amdgcn_readfirstlane(range_exp(m));
        auto pack = [&](uint64_t v) {
            return pack_f16x2(ldexpf(__uint_as_float((uint32_t)v), -he), ldexpf(__uint_as_float((uint32_t)(v >> 32)), -he));
        };
#pragma unroll
        for (int i = 0; i < kReg; i++) {
            const int p = threadIdx.x + i * kStride;
            if (p < np) xl[p] = pack(hv[i]);
        }
        for (int p = threadIdx.x + kReg * kStride; p < np; p += kStride) xl[p] = pack(ld_x(hp + p));
    }
    wait_vm_all();
    __syncthreads();
    if (stamp && threadIdx.x == 0) stamp[kStampDownStaged] = wall_clock64();
    if (!n) return 1;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    UnitPos p{first / cpr, first % cpr, first / cpr, 1.f / (float)cpr};
    int i = 0;
    for (; i + kRingD <= n; i += kRingD) {
#pragma unroll
        for (int r = 0; r < kRingD; r++) {
            load_codes(db, first + min(i + r + kRingD - 1, n - 1) * kPW, lane, bd[(r + kRingD - 1) % kRingD]);
            d_unit(bd[r], cb, xl, red, t0, cpr, wave, lane, p, acc);
        }
    }
#pragma unroll
    for (int r = 0; r < kRingD - 1; r++)
        if (i + r < n) d_unit(bd[r], cb, xl, red, t0, cpr, wave, lane, p, acc);
    red[((p.cur_t - t0) * kPW + wave) * 64 + lane] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    return 1;
}

// ---- Gate/up by table lookup (for experts with many rows per codebook).
// Within a 128-column chunk, group q (8 columns) of every row contributes
// C[a].x_q + C[b].x_q.  A table T[q][c] = C[c].x_q over all 4096 codebook
// rows c and the chunk's 16 groups (128 KiB of fp16) turns each group into
// two 2-byte LDS lookups in place of two 16-byte gathers; random 2-byte
// reads sustain about twice the lanes per clock of random 16-byte reads.
// Each table serves every row of the matrix that this workgroup streams for
// that chunk.
//
// The table is a small dense contraction, built on matrix cores:
// v_mfma_f32_16x16x16_f16, where lane l holds A[l%16][4(l/16)..+3],
// B[4(l/16)..+3][l%16] and D[4(l/16)..+3][l%16].  K half h of A holds
// codebook rows c0 + 16h + m; column n of B holds x of group n % 8 (of one
// half chunk) in K half n / 8 and zero in the other, so
// D[m][n] = C[c0 + 16(n/8) + m] . x_{n%8}: one instruction yields 32 rows x 8
// groups.  x enters as an fp16 pair hi + lo (two MFMAs into one fp32
// accumulator), so only the table entries themselves are rounded (to fp16).
// A wave keeps the A fragments of its 512 codebook rows in registers for the
// whole segment (the codebook never goes to LDS).
//
// LDS in this phase: the table, row q (group q) at kLutRowB q (the 64-byte
// pad puts consecutive rows 16 banks apart, so a table store is 2-way at
// worst), then the token's x (fp32, stored there by the routing pass).  The lookups address LDS
// from byte 0 (the kernel has no static LDS, so its dynamic LDS starts there;
// the host checks), with the row offset as the instruction's immediate
// where it fits (rows 0..7).
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const _Float16 lds_f16;
constexpr int kLutRowB = 2 * kCbRows + 64;                     // bytes per table row
constexpr int kLutX = 16 * kLutRowB;                           // x offset (132,096)
constexpr int kLutMaxH = (kDecRecs - kLutX) / 4;               // x must end below the routing tail
constexpr int kLutRing = 4;                                    // code buffers per wave (3 units ahead)
constexpr int kLutCbTiles = kCbRows / 32 / kPW;                // 32-row MFMA tiles each wave builds
typedef __attribute__((address_space(1))) const f16x4 gf16x4;  // global memory

// Group G's two lookups (row G of the table) as one fp16 pair.
template <int G>
__device__ __forceinline__ f16x2 lut_pair(const uint32_t (&d)[12]) {
    constexpr int bit = 24 * G, i = bit / 32, s = bit % 32;
    uint32_t v;
    if constexpr (s <= 8) v = d[i] >> s;
    else v = __builtin_amdgcn_alignbit(d[i + 1], d[i], s);
    constexpr uint32_t off = G * kLutRowB;
    const uint32_t aa = ((v << 1) & 0x1FFEu) + off;
    const uint32_t ba = ((v >> 11) & 0x1FFEu) + off;
    f16x2 p;
    p.x = *(lds_f16 *)(uintptr_t)aa;
    p.y = *(lds_f16 *)(uintptr_t)ba;
    return p;
}
template <int HF>
__device__ __forceinline__ void lut_read8(const uint32_t (&d)[12], f16x2 (&p)[8]) {
    p[0] = lut_pair<8 * HF + 0>(d);
    p[1] = lut_pair<8 * HF + 1>(d);
    p[2] = lut_pair<8 * HF + 2>(d);
    p[3] = lut_pair<8 * HF + 3>(d);
    p[4] = lut_pair<8 * HF + 4>(d);
    p[5] = lut_pair<8 * HF + 5>(d);
    p[6] = lut_pair<8 * HF + 6>(d);
    p[7] = lut_pair<8 * HF + 7>(d);
}
__device__ __forceinline__ float lut_sum8(f16x2 (&p)[8]) {
    // the values are complete here (waits for these lookups only)
    asm volatile("" : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]), "+v"(p[4]), "+v"(p[5]), "+v"(p[6]),
                 "+v"(p[7]));
    const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int g = 0; g < 8; g += 2) {
        a0 = __builtin_amdgcn_fdot2(p[g], one, a0, false);       // T[a] + T[b], exact in fp32
        a1 = __builtin_amdgcn_fdot2(p[g + 1], one, a1, false);
    }
    return a0 + a1;
}
// One 48-byte strip (16 groups): the second half's lookups are issued
// before the first half's sums.
__device__ __forceinline__ float lut_strip(const uint32_t (&d)[12]) {
    f16x2 p0[8], p1[8];
    lut_read8<0>(d, p0);
    lut_read8<1>(d, p1);
    const float s0 = lut_sum8(p0);
    return s0 + lut_sum8(p1);
}

// The lane id, computed afresh where it is used: left to the compiler, the
// lane-dependent addresses of the table builds are kept across the whole
// phase and spilled, and reloading a spill waits for every load in flight.
__device__ __forceinline__ int fresh_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// The table of one chunk from the A fragments; the chunk's 128 x values
// (fp32) are at LDS byte xo.
// Returns the chunk's exponent e: the table holds C[c].(x_q 2^-e) (range
// scaling, so that no entry overflows fp16), and each sum over the chunk is
// scaled back by 2^e.  Every wave reads all 128 values, so all find the same e.
__device__ __forceinline__ int lut_build(const f16x4 (&A)[kLutCbTiles], int xo, int wave) {
    const int lane = fresh_lane();
    const int n = lane & 15, g = lane >> 4;
    const bool valid = (g >> 1) == (n >> 3);
    const f16x4 z4 = {(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
    f16x4 bh[2], bl[2];
    float4 xr[2];
    float m = 0.f;
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
        xr[hf] = *(const float4 *)(dec_lds + xo + 4 * (64 * hf + 8 * (n & 7) + 4 * (g & 1)));
        m = fmaxf(m, fmaxf(fmaxf(fabsf(xr[hf].x), fabsf(xr[hf].y)), fmaxf(fabsf(xr[hf].z), fabsf(xr[hf].w))));
    }
    const int e = __builtin_amdgcn_readfirstlane(range_exp(wave_max(m)));
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
        const float4 xv = make_float4(ldexpf(xr[hf].x, -e), ldexpf(xr[hf].y, -e), ldexpf(xr[hf].z, -e),
                                      ldexpf(xr[hf].w, -e));
        bh[hf].x = (_Float16)xv.x; bh[hf].y = (_Float16)xv.y; bh[hf].z = (_Float16)xv.z; bh[hf].w = (_Float16)xv.w;
        bl[hf].x = (_Float16)(xv.x - (float)bh[hf].x);
        bl[hf].y = (_Float16)(xv.y - (float)bh[hf].y);
        bl[hf].z = (_Float16)(xv.z - (float)bh[hf].z);
        bl[hf].w = (_Float16)(xv.w - (float)bh[hf].w);
        if (!valid) { bh[hf] = z4; bl[hf] = z4; }
    }
    // this lane's entries: rows 8 hf + n % 8, codebook rows c0 + 16 (n / 8) + 4 g + 0..3;
    // two tiles (four independent accumulators) per step
    char *dst = dec_lds + (n & 7) * kLutRowB + 2 * (wave * kLutCbTiles * 32 + 16 * (n >> 3) + 4 * g);
#pragma unroll
    for (int t = 0; t < kLutCbTiles; t += 2) {
        f32x4 d[2][2];
#pragma unroll
        for (int u = 0; u < 2; u++)
#pragma unroll
            for (int hf = 0; hf < 2; hf++) {
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                d[u][hf] = __builtin_amdgcn_mfma_f32_16x16x16f16(A[t + u], bh[hf], z, 0, 0, 0);
            }
#pragma unroll
        for (int u = 0; u < 2; u++)
#pragma unroll
            for (int hf = 0; hf < 2; hf++)
                d[u][hf] = __builtin_amdgcn_mfma_f32_16x16x16f16(A[t + u], bl[hf], d[u][hf], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 2; u++)
#pragma unroll
            for (int hf = 0; hf < 2; hf++) {
                f16x4 o;
                o.x = (_Float16)d[u][hf].x; o.y = (_Float16)d[u][hf].y;
                o.z = (_Float16)d[u][hf].z; o.w = (_Float16)d[u][hf].w;
                *(f16x4 *)(dst + hf * 8 * kLutRowB + 64 * (t + u)) = o;
            }
    }
    return e;
}

// One segment of a table-lookup space: one matrix (codes at codes, codebook
// at cb, cpr chunks per row tile) of one expert, chunk c, row tiles
// [ta, ta + nt).  One table build, then the waves stream the tiles through
// register rings (no barriers) and store each tile's sum over the chunk as a
// row-pair partial at part + tstride * tile (the caller's part points at the
// segment's slot; tag: tag16 of the step).  Wave v's first kLutRing - 1 tiles are v, v + kPW, ...;
// after that each wave takes the next tile from a workgroup counter in LDS,
// so waves that run ahead take more tiles.  A tile is always summed whole by
// one wave, so the result does not depend on which.  pre() runs once the
// first code loads are in flight and before the build reads the chunk's x
// at LDS byte xo (down waits for h and stages its chunk there); it returns
// false if its wait failed, and so does the segment.
__device__ __forceinline__ int lut_next_tile(unsigned *ctr, int lane) {
    unsigned v = 0;
    if (lane == 0) v = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return (int)__builtin_amdgcn_readfirstlane(v);
}
template <class Pre>
__device__ __forceinline__ bool stream_lut(const u32x4 *codes, const u32x4 *cb, int cpr, int c, int xo, int ta, int nt,
                                           uint64_t *part, int tstride, unsigned tag, int wave, int lane, Pre pre,
                                           unsigned long long *built = nullptr) {
    gu32x4 *gb = (gu32x4 *)codes;
    unsigned *ctr = (unsigned *)(dec_lds + kDecCtr);
    // the A fragments first: the build waits for them alone, tile by tile,
    // while the code ring's loads stay in flight
    f16x4 A[kLutCbTiles];
    {
        const int nn = lane & 15, g = lane >> 4;
        gf16x4 *src = (gf16x4 *)((const char *)cb + (size_t)(wave * kLutCbTiles * 32 + 16 * (g >> 1) + nn) * 16 +
                                 8 * (g & 1));
#pragma unroll
        for (int t = 0; t < kLutCbTiles; t++) A[t] = src[t * 64];
    }
    // tiles past the segment load its last tile (never consumed)
    auto unit_addr = [&](int t) { return (ta + min(t, nt - 1)) * cpr + c; };
    uint32_t buf[kLutRing][12];
    int tile[kLutRing];
#pragma unroll
    for (int r = 0; r < kLutRing - 1; r++) {
        tile[r] = wave + kPW * r;
        load_codes(gb, unit_addr(tile[r]), lane, buf[r]);
    }
    if (!pre()) return false;
    lds_sync();                    // the previous table's readers and counter users are done
    if (threadIdx.x == 0) *ctr = kPW * (kLutRing - 1);
    const int e = lut_build(A, xo, wave);
    lds_sync();
    if (built && threadIdx.x == 0) *built = wall_clock64();   // profiling stamp: the table is ready
    // a wave's tiles only grow, so once one is past the segment, all later ones are
    for (;;) {
#pragma unroll
        for (int r = 0; r < kLutRing; r++) {
            const int nr = (r + kLutRing - 1) % kLutRing;
            tile[nr] = lut_next_tile(ctr, lane);
            load_codes(gb, unit_addr(tile[nr]), lane, buf[nr]);
            if (tile[r] < nt)
                st_pair(part + (size_t)(ta + tile[r]) * tstride, ldexpf(lut_strip(buf[r]), e), tag, lane);
        }
        if (tile[kLutRing - 1] >= nt) break;
    }
    return true;
}

// Workgroup whose down range holds the last unit of output tile td in the
// last rank: it combines the tile.
__device__ __forceinline__ int combiner_of(int td, int k, int tilesH, int cprI, int nD, int G) {
    return range_owner(nD, G, ((k - 1) * tilesH + td + 1) * cprI - 1);
}

// Output tile td, by one wave: out = sum_j w_j * sum_slots y_j + shared, in
// fixed (rank, contributor) order, from tagged partials polled until every
// contribution of this step is there.  Each poll loads RG ranks' partials (up
// to 4 contributors each) and, the first time, the shared output, so a layer
// of up to RG ranks needs one round trip once the last partial lands.
// Returns false on a failed wait.
template <int RG>
__device__ __forceinline__ bool combine_tile(int td, int s, unsigned tag, int k, int tilesH, int cprI, int nD,
                                             int G, int H, bool shared_on, const uint64_t *part_d, int slots_d,
                                             const uint64_t *ysh, float *out, const float *sw, unsigned *sync,
                                             int lane) {
    const int r = td * kTileRows + lane;
    float o = 0.f, sh = 0.f;
    long spins = 0;
    // ranks RG at a time, contributors 4 at a time: up to 4 RG partials (and
    // the shared output) in flight per poll
    for (int j0 = 0; j0 < k; j0 += RG) {
        float ya[RG];
        int cj[RG];
        const uint64_t *pj[RG];
        int cmax = 0;
#pragma unroll
        for (int jj = 0; jj < RG; jj++) {
            const int t = min(j0 + jj, k - 1) * tilesH + td;
            cj[jj] = range_owner(nD, G, (t + 1) * cprI - 1) - range_owner(nD, G, t * cprI) + 1;
            pj[jj] = part_d + (size_t)t * slots_d * 64 + lane;
            cmax = max(cmax, cj[jj]);
            ya[jj] = 0.f;
        }
        for (int q0 = 0; q0 < cmax; q0 += 4) {
            const bool with_shared = shared_on && j0 == 0 && q0 == 0;
            uint64_t v[RG][4], vs = 0;
            for (;;) {
                bool ok = true;
#pragma unroll
                for (int jj = 0; jj < RG; jj++)
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        v[jj][q] = ld_tagged(pj[jj] + (size_t)min(q0 + q, cj[jj] - 1) * 64);
                        ok = ok && tag_ok(v[jj][q], tag);
                    }
                if (with_shared) {
                    vs = ld_tagged(ysh + r);
                    ok = ok && tag_ok(vs, tag);
                }
                if (__all(ok)) break;
                if (!poll_more(sync, spins)) return false;
            }
#pragma unroll
            for (int jj = 0; jj < RG; jj++)
#pragma unroll
                for (int q = 0; q < 4; q++)
                    if (j0 + jj < k && q0 + q < cj[jj]) ya[jj] += tag_val(v[jj][q]);
            if (with_shared) sh = tag_val(vs);
        }
#pragma unroll
        for (int jj = 0; jj < RG; jj++)
            if (j0 + jj < k) o = fmaf(sw[j0 + jj], ya[jj], o);
    }
    if (shared_on) o += sh;
    out[(size_t)s * H + r] = o;
    return true;
}

// Output rows [16 sl, 16 sl + 16) for the table-lookup down, by the whole
// workgroup (H / 16 such slices spread over all workgroups, so each reads a
// 16th of a tile's partials: one 128-byte line per (rank, chunk)).  Lane l
// takes row 16 sl + l % 16 of the partials p = 4 (v + 8 q) + l / 16 (wave v,
// p = rank cprI + chunk, every load of a wave in flight together; polls after
// the first reload only the words still missing) and weights them by
// fj[rank][l % 16] = w_j s_j[row] (gate weight times row scale, in LDS, filled
// by the caller before the barrier below).  The four lanes of a row, then the
// waves in order, are added; wave 0 adds the shared output, writes the rows
// and counts the slice on the layer-done counter.  Returns false on a failed
// wait (the same on every wave).
constexpr int kSliceRows = 16;
template <int NB, int LC>
__device__ __forceinline__ bool combine_slice_lut(int sl, int s, unsigned tag, int k, int tilesH, int cprI, int H,
                                                  bool shared_on, const uint64_t *part_d, const uint64_t *ysh,
                                                  float *out, const float *fj, unsigned *sync, int *bcast, int wave,
                                                  int lane) {
    float *jr = (float *)(dec_lds + kLutX + 512 + MOE_MAX_K * kSliceRows * 4);   // [kPW][16] the waves' sums
    const int rr = lane & (kSliceRows - 1), pq = lane >> 4;
    const int r = sl * kSliceRows + rr, td = r / kTileRows;
    const int np = k * cprI;
    const unsigned t16 = tag16(s);
    float acc = 0.f;
    long spins = 0;
    bool ok = true;
    lds_sync();                              // fj is complete
    for (int p0 = 4 * wave + pq; __any(p0 < np) && ok; p0 += NB * 4 * kPW) {
        uint64_t v[NB];
        const uint64_t *pa[NB];
        int jq[NB];
#pragma unroll
        for (int q = 0; q < NB; q++) {
            const int p = min(p0 + q * 4 * kPW, np - 1);
            jq[q] = p / cprI;
            pa[q] = part_d + (((size_t)jq[q] * tilesH + td) * cprI + (p - jq[q] * cprI)) * 32 + (r & 31);
            v[q] = ld_tagged(pa[q]);
        }
        for (;;) {
            bool all = true;
#pragma unroll
            for (int q = 0; q < NB; q++) all = all && pair_ok(v[q], t16);
            if (__all(all)) break;
            if (!poll_more(sync, spins)) { ok = false; break; }
#pragma unroll
            for (int q = 0; q < NB; q++)
                if (!pair_ok(v[q], t16)) v[q] = ld_tagged(pa[q]);
        }
        if (!ok) break;
#pragma unroll
        for (int q = 0; q < NB; q++)
            if (p0 + q * 4 * kPW < np) acc = fmaf(fj[jq[q] * kSliceRows + rr], pair_val(v[q], r & 63), acc);
    }
    acc += __shfl_xor(acc, 16, 64);
    acc += __shfl_xor(acc, 32, 64);
    if (lane < kSliceRows) jr[wave * kSliceRows + lane] = acc;
    if (!ok && lane == 0) *bcast = 0;
    lds_sync();
    if (!*bcast) return false;
    if (wave == 0) {
        float o = 0.f;
#pragma unroll
        for (int v = 0; v < kPW; v++) o += jr[v * kSliceRows + rr];
        bool oks = true;
        if (shared_on) {
            uint64_t vs;
            for (;;) {
                vs = ld_tagged(ysh + r);
                if (__all(tag_ok(vs, tag))) break;
                if (!poll_more(sync, spins)) { oks = false; break; }
            }
            o += tag_val(vs);
        }
        if (oks) {
            if (lane < kSliceRows) out[(size_t)s * H + r] = o;
            // counted at once: nothing in this launch reads the outputs
            if (lane == 0)
                __hip_atomic_fetch_add(sync + kLayerDone + (sl % LC) * kLine, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        } else if (lane == 0) {
            *bcast = 0;
        }
    }
    lds_sync();
    return *bcast != 0;
}

struct DecArgs {
    const DecLayer *layers;  // [nL] in device memory
    int nL, T, H, I, k, E_max, G;
    int has_shared;
    const float *x;          // [T, nL, H]
    float *out;              // [T, nL, H]
    int32_t *idx_out;        // [T, nL, k] or null
    RecOffsets off;
    unsigned *sync;          // counters
    uint64_t *z;             // [E_max] tagged logits
    float *hh;               // [k][I] fp32 h per rank (gather down)
    uint64_t *hq;            // [k][I] tagged fp32 h per rank (down by table lookup)
    float *hs;               // [I] shared h
    uint64_t *ysh;           // [H] tagged shared y
    uint64_t *part_gu;       // [k*tilesI][slots_gu][128] tagged ([64] row pairs by table lookup)
    uint64_t *part_d;        // [k*tilesH][slots_d][64] tagged ([32] row pairs by table lookup)
    int slots_gu, slots_d;
    int slots_red_gu, slots_red_d;   // tiles one workgroup's range can touch (LDS sum slots)
    int lut;                 // kLutGateUp | kLutDown: the phases done by table lookup
                             // (part_gu, part_d then have one slot per chunk of
                             // H, I)
    unsigned long long *stamps;   // optional phase timestamps [steps][G][kDecStamps], or null
    int stamp_steps;
};

// LC: layer-done counter copies (8 where a step has few output units, 16
// where it has many: fewer adders per copy, more words per wait)
template <int LC>
__global__ __launch_bounds__(kPW * 64) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_decode_persistent(DecArgs a) {
    char *lds = dec_lds;
    const DecLds LL = dec_lds_layout(a.H, a.I);
    const float *red_gu = (const float *)(lds + LL.red_gu);     // [slot][kPW][2][64]
    const float *red_d = (const float *)(lds + LL.red_d);       // [slot][kPW][64]
    int *sidx = (int *)(lds + kDecTail);                        // [MOE_MAX_K]
    float *sw = (float *)(sidx + MOE_MAX_K);                    // [MOE_MAX_K]
    int *bcast = (int *)(sw + MOE_MAX_K);                       // [4]
    float *red = (float *)(bcast + 4);                          // [kPW] router partials
    uint64_t *recs = (uint64_t *)(red + kPW);                   // [MOE_MAX_K] records of the chosen experts
    float *lmax = (float *)(recs + MOE_MAX_K);                  // [kPW] the waves' largest magnitudes
    uint64_t *recs_all = (uint64_t *)(lds + kDecRecs);          // [E] until top-k

    // XCD-major work index: workgroup b runs on XCD b % 8 (the dispatcher
    // deals workgroups round-robin over the 8 XCDs), so with w as below the 32
    // workgroups of one XCD take a contiguous slice of every phase's unit
    // space: one XCD streams the tiles of one (expert, matrix) and its L2
    // fetches that codebook and that chunk of x once, instead of every XCD
    // fetching every codebook.
    const int G = a.G;
    const int w = G % kXcds == 0 ? (int)(blockIdx.x % kXcds) * (G / kXcds) + (int)(blockIdx.x / kXcds) : (int)blockIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int H = a.H, I = a.I, k = a.k;
    const int tilesI = I / kTileRows, tilesH = H / kTileRows;
    const int cprH = H / kChunkCols, cprI = I / kChunkCols;
    const int nGU = k * tilesI * cprH, nD = k * tilesH * cprI;
    const int gu0 = range_start(nGU, G, w), gu1 = range_start(nGU, G, w + 1);
    const int d0 = range_start(nD, G, w), d1 = range_start(nD, G, w + 1);
    unsigned *sync = a.sync;
    unsigned *h_ready = sync + kHReady;                          // [k+1], kLine apart
    const int steps = a.T * a.nL;
    // shared-expert row ranges
    const int shI0 = range_start(I, G, w), shI1 = range_start(I, G, w + 1);
    const int shH0 = range_start(H, G, w), shH1 = range_start(H, G, w + 1);
    const unsigned sh_gu_contrib = (unsigned)min(G, I);          // workgroups with shared gate/up rows
    // Whether this workgroup uses a step's routing result.  Which workgroups
    // own gate/up units, joins, down units or output units depends only on
    // the shape (workgroup w owns some of an n-unit space iff w < min(n, G)),
    // never on the experts chosen.  A workgroup that owns none of them skips
    // the logit poll: every workgroup that polls the step-tagged logits of
    // step s owns work that the step-(s+1) layer-done barrier waits for, so
    // no poller can still be reading step s's logits when they are retagged.
    const bool routed = [&] {
        const bool lg = a.lut & kLutGateUp, ld = a.lut & kLutDown;
        const long gu_units = lg ? (long)k * 2 * cprH * tilesI : nGU;
        const long join_units = lg ? (long)k * tilesI : 0;       // gather joins: owners of gate/up units
        const long d_units = ld ? (long)k * cprI : nD;           // table-lookup down: (rank, chunk) segments
        const long out_units = ld ? (long)(H / kSliceRows) : 0;  // gather combines: owners of down units
        return w == 0 || w < gu_units || w < join_units || w < d_units || w < out_units;
    }();

    unsigned long long *stamp = nullptr;
    auto mark = [&](int i) {
        if (stamp && threadIdx.x == 0) stamp[i] = wall_clock64();
    };
    for (int s = 0; s < steps; s++) {
        stamp = (a.stamps && s < a.stamp_steps) ? a.stamps + ((size_t)s * G + w) * kDecStamps : nullptr;
        mark(kStampStart);
        const int t = s / a.nL, L = s % a.nL;
        const DecLayer lay = a.layers[L];   // device memory, uniform
        const float *xs = a.x + ((size_t)t * a.nL + L) * H;
        const int E = lay.E, nE = min(E, G);
        const bool shared_on = a.has_shared && lay.shared;
        // the layer's record pointers, loaded while waiting (the table is
        // fixed during the launch): the chosen experts' loads can start right
        // after top-k
        for (int e = threadIdx.x; e < E; e += kPW * 64) recs_all[e] = gld((const uint64_t *)lay.records + e);
        // output units per step: 64-row tiles, or 16-row slices (down by table lookup)
        if (s > 0 && !wg_wait<LC>(sync, sync + kLayerDone,
                                 (unsigned)s * ((a.lut & kLutDown) ? H / kSliceRows : tilesH), bcast))
            return;
        if (s == 0) lds_sync();
        mark(kStampLayerWait);

        const unsigned tag = (unsigned)s + 1;
        {
            // the top-k's candidate list and count (LDS free since the last step ended)
            uint64_t *cand0 = (uint64_t *)(lds + kTopkScratch) + MOE_MAX_E;
            for (int i = threadIdx.x; i < kTopkGroups * MOE_MAX_K; i += kPW * 64) cand0[i] = 0u;
        }

        // ---- x as fp16 pairs into LDS (every workgroup, for gate/up), in
        // one pass with this workgroup's first logit row (e = w, if w < E):
        // thread t takes the float4 pieces c = 4t + 2048 m of x and of the
        // row, up to four pieces' loads in flight together, and multiplies
        // them in increasing m, the order of the row loop below (pieces past
        // H add fma(0, 0), as there)
        float acc_w = 0.f;
        int xe = 0;                 // gather gate/up: x enters as fp16 pairs scaled by 2^-xe
        // thread 0: the bias of logit row w, loaded together with x and the row
        const float bias_w = threadIdx.x == 0 && lay.bias && w < nE ? gld(lay.bias + w) : 0.f;
        {
            float *xst = (float *)(lds + kXStage);   // gathers: fp32 x, packed below once xe is known
            float xm = 0.f;
            const bool row_w = w < nE;
            const float *wr = lay.W + (size_t)(row_w ? w : 0) * H;
            const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
            constexpr int kPiece = kPW * 64 * 4;
            for (int c = threadIdx.x * 4; c < H; c += 4 * kPiece) {
                float4 xv[4], wv[4];
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const int cu = c + u * kPiece;
                    xv[u] = cu < H ? gld4(xs + cu) : zero4;
                    wv[u] = cu < H && row_w ? gld4(wr + cu) : zero4;
                }
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const int cu = c + u * kPiece;
                    if (cu < H && (a.lut & kLutGateUp)) {
                        *(float4 *)(lds + kLutX + 4 * cu) = xv[u];   // fp32, for the table builds
                    } else if (cu < H) {
                        *(float4 *)(xst + cu) = xv[u];
                        xm = fmaxf(xm, fmaxf(fmaxf(fabsf(xv[u].x), fabsf(xv[u].y)),
                                             fmaxf(fabsf(xv[u].z), fabsf(xv[u].w))));
                    }
                    acc_w = fmaf(wv[u].x, xv[u].x, acc_w);
                    acc_w = fmaf(wv[u].y, xv[u].y, acc_w);
                    acc_w = fmaf(wv[u].z, xv[u].z, acc_w);
                    acc_w = fmaf(wv[u].w, xv[u].w, acc_w);
                }
            }
            xm = wave_max(xm);
            if (lane == 0) lmax[wave] = xm;    // read after the logit poll's barrier
        }

        // ---- route: logits of rows e = w, w + G, ... (tagged, no counter)
        if (w < nE) {
            for (int e = w; e < E; e += G) {
                const float *wr = lay.W + (size_t)e * H;
                // thread 0: this row's bias, in flight with the row's loads
                const float be = threadIdx.x == 0 && lay.bias ? (e == w ? bias_w : gld(lay.bias + e)) : 0.f;
                float acc = e == w ? acc_w : 0.f;
                for (int c0 = threadIdx.x * 4; c0 < H && e != w; c0 += 2 * kPW * 64 * 4) {
                    // two chunks' loads in flight together
                    const int c1 = c0 + kPW * 64 * 4;
                    const float4 w0 = gld4(wr + c0), x0 = gld4(xs + c0);
                    const bool two = c1 < H;
                    const float4 w1 = two ? gld4(wr + c1) : make_float4(0.f, 0.f, 0.f, 0.f);
                    const float4 x1 = two ? gld4(xs + c1) : make_float4(0.f, 0.f, 0.f, 0.f);
                    acc = fmaf(w0.x, x0.x, acc);
                    acc = fmaf(w0.y, x0.y, acc);
                    acc = fmaf(w0.z, x0.z, acc);
                    acc = fmaf(w0.w, x0.w, acc);
                    acc = fmaf(w1.x, x1.x, acc);
                    acc = fmaf(w1.y, x1.y, acc);
                    acc = fmaf(w1.z, x1.z, acc);
                    acc = fmaf(w1.w, x1.w, acc);
                }
                acc = wave_sum(acc);
                lds_sync();
                if (lane == 0) red[wave] = acc;
                lds_sync();
                if (threadIdx.x == 0) {
                    float z = 0.f;
                    for (int v = 0; v < kPW; v++) z += red[v];
                    st_tagged(a.z + e, z + be, tag);
                }
            }
        }

        // ---- shared gate/up (independent of routing) on waves 1..7 while
        // wave 0 polls the logits.  The workgroup's rows go kShRows at a
        // time, each thread on 8 columns of every row of the group: all
        // weight loads are in flight together, then one reduction per group.
        // A workgroup with more than kShRows rows (I > kShRows * G) does the
        // further groups with all waves after the poll.
        const bool sh_rows = shared_on && shI1 > shI0;
        float *shred = (float *)lds;   // [kPW][2 * kShRows], codebook area (free until gate/up)
        // (NR rows per group: 4 where a workgroup has at most 4 rows)
        auto shared_partials = [&](auto nr_tag, int r0, int t, int nthr) {
            constexpr int NR = decltype(nr_tag)::value;
            const uint16_t *wg0 = lay.shared, *wu0 = lay.shared + (size_t)I * H;
            float g[NR], u[NR];
#pragma unroll
            for (int q = 0; q < NR; q++) g[q] = u[q] = 0.f;
            for (int c = t * 8; c < H; c += nthr * 8) {
                const float4 xa = gld4(xs + c), xb = gld4(xs + c + 4);
                uint4 gv[NR], uv[NR];
#pragma unroll
                for (int q = 0; q < NR; q++) {
                    const size_t o = (size_t)min(r0 + q, shI1 - 1) * H + c;
                    gv[q] = gldu4(wg0 + o);
                    uv[q] = gldu4(wu0 + o);
                }
                const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
                for (int q = 0; q < NR; q++) {
                    const uint32_t gq[4] = {gv[q].x, gv[q].y, gv[q].z, gv[q].w};
                    const uint32_t uq[4] = {uv[q].x, uv[q].y, uv[q].z, uv[q].w};
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        g[q] = fmaf(__uint_as_float(gq[i] << 16), xv[2 * i], g[q]);
                        g[q] = fmaf(__uint_as_float(gq[i] & 0xFFFF0000u), xv[2 * i + 1], g[q]);
                        u[q] = fmaf(__uint_as_float(uq[i] << 16), xv[2 * i], u[q]);
                        u[q] = fmaf(__uint_as_float(uq[i] & 0xFFFF0000u), xv[2 * i + 1], u[q]);
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < NR; q++) {
                g[q] = wave_sum(g[q]);
                u[q] = wave_sum(u[q]);
            }
            if (lane == 0) {
#pragma unroll
                for (int q = 0; q < NR; q++) {
                    shred[wave * 2 * kShRows + q] = g[q];
                    shred[wave * 2 * kShRows + kShRows + q] = u[q];
                }
            }
        };
        // wave 1 finishes a group from the waves' partials v0..kPW-1
        auto shared_finish = [&](int r0, int v0) {
            const int nr = min(kShRows, shI1 - r0);
            if (wave == 1 && lane < nr) {
                float gg = 0.f, uu = 0.f;
                for (int v = v0; v < kPW; v++) {
                    gg += shred[v * 2 * kShRows + lane];
                    uu += shred[v * 2 * kShRows + kShRows + lane];
                }
                st_x(a.hs + r0 + lane, gg / (1.f + __expf(-gg)) * uu);
            }
        };

        // ---- top-k: wave 0 polls the tagged logits into LDS as
        // order-preserving keys; then every thread ranks its experts by
        // counting the ones ahead of it in (logit desc, expert id asc) order
        // (no lane exchanges, no dependency chain); ranks below k land in
        // rank order, and wave 0 computes the weights in that order.
        // key of expert e: order_key(z) << 32 | (2^32 - 1 - e), so one 64-bit
        // comparison orders by logit, then by lower id
        uint64_t *zkey = (uint64_t *)(lds + kTopkScratch);    // [E rounded up to 32]
        float *sz = (float *)(zkey + MOE_MAX_E + kTopkGroups * MOE_MAX_K);   // [MOE_MAX_K] logits in rank order
        if (wave == 0 && !routed) {
            if (lane == 0) *bcast = 1;
        } else if (wave == 0) {
            long spins = 0;
            bool okw = true;
            for (;;) {
                bool ok = true;
#pragma unroll
                for (int i = 0; i < MOE_MAX_E / 64; i++) {
                    const int e = lane + 64 * i;
                    if (e < E) {
                        const uint64_t zz = ld_tagged(a.z + e);
                        ok = ok && tag_ok(zz, tag);
                        const float f = tag_val(zz);
                        zkey[e] = (uint64_t)order_key(f == f ? f : -INFINITY) << 32 | (0xFFFFFFFFu - (uint32_t)e);
                    } else if (e < ((E + 31) & ~31)) {
                        zkey[e] = 0u;   // padding: below every real key
                    }
                }
                if (__all(ok)) break;
                if (!poll_more(sync, spins)) { okw = false; break; }
            }
            if (lane == 0) *bcast = okw;
        } else if (sh_rows) {
            if (shI1 - shI0 <= 4)
                shared_partials(std::integral_constant<int, 4>{}, shI0, (int)threadIdx.x - 64, (kPW - 1) * 64);
            else
                shared_partials(std::integral_constant<int, kShRows>{}, shI0, (int)threadIdx.x - 64,
                                (kPW - 1) * 64);
        }
        lds_sync();
        if (!*bcast) return;
        if (!(a.lut & kLutGateUp)) {
            // x as fp16 pairs for the gathers, scaled by 2^-xe (xe from the
            // largest |x|, the same in every workgroup)
            float m = lmax[0];
#pragma unroll
            for (int v = 1; v < kPW; v++) m = fmaxf(m, lmax[v]);
            xe = __builtin_amdgcn_readfirstlane(range_exp(m));
            const float *xst = (const float *)(lds + kXStage);
            uint32_t *xl = (uint32_t *)(lds + LL.x_gu);
            for (int p = threadIdx.x; p < H / 2; p += kPW * 64) {
                const float2 v = *(const float2 *)(xst + 2 * p);
                xl[p] = pack_f16x2(ldexpf(v.x, -xe), ldexpf(v.y, -xe));
            }
        }
        if (routed) {
            // Exact top-k by counting: a key's rank is the number of keys
            // above it (keys are unique: logit bits above the inverted id).
            // For E > 64 in two levels: each key is first ranked within its
            // group (E split into kTopkGroups ranges of whole 32-key blocks);
            // keys of local rank < k are candidates (every global top-k key is
            // one), each in the slot (group, local rank), and are ranked among
            // themselves.
            const int kk = __builtin_amdgcn_readfirstlane(lay.k);
            const bool two = E > 64;
            const int gsz = two ? ((E + kTopkGroups - 1) / kTopkGroups + 31) & ~31 : (E + 31) & ~31;
            uint64_t *cand = zkey + MOE_MAX_E;                  // [kTopkGroups * MOE_MAX_K], zeroed while routing began
            // rank of key ke among the keys at list[q0, q1) (q0, q1 multiples of 32)
            auto count_above = [&](const uint64_t *list, int q0, int q1, uint64_t ke) {
                int r[4] = {0, 0, 0, 0};
                for (; q0 < q1 && r[0] + r[1] + r[2] + r[3] < kk; q0 += 32) {
                    uint64_t kv[32];
#pragma unroll
                    for (int i = 0; i < 16; i++) {   // 32 keys per step (broadcast reads)
                        const u32x4 tw = *(const u32x4 *)(list + q0 + 2 * i);
                        kv[2 * i] = (uint64_t)tw.y << 32 | tw.x;
                        kv[2 * i + 1] = (uint64_t)tw.w << 32 | tw.z;
                    }
#pragma unroll
                    for (int i = 0; i < 32; i++) r[i & 3] += kv[i] > ke;   // four independent counts
                }
                return r[0] + r[1] + r[2] + r[3];
            };
            auto place = [&](int rank, uint64_t ke) {
                sidx[rank] = (int)(0xFFFFFFFFu - (uint32_t)ke);
                sz[rank] = key_value((uint32_t)(ke >> 32));
            };
            for (int e = threadIdx.x; e < E; e += kPW * 64) {
                const uint64_t ke = zkey[e];
                const int g0 = e / gsz * gsz;
                const int rank = count_above(zkey, g0, min((E + 31) & ~31, g0 + gsz), ke);
                if (rank < kk) {
                    if (two) cand[e / gsz * kk + rank] = ke;   // a slot of its own: (group, local rank)
                    else place(rank, ke);
                }
            }
            if (two) {
                lds_sync();
                // the groups' candidates, zeros where a group had fewer than k
                // keys (zero is below every real key; the candidate area is
                // zeroed up to its end, kTopkGroups * MOE_MAX_K >= ncp).  Each
                // candidate is ranked by P threads (every thread of the
                // workgroup takes part), each counting a P-th of the list; the
                // P counts are added across their lanes.
                const int nc = (E + gsz - 1) / gsz * kk;
                int ncp = 32;
                while (ncp < nc) ncp <<= 1;
                const int P = max(1, kPW * 64 / ncp), len = ncp / P;
                const int c = threadIdx.x / P, q0 = (threadIdx.x % P) * len;
                const uint64_t ke = c < nc ? cand[c] : 0u;
                int rank = 0;
                for (int q = q0; q < q0 + len; q += 2) {
                    const u32x4 tw = *(const u32x4 *)(cand + q);
                    rank += ((uint64_t)tw.y << 32 | tw.x) > ke;
                    rank += ((uint64_t)tw.w << 32 | tw.z) > ke;
                }
                for (int o = 1; o < P; o <<= 1) rank += __shfl_xor(rank, o, 64);
                if (threadIdx.x % P == 0 && ke && rank < kk) place(rank, ke);
            }
        }
        lds_sync();
        if (routed && wave == 0) {
            // lane r < k scores rank r; the sum runs in rank order
            const int kk = __builtin_amdgcn_readfirstlane(lay.k);
            const float zmax = sz[0];
            float sc = 0.f;
            if (lane < kk) {
                const float z = sz[lane];
                sc = lay.score_fn == MOE_SCORE_SOFTMAX ? __expf(z - zmax) : 1.f / (1.f + __expf(-z));
            }
            float sum = 0.f;
            for (int r = 0; r < kk; r++) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), r));
            if (lane < kk) {
                const int e = sidx[lane];
                sw[lane] = sc / sum;
                recs[lane] = recs_all[e];
                if (w == 0 && a.idx_out) a.idx_out[(size_t)s * k + lane] = e;
            }
        }
        lds_sync();
        // the shared rows' SiLU(g) * u, stored after the top-k: a wave's
        // stores hold its later vector-memory waits (which the top-k's
        // register reuse brings in), and the shared down reads these rows
        // only after the gate/up phase
        if (sh_rows) {
            shared_finish(shI0, 1);
            for (int r0 = shI0 + kShRows; r0 < shI1; r0 += kShRows) {
                lds_sync();
                shared_partials(std::integral_constant<int, kShRows>{}, r0, threadIdx.x, kPW * 64);
                lds_sync();
                shared_finish(r0, 0);
            }
        }
        mark(kStampRouted);
        // wave 1 wrote every shared row of this workgroup: it counts them once
        // its stores are done, at the first point after routing where it
        // waits for its memory operations anyway (gathers: the codebook
        // staging) or, at the latest, before this workgroup's first wait on
        // another workgroup (the joins), so the count never waits on them
        bool sh_counted = !(sh_rows && wave == 1);
        // the shared h counter, loaded after the gate/up loop (its round trip
        // overlaps the joins): where it already shows every row, the shared
        // down needs no poll of its own
        unsigned sh_early = 0;
        auto count_shared = [&] {
            if (!sh_counted) {
                wait_vm_all();
                if (lane == 0)
                    __hip_atomic_fetch_add(h_ready + k * kLine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                sh_counted = true;
            }
        };

        if (a.lut & kLutGateUp) {
            // ---- gate/up by table lookup over this workgroup's range of the
            // (rank, matrix, chunk, tile) space, one segment (fixed rank,
            // matrix and chunk) at a time; each tile's sum over the chunk goes
            // out as a row-pair partial (slot = chunk; gate in words 0..31, up
            // in 32..63)
            // (32-bit index math: the host allows this path only where
            // nL * G fits an int)
            const int nL = k * 2 * cprH * tilesI;
            const int GaL = min(nL, G);
            const int l1 = w + 1 >= GaL ? nL : nL * (w + 1) / GaL;
            for (int ua = w >= GaL ? nL : nL * w / GaL; ua < l1;) {
                const int seg = ua / tilesI;
                const int ub = min(l1, (seg + 1) * tilesI);
                const int c = seg % cprH, m = (seg / cprH) & 1, j = seg / (2 * cprH);
                const uint8_t *rec = (const uint8_t *)recs[j];
                const int ta = ua - seg * tilesI;
                stream_lut((const u32x4 *)(rec + a.off.codes[m]), (const u32x4 *)(rec + a.off.cb[m]), cprH, c,
                           kLutX + 4 * kChunkCols * c, ta, ub - ua,
                           a.part_gu + ((size_t)j * tilesI * cprH + c) * 64 + m * 32, 64 * cprH, tag16(s), wave, lane,
                           [] { return true; }, stamp ? stamp + kStampGuStaged : nullptr);
                ua = ub;
            }
            lds_sync();
            mark(kStampGuLoop);
            count_shared();
            if (shared_on) sh_early = ld_cnt(h_ready + k * kLine);
            // joins: tiles tau = w + G i of all ranks' k * tilesI tiles, two at
            // a time.  Wave v polls slots v, v + kPW, ... of both tiles (all its
            // loads in flight together: one round trip once the partials have
            // landed) and sums them in slot order; the waves' sums meet in LDS,
            // and wave tt adds them in wave order for tile tt, scales, and
            // writes SiLU(g) * u: fp16 for a gather down, else fp32 as
            // step-tagged words (down by table lookup polls them per chunk).
            bool okj = true;
            const unsigned t16 = tag16(s);
            const int nTau = k * tilesI;
            const int nT = w < nTau ? (nTau - 1 - w) / G + 1 : 0;
            float *jred = (float *)lds;     // [2][kPW][128], table area (free now)
            for (int p0 = 0; p0 < nT; p0 += 2) {
                const int tn = min(2, nT - p0);
                float gs[2] = {0.f, 0.f}, us[2] = {0.f, 0.f};
                for (int s0 = wave; s0 < cprH && okj; s0 += 4 * kPW) {
                    uint64_t vg[2][4], vu[2][4];
                    const uint64_t *pp[2][4];
                    long spins = 0;
#pragma unroll
                    for (int tt = 0; tt < 2; tt++)
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            const int tau = w + G * (p0 + min(tt, tn - 1));
                            const int sl = min(s0 + q * kPW, cprH - 1);
                            pp[tt][q] = a.part_gu + ((size_t)tau * cprH + sl) * 64 + (lane & 31);
                            vg[tt][q] = ld_tagged(pp[tt][q]);
                            vu[tt][q] = ld_tagged(pp[tt][q] + 32);
                        }
                    // later polls reload only the words still missing
                    for (;;) {
                        bool ok = true;
#pragma unroll
                        for (int tt = 0; tt < 2; tt++)
#pragma unroll
                            for (int q = 0; q < 4; q++) ok = ok && pair_ok(vg[tt][q], t16) && pair_ok(vu[tt][q], t16);
                        if (__all(ok)) break;
                        if (!poll_more(sync, spins)) { okj = false; break; }
#pragma unroll
                        for (int tt = 0; tt < 2; tt++)
#pragma unroll
                            for (int q = 0; q < 4; q++) {
                                if (!pair_ok(vg[tt][q], t16)) vg[tt][q] = ld_tagged(pp[tt][q]);
                                if (!pair_ok(vu[tt][q], t16)) vu[tt][q] = ld_tagged(pp[tt][q] + 32);
                            }
                    }
                    if (!okj) break;
#pragma unroll
                    for (int tt = 0; tt < 2; tt++)
#pragma unroll
                        for (int q = 0; q < 4; q++)
                            if (s0 + q * kPW < cprH) {
                                gs[tt] += pair_val(vg[tt][q], lane);
                                us[tt] += pair_val(vu[tt][q], lane);
                            }
                }
#pragma unroll
                for (int tt = 0; tt < 2; tt++) {
                    jred[(tt * kPW + wave) * 128 + lane] = gs[tt];
                    jred[(tt * kPW + wave) * 128 + 64 + lane] = us[tt];
                }
                lds_sync();
                if (wave < tn) {
                    const int tau = w + G * (p0 + wave);
                    const int j = (int)(tau / tilesI);
                    const uint8_t *rec = (const uint8_t *)recs[j];
                    const int r = (int)(tau % tilesI) * kTileRows + lane;
                    float g = 0.f, uu = 0.f;
#pragma unroll
                    for (int v = 0; v < kPW; v++) {
                        g += jred[(wave * kPW + v) * 128 + lane];
                        uu += jred[(wave * kPW + v) * 128 + 64 + lane];
                    }
                    g *= (float)gld((const _Float16 *)(rec + a.off.scales[0]) + r);
                    uu *= (float)gld((const _Float16 *)(rec + a.off.scales[1]) + r);
                    const float hv = g / (1.f + __expf(-g)) * uu;
                    if (a.lut & kLutDown) {
                        st_tagged(a.hq + (size_t)j * I + r, hv, tag);   // read per chunk by down
                    } else {
                        st_x(a.hh + (size_t)j * I + r, hv);
                    }
                }
                lds_sync();
            }
            if (lane == 0 && !okj) *bcast = 0;
            if (a.lut & kLutDown) {
                // h is tagged: no wait for the stores, no counter
                lds_sync();
                if (!*bcast) return;
            } else {
                wait_vm_all();
                __syncthreads();
                if (!*bcast) return;
            }
            if (threadIdx.x == 0 && !(a.lut & kLutDown))
                for (int tau = w; tau < k * tilesI; tau += G)
                    __hip_atomic_fetch_add(h_ready + (tau / tilesI) * kLine, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        }
        // ---- gate/up over this workgroup's range of (rank, tile, chunk), one
        // expert segment at a time (a range spans at most two experts)
        for (int ea = (a.lut & kLutGateUp) ? gu1 : gu0; ea < gu1;) {
            const int j = ea / (tilesI * cprH);
            const int eb = min(gu1, (j + 1) * tilesI * cprH);
            const uint8_t *rec = (const uint8_t *)recs[j];
            const int base = j * tilesI * cprH;              // expert-local units
            stream_gateup((const u32x4 *)(rec + a.off.codes[0]), (const u32x4 *)(rec + a.off.codes[1]),
                          (const u32x4 *)(rec + a.off.cb[0]), (const u32x4 *)(rec + a.off.cb[1]), H, I, cprH,
                          ea - base, eb - base, ea / cprH - base / cprH, a.slots_red_gu, wave,
                          lane, stamp, sh_counted ? nullptr : h_ready + k * kLine);
            sh_counted = true;
            lds_sync();
            mark(kStampGuLoop);
            if (shared_on) sh_early = ld_cnt(h_ready + k * kLine);
            // one tagged partial per touched tile (wave v: tiles v, v + kPW,
            // ...); the workgroup owning a tile's last unit joins it (one
            // wave per tile) into fp16 SiLU(g) * u once every contributor's
            // partial of this step is there
            const int tA = ea / cprH;
            const int nt = (eb - 1) / cprH - tA + 1;
            for (int v = wave; v < nt; v += kPW) {
                const int tau = tA + v;
                const int slot = w - range_owner(nGU, G, tau * cprH);
                float g = 0.f, uu = 0.f;
#pragma unroll
                for (int q = 0; q < kPW; q++) {
                    g += red_gu[(v * kPW + q) * 128 + lane];
                    uu += red_gu[(v * kPW + q) * 128 + 64 + lane];
                }
                uint64_t *p = a.part_gu + ((size_t)tau * a.slots_gu + slot) * 128;
                st_tagged(p + lane, g, tag);
                st_tagged(p + 64 + lane, uu, tag);
            }
            int nj = 0;
            bool okj = true;
            for (int v = 0; v < nt; v++) {
                const int tau = tA + v;
                if (range_owner(nGU, G, (tau + 1) * cprH - 1) != w) continue;
                if (nj++ % kPW != wave) continue;
                const int first = range_owner(nGU, G, tau * cprH), ncontrib = w - first + 1;
                const int r = tau % tilesI * kTileRows + lane;
                const float sg = (float)gld((const _Float16 *)(rec + a.off.scales[0]) + r);
                const float su = (float)gld((const _Float16 *)(rec + a.off.scales[1]) + r);
                const uint64_t *pp = a.part_gu + (size_t)tau * a.slots_gu * 128 + lane;
                float g = 0.f, uu = 0.f;
                long spins = 0;
                for (int s0 = 0; s0 < ncontrib && okj; s0 += 4) {
                    uint64_t vg[4], vu[4];
                    for (;;) {
                        bool ok = true;
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            const size_t o = (size_t)min(s0 + q, ncontrib - 1) * 128;
                            vg[q] = ld_tagged(pp + o);
                            vu[q] = ld_tagged(pp + o + 64);
                            ok = ok && tag_ok(vg[q], tag) && tag_ok(vu[q], tag);
                        }
                        if (__all(ok)) break;
                        if (!poll_more(sync, spins)) { okj = false; break; }
                    }
#pragma unroll
                    for (int q = 0; q < 4; q++)
                        if (s0 + q < ncontrib) {
                            g += tag_val(vg[q]);
                            uu += tag_val(vu[q]);
                        }
                }
                g = ldexpf(g, xe) * sg;
                uu = ldexpf(uu, xe) * su;
                st_x(a.hh + (size_t)j * I + r, g / (1.f + __expf(-g)) * uu);
            }
            if (lane == 0 && !okj) *bcast = 0;
            wait_vm_all();
            __syncthreads();
            if (!*bcast) return;
            if (threadIdx.x == 0 && nj)
                __hip_atomic_fetch_add(h_ready + j * kLine, (unsigned)nj, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ea = eb;
        }

        mark(kStampGuDone);
        // ---- shared down rows, tagged: wave v takes the workgroup's rows
        // shH0 + v, shH0 + v + kPW, ..., kShDR at a time, lane l columns
        // 8 l + 512 m.  A wave issues its rows' weight loads, then waits for
        // the whole shared h (its own poll of the counter, unless the value
        // loaded after gate/up already showed it), then loads h (coherent
        // loads) and sums: no workgroup barrier, and the weights' round trip
        // overlaps the wait.
        count_shared();
        if (shared_on && shH1 > shH0) {
            const uint16_t *wd0 = lay.shared + 2 * (size_t)I * H;
            const unsigned h_target = (unsigned)(s + 1) * sh_gu_contrib;
            bool h_seen = false, oks = true;
            for (int rb = shH0 + wave; rb < shH1 && oks; rb += kPW * kShDR) {
                float acc[kShDR];
#pragma unroll
                for (int d = 0; d < kShDR; d++) acc[d] = 0.f;
                for (int c0 = 0; c0 < I && oks; c0 += 512 * kShCP) {
                    uint4 wv[kShDR][kShCP];
#pragma unroll
                    for (int d = 0; d < kShDR; d++)
#pragma unroll
                        for (int p = 0; p < kShCP; p++) {
                            const int r = rb + d * kPW, c = c0 + 512 * p + 8 * lane;
                            wv[d][p] = r < shH1 && c < I ? gldu4(wd0 + (size_t)r * I + c)
                                                         : make_uint4(0u, 0u, 0u, 0u);
                        }
                    if (!h_seen && sh_early < h_target) {
                        long spins = 0;
                        while (ld_cnt(h_ready + k * kLine) < h_target)
                            if (!poll_more(sync, spins)) { oks = false; break; }
                    }
                    h_seen = true;
                    if (!oks) break;
                    uint64_t hv[kShCP][4];
#pragma unroll
                    for (int p = 0; p < kShCP; p++) {
                        const int c = c0 + 512 * p + 8 * lane;
#pragma unroll
                        for (int q = 0; q < 4; q++)
                            hv[p][q] = c < I ? ld_x((const uint64_t *)(a.hs + c) + q) : 0u;
                    }
#pragma unroll
                    for (int p = 0; p < kShCP; p++) {
                        float hf[8];
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            hf[2 * q] = __uint_as_float((uint32_t)hv[p][q]);
                            hf[2 * q + 1] = __uint_as_float((uint32_t)(hv[p][q] >> 32));
                        }
#pragma unroll
                        for (int d = 0; d < kShDR; d++) {
                            const uint32_t dq[4] = {wv[d][p].x, wv[d][p].y, wv[d][p].z, wv[d][p].w};
#pragma unroll
                            for (int i = 0; i < 4; i++) {
                                acc[d] = fmaf(__uint_as_float(dq[i] << 16), hf[2 * i], acc[d]);
                                acc[d] = fmaf(__uint_as_float(dq[i] & 0xFFFF0000u), hf[2 * i + 1], acc[d]);
                            }
                        }
                    }
                }
#pragma unroll
                for (int d = 0; d < kShDR; d++) {
                    const float y = wave_sum(acc[d]);
                    const int r = rb + d * kPW;
                    if (oks && lane == 0 && r < shH1) st_tagged(a.ysh + r, y, tag);
                }
            }
            if (!oks && lane == 0) *bcast = 0;
            lds_sync();
            if (!*bcast) return;
        }

        mark(kStampSharedDown);
        if (a.lut & kLutDown) {
            // ---- down by table lookup over this workgroup's range of the
            // (rank, chunk of I, tile of H) space, one segment (fixed rank
            // and chunk) at a time; each tile's sum over the chunk goes out
            // as a row-pair partial (slot = chunk, 32 words).  A segment's table needs
            // only its chunk's 128 values of the rank's h, polled as tagged
            // words (no counter, no wait for the whole h).  Where every
            // segment has a workgroup of its own, each takes one whole
            // segment (one table build).
            // (32-bit index math: the host allows this path only where
            // nLd * G fits an int)
            // fj [k][16] (k 16 <= 512: one entry per thread): w_j s_j[row] of slice w, combined below
            float *fj = (float *)(lds + kLutX + 512);
            const int nSl = H / kSliceRows;
            auto scale_of = [&](int sl) -> _Float16 {
                const int j = threadIdx.x / kSliceRows;
                return gld((const _Float16 *)((const uint8_t *)recs[j] + a.off.scales[2]) + sl * kSliceRows +
                           threadIdx.x % kSliceRows);
            };
            const bool fj_entry = threadIdx.x < k * kSliceRows;
            bool fj_done = w >= nSl;
            const int nLd = k * cprI * tilesH;
            const int GaD = min(k * cprI, G);
            const int l1 = w + 1 >= GaD ? nLd : nLd * (w + 1) / GaD;
            for (int ua = w >= GaD ? nLd : nLd * w / GaD; ua < l1;) {
                const int seg = ua / tilesH;
                const int ub = min(l1, (seg + 1) * tilesH);
                const int c = seg % cprI, j = seg / cprI;
                const uint8_t *rec = (const uint8_t *)recs[j];
                const uint64_t *hsrc = a.hq + (size_t)j * I + kChunkCols * c;
                const bool ok = stream_lut(
                    (const u32x4 *)(rec + a.off.codes[2]), (const u32x4 *)(rec + a.off.cb[2]), cprI, c, kLutX,
                    ua - seg * tilesH, ub - ua, a.part_d + ((size_t)j * tilesH * cprI + c) * 32, 32 * cprI, tag16(s), wave,
                    lane, [&] {
                        // the first segment also loads slice w's row scales: issued here,
                        // after the A fragments and the code rings, stored after the poll
                        const bool fill = !fj_done && fj_entry;
                        _Float16 sv = (_Float16)0.f;
                        if (fill) sv = scale_of(w);
                        // the chunk's h, as fp32 where the build reads x
                        if (wave == 0) {
                            uint64_t v0, v1;
                            long spins = 0;
                            bool okh = true;
                            for (;;) {
                                v0 = ld_tagged(hsrc + 2 * lane);
                                v1 = ld_tagged(hsrc + 2 * lane + 1);
                                if (__all(tag_ok(v0, tag) && tag_ok(v1, tag))) break;
                                if (!poll_more(sync, spins)) { okh = false; break; }
                            }
                            *(float2 *)(lds + kLutX + 8 * lane) = make_float2(tag_val(v0), tag_val(v1));
                            if (lane == 0) bcast[1] = okh;   // its own word: others may still read bcast[0]
                        }
                        if (fill) fj[threadIdx.x] = sw[threadIdx.x / kSliceRows] * (float)sv;
                        fj_done = true;
                        lds_sync();
                        mark(kStampDownStaged);
                        return bcast[1] != 0;
                    });
                if (!ok) return;
                ua = ub;
            }
            lds_sync();
            mark(kStampDownLoop);
            // ---- output slices w, w + G, ... (whole workgroup each)
            for (int sl = w; sl < nSl; sl += G) {
                if (sl != w || !fj_done) {
                    if (sl != w) lds_sync();
                    if (fj_entry) fj[threadIdx.x] = sw[threadIdx.x / kSliceRows] * (float)scale_of(sl);
                    fj_done = true;
                }
                if (!combine_slice_lut<8, LC>(sl, s, tag, k, tilesH, cprI, H, shared_on, a.part_d, a.ysh, a.out, fj, sync,
                                          bcast, wave, lane))
                    return;
            }
            mark(kStampDownDone);
            continue;
        }
        // ---- down over this workgroup's range of (rank, tile of H, chunk),
        // one expert segment at a time: tagged partials per touched tile
        for (int ea = d0; ea < d1;) {
            const int j = ea / (tilesH * cprI);
            const int eb = min(d1, (j + 1) * tilesH * cprI);
            const uint8_t *rec = (const uint8_t *)recs[j];
            const int base = j * tilesH * cprI;
            const int tA = ea / cprI;
            const int nt = (eb - 1) / cprI - tA + 1;
            const _Float16 *dscale = (const _Float16 *)(rec + a.off.scales[2]);
            // the row scales of this wave's first tile, loaded before the
            // loop: the partial stores after it wait for no load
            const float sc0 = wave < nt ? (float)gld(dscale + (tA + wave) % tilesH * kTileRows + lane) : 0.f;
            int he = 0;
            if (!stream_down((const u32x4 *)(rec + a.off.codes[2]), (const u32x4 *)(rec + a.off.cb[2]),
                             a.hh + (size_t)j * I, sync, h_ready + j * kLine, (unsigned)(s + 1) * tilesI, bcast, lmax,
                             he, H, I, cprI, ea - base, eb - base, ea / cprI - base / cprI,
                             a.slots_red_d, wave, lane, stamp))
                return;
            lds_sync();
            mark(kStampDownLoop);
            for (int v = wave; v < nt; v += kPW) {
                const int tau = tA + v;
                float y = 0.f;
#pragma unroll
                for (int q = 0; q < kPW; q++) y += red_d[(v * kPW + q) * 64 + lane];
                const int r = tau % tilesH * kTileRows + lane;
                y = ldexpf(y, he) * (v == wave ? sc0 : (float)gld(dscale + r));
                st_tagged(a.part_d + ((size_t)tau * a.slots_d + (w - range_owner(nD, G, tau * cprI))) * 64 + lane, y,
                          tag);
            }
            lds_sync();
            ea = eb;
        }

        // ---- output tiles this workgroup combines (one wave each), each
        // counted on the layer-done counter by its wave
        {
            int nc = 0;
            bool okc = true;
            // candidates: the last rank's tiles that this workgroup's range touches
            const int lb0 = (k - 1) * tilesH * cprI;
            const int tdA = d1 > lb0 ? (max(d0, lb0) - lb0) / cprI : tilesH;
            const int tdB = d1 > lb0 ? (d1 - 1 - lb0) / cprI : -1;
            for (int td = tdA; td <= tdB; td++) {
                if (combiner_of(td, k, tilesH, cprI, nD, G) != w) continue;
                if (nc++ % kPW != wave || !okc) continue;
                okc = k <= 2 ? combine_tile<2>(td, s, tag, k, tilesH, cprI, nD, G, H, shared_on, a.part_d, a.slots_d,
                                               a.ysh, a.out, sw, sync, lane)
                             : combine_tile<8>(td, s, tag, k, tilesH, cprI, nD, G, H, shared_on, a.part_d, a.slots_d,
                                               a.ysh, a.out, sw, sync, lane);
                // counted at once: nothing in this launch reads the outputs, and
                // the partials it read are consumed (their values are used)
                if (okc && lane == 0)
                    __hip_atomic_fetch_add(sync + kLayerDone + (td % LC) * kLine, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            }
            if (lane == 0 && !okc) *bcast = 0;
            lds_sync();
            if (!*bcast) return;
        }
        mark(kStampDownDone);
    }
}

struct LayerPack {
    DecLayer layers[kDecMaxLayers];
    int n;
};

// copies the layer descriptors into device memory (indices are compile-time
// after unrolling, so the argument block is never indexed at run time)
__global__ void k_store_layers(LayerPack pack, DecLayer *dst) {
    if (threadIdx.x != 0) return;
#pragma unroll
    for (int l = 0; l < kDecMaxLayers; l++)
        if (l < pack.n) dst[l] = pack.layers[l];
}

// Zeroes the counters and tagged buffers before a launch, except the sticky
// status word, which keeps kDecodeStatusFailed and is set to
// kDecodeStatusClean if it holds neither value (a workspace's first use).
__global__ void k_decode_clear(unsigned *p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        if (i != (size_t)kStatus) {
            p[i] = 0;
        } else if (p[i] != (unsigned)kDecodeStatusFailed) {
            p[i] = (unsigned)kDecodeStatusClean;
        }
    }
}

size_t decode_lds() { return kDecLdsBytes; }

}  // namespace

// ---------------------------------------------------------------- host side
static long h_range_start(long n, int G, int w) {
    const int Ga = (int)std::min<long>(n, G);
    return w >= Ga ? n : n * w / Ga;
}
static int h_range_owner(long n, int G, long u) {
    const int Ga = (int)std::min<long>(n, G);
    return (int)(((u + 1) * Ga + n - 1) / n - 1);
}

static int max_contributors(long n_tiles, int cpr, int G) {
    const long n = n_tiles * cpr;
    int m = 1;
    for (long tau = 0; tau < n_tiles; tau++)
        m = std::max(m, h_range_owner(n, G, (tau + 1) * cpr - 1) - h_range_owner(n, G, tau * cpr) + 1);
    return m;
}

// most tiles (of cpr units each) that one workgroup's range of an n-unit space touches
static int max_tiles_per_range(long n_tiles, int cpr, int G) {
    const long n = n_tiles * cpr;
    int m = 1;
    for (int w = 0; w < G; w++) {
        const long a = h_range_start(n, G, w), b = h_range_start(n, G, w + 1);
        if (b > a) m = std::max(m, (int)((b - 1) / cpr - a / cpr + 1));
    }
    return m;
}

hipError_t decode_plan(int H, int I, int k, int lut_mode, DecodePlanOut *o) {
    // per device: the persistent grid and whether dynamic LDS starts at byte 0
    // (no static LDS)
    constexpr int kMaxDev = 64;
    static int Gdev[kMaxDev] = {};
    static bool lds_zero_dev[kMaxDev] = {};
    int dev = 0;
    hipError_t ed = hipGetDevice(&dev);
    if (ed != hipSuccess) return ed;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    int &G = Gdev[dev];
    bool &lds_at_zero = lds_zero_dev[dev];
    if (G == 0) {
        const void *fns[2] = {(const void *)k_decode_persistent<8>, (const void *)k_decode_persistent<16>};
        int cus = 0, per_min = 1 << 30;
        hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        lds_at_zero = true;
        for (const void *fn : fns) {
            hipFuncAttributes fa;
            if (e == hipSuccess) e = hipFuncGetAttributes(&fa, fn);
            if (e == hipSuccess) lds_at_zero = lds_at_zero && fa.sharedSizeBytes == 0;
            if (e == hipSuccess)
                e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)decode_lds());
            int per = 0;
            if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, kPW * 64, decode_lds());
            per_min = std::min(per_min, per);
        }
        if (e != hipSuccess) return e;
        if (per_min < 1) return hipErrorInvalidConfiguration;
        G = cus * per_min;
    }
    const int tilesI = I / kTileRows, tilesH = H / kTileRows, cprH = H / kChunkCols, cprI = I / kChunkCols;
    o->G = G;
    o->slots_gu = max_contributors((long)k * tilesI, cprH, G);
    o->slots_d = max_contributors((long)k * tilesH, cprI, G);
    o->slots_red_gu = max_tiles_per_range((long)k * tilesI, cprH, G);
    o->slots_red_d = max_tiles_per_range((long)k * tilesH, cprI, G);
    // Table lookup: a table costs about as much as streaming 4096 rows' groups
    // by gathers, so it pays when every table serves many more rows than that
    // (by default where I >= 8192: a gate/up table serves I rows; a down
    // table serves H rows, and by then the join that precedes down is
    // already per chunk); gate/up's x (fp32) must fit in LDS beside the table.
    const bool want = lut_mode > 0 || (lut_mode < 0 && I >= 2 * kCbRows);
    const bool gu_fits = lds_at_zero && H <= kLutMaxH && (long)k * 2 * cprH * tilesI * G < (1L << 31);
    // down by table lookup takes its h, per chunk, from gate/up's table-lookup joins
    const bool d_fits = gu_fits && (long)k * cprI * tilesH * G < (1L << 31);
    o->lut = (want && gu_fits ? kLutGateUp : 0) | (want && lut_mode != 2 && d_fits ? kLutDown : 0);
    if (o->lut & kLutGateUp) o->slots_gu = cprH;
    if (o->lut & kLutDown) o->slots_d = cprI;
    o->sync_words = kHReady + (size_t)(k + 1) * kLine;
    // LDS: the gathers' layouts of the phases done by gathers must fit below
    // the routing tail (a table-lookup phase uses the table area instead)
    const long red_gu = 2L * kCbRows * 16 + ((H * 2 + 255) & ~255) + (long)o->slots_red_gu * kPW * 128 * 4;
    const long red_d = (long)kCbRows * 16 + ((I * 2 + 255) & ~255) + (long)o->slots_red_d * kPW * 64 * 4;
    const bool gu_ok = (o->lut & kLutGateUp) || (red_gu <= kDecTail && kXStage + (long)H * 4 <= 2L * kCbRows * 16);
    const bool d_ok = (o->lut & kLutDown) || red_d <= kDecTail;
    o->lds_ok = gu_ok && d_ok;
    // the kernel's work-range arithmetic is 32-bit: n * (G + 1) < 2^31 for
    // every unit space it splits
    const long lim = (1L << 31) / (G + 1);
    o->units_ok = (long)k * tilesI * cprH < lim && (long)k * tilesH * cprI < lim && I < lim && H < lim;
    return hipSuccess;
}

hipError_t launch_decode_persistent(const DecodeLaunch &d, hipStream_t s) {
    const int tilesI = d.I / kTileRows, tilesH = d.H / kTileRows;
    const unsigned fill_blocks = (unsigned)std::min<size_t>(1024, (d.clear_words + 255) / 256);
    k_decode_clear<<<fill_blocks, 256, 0, s>>>(d.sync, d.clear_words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    DecArgs a{};
    LayerPack pack;
    for (int l = 0; l < kDecMaxLayers; l++) pack.layers[l] = l < d.nL ? d.layers[l] : DecLayer{};
    pack.n = d.nL;
    k_store_layers<<<1, 64, 0, s>>>(pack, d.layer_buf);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.layers = d.layer_buf;
    a.nL = d.nL;
    a.T = d.T;
    a.H = d.H;
    a.I = d.I;
    a.k = d.k;
    a.E_max = d.E_max;
    a.G = d.G;
    a.has_shared = d.has_shared;
    a.x = d.x;
    a.out = d.out;
    a.idx_out = d.idx_out;
    a.off = d.off;
    a.sync = d.sync;
    a.z = d.z;
    a.hh = d.hh;
    a.hq = d.hq;
    a.hs = d.hs;
    a.ysh = d.ysh;
    a.part_gu = d.part_gu;
    a.part_d = d.part_d;
    a.slots_gu = d.slots_gu;
    a.slots_d = d.slots_d;
    a.slots_red_gu = d.slots_red_gu;
    a.slots_red_d = d.slots_red_d;
    a.lut = d.lut;
    a.stamps = d.stamps;
    a.stamp_steps = d.stamp_steps;
    (void)tilesI;
    void *args[] = {&a};
    const int out_units = (d.lut & kLutDown) ? d.H / kSliceRows : tilesH;   // output units per step
    const void *fn = out_units >= 128 ? (const void *)k_decode_persistent<16> : (const void *)k_decode_persistent<8>;
    return hipLaunchCooperativeKernel(fn, dim3(d.G), dim3(kPW * 64), args, (unsigned)decode_lds(), s);
}

}  // namespace moe
