// HIP kernels for gfx950 (CDNA4): router logits, wavefront top-k, RVQ
// gate/up and down GEMVs on packed 24-bit code pairs, dense bf16 shared
// expert, fixed-order combine.
//
// Sources (pages on routed expert streaming):
//  "WISP -- 실행될 수 없는 것을 스트리밍하다", section "통찰": the model's own
//    router picks each token's experts (route + top-k below);
//  "2.78조 파라미터 모델을 노트북에서: NVMe 스트리밍 추론 엔진 WASTE", section
//    "유휴 가중치는 메모리가 아니라 제때 닿기만 하면 된다": experts are residual
//    vector quantised at 3.00 bits per weight and never expanded (the GEMVs
//    below decode codes on the fly; no weight matrix is ever written out).
//
// Numerics: logits, accumulation and the combine are fp32.  The RVQ GEMVs
// multiply the exact fp16 codebook entries by the input rounded to fp16
// (v_dot2_f32_f16: exact products, fp32 accumulation); the SwiGLU
// intermediate is kept in fp32 and rounded to fp16 when the down GEMV stages
// it.  Each rounding to fp16 follows a power-of-two range scaling of its
// block (range_exp), undone exactly after the fp32 sums.
#include <hip/hip_runtime.h>

#include "moe_internal.h"
#include "rvq_device.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- routing
// z[t, e] = W[e] . x[t] + b[e].  One workgroup per expert row and 8 tokens:
// its four waves take interleaved 256-column pieces of the row, four per step
// (loads in flight together), and their sums are added in wave order.
constexpr int kRouteTok = 8;

__global__ __launch_bounds__(256) void k_route_logits(const float *__restrict__ W, const float *__restrict__ bias,
                                                      int E, int H, const void *__restrict__ x, int x_dtype, int T,
                                                      float *__restrict__ z) {
    __shared__ float red[4][kRouteTok];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = blockIdx.x;
    const int t0 = blockIdx.y * kRouteTok;
    const int nt = min(kRouteTok, T - t0);
    float acc[kRouteTok];
#pragma unroll
    for (int i = 0; i < kRouteTok; i++) acc[i] = 0.f;
    const float *wr = W + (size_t)e * H;
    // wave v takes the 256-column pieces v, v + 4, ... of the row, four per
    // step (their loads in flight together)
    constexpr int kPieces = 4;
    const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c0 = wave * 256 + lane * 4; c0 < H; c0 += kPieces * 1024) {
        float4 wv[kPieces];
#pragma unroll
        for (int u = 0; u < kPieces; u++) {
            const int c = c0 + u * 1024;
            wv[u] = c < H ? *(const float4 *)(wr + c) : zero4;
        }
#pragma unroll
        for (int i = 0; i < kRouteTok; i++) {
            if (i < nt) {
                float4 xv[kPieces];
#pragma unroll
                for (int u = 0; u < kPieces; u++) {
                    const int c = c0 + u * 1024;
                    if (c >= H) {
                        xv[u] = zero4;
                    } else if (x_dtype == MOE_DTYPE_F32) {
                        xv[u] = *(const float4 *)((const float *)x + (size_t)(t0 + i) * H + c);
                    } else {
                        const uint2 b = *(const uint2 *)((const uint16_t *)x + (size_t)(t0 + i) * H + c);
                        xv[u] = make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u),
                                            __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xFFFF0000u));
                    }
                }
#pragma unroll
                for (int u = 0; u < kPieces; u++) {
                    acc[i] = fmaf(wv[u].x, xv[u].x, acc[i]);
                    acc[i] = fmaf(wv[u].y, xv[u].y, acc[i]);
                    acc[i] = fmaf(wv[u].z, xv[u].z, acc[i]);
                    acc[i] = fmaf(wv[u].w, xv[u].w, acc[i]);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kRouteTok; i++) {
        const float s = wave_sum(acc[i]);
        if (lane == 0) red[wave][i] = s;
    }
    __syncthreads();
    if (threadIdx.x < nt) {
        const int i = threadIdx.x;
        z[(size_t)(t0 + i) * E + e] = ((red[0][i] + red[1][i]) + (red[2][i] + red[3][i])) + (bias ? bias[e] : 0.f);
    }
}

// Router logits for many tokens (batched calls): a workgroup takes 64 tokens
// x 64 experts x one slice of H, staged through LDS in 64-column steps; each
// thread accumulates 4 tokens x 4 experts (tokens ty + 16i, experts tx + 16j,
// so the 16 expert rows a wave reads sit in 16 different bank groups of the
// 68-float padded rows).  Slices write fp32 partial sums; k_route_reduce adds
// them in slice order plus the bias, so the result does not depend on timing.
constexpr int kRbT = 64, kRbE = 64, kRbK = 64, kRbRow = 68;

__global__ __launch_bounds__(256) void k_route_blocked(const float *__restrict__ W, int E, int H,
                                                       const void *__restrict__ x, int x_dtype, int T, int kslice,
                                                       float *__restrict__ part) {
    __shared__ __align__(16) float xs[kRbT * kRbRow];
    __shared__ __align__(16) float ws[kRbE * kRbRow];
    const int t0 = blockIdx.x * kRbT, e0 = blockIdx.y * kRbE, ks = blockIdx.z;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int c_begin = ks * kslice, c_end = min(H, c_begin + kslice);
    float acc[4][4] = {};
    // loader: 64 rows x 64 columns = 1024 float4; four per thread
    for (int c0 = c_begin; c0 < c_end; c0 += kRbK) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int q = tid + 256 * r, row = q >> 4, c4 = (q & 15) * 4;
            const int t = min(t0 + row, T - 1), e = min(e0 + row, E - 1);
            float4 xv;
            if (x_dtype == MOE_DTYPE_F32) {
                xv = *(const float4 *)((const float *)x + (size_t)t * H + c0 + c4);
            } else {
                const uint2 b = *(const uint2 *)((const uint16_t *)x + (size_t)t * H + c0 + c4);
                xv = make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u),
                                 __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xFFFF0000u));
            }
            *(float4 *)(xs + row * kRbRow + c4) = xv;
            *(float4 *)(ws + row * kRbRow + c4) = *(const float4 *)(W + (size_t)e * H + c0 + c4);
        }
        __syncthreads();
#pragma unroll 4
        for (int c = 0; c < kRbK; c += 4) {
            float4 xv[4], wv[4];
#pragma unroll
            for (int i = 0; i < 4; i++) xv[i] = *(const float4 *)(xs + (ty + 16 * i) * kRbRow + c);
#pragma unroll
            for (int j = 0; j < 4; j++) wv[j] = *(const float4 *)(ws + (tx + 16 * j) * kRbRow + c);
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    float a = acc[i][j];
                    a = fmaf(xv[i].x, wv[j].x, a);
                    a = fmaf(xv[i].y, wv[j].y, a);
                    a = fmaf(xv[i].z, wv[j].z, a);
                    a = fmaf(xv[i].w, wv[j].w, a);
                    acc[i][j] = a;
                }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int t = t0 + ty + 16 * i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int e = e0 + tx + 16 * j;
            if (e < E) part[((size_t)ks * T + t) * E + e] = acc[i][j];
        }
    }
}

__global__ __launch_bounds__(256) void k_route_reduce(const float *__restrict__ part, const float *__restrict__ bias,
                                                      int E, int T, int KS, float *__restrict__ z) {
    const size_t n = (size_t)T * E;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        float s = 0.f;
        // eight slices' loads in flight at a time, added in slice order
        int ks = 0;
        for (; ks + 8 <= KS; ks += 8) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; q++) v[q] = part[(ks + q) * n + i];
#pragma unroll
            for (int q = 0; q < 8; q++) s += v[q];
        }
        for (; ks < KS; ks++) s += part[ks * n + i];
        z[i] = s + (bias ? bias[n <= 0xFFFFFFFFu ? (unsigned)i % (unsigned)E : i % E] : 0.f);
    }
}

// Top-k per token, one 256-thread workgroup per token, by counting: the
// rank of an expert is the number of experts ahead of it in (z desc, id asc)
// order.  Each logit becomes a 64-bit key (order-preserving logit bits above
// the inverted id; NaN ranks last, -0 and +0 tie), so a rank is a count of
// larger keys and all ranks differ.  For E > 64 in two levels: ranks within
// eighths of the experts first (whole 32-key blocks); the keys of local rank
// below k (every global top-k key is one) are then ranked among themselves.
// Weights: softmax over the selected logits, or sigmoid scores renormalised,
// summed in rank order.  With idx_host / w_host (page-locked host memory) the
// kernel also writes the ids and weights there, visible to the host once the
// kernel has completed (no separate device-to-host copy).
constexpr int kTopkThreads = 256, kTopkLvl = 8;
__device__ __forceinline__ uint32_t topk_order_key(float f) {
    f = f == f ? f : -INFINITY;
    uint32_t u = __float_as_uint(f);
    u = u == 0x80000000u ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float topk_key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__global__ __launch_bounds__(kTopkThreads) void k_topk(const float *__restrict__ z, int E, int k, int score_fn,
                                                       int32_t *__restrict__ idx, float *__restrict__ w,
                                                       int32_t *__restrict__ idx_host, float *__restrict__ w_host,
                                                       uint32_t *flag_host, uint32_t seq) {
    __shared__ __align__(16) uint64_t key[MOE_MAX_E];              // padded to a multiple of 32 with zeros
    __shared__ __align__(16) uint64_t cand[kTopkLvl * MOE_MAX_K];  // zeros past the candidates
    __shared__ int sidx[MOE_MAX_K];
    __shared__ float sz[MOE_MAX_K];
    const int t = blockIdx.x;
    const int Ep = (E + 31) & ~31;
    for (int e = threadIdx.x; e < Ep; e += kTopkThreads)
        key[e] = e < E ? (uint64_t)topk_order_key(z[(size_t)t * E + e]) << 32 | (0xFFFFFFFFu - (uint32_t)e) : 0u;
    for (int i = threadIdx.x; i < kTopkLvl * MOE_MAX_K; i += kTopkThreads) cand[i] = 0u;
    __syncthreads();
    const bool two = E > 64;
    const int gsz = two ? ((E + kTopkLvl - 1) / kTopkLvl + 31) & ~31 : Ep;
    // rank of ke among list[q0, q1), 32 keys per step; stops once it reaches k
    auto count_above = [&](const uint64_t *list, int q0, int q1, uint64_t ke) {
        int r[4] = {0, 0, 0, 0};
        for (; q0 < q1 && r[0] + r[1] + r[2] + r[3] < k; q0 += 32) {
            uint64_t kv[32];
#pragma unroll
            for (int i = 0; i < 32; i++) kv[i] = list[q0 + i];
#pragma unroll
            for (int i = 0; i < 32; i++) r[i & 3] += kv[i] > ke;
        }
        return r[0] + r[1] + r[2] + r[3];
    };
    auto place = [&](int rank, uint64_t ke) {
        sidx[rank] = (int)(0xFFFFFFFFu - (uint32_t)ke);
        sz[rank] = topk_key_value((uint32_t)(ke >> 32));
    };
    for (int e = threadIdx.x; e < E; e += kTopkThreads) {
        const uint64_t ke = key[e];
        const int g0 = e / gsz * gsz;
        const int rank = count_above(key, g0, min(Ep, g0 + gsz), ke);
        if (rank < k) {
            if (two) cand[e / gsz * k + rank] = ke;   // a slot of its own: (group, local rank)
            else place(rank, ke);
        }
    }
    if (two) {
        __syncthreads();
        // the groups' candidates, zeros where a group had fewer than k keys
        // (the candidate area is zeroed to its end, kTopkLvl * MOE_MAX_K >=
        // ncp).  Each candidate is ranked by P threads, each counting a P-th
        // of the list; the P counts are added across their lanes.
        const int nc = (E + gsz - 1) / gsz * k;
        int ncp = 32;
        while (ncp < nc) ncp <<= 1;
        const int P = max(1, kTopkThreads / ncp), len = ncp / P;
        const int c = threadIdx.x / P, q0 = (threadIdx.x % P) * len;
        const uint64_t ke = c < nc ? cand[c] : 0u;
        int r4[4] = {0, 0, 0, 0};
#pragma unroll 4
        for (int q = q0; q < q0 + len; q += 4) {   // len is a multiple of 4: four loads in flight
            const uint64_t k0 = cand[q], k1 = cand[q + 1], k2 = cand[q + 2], k3 = cand[q + 3];
            r4[0] += k0 > ke;
            r4[1] += k1 > ke;
            r4[2] += k2 > ke;
            r4[3] += k3 > ke;
        }
        int rank = (r4[0] + r4[1]) + (r4[2] + r4[3]);
        for (int o = 1; o < P; o <<= 1) rank += __shfl_xor(rank, o, 64);
        if (threadIdx.x % P == 0 && ke && rank < k) place(rank, ke);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        // lane r < k scores rank r; the sum runs in rank order
        const int lane = threadIdx.x;
        const float zmax = sz[0];
        float sc = 0.f;
        if (lane < k) sc = score_fn == MOE_SCORE_SOFTMAX ? __expf(sz[lane] - zmax) : 1.f / (1.f + __expf(-sz[lane]));
        float sum = 0.f;
        for (int r = 0; r < k; r++) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), r));
        if (lane < k) {
            idx[(size_t)t * k + lane] = sidx[lane];
            w[(size_t)t * k + lane] = sc / sum;
            if (idx_host) idx_host[(size_t)t * k + lane] = sidx[lane];
            if (w_host) w_host[(size_t)t * k + lane] = sc / sum;
        }
    }
    // then seq to flag_host: the host can read the ids as soon as it sees it,
    // before the kernel's completion is signalled.  Every id and weight was
    // written by wave 0 (k <= 32), whose stores the system-scope fence orders
    // before the flag's.
    if (flag_host && t == 0 && threadIdx.x == 0) {
        __threadfence_system();
        __hip_atomic_store(flag_host, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// x -> fp16 pairs (one dword per two consecutive elements), one workgroup
// per token: the token's values are scaled by 2^-xexp[t] (xexp from the
// largest |x_t|, range_exp) so that no pair overflows fp16; the gate/up sums
// are scaled back by 2^xexp[t].
__global__ __launch_bounds__(256) void k_pack_x(const void *__restrict__ x, int x_dtype, int H, int64_t x_stride,
                                                uint32_t *__restrict__ xh, int32_t *__restrict__ xexp) {
    __shared__ float wm[4];
    const int t = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    auto val = [&](int c) -> float {
        if (x_dtype == MOE_DTYPE_F32) return ((const float *)x + (size_t)t * x_stride)[c];
        return bf16_to_f32(((const uint16_t *)x + (size_t)t * x_stride)[c]);
    };
    float m = 0.f;
    for (int c = threadIdx.x; c < H; c += 256) m = fmaxf(m, fabsf(val(c)));
    m = wave_max(m);
    if (lane == 0) wm[wave] = m;
    __syncthreads();
    const int e = range_exp(fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3])));
    const int hp = H / 2;
    for (int p = threadIdx.x; p < hp; p += 256)
        xh[(size_t)t * hp + p] = pack_f16x2(ldexpf(val(2 * p), -e), ldexpf(val(2 * p + 1), -e));
    if (threadIdx.x == 0) xexp[t] = e;
}

// ------------------------------------------------------------- RVQ GEMVs
// Copies a codebook (kCbRows rows of 16 bytes) from global memory into LDS
// with NT threads, every load of a thread issued before its first LDS store.
// (Loads through a generic pointer cannot be moved past an LDS store, so a
// plain copy loop runs one memory round trip per row a thread copies.)
template <int NT>
__device__ __forceinline__ void stage_codebook(char *dst, const uint8_t *src) {
    gu32x4 *g = (gu32x4 *)src;
    constexpr int kPer = kCbRows / NT;
    static_assert(kPer * NT == kCbRows && kPer <= 16, "codebook staging layout");
    u32x4 v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; i++) v[i] = g[threadIdx.x + i * NT];
#pragma unroll
    for (int i = 0; i < kPer; i++) ((u32x4 *)dst)[threadIdx.x + i * NT] = v[i];
}

// Gate/up: one workgroup per (item, 64-row tile, matrix): gate and up are
// separate workgroups, each with its matrix's codebook staged in LDS (64 KiB,
// so two workgroups share a CU); lane = row, waves split the 128-column
// chunks; the input's fp16 pairs are wave-uniform (scalar loads).  Output:
// the scaled fp32 gate and up, gu[item][0][r] and gu[item][1][r]; the down
// kernel forms SiLU(g) * u from them.
constexpr int kGuWaves = 8;

__global__ __launch_bounds__(kGuWaves * 64) void k_rvq_gateup(RecSrc src, RecOffsets off, int H, int I,
                                                              const uint32_t *__restrict__ xh,
                                                              const int32_t *__restrict__ xexp,
                                                              float *__restrict__ gu) {
    extern __shared__ __align__(16) char lds[];
    char *cb = lds;
    float *red = (float *)(lds + kCbRows * 16);      // [kGuWaves][64]
    const int tiles = I / kTileRows;
    const int mat = blockIdx.x & 1, tile = (blockIdx.x >> 1) % tiles, local = (blockIdx.x >> 1) / tiles;
    int item;
    const uint8_t *rec = resolve_record(src, local, item);
    const int t = item / src.k;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int cpr = H / kChunkCols;
    const u32x4 *codes = (const u32x4 *)(rec + off.codes[mat]) + (size_t)tile * cpr * kTileVec;
    // a wave's first two strips are in flight during the codebook staging,
    // and each strip's dots run with the next two strips' loads in flight
    int c = wave;
    uint32_t dg[12], ng[12];
    if (c < cpr) load_strip(codes + (size_t)c * kTileVec, lane, dg);
    if (c + kGuWaves < cpr) load_strip(codes + (size_t)(c + kGuWaves) * kTileVec, lane, ng);
    stage_codebook<kGuWaves * 64>(cb, rec + off.cb[mat]);
    __syncthreads();
    const uint32_t *x = xh + (size_t)t * (H / 2);
    float ag[4] = {0.f, 0.f, 0.f, 0.f};
    while (c < cpr) {
        const int cn = c + 2 * kGuWaves;
        uint32_t nn[12];
        if (cn < cpr) load_strip(codes + (size_t)cn * kTileVec, lane, nn);
        strip_dot<0>(dg, cb, x + c * 64, ag);
#pragma unroll
        for (int i = 0; i < 12; i++) {
            dg[i] = ng[i];
            ng[i] = nn[i];
        }
        c += kGuWaves;
    }
    red[wave * 64 + lane] = (ag[0] + ag[1]) + (ag[2] + ag[3]);
    __syncthreads();
    if (wave == 0) {
        float g = 0.f;
#pragma unroll
        for (int wv = 0; wv < kGuWaves; wv++) g += red[wv * 64 + lane];
        const int r = tile * kTileRows + lane;
        const _Float16 sg = ((const _Float16 *)(rec + off.scales[mat]))[r];
        gu[((size_t)item * 2 + mat) * I + r] = ldexpf(g, xexp[t]) * (float)sg;
    }
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.f + __expf(-g)) * u; }

// Down: one workgroup per (item, 64-row tile of H, K-slice); down codebook in
// LDS (64 KiB), then the slice's h = SiLU(g) * u (fp32, from the gate/up
// outputs) as fp16 pairs scaled by 2^-e (e from the slice's largest |h|,
// range_exp); writes s_d[r] * 2^e * partial dot into ypart[item][ks][r].
constexpr int kDnWaves = 4;

__global__ __launch_bounds__(kDnWaves * 64) void k_rvq_down(RecSrc src, RecOffsets off, int H, int I, int KS,
                                                            const float *__restrict__ gu,
                                                            float *__restrict__ ypart) {
    extern __shared__ __align__(16) char lds[];
    char *cbd = lds;
    float *red = (float *)(lds + kCbRows * 16);           // [kDnWaves][64]
    float *wm = red + kDnWaves * 64;                      // [kDnWaves]
    uint32_t *xl = (uint32_t *)(wm + kDnWaves);           // the slice's h pairs
    const int tiles = H / kTileRows;
    const int ks = blockIdx.x % KS;
    const int tile = (blockIdx.x / KS) % tiles;
    const int local = blockIdx.x / (KS * tiles);
    int item;
    const uint8_t *rec = resolve_record(src, local, item);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int cpr = I / kChunkCols;
    const int c0 = cpr * ks / KS, c1 = cpr * (ks + 1) / KS;   // 32-bit: cpr * KS is small
    const float *hg = gu + (size_t)item * 2 * I + c0 * kChunkCols, *hu = hg + I;
    const int np = (c1 - c0) * kChunkCols / 2;
    const u32x4 *codes = (const u32x4 *)(rec + off.codes[2]) + (size_t)tile * cpr * kTileVec;
    // a wave's first two strips are in flight during the staging, and each
    // strip's dots run with the next two strips' loads in flight
    int c = c0 + wave;
    uint32_t d[12], nd[12];
    if (c < c1) load_strip(codes + (size_t)c * kTileVec, lane, d);
    if (c + kDnWaves < c1) load_strip(codes + (size_t)(c + kDnWaves) * kTileVec, lane, nd);
    // the slice's gate and up values: up to kHReg pairs per thread stay in
    // registers (loaded with the codebook, all in flight together); a longer
    // slice reloads the rest for the packing
    typedef float f2v __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(1))) const f2v gf2;
    gf2 *hg2 = (gf2 *)hg, *hu2 = (gf2 *)hu;
    constexpr int kHReg = 4, kNT = kDnWaves * 64;
    f2v gr[kHReg], ur[kHReg];
#pragma unroll
    for (int i = 0; i < kHReg; i++) {
        const int p = threadIdx.x + i * kNT;
        const f2v z = {0.f, 0.f};
        gr[i] = p < np ? hg2[p] : z;
        ur[i] = p < np ? hu2[p] : z;
    }
    stage_codebook<kNT>(cbd, rec + off.cb[2]);
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < kHReg; i++)
        if (threadIdx.x + i * kNT < np)
            m = fmaxf(m, fmaxf(fabsf(silu_mul(gr[i].x, ur[i].x)), fabsf(silu_mul(gr[i].y, ur[i].y))));
    for (int p = threadIdx.x + kHReg * kNT; p < np; p += kNT) {
        const f2v g = hg2[p], u = hu2[p];
        m = fmaxf(m, fmaxf(fabsf(silu_mul(g.x, u.x)), fabsf(silu_mul(g.y, u.y))));
    }
    m = wave_max(m);
    if (lane == 0) wm[wave] = m;
    __syncthreads();
    const int e = range_exp(fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3])));
#pragma unroll
    for (int i = 0; i < kHReg; i++) {
        const int p = threadIdx.x + i * kNT;
        if (p < np) xl[p] = pack_f16x2(ldexpf(silu_mul(gr[i].x, ur[i].x), -e), ldexpf(silu_mul(gr[i].y, ur[i].y), -e));
    }
    for (int p = threadIdx.x + kHReg * kNT; p < np; p += kNT) {
        const f2v g = hg2[p], u = hu2[p];
        xl[p] = pack_f16x2(ldexpf(silu_mul(g.x, u.x), -e), ldexpf(silu_mul(g.y, u.y), -e));
    }
    __syncthreads();
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    while (c < c1) {
        const int cn = c + 2 * kDnWaves;
        uint32_t nn[12];
        if (cn < c1) load_strip(codes + (size_t)cn * kTileVec, lane, nn);
        strip_dot<0>(d, cbd, xl + (c - c0) * 64, acc);
#pragma unroll
        for (int i = 0; i < 12; i++) {
            d[i] = nd[i];
            nd[i] = nn[i];
        }
        c += kDnWaves;
    }
    red[wave * 64 + lane] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    __syncthreads();
    if (wave == 0) {
        float y = 0.f;
#pragma unroll
        for (int wv = 0; wv < kDnWaves; wv++) y += red[wv * 64 + lane];
        const int r = tile * kTileRows + lane;
        const _Float16 sd = ((const _Float16 *)(rec + off.scales[2]))[r];
        ypart[((size_t)item * KS + ks) * H + r] = ldexpf(y, e) * (float)sd;
    }
}

// out[t, c] = (acc ? out : 0) + sum_j w[t, j] * sum_ks ypart[t*k+j][ks][c] + ysh[t, c]
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ ypart, int k, int KS, int H,
                                                 const float *__restrict__ w, const float *__restrict__ ysh,
                                                 float *__restrict__ out, int64_t out_stride, int T,
                                                 int accumulate) {
    const size_t n = (size_t)T * H;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        // 32-bit index division where the index fits (a 64-bit one is a long
        // instruction sequence); the branch is uniform
        size_t t, c;
        if (n <= 0xFFFFFFFFu) {
            const unsigned u = (unsigned)i;
            t = u / (unsigned)H;
            c = u - (unsigned)t * (unsigned)H;
        } else {
            t = i / H;
            c = i % H;
        }
        float acc = 0.f;
        for (int j = 0; j < k; j++) {
            const size_t item = t * k + j;
            float y = 0.f;
            for (int s = 0; s < KS; s++) y += ypart[(item * KS + s) * H + c];
            acc = fmaf(w ? w[item] : 1.f, y, acc);
        }
        if (ysh) acc += ysh[t * H + c];
        float *o = out + t * out_stride + c;
        *o = accumulate ? *o + acc : acc;
    }
}

// ------------------------------------------------------ dense shared expert
// hs[t, r] = SiLU(Wg[r] . x_t) * (Wu[r] . x_t); one wave per row, all tokens.
constexpr int kDenseTok = 4;

__global__ __launch_bounds__(256) void k_dense_gateup(const uint16_t *__restrict__ Wsh, int H, int I,
                                                      const void *__restrict__ x, int x_dtype, int64_t x_stride,
                                                      int T, float *__restrict__ hs) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + wave;
    if (r >= I) return;
    const uint16_t *wg = Wsh + (size_t)r * H;
    const uint16_t *wu = Wsh + (size_t)I * H + (size_t)r * H;
    for (int t0 = 0; t0 < T; t0 += kDenseTok) {
        float ag[kDenseTok] = {}, au[kDenseTok] = {};
        const int nt = min(kDenseTok, T - t0);
        for (int c = lane * 8; c < H; c += 512) {
            const uint4 gv = *(const uint4 *)(wg + c);
            const uint4 uv = *(const uint4 *)(wu + c);
            float gw[8], uw[8];
            const uint32_t gq[4] = {gv.x, gv.y, gv.z, gv.w}, uq[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                gw[2 * i] = __uint_as_float(gq[i] << 16); gw[2 * i + 1] = __uint_as_float(gq[i] & 0xFFFF0000u);
                uw[2 * i] = __uint_as_float(uq[i] << 16); uw[2 * i + 1] = __uint_as_float(uq[i] & 0xFFFF0000u);
            }
#pragma unroll
            for (int tt = 0; tt < kDenseTok; tt++) {
                if (tt < nt) {
                    float xv[8];
                    if (x_dtype == MOE_DTYPE_F32) {
                        const float *xr = (const float *)x + (size_t)(t0 + tt) * x_stride + c;
                        const float4 a = *(const float4 *)xr, b = *(const float4 *)(xr + 4);
                        xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
                        xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
                    } else {
                        const uint4 b = *(const uint4 *)((const uint16_t *)x + (size_t)(t0 + tt) * x_stride + c);
                        const uint32_t q[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            xv[2 * i] = __uint_as_float(q[i] << 16);
                            xv[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        ag[tt] = fmaf(gw[i], xv[i], ag[tt]);
                        au[tt] = fmaf(uw[i], xv[i], au[tt]);
                    }
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < kDenseTok; tt++) {
            const float g = wave_sum(ag[tt]), u = wave_sum(au[tt]);
            if (lane == 0 && tt < nt) hs[(size_t)(t0 + tt) * I + r] = g / (1.f + __expf(-g)) * u;
        }
    }
}

// ysh[t, c] = Wd[c] . hs_t; one wave per row.
__global__ __launch_bounds__(256) void k_dense_down(const uint16_t *__restrict__ Wsh, int H, int I,
                                                    const float *__restrict__ hs, int T, float *__restrict__ ysh) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + wave;
    if (r >= H) return;
    const uint16_t *wd = Wsh + 2 * (size_t)I * H + (size_t)r * I;
    for (int t0 = 0; t0 < T; t0 += kDenseTok) {
        float acc[kDenseTok] = {};
        const int nt = min(kDenseTok, T - t0);
        for (int c = lane * 8; c < I; c += 512) {
            const uint4 dv = *(const uint4 *)(wd + c);
            const uint32_t q[4] = {dv.x, dv.y, dv.z, dv.w};
            float wv[8];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                wv[2 * i] = __uint_as_float(q[i] << 16);
                wv[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
            }
#pragma unroll
            for (int tt = 0; tt < kDenseTok; tt++) {
                if (tt < nt) {
                    const float *h = hs + (size_t)(t0 + tt) * I + c;
                    const float4 a = *(const float4 *)h, b = *(const float4 *)(h + 4);
                    acc[tt] = fmaf(wv[0], a.x, acc[tt]); acc[tt] = fmaf(wv[1], a.y, acc[tt]);
                    acc[tt] = fmaf(wv[2], a.z, acc[tt]); acc[tt] = fmaf(wv[3], a.w, acc[tt]);
                    acc[tt] = fmaf(wv[4], b.x, acc[tt]); acc[tt] = fmaf(wv[5], b.y, acc[tt]);
                    acc[tt] = fmaf(wv[6], b.z, acc[tt]); acc[tt] = fmaf(wv[7], b.w, acc[tt]);
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < kDenseTok; tt++) {
            const float s = wave_sum(acc[tt]);
            if (lane == 0 && tt < nt) ysh[(size_t)(t0 + tt) * H + r] = s;
        }
    }
}

size_t gateup_lds() { return kCbRows * 16 + kGuWaves * 64 * sizeof(float); }
// codebook, wave sums, wave maxima, and the largest K-slice's h pairs
size_t down_lds(int I, int KS) {
    const int cpr = I / kChunkCols;
    return kCbRows * 16 + (kDnWaves * 64 + kDnWaves) * sizeof(float) + (size_t)((cpr + KS - 1) / KS) * kChunkCols * 2;
}
constexpr int kMaxLds = 160 * 1024;

}  // namespace

// ----------------------------------------------------------------- launchers
hipError_t launch_route_logits(const float *W, const float *bias, int E, int H, const void *x, int x_dtype,
                               int T, float *z, hipStream_t s) {
    dim3 grid(E, (T + kRouteTok - 1) / kRouteTok);
    k_route_logits<<<grid, 256, 0, s>>>(W, bias, E, H, x, x_dtype, T, z);
    return hipGetLastError();
}

int route_blocked_slices(int E, int H, int T) {
    const int tiles = ((T + kRbT - 1) / kRbT) * ((E + kRbE - 1) / kRbE);
    const int steps = H / kRbK;
    int ks = (1024 + tiles - 1) / tiles;   // about four workgroups per CU
    return std::max(1, std::min(ks, std::min(steps, kRouteMaxSlices)));
}

hipError_t launch_route_blocked(const float *W, const float *bias, int E, int H, const void *x, int x_dtype, int T,
                                float *part, float *z, hipStream_t s) {
    if (H % kRbK) return hipErrorInvalidValue;
    const int KS = route_blocked_slices(E, H, T);
    const int steps = H / kRbK;
    const int kslice = ((steps + KS - 1) / KS) * kRbK;
    const int ks_used = (H + kslice - 1) / kslice;
    dim3 grid((T + kRbT - 1) / kRbT, (E + kRbE - 1) / kRbE, ks_used);
    k_route_blocked<<<grid, 256, 0, s>>>(W, E, H, x, x_dtype, T, kslice, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t n = (size_t)T * E;
    k_route_reduce<<<(int)std::min<size_t>((n + 255) / 256, 4096), 256, 0, s>>>(part, bias, E, T, ks_used, z);
    return hipGetLastError();
}

hipError_t launch_topk(const float *z, int E, int k, int score_fn, int T, int32_t *idx, float *w,
                       hipStream_t s, int32_t *idx_host, float *w_host, uint32_t *flag_host, uint32_t seq) {
    k_topk<<<T, kTopkThreads, 0, s>>>(z, E, k, score_fn, idx, w, idx_host, w_host, flag_host, seq);
    return hipGetLastError();
}

hipError_t launch_pack_x(const void *x, int x_dtype, int T, int H, int64_t x_stride, uint32_t *xh, int32_t *xexp,
                         hipStream_t s) {
    if (T == 0) return hipSuccess;
    k_pack_x<<<T, 256, 0, s>>>(x, x_dtype, H, x_stride, xh, xexp);
    return hipGetLastError();
}

hipError_t launch_rvq_gateup(const RecSrc &src, const RecOffsets &off, int H, int I, int n_items,
                             const uint32_t *xh, const int32_t *xexp, float *gu, hipStream_t s) {
    if (n_items == 0) return hipSuccess;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)k_rvq_gateup, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)gateup_lds());
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int grid = n_items * (I / kTileRows) * 2;
    k_rvq_gateup<<<grid, kGuWaves * 64, gateup_lds(), s>>>(src, off, H, I, xh, xexp, gu);
    return hipGetLastError();
}

int down_splits(int H, int I, int n_items) {
    // enough workgroups to cover the chip twice (two 64 KiB workgroups per CU)
    const int tiles = n_items * (H / kTileRows);
    const int cpr = I / kChunkCols;
    int ks = 1;
    while (tiles * ks < 512 && ks * 2 <= cpr / 4) ks *= 2;
    return ks;
}

hipError_t launch_rvq_down(const RecSrc &src, const RecOffsets &off, int H, int I, int n_items, int KS,
                           const float *gu, float *ypart, hipStream_t s) {
    if (n_items == 0) return hipSuccess;
    const size_t lds = down_lds(I, KS);
    if (lds > (size_t)kMaxLds) return hipErrorInvalidValue;
    static bool attr = false;
    if (!attr) {
        hipError_t e =
            hipFuncSetAttribute((const void *)k_rvq_down, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int grid = n_items * (H / kTileRows) * KS;
    k_rvq_down<<<grid, kDnWaves * 64, lds, s>>>(src, off, H, I, KS, gu, ypart);
    return hipGetLastError();
}

hipError_t launch_combine(const float *ypart, int k, int KS, int H, const float *w, const float *ysh,
                          float *out, int64_t out_stride, int T, int accumulate, hipStream_t s) {
    const size_t n = (size_t)T * H;
    const int grid = (int)std::min<size_t>((n + 255) / 256, 4096);
    k_combine<<<grid, 256, 0, s>>>(ypart, k, KS, H, w, ysh, out, out_stride, T, accumulate);
    return hipGetLastError();
}

hipError_t launch_dense_gateup(const uint16_t *shared, int H, int I, const void *x, int x_dtype,
                               int64_t x_stride, int T, float *hs, hipStream_t s) {
    k_dense_gateup<<<(I + 3) / 4, 256, 0, s>>>(shared, H, I, x, x_dtype, x_stride, T, hs);
    return hipGetLastError();
}

hipError_t launch_dense_down(const uint16_t *shared, int H, int I, const float *hs, int T, float *ysh,
                             hipStream_t s) {
    k_dense_down<<<(H + 3) / 4, 256, 0, s>>>(shared, H, I, hs, T, ysh);
    return hipGetLastError();
}

// Plain streaming read of a buffer (the reference rate for expert-weight
// bandwidth): each workgroup XORs one contiguous block, four nontemporal
// 16-byte loads per thread in flight (4 KB apart; a grid-strided order, with
// a thread's loads 8 MB apart, measured 13% slower), and stores the XOR of
// its threads, so no read is dead code and the partials check the data.
__global__ __launch_bounds__(256) void k_hbm_read(const u32x4 *__restrict__ p, size_t n16, uint32_t *__restrict__ sink) {
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b0 = (size_t)blockIdx.x * per, b1 = b0 + per < n16 ? b0 + per : n16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    size_t i = b0 + threadIdx.x;
    for (; i + 3 * 256 < b1; i += 4 * 256) {
        const u32x4 a = __builtin_nontemporal_load(p + i), b = __builtin_nontemporal_load(p + i + 256);
        const u32x4 c = __builtin_nontemporal_load(p + i + 512), d = __builtin_nontemporal_load(p + i + 768);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < b1; i += 256) acc ^= __builtin_nontemporal_load(p + i);
    uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
    for (int o = 32; o > 0; o >>= 1) v ^= __shfl_xor(v, o);
    __shared__ uint32_t part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

hipError_t launch_hbm_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s) {
    k_hbm_read<<<MOE_HBM_READ_BLOCKS, 256, 0, s>>>((const u32x4 *)buf, bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace moe
