// Batched (multi-token) MoE layer on matrix cores for gfx950: group the
// (token, rank) pairs per expert, then per expert a GEMM whose weight operand
// is decoded from the RVQ codes straight into MFMA B fragments.
//
// Source: WASTE article ("2.78조 파라미터 모델을 노트북에서: NVMe 스트리밍 추론
// 엔진 WASTE"), section "실무자에게 남는 질문은 실현 가능성이 아니라
// 엔지니어링": an image becomes 256 prompt positions that each pass through
// every MoE layer like text, which makes a layer call a 256-token batch; same
// article, section "유휴 가중치는 메모리가 아니라 제때 닿기만 하면 된다":
// expert weights stay RVQ-coded (3.00 bits per weight) and are never expanded
// in memory.
//
// v_mfma_f32_16x16x32_bf16: A is 16 (tokens) x 32 (K), B is 32 (K) x 16
// (weight rows); lane l holds A[l%16][8*(l/16)+0..7], B[8*(l/16)+0..7][l%16]
// and D[4*(l/16)+0..3][l%16].  Eight consecutive K values of one weight row
// are exactly one RVQ group, so each lane decodes bf16(C[a] + C[b]) of one
// group into its B fragment.  Within a 128-column chunk, K-step s uses group
// 4*(l/16)+s in lane block l/16 (a fixed permutation of K, applied to A and B
// alike).  The weight row scale is applied to the fp32 accumulator.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGWaves = 8;          // waves per workgroup
constexpr int kTokBlocks = 2;
constexpr int kTwGateUp = 2;        // 16-row tiles per wave unit (gate/up)
constexpr int kTwDown = 5;          // 16-row tiles per wave unit (down)       // 16-token blocks per pass (32 tokens)

__device__ __forceinline__ uint32_t bf16_pair_from_f16_sum(uint32_t a, uint32_t b) {
    const f16x2 s = __builtin_bit_cast(f16x2, a) + __builtin_bit_cast(f16x2, b);   // v_pk_add_f16
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r;
    r.x = (__bf16)(float)s.x;
    r.y = (__bf16)(float)s.y;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 decode_group(const char *cb, uint32_t v) {
    const u32x4 ca = *(const u32x4 *)(cb + ((v << 4) & 0xFFF0u));
    const u32x4 cv = *(const u32x4 *)(cb + ((v >> 8) & 0xFFF0u));
    u32x4 r;
    r.x = bf16_pair_from_f16_sum(ca.x, cv.x);
    r.y = bf16_pair_from_f16_sum(ca.y, cv.y);
    r.z = bf16_pair_from_f16_sum(ca.z, cv.z);
    r.w = bf16_pair_from_f16_sum(ca.w, cv.w);
    return __builtin_bit_cast(bf16x8, r);
}

// The lane's 3 dwords (4 groups) of its row's 48-byte strip in a code tile.
__device__ __forceinline__ void load_quad(const uint8_t *tile, int row_in_tile, int g4, uint32_t &d0, uint32_t &d1,
                                          uint32_t &d2) {
    const int d = 3 * g4;
    auto at = [&](int dw) -> uint32_t {
        return __builtin_nontemporal_load((const uint32_t *)(tile + (dw >> 2) * 1024 + row_in_tile * 16 + (dw & 3) * 4));
    };
    d0 = at(d);
    d1 = at(d + 1);
    d2 = at(d + 2);
}

template <int S>
__device__ __forceinline__ uint32_t quad_code(uint32_t d0, uint32_t d1, uint32_t d2) {
    if constexpr (S == 0) return d0;
    else if constexpr (S == 1) return __builtin_amdgcn_alignbit(d1, d0, 24);
    else if constexpr (S == 2) return __builtin_amdgcn_alignbit(d2, d1, 16);
    else return d2 >> 8;
}

// ------------------------------------------------------------------ group
// One workgroup: histogram of expert ids, exclusive scan, scatter, then a
// per-expert insertion sort so every segment lists its pairs in ascending
// pair index (deterministic).
__global__ __launch_bounds__(1024) void k_group(const int32_t *__restrict__ idx, int n_pairs, int E,
                                                int32_t *__restrict__ perm, int32_t *__restrict__ inv,
                                                int32_t *__restrict__ counts, int32_t *__restrict__ offsets) {
    __shared__ int cnt[MOE_MAX_E + 1];
    __shared__ int off[MOE_MAX_E + 1];
    __shared__ int fill[MOE_MAX_E];
    for (int e = threadIdx.x; e <= E; e += blockDim.x) { cnt[e] = 0; fill[e < E ? e : 0] = 0; }
    __syncthreads();
    for (int p = threadIdx.x; p < n_pairs; p += blockDim.x) atomicAdd(&cnt[idx[p]], 1);
    __syncthreads();
    if (threadIdx.x == 0) {
        int s = 0;
        for (int e = 0; e < E; e++) { off[e] = s; s += cnt[e]; }
        off[E] = s;
    }
    __syncthreads();
    for (int p = threadIdx.x; p < n_pairs; p += blockDim.x) {
        const int e = idx[p];
        perm[off[e] + atomicAdd(&fill[e], 1)] = p;
    }
    __syncthreads();
    __threadfence_block();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int b = off[e], n = cnt[e];
        for (int i = 1; i < n; i++) {
            const int v = perm[b + i];
            int j = i - 1;
            while (j >= 0 && perm[b + j] > v) { perm[b + j + 1] = perm[b + j]; j--; }
            perm[b + j + 1] = v;
        }
        counts[e] = n;
        offsets[e] = b;
    }
    if (threadIdx.x == 0) offsets[E] = off[E];
    __syncthreads();
    for (int q = threadIdx.x; q < n_pairs; q += blockDim.x) inv[perm[q]] = q;
}

// x (fp32 or bf16) -> bf16 [T, H]
__global__ __launch_bounds__(256) void k_to_bf16(const void *__restrict__ x, int x_dtype, size_t n,
                                                 uint16_t *__restrict__ xb) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        if (x_dtype == MOE_DTYPE_BF16) {
            xb[i] = ((const uint16_t *)x)[i];
        } else {
            const __bf16 b = (__bf16)((const float *)x)[i];
            xb[i] = __builtin_bit_cast(uint16_t, b);
        }
    }
}

// --------------------------------------------------------- grouped GEMM
struct GroupedArgs {
    // weights
    const void *const *table;   // [dev] expert record pointers (RVQ experts)
    RecOffsets off;
    const uint16_t *dense;      // dense bf16 matrix rows [N, K] (shared expert), gate at dense, up at dense2
    const uint16_t *dense2;
    // tokens
    const int32_t *counts;      // [E] pairs per expert
    const int32_t *offsets;     // [E] first position of each expert's segment
    const int32_t *perm;        // [positions] -> pair index
    int k;                      // ranks per token (pair -> token = pair / k)
    int n_tokens;               // dense mode: number of tokens (positions = tokens)
    // operands
    const uint16_t *a;          // A rows: x bf16 [T, K] (gate/up) or h bf16 [positions, K] (down)
    int a_by_token;             // 1: A row of position p = token of p; 0: A row = p
    uint16_t *hout;             // gate/up: h bf16 [positions, N]
    float *yout;                // down: y fp32 [positions, N] (scaled)
    int N, K;                   // weight matrix rows (outputs) and columns (reduction)
    int splits;                 // workgroups per expert (row ranges)
    int mat;                    // RVQ matrix: 0 = gate (+up), 2 = down
};

// Work unit of a wave: TW 16-row tiles x one pass of up to 16*kTokBlocks
// tokens, swept over all 128-column chunks.  The codes (or dense weights) and
// the A fragments of chunk j+1 are loaded while chunk j is computed.
template <bool GATEUP, bool DENSE, int TW>
__global__ __launch_bounds__(kGWaves * 64) void k_grouped(GroupedArgs g) {
    extern __shared__ __align__(16) char lds[];
    const int slot = DENSE ? 0 : blockIdx.x / g.splits, split = DENSE ? 0 : blockIdx.x % g.splits;
    int cnt, pos0;
    const uint8_t *rec = nullptr;
    if constexpr (DENSE) {
        cnt = g.n_tokens;
        pos0 = 0;
    } else {
        cnt = g.counts[slot];
        pos0 = g.offsets[slot];
        if (cnt == 0) return;                 // uniform across the workgroup
        rec = (const uint8_t *)g.table[slot];
    }
    char *cb0 = lds, *cb1 = lds + kCbRows * 16;
    if constexpr (!DENSE) {
        const u32x4 *s0 = (const u32x4 *)(rec + g.off.cb[g.mat]);
        const u32x4 *s1 = (const u32x4 *)(rec + g.off.cb[1]);
        for (int i = threadIdx.x; i < kCbRows; i += kGWaves * 64) {
            ((u32x4 *)cb0)[i] = s0[i];
            if constexpr (GATEUP) ((u32x4 *)cb1)[i] = s1[i];
        }
        __syncthreads();
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int col = lane & 15, g4 = lane >> 4;
    const int rows_per_split = g.N / g.splits;          // multiple of 16
    const int r_begin = split * rows_per_split;
    const int tiles = rows_per_split / 16;
    const int tgroups = (tiles + TW - 1) / TW;
    const int cpr = g.K / kChunkCols;
    const uint8_t *codes0 = nullptr, *codes1 = nullptr;
    const _Float16 *sc0 = nullptr, *sc1 = nullptr;
    if constexpr (!DENSE) {
        codes0 = rec + g.off.codes[g.mat];
        codes1 = rec + g.off.codes[1];
        sc0 = (const _Float16 *)(rec + g.off.scales[g.mat]);
        sc1 = (const _Float16 *)(rec + g.off.scales[1]);
    }
    const int passes = (cnt + 16 * kTokBlocks - 1) / (16 * kTokBlocks);
    const int units = tgroups * passes;
    const int u_first = DENSE ? blockIdx.x * kGWaves + wave : wave;
    const int u_step = DENSE ? gridDim.x * kGWaves : kGWaves;
    for (int u = u_first; u < units; u += u_step) {
        const int tg = u % tgroups, pass = u / tgroups;
        const int ntw = min(TW, tiles - tg * TW);             // tiles in this unit (wave-uniform)
        int n[TW];
        const uint8_t *t0[TW], *t1[TW];
#pragma unroll
        for (int t = 0; t < TW; t++) {
            n[t] = r_begin + (tg * TW + min(t, ntw - 1)) * 16 + col;
            if constexpr (!DENSE) {
                t0[t] = codes0 + (size_t)(n[t] >> 6) * cpr * kTileBytes;
                t1[t] = codes1 + (size_t)(n[t] >> 6) * cpr * kTileBytes;
            }
        }
        const int m_base = pass * 16 * kTokBlocks;
        const int nblk = min(kTokBlocks, (cnt - m_base + 15) / 16);
        const uint16_t *arow[kTokBlocks];
#pragma unroll
        for (int b = 0; b < kTokBlocks; b++) {
            const int m = m_base + b * 16 + col;
            arow[b] = nullptr;
            if (b < nblk && m < cnt) {
                const int p = pos0 + m;
                const int row = DENSE ? p : (g.a_by_token ? g.perm[p] / g.k : p);
                arow[b] = g.a + (size_t)row * g.K;
            }
        }
        f32x4 acc0[TW][kTokBlocks], acc1[TW][kTokBlocks];
#pragma unroll
        for (int t = 0; t < TW; t++)
#pragma unroll
            for (int b = 0; b < kTokBlocks; b++) {
                acc0[t][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
                acc1[t][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
        // operand staging for one chunk
        struct Stage {
            uint32_t c0[TW][3], c1[TW][3];          // RVQ codes (4 groups) per tile
            bf16x8 w0[TW][4], w1[TW][4];            // dense weights per tile and K-step
            bf16x8 a[4][kTokBlocks];                // A fragments per K-step and block
        };
        auto load_stage = [&](int j, Stage &st) {
#pragma unroll
            for (int t = 0; t < TW; t++) {
                if (t < ntw) {
                    if constexpr (!DENSE) {
                        load_quad(t0[t] + (size_t)j * kTileBytes, n[t] & 63, g4, st.c0[t][0], st.c0[t][1], st.c0[t][2]);
                        if constexpr (GATEUP)
                            load_quad(t1[t] + (size_t)j * kTileBytes, n[t] & 63, g4, st.c1[t][0], st.c1[t][1],
                                      st.c1[t][2]);
                    } else {
#pragma unroll
                        for (int s = 0; s < 4; s++) {
                            const int kc = j * kChunkCols + (4 * g4 + s) * 8;
                            st.w0[t][s] = *(const bf16x8 *)(g.dense + (size_t)n[t] * g.K + kc);
                            if constexpr (GATEUP) st.w1[t][s] = *(const bf16x8 *)(g.dense2 + (size_t)n[t] * g.K + kc);
                        }
                    }
                }
            }
#pragma unroll
            for (int s = 0; s < 4; s++) {
                const int kc = j * kChunkCols + (4 * g4 + s) * 8;
#pragma unroll
                for (int b = 0; b < kTokBlocks; b++) {
                    st.a[s][b] = (bf16x8){};
                    if (b < nblk && arow[b]) st.a[s][b] = *(const bf16x8 *)(arow[b] + kc);
                }
            }
        };
        Stage cur, nxt;
        load_stage(0, cur);
        for (int j = 0; j < cpr; j++) {
            if (j + 1 < cpr) load_stage(j + 1, nxt);
#pragma unroll
            for (int s = 0; s < 4; s++) {
#pragma unroll
                for (int t = 0; t < TW; t++) {
                    if (t < ntw) {
                        bf16x8 B0, B1;
                        if constexpr (DENSE) {
                            B0 = cur.w0[t][s];
                            if constexpr (GATEUP) B1 = cur.w1[t][s];
                        } else {
                            const uint32_t *c0 = cur.c0[t], *c1 = cur.c1[t];
                            const uint32_t v0 = s == 0 ? quad_code<0>(c0[0], c0[1], c0[2])
                                              : s == 1 ? quad_code<1>(c0[0], c0[1], c0[2])
                                              : s == 2 ? quad_code<2>(c0[0], c0[1], c0[2])
                                                       : quad_code<3>(c0[0], c0[1], c0[2]);
                            B0 = decode_group(cb0, v0);
                            if constexpr (GATEUP) {
                                const uint32_t v1 = s == 0 ? quad_code<0>(c1[0], c1[1], c1[2])
                                                  : s == 1 ? quad_code<1>(c1[0], c1[1], c1[2])
                                                  : s == 2 ? quad_code<2>(c1[0], c1[1], c1[2])
                                                           : quad_code<3>(c1[0], c1[1], c1[2]);
                                B1 = decode_group(cb1, v1);
                            }
                        }
#pragma unroll
                        for (int b = 0; b < kTokBlocks; b++) {
                            if (b < nblk) {
                                acc0[t][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.a[s][b], B0, acc0[t][b], 0, 0, 0);
                                if constexpr (GATEUP)
                                    acc1[t][b] =
                                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.a[s][b], B1, acc1[t][b], 0, 0, 0);
                            }
                        }
                    }
                }
            }
            if (j + 1 < cpr) cur = nxt;
        }
        // epilogue: lane holds D[4*g4 + i][col] of each (tile, block)
#pragma unroll
        for (int t = 0; t < TW; t++) {
            if (t >= ntw) continue;
            float s0v = 1.f, s1v = 1.f;
            if constexpr (!DENSE) {
                s0v = (float)sc0[n[t]];
                if constexpr (GATEUP) s1v = (float)sc1[n[t]];
            }
#pragma unroll
            for (int b = 0; b < kTokBlocks; b++) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int m = m_base + b * 16 + 4 * g4 + i;
                    if (b < nblk && m < cnt) {
                        const size_t p = (size_t)(pos0 + m);
                        if constexpr (GATEUP) {
                            const float gg = acc0[t][b][i] * s0v, uu = acc1[t][b][i] * s1v;
                            const __bf16 h = (__bf16)(gg / (1.f + __expf(-gg)) * uu);
                            g.hout[p * g.N + n[t]] = __builtin_bit_cast(uint16_t, h);
                        } else {
                            g.yout[p * g.N + n[t]] = acc0[t][b][i] * s0v;
                        }
                    }
                }
            }
        }
    }
}

// out[t, c] = sum_j w[t, j] * y[inv[t*k+j], c] + ysh[t, c]
__global__ __launch_bounds__(256) void k_grouped_combine(const float *__restrict__ y, const int32_t *__restrict__ inv,
                                                         const float *__restrict__ w, int k, int H, int T,
                                                         const float *__restrict__ ysh, float *__restrict__ out) {
    const size_t n = (size_t)T * H;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const size_t t = i / H, c = i % H;
        float acc = 0.f;
        for (int j = 0; j < k; j++) acc = fmaf(w[t * k + j], y[(size_t)inv[t * k + j] * H + c], acc);
        if (ysh) acc += ysh[i];
        out[i] = acc;
    }
}

// dense shared-expert down output is written per token as fp32 by k_grouped<false, true>

}  // namespace

hipError_t launch_group(const int32_t *idx, int n_pairs, int E, int32_t *perm, int32_t *inv, int32_t *counts,
                        int32_t *offsets, hipStream_t s) {
    k_group<<<1, 1024, 0, s>>>(idx, n_pairs, E, perm, inv, counts, offsets);
    return hipGetLastError();
}

hipError_t launch_to_bf16(const void *x, int x_dtype, size_t n, uint16_t *xb, hipStream_t s) {
    const int grid = (int)std::min<size_t>((n + 255) / 256, 4096);
    k_to_bf16<<<grid, 256, 0, s>>>(x, x_dtype, n, xb);
    return hipGetLastError();
}

static int pick_splits(int N) {
    // row ranges per expert: whole 16-row tiles, about 8 tiles per wave
    int splits = 1;
    while ((N / (splits * 2)) % 64 == 0 && N / (splits * 2) >= 64 * kGWaves / 2 && splits < 8) splits *= 2;
    return splits;
}

hipError_t launch_grouped_rvq(const void *const *table, const RecOffsets &off, int E, int H, int I,
                              const int32_t *counts, const int32_t *offsets, const int32_t *perm, int k,
                              const uint16_t *xb, uint16_t *hbuf, float *ybuf, hipStream_t s) {
    GroupedArgs g{};
    g.table = table;
    g.off = off;
    g.counts = counts;
    g.offsets = offsets;
    g.perm = perm;
    g.k = k;
    // gate/up: N = I rows, K = H
    g.a = xb;
    g.a_by_token = 1;
    g.hout = hbuf;
    g.N = I;
    g.K = H;
    g.splits = pick_splits(I);
    g.mat = 0;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)k_grouped<true, false, kTwGateUp>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kCbRows * 16);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void *)k_grouped<false, false, kTwDown>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    kCbRows * 16);
        if (e != hipSuccess) return e;
        attr = true;
    }
    k_grouped<true, false, kTwGateUp><<<E * g.splits, kGWaves * 64, 2 * kCbRows * 16, s>>>(g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // down: N = H rows, K = I; A = h rows by position
    g.a = hbuf;
    g.a_by_token = 0;
    g.hout = nullptr;
    g.yout = ybuf;
    g.N = H;
    g.K = I;
    g.splits = pick_splits(H);
    g.mat = 2;
    k_grouped<false, false, kTwDown><<<E * g.splits, kGWaves * 64, kCbRows * 16, s>>>(g);
    return hipGetLastError();
}

hipError_t launch_grouped_dense(const uint16_t *shared, int H, int I, int T, const uint16_t *xb, uint16_t *hs,
                                float *ysh, hipStream_t s) {
    GroupedArgs g{};
    g.n_tokens = T;
    g.k = 1;
    g.a = xb;
    g.a_by_token = 0;
    g.dense = shared;
    g.dense2 = shared + (size_t)I * H;
    g.hout = hs;
    g.N = I;
    g.K = H;
    g.splits = 1;
    const int passes = (T + 16 * kTokBlocks - 1) / (16 * kTokBlocks);
    k_grouped<true, true, 1><<<std::max(1, (I / 16) * passes / kGWaves), kGWaves * 64, 0, s>>>(g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    g.a = hs;
    g.dense = shared + 2 * (size_t)I * H;
    g.dense2 = nullptr;
    g.hout = nullptr;
    g.yout = ysh;
    g.N = H;
    g.K = I;
    k_grouped<false, true, 1><<<std::max(1, (H / 16) * passes / kGWaves), kGWaves * 64, 0, s>>>(g);
    return hipGetLastError();
}

hipError_t launch_grouped_combine(const float *ybuf, const int32_t *inv, const float *w, int k, int H, int T,
                                  const float *ysh, float *out, hipStream_t s) {
    const size_t n = (size_t)T * H;
    const int grid = (int)std::min<size_t>((n + 255) / 256, 4096);
    k_grouped_combine<<<grid, 256, 0, s>>>(ybuf, inv, w, k, H, T, ysh, out);
    return hipGetLastError();
}

}  // namespace moe
