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
// are exactly one RVQ group, so one codebook row is one lane's B fragment.
// The codebooks are converted to bf16 in LDS once; a group then costs two
// gathers, C[a] and C[b], used as B fragments of two MFMAs that share the A
// fragment and the accumulator (W x = C[a] x + C[b] x, summed in fp32): no
// per-group arithmetic besides the addresses.  Within a 128-column chunk,
// K-step s uses group 4*(l/16)+s in lane block l/16 (a fixed permutation of
// K, applied to A and B alike).  The weight row scale is applied to the fp32
// accumulator.
//
// A workgroup multiplies by one matrix of one expert (gate, up or down): its
// LDS is one codebook plus the A ring (76 KB), so two workgroups share a CU
// and one's codebook staging and epilogue overlap the other's gathers.  Gate
// and up go to fp32 buffers and a separate elementwise kernel forms
// h = bf16(SiLU(gate) * up) for the down GEMM.
#include <hip/hip_runtime.h>

#include "moe_internal.h"
#include "rvq_device.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kNw = 8;              // waves per workgroup
constexpr int kTw = 2;              // 16-row tiles per wave unit

__device__ __forceinline__ uint32_t bf16_pair_from_f16_pair(uint32_t a) {
    const f16x2 h = __builtin_bit_cast(f16x2, a);
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r;
    r.x = (__bf16)(float)h.x;
    r.y = (__bf16)(float)h.y;
    return __builtin_bit_cast(uint32_t, r);
}

// fp16 codebook rows staged in LDS -> bf16 in place (each thread its rows)
__device__ __forceinline__ void codebook_to_bf16(char *cb) {
    for (int i = threadIdx.x; i < kCbRows; i += blockDim.x) {
        u32x4 v = ((u32x4 *)cb)[i];
        v.x = bf16_pair_from_f16_pair(v.x);
        v.y = bf16_pair_from_f16_pair(v.y);
        v.z = bf16_pair_from_f16_pair(v.z);
        v.w = bf16_pair_from_f16_pair(v.w);
        ((u32x4 *)cb)[i] = v;
    }
}

// B fragments of the stage-1 and stage-2 codebook rows of a group (24-bit
// code pair v) from a bf16 codebook in LDS
__device__ __forceinline__ void group_rows(const char *cb, uint32_t v, bf16x8 &ba, bf16x8 &bb) {
    ba = *(const bf16x8 *)(cb + ((v << 4) & 0xFFF0u));
    bb = *(const bf16x8 *)(cb + ((v >> 8) & 0xFFF0u));
}

template <int S>
__device__ __forceinline__ uint32_t quad_code(uint32_t d0, uint32_t d1, uint32_t d2) {
    if constexpr (S == 0) return d0;
    else if constexpr (S == 1) return __builtin_amdgcn_alignbit(d1, d0, 24);
    else if constexpr (S == 2) return __builtin_amdgcn_alignbit(d2, d1, 16);
    else return d2 >> 8;
}

// ------------------------------------------------------------------ group
// One workgroup: histogram of expert ids, exclusive scan (one wave), then
// every pair's position in its expert's segment, so that each segment lists
// its pairs in ascending pair index (deterministic).  Pair p is token p / k's
// rank p % k, and a token's k experts differ, so p's position in expert e's
// segment is the number of earlier tokens that chose e: with a bitmap of the
// tokens per expert in LDS (up to kGroupBitWords words), a popcount.  Larger
// cases scatter, then sort each segment by insertion (in LDS up to
// kGroupLdsPairs pairs, else in global memory).
constexpr int kGroupLdsPairs = 12288;
constexpr int kGroupBitWords = 8192;

__global__ __launch_bounds__(1024) void k_group(const int32_t *__restrict__ idx, int n_pairs, int k, int E,
                                                int32_t *__restrict__ perm, int32_t *__restrict__ inv,
                                                int32_t *__restrict__ counts, int32_t *__restrict__ offsets) {
    __shared__ int cnt[MOE_MAX_E + 1];
    __shared__ int off[MOE_MAX_E + 1];
    __shared__ int fill[MOE_MAX_E];
    __shared__ int sperm[kGroupLdsPairs];
    __shared__ uint32_t bits[kGroupBitWords];
    const int T = n_pairs / k, nw = (T + 31) / 32;   // tokens, bitmap words per expert
    const bool by_bits = (long)E * nw <= kGroupBitWords;
    const bool in_lds = n_pairs <= kGroupLdsPairs;
    int *P = in_lds ? sperm : perm;
    for (int e = threadIdx.x; e <= E; e += blockDim.x) { cnt[e] = 0; fill[e < E ? e : 0] = 0; }
    if (by_bits)
        for (int i = threadIdx.x; i < E * nw; i += blockDim.x) bits[i] = 0u;
    __syncthreads();
    for (int p = threadIdx.x; p < n_pairs; p += blockDim.x) {
        const int e = idx[p];
        atomicAdd(&cnt[e], 1);
        if (by_bits) {
            const int t = p / k;
            atomicOr(&bits[e * nw + (t >> 5)], 1u << (t & 31));
        }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        // lane l sums experts [l*per, (l+1)*per); a shuffle scan gives the bases
        const int lane = threadIdx.x, per = (E + 63) / 64;
        const int e0 = min(E, lane * per), e1 = min(E, e0 + per);
        int local = 0;
        for (int e = e0; e < e1; e++) local += cnt[e];
        int incl = local;
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        int base = incl - local;
        for (int e = e0; e < e1; e++) {
            off[e] = base;
            base += cnt[e];
        }
        if (lane == 63) off[E] = incl;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        counts[e] = cnt[e];
        offsets[e] = off[e];
    }
    if (threadIdx.x == 0) offsets[E] = off[E];
    if (by_bits) {
        for (int p = threadIdx.x; p < n_pairs; p += blockDim.x) {
            const int e = idx[p], t = p / k;
            const uint32_t *row = bits + e * nw;
            int rank = __popc(row[t >> 5] & ((1u << (t & 31)) - 1u));
            for (int i = 0; i < (t >> 5); i++) rank += __popc(row[i]);
            const int q = off[e] + rank;
            perm[q] = p;
            inv[p] = q;
        }
        return;
    }
    for (int p = threadIdx.x; p < n_pairs; p += blockDim.x) {
        const int e = idx[p];
        P[off[e] + atomicAdd(&fill[e], 1)] = p;
    }
    __syncthreads();
    __threadfence_block();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int b = off[e], n = cnt[e];
        for (int i = 1; i < n; i++) {
            const int v = P[b + i];
            int j = i - 1;
            while (j >= 0 && P[b + j] > v) { P[b + j + 1] = P[b + j]; j--; }
            P[b + j + 1] = v;
        }
    }
    __syncthreads();
    for (int q = threadIdx.x; q < n_pairs; q += blockDim.x) {
        const int p = P[q];
        if (in_lds) perm[q] = p;
        inv[p] = q;
    }
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
    // tokens
    const int32_t *counts;      // [E] pairs per expert
    const int32_t *offsets;     // [E] first position of each expert's segment
    const int32_t *perm;        // [positions] -> pair index
    int k;                      // ranks per token (pair -> token = pair / k)
    // operands
    const uint16_t *a;          // A rows: x bf16 [T, K] (gate/up) or h bf16 [positions, K] (down)
    int a_by_token;             // 1: A row of position p = token of p; 0: A row = p
    float *yout;                // y fp32 [positions, N] (scaled by the row scale) of matrix mat
    int N, K;                   // weight matrix rows (outputs) and columns (reduction)
    int splits;                 // workgroups per expert and matrix (row ranges)
    int mat;                    // first RVQ matrix: 0 = gate, 1 = up, 2 = down
    int mats;                   // matrices mat .. mat+mats-1, each by workgroups of its own
    size_t ymat_stride;         // elements between the outputs of consecutive matrices
    int xcd_group;              // 1: place each expert's workgroups on one XCD (expert count % 8 == 0)
};

// Dense bf16 GEMM for the shared expert over all T tokens: D[t][n] =
// sum_k A[t][k] W[n][k] (A = x or h in bf16 rows of K, W = weight rows),
// fp32 accumulation.  Workgroup tile: 64 weight rows x 32 MT tokens, 4 waves
// as 2 x 2 (a wave: two 16-row MFMA tiles x 16 MT tokens, per matrix); K goes
// through LDS in stages of 64 columns, double-buffered, the next stage's
// operands loaded into registers while this stage is multiplied.  Rows are
// padded to 144 bytes in LDS so the 16 lanes of a fragment read hit 16
// different bank groups.  K may be split over gridDim.z slices (contiguous
// stage ranges) so that a few-token GEMM still has several workgroups per CU
// in flight; each slice then writes fp32 partial sums, part[z][b][t][n] (b:
// gate, up) or part[z][t][n].  Gate/up with one slice writes
// h = bf16(SiLU(g) * u) directly.  Token rows past T are clamped on load and
// never written.
// MT: 16-token MFMA tiles per wave (a workgroup covers 32 MT tokens); gate/up
// takes MT = 4 (each weight tile is read from L2 by T / 128 workgroups instead
// of T / 32: 43.8 -> 23.5 us at 256 tokens), down MT = 1 (its K is short).
constexpr int kDnN = 64, kDnK = 64, kDnRow = 144;
constexpr int kDnMTGateUp = 4, kDnMTDown = 1;

template <bool GATEUP, int MT>
__global__ __launch_bounds__(256) void k_dense_mm(const uint16_t *__restrict__ A, const uint16_t *__restrict__ W0,
                                                  const uint16_t *__restrict__ W1, int T, int N, int K,
                                                  uint16_t *__restrict__ hout, float *__restrict__ part) {
    constexpr int NB = GATEUP ? 2 : 1;
    constexpr int kDnM = 32 * MT;
    constexpr int kStage = (kDnM + NB * kDnN) * kDnRow;
    __shared__ __align__(16) char lds[2 * kStage];
    const int n0 = blockIdx.x * kDnN, m0 = blockIdx.y * kDnM;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, g4 = lane >> 4;
    const int wn = (wave & 1) * 32, wm = (wave >> 1) * 16 * MT;
    // staging: A kDnM rows x 128 B (MT 16-byte pieces per thread), each
    // weight matrix 64 rows x 128 B (two pieces per thread)
    const int ar = tid >> 3, ap = tid & 7;
    const uint16_t *a_src[MT];
#pragma unroll
    for (int i = 0; i < MT; i++) a_src[i] = A + (size_t)min(m0 + ar + 32 * i, T - 1) * K + ap * 8;
    const uint16_t *w_src[NB][2];
#pragma unroll
    for (int b = 0; b < NB; b++)
#pragma unroll
        for (int h = 0; h < 2; h++) w_src[b][h] = (b ? W1 : W0) + (size_t)(n0 + ar + 32 * h) * K + ap * 8;
    u32x4 ra[MT], rw[NB][2];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < MT; i++) ra[i] = *(const u32x4 *)(a_src[i] + k0);
#pragma unroll
        for (int b = 0; b < NB; b++)
#pragma unroll
            for (int h = 0; h < 2; h++) rw[b][h] = *(const u32x4 *)(w_src[b][h] + k0);
    };
    auto stash = [&](int buf) {
        char *st = lds + buf * kStage;
#pragma unroll
        for (int i = 0; i < MT; i++) *(u32x4 *)(st + (ar + 32 * i) * kDnRow + ap * 16) = ra[i];
#pragma unroll
        for (int b = 0; b < NB; b++)
#pragma unroll
            for (int h = 0; h < 2; h++)
                *(u32x4 *)(st + (kDnM + b * kDnN + ar + 32 * h) * kDnRow + ap * 16) = rw[b][h];
    };
    f32x4 acc[MT][NB][2];
#pragma unroll
    for (int i = 0; i < MT; i++)
#pragma unroll
        for (int b = 0; b < NB; b++)
#pragma unroll
            for (int j = 0; j < 2; j++) acc[i][b][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int stages = K / kDnK, z = blockIdx.z, ks = gridDim.z;
    const int st_begin = z * stages / ks, st_end = (z + 1) * stages / ks;
    fetch(st_begin * kDnK);
    stash(0);
    __syncthreads();
    for (int st = st_begin; st < st_end; st++) {
        const int cur = (st - st_begin) & 1;
        if (st + 1 < st_end) fetch((st + 1) * kDnK);
        const char *L = lds + cur * kStage;
#pragma unroll
        for (int kk = 0; kk < kDnK / 32; kk++) {
            bf16x8 af[MT];
#pragma unroll
            for (int i = 0; i < MT; i++)
                af[i] = *(const bf16x8 *)(L + (wm + 16 * i + col) * kDnRow + kk * 64 + g4 * 16);
#pragma unroll
            for (int b = 0; b < NB; b++)
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const bf16x8 bfr =
                        *(const bf16x8 *)(L + (kDnM + b * kDnN + wn + 16 * j + col) * kDnRow + kk * 64 + g4 * 16);
#pragma unroll
                    for (int i = 0; i < MT; i++)
                        acc[i][b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr, acc[i][b][j], 0, 0, 0);
                }
        }
        if (st + 1 < st_end) stash(cur ^ 1);
        __syncthreads();
    }
    // lane holds D[token 16 mi + 4*g4 + i][row col] of each 16 x 16 tile
#pragma unroll
    for (int mi = 0; mi < MT; mi++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int n = n0 + wn + 16 * j + col;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int t = m0 + wm + 16 * mi + 4 * g4 + i;
                if (t >= T) continue;
                if (GATEUP && ks == 1) {
                    const float g = acc[mi][0][j][i], u = acc[mi][NB - 1][j][i];
                    const __bf16 h = (__bf16)(g / (1.f + __expf(-g)) * u);
                    hout[(size_t)t * N + n] = __builtin_bit_cast(uint16_t, h);
                } else {
#pragma unroll
                    for (int b = 0; b < NB; b++) part[(((size_t)z * NB + b) * T + t) * N + n] = acc[mi][b][j][i];
                }
            }
        }
}

// h[t][n] = bf16(SiLU(sum_z g_z) * sum_z u_z), slices added in order
__global__ __launch_bounds__(256) void k_dense_silu_reduce(const float *__restrict__ part, int ks, size_t tn,
                                                           uint16_t *__restrict__ h) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < tn; i += (size_t)gridDim.x * blockDim.x) {
        float g = 0.f, u = 0.f;
        for (int z = 0; z < ks; z++) {
            g += part[(2 * (size_t)z) * tn + i];
            u += part[(2 * (size_t)z + 1) * tn + i];
        }
        h[i] = __builtin_bit_cast(uint16_t, (__bf16)(g / (1.f + __expf(-g)) * u));
    }
}

// RVQ experts: one 16-token block per pass (experts average 10.7 tokens in
// the 256-token layer; the few with more take a second pass over their
// codes).  All waves of a workgroup sweep the 128-column chunks together:
//  - the A operand (16 token rows x 128 columns, 4 KB per chunk) goes
//    through a 3-slot ring in LDS, copied once per workgroup instead of once
//    per wave (the first four waves copy it, one 16-byte piece per lane, two
//    chunks ahead), with one workgroup barrier per chunk;
//  - each wave keeps its own codes in a 3-deep register ring (loads past the
//    last chunk re-read it and tiles past the last row re-use the last tile,
//    so the steady state has no branches around its loads);
//  - the codebook gathers run one K-step ahead of the MFMAs that use them.
// The epilogue writes real rows and tokens only.
constexpr int kBufNt = 2;                     // buffer load cache policy: non-temporal
constexpr int kBufWord3 = 0x00020000;         // buffer descriptor word 3 (32-bit data format)
constexpr int kASlot = 16 * kChunkCols * 2;   // bytes of one A ring slot
constexpr int kARing = 3;

// A lane's 4 groups are 12 bytes (dwords d0, d1, d2) of its row's 48-byte
// strip, which the record splits into three 16-byte parts 1 KB apart.  They
// come in one 8-byte and one 4-byte load: lane blocks 0 and 2 read (d0, d1)
// and d2, blocks 1 and 3 (whose 12 bytes straddle a part boundary) read
// (d1, d2) and d0.  Per wave and tile the two loads touch 10 cache lines
// where three 4-byte loads touched 18.
struct RvqQuadOff {
    int part8, byte8, part4, byte4;   // the 8-byte and the 4-byte load: strip part and byte in it
};
__device__ __forceinline__ RvqQuadOff rvq_quad_off(int g4) {
    switch (g4) {
    case 0: return {0, 0, 0, 8};
    case 1: return {1, 0, 0, 12};
    case 2: return {1, 8, 2, 0};
    default: return {2, 8, 2, 4};
    }
}

template <int TW>
struct RvqStage {
    // per tile: the 8-byte load in [0], [1], the 4-byte one in [2]
    uint32_t c0[TW][3];
};

// Codes of chunk j through buffer loads: rs describes the matrix's code
// section (reads past its end return zero), qoff[t] the lane's byte offsets
// of its two loads of tile t in chunk 0, and the chunk's offset goes in the
// scalar offset.  Streaming (nt) loads.
template <int TW>
__device__ __forceinline__ void rvq_load(RvqStage<TW> &st, __amdgpu_buffer_rsrc_t rs, const uint32_t (&qoff)[TW][2],
                                         int j) {
    const int soff = j * kTileBytes;
#pragma unroll
    for (int t = 0; t < TW; t++) {
        const auto q0 = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)qoff[t][0], soff, kBufNt);
        st.c0[t][0] = q0[0];
        st.c0[t][1] = q0[1];
        st.c0[t][2] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)qoff[t][1], soff, kBufNt);
    }
}

// (d0, d1, d2) from a tile's loads; odd: lane block 1 or 3
__device__ __forceinline__ void rvq_dwords(const uint32_t (&c)[3], bool odd, uint32_t &d0, uint32_t &d1,
                                           uint32_t &d2) {
    d0 = odd ? c[2] : c[0];
    d1 = odd ? c[0] : c[1];
    d2 = odd ? c[1] : c[2];
}

// Gathered B fragments of one K-step: C[a] and C[b] per tile.
template <int TW>
struct RvqGather {
    bf16x8 b[TW][2];
};

template <int TW, int S>
__device__ __forceinline__ void rvq_gather(const RvqStage<TW> &st, bool odd, const char *cb, RvqGather<TW> &g) {
#pragma unroll
    for (int t = 0; t < TW; t++) {
        uint32_t d0, d1, d2;
        rvq_dwords(st.c0[t], odd, d0, d1, d2);
        group_rows(cb, quad_code<S>(d0, d1, d2), g.b[t][0], g.b[t][1]);
    }
}

template <int TW>
__device__ __forceinline__ void rvq_mfma(const bf16x8 &a, const RvqGather<TW> &g, f32x4 (&acc)[TW]) {
#pragma unroll
    for (int t = 0; t < TW; t++) {
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, g.b[t][0], acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, g.b[t][1], acc[t], 0, 0, 0);
    }
}

// Wait until at most N LDS operations of this wave are outstanding, then a
// workgroup barrier; outstanding global loads are not waited for.
template <int N>
__device__ __forceinline__ void lds_wait_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));   // vmcnt(63) expcnt(7) lgkmcnt(N)
    asm volatile("s_barrier" ::: "memory");
}

// The A ring.  Token m's 16-byte piece q (columns 8q..8q+7 of the chunk)
// sits at m*256 + (q ^ m)*16 of a slot, so the 16 lanes of one lane block
// (16 tokens, one piece each) read 16 different bank groups.  Thread i < 256
// of the workgroup copies piece i to slot byte 16 i.
struct ARing {
    bool copy;                  // this wave copies (waves 0-3; wave-uniform)
    char *base;                 // slot 0
    const uint16_t *src;        // the lane's token row + its piece (columns 8q..)
    uint32_t wr;                // byte offset of the lane's piece in a slot
    uint32_t rd[4];             // byte offset of the lane's A fragment of K-step s in a slot
};

__device__ __forceinline__ u32x4 a_fetch(const ARing &r, int j) {
    return *(const u32x4 *)(r.src + (size_t)j * kChunkCols);
}
__device__ __forceinline__ void a_store(const ARing &r, int slot, const u32x4 &v) {
    *(u32x4 *)(r.base + slot * kASlot + r.wr) = v;
}

// One chunk (ring slot R, codes in cur): on entry g holds K-step 0 of this
// chunk's gathers and areg the A piece of chunk j+1 (copied here into the
// ring); areg leaves with chunk j+2's piece, fill with chunk j+2's codes
// and, with NEXT, g with K-step 0 of the next chunk (nxt).
template <int TW, bool NEXT, int R>
__device__ __forceinline__ void rvq_chunk(const RvqStage<TW> &cur, const RvqStage<TW> &nxt, RvqStage<TW> &fill,
                                          __amdgpu_buffer_rsrc_t rs, const uint32_t (&qoff)[TW][2], bool odd,
                                          int j, int cpr, const ARing &ar, u32x4 &areg, const char *cb,
                                          RvqGather<TW> &g, f32x4 (&acc)[TW]) {
    constexpr int kG = TW * 2;   // gathers per K-step
    static_assert(kG <= 15, "lgkmcnt range");
    if (ar.copy) a_store(ar, (R + 1) % kARing, areg);
    bf16x8 a[4];
    const char *slot = ar.base + R * kASlot;
#pragma unroll
    for (int s = 0; s < 4; s++) a[s] = *(const bf16x8 *)(slot + ar.rd[s]);
    if (ar.copy) areg = a_fetch(ar, min(j + 2, cpr - 1));
    rvq_load<TW>(fill, rs, qoff, min(j + 2, cpr - 1));
    __builtin_amdgcn_sched_barrier(0);
    RvqGather<TW> g1, g2;
    rvq_gather<TW, 1>(cur, odd, cb, g1);
    __builtin_amdgcn_sched_barrier(0);
    // the A copy of chunk j+1 (issued before the K-step 1 gathers) is done
    lds_wait_barrier<kG>();
    __builtin_amdgcn_sched_barrier(0);
    rvq_mfma<TW>(a[0], g, acc);
    __builtin_amdgcn_sched_barrier(0);
    rvq_gather<TW, 2>(cur, odd, cb, g2);
    __builtin_amdgcn_sched_barrier(0);
    rvq_mfma<TW>(a[1], g1, acc);
    __builtin_amdgcn_sched_barrier(0);
    rvq_gather<TW, 3>(cur, odd, cb, g1);
    __builtin_amdgcn_sched_barrier(0);
    rvq_mfma<TW>(a[2], g2, acc);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) rvq_gather<TW, 0>(nxt, odd, cb, g);
    __builtin_amdgcn_sched_barrier(0);
    rvq_mfma<TW>(a[3], g1, acc);
    __builtin_amdgcn_sched_barrier(0);
}

template <int TW, int NW>
__global__ __launch_bounds__(NW * 64) void k_grouped_rvq(GroupedArgs g) {
    static_assert(NW >= 4, "the A copy needs 256 lanes");
    extern __shared__ __align__(16) char lds[];
    // Workgroups are dealt to the 8 XCDs round-robin by index; when the
    // expert count is a multiple of 8, the row ranges of one expert all go to
    // one XCD (consecutive there), so its codebooks and A rows come from HBM
    // once and from that XCD's L2 after.
    // An expert's units are its matrices' row ranges (matrix-major).
    const int units = g.mats * g.splits;
    int slot, unit;
    if (g.xcd_group) {
        const int b = blockIdx.x, xcd = b & 7, idx = b >> 3;
        slot = (idx / units) * 8 + xcd;
        unit = idx % units;
    } else {
        slot = blockIdx.x / units;
        unit = blockIdx.x % units;
    }
    const int split = unit % g.splits, m = unit / g.splits;
    const int mat = g.mat + m;
    float *const yout = g.yout + m * g.ymat_stride;
    const int cnt = g.counts[slot], pos0 = g.offsets[slot];
    if (cnt == 0) return;                 // uniform across the workgroup
    const uint8_t *rec = (const uint8_t *)g.table[slot];
    char *cb = lds, *aring = lds + kCbRows * 16;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    // the codebook into LDS with direct copies (all in flight at once), then bf16
    stage_lds_waves<kLdsPlain, NW>(cb, rec + g.off.cb[mat], kCbRows * 16, wave, lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    codebook_to_bf16(cb);
    const int col = lane & 15, g4 = lane >> 4;
    const RvqQuadOff qo = rvq_quad_off(g4);
    const bool odd = (g4 & 1) != 0;
    const int rows_per_split = g.N / g.splits;          // multiple of 16
    const int r_begin = split * rows_per_split;
    const int tiles = rows_per_split / 16;
    const int tgroups = (tiles + TW - 1) / TW;
    const int rounds = (tgroups + NW - 1) / NW;
    const int cpr = g.K / kChunkCols;
    const int code_bytes = g.N / 64 * cpr * kTileBytes;   // the matrix's code section
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(rec + g.off.codes[mat]), 0, code_bytes, kBufWord3);
    const _Float16 *sc = (const _Float16 *)(rec + g.off.scales[mat]);
    const int passes = (cnt + 15) / 16;
    ARing ar;
    ar.copy = wave < 4;
    ar.base = aring;
    const int apiece = (wave * 64 + lane) & 255;   // A piece a copying lane copies: token apiece/16, piece apiece%16
    ar.wr = apiece * 16;
#pragma unroll
    for (int s = 0; s < 4; s++) ar.rd[s] = col * 256 + (((4 * g4 + s) ^ col) & 15) * 16;
    // Every wave runs every (pass, round) so the barriers line up; a wave
    // without a tile group in the last round repeats the last one and
    // writes nothing.
    for (int it = 0; it < passes * rounds; it++) {
        const int pass = it / rounds, tg_raw = (it % rounds) * NW + wave;
        const bool active = tg_raw < tgroups;                  // wave-uniform
        const int tg = min(tg_raw, tgroups - 1);
        const int ntw = min(TW, tiles - tg * TW);             // tiles in this unit (wave-uniform)
        int n[TW];
        uint32_t qoff[TW][2];
#pragma unroll
        for (int t = 0; t < TW; t++) {
            n[t] = r_begin + (tg * TW + min(t, ntw - 1)) * 16 + col;
            const uint32_t row0 = (uint32_t)((n[t] >> 6) * cpr) * kTileBytes + (n[t] & 63) * 16;
            qoff[t][0] = row0 + qo.part8 * 1024 + qo.byte8;
            qoff[t][1] = row0 + qo.part4 * 1024 + qo.byte4;
        }
        // the copying lanes' A rows: tokens past the pass's last real one
        // copy the last real row (their products are never written)
        {
            const int mloc = apiece >> 4;
            const int m = min(pass * 16 + mloc, cnt - 1);
            const int p = pos0 + m;
            const uint16_t *row = g.a + (size_t)(g.a_by_token ? g.perm[p] / g.k : p) * g.K;
            ar.src = row + (((lane & 15) ^ mloc) & 15) * 8;
        }
        f32x4 acc[TW];
#pragma unroll
        for (int t = 0; t < TW; t++) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
        // prologue: every wave is past the previous unit's last A reads (and
        // the codebook conversion) before slot 0 is rewritten
        u32x4 areg = {0u, 0u, 0u, 0u};
        if (ar.copy) areg = a_fetch(ar, 0);
        lds_wait_barrier<0>();
        if (ar.copy) {
            a_store(ar, 0, areg);
            areg = a_fetch(ar, min(1, cpr - 1));
        }
        RvqStage<TW> st[3];
        rvq_load<TW>(st[0], rs, qoff, 0);
        rvq_load<TW>(st[1], rs, qoff, min(1, cpr - 1));
        RvqGather<TW> g0;
        rvq_gather<TW, 0>(st[0], odd, cb, g0);
        lds_wait_barrier<0>();
        int j = 0;
        for (; j + 3 <= cpr; j += 3) {
            rvq_chunk<TW, true, 0>(st[0], st[1], st[2], rs, qoff, odd, j, cpr, ar, areg, cb, g0, acc);
            rvq_chunk<TW, true, 1>(st[1], st[2], st[0], rs, qoff, odd, j + 1, cpr, ar, areg, cb, g0, acc);
            rvq_chunk<TW, true, 2>(st[2], st[0], st[1], rs, qoff, odd, j + 2, cpr, ar, areg, cb, g0, acc);
        }
        // the last cpr - j (< 3) chunks are already in st[0], st[1]
        if (j + 2 == cpr) {
            rvq_chunk<TW, true, 0>(st[0], st[1], st[2], rs, qoff, odd, j, cpr, ar, areg, cb, g0, acc);
            rvq_chunk<TW, false, 1>(st[1], st[2], st[0], rs, qoff, odd, j + 1, cpr, ar, areg, cb, g0, acc);
        } else if (j + 1 == cpr) {
            rvq_chunk<TW, false, 0>(st[0], st[1], st[2], rs, qoff, odd, j, cpr, ar, areg, cb, g0, acc);
        }
        if (!active) continue;
        // epilogue: lane holds D[4*g4 + i][col] of each tile
#pragma unroll
        for (int t = 0; t < TW; t++) {
            if (t >= ntw) continue;
            const float sv = (float)sc[n[t]];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int mm = pass * 16 + 4 * g4 + i;
                if (mm >= cnt) continue;
                yout[(size_t)(pos0 + mm) * g.N + n[t]] = acc[t][i] * sv;
            }
        }
    }
}

// h = bf16(SiLU(g) * u) from the fp32 gate and up outputs, 4 per thread
__global__ __launch_bounds__(256) void k_silu_mul(const float4 *__restrict__ gv, const float4 *__restrict__ uv,
                                                  size_t n4, uint2 *__restrict__ h) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
        const float4 a = gv[i], b = uv[i];
        const float gg[4] = {a.x, a.y, a.z, a.w}, uu[4] = {b.x, b.y, b.z, b.w};
        uint16_t r[4];
#pragma unroll
        for (int j = 0; j < 4; j++)
            r[j] = __builtin_bit_cast(uint16_t, (__bf16)(gg[j] / (1.f + __expf(-gg[j])) * uu[j]));
        h[i] = make_uint2(r[0] | (uint32_t)r[1] << 16, r[2] | (uint32_t)r[3] << 16);
    }
}

// out[t, c] = sum_j w[t, j] * y[inv[t*k+j], c] + sum_z ysh[z, t, c], the
// ranks and the shared expert's slices in order.  Workgroup row blockIdx.y takes tokens blockIdx.y + i * gridDim.y; a
// thread takes V consecutive columns (V = 4 with 16-byte aligned rows).
template <int V>
__device__ __forceinline__ void load_v(const float *p, float (&v)[V]) {
    if constexpr (V == 4) {
        const float4 q = *(const float4 *)p;
        v[0] = q.x, v[1] = q.y, v[2] = q.z, v[3] = q.w;
    } else {
#pragma unroll
        for (int i = 0; i < V; i++) v[i] = p[i];
    }
}

template <int V>
__global__ __launch_bounds__(256) void k_grouped_combine(const float *__restrict__ y, const int32_t *__restrict__ inv,
                                                         const float *__restrict__ w, int k, int H, int T,
                                                         const float *__restrict__ ysh, int nsh,
                                                         float *__restrict__ out) {
    const int c = (blockIdx.x * blockDim.x + threadIdx.x) * V;
    if (c >= H) return;
    for (int t = blockIdx.y; t < T; t += gridDim.y) {
        float acc[V] = {};
        for (int j = 0; j < k; j++) {
            const float wj = w[(size_t)t * k + j];
            float v[V];
            load_v<V>(y + (size_t)inv[(size_t)t * k + j] * H + c, v);
#pragma unroll
            for (int i = 0; i < V; i++) acc[i] = fmaf(wj, v[i], acc[i]);
        }
        if (nsh > 0) {
            float sh[V] = {};
            for (int z = 0; z < nsh; z++) {
                float v[V];
                load_v<V>(ysh + ((size_t)z * T + t) * H + c, v);
#pragma unroll
                for (int i = 0; i < V; i++) sh[i] += v[i];
            }
#pragma unroll
            for (int i = 0; i < V; i++) acc[i] += sh[i];
        }
        float *o = out + (size_t)t * H + c;
        if constexpr (V == 4) {
            *(float4 *)o = make_float4(acc[0], acc[1], acc[2], acc[3]);
        } else {
#pragma unroll
            for (int i = 0; i < V; i++) o[i] = acc[i];
        }
    }
}

}  // namespace

hipError_t launch_group(const int32_t *idx, int n_pairs, int k, int E, int32_t *perm, int32_t *inv,
                        int32_t *counts, int32_t *offsets, hipStream_t s) {
    k_group<<<1, 1024, 0, s>>>(idx, n_pairs, k, E, perm, inv, counts, offsets);
    return hipGetLastError();
}

hipError_t launch_to_bf16(const void *x, int x_dtype, size_t n, uint16_t *xb, hipStream_t s) {
    const int grid = (int)std::min<size_t>((n + 255) / 256, 4096);
    k_to_bf16<<<grid, 256, 0, s>>>(x, x_dtype, n, xb);
    return hipGetLastError();
}

// Row ranges per expert: the most (up to 16) that divide N into whole rounds
// of the workgroup's tile groups (16 * TW * NW rows), else one range.
static int pick_splits(int N, int TW, int NW) {
    const int round_rows = 16 * TW * NW;
    for (int s = 16; s > 1; s--)
        if (N % s == 0 && (N / s) % round_rows == 0) return s;
    return 1;
}

constexpr int kLdsRvq = kCbRows * 16 + kARing * kASlot;   // 76 KB: two workgroups per CU

hipError_t launch_grouped_rvq(const void *const *table, const RecOffsets &off, int E, int H, int I, int n_pairs,
                              const int32_t *counts, const int32_t *offsets, const int32_t *perm, int k,
                              const uint16_t *xb, uint16_t *hbuf, float *ybuf, hipStream_t s) {
    GroupedArgs g{};
    g.table = table;
    g.off = off;
    g.counts = counts;
    g.offsets = offsets;
    g.perm = perm;
    g.k = k;
    g.xcd_group = E % 8 == 0;
    static bool attr = false;
    if (!attr) {
        const hipError_t e = hipFuncSetAttribute((const void *)k_grouped_rvq<kTw, kNw>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, kLdsRvq);
        if (e != hipSuccess) return e;
        attr = true;
    }
    // gate and up (N = I rows, K = H, A = x rows by token), each by its own
    // workgroups: gate into ybuf[0, pairs*I), up into ybuf[pairs*I, 2*pairs*I)
    g.a = xb;
    g.a_by_token = 1;
    g.N = I;
    g.K = H;
    g.mat = 0;
    g.mats = 2;
    g.ymat_stride = (size_t)n_pairs * I;
    g.yout = ybuf;
    g.splits = pick_splits(I, kTw, kNw);
    k_grouped_rvq<kTw, kNw><<<E * 2 * g.splits, kNw * 64, kLdsRvq, s>>>(g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // h = bf16(SiLU(gate) * up)
    const size_t n4 = (size_t)n_pairs * I / 4;
    const int grid = (int)std::min<size_t>((n4 + 255) / 256, 4096);
    k_silu_mul<<<grid, 256, 0, s>>>((const float4 *)ybuf, (const float4 *)(ybuf + g.ymat_stride), n4, (uint2 *)hbuf);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // down: N = H rows, K = I; A = h rows by position
    g.a = hbuf;
    g.a_by_token = 0;
    g.N = H;
    g.K = I;
    g.mat = 2;
    g.mats = 1;
    g.ymat_stride = 0;
    g.splits = pick_splits(H, kTw, kNw);
    k_grouped_rvq<kTw, kNw><<<E * g.splits, kNw * 64, kLdsRvq, s>>>(g);
    return hipGetLastError();
}

int dense_splits(int N, int T, int K, int M) {
    const int tiles = (N / kDnN) * ((T + M - 1) / M);
    const int ks = (1024 + tiles - 1) / tiles;   // about four workgroups per CU
    return std::max(1, std::min(ks, std::min(K / kDnK, 8)));
}

size_t dense_part_floats(int H, int I, int T) {
    const int kg = dense_splits(I, T, H, 32 * kDnMTGateUp), kd = dense_splits(H, T, I, 32 * kDnMTDown);
    return std::max(kg > 1 ? (size_t)kg * 2 * T * I : 0, (size_t)kd * T * H);
}

hipError_t launch_grouped_dense(const uint16_t *shared, int H, int I, int T, const uint16_t *xb, uint16_t *hs,
                                float *part, int *nsh, hipStream_t s) {
    *nsh = 0;
    if (T <= 0) return hipSuccess;
    if (I % kDnN || H % kDnN || H % kDnK || I % kDnK) return hipErrorInvalidValue;
    const uint16_t *wg = shared, *wu = shared + (size_t)I * H, *wd = shared + 2 * (size_t)I * H;
    constexpr int Mg = 32 * kDnMTGateUp, Md = 32 * kDnMTDown;
    const int kg = dense_splits(I, T, H, Mg), kd = dense_splits(H, T, I, Md);
    k_dense_mm<true, kDnMTGateUp><<<dim3(I / kDnN, (T + Mg - 1) / Mg, kg), 256, 0, s>>>(xb, wg, wu, T, I, H, hs, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (kg > 1) {
        const size_t tn = (size_t)T * I;
        k_dense_silu_reduce<<<(int)std::min<size_t>((tn + 255) / 256, 4096), 256, 0, s>>>(part, kg, tn, hs);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // down partials (kd slices of [T, H]) are added by the combine
    k_dense_mm<false, kDnMTDown><<<dim3(H / kDnN, (T + Md - 1) / Md, kd), 256, 0, s>>>(hs, wd, nullptr, T, H, I,
                                                                                     nullptr, part);
    *nsh = kd;
    return hipGetLastError();
}

hipError_t launch_grouped_combine(const float *ybuf, const int32_t *inv, const float *w, int k, int H, int T,
                                  const float *ysh, int nsh, float *out, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const dim3 block(256);
    const int rows = std::min(T, 65535);
    // y and ysh rows are 16-byte aligned (workspace, H % 128 == 0); out is the caller's
    if (H % 4 == 0 && (uintptr_t)out % 16 == 0)
        k_grouped_combine<4><<<dim3((H / 4 + 255) / 256, rows), block, 0, s>>>(ybuf, inv, w, k, H, T, ysh, nsh, out);
    else
        k_grouped_combine<1><<<dim3((H + 255) / 256, rows), block, 0, s>>>(ybuf, inv, w, k, H, T, ysh, nsh, out);
    return hipGetLastError();
}

}  // namespace moe
