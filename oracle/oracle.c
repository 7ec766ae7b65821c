/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the routed-expert MoE decode
 * path (router logits -> top-k -> per-expert SwiGLU on RVQ codes -> combine,
 * plus the LRU slot-cache trace).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP path; it reads the same input bytes.
 *
 * Everything is computed in double precision from the stored fp32 / fp16 /
 * bf16 values, which all convert to double exactly.  Loops are written in
 * the order the definitions state.  Optional threads split independent
 * output rows only, so results do not depend on the thread count.
 *
 * Sources (pages on routed expert streaming):
 *  [WISP]  "WISP -- 실행될 수 없는 것을 스트리밍하다" (molayo1419.me),
 *          sections "통찰" (the model's own router picks the experts of each
 *          token; an LRU cache promotes frequently used experts) and
 *          "Lesson 2" (the router is the scheduler; no heuristics).
 *  [WASTE] "2.78조 파라미터 모델을 노트북에서: NVMe 스트리밍 추론 엔진 WASTE"
 *          (ttj.ttj.kr), section "유휴 가중치는 메모리가 아니라 제때 닿기만
 *          하면 된다" (one aligned record per expert, gate/up/down adjacent;
 *          residual vector quantisation at 3.00 bits per weight, matrices
 *          never expanded) and section "병목은 산술이 아니라 저장장치와
 *          램이다" (every layer checked against a reference).
 *  [WARP]  "WARP 소개" (discuss.pytorch.kr), section "WARP의 캐시 설정에서
 *          드러나는 역설" (experts per token is a manifest parameter) and
 *          section "WARP가 모델을 램에 올리지 않는 방법" (prediction changes
 *          timing only, never results).
 * The pages give no formula for routing, SwiGLU or RVQ decoding.  The
 * readings taken here (documented with the repository's design notes):
 *  - weights are W[out, in], y = W x; a group is 8 consecutive input-dim
 *    weights of one row; W[r, 8q+i] = s_r * (C[a][i] + C[b][i]) with one
 *    4096x8 fp16 codebook per matrix shared by both stages;
 *  - selection orders experts by (logit desc, id asc) and keeps the first k;
 *    gate weights are softmax or sigmoid renormalised over the selected set;
 *  - expert FFN: y = W_d (SiLU(W_g x) * (W_u x)), SiLU(v) = v / (1 + e^-v);
 *  - layer output = sum_j w_j y_j + shared(x) (shared expert dense, weight 1);
 *  - cache: one LRU over keys layer*E + expert, lookups of one layer step in
 *    ascending expert id; a miss takes the lowest free slot, else evicts the
 *    least recently used key and reuses its slot.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_CB_ROWS 4096
#define ORC_GROUP 8

/* ---------------------------------------------------------------- values */

/* IEEE binary16 -> double, from the bit fields. */
static double half_to_double(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);
    return sign ? -v : v;
}

/* bfloat16 -> double: the upper half of an IEEE binary32. */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

double oracle_half_to_double(uint16_t h) { return half_to_double(h); }
double oracle_bf16_to_double(uint16_t b) { return bf16_to_double(b); }

/* ---------------------------------------------------------------- format */

static int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

/* Section offsets of one expert record: gate/up/down codes, gate/up/down
 * fp16 scales, gate/up/down fp16 codebooks; each section 256-byte aligned,
 * record padded to 4 KiB.  Returns 0, or -1 for dimensions the tiled code
 * layout cannot hold (H and I must be multiples of 128). */
int oracle_record_layout(int H, int I, int64_t off[9], int64_t size[9],
                         int64_t *nbytes, int64_t *padded)
{
    if (H <= 0 || I <= 0 || H % 128 || I % 128)
        return -1;
    int64_t s[9];
    s[0] = (int64_t)I * (H / ORC_GROUP) * 3;
    s[1] = s[0];
    s[2] = (int64_t)H * (I / ORC_GROUP) * 3;
    s[3] = 2 * (int64_t)I;
    s[4] = 2 * (int64_t)I;
    s[5] = 2 * (int64_t)H;
    s[6] = s[7] = s[8] = (int64_t)ORC_CB_ROWS * ORC_GROUP * 2;
    int64_t pos = 0;
    for (int i = 0; i < 9; i++) {
        pos = align_up(pos, 256);
        off[i] = pos;
        size[i] = s[i];
        pos += s[i];
    }
    *nbytes = pos;
    *padded = align_up(pos, 4096);
    return 0;
}

/* The 24-bit code pair of row r, group q of a matrix with K columns, stored
 * in 64-row x 128-column tiles of 3072 bytes: strip byte p of tile row l is
 * at (p / 16) * 1024 + l * 16 + p % 16; strip byte 3g+m is byte m
 * (little-endian) of group g's value. */
uint32_t oracle_code_pair(const uint8_t *sec, int K, int r, int q)
{
    int64_t t = r / 64, l = r % 64, j = q / 16, g = q % 16;
    const uint8_t *tile = sec + (t * (K / 128) + j) * 3072;
    uint32_t v = 0;
    for (int m = 0; m < 3; m++) {
        int p = 3 * (int)g + m;
        v |= (uint32_t)tile[(p / 16) * 1024 + l * 16 + (p % 16)] << (8 * m);
    }
    return v;
}

/* Decoded codebook in double: cbd[c*8+i] = C[c][i]. */
static void codebook_to_double(const uint16_t *cb, double *cbd)
{
    for (int c = 0; c < ORC_CB_ROWS * ORC_GROUP; c++)
        cbd[c] = half_to_double(cb[c]);
}

/* RVQ decode of one row: w[8q+i] = s_r * (C[a][i] + C[b][i]), a = v & 0xFFF,
 * b = v >> 12. */
static void decode_row(const uint8_t *sec, const double *cbd, double s_r,
                       int K, int r, double *w)
{
    for (int q = 0; q < K / ORC_GROUP; q++) {
        uint32_t v = oracle_code_pair(sec, K, r, q);
        uint32_t a = v & 0xFFF, b = v >> 12;
        for (int i = 0; i < ORC_GROUP; i++)
            w[q * ORC_GROUP + i] = s_r * (cbd[a * ORC_GROUP + i] + cbd[b * ORC_GROUP + i]);
    }
}

/* Public single-row decode (tests pin it against the closed form). */
int oracle_rvq_decode_row(const uint8_t *sec, const uint16_t *scales,
                          const uint16_t *codebook, int N, int K, int r, double *w)
{
    if (r < 0 || r >= N || K % 128 || N % 64)
        return -1;
    double *cbd = malloc(sizeof(double) * ORC_CB_ROWS * ORC_GROUP);
    if (!cbd)
        return -2;
    codebook_to_double(codebook, cbd);
    decode_row(sec, cbd, half_to_double(scales[r]), K, r, w);
    free(cbd);
    return 0;
}

/* ----------------------------------------------------- threaded row loops */

typedef struct {
    const uint8_t *sec;      /* codes of one matrix */
    const double *cbd;       /* decoded codebook */
    const uint16_t *scales;  /* fp16 [N] */
    int N, K, T;
    const double *x;         /* [T, K] */
    double *y;               /* [T, N] */
    int r0, r1;
} gemv_job;

static void *gemv_rows(void *arg)
{
    gemv_job *j = arg;
    double *w = malloc(sizeof(double) * j->K);
    if (!w)
        return (void *)1;
    for (int r = j->r0; r < j->r1; r++) {
        decode_row(j->sec, j->cbd, half_to_double(j->scales[r]), j->K, r, w);
        for (int t = 0; t < j->T; t++) {
            const double *xt = j->x + (int64_t)t * j->K;
            double acc = 0.0;
            for (int c = 0; c < j->K; c++)
                acc += w[c] * xt[c];
            j->y[(int64_t)t * j->N + r] = acc;
        }
    }
    free(w);
    return NULL;
}

static int g_threads = 1;

void oracle_set_threads(int n) { g_threads = n < 1 ? 1 : (n > 256 ? 256 : n); }
int oracle_get_threads(void) { return g_threads; }

/* y[t, r] = sum_c W[r, c] x[t, c] for an RVQ matrix [N, K]. */
static int rvq_gemv(const uint8_t *sec, const uint16_t *scales, const uint16_t *cb,
                    int N, int K, const double *x, int T, double *y)
{
    double *cbd = malloc(sizeof(double) * ORC_CB_ROWS * ORC_GROUP);
    if (!cbd)
        return -2;
    codebook_to_double(cb, cbd);
    int nt = g_threads < N ? g_threads : N;
    pthread_t th[256];
    gemv_job jobs[256];
    int rc = 0;
    for (int i = 0; i < nt; i++) {
        jobs[i] = (gemv_job){sec, cbd, scales, N, K, T, x, y,
                             (int)((int64_t)N * i / nt), (int)((int64_t)N * (i + 1) / nt)};
        if (nt == 1)
            rc |= gemv_rows(&jobs[i]) != NULL;
        else if (pthread_create(&th[i], NULL, gemv_rows, &jobs[i]))
            return -3;
    }
    if (nt > 1)
        for (int i = 0; i < nt; i++) {
            void *ret;
            pthread_join(th[i], &ret);
            rc |= ret != NULL;
        }
    free(cbd);
    return rc ? -2 : 0;
}

int oracle_rvq_gemv(const uint8_t *sec, const uint16_t *scales, const uint16_t *cb,
                    int N, int K, const double *x, int T, double *y)
{
    if (N % 64 || K % 128 || T < 0)
        return -1;
    return rvq_gemv(sec, scales, cb, N, K, x, T, y);
}

/* ------------------------------------------------------------ expert FFN */

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* One routed expert on T tokens: g = W_g x, u = W_u x, h = SiLU(g) * u,
 * y = W_d h.  record: the expert's record bytes; x [T, H]; y [T, H]. */
int oracle_expert_ffn(const uint8_t *record, int H, int I, const double *x, int T, double *y)
{
    int64_t off[9], size[9], nb, pad;
    if (oracle_record_layout(H, I, off, size, &nb, &pad))
        return -1;
    if (T == 0)
        return 0;
    double *g = malloc(sizeof(double) * (int64_t)T * I);
    double *u = malloc(sizeof(double) * (int64_t)T * I);
    if (!g || !u) {
        free(g);
        free(u);
        return -2;
    }
    const uint16_t *sg = (const uint16_t *)(record + off[3]);
    const uint16_t *su = (const uint16_t *)(record + off[4]);
    const uint16_t *sd = (const uint16_t *)(record + off[5]);
    const uint16_t *cg = (const uint16_t *)(record + off[6]);
    const uint16_t *cu = (const uint16_t *)(record + off[7]);
    const uint16_t *cd = (const uint16_t *)(record + off[8]);
    int rc = rvq_gemv(record + off[0], sg, cg, I, H, x, T, g);
    if (!rc)
        rc = rvq_gemv(record + off[1], su, cu, I, H, x, T, u);
    if (!rc) {
        for (int64_t i = 0; i < (int64_t)T * I; i++)
            g[i] = silu(g[i]) * u[i];        /* h, stored in g */
        rc = rvq_gemv(record + off[2], sd, cd, H, I, g, T, y);
    }
    free(g);
    free(u);
    return rc;
}

/* Dense shared expert, bf16 weights: gate [I, H] | up [I, H] | down [H, I]. */
int oracle_shared_ffn(const uint16_t *w, int H, int I, const double *x, int T, double *y)
{
    const uint16_t *wg = w, *wu = w + (int64_t)I * H, *wd = w + 2 * (int64_t)I * H;
    double *h = malloc(sizeof(double) * I);
    if (!h)
        return -2;
    for (int t = 0; t < T; t++) {
        const double *xt = x + (int64_t)t * H;
        for (int r = 0; r < I; r++) {
            double gg = 0.0, uu = 0.0;
            for (int c = 0; c < H; c++) {
                gg += bf16_to_double(wg[(int64_t)r * H + c]) * xt[c];
                uu += bf16_to_double(wu[(int64_t)r * H + c]) * xt[c];
            }
            h[r] = silu(gg) * uu;
        }
        for (int r = 0; r < H; r++) {
            double acc = 0.0;
            for (int c = 0; c < I; c++)
                acc += bf16_to_double(wd[(int64_t)r * I + c]) * h[c];
            y[(int64_t)t * H + r] = acc;
        }
    }
    free(h);
    return 0;
}

/* --------------------------------------------------------------- routing */

typedef struct {
    double z;
    int e;
} zkey;

/* (z desc, expert id asc) */
static int zkey_cmp(const void *pa, const void *pb)
{
    const zkey *a = pa, *b = pb;
    if (a->z > b->z)
        return -1;
    if (a->z < b->z)
        return 1;
    return a->e - b->e;
}

/* Router for T tokens.  W [E, H] fp32, bias [E] fp32 or NULL, x [T, H].
 * score_fn 0 = softmax, 1 = sigmoid; weights renormalised over the selected
 * set.  Outputs idx [T, k] in selection order, w [T, k], and (if z != NULL)
 * the logits z [T, E]. */
int oracle_route(const float *W, const float *bias, int E, int H, const double *x,
                 int T, int k, int score_fn, int32_t *idx, double *w, double *z)
{
    if (k < 1 || k > E || (score_fn != 0 && score_fn != 1))
        return -1;
    zkey *keys = malloc(sizeof(zkey) * E);
    if (!keys)
        return -2;
    for (int t = 0; t < T; t++) {
        const double *xt = x + (int64_t)t * H;
        for (int e = 0; e < E; e++) {
            double acc = 0.0;
            for (int h = 0; h < H; h++)
                acc += (double)W[(int64_t)e * H + h] * xt[h];
            if (bias)
                acc += (double)bias[e];
            keys[e].z = acc;
            keys[e].e = e;
            if (z)
                z[(int64_t)t * E + e] = acc;
        }
        qsort(keys, E, sizeof(zkey), zkey_cmp);
        double sum = 0.0, zmax = keys[0].z;
        for (int j = 0; j < k; j++) {
            double s = score_fn == 0 ? exp(keys[j].z - zmax) : 1.0 / (1.0 + exp(-keys[j].z));
            w[(int64_t)t * k + j] = s;
            idx[(int64_t)t * k + j] = keys[j].e;
            sum += s;
        }
        for (int j = 0; j < k; j++)
            w[(int64_t)t * k + j] /= sum;
    }
    free(keys);
    return 0;
}

/* ----------------------------------------------------------------- layer */

/* One MoE layer on T tokens: route, run each selected expert, combine
 * out_t = sum_j w_{t,j} y_j(x_t) + shared(x_t).  records[E] are host
 * pointers to expert records; shared may be NULL.  idx/w/z outputs may be
 * NULL. */
int oracle_layer(const float *W, const float *bias, int E, int k, int score_fn,
                 const uint8_t *const *records, const uint16_t *shared,
                 int H, int I, const double *x, int T, double *out,
                 int32_t *idx_out, double *w_out)
{
    if (T == 0)
        return 0;
    int32_t *idx = malloc(sizeof(int32_t) * (int64_t)T * k);
    double *w = malloc(sizeof(double) * (int64_t)T * k);
    double *y = malloc(sizeof(double) * H);
    int rc = (!idx || !w || !y) ? -2 : 0;
    if (!rc)
        rc = oracle_route(W, bias, E, H, x, T, k, score_fn, idx, w, NULL);
    for (int t = 0; !rc && t < T; t++) {
        const double *xt = x + (int64_t)t * H;
        double *ot = out + (int64_t)t * H;
        for (int c = 0; c < H; c++)
            ot[c] = 0.0;
        for (int j = 0; !rc && j < k; j++) {
            rc = oracle_expert_ffn(records[idx[(int64_t)t * k + j]], H, I, xt, 1, y);
            for (int c = 0; c < H; c++)
                ot[c] += w[(int64_t)t * k + j] * y[c];
        }
        if (!rc && shared) {
            rc = oracle_shared_ffn(shared, H, I, xt, 1, y);
            for (int c = 0; c < H; c++)
                ot[c] += y[c];
        }
    }
    if (!rc && idx_out)
        memcpy(idx_out, idx, sizeof(int32_t) * (int64_t)T * k);
    if (!rc && w_out)
        memcpy(w_out, w, sizeof(double) * (int64_t)T * k);
    free(idx);
    free(w);
    free(y);
    return rc;
}

/* ------------------------------------------------------------- LRU cache */

/* Plain LRU over integer keys with `capacity` slots, simulated with a doubly
 * linked list (most recent at the head) and a linear search.  For each key:
 * hit[i] = 1 if present (moved to the head); on a miss the key goes to the
 * lowest-numbered free slot, else the tail key is evicted and its slot is
 * reused; the new key goes to the head.  slot[i] = slot holding the key after
 * the access; evicted[i] = evicted key or -1. */
int oracle_lru(const int64_t *keys, int64_t n, int capacity,
               int32_t *hit, int32_t *slot, int64_t *evicted)
{
    if (capacity < 1)
        return -1;
    int64_t *key_of = malloc(sizeof(int64_t) * capacity);
    int *prev = malloc(sizeof(int) * capacity), *next = malloc(sizeof(int) * capacity);
    if (!key_of || !prev || !next) {
        free(key_of);
        free(prev);
        free(next);
        return -2;
    }
    int head = -1, tail = -1, used = 0;
    for (int64_t i = 0; i < n; i++) {
        int found = -1;
        for (int s = head; s != -1; s = next[s])
            if (key_of[s] == keys[i]) {
                found = s;
                break;
            }
        evicted[i] = -1;
        if (found >= 0) {
            hit[i] = 1;
            /* unlink, then push at the head */
            if (prev[found] != -1)
                next[prev[found]] = next[found];
            else
                head = next[found];
            if (next[found] != -1)
                prev[next[found]] = prev[found];
            else
                tail = prev[found];
        } else {
            hit[i] = 0;
            if (used < capacity) {
                found = used++;
            } else {
                found = tail;
                evicted[i] = key_of[found];
                tail = prev[found];
                if (tail != -1)
                    next[tail] = -1;
                else
                    head = -1;
            }
            key_of[found] = keys[i];
        }
        prev[found] = -1;
        next[found] = head;
        if (head != -1)
            prev[head] = found;
        head = found;
        if (tail == -1)
            tail = found;
        slot[i] = found;
    }
    free(key_of);
    free(prev);
    free(next);
    return 0;
}

/* Cache trace of a streamed decode: idx [steps, k] holds the selected
 * experts of each (token, layer) step in decode order (token-major; the
 * layer of step s is layer0 + s % nlayers).  Each step's keys
 * layer * E + expert are looked up in ascending expert id.  Outputs, per
 * lookup: key, hit, slot, evicted key (-1 if none). */
int oracle_stream_trace(const int32_t *idx, int64_t steps, int nlayers, int layer0,
                        int E, int k, int capacity, int64_t *key, int32_t *hit,
                        int32_t *slot, int64_t *evicted)
{
    if (k < 1 || capacity < k || nlayers < 1)
        return -1;
    int32_t *sorted = malloc(sizeof(int32_t) * k);
    if (!sorted)
        return -2;
    for (int64_t s = 0; s < steps; s++) {
        memcpy(sorted, idx + s * k, sizeof(int32_t) * k);
        for (int a = 1; a < k; a++)          /* insertion sort, ascending */
            for (int b = a; b > 0 && sorted[b - 1] > sorted[b]; b--) {
                int32_t tmp = sorted[b];
                sorted[b] = sorted[b - 1];
                sorted[b - 1] = tmp;
            }
        int64_t layer = layer0 + s % nlayers;
        for (int j = 0; j < k; j++)
            key[s * k + j] = layer * E + sorted[j];
    }
    free(sorted);
    return oracle_lru(key, steps * k, capacity, hit, slot, evicted);
}

/* --------------------------------------------- two tiers, exclusive LRU */

/* One LRU level with explicit slots: key_of[s] (-1 free), recency order as
 * a doubly linked list (most recent at the head).  Used by the two-tier
 * model below; written out on its own so that a freed slot is visible. */
typedef struct {
    int cap;
    int64_t *key_of;
    int *prev, *next;
    int head, tail;
} level_t;

static int level_init(level_t *L, int cap)
{
    L->cap = cap;
    L->key_of = malloc(sizeof(int64_t) * (cap > 0 ? cap : 1));
    L->prev = malloc(sizeof(int) * (cap > 0 ? cap : 1));
    L->next = malloc(sizeof(int) * (cap > 0 ? cap : 1));
    L->head = L->tail = -1;
    if (!L->key_of || !L->prev || !L->next)
        return -2;
    for (int s = 0; s < cap; s++)
        L->key_of[s] = -1;
    return 0;
}

static void level_free(level_t *L)
{
    free(L->key_of);
    free(L->prev);
    free(L->next);
}

static int level_find(const level_t *L, int64_t key)
{
    for (int s = L->head; s != -1; s = L->next[s])
        if (L->key_of[s] == key)
            return s;
    return -1;
}

static void level_unlink(level_t *L, int s)
{
    if (L->prev[s] != -1)
        L->next[L->prev[s]] = L->next[s];
    else
        L->head = L->next[s];
    if (L->next[s] != -1)
        L->prev[L->next[s]] = L->prev[s];
    else
        L->tail = L->prev[s];
}

static void level_push_head(level_t *L, int s)
{
    L->prev[s] = -1;
    L->next[s] = L->head;
    if (L->head != -1)
        L->prev[L->head] = s;
    L->head = s;
    if (L->tail == -1)
        L->tail = s;
}

/* Put key at the head: the lowest free slot, else the tail key's slot (that
 * key is evicted: *evicted, else -1).  Returns the slot. */
static int level_insert(level_t *L, int64_t key, int64_t *evicted)
{
    int s = -1;
    *evicted = -1;
    for (int f = 0; f < L->cap; f++)
        if (L->key_of[f] == -1) {
            s = f;
            break;
        }
    if (s < 0) {
        s = L->tail;
        *evicted = L->key_of[s];
        level_unlink(L, s);
    }
    L->key_of[s] = key;
    level_push_head(L, s);
    return s;
}

/* Two exclusive LRU tiers: an upper tier of c1 slots (the HBM cache) and a
 * lower tier of c2 slots (host memory) in front of a backing store (the
 * file).  Each key is looked up in the upper tier; a hit moves it to the
 * upper tier's head.  On a miss the key is looked up in the lower tier: if
 * there, it leaves the lower tier (its slot becomes free) and its record is
 * the source of the copy, else the record comes from the backing store.  The
 * key is then inserted in the upper tier like oracle_lru (lowest free slot,
 * else the upper tier's least recently used key is evicted), and an evicted
 * key moves down: it is inserted at the lower tier's head (lowest free slot,
 * else the lower tier's least recently used key leaves both tiers).  WISP
 * "통찰" (each lookup goes to the fastest tier that holds the expert; LRU
 * promotes the experts in use) read as an exclusive hierarchy: a record is in
 * at most one tier, the upper tier's victims fill the lower one.
 * Per key i:
 *   hit1, slot1, ev1: the upper tier, as oracle_lru;
 *   hit2: -1 (no lower lookup: upper hit), 0 absent, 1 found there;
 *   slot2: the lower slot the key was found in, else -1;
 *   dslot, dev: the lower slot the upper tier's evicted key went to and the
 *   key that left the lower tier for it (-1 if none). */
int oracle_two_tier(const int64_t *keys, int64_t n, int c1, int c2,
                    int32_t *hit1, int32_t *slot1, int64_t *ev1,
                    int32_t *hit2, int32_t *slot2, int32_t *dslot, int64_t *dev)
{
    if (c1 < 1 || c2 < 1)
        return -1;
    level_t up, lo;
    int rc = level_init(&up, c1);
    if (!rc)
        rc = level_init(&lo, c2);
    if (rc) {
        level_free(&up);
        return rc;
    }
    for (int64_t i = 0; i < n; i++) {
        hit2[i] = -1;
        slot2[i] = -1;
        dslot[i] = -1;
        dev[i] = -1;
        ev1[i] = -1;
        int s = level_find(&up, keys[i]);
        if (s >= 0) {
            hit1[i] = 1;
            level_unlink(&up, s);
            level_push_head(&up, s);
            slot1[i] = s;
            continue;
        }
        hit1[i] = 0;
        int h = level_find(&lo, keys[i]);
        hit2[i] = h >= 0;
        if (h >= 0) {
            slot2[i] = h;
            level_unlink(&lo, h);
            lo.key_of[h] = -1;
        }
        slot1[i] = level_insert(&up, keys[i], &ev1[i]);
        if (ev1[i] != -1)
            dslot[i] = level_insert(&lo, ev1[i], &dev[i]);
    }
    level_free(&up);
    level_free(&lo);
    return 0;
}
