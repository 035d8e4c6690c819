/*
 * CPU oracle for the forward pass of one DeepSeekMoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * statement of what the layer computes.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load it.  It shares no source,
 * header, table or helper with the HIP library; the two meet only through the
 * seeded input tensors.
 *
 * Sources (the pages; each function cites the passage it follows):
 *   [IFS]      "DeepSeek-V3 Technical Report" notes, learn.ifs.name/d/deepseekv3
 *              -- paragraphs on MoE routing, bias balancing, FP8 tiling and
 *              FP8 accumulation.
 *   [LINEAGE]  "DeepSeek-V3" milestone summary, nlp-lineage.vercel.app --
 *              section "The idea" (load balancing, FP8 training bullets) and
 *              the paragraph "The notation" (the MoE output equation).
 * Readings where the pages are silent are marked READING and listed with the
 * design notes.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * OpenMP only splits independent outputs across threads; every individual
 * sum runs sequentially in the order written, so results do not depend on the
 * thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif


/* ------------------------------------------------------------------------ */
/* Scalar helpers                                                             */
/* ------------------------------------------------------------------------ */

static float bits_to_f32(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

/* bfloat16 is the upper half of an IEEE binary32. */
static float bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/*
 * READING (router sigmoid).  The pages give the affinity as a sigmoid of the
 * token-centroid product ([IFS] MoE paragraph) but no arithmetic.  Bit-exact
 * routing needs one exactly specified sigmoid, so both sides implement:
 *
 *   exp_spec(y): y < -87 -> 0;  y > 88.72 -> +inf;  otherwise
 *     n = rint(fl(y * L2E))                      (round half to even)
 *     r = fma(-n, LN2_HI, y);  r = fma(-n, LN2_LO, r)   (Cody-Waite reduction)
 *     p = Horner Taylor polynomial of degree 7 in r, coefficients fl32(1/k!),
 *         every step one fma
 *     return p * 2^n                              (exact scaling)
 *   sigmoid_spec(x) = 1 / (1 + exp_spec(-x))      (IEEE binary32 add, divide)
 *
 * Cody and Waite's argument reduction and the Taylor series of exp are
 * textbook methods; the constants below are the binary32 roundings of log2(e),
 * of ln 2 split into a 16-bit head and a tail, and of 1/k!.
 */
static const float SPEC_L2E = 0x1.715476p+0f;
static const float SPEC_LN2_HI = 0x1.62e400p-1f;
static const float SPEC_LN2_LO = 0x1.7f7d1cp-20f;
static const float SPEC_C[8] = {
    1.0f, 1.0f, 0x1.000000p-1f, 0x1.555556p-3f, 0x1.555556p-5f,
    0x1.111112p-7f, 0x1.6c16c2p-10f, 0x1.a01a02p-13f};

float oracle_exp_spec(float y) {
    if (y < -87.0f) return 0.0f;
    if (y > 88.72f) return INFINITY;
    float n = rintf(y * SPEC_L2E);
    float r = fmaf(-n, SPEC_LN2_HI, y);
    r = fmaf(-n, SPEC_LN2_LO, r);
    float p = SPEC_C[7];
    for (int k = 6; k >= 0; --k) p = fmaf(p, r, SPEC_C[k]);
    return ldexpf(p, (int)n);
}

float oracle_sigmoid_spec(float x) {
    float e = oracle_exp_spec(-x);
    float den = 1.0f + e;
    return 1.0f / den;
}

/* ------------------------------------------------------------------------ */
/* OCP OFP8 E4M3 codec ([IFS] FP8 paragraph: the format is "FP8"; READING:   */
/* the OCP E4M3 variant, bias 7, no infinities, max 448, NaN = S.1111.111)    */
/* ------------------------------------------------------------------------ */

/* Value of a code, straight from the format definition. */
double oracle_e4m3_decode(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);          /* subnormal: m/8 * 2^-6 */
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);        /* normal: (1+m/8) * 2^(e-7) */
    return s ? -v : v;
}

/*
 * Round to nearest, ties to the code with an even mantissa, saturating finite
 * overflow to +-448; NaN maps to 0x7F with its sign (READING).  Magnitude codes
 * 0x00..0x7E are in increasing order of value, so this searches for the pair of
 * neighbouring codes around |x| and picks the nearer.
 */
uint8_t oracle_e4m3_encode(float x) {
    uint8_t sign = (f32_to_bits(x) >> 31) ? 0x80 : 0x00;
    if (isnan(x)) return sign | 0x7F;
    double a = fabs((double)x);
    if (a >= 448.0) return sign | 0x7E;
    int lo = 0, hi = 0x7E;                 /* invariant: value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (oracle_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid;
    }
    double vlo = oracle_e4m3_decode((uint8_t)lo), vhi = oracle_e4m3_decode((uint8_t)hi);
    int pick;
    if (a - vlo < vhi - a) pick = lo;
    else if (a - vlo > vhi - a) pick = hi;
    else pick = (lo % 2 == 0) ? lo : hi;   /* tie: even mantissa bit */
    return sign | (uint8_t)pick;
}

/* Element-wise versions, so tests can sweep millions of inputs. */
void oracle_sigmoid_spec_n(const float* x, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_sigmoid_spec(x[i]);
}

void oracle_exp_spec_n(const float* x, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_exp_spec(x[i]);
}

void oracle_e4m3_encode_n(const float* x, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i]);
}

/* ------------------------------------------------------------------------ */
/* A1: router affinity  s[t,i] = sigmoid(u_t . e_i)                          */
/* [IFS] MoE-routing paragraph: s = sigmoid of the token-centroid product;   */
/* [LINEAGE] "The notation" (score s_(i,t)).                                 */
/* READING: bf16 inputs; FP32 sum in increasing k, one fma per term (every   */
/* bf16*bf16 product is exact in FP32); no temperature, no 1/sqrt(d).        */
/* ------------------------------------------------------------------------ */
void oracle_router_scores(const uint16_t* u, const uint16_t* e, int64_t T, int d, int E,
                          float* s /* [T,E] */) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int i = 0; i < E; ++i) {
            float acc = 0.0f;
            for (int k = 0; k < d; ++k)
                acc = fmaf(bf16_to_f32(u[t * d + k]), bf16_to_f32(e[(int64_t)i * d + k]), acc);
            s[t * E + i] = oracle_sigmoid_spec(acc);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* A2: biased top-K selection and gate normalisation                         */
/* [IFS] bias paragraph: b_i shifts expert i's rank, not its gate.  [IFS]    */
/* MoE-routing paragraph: g = s / (sum of s over the chosen set).            */
/* [LINEAGE] "The notation": chosen iff s+b is among the top K; g uses s.    */
/* READING: key = fl32(s + b) with -0 -> +0 and NaN -> -inf; rank experts by */
/* (key descending, index ascending) and the first K are slots 0..K-1;       */
/* D = FP32 sum of the chosen raw s in slot order; g = fl32(s / D); if D = 0 */
/* every gate is 0.                                                          */
/* ------------------------------------------------------------------------ */
typedef struct { float key; int idx; } ranked_t;

static int cmp_ranked(const void* pa, const void* pb) {
    const ranked_t* a = (const ranked_t*)pa;
    const ranked_t* b = (const ranked_t*)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    return (a->idx > b->idx) - (a->idx < b->idx);
}

static float canonical_key(float v) {
    if (isnan(v)) return -INFINITY;
    if (v == 0.0f) return 0.0f;
    return v;
}

void oracle_topk_from_scores(const float* s, const float* bias, int64_t T, int E, int K,
                             int32_t* idx, float* gate) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        ranked_t* r = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)E);
        for (int i = 0; i < E; ++i) {
            r[i].key = canonical_key(s[t * E + i] + bias[i]);
            r[i].idx = i;
        }
        qsort(r, (size_t)E, sizeof(ranked_t), cmp_ranked);
        float D = 0.0f;
        for (int k = 0; k < K; ++k) D = D + s[t * E + r[k].idx];
        for (int k = 0; k < K; ++k) {
            idx[t * K + k] = r[k].idx;
            gate[t * K + k] = (D == 0.0f) ? 0.0f : s[t * E + r[k].idx] / D;
        }
        free(r);
    }
}

/* ------------------------------------------------------------------------ */
/* A2, group-limited variant.  [IFS] MoE-routing paragraph: each token is    */
/* sent to at most 4 nodes.  The pages give no rule for picking the nodes.   */
/* READING: the E experts form n_groups groups of E/n_groups consecutive     */
/* indices; a group's score is the largest key (as above) of its experts;    */
/* the topk_groups groups ranked first by (score descending, group index     */
/* ascending) are kept; the K experts are the first K of the kept groups'    */
/* experts ranked by (key descending, index ascending).  Gates as above.     */
/* ------------------------------------------------------------------------ */
void oracle_topk_grouped_from_scores(const float* s, const float* bias, int64_t T, int E, int K,
                                     int n_groups, int topk_groups, int32_t* idx, float* gate) {
    const int gs = E / n_groups;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        float* key = (float*)malloc(sizeof(float) * (size_t)E);
        ranked_t* grp = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)n_groups);
        ranked_t* r = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)E);
        for (int i = 0; i < E; ++i) key[i] = canonical_key(s[t * E + i] + bias[i]);
        for (int g = 0; g < n_groups; ++g) {
            float best = key[g * gs];
            for (int i = g * gs + 1; i < (g + 1) * gs; ++i)
                if (key[i] > best) best = key[i];
            grp[g].key = best;
            grp[g].idx = g;
        }
        qsort(grp, (size_t)n_groups, sizeof(ranked_t), cmp_ranked);
        int n = 0;
        for (int q = 0; q < topk_groups; ++q)
            for (int i = grp[q].idx * gs; i < (grp[q].idx + 1) * gs; ++i) {
                r[n].key = key[i];
                r[n].idx = i;
                ++n;
            }
        qsort(r, (size_t)n, sizeof(ranked_t), cmp_ranked);
        float D = 0.0f;
        for (int k = 0; k < K; ++k) D = D + s[t * E + r[k].idx];
        for (int k = 0; k < K; ++k) {
            idx[t * K + k] = r[k].idx;
            gate[t * K + k] = (D == 0.0f) ? 0.0f : s[t * E + r[k].idx] / D;
        }
        free(key);
        free(grp);
        free(r);
    }
}

/* ------------------------------------------------------------------------ */
/* Sequence-wise balance loss.  [IFS] bias paragraph: a tiny sequence-wise   */
/* loss remains against extreme imbalance.  No formula on the pages.         */
/* READING, per sequence q of L tokens [qL, qL+L):                           */
/*   f_i = E/(K L) * #{t in q : i among idx[t, 0..K-1]}                      */
/*   P_i = (1/L) sum_t s[t,i] / sum_j s[t,j]  (a row summing to 0 adds 0)    */
/*   loss[q] = alpha * sum_i f_i P_i, all in FP64.                           */
/* ------------------------------------------------------------------------ */
void oracle_seq_balance_loss(const float* s, const int32_t* idx, int64_t T, int E, int K, int L,
                             double alpha, double* loss) {
    const int64_t nseq = T / L;
    for (int64_t q = 0; q < nseq; ++q) {
        double* P = (double*)calloc((size_t)E, sizeof(double));
        double* f = (double*)calloc((size_t)E, sizeof(double));
        for (int64_t t = q * L; t < (q + 1) * L; ++t) {
            double rs = 0.0;
            for (int j = 0; j < E; ++j) rs += (double)s[t * E + j];
            if (rs != 0.0)
                for (int i = 0; i < E; ++i) P[i] += (double)s[t * E + i] / rs;
            for (int k = 0; k < K; ++k) {
                const int e = idx[t * K + k];
                if (e >= 0 && e < E) f[e] += 1.0;
            }
        }
        double sum = 0.0;
        for (int i = 0; i < E; ++i)
            sum += ((double)E / ((double)K * L) * f[i]) * (P[i] / L);
        loss[q] = alpha * sum;
        free(P);
        free(f);
    }
}

/* ------------------------------------------------------------------------ */
/* A3: dispatch.  Every (token, slot) assignment becomes one GEMM row; no     */
/* token is dropped ([LINEAGE] "The idea", load-balancing bullet).  READING: */
/* rows sorted by (expert, token); the shared expert's T rows follow the     */
/* routed rows in token order.                                               */
/*   count[e]        number of assignments to expert e                       */
/*   group_offset    exclusive scan of count, then T*K, then T*K+T if shared */
/*   row_token[r]    token of row r                                          */
/*   slot_row[t,k]   row that holds assignment (t, k)                        */
/* ------------------------------------------------------------------------ */
typedef struct { int32_t expert, token, slot; } assign_t;

static int cmp_assign(const void* pa, const void* pb) {
    const assign_t* a = (const assign_t*)pa;
    const assign_t* b = (const assign_t*)pb;
    if (a->expert != b->expert) return (a->expert > b->expert) - (a->expert < b->expert);
    return (a->token > b->token) - (a->token < b->token);
}

int oracle_dispatch(const int32_t* idx, int64_t T, int K, int E, int include_shared,
                    int32_t* count, int32_t* group_offset, int32_t* row_token, int32_t* slot_row) {
    int64_t n = T * K;
    for (int e = 0; e < E; ++e) count[e] = 0;
    for (int64_t j = 0; j < n; ++j) {
        if (idx[j] < 0 || idx[j] >= E) return -1;
        count[idx[j]]++;
    }
    int32_t run = 0;
    for (int e = 0; e < E; ++e) { group_offset[e] = run; run += count[e]; }
    group_offset[E] = run;
    if (include_shared) group_offset[E + 1] = run + (int32_t)T;

    assign_t* a = (assign_t*)malloc(sizeof(assign_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            a[t * K + k].expert = idx[t * K + k];
            a[t * K + k].token = (int32_t)t;
            a[t * K + k].slot = k;
        }
    qsort(a, (size_t)n, sizeof(assign_t), cmp_assign);
    for (int64_t r = 0; r < n; ++r) {
        row_token[r] = a[r].token;
        slot_row[(int64_t)a[r].token * K + a[r].slot] = (int32_t)r;
    }
    if (include_shared)
        for (int64_t t = 0; t < T; ++t) row_token[n + t] = (int32_t)t;
    free(a);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* A4/A5: block quantisation to E4M3 ([IFS] FP8 paragraph: activations per   */
/* 1x128 tile, weights per 128x128 block).  READING of the scale rule:       */
/*   amax = max |x| over the tile;                                           */
/*   if amax == 0 or 448/amax is not finite: scale = inv = 1                 */
/*   else inv = fl32(448/amax), scale = fl32(amax/448)                       */
/*   q = encode(fl32(x * inv));  the stored dequantisation factor is scale.  */
/* x is FP32 (bf16 inputs are widened exactly by the caller).                */
/* ------------------------------------------------------------------------ */
static void tile_scale(float amax, float* inv, float* scale) {
    float iv = 448.0f / amax;
    if (amax == 0.0f || !isfinite(iv)) { *inv = 1.0f; *scale = 1.0f; return; }
    *inv = iv;
    *scale = amax / 448.0f;
}

/* 1 x tile quantisation along rows: each row is cut into cols/128 tiles. */
void oracle_quant_1x128(const float* x, int64_t rows, int cols, uint8_t* q, float* scale) {
    int nt = cols / 128;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int j = 0; j < nt; ++j) {
            const float* p = x + r * cols + (int64_t)j * 128;
            float amax = 0.0f;
            for (int c = 0; c < 128; ++c) { float a = fabsf(p[c]); if (a > amax) amax = a; }
            float inv, sc;
            tile_scale(amax, &inv, &sc);
            for (int c = 0; c < 128; ++c) q[r * cols + (int64_t)j * 128 + c] = oracle_e4m3_encode(p[c] * inv);
            scale[r * nt + j] = sc;
        }
    }
}

/* 128 x 128 block quantisation of a [rows, cols] matrix; scale is [rows/128, cols/128]. */
void oracle_quant_128x128(const float* w, int64_t rows, int cols, uint8_t* q, float* scale) {
    int64_t nbr = rows / 128;
    int nbc = cols / 128;
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t br = 0; br < nbr; ++br) {
        for (int bc = 0; bc < nbc; ++bc) {
            float amax = 0.0f;
            for (int i = 0; i < 128; ++i)
                for (int c = 0; c < 128; ++c) {
                    float a = fabsf(w[(br * 128 + i) * cols + bc * 128 + c]);
                    if (a > amax) amax = a;
                }
            float inv, sc;
            tile_scale(amax, &inv, &sc);
            for (int i = 0; i < 128; ++i)
                for (int c = 0; c < 128; ++c) {
                    int64_t o = (br * 128 + i) * cols + bc * 128 + c;
                    q[o] = oracle_e4m3_encode(w[o] * inv);
                }
            scale[br * nbc + bc] = sc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* A6/A7/A10: block-scaled FP8 GEMM.  [IFS] FP8-accumulation paragraph:      */
/* every 128 elements of the inner dimension the partial sum is promoted to  */
/* full precision and the per-group scaling factors are applied there.       */
/*   C[m,n] = sum_j sa[m,j] * sb[n/128, j] * sum_{k in slice j} qa[m,k]qb[n,k] */
/* Here every slice sum and the outer sum are taken in FP64; each slice sum  */
/* of 128 E4M3 products is exact in FP64, so C is the value of the           */
/* dequantised operands up to one FP64 rounding per slice.                   */
/* A rows may be gathered: row m of the GEMM reads A row a_rows[m] (or m).   */
/* ------------------------------------------------------------------------ */
void oracle_gemm_blockscaled(const uint8_t* qa, const float* sa, const int32_t* a_rows, int64_t M,
                             const uint8_t* qb, const float* sb, int N, int K, double* out) {
    int ns = K / 128;
    double lut[256];
    for (int c = 0; c < 256; ++c) lut[c] = oracle_e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        int64_t am = a_rows ? a_rows[m] : m;
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int j = 0; j < ns; ++j) {
                double part = 0.0;
                for (int k = j * 128; k < j * 128 + 128; ++k)
                    part += lut[qa[am * K + k]] * lut[qb[(int64_t)n * K + k]];
                acc += (double)sa[am * ns + j] * (double)sb[(int64_t)(n / 128) * ns + j] * part;
            }
            out[m * N + n] = acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Expert FFN nonlinearity.  The pages write only FFN_i ([LINEAGE] "The      */
/* notation").  READING: SwiGLU, FFN(x) = W2 (SiLU(W1 x) * (W3 x)),          */
/* SiLU(z) = z * sigmoid(z), no bias terms.  FP64 throughout.                */
/* ------------------------------------------------------------------------ */
void oracle_swiglu(const double* zg, const double* zu, int64_t n, double* h) {
    for (int64_t i = 0; i < n; ++i) h[i] = zg[i] / (1.0 + exp(-zg[i])) * zu[i];
}

/* ------------------------------------------------------------------------ */
/* A8: combine.  [LINEAGE] "The notation":                                    */
/*   h'_t = u_t + sum_shared FFN_i(u_t) + sum_routed g_(i,t) FFN_i(u_t)      */
/* y holds one FFN output row per GEMM row; shared_row0 < 0 means no shared  */
/* term.  FP64 sums.                                                         */
/* ------------------------------------------------------------------------ */
void oracle_combine(const uint16_t* u, const double* y, int64_t shared_row0, const float* gate,
                    const int32_t* slot_row, int64_t T, int K, int d, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int c = 0; c < d; ++c) {
            double v = (double)bf16_to_f32(u[t * d + c]);
            if (shared_row0 >= 0) v += y[(shared_row0 + t) * d + c];
            for (int k = 0; k < K; ++k) v += (double)gate[t * K + k] * y[(int64_t)slot_row[t * K + k] * d + c];
            out[t * d + c] = v;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* A9: bias update.  [IFS] bias paragraph and [LINEAGE] "The idea": the    */
/* sign rule of the balancing bias, applied once per step.  READING:         */
/* count*E > T*K -> b - gamma; count*E < T*K -> b + gamma; equality (an     */
/* expert exactly at the batch mean) keeps b.  FP32 add.                     */
/* ------------------------------------------------------------------------ */
void oracle_bias_update(float* bias, const int32_t* count, int E, int64_t total_assignments, float gamma) {
    for (int e = 0; e < E; ++e) {
        int64_t lhs = (int64_t)count[e] * E;
        if (lhs > total_assignments) bias[e] = bias[e] - gamma;
        else if (lhs < total_assignments) bias[e] = bias[e] + gamma;
    }
}

/* ------------------------------------------------------------------------ */
/* Thread count of the OpenMP loops above (timing only: every output's       */
/* reduction is sequential, so the count never changes a result).            */
/* ------------------------------------------------------------------------ */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
