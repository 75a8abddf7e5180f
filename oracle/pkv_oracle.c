/*
 * pkv_oracle.c - plain CPU oracle for paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include,
 * link or call this file; only the tests, the package smoke check and the
 * CPU-baseline leg of the benchmark use it.  It shares no code, header,
 * table or constant with the HIP library.
 *
 * Sources (cited by page title and section):
 *   [P4] "vLLM 推理引擎源码级拆解：PagedAttention 显存虚拟化、Continuous
 *        Batching 调度与量化落地全指南" (chenxutan.com/d/5333)
 *   [P2] "vLLM 深度实战" (chenxutan.com/d/3332)
 *   [P3] "vLLM 深度剖析：PagedAttention 与连续批处理如何撑起大模型推理"
 *        (pgsm.cn/news/372185)
 *   [P1] "vLLM 0.5 深度拆解" (chenxutan.com/d/4924)
 *
 * What it computes.  Paging changes only where K/V live: a sequence is
 * logically contiguous while its blocks sit anywhere in a shared pool, found
 * through a per-sequence block table ([P4] §2.1-2.2).  The result of paged
 * decode is therefore exactly single-query softmax attention over the
 * gathered, logically ordered K/V; the online (running max / running sum)
 * softmax of the [P4] §2.3 kernel sketch is an evaluation order of that same
 * function.  So this oracle writes out the plain definition:
 *   1. gather K/V of one sequence and one KV head into contiguous arrays via
 *      the block table (address translation of [P4] §2.3),
 *   2. scores z_t = scale * <q, k_t>,
 *   3. textbook two-pass softmax (max, exp, sum),
 *   4. out = sum_t p_t v_t / sum_t p_t.
 * All arithmetic after the exact widening of the stored values is IEEE
 * double; build without -ffast-math.
 *
 * Readings taken where the pages are silent (all listed in the design notes):
 *   - element (b, o, h, d) of either cache sits at ((b*bs + o)*Hkv + h)*D + d;
 *     the [P4] §2.3 sketch omits the head term but declares the
 *     [num_blocks, block_size, num_heads, head_dim] layout.
 *   - GQA ([P4] §2.3 names it only): query head hq reads KV head hq / G,
 *     G = Hq / Hkv.
 *   - tokens t >= L never contribute, whatever the memory holds.
 *   - L <= 0 gives an all-zero output row.
 *   - FP8 KV ([P1] §4.2, [P3] §6.1, [P4] §6.4 give only the flag): OCP
 *     E4M3 with one scale per tensor, element = decode(code) * scale; codes
 *     are written as e4m3(x / scale), the division in fp32, round to nearest
 *     even, saturating at +-448.
 *   - split-K partials (not on the pages): per partition of P tokens,
 *     m_p = max z, l_p = sum exp(z - m_p), o_p = sum exp(z - m_p) v (not
 *     normalised), merged by out = sum e^(m_p-M) o_p / sum e^(m_p-M) l_p.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Storage type codes used by this oracle's own API. */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_E4M3 = 3 };

/* Error codes of this oracle's own API. */
enum { ORC_OK = 0, ORC_EARG = -1, ORC_EBLOCK = -2, ORC_ENOMEM = -3 };

static int orc_elem_bytes(int dt)
{
    switch (dt) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    case ORC_E4M3: return 1;
    default: return 0;
    }
}

/* ---------------------------------------------------------------------- */
/* Scalar format conversions, each written from its format definition.    */
/* ---------------------------------------------------------------------- */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double orc_bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = (m == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + m), e - 25);  /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* OCP FP8 E4M3: 1 sign, 4 exponent (bias 7), 3 fraction bits, no infinity,
 * S.1111.111 is NaN, largest finite 448, smallest subnormal 2^-9. */
double orc_e4m3_decode(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 15;
    int m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);               /* m/8 * 2^-6 */
    else
        v = ldexp((double)(8 + m), e - 10);     /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* Round-half-to-even of a non-negative double that holds an exact value. */
static double orc_rne(double q)
{
    double n = floor(q);
    double frac = q - n;
    if (frac > 0.5)
        return n + 1.0;
    if (frac < 0.5)
        return n;
    return (fmod(n, 2.0) == 0.0) ? n : n + 1.0;
}

/* fp32 -> OCP E4M3, round to nearest even, saturate finite overflow to
 * +-448, NaN -> S.1111.111.  Works on the exact value in double: a binary32
 * divided by a power of two is exact in binary64. */
uint8_t orc_e4m3_encode(float x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (isnan(x))
        return (uint8_t)(sign | 0x7F);
    if (isinf(x))
        return (uint8_t)(sign | 0x7E);     /* overflow saturates */
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: multiples of 2^-9; 8 * 2^-9 is the smallest
         * normal, whose code happens to be 8 as well. */
        double n = orc_rne(a * 512.0);
        return (uint8_t)(sign | (uint8_t)n);
    }
    int ex;
    (void)frexp(a, &ex);       /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;            /* a in [2^e, 2^(e+1)) */
    if (e > 8)
        return (uint8_t)(sign | 0x7E);
    double q = ldexp(a, 3 - e); /* in [8, 16): 3 fraction bits above the point */
    double n = orc_rne(q);
    if (n == 16.0) {
        n = 8.0;
        e += 1;
    }
    int biased = e + 7;
    int mant = (int)n - 8;
    if (biased > 15 || (biased == 15 && mant == 7))
        return (uint8_t)(sign | 0x7E);     /* above 448: saturate */
    return (uint8_t)(sign | (uint8_t)(biased << 3) | (uint8_t)mant);
}

/* Widen stored element i of a non-fp8 array to double (exact). */
static double orc_load(const void* base, size_t i, int dt)
{
    switch (dt) {
    case ORC_F32: return (double)((const float*)base)[i];
    case ORC_F16: return orc_f16_to_double(((const uint16_t*)base)[i]);
    case ORC_BF16: return orc_bf16_to_double(((const uint16_t*)base)[i]);
    default: return NAN;
    }
}

/* Stored value as the fp32 number the writer divides by the scale. */
static float orc_load_f32(const void* base, size_t i, int dt)
{
    return (float)orc_load(base, i, dt);   /* exact: f16/bf16/f32 fit fp32 */
}

/* Vectorised helpers for the Python side. */
void orc_e4m3_encode_array(const float* x, uint8_t* out, size_t n)
{
    for (size_t i = 0; i < n; i++)
        out[i] = orc_e4m3_encode(x[i]);
}

void orc_e4m3_decode_array(const uint8_t* c, double* out, size_t n)
{
    for (size_t i = 0; i < n; i++)
        out[i] = orc_e4m3_decode(c[i]);
}

void orc_widen_array(const void* x, int dt, double* out, size_t n)
{
    for (size_t i = 0; i < n; i++)
        out[i] = (dt == ORC_E4M3) ? orc_e4m3_decode(((const uint8_t*)x)[i])
                                  : orc_load(x, i, dt);
}

/* ---------------------------------------------------------------------- */
/* Cache writer: the append step.                                          */
/* ---------------------------------------------------------------------- */

/* For every new token i with slot_mapping[i] >= 0, slot = phys_block*bs +
 * offset ([P4] §2.2: a new token goes to the next free slot of the last block
 * or of a freshly appended block; the slot number itself is the caller's).
 * Writes key[i][h][:] and value[i][h][:] into cache[slot/bs][slot%bs][h][:].
 * Same storage type: a bit copy.  fp8 cache: e4m3(x / scale) with an fp32
 * divide.  Slots >= NB*bs are skipped like negative ones. */
int orc_reshape_and_cache(const void* key, const void* value, int src_dt,
                          void* k_cache, void* v_cache, int cache_dt,
                          const int64_t* slot_mapping, int T, int Hkv, int D,
                          int bs, int NB, float k_scale, float v_scale)
{
    if (!key || !value || !k_cache || !v_cache || !slot_mapping)
        return ORC_EARG;
    if (T < 0 || Hkv <= 0 || D <= 0 || bs <= 0 || NB <= 0)
        return ORC_EARG;
    int se = orc_elem_bytes(src_dt), ce = orc_elem_bytes(cache_dt);
    if (!se || !ce || src_dt == ORC_E4M3)
        return ORC_EARG;
    if (cache_dt != ORC_E4M3 && cache_dt != src_dt)
        return ORC_EARG;
    size_t row = (size_t)Hkv * D;               /* elements per token */
    int64_t nslots = (int64_t)NB * bs;
    for (int i = 0; i < T; i++) {
        int64_t slot = slot_mapping[i];
        if (slot < 0 || slot >= nslots)
            continue;
        int64_t b = slot / bs, o = slot % bs;
        size_t dst0 = ((size_t)b * bs + (size_t)o) * row;
        size_t src0 = (size_t)i * row;
        if (cache_dt == src_dt) {
            memcpy((char*)k_cache + dst0 * ce, (const char*)key + src0 * se, row * se);
            memcpy((char*)v_cache + dst0 * ce, (const char*)value + src0 * se, row * se);
        } else {
            uint8_t* kc = (uint8_t*)k_cache;
            uint8_t* vc = (uint8_t*)v_cache;
            for (size_t j = 0; j < row; j++) {
                float xk = orc_load_f32(key, src0 + j, src_dt);
                float xv = orc_load_f32(value, src0 + j, src_dt);
                volatile float qk = xk / k_scale;   /* one fp32 IEEE divide */
                volatile float qv = xv / v_scale;
                kc[dst0 + j] = orc_e4m3_encode(qk);
                vc[dst0 + j] = orc_e4m3_encode(qv);
            }
        }
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------- */
/* Decode attention.                                                       */
/* ---------------------------------------------------------------------- */

typedef struct {
    const void* query; int q_dt;
    const void* k_cache; const void* v_cache; int cache_dt;
    const int32_t* block_tables; int max_blocks;
    const int32_t* seq_lens;
    int S, Hq, Hkv, D, bs, NB;
    double scale, k_scale, v_scale;
    /* Mixed block sizes: tokens per block of each sequence, or NULL when
     * every block has bs tokens.  With it, bs and NB count pages. */
    const int32_t* seq_bs;
} orc_problem;

/* Stored cache element as a real number: exact widening, or the fp8 code's
 * value times its per-tensor scale. */
static double orc_cache_value(const orc_problem* p, const void* cache,
                              size_t i, double fp8_scale)
{
    if (p->cache_dt == ORC_E4M3)
        return orc_e4m3_decode(((const uint8_t*)cache)[i]) * fp8_scale;
    return orc_load(cache, i, p->cache_dt);
}

/* Step 1: gather tokens [t0, t1) of sequence s, KV head h, into K, V
 * ([t1-t0][D], row-major) through the block table ([P4] §2.2-2.3:
 * logical block t/bs, offset t%bs, physical block from the table).
 * Mixed block sizes ([P1] §1.3): sequence s has blocks of bs_s tokens, each
 * bs_s/bs consecutive pages of bs tokens from the page the table names, so
 * token t is row (entry * bs + t % bs_s) of the pool. */
static int orc_gather(const orc_problem* p, int s, int h, int t0, int t1,
                      double* K, double* V)
{
    int bs_s = p->seq_bs ? p->seq_bs[s] : p->bs;
    if (bs_s < p->bs || bs_s % p->bs != 0)
        return ORC_EARG;
    for (int t = t0; t < t1; t++) {
        int logical = t / bs_s;
        int offset = t % bs_s;
        if (logical >= p->max_blocks)
            return ORC_EBLOCK;
        int32_t b = p->block_tables[(size_t)s * p->max_blocks + logical];
        if (b < 0 || (int64_t)b + bs_s / p->bs > p->NB)
            return ORC_EBLOCK;
        size_t base = (((size_t)b * p->bs + (size_t)offset) * p->Hkv + (size_t)h) * p->D;
        for (int d = 0; d < p->D; d++) {
            K[(size_t)(t - t0) * p->D + d] = orc_cache_value(p, p->k_cache, base + d, p->k_scale);
            V[(size_t)(t - t0) * p->D + d] = orc_cache_value(p, p->v_cache, base + d, p->v_scale);
        }
    }
    return ORC_OK;
}

/* Step 2: z_t = scale * sum_d q[d] K[t][d], d ascending. */
static void orc_scores(const orc_problem* p, const double* q, const double* K,
                       int n, double* z)
{
    for (int t = 0; t < n; t++) {
        double acc = 0.0;
        for (int d = 0; d < p->D; d++)
            acc += q[d] * K[(size_t)t * p->D + d];
        z[t] = p->scale * acc;
    }
}

static void orc_query_row(const orc_problem* p, int s, int hq, double* q)
{
    size_t base = ((size_t)s * p->Hq + hq) * p->D;
    for (int d = 0; d < p->D; d++)
        q[d] = orc_load(p->query, base + d, p->q_dt);
}

static int orc_check(const orc_problem* p)
{
    if (!p->query || !p->k_cache || !p->v_cache || !p->block_tables || !p->seq_lens)
        return ORC_EARG;
    if (p->S <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->D <= 0 || p->bs <= 0 ||
        p->NB <= 0 || p->max_blocks <= 0)
        return ORC_EARG;
    if (p->Hq % p->Hkv != 0)
        return ORC_EARG;
    if (!orc_elem_bytes(p->cache_dt) || !orc_elem_bytes(p->q_dt) || p->q_dt == ORC_E4M3)
        return ORC_EARG;
    return ORC_OK;
}

/* One output row out[D]: query vector q[D] of a head reading KV head h of
 * sequence s, attending to tokens [0, n) of the sequence -- steps 1-4 of
 * the definition.  n <= 0 gives a zero row. */
static int orc_attend_row(const orc_problem* p, int s, int h, const double* q, int n,
                          double* out)
{
    if (n <= 0) {
        for (int d = 0; d < p->D; d++)
            out[d] = 0.0;
        return ORC_OK;
    }
    double* K = (double*)malloc(sizeof(double) * (size_t)n * p->D);
    double* V = (double*)malloc(sizeof(double) * (size_t)n * p->D);
    double* z = (double*)malloc(sizeof(double) * (size_t)n);
    int rc = ORC_OK;
    if (!K || !V || !z) {
        rc = ORC_ENOMEM;
        goto done;
    }
    rc = orc_gather(p, s, h, 0, n, K, V);
    if (rc != ORC_OK)
        goto done;
    orc_scores(p, q, K, n, z);
    /* Step 3: softmax, two passes. */
    double m = -INFINITY;
    for (int t = 0; t < n; t++)
        if (z[t] > m)
            m = z[t];
    double l = 0.0;
    for (int t = 0; t < n; t++) {
        z[t] = exp(z[t] - m);
        l += z[t];
    }
    /* Step 4: weighted sum of V rows, normalised. */
    for (int d = 0; d < p->D; d++) {
        double acc = 0.0;
        for (int t = 0; t < n; t++)
            acc += z[t] * V[(size_t)t * p->D + d];
        out[d] = acc / l;
    }
done:
    free(K);
    free(V);
    free(z);
    return rc;
}

/* Decode row (s, hq): the sequence's query against all its L tokens. */
static int orc_decode_row(const orc_problem* p, int s, int hq, double* out)
{
    int G = p->Hq / p->Hkv;
    double* q = (double*)malloc(sizeof(double) * p->D);
    if (!q)
        return ORC_ENOMEM;
    orc_query_row(p, s, hq, q);
    int rc = orc_attend_row(p, s, hq / G, q, p->seq_lens[s], out);
    free(q);
    return rc;
}

/* out[S][Hq][D] (double).  rows: optional list of n_rows flat indices
 * s*Hq + hq to compute (others untouched); NULL computes every row.
 * nthreads <= 0 uses the OpenMP default. */
static int orc_decode_rows(const orc_problem* pp, double* out, const int32_t* rows,
                           int n_rows, int nthreads)
{
    const orc_problem p = *pp;
    const int S = p.S, Hq = p.Hq, D = p.D;
    int rc = orc_check(&p);
    if (rc != ORC_OK || !out)
        return rc != ORC_OK ? rc : ORC_EARG;
    int n = rows ? n_rows : S * Hq;
    int err = ORC_OK;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int i = 0; i < n; i++) {
        int r = rows ? rows[i] : i;
        if (r < 0 || r >= S * Hq) {
            err = ORC_EARG;
            continue;
        }
        int e = orc_decode_row(&p, r / Hq, r % Hq, out + (size_t)r * D);
        if (e != ORC_OK)
            err = e;
    }
    (void)nthreads;
    return err;
}

int orc_paged_decode(double* out, const void* query, int q_dt,
                     const void* k_cache, const void* v_cache, int cache_dt,
                     const int32_t* block_tables, int max_blocks,
                     const int32_t* seq_lens, int S, int Hq, int Hkv, int D,
                     int bs, int NB, double scale, double k_scale,
                     double v_scale, const int32_t* rows, int n_rows,
                     int nthreads)
{
    orc_problem p = {query, q_dt, k_cache, v_cache, cache_dt, block_tables,
                     max_blocks, seq_lens, S, Hq, Hkv, D, bs, NB, scale,
                     k_scale, v_scale, NULL};
    return orc_decode_rows(&p, out, rows, n_rows, nthreads);
}

/* Decode over a pool of NP pages of `page` tokens whose sequences have
 * blocks of seq_bs[s] tokens (multiples of page; see orc_gather). */
int orc_paged_decode_mixed(double* out, const void* query, int q_dt,
                           const void* k_cache, const void* v_cache, int cache_dt,
                           const int32_t* block_tables, int max_blocks,
                           const int32_t* seq_lens, const int32_t* seq_bs, int S, int Hq,
                           int Hkv, int D, int page, int NP, double scale, double k_scale,
                           double v_scale, const int32_t* rows, int n_rows, int nthreads)
{
    if (!seq_bs)
        return ORC_EARG;
    orc_problem p = {query, q_dt, k_cache, v_cache, cache_dt, block_tables,
                     max_blocks, seq_lens, S, Hq, Hkv, D, page, NP, scale,
                     k_scale, v_scale, seq_bs};
    return orc_decode_rows(&p, out, rows, n_rows, nthreads);
}

/* Split-K partials for partition size P (> 0): for each (s, hq) and each
 * partition k < ceil(L/P) covering tokens [kP, min(L, (k+1)P)):
 *   m[s][hq][k] = max z,  l[s][hq][k] = sum exp(z - m),
 *   o[s][hq][k][:] = sum exp(z - m) v  (not normalised).
 * Arrays are [S][Hq][P_max] and [S][Hq][P_max][D]; entries with
 * k >= ceil(L/P) are left untouched. */
int orc_paged_partials(double* m_out, double* l_out, double* o_out,
                       const void* query, int q_dt, const void* k_cache,
                       const void* v_cache, int cache_dt,
                       const int32_t* block_tables, int max_blocks,
                       const int32_t* seq_lens, int S, int Hq, int Hkv, int D,
                       int bs, int NB, double scale, double k_scale,
                       double v_scale, int partition_size, int P_max,
                       int nthreads)
{
    orc_problem p = {query, q_dt, k_cache, v_cache, cache_dt, block_tables,
                     max_blocks, seq_lens, S, Hq, Hkv, D, bs, NB, scale,
                     k_scale, v_scale, NULL};
    int rc = orc_check(&p);
    if (rc != ORC_OK)
        return rc;
    if (!m_out || !l_out || !o_out || partition_size <= 0 || P_max <= 0)
        return ORC_EARG;
    int G = Hq / Hkv;
    int err = ORC_OK;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int r = 0; r < S * Hq; r++) {
        int s = r / Hq, hq = r % Hq, h = hq / G;
        int L = seq_lens[s];
        int nparts = L > 0 ? (L + partition_size - 1) / partition_size : 0;
        if (nparts > P_max) {
            err = ORC_EARG;
            continue;
        }
        double* q = (double*)malloc(sizeof(double) * D);
        double* K = (double*)malloc(sizeof(double) * (size_t)partition_size * D);
        double* V = (double*)malloc(sizeof(double) * (size_t)partition_size * D);
        double* z = (double*)malloc(sizeof(double) * (size_t)partition_size);
        if (!q || !K || !V || !z) {
            err = ORC_ENOMEM;
            free(q); free(K); free(V); free(z);
            continue;
        }
        orc_query_row(&p, s, hq, q);
        for (int k = 0; k < nparts; k++) {
            int t0 = k * partition_size;
            int t1 = t0 + partition_size < L ? t0 + partition_size : L;
            int n = t1 - t0;
            int e = orc_gather(&p, s, h, t0, t1, K, V);
            if (e != ORC_OK) {
                err = e;
                break;
            }
            orc_scores(&p, q, K, n, z);
            double m = -INFINITY;
            for (int t = 0; t < n; t++)
                if (z[t] > m)
                    m = z[t];
            double l = 0.0;
            for (int t = 0; t < n; t++) {
                z[t] = exp(z[t] - m);
                l += z[t];
            }
            size_t idx = ((size_t)s * Hq + hq) * P_max + k;
            m_out[idx] = m;
            l_out[idx] = l;
            for (int d = 0; d < D; d++) {
                double acc = 0.0;
                for (int t = 0; t < n; t++)
                    acc += z[t] * V[(size_t)t * D + d];
                o_out[idx * D + d] = acc;
            }
        }
        free(q); free(K); free(V); free(z);
    }
    (void)nthreads;
    return err;
}

/* Merge of split-K partials into out[S][Hq][D]:
 *   M = max_k m_k,  out = sum_k e^(m_k - M) o_k / sum_k e^(m_k - M) l_k,
 * over k < ceil(L/P), k ascending.  L <= 0 gives zeros. */
int orc_partition_reduce(double* out, const double* m_in, const double* l_in,
                         const double* o_in, const int32_t* seq_lens, int S,
                         int Hq, int D, int partition_size, int P_max)
{
    if (!out || !m_in || !l_in || !o_in || !seq_lens || S <= 0 || Hq <= 0 ||
        D <= 0 || partition_size <= 0 || P_max <= 0)
        return ORC_EARG;
    for (int s = 0; s < S; s++) {
        int L = seq_lens[s];
        int nparts = L > 0 ? (L + partition_size - 1) / partition_size : 0;
        if (nparts > P_max)
            return ORC_EARG;
        for (int hq = 0; hq < Hq; hq++) {
            size_t base = ((size_t)s * Hq + hq) * P_max;
            double* o = out + ((size_t)s * Hq + hq) * D;
            if (nparts == 0) {
                for (int d = 0; d < D; d++)
                    o[d] = 0.0;
                continue;
            }
            double M = -INFINITY;
            for (int k = 0; k < nparts; k++)
                if (m_in[base + k] > M)
                    M = m_in[base + k];
            double den = 0.0;
            for (int k = 0; k < nparts; k++)
                den += exp(m_in[base + k] - M) * l_in[base + k];
            for (int d = 0; d < D; d++) {
                double num = 0.0;
                for (int k = 0; k < nparts; k++)
                    num += exp(m_in[base + k] - M) * o_in[(base + k) * D + d];
                o[d] = num / den;
            }
        }
    }
    return ORC_OK;
}

/* Several new query tokens per sequence, as chunked prefill and speculative
 * verification use them ([P4] §6.3, §6.5; [P1] §2.3).  The Qn new tokens of
 * sequence s, Qn = query_start[s+1] - query_start[s], are the last Qn of its
 * L cached tokens (appended before attention, as in decode), so query token
 * i sits at position L - Qn + i and attends to tokens 0 .. L - Qn + i
 * (causal among the new tokens; all earlier tokens visible).  A query token
 * whose position is negative (Qn > L) gets a zero row.
 * query and out are [total_q][Hq][D] with total_q = query_start[S]; rows:
 * optional flat indices qtok * Hq + hq, NULL computes every row. */
int orc_paged_multi(double* out, const void* query, int q_dt,
                    const void* k_cache, const void* v_cache, int cache_dt,
                    const int32_t* block_tables, int max_blocks,
                    const int32_t* seq_lens, const int32_t* query_start, int S,
                    int Hq, int Hkv, int D, int bs, int NB, double scale,
                    double k_scale, double v_scale, const int32_t* rows,
                    int n_rows, int nthreads)
{
    orc_problem p = {query, q_dt, k_cache, v_cache, cache_dt, block_tables,
                     max_blocks, seq_lens, S, Hq, Hkv, D, bs, NB, scale,
                     k_scale, v_scale, NULL};
    int rc = orc_check(&p);
    if (rc != ORC_OK || !out || !query_start)
        return rc != ORC_OK ? rc : ORC_EARG;
    if (query_start[0] != 0)
        return ORC_EARG;
    for (int s = 0; s < S; s++)
        if (query_start[s + 1] < query_start[s])
            return ORC_EARG;
    int total_q = query_start[S];
    int* owner = (int*)malloc(sizeof(int) * (size_t)(total_q > 0 ? total_q : 1));
    if (!owner)
        return ORC_ENOMEM;
    for (int s = 0; s < S; s++)
        for (int i = query_start[s]; i < query_start[s + 1]; i++)
            owner[i] = s;
    int G = Hq / Hkv;
    int n = rows ? n_rows : total_q * Hq;
    int err = ORC_OK;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int i = 0; i < n; i++) {
        int r = rows ? rows[i] : i;
        if (r < 0 || r >= total_q * Hq) {
            err = ORC_EARG;
            continue;
        }
        int qt = r / Hq, hq = r % Hq;
        int s = owner[qt];
        int Qn = query_start[s + 1] - query_start[s];
        int pos = seq_lens[s] - Qn + (qt - query_start[s]);
        double* q = (double*)malloc(sizeof(double) * D);
        if (!q) {
            err = ORC_ENOMEM;
            continue;
        }
        size_t base = ((size_t)qt * Hq + hq) * D;
        for (int d = 0; d < D; d++)
            q[d] = orc_load(query, base + d, q_dt);
        int e = orc_attend_row(&p, s, hq / G, q, pos + 1, out + (size_t)r * D);
        free(q);
        if (e != ORC_OK)
            err = e;
    }
    (void)nthreads;
    free(owner);
    return err;
}

/* Gather only (step 1), exposed so tests can pin address translation:
 * K, V receive tokens [0, L) of (s, h) as doubles [L][D]. */
int orc_gather_sequence(double* K, double* V, const void* k_cache,
                        const void* v_cache, int cache_dt,
                        const int32_t* block_tables, int max_blocks,
                        const int32_t* seq_lens, int S, int Hkv, int D, int bs,
                        int NB, double k_scale, double v_scale, int s, int h)
{
    orc_problem p = {k_cache, ORC_F32, k_cache, v_cache, cache_dt,
                     block_tables, max_blocks, seq_lens, S, Hkv, Hkv, D, bs,
                     NB, 1.0, k_scale, v_scale, NULL};
    if (!K || !V || orc_check(&p) != ORC_OK || s < 0 || s >= S || h < 0 || h >= Hkv)
        return ORC_EARG;
    int L = seq_lens[s];
    if (L <= 0)
        return ORC_OK;
    return orc_gather(&p, s, h, 0, L, K, V);
}

int orc_openmp_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
