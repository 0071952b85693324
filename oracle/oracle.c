/*
 * fp64 CPU oracle for the fused inference attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code, header
 * or table with the GPU library; it is the plain definition written out, one
 * output row at a time, in double precision.
 *
 * What it computes (page "torch_npu.npu_prompt_flash_attention", function
 * description formula; page "torch_npu.npu_fused_infer_attention_score_v2",
 * function description formula and the softmax_lse output description):
 *
 *   for every batch b, query head h and valid query row i:
 *     g      = h / (QN / KVN)                  (GQA: contiguous head groups)
 *     J(i)   = { j < Lkv_b : allowed(b, i, j) }
 *     s_j    = scale * sum_d q[b,h,i,d] * k[b,g,j,d]
 *     m      = max_{j in J} s_j
 *     l      = sum_{j in J} exp(s_j - m)
 *     out_e  = sum_{j in J} exp(s_j - m) * v[b,g,j,e] / l
 *     lse    = m + log(l)                       (natural log)
 *   J(i) empty  ->  out = 0, lse = +inf        (parity unpinned: convention)
 *   rows past the valid length of a padded layout -> out = 0, lse = +inf
 *                                               (parity unpinned: convention)
 *
 * Masking is set membership, never the addition of -inf, so no NaN can arise
 * from a masked position and nothing outside J is ever read.
 *
 * allowed(b, i, j) follows the sparse_mode list of the v2 parameter
 * description, with delta = Lkv_b - Lq_b:
 *   mode 0, no mask : true
 *   mode 0, mask    : mask[i][j] == 0 and -pre <= j - i <= next
 *   mode 1          : mask[i][j] == 0
 *   mode 2          : j <= i                       (top-left causal)
 *   mode 3          : j <= i + delta               (bottom-right causal)
 *   mode 4          : -pre <= j - i - delta <= next (bottom-right band)
 * Decode (query S == 1 outside TND) ignores sparse_mode, pre and next (v2
 * parameter description of sparse_mode, pre_tokens, next_tokens); an
 * atten_mask there holds one value per (batch, kv token) (v2 atten_mask
 * description, query S == 1 shapes (B, KV_S), (B, 1, KV_S), (B, 1, 1, KV_S)):
 *   decode          : mask[b][j] == 0
 * A mask value of nonzero means "masked" (PFA parameter description of
 * atten_mask: padding is filled with 1).
 *
 * Block-sparse (page "aclnnBlockSparseAttentionV2", function description
 * formula and constraints): allowed(b, h, i, j) =
 *   M[b, h, i / X, j / Y] != 0 and i < Lq_b and j < Lkv_b,
 * with no causal mask and no atten_mask; the mask's head axis is the query
 * head.  The compacted schedule lists, per (b, h, q-block), the selected
 * kv-blocks kb < ceil(Lkv_b / Y) in ascending order (tail -1).
 *
 * Inputs are fp16/bf16 bit patterns, each read as its exact value in double.
 *
 * KV pseudo-quantization (v2 page, kv pseudo-quant parameters): key and value
 * hold int8 values x; each stands for scale * (x + offset) (the page's table
 * of the quantization formulas is lost; this affine reading is taken), with
 *   mode 0 (per channel): scale[g][d], offset[g][d] of kv head g, channel d;
 *   mode 1 (per token):   scale[b][j], offset[b][j] of batch b, kv token j;
 * the scales and offsets are passed in as exact double values.
 *
 * Block-sparse FP8 (page "aclnnBlockSparseAttentionV2", FP8 feature): query,
 * key and value hold FLOAT8_E4M3FN values, each standing for its value times
 * the fp32 scale of its block: query row i of (b, h) uses
 * qscale[b][h][i / qblk], key / value token j of (b, g) uses
 * kscale[b][g][j / kvblk] (vscale likewise).
 *
 * MLA (v2 page, query_rope / key_rope parameters and their constraints):
 * with both rope inputs given, the query and key vectors are extended by
 * their rope parts (width Dr, laid out like query and key with D = Dr), so
 *   s_j = scale * (sum_d q[b,h,i,d] k[b,g,j,d] + sum_r qr[b,h,i,r] kr[b,g,j,r]);
 * value and output keep D = Dv.  (The pages state the inputs and their
 * shapes, not a formula for the rope parts; concatenation is the reading:
 * parity unpinned against the pages.)
 * With sparse_mode 4 the bottom-right band of the mode list applies at query
 * S 1 too (the MLA constraints list that mode for S 1).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F16 = 0, OR_BF16 = 1 };
enum { OR_BNSD = 0, OR_BSND = 1, OR_TND = 2 };

/* Exact value of an IEEE binary16 / bfloat16 bit pattern. */
static double half_bits_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);   /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static double bf16_bits_to_double(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double elem(const uint16_t* p, int64_t idx, int dtype)
{
    return dtype == OR_BF16 ? bf16_bits_to_double(p[idx]) : half_bits_to_double(p[idx]);
}

/* Exported so a test can check the element reader against a library cast. */
double oracle_read_half(uint16_t bits, int dtype) { return elem(&bits, 0, dtype); }

/* Exact value of a FLOAT8_E4M3FN byte: 1 sign, 4 exponent (bias 7), 3
 * mantissa bits; no infinities, S.1111.111 is NaN. */
static double e4m3fn_to_double(uint8_t x)
{
    int sign = (x >> 7) & 1;
    int e = (x >> 3) & 0xf;
    int m = x & 7;
    double v;
    if (e == 0)
        v = ldexp((double)m, -9);                /* subnormal: m/8 * 2^-6 */
    else if (e == 15 && m == 7)
        v = NAN;
    else
        v = ldexp((double)(8 + m), e - 10);      /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

double oracle_read_e4m3fn(uint8_t bits) { return e4m3fn_to_double(bits); }

typedef struct {
    int32_t layout;          /* OR_BNSD, OR_BSND (also BSH), OR_TND */
    int32_t dtype;           /* OR_F16 or OR_BF16 (q, k, v alike) */
    int64_t B, QN, KVN;
    int64_t Sq, Skv;         /* padded S axes; TND: total rows */
    int64_t Dqk, Dv;
    const int64_t* lq;       /* [B] valid query lengths */
    const int64_t* lkv;      /* [B] valid kv lengths */
    const int64_t* q_start;  /* [B] TND first query row of each sequence */
    const int64_t* kv_start; /* [B] TND first kv row of each sequence */
    double scale;
    int32_t sparse_mode;
    int32_t decode;          /* 1: query S == 1 outside TND */
    int64_t pre_tokens, next_tokens;
    const uint8_t* mask;     /* explicit mask or NULL; nonzero = masked */
    int64_t mask_bstride;    /* elements between batches (0 = broadcast) */
    int64_t mask_rstride;    /* elements between mask rows */
    const int32_t* block_table; /* paged KV or NULL */
    int64_t bt_stride;
    int64_t block_size;
    int32_t pool_layout;     /* 0: (NB, KVN, bs, D)  1: (NB, bs, KVN*D) */
    /* block-sparse */
    const uint8_t* block_mask;  /* [B, QN, nqb, nkb], nonzero = selected */
    int64_t nqb, nkb, X, Y;
    /* optional row subset: n_rows triples (b, h, i); NULL = every row */
    const int64_t* rows;
    int64_t n_rows;
    /* int8 key/value (KV pseudo-quantization); offsets may be NULL (0) */
    int32_t kv_i8;
    int32_t kmode, vmode;            /* 0 per channel [KVN * D], 1 per token [B, tok_stride] */
    const double* k_scale;
    const double* k_off;
    const double* v_scale;
    const double* v_off;
    int64_t tok_stride;
    /* block-sparse FP8 (E4M3FN) inputs with per-block scales */
    int32_t fp8;
    const double* q_bscale;          /* [B, QN, nqs] */
    const double* k_bscale;          /* [B, KVN, nks] */
    const double* v_bscale;
    int64_t nqs, nks, qblk, kvblk;
    /* MLA (query_rope / key_rope given): the score adds q_rope . k_rope, both
     * of width Dr, laid out as the query and the key with D = Dr */
    const uint16_t* q_rope;
    const uint16_t* k_rope;
    int64_t Dr;
} oracle_args;

static int64_t q_off(const oracle_args* a, int64_t b, int64_t h, int64_t i, int64_t D)
{
    switch (a->layout) {
    case OR_BNSD: return ((b * a->QN + h) * a->Sq + i) * D;
    case OR_BSND: return ((b * a->Sq + i) * a->QN + h) * D;
    default:      return ((a->q_start[b] + i) * a->QN + h) * D;
    }
}

static int64_t kv_off(const oracle_args* a, int64_t b, int64_t g, int64_t j, int64_t D)
{
    if (a->block_table) {
        int64_t blk = a->block_table[b * a->bt_stride + j / a->block_size];
        int64_t t = j % a->block_size;
        if (a->pool_layout == 0)
            return ((blk * a->KVN + g) * a->block_size + t) * D;
        return ((blk * a->block_size + t) * a->KVN + g) * D;
    }
    switch (a->layout) {
    case OR_BNSD: return ((b * a->KVN + g) * a->Skv + j) * D;
    case OR_BSND: return ((b * a->Skv + j) * a->KVN + g) * D;
    default:      return ((a->kv_start[b] + j) * a->KVN + g) * D;
    }
}

static int allowed_dense(const oracle_args* a, int64_t b, int64_t i, int64_t j)
{
    /* MLA with a query D of 512 lists sparse_mode 4 (with the mask) at query
     * S 1 as well (v2 page, query_rope / key_rope constraints): there the
     * band applies to decode too, through the mode rules below */
    const int mla_band = a->Dr > 0 && a->sparse_mode == 4;
    if (a->decode && !mla_band)
        return a->mask ? a->mask[b * a->mask_bstride + j] == 0 : 1;
    int64_t delta = a->lkv[b] - a->lq[b];
    int masked_by_tensor = 0;
    if (a->mask && (a->sparse_mode == 0 || a->sparse_mode == 1))
        masked_by_tensor = a->mask[b * a->mask_bstride + i * a->mask_rstride + j] != 0;
    switch (a->sparse_mode) {
    case 0:
        if (!a->mask)
            return 1;
        return !masked_by_tensor && (j - i >= -a->pre_tokens) && (j - i <= a->next_tokens);
    case 1:
        return !masked_by_tensor;
    case 2:
        return j <= i;
    case 3:
        return j <= i + delta;
    case 4:
        return (j - i - delta >= -a->pre_tokens) && (j - i - delta <= a->next_tokens);
    default:
        return 0;
    }
}

static int allowed_bsa(const oracle_args* a, int64_t b, int64_t h, int64_t i, int64_t j)
{
    int64_t qb = i / a->X, kb = j / a->Y;
    return a->block_mask[((b * a->QN + h) * a->nqb + qb) * a->nkb + kb] != 0;
}

/* Element d of key (is_v = 0) or value (is_v = 1) token j of kv head g,
 * batch b, at flat index idx of the tensor. */
static double kv_elem(const oracle_args* a, const void* t, int64_t idx, int is_v, int64_t b,
                      int64_t g, int64_t j, int64_t d, int64_t D)
{
    if (a->fp8) {
        const double* sc = is_v ? a->v_bscale : a->k_bscale;
        return e4m3fn_to_double(((const uint8_t*)t)[idx]) * sc[(b * a->KVN + g) * a->nks + j / a->kvblk];
    }
    if (!a->kv_i8)
        return elem((const uint16_t*)t, idx, a->dtype);
    const double x = (double)((const int8_t*)t)[idx];
    const int md = is_v ? a->vmode : a->kmode;
    const double* sc = is_v ? a->v_scale : a->k_scale;
    const double* of = is_v ? a->v_off : a->k_off;
    const int64_t p = md == 0 ? g * D + d : b * a->tok_stride + j;
    return sc[p] * (x + (of ? of[p] : 0.0));
}

/* One output row: out[0..Dv) and *lse.  Returns 0, or -1 on allocation failure. */
static int one_row(const oracle_args* a, const uint16_t* q, const void* k,
                   const void* v, int bsa, int64_t b, int64_t h, int64_t i,
                   double* out, double* lse)
{
    int64_t e;
    for (e = 0; e < a->Dv; ++e)
        out[e] = 0.0;
    *lse = INFINITY;
    if (i >= (a->decode ? 1 : a->lq[b]))
        return 0;                                   /* padding row */
    int64_t L = a->lkv[b];
    if (L <= 0)
        return 0;                                   /* empty kv */
    int64_t G = a->QN / a->KVN;
    int64_t g = h / G;
    double* s = (double*)malloc(sizeof(double) * (size_t)L);
    unsigned char* in = (unsigned char*)malloc((size_t)L);
    if (!s || !in) {
        free(s);
        free(in);
        return -1;
    }
    const int64_t qo = q_off(a, b, h, i, a->Dqk);
    double m = -INFINITY;
    int64_t n_in = 0, j, d;
    for (j = 0; j < L; ++j) {
        in[j] = (unsigned char)(bsa ? allowed_bsa(a, b, h, i, j) : allowed_dense(a, b, i, j));
        if (!in[j])
            continue;
        const int64_t ko = kv_off(a, b, g, j, a->Dqk);
        double acc = 0.0;
        for (d = 0; d < a->Dqk; ++d) {
            const double qv = a->fp8 ? e4m3fn_to_double(((const uint8_t*)q)[qo + d]) *
                                           a->q_bscale[(b * a->QN + h) * a->nqs + i / a->qblk]
                                     : elem(q, qo + d, a->dtype);
            acc += qv * kv_elem(a, k, ko + d, 0, b, g, j, d, a->Dqk);
        }
        if (a->Dr > 0) {
            /* MLA: the rope parts extend the query and key vectors */
            const int64_t qro = q_off(a, b, h, i, a->Dr), kro = kv_off(a, b, g, j, a->Dr);
            for (d = 0; d < a->Dr; ++d)
                acc += elem(a->q_rope, qro + d, a->dtype) * elem(a->k_rope, kro + d, a->dtype);
        }
        s[j] = a->scale * acc;
        if (s[j] > m)
            m = s[j];
        ++n_in;
    }
    if (n_in > 0) {
        double l = 0.0;
        for (j = 0; j < L; ++j) {
            if (!in[j])
                continue;
            const double p = exp(s[j] - m);
            const int64_t vo = kv_off(a, b, g, j, a->Dv);
            l += p;
            for (e = 0; e < a->Dv; ++e)
                out[e] += p * kv_elem(a, v, vo + e, 1, b, g, j, e, a->Dv);
        }
        for (e = 0; e < a->Dv; ++e)
            out[e] /= l;
        *lse = m + log(l);
    }
    free(s);
    free(in);
    return 0;
}

/* Output addressing: out follows the query layout with D = Dv; lse is
 * [B, QN, Sq] (TND: [T, QN]).  With a row subset, out is [n_rows, Dv] and
 * lse is [n_rows]. */
static int run(const oracle_args* a, const uint16_t* q, const void* k, const void* v,
               int bsa, double* out, double* lse)
{
    int failed = 0;
    if (a->rows) {
        int64_t r;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
        for (r = 0; r < a->n_rows; ++r) {
            const int64_t* t = a->rows + 3 * r;
            failed |= one_row(a, q, k, v, bsa, t[0], t[1], t[2], out + r * a->Dv, lse + r) != 0;
        }
        return failed ? -1 : 0;
    }
    int64_t n_units, u;
    int64_t Sq_rows = a->decode ? 1 : a->Sq;
    if (a->layout == OR_TND)
        n_units = a->Sq * a->QN;                     /* every (row, head) */
    else
        n_units = a->B * a->QN * Sq_rows;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : failed)
    for (u = 0; u < n_units; ++u) {
        int64_t b, h, i, oo, lo;
        if (a->layout == OR_TND) {
            int64_t row = u / a->QN;
            h = u % a->QN;
            for (b = 0; b + 1 < a->B && a->q_start[b + 1] <= row; ++b) {
            }
            i = row - a->q_start[b];
            if (i >= a->lq[b])
                continue;                             /* rows past the last sequence */
            oo = (row * a->QN + h) * a->Dv;
            lo = row * a->QN + h;
        } else {
            b = u / (a->QN * Sq_rows);
            h = (u / Sq_rows) % a->QN;
            i = u % Sq_rows;
            oo = a->layout == OR_BNSD ? ((b * a->QN + h) * a->Sq + i) * a->Dv
                                      : ((b * a->Sq + i) * a->QN + h) * a->Dv;
            lo = (b * a->QN + h) * a->Sq + i;
        }
        failed |= one_row(a, q, k, v, bsa, b, h, i, out + oo, lse + lo) != 0;
    }
    return failed ? -1 : 0;
}

int oracle_attention(const oracle_args* a, const uint16_t* q, const void* k,
                     const void* v, double* out, double* lse)
{
    if (!a || !q || !k || !v || !out || !lse || a->KVN <= 0 || a->QN % a->KVN)
        return -2;
    if (a->kv_i8 && (!a->k_scale || !a->v_scale))
        return -2;
    return run(a, q, k, v, 0, out, lse);
}

int oracle_block_sparse(const oracle_args* a, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, double* out, double* lse)
{
    if (!a || !q || !k || !v || !out || !lse || !a->block_mask || a->X <= 0 || a->Y <= 0 ||
        a->KVN <= 0 || a->QN % a->KVN || a->kv_i8)
        return -2;
    if (a->fp8 && (!a->q_bscale || !a->k_bscale || !a->v_bscale || a->qblk <= 0 || a->kvblk <= 0))
        return -2;
    return run(a, q, k, v, 1, out, lse);
}

/* Compacted block schedule: cnt[b,h,qb] and idx[b,h,qb,0..nkb) ascending,
 * tail -1.  q-blocks at or past ceil(Lq_b / X) get an empty list. */
int oracle_bsa_compact(const uint8_t* mask, int64_t B, int64_t N, int64_t nqb, int64_t nkb,
                       const int64_t* lq, const int64_t* lkv, int64_t X, int64_t Y,
                       int32_t* idx, int32_t* cnt)
{
    int64_t b, h, qb, kb;
    for (b = 0; b < B; ++b) {
        const int64_t qlim = (lq[b] + X - 1) / X;
        const int64_t klim = (lkv[b] + Y - 1) / Y;
        for (h = 0; h < N; ++h) {
            for (qb = 0; qb < nqb; ++qb) {
                const int64_t row = (b * N + h) * nqb + qb;
                int32_t c = 0;
                for (kb = 0; kb < nkb; ++kb)
                    idx[row * nkb + kb] = -1;
                if (qb < qlim)
                    for (kb = 0; kb < nkb && kb < klim; ++kb)
                        if (mask[row * nkb + kb])
                            idx[row * nkb + c++] = (int32_t)kb;
                cnt[row] = c;
            }
        }
    }
    return 0;
}

/* Threads of the OpenMP loops over output rows (n >= 1); a timing knob only. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
