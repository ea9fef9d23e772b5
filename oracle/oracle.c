/*
 * CPU oracle for paged grouped-query attention over a block-table fp16 KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, single-threaded statement of what the
 * paged-attention path computes. Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load it. The HIP library never links, includes or calls it,
 * and it shares no code, header or table with the HIP library.
 *
 * Sources (three web pages):
 *   [append]   com.microsoft.SparseAttention, "sparse-kv-append.wgsl.jinja": the KV append pass
 *              (past-length rule, rotary pairing, one write per new row).
 *   [sparse]   alice-llm "sparse_attention_forward.wgsl": the block-sparse edge forward that
 *              emits per-(edge, q-head) partials (o, m, l) in fp32.
 *   [manifest] com.microsoft.PagedAttention "manifest.json": op inputs/outputs/attributes, the
 *              derived shapes, and the scatter -> split-attend -> merge passes.
 *
 * Precision. Attention, softmax and merge arithmetic run in float64 on values decoded exactly
 * from their fp16/fp32 storage, and results are rounded once (round-to-nearest-even) into the
 * output storage type. The rotary step runs in float32, because the append page writes it as
 * a float32 function: two float32 products, each rounded, then one float32 add or subtract,
 * then a cast to fp16. This file must be compiled with -ffp-contract=off so that the compiler
 * does not fuse those products.
 *
 * Parity pins for every function here live in the CPU test suite; see the test files named
 * after each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_ROTARY_NONE 0
#define ORACLE_ROTARY_NEOX 1
#define ORACLE_ROTARY_INTERLEAVED 2

/* ---------------------------------------------------------------------------------------- */
/* IEEE-754 binary16 <-> binary64, written from the format definition.                      */
/* ---------------------------------------------------------------------------------------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);    /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Round a binary64 value to the nearest binary16, ties to even. */
uint16_t oracle_f64_to_f16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00);
    double a = fabs(x);
    /* 65520 is halfway between 65504 (largest finite, odd significand) and 2^16: ties go to the
     * even side, which overflows to infinity. */
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; a rounded quotient of 1024 is the smallest normal */
        double r = nearbyint(a * 16777216.0);
        return (uint16_t)(sign | (uint16_t)r);
    }
    int e2;
    frexp(a, &e2);                      /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;                     /* unbiased exponent, -14..15 */
    double r = nearbyint(ldexp(a, 10 - E));   /* significand * 1024, in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        E += 1;
    }
    if (E > 15)
        return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)r - 1024));
}

uint16_t oracle_f32_to_f16(float x) { return oracle_f64_to_f16((double)x); }

/* The same decode, tabulated once: every fp16 bit pattern -> its float64 value. The oracle is
 * single-threaded, so the lazy fill needs no lock. */
static double f16_table[65536];
static int f16_table_ready = 0;

static double f16v(uint16_t h)
{
    if (!f16_table_ready) {
        for (int i = 0; i < 65536; ++i)
            f16_table[i] = oracle_f16_to_f64((uint16_t)i);
        f16_table_ready = 1;
    }
    return f16_table[h];
}

/* ---------------------------------------------------------------------------------------- */
/* [append] past-length rule for a padded batch.                                             */
/* ---------------------------------------------------------------------------------------- */

/* How much history precedes a padded batch's new tokens. When the scalar total sequence length
 * equals the new-token count the call is a prompt, and every row has no history; otherwise a
 * row's history is its own total minus the new-token count, and zero if that would be
 * negative. */
int oracle_past_length_padded(int total_sequence_length, int key_total_sequence_length,
                              int seq_len)
{
    if ((uint32_t)total_sequence_length == (uint32_t)seq_len)
        return 0;
    if ((uint32_t)key_total_sequence_length >= (uint32_t)seq_len)
        return (int)((uint32_t)key_total_sequence_length - (uint32_t)seq_len);
    return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* [append] rotary pairing.                                                                  */
/* ---------------------------------------------------------------------------------------- */

/* Cos/sin column used by component d: interleaved pairs (2i, 2i+1) share column i; the NeoX
 * split pairs d with d + R/2 and both use column d mod R/2. */
static int rotary_column(int d, int half, int mode)
{
    if (mode == ORACLE_ROTARY_INTERLEAVED)
        return d / 2;
    return d < half ? d : d - half;
}

static int rotary_partner(int d, int half, int mode)
{
    if (mode == ORACLE_ROTARY_INTERLEAVED)
        return (d % 2 == 0) ? d + 1 : d - 1;
    return d < half ? d + half : d - half;
}

static int rotary_is_first(int d, int half, int mode)
{
    if (mode == ORACLE_ROTARY_INTERLEAVED)
        return d % 2 == 0;
    return d < half;
}

/* The first member of a pair subtracts its partner's sine term; the second adds it. Float32,
 * products rounded separately (no contraction). */
static float rotary_component(float own, float partner, float cs, float sn, int first)
{
    float a = own * cs;
    float b = partner * sn;
    return first ? a - b : a + b;
}

/* ---------------------------------------------------------------------------------------- */
/* [append] + [manifest ScatterKV] fused KV append into the paged cache.                     */
/* ---------------------------------------------------------------------------------------- */

/*
 * For every sequence b and new token t < n_b (n_b = cu[b+1]-cu[b]): row i = cu[b]+t sits at
 * absolute position pos = past[b]+t. Its slot is slot_mapping[i] when a mapping is given, else
 * block_table[b][pos/bs]*bs + pos%bs. A negative slot writes nothing. For each kv head g the
 * key row (separate key input, or the packed row at column H*D + g*D) is rotated at pos over its
 * first rotary_dim components and written to key_cache[slot/bs][slot%bs][g][:]; the value row
 * (separate, or packed column (H+G)*D + g*D) is copied to value_cache at the same place. No
 * other cache element is written.
 */
void oracle_kv_append(int T, int B, int H, int G, int D, int bs, int MB, int packed,
                      const uint16_t *query, const uint16_t *key, const uint16_t *value,
                      uint16_t *key_cache, uint16_t *value_cache,
                      const int32_t *cu, const int32_t *past, const int32_t *block_table,
                      const int32_t *slot_mapping,
                      const uint16_t *cos_cache, const uint16_t *sin_cache,
                      int rotary_dim, int rotary_mode)
{
    (void)T;
    const int half = rotary_dim / 2;
    const long long qstride = (long long)(H + 2 * G) * D;
    for (int b = 0; b < B; ++b) {
        const int n = cu[b + 1] - cu[b];
        for (int t = 0; t < n; ++t) {
            const long long i = (long long)cu[b] + t;
            const long long pos = (long long)past[b] + t;
            long long slot;
            if (slot_mapping)
                slot = slot_mapping[i];
            else
                slot = (long long)block_table[(long long)b * MB + pos / bs] * bs + pos % bs;
            if (slot < 0)
                continue;
            for (int g = 0; g < G; ++g) {
                const uint16_t *ks, *vs;
                if (packed) {
                    ks = query + i * qstride + (long long)H * D + (long long)g * D;
                    vs = query + i * qstride + (long long)(H + G) * D + (long long)g * D;
                } else {
                    ks = key + i * G * D + (long long)g * D;
                    vs = value + i * G * D + (long long)g * D;
                }
                uint16_t *kd = key_cache + (slot * G + g) * D;
                uint16_t *vd = value_cache + (slot * G + g) * D;
                for (int d = 0; d < D; ++d) {
                    if (rotary_mode != ORACLE_ROTARY_NONE && d < rotary_dim) {
                        const int c = rotary_column(d, half, rotary_mode);
                        const float cs = (float)oracle_f16_to_f64(cos_cache[pos * half + c]);
                        const float sn = (float)oracle_f16_to_f64(sin_cache[pos * half + c]);
                        const float own = (float)oracle_f16_to_f64(ks[d]);
                        const float partner =
                            (float)oracle_f16_to_f64(ks[rotary_partner(d, half, rotary_mode)]);
                        kd[d] = oracle_f32_to_f16(
                            rotary_component(own, partner, cs, sn,
                                             rotary_is_first(d, half, rotary_mode)));
                    } else {
                        kd[d] = ks[d];
                    }
                    vd[d] = vs[d];
                }
            }
        }
    }
}

/* The [append] page's own pass over a contiguous BNSH cache [B, KVH, max_cache_seq, D]: one
 * write per (batch, kv head, new token t < seq_len, component d), at position
 * past + t with past = oracle_past_length_padded(total_sequence_length,
 * key_total_sequence_lengths[b], seq_len); the key is rotated at that position (as in
 * oracle_kv_append), the value copied. Sources: padded rows (b*seq_len + t) of packed
 * [Q | K | V] rows or of separate [B*seq_len, KVH*D] arrays. A row whose position falls at or
 * past max_cache_seq (or, with rotary, at or past rotary_positions) is not written: the page
 * leaves that to the caller, this oracle and the library skip it. */
void oracle_kv_append_bnsh(int B, int seq_len, int H, int KVH, int D, int max_cache_seq,
                           int packed, const uint16_t *query, const uint16_t *key,
                           const uint16_t *value, uint16_t *present_key,
                           uint16_t *present_value, int total_sequence_length,
                           const int32_t *key_total_sequence_lengths,
                           const uint16_t *cos_cache, const uint16_t *sin_cache,
                           int rotary_dim, int rotary_mode, int rotary_positions)
{
    const int half = rotary_dim / 2;
    const long long qstride = (long long)(H + 2 * KVH) * D;
    for (int b = 0; b < B; ++b) {
        const int past = oracle_past_length_padded(total_sequence_length,
                                                   key_total_sequence_lengths[b], seq_len);
        for (int h = 0; h < KVH; ++h) {
            for (int t = 0; t < seq_len; ++t) {
                const long long pos = (long long)past + t;
                if (pos >= max_cache_seq)
                    continue;
                if (rotary_mode != ORACLE_ROTARY_NONE && pos >= rotary_positions)
                    continue;
                const long long row = (long long)b * seq_len + t;
                const uint16_t *ks, *vs;
                if (packed) {
                    ks = query + row * qstride + (long long)H * D + (long long)h * D;
                    vs = query + row * qstride + (long long)(H + KVH) * D + (long long)h * D;
                } else {
                    ks = key + row * KVH * D + (long long)h * D;
                    vs = value + row * KVH * D + (long long)h * D;
                }
                const long long dst = (((long long)b * KVH + h) * max_cache_seq + pos) * D;
                for (int d = 0; d < D; ++d) {
                    if (rotary_mode != ORACLE_ROTARY_NONE && d < rotary_dim) {
                        const int c = rotary_column(d, half, rotary_mode);
                        const float cs = (float)oracle_f16_to_f64(cos_cache[pos * half + c]);
                        const float sn = (float)oracle_f16_to_f64(sin_cache[pos * half + c]);
                        const float own = (float)oracle_f16_to_f64(ks[d]);
                        const float partner =
                            (float)oracle_f16_to_f64(ks[rotary_partner(d, half, rotary_mode)]);
                        present_key[dst + d] = oracle_f32_to_f16(
                            rotary_component(own, partner, cs, sn,
                                             rotary_is_first(d, half, rotary_mode)));
                    } else {
                        present_key[dst + d] = ks[d];
                    }
                    present_value[dst + d] = vs[d];
                }
            }
        }
    }
}

/* Query rotation at the same positions (the first "next" step past the pages, which rotate only
 * keys in the append and hand queries to attention already positioned): new query row t of
 * sequence b sits at pos = past[b] + t, and each of its H head rows gets the same per-pair
 * float32 rotation the key path applies, with the same cos/sin rows; components past
 * rotary_dim are copied. Source rows are the Q part of packed rows or a separate [T, H*D]
 * array; q_out is [T, H*D] fp16 and every row of every sequence is written. */
void oracle_rotate_query(int B, int H, int G, int D, int packed, const uint16_t *query,
                         const int32_t *cu, const int32_t *past, const uint16_t *cos_cache,
                         const uint16_t *sin_cache, int rotary_dim, int rotary_mode,
                         uint16_t *q_out)
{
    const int half = rotary_dim / 2;
    const long long stride = packed ? (long long)(H + 2 * G) * D : (long long)H * D;
    for (int b = 0; b < B; ++b) {
        const int n = cu[b + 1] - cu[b];
        for (int t = 0; t < n; ++t) {
            const long long i = (long long)cu[b] + t;
            const long long pos = (long long)past[b] + t;
            for (int h = 0; h < H; ++h) {
                const uint16_t *qs = query + i * stride + (long long)h * D;
                uint16_t *qd = q_out + (i * H + h) * (long long)D;
                for (int d = 0; d < D; ++d) {
                    if (rotary_mode != ORACLE_ROTARY_NONE && d < rotary_dim) {
                        const int c = rotary_column(d, half, rotary_mode);
                        const float cs = (float)oracle_f16_to_f64(cos_cache[pos * half + c]);
                        const float sn = (float)oracle_f16_to_f64(sin_cache[pos * half + c]);
                        const float own = (float)oracle_f16_to_f64(qs[d]);
                        const float partner =
                            (float)oracle_f16_to_f64(qs[rotary_partner(d, half, rotary_mode)]);
                        qd[d] = oracle_f32_to_f16(
                            rotary_component(own, partner, cs, sn,
                                             rotary_is_first(d, half, rotary_mode)));
                    } else {
                        qd[d] = qs[d];
                    }
                }
            }
        }
    }
}

/* Edge list of the block-sparse forward from a kept-block mask (the [sparse] page's host step:
 * block_len from used_kv_lens clamped by the block). Rows (q, h) are taken in order, blocks in
 * order within a row; every nonzero mask[q][h][blk] gives edge (q, h, blk, b, block_len) with
 * b = q_batch[q] and block_len = clamp(used_kv_lens[b] - blk*block_size, 0, block_size).
 * group_ptr[q*hkv + h] is the index of the row's first edge, group_ptr[tq*hkv] the edge count.
 * edge_meta must hold as many edges as the mask has nonzero entries. */
void oracle_build_edges(int tq, int hkv, int nblk, int block_size, const uint8_t *mask,
                        const int32_t *q_batch, const int32_t *used_kv_lens, int32_t *edge_meta,
                        int32_t *group_ptr)
{
    long long e = 0;
    for (int q = 0; q < tq; ++q) {
        const int b = q_batch[q];
        for (int h = 0; h < hkv; ++h) {
            group_ptr[(long long)q * hkv + h] = (int32_t)e;
            for (int blk = 0; blk < nblk; ++blk) {
                if (!mask[((long long)q * hkv + h) * nblk + blk])
                    continue;
                long long len = (long long)used_kv_lens[b] - (long long)blk * block_size;
                if (len < 0)
                    len = 0;
                if (len > block_size)
                    len = block_size;
                int32_t *m = edge_meta + 5 * e;
                m[0] = q;
                m[1] = h;
                m[2] = blk;
                m[3] = b;
                m[4] = (int32_t)len;
                ++e;
            }
        }
    }
    group_ptr[(long long)tq * hkv] = (int32_t)e;
}

/* ---------------------------------------------------------------------------------------- */
/* Paged attention: gather to contiguous, then dense softmax attention.                      */
/* ---------------------------------------------------------------------------------------- */

/* Copy key (or value) rows 0..n-1 of sequence b, kv head g, out of the paged cache into a
 * contiguous float64 array [n, D]. Row j lives in block block_table[b][j/bs] at offset j%bs. */
static void gather_rows(const uint16_t *cache, const int32_t *block_table, int MB, int bs,
                        int G, int D, int b, int g, int n, double *dst)
{
    for (int j = 0; j < n; ++j) {
        const long long blk = block_table[(long long)b * MB + j / bs];
        const uint16_t *src = cache + ((blk * bs + j % bs) * G + g) * (long long)D;
        for (int d = 0; d < D; ++d)
            dst[(long long)j * D + d] = f16v(src[d]);
    }
}

/* Softmax attention of one query vector over keys K[0..n) and values V[0..n), unnormalised:
 * s_j = (q . k_j) * scale, m = max_j s_j, p_j = exp(s_j - m), l = sum_j p_j,
 * o = sum_j p_j v_j. n == 0 gives m = -inf, l = 0, o = 0. */
static void attend(const double *q, const double *K, const double *V, int n, int D, double scale,
                   double *o, double *m_out, double *l_out, double *s)
{
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += q[d] * K[(long long)j * D + d];
        s[j] = dot * scale;
        if (s[j] > m)
            m = s[j];
    }
    double l = 0.0;
    for (int d = 0; d < D; ++d)
        o[d] = 0.0;
    for (int j = 0; j < n; ++j) {
        const double p = exp(s[j] - m);
        l += p;
        for (int d = 0; d < D; ++d)
            o[d] += p * V[(long long)j * D + d];
    }
    *m_out = m;
    *l_out = l;
}

/* Keys visible to row t of sequence b: causal -> positions 0..past+t, else the whole sequence
 * past + n_b. */
static int visible_keys(const int32_t *cu, const int32_t *past, int b, int t, int causal)
{
    const int n = cu[b + 1] - cu[b];
    return causal ? past[b] + t + 1 : past[b] + n;
}

/*
 * Dense paged attention ([manifest] PagedAttention.Attend). Query head h of row i attends with
 * kv head g = h / (H/G) over the visible keys of its sequence; the output row
 * out[i][h*D + d] is the normalised softmax-weighted sum of values, rounded to fp16.
 * Query head h of row i starts at query[i*q_row_stride + h*D] (q_row_stride = H*D, or
 * (H+2G)*D for the packed layout).
 */
void oracle_paged_attention(int T, int B, int H, int G, int D, int bs, int MB,
                            const uint16_t *query, long long q_row_stride,
                            const uint16_t *key_cache, const uint16_t *value_cache,
                            const int32_t *cu, const int32_t *past, const int32_t *block_table,
                            double scale, int causal, uint16_t *out)
{
    (void)T;
    const int Q = H / G;
    int maxn = 1;
    for (int b = 0; b < B; ++b) {
        const int Lb = past[b] + cu[b + 1] - cu[b];
        if (Lb > maxn)
            maxn = Lb;
    }
    double *K = malloc(sizeof(double) * (size_t)maxn * D);
    double *V = malloc(sizeof(double) * (size_t)maxn * D);
    double *s = malloc(sizeof(double) * (size_t)maxn);
    double *q = malloc(sizeof(double) * (size_t)D);
    double *o = malloc(sizeof(double) * (size_t)D);
    for (int b = 0; b < B; ++b) {
        const int n_b = cu[b + 1] - cu[b];
        for (int t = 0; t < n_b; ++t) {
            const long long i = (long long)cu[b] + t;
            const int limit = visible_keys(cu, past, b, t, causal);
            for (int h = 0; h < H; ++h) {
                const int g = h / Q;
                gather_rows(key_cache, block_table, MB, bs, G, D, b, g, limit, K);
                gather_rows(value_cache, block_table, MB, bs, G, D, b, g, limit, V);
                for (int d = 0; d < D; ++d)
                    q[d] = f16v(query[i * q_row_stride + (long long)h * D + d]);
                double m, l;
                attend(q, K, V, limit, D, scale, o, &m, &l, s);
                for (int d = 0; d < D; ++d)
                    out[i * H * D + (long long)h * D + d] = oracle_f64_to_f16(o[d] / l);
            }
        }
    }
    free(K);
    free(V);
    free(s);
    free(q);
    free(o);
}

/*
 * Split-KV partials ([manifest] PagedAttention.AttendSplitK). The visible keys [0, limit) of
 * each (row i, head h) are cut into num_splits contiguous chunks of C keys, where
 * C = chunk_keys if chunk_keys > 0, else C = ceil(ceil(limit / num_splits) / bs) * bs. Chunk s
 * covers [s*C, min((s+1)*C, limit)) and emits the unnormalised (o, m, l) of attend() over it; an
 * empty chunk emits o = 0, m = -1e30, l = 0. Partial p = (i*num_splits + s)*H + h:
 * o_part[p*D + d], m_part[p], l_part[p], stored as float32.
 */
void oracle_paged_attention_partials(int T, int B, int H, int G, int D, int bs, int MB,
                                     const uint16_t *query, long long q_row_stride,
                                     const uint16_t *key_cache, const uint16_t *value_cache,
                                     const int32_t *cu, const int32_t *past,
                                     const int32_t *block_table, double scale, int causal,
                                     int num_splits, int chunk_keys,
                                     float *o_part, float *m_part, float *l_part)
{
    (void)T;
    const int Q = H / G;
    int maxn = 1;
    for (int b = 0; b < B; ++b) {
        const int Lb = past[b] + cu[b + 1] - cu[b];
        if (Lb > maxn)
            maxn = Lb;
    }
    double *K = malloc(sizeof(double) * (size_t)maxn * D);
    double *V = malloc(sizeof(double) * (size_t)maxn * D);
    double *s = malloc(sizeof(double) * (size_t)maxn);
    double *q = malloc(sizeof(double) * (size_t)D);
    double *o = malloc(sizeof(double) * (size_t)D);
    for (int b = 0; b < B; ++b) {
        const int n_b = cu[b + 1] - cu[b];
        for (int t = 0; t < n_b; ++t) {
            const long long i = (long long)cu[b] + t;
            const int limit = visible_keys(cu, past, b, t, causal);
            long long C = chunk_keys;
            if (C <= 0) {
                const long long per = (limit + num_splits - 1) / num_splits;
                C = (per + bs - 1) / bs * bs;
            }
            for (int h = 0; h < H; ++h) {
                const int g = h / Q;
                gather_rows(key_cache, block_table, MB, bs, G, D, b, g, limit, K);
                gather_rows(value_cache, block_table, MB, bs, G, D, b, g, limit, V);
                for (int d = 0; d < D; ++d)
                    q[d] = f16v(query[i * q_row_stride + (long long)h * D + d]);
                for (int sp = 0; sp < num_splits; ++sp) {
                    const long long p = (i * num_splits + sp) * H + h;
                    long long lo = sp * C, hi = (sp + 1) * C;
                    if (hi > limit)
                        hi = limit;
                    if (lo >= hi) {
                        for (int d = 0; d < D; ++d)
                            o_part[p * D + d] = 0.0f;
                        m_part[p] = -1e30f;
                        l_part[p] = 0.0f;
                        continue;
                    }
                    double m, l;
                    attend(q, K + lo * D, V + lo * D, (int)(hi - lo), D, scale, o, &m, &l, s);
                    for (int d = 0; d < D; ++d)
                        o_part[p * D + d] = (float)o[d];
                    m_part[p] = (float)m;
                    l_part[p] = (float)l;
                }
            }
        }
    }
    free(K);
    free(V);
    free(s);
    free(q);
    free(o);
}

/* ---------------------------------------------------------------------------------------- */
/* Log-sum-exp merge of partials ([manifest] PagedAttention.AttendSplitKMerge).              */
/* ---------------------------------------------------------------------------------------- */

/*
 * Group k owns partial units e in [e0, e1): e0 = group_ptr[k], e1 = group_ptr[k+1] when a CSR
 * offset array is given, else e0 = k*num_splits, e1 = e0 + num_splits. Each unit holds `lanes`
 * partials, p = e*lanes + lane. Output row r = k*lanes + lane:
 *   M = max_e m_p;  w_e = exp(m_p - M) if l_p > 0 else 0;  Lsum = sum_e w_e l_p;
 *   out[r][d] = (sum_e w_e o_p[d]) / Lsum, or 0 when Lsum == 0.
 * out_dtype 0 writes fp16 (RNE), 1 writes float32.
 */
void oracle_split_combine(const float *o_part, const float *m_part, const float *l_part,
                          const int32_t *group_ptr, int num_groups, int lanes, int num_splits,
                          int D, int out_dtype, void *out)
{
    double *acc = malloc(sizeof(double) * (size_t)D);
    for (int k = 0; k < num_groups; ++k) {
        const long long e0 = group_ptr ? group_ptr[k] : (long long)k * num_splits;
        const long long e1 = group_ptr ? group_ptr[k + 1] : e0 + num_splits;
        for (int lane = 0; lane < lanes; ++lane) {
            double M = -INFINITY;
            for (long long e = e0; e < e1; ++e) {
                const long long p = e * lanes + lane;
                if (l_part[p] > 0.0f && (double)m_part[p] > M)
                    M = m_part[p];
            }
            double Lsum = 0.0;
            for (int d = 0; d < D; ++d)
                acc[d] = 0.0;
            for (long long e = e0; e < e1; ++e) {
                const long long p = e * lanes + lane;
                if (!(l_part[p] > 0.0f))
                    continue;
                const double w = exp((double)m_part[p] - M);
                Lsum += w * (double)l_part[p];
                for (int d = 0; d < D; ++d)
                    acc[d] += w * (double)o_part[p * D + d];
            }
            const long long r = (long long)k * lanes + lane;
            for (int d = 0; d < D; ++d) {
                const double v = Lsum > 0.0 ? acc[d] / Lsum : 0.0;
                if (out_dtype == 0)
                    ((uint16_t *)out)[r * D + d] = oracle_f64_to_f16(v);
                else
                    ((float *)out)[r * D + d] = (float)v;
            }
        }
    }
    free(acc);
}

/* ---------------------------------------------------------------------------------------- */
/* [sparse] block-sparse edge forward.                                                        */
/* ---------------------------------------------------------------------------------------- */

/*
 * One partial per (edge e, q-head lane qh), p = e*qhead + qh, following the page's phases:
 * edge e = (q_idx, h, blk, batch, block_len) from edge_meta[5e..5e+4]; query row
 * q_buf[q_idx][h*qhead + qh][:]. A block_len <= 0 gives the sentinel o = 0, m = -1e30, l = 0.
 * Otherwise for t < block_len: page slot blk*(block_size/page_size) + t/page_size of the
 * batch's table row gives page id pid; pid < 0 gives score -1e30, else the key row
 * k_pages[pid][h][t % page_size][:] gives s_t = (q . k) * scale. m = max(-1e30, max_t s_t);
 * p_t = exp(s_t - m) when s_t > -5e29, else 0; l = sum_t p_t; o = sum over mapped t with
 * p_t != 0 of p_t * v_t. Results are stored as float32.
 * q_pos (int32 [Tq], or NULL for no mask) adds the right-aligned causal mask the page lists as
 * unimplemented: key t of the edge's block is seen only when blk*block_size + t <= q_pos[q_idx].
 */
void oracle_sparse_forward(int E, int hkv, int qhead, int D, int block_size, int page_size,
                           int max_pages, const float *q_buf, const float *k_pages,
                           const float *v_pages, const int32_t *edge_meta,
                           const int32_t *block_tables, double softmax_scale,
                           const int32_t *q_pos, float *o_partial, float *m_partial,
                           float *l_partial)
{
    const double NEG_LARGE = (double)-1.0e30f;
    const int hq = hkv * qhead;
    const int ppb = block_size / page_size;
    int maxlen = 1;
    for (long long e = 0; e < E; ++e)
        if (edge_meta[e * 5 + 4] > maxlen)
            maxlen = edge_meta[e * 5 + 4];
    double *s = malloc(sizeof(double) * (size_t)maxlen);
    double *o = malloc(sizeof(double) * (size_t)D);
    for (long long e = 0; e < E; ++e) {
        const int q_idx = edge_meta[e * 5 + 0];
        const int h = edge_meta[e * 5 + 1];
        const int blk = edge_meta[e * 5 + 2];
        const int batch = edge_meta[e * 5 + 3];
        const int len = edge_meta[e * 5 + 4] > 0 ? edge_meta[e * 5 + 4] : 0;
        for (int qh = 0; qh < qhead; ++qh) {
            const long long p = e * qhead + qh;
            if (len == 0) {
                for (int d = 0; d < D; ++d)
                    o_partial[p * D + d] = 0.0f;
                m_partial[p] = (float)NEG_LARGE;
                l_partial[p] = 0.0f;
                continue;
            }
            const float *q = q_buf + ((long long)q_idx * hq + (long long)h * qhead + qh) * D;
            double m = NEG_LARGE;
            for (int t = 0; t < len; ++t) {
                const int pid = block_tables[(long long)batch * max_pages +
                                             (long long)blk * ppb + t / page_size];
                double st = NEG_LARGE;
                /* causal (the mask the page leaves unimplemented): a key whose absolute position
                 * blk * block_size + t lies after the query row's position q_pos[q_idx] is
                 * excluded exactly like a key on an unmapped page */
                const int visible =
                    !q_pos || (long long)blk * block_size + t <= (long long)q_pos[q_idx];
                if (pid >= 0 && visible) {
                    const float *k =
                        k_pages + (((long long)pid * hkv + h) * page_size + t % page_size) * D;
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += (double)q[d] * (double)k[d];
                    st = dot * softmax_scale;
                }
                s[t] = st;
                if (st > m)
                    m = st;
            }
            double l = 0.0;
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            for (int t = 0; t < len; ++t) {
                const double pt = s[t] > NEG_LARGE * 0.5 ? exp(s[t] - m) : 0.0;
                l += pt;
                if (pt == 0.0)
                    continue;
                const int pid = block_tables[(long long)batch * max_pages +
                                             (long long)blk * ppb + t / page_size];
                if (pid < 0)
                    continue;
                const float *v =
                    v_pages + (((long long)pid * hkv + h) * page_size + t % page_size) * D;
                for (int d = 0; d < D; ++d)
                    o[d] += pt * (double)v[d];
            }
            for (int d = 0; d < D; ++d)
                o_partial[p * D + d] = (float)o[d];
            m_partial[p] = (float)m;
            l_partial[p] = (float)l;
        }
    }
    free(s);
    free(o);
}
