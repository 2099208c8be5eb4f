/*
 * oracle_mt.c -- the oracle's ZVC and RLE definitions run on several host
 * threads, for timing the oracle on every host core beside the GPU.
 *
 * TEST INFRASTRUCTURE ONLY, like oracle.c, whose single-threaded functions
 * and helpers it includes: the library built from this file holds both.  The
 * threaded forms compute exactly what the single-threaded loops compute (the
 * tests compare them byte for byte); the pins of the definitions themselves
 * are on oracle.c.
 */
#include "oracle.c"

/* ---- the same definitions on several host threads ------------------------ */
/*
 * For timing the oracle beside the GPU on all host cores.  Windows are
 * independent once each one's place in the stream is known, so every form
 * here is two-phase: each thread first counts what its own range of windows
 * holds, a prefix over the ranges places them, then each thread writes (or
 * decodes) its range.  The streams, outputs and error bits are exactly those
 * of the single-threaded functions above, which the tests check byte for byte.
 */
#include <pthread.h>
#include <stdlib.h>

typedef struct {
    const void *src;        /* elements (compress) */
    const uint8_t *stream;  /* stream (decompress) */
    uint64_t src_bytes;
    uint8_t *dst;
    uint64_t n, w_lo, w_hi; /* window range [w_lo, w_hi) */
    int esz;
    uint64_t count;         /* phase 1 result */
    uint64_t base;          /* phase 2 input: first value index of the range */
    uint32_t *p, *v;        /* RLE: per-window entries / nonzeros */
    uint32_t err;
    int phase;
} mt_job;

static int run_jobs(mt_job *jobs, int threads, void *(*fn)(void *))
{
    pthread_t tid[256];
    int started = 0;
    for (int k = 1; k < threads; k++) {
        if (pthread_create(&tid[k], NULL, fn, &jobs[k]) != 0)
            break;
        started = k;
    }
    fn(&jobs[0]);
    for (int k = started + 1; k < threads; k++)   /* threads that did not start: run here */
        fn(&jobs[k]);
    for (int k = 1; k <= started; k++)
        pthread_join(tid[k], NULL);
    return OR_OK;
}

static int split(mt_job *jobs, int threads, uint64_t windows)
{
    if (threads < 1)
        threads = 1;
    if (threads > 256)
        threads = 256;
    if ((uint64_t)threads > windows)
        threads = windows > 0 ? (int)windows : 1;
    for (int k = 0; k < threads; k++) {
        jobs[k].w_lo = windows * (uint64_t)k / (uint64_t)threads;
        jobs[k].w_hi = windows * (uint64_t)(k + 1) / (uint64_t)threads;
    }
    return threads;
}

static void *zvc_c_job(void *arg)
{
    mt_job *j = (mt_job *)arg;
    uint64_t lo = 32 * j->w_lo, hi = 32 * j->w_hi < j->n ? 32 * j->w_hi : j->n;
    if (j->phase == 0) {
        uint64_t nnz = 0;
        for (uint64_t i = lo; i < hi; i++)
            if (elem(j->src, i, j->esz) != 0)
                nnz++;
        j->count = nnz;
        return NULL;
    }
    for (uint64_t w = j->w_lo; w < j->w_hi; w++) {
        uint32_t mask = 0;
        for (int i = 0; i < 32; i++) {
            uint64_t idx = 32 * w + (uint64_t)i;
            if (idx < j->n && elem(j->src, idx, j->esz) != 0)
                mask |= (uint32_t)1 << i;
        }
        put_le(j->dst + 4 * w, mask, 4);
    }
    uint64_t pos = 4 * ((j->n + 31) / 32) + (uint64_t)j->esz * j->base;
    for (uint64_t i = lo; i < hi; i++) {
        uint64_t v = elem(j->src, i, j->esz);
        if (v != 0) {
            put_le(j->dst + pos, v, j->esz);
            pos += (uint64_t)j->esz;
        }
    }
    return NULL;
}

int oracle_zvc_compress_mt(const void *src, uint64_t n, int esz, uint8_t *dst, uint64_t capacity,
                           uint64_t *out_bytes, int threads)
{
    if (!esz_ok(esz) || !out_bytes)
        return OR_ERR_ARG;
    mt_job jobs[256];
    uint64_t W = (n + 31) / 32;
    int T = split(jobs, threads, W);
    for (int k = 0; k < T; k++) {
        jobs[k].src = src; jobs[k].n = n; jobs[k].esz = esz; jobs[k].dst = dst; jobs[k].phase = 0;
    }
    run_jobs(jobs, T, zvc_c_job);
    uint64_t nnz = 0;
    for (int k = 0; k < T; k++) {
        jobs[k].base = nnz;
        nnz += jobs[k].count;
        jobs[k].phase = 1;
    }
    *out_bytes = 4 * W + (uint64_t)esz * nnz;
    if (*out_bytes > capacity)
        return OR_ERR_CAPACITY;
    if (n > 0)
        run_jobs(jobs, T, zvc_c_job);
    return OR_OK;
}

static void *zvc_d_job(void *arg)
{
    mt_job *j = (mt_job *)arg;
    uint64_t lo = 32 * j->w_lo, hi = 32 * j->w_hi < j->n ? 32 * j->w_hi : j->n;
    if (j->phase == 0) {
        uint64_t c = 0;
        for (uint64_t idx = lo; idx < hi; idx++) {
            uint32_t mask = (uint32_t)get_stream(j->stream, j->src_bytes, 4 * (idx / 32), 4);
            c += (mask >> (idx % 32)) & 1u;
        }
        j->count = c;
        return NULL;
    }
    uint64_t pos = 4 * ((j->n + 31) / 32) + (uint64_t)j->esz * j->base;
    for (uint64_t idx = lo; idx < hi; idx++) {
        uint32_t mask = (uint32_t)get_stream(j->stream, j->src_bytes, 4 * (idx / 32), 4);
        uint64_t v = 0;
        if ((mask >> (idx % 32)) & 1u) {
            v = get_stream(j->stream, j->src_bytes, pos, j->esz);
            pos += (uint64_t)j->esz;
        }
        put_le(j->dst + idx * (uint64_t)j->esz, v, j->esz);
    }
    return NULL;
}

int oracle_zvc_decompress_mt(const uint8_t *src, uint64_t src_bytes, uint64_t n, int esz, void *dst,
                             uint32_t *err, int threads)
{
    if (!esz_ok(esz) || !err)
        return OR_ERR_ARG;
    mt_job jobs[256];
    uint64_t W = (n + 31) / 32;
    int T = split(jobs, threads, W);
    for (int k = 0; k < T; k++) {
        jobs[k].stream = src; jobs[k].src_bytes = src_bytes; jobs[k].n = n; jobs[k].esz = esz;
        jobs[k].dst = (uint8_t *)dst; jobs[k].phase = 0;
    }
    run_jobs(jobs, T, zvc_d_job);
    uint64_t c = 0;
    for (int k = 0; k < T; k++) {
        jobs[k].base = c;
        c += jobs[k].count;
        jobs[k].phase = 1;
    }
    run_jobs(jobs, T, zvc_d_job);
    uint32_t e = 0;
    if (n % 32 != 0) {
        uint32_t last = (uint32_t)get_stream(src, src_bytes, 4 * (W - 1), 4);
        if (last >> (n % 32))
            e |= OR_E_MASK_PAST_N;
    }
    if (4 * W + (uint64_t)esz * c != src_bytes)
        e |= OR_E_SIZE;
    *err = e;
    return OR_OK;
}

static void *rle_c_job(void *arg)
{
    mt_job *j = (mt_job *)arg;
    uint64_t E = rle_window(j->esz), Wr = (j->n + E - 1) / E;
    uint16_t runs[2050];
    for (uint64_t w = j->w_lo; w < j->w_hi; w++) {
        uint64_t lo = w * E, hi = lo + E < j->n ? lo + E : j->n, nz;
        if (j->phase == 0) {
            j->p[w] = (uint32_t)padded(window_runs(j->src, lo, hi, j->esz, NULL, 0, &nz), j->esz);
            j->v[w] = (uint32_t)nz;
            continue;
        }
        /* phase 1: p[] and v[] now hold exclusive prefixes (index Wr = totals) */
        uint64_t r = window_runs(j->src, lo, hi, j->esz, runs, 2050, &nz);
        uint64_t p = padded(r, j->esz);
        if (p > r)
            runs[r] = 0;
        uint64_t pos = 8 * (Wr + 1) + 2 * (uint64_t)j->p[w] + (uint64_t)j->esz * j->v[w];
        put_le(j->dst + 4 * w, j->p[w], 4);
        put_le(j->dst + 4 * (Wr + 1) + 4 * w, j->v[w], 4);
        for (uint64_t k = 0; k < p; k++) {
            put_le(j->dst + pos, runs[k], 2);
            pos += 2;
        }
        for (uint64_t i = lo; i < hi; i++) {
            uint64_t v = elem(j->src, i, j->esz);
            if (v != 0) {
                put_le(j->dst + pos, v, j->esz);
                pos += (uint64_t)j->esz;
            }
        }
    }
    return NULL;
}

int oracle_rle_compress_mt(const void *src, uint64_t n, int esz, uint8_t *dst, uint64_t capacity,
                           uint64_t *out_bytes, int threads)
{
    if (!esz_ok(esz) || !out_bytes)
        return OR_ERR_ARG;
    uint64_t E = rle_window(esz), Wr = (n + E - 1) / E;
    uint32_t *p = (uint32_t *)malloc(4 * (Wr + 1)), *v = (uint32_t *)malloc(4 * (Wr + 1));
    if (!p || !v) {
        free(p);
        free(v);
        return OR_ERR_ARG;
    }
    mt_job jobs[256];
    int T = split(jobs, threads, Wr);
    for (int k = 0; k < T; k++) {
        jobs[k].src = src; jobs[k].n = n; jobs[k].esz = esz; jobs[k].dst = dst;
        jobs[k].p = p; jobs[k].v = v; jobs[k].phase = 0;
    }
    if (Wr > 0)
        run_jobs(jobs, T, rle_c_job);
    uint64_t ent = 0, nnz = 0;
    for (uint64_t w = 0; w < Wr; w++) {  /* exclusive prefixes in place */
        uint64_t a = p[w], b = v[w];
        p[w] = (uint32_t)ent;
        v[w] = (uint32_t)nnz;
        ent += a;
        nnz += b;
    }
    *out_bytes = 8 * (Wr + 1) + 2 * ent + (uint64_t)esz * nnz;
    int rc = OR_OK;
    if (*out_bytes > capacity) {
        rc = OR_ERR_CAPACITY;
    } else {
        for (int k = 0; k < T; k++)
            jobs[k].phase = 1;
        if (Wr > 0)
            run_jobs(jobs, T, rle_c_job);
        put_le(dst + 4 * Wr, ent, 4);
        put_le(dst + 4 * (Wr + 1) + 4 * Wr, nnz, 4);
    }
    free(p);
    free(v);
    return rc;
}

/* one window of the RLE decoder; returns its error bits */
static uint32_t rle_d_window(const uint8_t *src, uint64_t src_bytes, uint64_t n, int esz, uint8_t *out,
                             uint64_t w)
{
    uint64_t E = rle_window(esz), Wr = (n + E - 1) / E, hdr = 8 * (Wr + 1);
    uint32_t e = 0;
    uint64_t r0 = get_stream(src, src_bytes, 4 * w, 4);
    uint64_t r1 = get_stream(src, src_bytes, 4 * (w + 1), 4);
    uint64_t v0 = get_stream(src, src_bytes, 4 * (Wr + 1) + 4 * w, 4);
    uint64_t v1 = get_stream(src, src_bytes, 4 * (Wr + 1) + 4 * (w + 1), 4);
    if (r1 < r0 || v1 < v0)
        return OR_E_INDEX;
    uint64_t lo = w * E, len_w = (lo + E < n ? lo + E : n) - lo;
    uint64_t p = r1 - r0, nv = v1 - v0;
    uint64_t rpos = hdr + 2 * r0 + (uint64_t)esz * v0;
    uint64_t vpos = rpos + 2 * p;
    uint64_t r = p;
    if (p == 0 || p > len_w + 2)
        return OR_E_RUN_FORM;
    if (esz == 4) {
        if (p & 1)
            e |= OR_E_RUN_FORM;
        else if (get_stream(src, src_bytes, rpos + 2 * (p - 1), 2) == 0)
            r = p - 1;
    }
    uint64_t at = 0, nzsum = 0, vk = 0;
    for (uint64_t k = 0; k < r; k++) {
        uint64_t len = get_stream(src, src_bytes, rpos + 2 * k, 2);
        if (len == 0 && k != 0)
            e |= OR_E_RUN_FORM;
        for (uint64_t jj = 0; jj < len; jj++, at++) {
            if (at >= len_w)
                continue;
            uint64_t v = 0;
            if (k & 1) {
                if (vk < nv)
                    v = get_stream(src, src_bytes, vpos + (uint64_t)esz * vk, esz);
                vk++;
            }
            put_le(out + (lo + at) * (uint64_t)esz, v, esz);
        }
        if (k & 1)
            nzsum += len;
    }
    if (at != len_w)
        e |= OR_E_RUN_SUM;
    if (nzsum != nv)
        e |= OR_E_VAL_COUNT;
    return e;
}

static void *rle_d_job(void *arg)
{
    mt_job *j = (mt_job *)arg;
    uint64_t E = rle_window(j->esz);
    uint32_t e = 0;
    for (uint64_t w = j->w_lo; w < j->w_hi; w++) {
        uint64_t lo = w * E, hi = lo + E < j->n ? lo + E : j->n;
        for (uint64_t i = lo * (uint64_t)j->esz; i < hi * (uint64_t)j->esz; i++)
            j->dst[i] = 0;
        e |= rle_d_window(j->stream, j->src_bytes, j->n, j->esz, j->dst, w);
    }
    j->err = e;
    return NULL;
}

int oracle_rle_decompress_mt(const uint8_t *src, uint64_t src_bytes, uint64_t n, int esz, void *dst,
                             uint32_t *err, int threads)
{
    if (!esz_ok(esz) || !err)
        return OR_ERR_ARG;
    uint64_t E = rle_window(esz), Wr = (n + E - 1) / E, hdr = 8 * (Wr + 1);
    uint32_t e = 0;
    if (get_stream(src, src_bytes, 0, 4) != 0 || get_stream(src, src_bytes, 4 * (Wr + 1), 4) != 0)
        e |= OR_E_INDEX;
    mt_job jobs[256];
    int T = split(jobs, threads, Wr);
    for (int k = 0; k < T; k++) {
        jobs[k].stream = src; jobs[k].src_bytes = src_bytes; jobs[k].n = n; jobs[k].esz = esz;
        jobs[k].dst = (uint8_t *)dst; jobs[k].err = 0;
    }
    if (Wr > 0)
        run_jobs(jobs, T, rle_d_job);
    for (int k = 0; k < T; k++)
        e |= jobs[k].err;
    uint64_t rt = get_stream(src, src_bytes, 4 * Wr, 4);
    uint64_t vt = get_stream(src, src_bytes, 4 * (Wr + 1) + 4 * Wr, 4);
    if (hdr + 2 * rt + (uint64_t)esz * vt != src_bytes)
        e |= OR_E_SIZE;
    *err = e;
    return OR_OK;
}
