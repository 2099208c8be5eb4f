/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header or constant table with the HIP library: both are written
 * independently from the same definition.
 *
 * Source: "Compressing DMA Engine: Leveraging Activation Sparsity for Training
 * Deep Neural Networks" (Rhu, O'Connor, Chatterjee, Pool, Keckler,
 * arXiv:1705.01626), §V.A Compression Algorithm, and §VII.A Compression
 * Efficiency for the 4 KB compression window.
 *
 * Every element is handled as its raw little-endian bit pattern of esz bytes
 * (esz = 4 for fp32, 2 for fp16/bf16).  An element is "zero" iff all of its
 * bits are 0; -0.0, denormals, NaN and Inf are nonzero and kept verbatim.
 *
 * ZVC (zero-value compression, §V.A).  Windows of 32 consecutive elements of
 * the flat buffer.  Each window gets a 32-bit mask whose bit i is 1 iff
 * element i of the window is nonzero (an all-zero window therefore becomes one
 * all-zero word: 32x for 4-byte words, as §V.A states); the nonzero elements
 * follow.  Stream = all W = ceil(n/32) masks (u32, little-endian), then every
 * nonzero element in ascending index order.  No header, no padding:
 *     size = 4 * ceil(n/32) + esz * nnz.
 *
 * RLE (run-length variant, §V.A; window of §VII.A).  Windows of E = 4096/esz
 * elements (4 KB).  Each window is described by maximal alternating runs,
 * zero-run first: z0, n0, z1, n1, ... (z0 may be 0, every other run >= 1, the
 * runs sum to the window length), each a u16.  For esz = 4 an odd run list is
 * followed by one 0 entry so the window's values start 4-byte aligned.  With
 * p_w entries (padding included) and v_w nonzeros in window w:
 *     [u32 run_off[Wr+1]] [u32 val_off[Wr+1]] [block_0] ... [block_{Wr-1}]
 *     run_off / val_off = exclusive prefix sums of p_w / v_w, index Wr = totals
 *     block_w = p_w u16 run entries, then its v_w nonzero elements
 *     size = 8(Wr+1) + 2 * sum p_w + esz * nnz.
 *
 * Decoding reads bytes at or beyond src_bytes as 0 and reports what it finds
 * as bits in *err (see OR_E_*).
 */
#include <stdint.h>
#include <stddef.h>

#define OR_OK 0
#define OR_ERR_ARG 1
#define OR_ERR_CAPACITY 2

#define OR_E_MASK_PAST_N   (1u << 0) /* ZVC: a mask bit set for an index >= n */
#define OR_E_SIZE          (1u << 1) /* stream size differs from what it describes */
#define OR_E_INDEX         (1u << 3) /* RLE: index does not start at 0 or decreases */
#define OR_E_RUN_SUM       (1u << 4) /* RLE: runs do not sum to the window length */
#define OR_E_VAL_COUNT     (1u << 5) /* RLE: nonzero runs disagree with val_off */
#define OR_E_RUN_FORM      (1u << 6) /* RLE: zero-length run or bad padding */

/* ---- little-endian byte access ---------------------------------------- */

static uint64_t get_le(const uint8_t *p, int nbytes)
{
    uint64_t v = 0;
    for (int b = 0; b < nbytes; b++)
        v |= (uint64_t)p[b] << (8 * b);
    return v;
}

static void put_le(uint8_t *p, uint64_t v, int nbytes)
{
    for (int b = 0; b < nbytes; b++)
        p[b] = (uint8_t)(v >> (8 * b));
}

/* read nbytes at stream offset off; bytes at or past src_bytes read as 0 */
static uint64_t get_stream(const uint8_t *s, uint64_t src_bytes, uint64_t off, int nbytes)
{
    uint64_t v = 0;
    for (int b = 0; b < nbytes; b++)
        if (off + b < src_bytes)
            v |= (uint64_t)s[off + b] << (8 * b);
    return v;
}

static uint64_t elem(const void *src, uint64_t i, int esz)
{
    return get_le((const uint8_t *)src + i * (uint64_t)esz, esz);
}

static int esz_ok(int esz) { return esz == 2 || esz == 4; }

/* ---- ZVC ---------------------------------------------------------------- */

uint64_t oracle_zvc_size(const void *src, uint64_t n, int esz)
{
    uint64_t nnz = 0;
    for (uint64_t i = 0; i < n; i++)
        if (elem(src, i, esz) != 0)
            nnz++;
    return 4 * ((n + 31) / 32) + (uint64_t)esz * nnz;
}

int oracle_zvc_compress(const void *src, uint64_t n, int esz,
                        uint8_t *dst, uint64_t capacity, uint64_t *out_bytes)
{
    if (!esz_ok(esz) || !out_bytes)
        return OR_ERR_ARG;
    uint64_t size = oracle_zvc_size(src, n, esz);
    *out_bytes = size;
    if (size > capacity)
        return OR_ERR_CAPACITY;
    uint64_t W = (n + 31) / 32;
    /* masks: bit i of word w <-> element 32w+i is nonzero */
    for (uint64_t w = 0; w < W; w++) {
        uint32_t mask = 0;
        for (int i = 0; i < 32; i++) {
            uint64_t idx = 32 * w + (uint64_t)i;
            if (idx < n && elem(src, idx, esz) != 0)
                mask |= (uint32_t)1 << i;
        }
        put_le(dst + 4 * w, mask, 4);
    }
    /* values: nonzero elements in ascending index order */
    uint64_t pos = 4 * W;
    for (uint64_t idx = 0; idx < n; idx++) {
        uint64_t v = elem(src, idx, esz);
        if (v != 0) {
            put_le(dst + pos, v, esz);
            pos += (uint64_t)esz;
        }
    }
    return OR_OK;
}

int oracle_zvc_decompress(const uint8_t *src, uint64_t src_bytes, uint64_t n, int esz,
                          void *dst, uint32_t *err)
{
    if (!esz_ok(esz) || !err)
        return OR_ERR_ARG;
    uint8_t *out = (uint8_t *)dst;
    uint64_t W = (n + 31) / 32;
    uint64_t pos = 4 * W;
    uint32_t e = 0;
    for (uint64_t idx = 0; idx < n; idx++) {
        uint32_t mask = (uint32_t)get_stream(src, src_bytes, 4 * (idx / 32), 4);
        uint64_t v = 0;
        if ((mask >> (idx % 32)) & 1u) {
            v = get_stream(src, src_bytes, pos, esz);
            pos += (uint64_t)esz;
        }
        put_le(out + idx * (uint64_t)esz, v, esz);
    }
    if (n % 32 != 0) {
        uint32_t last = (uint32_t)get_stream(src, src_bytes, 4 * (W - 1), 4);
        if (last >> (n % 32))
            e |= OR_E_MASK_PAST_N;
    }
    if (pos != src_bytes)
        e |= OR_E_SIZE;
    *err = e;
    return OR_OK;
}

/* ---- RLE ---------------------------------------------------------------- */

static uint64_t rle_window(int esz) { return 4096u / (unsigned)esz; }

/*
 * Runs of one window [lo, hi): writes up to cap entries into runs (u16) and
 * returns the entry count before padding.  Zero-run first; a window starting
 * with a nonzero element gets a leading zero-length run.
 */
static uint64_t window_runs(const void *src, uint64_t lo, uint64_t hi, int esz,
                            uint16_t *runs, uint64_t cap, uint64_t *nzcount)
{
    uint64_t r = 0, len = 0, nz = 0;
    int kind = 0; /* 0 = zero run, 1 = nonzero run */
    for (uint64_t i = lo; i < hi; i++) {
        int k = elem(src, i, esz) != 0;
        nz += (uint64_t)k;
        if (k == kind) {
            len++;
        } else {
            if (runs && r < cap)
                runs[r] = (uint16_t)len;
            r++;
            kind = k;
            len = 1;
        }
    }
    if (runs && r < cap)
        runs[r] = (uint16_t)len;
    r++;
    *nzcount = nz;
    return r;
}

static uint64_t padded(uint64_t r, int esz) { return (esz == 4 && (r & 1)) ? r + 1 : r; }

uint64_t oracle_rle_size(const void *src, uint64_t n, int esz)
{
    uint64_t E = rle_window(esz), Wr = (n + E - 1) / E, ent = 0, nnz = 0;
    for (uint64_t w = 0; w < Wr; w++) {
        uint64_t lo = w * E, hi = lo + E < n ? lo + E : n, nz;
        ent += padded(window_runs(src, lo, hi, esz, NULL, 0, &nz), esz);
        nnz += nz;
    }
    return 8 * (Wr + 1) + 2 * ent + (uint64_t)esz * nnz;
}

int oracle_rle_compress(const void *src, uint64_t n, int esz,
                        uint8_t *dst, uint64_t capacity, uint64_t *out_bytes)
{
    if (!esz_ok(esz) || !out_bytes)
        return OR_ERR_ARG;
    uint64_t size = oracle_rle_size(src, n, esz);
    *out_bytes = size;
    if (size > capacity)
        return OR_ERR_CAPACITY;
    uint64_t E = rle_window(esz), Wr = (n + E - 1) / E;
    uint16_t runs[2050];
    uint64_t ent = 0, nnz = 0;
    uint64_t pos = 8 * (Wr + 1);
    for (uint64_t w = 0; w < Wr; w++) {
        uint64_t lo = w * E, hi = lo + E < n ? lo + E : n, nz;
        uint64_t r = window_runs(src, lo, hi, esz, runs, 2050, &nz);
        uint64_t p = padded(r, esz);
        if (p > r)
            runs[r] = 0;
        put_le(dst + 4 * w, ent, 4);             /* run_off[w] */
        put_le(dst + 4 * (Wr + 1) + 4 * w, nnz, 4); /* val_off[w] */
        for (uint64_t k = 0; k < p; k++) {
            put_le(dst + pos, runs[k], 2);
            pos += 2;
        }
        for (uint64_t i = lo; i < hi; i++) {
            uint64_t v = elem(src, i, esz);
            if (v != 0) {
                put_le(dst + pos, v, esz);
                pos += (uint64_t)esz;
            }
        }
        ent += p;
        nnz += nz;
    }
    put_le(dst + 4 * Wr, ent, 4);
    put_le(dst + 4 * (Wr + 1) + 4 * Wr, nnz, 4);
    return OR_OK;
}

int oracle_rle_decompress(const uint8_t *src, uint64_t src_bytes, uint64_t n, int esz,
                          void *dst, uint32_t *err)
{
    if (!esz_ok(esz) || !err)
        return OR_ERR_ARG;
    uint8_t *out = (uint8_t *)dst;
    uint64_t E = rle_window(esz), Wr = (n + E - 1) / E;
    uint64_t hdr = 8 * (Wr + 1);
    uint32_t e = 0;
    for (uint64_t i = 0; i < n * (uint64_t)esz; i++)
        out[i] = 0;
    if (get_stream(src, src_bytes, 0, 4) != 0 || get_stream(src, src_bytes, 4 * (Wr + 1), 4) != 0)
        e |= OR_E_INDEX;
    for (uint64_t w = 0; w < Wr; w++) {
        uint64_t r0 = get_stream(src, src_bytes, 4 * w, 4);
        uint64_t r1 = get_stream(src, src_bytes, 4 * (w + 1), 4);
        uint64_t v0 = get_stream(src, src_bytes, 4 * (Wr + 1) + 4 * w, 4);
        uint64_t v1 = get_stream(src, src_bytes, 4 * (Wr + 1) + 4 * (w + 1), 4);
        if (r1 < r0 || v1 < v0) {
            e |= OR_E_INDEX;
            continue;
        }
        uint64_t lo = w * E, len_w = (lo + E < n ? lo + E : n) - lo;
        uint64_t p = r1 - r0, nv = v1 - v0;
        uint64_t rpos = hdr + 2 * r0 + (uint64_t)esz * v0; /* block start */
        uint64_t vpos = rpos + 2 * p;                      /* values start */
        /* number of real runs: padding is a trailing 0 after an odd list */
        uint64_t r = p;
        if (p == 0 || p > len_w + 2) {
            e |= OR_E_RUN_FORM;
            continue;
        }
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
            for (uint64_t j = 0; j < len; j++, at++) {
                if (at >= len_w)
                    continue;
                uint64_t v = 0;
                if (k & 1) { /* odd entries are nonzero runs */
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
    }
    {
        uint64_t rt = get_stream(src, src_bytes, 4 * Wr, 4);
        uint64_t vt = get_stream(src, src_bytes, 4 * (Wr + 1) + 4 * Wr, 4);
        if (hdr + 2 * rt + (uint64_t)esz * vt != src_bytes)
            e |= OR_E_SIZE;
    }
    *err = e;
    return OR_OK;
}

/* ---- ZVC, per-window interleaved form with a block index ----------------- */
/*
 * The page's literal description of ZVC (§V.A): a window's 32-bit mask is
 * followed by that window's nonzero values.  Windows follow each other in
 * order; an index of u32 val_off[Wr+1] (nonzeros before each block of
 * E = 4096/esz elements, the 4 KB window of §VII.A; entry Wr = the total) lets
 * each block be found without reading the ones before it:
 *     [u32 val_off[Wr+1]] [mask_0][values_0] [mask_1][values_1] ...
 *     block b starts at 4(Wr+1) + 4 * b * (E/32) + esz * val_off[b]
 *     size = 4(Wr+1) + 4 * ceil(n/32) + esz * nnz.
 */
static uint64_t zvci_block(int esz) { return (uint64_t)(4096 / esz); } /* elements per 4 KB */

uint64_t oracle_zvci_size(const void *src, uint64_t n, int esz)
{
    uint64_t E = zvci_block(esz), Wr = (n + E - 1) / E, nnz = 0;
    for (uint64_t i = 0; i < n; i++)
        if (elem(src, i, esz) != 0)
            nnz++;
    return 4 * (Wr + 1) + 4 * ((n + 31) / 32) + (uint64_t)esz * nnz;
}

int oracle_zvci_compress(const void *src, uint64_t n, int esz,
                         uint8_t *dst, uint64_t capacity, uint64_t *out_bytes)
{
    if (!esz_ok(esz) || !out_bytes)
        return OR_ERR_ARG;
    uint64_t size = oracle_zvci_size(src, n, esz);
    *out_bytes = size;
    if (size > capacity)
        return OR_ERR_CAPACITY;
    uint64_t E = zvci_block(esz), Wr = (n + E - 1) / E, W = (n + 31) / 32;
    uint64_t pos = 4 * (Wr + 1), nnz = 0;
    for (uint64_t w = 0; w < W; w++) {
        if ((32 * w) % E == 0)
            put_le(dst + 4 * ((32 * w) / E), nnz, 4); /* val_off of the block w opens */
        uint32_t mask = 0;
        for (int i = 31; i >= 0; i--) { /* bit i <-> element 32w + i */
            uint64_t idx = 32 * w + (uint64_t)i;
            mask <<= 1;
            if (idx < n && elem(src, idx, esz))
                mask |= 1u;
        }
        put_le(dst + pos, mask, 4);
        pos += 4;
        for (int i = 0; i < 32; i++) {
            uint64_t idx = 32 * w + (uint64_t)i;
            if ((mask >> i) & 1u) {
                put_le(dst + pos, elem(src, idx, esz), esz);
                pos += (uint64_t)esz;
                nnz++;
            }
        }
    }
    put_le(dst + 4 * Wr, nnz, 4);
    return OR_OK;
}

int oracle_zvci_decompress(const uint8_t *src, uint64_t src_bytes, uint64_t n, int esz,
                           void *dst, uint32_t *err)
{
    if (!esz_ok(esz) || !err)
        return OR_ERR_ARG;
    uint8_t *out = (uint8_t *)dst;
    uint64_t E = zvci_block(esz), Wr = (n + E - 1) / E, W = (n + 31) / 32;
    uint64_t hdr = 4 * (Wr + 1), wpb = E / 32;
    uint32_t e = 0;
    for (uint64_t i = 0; i < n * (uint64_t)esz; i++)
        out[i] = 0;
    if (get_stream(src, src_bytes, 0, 4) != 0)
        e |= OR_E_INDEX;
    for (uint64_t b = 0; b < Wr; b++) {
        uint64_t v0 = get_stream(src, src_bytes, 4 * b, 4);
        uint64_t v1 = get_stream(src, src_bytes, 4 * (b + 1), 4);
        if (v1 < v0) {
            e |= OR_E_INDEX;
            continue;
        }
        /* every block is decoded from its own index entry */
        uint64_t pos = hdr + 4 * b * wpb + (uint64_t)esz * v0, count = 0;
        for (uint64_t w = b * wpb; w < W && w < (b + 1) * wpb; w++) {
            uint32_t mask = (uint32_t)get_stream(src, src_bytes, pos, 4);
            pos += 4;
            for (int i = 0; i < 32; i++) {
                if (!((mask >> i) & 1u))
                    continue;
                uint64_t idx = 32 * w + (uint64_t)i;
                count++;
                if (idx >= n) {
                    e |= OR_E_MASK_PAST_N;
                    continue;
                }
                put_le(out + idx * (uint64_t)esz, get_stream(src, src_bytes, pos, esz), esz);
                pos += (uint64_t)esz;
            }
        }
        if (count != v1 - v0)
            e |= OR_E_VAL_COUNT;
    }
    if (hdr + 4 * W + (uint64_t)esz * get_stream(src, src_bytes, 4 * Wr, 4) != src_bytes)
        e |= OR_E_SIZE;
    *err = e;
    return OR_OK;
}

/* ---- ReLU of the producing layer (fused epilogue) ------------------------ */
/*
 * ReLU(x) = max(x, 0), written out on the element's sign, exponent and
 * mantissa fields (IEEE-754 binary32 / binary16, and bfloat16 = the top half
 * of a binary32).  A NaN (exponent all ones, mantissa not zero) passes
 * unchanged whatever its sign; any other value whose sign bit is set
 * (-0.0, negative denormals and normals, -inf) becomes +0.0; everything else
 * passes unchanged.  fmt: 0 = fp32, 1 = fp16, 2 = bf16.
 */
int oracle_relu(const void *src, uint64_t n, int fmt, void *dst)
{
    int esz, exp_bits, man_bits;
    if (fmt == 0) { esz = 4; exp_bits = 8; man_bits = 23; }
    else if (fmt == 1) { esz = 2; exp_bits = 5; man_bits = 10; }
    else if (fmt == 2) { esz = 2; exp_bits = 8; man_bits = 7; }
    else return OR_ERR_ARG;
    for (uint64_t i = 0; i < n; i++) {
        uint64_t v = elem(src, i, esz);
        uint64_t sign = v >> (exp_bits + man_bits);
        uint64_t exponent = (v >> man_bits) & (((uint64_t)1 << exp_bits) - 1);
        uint64_t mantissa = v & (((uint64_t)1 << man_bits) - 1);
        int is_nan = exponent == ((uint64_t)1 << exp_bits) - 1 && mantissa != 0;
        uint64_t y = (sign && !is_nan) ? 0 : v;
        put_le((uint8_t *)dst + i * (uint64_t)esz, y, esz);
    }
    return OR_OK;
}
