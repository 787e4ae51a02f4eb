/*
 * rans_oracle.c -- plain, single-threaded CPU reference of indexed rANS64.
 *
 * TEST INFRASTRUCTURE ONLY (see rans_oracle.h): called by the tests, the
 * smoke check and the benchmark's CPU-baseline leg, never by the product.
 *
 * The pages name the coder but do not print its procedure:
 *   - kompressor README, "Why" and "Credits": a faithful port of CompressAI's
 *     rANS coder, 64-bit rANS in the style of ryg_rans;
 *   - torch_ans 0.3.0, "Usage" table: rans64 has a 64-bit state, 32-bit
 *     stream words and at most 16 frequency bits, and in the legend
 *     State Bits > Stream Bits + Max Freq Bits;
 *   - torch_ans 0.3.0, "Low-level API Reference", rans*_push: symbols are
 *     chosen per position by an index into batched CDF tables with sizes and
 *     offsets; the coded range is [offset, offset + cdf_size - 2); a symbol
 *     outside it is zig-zag encoded into a raw value and sent by bypass
 *     coding with bypass_precision bits at a time;
 *   - kompressor BENCHMARKS.md, section 4: CompressAI's decoder finds the
 *     symbol by a linear scan of the CDF row (std::find_if) -- this oracle
 *     does exactly that, the plainest lookup there is.
 *
 * Readings taken where the pages are silent:
 *   R1  state interval [L0, 2^63) with L0 = 2^31, the interval of 64-bit
 *       ryg_rans with 32-bit output; with 16-bit precision a REG put
 *       renormalises when x >= f * 2^47 and a 4-bit put when x >= 2^59;
 *   R3  the encoder starts every lane at x = L0, so a clean decode ends at
 *       x = L0 with every lane word consumed;
 *   R4  bypass_precision = 4;
 *   R5  the raw value is sent as a count of 4-bit groups nb (base-15
 *       continuation: 15 means "add the next group"), then the nb groups
 *       least significant first; raw < 2^31 so nb <= 8;
 *   R6  zig-zag: v < 0 -> raw = -2v-1 (odd); v >= mv -> raw = 2(v-mv) (even);
 *   R7  a 4-bit put is x <- 16x + b (not a REG put with frequency 2^12);
 *   R8  raw >= 2^31 is rejected with ORACLE_E_SYMBOL_RANGE;
 *   R9  the terminal CDF entry is exactly 65536 and every frequency >= 1;
 *   R10 lane j covers [floor(j n / L), floor((j+1) n / L));
 *   R11 container [L, end_0..end_{L-1}] + lane streams;
 *   R2  each lane stream starts with the final state as two words (low then
 *       high), followed by the renormalisation words in the order the
 *       decoder consumes them (the reverse of the order they were emitted).
 */
#include "rans_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define PREC 16u
#define TOTAL_FREQ (1u << PREC)
#define STATE_LOW (1ull << 31)      /* L0 */
#define BYPASS_BITS 4u
#define BYPASS_MAX 15u              /* 2^BYPASS_BITS - 1: count continuation */
#define RAW_LIMIT (1ll << 31)

uint64_t oracle_lane_begin(uint64_t n, uint32_t num_lanes, uint32_t j)
{
    /* floor(j * n / L) without overflow: n < 2^63 and j <= L < 2^32, so
     * split n = a*L + b: j*n/L = j*a + j*b/L with j*b < 2^64. */
    uint64_t a = n / num_lanes, b = n % num_lanes;
    return (uint64_t)j * a + ((uint64_t)j * b) / num_lanes;
}

int oracle_check_tables(const int32_t *cdf, const int32_t *lengths,
                        int32_t num_tables, int32_t stride)
{
    if (num_tables <= 0 || stride < 3)
        return ORACLE_E_ARG;
    for (int32_t r = 0; r < num_tables; ++r) {
        int32_t len = lengths[r];
        const int32_t *row = cdf + (int64_t)r * stride;
        if (len < 3 || len > stride)
            return ORACLE_E_TABLE;
        if (row[0] != 0 || row[len - 1] != (int32_t)TOTAL_FREQ)
            return ORACLE_E_TABLE;
        for (int32_t k = 0; k + 1 < len; ++k)
            if (row[k + 1] <= row[k])
                return ORACLE_E_TABLE;
    }
    return ORACLE_OK;
}

/* One elementary coding step, in the order the decoder meets it. */
typedef struct {
    uint32_t start;   /* REG: cumulative frequency; BITS: the 4-bit value */
    uint32_t freq;    /* REG: frequency; BITS: 0 */
} put_t;

typedef struct {
    put_t *v;
    size_t n, cap;
} put_list;

static int put_push(put_list *l, uint32_t start, uint32_t freq)
{
    if (l->n == l->cap) {
        size_t nc = l->cap ? 2 * l->cap : 64;
        put_t *nv = (put_t *)realloc(l->v, nc * sizeof(put_t));
        if (!nv)
            return ORACLE_E_ARG;
        l->v = nv;
        l->cap = nc;
    }
    l->v[l->n].start = start;
    l->v[l->n].freq = freq;
    l->n++;
    return ORACLE_OK;
}

/* Forward-order puts of one symbol (torch_ans rans*_push range rule). */
static int symbol_puts(put_list *l, int32_t symbol, int32_t index,
                       const int32_t *cdf, const int32_t *lengths,
                       const int32_t *offsets, int32_t num_tables, int32_t stride)
{
    if (index < 0 || index >= num_tables)
        return ORACLE_E_INDEX;
    const int32_t *row = cdf + (int64_t)index * stride;
    int64_t mv = (int64_t)lengths[index] - 2;  /* escape slot */
    int64_t v = (int64_t)symbol - (int64_t)offsets[index];
    int64_t raw = 0;
    int escape = 0;
    if (v < 0) {
        raw = -2 * v - 1;
        v = mv;
        escape = 1;
    } else if (v >= mv) {
        raw = 2 * (v - mv);
        v = mv;
        escape = 1;
    }
    if (raw >= RAW_LIMIT)
        return ORACLE_E_SYMBOL_RANGE;
    int rc = put_push(l, (uint32_t)row[v], (uint32_t)(row[v + 1] - row[v]));
    if (rc)
        return rc;
    if (escape) {
        uint32_t nb = 0;
        while (nb < 16 && ((uint64_t)raw >> (BYPASS_BITS * nb)) != 0)
            ++nb;
        uint32_t t = nb;
        while (t >= BYPASS_MAX) {
            if ((rc = put_push(l, BYPASS_MAX, 0)))
                return rc;
            t -= BYPASS_MAX;
        }
        if ((rc = put_push(l, t, 0)))
            return rc;
        for (uint32_t k = 0; k < nb; ++k)
            if ((rc = put_push(l, (uint32_t)(((uint64_t)raw >> (BYPASS_BITS * k)) & BYPASS_MAX), 0)))
                return rc;
    }
    return ORACLE_OK;
}

/* Apply one put to state *x (S3), appending the word a renormalisation
 * emits to emitted[*ne]. */
static void apply_put(uint64_t *x, put_t p, uint32_t *emitted, size_t *ne)
{
    if (p.freq == 0) {
        /* 4-bit put: keep 16x + b below 2^63. */
        if (*x >= (1ull << (63 - BYPASS_BITS))) {
            emitted[(*ne)++] = (uint32_t)*x;
            *x >>= 32;
        }
        *x = (*x << BYPASS_BITS) + p.start;
    } else {
        /* REG put: keep floor(x/f)*2^16 + (x mod f) + start below 2^63. */
        uint64_t x_max = (uint64_t)p.freq << (63 - PREC);
        if (*x >= x_max) {
            emitted[(*ne)++] = (uint32_t)*x;
            *x >>= 32;
        }
        *x = (*x / p.freq) * TOTAL_FREQ + (*x % p.freq) + p.start;
    }
}

/* One lane; with num_cuts > 0 it also records, for each cut position c
 * (ascending, begin <= c <= end), the state once every position from c on
 * has been coded and the number of words emitted so far: the state a
 * decoder holds just before position c, and the count of lane words still
 * unread there (split metadata). */
static int encode_lane_cuts(const int32_t *symbols, const int32_t *indexes,
                            uint64_t begin, uint64_t end,
                            const int32_t *cdf, const int32_t *lengths,
                            const int32_t *offsets, int32_t num_tables, int32_t stride,
                            uint32_t *out, uint64_t cap, uint64_t *words,
                            const uint64_t *cuts, uint32_t num_cuts, uint32_t *cut_meta)
{
    put_list puts = {0, 0, 0};
    int rc = ORACLE_OK;
    /* first put of each position, and one past the last position's */
    size_t *first = (size_t *)malloc((end - begin + 1) * sizeof(size_t));
    if (!first)
        return ORACLE_E_ARG;
    for (uint64_t i = begin; i < end && rc == ORACLE_OK; ++i) {
        first[i - begin] = puts.n;
        rc = symbol_puts(&puts, symbols[i], indexes[i], cdf, lengths, offsets,
                         num_tables, stride);
    }
    first[end - begin] = puts.n;
    if (rc) {
        free(first);
        free(puts.v);
        return rc;
    }

    /* Emitted words, in emission order; at most one per put. */
    uint32_t *emitted = (uint32_t *)malloc((puts.n + 1) * sizeof(uint32_t));
    if (!emitted) {
        free(first);
        free(puts.v);
        return ORACLE_E_ARG;
    }
    size_t ne = 0;
    uint64_t x = STATE_LOW;
    /* positions last to first; each position's puts last to first */
    for (uint64_t i = end + 1; i-- > begin;) {
        if (i < end) {
            for (size_t k = first[i + 1 - begin]; k-- > first[i - begin];)
                apply_put(&x, puts.v[k], emitted, &ne);
        }
        for (uint32_t c = 0; c < num_cuts; ++c)
            if (cuts[c] == i) {
                cut_meta[3 * c] = (uint32_t)x;
                cut_meta[3 * c + 1] = (uint32_t)(x >> 32);
                cut_meta[3 * c + 2] = (uint32_t)ne;
            }
    }
    free(first);
    uint64_t total = 2 + ne;
    *words = total;
    if (total <= cap) {
        out[0] = (uint32_t)x;
        out[1] = (uint32_t)(x >> 32);
        for (size_t k = 0; k < ne; ++k)
            out[2 + k] = emitted[ne - 1 - k];
    } else {
        rc = ORACLE_E_CAPACITY;
    }
    free(emitted);
    free(puts.v);
    return rc;
}

int oracle_encode_lane(const int32_t *symbols, const int32_t *indexes,
                       uint64_t begin, uint64_t end,
                       const int32_t *cdf, const int32_t *lengths,
                       const int32_t *offsets, int32_t num_tables, int32_t stride,
                       uint32_t *out, uint64_t cap, uint64_t *words)
{
    return encode_lane_cuts(symbols, indexes, begin, end, cdf, lengths, offsets, num_tables,
                            stride, out, cap, words, NULL, 0, NULL);
}

typedef struct {
    uint64_t x;
    const uint32_t *w;
    uint64_t pos, words;
} dec_t;

/* x < L0 after a step means the encoder emitted a word there: read it back. */
static int dec_refill(dec_t *d)
{
    if (d->x < STATE_LOW) {
        if (d->pos >= d->words)
            return ORACLE_E_CORRUPT;
        d->x = (d->x << 32) | d->w[d->pos++];
    }
    return ORACLE_OK;
}

static int dec_bits(dec_t *d, uint32_t *b)
{
    *b = (uint32_t)(d->x & BYPASS_MAX);
    d->x >>= BYPASS_BITS;
    return dec_refill(d);
}

/* Decode positions [begin, end) from state d->x, reading lane words from
 * d->pos on. */
static int decode_range(dec_t *dd, const int32_t *indexes, uint64_t begin, uint64_t end,
                        const int32_t *cdf, const int32_t *lengths,
                        const int32_t *offsets, int32_t num_tables, int32_t stride,
                        int32_t *symbols_out)
{
    dec_t d = *dd;
    for (uint64_t i = begin; i < end; ++i) {
        int32_t index = indexes[i];
        if (index < 0 || index >= num_tables)
            return ORACLE_E_INDEX;
        const int32_t *row = cdf + (int64_t)index * stride;
        int32_t len = lengths[index];
        int64_t mv = (int64_t)len - 2;
        uint32_t cum = (uint32_t)(d.x & (TOTAL_FREQ - 1));
        /* linear scan: first entry above cum, minus one */
        int32_t s = 0;
        while (s + 1 < len && (uint32_t)row[s + 1] <= cum)
            ++s;
        uint32_t start = (uint32_t)row[s];
        uint32_t freq = (uint32_t)(row[s + 1] - row[s]);
        d.x = (uint64_t)freq * (d.x >> PREC) + cum - start;
        if (dec_refill(&d))
            return ORACLE_E_CORRUPT;
        int64_t value = s;
        if (s == mv) {
            uint32_t t, nb;
            if (dec_bits(&d, &t))
                return ORACLE_E_CORRUPT;
            nb = t;
            while (t == BYPASS_MAX) {
                if (dec_bits(&d, &t))
                    return ORACLE_E_CORRUPT;
                nb += t;
                if (nb > 8)
                    return ORACLE_E_CORRUPT;
            }
            if (nb > 8)
                return ORACLE_E_CORRUPT;
            uint64_t raw = 0;
            for (uint32_t k = 0; k < nb; ++k) {
                uint32_t b;
                if (dec_bits(&d, &b))
                    return ORACLE_E_CORRUPT;
                raw |= (uint64_t)b << (BYPASS_BITS * k);
            }
            if (raw >= (uint64_t)RAW_LIMIT)
                return ORACLE_E_CORRUPT;
            if (raw & 1)
                value = -(int64_t)(raw >> 1) - 1;
            else
                value = (int64_t)(raw >> 1) + mv;
        }
        int64_t sym = value + offsets[index];
        if (sym < INT32_MIN || sym > INT32_MAX)
            return ORACLE_E_CORRUPT;
        symbols_out[i] = (int32_t)sym;
    }
    *dd = d;
    return ORACLE_OK;
}

int oracle_decode_lane(const uint32_t *lane, uint64_t words,
                       const int32_t *indexes, uint64_t begin, uint64_t end,
                       const int32_t *cdf, const int32_t *lengths,
                       const int32_t *offsets, int32_t num_tables, int32_t stride,
                       int32_t *symbols_out)
{
    if (words < 2)
        return ORACLE_E_CORRUPT;
    dec_t d;
    d.x = (uint64_t)lane[0] | ((uint64_t)lane[1] << 32);
    d.w = lane;
    d.pos = 2;
    d.words = words;
    int rc = decode_range(&d, indexes, begin, end, cdf, lengths, offsets, num_tables, stride,
                          symbols_out);
    if (rc)
        return rc;
    if (d.x != STATE_LOW || d.pos != d.words)
        return ORACLE_E_CORRUPT;
    return ORACLE_OK;
}

/* Piece s of a lane [b, e) starts at b + floor(s (e - b) / pieces). */
static uint64_t piece_begin(uint64_t b, uint64_t e, uint32_t pieces, uint32_t s)
{
    return b + (uint64_t)(((unsigned __int128)(e - b) * s) / pieces);
}

int oracle_encode_split(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                        const int32_t *cdf, const int32_t *lengths, const int32_t *offsets,
                        int32_t num_tables, int32_t stride, uint32_t num_lanes,
                        uint32_t pieces, uint32_t *out, uint64_t cap, uint64_t *out_words,
                        uint32_t *split_meta)
{
    if (num_lanes == 0 || pieces == 0 || (n && (!symbols || !indexes)) || !cdf || !lengths ||
        !offsets || (pieces > 1 && !split_meta))
        return ORACLE_E_ARG;
    uint64_t cuts[64];
    if (pieces > 65)
        return ORACLE_E_ARG;
    int rc = oracle_check_tables(cdf, lengths, num_tables, stride);
    if (rc)
        return rc;
    uint64_t head = 1 + (uint64_t)num_lanes;
    uint64_t used = 0;   /* payload words so far */
    int cap_hit = 0;
    uint32_t *scratch = NULL;
    uint64_t scratch_cap = 0;
    for (uint32_t j = 0; j < num_lanes; ++j) {
        uint64_t b = oracle_lane_begin(n, num_lanes, j);
        uint64_t e = oracle_lane_begin(n, num_lanes, j + 1);
        /* a generous bound: each symbol makes at most 10 puts, one word each */
        uint64_t need = 2 + 10 * (e - b);
        if (need > scratch_cap) {
            free(scratch);
            scratch = (uint32_t *)malloc(need * sizeof(uint32_t));
            if (!scratch)
                return ORACLE_E_ARG;
            scratch_cap = need;
        }
        uint64_t w = 0;
        for (uint32_t s = 1; s < pieces; ++s)
            cuts[s - 1] = piece_begin(b, e, pieces, s);
        rc = encode_lane_cuts(symbols, indexes, b, e, cdf, lengths, offsets, num_tables, stride,
                              scratch, scratch_cap, &w, cuts, pieces - 1,
                              pieces > 1 ? split_meta + 3ull * (pieces - 1) * j : NULL);
        if (rc) {
            free(scratch);
            return rc;
        }
        if (head + used + w <= cap && !cap_hit)
            memcpy(out + head + used, scratch, w * sizeof(uint32_t));
        else
            cap_hit = 1;
        used += w;
        if (used > 0xFFFFFFFFull) {
            free(scratch);
            return ORACLE_E_ARG;
        }
        if (1 + j < cap)
            out[1 + j] = (uint32_t)used;
    }
    free(scratch);
    if (cap >= 1)
        out[0] = num_lanes;
    *out_words = head + used;
    return (cap_hit || head > cap) ? ORACLE_E_CAPACITY : ORACLE_OK;
}

int oracle_encode(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                  const int32_t *cdf, const int32_t *lengths, const int32_t *offsets,
                  int32_t num_tables, int32_t stride, uint32_t num_lanes,
                  uint32_t *out, uint64_t cap, uint64_t *out_words)
{
    return oracle_encode_split(symbols, indexes, n, cdf, lengths, offsets, num_tables, stride,
                               num_lanes, 1, out, cap, out_words, NULL);
}

int oracle_decode_split(const uint32_t *stream, uint64_t stream_words,
                        const int32_t *indexes, uint64_t n,
                        const int32_t *cdf, const int32_t *lengths, const int32_t *offsets,
                        int32_t num_tables, int32_t stride, uint32_t num_lanes,
                        uint32_t pieces, const uint32_t *split_meta, int32_t *symbols_out)
{
    if (num_lanes == 0 || pieces == 0 || pieces > 65 || !stream ||
        (n && (!indexes || !symbols_out)) || (pieces > 1 && !split_meta))
        return ORACLE_E_ARG;
    int rc = oracle_check_tables(cdf, lengths, num_tables, stride);
    if (rc)
        return rc;
    uint64_t head = 1 + (uint64_t)num_lanes;
    if (stream_words < head || stream[0] != num_lanes)
        return ORACLE_E_CORRUPT;
    uint64_t prev = 0;
    for (uint32_t j = 0; j < num_lanes; ++j) {
        uint64_t endj = stream[1 + j];
        if (endj < prev + 2 || head + endj > stream_words)
            return ORACLE_E_CORRUPT;
        prev = endj;
    }
    prev = 0;
    for (uint32_t j = 0; j < num_lanes; ++j) {
        uint64_t endj = stream[1 + j];
        uint64_t b = oracle_lane_begin(n, num_lanes, j);
        uint64_t e = oracle_lane_begin(n, num_lanes, j + 1);
        const uint32_t *lane = stream + head + prev;
        uint64_t W = endj - prev;
        /* piece s starts from the lane's flushed state (s = 0) or from its
         * split record: the state, and the count of lane words left unread */
        for (uint32_t s = 0; s < pieces; ++s) {
            dec_t d;
            d.w = lane;
            d.words = W;
            if (s == 0) {
                d.x = (uint64_t)lane[0] | ((uint64_t)lane[1] << 32);
                d.pos = 2;
            } else {
                const uint32_t *m = split_meta + 3ull * ((uint64_t)(pieces - 1) * j + s - 1);
                if ((uint64_t)m[2] > W - 2)
                    return ORACLE_E_CORRUPT;
                d.x = (uint64_t)m[0] | ((uint64_t)m[1] << 32);
                d.pos = W - m[2];
            }
            rc = decode_range(&d, indexes, piece_begin(b, e, pieces, s),
                              piece_begin(b, e, pieces, s + 1), cdf, lengths, offsets,
                              num_tables, stride, symbols_out);
            if (rc)
                return rc;
            uint64_t want_x = STATE_LOW, want_pos = W;
            if (s + 1 < pieces) {
                const uint32_t *m = split_meta + 3ull * ((uint64_t)(pieces - 1) * j + s);
                if ((uint64_t)m[2] > W - 2)
                    return ORACLE_E_CORRUPT;
                want_x = (uint64_t)m[0] | ((uint64_t)m[1] << 32);
                want_pos = W - m[2];
            }
            if (d.x != want_x || d.pos != want_pos)
                return ORACLE_E_CORRUPT;
        }
        prev = endj;
    }
    return ORACLE_OK;
}

int oracle_decode(const uint32_t *stream, uint64_t stream_words,
                  const int32_t *indexes, uint64_t n,
                  const int32_t *cdf, const int32_t *lengths, const int32_t *offsets,
                  int32_t num_tables, int32_t stride, uint32_t num_lanes,
                  int32_t *symbols_out)
{
    return oracle_decode_split(stream, stream_words, indexes, n, cdf, lengths, offsets,
                               num_tables, stride, num_lanes, 1, NULL, symbols_out);
}

/* ---- Quantised CDF tables ------------------------------------------------
 *
 * What the pages fix: the coder consumes 16-bit quantised CDF rows, one per
 * distribution, each holding the alphabet, an escape slot for bypass coding
 * and the terminal entry (torch_ans 0.3.0, "Range limit" under rans*_push);
 * the coder itself turns batched pmfs into such rows ("Parameter Setup" and
 * "Other Features": init_params converts PMF to CDF internally), and the
 * mean-scale model's y latent uses 64 rows of at most 3133 entries
 * (kompressor BENCHMARKS.md, section 4: 200,512 marshalled cdf entries).
 * The quantisation procedure and the discretised Gaussian are readings:
 *   T1  pmf entry k becomes f_k = max(1, round-half-even(p_k * 2^16)), the
 *       escape slot being the last entry of the pmf row;
 *   T2  the frequencies are then brought to a sum of exactly 2^16 one unit
 *       at a time, each unit taken from (surplus) or given to (deficit) the
 *       currently largest frequency, the lowest slot among equals; a
 *       frequency never drops below 1 (possible whenever the row has at most
 *       2^16 entries);
 *   T3  the Gaussian row of scale s: half-width c = ceil(s * z) for a given
 *       standard-normal quantile z (z = 6.1094... for a two-sided tail mass
 *       of 1e-9); slot k = 0..2c holds symbol v = k - c with mass
 *       Phi((v + 1/2) / s) - Phi((v - 1/2) / s); the escape slot holds the
 *       mass of both tails beyond c + 1/2, 2 Phi(-(c + 1/2) / s); offset -c,
 *       length 2c + 3, entries past the length set to 2^16;
 *   T4  Phi(x) = erfc(-x / sqrt(2)) / 2, all of it in double precision.
 */

static double std_normal_cdf(double x)
{
    return 0.5 * erfc(-x * 0.70710678118654752440);
}

int oracle_quantize_pmf(const double *pmf, int32_t m, int32_t *cdf)
{
    if (!pmf || !cdf || m < 2 || m > (int32_t)TOTAL_FREQ)
        return ORACLE_E_ARG;
    int64_t *f = (int64_t *)malloc((size_t)m * sizeof(int64_t));
    if (!f)
        return ORACLE_E_ARG;
    int64_t sum = 0;
    for (int32_t k = 0; k < m; ++k) {
        double p = pmf[k];
        if (!(p >= 0.0 && p <= 1.0)) {   /* also refuses NaN */
            free(f);
            return ORACLE_E_TABLE;
        }
        f[k] = (int64_t)rint(p * TOTAL_FREQ);   /* default rounding: half to even */
        if (f[k] < 1)
            f[k] = 1;
        sum += f[k];
    }
    int64_t excess = sum - (int64_t)TOTAL_FREQ;
    while (excess != 0) {
        int32_t top = 0;   /* the first slot of the largest frequency */
        for (int32_t k = 1; k < m; ++k)
            if (f[k] > f[top])
                top = k;
        if (excess > 0) {
            f[top] -= 1;   /* f[top] >= 2 here: sum > 2^16 >= m */
            excess -= 1;
        } else {
            f[top] += 1;
            excess += 1;
        }
    }
    cdf[0] = 0;
    for (int32_t k = 0; k < m; ++k)
        cdf[k + 1] = cdf[k] + (int32_t)f[k];
    free(f);
    return ORACLE_OK;
}

int oracle_gaussian_row(double scale, double tail_z, int32_t stride, int32_t *cdf_row,
                        int32_t *length, int32_t *offset)
{
    if (!cdf_row || !length || !offset || stride < 3)
        return ORACLE_E_ARG;
    if (!(scale > 0.0) || !(tail_z > 0.0))
        return ORACLE_E_TABLE;
    double cw = ceil(scale * tail_z);
    if (!(2.0 * cw + 3.0 <= (double)stride))
        return ORACLE_E_TABLE;
    int32_t c = (int32_t)cw;
    int32_t m = 2 * c + 2;   /* 2c + 1 symbols and the escape slot */
    double *pmf = (double *)malloc((size_t)m * sizeof(double));
    if (!pmf)
        return ORACLE_E_ARG;
    for (int32_t k = 0; k <= 2 * c; ++k) {
        double v = (double)(k - c);
        pmf[k] = std_normal_cdf((v + 0.5) / scale) - std_normal_cdf((v - 0.5) / scale);
    }
    pmf[m - 1] = 2.0 * std_normal_cdf(-((double)c + 0.5) / scale);
    int rc = oracle_quantize_pmf(pmf, m, cdf_row);
    free(pmf);
    if (rc)
        return rc;
    for (int32_t k = m + 1; k < stride; ++k)
        cdf_row[k] = (int32_t)TOTAL_FREQ;
    *length = m + 1;
    *offset = -c;
    return ORACLE_OK;
}

int oracle_gaussian_tables(const double *scales, int32_t num_tables, double tail_z,
                           int32_t stride, int32_t *cdf, int32_t *lengths, int32_t *offsets)
{
    if (!scales || num_tables <= 0)
        return ORACLE_E_ARG;
    for (int32_t r = 0; r < num_tables; ++r) {
        int rc = oracle_gaussian_row(scales[r], tail_z, stride, cdf + (int64_t)r * stride,
                                     lengths + r, offsets + r);
        if (rc)
            return rc;
    }
    return ORACLE_OK;
}

/* ---- Latent front end ------------------------------------------------------
 *
 * The pages time a mean-scale codec's steps around the coder: build_indexes
 * on the GPU, then the coder, for the y latent (kompressor BENCHMARKS.md,
 * section 3), and the symbols reach the coder as int32 tensors (section 4).
 * Readings:
 *   Q1  symbol = round-half-even(y - mean), the subtraction and the rounding
 *       in single precision (the latent's dtype); a value that int32 cannot
 *       hold saturates (NaN to INT32_MIN), so the coder refuses it as out of
 *       range rather than coding a wrapped value;
 *   Q2  index = the first table slot whose scale is at least the predicted
 *       scale, the last slot when none is (or the scale is NaN): written as
 *       (K - 1) - #{k < K - 1 : scale <= table[k]}, which holds for any table;
 *   Q3  dequantisation y_hat = (float)symbol + mean in single precision.
 */

static int32_t saturate_round(float d)
{
    if (d != d)
        return INT32_MIN;
    float r = rintf(d);   /* default rounding: half to even */
    if (r >= 2147483648.0f)
        return INT32_MAX;
    if (r < -2147483648.0f)
        return INT32_MIN;
    return (int32_t)r;
}

int oracle_latent_symbols(const float *y, const float *means, const float *scales, uint64_t n,
                          const float *scale_table, int32_t num_scales, int32_t *symbols,
                          int32_t *indexes)
{
    if (num_scales < 1 || (n && (!y || !means || !scales || !symbols || !indexes)) ||
        !scale_table)
        return ORACLE_E_ARG;
    for (uint64_t i = 0; i < n; ++i) {
        float d = y[i] - means[i];
        symbols[i] = saturate_round(d);
        int32_t idx = num_scales - 1;
        for (int32_t k = 0; k < num_scales - 1; ++k)
            if (scales[i] <= scale_table[k])
                idx -= 1;
        indexes[i] = idx;
    }
    return ORACLE_OK;
}

int oracle_dequantize(const int32_t *symbols, const float *means, uint64_t n, float *y_hat)
{
    if (n && (!symbols || !means || !y_hat))
        return ORACLE_E_ARG;
    for (uint64_t i = 0; i < n; ++i)
        y_hat[i] = (float)symbols[i] + means[i];
    return ORACLE_OK;
}

/* ---- Interleaved streams -------------------------------------------------
 *
 * The pages' fastest GPU decoder codes one stream per warp with one state
 * per warp lane and one shared word cursor, in a layout the CPU coder shares
 * word for word (torch_ans 0.3.0, "Usage" legend, Interleaved States).
 * Readings for the rans64 format here:
 *   IL1 the n symbols form S streams, stream t = [floor(t n / S),
 *       floor((t+1) n / S));
 *   IL2 symbol k of a stream (k from 0) is coded by state k mod W; every
 *       state starts at 2^31; a step is W consecutive symbols;
 *   IL3 a decoder takes the steps in order; within a step the put slots in
 *       order (slot 0 is every symbol's REG put, later slots the bypass puts
 *       of escaping symbols, in their S2 order); within a slot the states in
 *       ascending order; each put is followed by its renormalisation, which
 *       may read the next word from the stream's one shared cursor.  The
 *       encoder applies the puts in exactly the reverse order, so its
 *       emitted words, reversed, are the decoder's reading order;
 *   IL4 a stream is [x_0 low, x_0 high, .., x_{W-1} low, x_{W-1} high] (the
 *       final states in state order) followed by the words in reading
 *       order; the container is [S, end_0 .. end_{S-1}] and the streams, as
 *       for lanes;
 *   IL5 a clean decode leaves every state at 2^31 with every word read.
 * With W = 1 a stream is exactly a lane stream, and the container the lane
 * container with S lanes. */

#define MAX_PUTS 16   /* a symbol makes at most 10 puts (REG, count, 8 groups) */

int oracle_encode_interleaved(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                              const int32_t *cdf, const int32_t *lengths,
                              const int32_t *offsets, int32_t num_tables, int32_t stride,
                              uint32_t num_streams, uint32_t width, uint32_t *out, uint64_t cap,
                              uint64_t *out_words)
{
    if (num_streams == 0 || width == 0 || width > 1024 || (n && (!symbols || !indexes)))
        return ORACLE_E_ARG;
    int rc = oracle_check_tables(cdf, lengths, num_tables, stride);
    if (rc)
        return rc;
    uint64_t head = 1 + (uint64_t)num_streams;
    uint64_t used = 0;
    int cap_hit = 0;
    uint64_t *x = (uint64_t *)malloc(width * sizeof(uint64_t));
    put_t *step_puts = (put_t *)malloc((size_t)width * MAX_PUTS * sizeof(put_t));
    uint32_t *nputs = (uint32_t *)malloc(width * sizeof(uint32_t));
    if (!x || !step_puts || !nputs) {
        free(x); free(step_puts); free(nputs);
        return ORACLE_E_ARG;
    }
    for (uint32_t t = 0; t < num_streams && rc == ORACLE_OK; ++t) {
        uint64_t b = oracle_lane_begin(n, num_streams, t);
        uint64_t e = oracle_lane_begin(n, num_streams, t + 1);
        uint64_t m = e - b;
        /* at most one word per put */
        uint32_t *emitted = (uint32_t *)malloc((10 * m + 1) * sizeof(uint32_t));
        if (!emitted) {
            rc = ORACLE_E_ARG;
            break;
        }
        size_t ne = 0;
        for (uint32_t l = 0; l < width; ++l)
            x[l] = STATE_LOW;
        uint64_t steps = (m + width - 1) / width;
        for (uint64_t g = steps; g-- > 0 && rc == ORACLE_OK;) {
            /* the step's puts, per state */
            uint32_t max_slot = 0;
            for (uint32_t l = 0; l < width; ++l) {
                nputs[l] = 0;
                uint64_t k = g * width + l;
                if (k >= m)
                    continue;
                put_list one = {0, 0, 0};
                rc = symbol_puts(&one, symbols[b + k], indexes[b + k], cdf, lengths, offsets,
                                 num_tables, stride);
                if (rc == ORACLE_OK && one.n > MAX_PUTS)
                    rc = ORACLE_E_ARG;
                if (rc == ORACLE_OK) {
                    memcpy(step_puts + (size_t)l * MAX_PUTS, one.v, one.n * sizeof(put_t));
                    nputs[l] = (uint32_t)one.n;
                    if (one.n > max_slot)
                        max_slot = (uint32_t)one.n;
                }
                free(one.v);
                if (rc)
                    break;
            }
            /* slots last to first, states last to first */
            for (uint32_t s = max_slot; s-- > 0 && rc == ORACLE_OK;) {
                for (uint32_t l = width; l-- > 0;) {
                    if (s >= nputs[l])
                        continue;
                    apply_put(&x[l], step_puts[(size_t)l * MAX_PUTS + s], emitted, &ne);
                }
            }
        }
        if (rc == ORACLE_OK) {
            uint64_t w = 2ull * width + ne;
            if (head + used + w <= cap && !cap_hit) {
                uint32_t *o = out + head + used;
                for (uint32_t l = 0; l < width; ++l) {
                    o[2 * l] = (uint32_t)x[l];
                    o[2 * l + 1] = (uint32_t)(x[l] >> 32);
                }
                for (size_t k = 0; k < ne; ++k)
                    o[2 * width + k] = emitted[ne - 1 - k];
            } else {
                cap_hit = 1;
            }
            used += w;
            if (used > 0xFFFFFFFFull)
                rc = ORACLE_E_ARG;
            if (1 + t < cap)
                out[1 + t] = (uint32_t)used;
        }
        free(emitted);
    }
    free(x); free(step_puts); free(nputs);
    if (rc)
        return rc;
    if (cap >= 1)
        out[0] = num_streams;
    *out_words = head + used;
    return (cap_hit || head > cap) ? ORACLE_E_CAPACITY : ORACLE_OK;
}

/* Decoder side of one symbol, one put at a time: the phase of state l says
 * which put comes next (0: REG; 1: a count nibble; 2: a group nibble). */
typedef struct {
    int phase;
    int32_t index;
    int64_t slot, mv;
    uint32_t nb, got;
    uint64_t raw;
} il_sym_t;

int oracle_decode_interleaved(const uint32_t *stream, uint64_t stream_words,
                              const int32_t *indexes, uint64_t n,
                              const int32_t *cdf, const int32_t *lengths,
                              const int32_t *offsets, int32_t num_tables, int32_t stride,
                              uint32_t num_streams, uint32_t width, int32_t *symbols_out)
{
    if (num_streams == 0 || width == 0 || width > 1024 || !stream ||
        (n && (!indexes || !symbols_out)))
        return ORACLE_E_ARG;
    int rc = oracle_check_tables(cdf, lengths, num_tables, stride);
    if (rc)
        return rc;
    uint64_t head = 1 + (uint64_t)num_streams;
    if (stream_words < head || stream[0] != num_streams)
        return ORACLE_E_CORRUPT;
    uint64_t prev = 0;
    for (uint32_t t = 0; t < num_streams; ++t) {
        uint64_t endt = stream[1 + t];
        if (endt < prev + 2ull * width || head + endt > stream_words)
            return ORACLE_E_CORRUPT;
        prev = endt;
    }
    uint64_t *x = (uint64_t *)malloc(width * sizeof(uint64_t));
    il_sym_t *st = (il_sym_t *)malloc(width * sizeof(il_sym_t));
    if (!x || !st) {
        free(x); free(st);
        return ORACLE_E_ARG;
    }
    prev = 0;
    for (uint32_t t = 0; t < num_streams && rc == ORACLE_OK; ++t) {
        uint64_t endt = stream[1 + t];
        const uint32_t *w = stream + head + prev;
        uint64_t words = endt - prev, pos = 2ull * width;
        uint64_t b = oracle_lane_begin(n, num_streams, t);
        uint64_t e = oracle_lane_begin(n, num_streams, t + 1);
        uint64_t m = e - b;
        for (uint32_t l = 0; l < width; ++l)
            x[l] = (uint64_t)w[2 * l] | ((uint64_t)w[2 * l + 1] << 32);
        for (uint64_t g = 0; g * width < m && rc == ORACLE_OK; ++g) {
            int pending = 0;
            for (uint32_t l = 0; l < width; ++l) {
                uint64_t k = g * width + l;
                st[l].phase = k < m ? 0 : -1;
                if (k < m) {
                    st[l].index = indexes[b + k];
                    if (st[l].index < 0 || st[l].index >= num_tables) {
                        rc = ORACLE_E_INDEX;
                        break;
                    }
                    pending = 1;
                }
            }
            /* one slot at a time, states in ascending order */
            while (pending && rc == ORACLE_OK) {
                pending = 0;
                for (uint32_t l = 0; l < width && rc == ORACLE_OK; ++l) {
                    il_sym_t *s = &st[l];
                    if (s->phase < 0)
                        continue;
                    if (s->phase == 0) {
                        const int32_t *row = cdf + (int64_t)s->index * stride;
                        int32_t len = lengths[s->index];
                        uint32_t cum = (uint32_t)(x[l] & (TOTAL_FREQ - 1));
                        int32_t v = 0;
                        while (v + 1 < len && (uint32_t)row[v + 1] <= cum)
                            ++v;
                        uint32_t start = (uint32_t)row[v];
                        uint32_t freq = (uint32_t)(row[v + 1] - row[v]);
                        x[l] = (uint64_t)freq * (x[l] >> PREC) + cum - start;
                        s->slot = v;
                        s->mv = (int64_t)len - 2;
                        s->nb = 0;
                        s->got = 0;
                        s->raw = 0;
                        s->phase = v == s->mv ? 1 : 3;
                    } else {
                        uint32_t bits = (uint32_t)(x[l] & BYPASS_MAX);
                        x[l] >>= BYPASS_BITS;
                        if (s->phase == 1) {
                            s->nb += bits;
                            if (s->nb > 8)
                                rc = ORACLE_E_CORRUPT;
                            else if (bits != BYPASS_MAX)
                                s->phase = s->nb ? 2 : 3;
                        } else {
                            s->raw |= (uint64_t)bits << (BYPASS_BITS * s->got);
                            if (++s->got == s->nb)
                                s->phase = 3;
                        }
                    }
                    if (rc)
                        break;
                    /* renormalise after the put */
                    if (x[l] < STATE_LOW) {
                        if (pos >= words) {
                            rc = ORACLE_E_CORRUPT;
                            break;
                        }
                        x[l] = (x[l] << 32) | w[pos++];
                    }
                    if (s->phase == 3) {
                        int64_t value = s->slot;
                        if (s->slot == s->mv) {
                            if (s->raw >= (uint64_t)RAW_LIMIT) {
                                rc = ORACLE_E_CORRUPT;
                                break;
                            }
                            value = (s->raw & 1) ? -(int64_t)(s->raw >> 1) - 1
                                                 : (int64_t)(s->raw >> 1) + s->mv;
                        }
                        int64_t sym = value + offsets[s->index];
                        if (sym < INT32_MIN || sym > INT32_MAX) {
                            rc = ORACLE_E_CORRUPT;
                            break;
                        }
                        symbols_out[b + g * width + l] = (int32_t)sym;
                        s->phase = -1;
                    } else {
                        pending = 1;
                    }
                }
            }
        }
        if (rc == ORACLE_OK) {
            for (uint32_t l = 0; l < width; ++l)
                if (x[l] != STATE_LOW)
                    rc = ORACLE_E_CORRUPT;
            if (pos != words)
                rc = ORACLE_E_CORRUPT;
        }
        prev = endt;
    }
    free(x); free(st);
    return rc;
}
