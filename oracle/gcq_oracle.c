/*
 * gcq_oracle.c -- plain, slow, single-threaded CPU oracle for the
 * gradient-compression hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load this
 * library: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
 * leg call it.  It shares no code, header, table or constant with the HIP
 * library; every routine is written from the pages' statement of the method.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared (no -ffast-math,
 * which would enable flush-to-zero on x86 and break IEEE round-to-nearest).
 * On x86-64 float arithmetic is evaluated in single precision (SSE), so every
 * float expression below rounds once per operation, to nearest-even.
 *
 * Sources (cited by page title and section):
 *   [MX]  apache/mxnet pull request "2bit gradient compression":
 *         sections "Two bit quantization", "Format of compressed gradient",
 *         "Local kvstore", "Dist kvstore".
 *   [CD]  "CD-SGD: Distributed Stochastic Gradient Descent with Compression
 *         and Delay Compensation": section 3.4.1 "Update Rules" (eq. 10,
 *         11), section 3.2.1 "Implementation on MXNet" (Algorithm 1, the
 *         k-step switch) and Figure 4(b) (comm_buf, loc_buf).
 *   [QS]  "QSGD: Communication-Efficient SGD via Gradient Quantization and
 *         Encoding" (chapterpal summary): Knowl 1 (the Q_s operator),
 *         Knowl 2 (the (norm, sign, level) tuple), Knowl 3 (decode and
 *         average), Knowl 8 (bucketing, max-norm scaling).
 *   [EL]  P. Elias, "Universal codeword sets and representations of the
 *         integers" (IEEE Trans. Inf. Theory, 1975): the omega code, as used
 *         by [QS] Knowl 2.
 *   [SA]  "Communication-Efficient Decentralized Learning with Sparsification
 *         and Adaptive Peer Selection": the shared-seed Bernoulli(1/c)
 *         sparsification mask and the single-peer gossip exchange.
 *   [PH]  Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 *         1, 2, 3" (SC'11): the Philox-4x32 counter-based generator,
 *         pinned to the authors' published known-answer vectors.  The pages
 *         name no random source, so the choice of this generator and of the
 *         (seed, index) -> (key, counter) map is a frozen reading, not
 *         something the pages fix; any independent uniforms would be correct.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* 2-bit threshold quantizer with error-feedback residual              */
/* ------------------------------------------------------------------ */

/*
 * [MX] "Two bit quantization": a value at or above +t becomes code 11, a
 * value at or below -t becomes code 10, anything else code 00.  The
 * quantization error is kept as a residual and added to the next gradient
 * before it is quantized.  [CD] 3.4.1: a value that passes the threshold is
 * sent as the threshold itself, so 11 stands for +t and 10 for -t.
 * [MX] "Format of compressed gradient": 16 codes per 32-bit element, the
 * first code in the leftmost (most significant) bit pair; unused trailing
 * pairs are zero.
 *
 * g[n] is read, r[n] is read and overwritten with the new residual,
 * out[ceil(n/16)] is overwritten.
 */
void oracle_gc2_quantize(const float *g, float *r, size_t n, float t,
                         uint32_t *out)
{
    size_t nwords = (n + 15) / 16;
    for (size_t w = 0; w < nwords; w++)
        out[w] = 0u;
    for (size_t i = 0; i < n; i++) {
        float v = g[i] + r[i];          /* residual added before quantizing */
        uint32_t code;
        float sent;
        if (v >= t) {
            code = 3u;
            sent = t;
        } else if (v <= -t) {
            code = 2u;
            sent = -t;
        } else {
            code = 0u;
            sent = 0.0f;
        }
        r[i] = v - sent;                /* what was not sent is carried */
        out[i / 16] |= code << (30u - 2u * (unsigned)(i % 16));
    }
}

/*
 * [CD] 3.4.1 eq. (11): the local weights for the next iteration are the
 * pulled global weights minus eta times the local gradient.  [CD] 3.2.1 and
 * Figure 4(b): loc_buf holds the pulled weights and is updated with the
 * gradient in comm_buf; in the same iteration the gradient is compressed
 * (Algorithm 1: when count % k != 0), and both read comm_buf without
 * modifying it.  Reading taken: the step is the literal w - eta * g in
 * float32, the product rounded, then the difference rounded (no fused
 * multiply-add).
 *
 * w[n] is read and overwritten; g[n] is only read.
 */
void oracle_cdsgd_local_update(const float *g, float *w, size_t n, float eta)
{
    for (size_t i = 0; i < n; i++) {
        float step = eta * g[i];
        w[i] = w[i] - step;
    }
}

/*
 * A compressing iteration of [CD] Algorithm 1 on one buffer: the local
 * update of w and the 2-bit quantizer of g with residual r, as two
 * independent uses of the same gradient.
 */
void oracle_cdsgd_update_quantize(const float *g, float *r, float *w, size_t n,
                                  float t, float eta, uint32_t *out)
{
    oracle_cdsgd_local_update(g, w, n, eta);
    oracle_gc2_quantize(g, r, n, t, out);
}

/* Value a single 2-bit code stands for ([CD] 3.4.1).  01 is never produced
 * by the quantizer; it is read as zero, like 00. */
static float oracle_code_value(uint32_t code, float t)
{
    if (code == 3u)
        return t;
    if (code == 2u)
        return -t;
    return 0.0f;
}

/*
 * [MX] "Local kvstore": every device quantizes, device 0 dequantizes the
 * packed data of all devices and sums it.  Here the W devices are W packed
 * buffers; the sum starts at +0 and adds worker 0, 1, ..., W-1 in that order
 * in float32 (the order fixes the rounding).  acc[n] is overwritten.
 */
void oracle_gc2_dequant_reduce(const uint32_t *const *words, uint32_t W,
                               size_t n, float t, float *acc)
{
    for (size_t i = 0; i < n; i++) {
        float a = 0.0f;
        for (uint32_t w = 0; w < W; w++) {
            uint32_t code = (words[w][i / 16] >> (30u - 2u * (unsigned)(i % 16))) & 3u;
            a = a + oracle_code_value(code, t);
        }
        acc[i] = a;
    }
}

/* ------------------------------------------------------------------ */
/* Counter-based uniforms: Philox-4x32 with 10 rounds [PH]             */
/* ------------------------------------------------------------------ */

/*
 * One Philox-4x32 round: two 32x32->64 multiplications of counter words 0
 * and 2 by the round multipliers; the high halves are xored with the other
 * two counter words and the round key, and the four words are permuted.
 * Between rounds the two key words are bumped by the Weyl constants (the
 * golden ratio and sqrt(3)-1, as 32-bit fractions).
 */
void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                          uint32_t out[4])
{
    const uint32_t mul0 = 0xD2511F53u, mul1 = 0xCD9E8D57u;
    const uint32_t weyl0 = 0x9E3779B9u, weyl1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; round++) {
        if (round > 0) {
            k0 += weyl0;
            k1 += weyl1;
        }
        uint64_t p0 = (uint64_t)mul0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)mul1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/*
 * Uniform for element i under a 64-bit seed: counter = (i/4 low word,
 * i/4 high word, 0, 0), key = (seed low word, seed high word); output word
 * i%4, top 24 bits, scaled by 2^-24.  The value lies in [0, 1) and is exact
 * in float32.  It depends only on (seed, i), never on how work is split.
 */
float oracle_uniform(uint64_t seed, uint64_t i)
{
    uint64_t q = i >> 2;
    uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t o[4];
    oracle_philox4x32_10(ctr, key, o);
    uint32_t word = o[i & 3u];
    return (float)(word >> 8) * (1.0f / 16777216.0f);
}

/* ------------------------------------------------------------------ */
/* QSGD bucketed s-level stochastic quantizer                          */
/* ------------------------------------------------------------------ */

/*
 * [QS] Knowl 8 "Gradient Bucketing": the vector is cut into contiguous
 * buckets of d elements (the last may be shorter) and each bucket is scaled
 * by its own L2 norm [QS] Knowl 1.  The sum of squares is taken in double
 * in index order, its square root in double, rounded once to float.
 */
void oracle_qsgd_norms(const float *g, size_t n, uint32_t d, float *norms)
{
    size_t nb = (n + d - 1) / d;
    for (size_t b = 0; b < nb; b++) {
        size_t lo = b * (size_t)d;
        size_t hi = lo + d < n ? lo + d : n;
        double s = 0.0;
        for (size_t i = lo; i < hi; i++)
            s += (double)g[i] * (double)g[i];
        norms[b] = (float)sqrt(s);
    }
}

/*
 * [QS] Knowl 1: with a = |v_i| / ||v||, and l the integer with
 * a in [l/s, (l+1)/s], the level is l+1 with probability a*s - l and l
 * otherwise; Q_s(0) = 0.  Taken in float32, in this order:
 *   a = |g| / norm (one correctly rounded division), x = a * s,
 *   l = floor(x), p = x - l (exact), level = l + [u < p], clamped to s;
 *   a zero norm (or x not a number) gives level 0.
 * Sign bit = [g < 0] (sgn(0) = +1, so -0 is stored as positive).
 * [QS] Knowl 2: the (norm, sign, level) tuple is stored here as one nibble
 * per element: sign in bit 3, level in bits 2..0; 8 nibbles per 32-bit word,
 * the first element in the most significant nibble; unused nibbles zero.
 *
 * The norms are GIVEN (so a GPU's norms can be fed in to compare levels).
 * The slice g[0..n) holds elements whose global indices start at
 * index_base, which must be a multiple of both d and 8: buckets and words
 * are counted from the start of the slice, the uniform uses the global
 * index.  nibbles[ceil(n/8)] is overwritten.
 */
void oracle_qsgd_levels(const float *g, size_t n, uint32_t d, uint32_t s,
                        uint64_t seed, uint64_t index_base,
                        const float *norms, uint32_t *nibbles)
{
    size_t nwords = (n + 7) / 8;
    for (size_t w = 0; w < nwords; w++)
        nibbles[w] = 0u;
    const float sf = (float)s;
    for (size_t i = 0; i < n; i++) {
        float norm = norms[i / d];
        uint32_t level;
        if (norm == 0.0f) {
            level = 0u;
        } else {
            float a = fabsf(g[i]) / norm;
            float x = a * sf;
            if (x != x) {
                level = 0u;
            } else if (x >= sf) {
                level = s;
            } else {
                float l = floorf(x);
                float p = x - l;
                float u = oracle_uniform(seed, index_base + i);
                level = (uint32_t)l + (u < p ? 1u : 0u);
            }
        }
        uint32_t sign = g[i] < 0.0f ? 1u : 0u;
        uint32_t nib = (sign << 3) | level;
        nibbles[i / 8] |= nib << (28u - 4u * (unsigned)(i % 8));
    }
}

/* Norms then levels, as one call (the whole quantizer). */
void oracle_qsgd_quantize(const float *g, size_t n, uint32_t d, uint32_t s,
                          uint64_t seed, float *norms, uint32_t *nibbles)
{
    oracle_qsgd_norms(g, n, d, norms);
    oracle_qsgd_levels(g, n, d, s, seed, 0u, norms, nibbles);
}

/*
 * [QS] Knowl 1 and Knowl 3 "Decode": Q_s(v_i) = ||v|| * sgn(v_i) * level/s,
 * evaluated in float32 as (norm * level) / s, then the sign applied.
 * The level field is used as stored.  out[n] is overwritten.
 */
void oracle_qsgd_dequant(const float *norms, const uint32_t *nibbles,
                         size_t n, uint32_t d, uint32_t s, float *out)
{
    const float sf = (float)s;
    for (size_t i = 0; i < n; i++) {
        uint32_t nib = (nibbles[i / 8] >> (28u - 4u * (unsigned)(i % 8))) & 15u;
        uint32_t sign = nib >> 3;
        float level = (float)(nib & 7u);
        float m = norms[i / d] * level;
        m = m / sf;
        out[i] = sign ? -m : m;
    }
}

/*
 * [QS] Knowl 8, max-norm scaling: a bucket is scaled by its largest
 * coordinate magnitude instead of its L2 norm.  The maximum is exact.
 * Reading taken for NaN: an element takes part only when its magnitude
 * compares greater than the running maximum, so NaNs never become the scale
 * (and, as with any scale, quantize to level 0).  scales[ceil(n/d)].
 */
void oracle_qsgd_maxnorms(const float *g, size_t n, uint32_t d, float *scales)
{
    size_t nb = (n + d - 1) / d;
    for (size_t b = 0; b < nb; b++) {
        size_t lo = b * (size_t)d;
        size_t hi = lo + d < n ? lo + d : n;
        float m = 0.0f;
        for (size_t i = lo; i < hi; i++) {
            float a = fabsf(g[i]);
            if (a > m)
                m = a;
        }
        scales[b] = m;
    }
}

/* Q_s with max-norm bucket scales: the same levels as the L2 quantizer,
 * given the scales. */
void oracle_qsgd_quantize_maxnorm(const float *g, size_t n, uint32_t d, uint32_t s,
                                  uint64_t seed, float *scales, uint32_t *nibbles)
{
    oracle_qsgd_maxnorms(g, n, d, scales);
    oracle_qsgd_levels(g, n, d, s, seed, 0u, scales, nibbles);
}

/*
 * [QS] Knowl 3: every processor decodes the messages of all K peers and
 * averages them, g_bar = (1/K) sum_l Decode(M_l).  Reading taken: for each
 * element, the K decoded values (each exactly as oracle_qsgd_dequant) are
 * added in float32 in worker order 0..K-1 starting from +0, and the sum is
 * divided by K once (correctly rounded).  scales[l] and nibbles[l] are the
 * l-th worker's bucket scales and nibble words.
 */
void oracle_qsgd_dequant_average(const float *const *scales, const uint32_t *const *nibbles,
                                 uint32_t K, size_t n, uint32_t d, uint32_t s, float *out)
{
    const float sf = (float)s;
    const float kf = (float)K;
    for (size_t i = 0; i < n; i++) {
        float acc = 0.0f;
        for (uint32_t l = 0; l < K; l++) {
            uint32_t nib = (nibbles[l][i / 8] >> (28u - 4u * (unsigned)(i % 8))) & 15u;
            uint32_t sign = nib >> 3;
            float level = (float)(nib & 7u);
            float m = scales[l][i / d] * level;
            m = m / sf;
            acc = acc + (sign ? -m : m);
        }
        out[i] = acc / kf;
    }
}

/* ------------------------------------------------------------------ */
/* SAPS: shared-seed random sparsification and single-peer exchange    */
/* ------------------------------------------------------------------ */

/*
 * [SA] The model is sparsified by a mask whose entries follow a Bernoulli
 * distribution with probability 1/c, generated from a seed that the
 * coordinator hands every worker, so all workers mask the same components
 * and only the components at mask positions travel (the receiver knows the
 * positions from the seed).  Reading taken: element i is kept when
 * u_i * c < 1, evaluated exactly (u_i is oracle_uniform(seed, i), a 24-bit
 * fraction; the product of it and a float fits a double exactly).
 */
int oracle_saps_keep(uint64_t seed, uint64_t i, float c)
{
    double u = (double)oracle_uniform(seed, i);
    return u * (double)c < 1.0;
}

/* keep[j] = oracle_saps_keep(seed, start + j, c) for j < n, one byte each. */
void oracle_saps_keep_range(uint64_t seed, uint64_t start, size_t n, float c,
                            unsigned char *keep)
{
    for (size_t j = 0; j < n; j++)
        keep[j] = (unsigned char)oracle_saps_keep(seed, start + j, c);
}

/* The kept components of x, in index order; returns how many. */
size_t oracle_saps_gather(const float *x, size_t n, float c, uint64_t seed, float *values)
{
    size_t k = 0;
    for (size_t i = 0; i < n; i++)
        if (oracle_saps_keep(seed, i, c))
            values[k++] = x[i];
    return k;
}

/*
 * [SA] single-peer gossip: each row of the gossip matrix has two non-zero
 * entries and the matrix is doubly stochastic.  Reading taken: an exchanged
 * component becomes the average of the two workers' values, (x + y) * 0.5
 * in float32 (the sum rounded, the halving exact); components outside the
 * mask are left as they are.  peer holds the peer's kept values in index
 * order; returns how many were used.
 */
size_t oracle_saps_merge(float *x, size_t n, float c, uint64_t seed, const float *peer)
{
    size_t k = 0;
    for (size_t i = 0; i < n; i++) {
        if (oracle_saps_keep(seed, i, c)) {
            x[i] = (x[i] + peer[k]) * 0.5f;
            k++;
        }
    }
    return k;
}

/* ------------------------------------------------------------------ */
/* QSGD message coding with Elias omega codes                          */
/* ------------------------------------------------------------------ */

/*
 * [EL] omega code of a positive integer k: start from the single bit 0;
 * while k > 1, put the binary form of k (which starts with a 1) in front
 * and continue with k = (its number of digits) - 1.  omega(1) = 0,
 * omega(2) = 100, omega(3) = 110, omega(4) = 101000.
 */
static unsigned oracle_bit_length(uint64_t k)
{
    unsigned len = 0;
    while (k) {
        len++;
        k >>= 1;
    }
    return len;
}

/* Appends `nbits` low bits of v, most significant first, at bit *pos of out
 * (bit 31 of a word is its first bit); out must be zeroed. */
static void oracle_put_bits(uint32_t *out, uint64_t *pos, uint64_t v, unsigned nbits)
{
    for (unsigned b = nbits; b-- > 0;) {
        if ((v >> b) & 1u)
            out[*pos / 32] |= 1u << (31u - (unsigned)(*pos % 32));
        (*pos)++;
    }
}

static uint32_t oracle_get_bit(const uint32_t *in, uint64_t *pos)
{
    uint32_t bit = (in[*pos / 32] >> (31u - (unsigned)(*pos % 32))) & 1u;
    (*pos)++;
    return bit;
}

static void oracle_omega_put(uint32_t *out, uint64_t *pos, uint64_t k)
{
    uint64_t groups[64];
    unsigned lens[64];
    int ng = 0;
    while (k > 1) {
        unsigned len = oracle_bit_length(k);
        groups[ng] = k;
        lens[ng] = len;
        ng++;
        k = len - 1;
    }
    for (int g = ng - 1; g >= 0; g--)      /* the last group found comes first */
        oracle_put_bits(out, pos, groups[g], lens[g]);
    oracle_put_bits(out, pos, 0, 1);
}

static uint64_t oracle_omega_get(const uint32_t *in, uint64_t *pos)
{
    uint64_t k = 1;
    while (oracle_get_bit(in, pos)) {      /* a group: a 1 and k more digits */
        uint64_t v = 1;
        for (uint64_t b = 0; b < k; b++)
            v = (v << 1) | oracle_get_bit(in, pos);
        k = v;
    }
    return k;
}

/* Code length of omega(k), in bits. */
unsigned oracle_omega_length(uint64_t k)
{
    unsigned len = 1;
    while (k > 1) {
        unsigned b = oracle_bit_length(k);
        len += b;
        k = b - 1;
    }
    return len;
}

/*
 * [QS] Knowl 2: a quantized bucket is the tuple (norm, signs, levels); the
 * norm takes 32 bits and the non-zero coordinates are coded by the omega
 * code of the distance from the previous non-zero coordinate, with their
 * sign and their level.  Readings taken (the format is not spelled out): per
 * bucket, the 32 bits of the float norm, then for each coordinate i (index
 * within the bucket) whose level is not 0, in order: omega(i - prev) with
 * prev the previous such index (-1 before the first), one sign bit (1 =
 * negative), omega(level).  Buckets follow each other with no padding;
 * bit_offsets[b] is where bucket b starts and bit_offsets[nb] the total
 * length (the message lengths, which delimit the buckets).  Bits are written
 * most significant first into 32-bit words.  Signs of level-0 coordinates are
 * not coded.
 *
 * out must hold ceil(total/32) words; it is zeroed here first up to
 * out_words.  Returns the total length in bits.
 */
uint64_t oracle_qsgd_elias_encode(const float *norms, const uint32_t *nibbles, size_t n,
                                  uint32_t d, uint64_t *bit_offsets, uint32_t *out,
                                  size_t out_words)
{
    size_t nb = (n + d - 1) / d;
    for (size_t w = 0; w < out_words; w++)
        out[w] = 0u;
    uint64_t pos = 0;
    for (size_t b = 0; b < nb; b++) {
        bit_offsets[b] = pos;
        uint32_t normbits;
        memcpy(&normbits, &norms[b], 4);
        oracle_put_bits(out, &pos, normbits, 32);
        size_t lo = b * (size_t)d;
        size_t hi = lo + d < n ? lo + d : n;
        int64_t prev = -1;
        for (size_t i = lo; i < hi; i++) {
            uint32_t nib = (nibbles[i / 8] >> (28u - 4u * (unsigned)(i % 8))) & 15u;
            uint32_t level = nib & 7u;
            if (level == 0)
                continue;
            int64_t li = (int64_t)(i - lo);
            oracle_omega_put(out, &pos, (uint64_t)(li - prev));
            oracle_put_bits(out, &pos, nib >> 3, 1);
            oracle_omega_put(out, &pos, level);
            prev = li;
        }
    }
    bit_offsets[nb] = pos;
    return pos;
}

/* The inverse: norms and nibble words from the coded buckets (every
 * nibble of a coordinate the code does not name is 0). */
void oracle_qsgd_elias_decode(const uint32_t *in, const uint64_t *bit_offsets, size_t n,
                              uint32_t d, float *norms, uint32_t *nibbles)
{
    size_t nb = (n + d - 1) / d;
    for (size_t w = 0; w < (n + 7) / 8; w++)
        nibbles[w] = 0u;
    for (size_t b = 0; b < nb; b++) {
        uint64_t pos = bit_offsets[b];
        uint32_t normbits = 0;
        for (int k = 0; k < 32; k++)
            normbits = (normbits << 1) | oracle_get_bit(in, &pos);
        memcpy(&norms[b], &normbits, 4);
        size_t lo = b * (size_t)d;
        int64_t prev = -1;
        while (pos < bit_offsets[b + 1]) {
            int64_t li = prev + (int64_t)oracle_omega_get(in, &pos);
            uint32_t sign = oracle_get_bit(in, &pos);
            uint32_t level = (uint32_t)oracle_omega_get(in, &pos);
            size_t i = lo + (size_t)li;
            nibbles[i / 8] |= ((sign << 3) | level) << (28u - 4u * (unsigned)(i % 8));
            prev = li;
        }
    }
}
