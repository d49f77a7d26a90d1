/*
 * gcq.h -- C ABI of the MI355X (gfx950) gradient-compression library
 * (libgcq.so).
 *
 * The calls follow the statement of the problem on these pages:
 *   - apache/mxnet pull request "2bit gradient compression": sections "Two
 *     bit quantization", "Format of compressed gradient", "Local kvstore",
 *     "Dist kvstore", and the review thread (no default threshold; a new
 *     threshold takes effect on later calls).
 *   - "CD-SGD: Distributed Stochastic Gradient Descent with Compression and
 *     Delay Compensation": 3.4.1 "Update Rules" (a code that passes the
 *     threshold is worth the threshold itself; eq. (11), the local update),
 *     3.2.1 Algorithm 1 and Figure 4(b) (the local update and the
 *     compression read the same gradient buffer).
 *   - "QSGD: Communication-Efficient SGD via Gradient Quantization and
 *     Encoding" (chapterpal summary): Knowl 1 (Q_s), Knowl 2 (the
 *     (norm, sign, level) tuple and its Elias coding), Knowl 3 (encode,
 *     broadcast, decode, average), Knowl 8 (bucketing, max-norm scaling).
 *   - blog "IMerge修改（Design）": consecutive layers merged into
 *     transmission units (fusion buckets), one unit per message.
 *   - "Communication-Efficient Decentralized Learning with Sparsification
 *     and Adaptive Peer Selection": the shared-seed Bernoulli(1/c) mask and
 *     the single-peer gossip exchange.
 *
 * Conventions shared by every call:
 *   - Array pointers are DEVICE pointers (HIP device memory, e.g. torch
 *     tensors on a ROCm device) owned by the caller; the library keeps no
 *     reference to them after the call.  Host arrays are marked "host".
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *     call only enqueues work on that stream and returns; it never
 *     synchronizes, with one exception: a gc2_quantize_buckets call with
 *     more buckets than any earlier call on the device grows the library's
 *     device tables, which allocates device memory and first waits on the
 *     host for the kernels still reading the old tables.  Faults during
 *     execution surface at the caller's next synchronization with the
 *     stream.
 *   - Every argument is checked on the host before anything is enqueued; a
 *     call that returns an error has enqueued nothing and changed nothing.
 *   - Return value: GCQ_OK (0) or a negative GCQ_ERR_* status;
 *     gcq_status_string() names it.
 *   - n == 0 (or W == 0 buckets of work) is a successful no-op.
 *   - Element counts above 2^60 (GCQ_MAX_ELEMS) are rejected with
 *     GCQ_ERR_PARAM, so that no byte count or end address can wrap.
 *   - Arithmetic is IEEE float32 with round-to-nearest-even, denormals kept,
 *     no contraction into fused multiply-add where it would change a result.
 */
#ifndef GCQ_H
#define GCQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gcq_status {
    GCQ_OK = 0,
    GCQ_ERR_NULL = -1,      /* a required pointer is NULL while n > 0 */
    GCQ_ERR_THRESHOLD = -2, /* threshold t is not finite or t <= 0 */
    GCQ_ERR_PARAM = -3,     /* n, s, d, W or a bucket count out of range */
    GCQ_ERR_ALIGN = -4,     /* a pointer is not aligned as documented */
    GCQ_ERR_OVERLAP = -5,   /* an output range intersects another operand */
    GCQ_ERR_LAUNCH = -6,    /* the HIP runtime rejected a launch or copy */
    GCQ_ERR_NOMEM = -7      /* a library-owned buffer could not be grown */
};

/* Largest W accepted by gc2_dequant_reduce. */
#define GCQ_MAX_WORKERS 64

/* Largest element count n of any call (and of all buckets of one
 * gc2_quantize_buckets call together). */
#define GCQ_MAX_ELEMS ((size_t)1 << 60)

/* ------------------------------------------------------------------ */
/* 2-bit threshold quantizer with error-feedback residual              */
/* ------------------------------------------------------------------ */

/*
 * gc2_quantize -- one quantization step of the MXNet PR's 2-bit scheme
 * ("Two bit quantization", "Format of compressed gradient"), with the
 * residual of CD-SGD 3.4.1.
 *
 * For every i < n, in float32:
 *     v = g[i] + r[i]
 *     code = 11 if v >= t, 10 if v <= -t, else 00
 *     r[i] = v - (+t | -t | +0)          (the value the code stands for)
 * and code i is written to bits [31-2(i%16) : 30-2(i%16)] of
 * out_words[i/16], i.e. 16 codes per 32-bit word, first element in the most
 * significant bit pair; pairs past n in the last word are 00.
 *
 *   g          in,     float32[n], 16-byte aligned
 *   r          in/out, float32[n], 16-byte aligned; the residual carried
 *              between steps (the only state of the method)
 *   n          element count (any value, including a ragged tail)
 *   t          threshold, finite and > 0 (there is no default)
 *   out_words  out,    uint32[ceil(n/16)], 4-byte aligned, overwritten
 *   stream     hipStream_t
 *
 * Errors: GCQ_ERR_NULL, GCQ_ERR_THRESHOLD, GCQ_ERR_ALIGN, GCQ_ERR_OVERLAP
 * (g, r and out_words must be pairwise disjoint), GCQ_ERR_LAUNCH.
 */
int gc2_quantize(const float *g, float *r, size_t n, float t, uint32_t *out_words,
                 void *stream);

/* One fusion bucket: its own gradient, residual, packed output and
 * threshold.  Field meaning and alignment as in gc2_quantize. */
typedef struct gc2_bucket {
    const float *g;
    float *r;
    uint32_t *out_words;
    size_t n;
    float t;
} gc2_bucket;

/*
 * gc2_quantize_buckets -- gc2_quantize applied to each of num_buckets
 * buckets in ONE kernel launch (IMerge-style merged transmission units).
 * Each bucket is quantized exactly as gc2_quantize would quantize it alone:
 * its packing starts at its own out_words[0], its tail pairs are 00.
 *
 *   buckets      host array of num_buckets descriptors; read during the
 *                call only.  The library writes it into one of 8 device
 *                tables it owns per device, with small kernels whose
 *                arguments carry the descriptors, or reuses a table it
 *                already holds when the descriptors match.  The caller's
 *                stream waits on the device for the table's earlier
 *                readers, so calls on different streams may share tables;
 *                the host does not wait.  The tables are allocated on the
 *                first call and grown (with the host wait described in the
 *                conventions above) when a call has more buckets than they
 *                hold.
 *   num_buckets  0 .. 2^31-1
 *   stream       hipStream_t
 *
 * Errors: as gc2_quantize for any bucket (nothing is launched if one bucket
 * is invalid); GCQ_ERR_PARAM when the buckets hold more than GCQ_MAX_ELEMS
 * elements together; GCQ_ERR_OVERLAP also when two buckets' writable ranges
 * (r, out_words) intersect each other or another bucket's g; GCQ_ERR_NOMEM.
 */
int gc2_quantize_buckets(const gc2_bucket *buckets, uint32_t num_buckets, void *stream);

/*
 * gc2_quantize_buckets_noalloc -- gc2_quantize_buckets for callers that
 * cannot allocate memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, checks and results.  It
 * calls no hipMalloc or hipFree and allocates no host memory: the
 * descriptor table lives in a fixed device array of the library (room for
 * GC2_NOALLOC_MAX_BUCKETS descriptors, 48 bytes each, 192 KiB per device,
 * held until the process ends), which every call rewrites with small
 * kernels on `stream` before the quantizer reads it.  Calls on one device
 * therefore share that array: calls ordered on one stream are safe, but two
 * calls that may run at the same time on one device (on different streams
 * without an ordering between them) race on it and must not be made.
 *
 * Errors: as gc2_quantize_buckets, and GCQ_ERR_PARAM when num_buckets
 * exceeds GC2_NOALLOC_MAX_BUCKETS.
 */
#define GC2_NOALLOC_MAX_BUCKETS 4096
int gc2_quantize_buckets_noalloc(const gc2_bucket *buckets, uint32_t num_buckets, void *stream);

/*
 * gc2_dequant_reduce -- the receiving side of the MXNet PR's "Local
 * kvstore" (device 0 dequantizes every device's packed gradient and sums
 * them) and "Dist kvstore" (the server dequantizes to full size).  With
 * code(w, i) read as in gc2_quantize and 11 -> +t, 10 -> -t, 00 and 01 -> 0:
 *     acc[i] = ((+0 + val(0, i)) + val(1, i)) + ... + val(W-1, i)
 * in float32, workers added in the order 0, 1, ..., W-1 (the order fixes
 * the rounding; the result is bit-exact with that sequential sum).
 *
 *   words   host array of W device pointers, each uint32[ceil(n/16)],
 *           4-byte aligned, read only (they may alias one another)
 *   W       1 .. GCQ_MAX_WORKERS
 *   n       element count
 *   t       threshold the codes were made with, finite and > 0
 *   acc     out, float32[n], 16-byte aligned, overwritten (not accumulated)
 *   stream  hipStream_t
 *
 * Errors: GCQ_ERR_NULL, GCQ_ERR_PARAM (W), GCQ_ERR_THRESHOLD, GCQ_ERR_ALIGN,
 * GCQ_ERR_OVERLAP (acc intersects a words buffer), GCQ_ERR_LAUNCH.
 */
int gc2_dequant_reduce(const uint32_t *const *words, uint32_t W, size_t n, float t,
                       float *acc, void *stream);

/* ------------------------------------------------------------------ */
/* CD-SGD: local update fused with the 2-bit quantizer                 */
/* ------------------------------------------------------------------ */

/*
 * cdsgd_update_quantize -- a compressing iteration of CD-SGD's worker
 * (Algorithm 1 in 3.2.1: count % k != 0) on one buffer.  Figure 4(b): the
 * local weights in loc_buf are updated with the gradient in comm_buf, and
 * the same gradient is compressed; eq. (11) of 3.4.1: the next local
 * weights are the pulled global weights minus eta times the gradient.
 * One pass reads g once; for every i < n, in float32:
 *     w_loc[i] = w_loc[i] - (eta * g[i])     (product rounded, then the
 *                                              difference; no fused multiply-add)
 * and exactly gc2_quantize's step on (g[i], r[i]) into out_words.
 *
 *   g          in,     float32[n], 16-byte aligned (comm_buf; not modified)
 *   r          in/out, float32[n], 16-byte aligned (residual)
 *   w_loc      in/out, float32[n], 16-byte aligned (loc_buf: holds the pulled
 *              weights on entry, the next local weights on return)
 *   n          element count (any value)
 *   t          threshold, finite and > 0
 *   eta        local learning rate, finite and >= 0
 *   out_words  out,    uint32[ceil(n/16)], 4-byte aligned
 *   stream     hipStream_t
 *
 * Errors: GCQ_ERR_NULL, GCQ_ERR_THRESHOLD, GCQ_ERR_PARAM (eta), GCQ_ERR_ALIGN,
 * GCQ_ERR_OVERLAP (g, r, w_loc and out_words pairwise disjoint),
 * GCQ_ERR_LAUNCH.
 */
int cdsgd_update_quantize(const float *g, float *r, float *w_loc, size_t n, float t, float eta,
                          uint32_t *out_words, void *stream);

/*
 * cdsgd_local_update -- the local update alone, for CD-SGD's uncompressed
 * correction iterations (Algorithm 1: count % k == 0, when the full-precision
 * gradient is pushed): w_loc[i] = w_loc[i] - (eta * g[i]) as above.  The
 * residual is not touched.
 *
 *   g      in,     float32[n], 16-byte aligned
 *   w_loc  in/out, float32[n], 16-byte aligned
 *   eta    finite and >= 0
 *
 * Errors: GCQ_ERR_NULL, GCQ_ERR_PARAM, GCQ_ERR_ALIGN, GCQ_ERR_OVERLAP,
 * GCQ_ERR_LAUNCH.
 */
int cdsgd_local_update(const float *g, float *w_loc, size_t n, float eta, void *stream);

/* ------------------------------------------------------------------ */
/* QSGD: bucketed s-level stochastic quantizer                         */
/* ------------------------------------------------------------------ */

/*
 * qsgd_quantize -- Q_s of the QSGD summary (Knowl 1) applied per bucket of d
 * contiguous elements (Knowl 8), each bucket scaled by its own L2 norm; the
 * output is the (norm, sign, level) tuple of Knowl 2 as fixed-width
 * nibbles.
 *
 * Bucket b covers elements [b*d, min(b*d + d, n)).  norms[b] is its L2
 * norm, accumulated in float64 and rounded once to float32.  For element i
 * of bucket b, in float32:
 *     if norms[b] == 0: level = 0                       (Q_s(0) = 0)
 *     else: a = |g[i]| / norms[b]  (correctly rounded), x = a * s,
 *           x >= s -> level s; x NaN -> level 0; otherwise
 *           l = floor(x), p = x - l, level = l + (u_i < p)
 *     sign = (g[i] < 0)                                 (sgn(0) = +1)
 *     nibble = sign << 3 | level, 8 nibbles per uint32 word, first element
 *     in the most significant nibble, nibbles past n zero.
 * u_i = (word >> 8) * 2^-24 where word is output word (i % 4) of
 * Philox-4x32-10 (Salmon et al., SC'11) with counter (i/4 low 32 bits,
 * i/4 high 32 bits, 0, 0) and key (seed low 32 bits, seed high 32 bits).
 * u_i depends only on (seed, i), never on how the work is split.
 *
 *   g        in,  float32[n], 16-byte aligned
 *   n        element count
 *   d        bucket length, >= 1
 *   s        number of levels, 1 .. 7 (a level must fit in 3 bits)
 *   seed     64-bit seed of the uniforms (one per step)
 *   norms    out, float32[ceil(n/d)], 4-byte aligned, overwritten
 *   nibbles  out, uint32[ceil(n/8)], 4-byte aligned, overwritten
 *   stream   hipStream_t
 *
 * Errors: GCQ_ERR_NULL, GCQ_ERR_PARAM (d, s), GCQ_ERR_ALIGN,
 * GCQ_ERR_OVERLAP (g, norms, nibbles pairwise disjoint), GCQ_ERR_LAUNCH.
 */
int qsgd_quantize(const float *g, size_t n, uint32_t d, uint32_t s, uint64_t seed,
                  float *norms, uint32_t *nibbles, void *stream);

/*
 * qsgd_dequant -- "Decode" of the QSGD summary's Knowl 3: with level and
 * sign read from nibble i as stored (no clamping), in float32:
 *     out[i] = +-( (norms[i/d] * level) / s )    (- when the sign bit is 1)
 *
 *   norms    in,  float32[ceil(n/d)], 4-byte aligned
 *   nibbles  in,  uint32[ceil(n/8)], 4-byte aligned
 *   n, d, s  as in qsgd_quantize
 *   out      out, float32[n], 16-byte aligned, overwritten
 *   stream   hipStream_t
 *
 * Errors: GCQ_ERR_NULL, GCQ_ERR_PARAM, GCQ_ERR_ALIGN, GCQ_ERR_OVERLAP
 * (out intersects an input), GCQ_ERR_LAUNCH.
 */
int qsgd_dequant(const float *norms, const uint32_t *nibbles, size_t n, uint32_t d,
                 uint32_t s, float *out, void *stream);

/*
 * qsgd_quantize_maxnorm -- qsgd_quantize with the max-norm bucket scale of
 * the QSGD summary's Knowl 8: each bucket is normalized by its largest
 * coordinate magnitude instead of its L2 norm.  scales[b] = max |g_i| over
 * bucket b (exact; a NaN element never becomes the scale and quantizes to
 * level 0; an all-zero bucket has scale +0 and levels 0).  Levels, signs,
 * nibbles, uniforms and arguments exactly as qsgd_quantize, with scales in
 * place of norms; qsgd_dequant decodes the result.
 *
 * Errors: as qsgd_quantize.
 */
int qsgd_quantize_maxnorm(const float *g, size_t n, uint32_t d, uint32_t s, uint64_t seed,
                          float *scales, uint32_t *nibbles, void *stream);

/*
 * qsgd_dequant_average -- the receiving side of the QSGD summary's Knowl 3:
 * decode the messages of all K workers and average them,
 *     out[i] = ( sum over l = 0..K-1, in this order, starting from +0,
 *                of +-((scales[l][i/d] * level_l,i) / s) ) / K
 * in float32, each decoded value exactly as qsgd_dequant computes it, and
 * the sum divided by K once (correctly rounded).  Works with L2 norms or
 * max-norm scales.
 *
 *   scales   host array of K device pointers, float32[ceil(n/d)] each,
 *            4-byte aligned
 *   nibbles  host array of K device pointers, uint32[ceil(n/8)] each,
 *            4-byte aligned
 *   K        1..GCQ_MAX_WORKERS
 *   n, d, s  as qsgd_dequant
 *   out      out, float32[n], 16-byte aligned
 *
 * Errors: GCQ_ERR_PARAM (K, d or s), GCQ_ERR_NULL, GCQ_ERR_ALIGN,
 * GCQ_ERR_OVERLAP (out intersects an input), GCQ_ERR_LAUNCH.
 */
int qsgd_dequant_average(const float *const *scales, const uint32_t *const *nibbles, uint32_t K,
                         size_t n, uint32_t d, uint32_t s, float *out, void *stream);

/*
 * qsgd_elias_encode -- the QSGD summary's Knowl 2 coding of quantized
 * buckets with Elias omega codes (P. Elias, "Universal codeword sets and
 * representations of the integers", 1975: omega(1) = 0; for k > 1 the
 * binary digits of k, preceded by omega-style groups for its length - 1,
 * then a final 0).  Per bucket: the 32 bits of the norm, then for every
 * coordinate i (index within the bucket) whose level is not 0, in order:
 * omega(i - prev) with prev the previous such index (-1 before the first),
 * one sign bit (1 = negative), omega(level).  Buckets follow each other
 * without padding; bits are written most significant first into 32-bit
 * words.  Signs of level-0 coordinates are not coded.
 *
 *   norms, nibbles  a qsgd_quantize output (device), 4-byte aligned
 *   n, d            d a multiple of 8, 8 <= d <= 2048
 *   bit_offsets     out, uint64[ceil(n/d) + 1], 8-byte aligned: where bucket
 *                   b starts; the last entry is the total length in bits
 *   out_words       out, uint32[capacity_words]; words past the capacity are
 *                   not written (qsgd_elias_max_words bounds what is needed)
 *
 * Errors: GCQ_ERR_PARAM (d), GCQ_ERR_NULL, GCQ_ERR_ALIGN, GCQ_ERR_OVERLAP,
 * GCQ_ERR_LAUNCH.
 */
int qsgd_elias_encode(const float *norms, const uint32_t *nibbles, size_t n, uint32_t d,
                      uint64_t *bit_offsets, uint32_t *out_words, size_t capacity_words,
                      void *stream);

/*
 * qsgd_elias_decode -- the inverse: norms and nibble words from coded buckets
 * (in_words holds in_count words; nothing past them or past a bucket's end
 * is read, and a malformed bucket stops at its last whole coordinate).
 * Coordinates the code does not name get nibble 0.
 *
 * Errors: as qsgd_elias_encode.
 */
int qsgd_elias_decode(const uint32_t *in_words, size_t in_count, const uint64_t *bit_offsets,
                      size_t n, uint32_t d, float *norms, uint32_t *nibbles, void *stream);

/* ------------------------------------------------------------------ */
/* SAPS: shared-seed random sparsification, single-peer exchange       */
/* ------------------------------------------------------------------ */

/*
 * saps_mask -- the sparsification mask of "Communication-Efficient
 * Decentralized Learning with Sparsification and Adaptive Peer Selection":
 * entries Bernoulli(1/c) drawn from a seed that every worker shares, so all
 * workers keep the same components.  Element i is kept when u_i * c < 1
 * (exactly), u_i = the 24-bit uniform of qsgd_quantize's generator for
 * (seed, i).
 *
 *   n             element count
 *   c             finite, >= 1 (the compression ratio; 1 keeps everything)
 *   seed          the shared seed
 *   mask_words    out, uint32[saps_mask_words(n)], 4-byte aligned; bit j of
 *                 word w is element 32w + j (bits past n are 0)
 *   tile_offsets  out, uint64[saps_num_tiles(n) + 1], 8-byte aligned: entry t
 *                 is the number of kept elements before element 8192 t (an
 *                 exclusive prefix over 8192-element tiles); the last entry
 *                 is the total kept count (read it after a synchronize to
 *                 size the value buffer)
 *
 * Errors: GCQ_ERR_PARAM (c), GCQ_ERR_NULL, GCQ_ERR_ALIGN, GCQ_ERR_OVERLAP,
 * GCQ_ERR_LAUNCH.
 */
int saps_mask(size_t n, float c, uint64_t seed, uint32_t *mask_words, uint64_t *tile_offsets,
              void *stream);

/*
 * saps_gather -- the components a worker sends: values[r] = x[i_r] for the
 * kept indices i_0 < i_1 < ... (mask and offsets from saps_mask).  Only
 * ranks below `capacity` are written (size the buffer with the total count).
 *
 *   x         in, float32[n], 4-byte aligned
 *   values    out, float32[capacity], 4-byte aligned
 *
 * Errors: GCQ_ERR_PARAM, GCQ_ERR_NULL, GCQ_ERR_ALIGN, GCQ_ERR_OVERLAP,
 * GCQ_ERR_LAUNCH.
 */
int saps_gather(const float *x, size_t n, const uint32_t *mask_words,
                const uint64_t *tile_offsets, float *values, size_t capacity, void *stream);

/*
 * saps_merge -- the receiving side of the single-peer exchange: each row of
 * the gossip matrix has two non-zero entries and the matrix is doubly
 * stochastic, read as an equal-weight average: for every kept index i_r
 * with r < capacity, x[i_r] = (x[i_r] + peer_values[r]) * 0.5 in float32;
 * other components are unchanged.  The peer used the same seed, so its
 * values are in the same order.
 *
 *   x            in/out, float32[n], 4-byte aligned
 *   peer_values  in, float32[capacity], 4-byte aligned
 *
 * Errors: as saps_gather.
 */
int saps_merge(float *x, size_t n, const uint32_t *mask_words, const uint64_t *tile_offsets,
               const float *peer_values, size_t capacity, void *stream);

/* ------------------------------------------------------------------ */
/* Sizes and status names (pure host functions, no device access)      */
/* ------------------------------------------------------------------ */

/* ceil(n/16): packed 2-bit words for n elements (MXNet PR, "Format of
 * compressed gradient": 16 codes per 32-bit element, 1/16 the size). */
size_t gc2_packed_words(size_t n);
/* ceil(n/d): QSGD buckets of d consecutive coordinates, the last one ragged
 * (QSGD summary, Knowl 8: the vector is split into buckets of size d, each
 * quantized with its own scale); returns 0 for d == 0. */
size_t qsgd_num_buckets(size_t n, uint32_t d);
/* ceil(n/8): 32-bit words of the nibble stream.  Knowl 2 sends a sign and a
 * level per coordinate; with s <= 7 both fit one 4-bit nibble (bit 3 the
 * sign, bits 2..0 the level), 8 per word. */
size_t qsgd_nibble_words(size_t n);
/* An upper bound of the words qsgd_elias_encode writes (0 for a bad d). */
size_t qsgd_elias_max_words(size_t n, uint32_t d);
/* ceil(n/32): SAPS mask words. */
size_t saps_mask_words(size_t n);
/* ceil(n/8192): SAPS tiles (saps_mask writes one more offset than this). */
size_t saps_num_tiles(size_t n);
/* Static, never-NULL name of a status code. */
const char *gcq_status_string(int status);

/* ------------------------------------------------------------------ */
/* Measurement probes (not part of the method)                         */
/* ------------------------------------------------------------------ */

/*
 * Kernels with a hot-path kernel's HBM access pattern and none of its
 * arithmetic.  Timed beside that kernel they give the practical ceiling of
 * its access pattern on the device at hand, against which its own time is
 * judged (the 8 TB/s HBM peak is not reachable by any access pattern).
 *
 * gcq_probe_stream -- the 2-bit quantizer's pattern (its default launch
 * geometry, 1024 elements per 256-thread workgroup, one float4 per lane
 * and stream): reads a (and b, unless NULL), writes c, and, unless words is
 * NULL, one 32-bit word per 16 elements in 64-byte runs.  c = a XOR b bit for
 * bit (c = a without b); word 16k + L holds the bits of c[256k + 4L] (L < 16).
 * With a, b, c and words it moves the quantizer's 12.25 bytes per element;
 * with a and c alone it is a copy.
 *   a, b, c  float32[n], 16-byte aligned; words uint32[n/16], 4-byte aligned
 *   n        a multiple of 1024
 * Errors: GCQ_ERR_PARAM (n), GCQ_ERR_NULL (a or c), GCQ_ERR_ALIGN,
 * GCQ_ERR_OVERLAP (c or words intersects another operand; c may be b
 * itself, in place, as the quantizer updates r), GCQ_ERR_LAUNCH.
 *
 * gcq_probe_reduce -- gc2_dequant_reduce's own kernel and launch (the same
 * loads, LDS staging, stores, launch knobs and checks, no threshold) with
 * the decode replaced by an XOR: acc[16i] holds the XOR of the W workers'
 * word i, the other 15 sums of each word are +0.
 */
int gcq_probe_stream(const float *a, const float *b, float *c, uint32_t *words, size_t n,
                     void *stream);
int gcq_probe_reduce(const uint32_t *const *words, uint32_t W, size_t n, float *acc,
                     void *stream);

/* ------------------------------------------------------------------ */
/* Launch knobs: they change speed, never results                      */
/* ------------------------------------------------------------------ */

/*
 * How the kernels map work onto the GPU.  Every setting produces
 * bit-identical outputs; only the time differs.
 */
typedef struct gcq_tuning {
    int gc2_unroll;        /* 2-bit quantizer: float4 per lane and stream,
                              1, 2 or 4.  A workgroup quantizes 1024 * U
                              consecutive elements of a bucket, each lane U
                              float4 of g and of r; quads of lanes assemble
                              the packed words.  Default 1 */
    int gc2_nt;            /* non-temporal hints in the 2-bit quantizer, a mask:
                              1 g loads, 2 r loads, 4 r stores, 8 packed-word
                              stores (default 7: all but the packed words) */
    int gc2_blocks_per_cu; /* 0: one tile per workgroup (default);
                              k > 0: k workgroups per compute unit, grid-stride */
    int dq_nt_loads;       /* 1: non-temporal loads of the packed words in
                              gc2_dequant_reduce */
    int dq_nt_stores;      /* 1: non-temporal stores of the sums */
    int dq_lds_stores;     /* 1: stage each wavefront's sums through LDS so
                              every store instruction writes 1 KiB of
                              consecutive memory; 0: each lane stores its 16
                              consecutive sums directly */
    int dq_blocks_per_cu;  /* 0: one packed word position per thread (default);
                              k > 0: k workgroups per compute unit, grid-stride */
    int dq_fp4_decode;     /* 1: decode two codes per instruction with the FP4
                              conversion (default); 0: one signed-byte
                              conversion per code */
    int qsgd_nt;           /* 1: non-temporal hints in the QSGD quantizer
                              (default) */
    int qsgd_rcp;          /* 1: division-free level arithmetic in the QSGD
                              quantizer that provably reproduces the results of
                              the per-element IEEE division, with an exact
                              fallback where it cannot (default); 0: one IEEE
                              division per element */
    int qsgd_dequant_nt;   /* 1: non-temporal hints in qsgd_dequant */
    int qsgd_blocks_per_cu; /* fused QSGD quantizer (d a multiple of 256, up to
                               2048): 0: one wavefront per group of buckets
                               (default); k > 0: k workgroups per compute
                               unit, each wavefront strides over many groups */
    int qsgd_dequant_blocks_per_cu; /* qsgd_dequant: 0: one wavefront per
                               1024 elements; k > 0: k workgroups per compute
                               unit, grid-stride (default 0) */
    int qsgd_buckets_per_wave; /* fused QSGD quantizer: buckets H a
                               wavefront takes at once, one per group of 64/H
                               lanes: 1, 2 or 4, limited to d H <= 1024; 0:
                               H = 1024/d for d <= 1024, else 1 (default) */
    int dq_words_per_thread; /* gc2_dequant_reduce: packed words per thread,
                               1 or 2 (8-byte loads, used when every worker
                               array is 8-byte aligned, else 1); 0: 2 from
                               2^22 words (2^26 elements) per launch, else 1
                               (default) */
    int dq_resident_per_cu; /* gc2_dequant_reduce: at most this many
                               workgroups resident per compute unit, set through
                               the kernel's LDS allocation: 0 (no cap) or 2..8
                               (default 3) */
    int gc2_resident_per_cu; /* the 2-bit quantizer: the same cap, 0 (no cap,
                               default) or 2..8 */
    int cdsgd_resident_per_cu; /* the CD-SGD kernels (update fused with the
                               quantizer, update alone): the same cap, 0 (no
                               cap) or 2..8 (default 5) */
    int qsgd_avg_resident_per_cu; /* qsgd_dequant_average: the same cap, 0
                               (no cap, default) or 2..8 */
} gcq_tuning;

/*
 * gcq_get_tuning -- copy the current knobs into *out (host struct).  The
 * initial values are the library defaults, overridden by the environment
 * variables GCQ_GC2_UNROLL, GCQ_GC2_NT, GCQ_GC2_BLOCKS_PER_CU,
 * GCQ_DQ_NT_LOADS, GCQ_DQ_NT_STORES, GCQ_DQ_LDS_STORES, GCQ_DQ_FP4_DECODE,
 * GCQ_DQ_BLOCKS_PER_CU, GCQ_DQ_WORDS_PER_THREAD, GCQ_DQ_RESIDENT_PER_CU,
 * GCQ_GC2_RESIDENT_PER_CU, GCQ_CDSGD_RESIDENT_PER_CU, GCQ_QSGD_AVG_RESIDENT_PER_CU,
 * GCQ_QSGD_NT, GCQ_QSGD_RCP,
 * GCQ_QSGD_DEQUANT_NT, GCQ_QSGD_BLOCKS_PER_CU, GCQ_QSGD_DEQUANT_BLOCKS_PER_CU
 * and GCQ_QSGD_BUCKETS_PER_WAVE when set (block counts and gc2_nt are
 * clamped into range, a flag reads any nonzero value as 1, and any other
 * invalid value takes the default).
 * Errors: GCQ_ERR_NULL.
 *
 * gcq_set_tuning -- replace the knobs with *t (host struct).  Takes effect
 * for calls made after it returns; it must not run concurrently with
 * another call of this library.  Errors: GCQ_ERR_NULL, GCQ_ERR_PARAM (a
 * flag not 0/1, gc2_nt outside 0..15, gc2_unroll not 1/2/4, a block
 * count outside 0..1024, qsgd_buckets_per_wave not 0/1/2/4,
 * dq_words_per_thread not 0..2, a *_resident_per_cu knob not 0 or 2..8); on
 * error
 * nothing changes.
 */
int gcq_get_tuning(gcq_tuning *out);
int gcq_set_tuning(const gcq_tuning *t);

#ifdef __cplusplus
}
#endif

#endif /* GCQ_H */
