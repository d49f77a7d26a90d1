// elias.hip -- Elias-omega coding of QSGD buckets ("QSGD: Communication-
// Efficient SGD via Gradient Quantization and Encoding", chapterpal summary,
// Knowl 2: the norm in 32 bits, the non-zero coordinates coded by the omega
// code of the distance between them, with their sign and level; the omega
// code of P. Elias, "Universal codeword sets and representations of the
// integers", 1975) for gfx950.
//
// Layout: per bucket, the 32 norm bits, then for each coordinate whose
// level is not 0, omega(distance from the previous one; the first from -1),
// one sign bit, omega(level); buckets follow each other unpadded, bits most
// significant first in 32-bit words; bit_offsets[b] is where bucket b starts
// and bit_offsets[nb] the total length.
//
// Encode, one wavefront per bucket (d a multiple of 8, at most 2048):
//   lengths -- per chunk of 64 coordinates, a ballot of the non-zero ones
//              gives each its predecessor and code length; the bucket's
//              length goes to the offsets array, then an exclusive scan;
//   zero    -- each bucket that starts inside a word clears that word (it is
//              shared with the previous bucket);
//   write   -- the wavefront assembles its bucket's bits in LDS (LDS atomic
//              ORs at the scanned positions) and writes the words out: plain
//              stores, atomic ORs for the two words it may share.
// Decode is sequential per bucket (variable-length codes): one thread per
// bucket, every read checked against the bucket's end.
#include "gcq_device.h"
#include "gcq_internal.h"

namespace gcq {

namespace {

__device__ __host__ __forceinline__ uint32_t bit_length(uint32_t k)
{
    return k ? 32u - (uint32_t)__builtin_clz(k) : 0u;
}

// omega(k) as a right-aligned bit string and its length (k >= 1, at most 32
// bits for the values here: distances up to 2048, levels up to 7).
__device__ __forceinline__ uint32_t omega_code(uint32_t k, uint32_t &len)
{
    uint64_t code = 0;   // the final 0
    len = 1;
    while (k > 1) {
        const uint32_t b = bit_length(k);
        code |= (uint64_t)k << len;
        len += b;
        k = b - 1;
    }
    return (uint32_t)code;
}

__device__ __host__ __forceinline__ uint32_t omega_length(uint32_t k)
{
    uint32_t len = 1;
    while (k > 1) {
        const uint32_t b = bit_length(k);
        len += b;
        k = b - 1;
    }
    return len;
}

// The per-coordinate step shared by both encode passes: for coordinate li of
// the bucket (one per lane in this chunk), its nibble, whether it is coded,
// its code length, and the exclusive bit position within the bucket's codes.
struct Coord {
    uint32_t nib, len, code_d, len_d;
    uint64_t pos;
};

__device__ __forceinline__ Coord coord_step(const uint32_t *__restrict__ nibbles, uint64_t lo,
                                            uint32_t li, uint32_t bucket_len, uint32_t lane,
                                            int32_t &prev, uint64_t &bits)
{
    Coord c;
    c.nib = 0;
    if (li < bucket_len) {
        const uint64_t i = lo + li;
        c.nib = (nibbles[i >> 3] >> (28u - 4u * (uint32_t)(i & 7u))) & 15u;
    }
    const bool nz = (c.nib & 7u) != 0u;
    const uint64_t mask = __ballot(nz);
    const uint64_t below = mask & ((1ull << lane) - 1ull);
    const int32_t chunk0 = (int32_t)(li - lane);
    const int32_t p = below ? chunk0 + 63 - (int32_t)__builtin_clzll(below) : prev;
    c.code_d = 0;
    c.len_d = 0;
    c.len = 0;
    if (nz) {
        c.code_d = omega_code((uint32_t)((int32_t)li - p), c.len_d);
        c.len = c.len_d + 1u + omega_length(c.nib & 7u);
    }
    // exclusive scan of the lengths across the wavefront
    uint32_t incl = c.len;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off, kWave);
        if (lane >= (uint32_t)off)
            incl += y;
    }
    c.pos = bits + incl - c.len;
    bits += __shfl(incl, kWave - 1, kWave);
    if (mask)
        prev = chunk0 + 63 - (int32_t)__builtin_clzll(mask);
    return c;
}

__global__ __launch_bounds__(kWave) void elias_length_kernel(const uint32_t *__restrict__ nibbles,
                                                              uint64_t n, uint32_t d, uint64_t nb,
                                                              uint64_t *__restrict__ offs)
{
    const uint32_t lane = threadIdx.x;
    for (uint64_t b = blockIdx.x; b < nb; b += gridDim.x) {
        const uint64_t lo = b * d;
        const uint32_t blen = (uint32_t)(lo + d < n ? d : n - lo);
        int32_t prev = -1;
        uint64_t bits = 0;
        for (uint32_t c0 = 0; c0 < blen; c0 += kWave)
            (void)coord_step(nibbles, lo, c0 + lane, blen, lane, prev, bits);
        if (lane == 0)
            offs[b] = 32u + bits;
    }
}

__global__ __launch_bounds__(kBlockThreads) void elias_zero_kernel(const uint64_t *__restrict__ offs,
                                                                    uint64_t nb,
                                                                    uint32_t *__restrict__ out,
                                                                    uint64_t cap)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t b = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += stride) {
        const uint64_t o = offs[b];
        if ((o & 31u) && (o >> 5) < cap)
            out[o >> 5] = 0u;
    }
}

__global__ __launch_bounds__(kWave) void elias_write_kernel(const float *__restrict__ norms,
                                                             const uint32_t *__restrict__ nibbles,
                                                             uint64_t n, uint32_t d, uint64_t nb,
                                                             const uint64_t *__restrict__ offs,
                                                             uint32_t *__restrict__ out,
                                                             uint64_t cap, uint32_t lds_words)
{
    extern __shared__ uint32_t bucket_bits[];
    const uint32_t lane = threadIdx.x;
    for (uint64_t b = blockIdx.x; b < nb; b += gridDim.x) {
        const uint64_t lo = b * d;
        const uint32_t blen = (uint32_t)(lo + d < n ? d : n - lo);
        const uint64_t start = offs[b], end = offs[b + 1];
        const uint32_t sh = (uint32_t)(start & 31u);
        for (uint32_t k = lane; k < lds_words; k += kWave)
            bucket_bits[k] = 0u;
        __syncthreads();
        if (lane == 0) {
            const uint64_t v = (uint64_t)__float_as_uint(norms[b]) << (32u - sh);
            atomicOr(&bucket_bits[0], (uint32_t)(v >> 32));
            atomicOr(&bucket_bits[1], (uint32_t)v);
        }
        int32_t prev = -1;
        uint64_t bits = 0;
        for (uint32_t c0 = 0; c0 < blen; c0 += kWave) {
            const Coord c = coord_step(nibbles, lo, c0 + lane, blen, lane, prev, bits);
            if (c.len) {
                // code = omega(dist) | sign | omega(level), c.len <= 26 bits
                uint32_t len_l;
                const uint32_t code_l = omega_code(c.nib & 7u, len_l);
                const uint64_t code = ((((uint64_t)c.code_d << 1) | (c.nib >> 3)) << len_l) | code_l;
                const uint64_t p = (uint64_t)sh + 32u + c.pos;     // < lds_words * 32
                const uint32_t w = (uint32_t)(p >> 5), o = (uint32_t)(p & 31u);
                const uint64_t v = code << (64u - c.len - o);
                atomicOr(&bucket_bits[w], (uint32_t)(v >> 32));
                if ((uint32_t)v)
                    atomicOr(&bucket_bits[w + 1], (uint32_t)v);
            }
        }
        __syncthreads();
        const uint64_t nw = (sh + (end - start) + 31u) >> 5;
        const bool shares_last = ((end & 31u) != 0u) && (b + 1 < nb);
        for (uint64_t k = lane; k < nw; k += kWave) {
            const uint64_t gw = (start >> 5) + k;
            if (gw >= cap)
                continue;
            const uint32_t v = bucket_bits[k];
            if ((k == 0 && sh) || (k == nw - 1 && shares_last))
                atomicOr(&out[gw], v);
            else
                out[gw] = v;
        }
        __syncthreads();
    }
}

// Sequential decode of one bucket per thread.  The bits stream through a
// 64-bit register window refilled a word at a time (one load per 32 bits
// consumed); the bucket's nibble words are built in a register and stored
// once each.  Nothing past the bucket's end or the input is read; a code
// that would run past the end stops the bucket (it then keeps the
// coordinates decoded so far).
struct BitReader {
    const uint32_t *in;
    uint64_t word;        // next word to load
    uint64_t left;        // bits of the bucket not yet consumed
    uint64_t buf;         // window, next bit in bit 63
    uint32_t avail;       // valid bits in the window
    bool ok;

    __device__ void refill()
    {
        while (avail <= 32u && (uint64_t)avail < left) {
            buf |= (uint64_t)in[word++] << (32u - avail);
            avail += 32u;
        }
    }
    __device__ uint32_t get(uint32_t nbits)   // 1..32 bits
    {
        if (!ok || nbits > left) {
            ok = false;
            return 0u;
        }
        refill();
        const uint32_t v = (uint32_t)(buf >> (64u - nbits));
        buf <<= nbits;
        avail -= nbits;
        left -= nbits;
        return v;
    }
    __device__ uint32_t omega()
    {
        uint32_t k = 1;
        while (ok && get(1)) {
            if (k >= 31u) {
                ok = false;
                return 0u;
            }
            k = (1u << k) | get(k);
        }
        return k;
    }
};

__global__ __launch_bounds__(kBlockThreads) void elias_decode_kernel(
    const uint32_t *__restrict__ in, const uint64_t *__restrict__ offs, uint64_t n, uint32_t d,
    uint64_t nb, uint64_t in_words, float *__restrict__ norms, uint32_t *__restrict__ nibbles)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t b = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += stride) {
        const uint64_t lo = b * d;
        const uint32_t blen = (uint32_t)(lo + d < n ? d : n - lo);
        const uint32_t nw = (blen + 7u) / 8u;
        uint32_t *nib = nibbles + (lo >> 3);
        uint64_t start = offs[b], end = offs[b + 1];
        if (end > in_words * 32u)
            end = in_words * 32u;
        if (start > end)
            start = end;
        BitReader r{in, start >> 5, end - start, 0u, 0u, true};
        // the first word may begin mid-word: load it and drop the bits before
        // the bucket
        const uint32_t skip = (uint32_t)(start & 31u);
        if (end > start) {
            r.buf = (uint64_t)in[r.word++] << 32;
            r.avail = 32u;
            r.buf <<= skip;
            r.avail -= skip;
        }
        norms[b] = __uint_as_float(r.get(32));
        int64_t prev = -1;
        uint32_t cur = 0, cur_w = 0;   // nibble word being built, and its index
        while (r.ok && r.left) {
            const int64_t li = prev + (int64_t)r.omega();
            const uint32_t sign = r.get(1);
            const uint32_t level = r.omega();
            if (!r.ok || li >= (int64_t)blen || level > 7u)
                break;
            const uint32_t w = (uint32_t)li >> 3;
            while (cur_w < w) {            // words before this coordinate are done
                nib[cur_w++] = cur;
                cur = 0;
            }
            cur |= ((sign << 3) | level) << (28u - 4u * ((uint32_t)li & 7u));
            prev = li;
        }
        while (cur_w < nw) {
            nib[cur_w++] = cur;
            cur = 0;
        }
    }
}

// Largest code of one coordinate for bucket length d: omega(d) + 1 + omega(7).
uint32_t max_coord_bits(uint32_t d) { return omega_length(d) + 1u + omega_length(7u); }

}  // namespace

uint64_t elias_max_words(uint64_t n, uint32_t d)
{
    if (!d)
        return 0;
    const uint64_t nb = (n + d - 1) / d;
    return (nb * 32u + n * (uint64_t)max_coord_bits(d) + 31u) / 32u + 1u;
}

hipError_t launch_elias_encode(const float *norms, const uint32_t *nibbles, uint64_t n, uint32_t d,
                               uint64_t *offs, uint32_t *out, uint64_t cap, hipStream_t stream)
{
    const uint64_t nb = (n + d - 1) / d;
    if (nb) {
        const uint32_t grid = grid_for(nb, 0);
        elias_length_kernel<<<grid, kWave, 0, stream>>>(nibbles, n, d, nb, offs);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    hipError_t e = launch_exclusive_scan_u64(offs, nb, stream);
    if (e != hipSuccess || !nb)
        return e;
    elias_zero_kernel<<<grid_for((nb + kBlockThreads - 1) / kBlockThreads, 0), kBlockThreads, 0,
                        stream>>>(offs, nb, out, cap);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    // LDS for one bucket: shift + norm + every coordinate at its longest code,
    // plus the word a code may spill into
    const uint32_t lds_words = (31u + 32u + d * max_coord_bits(d) + 31u) / 32u + 1u;
    elias_write_kernel<<<grid_for(nb, 0), kWave, (size_t)lds_words * 4u, stream>>>(
        norms, nibbles, n, d, nb, offs, out, cap, lds_words);
    return hipGetLastError();
}

hipError_t launch_elias_decode(const uint32_t *in, const uint64_t *offs, uint64_t n, uint32_t d,
                               uint64_t in_words, float *norms, uint32_t *nibbles,
                               hipStream_t stream)
{
    const uint64_t nb = (n + d - 1) / d;
    if (!nb)
        return hipSuccess;
    elias_decode_kernel<<<grid_for((nb + kBlockThreads - 1) / kBlockThreads, 0), kBlockThreads, 0,
                          stream>>>(in, offs, n, d, nb, in_words, norms, nibbles);
    return hipGetLastError();
}

}  // namespace gcq
