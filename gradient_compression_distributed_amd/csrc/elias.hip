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
// Encode (d a multiple of 8, at most 2048): one lane per bucket, a
// wavefront per 64 consecutive buckets.  A lane loads its bucket's nibble
// words 512 coordinates at a time, all sixteen 16-byte blocks at once (the
// lanes' loads are 256 bytes apart; issued together, the requests for one
// cache line arrive together), and works on them from registers:
//   lengths -- per nibble word, the code bits of its coordinates from
//              popcounts, plus the omega length of its first distance; the
//              lengths go through an exclusive scan into the offsets;
//   zero    -- each bucket that starts inside a word clears that word (it is
//              shared with the previous bucket);
//   write   -- block by block (32 coordinates), each lane appends the codes
//              of its coded coordinates to a 64-bit window and hands each
//              completed word to the wavefront's LDS stage (an OR: a word two
//              buckets share gets both), which leaves with coalesced stores;
//              a wavefront whose words exceed the stage stores directly,
//              atomic ORs on the shared words.
// Decode: one lane per bucket (variable-length codes are read in order), a
// wavefront per 64 consecutive buckets.  Their bits, one contiguous range,
// are first copied into LDS with coalesced loads; each coordinate is then
// parsed from a 64-bit register window and ORed into the lane's nibble
// chunk in LDS, which leaves as one 16-byte store per 32 coordinates.
// Every read stays inside the bucket and the input.
#include "gcq_device.h"
#include "gcq_internal.h"

namespace gcq {

namespace {

__device__ __host__ __forceinline__ uint32_t bit_length(uint32_t k)
{
    return k ? 32u - (uint32_t)__builtin_clz(k) : 0u;
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

// omega lengths L(k) = b + L(b - 1), b the bit length of k, L(0) = 0: for
// k <= 11 the table below (4 bits per entry, entry k at bit 4k), so for
// 1 <= k <= 4095 one lookup after the bit length.
constexpr uint64_t kOmegaLenTable = 0x777766663310ull;

__device__ __forceinline__ uint32_t omega_len_small(uint32_t k)   // 0 <= k <= 11
{
    return (uint32_t)(kOmegaLenTable >> (4u * k)) & 15u;
}

__device__ __forceinline__ uint32_t omega_len_fast(uint32_t k)   // 1 <= k <= 4095
{
    const uint32_t b = 32u - (uint32_t)__builtin_clz(k);
    return b + omega_len_small(b - 1u);
}

// omega(k) right-aligned, 1 <= k <= 4095: at most three groups (the binary
// digits of k, of its bit length - 1, ...), the last one found first in the
// code, then the final 0.
__device__ __forceinline__ uint32_t omega_code_fast(uint32_t k, uint32_t &len)
{
    uint32_t code = 0, n = 1;
#pragma unroll
    for (int g = 0; g < 3; ++g) {
        if (k > 1u) {
            const uint32_t b = 32u - (uint32_t)__builtin_clz(k);
            code |= k << n;
            n += b;
            k = b - 1u;
        }
    }
    len = n;
    return code;
}

// Per nibble word: bit 4k set when nibble k (from the least significant
// end) has a non-zero level.  Coordinate j of the word is nibble 7 - j: its
// level in bits 28 - 4j .. 30 - 4j, its sign in bit 31 - 4j.
__device__ __forceinline__ uint32_t nonzero_nibbles(uint32_t w)
{
    return (w | (w >> 1) | (w >> 2)) & 0x11111111u;
}

// Coded coordinates of a nibble word as an 8-bit mask, coordinate j of the
// word in bit 7 - j (so the previous coordinate is one bit higher).
__device__ __forceinline__ uint32_t coord_mask8(uint32_t w)
{
    uint32_t m = nonzero_nibbles(w);       // bit 4k: nibble k from the least significant
    m = (m | (m >> 3)) & 0x03030303u;
    m = (m | (m >> 6)) & 0x000F000Fu;
    return (m | (m >> 12)) & 0xFFu;
}

// Code bits of a nibble word's coordinates except the omega code of its
// first coordinate's distance (which depends on earlier words), from
// nz = nonzero_nibbles(w) (bit 4k set: nibble k, coordinate 7 - k, coded):
//   sign + omega(level): 1 + L(level) = 2, 4 or 7 bits for levels 1, 2-3,
//   4-7, counted with popcounts of the level bits;
//   omega(gap) for each later coordinate of the word, gap <= 7: L = 1, 3 or
//   6, i.e. 1 + 2 [gap >= 2] + 3 [gap >= 4], where gap >= 2 means the
//   coordinate just before (one nibble higher) is not coded, gap >= 4 the
//   three before.
__device__ __forceinline__ uint32_t word_code_bits(uint32_t w, uint32_t nz)
{
    const uint32_t ge2 = ((w >> 1) | (w >> 2)) & 0x11111111u;
    const uint32_t ge4 = (w >> 2) & 0x11111111u;
    const uint32_t rest = nz ? nz & ~(0x80000000u >> (uint32_t)__builtin_clz(nz)) : 0u;
    const uint32_t gap2 = rest & ~(nz >> 4);
    const uint32_t gap4 = gap2 & ~(nz >> 8) & ~(nz >> 12);
    return 2u * (uint32_t)__builtin_popcount(nz) + 2u * (uint32_t)__builtin_popcount(ge2) +
           3u * (uint32_t)__builtin_popcount(ge4) + (uint32_t)__builtin_popcount(rest) +
           2u * (uint32_t)__builtin_popcount(gap2) + 3u * (uint32_t)__builtin_popcount(gap4);
}

// Encode: one lane per bucket, a wavefront per 64 consecutive buckets (the
// decode's layout).  A lane reads its bucket's nibble words in order, 16
// bytes at a time with the next 16 in flight.

// Block k (words 4k .. 4k+3) of a bucket of nw nibble words at p, zeros
// past nw.  Vec: p is 16-byte aligned, and a block wholly inside the
// bucket is one 16-byte load; other blocks are read word by word.
template <bool Vec>
__device__ __forceinline__ uint4 nib_block(const uint32_t *__restrict__ p, uint32_t k, uint32_t nw)
{
    const uint32_t w0 = 4u * k;
    if (Vec && w0 + 4u <= nw)
        return reinterpret_cast<const uint4 *>(p)[k];
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (w0 < nw)
        v.x = p[w0];
    if (w0 + 1u < nw)
        v.y = p[w0 + 1u];
    if (w0 + 2u < nw)
        v.z = p[w0 + 2u];
    if (w0 + 3u < nw)
        v.w = p[w0 + 3u];
    return v;
}

// Nibble word j of a bucket of blen coordinates, the coordinates at or past
// blen cleared.
__device__ __forceinline__ uint32_t clip_word(uint32_t w, uint32_t j, uint32_t blen)
{
    const uint32_t li0 = 8u * j;
    if (li0 + 8u <= blen)
        return w;
    return li0 < blen ? w & (~0u << (4u * (li0 + 8u - blen))) : 0u;
}

__device__ __forceinline__ uint32_t word_of(uint4 v, uint32_t q)   // word q (0..3) of a block
{
    return q == 0u ? v.x : q == 1u ? v.y : q == 2u ? v.z : v.w;
}

// Bucket lengths in bits: the norm's 32, then per nibble word the code bits
// of its coordinates (word_code_bits) and the omega length of its first
// coordinate's distance from the lane's previous coded coordinate.
template <bool Vec>
__global__ __launch_bounds__(kBlockThreads) void elias_length_kernel(
    const uint32_t *__restrict__ nibbles, uint64_t n, uint32_t d, uint64_t nb,
    uint64_t *__restrict__ offs)
{
    const uint64_t b = (uint64_t)blockIdx.x * kBlockThreads + threadIdx.x;
    if (b >= nb)
        return;
    const uint64_t lo = b * d;
    const uint32_t blen = (uint32_t)(lo + d < n ? d : n - lo);
    const uint32_t nw = (blen + 7u) / 8u;
    const uint32_t nblk = (nw + 3u) / 4u;
    const uint32_t *p = nibbles + (lo >> 3);
    uint32_t bits = 32u;
    int32_t prev = -1;
    // 512 coordinates at a time: their 16 blocks loaded together
    constexpr uint32_t kB = 16;
    for (uint32_t k0 = 0; k0 < nblk; k0 += kB) {
        uint4 blk[kB];
#pragma unroll
        for (uint32_t t = 0; t < kB; ++t)
            blk[t] = k0 + t < nblk ? nib_block<Vec>(p, k0 + t, nw) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (uint32_t t = 0; t < kB; ++t) {
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q) {
                const uint32_t j = 4u * (k0 + t) + q;
                const uint32_t w = clip_word(word_of(blk[t], q), j, blen);
                const uint32_t nz = nonzero_nibbles(w);
                // the word's first and last coded coordinates: its highest and
                // lowest set bits (bit 4k is coordinate 7 - k)
                const int32_t first = (int32_t)(8u * j + ((uint32_t)__builtin_clz(nz | 1u) >> 2));
                const int32_t gap = first - prev > 1 ? first - prev : 1;   // >= 1 when nz != 0
                const uint32_t add = word_code_bits(w, nz) + omega_len_fast((uint32_t)gap);
                bits += nz ? add : 0u;
                prev = nz ? (int32_t)(8u * j + 7u - ((uint32_t)__builtin_ctz(nz) >> 2)) : prev;
            }
        }
    }
    offs[b] = bits;
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

// Staged output words per wavefront (as the decode stages its input): with
// the omega table of 1..d, four workgroups fit a compute unit for d <= 2048.
constexpr uint32_t kEncodeStageWords = 31u * kWave;

// The code words.  LDS: the omega codes of 1..d ((length << 24) | code, one
// word each, shared by the workgroup), then per wavefront the stage of its
// 64 buckets' words.  Each lane appends its bucket's codes to a 64-bit
// window (next free bit `fill` of word wi) and hands each word on as it
// completes: ORed into the stage, which the wavefront then stores with
// coalesced stores, or, when the wavefront's words do not fit the stage,
// stored directly.  A word two buckets share is ORed by both: in the stage,
// or, in memory, with an atomic OR on the word the zero kernel cleared.
template <bool Vec>
__global__ __launch_bounds__(kBlockThreads) void elias_write_kernel(
    const float *__restrict__ norms, const uint32_t *__restrict__ nibbles, uint64_t n, uint32_t d,
    uint64_t nb, const uint64_t *__restrict__ offs, uint32_t *__restrict__ out, uint64_t cap)
{
    extern __shared__ uint32_t elias_lds[];
    const uint32_t lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    uint32_t *codes = elias_lds;
    uint32_t *stage = elias_lds + (d + 1u) + wave * kEncodeStageWords;
    for (uint32_t k = threadIdx.x + 1u; k <= d; k += kBlockThreads) {
        uint32_t len;
        const uint32_t c = omega_code_fast(k, len);
        codes[k] = (len << 24) | c;
    }
    __syncthreads();
    const uint64_t b0 = ((uint64_t)blockIdx.x * kBlockWaves + wave) * kWave;
    if (b0 >= nb)
        return;   // (no barrier below)
    const uint64_t b = b0 + lane;
    const bool valid = b < nb;
    const uint32_t last = (uint32_t)(nb - b0 < kWave ? nb - b0 - 1u : kWave - 1u);
    uint64_t start = 0, end = 0;
    if (valid) {
        start = offs[b];
        end = offs[b + 1];
    }
    // the wavefront's words [wlo, whi): its buckets are consecutive
    const uint64_t s0 = __shfl(start, 0, kWave);
    const uint64_t e_last = __shfl(end, (int)last, kWave);
    const uint64_t wlo = s0 >> 5, whi = (e_last + 31u) >> 5;
    const bool staged = whi - wlo <= kEncodeStageWords;
    if (staged)
        for (uint64_t k = lane; k < whi - wlo; k += kWave)
            stage[k] = 0u;
    // LDS operations of a wavefront take effect in order; keep the compiler
    // from moving the ORs below above the clears
    __builtin_amdgcn_wave_barrier();
    const bool share_first = (start & 31u) != 0u;
    const bool share_last = (end & 31u) != 0u && b + 1 < nb;
    auto emit = [&](uint64_t gw, uint32_t v) {
        if (staged) {
            __hip_atomic_fetch_or(stage + (gw - wlo), v, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_WORKGROUP);
        } else if (gw < cap) {
            if ((gw == (start >> 5) && share_first) || (gw == ((end - 1u) >> 5) && share_last))
                atomicOr(out + gw, v);
            else
                out[gw] = v;
        }
    };
    const uint64_t lo = valid ? b * d : 0u;
    const uint32_t blen = valid ? (uint32_t)(lo + d < n ? d : n - lo) : 0u;
    const uint32_t nw = (blen + 7u) / 8u;
    const uint32_t *p = nibbles + (lo >> 3);
    uint64_t wi = start >> 5;
    uint32_t fill = (uint32_t)(start & 31u);
    uint64_t acc = 0;
    if (valid) {   // the norm's 32 bits complete the first word
        acc = (uint64_t)__float_as_uint(norms[b]) << (32u - fill);
        emit(wi, (uint32_t)(acc >> 32));
        acc <<= 32;
        ++wi;
    }
    // 512 coordinates at a time: their 16 blocks of nibble words loaded
    // together, then coded block by block; within a block each lane takes its
    // coded coordinates in order (coordinate c of the block at bit 31 - c of
    // m32, its nibble in the 64-bit half c / 16)
    constexpr uint32_t kB = 16;
    const uint32_t nblk = (nw + 3u) / 4u;
    const uint32_t nblk_full = (d / 8u + 3u) / 4u;   // any bucket's, wave-uniform
    int32_t prev = -1;
    for (uint32_t k0 = 0; k0 < nblk_full; k0 += kB) {
        uint4 blk[kB];
#pragma unroll
        for (uint32_t t = 0; t < kB; ++t)
            blk[t] = k0 + t < nblk ? nib_block<Vec>(p, k0 + t, nw) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (uint32_t t = 0; t < kB; ++t) {
            const uint32_t k = k0 + t;
            if (k >= nblk_full)
                continue;   // (wave-uniform)
            const uint32_t w0 = clip_word(blk[t].x, 4u * k, blen);
            const uint32_t w1 = clip_word(blk[t].y, 4u * k + 1u, blen);
            const uint32_t w2 = clip_word(blk[t].z, 4u * k + 2u, blen);
            const uint32_t w3 = clip_word(blk[t].w, 4u * k + 3u, blen);
            const uint64_t half0 = ((uint64_t)w0 << 32) | w1, half1 = ((uint64_t)w2 << 32) | w3;
            uint32_t m32 = (coord_mask8(w0) << 24) | (coord_mask8(w1) << 16) |
                           (coord_mask8(w2) << 8) | coord_mask8(w3);
            while (__any(m32 != 0u)) {
                if (m32) {
                    const uint32_t c = (uint32_t)__builtin_clz(m32);
                    const uint32_t li = 32u * k + c;
                    const uint32_t nibv =
                        (uint32_t)((c < 16u ? half0 : half1) >> (60u - 4u * (c & 15u))) & 15u;
                    const uint32_t cd = codes[(uint32_t)((int32_t)li - prev)];   // in [1, d]
                    const uint32_t cl = codes[nibv & 7u];                         // level 1..7
                    const uint32_t llen = cl >> 24;
                    const uint32_t code =
                        ((((cd & 0xFFFFFFu) << 1) | (nibv >> 3)) << llen) | (cl & 0xFFFFFFu);
                    const uint32_t len = (cd >> 24) + 1u + llen;   // <= 26 bits
                    acc |= (uint64_t)code << (64u - fill - len);
                    fill += len;
                    prev = (int32_t)li;
                    m32 &= ~(0x80000000u >> c);
                    if (fill >= 32u) {
                        emit(wi, (uint32_t)(acc >> 32));
                        acc <<= 32;
                        fill -= 32u;
                        ++wi;
                    }
                }
            }
        }
    }
    if (valid && fill)   // the last, partial word
        emit(wi, (uint32_t)(acc >> 32));
    __builtin_amdgcn_wave_barrier();
    if (staged) {
        // the wavefront's first and last words may be shared with the
        // neighbouring wavefronts' buckets
        const uint64_t nwords = whi - wlo;
        const bool first_shared = (s0 & 31u) != 0u;
        const bool last_shared = (e_last & 31u) != 0u && b0 + last + 1 < nb;
        for (uint64_t k = lane; k < nwords; k += kWave) {
            const uint64_t gw = wlo + k;
            if (gw >= cap)
                continue;
            const uint32_t v = stage[k];
            if ((k == 0 && first_shared) || (k == nwords - 1u && last_shared))
                atomicOr(out + gw, v);
            else
                out[gw] = v;
        }
    }
}

// Decode.  A reader over one bucket's bits: a 64-bit window (next bit in
// bit 63) refilled one word at a time from `src` (the staged copy in LDS, or
// the input).  `left` counts the bucket's bits not yet consumed; it is
// capped at 2^31, more than any bucket can consume before it stops (every
// coordinate advances the index, and the reader fails on any omega group
// of 31 or more digits).
template <typename Src>
struct BitReader {
    Src src;              // the bucket's first word
    uint32_t word;        // next word to load, relative to src
    uint32_t left;
    uint64_t buf;         // window
    uint32_t avail;       // valid bits in the window
    bool ok;

    __device__ void refill()
    {
        while (avail <= 32u && avail < left) {
            buf |= (uint64_t)src[word++] << (32u - avail);
            avail += 32u;
        }
    }
    __device__ void consume(uint32_t nbits)
    {
        buf <<= nbits;
        avail -= nbits;
        left -= nbits;
    }
    __device__ uint32_t get(uint32_t nbits)   // 1..32 bits
    {
        if (!ok || nbits > left) {
            ok = false;
            return 0u;
        }
        refill();
        const uint32_t v = (uint32_t)(buf >> (64u - nbits));
        consume(nbits);
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

// Omega codes read from the top 32 bits x of the window (next bit in bit
// 31) with shifts and selects, no branches.  An omega code is groups, each a
// 1 and k more digits making the next k, ended by a 0; the first group
// starts from k = 1.
//
// omega(dist) with at most 3 groups: its length (<= 23), or 0 when it needs
// more groups.
__device__ __forceinline__ uint32_t dist_peek(uint32_t x, uint32_t &dist)
{
    // continuation bits c0..c3, group values k1 (2 bits), k2 (k1 + 1 bits),
    // k3 (k2 + 1 bits)
    const uint32_t c0 = x >> 31;
    const uint32_t k1 = 2u | ((x >> 30) & 1u);
    const uint32_t c1 = (x >> 29) & 1u;
    const uint32_t k2 = (x << 2) >> (31u - k1);                  // k1 <= 3
    const uint32_t c2 = (x << (3u + k1)) >> 31;
    const uint32_t k3 = (x << (3u + k1)) >> (31u - k2);          // k2 <= 15
    const uint32_t c3 = (x << (4u + k1 + k2)) >> 31;
    dist = !c0 ? 1u : !c1 ? k1 : !c2 ? k2 : k3;
    const uint32_t dlen = !c0 ? 1u : !c1 ? 3u : !c2 ? 4u + k1 : 5u + k1 + k2;
    return !c0 || !c1 || !c2 || !c3 ? dlen : 0u;
}

// The sign bit, then omega(level) with at most 2 groups: their length
// (<= 8), or 0 when the level code needs more groups.
__device__ __forceinline__ uint32_t sign_level_peek(uint32_t x, uint32_t &sign, uint32_t &level)
{
    sign = x >> 31;
    const uint32_t y = x << 1;
    const uint32_t l0 = y >> 31;
    const uint32_t m1 = 2u | ((y >> 30) & 1u);
    const uint32_t l1 = (y >> 29) & 1u;
    const uint32_t m2 = (y << 2) >> (31u - m1);
    const uint32_t l2 = (y << (3u + m1)) >> 31;
    level = !l0 ? 1u : !l1 ? m1 : m2;
    const uint32_t llen = !l0 ? 1u : !l1 ? 3u : 4u + m1;
    return !l0 || !l1 || !l2 ? 1u + llen : 0u;
}

// One coordinate: omega(dist), the sign, omega(level).  Returns the code's
// length (<= 31), or 0 when it needs more groups; the caller checks it
// against the bits the window holds.
__device__ __forceinline__ uint32_t coord_peek(uint32_t x, uint32_t &dist, uint32_t &sign,
                                               uint32_t &level)
{
    const uint32_t dlen = dist_peek(x, dist);
    const uint32_t slen = sign_level_peek(x << (dlen ? dlen : 1u), sign, level);
    return dlen && slen ? dlen + slen : 0u;
}

// Staged input words per wavefront: 31 per lane, so that with the decode
// tables and the nibble chunks (40,064 bytes a workgroup) four workgroups fit
// a compute unit's 160 KiB of LDS.
constexpr uint32_t kDecodeStageWords = 31u * kWave;
static_assert(kDecodeStageWords % kWave == 0, "the staging copy moves whole wavefront rows");

// Decode tables for the common short codes (built per workgroup):
//   distance table, indexed by the window's next 11 bits: (length << 8) |
//   distance when omega(distance) fits those 11 bits (distances up to 31),
//   else 0;
//   sign-and-level table, indexed by the next 7 bits after the distance:
//   ((1 + length) << 4) | nibble when the sign bit and omega(level) fit them
//   with a level up to 7, else 0.
// A coordinate whose codes miss either table goes through coord_peek.
constexpr uint32_t kDistBits = 11, kLevelBits = 7;

__device__ __forceinline__ uint32_t dist_entry(uint32_t i)
{
    uint32_t dist;
    const uint32_t dlen = dist_peek(i << (32u - kDistBits), dist);
    return dlen && dlen <= kDistBits ? (dlen << 8) | dist : 0u;
}

__device__ __forceinline__ uint32_t level_entry(uint32_t j)
{
    uint32_t sign, level;
    const uint32_t slen = sign_level_peek(j << (32u - kLevelBits), sign, level);
    return slen && slen <= kLevelBits && level <= 7u ? (slen << 4) | (sign << 3) | level : 0u;
}

// The nibble words being built, CW per thread, in LDS: word k of thread t
// at lds[k * kBlockThreads + t], so the lanes of a wavefront touch
// consecutive banks.  Each thread owns its words (no barrier needed); a
// coordinate is ORed in with one LDS atomic, no register state to select
// among or carry through the loop.
template <uint32_t CW>
struct LdsChunk {
    uint32_t *own;   // word 0 of this thread
    __device__ void clear() const
    {
#pragma unroll
        for (uint32_t k = 0; k < CW; ++k)
            own[k * kBlockThreads] = 0u;
    }
    __device__ void put(uint32_t k, uint32_t v) const   // word k of the chunk |= v
    {
        __hip_atomic_fetch_or(own + k * kBlockThreads, v, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    // chunk ch of the bucket's nw words, from LDS (or zeros)
    template <bool Zero>
    __device__ void store(uint32_t *__restrict__ nib, uint32_t ch, uint32_t nw) const
    {
        uint32_t c[CW];
#pragma unroll
        for (uint32_t k = 0; k < CW; ++k)
            c[k] = Zero ? 0u : own[k * kBlockThreads];
        if constexpr (CW == 4) {
            if (ch * 4u + 4u <= nw) {
                uint4 v;
                v.x = c[0];
                v.y = c[1];
                v.z = c[2];
                v.w = c[3];
                reinterpret_cast<uint4 *>(nib)[ch] = v;
                return;
            }
        }
#pragma unroll
        for (uint32_t k = 0; k < CW; ++k)
            if (ch * CW + k < nw)
                nib[ch * CW + k] = c[k];
    }
};

template <uint32_t CW, typename Src>
__device__ __forceinline__ void decode_bucket(Src src, uint64_t start, uint64_t end, uint32_t blen,
                                              bool valid, float *norm_out,
                                              uint32_t *__restrict__ nib,
                                              const uint16_t *dist_tab, const uint8_t *level_tab,
                                              LdsChunk<CW> chunk)
{
    const uint64_t span = valid ? end - start : 0u;
    BitReader<Src> r{src, 0u, span < (1ull << 31) ? (uint32_t)span : (1u << 31), 0u, 0u, valid};
    const uint32_t lastw = span ? (uint32_t)(((end - 1u) >> 5) - (start >> 5)) : 0u;
    const uint32_t nw = (blen + 7u) / 8u;                 // 0 for a lane with no bucket
    const uint32_t nch = (nw + CW - 1u) / CW;
    // the first word may begin mid-word: load it and drop the bits before
    // the bucket
    if (span) {
        const uint32_t skip = (uint32_t)(start & 31u);
        r.buf = ((uint64_t)src[r.word++] << 32) << skip;
        r.avail = 32u - skip;
    }
    const float norm = __uint_as_float(r.get(32));
    if (valid)
        *norm_out = norm;
    bool active = r.ok && r.left;
    int32_t prev = -1;
    chunk.clear();
    uint32_t cur = 0;   // index of the chunk being built
    // the word the next refill takes, read an iteration ahead so that its
    // latency overlaps the decode (reread where the slow path moves on)
    uint32_t wv = span ? src[r.word < lastw ? r.word : lastw] : 0u;
    while (__any(active)) {
        const bool need = active && r.avail <= 32u && r.avail < r.left;
        r.buf |= need ? (uint64_t)wv << (32u - r.avail) : 0u;
        r.word += need ? 1u : 0u;
        r.avail += need ? 32u : 0u;
        wv = span ? src[r.word < lastw ? r.word : lastw] : 0u;
        const uint32_t lim = r.avail < r.left ? r.avail : r.left;
        const uint32_t x = (uint32_t)(r.buf >> 32);
        const uint32_t e1 = dist_tab[x >> (32u - kDistBits)];
        const uint32_t e2 = level_tab[(x << (e1 >> 8)) >> (32u - kLevelBits)];
        uint32_t dist = e1 & 0xFFu, sign = (e2 >> 3) & 1u, level = e2 & 7u;
        uint32_t len = e1 && e2 ? (e1 >> 8) + (e2 >> 4) : 0u;
        if (active && !len)   // a code the tables do not hold
            len = coord_peek(x, dist, sign, level);
        const bool fast = len && len <= lim;
        const uint32_t take = active && fast ? len : 0u;
        r.buf <<= take;
        r.avail -= take;
        r.left -= take;
        if (active && !fast) {
            dist = r.omega();
            sign = r.get(1);
            level = r.omega();
            wv = span ? src[r.word < lastw ? r.word : lastw] : 0u;
        }
        // li < blen <= 2048 unless the bucket stops here (dist < 2^31)
        const uint32_t li = (uint32_t)(prev + 1) + (dist - 1u);
        const bool ins = active && r.ok && li < blen && level <= 7u;
        const uint32_t ch = li / (8u * CW);
        if (ins && ch != cur) {   // later chunks only: the chunk before is done
            chunk.template store<false>(nib, cur, nw);
            chunk.clear();
            while (++cur < ch)
                chunk.template store<true>(nib, cur, nw);
        }
        // every lane ORs (0 where nothing is inserted: no branch, and the
        // word is the lane's own)
        chunk.put((li >> 3) % CW, ins ? ((sign << 3) | level) << (28u - 4u * (li & 7u)) : 0u);
        prev = ins ? (int32_t)li : prev;
        active = ins && r.left;
    }
    // the last chunk, then zeros to the bucket's end
    if (nch) {
        chunk.template store<false>(nib, cur, nw);
        while (++cur < nch)
            chunk.template store<true>(nib, cur, nw);
    }
}

// Vec: 16-byte nibble stores (d a multiple of 32, output 16-byte aligned).
template <bool Vec>
__global__ __launch_bounds__(kBlockThreads) void elias_decode_kernel(
    const uint32_t *__restrict__ in, const uint64_t *__restrict__ offs, uint64_t n, uint32_t d,
    uint64_t nb, uint64_t in_words, float *__restrict__ norms, uint32_t *__restrict__ nibbles)
{
    __shared__ uint32_t stage[kBlockWaves][kDecodeStageWords];
    __shared__ uint16_t dist_tab[1u << kDistBits];
    __shared__ uint8_t level_tab[1u << kLevelBits];
    constexpr uint32_t CW = Vec ? 4u : 1u;
    __shared__ uint32_t chunk_lds[CW * kBlockThreads];
    const LdsChunk<CW> chunk{chunk_lds + threadIdx.x};
    const uint32_t lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    for (uint32_t i = threadIdx.x; i < (1u << kDistBits); i += kBlockThreads)
        dist_tab[i] = (uint16_t)dist_entry(i);
    for (uint32_t j = threadIdx.x; j < (1u << kLevelBits); j += kBlockThreads)
        level_tab[j] = (uint8_t)level_entry(j);
    // (the first __syncthreads below orders the tables before any use)
    const uint64_t nlanes_groups = (nb + kWave - 1) / kWave;                  // 64 buckets each
    const uint64_t ngroups = (nlanes_groups + kBlockWaves - 1) / kBlockWaves;  // per workgroup
    const uint64_t limit = in_words * 32u;
    for (uint64_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
        const uint64_t b = (grp * kBlockWaves + wave) * kWave + lane;
        const bool valid = b < nb;
        uint64_t start = 0, end = 0;
        if (valid) {
            start = offs[b];
            end = offs[b + 1];
            end = end < limit ? end : limit;
            start = start < end ? start : end;
        }
        // the wavefront's word range: staged when it fits
        uint64_t wlo = valid && end > start ? start >> 5 : ~0ull;
        uint64_t whi = valid && end > start ? (end + 31u) >> 5 : 0u;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const uint64_t a = __shfl_xor(wlo, off, kWave), c = __shfl_xor(whi, off, kWave);
            wlo = a < wlo ? a : wlo;
            whi = c > whi ? c : whi;
        }
        const bool staged = whi <= wlo || whi - wlo <= kDecodeStageWords;
        if (staged && whi > wlo) {
            // every load issued before the first LDS store
            const uint32_t cnt = (uint32_t)(whi - wlo);
            uint32_t t[kDecodeStageWords / kWave];
#pragma unroll
            for (uint32_t j = 0; j < kDecodeStageWords / kWave; ++j)
                if (lane + j * kWave < cnt)
                    t[j] = in[wlo + lane + j * kWave];
#pragma unroll
            for (uint32_t j = 0; j < kDecodeStageWords / kWave; ++j)
                if (lane + j * kWave < cnt)
                    stage[wave][lane + j * kWave] = t[j];
        }
        __syncthreads();
        {
            // every lane runs the loop (its trip count is the wavefront's);
            // lanes past the last bucket read and store nothing
            const uint64_t lo = valid ? b * d : 0u;
            const uint32_t blen = valid ? (uint32_t)(lo + d < n ? d : n - lo) : 0u;
            // separate calls, so that each reads through its own address space
            // (LDS reads for the staged copy, not generic loads)
            if (staged)
                decode_bucket<CW, const uint32_t *>(
                    stage[wave] + (end > start ? (start >> 5) - wlo : 0u), start, end, blen, valid,
                    norms + b, nibbles + (lo >> 3), dist_tab, level_tab, chunk);
            else
                decode_bucket<CW, const uint32_t *>(in + (start >> 5), start, end, blen, valid,
                                                    norms + b, nibbles + (lo >> 3), dist_tab,
                                                    level_tab, chunk);
        }
        __syncthreads();   // the stage is rewritten by the next group
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
    // 16-byte nibble loads when every bucket starts 16-byte aligned
    const bool vec = d % 32u == 0 && ((uintptr_t)nibbles & 15u) == 0;
    const uint32_t grid = grid_for((nb + kBlockThreads - 1) / kBlockThreads, 0);
    if (nb) {
        if (vec)
            elias_length_kernel<true><<<grid, kBlockThreads, 0, stream>>>(nibbles, n, d, nb, offs);
        else
            elias_length_kernel<false><<<grid, kBlockThreads, 0, stream>>>(nibbles, n, d, nb, offs);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    hipError_t e = launch_exclusive_scan_u64(offs, nb, stream);
    if (e != hipSuccess || !nb)
        return e;
    elias_zero_kernel<<<grid, kBlockThreads, 0, stream>>>(offs, nb, out, cap);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const size_t lds = ((size_t)d + 1u + (size_t)kBlockWaves * kEncodeStageWords) * 4u;
    if (vec)
        elias_write_kernel<true><<<grid, kBlockThreads, lds, stream>>>(norms, nibbles, n, d, nb,
                                                                        offs, out, cap);
    else
        elias_write_kernel<false><<<grid, kBlockThreads, lds, stream>>>(norms, nibbles, n, d, nb,
                                                                         offs, out, cap);
    return hipGetLastError();
}

hipError_t launch_elias_decode(const uint32_t *in, const uint64_t *offs, uint64_t n, uint32_t d,
                               uint64_t in_words, float *norms, uint32_t *nibbles,
                               hipStream_t stream)
{
    const uint64_t nb = (n + d - 1) / d;
    if (!nb)
        return hipSuccess;
    const uint64_t ngroups = ((nb + kWave - 1) / kWave + kBlockWaves - 1) / kBlockWaves;
    if (d % 32u == 0 && ((uintptr_t)nibbles & 15u) == 0)
        elias_decode_kernel<true><<<grid_for(ngroups, 0), kBlockThreads, 0, stream>>>(
            in, offs, n, d, nb, in_words, norms, nibbles);
    else
        elias_decode_kernel<false><<<grid_for(ngroups, 0), kBlockThreads, 0, stream>>>(
            in, offs, n, d, nb, in_words, norms, nibbles);
    return hipGetLastError();
}

}  // namespace gcq
