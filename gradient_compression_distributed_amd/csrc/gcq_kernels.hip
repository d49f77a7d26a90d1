// gcq_kernels.hip -- HIP kernels for gfx950 (CDNA4, wave64) of the
// gradient-compression hot path.
//
// Everything here is HBM-streaming work: no dense contraction, so no MFMA.
// Each kernel reads its inputs once with 16-byte (dwordx4) loads and writes
// each output byte once; cross-lane assembly of packed words uses DPP quad
// permutes instead of LDS round trips.
//
// Arithmetic follows the pages (see include/gcq.h for the passages); all
// float work is IEEE float32 round-to-nearest with denormals kept, and the
// library is compiled with -ffp-contract=off so no a*b+c is fused unless
// written as an explicit fma whose product is exact.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>

#include "gcq_internal.h"

namespace gcq {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// Pointers the compiler cannot trace to a kernel argument (those read from
// the bucket table) would otherwise be accessed with flat instructions;
// qualifying them as global memory keeps global_load/store (vmcnt only).
#define GLOBAL __attribute__((address_space(1)))

template <bool NT, typename P>
__device__ __forceinline__ auto ld(P p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <bool NT, typename P, typename T>
__device__ __forceinline__ void st(P p, T v)
{
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// DPP quad permutes: broadcast lane q of each group of 4 lanes, and swap
// neighbouring lanes.
template <int Ctrl>
__device__ __forceinline__ uint32_t dpp(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, Ctrl, 0xF, 0xF, false);
}
constexpr int kQuadBcast0 = 0x00, kQuadBcast1 = 0x55, kQuadBcast2 = 0xAA, kQuadBcast3 = 0xFF;
constexpr int kSwapPairs = 0xB1;  // quad_perm [1,0,3,2]

// ------------------------------------------------------------------------
// 2-bit threshold quantizer (MXNet PR "Two bit quantization"; CD-SGD 3.4.1)
// ------------------------------------------------------------------------

// 11 at or above +t, 10 at or below -t, 00 otherwise (NaN compares false).
__device__ __forceinline__ uint32_t gc2_code(float v, float t)
{
    const uint32_t up = v >= t ? 1u : 0u;
    const uint32_t dn = v <= -t ? 1u : 0u;
    return ((up | dn) << 1) | up;
}

// What is not sent stays in the residual: 11 sends +t, 10 sends -t.
__device__ __forceinline__ float gc2_residual(float v, uint32_t code, float t)
{
    const float sent = code == 3u ? t : (code == 2u ? -t : 0.0f);
    return v - sent;
}

// Full wave tile, layout 0.  Lane L loads elements 256k + 4L .. +3 of the
// tile for k = 0..3, so every dwordx4 load of the wave covers 1 KiB of
// consecutive memory.  Those four elements are byte (L % 4) of packed word
// 16k + L/4 (byte 0 = most significant).  A quad of lanes therefore holds
// the four bytes of four words; one DPP broadcast per source lane lets lane
// 4m + j assemble word 16j + m, so the wave stores its 64 words as one
// 256-byte block.
template <bool NT>
__device__ __forceinline__ void gc2_tile_coalesced(const GLOBAL float *__restrict__ g,
                                                   GLOBAL float *__restrict__ r,
                                                   GLOBAL uint32_t *__restrict__ out, float t,
                                                   uint32_t lane)
{
    const GLOBAL v4f *g4 = (const GLOBAL v4f *)g;
    GLOBAL v4f *r4 = (GLOBAL v4f *)r;
    v4f gv[4], rv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        gv[k] = ld<NT>(g4 + k * kWave + lane);
        rv[k] = ld<NT>(r4 + k * kWave + lane);
    }
    uint32_t bytes = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const v4f v = gv[k] + rv[k];
        const uint32_t c0 = gc2_code(v.x, t), c1 = gc2_code(v.y, t);
        const uint32_t c2 = gc2_code(v.z, t), c3 = gc2_code(v.w, t);
        v4f rn;
        rn.x = gc2_residual(v.x, c0, t);
        rn.y = gc2_residual(v.y, c1, t);
        rn.z = gc2_residual(v.z, c2, t);
        rn.w = gc2_residual(v.w, c3, t);
        st<NT>(r4 + k * kWave + lane, rn);
        bytes |= ((c0 << 6) | (c1 << 4) | (c2 << 2) | c3) << (8 * k);
    }
    const uint32_t x0 = dpp<kQuadBcast0>(bytes), x1 = dpp<kQuadBcast1>(bytes);
    const uint32_t x2 = dpp<kQuadBcast2>(bytes), x3 = dpp<kQuadBcast3>(bytes);
    const uint32_t j = lane & 3u, sh = 8u * j;
    const uint32_t word = (((x0 >> sh) & 0xFFu) << 24) | (((x1 >> sh) & 0xFFu) << 16) |
                          (((x2 >> sh) & 0xFFu) << 8) | ((x3 >> sh) & 0xFFu);
    st<NT>(out + 16u * j + (lane >> 2), word);
}

// Full wave tile, layout 1: lane L owns elements 16L .. 16L+15 (a 64-byte
// run, four dwordx4 loads 64 bytes apart across lanes) and packs its own
// word with no cross-lane traffic.
template <bool NT>
__device__ __forceinline__ void gc2_tile_runs(const GLOBAL float *__restrict__ g,
                                              GLOBAL float *__restrict__ r,
                                              GLOBAL uint32_t *__restrict__ out, float t,
                                              uint32_t lane)
{
    const GLOBAL v4f *g4 = (const GLOBAL v4f *)g + 4u * lane;
    GLOBAL v4f *r4 = (GLOBAL v4f *)r + 4u * lane;
    v4f gv[4], rv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        gv[k] = ld<NT>(g4 + k);
        rv[k] = ld<NT>(r4 + k);
    }
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const v4f v = gv[k] + rv[k];
        const uint32_t c0 = gc2_code(v.x, t), c1 = gc2_code(v.y, t);
        const uint32_t c2 = gc2_code(v.z, t), c3 = gc2_code(v.w, t);
        v4f rn;
        rn.x = gc2_residual(v.x, c0, t);
        rn.y = gc2_residual(v.y, c1, t);
        rn.z = gc2_residual(v.z, c2, t);
        rn.w = gc2_residual(v.w, c3, t);
        st<NT>(r4 + k, rn);
        word |= ((c0 << 6) | (c1 << 4) | (c2 << 2) | c3) << (24 - 8 * k);
    }
    st<NT>(out + lane, word);
}

// Wave tile that runs past the end of its bucket: lane L packs word
// (e0/16 + L) element by element with bounds checks; pairs past n stay 00.
__device__ __forceinline__ void gc2_tile_partial(const GLOBAL float *__restrict__ g,
                                                 GLOBAL float *__restrict__ r,
                                                 GLOBAL uint32_t *__restrict__ out, uint64_t n,
                                                 uint64_t e0, float t, uint32_t lane)
{
    const uint64_t w = (e0 >> 4) + lane;
    const uint64_t base = w << 4;
    if (base >= n)
        return;
    uint32_t word = 0;
    for (uint32_t p = 0; p < 16; ++p) {
        const uint64_t e = base + p;
        if (e < n) {
            const float v = g[e] + r[e];
            const uint32_t c = gc2_code(v, t);
            r[e] = gc2_residual(v, c, t);
            word |= c << (30u - 2u * p);
        }
    }
    out[w] = word;
}

// One kernel for the single-buffer call (Table = false: the descriptor is a
// kernel argument) and the fused multi-bucket call (Table = true: a device
// table of buckets, each owning a contiguous range of block tiles).  The
// block -> tile map is a grid-stride loop; with a grid of one block per
// tile it runs once.  Tiles of a bucket are contiguous and 16 KiB-aligned
// in memory, so no cache line is shared between workgroups (and thus
// between the XCDs' L2s).
template <int Layout, bool NT, bool Table>
__global__ __launch_bounds__(kBlockThreads) void gc2_quantize_kernel(
    Gc2Desc one, const Gc2Desc *__restrict__ table, uint32_t nbuckets, uint64_t total_tiles)
{
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = threadIdx.x / kWave;
    uint64_t tile = blockIdx.x;
    if (tile >= total_tiles)
        return;
    uint32_t b = 0;
    if constexpr (Table) {
        // last bucket whose first tile is <= tile (empty buckets share their
        // successor's first tile and are skipped)
        uint32_t lo = 0, hi = nbuckets - 1;
        while (lo < hi) {
            const uint32_t mid = (lo + hi + 1) >> 1;
            if (table[mid].tile_begin <= tile)
                lo = mid;
            else
                hi = mid - 1;
        }
        b = lo;
    }
    for (; tile < total_tiles; tile += gridDim.x) {
        Gc2Desc d;
        if constexpr (Table) {
            while (b + 1 < nbuckets && table[b + 1].tile_begin <= tile)
                ++b;
            d = table[b];
        } else {
            d = one;
        }
        const GLOBAL float *g = (const GLOBAL float *)d.g;
        GLOBAL float *r = (GLOBAL float *)d.r;
        GLOBAL uint32_t *out = (GLOBAL uint32_t *)d.out;
        const uint64_t e0 = (tile - d.tile_begin) * kTileElems + (uint64_t)wave * kWaveElems;
        if (e0 + kWaveElems <= d.n) {
            if constexpr (Layout == 0)
                gc2_tile_coalesced<NT>(g + e0, r + e0, out + (e0 >> 4), d.t, lane);
            else
                gc2_tile_runs<NT>(g + e0, r + e0, out + (e0 >> 4), d.t, lane);
        } else if (e0 < d.n) {
            gc2_tile_partial(g, r, out, d.n, e0, d.t, lane);
        }
    }
}

// ------------------------------------------------------------------------
// Dequantize-and-reduce over W packed buffers (MXNet PR "Local kvstore")
// ------------------------------------------------------------------------

// Re-encode the sixteen 2-bit codes of a word as 2-bit two's-complement
// values of what they stand for: 11 (+t) -> 01 (+1), 10 (-t) -> 11 (-1),
// 00 and 01 (read as zero) -> 00.
__device__ __forceinline__ uint32_t gc2_signed_pairs(uint32_t w)
{
    const uint32_t hi = w & 0xAAAAAAAAu;
    const uint32_t lo_at_hi = (w << 1) & 0xAAAAAAAAu;
    return (hi & ~lo_at_hi) | (hi >> 1);
}

// Add worker word `w` (16 codes) into the 16 running sums.  Element k's
// value f_k in {-1, 0, +1} is moved to the top two bits of a byte
// (m_r = (pairs << 2r) & 0xC0C0C0C0 holds elements r, 4+r, 8+r, 12+r in
// bytes 3, 2, 1, 0), so one signed-byte conversion (an SDWA v_cvt) yields
// 64 f_k exactly.  With tq = t/64 (exact: t >= 2^-120), fma(tq, 64 f_k, a)
// rounds t f_k + a once -- the same result as a + (+t | -t | 0) in float32.
// Scaled = false is the same with f_k itself and tq = t (for tiny t).
template <bool Scaled>
__device__ __forceinline__ void dq_accumulate(float (&a)[16], uint32_t w, float tq)
{
    const uint32_t pairs = gc2_signed_pairs(w);
    if constexpr (Scaled) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t m = (pairs << (2 * r)) & 0xC0C0C0C0u;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int k = 4 * (3 - b) + r;
                const float v = (float)(int8_t)(m >> (8 * b));
                a[k] = __builtin_fmaf(tq, v, a[k]);
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const float v = (float)((int32_t)(pairs << (2 * k)) >> 30);
            a[k] = __builtin_fmaf(tq, v, a[k]);
        }
    }
}

constexpr int kDqChunk = 16;  // worker words loaded before they are decoded

// Each thread owns one packed word position (16 elements) per iteration:
// loads of a worker's words are 256 B per wave instruction; workers are
// added strictly in the order 0..W-1.
template <bool Scaled, bool NT>
__global__ __launch_bounds__(kBlockThreads) void dq_reduce_kernel(DqWorkers ws, uint32_t W,
                                                                  uint64_t n, float tq,
                                                                  float *__restrict__ acc)
{
    const uint64_t nwords = (n + 15) >> 4;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t wi = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; wi < nwords;
         wi += stride) {
        float a[16];
#pragma unroll
        for (int k = 0; k < 16; ++k)
            a[k] = 0.0f;
        for (uint32_t w0 = 0; w0 < W; w0 += kDqChunk) {
            uint32_t wd[kDqChunk];
#pragma unroll
            for (int j = 0; j < kDqChunk; ++j)
                wd[j] = (w0 + j < W) ? ld<NT>((const GLOBAL uint32_t *)ws.w[w0 + j] + wi) : 0u;
#pragma unroll
            for (int j = 0; j < kDqChunk; ++j)
                if (w0 + j < W)
                    dq_accumulate<Scaled>(a, wd[j], tq);
        }
        const uint64_t e = wi << 4;
        if (e + 16 <= n) {
            v4f *o = reinterpret_cast<v4f *>(acc + e);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v4f x;
                x.x = a[4 * q];
                x.y = a[4 * q + 1];
                x.z = a[4 * q + 2];
                x.w = a[4 * q + 3];
                st<NT>(o + q, x);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k)
                if (e + k < n)
                    acc[e + k] = a[k];
        }
    }
}

// ------------------------------------------------------------------------
// QSGD (Knowl 1, 2, 8 of the QSGD summary)
// ------------------------------------------------------------------------

// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64-bit products; the high halves are xored with the other counter
// words and the round key, the words permuted; the key advances by the
// Weyl increments between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t a = c[0], b = c[2];
        const uint32_t lo0 = 0xD2511F53u * a, hi0 = __umulhi(0xD2511F53u, a);
        const uint32_t lo1 = 0xCD9E8D57u * b, hi1 = __umulhi(0xCD9E8D57u, b);
        c[0] = hi1 ^ c[1] ^ k0;
        c[1] = lo1;
        c[2] = hi0 ^ c[3] ^ k1;
        c[3] = lo0;
    }
}

// The four uniforms of elements 4q .. 4q+3: top 24 bits of each output
// word, times 2^-24 (exact in float32).
__device__ __forceinline__ void uniforms4(uint64_t q, uint32_t k0, uint32_t k1, float (&u)[4])
{
    uint32_t c[4] = {(uint32_t)q, (uint32_t)(q >> 32), 0u, 0u};
    philox4x32_10(c, k0, k1);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        u[j] = (float)(c[j] >> 8) * 0x1p-24f;
}

// Level of one element (Knowl 1): a = |g|/norm, x = a s, l = floor(x),
// level l+1 with probability x - l; zero norm -> 0; x >= s -> s; NaN -> 0.
__device__ __forceinline__ uint32_t qsgd_level(float gabs, float norm, float sf, uint32_t s,
                                               float u)
{
    const float a = gabs / norm;
    const float x = a * sf;
    const bool below_top = x < sf;           // false for x >= s and for NaN
    const float xs = below_top ? x : 0.0f;   // keeps the conversion in [0, s)
    const float l = floorf(xs);
    const float p = xs - l;
    uint32_t level = (uint32_t)l + (u < p ? 1u : 0u);
    if (!below_top)
        level = x >= sf ? s : 0u;
    if (norm == 0.0f)
        level = 0u;
    return level;
}

__device__ __forceinline__ uint32_t qsgd_nibble(float gv, float norm, float sf, uint32_t s,
                                                float u)
{
    const uint32_t sign = gv < 0.0f ? 8u : 0u;
    return sign | qsgd_level(fabsf(gv), norm, sf, s, u);
}

__device__ __forceinline__ double wave_sum(double x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x += __shfl_xor(x, off, kWave);
    return x;
}

// Fused norm + levels + nibbles for buckets of D = 256*C elements held in
// registers: one wavefront per bucket, lane L holds elements 256c + 4L .. +3
// (dwordx4 loads, 1 KiB per wave instruction).  The sum of squares is
// accumulated in float64 (each square exact), reduced across the wave by
// butterfly shuffles, square-rooted in float64 and rounded once to float32.
// Nibble words: lane pairs (2m, 2m+1) hold the two halves of word 32c + m
// of chunk c; one DPP neighbour swap per two chunks lets even lanes store
// chunk c's words and odd lanes chunk c+1's.
template <int C, bool NT>
__global__ __launch_bounds__(kBlockThreads) void qsgd_fused_kernel(
    const float *__restrict__ g, uint32_t s, uint32_t k0, uint32_t k1, float *__restrict__ norms,
    uint32_t *__restrict__ nib, uint64_t nb_full)
{
    constexpr uint64_t D = 256u * C;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const float sf = (float)s;
    const uint64_t wstride = (uint64_t)gridDim.x * kBlockWaves;
    for (uint64_t b = (uint64_t)blockIdx.x * kBlockWaves + threadIdx.x / kWave; b < nb_full;
         b += wstride) {
        const uint64_t base = b * D;
        v4f v[C];
#pragma unroll
        for (int c = 0; c < C; ++c)
            v[c] = ld<NT>(reinterpret_cast<const v4f *>(g + base + 256u * c) + lane);
        double ss = 0.0;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            ss = __builtin_fma((double)v[c].x, (double)v[c].x, ss);
            ss = __builtin_fma((double)v[c].y, (double)v[c].y, ss);
            ss = __builtin_fma((double)v[c].z, (double)v[c].z, ss);
            ss = __builtin_fma((double)v[c].w, (double)v[c].w, ss);
        }
        ss = wave_sum(ss);
        const float norm = (float)__builtin_sqrt(ss);
        if (lane == 0)
            norms[b] = norm;
        uint32_t h[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            float u[4];
            uniforms4((base + 256u * c + 4u * lane) >> 2, k0, k1, u);
            h[c] = (qsgd_nibble(v[c].x, norm, sf, s, u[0]) << 12) |
                   (qsgd_nibble(v[c].y, norm, sf, s, u[1]) << 8) |
                   (qsgd_nibble(v[c].z, norm, sf, s, u[2]) << 4) |
                   qsgd_nibble(v[c].w, norm, sf, s, u[3]);
        }
        uint32_t *out = nib + (base >> 3);
        const bool odd = (lane & 1u) != 0;
#pragma unroll
        for (int c = 0; c < C; c += 2) {
            if (c + 1 < C) {
                const uint32_t y = dpp<kSwapPairs>(odd ? h[c] : h[c + 1]);
                if (odd)
                    st<NT>(out + 32u * (c + 1) + (lane >> 1), (y << 16) | h[c + 1]);
                else
                    st<NT>(out + 32u * c + (lane >> 1), (h[c] << 16) | y);
            } else {
                const uint32_t y = dpp<kSwapPairs>(h[c]);
                if (!odd)
                    st<NT>(out + 32u * c + (lane >> 1), (h[c] << 16) | y);
            }
        }
    }
}

// Generic norms, any d: one thread per bucket (d <= 32, the bucket summed
// in index order) or one wavefront per bucket (lanes stride the bucket).
__global__ __launch_bounds__(kBlockThreads) void qsgd_norms_thread_kernel(
    const float *__restrict__ g, uint64_t n, uint32_t d, uint64_t b0, uint64_t nb,
    float *__restrict__ norms)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t b = b0 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += stride) {
        const uint64_t lo = b * d;
        const uint64_t hi = lo + d < n ? lo + d : n;
        double ss = 0.0;
        for (uint64_t e = lo; e < hi; ++e)
            ss = __builtin_fma((double)g[e], (double)g[e], ss);
        norms[b] = (float)__builtin_sqrt(ss);
    }
}

__global__ __launch_bounds__(kBlockThreads) void qsgd_norms_wave_kernel(
    const float *__restrict__ g, uint64_t n, uint32_t d, uint64_t b0, uint64_t nb,
    float *__restrict__ norms)
{
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint64_t wstride = (uint64_t)gridDim.x * kBlockWaves;
    for (uint64_t b = b0 + (uint64_t)blockIdx.x * kBlockWaves + threadIdx.x / kWave; b < nb;
         b += wstride) {
        const uint64_t lo = b * d;
        const uint64_t hi = lo + d < n ? lo + d : n;
        double ss = 0.0;
        for (uint64_t e = lo + lane; e < hi; e += kWave)
            ss = __builtin_fma((double)g[e], (double)g[e], ss);
        ss = wave_sum(ss);
        if (lane == 0)
            norms[b] = (float)__builtin_sqrt(ss);
    }
}

// Generic levels, any d: one thread per nibble word (8 elements, two
// Philox calls), each element reading its bucket's norm.
__global__ __launch_bounds__(kBlockThreads) void qsgd_levels_generic_kernel(
    const float *__restrict__ g, uint64_t n, uint32_t d, uint32_t s, uint32_t k0, uint32_t k1,
    const float *__restrict__ norms, uint32_t *__restrict__ nib, uint64_t w0, uint64_t nwords)
{
    const float sf = (float)s;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t w = w0 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwords;
         w += stride) {
        uint32_t word = 0;
        for (uint32_t half = 0; half < 2; ++half) {
            const uint64_t eb = (w << 3) + 4u * half;
            if (eb >= n)
                break;
            float u[4];
            uniforms4(eb >> 2, k0, k1, u);
            for (uint32_t q = 0; q < 4; ++q) {
                const uint64_t e = eb + q;
                if (e < n) {
                    const uint32_t nbl = qsgd_nibble(g[e], norms[e / d], sf, s, u[q]);
                    word |= nbl << (28u - 4u * (4u * half + q));
                }
            }
        }
        nib[w] = word;
    }
}

// Decode (Knowl 3): out = +-((norm * level) / s).  One thread per group of 4
// elements (a 16-byte store); lanes 2m and 2m+1 read the two halves of one
// nibble word.  Pow2: d is a power of two >= 4, so the group shares one
// bucket and the bucket index is a shift.
template <bool Pow2, bool NT>
__global__ __launch_bounds__(kBlockThreads) void qsgd_dequant_kernel(
    const float *__restrict__ norms, const uint32_t *__restrict__ nib, uint64_t n, uint32_t d,
    uint32_t dshift, uint32_t s, float *__restrict__ out)
{
    const float sf = (float)s;
    const uint64_t ngroups = (n + 3) >> 2;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t gi = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < ngroups;
         gi += stride) {
        const uint64_t e = gi << 2;
        const uint32_t word = ld<NT>(nib + (e >> 3));
        const uint32_t h = (gi & 1u) ? (word & 0xFFFFu) : (word >> 16);
        float o[4];
        if constexpr (Pow2) {
            const float norm = norms[e >> dshift];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t nb = (h >> (12 - 4 * q)) & 0xFu;
                const float m = (norm * (float)(nb & 7u)) / sf;
                o[q] = (nb & 8u) ? -m : m;
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint64_t ei = e + q < n ? e + q : e;
                const uint32_t nb = (h >> (12 - 4 * q)) & 0xFu;
                const float m = (norms[ei / d] * (float)(nb & 7u)) / sf;
                o[q] = (nb & 8u) ? -m : m;
            }
        }
        if (e + 4 <= n) {
            v4f x;
            x.x = o[0];
            x.y = o[1];
            x.z = o[2];
            x.w = o[3];
            st<NT>(reinterpret_cast<v4f *>(out + e), x);
        } else {
            for (int q = 0; q < 4; ++q)
                if (e + q < n)
                    out[e + q] = o[q];
        }
    }
}

int env_int(const char *name, int dflt)
{
    const char *v = getenv(name);
    return (v && *v) ? atoi(v) : dflt;
}

uint32_t grid_for(uint64_t work_blocks, int blocks_per_cu)
{
    uint64_t g = work_blocks;
    if (blocks_per_cu > 0) {
        const uint64_t cap = (uint64_t)device_cus() * (uint64_t)blocks_per_cu;
        g = g < cap ? g : cap;
    }
    if (g < 1)
        g = 1;
    if (g > 0x7FFFFFFFu)
        g = 0x7FFFFFFFu;
    return (uint32_t)g;
}

}  // namespace

namespace {
std::mutex g_tuning_mu;
bool g_tuning_init = false;
Tuning g_tuning;
}  // namespace

Tuning tuning()
{
    std::lock_guard<std::mutex> lock(g_tuning_mu);
    if (!g_tuning_init) {
        g_tuning.gc2_layout = env_int("GCQ_GC2_LAYOUT", 0) ? 1 : 0;
        g_tuning.nt = env_int("GCQ_NT", 1) ? 1 : 0;
        g_tuning.blocks_per_cu = std::max(0, std::min(1024, env_int("GCQ_BLOCKS_PER_CU", 0)));
        g_tuning.dq_blocks_per_cu =
            std::max(0, std::min(1024, env_int("GCQ_DQ_BLOCKS_PER_CU", 0)));
        g_tuning_init = true;
    }
    return g_tuning;
}

void set_tuning(const Tuning &t)
{
    (void)tuning();
    std::lock_guard<std::mutex> lock(g_tuning_mu);
    g_tuning = t;
}

int device_cus()
{
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (!cache[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

template <bool Table>
static hipError_t launch_gc2(const Gc2Desc &one, const Gc2Desc *table, uint32_t nb,
                             uint64_t total_tiles, hipStream_t stream)
{
    const Tuning tu = tuning();
    const uint32_t grid = grid_for(total_tiles, tu.blocks_per_cu);
    const dim3 block(kBlockThreads);
    if (tu.gc2_layout == 0) {
        if (tu.nt)
            gc2_quantize_kernel<0, true, Table><<<grid, block, 0, stream>>>(one, table, nb, total_tiles);
        else
            gc2_quantize_kernel<0, false, Table><<<grid, block, 0, stream>>>(one, table, nb, total_tiles);
    } else {
        if (tu.nt)
            gc2_quantize_kernel<1, true, Table><<<grid, block, 0, stream>>>(one, table, nb, total_tiles);
        else
            gc2_quantize_kernel<1, false, Table><<<grid, block, 0, stream>>>(one, table, nb, total_tiles);
    }
    return hipGetLastError();
}

hipError_t launch_gc2_single(const Gc2Desc &one, hipStream_t stream)
{
    const uint64_t tiles = (one.n + kTileElems - 1) / kTileElems;
    if (!tiles)
        return hipSuccess;
    return launch_gc2<false>(one, nullptr, 1, tiles, stream);
}

hipError_t launch_gc2_table(const Gc2Desc *dev_table, uint32_t nbuckets, uint64_t total_tiles,
                            hipStream_t stream)
{
    if (!total_tiles || !nbuckets)
        return hipSuccess;
    Gc2Desc none = {};
    return launch_gc2<true>(none, dev_table, nbuckets, total_tiles, stream);
}

hipError_t launch_dequant_reduce(const DqWorkers &w, uint32_t W, uint64_t n, float t, float *acc,
                                 hipStream_t stream)
{
    const uint64_t nwords = (n + 15) >> 4;
    if (!nwords)
        return hipSuccess;
    const Tuning tu = tuning();
    const uint32_t grid = grid_for((nwords + kBlockThreads - 1) / kBlockThreads,
                                   tu.dq_blocks_per_cu);
    // t/64 is exact (a power-of-two scaling that stays normal) for t >= 2^-120.
    const bool scaled = t >= 0x1p-120f;
    const float tq = scaled ? t * 0x1p-6f : t;
    if (scaled) {
        if (tu.nt)
            dq_reduce_kernel<true, true><<<grid, kBlockThreads, 0, stream>>>(w, W, n, tq, acc);
        else
            dq_reduce_kernel<true, false><<<grid, kBlockThreads, 0, stream>>>(w, W, n, tq, acc);
    } else {
        dq_reduce_kernel<false, false><<<grid, kBlockThreads, 0, stream>>>(w, W, n, tq, acc);
    }
    return hipGetLastError();
}

hipError_t launch_qsgd_quantize(const float *g, uint64_t n, uint32_t d, uint32_t s, uint64_t seed,
                                float *norms, uint32_t *nibbles, hipStream_t stream)
{
    if (!n)
        return hipSuccess;
    const Tuning tu = tuning();
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const uint64_t nb = (n + d - 1) / d;
    const uint64_t nwords = (n + 7) >> 3;
    uint64_t nb_done = 0;  // buckets (and their words) finished by the fused kernel
    const uint32_t C = d % 256u == 0 ? d / 256u : 0u;
    if (C == 1 || C == 2 || C == 4 || C == 8) {
        nb_done = n / d;
        if (nb_done) {
            const uint32_t grid = grid_for((nb_done + kBlockWaves - 1) / kBlockWaves, 0);
#define GCQ_FUSED(CC)                                                                              \
    if (tu.nt)                                                                                     \
        qsgd_fused_kernel<CC, true><<<grid, kBlockThreads, 0, stream>>>(g, s, k0, k1, norms,     \
                                                                         nibbles, nb_done);      \
    else                                                                                           \
        qsgd_fused_kernel<CC, false><<<grid, kBlockThreads, 0, stream>>>(g, s, k0, k1, norms,    \
                                                                          nibbles, nb_done);
            switch (C) {
            case 1: GCQ_FUSED(1) break;
            case 2: GCQ_FUSED(2) break;
            case 4: GCQ_FUSED(4) break;
            default: GCQ_FUSED(8) break;
            }
#undef GCQ_FUSED
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
    }
    if (nb_done < nb) {
        const uint64_t left = nb - nb_done;
        if (d <= 32) {
            const uint32_t grid = grid_for((left + kBlockThreads - 1) / kBlockThreads, 0);
            qsgd_norms_thread_kernel<<<grid, kBlockThreads, 0, stream>>>(g, n, d, nb_done, nb,
                                                                         norms);
        } else {
            const uint32_t grid = grid_for((left + kBlockWaves - 1) / kBlockWaves, 0);
            qsgd_norms_wave_kernel<<<grid, kBlockThreads, 0, stream>>>(g, n, d, nb_done, nb,
                                                                       norms);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        // the fused kernel ends on a word boundary (d is a multiple of 8 there)
        const uint64_t w0 = (nb_done * d) >> 3;
        const uint32_t grid = grid_for((nwords - w0 + kBlockThreads - 1) / kBlockThreads, 0);
        qsgd_levels_generic_kernel<<<grid, kBlockThreads, 0, stream>>>(g, n, d, s, k0, k1, norms,
                                                                       nibbles, w0, nwords);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_qsgd_dequant(const float *norms, const uint32_t *nibbles, uint64_t n, uint32_t d,
                               uint32_t s, float *out, hipStream_t stream)
{
    if (!n)
        return hipSuccess;
    const Tuning tu = tuning();
    const uint64_t ngroups = (n + 3) >> 2;
    const uint32_t grid = grid_for((ngroups + kBlockThreads - 1) / kBlockThreads, 0);
    const bool pow2 = d >= 4 && (d & (d - 1)) == 0;
    const uint32_t dshift = pow2 ? (uint32_t)__builtin_ctz(d) : 0u;
    if (pow2) {
        if (tu.nt)
            qsgd_dequant_kernel<true, true><<<grid, kBlockThreads, 0, stream>>>(norms, nibbles, n, d,
                                                                                dshift, s, out);
        else
            qsgd_dequant_kernel<true, false><<<grid, kBlockThreads, 0, stream>>>(
                norms, nibbles, n, d, dshift, s, out);
    } else {
        qsgd_dequant_kernel<false, false><<<grid, kBlockThreads, 0, stream>>>(norms, nibbles, n, d,
                                                                              dshift, s, out);
    }
    return hipGetLastError();
}

}  // namespace gcq
