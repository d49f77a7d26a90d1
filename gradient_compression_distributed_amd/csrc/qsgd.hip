// qsgd.hip -- QSGD bucketed s-level stochastic quantizer and its decode
// ("QSGD: Communication-Efficient SGD via Gradient Quantization and
// Encoding", chapterpal summary: Knowl 1 the Q_s operator, Knowl 2 the
// (norm, sign, level) tuple, Knowl 3 decode, Knowl 8 bucketing) for gfx950.
//
// Per element: 4 B of gradient read, a 4-bit nibble (sign + 3-bit level)
// and a 4/d-byte share of the bucket norm written; decode reads those and
// writes 4 B.  The uniforms come from a counter-based generator, so a
// draw depends only on (seed, element index), never on the launch shape.
#include <math.h>

#include "gcq_device.h"
#include "gcq_internal.h"

namespace gcq {

namespace {

using dev::ld;
using dev::st;
using dev::v4f;

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
                const uint32_t y = dev::dpp<dev::kSwapPairs>(odd ? h[c] : h[c + 1]);
                if (odd)
                    st<NT>(out + 32u * (c + 1) + (lane >> 1), (y << 16) | h[c + 1]);
                else
                    st<NT>(out + 32u * c + (lane >> 1), (h[c] << 16) | y);
            } else {
                const uint32_t y = dev::dpp<dev::kSwapPairs>(h[c]);
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

}  // namespace

hipError_t launch_qsgd_quantize(const float *g, uint64_t n, uint32_t d, uint32_t s, uint64_t seed,
                                float *norms, uint32_t *nibbles, hipStream_t stream)
{
    if (!n)
        return hipSuccess;
    const gcq_tuning tu = tuning();
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
    if (tu.qsgd_nt)                                                                                     \
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
    const gcq_tuning tu = tuning();
    const uint64_t ngroups = (n + 3) >> 2;
    const uint32_t grid = grid_for((ngroups + kBlockThreads - 1) / kBlockThreads, 0);
    const bool pow2 = d >= 4 && (d & (d - 1)) == 0;
    const uint32_t dshift = pow2 ? (uint32_t)__builtin_ctz(d) : 0u;
    if (pow2) {
        if (tu.qsgd_nt)
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
