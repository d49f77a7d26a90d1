// qsgd.hip -- QSGD bucketed s-level stochastic quantizer and its decode
// ("QSGD: Communication-Efficient SGD via Gradient Quantization and
// Encoding", chapterpal summary: Knowl 1 the Q_s operator, Knowl 2 the
// (norm, sign, level) tuple, Knowl 3 decode and the K-worker average,
// Knowl 8 bucketing and max-norm scaling) for gfx950.
//
// Per element: 4 B of gradient read, a 4-bit nibble (sign + 3-bit level)
// and a 4/d-byte share of the bucket norm written; decode reads those and
// writes 4 B.  The uniforms come from a counter-based generator, so a
// draw depends only on (seed, element index), never on the launch shape.
#include <math.h>

#include <type_traits>

#include "gcq_device.h"
#include "gcq_internal.h"

namespace gcq {

namespace {

using dev::ld;
using dev::st;
using dev::v4f;

using dev::philox4x32_10;

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

// The four raw output words behind those uniforms (u = (c >> 8) 2^-24).
__device__ __forceinline__ void philox_words4(uint64_t q, uint32_t k0, uint32_t k1,
                                              uint32_t (&c)[4])
{
    c[0] = (uint32_t)q;
    c[1] = (uint32_t)(q >> 32);
    c[2] = 0u;
    c[3] = 0u;
    philox4x32_10(c, k0, k1);
}

// Level of one element (Knowl 1), exactly as defined: a = |g|/norm (one
// correctly rounded division), x = a s, l = floor(x), level l+1 when
// u < x - l; zero norm -> 0; x >= s -> s; NaN -> 0.
__device__ __forceinline__ uint32_t qsgd_level_exact(float gabs, float norm, float sf, uint32_t s,
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

// The same level without a division per element.  With l = floor(x) and
// p = x - l, the level l + [u < p] equals ceil(x - u) in exact arithmetic
// (u in [0, 1); the integer case x - u = l is p = u, level l).  With
// T = x + 1 - u > 0 that is trunc(T) whenever T is not an integer.  The
// clamp needs no case of its own: |g| <= norm for the L2 norm (the float64
// sum of exact squares only rounds towards values >= g^2, and bucket_norm's
// square root is within 2^-40 of exact before its rounding to float, which
// cannot fall below the float |g|) and for the largest magnitude, so
// a = RN(|g|/norm) <= 1 and x <= s; x = s gives T in (s, s + 1], whose trunc
// is s unless T = s + 1 (u = 0), an integer.
//
// The kernel computes d = RN(t - U' 2^-32) with t = RN(|g| rs + 1 + kGuard)
// (one fma), rs = RN(r s) for r the reciprocal of the norm from
// recip_refined (within one ulp of 1/norm, in fact within one rounding and
// 2^-45), and U' = RN(c) the raw 32-bit Philox word converted to float (no
// shift).  For a bucket norm in [2^-120, 2^120]:
//   |g| rs is within 5 relative half-ulps of x (two roundings in x, the
//     ulp of r and the rounding of rs, on a value below 7.0001):
//     35.1 * 2^-24;
//   t rounds |g| rs + 1 + kGuard < 9 once: at most 2^-21 = 8 * 2^-24;
//   U' 2^-32 is within 2^-24 (the 8 dropped bits) + 2^-25 (the conversion)
//     of u = (c >> 8) 2^-24: 1.5 * 2^-24;
//   the fma rounds t - U' 2^-32 < 9 once: 8 * 2^-24;
// so |d - (T + kGuard)| < 53 * 2^-24 < kGuard = 2^-18.  When fract(d) >= 2
// kGuard, T lies strictly between trunc(d) and trunc(d) + 1: trunc(d) =
// trunc(T), the exact level (T <= s + 1 then keeps it at most s, within its
// 3 bits).  The shortcut only runs for finite buckets (a NaN or Inf element
// makes the norm NaN or Inf, outside the range), so d is finite and d > 0.
constexpr float kGuard = 0x1p-18f;
// fract(d) is exact for d in [0, 9); one comparison per element group.
constexpr float kSafeFrac = 2.0f * kGuard;

// Level from the shortcut; `frac` = fract(d), safe when >= kSafeFrac (an
// unsafe lane's return value is not used).
__device__ __forceinline__ uint32_t qsgd_level_fast(float gabs, float rs, uint32_t c, float &frac)
{
    const float t = __builtin_fmaf(gabs, rs, 1.0f + kGuard);
    const float d = __builtin_fmaf((float)c, -0x1p-32f, t);
    frac = __builtin_amdgcn_fractf(d);
    return (uint32_t)d;                      // d in (0, s + 2): in range
}

// 1/x for x in [2^-120, 2^120]: the hardware reciprocal (documented within
// one ulp) and one Newton step, r (2 - x r), rounded once: the unrounded
// step is within e^2 (plus 2^-47 from rounding 1 - x r) of 1/x for an
// estimate within e, so the result is within one rounding and 2^-45 of 1/x.
__device__ __forceinline__ float recip_refined(float x)
{
    const float r0 = __builtin_amdgcn_rcpf(x);
    const float e = __builtin_fmaf(-x, r0, 1.0f);
    return __builtin_fmaf(e, r0, r0);
}

// A bucket's L2 norm from its float64 sum of squares ss (every partial sum
// of exact squares of floats, so 0 or in [2^-298, 2^266]): RN32(sqrt(ss)).
// The hardware reciprocal square root y (an estimate within b of 1/sqrt(ss))
// and h = ss y, then two corrections h += (ss - h^2) y / 2, each of which
// takes a relative error a to about -(a b + a^2 / 2): from b to within 1.5
// b^3 + 2^-52, below 2^-40 for any b <= 2^-13.  The float rounding then
// equals the correctly rounded one except within 2^-40 of a halfway point,
// and never undershoots the float |g| of any element.  ss = 0, Inf or NaN
// gives ss itself.
__device__ __forceinline__ float bucket_norm(double ss)
{
    const double y = __builtin_amdgcn_rsq(ss);
    const double hy = 0.5 * y;
    double h = ss * y;
    h = __builtin_fma(__builtin_fma(-h, h, ss), hy, h);
    h = __builtin_fma(__builtin_fma(-h, h, ss), hy, h);
    return ss > 0.0 && ss < __builtin_inf() ? (float)h : (float)ss;
}

__device__ __forceinline__ uint32_t sign_bit(float gv) { return gv < 0.0f ? 8u : 0u; }

// Float4 q (0..3) of lane L of a full 1024-output wave tile at `tile`
// (wave-uniform), elements 256q + 4L .. +3.  NT: a buffer store with the nt
// and sc1 cache-policy bits (the lane-table decode at 2^30, d = 512: 0.74 ms
// against 0.77 ms with nt alone, in one process); else a plain store.
template <bool NT>
__device__ __forceinline__ void st_tile_f4(float *tile, int q, uint32_t lane, v4f x)
{
    if constexpr (NT) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)tile, 0, (int)(kWaveElems * 4), dev::kBufferRsrcWord3);
        __builtin_amdgcn_raw_buffer_store_b128(x, rs, (int)((256u * q + 4u * lane) * 4u), 0,
                                               dev::kCpolNt | dev::kCpolSc1);
    } else {
        *reinterpret_cast<v4f *>(tile + 256u * q + 4u * lane) = x;
    }
}

// 16 bits of nibbles for four elements, first element in the top nibble:
// nibble = sign << 3 | level, sign = [g < 0].  pack4_exact tests g < 0 per
// element.  pack4 takes the sign bits from the bit patterns of g + 0.0
// (which turns -0.0 into +0.0, so the sign bit is set exactly when g < 0,
// NaNs aside: callers route NaNs to pack4_exact): the top bytes of g0 and
// g2 go to bytes 1 and 0 of one word, those of g1 and g3 to another, which
// is then shifted down by a nibble.
__device__ __forceinline__ uint32_t pack4_exact(const float (&gq)[4], const uint32_t (&lv)[4])
{
    uint32_t h = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        h |= (sign_bit(gq[q]) | lv[q]) << (12 - 4 * q);
    return h;
}

__device__ __forceinline__ uint32_t pack4(const float (&gq)[4], const uint32_t (&lv)[4])
{
    const uint32_t a = __builtin_amdgcn_perm(__float_as_uint(gq[0] + 0.0f),
                                             __float_as_uint(gq[2] + 0.0f), 0x0C0C0703u);
    const uint32_t b = __builtin_amdgcn_perm(__float_as_uint(gq[1] + 0.0f),
                                             __float_as_uint(gq[3] + 0.0f), 0x0C0C0703u);
    uint32_t h = (((((lv[0] << 4) | lv[1]) << 4) | lv[2]) << 4) | lv[3];
    h |= a & 0x8080u;
    h |= (b >> 4) & 0x0808u;
    return h;
}

// A bucket takes the division-free level path when its norm is in this
// range (false for 0, Inf and NaN norms, which take the exact path).
__device__ __forceinline__ bool rcp_norm_ok(float norm)
{
    return norm >= 0x1p-120f && norm <= 0x1p120f;
}

__device__ __forceinline__ float uniform_f(float x)
{
    return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(x)));
}

// Max-norm scaling (QSGD summary, Knowl 8): the running maximum of |g| that
// a NaN never enters (compare, then select), and its wave reduction (the
// maximum is exact, so the order does not matter).
__device__ __forceinline__ float max_in(float m, float a) { return a > m ? a : m; }

// Sum, maximum and "any" over the G lanes of an aligned lane group (G a
// power of two dividing the wavefront): butterflies that stay in the group.
template <uint32_t G>
__device__ __forceinline__ double group_sum(double x)
{
#pragma unroll
    for (uint32_t off = G / 2; off > 0; off >>= 1)
        x += __shfl_xor(x, off, kWave);
    return x;
}

template <uint32_t G>
__device__ __forceinline__ float group_max(float x)
{
#pragma unroll
    for (uint32_t off = G / 2; off > 0; off >>= 1) {
        const float y = __shfl_xor(x, off, kWave);
        x = max_in(x, y);
    }
    return x;
}

template <uint32_t G>
__device__ __forceinline__ bool group_any(bool p, uint32_t grp)
{
    const uint64_t m = __ballot(p);
    if constexpr (G == kWave)
        return m != 0;
    else
        return ((m >> (grp * G)) & ((1ull << G) - 1u)) != 0;
}

// The last bucket when it is shorter than the fused kernel's D (elements
// e0 .. n - 1, e0 a multiple of 8), after the fused kernel: one wavefront,
// norm and nibbles in one launch, with the arithmetic of the generic kernels
// below (lanes stride the bucket for the float64 sum of squares or the
// largest magnitude; lanes stride its nibble words, each element taking the
// level as defined).
template <bool Max>
__global__ __launch_bounds__(kWave) void qsgd_tail_kernel(const float *__restrict__ g, uint64_t n,
                                                           uint64_t e0, uint64_t b, uint32_t s,
                                                           uint32_t k0, uint32_t k1,
                                                           float *__restrict__ norms,
                                                           uint32_t *__restrict__ nib)
{
    const uint32_t lane = threadIdx.x;
    float norm;
    if constexpr (Max) {
        float m = 0.0f;
        for (uint64_t e = e0 + lane; e < n; e += kWave)
            m = max_in(m, fabsf(g[e]));
        norm = group_max<kWave>(m);
    } else {
        double ss = 0.0;
        for (uint64_t e = e0 + lane; e < n; e += kWave)
            ss = __builtin_fma((double)g[e], (double)g[e], ss);
        ss = group_sum<kWave>(ss);
        norm = bucket_norm(ss);
    }
    if (lane == 0)
        norms[b] = norm;
    const float sf = (float)s;
    const uint64_t w1 = (n + 7) >> 3;
    for (uint64_t w = (e0 >> 3) + lane; w < w1; w += kWave) {
        uint32_t word = 0;
#pragma unroll
        for (uint32_t half = 0; half < 2; ++half) {
            const uint64_t eb = (w << 3) + 4u * half;
            float u[4];
            uniforms4(eb >> 2, k0, k1, u);
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q) {
                const uint64_t e = eb + q;
                if (e < n)
                    word |= (sign_bit(g[e]) | qsgd_level_exact(fabsf(g[e]), norm, sf, s, u[q]))
                            << (28u - 4u * (4u * half + q));
            }
        }
        nib[w] = word;
    }
}

// Fused norm + levels + nibbles for buckets of D = 256*C elements held in
// registers.  A wavefront owns H consecutive buckets at a time, one per
// aligned group of G = 64/H lanes; lane l of a group holds elements
// 4G r + 4l .. +3 of its bucket for r = 0 .. R-1, R = C H (dwordx4 loads,
// 16 G contiguous bytes per group and instruction).  The sum of squares is
// accumulated in float64 (each square exact), reduced across the group by
// butterfly shuffles, square-rooted in float64 and rounded once to float32.
// Everything a bucket costs beyond its elements (the reduction, the square
// root, the reciprocal) is one instruction sequence for the H buckets
// together, so H > 1 spreads it over more elements per lane.  Nibble words:
// lane pairs (2m, 2m+1) of a group hold the two halves of word (G/2) r + m
// of the bucket; one DPP neighbour swap per two chunks lets even lanes store
// chunk r's words and odd lanes chunk r+1's.  In the last round a group past
// the final bucket redoes that bucket and stores nothing.
//
// Max = true scales each bucket by its largest magnitude instead (Knowl 8).
// A NaN does not enter that scale, so a bucket holding one takes the exact
// level path (the division-free shortcut assumes finite inputs).
template <int C, int H, bool NT, bool Rcp, bool Max>
__global__ __launch_bounds__(kBlockThreads, C * H > 4 ? 4 : 7) void qsgd_fused_kernel(
    const float *__restrict__ g, uint32_t s, uint32_t k0, uint32_t k1, float *__restrict__ norms,
    uint32_t *__restrict__ nib, uint64_t nb_full)
{
    constexpr uint64_t D = 256u * C;
    constexpr uint32_t G = kWave / H;   // lanes per bucket
    constexpr int R = C * H;            // float4 chunks per lane
    constexpr uint32_t CH = 4u * G;     // elements per chunk
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t grp = lane / G, l = lane % G;
    const float sf = (float)s;
    const uint64_t ngroups = (nb_full + H - 1) / H;
    const uint64_t wstride = (uint64_t)gridDim.x * kBlockWaves;
    for (uint64_t bw = (uint64_t)blockIdx.x * kBlockWaves + threadIdx.x / kWave; bw < ngroups;
         bw += wstride) {
        const uint64_t braw = bw * H + grp;
        const bool own = braw < nb_full;
        const uint64_t b = own ? braw : nb_full - 1;
        const uint64_t base = b * D;
        v4f v[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            v[r] = ld<NT>(reinterpret_cast<const v4f *>(g + base + CH * r) + l);
        float norm;
        bool finite_bucket = true;
        if constexpr (Max) {
            float m = 0.0f;
            bool nan = false;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                m = max_in(m, fabsf(v[r].x));
                m = max_in(m, fabsf(v[r].y));
                m = max_in(m, fabsf(v[r].z));
                m = max_in(m, fabsf(v[r].w));
                nan = nan | (v[r].x != v[r].x) | (v[r].y != v[r].y) | (v[r].z != v[r].z) |
                      (v[r].w != v[r].w);
            }
            norm = group_max<G>(m);
            finite_bucket = !group_any<G>(nan, grp);
        } else {
            double ss = 0.0;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                ss = __builtin_fma((double)v[r].x, (double)v[r].x, ss);
                ss = __builtin_fma((double)v[r].y, (double)v[r].y, ss);
                ss = __builtin_fma((double)v[r].z, (double)v[r].z, ss);
                ss = __builtin_fma((double)v[r].w, (double)v[r].w, ss);
            }
            ss = group_sum<G>(ss);
            norm = bucket_norm(ss);
        }
        if constexpr (H == 1)
            norm = uniform_f(norm);   // wave-uniform: scalar registers from here on
        if (own && l == 0)
            norms[b] = norm;
        const bool fast = Rcp && rcp_norm_ok(norm) && finite_bucket;
        const float rs = fast ? recip_refined(norm) * sf : 0.0f;
        uint32_t h[R];
        // The chunk loop in two copies: AllFast when every bucket the
        // wavefront holds takes the division-free path (the common case),
        // where the choice between the two nibble packings is known at
        // compile time; otherwise each lane follows its own bucket and both
        // packings are formed and selected.
        auto chunks = [&](auto all_fast) {
            constexpr bool AllFast = decltype(all_fast)::value;
            const bool f = AllFast || fast;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float gq[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
                uint32_t cw[4];
                philox_words4((base + CH * r + 4u * l) >> 2, k0, k1, cw);
                uint32_t lv[4];
                bool all_ok = false;
                if (f) {
                    float fr[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        lv[e] = qsgd_level_fast(fabsf(gq[e]), rs, cw[e], fr[e]);
                    all_ok = fminf(fminf(fr[0], fr[1]), fminf(fr[2], fr[3])) >= kSafeFrac;
                }
                if (!all_ok) {
                    // rare: the exact level where the shortcut cannot decide
                    // (its test redone here, so the fast path keeps nothing)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float fe = 0.0f;
                        if (f)
                            (void)qsgd_level_fast(fabsf(gq[e]), rs, cw[e], fe);
                        if (!(fe >= kSafeFrac))
                            lv[e] = qsgd_level_exact(fabsf(gq[e]), norm, sf, s,
                                                     (float)(cw[e] >> 8) * 0x1p-24f);
                    }
                }
                // a fast bucket holds no NaN, so its signs may come from the bits
                if constexpr (AllFast)
                    h[r] = pack4(gq, lv);
                else
                    h[r] = f ? pack4(gq, lv) : pack4_exact(gq, lv);
            }
        };
        if (__all(fast))
            chunks(std::true_type{});
        else
            chunks(std::false_type{});
        uint32_t *out = nib + (base >> 3) + (l >> 1);
        const bool odd = (lane & 1u) != 0;
#pragma unroll
        for (int r = 0; r < R; r += 2) {
            if (r + 1 < R) {
                const uint32_t y = dev::dpp<dev::kSwapPairs>(odd ? h[r] : h[r + 1]);
                if (own) {
                    if (odd)
                        st<NT>(out + (G / 2u) * (r + 1), (y << 16) | h[r + 1]);
                    else
                        st<NT>(out + (G / 2u) * r, (h[r] << 16) | y);
                }
            } else {
                const uint32_t y = dev::dpp<dev::kSwapPairs>(h[r]);
                if (own && !odd)
                    st<NT>(out + (G / 2u) * r, (h[r] << 16) | y);
            }
        }
    }
}

// Generic norms, any d: one thread per bucket (d <= 32, the bucket summed
// in index order) or one wavefront per bucket (lanes stride the bucket).
// (Max: the largest magnitude instead of the L2 norm.)
template <bool Max>
__global__ __launch_bounds__(kBlockThreads) void qsgd_norms_thread_kernel(
    const float *__restrict__ g, uint64_t n, uint32_t d, uint64_t b0, uint64_t nb,
    float *__restrict__ norms)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t b = b0 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += stride) {
        const uint64_t lo = b * d;
        const uint64_t hi = lo + d < n ? lo + d : n;
        if constexpr (Max) {
            float m = 0.0f;
            for (uint64_t e = lo; e < hi; ++e)
                m = max_in(m, fabsf(g[e]));
            norms[b] = m;
        } else {
            double ss = 0.0;
            for (uint64_t e = lo; e < hi; ++e)
                ss = __builtin_fma((double)g[e], (double)g[e], ss);
            norms[b] = bucket_norm(ss);
        }
    }
}

template <bool Max>
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
        if constexpr (Max) {
            float m = 0.0f;
            for (uint64_t e = lo + lane; e < hi; e += kWave)
                m = max_in(m, fabsf(g[e]));
            m = group_max<kWave>(m);
            if (lane == 0)
                norms[b] = m;
        } else {
            double ss = 0.0;
            for (uint64_t e = lo + lane; e < hi; e += kWave)
                ss = __builtin_fma((double)g[e], (double)g[e], ss);
            ss = group_sum<kWave>(ss);
            if (lane == 0)
                norms[b] = bucket_norm(ss);
        }
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
                    const uint32_t nbl =
                        sign_bit(g[e]) | qsgd_level_exact(fabsf(g[e]), norms[e / d], sf, s, u[q]);
                    word |= nbl << (28u - 4u * (4u * half + q));
                }
            }
        }
        nib[w] = word;
    }
}

// Decode (Knowl 3): out = +-((norm * level) / s), one division per element
// (buckets shorter than 341 elements; longer ones take the lane-table kernel
// below, which computes the same quotients).  A wavefront owns 1024
// consecutive outputs; lane L decodes elements 256q + 4L .. +3 (q = 0..3),
// so every 16-byte store instruction of the wave writes 1 KiB of
// consecutive memory.  Lanes 2m and 2m+1 read the two halves of one nibble
// word.  All loads of a lane are issued before any arithmetic (indices past
// n are clamped to element 0 and their results dropped).  Pow2: d is a
// power of two >= 4, so the 4 elements of a group share one bucket and the
// bucket index is a shift.
template <bool Pow2, bool NT>
__global__ __launch_bounds__(kBlockThreads) void qsgd_dequant_kernel(
    const float *__restrict__ norms, const uint32_t *__restrict__ nib, uint64_t n, uint32_t d,
    uint32_t dshift, uint32_t s, float *__restrict__ out)
{
    const float sf = (float)s;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint64_t ntiles = (n + kWaveElems - 1) / kWaveElems;
    const uint64_t wstride = (uint64_t)gridDim.x * kBlockWaves;
    for (uint64_t t = (uint64_t)blockIdx.x * kBlockWaves + threadIdx.x / kWave; t < ntiles;
         t += wstride) {
        uint64_t e[4];
        uint32_t word[4];
        float nrm[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            e[q] = t * kWaveElems + 256u * q + 4u * lane;
            const uint64_t es = e[q] < n ? e[q] : 0;
            word[q] = ld<NT>(nib + (es >> 3));
            if constexpr (Pow2) {
                nrm[q][0] = norms[es >> dshift];
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    nrm[q][j] = norms[(es + j < n ? es + j : es) / d];
            }
        }
        float o[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t h = (lane & 1u) ? (word[q] & 0xFFFFu) : (word[q] >> 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t nb = (h >> (12 - 4 * j)) & 0xFu;
                const float m = (Pow2 ? nrm[q][0] : nrm[q][j]) * (float)(nb & 7u);
                const float v = m / sf;
                o[q][j] = (nb & 8u) ? -v : v;
            }
        }
        const uint64_t et0 = t * kWaveElems;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v4f x;
            x.x = o[q][0];
            x.y = o[q][1];
            x.z = o[q][2];
            x.w = o[q][3];
            if (et0 + kWaveElems <= n) {
                st_tile_f4<NT>(out + et0, q, lane, x);
            } else if (e[q] + 4 <= n) {
                st<NT>(reinterpret_cast<v4f *>(out + e[q]), x);
            } else {
                for (int j = 0; j < 4; ++j)
                    if (e[q] + j < n)
                        out[e[q] + j] = o[q][j];
            }
        }
    }
}

// Decode through a lane table, for 341 <= d <= 2^30: the 1024 outputs of a
// wavefront touch at most 4 buckets (rel + 1023 < 4d for every offset rel < d
// of the tile into its first bucket), so the 64 values +-((norm * level) / s)
// of those buckets, slot L / 16 and nibble L % 16, are one per lane.  Each
// lane computes its one quotient exactly as the per-element decode does (-0
// for a sign-bit-set level 0 included), and every output is fetched from the
// lane that holds it with ds_bpermute: per element a nibble extract, an
// address and a cross-lane read, no division.  Tile layout, loads and
// stores as above.
template <bool Pow2, bool NT>
__global__ __launch_bounds__(kBlockThreads) void qsgd_dequant_lanes_kernel(
    const float *__restrict__ norms, const uint32_t *__restrict__ nib, uint64_t n, uint32_t d,
    uint32_t dshift, uint32_t s, float *__restrict__ out)
{
    const float sf = (float)s;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint64_t ntiles = (n + kWaveElems - 1) / kWaveElems;
    const uint64_t nbuckets = (n + d - 1) / d;
    const uint64_t wstride = (uint64_t)gridDim.x * kBlockWaves;
    const uint32_t tnib = lane & 15u;
    const float tlev = (float)(tnib & 7u);
    for (uint64_t t = (uint64_t)blockIdx.x * kBlockWaves + threadIdx.x / kWave; t < ntiles;
         t += wstride) {
        const uint64_t et = t * kWaveElems;
        const uint64_t b0 = Pow2 ? et >> dshift : et / d;
        const uint32_t rel0 = (uint32_t)(et - b0 * d);   // < d
        uint64_t e[4];
        uint32_t word[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            e[q] = et + 256u * q + 4u * lane;
            const uint64_t es = e[q] < n ? e[q] : 0;
            word[q] = ld<NT>(nib + (es >> 3));
        }
        const uint64_t bl = b0 + (lane >> 4);
        const float nrm = bl < nbuckets ? norms[bl] : 0.0f;
        const float m = nrm * tlev;
        const float v = m / sf;
        const int tv = __float_as_int((tnib & 8u) ? -v : v);
        float o[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t h = (lane & 1u) ? (word[q] & 0xFFFFu) : (word[q] >> 16);
            const uint32_t rel = rel0 + 256u * q + 4u * lane;
            uint32_t slot[4];
            if constexpr (Pow2) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    slot[j] = rel >> dshift;   // d >= 512: one bucket per 4 elements
            } else {
                const uint32_t s0 = (rel >= d ? 1u : 0u) + (rel >= 2u * d ? 1u : 0u) +
                                    (rel >= 3u * d ? 1u : 0u);
                const uint32_t brk = (s0 + 1u) * d - rel;   // first j in the next bucket
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    slot[j] = s0 + ((uint32_t)j >= brk ? 1u : 0u);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t nb = (h >> (12 - 4 * j)) & 0xFu;
                const int addr = (int)(((slot[j] << 4) | nb) << 2);   // < 256 for slot <= 3
                o[q][j] = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, tv));
            }
        }
        const uint64_t et0 = t * kWaveElems;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v4f x;
            x.x = o[q][0];
            x.y = o[q][1];
            x.z = o[q][2];
            x.w = o[q][3];
            if (et0 + kWaveElems <= n) {
                st_tile_f4<NT>(out + et0, q, lane, x);
            } else if (e[q] + 4 <= n) {
                st<NT>(reinterpret_cast<v4f *>(out + e[q]), x);
            } else {
                for (int j = 0; j < 4; ++j)
                    if (e[q] + j < n)
                        out[e[q] + j] = o[q][j];
            }
        }
    }
}

// ---- K-worker decode-average (QSGD summary, Knowl 3) --------------------
// out_i = (sum over workers l = 0..K-1, in order, from +0, of the decoded
// value of worker l's nibble i) / K, each decoded value exactly
// qsgd_dequant's +-((scale * level) / s).
//
// A workgroup owns a tile of 2048 elements (one nibble word per thread).
// It first writes an LDS table: for worker l and each bucket the tile
// touches, the 16 decoded values of the 16 possible nibbles (one IEEE
// division per level, written with both signs).  Then each element and
// worker costs a nibble extract, a table read and an add; no division per
// element.  Sums are staged through LDS so every store instruction writes
// 1 KiB.
constexpr uint64_t kAvgTileElems = 8u * kBlockThreads;
constexpr uint32_t kAvgChunk = 16;   // worker words loaded before they are decoded
// table rows per worker: the buckets a 2048-element tile can touch when
// d >= 228 (2047/d + 2 <= 10); smaller buckets take the per-element kernel
constexpr uint32_t kAvgSlots = 10;
constexpr uint32_t kAvgWorkerBytes = kAvgSlots * 64u;

// Add one worker's nibble word (8 elements) into the running sums: the
// nibbles, times 4 (a byte offset into a 16-float table row), are spread
// one per byte -- elements 0, 2, 4, 6 in `hi`, 1, 3, 5, 7 in `lo`, first
// element in the top byte -- so each element's table address is its row
// (off, which already holds the group's worker base) plus one byte of a
// register, and the worker's place in the group is the LDS instruction's
// immediate offset.  The empty asm keeps the compiler from folding the
// byte extraction back into a shift-and-mask per element.  All eight table
// reads are issued before the additions.  Uni: the word's eight elements
// share one bucket (d a multiple of 8), and off[0] is every element's row.
template <uint32_t J, bool Uni>
__device__ __forceinline__ void avg_word(float (&a)[8], uint32_t w, const char *tb,
                                         const uint32_t (&off)[8])
{
    uint32_t hi = (w >> 2) & 0x3C3C3C3Cu;
    uint32_t lo = (w << 2) & 0x3C3C3C3Cu;
    asm volatile("" : "+v"(hi), "+v"(lo));
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t src = (e & 1) ? lo : hi;
        const uint32_t byte = (src >> (8 * (3 - e / 2))) & 0xFFu;
        t[e] = *(const float *)(tb + (off[Uni ? 0 : e] + byte) + J * kAvgWorkerBytes);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
        a[e] += t[e];
}

// Workers l .. l+N-1 (their words w[0..N-1] already loaded), in order.
template <uint32_t N, bool Uni, uint32_t J = 0>
__device__ __forceinline__ void avg_words(float (&a)[8], const uint32_t (&w)[kAvgChunk],
                                          const char *tb, const uint32_t (&offc)[8])
{
    if constexpr (J < N) {
        avg_word<J, Uni>(a, w[J], tb, offc);
        avg_words<N, Uni, J + 1>(a, w, tb, offc);
    }
}

template <uint32_t N, bool NT, bool Uni>
__device__ __forceinline__ void avg_group(float (&a)[8], uint32_t (&w)[kAvgChunk], bool loaded,
                                          const QsgdMsgs &ms, uint32_t l, uint64_t wi,
                                          const char *tb, const uint32_t (&off)[8])
{
    if (!loaded) {
#pragma unroll
        for (uint32_t j = 0; j < N; ++j)
            w[j] = ld<NT>((const GCQ_GLOBAL uint32_t *)ms.nibbles[l + j] + wi);
    }
    uint32_t offc[8];
#pragma unroll
    for (int e = 0; e < (Uni ? 1 : 8); ++e) {
        offc[e] = off[e] + l * kAvgWorkerBytes;
        asm volatile("" : "+v"(offc[e]));   // one add per group, not per read
    }
    avg_words<N, Uni>(a, w, tb, offc);
}

// Uni: at most 64 VGPRs, so 8 wavefronts share a SIMD (the 18 KiB of LDS a
// 16-worker workgroup takes allow 8 workgroups per CU); left to itself the
// compiler takes 65, which allows 7.  The general case needs more registers
// and keeps the default.
template <bool Pow2K, bool NT, bool Uni>
__global__ __launch_bounds__(kBlockThreads, Uni ? 8 : 1) void qsgd_average_kernel(QsgdMsgs ms, uint32_t K,
                                                                      uint64_t n, uint32_t d,
                                                                      uint32_t s,
                                                                      float kf, uint64_t ntiles,
                                                                      float *__restrict__ out)
{
    extern __shared__ v4f avg_lds[];
    float *table = (float *)avg_lds;                     // K * kAvgSlots * 16 floats
    v4f *stage = avg_lds + (size_t)K * kAvgSlots * 4;    // 2048 floats
    const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const float sf = (float)s;
    const uint64_t nwords = (n + 7) >> 3;
    // one block per tile (the default): XCD-contiguous runs of tiles, so the
    // scale lines a run of tiles shares are fetched into one L2
    const uint64_t first = gridDim.x == ntiles ? dev::xcd_tile(blockIdx.x, gridDim.x) : blockIdx.x;
    for (uint64_t tile = first; tile < ntiles; tile += gridDim.x) {
        const uint64_t e_tile = tile * kAvgTileElems;
        const uint64_t e_end = e_tile + kAvgTileElems < n ? e_tile + kAvgTileElems : n;
        const uint64_t b0 = e_tile / d;
        const uint32_t nbk = (uint32_t)((e_end - 1) / d - b0 + 1);   // <= kAvgSlots
        __syncthreads();   // the previous tile is done with the table and the stage
        const uint64_t wi = (e_tile >> 3) + tid;
        const bool valid = wi < nwords;
        // the first group's nibble words do not depend on the table: their
        // loads are issued before it is built (16 workers, 8 for K < 16,
        // all K for K < 8)
        uint32_t w[kAvgChunk];
        const uint32_t first = K >= 16u ? 16u : (K >= 8u ? 8u : K);
        if (valid) {
            if (first >= 8u) {
#pragma unroll
                for (uint32_t j = 0; j < 8; ++j)
                    w[j] = ld<NT>((const GCQ_GLOBAL uint32_t *)ms.nibbles[j] + wi);
                if (first == 16u) {
#pragma unroll
                    for (uint32_t j = 8; j < 16; ++j)
                        w[j] = ld<NT>((const GCQ_GLOBAL uint32_t *)ms.nibbles[j] + wi);
                }
            } else {
#pragma unroll
                for (uint32_t j = 0; j < 7; ++j)
                    if (j < first)
                        w[j] = ld<NT>((const GCQ_GLOBAL uint32_t *)ms.nibbles[j] + wi);
            }
        }
        // thread (l, lev) = (tid / 8 + 32 j, tid % 8) fills level lev of
        // worker l, both signs (nibbles lev and 8 | lev: one division), for
        // every bucket of the tile; its scale loads are issued together.
        // With K <= 16 the upper half of the workgroup has no entries.
        {
            const uint32_t lev = tid & 7u;
            const float levf = (float)lev;
            for (uint32_t l = tid >> 3; l < K; l += kBlockThreads / 8u) {
                const GCQ_GLOBAL float *sc = (const GCQ_GLOBAL float *)ms.scales[l] + b0;
                float v[kAvgSlots];
#pragma unroll
                for (uint32_t bb = 0; bb < kAvgSlots; ++bb)
                    v[bb] = bb < nbk ? sc[bb] : 0.0f;
                float *tl = table + l * (kAvgWorkerBytes / 4u) + lev;
#pragma unroll
                for (uint32_t bb = 0; bb < kAvgSlots; ++bb) {
                    if (bb < nbk) {
                        float m = v[bb] * levf;
                        m = m / sf;
                        tl[16u * bb] = m;
                        tl[16u * bb + 8u] = -m;
                    }
                }
            }
        }
        __syncthreads();
        float a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            a[e] = 0.0f;
        if (valid) {
            // bucket slot of each of the thread's 8 elements: at most one
            // bucket boundary falls inside them (d >= 8 on this path).
            // Elements past n may map to a slot that holds no table; their
            // reads stay inside the allocation and they are never stored.
            const uint32_t rel = (uint32_t)(wi * 8u - b0 * d);
            const uint32_t bb0 = rel / d;
            const uint32_t brk = (bb0 + 1u) * d - rel;   // >= 8 when Uni
            uint32_t off[8];   // byte offset of each element's table row
#pragma unroll
            for (int e = 0; e < 8; ++e)
                off[e] = (bb0 + (!Uni && (uint32_t)e >= brk ? 1u : 0u)) * 64u;
            const char *tb = (const char *)table;
            // groups of 16, then 8 workers, then the last K mod 8 (uniform
            // branches per word): every load of a group issued, then
            // decoded in worker order
            uint32_t l = 0;
            for (; l + 16u <= K; l += 16u)
                avg_group<16, NT, Uni>(a, w, l == 0, ms, l, wi, tb, off);
            for (; l + 8u <= K; l += 8u)
                avg_group<8, NT, Uni>(a, w, l == 0, ms, l, wi, tb, off);
            const uint32_t rem = K - l;   // 0 .. 7, uniform
            if (rem) {
                if (l != 0) {
#pragma unroll
                    for (uint32_t j = 0; j < 7; ++j)
                        if (j < rem)
                            w[j] = ld<NT>((const GCQ_GLOBAL uint32_t *)ms.nibbles[l + j] + wi);
                }
                uint32_t offc[8];
#pragma unroll
                for (int e = 0; e < (Uni ? 1 : 8); ++e)
                    offc[e] = off[e] + l * kAvgWorkerBytes;
                if (rem > 0u) avg_word<0, Uni>(a, w[0], tb, offc);
                if (rem > 1u) avg_word<1, Uni>(a, w[1], tb, offc);
                if (rem > 2u) avg_word<2, Uni>(a, w[2], tb, offc);
                if (rem > 3u) avg_word<3, Uni>(a, w[3], tb, offc);
                if (rem > 4u) avg_word<4, Uni>(a, w[4], tb, offc);
                if (rem > 5u) avg_word<5, Uni>(a, w[5], tb, offc);
                if (rem > 6u) avg_word<6, Uni>(a, w[6], tb, offc);
            }
        }
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[e] = Pow2K ? a[e] * kf : a[e] / kf;   // kf = 1/K (exact) or K
        if (e_tile + kAvgTileElems <= n) {
            v4f x0, x1;
            x0.x = o[0]; x0.y = o[1]; x0.z = o[2]; x0.w = o[3];
            x1.x = o[4]; x1.y = o[5]; x1.z = o[6]; x1.w = o[7];
            stage[2 * tid] = x0;
            stage[2 * tid + 1] = x1;
            __syncthreads();
            GCQ_GLOBAL v4f *o4 = (GCQ_GLOBAL v4f *)(out + e_tile + 512u * wave);
#pragma unroll
            for (int q = 0; q < 2; ++q)
                st<NT>(o4 + 64 * q + lane, stage[128 * wave + 64 * q + lane]);
        } else if (wi < nwords) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (wi * 8u + e < n)
                    out[wi * 8u + e] = o[e];
        }
    }
}

// Any d and K: one thread per element, the division per worker as defined.
template <bool Pow2K>
__global__ __launch_bounds__(kBlockThreads) void qsgd_average_generic_kernel(
    QsgdMsgs ms, uint32_t K, uint64_t n, uint32_t d, uint32_t s, float kf, float *__restrict__ out)
{
    const float sf = (float)s;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint64_t b = i / d;
        const uint32_t sh = 28u - 4u * (uint32_t)(i & 7u);
        float acc = 0.0f;
        for (uint32_t l = 0; l < K; ++l) {
            const uint32_t nib = (ms.nibbles[l][i >> 3] >> sh) & 15u;
            float m = ms.scales[l][b] * (float)(nib & 7u);
            m = m / sf;
            acc += (nib & 8u) ? -m : m;
        }
        out[i] = Pow2K ? acc * kf : acc / kf;
    }
}

template <int CC, int H, bool Max>
void launch_fused(const gcq_tuning &tu, const float *g, uint64_t n, uint32_t s, uint32_t k0,
                  uint32_t k1, float *norms, uint32_t *nibbles, uint64_t nb_done, hipStream_t stream)
{
    constexpr uint64_t D = 256u * CC;
    const uint64_t waves = (nb_done + H - 1) / H;
    const uint32_t grid = grid_for((waves + kBlockWaves - 1) / kBlockWaves, tu.qsgd_blocks_per_cu);
    if (tu.qsgd_nt && tu.qsgd_rcp)
        qsgd_fused_kernel<CC, H, true, true, Max>
            <<<grid, kBlockThreads, 0, stream>>>(g, s, k0, k1, norms, nibbles, nb_done);
    else if (tu.qsgd_nt)
        qsgd_fused_kernel<CC, H, true, false, Max>
            <<<grid, kBlockThreads, 0, stream>>>(g, s, k0, k1, norms, nibbles, nb_done);
    else if (tu.qsgd_rcp)
        qsgd_fused_kernel<CC, H, false, true, Max>
            <<<grid, kBlockThreads, 0, stream>>>(g, s, k0, k1, norms, nibbles, nb_done);
    else
        qsgd_fused_kernel<CC, H, false, false, Max>
            <<<grid, kBlockThreads, 0, stream>>>(g, s, k0, k1, norms, nibbles, nb_done);
    if (n > nb_done * D)   // a short last bucket
        qsgd_tail_kernel<Max><<<1, kWave, 0, stream>>>(g, n, nb_done * D, nb_done, s, k0, k1, norms,
                                                      nibbles);
}

// Buckets per wavefront: the knob (0: as many as make 4 float4 chunks per
// lane, which measured fastest), limited to C H <= 4 chunks per lane
// (register budget).
template <bool Max>
void launch_fused_c(uint32_t C, const gcq_tuning &tu, const float *g, uint64_t n, uint32_t s,
                    uint32_t k0, uint32_t k1, float *norms, uint32_t *nibbles, uint64_t nb_done,
                    hipStream_t stream)
{
    const uint32_t hmax = C <= 4 ? 4u / C : 1u;
    const uint32_t want = tu.qsgd_buckets_per_wave ? (uint32_t)tu.qsgd_buckets_per_wave : hmax;
    const uint32_t H = want < hmax ? want : hmax;
#define GCQ_F(CC, HH) \
    launch_fused<CC, HH, Max>(tu, g, n, s, k0, k1, norms, nibbles, nb_done, stream)
    switch (C) {
    case 1:
        if (H >= 4)
            GCQ_F(1, 4);
        else if (H == 2)
            GCQ_F(1, 2);
        else
            GCQ_F(1, 1);
        break;
    case 2:
        if (H >= 2)
            GCQ_F(2, 2);
        else
            GCQ_F(2, 1);
        break;
    case 4: GCQ_F(4, 1); break;
    default: GCQ_F(8, 1); break;
    }
#undef GCQ_F
}

}  // namespace

hipError_t launch_qsgd_quantize(const float *g, uint64_t n, uint32_t d, uint32_t s, uint64_t seed,
                                float *norms, uint32_t *nibbles, bool maxnorm, hipStream_t stream)
{
    if (!n)
        return hipSuccess;
    const gcq_tuning tu = tuning();
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const uint64_t nb = (n + d - 1) / d;
    const uint64_t nwords = (n + 7) >> 3;
    uint64_t nb_done = 0;  // buckets (and their words) finished by the fused kernel
    const uint32_t C = d % 256u == 0 ? d / 256u : 0u;
    if ((C == 1 || C == 2 || C == 4 || C == 8) && n >= d) {
        // the full buckets, then a short last one in a one-wavefront launch
        if (maxnorm)
            launch_fused_c<true>(C, tu, g, n, s, k0, k1, norms, nibbles, n / d, stream);
        else
            launch_fused_c<false>(C, tu, g, n, s, k0, k1, norms, nibbles, n / d, stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        nb_done = nb;
    }
    if (nb_done < nb) {
        const uint64_t left = nb - nb_done;
        if (d <= 32) {
            const uint32_t grid = grid_for((left + kBlockThreads - 1) / kBlockThreads, 0);
            if (maxnorm)
                qsgd_norms_thread_kernel<true>
                    <<<grid, kBlockThreads, 0, stream>>>(g, n, d, nb_done, nb, norms);
            else
                qsgd_norms_thread_kernel<false>
                    <<<grid, kBlockThreads, 0, stream>>>(g, n, d, nb_done, nb, norms);
        } else {
            const uint32_t grid = grid_for((left + kBlockWaves - 1) / kBlockWaves, 0);
            if (maxnorm)
                qsgd_norms_wave_kernel<true>
                    <<<grid, kBlockThreads, 0, stream>>>(g, n, d, nb_done, nb, norms);
            else
                qsgd_norms_wave_kernel<false>
                    <<<grid, kBlockThreads, 0, stream>>>(g, n, d, nb_done, nb, norms);
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
    const uint64_t ntiles = (n + kWaveElems - 1) / kWaveElems;
    const uint32_t grid =
        grid_for((ntiles + kBlockWaves - 1) / kBlockWaves, tu.qsgd_dequant_blocks_per_cu);
    const bool pow2 = d >= 4 && (d & (d - 1)) == 0;
    const uint32_t dshift = pow2 ? (uint32_t)__builtin_ctz(d) : 0u;
    const bool lanes = d >= 341 && d <= (1u << 30);
#define GCQ_DQ(P, NT)                                                                           \
    do {                                                                                        \
        if (lanes)                                                                              \
            qsgd_dequant_lanes_kernel<P, NT>                                                    \
                <<<grid, kBlockThreads, 0, stream>>>(norms, nibbles, n, d, dshift, s, out);     \
        else                                                                                    \
            qsgd_dequant_kernel<P, NT>                                                          \
                <<<grid, kBlockThreads, 0, stream>>>(norms, nibbles, n, d, dshift, s, out);     \
    } while (0)
    if (pow2) {
        if (tu.qsgd_dequant_nt)
            GCQ_DQ(true, true);
        else
            GCQ_DQ(true, false);
    } else {
        if (tu.qsgd_dequant_nt)
            GCQ_DQ(false, true);
        else
            GCQ_DQ(false, false);
    }
#undef GCQ_DQ
    return hipGetLastError();
}

hipError_t launch_qsgd_average(const QsgdMsgs &ms, uint32_t K, uint64_t n, uint32_t d, uint32_t s,
                               float *out, hipStream_t stream)
{
    if (!n)
        return hipSuccess;
    const gcq_tuning tu = tuning();
    const bool pow2 = (K & (K - 1u)) == 0u;
    const float kf = pow2 ? 1.0f / (float)K : (float)K;   // 1/K is exact for K = 2^j
    // buckets a 2048-element tile can touch
    const uint64_t slots = (kAvgTileElems - 1) / d + 2;
    const uint64_t lds = ((uint64_t)K * kAvgSlots * 16u + kAvgTileElems) * 4u;
    if (slots <= kAvgSlots && d <= (1u << 30) && lds <= 64u * 1024u) {
        const uint64_t ntiles = (n + kAvgTileElems - 1) / kAvgTileElems;
        const uint32_t grid = grid_for(ntiles, tu.qsgd_dequant_blocks_per_cu);
        // a nibble word never straddles a bucket boundary when 8 divides d
        const bool uni = (d & 7u) == 0u;
        const uint64_t lds_run = lds + resident_lds_pad((uint32_t)lds, tu.qsgd_avg_resident_per_cu);
#define GCQ_AVG(P, NT, U)                                                                     \
    qsgd_average_kernel<P, NT, U><<<grid, kBlockThreads, (size_t)lds_run, stream>>>(          \
        ms, K, n, d, s, kf, ntiles, out)
#define GCQ_AVG_U(P, NT)                                                                      \
    do {                                                                                      \
        if (uni)                                                                              \
            GCQ_AVG(P, NT, true);                                                             \
        else                                                                                  \
            GCQ_AVG(P, NT, false);                                                            \
    } while (0)
        if (pow2) {
            if (tu.qsgd_dequant_nt)
                GCQ_AVG_U(true, true);
            else
                GCQ_AVG_U(true, false);
        } else {
            if (tu.qsgd_dequant_nt)
                GCQ_AVG_U(false, true);
            else
                GCQ_AVG_U(false, false);
        }
#undef GCQ_AVG_U
#undef GCQ_AVG
    } else {
        const uint32_t grid = grid_for((n + kBlockThreads - 1) / kBlockThreads, 0);
        if (pow2)
            qsgd_average_generic_kernel<true>
                <<<grid, kBlockThreads, 0, stream>>>(ms, K, n, d, s, kf, out);
        else
            qsgd_average_generic_kernel<false>
                <<<grid, kBlockThreads, 0, stream>>>(ms, K, n, d, s, kf, out);
    }
    return hipGetLastError();
}

}  // namespace gcq
