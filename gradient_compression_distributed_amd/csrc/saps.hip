// saps.hip -- SAPS shared-seed random sparsification ("Communication-
// Efficient Decentralized Learning with Sparsification and Adaptive Peer
// Selection": a Bernoulli(1/c) mask drawn from a seed every worker shares,
// only the kept components exchanged, single-peer gossip) for gfx950.
//
// Three steps over tiles of 8192 elements (256 threads x 32 elements):
//   mask   -- each thread draws its 32 uniforms (8 Philox calls, the QSGD
//             quantizer's stream), keeps element i when U_i < T with
//             T = ceil(2^24 / c) (exactly u_i c < 1), tested on the raw
//             32-bit word as c_i <= 256 T - 1 (U_i = c_i >> 8; T is in
//             [1, 2^24] for c in [1, inf), so 256 T - 1 fits 32 bits) by
//             the carry of a 64-bit add,
//             writes one 32-bit mask word (bit j = element 32w + j) and the
//             tile's kept count;
//   scan   -- the tile counts become exclusive offsets (and the total);
//   apply  -- per tile, a block scan of the threads' popcounts gives each
//             thread its first rank; it then gathers x at its set bits into
//             values[rank], or merges a peer's values there.  Only the cache
//             lines holding kept elements are read: at c = 100 about a
//             quarter of them.
#include "gcq_device.h"
#include "gcq_internal.h"

namespace gcq {

namespace {

using dev::ld;
using dev::philox4x32_10;
using dev::st;

constexpr uint32_t kSapsThreads = 256;
constexpr uint64_t kSapsTileElems = 32u * kSapsThreads;

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x += __shfl_xor(x, off, kWave);
    return x;
}

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x, uint32_t lane)
{
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, kWave);
        if (lane >= (uint32_t)off)
            x += y;
    }
    return x;
}

__global__ __launch_bounds__(kSapsThreads) void saps_mask_kernel(uint64_t n, uint32_t Tm,
                                                                  uint32_t k0, uint32_t k1,
                                                                  uint32_t *__restrict__ mask,
                                                                  uint64_t *__restrict__ offs,
                                                                  uint64_t ntiles)
{
    __shared__ uint32_t wsum[kSapsThreads / kWave];
    const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    // Element dropped when c > Tm, i.e. when c + (2^32 - 1 - Tm) carries
    // into bit 32.  With a factor of 1 the compiler cannot see, c * one + m
    // is one v_mad_u64_u32 whose high word is that carry, and the bit goes
    // into place with one shift-or: two instructions per element, where a
    // compare, a select and an or take three or more.
    const uint64_t m = 0xFFFFFFFFull - Tm;
    uint32_t one = 1;
    asm volatile("" : "+s"(one));
    for (uint64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const uint64_t wi = tile * kSapsThreads + tid;
        const uint64_t e0 = wi * 32u;
        uint32_t word = 0;
        if (e0 < n) {
            uint32_t drop = 0;
#pragma unroll
            for (uint32_t j = 0; j < 8; ++j) {
                const uint64_t q = (e0 >> 2) + j;
                uint32_t c[4] = {(uint32_t)q, (uint32_t)(q >> 32), 0u, 0u};
                philox4x32_10(c, k0, k1);
#pragma unroll
                for (uint32_t r = 0; r < 4; ++r) {
                    uint32_t carry = (uint32_t)(((uint64_t)c[r] * one + m) >> 32);
                    asm("" : "+v"(carry));   // keeps the shift-or from folding into the product
                    drop |= carry << (4 * j + r);
                }
            }
            word = ~drop;
            if (n - e0 < 32u)
                word &= (1u << (uint32_t)(n - e0)) - 1u;   // elements past n are not kept
            st<true>((GCQ_GLOBAL uint32_t *)mask + wi, word);
        }
        const uint32_t cnt = wave_sum_u32((uint32_t)__builtin_popcount(word));
        if (lane == 0)
            wsum[wave] = cnt;
        __syncthreads();
        if (tid == 0)
            offs[tile] = (uint64_t)wsum[0] + wsum[1] + wsum[2] + wsum[3];
        __syncthreads();
    }
}

// In-place exclusive scan of a[0..count) with a[count] = the total (the SAPS
// tile offsets and the Elias coder's bucket offsets), in three passes and no
// workspace, over chunks of kScanChunk entries:
//   sums  -- each chunk's sum replaces its last entry (that entry's own value
//            is never needed again: no exclusive prefix includes it);
//   top   -- one workgroup scans those last entries (exclusive, in place)
//            and writes the total;
//   local -- each chunk scans its other entries from its offset, and its
//            last entry gets the offset plus all of them.
constexpr uint32_t kScanThreads = 1024;
constexpr uint64_t kScanChunk = 8u * kScanThreads;

__device__ __forceinline__ uint64_t block_exclusive_scan(uint64_t v, uint64_t *part,
                                                          uint64_t &total)
{
    const uint32_t tid = threadIdx.x;
    part[tid] = v;
    __syncthreads();
    for (uint32_t off = 1; off < kScanThreads; off <<= 1) {
        const uint64_t t = tid >= off ? part[tid - off] : 0u;
        __syncthreads();
        part[tid] += t;
        __syncthreads();
    }
    total = part[kScanThreads - 1];
    const uint64_t excl = part[tid] - v;
    __syncthreads();
    return excl;
}

__global__ __launch_bounds__(kScanThreads) void scan_sums_kernel(uint64_t *__restrict__ a,
                                                                  uint64_t count)
{
    __shared__ uint64_t part[kScanThreads];
    const uint64_t c0 = (uint64_t)blockIdx.x * kScanChunk;
    const uint64_t c1 = c0 + kScanChunk < count ? c0 + kScanChunk : count;
    uint64_t local = 0;
    for (uint64_t i = c0 + threadIdx.x; i < c1; i += kScanThreads)
        local += a[i];
    uint64_t total;
    (void)block_exclusive_scan(local, part, total);
    if (threadIdx.x == 0)
        a[c1 - 1] = total;
}

// Exclusive scan of the chunks' last entries, one workgroup, with the total
// written to a[count].
__global__ __launch_bounds__(kScanThreads) void scan_top_kernel(uint64_t *__restrict__ a,
                                                                 uint64_t count, uint64_t nchunks)
{
    __shared__ uint64_t part[kScanThreads];
    uint64_t carry = 0;
    for (uint64_t base = 0; base < nchunks; base += kScanThreads) {
        const uint64_t c = base + threadIdx.x;
        const uint64_t idx = c < nchunks ? ((c + 1) * kScanChunk < count ? (c + 1) * kScanChunk
                                                                          : count) - 1
                                         : 0;
        const uint64_t v = c < nchunks ? a[idx] : 0u;
        uint64_t total;
        const uint64_t excl = block_exclusive_scan(v, part, total);
        if (c < nchunks)
            a[idx] = carry + excl;
        carry += total;
    }
    if (threadIdx.x == 0)
        a[count] = carry;
}

__global__ __launch_bounds__(kScanThreads) void scan_local_kernel(uint64_t *__restrict__ a,
                                                                   uint64_t count)
{
    __shared__ uint64_t part[kScanThreads];
    __shared__ uint64_t offset;
    const uint64_t c0 = (uint64_t)blockIdx.x * kScanChunk;
    const uint64_t c1 = c0 + kScanChunk < count ? c0 + kScanChunk : count;
    if (threadIdx.x == 0)
        offset = a[c1 - 1];
    // thread t owns entries c0 + 8t .. +7; the chunk's last entry counts as 0
    uint64_t v[8];
    uint64_t local = 0;
#pragma unroll
    for (uint32_t j = 0; j < 8; ++j) {
        const uint64_t i = c0 + 8u * threadIdx.x + j;
        v[j] = i < c1 - 1 ? a[i] : 0u;
        local += v[j];
    }
    uint64_t total;
    uint64_t excl = block_exclusive_scan(local, part, total);   // its barriers order `offset`
    excl += offset;
#pragma unroll
    for (uint32_t j = 0; j < 8; ++j) {
        const uint64_t i = c0 + 8u * threadIdx.x + j;
        if (i < c1)
            a[i] = excl;
        excl += v[j];
    }
}

// Merge = false: values[rank] = x[i] for every kept i (rank < cap).
// Merge = true:  x[i] = (x[i] + values[rank]) * 0.5 for every kept i.
template <bool Merge>
__global__ __launch_bounds__(kSapsThreads) void saps_apply_kernel(
    float *__restrict__ x, uint64_t n, const uint32_t *__restrict__ mask,
    const uint64_t *__restrict__ offs, float *__restrict__ values, uint64_t cap, uint64_t ntiles)
{
    __shared__ uint32_t wsum[kSapsThreads / kWave];
    const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    GCQ_GLOBAL float *xg = (GCQ_GLOBAL float *)x;
    GCQ_GLOBAL float *vg = (GCQ_GLOBAL float *)values;
    for (uint64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const uint64_t wi = tile * kSapsThreads + tid;
        const uint64_t e0 = wi * 32u;
        uint32_t word = e0 < n ? ld<true>((const GCQ_GLOBAL uint32_t *)mask + wi) : 0u;
        const uint32_t cnt = (uint32_t)__builtin_popcount(word);
        const uint32_t incl = wave_inclusive_scan(cnt, lane);
        if (lane == kWave - 1)
            wsum[wave] = incl;
        __syncthreads();
        uint32_t before = 0;
        for (uint32_t w = 0; w < wave; ++w)
            before += wsum[w];
        uint64_t rank = offs[tile] + before + incl - cnt;
        while (word) {
            const uint32_t j = (uint32_t)__builtin_ctz(word);
            word &= word - 1u;
            if (rank < cap) {
                if constexpr (Merge)
                    xg[e0 + j] = (xg[e0 + j] + vg[rank]) * 0.5f;
                else
                    vg[rank] = xg[e0 + j];
            }
            ++rank;
        }
        __syncthreads();
    }
}

}  // namespace

uint32_t saps_threshold(float c)
{
    // smallest integer T with T * c >= 2^24 (products exact in double)
    const double two24 = 16777216.0, cd = (double)c;
    double t = __builtin_ceil(two24 / cd);
    while (t > 0.0 && (t - 1.0) * cd >= two24)
        t -= 1.0;
    while (t * cd < two24)
        t += 1.0;
    return (uint32_t)(t < two24 ? t : two24);
}

hipError_t launch_saps_mask(uint64_t n, float c, uint64_t seed, uint32_t *mask, uint64_t *offs,
                            hipStream_t stream)
{
    const uint64_t ntiles = (n + kSapsTileElems - 1) / kSapsTileElems;
    if (ntiles) {
        const uint32_t grid = grid_for(ntiles, 0);
        const uint32_t Tm = (uint32_t)(256u * (uint64_t)saps_threshold(c) - 1u);
        saps_mask_kernel<<<grid, kSapsThreads, 0, stream>>>(n, Tm, (uint32_t)seed,
                                                            (uint32_t)(seed >> 32), mask, offs,
                                                            ntiles);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return launch_exclusive_scan_u64(offs, ntiles, stream);
}

hipError_t launch_exclusive_scan_u64(uint64_t *a, uint64_t count, hipStream_t stream)
{
    const uint64_t nchunks = (count + kScanChunk - 1) / kScanChunk;
    if (nchunks) {
        if (nchunks > 0x7FFFFFFFu)
            return hipErrorInvalidValue;
        scan_sums_kernel<<<(uint32_t)nchunks, kScanThreads, 0, stream>>>(a, count);
    }
    scan_top_kernel<<<1, kScanThreads, 0, stream>>>(a, count, nchunks);
    if (nchunks)
        scan_local_kernel<<<(uint32_t)nchunks, kScanThreads, 0, stream>>>(a, count);
    return hipGetLastError();
}

hipError_t launch_saps_apply(float *x, uint64_t n, const uint32_t *mask, const uint64_t *offs,
                             float *values, uint64_t cap, bool merge, hipStream_t stream)
{
    const uint64_t ntiles = (n + kSapsTileElems - 1) / kSapsTileElems;
    if (!ntiles)
        return hipSuccess;
    const uint32_t grid = grid_for(ntiles, 0);
    if (merge)
        saps_apply_kernel<true>
            <<<grid, kSapsThreads, 0, stream>>>(x, n, mask, offs, values, cap, ntiles);
    else
        saps_apply_kernel<false>
            <<<grid, kSapsThreads, 0, stream>>>(x, n, mask, offs, values, cap, ntiles);
    return hipGetLastError();
}

}  // namespace gcq
