// dequant_reduce.hip -- dequantize-and-reduce over W packed 2-bit buffers
// (MXNet PR "2bit gradient compression", "Local kvstore": device 0 decodes
// every device's packed gradient and sums them; CD-SGD 3.4.1: 11 -> +t,
// 10 -> -t) for gfx950.
//
// Per element: W/4 bytes of codes read, 4 bytes of sum written (8 B at
// W = 16) and, per worker, one exact float32 fma.  The workers are added
// strictly in the order 0..W-1, so the result is bit-identical to the
// sequential float32 sum.
#include "gcq_device.h"
#include "gcq_internal.h"

namespace gcq {

namespace {

using dev::ld;
using dev::st;
using dev::v4f;

// Re-encode the sixteen 2-bit codes of a word as 2-bit two's-complement
// values of what they stand for: 11 (+t) -> 01 (+1), 10 (-t) -> 11 (-1),
// 00 and 01 (read as zero) -> 00.
__device__ __forceinline__ uint32_t signed_pairs(uint32_t w)
{
    const uint32_t hi = w & 0xAAAAAAAAu;
    const uint32_t lo_at_hi = (w << 1) & 0xAAAAAAAAu;
    return (hi & ~lo_at_hi) | (hi >> 1);
}

// Add one worker's word (16 codes) into the 16 running sums.  Element k's
// value f_k in {-1, 0, +1} is moved to the top two bits of a byte
// (m_r = (pairs << 2r) & 0xC0C0C0C0 holds elements r, 4+r, 8+r, 12+r in
// bytes 3, 2, 1, 0), so one signed-byte conversion (an SDWA v_cvt) yields
// 64 f_k exactly.  With tq = t/64 (exact: t >= 2^-120), fma(tq, 64 f_k, a)
// rounds t f_k + a once: the same result as a + (+t | -t | 0) in float32.
// Scaled = false does the same with f_k itself and tq = t (tiny t).
template <bool Scaled>
__device__ __forceinline__ void accumulate(float (&a)[16], uint32_t w, float tq)
{
    const uint32_t pairs = signed_pairs(w);
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

constexpr int kChunk = 16;      // worker words loaded before they are decoded
constexpr int kLdsRow = 16;     // floats per staged row (one packed word's sums)

// One thread per packed word position (16 elements) per iteration; the
// loop is uniform per workgroup (block tiles of 256 words).  Word offsets
// are 32-bit (the host splits larger inputs), so each load is a global
// load with a scalar base and a 32-bit vector offset.
//
// Lds = true: a full block tile stages each wavefront's 64 x 16 sums in
// LDS and reads them back transposed, so lane L stores elements
// 256q + 4L .. +3 (q = 0..3): every store instruction writes 1 KiB of
// consecutive memory instead of 64 scattered 16-byte pieces.
template <bool Scaled, bool NTL, bool NTS, bool Lds>
__global__ __launch_bounds__(kBlockThreads) void dq_reduce_kernel(DqWorkers ws, uint32_t W,
                                                                  uint32_t nwords, uint64_t n,
                                                                  float tq, float *__restrict__ acc)
{
    __shared__ v4f stage[Lds ? kBlockWaves * kWave * kLdsRow / 4 : 1];
    const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    GCQ_GLOBAL float *out = (GCQ_GLOBAL float *)acc;
    for (uint32_t base = blockIdx.x * kBlockThreads; base < nwords;
         base += gridDim.x * kBlockThreads) {
        const uint32_t wi = base + tid;
        const bool valid = wi < nwords;
        float a[16];
#pragma unroll
        for (int k = 0; k < 16; ++k)
            a[k] = 0.0f;
        if (valid) {
            const uint32_t boff = wi * 4u;
            for (uint32_t w0 = 0; w0 < W; w0 += kChunk) {
                uint32_t wd[kChunk];
#pragma unroll
                for (int j = 0; j < kChunk; ++j)
                    wd[j] = (w0 + j < W)
                                ? ld<NTL>((const GCQ_GLOBAL uint32_t *)(
                                      (const GCQ_GLOBAL char *)ws.w[w0 + j] + boff))
                                : 0u;
#pragma unroll
                for (int j = 0; j < kChunk; ++j)
                    if (w0 + j < W)
                        accumulate<Scaled>(a, wd[j], tq);
            }
        }
        const uint64_t e = (uint64_t)wi * 16u;
        if (Lds && ((uint64_t)base + kBlockThreads) * 16u <= n) {
            v4f *rowp = stage + (wave * kWave + lane) * (kLdsRow / 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v4f x;
                x.x = a[4 * q];
                x.y = a[4 * q + 1];
                x.z = a[4 * q + 2];
                x.w = a[4 * q + 3];
                rowp[q] = x;
            }
            __syncthreads();
            const uint64_t e0 = ((uint64_t)base + (uint64_t)wave * kWave) * 16u;
            const v4f *wstage = stage + wave * kWave * (kLdsRow / 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // element 256q + 4L of the wave tile: row 16q + L/4, column 4(L%4)
                const v4f x = wstage[(16 * q + (lane >> 2)) * (kLdsRow / 4) + (lane & 3)];
                st<NTS>((GCQ_GLOBAL v4f *)(out + e0) + 64 * q + lane, x);
            }
            __syncthreads();
        } else if (valid) {
            if (e + 16 <= n) {
                GCQ_GLOBAL v4f *o = (GCQ_GLOBAL v4f *)(out + e);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v4f x;
                    x.x = a[4 * q];
                    x.y = a[4 * q + 1];
                    x.z = a[4 * q + 2];
                    x.w = a[4 * q + 3];
                    st<NTS>(o + q, x);
                }
            } else {
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    if (e + k < n)
                        out[e + k] = a[k];
            }
        }
    }
}

template <bool Scaled, bool NTL, bool NTS, bool Lds>
void launch_one(uint32_t grid, hipStream_t stream, const DqWorkers &ws, uint32_t W,
                uint32_t nwords, uint64_t n, float tq, float *acc)
{
    dq_reduce_kernel<Scaled, NTL, NTS, Lds>
        <<<grid, kBlockThreads, 0, stream>>>(ws, W, nwords, n, tq, acc);
}

template <bool Scaled>
void dispatch(const gcq_tuning &tu, uint32_t grid, hipStream_t stream, const DqWorkers &ws,
              uint32_t W, uint32_t nwords, uint64_t n, float tq, float *acc)
{
    const int key = tu.dq_nt_loads * 4 + tu.dq_nt_stores * 2 + tu.dq_lds_stores;
    switch (key) {
    case 0: launch_one<Scaled, false, false, false>(grid, stream, ws, W, nwords, n, tq, acc); break;
    case 1: launch_one<Scaled, false, false, true>(grid, stream, ws, W, nwords, n, tq, acc); break;
    case 2: launch_one<Scaled, false, true, false>(grid, stream, ws, W, nwords, n, tq, acc); break;
    case 3: launch_one<Scaled, false, true, true>(grid, stream, ws, W, nwords, n, tq, acc); break;
    case 4: launch_one<Scaled, true, false, false>(grid, stream, ws, W, nwords, n, tq, acc); break;
    case 5: launch_one<Scaled, true, false, true>(grid, stream, ws, W, nwords, n, tq, acc); break;
    case 6: launch_one<Scaled, true, true, false>(grid, stream, ws, W, nwords, n, tq, acc); break;
    default: launch_one<Scaled, true, true, true>(grid, stream, ws, W, nwords, n, tq, acc); break;
    }
}

// Words per launch: keeps every byte offset of a word array below 2^32.
constexpr uint64_t kMaxWordsPerLaunch = (uint64_t)1 << 30;

}  // namespace

hipError_t launch_dequant_reduce(const DqWorkers &w, uint32_t W, uint64_t n, float t, float *acc,
                                 hipStream_t stream)
{
    const uint64_t nwords = (n + 15) >> 4;
    if (!nwords)
        return hipSuccess;
    const gcq_tuning tu = tuning();
    // t/64 is exact (a power-of-two scaling that stays normal) for t >= 2^-120.
    const bool scaled = t >= 0x1p-120f;
    const float tq = scaled ? t * 0x1p-6f : t;
    for (uint64_t w0 = 0; w0 < nwords; w0 += kMaxWordsPerLaunch) {
        const uint64_t cw = nwords - w0 < kMaxWordsPerLaunch ? nwords - w0 : kMaxWordsPerLaunch;
        const uint64_t cn = (n - w0 * 16) < cw * 16 ? (n - w0 * 16) : cw * 16;
        DqWorkers ws = w;
        for (uint32_t k = 0; k < W; ++k)
            ws.w[k] = w.w[k] + w0;
        const uint32_t grid =
            grid_for((cw + kBlockThreads - 1) / kBlockThreads, tu.dq_blocks_per_cu);
        if (scaled)
            dispatch<true>(tu, grid, stream, ws, W, (uint32_t)cw, cn, tq, acc + w0 * 16);
        else
            dispatch<false>(tu, grid, stream, ws, W, (uint32_t)cw, cn, tq, acc + w0 * 16);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace gcq
