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

using dev::kBufferRsrcWord3;
using dev::kCpolNt;
using dev::kCpolSc1;
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

// Add one worker's word (16 codes) into the 16 running sums, in one of
// three decodes (Mode), each exact:
//
// kDecodeFp4: the signed pairs are masked to the top two bits of each
//   nibble (me: pairs 0, 2, .., 14; mo: pairs 1, 3, .., 15, in nibbles 7..0),
//   which makes each nibble the FP4 (E2M1) code of +2.0 (0100), -2.0 (1100)
//   or 0 (0000).  One v_cvt_scalef32_pk_f32_fp4 (scale 1) turns a byte, i.e.
//   two elements, into two exact floats (low nibble -> .x).  With
//   tq = t/2 (exact for t >= 2^-120), fma(tq, 2 f, a) rounds t f + a once:
//   the same result as a + (+t | -t | 0) in float32.
// kDecodeSdwa: the pairs are masked to the top of each byte (m_r =
//   (pairs << 2r) & 0xC0C0C0C0 holds elements r, 4+r, 8+r, 12+r in bytes
//   3..0) and one signed-byte conversion (SDWA v_cvt) gives 64 f exactly;
//   tq = t/64.
// kDecodePlain: f from a sign-extending shift, tq = t (any t, including
//   t < 2^-120, where t/2 or t/64 would not be exact).
// kProbe (measurement only): no decode at all, the word is XORed into the
//   first sum, so the kernel keeps its loads, staging and stores and does
//   no arithmetic (gcq_probe_reduce).
enum { kDecodeFp4 = 0, kDecodeSdwa = 1, kDecodePlain = 2, kProbe = 3 };
typedef float v2f __attribute__((ext_vector_type(2)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

// Byte B of the masked words: nibble 2B holds pair 14-4B (me) / 15-4B (mo),
// nibble 2B+1 pair 12-4B / 13-4B.
template <int B>
__device__ __forceinline__ void fp4_byte(float (&a)[16], uint32_t me, uint32_t mo, float tq)
{
    const v2f e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(me, 1.0f, B);
    const v2f o = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(mo, 1.0f, B);
    a[14 - 4 * B] = __builtin_fmaf(tq, e.x, a[14 - 4 * B]);
    a[12 - 4 * B] = __builtin_fmaf(tq, e.y, a[12 - 4 * B]);
    a[15 - 4 * B] = __builtin_fmaf(tq, o.x, a[15 - 4 * B]);
    a[13 - 4 * B] = __builtin_fmaf(tq, o.y, a[13 - 4 * B]);
}

template <int Mode>
__device__ __forceinline__ void accumulate(float (&a)[16], uint32_t w, float tq)
{
    if constexpr (Mode == kProbe) {
        a[0] = __uint_as_float(__float_as_uint(a[0]) ^ w);
        return;
    }
    const uint32_t pairs = signed_pairs(w);
    if constexpr (Mode == kDecodeFp4) {
        const uint32_t me = pairs & 0xCCCCCCCCu;
        const uint32_t mo = (pairs << 2) & 0xCCCCCCCCu;
        fp4_byte<0>(a, me, mo, tq);
        fp4_byte<1>(a, me, mo, tq);
        fp4_byte<2>(a, me, mo, tq);
        fp4_byte<3>(a, me, mo, tq);
    } else if constexpr (Mode == kDecodeSdwa) {
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

// Store of 16 bytes of a full tile's sums, `off` bytes into a wavefront's
// run of `bytes` consecutive bytes at `base`.  NTS: a buffer store with the
// nt and sc1 cache-policy bits, which ran the 2^30-element, 16-worker reduce
// about 2% faster than nt alone; otherwise a plain store.
template <bool NTS>
__device__ __forceinline__ void st_run(GCQ_GLOBAL float *base, uint32_t bytes, uint32_t off,
                                       v4f x)
{
    if constexpr (NTS) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)bytes, kBufferRsrcWord3);
        __builtin_amdgcn_raw_buffer_store_b128(x, rs, (int)off, 0, kCpolNt | kCpolSc1);
    } else {
        *(GCQ_GLOBAL v4f *)((GCQ_GLOBAL char *)base + off) = x;
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
template <int Mode, bool NTL, bool NTS, bool Lds>
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
            uint32_t w0 = 0;
            // whole groups of kChunk workers: all loads issued, then decoded
            for (; w0 + kChunk <= W; w0 += kChunk) {
                uint32_t wd[kChunk];
#pragma unroll
                for (int j = 0; j < kChunk; ++j)
                    wd[j] = ld<NTL>((const GCQ_GLOBAL uint32_t *)(
                        (const GCQ_GLOBAL char *)ws.w[w0 + j] + boff));
#pragma unroll
                for (int j = 0; j < kChunk; ++j)
                    accumulate<Mode>(a, wd[j], tq);
            }
            // the rest, one worker at a time (still in worker order)
            for (; w0 < W; ++w0)
                accumulate<Mode>(a,
                                 ld<NTL>((const GCQ_GLOBAL uint32_t *)(
                                     (const GCQ_GLOBAL char *)ws.w[w0] + boff)),
                                 tq);
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
                st_run<NTS>(out + e0, kWave * 16 * 4, (64 * q + lane) * 16, x);
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

// Two packed words per thread (32 elements): one 8-byte load per worker
// (the word arrays 8-byte aligned), a block tile of 512 words.  Sums of a
// full tile leave through LDS as in dq_reduce_kernel: rows of 32 floats
// padded to 36 (a 144-byte stride spreads the lanes' rows over the banks),
// read back so that lane L stores elements 256q + 4L .. +3 (q = 0..7).
constexpr int kRow2 = 36;   // floats per staged row

template <int Mode, bool NTL, bool NTS>
__global__ __launch_bounds__(kBlockThreads) void dq_reduce2_kernel(DqWorkers ws, uint32_t W,
                                                                   uint32_t nwords, uint64_t n,
                                                                   float tq, float *__restrict__ acc)
{
    __shared__ v4f stage[kBlockWaves * kWave * kRow2 / 4];
    const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    GCQ_GLOBAL float *out = (GCQ_GLOBAL float *)acc;
    for (uint32_t base = blockIdx.x * 2u * kBlockThreads; base < nwords;
         base += gridDim.x * 2u * kBlockThreads) {
        const uint32_t wi = base + 2u * tid;   // the thread's first word
        float a[16], b[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            a[k] = 0.0f;
            b[k] = 0.0f;
        }
        if (wi + 1u < nwords) {
            const uint32_t boff = wi * 4u;
            uint32_t w0 = 0;
            for (; w0 + kChunk <= W; w0 += kChunk) {
                v2u wd[kChunk];
#pragma unroll
                for (int j = 0; j < kChunk; ++j)
                    wd[j] = ld<NTL>((const GCQ_GLOBAL v2u *)(
                        (const GCQ_GLOBAL char *)ws.w[w0 + j] + boff));
#pragma unroll
                for (int j = 0; j < kChunk; ++j) {
                    accumulate<Mode>(a, wd[j].x, tq);
                    accumulate<Mode>(b, wd[j].y, tq);
                }
            }
            for (; w0 < W; ++w0) {
                const v2u wd = ld<NTL>((const GCQ_GLOBAL v2u *)(
                    (const GCQ_GLOBAL char *)ws.w[w0] + boff));
                accumulate<Mode>(a, wd.x, tq);
                accumulate<Mode>(b, wd.y, tq);
            }
        } else if (wi < nwords) {   // the last word alone
            const uint32_t boff = wi * 4u;
            for (uint32_t w0 = 0; w0 < W; ++w0)
                accumulate<Mode>(a,
                                 ld<NTL>((const GCQ_GLOBAL uint32_t *)(
                                     (const GCQ_GLOBAL char *)ws.w[w0] + boff)),
                                 tq);
        }
        const uint64_t e = (uint64_t)wi * 16u;
        if (((uint64_t)base + 2u * kBlockThreads) * 16u <= n) {
            v4f *rowp = stage + (wave * kWave + lane) * (kRow2 / 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v4f x, y;
                x.x = a[4 * q];
                x.y = a[4 * q + 1];
                x.z = a[4 * q + 2];
                x.w = a[4 * q + 3];
                y.x = b[4 * q];
                y.y = b[4 * q + 1];
                y.z = b[4 * q + 2];
                y.w = b[4 * q + 3];
                rowp[q] = x;
                rowp[4 + q] = y;
            }
            __syncthreads();
            const uint64_t e0 = ((uint64_t)base + 2u * (uint64_t)wave * kWave) * 16u;
            const v4f *wstage = stage + wave * kWave * (kRow2 / 4);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                // element 256q + 4L of the wave tile: row 8q + L/8, column 4(L%8)
                const v4f x = wstage[(8 * q + (lane >> 3)) * (kRow2 / 4) + (lane & 7)];
                st_run<NTS>(out + e0, kWave * 32 * 4, (64 * q + lane) * 16, x);
            }
            __syncthreads();
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                if (e + k < n)
                    out[e + k] = a[k];
                if (e + 16 + k < n)
                    out[e + 16 + k] = b[k];
            }
        }
    }
}

template <int Mode, bool NTL, bool NTS, bool Lds>
void launch_one(uint32_t grid, uint32_t pad, hipStream_t stream, const DqWorkers &ws, uint32_t W,
                uint32_t nwords, uint64_t n, float tq, float *acc)
{
    dq_reduce_kernel<Mode, NTL, NTS, Lds>
        <<<grid, kBlockThreads, pad, stream>>>(ws, W, nwords, n, tq, acc);
}

template <int Mode>
void dispatch(const gcq_tuning &tu, uint32_t grid, hipStream_t stream, const DqWorkers &ws,
              uint32_t W, uint32_t nwords, uint64_t n, float tq, float *acc, bool two)
{
    if (two) {
        const uint32_t grid2 = grid_for((nwords + 2u * kBlockThreads - 1) / (2u * kBlockThreads),
                                        tu.dq_blocks_per_cu);
        const uint32_t pad = resident_lds_pad(kBlockWaves * kWave * kRow2 * 4, tu.dq_resident_per_cu);
        const int k2 = tu.dq_nt_loads * 2 + tu.dq_nt_stores;
        if (k2 == 3)
            dq_reduce2_kernel<Mode, true, true><<<grid2, kBlockThreads, pad, stream>>>(ws, W, nwords, n, tq, acc);
        else if (k2 == 2)
            dq_reduce2_kernel<Mode, true, false><<<grid2, kBlockThreads, pad, stream>>>(ws, W, nwords, n, tq, acc);
        else if (k2 == 1)
            dq_reduce2_kernel<Mode, false, true><<<grid2, kBlockThreads, pad, stream>>>(ws, W, nwords, n, tq, acc);
        else
            dq_reduce2_kernel<Mode, false, false><<<grid2, kBlockThreads, pad, stream>>>(ws, W, nwords, n, tq, acc);
        return;
    }
    const uint32_t pad = resident_lds_pad(tu.dq_lds_stores ? kBlockWaves * kWave * kLdsRow * 4 : 16,
                                 tu.dq_resident_per_cu);
    const int key = tu.dq_nt_loads * 4 + tu.dq_nt_stores * 2 + tu.dq_lds_stores;
    switch (key) {
    case 0: launch_one<Mode, false, false, false>(grid, pad, stream, ws, W, nwords, n, tq, acc); break;
    case 1: launch_one<Mode, false, false, true>(grid, pad, stream, ws, W, nwords, n, tq, acc); break;
    case 2: launch_one<Mode, false, true, false>(grid, pad, stream, ws, W, nwords, n, tq, acc); break;
    case 3: launch_one<Mode, false, true, true>(grid, pad, stream, ws, W, nwords, n, tq, acc); break;
    case 4: launch_one<Mode, true, false, false>(grid, pad, stream, ws, W, nwords, n, tq, acc); break;
    case 5: launch_one<Mode, true, false, true>(grid, pad, stream, ws, W, nwords, n, tq, acc); break;
    case 6: launch_one<Mode, true, true, false>(grid, pad, stream, ws, W, nwords, n, tq, acc); break;
    default: launch_one<Mode, true, true, true>(grid, pad, stream, ws, W, nwords, n, tq, acc); break;
    }
}

// Words per launch: keeps every byte offset of a word array below 2^32.
constexpr uint64_t kMaxWordsPerLaunch = (uint64_t)1 << 30;

}  // namespace

constexpr uint64_t kTwoWordsFrom = 1ull << 22;

hipError_t launch_dequant_reduce(const DqWorkers &w, uint32_t W, uint64_t n, float t, float *acc,
                                 hipStream_t stream, bool probe)
{
    const uint64_t nwords = (n + 15) >> 4;
    if (!nwords)
        return hipSuccess;
    const gcq_tuning tu = tuning();
    // t/2 and t/64 are exact (power-of-two scalings that stay normal) for
    // t >= 2^-120; smaller thresholds use the plain decode.
    const int mode = probe ? kProbe
                           : t < 0x1p-120f ? kDecodePlain
                                           : (tu.dq_fp4_decode ? kDecodeFp4 : kDecodeSdwa);
    const float tq = mode == kDecodeFp4 ? t * 0.5f : (mode == kDecodeSdwa ? t * 0x1p-6f : t);
    for (uint64_t w0 = 0; w0 < nwords; w0 += kMaxWordsPerLaunch) {
        const uint64_t cw = nwords - w0 < kMaxWordsPerLaunch ? nwords - w0 : kMaxWordsPerLaunch;
        const uint64_t cn = (n - w0 * 16) < cw * 16 ? (n - w0 * 16) : cw * 16;
        DqWorkers ws = w;
        for (uint32_t k = 0; k < W; ++k)
            ws.w[k] = w.w[k] + w0;
        const uint32_t grid =
            grid_for((cw + kBlockThreads - 1) / kBlockThreads, tu.dq_blocks_per_cu);
        // two words per thread when every word array is 8-byte aligned here:
        // by default from kTwoWordsFrom words per launch (below, the one-word
        // kernel's finer grid wins: 39 against 46 us at 1.6 M words, W = 16;
        // at 4 M words the two are level)
        bool two = tu.dq_words_per_thread == 2 ||
                   (tu.dq_words_per_thread == 0 && cw >= kTwoWordsFrom);
        for (uint32_t k = 0; k < W; ++k)
            two = two && ((uintptr_t)ws.w[k] & 7u) == 0;
        if (mode == kProbe)
            dispatch<kProbe>(tu, grid, stream, ws, W, (uint32_t)cw, cn, tq, acc + w0 * 16, two);
        else if (mode == kDecodeFp4)
            dispatch<kDecodeFp4>(tu, grid, stream, ws, W, (uint32_t)cw, cn, tq, acc + w0 * 16, two);
        else if (mode == kDecodeSdwa)
            dispatch<kDecodeSdwa>(tu, grid, stream, ws, W, (uint32_t)cw, cn, tq, acc + w0 * 16, two);
        else
            dispatch<kDecodePlain>(tu, grid, stream, ws, W, (uint32_t)cw, cn, tq, acc + w0 * 16, two);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace gcq
