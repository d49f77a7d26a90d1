// probe.hip -- a streaming probe for measurement (gcq_probe_stream): the
// 2-bit quantizer's HBM access pattern with none of its arithmetic.  Same
// geometry as the quantizer's default launch: 256-thread workgroups, one
// tile of 1024 elements each, lane L of a wavefront loading one float4 per
// input stream at 4L of its 256-element tile (non-temporal), storing one
// float4 of the output (non-temporal) and, for lanes 0..15, one 32-bit word
// of the packed stream (plain store), so each wavefront writes a 64-byte
// run of words as the quantizer does.  c = a XOR b, bit for bit (c = a with
// one input); word 16k + L of the stream holds the bits of c[256k + 4L].
// Timed beside the hot-path kernels, it is their practical ceiling.
#include "gcq_device.h"
#include "gcq_internal.h"

namespace gcq {

namespace {

using dev::v4f;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <bool TwoInputs, bool Words>
__global__ __launch_bounds__(kBlockThreads) void probe_stream_kernel(const float *__restrict__ a,
                                                                     const float *__restrict__ b,
                                                                     float *__restrict__ c,
                                                                     uint32_t *__restrict__ words)
{
    const uint32_t lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const uint64_t e0 = (uint64_t)blockIdx.x * 1024u + (uint64_t)wave * 256u;
    const GCQ_GLOBAL v4u *a4 = (const GCQ_GLOBAL v4u *)(a + e0);
    v4u x = __builtin_nontemporal_load(a4 + lane);
    if constexpr (TwoInputs) {
        const GCQ_GLOBAL v4u *b4 = (const GCQ_GLOBAL v4u *)(b + e0);
        x ^= __builtin_nontemporal_load(b4 + lane);
    }
    __builtin_nontemporal_store(x, (GCQ_GLOBAL v4u *)(c + e0) + lane);
    if constexpr (Words) {
        if (lane < 16)
            ((GCQ_GLOBAL uint32_t *)words)[(e0 >> 4) + lane] = x.x;
    }
}

}  // namespace

hipError_t launch_probe_stream(const float *a, const float *b, float *c, uint32_t *words,
                               uint64_t n, hipStream_t stream)
{
    const uint64_t tiles = n / 1024u;
    if (!tiles)
        return hipSuccess;
    for (uint64_t t0 = 0; t0 < tiles; t0 += 0x7FFFFFFFu) {
        const uint32_t g = (uint32_t)(tiles - t0 < 0x7FFFFFFFu ? tiles - t0 : 0x7FFFFFFFu);
        const uint64_t e = t0 * 1024u;
        const float *bb = b ? b + e : nullptr;
        uint32_t *ww = words ? words + e / 16 : nullptr;
        if (b && words)
            probe_stream_kernel<true, true><<<g, kBlockThreads, 0, stream>>>(a + e, bb, c + e, ww);
        else if (b)
            probe_stream_kernel<true, false><<<g, kBlockThreads, 0, stream>>>(a + e, bb, c + e, ww);
        else if (words)
            probe_stream_kernel<false, true><<<g, kBlockThreads, 0, stream>>>(a + e, bb, c + e, ww);
        else
            probe_stream_kernel<false, false><<<g, kBlockThreads, 0, stream>>>(a + e, bb, c + e, ww);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

}  // namespace gcq
