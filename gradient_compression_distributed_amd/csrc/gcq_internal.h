// gcq_internal.h -- declarations shared by the kernel files and the C ABI
// (gcq_api.hip).  Not installed; the public interface is include/gcq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gcq.h"

namespace gcq {

// Launch geometry: 64-lane wavefronts in 256-thread workgroups.  A "wave
// tile" of 1024 elements (one float4 per lane in each of four 1 KiB runs)
// is the unit of the QSGD kernels; the 2-bit quantizer's tile size is a
// launch knob (gc2_tile_elems).
constexpr int kWave = 64;
constexpr int kBlockThreads = 256;
constexpr int kBlockWaves = kBlockThreads / kWave;
constexpr uint64_t kWaveElems = 1024;

// Device-side bucket descriptor of the fused multi-bucket launch.
struct Gc2Desc {
    const float *g;
    float *r;
    uint32_t *out;
    uint64_t n;
    uint64_t tile_begin;  // first block tile of this bucket in the flat tile space
    float t;
    uint32_t pad;
};

// Worker pointers of the reduce, passed by value in the kernel arguments.
struct DqWorkers {
    const uint32_t *w[GCQ_MAX_WORKERS];
};

// The K messages of qsgd_dequant_average (bucket scales and nibble words
// per worker), passed by value in the kernel arguments.
struct QsgdMsgs {
    const float *scales[GCQ_MAX_WORKERS];
    const uint32_t *nibbles[GCQ_MAX_WORKERS];
};

// Launch knobs (gcq_get_tuning / gcq_set_tuning).  They change the launch
// shape only, never a result.
gcq_tuning tuning();
void set_tuning(const gcq_tuning &t);
bool tuning_valid(const gcq_tuning &t);

// Number of compute units of the current device (cached per device).
int device_cus();

// Dynamic LDS (bytes, never touched by the kernel) that leaves room for at
// most `resident` workgroups per compute unit when each also holds
// `static_bytes` of its own: a cap on resident workgroups set through the
// LDS allocation.  0: no cap.  Fewer resident workgroups keep fewer read and
// write windows open in HBM at once, which the streaming kernels measured
// faster at some settings (the launch knobs choose).
uint32_t resident_lds_pad(uint32_t static_bytes, int resident);

// Grid size for `work_blocks` workgroups of work: all of them when
// blocks_per_cu == 0, else at most blocks_per_cu per compute unit (the
// kernel then strides); clamped to [1, 2^31 - 1].
uint32_t grid_for(uint64_t work_blocks, int blocks_per_cu);

// ---- launchers (return the hipError_t of the launch) -------------------
// Elements per workgroup tile of the 2-bit quantizer under tuning `tu`
// (the unit of Gc2Desc::tile_begin).
uint64_t gc2_tile_elems(const gcq_tuning &tu);
hipError_t launch_gc2_single(const Gc2Desc &one, hipStream_t stream);
// `tu` is the tuning the table's tile_begin values were computed with.
// tiles_per_bucket > 0 when every bucket spans exactly that many tiles
// (the kernel then finds its bucket by a division instead of a search).
hipError_t launch_gc2_table(const gcq_tuning &tu, const Gc2Desc *dev_table, uint32_t nbuckets,
                            uint64_t total_tiles, uint32_t tiles_per_bucket, hipStream_t stream);
// Copies count host descriptors into the device table with small kernels
// whose arguments carry the descriptors (kFillChunk per launch), ordered on
// `stream`; the host array is not referenced after the call returns.
constexpr uint32_t kFillChunk = 64;
hipError_t launch_gc2_table_fill(const Gc2Desc *descs, uint32_t count, Gc2Desc *dev_table,
                                 hipStream_t stream);
// CD-SGD local update (Quant = false) or update fused with the quantizer.
hipError_t launch_cdsgd(const float *g, float *r, float *w, uint32_t *out, uint64_t n, float t,
                        float eta, bool quant, hipStream_t stream);
// In place: a[0..count) -> exclusive prefix sums, a[count] = the total.
hipError_t launch_exclusive_scan_u64(uint64_t *a, uint64_t count, hipStream_t stream);
// Elias-omega coding of QSGD buckets (d a multiple of 8, at most 2048).
uint64_t elias_max_words(uint64_t n, uint32_t d);
hipError_t launch_elias_encode(const float *norms, const uint32_t *nibbles, uint64_t n, uint32_t d,
                               uint64_t *offs, uint32_t *out, uint64_t cap, hipStream_t stream);
hipError_t launch_elias_decode(const uint32_t *in, const uint64_t *offs, uint64_t n, uint32_t d,
                               uint64_t in_words, float *norms, uint32_t *nibbles,
                               hipStream_t stream);
// SAPS: T = ceil(2^24 / c), the keep threshold of the 24-bit draw (u c < 1).
uint32_t saps_threshold(float c);
hipError_t launch_saps_mask(uint64_t n, float c, uint64_t seed, uint32_t *mask, uint64_t *offs,
                            hipStream_t stream);
hipError_t launch_saps_apply(float *x, uint64_t n, const uint32_t *mask, const uint64_t *offs,
                             float *values, uint64_t cap, bool merge, hipStream_t stream);
// probe: the same kernel and launch with the decode replaced by an XOR of
// the words (gcq_probe_reduce).
hipError_t launch_dequant_reduce(const DqWorkers &w, uint32_t W, uint64_t n, float t,
                                 float *acc, hipStream_t stream, bool probe = false);
// The streaming probe (gcq_probe_stream).
hipError_t launch_probe_stream(const float *a, const float *b, float *c, uint32_t *words,
                               uint64_t n, hipStream_t stream);
// maxnorm: bucket scale = largest magnitude (else the L2 norm).
hipError_t launch_qsgd_quantize(const float *g, uint64_t n, uint32_t d, uint32_t s, uint64_t seed,
                                float *norms, uint32_t *nibbles, bool maxnorm, hipStream_t stream);
hipError_t launch_qsgd_average(const QsgdMsgs &ms, uint32_t K, uint64_t n, uint32_t d, uint32_t s,
                               float *out, hipStream_t stream);
hipError_t launch_qsgd_dequant(const float *norms, const uint32_t *nibbles, uint64_t n, uint32_t d,
                               uint32_t s, float *out, hipStream_t stream);

}  // namespace gcq
