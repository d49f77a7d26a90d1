// gcq_internal.h -- declarations shared by the kernels (gcq_kernels.hip) and
// the C ABI (gcq_api.hip).  Not installed; the public interface is
// include/gcq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gcq {

// Geometry of the 2-bit quantizer.  A wavefront (64 lanes) owns a "wave
// tile" of 1024 consecutive elements = 64 packed words, one word per lane
// on the way out; a 256-thread workgroup owns a block tile of 4 wave tiles.
constexpr int kWave = 64;
constexpr int kBlockThreads = 256;
constexpr int kBlockWaves = kBlockThreads / kWave;
constexpr uint64_t kWaveElems = 1024;
constexpr uint64_t kTileElems = kWaveElems * kBlockWaves;

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
    const uint32_t *w[64];
};

// Launch knobs (gcq_set_tuning in include/gcq.h); initial values from the
// environment.  They change the launch shape only, never a result.
struct Tuning {
    int gc2_layout;        // 0: quad-assembled coalesced words, 1: per-lane runs
    int nt;                // non-temporal hints on streamed data
    int blocks_per_cu;     // 2-bit quantizer workgroups per CU (0: one tile each)
    int dq_blocks_per_cu;  // reduce workgroups per CU (0: one word per thread)
};
Tuning tuning();
void set_tuning(const Tuning &t);

// Number of compute units of the current device (cached per device).
int device_cus();

// ---- launchers (return a hipError_t of the launch) --------------------
hipError_t launch_gc2_single(const Gc2Desc &one, hipStream_t stream);
hipError_t launch_gc2_table(const Gc2Desc *dev_table, uint32_t nbuckets, uint64_t total_tiles,
                            hipStream_t stream);
hipError_t launch_dequant_reduce(const DqWorkers &w, uint32_t W, uint64_t n, float t,
                                 float *acc, hipStream_t stream);
hipError_t launch_qsgd_quantize(const float *g, uint64_t n, uint32_t d, uint32_t s, uint64_t seed,
                                float *norms, uint32_t *nibbles, hipStream_t stream);
hipError_t launch_qsgd_dequant(const float *norms, const uint32_t *nibbles, uint64_t n, uint32_t d,
                               uint32_t s, float *out, hipStream_t stream);

}  // namespace gcq
