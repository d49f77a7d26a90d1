// gcq_runtime.hip -- host-side runtime state shared by the launchers:
// launch knobs (defaults measured on MI355X, overridable from the
// environment) and the per-device compute-unit count.
#include <stdlib.h>

#include <algorithm>
#include <mutex>

#include "gcq_device.h"
#include "gcq_internal.h"

namespace gcq {

namespace {

std::mutex g_mu;
bool g_init = false;
gcq_tuning g_tuning;

int env_int(const char *name, int dflt)
{
    const char *v = getenv(name);
    return (v && *v) ? atoi(v) : dflt;
}

int env_flag(const char *name, int dflt) { return env_int(name, dflt) ? 1 : 0; }

bool resident_ok(int v) { return v == 0 || (v >= 2 && v <= 8); }

int env_count(const char *name, int dflt)
{
    return std::max(0, std::min(1024, env_int(name, dflt)));
}

void init_locked()
{
    if (g_init)
        return;
    // Defaults: the fastest settings measured on MI355X at 2^30 elements.
    g_tuning.gc2_unroll = env_int("GCQ_GC2_UNROLL", 1);
    if (g_tuning.gc2_unroll != 2 && g_tuning.gc2_unroll != 4)
        g_tuning.gc2_unroll = 1;
    g_tuning.gc2_nt = std::max(0, std::min(15, env_int("GCQ_GC2_NT", 7)));
    g_tuning.gc2_blocks_per_cu = env_count("GCQ_GC2_BLOCKS_PER_CU", 0);
    g_tuning.dq_nt_loads = env_flag("GCQ_DQ_NT_LOADS", 1);
    g_tuning.dq_nt_stores = env_flag("GCQ_DQ_NT_STORES", 1);
    g_tuning.dq_lds_stores = env_flag("GCQ_DQ_LDS_STORES", 1);
    g_tuning.dq_blocks_per_cu = env_count("GCQ_DQ_BLOCKS_PER_CU", 0);
    g_tuning.dq_fp4_decode = env_flag("GCQ_DQ_FP4_DECODE", 1);
    g_tuning.qsgd_nt = env_flag("GCQ_QSGD_NT", 1);
    g_tuning.qsgd_rcp = env_flag("GCQ_QSGD_RCP", 1);
    g_tuning.qsgd_dequant_nt = env_flag("GCQ_QSGD_DEQUANT_NT", 1);
    g_tuning.qsgd_blocks_per_cu = env_count("GCQ_QSGD_BLOCKS_PER_CU", 0);
    g_tuning.qsgd_dequant_blocks_per_cu = env_count("GCQ_QSGD_DEQUANT_BLOCKS_PER_CU", 0);
    g_tuning.qsgd_buckets_per_wave = env_int("GCQ_QSGD_BUCKETS_PER_WAVE", 0);
    if (g_tuning.qsgd_buckets_per_wave != 1 && g_tuning.qsgd_buckets_per_wave != 2 &&
        g_tuning.qsgd_buckets_per_wave != 4)
        g_tuning.qsgd_buckets_per_wave = 0;
    {
        const int wpt = env_int("GCQ_DQ_WORDS_PER_THREAD", 0);
        g_tuning.dq_words_per_thread = wpt == 1 || wpt == 2 ? wpt : 0;
    }
    g_tuning.dq_resident_per_cu = env_int("GCQ_DQ_RESIDENT_PER_CU", 3);
    if (!resident_ok(g_tuning.dq_resident_per_cu))
        g_tuning.dq_resident_per_cu = 3;
    g_tuning.gc2_resident_per_cu = env_int("GCQ_GC2_RESIDENT_PER_CU", 0);
    if (!resident_ok(g_tuning.gc2_resident_per_cu))
        g_tuning.gc2_resident_per_cu = 0;
    g_tuning.cdsgd_resident_per_cu = env_int("GCQ_CDSGD_RESIDENT_PER_CU", 5);
    if (!resident_ok(g_tuning.cdsgd_resident_per_cu))
        g_tuning.cdsgd_resident_per_cu = 5;
    g_tuning.qsgd_avg_resident_per_cu = env_int("GCQ_QSGD_AVG_RESIDENT_PER_CU", 0);
    if (!resident_ok(g_tuning.qsgd_avg_resident_per_cu))
        g_tuning.qsgd_avg_resident_per_cu = 0;
    g_init = true;
}

bool flag_ok(int v) { return v == 0 || v == 1; }
bool count_ok(int v) { return v >= 0 && v <= 1024; }

}  // namespace

gcq_tuning tuning()
{
    std::lock_guard<std::mutex> lock(g_mu);
    init_locked();
    return g_tuning;
}

bool tuning_valid(const gcq_tuning &t)
{
    return (t.gc2_unroll == 1 || t.gc2_unroll == 2 || t.gc2_unroll == 4) && t.gc2_nt >= 0 && t.gc2_nt <= 15 && count_ok(t.gc2_blocks_per_cu) &&
           flag_ok(t.dq_nt_loads) && flag_ok(t.dq_nt_stores) && flag_ok(t.dq_lds_stores) &&
           count_ok(t.dq_blocks_per_cu) && flag_ok(t.dq_fp4_decode) && flag_ok(t.qsgd_nt) &&
           flag_ok(t.qsgd_rcp) && flag_ok(t.qsgd_dequant_nt) && count_ok(t.qsgd_blocks_per_cu) &&
           count_ok(t.qsgd_dequant_blocks_per_cu) &&
           (t.qsgd_buckets_per_wave == 0 || t.qsgd_buckets_per_wave == 1 ||
            t.qsgd_buckets_per_wave == 2 || t.qsgd_buckets_per_wave == 4) &&
           (t.dq_words_per_thread >= 0 && t.dq_words_per_thread <= 2) &&
           resident_ok(t.dq_resident_per_cu) && resident_ok(t.gc2_resident_per_cu) &&
           resident_ok(t.cdsgd_resident_per_cu) && resident_ok(t.qsgd_avg_resident_per_cu);
}

void set_tuning(const gcq_tuning &t)
{
    std::lock_guard<std::mutex> lock(g_mu);
    init_locked();
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

// Largest LDS allocation of one workgroup on the current device (cached).
uint32_t device_max_lds()
{
    static std::mutex mu;
    static uint32_t cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 64u * 1024u;
    std::lock_guard<std::mutex> lock(mu);
    if (!cache[dev]) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            v <= 0)
            v = 64 * 1024;
        cache[dev] = (uint32_t)v;
    }
    return cache[dev];
}

uint32_t resident_lds_pad(uint32_t static_bytes, int resident)
{
    if (resident <= 0)
        return 0;
    const uint32_t per = dev::kLdsBytesPerCu / (uint32_t)resident - 1024u;
    const uint32_t cap = device_max_lds();
    const uint32_t want = per < cap ? per : cap;
    return want > static_bytes ? want - static_bytes : 0u;
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

}  // namespace gcq
