// gcq_api.hip -- the C ABI of libgcq.so (declared and documented in
// include/gcq.h): host-side argument checks, launch geometry, and the
// stream-ordered device table of the fused multi-bucket launch.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "gcq.h"
#include "gcq_internal.h"

namespace {

using gcq::Gc2Desc;

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
    uintptr_t lo, hi;
    bool writable;
};

Range range(const void *p, size_t bytes, bool writable)
{
    return Range{(uintptr_t)p, (uintptr_t)p + bytes, writable};
}

// True when a writable range intersects any other range.  Sorted sweep:
// a pair (A before B in start order) overlaps iff B.lo < A.hi, so it is
// enough to track the largest end so far among writable and among all
// ranges.  Read-only ranges may overlap one another.
bool any_write_overlap(Range *first, Range *last)
{
    std::sort(first, last, [](const Range &a, const Range &b) { return a.lo < b.lo; });
    uintptr_t end_all = 0, end_w = 0;
    for (const Range *p = first; p != last; ++p) {
        const Range &r = *p;
        if (r.hi == r.lo)
            continue;
        if (r.lo < end_w || (r.writable && r.lo < end_all))
            return true;
        end_all = std::max(end_all, r.hi);
        if (r.writable)
            end_w = std::max(end_w, r.hi);
    }
    return false;
}

bool any_write_overlap(std::vector<Range> &rs) { return any_write_overlap(rs.data(), rs.data() + rs.size()); }

// A fixed array that check_gc2 appends to (for the path that allocates
// nothing, not even host memory).
struct RangeArray {
    Range *p;
    size_t n;
    void push_back(const Range &r) { p[n++] = r; }
};

bool valid_threshold(float t) { return isfinite(t) && t > 0.0f; }

bool valid_rate(float eta) { return isfinite(eta) && eta >= 0.0f; }

// Largest element count of a call: with at most 8 bytes per element every
// byte count stays below 2^63, and with device addresses below 2^48 no
// range's end address wraps.
constexpr size_t kMaxElems = GCQ_MAX_ELEMS;

template <class Ranges>
int check_gc2(const float *g, const float *r, size_t n, float t, const uint32_t *out,
              Ranges *ranges)
{
    if (!valid_threshold(t))
        return GCQ_ERR_THRESHOLD;
    if (n > kMaxElems)
        return GCQ_ERR_PARAM;
    if (n == 0)
        return GCQ_OK;
    if (!g || !r || !out)
        return GCQ_ERR_NULL;
    if (!aligned(g, 16) || !aligned(r, 16) || !aligned(out, 4))
        return GCQ_ERR_ALIGN;
    ranges->push_back(range(g, n * 4, false));
    ranges->push_back(range(r, n * 4, true));
    ranges->push_back(range(out, gc2_packed_words(n) * 4, true));
    return GCQ_OK;
}

int launch_status(hipError_t e)
{
    if (e == hipSuccess)
        return GCQ_OK;
    if (e == hipErrorOutOfMemory)
        return GCQ_ERR_NOMEM;
    return GCQ_ERR_LAUNCH;
}

// Device tables of the fused launch: per device a cache of slots, each a
// device buffer, a host record of the descriptors it holds (to recognise a
// repeated bucket list) and an event recorded after the last kernel that
// read it.  A call whose descriptors match a slot's reuses that slot's
// table.  A new table goes to the least recently used slot.  Either way the
// caller's stream first waits, on the device, for the slot's event, so a
// table is read only after its fill and rewritten only after its last
// reader, whatever streams they ran on; the host never waits.  The fill is a
// kernel whose arguments carry the descriptors (nothing is staged in host
// memory).  All slots are allocated together on the first call; a call with
// more buckets than they hold grows them, which is the one case where the
// host waits (for the kernels still reading the old buffers) and device
// memory is allocated.
constexpr int kRing = 8;
constexpr int kMaxDevices = 64;

struct Slot {
    std::vector<Gc2Desc> descs;  // the table it holds (empty: none)
    Gc2Desc *dev = nullptr;
    size_t cap = 0;
    uint64_t used = 0;           // call number of its last use
    hipEvent_t ev = nullptr;
    bool pending = false;        // ev recorded after a kernel that read the table
};

struct DeviceRing {
    std::mutex mu;
    Slot slots[kRing];
    uint64_t calls = 0;
};

DeviceRing g_rings[kMaxDevices];

// A slot able to hold nb descriptors.  Growing frees the old buffer, so the
// host first waits for the slot's last reader.
int ensure_capacity(Slot &s, size_t nb)
{
    if (!s.ev && hipEventCreateWithFlags(&s.ev, hipEventDisableTiming) != hipSuccess)
        return GCQ_ERR_NOMEM;
    if (s.cap >= nb)
        return GCQ_OK;
    if (s.pending) {
        if (hipEventSynchronize(s.ev) != hipSuccess)
            return GCQ_ERR_LAUNCH;
        s.pending = false;
    }
    size_t cap = std::max<size_t>(nb, 2 * s.cap);
    if (s.dev)
        (void)hipFree(s.dev);
    s.dev = nullptr;
    s.cap = 0;
    s.descs.clear();
    if (hipMalloc((void **)&s.dev, cap * sizeof(Gc2Desc)) != hipSuccess)
        return GCQ_ERR_NOMEM;
    s.cap = cap;
    return GCQ_OK;
}

// The device table of gc2_quantize_buckets_noalloc: a fixed array of the
// library, one copy per device, held until the process ends.  Host code
// never passes `scratch` itself to a kernel (in host code the name stands
// for a host-side shadow, not the device copy); it uses the device address
// hipGetSymbolAddress returns for the current device, kept per device.
static_assert(sizeof(Gc2Desc) == 48, "the header states 48 bytes per descriptor");
static __device__ __align__(256) Gc2Desc scratch[GC2_NOALLOC_MAX_BUCKETS];

std::mutex g_scratch_mu;
Gc2Desc *g_scratch_ptr[kMaxDevices];
// Host-side working arrays of the no-alloc call (so it allocates no host
// memory either), used under g_scratch_mu.
Range g_na_ranges[3 * GC2_NOALLOC_MAX_BUCKETS];
Gc2Desc g_na_descs[GC2_NOALLOC_MAX_BUCKETS];

// The current device's copy of `scratch` (looked up once per device).
int scratch_table(int dev, Gc2Desc **out)
{
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return GCQ_ERR_LAUNCH;
        g_scratch_ptr[dev] = (Gc2Desc *)p;
    }
    *out = g_scratch_ptr[dev];
    return GCQ_OK;
}

// Checks every bucket of a fused call and builds its device descriptors:
// ranges receives up to 3 per bucket, descs one per bucket.  tpb is the
// tile count shared by every bucket (0 if they differ): the kernel then
// finds a tile's bucket by one division.
int prepare_buckets(const gc2_bucket *buckets, uint32_t num_buckets, const gcq_tuning &tu,
                    RangeArray *ranges, Gc2Desc *descs, uint64_t *total_tiles, uint64_t *tpb)
{
    uint64_t tiles_total = 0, total_elems = 0;
    const uint64_t te = gcq::gc2_tile_elems(tu);
    uint64_t same = (buckets[0].n + te - 1) / te;
    for (uint32_t b = 0; b < num_buckets; ++b) {
        const gc2_bucket &k = buckets[b];
        int st = check_gc2(k.g, k.r, k.n, k.t, k.out_words, ranges);
        if (st != GCQ_OK)
            return st;
        total_elems += k.n;   // each term <= 2^60, checked as it grows: no wrap
        if (total_elems > kMaxElems)
            return GCQ_ERR_PARAM;
        const uint64_t tiles = (k.n + te - 1) / te;
        if (tiles != same)
            same = 0;
        descs[b] = Gc2Desc{k.g, k.r, k.out_words, (uint64_t)k.n, tiles_total, k.t, 0};
        tiles_total += tiles;
    }
    if (same > 0xFFFFFFFFu)
        same = 0;
    if (any_write_overlap(ranges->p, ranges->p + ranges->n))
        return GCQ_ERR_OVERLAP;
    *total_tiles = tiles_total;
    *tpb = same;
    return GCQ_OK;
}

}  // namespace

extern "C" {

size_t gc2_packed_words(size_t n) { return n / 16 + (n % 16 != 0); }

size_t qsgd_num_buckets(size_t n, uint32_t d) { return d ? n / d + (n % d != 0) : 0; }

size_t qsgd_nibble_words(size_t n) { return n / 8 + (n % 8 != 0); }

const char *gcq_status_string(int status)
{
    switch (status) {
    case GCQ_OK: return "ok";
    case GCQ_ERR_NULL: return "null pointer with n > 0";
    case GCQ_ERR_THRESHOLD: return "threshold must be finite and > 0";
    case GCQ_ERR_PARAM: return "parameter out of range";
    case GCQ_ERR_ALIGN: return "pointer misaligned (float arrays 16 B, word arrays 4 B)";
    case GCQ_ERR_OVERLAP: return "an output range overlaps another operand";
    case GCQ_ERR_LAUNCH: return "HIP launch or copy failed";
    case GCQ_ERR_NOMEM: return "could not allocate a library buffer";
    default: return "unknown status";
    }
}

int gcq_get_tuning(gcq_tuning *out)
{
    if (!out)
        return GCQ_ERR_NULL;
    *out = gcq::tuning();
    return GCQ_OK;
}

int gcq_set_tuning(const gcq_tuning *t)
{
    if (!t)
        return GCQ_ERR_NULL;
    if (!gcq::tuning_valid(*t))
        return GCQ_ERR_PARAM;
    gcq::set_tuning(*t);
    return GCQ_OK;
}

int gc2_quantize(const float *g, float *r, size_t n, float t, uint32_t *out_words, void *stream)
{
    std::vector<Range> ranges;
    int st = check_gc2(g, r, n, t, out_words, &ranges);
    if (st != GCQ_OK || n == 0)
        return st;
    if (any_write_overlap(ranges))
        return GCQ_ERR_OVERLAP;
    Gc2Desc d = {g, r, out_words, (uint64_t)n, 0, t, 0};
    return launch_status(gcq::launch_gc2_single(d, (hipStream_t)stream));
}

int gc2_quantize_buckets(const gc2_bucket *buckets, uint32_t num_buckets, void *stream)
{
    if (num_buckets == 0)
        return GCQ_OK;
    if (!buckets)
        return GCQ_ERR_NULL;
    if (num_buckets > 0x7FFFFFFFu)
        return GCQ_ERR_PARAM;
    // host working arrays sized by the caller's count: a failed allocation
    // is reported, never thrown across the C boundary
    std::vector<Range> ranges;
    std::vector<Gc2Desc> descs;
    try {
        ranges.resize(3 * (size_t)num_buckets);
        descs.resize(num_buckets);
    } catch (const std::bad_alloc &) {
        return GCQ_ERR_NOMEM;
    }
    const gcq_tuning tu = gcq::tuning();
    RangeArray ra{ranges.data(), 0};
    uint64_t total_tiles = 0, tpb = 0;
    int st = prepare_buckets(buckets, num_buckets, tu, &ra, descs.data(), &total_tiles, &tpb);
    if (st != GCQ_OK || total_tiles == 0)
        return st;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return GCQ_ERR_LAUNCH;
    const size_t bytes = num_buckets * sizeof(Gc2Desc);
    hipStream_t hs = (hipStream_t)stream;
    DeviceRing &ring = g_rings[dev];
    std::lock_guard<std::mutex> lock(ring.mu);
    ++ring.calls;
    // The same buckets as an earlier call (the usual case: fusion buckets are
    // fixed across training steps, possibly a few alternating sets): the
    // table already on the device is reused as is.
    Slot *sp = nullptr;
    for (Slot &c : ring.slots) {
        if (c.descs.size() == num_buckets && memcmp(c.descs.data(), descs.data(), bytes) == 0) {
            sp = &c;
            break;
        }
    }
    bool fill = false;
    if (!sp) {
        Slot *lru = &ring.slots[0];
        for (Slot &c : ring.slots)
            if (c.used < lru->used)
                lru = &c;
        if (lru->cap < num_buckets) {
            // every slot grows with it, so later new tables of this size
            // allocate nothing
            for (Slot &c : ring.slots) {
                int st = ensure_capacity(c, num_buckets);
                if (st != GCQ_OK)
                    return st;
            }
        }
        sp = lru;
        sp->descs.clear();
        fill = true;
    }
    Slot &s = *sp;
    if (s.pending && hipStreamWaitEvent(hs, s.ev, 0) != hipSuccess)
        return GCQ_ERR_LAUNCH;
    if (fill) {
        hipError_t e = gcq::launch_gc2_table_fill(descs.data(), num_buckets, s.dev, hs);
        if (e != hipSuccess)
            return launch_status(e);
        s.descs = std::move(descs);
    }
    s.used = ring.calls;
    hipError_t e = gcq::launch_gc2_table(tu, s.dev, num_buckets, total_tiles, (uint32_t)tpb, hs);
    if (e != hipSuccess)
        return launch_status(e);
    if (hipEventRecord(s.ev, hs) != hipSuccess)
        return GCQ_ERR_LAUNCH;
    s.pending = true;
    return GCQ_OK;
}

int gc2_quantize_buckets_noalloc(const gc2_bucket *buckets, uint32_t num_buckets, void *stream)
{
    if (num_buckets == 0)
        return GCQ_OK;
    if (!buckets)
        return GCQ_ERR_NULL;
    if (num_buckets > GC2_NOALLOC_MAX_BUCKETS)
        return GCQ_ERR_PARAM;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    const gcq_tuning tu = gcq::tuning();
    RangeArray ra{g_na_ranges, 0};
    uint64_t total_tiles = 0, tpb = 0;
    int st = prepare_buckets(buckets, num_buckets, tu, &ra, g_na_descs, &total_tiles, &tpb);
    if (st != GCQ_OK || total_tiles == 0)
        return st;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return GCQ_ERR_LAUNCH;
    Gc2Desc *table = nullptr;
    st = scratch_table(dev, &table);
    if (st != GCQ_OK)
        return st;
    hipStream_t hs = (hipStream_t)stream;
    hipError_t e = gcq::launch_gc2_table_fill(g_na_descs, num_buckets, table, hs);
    if (e != hipSuccess)
        return launch_status(e);
    return launch_status(
        gcq::launch_gc2_table(tu, table, num_buckets, total_tiles, (uint32_t)tpb, hs));
}

int cdsgd_update_quantize(const float *g, float *r, float *w_loc, size_t n, float t, float eta,
                          uint32_t *out_words, void *stream)
{
    std::vector<Range> ranges;
    int st = check_gc2(g, r, n, t, out_words, &ranges);
    if (st != GCQ_OK)
        return st;
    if (!valid_rate(eta))
        return GCQ_ERR_PARAM;
    if (n == 0)
        return GCQ_OK;
    if (!w_loc)
        return GCQ_ERR_NULL;
    if (!aligned(w_loc, 16))
        return GCQ_ERR_ALIGN;
    ranges.push_back(range(w_loc, n * 4, true));
    if (any_write_overlap(ranges))
        return GCQ_ERR_OVERLAP;
    return launch_status(
        gcq::launch_cdsgd(g, r, w_loc, out_words, n, t, eta, true, (hipStream_t)stream));
}

int cdsgd_local_update(const float *g, float *w_loc, size_t n, float eta, void *stream)
{
    if (!valid_rate(eta) || n > kMaxElems)
        return GCQ_ERR_PARAM;
    if (n == 0)
        return GCQ_OK;
    if (!g || !w_loc)
        return GCQ_ERR_NULL;
    if (!aligned(g, 16) || !aligned(w_loc, 16))
        return GCQ_ERR_ALIGN;
    std::vector<Range> ranges = {range(g, n * 4, false), range(w_loc, n * 4, true)};
    if (any_write_overlap(ranges))
        return GCQ_ERR_OVERLAP;
    return launch_status(gcq::launch_cdsgd(g, nullptr, w_loc, nullptr, n, 1.0f, eta, false,
                                           (hipStream_t)stream));
}

namespace {

// The reduce's checks and launch; probe = true runs gcq_probe_reduce.
int dequant_reduce(const uint32_t *const *words, uint32_t W, size_t n, float t, float *acc,
                   void *stream, bool probe)
{
    if (W == 0 || W > GCQ_MAX_WORKERS)
        return GCQ_ERR_PARAM;
    if (!valid_threshold(t))
        return GCQ_ERR_THRESHOLD;
    if (n > kMaxElems)
        return GCQ_ERR_PARAM;
    if (n == 0)
        return GCQ_OK;
    if (!words || !acc)
        return GCQ_ERR_NULL;
    gcq::DqWorkers ws;
    memset(&ws, 0, sizeof ws);
    std::vector<Range> ranges;
    const size_t wbytes = gc2_packed_words(n) * 4;
    for (uint32_t w = 0; w < W; ++w) {
        if (!words[w])
            return GCQ_ERR_NULL;
        if (!aligned(words[w], 4))
            return GCQ_ERR_ALIGN;
        ws.w[w] = words[w];
        ranges.push_back(range(words[w], wbytes, false));
    }
    if (!aligned(acc, 16))
        return GCQ_ERR_ALIGN;
    ranges.push_back(range(acc, n * 4, true));
    if (any_write_overlap(ranges))
        return GCQ_ERR_OVERLAP;
    return launch_status(gcq::launch_dequant_reduce(ws, W, n, t, acc, (hipStream_t)stream, probe));
}

}  // namespace

int gc2_dequant_reduce(const uint32_t *const *words, uint32_t W, size_t n, float t, float *acc,
                       void *stream)
{
    return dequant_reduce(words, W, n, t, acc, stream, false);
}

int gcq_probe_reduce(const uint32_t *const *words, uint32_t W, size_t n, float *acc, void *stream)
{
    return dequant_reduce(words, W, n, 1.0f, acc, stream, true);
}

int gcq_probe_stream(const float *a, const float *b, float *c, uint32_t *words, size_t n,
                     void *stream)
{
    if (n > kMaxElems || n % 1024 != 0)
        return GCQ_ERR_PARAM;
    if (n == 0)
        return GCQ_OK;
    if (!a || !c)
        return GCQ_ERR_NULL;
    if (!aligned(a, 16) || !aligned(c, 16) || (b && !aligned(b, 16)) || (words && !aligned(words, 4)))
        return GCQ_ERR_ALIGN;
    std::vector<Range> ranges;
    ranges.push_back(range(a, n * 4, false));
    if (b && b != c)   // c may be b itself: in place, as the quantizer updates r
        ranges.push_back(range(b, n * 4, false));
    ranges.push_back(range(c, n * 4, true));
    if (words)
        ranges.push_back(range(words, n / 16 * 4, true));
    if (any_write_overlap(ranges))
        return GCQ_ERR_OVERLAP;
    return launch_status(gcq::launch_probe_stream(a, b, c, words, n, (hipStream_t)stream));
}

static int qsgd_quantize_impl(const float *g, size_t n, uint32_t d, uint32_t s, uint64_t seed,
                              float *norms, uint32_t *nibbles, bool maxnorm, void *stream)
{
    if (d == 0 || s < 1 || s > 7 || n > kMaxElems)
        return GCQ_ERR_PARAM;
    if (n == 0)
        return GCQ_OK;
    if (!g || !norms || !nibbles)
        return GCQ_ERR_NULL;
    if (!aligned(g, 16) || !aligned(norms, 4) || !aligned(nibbles, 4))
        return GCQ_ERR_ALIGN;
    std::vector<Range> ranges = {range(g, n * 4, false),
                                 range(norms, qsgd_num_buckets(n, d) * 4, true),
                                 range(nibbles, qsgd_nibble_words(n) * 4, true)};
    if (any_write_overlap(ranges))
        return GCQ_ERR_OVERLAP;
    return launch_status(gcq::launch_qsgd_quantize(g, n, d, s, seed, norms, nibbles, maxnorm,
                                                   (hipStream_t)stream));
}

int qsgd_quantize(const float *g, size_t n, uint32_t d, uint32_t s, uint64_t seed, float *norms,
                  uint32_t *nibbles, void *stream)
{
    return qsgd_quantize_impl(g, n, d, s, seed, norms, nibbles, false, stream);
}

int qsgd_quantize_maxnorm(const float *g, size_t n, uint32_t d, uint32_t s, uint64_t seed,
                          float *scales, uint32_t *nibbles, void *stream)
{
    return qsgd_quantize_impl(g, n, d, s, seed, scales, nibbles, true, stream);
}

int qsgd_dequant(const float *norms, const uint32_t *nibbles, size_t n, uint32_t d, uint32_t s,
                 float *out, void *stream)
{
    if (d == 0 || s < 1 || s > 7 || n > kMaxElems)
        return GCQ_ERR_PARAM;
    if (n == 0)
        return GCQ_OK;
    if (!norms || !nibbles || !out)
        return GCQ_ERR_NULL;
    if (!aligned(norms, 4) || !aligned(nibbles, 4) || !aligned(out, 16))
        return GCQ_ERR_ALIGN;
    std::vector<Range> ranges = {range(norms, qsgd_num_buckets(n, d) * 4, false),
                                 range(nibbles, qsgd_nibble_words(n) * 4, false),
                                 range(out, n * 4, true)};
    if (any_write_overlap(ranges))
        return GCQ_ERR_OVERLAP;
    return launch_status(
        gcq::launch_qsgd_dequant(norms, nibbles, n, d, s, out, (hipStream_t)stream));
}

int qsgd_dequant_average(const float *const *scales, const uint32_t *const *nibbles, uint32_t K,
                         size_t n, uint32_t d, uint32_t s, float *out, void *stream)
{
    if (K == 0 || K > GCQ_MAX_WORKERS || d == 0 || s < 1 || s > 7 || n > kMaxElems)
        return GCQ_ERR_PARAM;
    if (n == 0)
        return GCQ_OK;
    if (!scales || !nibbles || !out)
        return GCQ_ERR_NULL;
    if (!aligned(out, 16))
        return GCQ_ERR_ALIGN;
    gcq::QsgdMsgs ms;
    memset(&ms, 0, sizeof ms);
    std::vector<Range> ranges = {range(out, n * 4, true)};
    for (uint32_t l = 0; l < K; ++l) {
        if (!scales[l] || !nibbles[l])
            return GCQ_ERR_NULL;
        if (!aligned(scales[l], 4) || !aligned(nibbles[l], 4))
            return GCQ_ERR_ALIGN;
        ms.scales[l] = scales[l];
        ms.nibbles[l] = nibbles[l];
        ranges.push_back(range(scales[l], qsgd_num_buckets(n, d) * 4, false));
        ranges.push_back(range(nibbles[l], qsgd_nibble_words(n) * 4, false));
    }
    if (any_write_overlap(ranges))
        return GCQ_ERR_OVERLAP;
    return launch_status(
        gcq::launch_qsgd_average(ms, K, n, d, s, out, (hipStream_t)stream));
}

static bool elias_d_ok(uint32_t d) { return d >= 8 && d <= 2048 && d % 8 == 0; }

size_t qsgd_elias_max_words(size_t n, uint32_t d)
{
    return elias_d_ok(d) && n <= kMaxElems ? (size_t)gcq::elias_max_words(n, d) : 0;
}

int qsgd_elias_encode(const float *norms, const uint32_t *nibbles, size_t n, uint32_t d,
                      uint64_t *bit_offsets, uint32_t *out_words, size_t capacity_words,
                      void *stream)
{
    if (!elias_d_ok(d) || n > kMaxElems || capacity_words > kMaxElems)
        return GCQ_ERR_PARAM;
    if (!bit_offsets || (n && (!norms || !nibbles || (capacity_words && !out_words))))
        return GCQ_ERR_NULL;
    if (!aligned(norms, 4) || !aligned(nibbles, 4) || !aligned(bit_offsets, 8) ||
        !aligned(out_words, 4))
        return GCQ_ERR_ALIGN;
    const size_t nb = qsgd_num_buckets(n, d);
    std::vector<Range> ranges = {range(norms, nb * 4, false),
                                 range(nibbles, qsgd_nibble_words(n) * 4, false),
                                 range(bit_offsets, (nb + 1) * 8, true),
                                 range(out_words, capacity_words * 4, true)};
    if (any_write_overlap(ranges))
        return GCQ_ERR_OVERLAP;
    return launch_status(gcq::launch_elias_encode(norms, nibbles, n, d, bit_offsets, out_words,
                                                  capacity_words, (hipStream_t)stream));
}

int qsgd_elias_decode(const uint32_t *in_words, size_t in_count, const uint64_t *bit_offsets,
                      size_t n, uint32_t d, float *norms, uint32_t *nibbles, void *stream)
{
    if (!elias_d_ok(d) || n > kMaxElems || in_count > kMaxElems)
        return GCQ_ERR_PARAM;
    if (n == 0)
        return GCQ_OK;
    if (!bit_offsets || !norms || !nibbles || (in_count && !in_words))
        return GCQ_ERR_NULL;
    if (!aligned(in_words, 4) || !aligned(bit_offsets, 8) || !aligned(norms, 4) ||
        !aligned(nibbles, 4))
        return GCQ_ERR_ALIGN;
    const size_t nb = qsgd_num_buckets(n, d);
    std::vector<Range> ranges = {range(in_words, in_count * 4, false),
                                 range(bit_offsets, (nb + 1) * 8, false),
                                 range(norms, nb * 4, true),
                                 range(nibbles, qsgd_nibble_words(n) * 4, true)};
    if (any_write_overlap(ranges))
        return GCQ_ERR_OVERLAP;
    return launch_status(gcq::launch_elias_decode(in_words, bit_offsets, n, d, in_count, norms,
                                                  nibbles, (hipStream_t)stream));
}

size_t saps_mask_words(size_t n) { return n / 32 + (n % 32 != 0); }

size_t saps_num_tiles(size_t n) { return n / 8192 + (n % 8192 != 0); }

int saps_mask(size_t n, float c, uint64_t seed, uint32_t *mask_words, uint64_t *tile_offsets,
              void *stream)
{
    if (!(isfinite(c) && c >= 1.0f) || n > kMaxElems)
        return GCQ_ERR_PARAM;
    if (!tile_offsets || (n && !mask_words))
        return GCQ_ERR_NULL;
    if (!aligned(mask_words, 4) || !aligned(tile_offsets, 8))
        return GCQ_ERR_ALIGN;
    std::vector<Range> ranges = {range(mask_words, saps_mask_words(n) * 4, true),
                                 range(tile_offsets, (saps_num_tiles(n) + 1) * 8, true)};
    if (any_write_overlap(ranges))
        return GCQ_ERR_OVERLAP;
    return launch_status(
        gcq::launch_saps_mask(n, c, seed, mask_words, tile_offsets, (hipStream_t)stream));
}

static int saps_apply(float *x, size_t n, const uint32_t *mask_words, const uint64_t *tile_offsets,
                      float *values, size_t capacity, bool merge, void *stream)
{
    if (n > kMaxElems || capacity > kMaxElems)
        return GCQ_ERR_PARAM;
    if (n == 0)
        return GCQ_OK;
    if (!x || !mask_words || !tile_offsets || (capacity && !values))
        return GCQ_ERR_NULL;
    if (!aligned(x, 4) || !aligned(mask_words, 4) || !aligned(tile_offsets, 8) ||
        !aligned(values, 4))
        return GCQ_ERR_ALIGN;
    std::vector<Range> ranges = {range(x, n * 4, merge),
                                 range(mask_words, saps_mask_words(n) * 4, false),
                                 range(tile_offsets, (saps_num_tiles(n) + 1) * 8, false),
                                 range(values, capacity * 4, !merge)};
    if (any_write_overlap(ranges))
        return GCQ_ERR_OVERLAP;
    return launch_status(gcq::launch_saps_apply(x, n, mask_words, tile_offsets, values, capacity,
                                                merge, (hipStream_t)stream));
}

int saps_gather(const float *x, size_t n, const uint32_t *mask_words,
                const uint64_t *tile_offsets, float *values, size_t capacity, void *stream)
{
    return saps_apply((float *)x, n, mask_words, tile_offsets, values, capacity, false, stream);
}

int saps_merge(float *x, size_t n, const uint32_t *mask_words, const uint64_t *tile_offsets,
               const float *peer_values, size_t capacity, void *stream)
{
    return saps_apply(x, n, mask_words, tile_offsets, (float *)peer_values, capacity, true,
                      stream);
}

}  // extern "C"
