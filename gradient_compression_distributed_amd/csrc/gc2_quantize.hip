// gc2_quantize.hip -- the 2-bit threshold quantizer with error-feedback
// residual (MXNet PR "2bit gradient compression": "Two bit quantization",
// "Format of compressed gradient"; CD-SGD 3.4.1 "Update Rules") for gfx950,
// single buffer and fused multi-bucket (IMerge-style merged transmission
// units) launches; and CD-SGD's local update of the weights, alone or fused
// with the quantizer (CD-SGD 3.4.1 eq. (11); 3.2.1 Algorithm 1 and Figure
// 4(b): both read the same gradient buffer).
//
// HBM-bound: per element 4 B of g and 4 B of r are read, 4 B of r and 1/4 B
// of packed code written (12.25 B), ~10 VALU ops of arithmetic.  No MFMA.
// Float work is IEEE float32 round-to-nearest; the library is built with
// -ffp-contract=off.
#include "gcq_device.h"
#include "gcq_internal.h"

namespace gcq {

namespace {

using dev::ld;
using dev::st;
using dev::v4f;

// 11 at or above +t, 10 at or below -t, 00 otherwise (NaN compares false).
__device__ __forceinline__ uint32_t gc2_code(float v, float t)
{
    const uint32_t up = v >= t ? 1u : 0u;
    const uint32_t dn = v <= -t ? 1u : 0u;
    return ((up | dn) << 1) | up;
}

// What is not sent stays in the residual: 11 sends +t, 10 sends -t.
__device__ __forceinline__ float gc2_residual(float v, uint32_t code, float t)
{
    const float sent = code == 3u ? t : (code == 2u ? -t : 0.0f);
    return v - sent;
}

// Non-temporal hints per operand (a bit mask): g loads, r loads, r stores,
// packed-word stores.  A non-temporal r (or w) store is a buffer store with
// the nt and sc1 cache-policy bits: about 1% faster for the fused launch at
// 2^30 than nt alone (1.98 against 2.01 ms in one process, every buffer).
constexpr int kNtG = 1, kNtR = 2, kNtRStore = 4, kNtOut = 8;

// Stores float4 k*64 + lane of a wavefront run of 256*U floats at `base`
// (wave-uniform); NT: buffer store with nt and sc1.
template <bool NT, int U>
__device__ __forceinline__ void st_wave_f4(GCQ_GLOBAL v4f *base, int k, uint32_t lane, v4f x)
{
    if constexpr (NT) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)base, 0, 1024 * U, dev::kBufferRsrcWord3);
        __builtin_amdgcn_raw_buffer_store_b128(x, rs, (int)((k * kWave + lane) * 16u), 0,
                                               dev::kCpolNt | dev::kCpolSc1);
    } else {
        base[k * kWave + lane] = x;
    }
}

// Four elements -> their residuals (rn) and one byte of codes, first
// element in the top bit pair.
__device__ __forceinline__ uint32_t gc2_quad(v4f g, v4f r, float t, v4f &rn)
{
    const v4f v = g + r;
    const uint32_t c0 = gc2_code(v.x, t), c1 = gc2_code(v.y, t);
    const uint32_t c2 = gc2_code(v.z, t), c3 = gc2_code(v.w, t);
    rn.x = gc2_residual(v.x, c0, t);
    rn.y = gc2_residual(v.y, c1, t);
    rn.z = gc2_residual(v.z, c2, t);
    rn.w = gc2_residual(v.w, c3, t);
    return (c0 << 6) | (c1 << 4) | (c2 << 2) | c3;
}

// CD-SGD local update of four weights: w - eta * g, the product and the
// difference each rounded once (no fma: the library is built with
// -ffp-contract=off).
__device__ __forceinline__ v4f local_step(v4f w, v4f g, float eta)
{
    const v4f step = eta * g;
    return w - step;
}

// Full wave tile of 256*U elements (U = 1, 2 or 4 float4 per stream per
// lane).  Lane L loads elements 256k + 4L .. +3 of the tile for k < U, so
// every dwordx4 load of the wave covers 1 KiB of consecutive memory.  Those
// four elements are byte (L % 4) of packed word 16k + L/4 (byte 0 = most
// significant).  A quad of lanes therefore holds the four bytes of U words;
// one DPP broadcast per source lane lets lane 4m + j (j < U) assemble word
// 16j + m, so the wave stores its 16U words as U runs of 64 bytes.
//
// The tile size sets how far apart the in-flight accesses of the chip lie:
// with one float4 per lane (U = 1) a workgroup touches 4 KiB per stream and
// the resident workgroups cover one compact window of each buffer, which
// streams faster on HBM3E than four float4 per lane.
//
// Loc = true adds CD-SGD's local update: the weights w (same layout, same
// hints as r) are loaded with g and r and stored updated, so the gradient is
// read once for both uses.
template <int U, int NT, bool Loc>
__device__ __forceinline__ void gc2_wave_tile(const GCQ_GLOBAL float *__restrict__ g,
                                              GCQ_GLOBAL float *__restrict__ r,
                                              GCQ_GLOBAL uint32_t *__restrict__ out, float t,
                                              uint32_t lane, GCQ_GLOBAL float *__restrict__ w,
                                              float eta)
{
    const GCQ_GLOBAL v4f *g4 = (const GCQ_GLOBAL v4f *)g;
    GCQ_GLOBAL v4f *r4 = (GCQ_GLOBAL v4f *)r;
    GCQ_GLOBAL v4f *w4 = (GCQ_GLOBAL v4f *)w;
    v4f gv[U], rv[U], wv[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        gv[k] = ld<(NT & kNtG) != 0>(g4 + k * kWave + lane);
        rv[k] = ld<(NT & kNtR) != 0>(r4 + k * kWave + lane);
        if constexpr (Loc)
            wv[k] = ld<(NT & kNtR) != 0>(w4 + k * kWave + lane);
    }
    if constexpr (Loc) {
#pragma unroll
        for (int k = 0; k < U; ++k)
            st_wave_f4<(NT & kNtRStore) != 0, U>(w4, k, lane, local_step(wv[k], gv[k], eta));
    }
    uint32_t bytes = 0;
#pragma unroll
    for (int k = 0; k < U; ++k) {
        v4f rn;
        bytes |= gc2_quad(gv[k], rv[k], t, rn) << (8 * k);
        st_wave_f4<(NT & kNtRStore) != 0, U>(r4, k, lane, rn);
    }
    const uint32_t x0 = dev::dpp<dev::kQuadBcast0>(bytes), x1 = dev::dpp<dev::kQuadBcast1>(bytes);
    const uint32_t x2 = dev::dpp<dev::kQuadBcast2>(bytes), x3 = dev::dpp<dev::kQuadBcast3>(bytes);
    const uint32_t j = lane & 3u, sh = 8u * j;
    const uint32_t word = (((x0 >> sh) & 0xFFu) << 24) | (((x1 >> sh) & 0xFFu) << 16) |
                          (((x2 >> sh) & 0xFFu) << 8) | ((x3 >> sh) & 0xFFu);
    if (U == 4 || j < (uint32_t)U)
        st<(NT & kNtOut) != 0>(out + 16u * j + (lane >> 2), word);
}

// Wave tile of 256*U elements that runs past the end of its bucket: lane
// L < 16U packs word (e0/16 + L) element by element with bounds checks;
// pairs past n stay 00.
template <int U, bool Loc>
__device__ __forceinline__ void gc2_tile_partial(const GCQ_GLOBAL float *__restrict__ g,
                                                 GCQ_GLOBAL float *__restrict__ r,
                                                 GCQ_GLOBAL uint32_t *__restrict__ out, uint64_t n,
                                                 uint64_t e0, float t, uint32_t lane,
                                                 GCQ_GLOBAL float *__restrict__ wl, float eta)
{
    if (lane >= 16u * U)
        return;
    const uint64_t w = (e0 >> 4) + lane;
    const uint64_t base = w << 4;
    if (base >= n)
        return;
    uint32_t word = 0;
    for (uint32_t p = 0; p < 16; ++p) {
        const uint64_t e = base + p;
        if (e < n) {
            if constexpr (Loc)
                wl[e] = wl[e] - eta * g[e];
            const float v = g[e] + r[e];
            const uint32_t c = gc2_code(v, t);
            r[e] = gc2_residual(v, c, t);
            word |= c << (30u - 2u * p);
        }
    }
    out[w] = word;
}

// Bucket of block tile `tile`: a division when every bucket spans `tpb`
// tiles, else a binary search for the last bucket whose first tile is
// <= tile (empty buckets share their successor's first tile and are
// skipped).  Uniform per workgroup, so it runs on the scalar unit.
__device__ __forceinline__ uint32_t gc2_find_bucket(const Gc2Desc *__restrict__ table,
                                                    uint32_t nbuckets, uint64_t tile, uint32_t tpb)
{
    if (tpb)
        return (uint32_t)(tile / tpb);
    uint32_t lo = 0, hi = nbuckets - 1;
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (table[mid].tile_begin <= tile)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// One kernel for the single-buffer call (Table = false: the descriptor is a
// kernel argument) and the fused multi-bucket call (Table = true: a device
// table of buckets, each owning a contiguous range of block tiles of
// 1024*U elements).  The block -> tile map is a grid-stride loop; with a
// grid of one block per tile (the default) it runs once, and tiles are
// handed out in address order.  A block tile is 4U KiB-aligned within its
// bucket, so no cache line of a bucket is shared between workgroups, and
// thus between the XCDs' L2 caches.
//
// Loc = true (single buffer only) is CD-SGD's compressing iteration: the
// local update of w is fused in (w and eta are unused otherwise).
template <int U, int NT, bool Table, bool Loc>
__global__ __launch_bounds__(kBlockThreads) void gc2_quantize_kernel(
    Gc2Desc one, const Gc2Desc *__restrict__ table, uint32_t nbuckets, uint64_t total_tiles,
    uint32_t tiles_per_bucket, float *__restrict__ wloc, float eta)
{
    static_assert(!(Table && Loc), "the local update is single-buffer");
    constexpr uint64_t kWaveTile = 256u * U, kBlockTile = kWaveTile * kBlockWaves;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = threadIdx.x / kWave;
    uint64_t tile = blockIdx.x;
    if (tile >= total_tiles)
        return;
    uint32_t b = 0;
    if constexpr (Table)
        b = gc2_find_bucket(table, nbuckets, tile, tiles_per_bucket);
    for (; tile < total_tiles; tile += gridDim.x) {
        Gc2Desc d;
        if constexpr (Table) {
            if (tiles_per_bucket)
                b = (uint32_t)(tile / tiles_per_bucket);
            else
                while (b + 1 < nbuckets && table[b + 1].tile_begin <= tile)
                    ++b;
            d = table[b];
        } else {
            d = one;
        }
        const GCQ_GLOBAL float *g = (const GCQ_GLOBAL float *)d.g;
        GCQ_GLOBAL float *r = (GCQ_GLOBAL float *)d.r;
        GCQ_GLOBAL uint32_t *out = (GCQ_GLOBAL uint32_t *)d.out;
        const uint64_t e0 = (tile - d.tile_begin) * kBlockTile + (uint64_t)wave * kWaveTile;
        GCQ_GLOBAL float *w = (GCQ_GLOBAL float *)wloc;
        if (e0 + kWaveTile <= d.n)
            gc2_wave_tile<U, NT, Loc>(g + e0, r + e0, out + (e0 >> 4), d.t, lane,
                                      Loc ? w + e0 : w, eta);
        else if (e0 < d.n)
            gc2_tile_partial<U, Loc>(g, r, out, d.n, e0, d.t, lane, w, eta);
    }
}

template <int U, bool Table>
void launch_nt(int nt, uint32_t grid, uint32_t pad, const Gc2Desc &one, const Gc2Desc *table,
               uint32_t nb, uint64_t total_tiles, uint32_t tpb, hipStream_t stream)
{
    const dim3 block(kBlockThreads);
#define GCQ_GC2(NT)                                                                            \
    gc2_quantize_kernel<U, NT, Table, false>                                                   \
        <<<grid, block, pad, stream>>>(one, table, nb, total_tiles, tpb, nullptr, 0.0f)
    switch (nt) {
    case 0: GCQ_GC2(0); break;
    case 1: GCQ_GC2(1); break;
    case 2: GCQ_GC2(2); break;
    case 3: GCQ_GC2(3); break;
    case 4: GCQ_GC2(4); break;
    case 5: GCQ_GC2(5); break;
    case 6: GCQ_GC2(6); break;
    case 7: GCQ_GC2(7); break;
    case 8: GCQ_GC2(8); break;
    case 9: GCQ_GC2(9); break;
    case 10: GCQ_GC2(10); break;
    case 11: GCQ_GC2(11); break;
    case 12: GCQ_GC2(12); break;
    case 13: GCQ_GC2(13); break;
    case 14: GCQ_GC2(14); break;
    default: GCQ_GC2(15); break;
    }
#undef GCQ_GC2
}

template <bool Table>
hipError_t launch(const gcq_tuning &tu, const Gc2Desc &one, const Gc2Desc *table, uint32_t nb,
                  uint64_t total_tiles, uint32_t tpb, hipStream_t stream)
{
    const uint32_t grid = grid_for(total_tiles, tu.gc2_blocks_per_cu);
    const uint32_t pad = resident_lds_pad(0, tu.gc2_resident_per_cu);
    switch (tu.gc2_unroll) {
    case 1: launch_nt<1, Table>(tu.gc2_nt, grid, pad, one, table, nb, total_tiles, tpb, stream); break;
    case 2: launch_nt<2, Table>(tu.gc2_nt, grid, pad, one, table, nb, total_tiles, tpb, stream); break;
    default: launch_nt<4, Table>(tu.gc2_nt, grid, pad, one, table, nb, total_tiles, tpb, stream); break;
    }
    return hipGetLastError();
}

// CD-SGD local update alone (a correction iteration): w - eta * g over
// wave tiles of 256*U elements, lane L owning float4 k*64 + L (k < U).
template <int U, int NT>
__global__ __launch_bounds__(kBlockThreads) void local_update_kernel(const float *__restrict__ g,
                                                                      float *__restrict__ w,
                                                                      uint64_t n, uint64_t tiles,
                                                                      float eta)
{
    constexpr uint64_t kWaveTile = 256u * U, kBlockTile = kWaveTile * kBlockWaves;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = threadIdx.x / kWave;
    const GCQ_GLOBAL float *gg = (const GCQ_GLOBAL float *)g;
    GCQ_GLOBAL float *ww = (GCQ_GLOBAL float *)w;
    for (uint64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const uint64_t e0 = tile * kBlockTile + (uint64_t)wave * kWaveTile;
        if (e0 + kWaveTile <= n) {
            const GCQ_GLOBAL v4f *g4 = (const GCQ_GLOBAL v4f *)(gg + e0);
            GCQ_GLOBAL v4f *w4 = (GCQ_GLOBAL v4f *)(ww + e0);
            v4f gv[U], wv[U];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                gv[k] = ld<(NT & kNtG) != 0>(g4 + k * kWave + lane);
                wv[k] = ld<(NT & kNtR) != 0>(w4 + k * kWave + lane);
            }
#pragma unroll
            for (int k = 0; k < U; ++k)
                st_wave_f4<(NT & kNtRStore) != 0, U>(w4, k, lane, local_step(wv[k], gv[k], eta));
        } else if (e0 < n) {
            for (uint64_t e = e0 + lane; e < n && e < e0 + kWaveTile; e += kWave)
                ww[e] = ww[e] - eta * gg[e];
        }
    }
}

// The CD-SGD launches take the quantizer's unroll and block-count knobs,
// and its non-temporal mask reduced to none (0), all (15) or the default
// set (g, r and w loads, r and w stores: 7).
template <int U, int NT>
void launch_cdsgd_u(bool quant, uint32_t grid, uint32_t pad, const Gc2Desc &one, float *w,
                    float eta, uint64_t tiles, hipStream_t stream)
{
    if (quant)
        gc2_quantize_kernel<U, NT, false, true>
            <<<grid, kBlockThreads, pad, stream>>>(one, nullptr, 1, tiles, 0, w, eta);
    else
        local_update_kernel<U, NT>
            <<<grid, kBlockThreads, pad, stream>>>(one.g, w, one.n, tiles, eta);
}

template <int U>
void launch_cdsgd_nt(int nt, bool quant, uint32_t grid, uint32_t pad, const Gc2Desc &one,
                     float *w, float eta, uint64_t tiles, hipStream_t stream)
{
    if (nt == 0)
        launch_cdsgd_u<U, 0>(quant, grid, pad, one, w, eta, tiles, stream);
    else if (nt == 15)
        launch_cdsgd_u<U, 15>(quant, grid, pad, one, w, eta, tiles, stream);
    else
        launch_cdsgd_u<U, 7>(quant, grid, pad, one, w, eta, tiles, stream);
}

// Writes descriptors that arrive by value in the kernel arguments into a
// device table: one launch per kFillChunk descriptors, thread i storing
// descriptor i.  Nothing is staged in host memory, so the caller's array may
// be reused as soon as the launch call returns, and a table slot is ordered
// against its earlier readers on the device alone.
struct Gc2FillChunk {
    Gc2Desc d[kFillChunk];
};

__global__ __launch_bounds__(kFillChunk) void gc2_table_fill_kernel(Gc2FillChunk chunk,
                                                                     Gc2Desc *__restrict__ dst,
                                                                     uint32_t count)
{
    const uint32_t i = threadIdx.x;
    if (i < count)
        dst[i] = chunk.d[i];
}

}  // namespace

uint64_t gc2_tile_elems(const gcq_tuning &tu) { return 1024u * (uint64_t)tu.gc2_unroll; }

hipError_t launch_gc2_table_fill(const Gc2Desc *descs, uint32_t count, Gc2Desc *dev_table,
                                 hipStream_t stream)
{
    for (uint32_t b0 = 0; b0 < count; b0 += kFillChunk) {
        const uint32_t c = count - b0 < kFillChunk ? count - b0 : kFillChunk;
        Gc2FillChunk chunk = {};
        for (uint32_t i = 0; i < c; ++i)
            chunk.d[i] = descs[b0 + i];
        gc2_table_fill_kernel<<<1, kFillChunk, 0, stream>>>(chunk, dev_table + b0, c);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_gc2_single(const Gc2Desc &one, hipStream_t stream)
{
    const gcq_tuning tu = tuning();
    const uint64_t te = gc2_tile_elems(tu);
    const uint64_t tiles = (one.n + te - 1) / te;
    if (!tiles)
        return hipSuccess;
    return launch<false>(tu, one, nullptr, 1, tiles, 0, stream);
}

hipError_t launch_cdsgd(const float *g, float *r, float *w, uint32_t *out, uint64_t n, float t,
                        float eta, bool quant, hipStream_t stream)
{
    const gcq_tuning tu = tuning();
    const uint64_t te = gc2_tile_elems(tu);
    const uint64_t tiles = (n + te - 1) / te;
    if (!tiles)
        return hipSuccess;
    const Gc2Desc one = {g, r, out, n, 0, t, 0};
    const uint32_t grid = grid_for(tiles, tu.gc2_blocks_per_cu);
    const uint32_t pad = resident_lds_pad(0, tu.cdsgd_resident_per_cu);
    switch (tu.gc2_unroll) {
    case 1: launch_cdsgd_nt<1>(tu.gc2_nt, quant, grid, pad, one, w, eta, tiles, stream); break;
    case 2: launch_cdsgd_nt<2>(tu.gc2_nt, quant, grid, pad, one, w, eta, tiles, stream); break;
    default: launch_cdsgd_nt<4>(tu.gc2_nt, quant, grid, pad, one, w, eta, tiles, stream); break;
    }
    return hipGetLastError();
}

hipError_t launch_gc2_table(const gcq_tuning &tu, const Gc2Desc *dev_table, uint32_t nbuckets,
                            uint64_t total_tiles, uint32_t tiles_per_bucket, hipStream_t stream)
{
    if (!total_tiles || !nbuckets)
        return hipSuccess;
    Gc2Desc none = {};
    return launch<true>(tu, none, dev_table, nbuckets, total_tiles, tiles_per_bucket, stream);
}

}  // namespace gcq
