// gcq_device.h -- device-side helpers shared by the kernels: 16-byte vector
// type, global-address-space qualifier, (non-temporal) loads and stores, DPP
// lane permutes, and the counter-based generator of the random draws.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gcq {
namespace dev {

typedef float v4f __attribute__((ext_vector_type(4)));

// Pointers the compiler cannot trace to a kernel argument (read from a table
// or indexed out of a struct) would otherwise get flat instructions;
// qualifying them as global memory keeps global_load/store.
#define GCQ_GLOBAL __attribute__((address_space(1)))

template <bool NT, typename P>
__device__ __forceinline__ auto ld(P p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <bool NT, typename P, typename T>
__device__ __forceinline__ void st(P p, T v)
{
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// Buffer resources and cache-policy bits (gfx950): word 3 of a raw
// (stride 0, byte-addressed) buffer resource, and the aux bits of the
// buffer load/store builtins: sc0 1, nt 2, sc1 16.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kCpolSc0 = 1;
constexpr int kCpolNt = 2;
constexpr int kCpolSc1 = 16;

// LDS per compute unit on gfx950.
constexpr uint32_t kLdsBytesPerCu = 160u * 1024u;

// DPP quad permutes (within each aligned group of 4 lanes): broadcast lane
// q, or swap neighbouring lanes.  All lanes must be active.
template <int Ctrl>
__device__ __forceinline__ uint32_t dpp(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, Ctrl, 0xF, 0xF, false);
}
constexpr int kQuadBcast0 = 0x00;  // quad_perm [0,0,0,0]
constexpr int kQuadBcast1 = 0x55;  // quad_perm [1,1,1,1]
constexpr int kQuadBcast2 = 0xAA;  // quad_perm [2,2,2,2]
constexpr int kQuadBcast3 = 0xFF;  // quad_perm [3,3,3,3]
constexpr int kSwapPairs = 0xB1;   // quad_perm [1,0,3,2]

// Block -> tile for a grid of exactly one block per tile (G blocks).  The
// dispatcher hands consecutive workgroups to the 8 XCDs in turn, and each
// XCD has its own L2; this gives XCD x the contiguous run of tiles
// [x q + min(x, r), +q + [x < r]) (q = G / 8, r = G mod 8), so neighbouring
// tiles share their L2 lines (e.g. the bucket scales several tiles read).
// It is a bijection of [0, G) for any G, whatever the dispatch order.
constexpr uint32_t kXcds = 8;

__device__ __forceinline__ uint64_t xcd_tile(uint32_t b, uint32_t G)
{
    const uint32_t x = b % kXcds, i = b / kXcds, q = G / kXcds, r = G % kXcds;
    return (uint64_t)x * q + (x < r ? x : r) + i;
}

// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64-bit products; the high halves are xored with the other counter
// words and the round key, the words permuted; the key advances by the
// Weyl increments between rounds.  Each product is one v_mad_u64_u32 and
// each three-way xor one v_bitop3_b32 (truth table 0x96) on gfx950.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)c[0] * 0xD2511F53u;
        const uint64_t p1 = (uint64_t)c[2] * 0xCD9E8D57u;
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c[1], k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c[3], k1, 0x96);
        c[0] = n0;
        c[1] = (uint32_t)p1;
        c[2] = n2;
        c[3] = (uint32_t)p0;
    }
}

}  // namespace dev
}  // namespace gcq
