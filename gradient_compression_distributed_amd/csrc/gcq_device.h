// gcq_device.h -- device-side helpers shared by the kernels: 16-byte vector
// type, global-address-space qualifier, (non-temporal) loads and stores, DPP
// lane permutes.
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

}  // namespace dev
}  // namespace gcq
