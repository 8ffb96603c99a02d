// Checked-build instrumentation of the attention kernels (compiled only with
// H3ATTN_CHECKED, i.e. into libh3attn_checked.so; in the product library the
// macros below expand to nothing).
//
// Each translation unit that includes this header gets its own flag words and
// jitter seed (file-scope device variables) and reads or sets them through
// checked_state_here from its own host code.
//   H3_CHECK(ok, kind)       records a violated invariant: flag word `kind`
//                            (CheckKind) becomes nonzero.
//   H3_JITTER(wave, j, where) with a nonzero seed, the wave sleeps a
//                            pseudo-random 0..3 x 128 cycles.  Placed before
//                            tile fills and compute phases, it moves waves and
//                            their direct-to-LDS fills against each other
//                            without changing any wait or barrier, so a race
//                            between a fill and a fragment read shows up as
//                            different output bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3_internal.h"

namespace h3 {

#ifdef H3ATTN_CHECKED
static __device__ uint32_t h3_check_flags[kCheckKinds];
static __device__ uint32_t h3_jitter_seed;

__device__ __forceinline__ void check_invariant(bool ok, int kind)
{
    if (!ok) atomicOr(&h3_check_flags[kind], 1u);
}

__device__ __forceinline__ void jitter(int wave, int j, int where)
{
    const uint32_t seed = h3_jitter_seed;
    if (seed == 0) return;
    uint32_t x = seed ^ ((uint32_t)blockIdx.x * 0x9E3779B1u) ^ ((uint32_t)wave * 0x85EBCA77u) ^
                 ((uint32_t)j * 0xC2B2AE3Du) ^ ((uint32_t)where * 0x27D4EB2Fu);
    x ^= x >> 15;
    x *= 0x2C1B3C6Du;
    x ^= x >> 12;
    const int nap = __builtin_amdgcn_readfirstlane((int)(x >> 30));
    for (int i = 0; i < nap; ++i) __builtin_amdgcn_s_sleep(2);
}

// Host: OR this unit's flag words into or_into (HOST [kCheckKinds]; may be
// null), clear them if asked, and set the jitter seed of later launches.  The
// caller has synchronised the device.
static inline hipError_t checked_state_here(uint32_t *or_into, bool clear, uint32_t jitter_seed)
{
    uint32_t f[kCheckKinds] = {};
    hipError_t e = hipMemcpyFromSymbol(f, HIP_SYMBOL(h3_check_flags), sizeof f);
    if (e == hipSuccess && or_into)
        for (int i = 0; i < kCheckKinds; ++i) or_into[i] |= f[i];
    if (e == hipSuccess && clear) {
        const uint32_t zeros[kCheckKinds] = {};
        e = hipMemcpyToSymbol(HIP_SYMBOL(h3_check_flags), zeros, sizeof zeros);
    }
    if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(h3_jitter_seed), &jitter_seed, sizeof jitter_seed);
    return e;
}

#define H3_CHECK(ok, kind) ::h3::check_invariant((ok), (kind))
#define H3_JITTER(wave, j, where) ::h3::jitter((wave), (j), (where))
#else
#define H3_CHECK(ok, kind) ((void)0)
#define H3_JITTER(wave, j, where) ((void)0)
#endif

}  // namespace h3
