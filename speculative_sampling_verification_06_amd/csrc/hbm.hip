// hbm.hip - plain streaming kernels that measure the HBM rate this GPU
// reaches: the achievable ceiling the verify kernels are compared with (a
// datasheet peak is not reached by any access pattern).  Not part of the
// verify step.
//
// k_hbm_read: every lane keeps four 16-byte non-temporal loads in flight per
// pass over a grid-stride range and folds them into one word (XOR), so no
// load is dead; each wave writes one word.  k_hbm_copy: the same loads, each
// stored to the destination.  The grid is eight 256-thread workgroups per
// compute unit (the resident limit at these register counts), every one
// streaming until the range ends.

#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>

#include "spec_verify.h"
#include "sv_internal.h"

namespace svhbm {

constexpr int NT = 256;
constexpr int U = 4;                 // 16-byte loads in flight per lane
constexpr int WG_PER_CU = 8;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }

__global__ __launch_bounds__(NT) void k_hbm_read(const u32x4* __restrict__ src, int64_t n16,
                                                 uint32_t* __restrict__ out)
{
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * NT * U;
    for (int64_t i = (int64_t)blockIdx.x * NT * U + threadIdx.x; i < n16; i += stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = i + (int64_t)u * NT;
            v[u] = j < n16 ? ld_nt(src + j) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0) out[blockIdx.x * (NT / 64) + (threadIdx.x >> 6)] = acc;
}

__global__ __launch_bounds__(NT) void k_hbm_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * NT * U;
    for (int64_t i = (int64_t)blockIdx.x * NT * U + threadIdx.x; i < n16; i += stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = i + (int64_t)u * NT;
            if (j < n16) v[u] = ld_nt(src + j);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = i + (int64_t)u * NT;
            if (j < n16) __builtin_nontemporal_store(v[u], dst + j);
        }
    }
}

static int grid_for_device()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        return -1;
    return cus * WG_PER_CU;
}

}  // namespace svhbm

extern "C" {

int32_t sv_hbm_probe_words(void)
{
    const int g = svhbm::grid_for_device();
    return g < 0 ? -1 : g * (svhbm::NT / 64);
}

int sv_hbm_probe(int32_t kind, const void* src, void* dst, size_t bytes, void* stream)
{
    if (kind != SV_PROBE_READ && kind != SV_PROBE_COPY) return SV_EINVAL;
    if (!src || !dst || bytes == 0 || bytes % 16 != 0) return SV_EINVAL;
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0) return SV_EINVAL;
    const int64_t n16 = (int64_t)(bytes / 16);
    if (kind == SV_PROBE_COPY) {
        const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
        if (s0 < d0 + bytes && d0 < s0 + bytes) return SV_EINVAL;      // overlapping ranges
    }
    const int grid_max = svhbm::grid_for_device();
    if (grid_max < 0) return SV_ELAUNCH;
    const int64_t per_wg = (int64_t)svhbm::NT * svhbm::U;
    const int grid = (int)((n16 + per_wg - 1) / per_wg < grid_max ? (n16 + per_wg - 1) / per_wg : grid_max);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const auto* s = static_cast<const svhbm::u32x4*>(src);
    sv_launch_begin();
    if (kind == SV_PROBE_READ)
        hipLaunchKernelGGL(svhbm::k_hbm_read, dim3(grid), dim3(svhbm::NT), 0, st, s, n16, static_cast<uint32_t*>(dst));
    else
        hipLaunchKernelGGL(svhbm::k_hbm_copy, dim3(grid), dim3(svhbm::NT), 0, st, s, static_cast<svhbm::u32x4*>(dst), n16);
    return sv_launch_status();
}

}  // extern "C"
