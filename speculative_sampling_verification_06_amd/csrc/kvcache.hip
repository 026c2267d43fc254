// kvcache.hip - commit of the accepted prefix into a key/value cache.
//
// The target pass computes state for every candidate position before anyone
// knows which candidates survive; after verification the entries of the
// discarded suffix must not become part of the committed decoding state, and
// the draft's own cache must follow the accepted prefix too ([NL]
// "Verifikasi mengubah jalur cache": truncation, staged writes or index
// management all meet that requirement).
//
// Staged writes (sv_kv_commit with a staging buffer): the pass wrote S entries
// per sequence and plane into staged [P, B, S, row_bytes]; the committed count
// is c_b = accepted_len[b] + offset, where offset = 1 when the staging block
// starts with the previous round's final token (its entry is computed in this
// pass) and 0 otherwise.  k_kv_copy copies staged[p, b, 0:c_b] to
// cache[p, b, len_b : len_b + c_b] for every plane p (e.g. 2 per layer: keys
// and values); k_kv_len then sets len_b += c_b.  Two launches, because every
// copy workgroup reads len_b.  In-place writes (staged == NULL): the entries
// already sit at cache[p, b, len_b : len_b + S), so committing is the length
// update alone and the rest of that region is never read again.
//
// Sequences with accepted_len = -1 (invalid input) or whose commit would pass
// L_max are left unchanged; status[b] says which (0 committed, 1 invalid,
// 2 would overflow).  HBM-bound copy: 16-byte vector loads and stores when
// row_bytes and both base pointers are 16-byte aligned, bytes otherwise.

#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>

#include "spec_verify.h"
#include "sv_internal.h"

namespace svkv {

constexpr int NT = 256;
constexpr int64_t CHUNK = 64 * 1024;      // staged bytes per workgroup

struct KvParams {
    char* cache;
    const int32_t* len;
    const char* staged;
    const int32_t* acc;
    int32_t B, S, offset;
    int64_t lmax, row_bytes;
    int32_t chunks;                       // per (plane, sequence)
    bool vec;
};

__device__ __forceinline__ int32_t commit_count(const KvParams& P, int b, int32_t len)
{
    const int32_t n = P.acc[b];
    if (n < 0 || n > P.S - P.offset) return -1;                       // invalid sequence
    const int32_t c = n + P.offset;
    if (len < 0 || (int64_t)len + c > P.lmax) return -2;               // would overflow
    return c;
}

__global__ __launch_bounds__(NT) void k_kv_copy(const KvParams P)
{
    const int64_t per_plane = (int64_t)P.B * P.chunks;
    const int64_t g = blockIdx.x;
    const int p = (int)(g / per_plane);
    const int b = (int)((g - (int64_t)p * per_plane) / P.chunks);
    const int ch = (int)(g - (int64_t)p * per_plane - (int64_t)b * P.chunks);
    const int32_t len = P.len[b];
    const int32_t c = commit_count(P, b, len);
    if (c <= 0) return;
    const int64_t bytes = (int64_t)c * P.row_bytes;
    const int64_t lo = (int64_t)ch * CHUNK;
    if (lo >= bytes) return;
    const int64_t hi = lo + CHUNK < bytes ? lo + CHUNK : bytes;
    const char* src = P.staged + (((int64_t)p * P.B + b) * P.S) * P.row_bytes;
    char* dst = P.cache + (((int64_t)p * P.B + b) * P.lmax + len) * P.row_bytes;
    if (P.vec) {
        for (int64_t o = lo + (int64_t)threadIdx.x * 16; o < hi; o += (int64_t)NT * 16)
            *reinterpret_cast<uint4*>(dst + o) = *reinterpret_cast<const uint4*>(src + o);
    } else {
        for (int64_t o = lo + threadIdx.x; o < hi; o += NT) dst[o] = src[o];
    }
}

__global__ __launch_bounds__(NT) void k_kv_len(const KvParams P, int32_t* len, int32_t* status)
{
    const int b = blockIdx.x * NT + threadIdx.x;
    if (b >= P.B) return;
    const int32_t l = len[b];
    const int32_t c = commit_count(P, b, l);
    if (c >= 0) len[b] = l + c;
    if (status) status[b] = c >= 0 ? 0 : (c == -1 ? 1 : 2);
}

static bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace svkv

extern "C" {

int sv_kv_commit(void* cache, int32_t* cache_len, const void* staged, const int32_t* accepted_len,
                 int32_t planes, int32_t B, int32_t K, int32_t offset, int64_t l_max, int64_t row_bytes,
                 int32_t* status, void* stream)
{
    if (planes < 1 || B < 0 || K < 0 || K > SV_MAX_K || (offset != 0 && offset != 1) || l_max < 1 || row_bytes < 1)
        return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!cache_len || !accepted_len || (staged && !cache)) return SV_EINVAL;
    if (!svkv::aligned_to(cache_len, 4) || !svkv::aligned_to(accepted_len, 4) || (status && !svkv::aligned_to(status, 4)))
        return SV_EINVAL;
    svkv::KvParams P;
    P.cache = static_cast<char*>(cache);
    P.len = cache_len;
    P.staged = static_cast<const char*>(staged);
    P.acc = accepted_len;
    P.B = B;
    P.S = K + offset;
    P.offset = offset;
    P.lmax = l_max;
    P.row_bytes = row_bytes;
    const int64_t region = (int64_t)P.S * row_bytes;
    const int64_t chunks = (region + svkv::CHUNK - 1) / svkv::CHUNK;
    // S = K + offset = 0 (K = 0, offset 0): no staged entries, so nothing to
    // copy; the length update and the status still run
    if ((int64_t)planes * B * chunks > INT_MAX) return SV_EINVAL;
    P.chunks = (int32_t)chunks;
    P.vec = row_bytes % 16 == 0 && svkv::aligned_to(cache, 16) && (!staged || svkv::aligned_to(staged, 16));
    hipStream_t st = static_cast<hipStream_t>(stream);
    sv_launch_begin();
    if (staged && chunks > 0)
        hipLaunchKernelGGL(svkv::k_kv_copy, dim3((unsigned)((int64_t)planes * B * chunks)), dim3(svkv::NT), 0, st, P);
    hipLaunchKernelGGL(svkv::k_kv_len, dim3((unsigned)((B + svkv::NT - 1) / svkv::NT)), dim3(svkv::NT), 0, st, P,
                       cache_len, status);
    return sv_launch_status();
}

}  // extern "C"
