// lookup.hip - prompt-lookup proposer: candidate tokens without a draft model.
//
// The candidates are the tokens that followed an earlier occurrence of the
// history's current ending ([QH] "Vấn đề 3: Làm sao khi không muốn train
// drafter?": match the text being generated against the prompt and earlier
// output, propose the continuation, let the target verify it).  The ending
// tried is the last n tokens for n from n_max down to n_min; for the first n
// with an earlier occurrence (one that leaves at least one token after it
// inside the history) the earliest such occurrence is used, and the up to K
// tokens after it, clipped at the history's end, are the candidates.
//
// One workgroup per sequence.  For every continuation start c in [1, L-1]
// the match length l(c) is the number of tokens before c that agree with the
// ending, read backwards (at most n_max, at most c).  The rule above picks
// the largest n with some l(c) >= n, then the smallest such c; since that n
// is the largest l(c), it is the pair maximising (l(c), -c), found with one
// block reduction.  The comparison loop depends on the data (it runs on only
// while tokens agree), so read from global memory each start's first token
// was a round trip of its own, one after another per thread; histories of up
// to HCAP tokens are staged in LDS by one coalesced pass over the whole row
// (issued before the row's length arrives) and compared there, the ending and
// the candidates read back from LDS (B=256 histories of 2-4k tokens: 19.4 ->
// 11.0 us per call); longer ones are compared in global memory.  Reads the
// history once.

#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>

#include "spec_verify.h"
#include "sv_internal.h"

namespace svpl {

constexpr int NT = 256;
constexpr int NW = NT / 64;
constexpr int HCAP = 15360;               // history tokens staged in LDS (60 KB)

struct LookupParams {
    const int32_t* hist;
    const int32_t* hist_len;
    int32_t* cand;
    int32_t* klen;
    int32_t B, Lmax, n_max, n_min, K;
};

// STAGE: the history (Lmax <= HCAP tokens) is compared in LDS, filled with
// dynamic shared memory of Lmax tokens.
template <bool STAGE>
__global__ __launch_bounds__(NT) void k_lookup(const LookupParams P)
{
    extern __shared__ int32_t sh_h[];
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t* h = P.hist + (int64_t)b * P.Lmax;
    int32_t* cand = P.cand + (int64_t)b * P.K;
    __shared__ int32_t sfx[SV_MAX_NGRAM];         // the ending, last token first
    __shared__ uint64_t sh_best[NW];
    __shared__ int32_t sh_c, sh_k;

    const int32_t L = P.hist_len[b];
    if constexpr (STAGE) {
        // the whole row of Lmax tokens, loaded without waiting for its length
        constexpr int U = 16;                      // independent loads in flight per thread (4096 tokens: one pass)
        for (int i0 = 0; i0 < P.Lmax; i0 += NT * U) {
            int32_t v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * NT + tid;
                v[u] = i < P.Lmax ? h[i] : 0;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * NT + tid;
                if (i < P.Lmax) sh_h[i] = v[u];
            }
        }
    }
    if (L < 0 || L > P.Lmax) {                     // invalid length (uniform): the sequence gets klen -1
        for (int j = tid; j < P.K; j += NT) cand[j] = -1;
        if (tid == 0) P.klen[b] = -1;
        return;
    }
    const int ns = min(P.n_max, L);
    if constexpr (STAGE) {
        __syncthreads();
        if (tid < ns) sfx[tid] = sh_h[L - 1 - tid];
    } else {
        if (tid < ns) sfx[tid] = h[L - 1 - tid];
    }
    __syncthreads();
    const int32_t* hc = STAGE ? sh_h : h;          // where the comparisons read

    // key = (l << 32) | ~c: the maximum has the longest match, then the smallest c
    uint64_t best = 0;
    for (int32_t c = 1 + tid; c < L; c += NT) {
        const int lim = min(P.n_max, c);
        int l = 0;
        while (l < lim && hc[c - 1 - l] == sfx[l]) ++l;
        const uint64_t key = ((uint64_t)(uint32_t)l << 32) | (uint32_t)~(uint32_t)c;
        best = key > best ? key : best;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t o = __shfl_xor(best, off, 64);
        best = o > best ? o : best;
    }
    if (lane == 0) sh_best[wave] = best;
    __syncthreads();
    if (tid == 0) {
        uint64_t m = sh_best[0];
        for (int w = 1; w < NW; ++w) m = sh_best[w] > m ? sh_best[w] : m;
        const int l = (int)(m >> 32);
        int32_t k = 0, c = 0;
        if (l >= P.n_min && l >= 1) {
            c = (int32_t)~(uint32_t)(m & 0xffffffffu);
            k = min(P.K, L - c);
        }
        sh_c = c;
        sh_k = k;
        P.klen[b] = k;
    }
    __syncthreads();
    const int32_t c = sh_c, k = sh_k;
    for (int j = tid; j < P.K; j += NT) cand[j] = j < k ? hc[c + j] : -1;
}

static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace svpl

extern "C" {

int sv_lookup_propose(const int32_t* history, const int32_t* hist_len, int32_t B, int32_t Lmax, int32_t n_max,
                      int32_t n_min, int32_t K, int32_t* cand, int32_t* klen, void* stream)
{
    if (B < 0 || Lmax < 0 || n_min < 1 || n_max < n_min || n_max > SV_MAX_NGRAM || K < 0 || K > SV_MAX_K)
        return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!hist_len || !klen || (Lmax > 0 && !history) || (K > 0 && !cand)) return SV_EINVAL;
    if (!svpl::aligned4(hist_len) || !svpl::aligned4(klen) || (history && !svpl::aligned4(history)) ||
        (cand && !svpl::aligned4(cand)))
        return SV_EINVAL;
    svpl::LookupParams P;
    P.hist = history;
    P.hist_len = hist_len;
    P.cand = cand;
    P.klen = klen;
    P.B = B;
    P.Lmax = Lmax;
    P.n_max = n_max;
    P.n_min = n_min;
    P.K = K;
    sv_launch_begin();
    if (Lmax <= svpl::HCAP)
        hipLaunchKernelGGL(svpl::k_lookup<true>, dim3((unsigned)B), dim3(svpl::NT), (size_t)Lmax * sizeof(int32_t),
                           static_cast<hipStream_t>(stream), P);
    else
        hipLaunchKernelGGL(svpl::k_lookup<false>, dim3((unsigned)B), dim3(svpl::NT), 0, static_cast<hipStream_t>(stream),
                           P);
    return sv_launch_status();
}

}  // extern "C"
