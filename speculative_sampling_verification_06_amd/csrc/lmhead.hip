// lmhead.hip - gfx950 bf16 MFMA LM head for the fused LM-head verify path.
//
// The target model's last step maps each final hidden vector (d values) to one
// score per vocabulary token ([QH] "Hidden state": the LM head turns the last
// hidden state into the table over the vocabulary).  For the verify step the
// K+1 positions of B sequences share the weight, so
//     logits[m, v] = sum_k hidden[m, k] * W[k, v],   m < M = B*(K+1), v < V,
// a tall-skinny dense contraction (M = 192, d = 4096, V = 128256 in the fused
// workload).  At M = 192 it does 2*M flops per weight element: HBM-bound on
// streaming W once (1.05 GB), with MFMA needed at about half its peak.
//
// Layout: W is static, so it is packed once (k_pack) from [d, V] into
// Wt = W^T [V, d] (the usual [out_features, in_features] weight layout), which
// makes both MFMA operands contiguous along k.  k_lmhead: one workgroup = 4
// waves; each wave owns 64 vocabulary rows of Wt (two 32-wide MFMA tiles) and
// all 192 hidden rows (six 32-row tiles) of an M block, so every Wt element
// is read from HBM exactly once and each 16-k step issues 12
// v_mfma_f32_32x32x16_bf16.  Wt fragments stream into a register ring two
// 64-k blocks deep; the hidden states (1.5 MB, L2-resident) come through a
// double-buffered LDS block shared by the four waves, the next block's loads
// in flight while the current one is multiplied.
// Accumulation is fp32; bf16 x bf16 products are exact in fp32.
//
// MFMA 32x32x16 operand layout (lane l, 8 bf16 per operand):
//   A (32 x 16): row l % 32, k = 8 * (l / 32) .. +7
//   B (16 x 32): column l % 32, k = 8 * (l / 32) .. +7
//   D (32 x 32, 16 fp32): column l % 32, element r -> row 8*(r/4) + 4*(l/32) + r%4

#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>

#include "spec_verify.h"
#include "sv_internal.h"

namespace svlm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NT = 256;           // four wave64
constexpr int WN = 64;            // vocabulary rows per wave
constexpr int BN = 4 * WN;        // per workgroup
constexpr int MT = 6;             // 32-row tiles per M block
constexpr int MB = 32 * MT;       // 192 hidden rows per M block

__device__ __forceinline__ bf16x8 ld16(const uint16_t* p)
{
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    return __builtin_bit_cast(bf16x8, v);
}

__global__ __launch_bounds__(256) void k_pack(const uint16_t* __restrict__ W, uint16_t* __restrict__ Wt,
                                              int d, int V)
{
    __shared__ uint16_t tile[64][66];
    const int k0 = blockIdx.y * 64, v0 = blockIdx.x * 64;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int r = i >> 6, c = i & 63;
        const int k = k0 + r, v = v0 + c;
        tile[r][c] = (k < d && v < V) ? W[(int64_t)k * V + v] : (uint16_t)0;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int r = i >> 6, c = i & 63;
        const int v = v0 + r, k = k0 + c;
        if (v < V && k < d) Wt[(int64_t)v * d + k] = tile[c][r];
    }
}

// Hidden-state block of BK k-columns for all MB rows, staged in LDS and
// shared by the four waves.  Rows are padded to A_LD bf16 (144 bytes) so the
// 16 lanes of each ds_read_b128 group hit all 64 banks once.
constexpr int BK = 64;                 // k per LDS block
constexpr int KS = BK / 16;            // MFMA k-steps per block
constexpr int A_LD = BK + 8;           // padded LDS row stride, bf16
constexpr int A_PIECES = MB * BK / 8;  // 16-byte pieces per block
constexpr int A_PER_T = A_PIECES / NT; // per thread (6)
constexpr int WPF = 2 * KS;            // Wt prefetch depth in k-steps (two blocks)
static_assert(A_PIECES % NT == 0, "block pieces must split evenly");

__global__ __launch_bounds__(NT, 1) void k_lmhead(const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wt,
                                                  float* __restrict__ out, int M, int d, int V)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][MB * A_LD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, kg = lane >> 5;
    const int n0 = blockIdx.x * BN + wave * WN;
    const int m0 = blockIdx.y * MB;
    const int nsteps = (d + 15) / 16;
    const int nblk = (d + BK - 1) / BK;
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    const bf16x8 zero = {};

    // rows past V read the last valid row; their results are not stored
    const uint16_t* bp[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int v = min(n0 + 32 * c + li, V - 1);
        bp[c] = Wt + (int64_t)v * d + 8 * kg;
    }
    auto ldw = [&](int c, int step) -> bf16x8 {
        return (step < nsteps && step * 16 + 8 * kg < d) ? ld16(bp[c] + step * 16) : zero;
    };
    // this thread's share of a hidden-state block: pieces tid + i*NT, i < 6,
    // held in six named registers (an indexable array would be moved to LDS)
    static_assert(A_PER_T == 6, "staging below is written out for six pieces");
    const int ar = tid >> 3, ac = (tid & 7) * 8;               // piece i: row ar + 32*i
#define LM_SRC(i) (H + (int64_t)min(m0 + ar + 32 * (i), M - 1) * d + ac)
    const uint16_t* hs0 = LM_SRC(0);
    const uint16_t* hs1 = LM_SRC(1);
    const uint16_t* hs2 = LM_SRC(2);
    const uint16_t* hs3 = LM_SRC(3);
    const uint16_t* hs4 = LM_SRC(4);
    const uint16_t* hs5 = LM_SRC(5);
#undef LM_SRC
    uint4 s0, s1, s2, s3, s4, s5;
#define LM_LOAD_A(kb)                                                                          \
    do {                                                                                       \
        const bool ok_ = (kb) < nblk && (kb) * BK + ac < d;                                   \
        const int64_t o_ = (int64_t)(kb) * BK;                                                \
        s0 = ok_ ? *reinterpret_cast<const uint4*>(hs0 + o_) : z4;                             \
        s1 = ok_ ? *reinterpret_cast<const uint4*>(hs1 + o_) : z4;                             \
        s2 = ok_ ? *reinterpret_cast<const uint4*>(hs2 + o_) : z4;                             \
        s3 = ok_ ? *reinterpret_cast<const uint4*>(hs3 + o_) : z4;                             \
        s4 = ok_ ? *reinterpret_cast<const uint4*>(hs4 + o_) : z4;                             \
        s5 = ok_ ? *reinterpret_cast<const uint4*>(hs5 + o_) : z4;                             \
    } while (0)
#define LM_STORE_A(buf)                                                                        \
    do {                                                                                       \
        uint16_t* a_ = &As[buf][ar * A_LD + ac];                                              \
        *reinterpret_cast<uint4*>(a_ + 0 * 32 * A_LD) = s0;                                   \
        *reinterpret_cast<uint4*>(a_ + 1 * 32 * A_LD) = s1;                                   \
        *reinterpret_cast<uint4*>(a_ + 2 * 32 * A_LD) = s2;                                   \
        *reinterpret_cast<uint4*>(a_ + 3 * 32 * A_LD) = s3;                                   \
        *reinterpret_cast<uint4*>(a_ + 4 * 32 * A_LD) = s4;                                   \
        *reinterpret_cast<uint4*>(a_ + 5 * 32 * A_LD) = s5;                                   \
    } while (0)

    f32x16 acc[MT][2];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        acc[t][0] = f32x16{};
        acc[t][1] = f32x16{};
    }
    bf16x8 wb[WPF][2];
#pragma unroll
    for (int q = 0; q < WPF; ++q) {
        wb[q][0] = ldw(0, q);
        wb[q][1] = ldw(1, q);
    }
    LM_LOAD_A(0);
    LM_STORE_A(0);
    LM_LOAD_A(1);
    __syncthreads();

    // blocks in pairs so every Wt ring slot index is a compile-time constant
    for (int kb0 = 0; kb0 < nblk; kb0 += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kb = kb0 + h;
            if (kb < nblk) {
                const uint16_t* as = As[h] + li * A_LD + 8 * kg;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int step = kb * KS + ks;
                    const int slot = h * KS + ks;
                    const bf16x8 b0 = wb[slot][0], b1 = wb[slot][1];
                    wb[slot][0] = ldw(0, step + WPF);
                    wb[slot][1] = ldw(1, step + WPF);
                    if (step < nsteps) {
#pragma unroll
                        for (int t = 0; t < MT; ++t) {
                            const bf16x8 a = *reinterpret_cast<const bf16x8*>(as + t * 32 * A_LD + ks * 16);
                            acc[t][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[t][0], 0, 0, 0);
                            acc[t][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[t][1], 0, 0, 0);
                        }
                    }
                }
                // block kb+1 (in registers) into the other buffer; every wave
                // finished reading that buffer before the previous barrier
                LM_STORE_A(h ^ 1);
                __syncthreads();
                LM_LOAD_A(kb + 2);
            }
        }
    }

#undef LM_LOAD_A
#undef LM_STORE_A
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int col = n0 + 32 * c + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + 32 * t + 8 * (r >> 2) + 4 * kg + (r & 3);
                if (row < M && col < V) out[(int64_t)row * V + col] = acc[t][c][r];
            }
        }
    }
}

static bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static int check_gemm(const void* hidden, const void* w_vd, int32_t M, int32_t d, int32_t V, const float* logits)
{
    if (M < 0 || d < 8 || d % 8 != 0 || V < 1) return SV_EINVAL;
    if (M == 0) return SV_OK;
    if (!hidden || !w_vd || !logits) return SV_EINVAL;
    if (!aligned_to(hidden, 16) || !aligned_to(w_vd, 16) || !aligned_to(logits, 4)) return SV_EINVAL;
    if ((V + (int64_t)BN - 1) / BN > INT_MAX || (M + (int64_t)MB - 1) / MB > 65535) return SV_EINVAL;
    return 1;
}

}  // namespace svlm

extern "C" {

int sv_lmhead_pack(const void* w_dv, void* w_vd, int32_t d, int32_t V, void* stream)
{
    if (d < 1 || V < 1 || !w_dv || !w_vd) return SV_EINVAL;
    if (!svlm::aligned_to(w_dv, 2) || !svlm::aligned_to(w_vd, 2)) return SV_EINVAL;
    if ((d + 63) / 64 > 65535) return SV_EINVAL;
    const dim3 grid((unsigned)((V + 63) / 64), (unsigned)((d + 63) / 64));
    sv_launch_begin();
    hipLaunchKernelGGL(svlm::k_pack, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint16_t*>(w_dv), static_cast<uint16_t*>(w_vd), d, V);
    return sv_launch_status();
}

int sv_lmhead(const void* hidden, const void* w_vd, int32_t M, int32_t d, int32_t V, float* logits,
              void* stream)
{
    const int rc = svlm::check_gemm(hidden, w_vd, M, d, V, logits);
    if (rc <= 0) return rc;
    const dim3 grid((unsigned)((V + svlm::BN - 1) / svlm::BN), (unsigned)((M + svlm::MB - 1) / svlm::MB));
    sv_launch_begin();
    hipLaunchKernelGGL(svlm::k_lmhead, grid, dim3(svlm::NT), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(w_vd), logits, M, d, V);
    return sv_launch_status();
}

int spec_lmhead_verify(const void* hidden, const void* w_vd, int32_t d, float* target_logits,
                       const void* draft_logits, int32_t draft_dtype, const int32_t* draft_tokens,
                       const float* uniforms, float temperature, const uint8_t* greedy_flag,
                       int32_t B, int32_t K, int32_t V, int32_t* accepted_len, int32_t* out_tokens,
                       const sv_diag* diag, void* workspace, size_t workspace_bytes, void* stream)
{
    if (B < 0 || K < 0 || K > SV_MAX_K) return SV_EINVAL;
    if ((int64_t)B * (K + 1) > INT_MAX) return SV_EINVAL;
    const int32_t M = B * (K + 1);
    int rc = svlm::check_gemm(hidden, w_vd, M, d, V, target_logits);
    if (rc < 0) return rc;
    if (B == 0) return SV_OK;
    // every check of the verify step runs before anything is launched
    rc = sv_verify_mixed(target_logits, draft_logits, draft_tokens, uniforms, temperature, greedy_flag, B, K,
                         V, SV_F32, draft_dtype, accepted_len, out_tokens, diag, workspace, workspace_bytes,
                         stream, 1);
    if (rc != SV_OK) return rc;
    rc = sv_lmhead(hidden, w_vd, M, d, V, target_logits, stream);
    if (rc != SV_OK) return rc;
    return sv_verify_mixed(target_logits, draft_logits, draft_tokens, uniforms, temperature, greedy_flag, B, K,
                           V, SV_F32, draft_dtype, accepted_len, out_tokens, diag, workspace, workspace_bytes,
                           stream, 0);
}

}  // extern "C"
