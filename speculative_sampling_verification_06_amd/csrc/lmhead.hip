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
// Layout: W is static, so it is packed once (k_pack) from [d, V] into MFMA
// operand tiles: tile (vt, kt) holds the 32 vocabulary columns vt*32.. and the
// 16 k values kt*16.. of W as 64 lanes x 8 bf16 in the B-operand lane order
// below (1 KB), zero past V and past d; the 8 tiles of one workgroup's 256
// columns alternate per k-tile (tile_off).  Each wave load of a weight
// fragment is one contiguous kilobyte and a workgroup's k-step reads one
// contiguous 8 KB, where reading 32 rows of W^T 32 bytes at a time left DRAM
// rows half used (351 -> 271 us for the workload above).  k_lmhead: one
// workgroup = 4 waves, one per SIMD; each wave owns two vocabulary tiles (64
// columns) and all 192 hidden rows (six 32-row tiles) of an M block, so every
// W element is read from HBM exactly once and each 16-k step issues 12
// v_mfma_f32_32x32x16_bf16 on one A fragment per tile pair (the 192
// accumulators sit in AGPRs).  Weight tiles stream into a register ring RB
// 64-k blocks deep, with non-temporal loads; the hidden states (1.5 MB,
// L2-resident) come through a double-buffered LDS block shared by the four
// waves, the next block's loads in flight while the current one is
// multiplied, and each wave reads the A fragments of the next 16-k step from
// LDS while the matrix cores work on the current one.
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
constexpr int NC = 2;             // 32-wide vocabulary tiles per wave
constexpr int WN = 32 * NC;       // vocabulary rows per wave
constexpr int WPS = 1;            // waves per SIMD the register budget allows
constexpr int BN = 4 * WN;        // per workgroup
constexpr int MT = 6;             // 32-row tiles per M block
constexpr int MB = 32 * MT;       // 192 hidden rows per M block
constexpr int TG = BN / 32;       // vocabulary tiles interleaved per k-tile in the packed weight

// Element offset of packed tile (vt, kt) for KT k-tiles: the TG tiles of one
// workgroup alternate per k-tile, so its four waves read one contiguous
// TG KB per k-step.
__host__ __device__ __forceinline__ int64_t tile_off(int vt, int kt, int KT)
{
    return (((int64_t)(vt / TG) * KT + kt) * TG + vt % TG) * 512;
}

// Barrier for the LDS hand-over only: this wave's LDS stores complete
// (lgkmcnt 0), then s_barrier.  __syncthreads() would also wait for every
// outstanding global load (vmcnt 0), draining the weight prefetch ring each
// block.  The signal fences keep the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void lds_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);    // gfx9 encoding: lgkmcnt(0), vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ uint4 and4(uint4 v, uint32_t m) { return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m); }

// Weight fragments are read once: non-temporal loads (evict first), so the
// stream does not push the hidden states, and the logits the verify step
// reads next, out of the caches.
__device__ __forceinline__ bf16x8 ld16(const uint16_t* p)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return __builtin_bit_cast(bf16x8, v);
}

// Packed offset of element (lane l, e) of tile (vt, kt): ((vt * KT + kt) * 64
// + l) * 8 + e, holding W[kt*16 + 8*(l/32) + e][vt*32 + l%32] (0 outside).
// One workgroup per (vocabulary tile, 64 k): W[k0..k0+63][v0..v0+31] through
// LDS, then four tiles written contiguously.
__global__ __launch_bounds__(256) void k_pack(const uint16_t* __restrict__ W, uint16_t* __restrict__ P,
                                              int d, int V, int KT)
{
    __shared__ uint16_t tile[64][34];
    const int vt = blockIdx.x, k0 = blockIdx.y * 64, v0 = vt * 32;
    for (int i = threadIdx.x; i < 64 * 32; i += 256) {
        const int r = i >> 5, c = i & 31;
        const int k = k0 + r, v = v0 + c;
        tile[r][c] = (k < d && v < V) ? W[(int64_t)k * V + v] : (uint16_t)0;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 4 * 512; i += 256) {
        const int q = i >> 9, l = (i >> 3) & 63, e = i & 7;    // k-tile in block, lane, element
        const int kt = blockIdx.y * 4 + q;
        if (kt < KT) P[tile_off(vt, kt, KT) + l * 8 + e] = tile[q * 16 + 8 * (l >> 5) + e][l & 31];
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
constexpr int RB = 2;                  // weight ring depth in LDS blocks
constexpr int WPF = RB * KS;           // weight prefetch depth in k-steps
static_assert(A_PIECES % NT == 0, "block pieces must split evenly");
static_assert(RB % 2 == 0, "block groups must start on an even block (hidden-state register sets alternate)");

__global__ __launch_bounds__(NT, WPS) void k_lmhead(const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wp,
                                                  float* __restrict__ out, int M, int d, int V)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][MB * A_LD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, kg = lane >> 5;
    const int n0 = blockIdx.x * BN + wave * WN;
    const int m0 = blockIdx.y * MB;
    const int nsteps = (d + 15) / 16;          // k-tiles per vocabulary tile
    const int nvt = (V + 31) / 32;
    const int nblk = (d + BK - 1) / BK;

    // this lane's fragment of each k-tile of its vocabulary tile; tiles past
    // the last read the last one (their results are not stored)
    const uint16_t* bp[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int vt = min((n0 + 32 * c) / 32, nvt - 1);
        bp[c] = Wp + tile_off(vt, 0, nsteps) + lane * 8;
    }
    // every load is issued, from an in-range address (a fixed count of loads
    // per step lets the compiler wait for exactly the ones a use needs); a
    // fragment past the last k-tile is never multiplied, so no select on the
    // loaded value (one would make the block's end wait for the whole ring)
    auto ldw = [&](int c, int step) -> bf16x8 { return ld16(bp[c] + (int64_t)(step < nsteps ? step : 0) * (TG * 512)); };
    // this thread's share of a hidden-state block: A_PER_T pieces, rows
    // ar + RP*i, columns ac .. ac+7 of the block
    constexpr int PPR = BK / 8;                                 // pieces per row
    constexpr int RP = NT / PPR;                                // rows per pass
    const int ar = tid / PPR, ac = (tid % PPR) * 8;
    const uint16_t* hs[A_PER_T];
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) hs[i] = H + (int64_t)min(m0 + ar + RP * i, M - 1) * d + ac;
    // columns past d are stored as zero (the weight's are zero there too,
    // and a finite 0 * 0 keeps a non-finite hidden value elsewhere out); the
    // select sits at the store, which waits for the loads anyway.  Two
    // register sets: a block is loaded two blocks (2*KS k-steps) before its
    // store, so the store's wait, which also covers every weight fragment
    // issued before those loads (the counter completes in issue order), asks
    // only for fragments whose k-step has come: the weight ring keeps its
    // full lead at block boundaries (one block ahead it fell to half, ~18 us
    // of the 104 us main loop at B*(K+1) = 192, d = 4096, V = 128256).
    uint4 sa[2][A_PER_T];
    uint32_t amask[2];                  // all ones while the loaded columns are below d
#define LM_LOAD_A(kb, set)                                                                     \
    do {                                                                                       \
        const bool ok_ = (kb) < nblk && (kb) * BK + ac < d;                                   \
        amask[set] = ok_ ? ~0u : 0u;                                                          \
        const int64_t o_ = ok_ ? (int64_t)(kb) * BK : 0;                                      \
        _Pragma("unroll") for (int i_ = 0; i_ < A_PER_T; ++i_)                               \
            sa[set][i_] = *reinterpret_cast<const uint4*>(hs[i_] + o_);                       \
    } while (0)
#define LM_STORE_A(buf, set)                                                                   \
    do {                                                                                       \
        uint16_t* a_ = &As[buf][ar * A_LD + ac];                                              \
        _Pragma("unroll") for (int i_ = 0; i_ < A_PER_T; ++i_)                               \
            *reinterpret_cast<uint4*>(a_ + i_ * RP * A_LD) = and4(sa[set][i_], amask[set]);   \
    } while (0)

    f32x16 acc[MT][NC];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[t][c] = f32x16{};
    bf16x8 wb[WPF][NC];
#pragma unroll
    for (int q = 0; q < WPF; ++q)
#pragma unroll
        for (int c = 0; c < NC; ++c) wb[q][c] = ldw(c, q);
    LM_LOAD_A(0, 0);
    LM_STORE_A(0, 0);
    LM_LOAD_A(1, 1);
    LM_LOAD_A(2, 0);
    __syncthreads();

    // blocks in groups of RB so every weight ring slot index is a compile-time
    // constant; the hidden-state block alternates between the two LDS buffers
    for (int kb0 = 0; kb0 < nblk; kb0 += RB) {
#pragma unroll
        for (int h = 0; h < RB; ++h) {
            const int kb = kb0 + h;
            if (kb < nblk) {
                const int buf = kb & 1;
                const uint16_t* as = As[buf] + li * A_LD + 8 * kg;
                // the A fragments of k-step ks+1 are read from LDS while the
                // matrix cores work on k-step ks
                bf16x8 af[2][MT];
#pragma unroll
                for (int t = 0; t < MT; ++t) af[0][t] = *reinterpret_cast<const bf16x8*>(as + t * 32 * A_LD);
                // all six reads go out before the first k-step's matrix ops: left
                // to itself the scheduler sank them into one register set, each
                // read then waiting on its own (GEMM 234-238 -> 228-229 us)
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int step = kb * KS + ks;
                    const int slot = h * KS + ks;
                    if (ks + 1 < KS) {
#pragma unroll
                        for (int t = 0; t < MT; ++t)
                            af[(ks + 1) & 1][t] = *reinterpret_cast<const bf16x8*>(as + t * 32 * A_LD + (ks + 1) * 16);
                    }
                    bf16x8 bc[NC];
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        bc[c] = wb[slot][c];
                        wb[slot][c] = ldw(c, step + WPF);
                    }
                    if (step < nsteps) {
#pragma unroll
                        for (int t = 0; t < MT; ++t)
#pragma unroll
                            for (int c = 0; c < NC; ++c)
                                acc[t][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][t], bc[c], acc[t][c], 0, 0, 0);
                    }
                }
                // block kb+1 (register set (kb+1) & 1 = (h+1) & 1, kb0 being
                // even) into the other buffer; every wave finished reading that
                // buffer before the previous barrier; then block kb+3 into the
                // freed set
                LM_STORE_A(buf ^ 1, (h + 1) & 1);
                lds_barrier();
                LM_LOAD_A(kb + 3, (h + 1) & 1);
            }
        }
    }

#undef LM_LOAD_A
#undef LM_STORE_A
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
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

static int check_gemm(const void* hidden, const void* w_packed, int32_t M, int32_t d, int32_t V, const float* logits)
{
    if (M < 0 || d < 8 || d % 8 != 0 || V < 1) return SV_EINVAL;
    if (M == 0) return SV_OK;
    if (!hidden || !w_packed || !logits) return SV_EINVAL;
    if (!aligned_to(hidden, 16) || !aligned_to(w_packed, 16) || !aligned_to(logits, 4)) return SV_EINVAL;
    if ((V + (int64_t)BN - 1) / BN > INT_MAX || (M + (int64_t)MB - 1) / MB > 65535) return SV_EINVAL;
    return 1;
}

}  // namespace svlm

extern "C" {

size_t sv_lmhead_packed_bytes(int32_t d, int32_t V)
{
    if (d < 1 || V < 1) return 0;
    const size_t groups = ((size_t)V + 32 * svlm::TG - 1) / (32 * svlm::TG);
    return groups * svlm::TG * (size_t)((d + 15) / 16) * 512 * sizeof(uint16_t);
}

int sv_lmhead_pack(const void* w_dv, void* w_packed, int32_t d, int32_t V, void* stream)
{
    if (d < 1 || V < 1 || !w_dv || !w_packed) return SV_EINVAL;
    if (!svlm::aligned_to(w_dv, 2) || !svlm::aligned_to(w_packed, 16)) return SV_EINVAL;
    if ((d + 63) / 64 > 65535) return SV_EINVAL;
    const dim3 grid((unsigned)((V + 31) / 32), (unsigned)((d + 63) / 64));
    sv_launch_begin();
    hipLaunchKernelGGL(svlm::k_pack, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint16_t*>(w_dv), static_cast<uint16_t*>(w_packed), d, V, (d + 15) / 16);
    return sv_launch_status();
}

int sv_lmhead(const void* hidden, const void* w_packed, int32_t M, int32_t d, int32_t V, float* logits,
              void* stream)
{
    const int rc = svlm::check_gemm(hidden, w_packed, M, d, V, logits);
    if (rc <= 0) return rc;
    const dim3 grid((unsigned)((V + svlm::BN - 1) / svlm::BN), (unsigned)((M + svlm::MB - 1) / svlm::MB));
    sv_launch_begin();
    hipLaunchKernelGGL(svlm::k_lmhead, grid, dim3(svlm::NT), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(w_packed), logits, M, d, V);
    return sv_launch_status();
}

}  // extern "C"

namespace svlm {

// spec_lmhead_verify's launches: part 1 the GEMM, part 2 the verify step on
// its logits, 3 both.  Every host check of both runs first.
static int lmhead_verify_parts(int parts, const void* hidden, const void* w_packed, int32_t d, float* target_logits,
                               const void* draft_logits, int32_t draft_dtype, const int32_t* draft_tokens,
                               const float* uniforms, float temperature, const uint8_t* greedy_flag, int32_t B,
                               int32_t K, int32_t V, int32_t* accepted_len, int32_t* out_tokens,
                               const sv_diag* diag, void* workspace, size_t workspace_bytes, void* stream)
{
    if (B < 0 || K < 0 || K > SV_MAX_K) return SV_EINVAL;
    if ((int64_t)B * (K + 1) > INT_MAX) return SV_EINVAL;
    const int32_t M = B * (K + 1);
    int rc = check_gemm(hidden, w_packed, M, d, V, target_logits);
    if (rc < 0) return rc;
    if (B == 0) return SV_OK;
    // every check of the verify step runs before anything is launched
    rc = sv_verify_mixed(target_logits, draft_logits, draft_tokens, uniforms, temperature, greedy_flag, B, K,
                         V, SV_F32, draft_dtype, accepted_len, out_tokens, diag, workspace, workspace_bytes,
                         stream, 1);
    if (rc != SV_OK) return rc;
    if (parts & 1) {
        rc = sv_lmhead(hidden, w_packed, M, d, V, target_logits, stream);
        if (rc != SV_OK) return rc;
    }
    if (!(parts & 2)) return SV_OK;
    return sv_verify_mixed(target_logits, draft_logits, draft_tokens, uniforms, temperature, greedy_flag, B, K,
                           V, SV_F32, draft_dtype, accepted_len, out_tokens, diag, workspace, workspace_bytes,
                           stream, 0);
}

}  // namespace svlm

extern "C" {

#define SV_LMV_ARGS                                                                                  \
    const void *hidden, const void *w_packed, int32_t d, float *target_logits, const void *draft_logits, \
        int32_t draft_dtype, const int32_t *draft_tokens, const float *uniforms, float temperature,     \
        const uint8_t *greedy_flag, int32_t B, int32_t K, int32_t V, int32_t *accepted_len,              \
        int32_t *out_tokens, const sv_diag *diag, void *workspace, size_t workspace_bytes, void *stream
#define SV_LMV_PASS                                                                                  \
    hidden, w_packed, d, target_logits, draft_logits, draft_dtype, draft_tokens, uniforms, temperature, \
        greedy_flag, B, K, V, accepted_len, out_tokens, diag, workspace, workspace_bytes, stream

int spec_lmhead_verify(SV_LMV_ARGS) { return svlm::lmhead_verify_parts(3, SV_LMV_PASS); }
int sv_lmhead_verify_gemm(SV_LMV_ARGS) { return svlm::lmhead_verify_parts(1, SV_LMV_PASS); }
int sv_lmhead_verify_rest(SV_LMV_ARGS) { return svlm::lmhead_verify_parts(2, SV_LMV_PASS); }

}  // extern "C"
