// spec_verify.hip - gfx950 (MI355X) kernels and C ABI of the speculative-sampling
// verify step.  Page citations ([QH], [NL], [MC]) are spelled out in
// include/spec_verify.h next to the declarations.
//
// Launches on the caller's stream; kernel boundaries are the only
// synchronisation between workgroups (no fences, no counters):
//
//   row statistics, one of two schedules:
//   k_rowstats       eager: one launch, one workgroup per (sequence b, row r,
//                    vocab chunk c); rows r = 0..K are target rows, K+1..2K
//                    draft rows.
//   k_rowstats_lazy  lazy: one launch per position j = 0..K, rows of position
//                    j only for sequences that reach j (rows past the first
//                    rejection are never read).
//                    Either way a workgroup streams its chunk once with
//                    16-byte loads (UNROLL in flight per lane); sampling rows
//                    keep an online softmax state (running max m and sum z of
//                    exp2(x*s - m*s), s = log2(e)/T), greedy rows a
//                    lowest-index argmax; one 16-byte partial per chunk.
//   k_tiles          one workgroup per (sequence, vocab tile).  Each merges
//                    its sequence's partials in chunk order, runs the K tests
//                    on wave 0 and finds the first rejection n with one
//                    ballot (tile 0 writes accepted_len, the accepted prefix,
//                    the greedy token, the diagnostics and a record for the
//                    search); sampling sequences then sum the draw weights of
//                    row n (residual max(0, p - q) scaled by Z_p, or p for the
//                    bonus) per 512-element segment.
//   k_search         one workgroup per sampling sequence: scans the segment
//                    sums for u*S, re-reads that one segment, walks it.
//
// Numerics: every term is exp2(fma(x, s, -c)) with c = m*s held as an exact
// shift, so the row's own rounding of c cancels out of every ratio; partial
// states are merged by rescaling with exp2(c_i - c), c_i the rounded shifts
// the terms were computed with (built with -ffp-contract=off so this stays
// exact).  Sums are fp32 trees (window, wave butterfly, fixed-order merges),
// never float atomics, so results are bitwise deterministic.  The max is
// NaN-propagating, so a NaN anywhere in a row turns its sum into NaN and the
// row is reported invalid.

#include <hip/hip_runtime.h>

#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "spec_verify.h"
#include "sv_internal.h"

namespace sv {

constexpr int NT = 256;               // threads per workgroup: four wave64
constexpr int NWAVE = NT / 64;
constexpr int UNROLL = 4;             // 16-byte loads in flight per lane and row
constexpr int SPW = 4;                // draw: segments per wave per tile
constexpr int SPT = NWAVE * SPW;      // draw: segments per tile
constexpr int MAXR = 2 * SV_MAX_K + 1;
constexpr float NEG_INF = -__builtin_inff();
constexpr float POS_INF = __builtin_inff();
constexpr float LN2 = 0.693147180559945309417f;

template <int DT> struct Fmt;
template <> struct Fmt<SV_F32> {
    static constexpr int E = 4, BYTES = 4;
    static constexpr uint32_t NEG_INF_WORD = 0xff800000u;
};
template <> struct Fmt<SV_BF16> {
    static constexpr int E = 8, BYTES = 2;
    static constexpr uint32_t NEG_INF_WORD = 0xff80ff80u;
};

struct Partial {      // one (row, chunk): softmax {m, z} or argmax {m = value, idx, bad}
    float m;
    float z;
    int32_t idx;
    uint32_t bad;
};

struct SeqRec {       // what tile 0 of k_tiles leaves for k_search
    int32_t n;
    int32_t status;   // 1 = sampling sequence, valid, draw pending
    float mp, zp;     // target row n
    float mq, zq;     // draft row n (n below the sequence's proposal count)
    float u;          // uniforms[b, K]
    int32_t bonus;    // n equals the proposal count: draw from p_n
    int32_t xn;       // one-hot proposals: the token proposed at n (its draft row is implicit)
    int32_t pad;
};

struct Params {
    const void* target;
    const void* draft;
    const int32_t* tokens;
    const float* uniforms;
    const uint8_t* greedy;
    int32_t* acc;
    int32_t* out;
    float* p_tok;
    float* q_tok;
    float* lse_p;
    float* lse_q;
    float* res_mass;
    Partial* part;
    SeqRec* rec;
    int32_t* reach;   // lazy mode: last position each sequence was seen alive at
    float* seg;       // [2][B][nseg]: residual sums, then p sums
    uint64_t* slots;  // grouped per-sequence schedule: tagged words the G workgroups of a sequence exchange
    uint32_t* gep;    // grouped schedule: per-sequence call counter (tags)
    int32_t B, K, V, C;
    int32_t nseg, tiles;
    int32_t G, gsegs; // grouped schedule: workgroups per sequence, segments per workgroup slice
    int32_t qd, ncu;  // grouped schedule with lookahead: sequence slots and compute units per die
                      // for the turned placement (ncu 0: the plain one)
    uint32_t salt;    // grouped schedule: shape hash folded into the tags
    uint32_t nonce;   // grouped schedule: per-call host counter folded into the tags
    int32_t spin;     // grouped schedule: polls before a wait gives up
    const int32_t* klen;  // proposals per sequence (prompt lookup), null = K for all
    int32_t onehot;   // draft distribution = one-hot at the proposed token (no draft logits)
    float s;          // log2(e) / T
};

// ---------------------------------------------------------------- helpers --

__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float shift_of(float m, float s) { return m == NEG_INF ? 0.f : m * s; }

template <int N>
__device__ __forceinline__ float tree_max(const float* x)
{
    if constexpr (N == 1) {
        return x[0];
    } else if constexpr (N == 2) {
        return vmax(x[0], x[1]);
    } else {
        constexpr int M = (N + 2) / 3;
        float a[M];
#pragma unroll
        for (int k = 0; k < N / 3; ++k) a[k] = vmax(vmax(x[3 * k], x[3 * k + 1]), x[3 * k + 2]);
        if constexpr (N % 3 == 1) a[N / 3] = x[N - 1];
        if constexpr (N % 3 == 2) a[N / 3] = vmax(x[N - 2], x[N - 1]);
        return tree_max<M>(a);
    }
}

template <int N>
__device__ __forceinline__ float tree_sum(float* t)
{
    if constexpr (N == 1) {
        return t[0];
    } else {
        constexpr int H = N / 2;
#pragma unroll
        for (int k = 0; k < H; ++k) t[k] = t[k] + t[k + (N - H)];
        return tree_sum<N - H>(t);
    }
}

template <int DT> __device__ __forceinline__ void unpack(const uint4& v, float* x);
template <> __device__ __forceinline__ void unpack<SV_F32>(const uint4& v, float* x)
{
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
}
template <> __device__ __forceinline__ void unpack<SV_BF16>(const uint4& v, float* x)
{
    x[0] = __uint_as_float(v.x << 16);
    x[1] = __uint_as_float(v.x & 0xffff0000u);
    x[2] = __uint_as_float(v.y << 16);
    x[3] = __uint_as_float(v.y & 0xffff0000u);
    x[4] = __uint_as_float(v.z << 16);
    x[5] = __uint_as_float(v.z & 0xffff0000u);
    x[6] = __uint_as_float(v.w << 16);
    x[7] = __uint_as_float(v.w & 0xffff0000u);
}

template <int DT>
__device__ __forceinline__ float load1(const char* row, int64_t i)
{
    if constexpr (DT == SV_F32) return reinterpret_cast<const float*>(row)[i];
    else return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[i] << 16);
}

// Eight consecutive elements starting at e (a multiple of 8); -inf past V.
// One 16-byte load for bf16, two for fp32, when the row is 16-byte aligned.
constexpr int LE = 8;                  // draw: elements per lane per segment
constexpr int SEG = 64 * LE;           // draw: elements per segment (one wave)

template <int DT>
__device__ __forceinline__ void load8(const char* row, int64_t e, int64_t V, bool aligned, float* x)
{
    if (aligned && e + LE <= V) {
        const uint4* p = reinterpret_cast<const uint4*>(row + e * Fmt<DT>::BYTES);
        if constexpr (DT == SV_BF16) {
            unpack<SV_BF16>(p[0], x);
        } else {
            unpack<SV_F32>(p[0], x);
            unpack<SV_F32>(p[1], x + 4);
        }
    } else {
#pragma unroll
        for (int k = 0; k < LE; ++k) x[k] = (e + k < V) ? load1<DT>(row, e + k) : NEG_INF;
    }
}

// ------------------------------------------------- online softmax / argmax --

struct SmState { float m, z; };
struct AmState { float v; int32_t i; uint32_t bad; };

__device__ __forceinline__ SmState sm_merge(SmState a, SmState b, float s)
{
    const float mn = vmax(a.m, b.m);
    const float cn = shift_of(mn, s);
    const float fa = (a.m == NEG_INF) ? 0.f : ex2(shift_of(a.m, s) - cn);
    const float fb = (b.m == NEG_INF) ? 0.f : ex2(shift_of(b.m, s) - cn);
    return {mn, __builtin_fmaf(a.z, fa, b.z * fb)};
}

__device__ __forceinline__ AmState am_merge(AmState a, AmState b)
{
    AmState r = (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
    r.bad = a.bad | b.bad;
    return r;
}

// Online softmax over one window of N elements: the running max m and the
// sum z of exp2((x - m) s), rescaled when the max moves.  KEEP: once every
// lane of the wave holds a finite m, a window's exps are taken against m as
// it stands and added (fp32 sums are scale-invariant, so this is as exact as
// rescaling, and it spares the window max and the rescale exp; m is then a
// reference at or below the max); a window whose sum is not below 2^64 on
// some lane (an element far above m, +Inf or NaN) takes the max and
// rescales.  KEEP costs registers (the window stays live through its exps).
template <int N, bool KEEP = false>
__device__ __forceinline__ void sm_window(const float* x, float s, SmState& st)
{
    if (KEEP && __all(st.m > NEG_INF && st.m < POS_INF)) {
        const float c = st.m * s;
        float t[N];
#pragma unroll
        for (int k = 0; k < N; ++k) t[k] = ex2(__builtin_fmaf(x[k], s, -c));
        const float ws = tree_sum<N>(t);
        if (__all(ws < 0x1p64f)) {
            st.z += ws;
            return;
        }
    }
    const float wm = tree_max<N>(x);
    const float mn = vmax(st.m, wm);
    const float cn = shift_of(mn, s);
    const float sc = (st.m == NEG_INF) ? 0.f : ex2(shift_of(st.m, s) - cn);
    float t[N];
#pragma unroll
    for (int k = 0; k < N; ++k) t[k] = ex2(__builtin_fmaf(x[k], s, -cn));
    const float ws = tree_sum<N>(t);
    st.z = __builtin_fmaf(st.z, sc, ws);
    st.m = mn;
}

// idx(k) gives the row index of x[k]; increasing in k.
template <int N, typename IdxF>
__device__ __forceinline__ void am_window(const float* x, IdxF idx, AmState& st)
{
    const float wm = tree_max<N>(x);
    if (wm != wm || wm == POS_INF) st.bad = 1u;
    if (wm > st.v) {
        int kk = N - 1;
#pragma unroll
        for (int k = N - 1; k >= 0; --k)
            if (x[k] == wm) kk = k;
        st.v = wm;
        st.i = (int32_t)idx(kk);
    }
}

// Stream elements [e0, e1) of one row (e0 a multiple of E) into the state;
// BT threads, U 16-byte loads in flight per lane.
template <int DT, bool GREEDY, int BT = NT, int U = UNROLL, bool KEEP = false>
__device__ __forceinline__ void scan_chunk(const char* row, int64_t e0, int64_t e1, float s,
                                           SmState& sm, AmState& am)
{
    constexpr int E = Fmt<DT>::E;
    constexpr int W = U * E;
    const int tid = threadIdx.x;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
    if (aligned) {
        const uint4* vrow = reinterpret_cast<const uint4*>(row);
        const int64_t v0 = e0 / E, v1 = e1 / E;
        for (int64_t base = v0 + tid; base < v1; base += (int64_t)BT * U) {
            uint4 raw[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t vi = base + (int64_t)u * BT;
                if (vi < v1) raw[u] = vrow[vi];
                else raw[u] = make_uint4(Fmt<DT>::NEG_INF_WORD, Fmt<DT>::NEG_INF_WORD,
                                         Fmt<DT>::NEG_INF_WORD, Fmt<DT>::NEG_INF_WORD);
            }
            float x[W];
#pragma unroll
            for (int u = 0; u < U; ++u) unpack<DT>(raw[u], x + u * E);
            if constexpr (GREEDY)
                am_window<W>(x, [base](int k) { return (base + (int64_t)(k / E) * BT) * E + (k % E); }, am);
            else
                sm_window<W, KEEP>(x, s, sm);
        }
        const int64_t t0 = v1 * E;             // ragged tail of the row (< E elements)
        if (t0 + tid < e1) {
            float x1[1] = {load1<DT>(row, t0 + tid)};
            const int64_t i1 = t0 + tid;
            if constexpr (GREEDY) am_window<1>(x1, [i1](int) { return i1; }, am);
            else sm_window<1, KEEP>(x1, s, sm);
        }
    } else {
        for (int64_t base = e0 + tid; base < e1; base += (int64_t)BT * W) {
            float x[W];
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int64_t i = base + (int64_t)k * BT;
                x[k] = (i < e1) ? load1<DT>(row, i) : NEG_INF;
            }
            if constexpr (GREEDY)
                am_window<W>(x, [base](int k) { return base + (int64_t)k * BT; }, am);
            else
                sm_window<W, KEEP>(x, s, sm);
        }
    }
}

// ------------------------------------------------------- block reductions --

// Cross-lane moves within the wave by DPP (data-parallel primitives: a VALU
// operand modifier, no LDS round trip as with ds_bpermute).  Lanes whose
// source is outside the pattern, or rows the mask leaves out, read 0.
// gfx9 DPP controls: quad_perm 0x00-0xFF, row_shr:n 0x110+n, row_mirror
// 0x140, row_half_mirror 0x141, row_bcast:15 0x142, row_bcast:31 0x143.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_i(int v, int old)
{
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp(float v, float old = 0.f)
{
    return __builtin_bit_cast(float, dpp_i<CTRL, ROW_MASK>(__builtin_bit_cast(int, v), __builtin_bit_cast(int, old)));
}
// lane l's value on every lane (l uniform over the wave)
__device__ __forceinline__ float lane_f(float v, int l)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ int lane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// The reduction order every cross-lane merge below uses: lane ^ 1, lane ^ 2,
// the other quad of the half row, the other half of the row, rows 0 + 1 and
// 2 + 3, then the two halves; the result is lane 63's, read by every lane.
// A lane whose partner a row broadcast leaves out merges the identity.

// Softmax states {max, sum} merged over the wave.
__device__ __forceinline__ SmState wave_reduce_sm(SmState v, float s)
{
    v = sm_merge(v, {dpp<0xb1>(v.m, NEG_INF), dpp<0xb1>(v.z)}, s);
    v = sm_merge(v, {dpp<0x4e>(v.m, NEG_INF), dpp<0x4e>(v.z)}, s);
    v = sm_merge(v, {dpp<0x141>(v.m, NEG_INF), dpp<0x141>(v.z)}, s);
    v = sm_merge(v, {dpp<0x140>(v.m, NEG_INF), dpp<0x140>(v.z)}, s);
    v = sm_merge(v, {dpp<0x142, 0xa>(v.m, NEG_INF), dpp<0x142, 0xa>(v.z)}, s);
    v = sm_merge(v, {dpp<0x143, 0xc>(v.m, NEG_INF), dpp<0x143, 0xc>(v.z)}, s);
    return {lane_f(v.m, 63), lane_f(v.z, 63)};
}

// Greedy states {max, lowest index of the max, invalid flag} merged over the
// wave (the merge is symmetric, so the order only fixes the work).
__device__ __forceinline__ AmState wave_reduce_am(AmState v)
{
#define SV_AM_STEP(CTRL, MASK)                                                                     \
    v = am_merge(v, {dpp<CTRL, MASK>(v.v, NEG_INF), dpp_i<CTRL, MASK>(v.i, INT_MAX),              \
                     (uint32_t)dpp_i<CTRL, MASK>((int)v.bad, 0)})
    SV_AM_STEP(0xb1, 0xf);
    SV_AM_STEP(0x4e, 0xf);
    SV_AM_STEP(0x141, 0xf);
    SV_AM_STEP(0x140, 0xf);
    SV_AM_STEP(0x142, 0xa);
    SV_AM_STEP(0x143, 0xc);
#undef SV_AM_STEP
    return {lane_f(v.v, 63), lane_i(v.i, 63), (uint32_t)lane_i((int)v.bad, 63)};
}

// Workgroup of BT threads; sh holds BT/64 states.  Every thread returns the
// waves' states merged in wave order.
template <int BT = NT>
__device__ __forceinline__ SmState block_reduce_sm(SmState v, float s, SmState* sh)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_reduce_sm(v, s);
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    SmState r = sh[0];
#pragma unroll
    for (int w = 1; w < BT / 64; ++w) r = sm_merge(r, sh[w], s);
    return r;
}

template <int BT = NT>
__device__ __forceinline__ AmState block_reduce_am(AmState v, AmState* sh)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_reduce_am(v);
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    AmState r = sh[0];
#pragma unroll
    for (int w = 1; w < BT / 64; ++w) r = am_merge(r, sh[w]);
    return r;
}

// Sum over the wave in a fixed order (pairs, quads, half rows, rows, then
// rows 0+1 and 2+3, then the two halves); every lane gets the total.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp<0xb1>(v);                  // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp<0x4e>(v);                  // quad_perm [2,3,0,1]: lane ^ 2
    v += dpp<0x141>(v);                 // row_half_mirror: the other quad of the half row
    v += dpp<0x140>(v);                 // row_mirror: the other half of the row
    v += dpp<0x142, 0xa>(v);            // rows 1, 3 += last lane of rows 0, 2
    v += dpp<0x143, 0xc>(v);            // rows 2, 3 += lane 31 (rows 0 + 1)
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Largest value over the wave (NaN-propagating), the same butterfly as wave_sum.
__device__ __forceinline__ float wave_max(float v)
{
    v = vmax(v, dpp<0xb1>(v, NEG_INF));
    v = vmax(v, dpp<0x4e>(v, NEG_INF));
    v = vmax(v, dpp<0x141>(v, NEG_INF));
    v = vmax(v, dpp<0x140>(v, NEG_INF));
    v = vmax(v, dpp<0x142, 0xa>(v, NEG_INF));
    v = vmax(v, dpp<0x143, 0xc>(v, NEG_INF));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Inclusive scan over the wave (lane order): within each row of 16 lanes by
// shifts of 1, 2, 4 and 8, then the rows' totals carried forward.
__device__ __forceinline__ float wave_incl_scan(float v)
{
    v += dpp<0x111>(v);                 // row_shr:1
    v += dpp<0x112>(v);                 // row_shr:2
    v += dpp<0x114>(v);                 // row_shr:4
    v += dpp<0x118>(v);                 // row_shr:8
    v += dpp<0x142, 0xa>(v);            // rows 1, 3 += total of rows 0, 2
    v += dpp<0x143, 0xc>(v);            // rows 2, 3 += total of rows 0, 1
    return v;
}

// Inclusive scan over a workgroup of BT threads; *total gets the sum of all
// BT values.  sh holds BT/64 floats.
template <int BT = NT>
__device__ __forceinline__ float block_incl_scan(float v, float* sh, float* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_incl_scan(v);
    if (lane == 63) sh[wave] = v;
    __syncthreads();
    float off = 0.f, tot = 0.f;
#pragma unroll
    for (int w = 0; w < BT / 64; ++w) {
        if (w < wave) off += sh[w];
        tot += sh[w];
    }
    __syncthreads();
    *total = tot;
    return v + off;
}

template <int DT>
__device__ __forceinline__ const char* target_row(const Params& P, int b, int j)
{
    return reinterpret_cast<const char*>(P.target) +
           ((int64_t)b * (P.K + 1) + j) * (int64_t)P.V * Fmt<DT>::BYTES;
}
template <int DT>
__device__ __forceinline__ const char* draft_row(const Params& P, int b, int j)
{
    return reinterpret_cast<const char*>(P.draft) +
           ((int64_t)b * P.K + j) * (int64_t)P.V * Fmt<DT>::BYTES;
}

__device__ __forceinline__ void put(float* a, int64_t i, float v) { if (a) a[i] = v; }

// --------------------------------------------- k_rowstats: one row chunk --

template <int DT>
__device__ __forceinline__ void rowstats_body(const Params& P, const char* row, int64_t e0, int64_t e1,
                                              bool greedy, Partial* dst, SmState* sh_sm, AmState* sh_am)
{
    SmState sm = {NEG_INF, 0.f};
    AmState am = {NEG_INF, INT_MAX, 0u};
    if (greedy) {
        if (e0 < e1) scan_chunk<DT, true>(row, e0, e1, P.s, sm, am);
        am = block_reduce_am(am, sh_am);
        if (threadIdx.x == 0) *dst = {am.v, 0.f, am.i, am.bad};
    } else {
        if (e0 < e1) scan_chunk<DT, false, NT, UNROLL, true>(row, e0, e1, P.s, sm, am);
        sm = block_reduce_sm(sm, P.s, sh_sm);
        if (threadIdx.x == 0) *dst = {sm.m, sm.z, 0, 0u};
    }
}

// Chunk c of a row covers [c*cl, min((c+1)*cl, V)), cl a multiple of 8 elements.
__device__ __forceinline__ int64_t chunk_len(int V, int C)
{
    const int64_t n8 = ((int64_t)V + 7) / 8;
    return ((n8 + C - 1) / C) * 8;
}

// Six waves per SIMD for the bf16 row streams (80 registers): the merges at
// the end would otherwise cost a wave per SIMD for a few registers.
template <int DTT, int DTD>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(6, 8))) void k_rowstats(const Params P)
{
    const int K = P.K, R = 2 * K + 1;
    const int per_seq = R * P.C;
    const int b = blockIdx.x / per_seq;
    const int rem = blockIdx.x - b * per_seq;
    const int r = rem / P.C;
    const int c = rem - r * P.C;
    const bool greedy = P.greedy != nullptr && P.greedy[b] != 0;
    const bool is_draft = r > K;
    __shared__ SmState sh_sm[NWAVE];
    __shared__ AmState sh_am[NWAVE];

    if (is_draft && (greedy || P.draft == nullptr)) return;      // never read
    if (!is_draft && P.klen) {                                   // rows past the proposals: never examined
        const int kb = P.klen[b];
        if (kb < 0 || kb > K || r > kb) return;
    }
    const int64_t cl = chunk_len(P.V, P.C);
    const int64_t e0 = (int64_t)c * cl;
    const int64_t e1 = e0 + cl < (int64_t)P.V ? e0 + cl : (int64_t)P.V;
    Partial* dst = P.part + ((int64_t)b * R + r) * P.C + c;
    if (is_draft)
        rowstats_body<DTD>(P, draft_row<DTD>(P, b, r - K - 1), e0, e1, false, dst, sh_sm, sh_am);
    else
        rowstats_body<DTT>(P, target_row<DTT>(P, b, r), e0, e1, greedy, dst, sh_sm, sh_am);
}

// ------------------------------------------ decide: n for one sequence --

struct Decision {
    int32_t n;
    int32_t ok;       // valid sequence
    float mp, zp, mq, zq, u;
};

// Merged statistics of one row.
struct RowStat {
    float m, z;       // softmax: running max and sum; greedy: max value (z unused)
    int32_t i;        // greedy: lowest index of the max
    int32_t ok;       // row valid
};

__device__ __forceinline__ RowStat rowstat_am(const AmState& am)
{
    return {am.v, 0.f, am.i, (am.bad == 0u) && am.v > NEG_INF && am.v < POS_INF};
}

__device__ __forceinline__ RowStat rowstat_sm(const SmState& sm)
{
    return {sm.m, sm.z, 0, (sm.z > 0.f) && (sm.z < POS_INF) && sm.m > NEG_INF && sm.m < POS_INF};
}

// Partials are loaded sixteen at a time (independent loads, one round trip
// for rows of up to 16 chunks: the fused LM-head verify's rows have 12, and
// its decision then waits one round trip less: 43.8 -> 43.2 us per verify)
// and merged in chunk order, so every caller gets the same bits.
constexpr int MERGE_BATCH = 16;

__device__ __forceinline__ RowStat merge_row(const Partial* pp, int C, float s, bool greedy)
{
    AmState am = {NEG_INF, INT_MAX, 0u};
    SmState sm = {NEG_INF, 0.f};
    for (int c0 = 0; c0 < C; c0 += MERGE_BATCH) {
        Partial t[MERGE_BATCH];
#pragma unroll
        for (int u = 0; u < MERGE_BATCH; ++u)
            if (c0 + u < C) t[u] = pp[c0 + u];
#pragma unroll
        for (int u = 0; u < MERGE_BATCH; ++u) {
            if (c0 + u < C) {
                if (greedy) am = am_merge(am, {t[u].m, t[u].idx, t[u].bad});
                else sm = sm_merge(sm, {t[u].m, t[u].z}, s);
            }
        }
    }
    return greedy ? rowstat_am(am) : rowstat_sm(sm);
}

struct TestOut {
    bool stop, inval;
    float ptok, qtok;
};

// What the test at position j reads besides the row statistics: the draft
// token x, its uniform u, and the target and draft logits at x.  For j = K
// only u (the draw's uniform) is meaningful.
struct TestIn {
    int32_t x;
    float u, lx, dx;
};

// The test at position j (j < K): greedy keeps x_j iff it is the lowest-index
// argmax of target row j; sampling keeps it iff u_j * q_j(x_j) < p_j(x_j).
// stop = rejected or invalid.  t, d: merged target row j and draft row j; lx
// and dx are read only when the test is valid.
__device__ __forceinline__ TestOut test_from(int V, float s, bool greedy, const RowStat& t, const RowStat& d,
                                             int32_t x, float u, float lx, float dx)
{
    TestOut o = {true, true, NAN, NAN};
    const bool tok_ok = x >= 0 && x < V;
    if (greedy) {
        o.inval = !(t.ok && tok_ok);
        o.stop = o.inval || x != t.i;
        return o;
    }
    const bool u_ok = u >= 0.f && u < 1.f;
    o.inval = !(t.ok && d.ok && tok_ok && u_ok);
    if (o.inval) return o;
    o.ptok = ex2(__builtin_fmaf(lx, s, -shift_of(t.m, s))) / t.z;
    o.qtok = ex2(__builtin_fmaf(dx, s, -shift_of(d.m, s))) / d.z;
    o.stop = !(u * o.qtok < o.ptok);
    return o;
}

template <int DTT, int DTD>
__device__ __forceinline__ TestOut position_test(const Params& P, int b, int j, bool greedy, const RowStat& t,
                                                 const RowStat& d, int32_t x, float u)
{
    float lx = 0.f, dx = 0.f;                      // one-hot proposals: the draft logit at x is 0
    if (!greedy && t.ok && d.ok && x >= 0 && x < P.V && u >= 0.f && u < 1.f) {
        lx = load1<DTT>(target_row<DTT>(P, b, j), x);
        if (!P.onehot) dx = load1<DTD>(draft_row<DTD>(P, b, j), x);
    }
    return test_from(P.V, P.s, greedy, t, d, x, u, lx, dx);
}

// Test inputs of position j <= K, loaded before the row statistics exist (the
// logits at x are read whenever x is in range).
template <int DTT, int DTD>
__device__ __forceinline__ TestIn load_test_in(const Params& P, int b, int j, bool greedy)
{
    const int K = P.K;
    TestIn r = {-1, 0.f, 0.f, 0.f};
    if (!greedy) r.u = P.uniforms[(int64_t)b * (K + 1) + j];
    if (j < K) {
        r.x = P.tokens[(int64_t)b * K + j];
        if (!greedy && r.x >= 0 && r.x < P.V) {
            r.lx = load1<DTT>(target_row<DTT>(P, b, j), r.x);
            if (P.draft && !P.onehot) r.dx = load1<DTD>(draft_row<DTD>(P, b, j), r.x);
        }
    }
    return r;
}

// Runs the K tests on wave 0 from the merged row statistics f_rs (target rows
// 0..K, then draft rows 0..K-1) and finds the first rejection n with one
// ballot; every workgroup that needs n reaches the same result bit for bit.
// Rows past the first rejection may hold anything: only examined positions
// matter.  ti: test inputs already loaded (K+1 entries), or null to load them
// here.  With write_out, also writes accepted_len, the accepted prefix, the
// greedy token, the diagnostics and the record the search launch reads;
// draw_here leaves out_tokens[b, n] and res_mass of a sampling sequence to a
// draw in the same workgroup.  Every thread must call it; *dec is valid for
// all threads on return.
// RAGGED: per-sequence proposal counts P.klen (prompt lookup); compiled out
// of the plain verify step.
template <int DTT, int DTD, bool RAGGED = false>
__device__ void decide_core(const Params& P, int b, bool greedy, bool write_out, bool draw_here,
                            const RowStat* f_rs, const TestIn* ti, Decision* dec, bool acc_by_draw = false)
{
    const int K = P.K;
    const float s = P.s;
    const int tid = threadIdx.x;

    if (tid < 64) {
        const int j = tid;
        const int64_t ub = (int64_t)b * (K + 1);
        // proposals of this sequence: K, or its own count (prompt lookup)
        const int Kb = RAGGED ? P.klen[b] : K;
        const bool kb_bad = RAGGED && (Kb < 0 || Kb > K);
        bool stop = false, inval = false;
        float ptok = NAN, qtok = NAN;
        int32_t x = -1;
        if (j < K && (kb_bad || j >= Kb)) {
            stop = true;                           // past the proposals: no test
        } else if (j < K) {
            TestOut o;
            if (ti) {
                x = ti[j].x;
                o = test_from(P.V, s, greedy, f_rs[j], f_rs[K + 1 + j], x, ti[j].u, ti[j].lx, ti[j].dx);
            } else {
                x = P.tokens[(int64_t)b * K + j];
                const float u = greedy ? 0.f : P.uniforms[ub + j];
                o = position_test<DTT, DTD>(P, b, j, greedy, f_rs[j], f_rs[K + 1 + j], x, u);
            }
            stop = o.stop;
            inval = o.inval;
            ptok = o.ptok;
            qtok = o.qtok;
        }
        const uint64_t smask = __ballot(stop);
        const uint64_t imask = __ballot(inval);
        const int n = smask ? (__ffsll((unsigned long long)smask) - 1) : K;
        bool bad = kb_bad || ((n < K) && ((imask >> n) & 1ull));
        const bool at_end = n == Kb;               // every proposal accepted: the bonus row
        float uK = 0.f;
        if (!bad && at_end) bad = !f_rs[n].ok;
        if (!bad && !greedy) {
            uK = ti ? ti[K].u : P.uniforms[ub + K];
            bad = !(uK >= 0.f && uK < 1.f);
        }
        if (j == 0) {
            dec->n = n;
            dec->ok = !bad;
            dec->mp = bad || greedy ? 0.f : f_rs[n].m;
            dec->zp = bad || greedy ? 1.f : f_rs[n].z;
            dec->mq = (bad || greedy || at_end) ? 0.f : f_rs[K + 1 + n].m;
            dec->zq = (bad || greedy || at_end) ? 1.f : f_rs[K + 1 + n].z;
            dec->u = uK;
        }
        if (write_out) {
            int32_t* out = P.out + ub;
            if (bad) {
                if (j <= K) out[j] = -1;
                if (j < K) {
                    put(P.p_tok, (int64_t)b * K + j, NAN);
                    put(P.q_tok, (int64_t)b * K + j, NAN);
                    put(P.lse_q, (int64_t)b * K + j, NAN);
                }
                if (j <= K) put(P.lse_p, ub + j, NAN);
                if (j == 0) {
                    P.acc[b] = -1;
                    put(P.res_mass, b, NAN);
                }
            } else {
                const bool drawn_later = draw_here && !greedy && j == n;
                if (j <= K && !drawn_later) out[j] = (j < n) ? x : ((j == n && greedy) ? f_rs[n].i : -1);
                const bool seen = !greedy && j <= n;
                const bool seen_q = seen && j < Kb;      // draft row j examined (tested)
                if (j < K) {
                    put(P.p_tok, (int64_t)b * K + j, seen ? ptok : NAN);
                    put(P.q_tok, (int64_t)b * K + j, seen ? qtok : NAN);
                    put(P.lse_q, (int64_t)b * K + j,
                        seen_q ? (shift_of(f_rs[K + 1 + j].m, s) + log2f(f_rs[K + 1 + j].z)) * LN2 : NAN);
                }
                if (j <= K) put(P.lse_p, ub + j, seen ? (shift_of(f_rs[j].m, s) + log2f(f_rs[j].z)) * LN2 : NAN);
                if (j == 0) {
                    if (greedy || !acc_by_draw) P.acc[b] = n;
                    if (greedy) put(P.res_mass, b, 0.f);
                }
            }
            if (j == n && !draw_here) {           // lane n holds x_n
                SeqRec r;
                r.n = n;
                r.status = (!bad && !greedy) ? 1 : 0;
                r.mp = f_rs[n].m;
                r.zp = greedy ? 1.f : f_rs[n].z;
                r.mq = (greedy || at_end) ? 0.f : f_rs[K + 1 + n].m;
                r.zq = (greedy || at_end) ? 1.f : f_rs[K + 1 + n].z;
                r.u = uK;
                r.bonus = at_end ? 1 : 0;
                r.xn = x;
                r.pad = 0;
                P.rec[b] = r;
            }
        }
    }
    __syncthreads();
}

// Merges the sequence's chunk partials into row statistics, then decides.
// The last wave loads the tests' inputs (tokens, uniforms, the two logits at
// each token) while the rows merge, so the decision waits for one round trip
// instead of two after the merge.
template <int DTT, int DTD>
__device__ void decide_seq(const Params& P, int b, bool greedy, bool write_out, Decision* dec)
{
    const int K = P.K, C = P.C, R = 2 * K + 1;
    const int tid = threadIdx.x;
    __shared__ RowStat f_rs[MAXR];
    __shared__ TestIn ti[SV_MAX_K + 1];

    const int tw = (NWAVE - 1) * 64;               // R <= 127 rows merge on the waves before it
    if (tid >= tw && tid - tw <= K) {
        const int j = tid - tw;
        // prompt lookup: positions at or past the sequence's own count are
        // never tested (their proposals and rows stay unread)
        const int kb = P.klen ? P.klen[b] : K;
        const bool tested = j == K || (kb >= 0 && kb <= K && j < kb);
        ti[j] = tested ? load_test_in<DTT, DTD>(P, b, j, greedy) : TestIn{-1, 0.f, 0.f, 0.f};
    }
    if (tid < R) {
        const Partial* pp = P.part + ((int64_t)b * R + tid) * C;
        const bool draft_row_ = tid > K;
        if (draft_row_ && P.onehot) f_rs[tid] = {0.f, 1.f, 0, 1};   // logit 0 at x_j, -inf elsewhere
        else if (draft_row_ && (greedy || P.draft == nullptr)) f_rs[tid] = {0.f, 0.f, 0, 0};
        else f_rs[tid] = merge_row(pp, C, P.s, greedy);
    }
    __syncthreads();
    if (P.klen) decide_core<DTT, DTD, true>(P, b, greedy, write_out, false, f_rs, ti, dec);
    else decide_core<DTT, DTD, false>(P, b, greedy, write_out, false, f_rs, ti, dec);
}

// --------------------------- k_rowstats_lazy: position j, live rows only --
//
// Lazy mode streams position j only for sequences that reach it, in one launch
// per position (j = 0..K): the method never examines rows after the first
// rejection, so they are never read.  Grid: B x (2 rows, or 1 at j = K) x C.
// A workgroup first settles whether its sequence reaches j: reach[b] (written
// by launch j-1) says position j-1 was streamed, and thread 0 re-runs the test
// at j-1 from that position's partials with the same merge and test code
// k_tiles uses, so the two can never disagree.

template <int DTT, int DTD>
__device__ bool reaches(const Params& P, int b, int j, bool greedy)
{
    if (j == 0) return true;
    // most sequences are gone after a few positions: one load settles those
    if (P.reach[b] < j - 1) return false;
    const int K = P.K, C = P.C, R = 2 * K + 1, jp = j - 1;
    // independent loads together: token, uniform and the partials
    const int32_t x = P.tokens[(int64_t)b * K + jp];
    const float u = greedy ? 0.f : P.uniforms[(int64_t)b * (K + 1) + jp];
    const RowStat t = merge_row(P.part + ((int64_t)b * R + jp) * C, C, P.s, greedy);
    RowStat d = {0.f, 0.f, 0, 0};
    if (!greedy && P.draft != nullptr) d = merge_row(P.part + ((int64_t)b * R + K + 1 + jp) * C, C, P.s, false);
    return !position_test<DTT, DTD>(P, b, jp, greedy, t, d, x, u).stop;
}

template <int DTT, int DTD>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(6, 8))) void k_rowstats_lazy(const Params P, const int j)
{
    const int K = P.K, R = 2 * K + 1;
    const int Rj = j < K ? 2 : 1;
    const int per_seq = Rj * P.C;
    const int b = blockIdx.x / per_seq;
    const int rem = blockIdx.x - b * per_seq;
    const int r = rem / P.C;                       // 0: target row j, 1: draft row j
    const int c = rem - r * P.C;
    const bool greedy = P.greedy != nullptr && P.greedy[b] != 0;
    __shared__ SmState sh_sm[NWAVE];
    __shared__ AmState sh_am[NWAVE];
    __shared__ int sh_go;

    if (r == 1 && (greedy || P.draft == nullptr)) return;       // never read
    if (threadIdx.x == 0) sh_go = reaches<DTT, DTD>(P, b, j, greedy) ? 1 : 0;
    __syncthreads();
    if (!sh_go) return;
    if (threadIdx.x == 0 && r == 0 && c == 0) P.reach[b] = j;

    const int64_t cl = chunk_len(P.V, P.C);
    const int64_t e0 = (int64_t)c * cl;
    const int64_t e1 = e0 + cl < (int64_t)P.V ? e0 + cl : (int64_t)P.V;
    const int row = r == 0 ? j : K + 1 + j;
    Partial* dst = P.part + ((int64_t)b * R + row) * P.C + c;
    if (r == 1)
        rowstats_body<DTD>(P, draft_row<DTD>(P, b, j), e0, e1, false, dst, sh_sm, sh_am);
    else
        rowstats_body<DTT>(P, target_row<DTT>(P, b, j), e0, e1, greedy, dst, sh_sm, sh_am);
}

// ----------------------------------------------------- draw: final token --

// Draw weight of one element: residual max(0, p - q) scaled by Z_p, or p*Z_p.
__device__ __forceinline__ float weight(float l, float d, float s, float cp, float cq, float w, int mode)
{
    const float ep = ex2(__builtin_fmaf(l, s, -cp));
    if (mode != 0) return ep;                       // bonus row or p fallback
    const float eq = ex2(__builtin_fmaf(d, s, -cq));
    return fmaxf(0.f, __builtin_fmaf(-w, eq, ep));
}

// Draw inputs of a one-hot draft row (all of q on the proposed token x): -inf
// (q = 0) away from x; at x the residual max(0, p(x) - 1) is exactly 0, which
// +inf gives in weight() (fma(-w, +inf, e_p) = -inf, then max with 0), free
// of the rounding of Z_p.
__device__ __forceinline__ void onehot8(int64_t e, int32_t x, float* xd)
{
#pragma unroll
    for (int k = 0; k < LE; ++k) xd[k] = (e + k == (int64_t)x) ? POS_INF : NEG_INF;
}

// k_decide: one workgroup per sequence settles n and writes the outputs and
// the record the draw launches read.
template <int DTT, int DTD>
__global__ __launch_bounds__(NT) void k_decide(const Params P)
{
    const int b = blockIdx.x;
    const bool greedy = P.greedy != nullptr && P.greedy[b] != 0;
    __shared__ Decision dec;
    decide_seq<DTT, DTD>(P, b, greedy, true, &dec);
}

// k_tiles: one workgroup per (sequence b, vocabulary tile t of NWAVE*SW segments): the draw
// weights of row n (residual max(0, p - q) scaled by Z_p, or p for the bonus)
// summed per segment of 64*8 elements (one per wave iteration).  DECIDE:
// every workgroup of a sampling sequence first settles the sequence's
// decision itself (the merge of its partials and the tests, a few
// microseconds; tile 0 of every sequence writes the outputs and the record
// k_search reads), in place of a k_decide launch; worth it while the grid
// fits the device at once, since each workgroup pays the decision.
// Otherwise the record k_decide left says what to draw.
template <int DTT, int DTD, bool DECIDE, int SW = SPW>
__global__ __launch_bounds__(NT) void k_tiles(const Params P)
{
    const int b = blockIdx.x / P.tiles;
    const int t = blockIdx.x - b * P.tiles;
    int n;
    bool bonus;
    float mp, zp, mq, zq;
    int32_t xn;
    if constexpr (DECIDE) {
        const bool greedy = P.greedy != nullptr && P.greedy[b] != 0;
        if (t != 0 && greedy) return;              // nothing to draw, outputs from tile 0
        __shared__ Decision dec;
        decide_seq<DTT, DTD>(P, b, greedy, t == 0, &dec);
        if (greedy || !dec.ok) return;             // uniform across the workgroup
        n = dec.n;
        bonus = n == (P.klen ? P.klen[b] : P.K);   // valid sequence: the count is in [0, K]
        mp = dec.mp; zp = dec.zp; mq = dec.mq; zq = dec.zq;
        xn = (P.onehot && !bonus) ? P.tokens[(int64_t)b * P.K + n] : -1;
    } else {
        const SeqRec rec = P.rec[b];
        if (rec.status != 1) return;               // greedy, invalid: nothing to draw
        n = rec.n;
        bonus = rec.bonus != 0;
        mp = rec.mp; zp = rec.zp; mq = rec.mq; zq = rec.zq;
        xn = rec.xn;
    }

    const int V = P.V, nseg = P.nseg;
    const float s = P.s;
    const bool oh = P.onehot != 0;
    const char* trow = target_row<DTT>(P, b, n);
    const char* drow = (bonus || oh) ? nullptr : draft_row<DTD>(P, b, n);
    const float cp = shift_of(mp, s);
    const float cq = bonus ? 0.f : shift_of(mq, s);
    const float w = bonus ? 0.f : zp / zq;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool t_al = (reinterpret_cast<uintptr_t>(trow) & 15u) == 0;
    const bool d_al = drow != nullptr && (reinterpret_cast<uintptr_t>(drow) & 15u) == 0;

    float xl[SW][LE], xd[SW][LE];
#pragma unroll
    for (int k = 0; k < SW; ++k) {
        const int seg = t * (NWAVE * SW) + wave * SW + k;
        const int64_t e = (int64_t)seg * SEG + (int64_t)lane * LE;
        load8<DTT>(trow, e, V, t_al, xl[k]);
        if (!bonus) {
            if (oh) onehot8(e, xn, xd[k]);
            else load8<DTD>(drow, e, V, d_al, xd[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < SW; ++k) {
        const int seg = t * (NWAVE * SW) + wave * SW + k;
        float sr = 0.f, sp = 0.f;
#pragma unroll
        for (int q = 0; q < LE; ++q) {
            const float ep = ex2(__builtin_fmaf(xl[k][q], s, -cp));
            sp += ep;
            sr += bonus ? ep : weight(xl[k][q], xd[k][q], s, cp, cq, w, 0);
        }
        sr = wave_sum(sr);
        sp = wave_sum(sp);
        if (lane == 0 && seg < nseg) {
            P.seg[(int64_t)b * nseg + seg] = sr;
            P.seg[((int64_t)P.B + b) * nseg + seg] = sp;
        }
    }
}

// Where the draw lands: the segment g holding u*S and the weight before it.
struct Pick {
    int mode;         // 0 residual, 1 bonus row p, 2 p fallback (residual rounded to nothing)
    int g;            // segment, -1 if no segment has positive weight
    bool overrun;     // rounding put u*S past the total: last positive weight
    float S, thr, lo;
};

struct Locate {
    int g;            // segment, -1 if none has positive weight
    bool overrun;     // no running sum exceeded thr: g is the last positive segment
    float lo;         // running sum before g
};

// First segment with positive weight whose running sum exceeds thr (chunked
// block scans of BT values, the order the totals are taken in); only
// segments with positive weight can hit, so rounding in the tree prefix never
// picks an empty one.  Without a hit: the last segment with positive weight.
// sh_scan and sh_seg hold BT/64 entries.  The sums may sit in global memory
// or LDS.
template <int BT>
__device__ Locate locate_segment(const float* sums, int nseg, float thr, float* sh_scan, int* sh_seg, float* sh_lo)
{
    constexpr int NW = BT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int g = -1;
    float lo = 0.f;
    float off = 0.f;
    for (int base = 0; base < nseg; base += BT) {
        const float v = (base + tid < nseg) ? sums[base + tid] : 0.f;
        float tot;
        const float incl = block_incl_scan<BT>(v, sh_scan, &tot);
        const bool hit = (base + tid < nseg) && v > 0.f && (off + incl > thr);
        const uint64_t m = __ballot(hit);
        if (lane == 0) sh_seg[wave] = m ? base + wave * 64 + (__ffsll((unsigned long long)m) - 1) : INT_MAX;
        __syncthreads();
        int best = INT_MAX;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) best = min(best, sh_seg[w2]);
        if (best != INT_MAX) {                    // uniform across the workgroup
            if (base + tid == best) sh_lo[0] = off + (incl - v);
            __syncthreads();
            g = best;
            lo = sh_lo[0];
            break;
        }
        off += tot;
        __syncthreads();
    }
    const bool overrun = g < 0;
    if (overrun) {
        for (int base = ((nseg - 1) / BT) * BT; base >= 0 && g < 0; base -= BT) {
            const bool pos = (base + tid < nseg) && sums[base + tid] > 0.f;
            const uint64_t m = __ballot(pos);
            if (lane == 0) sh_seg[wave] = m ? base + wave * 64 + (63 - __clzll((long long)m)) : -1;
            __syncthreads();
            int bestl = -1;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) bestl = max(bestl, sh_seg[w2]);
            g = bestl;
            __syncthreads();
        }
    }
    return {g, overrun, lo};
}

// Total weight of the segment sums: residual sums_r, or p sums sums_p when
// the residual rounded to nothing; then the segment holding u*S.  first_r:
// this thread's entry of the first BT residual sums when the caller already
// loaded it (NAN: not loaded).
template <int BT>
__device__ Pick find_segment(const float* sums_r, const float* sums_p, int nseg, float u, bool bonus,
                             float* sh_scan, int* sh_seg, float* sh_lo, float first_r = NAN)
{
    const int tid = threadIdx.x;
    Pick pk;
    float S = 0.f;
    for (int base = 0; base < nseg; base += BT) {
        const float v = (base == 0 && !(first_r != first_r)) ? first_r
                                                            : ((base + tid < nseg) ? sums_r[base + tid] : 0.f);
        float tot;
        block_incl_scan<BT>(v, sh_scan, &tot);
        S += tot;
    }
    pk.mode = bonus ? 1 : 0;
    const float* sums = sums_r;
    if (!(S > 0.f)) {                              // residual rounded to nothing: draw from p_n
        pk.mode = 2;
        sums = sums_p;
        S = 0.f;
        for (int base = 0; base < nseg; base += BT) {
            const float v = (base + tid < nseg) ? sums[base + tid] : 0.f;
            float tot;
            block_incl_scan<BT>(v, sh_scan, &tot);
            S += tot;
        }
    }
    const float thr = u * S;
    const Locate L = locate_segment<BT>(sums, nseg, thr, sh_scan, sh_seg, sh_lo);
    pk.g = L.g;
    pk.overrun = L.overrun;
    pk.S = S;
    pk.thr = thr;
    pk.lo = L.lo;
    return pk;
}

// One segment on one wave: lane exclusive prefix, then an in-lane walk.  Only
// a positive weight can be chosen; a segment with a positive sum always holds
// one.  Returns the drawn index on every lane.

// ox >= 0: the draft row is one-hot at token ox (drow unused).
template <int DTT, int DTD>
__device__ int walk_segment(const char* trow, const char* drow, int V, const Pick& pk, float s, float cp,
                            float cq, float w, int32_t ox = -1)
{
    const int lane = threadIdx.x & 63;
    const bool t_al = (reinterpret_cast<uintptr_t>(trow) & 15u) == 0;
    const bool d_al = drow != nullptr && (reinterpret_cast<uintptr_t>(drow) & 15u) == 0;
    const int g = pk.g, mode = pk.mode;
    const int64_t e = (int64_t)g * SEG + (int64_t)lane * LE;
    float xl[LE], xd[LE], wv[LE];
    load8<DTT>(trow, e, V, t_al, xl);
    if (mode == 0) {
        if (ox >= 0) onehot8(e, ox, xd);
        else load8<DTD>(drow, e, V, d_al, xd);
    }
    float ls = 0.f;
#pragma unroll
    for (int k = 0; k < LE; ++k) {
        wv[k] = weight(xl[k], mode == 0 ? xd[k] : 0.f, s, cp, cq, w, mode);
        ls += wv[k];
    }
    const float incl = wave_incl_scan(ls);
    const float thr2 = pk.thr - pk.lo;
    float run = incl - ls;
    int cand = -1;
#pragma unroll
    for (int k = 0; k < LE; ++k) {
        run += wv[k];
        if (cand < 0 && wv[k] > 0.f && run > thr2) cand = k;
    }
    const uint64_t m = pk.overrun ? 0ull : __ballot(cand >= 0);
    if (m) {
        const int L = __ffsll((unsigned long long)m) - 1;
        return (int)((int64_t)g * SEG + (int64_t)L * LE + lane_i(cand, L));
    }
    int lastk = -1;
#pragma unroll
    for (int k = 0; k < LE; ++k)
        if (wv[k] > 0.f) lastk = k;
    const uint64_t mp = __ballot(lastk >= 0);
    const int L = mp ? 63 - __clzll((long long)mp) : 0;
    const int kk = lane_i(lastk, L);
    return (int)((int64_t)g * SEG + (int64_t)L * LE + (kk < 0 ? 0 : kk));
}

// k_search: one workgroup per sequence.  Scans the segment sums for the one
// segment holding u*S, then walks that segment lane by lane.
template <int DTT, int DTD>
__global__ __launch_bounds__(NT) void k_search(const Params P)
{
    const int b = blockIdx.x;
    const int nseg = P.nseg;
    // the first residual sums load with the record (the search needs them
    // whenever the record says there is a draw)
    const float* sums_r = P.seg + (int64_t)b * nseg;
    const float first_r = (int)threadIdx.x < nseg ? sums_r[threadIdx.x] : 0.f;
    const SeqRec rec = P.rec[b];
    if (rec.status != 1) return;
    const int K = P.K;
    const float s = P.s;
    const int n = rec.n;
    const bool bonus = rec.bonus != 0;
    const bool oh = P.onehot != 0;
    const char* trow = target_row<DTT>(P, b, n);
    const char* drow = (bonus || oh) ? nullptr : draft_row<DTD>(P, b, n);
    const float cp = shift_of(rec.mp, s);
    const float cq = bonus ? 0.f : shift_of(rec.mq, s);
    const float w = bonus ? 0.f : rec.zp / rec.zq;
    __shared__ float sh_scan[NWAVE];
    __shared__ int sh_seg[NWAVE];
    __shared__ float sh_lo[1];

    const float* sums_p = P.seg + ((int64_t)P.B + b) * nseg;
    const Pick pk = find_segment<NT>(sums_r, sums_p, nseg, rec.u, bonus, sh_scan, sh_seg, sh_lo, first_r);
    if ((threadIdx.x >> 6) == 0 && pk.g >= 0) {
        const int y = walk_segment<DTT, DTD>(trow, drow, P.V, pk, s, cp, cq, w, (oh && !bonus) ? rec.xn : -1);
        if (threadIdx.x == 0) {
            P.out[(int64_t)b * (K + 1) + n] = y;
            put(P.res_mass, b, pk.mode == 2 ? 0.f : pk.S / rec.zp);
        }
    }
}

// ------------------------------------ k_seq: one workgroup per sequence --
//
// One workgroup of QT threads owns sequence b and walks its positions itself:
// it streams target row j and draft row j together, merges them on thread 0,
// runs the test at j and stops at the first rejection, so rows past it are
// never read and no other workgroup is ever waited for.  The decision, the
// diagnostics and the draw from row n (its segment sums kept in LDS, the rows
// just streamed likely still cached) follow in the same launch.  Fills the
// chip when B is at least about the number of compute units.

constexpr int QT = 1024;              // threads per workgroup: sixteen wave64
constexpr int QW = QT / 64;
constexpr int QU = 4;                 // 16-byte loads in flight per lane and row
constexpr int QSPW = 4;               // draw: segments per wave per step
constexpr int QMAXSEG = 4096;         // segment sums held in LDS: V <= QMAXSEG * SEG

// Online softmax of elements [e0, e1) of target row trow and draft row drow
// (may be null), both streamed in the same loop by BT threads with U 16-byte
// loads in flight per lane and row.  e0 is a multiple of 8 elements; e1 is a
// multiple of 8 or the row end.
// Fair share for a stream every wave of the chip runs at once: the SIMD issues
// the oldest ready wave first, so the waves dispatched last would get the
// least issue and memory bandwidth and finish last.  Each wave lowers its
// priority as it gets through its share (3 at the start, 0 in its last
// quarter): waves that are ahead yield to the ones behind, and all finish
// together.  `it` and `n` are uniform over the wave.
__device__ __forceinline__ void fair_priority(int it, int n)
{
    const int p = 3 - (4 * it) / (n > 0 ? n : 1);
    if (p >= 3) __builtin_amdgcn_s_setprio(3);
    else if (p == 2) __builtin_amdgcn_s_setprio(2);
    else if (p == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

template <int DTT, int DTD, int BT, int U, bool FAIR = false>
__device__ __forceinline__ void stream_pair(const char* trow, const char* drow, int64_t e0, int64_t e1, float s,
                                            SmState& st, SmState& sd)
{
    constexpr int ET = Fmt<DTT>::E, ED = Fmt<DTD>::E;
    const int tid = threadIdx.x;
    const bool al = (reinterpret_cast<uintptr_t>(trow) & 15u) == 0 &&
                    (drow == nullptr || (reinterpret_cast<uintptr_t>(drow) & 15u) == 0);
    if (al) {
        const uint4* vt = reinterpret_cast<const uint4*>(trow);
        const uint4* vd = reinterpret_cast<const uint4*>(drow);
        const int64_t t0 = e0 / ET, t1 = e1 / ET;          // whole vectors of the range
        const int64_t d0 = e0 / ED, d1 = drow ? e1 / ED : d0;
        const int64_t nt = t1 - t0, nd = d1 - d0;
        const int64_t nv = nt > nd ? nt : nd;
        const int niter = (int)((nv + (int64_t)BT * U - 1) / ((int64_t)BT * U));
        int it = 0;
        for (int64_t k = tid; k < nv; k += (int64_t)BT * U, ++it) {
            if constexpr (FAIR) fair_priority(it, niter);
            uint4 rt[U], rd[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t vi = k + (int64_t)u * BT;
                rt[u] = vi < nt ? vt[t0 + vi]
                                : make_uint4(Fmt<DTT>::NEG_INF_WORD, Fmt<DTT>::NEG_INF_WORD,
                                             Fmt<DTT>::NEG_INF_WORD, Fmt<DTT>::NEG_INF_WORD);
            }
            if (drow) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t vi = k + (int64_t)u * BT;
                    rd[u] = vi < nd ? vd[d0 + vi]
                                    : make_uint4(Fmt<DTD>::NEG_INF_WORD, Fmt<DTD>::NEG_INF_WORD,
                                                 Fmt<DTD>::NEG_INF_WORD, Fmt<DTD>::NEG_INF_WORD);
                }
            }
            if (k < nt) {
                float x[U * ET];
#pragma unroll
                for (int u = 0; u < U; ++u) unpack<DTT>(rt[u], x + u * ET);
                sm_window<U * ET>(x, s, st);
            }
            if (drow && k < nd) {
                float x[U * ED];
#pragma unroll
                for (int u = 0; u < U; ++u) unpack<DTD>(rd[u], x + u * ED);
                sm_window<U * ED>(x, s, sd);
            }
        }
        const int64_t tt = t1 * ET;              // ragged tails (< E elements each)
        if (tt + tid < e1) {
            float x1[1] = {load1<DTT>(trow, tt + tid)};
            sm_window<1>(x1, s, st);
        }
        if (drow) {
            const int64_t dt = d1 * ED;
            if (dt + tid < e1) {
                float x1[1] = {load1<DTD>(drow, dt + tid)};
                sm_window<1>(x1, s, sd);
            }
        }
    } else {
        constexpr int W = U * 4;
        for (int64_t base = e0 + tid; base < e1; base += (int64_t)BT * W) {
            float x[W], y[W];
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int64_t i = base + (int64_t)k * BT;
                x[k] = (i < e1) ? load1<DTT>(trow, i) : NEG_INF;
                y[k] = (drow && i < e1) ? load1<DTD>(drow, i) : NEG_INF;
            }
            sm_window<W>(x, s, st);
            if (drow) sm_window<W>(y, s, sd);
        }
    }
}

// OH: one-hot proposals (prompt lookup), a separate instance so the plain
// verify step's register budget is unaffected.
template <int DTT, int DTD, bool OH = false>
__global__ __launch_bounds__(QT) void k_seq(const Params P)
{
    const int b = blockIdx.x;
    const int K = P.K, V = P.V, R = 2 * K + 1;
    const float s = P.s;
    const bool greedy = P.greedy != nullptr && P.greedy[b] != 0;
    const bool has_draft = !greedy && P.draft != nullptr;
    // proposals of this sequence (prompt lookup: its own count; invalid counts
    // stop at once and decide_core reports the sequence invalid)
    const int Kb = OH ? P.klen[b] : K;
    const int Ke = OH ? ((Kb >= 0 && Kb <= K) ? Kb : 0) : K;
    const RowStat d0 = OH ? RowStat{0.f, 1.f, 0, 1} : RowStat{0.f, 0.f, 0, 0};
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ RowStat f_rs[MAXR];
    __shared__ TestIn ti[SV_MAX_K + 1];
    __shared__ SmState sh_t[QW], sh_d[QW];
    __shared__ AmState sh_a[QW];
    __shared__ int sh_stop;
    __shared__ Decision dec;
    __shared__ float seg_r[QMAXSEG], seg_p[QMAXSEG];
    __shared__ float sh_scan[QW];
    __shared__ int sh_seg[QW];
    __shared__ float sh_lo[1];

    // rows never streamed stay invalid; the test inputs load while position 0
    // streams (the first barrier below orders both before any read)
    if (tid < R) f_rs[tid] = tid > K ? d0 : RowStat{0.f, 0.f, 0, 0};
    const int tw = (QW - 1) * 64;                  // last wave loads the test inputs
    if (tid >= tw && tid - tw <= K) ti[tid - tw] = load_test_in<DTT, DTD>(P, b, tid - tw, greedy);

    for (int j = 0; j <= Ke; ++j) {
        const char* trow = target_row<DTT>(P, b, j);
        const bool dj = has_draft && j < K;
        if (greedy) {
            SmState sm = {NEG_INF, 0.f};
            AmState am = {NEG_INF, INT_MAX, 0u};
            scan_chunk<DTT, true, QT, QU>(trow, 0, V, s, sm, am);
            am = wave_reduce_am(am);
            if (lane == 0) sh_a[wave] = am;
        } else {
            SmState st = {NEG_INF, 0.f}, sd = {NEG_INF, 0.f};
            stream_pair<DTT, DTD, QT, QU>(trow, dj ? draft_row<DTD>(P, b, j) : nullptr, 0, V, s, st, sd);
            st = wave_reduce_sm(st, s);
            if (dj) sd = wave_reduce_sm(sd, s);
            if (lane == 0) {
                sh_t[wave] = st;
                sh_d[wave] = sd;
            }
        }
        __syncthreads();
        if (tid == 0) {
            RowStat t, d = d0;
            if (greedy) {
                AmState am = sh_a[0];
                for (int w2 = 1; w2 < QW; ++w2) am = am_merge(am, sh_a[w2]);
                t = rowstat_am(am);
            } else {
                SmState st = sh_t[0];
                for (int w2 = 1; w2 < QW; ++w2) st = sm_merge(st, sh_t[w2], s);
                t = rowstat_sm(st);
                if (dj) {
                    SmState sd = sh_d[0];
                    for (int w2 = 1; w2 < QW; ++w2) sd = sm_merge(sd, sh_d[w2], s);
                    d = rowstat_sm(sd);
                    f_rs[K + 1 + j] = d;
                }
            }
            f_rs[j] = t;
            bool stop = true;
            if (j < Ke) stop = test_from(V, s, greedy, t, d, ti[j].x, ti[j].u, ti[j].lx, ti[j].dx).stop;
            sh_stop = stop;
        }
        __syncthreads();
        if (sh_stop) break;
    }

    decide_core<DTT, DTD, OH>(P, b, greedy, true, true, f_rs, ti, &dec);
    if (greedy || !dec.ok) return;                 // uniform across the workgroup

    // draw from row n: residual max(0, p - q) scaled by Z_p, or p for the bonus
    const int n = dec.n, nseg = P.nseg;
    const bool bonus = n == Kb;                    // valid sequence: Kb in [0, K]
    const int32_t ox = (OH && !bonus) ? ti[n].x : -1;   // one-hot draft row at n
    const char* trow = target_row<DTT>(P, b, n);
    const char* drow = (bonus || OH) ? nullptr : draft_row<DTD>(P, b, n);
    const float cp = shift_of(dec.mp, s);
    const float cq = bonus ? 0.f : shift_of(dec.mq, s);
    const float w = bonus ? 0.f : dec.zp / dec.zq;
    const bool t_al = (reinterpret_cast<uintptr_t>(trow) & 15u) == 0;
    const bool d_al = drow != nullptr && (reinterpret_cast<uintptr_t>(drow) & 15u) == 0;
    for (int g0 = wave * QSPW; g0 < nseg; g0 += QW * QSPW) {
        float xl[QSPW][LE], xd[QSPW][LE];
#pragma unroll
        for (int k = 0; k < QSPW; ++k) {
            const int64_t e = (int64_t)(g0 + k) * SEG + (int64_t)lane * LE;
            load8<DTT>(trow, e, V, t_al, xl[k]);
            if (!bonus) {
                if constexpr (OH) onehot8(e, ox, xd[k]);
                else load8<DTD>(drow, e, V, d_al, xd[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < QSPW; ++k) {
            float sr = 0.f, sp = 0.f;
#pragma unroll
            for (int q = 0; q < LE; ++q) {
                const float ep = ex2(__builtin_fmaf(xl[k][q], s, -cp));
                sp += ep;
                sr += bonus ? ep : weight(xl[k][q], xd[k][q], s, cp, cq, w, 0);
            }
            sr = wave_sum(sr);
            sp = wave_sum(sp);
            if (lane == 0 && g0 + k < nseg) {
                seg_r[g0 + k] = sr;
                seg_p[g0 + k] = sp;
            }
        }
    }
    __syncthreads();
    const Pick pk = find_segment<QT>(seg_r, seg_p, nseg, dec.u, bonus, sh_scan, sh_seg, sh_lo);
    if (wave == 0) {
        const int y = pk.g >= 0 ? walk_segment<DTT, DTD>(trow, drow, V, pk, s, cp, cq, w, ox) : -1;
        if (lane == 0) {
            P.out[(int64_t)b * (K + 1) + n] = y;
            put(P.res_mass, b, pk.g < 0 ? NAN : (pk.mode == 2 ? 0.f : pk.S / dec.zp));
        }
    }
}

// ------------------------ k_seqg: G workgroups per sequence, one launch --
//
// The per-sequence walk of k_seq with each row split over the G workgroups of
// the sequence (slice g: segments [g*gsegs, (g+1)*gsegs) of SEG elements), so
// a sequence's later positions and its draw run on G compute units instead of
// one.  After streaming its slice of position j a workgroup publishes its
// partial statistics; every member waits for all G partials, merges them in
// the same fixed order and takes the same decision bit for bit, so no member
// ever needs another's decision.  The draw exchanges slice totals the same
// way; the member whose slice holds u*S finds and walks the segment.
//
// Exchange: each published value travels in one 64-bit word with a 32-bit tag
// in its upper half, stored and loaded as relaxed agent-scope atomics, so a
// word is valid on its own and needs no fence.  Values go in pairs whose two
// tags hash the sequence's call counter gep[b], the shape and the word's
// index: a word left by an earlier call, or any other content, passes both
// checks of a pair with probability 2^-64.  Member 0 advances gep[b] once all
// G members have published position 0 (so all of them have read it).
//
// Waits spin on the loads with a bound; the host launches no more
// workgroups than the device holds at once, so every member is resident and
// the bound is never reached in practice.  A wait that reaches it marks the
// sequence invalid (accepted_len -1) instead of hanging.

constexpr int GT = 256;               // threads per workgroup
constexpr int GW = GT / 64;
constexpr int GU = 3;                 // 16-byte loads in flight per lane and row
// Draw: 16-byte pieces in flight per lane.  With proposals (K > 0) the
// sequences that reject at their first position draw while the few long
// chains of positions are still streaming; those draws go shallow and paced
// (GDV_EARLY pieces, DRAW_PACE x 64 cycles of sleep per wave step), which
// leaves the latency-bound chains more of HBM, and finish well before the
// chains do.  Every other draw, and every draw at K = 0 (all sequences draw
// at once, nothing else streams), goes deep (GDV_DEEP).
constexpr int GDV_EARLY = 2;
constexpr int GDV_DEEP = 8;
constexpr int DRAW_PACE = 16;
// Wave priorities (s_setprio): position 0 of every sequence streams with a
// fair share (3 falling to 0 with progress); a sequence past it is on its way
// to a decision and maybe a long chain of positions, ahead of every stream of
// position 0; its draw, the end of a sequence, behind the chains.
constexpr int PRIO_CHAIN = 3;
constexpr int PRIO_DRAW = 1;
constexpr int GMAXG = 64;             // members per sequence at most (one wave gathers them)
constexpr int GMAXSEG = 2048;         // segment sums of one slice held in LDS
constexpr int GCAP = 4096;            // workgroups per launch at most (workspace sizing)
constexpr int XCDS = 8;               // workgroup i runs on accelerator die i % 8
constexpr int GSPIN = 1 << 20;        // polls before a wait gives up

__device__ __forceinline__ uint32_t mix32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

__device__ __forceinline__ uint32_t word_tag(uint32_t ep, uint32_t salt, uint32_t widx)
{
    const uint32_t t = mix32(ep * 0x9e3779b9u ^ salt ^ mix32(widx + 0x632be5abu));
    return t ? t : 1u;                // never 0: zeroed memory is never valid
}

__device__ __forceinline__ void put_word(uint64_t* w, uint32_t tag, uint32_t v)
{
    __hip_atomic_store(w, ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t get_word(const uint64_t* w)
{
    return __hip_atomic_load(const_cast<uint64_t*>(w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Word layout of one sequence's region: position j, member g, word w < 4 at
// (j*G + g)*4 + w (target pair, then draft pair); draw totals of member g,
// word w < 2 at (K+1)*G*4 + g*2 + w.
__device__ __forceinline__ int pos_word(int K, int G, int j, int g, int w) { (void)K; return (j * G + g) * 4 + w; }
__device__ __forceinline__ int draw_word(int K, int G, int g, int w) { return (K + 1) * G * 4 + g * 2 + w; }

// Wave 0: lane l < G waits for the NW words of member l starting at word
// index first(l) (consecutive), tags checked; v gets the values.  Returns
// whether every member's words arrived (uniform over the wave).
template <int NW>
__device__ __forceinline__ bool gather(const uint64_t* region, int G, uint32_t ep, uint32_t salt, int first,
                                       int spin, uint32_t (&v)[NW])
{
    const int l = threadIdx.x & 63;
    bool ready = l >= G;
    uint32_t tg[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        tg[k] = word_tag(ep, salt, (uint32_t)(first + k));
        v[k] = 0u;
    }
    for (int it = 0;; ++it) {
        if (!ready) {
            uint64_t w[NW];
#pragma unroll
            for (int k = 0; k < NW; ++k) w[k] = get_word(region + first + k);
            bool ok = true;
#pragma unroll
            for (int k = 0; k < NW; ++k) ok = ok && (uint32_t)(w[k] >> 32) == tg[k];
            if (ok) {
#pragma unroll
                for (int k = 0; k < NW; ++k) v[k] = (uint32_t)w[k];
                ready = true;
            }
        }
        if (__all(ready)) return true;
        if (it >= spin) return false;
        __builtin_amdgcn_s_sleep(2);
    }
}

// A member whose bounded wait ran out (some member of its sequence did not run
// at the same time): the sequence reports SV_GAVE_UP.  It writes the length
// only: the row is written by the members that complete (member 0 the prefix
// and padding, the drawing member the final token, then the length), so a
// valid length, if it is the store that lands last, always stands next to a
// whole row; under SV_GAVE_UP the row is unspecified (see sv_set_wait_limit).
__device__ __forceinline__ void give_up(const Params& P, int b)
{
    if (threadIdx.x == 0) P.acc[b] = SV_GAVE_UP;
}

// Draw pass of one member over its slice (segments sg0 .. sg0+nl-1) of row
// n: per segment, the sum of the draw weights (seg_r: residual max(0, p-q),
// or p for the bonus row, both scaled by Z_p) and of p (seg_p).  Full
// segments of 16-byte aligned rows go DSEG per wave step with every load of
// the step issued, unconditionally and from in-range addresses, before any is
// used, kept as raw 16-byte pieces (half the registers of unpacked floats);
// a partial last segment or unaligned rows go one segment per wave at a
// time.  Per element the arithmetic and its order are the walk's.  DV: the
// 16-byte pieces per lane of a wave step (DSEG = DV / pieces per segment, at
// least one); a GDV_EARLY draw also sleeps DRAW_PACE x 64 cycles after each
// step.
template <int DTT, int DTD, bool OH, bool BONUS, int DV>
__device__ __forceinline__ void draw_sums(const char* trow, const char* drow, int V, int nseg, int sg0, int nl,
                                          float s, float cp, float cq, float w, int32_t ox, bool fast_rows,
                                          float* seg_r, float* seg_p)
{
    constexpr int VT = Fmt<DTT>::BYTES / 2;        // 16-byte pieces per eight elements
    constexpr int VD = Fmt<DTD>::BYTES / 2;
    constexpr bool LD = !BONUS && !OH;             // a draft row to load
    constexpr int DSEG = DV / (VT + VD) > 0 ? DV / (VT + VD) : 1;   // segments per wave step
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool partial = (V % SEG) != 0 && sg0 + nl == nseg && nl > 0;
    const int nfast = fast_rows ? nl - (partial ? 1 : 0) : 0;
    for (int l0 = wave * DSEG; l0 < nfast; l0 += GW * DSEG) {
        uint4 rt[DSEG][VT], rd[DSEG][LD ? VD : 1];
#pragma unroll
        for (int k = 0; k < DSEG; ++k) {
            const int64_t e = (int64_t)(sg0 + min(l0 + k, nfast - 1)) * SEG + (int64_t)lane * LE;
            const uint4* pt = reinterpret_cast<const uint4*>(trow + e * Fmt<DTT>::BYTES);
#pragma unroll
            for (int v = 0; v < VT; ++v) rt[k][v] = pt[v];
            if constexpr (LD) {
                const uint4* pd = reinterpret_cast<const uint4*>(drow + e * Fmt<DTD>::BYTES);
#pragma unroll
                for (int v = 0; v < VD; ++v) rd[k][v] = pd[v];
            }
        }
#pragma unroll
        for (int k = 0; k < DSEG; ++k) {
            float xl[LE], xd[LE];
#pragma unroll
            for (int v = 0; v < VT; ++v) unpack<DTT>(rt[k][v], xl + v * (LE / VT));
            if constexpr (LD) {
#pragma unroll
                for (int v = 0; v < VD; ++v) unpack<DTD>(rd[k][v], xd + v * (LE / VD));
            } else if constexpr (OH && !BONUS) {
                onehot8((int64_t)(sg0 + l0 + k) * SEG + (int64_t)lane * LE, ox, xd);
            }
            float sr = 0.f, sp = 0.f;
#pragma unroll
            for (int qq = 0; qq < LE; ++qq) {
                const float ep2 = ex2(__builtin_fmaf(xl[qq], s, -cp));
                sp += ep2;
                if constexpr (BONUS) sr += ep2;
                else sr += weight(xl[qq], xd[qq], s, cp, cq, w, 0);
            }
            sr = wave_sum(sr);
            sp = wave_sum(sp);
            if (lane == 0 && l0 + k < nfast) {
                seg_r[l0 + k] = sr;
                seg_p[l0 + k] = sp;
            }
        }
        if constexpr (DV == GDV_EARLY) __builtin_amdgcn_s_sleep(DRAW_PACE);
    }
    const bool t_al = (reinterpret_cast<uintptr_t>(trow) & 15u) == 0;
    const bool d_al = drow != nullptr && (reinterpret_cast<uintptr_t>(drow) & 15u) == 0;
    for (int l = nfast + wave; l < nl; l += GW) {
        const int64_t e = (int64_t)(sg0 + l) * SEG + (int64_t)lane * LE;
        float xl[LE], xd[LE];
        load8<DTT>(trow, e, V, t_al, xl);
        if constexpr (LD) load8<DTD>(drow, e, V, d_al, xd);
        else if constexpr (OH && !BONUS) onehot8(e, ox, xd);
        float sr = 0.f, sp = 0.f;
#pragma unroll
        for (int qq = 0; qq < LE; ++qq) {
            const float ep2 = ex2(__builtin_fmaf(xl[qq], s, -cp));
            sp += ep2;
            if constexpr (BONUS) sr += ep2;
            else sr += weight(xl[qq], xd[qq], s, cp, cq, w, 0);
        }
        sr = wave_sum(sr);
        sp = wave_sum(sp);
        if (lane == 0) {
            seg_r[l] = sr;
            seg_p[l] = sp;
        }
    }
}

// A row's slice in one pass with its segment sums (16-byte aligned rows of
// whole vectors): a segment of 512 elements is VS = 512 / (64 * E) vectors
// per lane of one wave (E elements per 16-byte vector: 1 for bf16, 2 for
// fp32), lane l holding vectors l, l + 64, ... of the segment, and load
// group u of iteration it of wave w covers segment (it*US + u)*(BT/64) + w
// (US = U / VS groups), so a segment's sum is one wave reduction.  The exps
// are taken against a wave-uniform reference, the first finite segment max,
// kept while the segments' sums stay below 2^64 (fp32 sums are
// scale-invariant); a segment that reaches it (an element far above, +Inf
// or NaN) takes its own max and the reference moves there.  seg_m / seg_z
// get each segment's reference and sum, so the draw can rescale them to the
// row's max instead of reading the row again.  Returns the slice's state,
// uniform over the wave.
template <int DT, int BT, int U, bool FAIR>
__device__ __forceinline__ SmState stream_bonus(const char* trow, int64_t e0, int64_t e1, float s, float* seg_m,
                                                float* seg_z)
{
    constexpr int E = Fmt<DT>::E;                       // elements per 16-byte vector
    constexpr int VS = SEG / (64 * E);                  // vectors per lane per segment
    constexpr int US = (U + VS - 1) / VS;               // segments per lane and iteration
    constexpr int NWV = BT / 64;
    constexpr int N = VS * E;                           // elements per lane per segment (8)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint4* vt = reinterpret_cast<const uint4*>(trow) + e0 / E;
    const int64_t nv = (e1 - e0) / E;                   // whole vectors: e1 - e0 is a multiple of 8
    const int nl = (int)((e1 - e0 + SEG - 1) / SEG);    // segments of the slice
    const int niter = (nl + US * NWV - 1) / (US * NWV);
    constexpr uint32_t NI = Fmt<DT>::NEG_INF_WORD;
    SmState st = {NEG_INF, 0.f};                       // m: the reference while finite
    for (int it = 0; it < niter; ++it) {
        if constexpr (FAIR) fair_priority(it, niter);
        uint4 raw[US][VS];
#pragma unroll
        for (int u = 0; u < US; ++u) {
#pragma unroll
            for (int v = 0; v < VS; ++v) {
                const int64_t k = (int64_t)((it * US + u) * NWV + wave) * (64 * VS) + v * 64 + lane;
                raw[u][v] = k < nv ? vt[k] : make_uint4(NI, NI, NI, NI);
            }
        }
#pragma unroll
        for (int u = 0; u < US; ++u) {
            const int seg = (it * US + u) * NWV + wave;
            if (seg < nl) {                             // uniform over the wave
                float x[N], t[N];
#pragma unroll
                for (int v = 0; v < VS; ++v) unpack<DT>(raw[u][v], x + v * E);
                bool done = false;
                if (st.m > NEG_INF && st.m < POS_INF) {
                    const float c = st.m * s;
#pragma unroll
                    for (int q = 0; q < N; ++q) t[q] = ex2(__builtin_fmaf(x[q], s, -c));
                    const float wz = wave_sum(tree_sum<N>(t));
                    if (wz < 0x1p64f) {                 // uniform
                        if (lane == 0) {
                            seg_m[seg] = st.m;
                            seg_z[seg] = wz;
                        }
                        st.z += wz;
                        done = true;
                    }
                }
                if (!done) {                            // first finite segment, or the reference moves
                    const float wm = vmax(wave_max(tree_max<N>(x)), st.m);
                    const float c = shift_of(wm, s);
#pragma unroll
                    for (int q = 0; q < N; ++q) t[q] = ex2(__builtin_fmaf(x[q], s, -c));
                    const float wz = wave_sum(tree_sum<N>(t));
                    if (lane == 0) {
                        seg_m[seg] = wm;
                        seg_z[seg] = wz;
                    }
                    st = sm_merge(st, {wm, wz}, s);
                }
            }
        }
    }
    return st;
}

// DV: the draw's 16-byte pieces in flight per lane after a rejection at the
// first position (GDV_EARLY with proposals, GDV_DEEP at K = 0).
// LA: lookahead.  With LA = 0 a member streams position j only once j-1 is
// settled.  With LA = 1 it streams (and publishes) position j+1 before it
// gathers the partials of j, so the exchange's round trip and the wait for
// the sequence's slowest member hide behind a stream; the price is one
// position streamed past the first rejection (its partial is never used).
// Worth it where the chain's latency, not HBM, sets the kernel's length.
template <int DTT, int DTD, bool OH = false, int DV = GDV_EARLY, int LA = 0>
__global__ __launch_bounds__(GT) __attribute__((amdgpu_waves_per_eu(5, 8))) void k_seqg(const Params P)
{
    const int G = P.G;
    const int xcd = (int)(blockIdx.x % XCDS), loc = (int)(blockIdx.x / XCDS);
    // members of a sequence share a die (workgroup i runs on die i % 8):
    // slot q of die x holds sequence 8q + x, members in consecutive slots;
    // under lookahead 8q + (x + q) mod 8, so a pattern over the sequence
    // index with period 2, 4 or 8 (e.g. every other sequence greedy) is
    // spread over all dies
    int slot = loc;
    if (LA > 0 && P.ncu > 0) {
        // a die fills its ncu compute units in turn (its workgroup `loc` on
        // unit loc % ncu, round loc / ncu); every full round after the first
        // is turned by half the units, so the slots that share a unit come
        // from different halves of the rounds' sequences (with the pattern
        // above: sampling and greedy members side by side, instead of units
        // that hold only sampling members' rows, exps and draws).  A
        // rotation within each round keeps every sequence's members in the
        // rounds they had: a bijection, the same dispatch order.
        const int ncu = P.ncu, r = loc / ncu, c = loc - r * ncu;
        if (r < P.qd * G / ncu) slot = r * ncu + (c + ncu - (r * (ncu / 2)) % ncu) % ncu;
    }
    const int q = slot / G;
    const int b = LA > 0 ? XCDS * q + (xcd + q) % XCDS : xcd + XCDS * q;
    const int g = slot - q * G;
    if (b >= P.B) return;
    const int K = P.K, V = P.V, R = 2 * K + 1;
    const float s = P.s;
    const bool greedy = P.greedy != nullptr && P.greedy[b] != 0;
    const bool has_draft = !greedy && P.draft != nullptr;
    // proposals of this sequence (prompt lookup: its own count; invalid counts
    // stop at once and decide_core reports the sequence invalid)
    const int Kb = OH ? P.klen[b] : K;
    const int Ke = OH ? ((Kb >= 0 && Kb <= K) ? Kb : 0) : K;
    const RowStat d0 = OH ? RowStat{0.f, 1.f, 0, 1} : RowStat{0.f, 0.f, 0, 0};
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t salt = P.salt;
    uint64_t* region = P.slots + (int64_t)b * (((int64_t)K + 1) * G * 4 + (int64_t)G * 2);
    const int sg0 = g * P.gsegs;
    const int sg1 = min(sg0 + P.gsegs, P.nseg);
    const int nl = max(sg1 - sg0, 0);              // segments of this slice
    const int64_t e0 = (int64_t)sg0 * SEG;
    const int64_t e1 = min((int64_t)sg1 * SEG, (int64_t)V);

    __shared__ RowStat f_rs[MAXR];
    __shared__ TestIn ti[SV_MAX_K + 1];
    __shared__ SmState sh_t[2][GW], sh_d[2][GW];   // per wave, two positions in flight
    __shared__ AmState sh_a[2][GW];
    __shared__ int sh_stop;                        // 0 go on, 1 stop, 2 a wait gave up
    __shared__ Decision dec;
    __shared__ float seg_r[GMAXSEG], seg_p[GMAXSEG];
    __shared__ float sh_scan[GW];
    __shared__ int sh_seg[GW];
    __shared__ float sh_lo[1];
    __shared__ int sh_pick_g, sh_pick_mode, sh_pick_over;
    __shared__ float sh_pick_S, sh_pick_thr;

    // call identity in the tags: the device counter (fresh for every replay of
    // a captured launch) and the host's per-call nonce (so that words a
    // member left in a call whose waits gave up never match a later call, even
    // if that member read the counter after member 0 advanced it)
    uint32_t ep0 = 0, ep = 0;
    if (wave == 0) {
        ep0 = (uint32_t)__hip_atomic_load(P.gep + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ep = ep0 ^ mix32(P.nonce + 0x7f4a7c15u);
    }
    if (tid < R) f_rs[tid] = tid > K ? d0 : RowStat{0.f, 0.f, 0, 0};
    const int tw = (GW - 1) * 64;                  // last wave loads the test inputs
    if (tid >= tw && tid - tw <= K) ti[tid - tw] = load_test_in<DTT, DTD>(P, b, tid - tw, greedy);

    // the bonus row (position Kb) of a sampling sequence streamed in one pass
    // with its segment sums (rows of whole 16-byte vectors, no lookahead: there
    // the bonus row is rarely reached and the path's registers would spill);
    // segs_pos is the position whose sums the LDS holds
    const bool seg_pass = !greedy && (V & 7) == 0;
    int segs_pos = -1;
    // s: last position streamed and published; d: last position settled
    // (both uniform over the workgroup).  Stream while at most LA positions
    // are streamed but unsettled, then settle the oldest.
    // with lookahead the slices are small (few sequences): four loads per lane
    // and row cover a 16 KB slice in one round trip
    constexpr int SU = LA > 0 ? 4 : GU;
    // the sampling step (K = 0; the only use of the deep-draw instance without
    // lookahead) streams one row, not a pair: six loads per lane keep a pair's
    // bytes in flight (V=152064 bf16, B=64: 19.0 -> 18.1 us; B=256 22.4 -> 22.2)
    constexpr int SB = (DV == GDV_DEEP && LA == 0) ? 2 * GU : SU;
    int s_ = -1, d_ = -1;
    for (;;) {
        if (s_ < Ke && s_ - d_ <= LA) {
            const int j = ++s_, bi = j & 1;
            const char* trow = target_row<DTT>(P, b, j);
            const bool dj = has_draft && j < K;
            if (greedy) {
                SmState sm = {NEG_INF, 0.f};
                AmState am = {NEG_INF, INT_MAX, 0u};
                if (e0 < e1) scan_chunk<DTT, true, GT, SU>(trow, e0, e1, s, sm, am);
                if (j == 0) __builtin_amdgcn_s_setprio(PRIO_CHAIN);
                am = wave_reduce_am(am);
                if (lane == 0) sh_a[bi][wave] = am;
            } else {
                SmState st = {NEG_INF, 0.f}, sd = {NEG_INF, 0.f};
                // position 0: every sequence streams at once (fair share); later
                // positions: the few long sequences, oldest-first is fine
                const char* drow = dj ? draft_row<DTD>(P, b, j) : nullptr;
                // the bonus row in one pass, its segment sums kept for the draw
                const bool one = LA == 0 && j == Kb && seg_pass && (reinterpret_cast<uintptr_t>(trow) & 15u) == 0;
                if (e0 < e1) {
                    if (one) {
                        if (j == 0) st = stream_bonus<DTT, GT, SB, true>(trow, e0, e1, s, seg_r, seg_p);
                        else st = stream_bonus<DTT, GT, SB, false>(trow, e0, e1, s, seg_r, seg_p);
                    } else if constexpr (OH) {
                        // a one-hot proposal has no draft row: one more load per lane on
                        // the single row (B=256 prompt lookup: 92.6 -> 89.8 us per verify;
                        // six spill and lose)
                        if (j == 0) stream_pair<DTT, DTD, GT, SU + 1, true>(trow, nullptr, e0, e1, s, st, sd);
                        else stream_pair<DTT, DTD, GT, SU + 1>(trow, nullptr, e0, e1, s, st, sd);
                    } else if (j == 0) {
                        // the fair share is for the many position-0 streams of a large
                        // batch; under lookahead (B <= 64) it only delays some members
                        // (B=64 40.5 -> 39.8 us cache-flushed)
                        stream_pair<DTT, DTD, GT, SU, LA == 0>(trow, drow, e0, e1, s, st, sd);
                    } else {
                        stream_pair<DTT, DTD, GT, SU>(trow, drow, e0, e1, s, st, sd);
                    }
                }
                if (one) segs_pos = j;
                if (j == 0) __builtin_amdgcn_s_setprio(PRIO_CHAIN);
                if (!one) st = wave_reduce_sm(st, s);      // the one-pass state is uniform already
                if (dj) sd = wave_reduce_sm(sd, s);
                if (lane == 0) {
                    sh_t[bi][wave] = st;
                    sh_d[bi][wave] = sd;
                }
            }
            __syncthreads();
            // this member's partial of position j, merged over its waves in
            // order, published (the buffer bi is rewritten two streams later,
            // after the barrier that ends the next stream)
            if (wave == 0 && lane == 0) {
                uint64_t* w = region + pos_word(K, G, j, g, 0);
                const int wi = pos_word(K, G, j, g, 0);
                if (greedy) {
                    AmState am = sh_a[bi][0];
                    for (int w2 = 1; w2 < GW; ++w2) am = am_merge(am, sh_a[bi][w2]);
                    put_word(w, word_tag(ep, salt, wi), __float_as_uint(am.v));
                    put_word(w + 1, word_tag(ep, salt, wi + 1), (uint32_t)am.i | (am.bad ? 0x80000000u : 0u));
                } else {
                    SmState st = sh_t[bi][0], sd = sh_d[bi][0];
                    for (int w2 = 1; w2 < GW; ++w2) st = sm_merge(st, sh_t[bi][w2], s);
                    for (int w2 = 1; w2 < GW; ++w2) sd = sm_merge(sd, sh_d[bi][w2], s);
                    put_word(w, word_tag(ep, salt, wi), __float_as_uint(st.m));
                    put_word(w + 1, word_tag(ep, salt, wi + 1), __float_as_uint(st.z));
                    if (dj) {
                        put_word(w + 2, word_tag(ep, salt, wi + 2), __float_as_uint(sd.m));
                        put_word(w + 3, word_tag(ep, salt, wi + 3), __float_as_uint(sd.z));
                    }
                }
            }
            if (s_ < Ke && s_ - d_ <= LA) continue;      // stream the next position first
        }
        // settle position j = d+1: all members' partials, merged in lane order
        // on every member
        const int j = d_ + 1;
        const bool dj = has_draft && j < K;
        if (wave == 0) {
            bool ok;
            RowStat t, d = d0;
            const int first = pos_word(K, G, j, lane, 0);
            if (greedy) {
                uint32_t v[2];
                ok = gather<2>(region, G, ep, salt, first, P.spin, v);
                AmState am = {NEG_INF, INT_MAX, 0u};
                if (lane < G) am = {__uint_as_float(v[0]), (int32_t)(v[1] & 0x7fffffffu), v[1] >> 31};
                t = rowstat_am(wave_reduce_am(am));
            } else if (dj) {
                uint32_t v[4];
                ok = gather<4>(region, G, ep, salt, first, P.spin, v);
                SmState st = {NEG_INF, 0.f}, sd = {NEG_INF, 0.f};
                if (lane < G) {
                    st = {__uint_as_float(v[0]), __uint_as_float(v[1])};
                    sd = {__uint_as_float(v[2]), __uint_as_float(v[3])};
                }
                t = rowstat_sm(wave_reduce_sm(st, s));
                d = rowstat_sm(wave_reduce_sm(sd, s));
            } else {
                uint32_t v[2];
                ok = gather<2>(region, G, ep, salt, first, P.spin, v);
                SmState st = {NEG_INF, 0.f};
                if (lane < G) st = {__uint_as_float(v[0]), __uint_as_float(v[1])};
                t = rowstat_sm(wave_reduce_sm(st, s));
            }
            // every member has read the counter once position 0 is in
            if (j == 0 && g == 0 && lane == 0)
                __hip_atomic_store(P.gep + b, ep0 + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (lane == 0) {
                f_rs[j] = t;
                if (dj) f_rs[K + 1 + j] = d;
                bool stop = true;
                if (j < Ke) stop = test_from(V, s, greedy, t, d, ti[j].x, ti[j].u, ti[j].lx, ti[j].dx).stop;
                sh_stop = ok ? (stop ? 1 : 0) : 2;
            }
        }
        __syncthreads();
        d_ = j;
        if (sh_stop) break;
    }
    if (sh_stop == 2) {                            // a wait gave up
        give_up(P, b);
        return;
    }

    // a valid sampling sequence's accepted length is written by the member
    // that draws, after the drawn token: a member whose wait gave up writes
    // -1, and a length can then only stand next to a token that was written
    decide_core<DTT, DTD, OH>(P, b, greedy, g == 0, true, f_rs, ti, &dec, true);
    if (greedy || !dec.ok) return;                 // uniform across the workgroup

    // draw from row n: this member's slice of segment sums, then the totals
    const int n = dec.n;
    const bool bonus = n == Kb;                    // valid sequence: Kb in [0, K]
    const int32_t ox = (OH && !bonus) ? ti[n].x : -1;   // one-hot draft row at n
    const char* trow = target_row<DTT>(P, b, n);
    const char* drow = (bonus || OH) ? nullptr : draft_row<DTD>(P, b, n);
    const float cp = shift_of(dec.mp, s);
    const float cq = bonus ? 0.f : shift_of(dec.mq, s);
    const float w = bonus ? 0.f : dec.zp / dec.zq;
    const bool t_al = (reinterpret_cast<uintptr_t>(trow) & 15u) == 0;
    const bool d_al = drow != nullptr && (reinterpret_cast<uintptr_t>(drow) & 15u) == 0;
    const bool fast_rows = t_al && (bonus || OH || d_al);
    __builtin_amdgcn_s_setprio(PRIO_DRAW);
    if (bonus && segs_pos == n) {
        // the segment sums of the one-pass stream, rescaled to the row's max
        for (int l = tid; l < nl; l += GT) {
            const float v = seg_p[l] * ex2(shift_of(seg_r[l], s) - cp);
            seg_r[l] = v;
            seg_p[l] = v;
        }
    } else if (bonus)
        draw_sums<DTT, DTD, OH, true, GDV_DEEP>(trow, drow, V, P.nseg, sg0, nl, s, cp, cq, w, ox, fast_rows, seg_r,
                                                seg_p);
    else if (n == 0)
        draw_sums<DTT, DTD, OH, false, DV>(trow, drow, V, P.nseg, sg0, nl, s, cp, cq, w, ox, fast_rows, seg_r, seg_p);
    else
        draw_sums<DTT, DTD, OH, false, GDV_DEEP>(trow, drow, V, P.nseg, sg0, nl, s, cp, cq, w, ox, fast_rows, seg_r,
                                                 seg_p);
    __syncthreads();
    float tr = 0.f, tp = 0.f;                      // slice totals, in the scan order the search uses
    for (int base = 0; base < nl; base += GT) {
        float tot;
        block_incl_scan<GT>((base + tid < nl) ? seg_r[base + tid] : 0.f, sh_scan, &tot);
        tr += tot;
        block_incl_scan<GT>((base + tid < nl) ? seg_p[base + tid] : 0.f, sh_scan, &tot);
        tp += tot;
    }
    if (wave == 0) {
        if (lane == 0) {
            const int wi = draw_word(K, G, g, 0);
            put_word(region + wi, word_tag(ep, salt, wi), __float_as_uint(tr));
            put_word(region + wi + 1, word_tag(ep, salt, wi + 1), __float_as_uint(tp));
        }
        uint32_t v[2];
        const bool ok = gather<2>(region, G, ep, salt, draw_word(K, G, lane, 0), P.spin, v);
        const float mr = lane < G ? __uint_as_float(v[0]) : 0.f;
        const float mp = lane < G ? __uint_as_float(v[1]) : 0.f;
        // every lane walks the member totals in member order (same bits on all)
        float S = 0.f;
        for (int l = 0; l < G; ++l) S += lane_f(mr, l);
        int mode = bonus ? 1 : 0;
        const bool use_p = !(S > 0.f);             // residual rounded to nothing: draw from p_n
        if (use_p) {
            mode = 2;
            S = 0.f;
            for (int l = 0; l < G; ++l) S += lane_f(mp, l);
        }
        const float mine = use_p ? mp : mr;
        const float thr = dec.u * S;
        int gs = -1, over = 0;
        float cum = 0.f, lo = 0.f;
        for (int l = 0; l < G; ++l) {
            const float v2 = lane_f(mine, l);
            if (gs < 0) {
                if (v2 > 0.f && cum + v2 > thr) {
                    gs = l;
                    lo = cum;
                } else {
                    cum += v2;
                }
            }
        }
        if (gs < 0) {                              // rounding overrun: the last slice with weight
            over = 1;
            for (int l = G - 1; l >= 0; --l) {
                const float v2 = lane_f(mine, l);
                if (gs < 0 && v2 > 0.f) gs = l;
            }
        }
        if (lane == 0) {
            sh_pick_g = ok ? gs : -2;
            sh_pick_mode = mode;
            sh_pick_over = over;
            sh_pick_S = S;
            sh_pick_thr = over ? POS_INF : thr - lo;
        }
    }
    __syncthreads();
    if (sh_pick_g == -2) {                         // the wait for the slice totals gave up
        give_up(P, b);
        return;
    }
    if (sh_pick_g != g) return;                    // another member's slice holds the draw
    Pick pk;
    pk.mode = sh_pick_mode;
    pk.S = sh_pick_S;
    const Locate L = locate_segment<GT>(pk.mode == 2 ? seg_p : seg_r, nl, sh_pick_thr, sh_scan, sh_seg, sh_lo);
    pk.g = L.g < 0 ? -1 : sg0 + L.g;
    pk.overrun = L.overrun || sh_pick_over;
    pk.thr = sh_pick_thr;
    pk.lo = L.lo;
    if (wave == 0) {
        const int y = pk.g >= 0 ? walk_segment<DTT, DTD>(trow, drow, V, pk, s, cp, cq, w, ox) : -1;
        if (lane == 0) {
            P.out[(int64_t)b * (K + 1) + n] = y;
            put(P.res_mass, b, pk.g < 0 ? NAN : (pk.mode == 2 ? 0.f : pk.S / dec.zp));
            P.acc[b] = n;
        }
    }
}

// -------------------------------------------------------------- host side --

enum Sched { EAGER = 0, LAZY = 1, SEQ = 2 };

struct Plan {
    int C, nseg, tiles;
    Sched sched;
    bool lazy;
    int gmax;         // grouped per-sequence schedule: workgroups per sequence the workspace holds
    int G, gsegs;     // and the ones this call uses (G < 2: one 1024-thread workgroup per sequence)
    int la;           // grouped schedule: lookahead (positions streamed before the oldest is settled)
    size_t off_rec, off_reach, off_part, off_seg, off_gep, off_slots, total;
};

// SV_MODE_AUTO / EAGER / LAZY / SEQ (sv_set_mode; SV_MODE in the environment)
static std::atomic<int> g_mode{-1};
// most workgroups per sequence under SV_MODE_SEQ, 0 = as many as fit
// (sv_set_seq_groups; SV_SEQ_GROUPS in the environment)
static std::atomic<int> g_groups{-1};
// polls before a wait of the grouped schedule gives up (sv_set_wait_limit)
static std::atomic<int> g_spin{GSPIN};
// per-call nonce of the grouped schedule's tags
static std::atomic<uint32_t> g_nonce{0};
// lookahead of the grouped schedule: -1 = by shape (sv_set_seq_lookahead;
// SV_SEQ_LOOKAHEAD in the environment), else 0, 1 or 2
static std::atomic<int> g_la{-2};

static int la_knob()
{
    int m = g_la.load(std::memory_order_relaxed);
    if (m == -2) {
        const char* e = getenv("SV_SEQ_LOOKAHEAD");
        m = (e && (!strcmp(e, "0") || !strcmp(e, "1") || !strcmp(e, "2"))) ? (int)(e[0] - '0') : -1;
        int expect = -2;
        g_la.compare_exchange_strong(expect, m);
        m = g_la.load(std::memory_order_relaxed);
    }
    return m;
}

static int groups_now()
{
    int m = g_groups.load(std::memory_order_relaxed);
    if (m < 0) {
        const char* e = getenv("SV_SEQ_GROUPS");
        long v = e ? strtol(e, nullptr, 10) : 0;
        m = (v >= 1 && v <= GMAXG) ? (int)v : 0;
        int expect = -1;
        g_groups.compare_exchange_strong(expect, m);
        m = g_groups.load(std::memory_order_relaxed);
    }
    return m;
}

static int mode_now()
{
    int m = g_mode.load(std::memory_order_relaxed);
    if (m < 0) {
        const char* e = getenv("SV_MODE");
        m = SV_MODE_AUTO;
        if (e && !strcmp(e, "eager")) m = SV_MODE_EAGER;
        if (e && !strcmp(e, "lazy")) m = SV_MODE_LAZY;
        if (e && !strcmp(e, "seq")) m = SV_MODE_SEQ;
        int expect = -1;
        g_mode.compare_exchange_strong(expect, m);
        m = g_mode.load(std::memory_order_relaxed);
    }
    return m;
}

static int64_t nseg_of(int32_t V) { return ((int64_t)V + SEG - 1) / SEG; }

// Sequences are laid out eight to a die: the grouped launch has 8*ceil(B/8)
// groups of G workgroups.
static int64_t group_slots(int32_t B) { return 8 * (((int64_t)B + 7) / 8); }

// Workgroups per sequence the workspace is sized for (device independent).
static int group_max(int32_t B)
{
    const int64_t gm = GCAP / group_slots(B);
    return (int)(gm < GMAXG ? gm : GMAXG);
}

// k_seqg workgroups the current device holds at once, per storage-type pair
// (0 when unknown: the grouped launch is then not used); the smaller of the
// two draw depths' counts, so either instance's grid is resident.
template <int DTT, int DTD, bool OH>
static int group_capacity_t()
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 0;
    }
    static std::atomic<int> cache[64];
    static std::atomic<bool> init[64];
    if (init[dev].load(std::memory_order_acquire)) return cache[dev].load(std::memory_order_relaxed);
    int per_cu2 = 0, per_cu3 = 0, per_cu4 = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&k_seqg<DTT, DTD, OH, GDV_EARLY>), GT, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu2, reinterpret_cast<const void*>(&k_seqg<DTT, DTD, OH, GDV_DEEP>), GT, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu3, reinterpret_cast<const void*>(OH ? &k_seqg<DTT, DTD, OH, GDV_DEEP>
                                                       : &k_seqg<DTT, DTD, OH, GDV_DEEP, 1>), GT, 0) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu4, reinterpret_cast<const void*>(OH ? &k_seqg<DTT, DTD, OH, GDV_DEEP>
                                                       : &k_seqg<DTT, DTD, OH, GDV_DEEP, 2>), GT, 0) != hipSuccess) {
        (void)hipGetLastError();                   // unknown capacity: one workgroup per sequence
        return 0;
    }
    if (per_cu2 < per_cu) per_cu = per_cu2;
    if (per_cu3 < per_cu) per_cu = per_cu3;
    if (per_cu4 < per_cu) per_cu = per_cu4;
    cache[dev].store(cus * per_cu, std::memory_order_relaxed);
    init[dev].store(true, std::memory_order_release);
    return cus * per_cu;
}

// Compute units per accelerator die of the current device, cached per
// device (0 if unknown: the plain placement is used).
static int cus_per_die()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 0;
    }
    static std::atomic<int> cache[64];
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    const int per = cus % XCDS == 0 ? cus / XCDS : 0;
    if (per > 0) cache[dev].store(per, std::memory_order_relaxed);
    return per;
}

static int group_capacity(int32_t dtt, int32_t dtd, bool onehot)
{
    if (onehot) return dtt == SV_BF16 ? group_capacity_t<SV_BF16, SV_BF16, true>()
                                      : group_capacity_t<SV_F32, SV_F32, true>();
    if (dtt == SV_BF16 && dtd == SV_BF16) return group_capacity_t<SV_BF16, SV_BF16, false>();
    if (dtt == SV_F32 && dtd == SV_F32) return group_capacity_t<SV_F32, SV_F32, false>();
    if (dtt == SV_F32 && dtd == SV_BF16) return group_capacity_t<SV_F32, SV_BF16, false>();
    return group_capacity_t<SV_BF16, SV_F32, false>();
}

// Bytes position 0 streams: every target row, and draft rows (K > 0).
static double pos0_bytes(int32_t B, int32_t K, int32_t V, int32_t dtt, int32_t dtd)
{
    const double bt = dtt == SV_BF16 ? 2 : 4, bd = dtd == SV_BF16 ? 2 : 4;
    return (double)B * V * (bt + (K > 0 ? bd : 0.0));
}

// Lookahead of the per-sequence schedule for this shape: 1 while position 0
// alone streams less than 64 MiB (the chains of positions, not HBM, then set
// the kernel's length), else 0; sv_set_seq_lookahead overrides.
static int lookahead_for(int32_t B, int32_t K, int32_t V, int32_t dtt, int32_t dtd)
{
    const int k = la_knob();
    if (k >= 0) return k;
    return pos0_bytes(B, K, V, dtt, dtd) >= 64.0 * (1 << 20) ? 0 : 1;
}

// Automatic choice.  The per-sequence schedule (one launch, no row past a
// rejection read, draws overlapping other sequences' streams) wins once
// position 0 alone streams at least 64 MiB, enough to fill the chip, and
// with lookahead from 16 MiB for up to 64 sequences of bf16 rows when there
// are positions to test, and for the sampling step (K = 0) on rows of whole
// vectors; it needs the vocabulary's segment sums to fit in LDS.  Otherwise lazy mode,
// which pays one latency-bound launch per position (5-20 us each on
// gfx950), wins once the eager stream is long against K+1 such launches: at
// least 64 MiB of logits per position; else eager.
// mode: the schedule asked for (SV_MODE_*); SV_MODE_AUTO applies the rule
// below.  -1: the process-wide mode (sv_set_mode).
static Sched choose_sched(int32_t B, int32_t K, int32_t V, int32_t dtt, int32_t dtd, bool onehot = false,
                          int mode = -1)
{
    const int m = mode >= 0 ? mode : mode_now();
    if (onehot) {                                  // no draft rows; lazy launches do not take one-hot rows
        const double bt = dtt == SV_BF16 ? 2 : 4;
        const bool seq_ok = nseg_of(V) <= QMAXSEG;
        if (m == SV_MODE_SEQ) return seq_ok ? SEQ : EAGER;
        if (m == SV_MODE_EAGER || m == SV_MODE_LAZY) return EAGER;
        return (seq_ok && (double)B * V * bt >= 64.0 * (1 << 20)) ? SEQ : EAGER;
    }
    const bool seq_ok = nseg_of(V) <= QMAXSEG;
    if (m == SV_MODE_SEQ) return seq_ok ? SEQ : (K == 0 ? EAGER : LAZY);
    if (m == SV_MODE_EAGER) return EAGER;
    if (m == SV_MODE_LAZY) return K == 0 ? EAGER : LAZY;
    const double bt = dtt == SV_BF16 ? 2 : 4, bd = dtd == SV_BF16 ? 2 : 4;
    const double mib64 = 64.0 * (1 << 20);
    const double p0 = pos0_bytes(B, K, V, dtt, dtd);
    if (seq_ok && p0 >= mib64) return SEQ;
    // a few long bf16 rows per sequence: the per-sequence schedule with
    // lookahead (measured per step with the caches warm: B=64 K=5 V=128256
    // 33.7 against 41 us eager, B=32 K=8 V=152064 29.0 against 47 us); not
    // at B=256 over a 19008-token shard (45.7 against 45.8 us) nor for fp32
    // target rows (50 against 42-44 us)
    if (seq_ok && K > 0 && p0 >= mib64 / 4 && B <= 64 && dtt == SV_BF16) return SEQ;
    // the sampling step on rows of whole 16-byte vectors: the per-sequence
    // launch reads each row once (the bonus row's segment sums are kept for
    // the draw) against twice for eager (V=152064, per call, bf16 / fp32:
    // B=1 10.6 / 11.4 against 15.1 / 14.2 us, B=64 19.0 / 20.5 against
    // 22.1 / 25.9, B=256 22.2 / 31.0 against 46.6 / 58.2)
    if (K == 0 && seq_ok && V % 8 == 0) return SEQ;
    if (K == 0) return EAGER;
    const double bytes = (double)B * V * ((double)(K + 1) * bt + (double)K * bd);
    return bytes >= (double)(K + 1) * mib64 ? LAZY : EAGER;
}

static int env_int(const char* name, int dflt)
{
    const char* v = getenv(name);
    if (!v || !*v) return dflt;
    char* end = nullptr;
    long x = strtol(v, &end, 10);
    return (end && *end == '\0' && x > 0 && x < INT_MAX) ? (int)x : dflt;
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static bool make_plan(int32_t B, int32_t K, int32_t V, Sched sched, Plan* pl)
{
    const bool lazy = sched == LAZY;
    const int64_t R = 2 * (int64_t)K + 1;
    const int64_t rows = (int64_t)B * R;
    const int64_t rows_per_launch = lazy ? (int64_t)B * 2 : rows;
    const int64_t n8 = ((int64_t)V + 7) / 8;
    int64_t max_c = n8 / ((int64_t)NT * UNROLL);        // at least one full window per lane
    if (max_c < 1) max_c = 1;
    static const int target_items = env_int("SV_TARGET_ITEMS", 4096);
    static const int forced_c = env_int("SV_CHUNKS", 0);
    int64_t C = rows_per_launch > 0 ? (target_items + rows_per_launch - 1) / rows_per_launch : 1;
    if (forced_c > 0) C = forced_c;
    if (C > max_c) C = max_c;
    if (C < 1) C = 1;
    pl->C = (int)C;
    pl->sched = sched;
    pl->lazy = lazy;
    pl->nseg = (int)(((int64_t)V + SEG - 1) / SEG);
    pl->tiles = (pl->nseg + SPT - 1) / SPT;
    if (rows * C > INT_MAX || (int64_t)B * pl->tiles > INT_MAX) return false;
    size_t o = 0;
    pl->off_rec = o;  o = align_up(o + sizeof(SeqRec) * (size_t)B, 256);
    pl->off_reach = o; o = align_up(o + sizeof(int32_t) * (size_t)B, 256);
    pl->off_part = o; o = align_up(o + sizeof(Partial) * (size_t)(rows * C), 256);
    pl->off_seg = o;  o = align_up(o + sizeof(float) * 2 * (size_t)B * (size_t)pl->nseg, 256);
    pl->gmax = group_max(B);
    pl->G = 1;
    pl->gsegs = pl->nseg;
    pl->la = 0;
    pl->off_gep = o;  o = align_up(o + sizeof(uint32_t) * (size_t)B, 256);
    pl->off_slots = o;
    o = align_up(o + sizeof(uint64_t) * (size_t)B * (size_t)pl->gmax * (((size_t)K + 1) * 4 + 2), 256);
    pl->total = o;
    return true;
}

static bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static bool dtype_ok(int32_t dt) { return dt == SV_F32 || dt == SV_BF16; }
static size_t dtype_bytes(int32_t dt) { return dt == SV_BF16 ? 2 : 4; }

// force: a schedule the call must use (-1: the mode's choice).
static int prepare(const void* target, const void* draft, const int32_t* tokens, const float* uniforms,
                   float T, const uint8_t* greedy, int32_t B, int32_t K, int32_t V, int32_t dtt, int32_t dtd,
                   int32_t* acc, int32_t* out, const sv_diag* diag, void* ws, size_t ws_bytes,
                   Params* P, Plan* pl, int force = -1, bool onehot = false)
{
    (void)greedy;
    if (B < 0 || K < 0 || K > SV_MAX_K || V < 1) return SV_EINVAL;
    if (!dtype_ok(dtt) || !dtype_ok(dtd)) return SV_EINVAL;
    if (!(T > 0.f) || !isfinite(T)) return SV_EINVAL;
    const double sd = 1.4426950408889634074 / (double)T;
    const float s = (float)sd;
    if (!isfinite(s) || !(s >= 1.17549435e-38f)) return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!target || !uniforms || !acc || !out) return SV_EINVAL;
    if (K > 0 && !tokens) return SV_EINVAL;
    if (!aligned_to(target, dtype_bytes(dtt)) || (draft && !aligned_to(draft, dtype_bytes(dtd)))) return SV_EINVAL;
    if (!aligned_to(uniforms, 4) || !aligned_to(acc, 4) || !aligned_to(out, 4) ||
        (tokens && !aligned_to(tokens, 4)))
        return SV_EINVAL;
    if (diag) {
        const float* d[5] = {diag->p_tok, diag->q_tok, diag->lse_p, diag->lse_q, diag->res_mass};
        for (const float* q : d)
            if (q && !aligned_to(q, 4)) return SV_EINVAL;
    }
    const Sched sched = force >= 0 ? (Sched)force : choose_sched(B, K, V, dtt, dtd);
    if (!make_plan(B, K, V, sched, pl)) return SV_EINVAL;
    if (!ws || !aligned_to(ws, 16) || ws_bytes < pl->total) return SV_EWORKSPACE;
    char* w = static_cast<char*>(ws);
    P->target = target;
    P->draft = K > 0 ? draft : nullptr;
    P->tokens = tokens;
    P->uniforms = uniforms;
    P->greedy = greedy;
    P->acc = acc;
    P->out = out;
    P->p_tok = diag ? diag->p_tok : nullptr;
    P->q_tok = diag ? diag->q_tok : nullptr;
    P->lse_p = diag ? diag->lse_p : nullptr;
    P->lse_q = diag ? diag->lse_q : nullptr;
    P->res_mass = diag ? diag->res_mass : nullptr;
    P->rec = reinterpret_cast<SeqRec*>(w + pl->off_rec);
    P->reach = reinterpret_cast<int32_t*>(w + pl->off_reach);
    P->part = reinterpret_cast<Partial*>(w + pl->off_part);
    P->seg = reinterpret_cast<float*>(w + pl->off_seg);
    P->B = B;
    P->K = K;
    P->V = V;
    P->C = pl->C;
    P->nseg = pl->nseg;
    P->tiles = pl->tiles;
    P->s = s;
    P->gep = reinterpret_cast<uint32_t*>(w + pl->off_gep);
    P->slots = reinterpret_cast<uint64_t*>(w + pl->off_slots);
    P->G = 1;
    P->gsegs = pl->nseg;
    P->qd = 0;
    P->ncu = 0;
    P->salt = 0;
    P->nonce = 0;
    P->spin = GSPIN;
    P->klen = nullptr;
    P->onehot = onehot ? 1 : 0;
    if (pl->sched == SEQ) {
        // as many workgroups per sequence as fit on the device at once (each
        // waits for the others), within the workspace's and LDS's limits
        int64_t G = group_capacity(dtt, dtd, onehot) / group_slots(B);
        if (G > pl->gmax) G = pl->gmax;
        const int la = onehot ? 0 : lookahead_for(B, K, V, dtt, dtd);
        if (la > 0) {
            // with lookahead, the fewest members whose slices a single pass of
            // four 16-byte loads per lane covers (16 bf16 / 8 fp32 segments):
            // a position is then one load round trip, the draw one wave step,
            // and further members only lengthen every exchange (measured at
            // B=32 V=152064: 20 members 34.9 us against 40 by capacity 42.4)
            const int per = (dtt == SV_F32 || dtd == SV_F32) ? 8 : 16;
            const int64_t gl = ((int64_t)pl->nseg + per - 1) / per;
            if (G > gl) G = gl;
        }
        const int lim = groups_now();
        if (lim > 0 && G > lim) G = lim;
        if (G > pl->nseg) G = pl->nseg;
        int64_t gsegs = G >= 2 ? (pl->nseg + G - 1) / G : pl->nseg;
        if (G >= 2 && gsegs <= GMAXSEG) {
            pl->G = (int)G;
            pl->gsegs = (int)gsegs;
            pl->la = la;
            uint32_t h = 0x811c9dc5u;
            const uint32_t f[7] = {(uint32_t)B, (uint32_t)K, (uint32_t)V, (uint32_t)G, (uint32_t)dtt,
                                   (uint32_t)dtd, (uint32_t)gsegs};
            for (uint32_t x : f) h = (h ^ x) * 0x01000193u;
            P->G = pl->G;
            P->gsegs = pl->gsegs;
            // turned placement under lookahead (sequence slots per die, units per die)
            const int ncu = la > 0 ? cus_per_die() : 0;
            if (ncu >= 2) {
                P->qd = (B + XCDS - 1) / XCDS;
                P->ncu = ncu;
            }
            P->salt = h;
            P->nonce = g_nonce.fetch_add(1u, std::memory_order_relaxed);
            P->spin = g_spin.load(std::memory_order_relaxed);
        }
    }
    return 1;   // ready to launch
}

template <int DTT, int DTD>
static void launch_rowstats_t(const Params& P, const Plan& pl, hipStream_t st)
{
    if (pl.sched == SEQ) {                         // the whole step in one launch
        const dim3 gg((unsigned)(group_slots(P.B) * pl.G));
        if (P.onehot) {                            // one storage type: no draft logits
            if constexpr (DTT == DTD) {
                if (pl.G < 2) hipLaunchKernelGGL((k_seq<DTT, DTT, true>), dim3((unsigned)P.B), dim3(QT), 0, st, P);
                else if (P.K > 0) hipLaunchKernelGGL((k_seqg<DTT, DTT, true, GDV_EARLY>), gg, dim3(GT), 0, st, P);
                else hipLaunchKernelGGL((k_seqg<DTT, DTT, true, GDV_DEEP>), gg, dim3(GT), 0, st, P);
            }
        } else if (pl.G >= 2) {
            if (P.K > 0 && pl.la > 1) hipLaunchKernelGGL((k_seqg<DTT, DTD, false, GDV_DEEP, 2>), gg, dim3(GT), 0, st, P);
            else if (P.K > 0 && pl.la > 0) hipLaunchKernelGGL((k_seqg<DTT, DTD, false, GDV_DEEP, 1>), gg, dim3(GT), 0, st, P);
            else if (P.K > 0) hipLaunchKernelGGL((k_seqg<DTT, DTD, false, GDV_EARLY>), gg, dim3(GT), 0, st, P);
            else hipLaunchKernelGGL((k_seqg<DTT, DTD, false, GDV_DEEP>), gg, dim3(GT), 0, st, P);
        } else {
            hipLaunchKernelGGL((k_seq<DTT, DTD>), dim3((unsigned)P.B), dim3(QT), 0, st, P);
        }
        return;
    }
    if (!pl.lazy) {
        const dim3 grid((unsigned)((int64_t)P.B * (2 * P.K + 1) * pl.C));
        hipLaunchKernelGGL((k_rowstats<DTT, DTD>), grid, dim3(NT), 0, st, P);
        return;
    }
    for (int j = 0; j <= P.K; ++j) {
        const dim3 grid((unsigned)((int64_t)P.B * (j < P.K ? 2 : 1) * pl.C));
        hipLaunchKernelGGL((k_rowstats_lazy<DTT, DTD>), grid, dim3(NT), 0, st, P, j);
    }
}

// Workgroups of k_tiles<DTT, DTD, true> the current device holds at once,
// cached per device (0 if the query fails: then the separate decision launch
// is used, and the failed query leaves no error behind).
template <int DTT, int DTD, int SW = SPW>
static int64_t tiles_capacity()
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 0;
    }
    static std::atomic<int> cache[64];
    static std::atomic<bool> init[64];
    if (init[dev].load(std::memory_order_acquire)) return cache[dev].load(std::memory_order_relaxed);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&k_tiles<DTT, DTD, true, SW>),
                                                     NT, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    cache[dev].store(cus * per_cu, std::memory_order_relaxed);
    init[dev].store(true, std::memory_order_release);
    return cus * per_cu;
}

template <int DTT, int DTD>
static void launch_draw_t(const Params& P, const Plan& pl, hipStream_t st)
{
    if (pl.sched == SEQ) return;                   // k_seq already drew
    // few sequences: tiles of one segment per wave, so the grid still fits the
    // device at once but spreads row n over four times the workgroups (B=8
    // V=32000 fp32: 21.5 -> 18.9 us per step); otherwise SPW segments per wave
    const int64_t t1 = (pl.nseg + NWAVE - 1) / NWAVE;
    if ((int64_t)P.B * t1 <= tiles_capacity<DTT, DTD, 1>()) {
        Params Q = P;
        Q.tiles = (int32_t)t1;
        hipLaunchKernelGGL((k_tiles<DTT, DTD, true, 1>), dim3((unsigned)(P.B * t1)), dim3(NT), 0, st, Q);
        hipLaunchKernelGGL((k_search<DTT, DTD>), dim3((unsigned)P.B), dim3(NT), 0, st, P);
        return;
    }
    // then two segments per wave (B=256 over a 19008-token shard: 44.1 -> 42.6 us hot)
    const int64_t t2 = (pl.nseg + 2 * NWAVE - 1) / (2 * NWAVE);
    if ((int64_t)P.B * t2 <= tiles_capacity<DTT, DTD, 2>()) {
        Params Q = P;
        Q.tiles = (int32_t)t2;
        hipLaunchKernelGGL((k_tiles<DTT, DTD, true, 2>), dim3((unsigned)(P.B * t2)), dim3(NT), 0, st, Q);
        hipLaunchKernelGGL((k_search<DTT, DTD>), dim3((unsigned)P.B), dim3(NT), 0, st, P);
        return;
    }
    const int64_t nt = (int64_t)P.B * pl.tiles;
    if (nt <= tiles_capacity<DTT, DTD>()) {
        hipLaunchKernelGGL((k_tiles<DTT, DTD, true>), dim3((unsigned)nt), dim3(NT), 0, st, P);
    } else {
        hipLaunchKernelGGL((k_decide<DTT, DTD>), dim3((unsigned)P.B), dim3(NT), 0, st, P);
        hipLaunchKernelGGL((k_tiles<DTT, DTD, false>), dim3((unsigned)nt), dim3(NT), 0, st, P);
    }
    hipLaunchKernelGGL((k_search<DTT, DTD>), dim3((unsigned)P.B), dim3(NT), 0, st, P);
}

#define SV_DISPATCH(FN, dtt, dtd, ...)                                                         \
    do {                                                                                       \
        if (dtt == SV_BF16 && dtd == SV_BF16) FN<SV_BF16, SV_BF16>(__VA_ARGS__);               \
        else if (dtt == SV_F32 && dtd == SV_F32) FN<SV_F32, SV_F32>(__VA_ARGS__);              \
        else if (dtt == SV_F32 && dtd == SV_BF16) FN<SV_F32, SV_BF16>(__VA_ARGS__);            \
        else FN<SV_BF16, SV_F32>(__VA_ARGS__);                                                 \
    } while (0)

static int launch_stats(const Params& P, const Plan& pl, int32_t dtt, int32_t dtd, hipStream_t st)
{
    sv_launch_begin();
    SV_DISPATCH(launch_rowstats_t, dtt, dtd, P, pl, st);
    return sv_launch_status();
}

static int launch_draw(const Params& P, const Plan& pl, int32_t dtt, int32_t dtd, hipStream_t st)
{
    sv_launch_begin();
    SV_DISPATCH(launch_draw_t, dtt, dtd, P, pl, st);
    return sv_launch_status();
}

}  // namespace sv

static thread_local int g_last_hip = 0;

void sv_launch_begin(void) { (void)hipGetLastError(); }

int sv_launch_status(void)
{
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) return SV_OK;
    g_last_hip = (int)e;
    return SV_ELAUNCH;
}

// Verify step with separate storage types for target and draft logits (the
// fused LM-head path feeds fp32 target logits and bf16 draft logits).
int sv_verify_mixed(const void* target, const void* draft, const int32_t* tokens, const float* uniforms,
                    float T, const uint8_t* greedy, int32_t B, int32_t K, int32_t V, int32_t dtt,
                    int32_t dtd, int32_t* acc, int32_t* out, const sv_diag* diag, void* ws,
                    size_t ws_bytes, void* stream, int check_only)
{
    sv::Params P;
    sv::Plan pl;
    int rc = sv::prepare(target, draft, tokens, uniforms, T, greedy, B, K, V, dtt, dtd, acc, out, diag,
                         ws, ws_bytes, &P, &pl);
    if (rc <= 0 || check_only) return rc <= 0 ? rc : SV_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    rc = sv::launch_stats(P, pl, dtt, dtd, st);
    if (rc != SV_OK) return rc;
    return sv::launch_draw(P, pl, dtt, dtd, st);
}

namespace sv {

// Scratch of spec_verify_noalloc, for callers that cannot allocate: one
// call's workspace in a file-scope device array that every GPU the library
// runs on holds until the process ends.  On the host this name is only a
// stand-in for the symbol, never a device address: host code uses the
// address hipGetSymbolAddress gives for the current device, kept per device.
constexpr size_t SCRATCH_BYTES = (size_t)16 << 20;
constexpr int SCRATCH_DEVS = 64;
__device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

// The current device's copy of `scratch`, looked up once per device with
// that device current (the first spec_verify_noalloc call on it).  Null on
// failure, with the HIP error kept for sv_last_hip_error().
static void* scratch_ptr(int* hip_err)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= SCRATCH_DEVS)) e = hipErrorInvalidDevice;
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *hip_err = (int)e;
        return nullptr;
    }
    static std::atomic<void*> ptrs[SCRATCH_DEVS];
    void* p = ptrs[dev].load(std::memory_order_acquire);
    if (p) return p;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
        (void)hipGetLastError();
        *hip_err = (int)(e != hipSuccess ? e : hipErrorInvalidSymbol);
        return nullptr;
    }
    ptrs[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace sv

// ------------------------------------------------------------------ C ABI --

extern "C" {

size_t sv_workspace_bytes(int32_t B, int32_t K, int32_t V, int32_t dtype)
{
    if (B <= 0 || K < 0 || K > SV_MAX_K || V < 1 || !sv::dtype_ok(dtype)) return 0;
    sv::Plan pe, pz;
    if (!sv::make_plan(B, K, V, sv::EAGER, &pe) || !sv::make_plan(B, K, V, sv::LAZY, &pz)) return 0;
    return pe.total > pz.total ? pe.total : pz.total;
}

#define SV_ARGS_DECL                                                                           \
    const void *target_logits, const void *draft_logits, const int32_t *draft_tokens,          \
        const float *uniforms, float temperature, const uint8_t *greedy_flag, int32_t B,       \
        int32_t K, int32_t V, int32_t dtype, int32_t *accepted_len, int32_t *out_tokens,      \
        const sv_diag *diag, void *workspace, size_t workspace_bytes, void *stream

#define SV_PREPARE                                                                             \
    sv::Params P;                                                                              \
    sv::Plan pl;                                                                               \
    int rc = sv::prepare(target_logits, draft_logits, draft_tokens, uniforms, temperature,     \
                         greedy_flag, B, K, V, dtype, dtype, accepted_len, out_tokens, diag,   \
                         workspace, workspace_bytes, &P, &pl);                                 \
    if (rc <= 0) return rc;                                                                    \
    hipStream_t st = static_cast<hipStream_t>(stream)

int spec_verify(SV_ARGS_DECL)
{
    SV_PREPARE;
    rc = sv::launch_stats(P, pl, dtype, dtype, st);
    if (rc != SV_OK) return rc;
    return sv::launch_draw(P, pl, dtype, dtype, st);
}

int spec_verify_mode(int mode, SV_ARGS_DECL)
{
    if (mode < SV_MODE_AUTO || mode > SV_MODE_SEQ) return SV_EINVAL;
    if (B < 0 || K < 0 || K > SV_MAX_K || V < 1 || !sv::dtype_ok(dtype)) return SV_EINVAL;
    // SV_MODE_AUTO here means the automatic rule, whatever sv_set_mode says
    const int force = sv::choose_sched(B, K, V, dtype, dtype, false, mode);
    sv::Params P;
    sv::Plan pl;
    int rc = sv::prepare(target_logits, draft_logits, draft_tokens, uniforms, temperature, greedy_flag, B, K, V,
                         dtype, dtype, accepted_len, out_tokens, diag, workspace, workspace_bytes, &P, &pl, force);
    if (rc <= 0) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    rc = sv::launch_stats(P, pl, dtype, dtype, st);
    if (rc != SV_OK) return rc;
    return sv::launch_draw(P, pl, dtype, dtype, st);
}

int sv_stats(SV_ARGS_DECL)
{
    SV_PREPARE;
    return sv::launch_stats(P, pl, dtype, dtype, st);
}

int spec_verify_ex(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                   const float* uniforms, float temperature, const uint8_t* greedy_flag, int32_t B, int32_t K,
                   int32_t V, int32_t target_dtype, int32_t draft_dtype, int32_t* accepted_len,
                   int32_t* out_tokens, const sv_diag* diag, void* workspace, size_t workspace_bytes,
                   void* stream)
{
    return sv_verify_mixed(target_logits, draft_logits, draft_tokens, uniforms, temperature, greedy_flag, B, K,
                           V, target_dtype, draft_dtype, accepted_len, out_tokens, diag, workspace,
                           workspace_bytes, stream, 0);
}

int spec_verify_noalloc(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                        const float* uniforms, float temperature, const uint8_t* greedy_flag, int32_t B, int32_t K,
                        int32_t V, int32_t dtype, int32_t* accepted_len, int32_t* out_tokens, const sv_diag* diag,
                        void* stream)
{
    // the workspace is the device's scratch array: the shape must fit it; no
    // part of the workspace needs initialising, so nothing is cleared
    const size_t need = sv_workspace_bytes(B, K, V, dtype);
    if (need > sv::SCRATCH_BYTES) return SV_ESCRATCH;
    // the host checks of spec_verify first (an aligned stand-in address of
    // the scratch's size: checked, never dereferenced, nothing launched)
    alignas(256) static char stand_in[256];
    const int rc = sv_verify_mixed(target_logits, draft_logits, draft_tokens, uniforms, temperature, greedy_flag,
                                   B, K, V, dtype, dtype, accepted_len, out_tokens, diag,
                                   need > 0 ? stand_in : nullptr, need > 0 ? sv::SCRATCH_BYTES : 0, stream, 1);
    if (rc != SV_OK || need == 0) return rc;
    void* ws = nullptr;
    {
        int err = 0;
        ws = sv::scratch_ptr(&err);
        if (!ws) {
            g_last_hip = err;
            return SV_ELAUNCH;
        }
    }
    return spec_verify(target_logits, draft_logits, draft_tokens, uniforms, temperature, greedy_flag, B, K, V,
                       dtype, accepted_len, out_tokens, diag, ws, ws ? sv::SCRATCH_BYTES : 0, stream);
}

size_t sv_noalloc_scratch_bytes(void) { return sv::SCRATCH_BYTES; }

int sv_draw(SV_ARGS_DECL)
{
    SV_PREPARE;
    return sv::launch_draw(P, pl, dtype, dtype, st);
}

size_t sv_sample_workspace_bytes(int32_t B, int32_t V, int32_t dtype)
{
    const size_t w = sv_workspace_bytes(B, 0, V, dtype);
    return w ? w + sv::align_up(sizeof(int32_t) * (size_t)B, 256) : 0;
}

int sv_sample(const void* logits, int32_t dtype, const float* uniforms, float temperature,
              const uint8_t* greedy_flag, int32_t B, int32_t V, int32_t* tokens, float* lse,
              void* workspace, size_t workspace_bytes, void* stream)
{
    // the verify step with K = 0: no tests, the final draw from p_0
    if (B < 0 || V < 1) return SV_EINVAL;
    if (B == 0) return SV_OK;
    const size_t w0 = sv_workspace_bytes(B, 0, V, dtype);
    if (w0 == 0) return SV_EINVAL;
    if (!workspace || workspace_bytes < sv_sample_workspace_bytes(B, V, dtype)) return SV_EWORKSPACE;
    int32_t* acc = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + w0);
    sv_diag dg = {nullptr, nullptr, lse, nullptr, nullptr};
    return sv_verify_mixed(logits, nullptr, nullptr, uniforms, temperature, greedy_flag, B, 0, V, dtype, dtype,
                           acc, tokens, lse ? &dg : nullptr, workspace, w0, stream, 0);
}

int spec_verify_lookup(const void* target_logits, int32_t dtype, const int32_t* cand, const int32_t* klen,
                       const float* uniforms, float temperature, const uint8_t* greedy_flag, int32_t B, int32_t K,
                       int32_t V, int32_t* accepted_len, int32_t* out_tokens, const sv_diag* diag, void* workspace,
                       size_t workspace_bytes, void* stream)
{
    // one-hot draft rows that are never stored; target rows past each
    // sequence's proposals are never read.  Eager, or per-sequence when the
    // mode (or the automatic rule on the target rows alone) picks it
    sv::Params P;
    sv::Plan pl;
    if (B > 0 && (!klen || (reinterpret_cast<uintptr_t>(klen) & 3u))) return SV_EINVAL;
    int rc = sv::prepare(target_logits, nullptr, cand, uniforms, temperature, greedy_flag, B, K, V, dtype, dtype,
                         accepted_len, out_tokens, diag, workspace, workspace_bytes, &P, &pl,
                         sv::choose_sched(B, K, V, dtype, dtype, true), true);
    if (rc <= 0) return rc;
    P.klen = klen;
    hipStream_t st = static_cast<hipStream_t>(stream);
    rc = sv::launch_stats(P, pl, dtype, dtype, st);
    if (rc != SV_OK) return rc;
    return sv::launch_draw(P, pl, dtype, dtype, st);
}

int sv_set_mode(int mode)
{
    if (mode < SV_MODE_AUTO || mode > SV_MODE_SEQ) return SV_EINVAL;
    sv::g_mode.store(mode, std::memory_order_relaxed);
    return SV_OK;
}

int sv_get_mode(void) { return sv::mode_now(); }

int sv_last_hip_error(void) { return g_last_hip; }

int sv_set_seq_groups(int groups)
{
    if (groups < 0 || groups > sv::GMAXG) return SV_EINVAL;
    sv::g_groups.store(groups, std::memory_order_relaxed);
    return SV_OK;
}

int sv_set_seq_lookahead(int lookahead)
{
    if (lookahead < -1 || lookahead > 2) return SV_EINVAL;
    sv::g_la.store(lookahead, std::memory_order_relaxed);
    return SV_OK;
}

int sv_seq_lookahead(int32_t B, int32_t K, int32_t V, int32_t target_dtype, int32_t draft_dtype)
{
    if (B < 1 || K < 0 || K > SV_MAX_K || V < 1 || !sv::dtype_ok(target_dtype) || !sv::dtype_ok(draft_dtype))
        return SV_EINVAL;
    if (sv::choose_sched(B, K, V, target_dtype, draft_dtype) != sv::SEQ) return 0;
    // the plan of a call on dummy (aligned, non-null) pointers, nothing launched
    sv::Params P;
    sv::Plan pl;
    alignas(16) static char dummy[16];
    const int rc = sv::prepare(dummy, dummy, reinterpret_cast<const int32_t*>(dummy),
                               reinterpret_cast<const float*>(dummy), 1.f, nullptr, B, K, V, target_dtype,
                               draft_dtype, reinterpret_cast<int32_t*>(dummy), reinterpret_cast<int32_t*>(dummy),
                               nullptr, dummy, (size_t)-1, &P, &pl);
    return rc == 1 ? (pl.G >= 2 && K > 0 ? pl.la : 0) : SV_EINVAL;
}

int sv_set_wait_limit(int32_t polls)
{
    if (polls < 0 || polls > sv::GSPIN) return SV_EINVAL;
    sv::g_spin.store(polls == 0 ? sv::GSPIN : polls, std::memory_order_relaxed);
    return SV_OK;
}

int sv_seq_groups(int32_t B, int32_t K, int32_t V, int32_t target_dtype, int32_t draft_dtype)
{
    if (B < 1 || K < 0 || K > SV_MAX_K || V < 1 || !sv::dtype_ok(target_dtype) || !sv::dtype_ok(draft_dtype))
        return SV_EINVAL;
    if (sv::choose_sched(B, K, V, target_dtype, draft_dtype) != sv::SEQ) return 0;
    // the plan of a call on dummy (aligned, non-null) pointers, nothing launched
    sv::Params P;
    sv::Plan pl;
    alignas(16) static char dummy[16];
    const int rc = sv::prepare(dummy, dummy, reinterpret_cast<const int32_t*>(dummy),
                               reinterpret_cast<const float*>(dummy), 1.f, nullptr, B, K, V, target_dtype,
                               draft_dtype, reinterpret_cast<int32_t*>(dummy), reinterpret_cast<int32_t*>(dummy),
                               nullptr, dummy, (size_t)-1, &P, &pl);
    return rc == 1 ? pl.G : SV_EINVAL;
}

int sv_schedule(int32_t B, int32_t K, int32_t V, int32_t target_dtype, int32_t draft_dtype)
{
    if (B < 0 || K < 0 || K > SV_MAX_K || V < 1 || !sv::dtype_ok(target_dtype) || !sv::dtype_ok(draft_dtype))
        return SV_EINVAL;
    switch (sv::choose_sched(B, K, V, target_dtype, draft_dtype)) {
    case sv::SEQ: return SV_MODE_SEQ;
    case sv::LAZY: return SV_MODE_LAZY;
    default: return SV_MODE_EAGER;
    }
}

const char* sv_strerror(int code)
{
    switch (code) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument (shape, dtype, temperature, pointer or alignment)";
    case SV_EWORKSPACE: return "workspace missing, misaligned or too small";
    case SV_ELAUNCH: return "HIP kernel launch failed";
    case SV_ESCRATCH: return "shape needs more workspace than the library's static scratch holds (spec_verify_noalloc)";
    default: return "unknown error";
    }
}

int sv_version(void) { return 1; }

}  // extern "C"
