// One 64-key tile of the flash-attention inner loop on gfx950 matrix cores,
// shared by the prefill and decode kernels. A wave owns 32 "columns" of the
// score block S^T = K Q^T: 32 query rows of one head (prefill) or the query
// heads of one KV group (decode). Lane 32 g + x holds column x; the operand
// layouts are described in dca_internal.h.
#pragma once

#include <hip/hip_runtime.h>

#include "dca_internal.h"
#include "frag.h"

namespace dca {

__device__ inline float lane_swap32(float x) { return __shfl_xor(x, 32, 64); }

// Registers one wave carries across key tiles.
template <typename T, int D>
struct WaveState {
    using vec = typename Frag<T>::vec;
    static constexpr int NU = D / (2 * Frag<T>::E);
    static constexpr int NDB = D / 32;
    vec qfrag[NU];
    int region;
    bool first;    // no tile of this row block seen yet (reference max unset)
    f32x16 oacc[NDB];
    float mref;    // reference max of the row's scores (base-2 exponent units)
    float l_run;   // sum of 2^(s - mref) over this lane's keys
};

// The pre-pass scales the rotated keys by yarn * sigma * log2 e, so the
// matrix cores deliver scores s in base-2 exponent units. Each 32x32 score
// accumulator starts at -mref (every value of a lane belongs to the lane's
// row), so it ends as s - mref and P = 2^(s - mref) needs no further
// arithmetic. Masked pairs hold -inf (P = 0).
//
// The row max is not taken on the common path. mref is only a reference: P
// stays exact whatever its value as long as nothing overflows, so a tile is
// accepted when every lane's sum of P over its 32 keys is finite and at most
// 2^20 (then every P <= 2^20). Otherwise -- and on a row block's first tile --
// the exact tile max is taken, mref raised to it (O and l rescaled), and P
// recomputed.
constexpr float kPsumLimit = 1048576.0f;   // 2^20

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedDsRead = 0x100;

// S^T (64 keys x 32 columns) = K Q^T for one key tile, K fragments at kl
// (LDS or global memory). LDS_SCHED: schedule the LDS fragment reads ahead of
// the matrix-core ops that consume them.
template <typename T, int D, bool LDS_SCHED>
__device__ __forceinline__ void tile_scores(int lane, const WaveState<T, D> &st, const char *__restrict__ kl,
                                            f32x16 (&s)[2]) {
    using F = Frag<T>;
    using vec = typename F::vec;
    constexpr int NU = WaveState<T, D>::NU;
    const vec *k = (const vec *)kl;
    const float init = st.first ? 0.f : -st.mref;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] = init;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) F::mma(k[(kb * NU + u) * 64 + lane], st.qfrag[u], s[kb]);
    if constexpr (LDS_SCHED && sizeof(T) == 2) {
        // schedule: the accumulator set-up, then K fragment reads kept
        // AHEAD deep in front of the matrix-core ops that consume them
        constexpr int N = 2 * NU, AHEAD = N < 4 ? N : 4;
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 16, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, AHEAD, 0);
#pragma unroll
        for (int i = 0; i < N - AHEAD; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, AHEAD, 0);
    }
}

// The same with the accumulators started from c0, a tuple the caller keeps
// equal to the start value (-mref, or 0 before the first tile): the first
// matrix-core op of each accumulator reads c0 and writes a fresh result, so
// no per-tile initialisation runs on the vector ALU.
// The wave raises its issue priority for these reads and products: of the
// two waves sharing a SIMD, the one starting its scores goes first, so the
// other's softmax and PV fill in behind it rather than the two running the
// same phase side by side (3% faster dense, 6% vertical-slash, measured).
// HOLD leaves the priority raised on return; the caller lowers it before PV.
template <typename T, int D, bool LDS_SCHED, bool HOLD = false>
__device__ __forceinline__ void tile_scores_from(int lane, const WaveState<T, D> &st, const f32x16 &c0,
                                                 const char *__restrict__ kl, f32x16 (&s)[2]) {
    using F = Frag<T>;
    using vec = typename F::vec;
    constexpr int NU = WaveState<T, D>::NU;
    const vec *k = (const vec *)kl;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb] = F::mma_from(k[(kb * NU) * 64 + lane], st.qfrag[0], c0);
#pragma unroll
    for (int u = 1; u < NU; ++u)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) F::mma(k[(kb * NU + u) * 64 + lane], st.qfrag[u], s[kb]);
    if constexpr (LDS_SCHED && sizeof(T) == 2) {
        constexpr int N = 2 * NU, AHEAD = N < 4 ? N : 4;
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, AHEAD, 0);
#pragma unroll
        for (int i = 0; i < N - AHEAD; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, AHEAD, 0);
    }
    if constexpr (!HOLD) __builtin_amdgcn_s_setprio(0);
}

// P = 2^s rounded to the operand type, in PV fragment order; returns this
// lane's sum of the rounded P.
template <typename T>
__device__ __forceinline__ float tile_p(const f32x16 (&s)[2], typename Frag<T>::vec (&p)[2][kBlk / (2 * Frag<T>::E)]) {
    using F = Frag<T>;
    constexpr int E = F::E;
    constexpr int NUV = kBlk / (2 * E);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) F::set(p[kb][v / E], v % E, F::from_float(__builtin_amdgcn_exp2f(s[kb][v])));
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < NUV; ++u) sum = F::sum_into(p[kb][u], sum);
    return sum;
}

// Raise mref to the tile's row max (or set it on the first tile), shift the
// scores to the new reference and rescale O and l.
template <typename T, int D>
__device__ __forceinline__ void raise_ref(WaveState<T, D> &st, f32x16 (&s)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    mx = fmaxf(mx, lane_swap32(mx));
    // rows of an active wave always hold a finite score in every tile they visit
    const float d = st.first ? mx : fmaxf(mx, 0.f);
    const float alpha = st.first ? 0.f : __builtin_amdgcn_exp2f(-d);
    st.mref = (st.first ? 0.f : st.mref) + d;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] -= d;
    st.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < WaveState<T, D>::NDB; ++db) st.oacc[db] *= alpha;
    st.first = false;
}

// V^T fragments of one tile, in the order the PV loop consumes them (read
// while the softmax runs).
template <typename T, int D>
struct VFrags {
    typename Frag<T>::vec v[2][kBlk / (2 * Frag<T>::E)][D / 32];
};
template <typename T, int D>
__device__ __forceinline__ void load_v(int lane, const char *__restrict__ vlds, VFrags<T, D> &vf) {
    using vec = typename Frag<T>::vec;
    constexpr int NDB = D / 32;
    constexpr int NUV = kBlk / (2 * Frag<T>::E);
    const vec *vl = (const vec *)vlds;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < NUV; ++u)
#pragma unroll
            for (int db = 0; db < NDB; ++db) vf.v[kb][u][db] = vl[((kb * NDB + db) * NUV + u) * 64 + lane];
}
// O^T += V^T P^T
template <typename T, int D>
__device__ __forceinline__ void tile_pv(WaveState<T, D> &st, const VFrags<T, D> &vf,
                                             const typename Frag<T>::vec (&p)[2][kBlk / (2 * Frag<T>::E)]) {
    using F = Frag<T>;
    constexpr int NDB = D / 32;
    constexpr int NUV = kBlk / (2 * F::E);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < NUV; ++u)
#pragma unroll
            for (int db = 0; db < NDB; ++db) F::mma(vf.v[kb][u][db], p[kb][u], st.oacc[db]);
}

}  // namespace dca
