// DCA causal GQA flash attention for gfx950 (one pass, online softmax).
//
// [mizuki, 核心思想]: the L x L score matrix splits into intra-chunk,
// successive-chunk and inter-chunk parts, merged by one softmax per row.
// Chunks are multiples of 64 rows, so a 64-key tile lies inside one chunk and
// a 32-row wave block inside one chunk: the region -- and with it the query
// variant -- is fixed per (wave, key tile) and needs no per-element select.
// Each wave walks its keys in ascending order: inter tiles (chunks <= c-2),
// successive tiles (chunk c-1), intra tiles (chunk c, up to the diagonal),
// reloading its query fragments twice at most.
//
// Per workgroup: NW waves x 32 query rows of one query head; 64-key K and V
// tiles staged through LDS (double-buffered, one barrier per tile). Per wave
// and tile:
//   S^T (64 keys x 32 rows) = K_rot Q_x^T     2 x (D/16) bf16 MFMA 32x32x16
//   online softmax (exp2 domain, scale tau * sigma * log2 e); a lane holds 32
//     scores of one row, the row max is completed with one lane swap
//   O^T (D x 32 rows) += V^T P^T               (D/32) x 4 MFMA 32x32x16
// The accumulator of S^T leaves scores in exactly the order the PV op wants
// them (see dca_internal.h), so P never touches LDS.
//
// Vertical-slash mode [mizuki, MInference sections]: the workgroup visits
// the union of the active key tiles of its 64-row query tiles, merging each
// head's sorted tile list VT and distance list D on the fly; a wave skips
// tiles inactive for its own query tile.
//
// Grid order: heaviest row tiles first; the work list is cut into per-XCD
// streams so that the workgroups resident on one XCD (workgroup i lands on
// XCD i mod 8) share one KV head and sweep the same keys through that XCD's
// L2.
#include <hip/hip_runtime.h>

#include "dca_internal.h"
#include "frag.h"

namespace dca {

struct AttnArgs {
    const void *qf[3];
    const void *kf;
    const void *vf;
    void *out;
    float *lse;
    int64_t S, C;
    int32_t Hq, Hkv, G, nblk;
    float ks;                 // tau * sigma * log2(e)
    // work decode
    int32_t n_rt, KVH, s_split, M, per_xcd;
    // vertical-slash lists
    const int32_t *vt, *vt_n, *dl, *dl_n;
    int32_t list_stride;
    int32_t sparse;
};

constexpr int kNone = 0x7fffffff;
// A row's running max is raised (and O rescaled) only when a new tile's max
// exceeds it by more than this many powers of two; until then scores are
// exponentiated against the stale max, which bounds every P by 2^8.
constexpr float kLazyRescale = 8.0f;

__device__ inline float lane_swap32(float x) { return __shfl_xor(x, 32, 64); }

typedef __attribute__((address_space(3))) void lds_void;

// Key tiles a workgroup visits, ascending. Dense: 0 .. kt_last. Vertical-
// slash: the union over the workgroup's 64-row query tiles t of
// {kt in VT : kt <= t} and {t - delta : delta in D, delta <= t}, merged on
// the fly from the head's sorted lists; the mask gets one bit per query tile
// for which the returned tile is active.
template <int NT>
struct TileIter {
    // the lists are read through the constant address space: scalar loads,
    // counted apart from the vector loads that fill the LDS rings
    typedef const __attribute__((address_space(4))) int32_t *cptr;
    int32_t pv[NT], pd[NT], tq[NT];
    cptr vt, dl;
    int32_t nv;
    int kt_dense, kt_last;
    bool sparse;

    __device__ __forceinline__ void init(const AttnArgs &a, int h, int i0, int S, int last) {
        kt_dense = 0;
        kt_last = last;
        sparse = a.sparse != 0;
        vt = dl = nullptr;
        nv = 0;
        if (!sparse) return;
        vt = (cptr)(a.vt + (int64_t)h * a.list_stride);
        dl = (cptr)(a.dl + (int64_t)h * a.list_stride);
        nv = ((cptr)a.vt_n)[h];
        const int32_t nd = ((cptr)a.dl_n)[h];
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            tq[q] = i0 / kTile + q;
            pv[q] = 0;
            int lo = 0, hi = nd;             // pd = index of the last D entry <= t
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (dl[mid] <= tq[q]) lo = mid + 1; else hi = mid;
            }
            pd[q] = lo - 1;
            if (tq[q] * kTile >= S) { pv[q] = nv; pd[q] = -1; }
        }
    }

    __device__ __forceinline__ int next(unsigned &m_out) {
        if (!sparse) {
            if (kt_dense > kt_last) return -1;
            m_out = (1u << NT) - 1;
            return kt_dense++;
        }
        int32_t best = kNone;
        int32_t ca[NT], cb[NT];
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            ca[q] = (pv[q] < nv && vt[pv[q]] <= tq[q]) ? vt[pv[q]] : kNone;
            cb[q] = (pd[q] >= 0) ? tq[q] - dl[pd[q]] : kNone;
            const int32_t c = ca[q] < cb[q] ? ca[q] : cb[q];
            best = c < best ? c : best;
        }
        if (best == kNone) return -1;
        unsigned m = 0;
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            bool hit = false;
            if (ca[q] == best) { ++pv[q]; hit = true; }
            if (cb[q] == best) { --pd[q]; hit = true; }
            if (hit) m |= 1u << q;
        }
        m_out = m;
        return best;
    }
};

// Per-wave constants of the tile loop.
// Per-wave constants of the tile loop.
struct WaveCtx {
    int lane, x, gsel, wave, r0, tb_succ, tb_intra, wave_qt;
    bool active_rows;
    float ks;
    int64_t qbase;               // element offset of this wave's 32-row block in a Q variant
    const char *kbytes, *vbytes; // this KV head's fragment-ordered K and V
};

// One K (or V) tile -> an LDS buffer, straight from global memory: each wave
// moves its share of the tile's contiguous 1 KB pieces (16 bytes per lane,
// written to LDS at M0 + 16 * lane). Issued as inline asm so that the
// compiler does not make every later LDS read wait for these loads: the loop
// waits for them explicitly (s_waitcnt vmcnt(0) + barrier) before any wave
// reads the buffer. The asm has no register outputs; M0 is set inside the
// block with the one wait state an SALU write of M0 needs before an LDS DMA
// reads it.
template <typename T, int D, int NW>
__device__ __forceinline__ void dma_tile(const WaveCtx &c, const char *base, int kt, uint32_t dst) {
    constexpr int TILE_BYTES = 2 * kBlk * D * (int)sizeof(T);
    constexpr int WAVE_CHUNKS = TILE_BYTES / 1024 / NW;
    static_assert(TILE_BYTES % (1024 * NW) == 0, "tile split");
#pragma unroll
    for (int i = 0; i < WAVE_CHUNKS; ++i) {
        const int chunk = c.wave * WAVE_CHUNKS + i;
        const char *src = base + (int64_t)kt * TILE_BYTES + chunk * 1024 + c.lane * 16;
        const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(dst + chunk * 1024);
        asm volatile(
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %0, off"
            :
            : "v"(src), "s"(lds_addr)
            : "memory", "m0");
    }
}

// Registers one wave carries across key tiles.
template <typename T, int D>
struct WaveState {
    using vec = typename Frag<T>::vec;
    static constexpr int NU = D / (2 * Frag<T>::E);
    static constexpr int NDB = D / 32;
    vec qfrag[NU];
    int region;
    f32x16 oacc[NDB];
    float m_ref;   // reference max of raw scores (this row); raised lazily
    float l_run;   // sum of 2^((s - m_ref) ks) over this lane's keys
};

template <typename T, int D>
__device__ __forceinline__ void load_q(const AttnArgs &a, const WaveCtx &c, WaveState<T, D> &st, int region) {
    using vec = typename Frag<T>::vec;
    if (region == st.region) return;
    const vec *qs = (const vec *)a.qf[region] + c.qbase / Frag<T>::E;
#pragma unroll
    for (int u = 0; u < WaveState<T, D>::NU; ++u) st.qfrag[u] = qs[u * 64 + c.lane];
    st.region = region;
    // land them here (twice per row block at most): no compiler-counted load
    // is then outstanding while tile loads are in flight
    __builtin_amdgcn_s_waitcnt(0);
}

// S^T (64 keys x 32 rows) = K_rot Q^T: two 32-key blocks.
template <typename T, int D>
__device__ __forceinline__ void qk(const WaveCtx &c, const WaveState<T, D> &st, const char *__restrict__ kl,
                                   f32x16 (&s)[2]) {
    using F = Frag<T>;
    using vec = typename F::vec;
    constexpr int NU = WaveState<T, D>::NU;
    const vec *k = (const vec *)kl;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int u = 0; u < NU; ++u) F::mma(k[(kb * NU + u) * 64 + c.lane], st.qfrag[u], s[kb]);
    }
}

// Causal mask of the tile that holds this wave's diagonal (keys past the row).
__device__ __forceinline__ void mask_diag(const WaveCtx &c, int j0, f32x16 (&s)[2]) {
    const int lim = c.r0 + c.x - j0 - 4 * c.gsel;     // key offset k is kept iff k <= lim
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            if (kBlk * kb + 8 * (v / 4) + (v % 4) > lim) s[kb][v] = -INFINITY;
}

__device__ __forceinline__ float tile_max(const f32x16 (&s)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    return mx;
}

// Raise the reference max when the tile's row max exceeds it by more than
// 2^kLazyRescale (always on a row's first tile), rescaling O and l.
template <typename T, int D>
__device__ __forceinline__ void maybe_raise(const WaveCtx &c, WaveState<T, D> &st, float mx) {
    mx = fmaxf(mx, lane_swap32(mx));
    const bool raise = (mx - st.m_ref) * c.ks > kLazyRescale;   // true while m_ref = -inf
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = fmaxf(st.m_ref, mx);
        const float alpha = __builtin_amdgcn_exp2f((st.m_ref - m_new) * c.ks);   // 0 on a first tile
        st.l_run *= alpha;
#pragma unroll
        for (int db = 0; db < WaveState<T, D>::NDB; ++db) st.oacc[db] *= alpha;
        st.m_ref = m_new;
    }
}

// P = 2^(s ks + neg) rounded to the operand type, in PV fragment order, with
// neg = -m_ref ks (or -inf: P = 0); the row sum of the rounded P is added to l.
template <typename T, int D>
__device__ __forceinline__ void softmax_p(const WaveCtx &c, WaveState<T, D> &st, const f32x16 (&s)[2], float neg,
                                          typename Frag<T>::vec (&p)[2][kBlk / (2 * Frag<T>::E)]) {
    using F = Frag<T>;
    constexpr int E = F::E;
    constexpr int NUV = kBlk / (2 * E);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            F::set(p[kb][v / E], v % E, F::from_float(__builtin_amdgcn_exp2f(fmaf(s[kb][v], c.ks, neg))));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < NUV; ++u) st.l_run = F::sum_into(p[kb][u], st.l_run);
}

// O^T += V^T P^T
template <typename T, int D>
__device__ __forceinline__ void pv(const WaveCtx &c, WaveState<T, D> &st, const char *__restrict__ vlds,
                                   const typename Frag<T>::vec (&p)[2][kBlk / (2 * Frag<T>::E)]) {
    using F = Frag<T>;
    using vec = typename F::vec;
    constexpr int NDB = WaveState<T, D>::NDB;
    constexpr int NUV = kBlk / (2 * F::E);
    const vec *vl = (const vec *)vlds;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < NUV; ++u) F::mma(vl[((kb * NDB + db) * NUV + u) * 64 + c.lane], p[kb][u], st.oacc[db]);
}

// Tile pipeline window: kt_n .. kt_{n+NS} with their query-tile masks (-1
// past the end), whether this wave works on kt_n, and how many loads this
// wave issued in the previous step (still in flight at the next step's top).
template <int NS>
struct Pipe {
    int t[NS + 1];
    unsigned m[NS + 1];
    int n;
    int prev_loads;
    bool act0;
};

// s_waitcnt vmcnt(N) (expcnt, lgkmcnt not waited), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ bool active(const WaveCtx &c, int kt, unsigned m) {
    return c.active_rows && kt * kTile <= c.r0 + kBlk - 1 && ((m >> c.wave_qt) & 1u);
}
__device__ __forceinline__ int region_of_tile(const WaveCtx &c, int kt) {
    return kt < c.tb_succ ? 2 : (kt < c.tb_intra ? 1 : 0);
}
// the one tile of a wave that can hold keys past its rows
__device__ __forceinline__ bool is_diag(const WaveCtx &c, int kt) { return kt * kTile + kTile - 1 > c.r0; }

// Instruction order of one fused step (bf16, d = 128): two LDS reads run
// ahead; each of the 16 QK^T matrix ops is followed by a share of the
// softmax VALU work (exp2, bf16 packing, row sums) and the LDS read two ops
// ahead, so the matrix cores and the VALU stay busy together; the 16 PV ops
// follow with their V reads. Masks: 0x2 VALU, 0x8 MFMA, 0x100 LDS read.
template <typename T, int D>
__device__ __forceinline__ void interleave_step() {
    if constexpr (sizeof(T) == 2 && D == 128) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    }
}

// Step n of the pipeline over an NS-slot ring for K and one for V (tile
// kt_j lives in slot j mod NS): wait until K(kt_{n+1}) and V(kt_n) have
// landed (loads of the last NS - 2 steps may stay in flight), start K of
// kt_{n+NS} and V of kt_{n+NS-1}, mask and take the row max of kt_n, then
// the scores of kt_{n+1} on the matrix cores alongside the softmax of kt_n
// on the VALU, and the PV of kt_n.
// The block is the same whether or not this wave works on kt_n and kt_{n+1}
// (a tile past a wave's diagonal, an inactive vertical-slash tile, the last
// step): inactive work is neutralised instead of skipped -- P of an inactive
// kt_n is exactly 0 (exponent offset -inf), and an inactive kt_{n+1} is
// neither masked nor used for the reference max -- so the hot block has no
// data-dependent branches besides the rare max raise and query reload.
template <typename T, int D, int NW, int NS, int NT>
__device__ __forceinline__ void pipe_step(const AttnArgs &a, const WaveCtx &c, WaveState<T, D> &st,
                                          TileIter<NT> &it, Pipe<NS> &pp, const char *lds, uint32_t lds_base,
                                          f32x16 (&s_cur)[2], f32x16 (&s_next)[2]) {
    using vec = typename Frag<T>::vec;
    constexpr int NUV = kBlk / (2 * Frag<T>::E);
    constexpr int TILE_BYTES = 2 * kBlk * D * (int)sizeof(T);
    constexpr int STEP_LOADS = 2 * (TILE_BYTES / 1024 / NW);   // per wave: one K and one V tile share
    if constexpr (NS >= 3) {
        if (pp.prev_loads == STEP_LOADS) wait_vmcnt<STEP_LOADS>(); else __builtin_amdgcn_s_waitcnt(0);
    } else {
        __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();                    // every wave's loads landed; the slots refilled below are free
    const bool has1 = pp.t[1] >= 0;
    const bool act1 = has1 && active(c, pp.t[1], pp.m[1]);
    if (has1) load_q(a, c, st, region_of_tile(c, pp.t[1]));
    // LDS: K slots at [0, NS TILE_BYTES), V slots at [NS TILE_BYTES, 2 NS TILE_BYTES)
    int loads = 0;
    if (pp.t[NS] >= 0) {
        dma_tile<T, D, NW>(c, c.kbytes, pp.t[NS], lds_base + ((pp.n + NS) % NS) * TILE_BYTES);
        loads += STEP_LOADS / 2;
    }
    if (pp.t[NS - 1] >= 0) {
        dma_tile<T, D, NW>(c, c.vbytes, pp.t[NS - 1], lds_base + (NS + (pp.n + NS - 1) % NS) * TILE_BYTES);
        loads += STEP_LOADS / 2;
    }
    pp.prev_loads = loads;
    const char *klds_next = lds + ((pp.n + 1) % NS) * TILE_BYTES;
    const char *vlds_cur = lds + (NS + pp.n % NS) * TILE_BYTES;

    // kt_n: causal mask if it holds the diagonal, then its row max (and a
    // rare raise of the reference max) before its P is formed
    if (pp.act0) {
        if (is_diag(c, pp.t[0])) mask_diag(c, pp.t[0] * kTile, s_cur);
        maybe_raise(c, st, tile_max(s_cur));
    }
    vec p[2][NUV];
    const float neg = pp.act0 ? -st.m_ref * c.ks : -INFINITY;
    qk<T, D>(c, st, klds_next, s_next);
    softmax_p(c, st, s_cur, neg, p);
    pv<T, D>(c, st, vlds_cur, p);
    interleave_step<T, D>();

    pp.act0 = act1;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        pp.t[i] = pp.t[i + 1];
        pp.m[i] = pp.m[i + 1];
    }
    pp.t[NS] = pp.t[NS] >= 0 ? it.next(pp.m[NS]) : -1;
    ++pp.n;
}

template <typename T, int D, int NW, int NS>
// second bound: at least two waves per SIMD (256 registers per wave)
__global__ __launch_bounds__(NW * 64, 2) void dca_attention_kernel(AttnArgs a) {
    using F = Frag<T>;
    using vec = typename F::vec;
    constexpr int E = F::E;
    constexpr int NUV = kBlk / (2 * E);
    constexpr int NDB = D / 32;
    constexpr int BM = kBlk * NW;              // rows per workgroup
    constexpr int NT = BM / kTile;             // 64-row query tiles per workgroup
    constexpr int BLK_ELEMS = kBlk * D;
    constexpr int TILE_BYTES = 2 * BLK_ELEMS * (int)sizeof(T);   // one 64-key tile of K (or V)
    static_assert(NT >= 1 && BM % kTile == 0, "workgroup rows must cover whole 64-row tiles");

    // LDS: a ring of NS K tiles and a ring of NS V tiles. K runs one tile
    // ahead of V: while tile n's P meets V(n), tile n+1's scores are formed
    // from K(n+1); loads of the next NS - 1 tiles are in flight.
    extern __shared__ __attribute__((aligned(1024))) char lds_dyn[];
    char *lds = lds_dyn;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void *)lds;

    // ---- decode the work item -------------------------------------------
    const int bid = blockIdx.x;
    const int xcd = bid % kXcds;
    const int slot = bid / kXcds;
    const int gg = slot % a.G;
    const int mm = (slot / a.G) % a.M;
    const int tt = slot / (a.G * a.M);
    const int sigma = xcd + kXcds * mm;
    const int kvg = sigma % a.KVH;
    const int kres = sigma / a.KVH;
    const int rt_desc = kres + a.s_split * tt;
    if (slot >= a.per_xcd || rt_desc >= a.n_rt) return;
    const int rt = a.n_rt - 1 - rt_desc;
    const int b = kvg / a.Hkv;
    const int kvh = kvg % a.Hkv;
    const int h = kvh * a.G + gg;
    const int64_t bh = (int64_t)b * a.Hq + h;
    const int64_t bkv = (int64_t)b * a.Hkv + kvh;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64;
    const int S = (int)a.S;
    const int i0 = rt * BM;
    const int last_row = (i0 + BM < S ? i0 + BM : S) - 1;
    WaveCtx c;
    c.lane = lane;
    c.x = lane % 32;
    c.gsel = lane / 32;
    c.wave = wave;
    c.r0 = i0 + kBlk * wave;                       // this wave's first row
    c.active_rows = c.r0 < S;
    // key-tile boundaries of this wave's regions: tiles [0, tb_succ) are
    // inter-chunk, [tb_succ, tb_intra) successive, [tb_intra, ...) intra
    const int tiles_per_chunk = (int)(a.C / kTile);
    const int cq = c.r0 / (int)a.C;
    c.tb_intra = cq * tiles_per_chunk;
    c.tb_succ = cq >= 1 ? c.tb_intra - tiles_per_chunk : 0;
    c.wave_qt = (kBlk * wave) / kTile;
    c.ks = a.ks;
    c.qbase = (bh * a.nblk + c.r0 / kBlk) * (int64_t)BLK_ELEMS;
    c.kbytes = (const char *)a.kf + bkv * a.nblk * (int64_t)BLK_ELEMS * (int64_t)sizeof(T);
    c.vbytes = (const char *)a.vf + bkv * a.nblk * (int64_t)BLK_ELEMS * (int64_t)sizeof(T);

    WaveState<T, D> st;
    st.region = -1;
#pragma unroll
    for (int db = 0; db < NDB; ++db) st.oacc[db] = f32x16{};
    st.m_ref = -INFINITY;
    st.l_run = 0.f;

    // ---- pipeline prologue ---------------------------------------------------
    TileIter<NT> it;
    it.init(a, h, i0, S, last_row / kTile);
    Pipe<NS> pp;
    pp.t[0] = it.next(pp.m[0]);
#pragma unroll
    for (int i = 1; i <= NS; ++i) {
        pp.m[i] = 0;
        pp.t[i] = pp.t[i - 1] >= 0 ? it.next(pp.m[i]) : -1;
    }
    pp.n = 0;
    // slots: K(kt_j), V(kt_j) -> j mod NS. Step 0 needs K(kt_0), K(kt_1) and
    // V(kt_0) landed; with three slots, K(kt_2) and V(kt_1) (the loads a step
    // leaves in flight) may still be on their way.
    static_assert(NS == 2 || NS == 3, "two or three ring slots");
    constexpr int STEP_LOADS = 2 * (TILE_BYTES / 1024 / NW);
    if (pp.t[0] >= 0) {
        dma_tile<T, D, NW>(c, c.kbytes, pp.t[0], lds_base);
        dma_tile<T, D, NW>(c, c.vbytes, pp.t[0], lds_base + NS * TILE_BYTES);
    }
    if (pp.t[1] >= 0) dma_tile<T, D, NW>(c, c.kbytes, pp.t[1], lds_base + TILE_BYTES);
    pp.prev_loads = 0;
    if constexpr (NS == 3) {
        if (pp.t[2] >= 0) {
            dma_tile<T, D, NW>(c, c.kbytes, pp.t[2], lds_base + 2 * TILE_BYTES);
            pp.prev_loads += STEP_LOADS / 2;
        }
        if (pp.t[1] >= 0) {
            dma_tile<T, D, NW>(c, c.vbytes, pp.t[1], lds_base + (NS + 1) * TILE_BYTES);
            pp.prev_loads += STEP_LOADS / 2;
        }
        if (pp.prev_loads == STEP_LOADS) wait_vmcnt<STEP_LOADS>(); else __builtin_amdgcn_s_waitcnt(0);
    } else {
        __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    f32x16 sa[2], sb[2];          // scores of the current and the next tile (roles alternate)
    sa[0] = sa[1] = f32x16{};
    pp.act0 = pp.t[0] >= 0 && active(c, pp.t[0], pp.m[0]);
    if (pp.act0) {
        load_q(a, c, st, region_of_tile(c, pp.t[0]));
        qk<T, D>(c, st, lds, sa);
    }

    // ---- steady state: step n works on tiles kt_n and kt_{n+1} ---------------
    while (pp.t[0] >= 0) {
        pipe_step<T, D, NW, NS>(a, c, st, it, pp, lds, lds_base, sa, sb);
        if (pp.t[0] < 0) break;
        pipe_step<T, D, NW, NS>(a, c, st, it, pp, lds, lds_base, sb, sa);
    }

    // ---- epilogue -----------------------------------------------------------
    const int row = c.r0 + c.x;
    if (!c.active_rows || row >= S) return;
    const float l_tot = st.l_run + lane_swap32(st.l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T *orow = (T *)a.out + (bh * a.S + row) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
            const int d0 = 32 * db + 8 * vq + 4 * c.gsel;
#pragma unroll
            for (int e = 0; e < 4; ++e) orow[d0 + e] = F::from_float(st.oacc[db][4 * vq + e] * inv);
        }
    if (a.lse != nullptr && c.gsel == 0) {
        a.lse[bh * a.S + row] = l_tot > 0.f ? (st.m_ref * c.ks + log2f(l_tot)) * 0.69314718055994531f
                                            : -INFINITY;
    }
}

template <typename T, int D, int NW, int NS>
static int launch_attn_t(const Problem &p, const AttnArgs &a0, void *stream) {
    constexpr int BM = kBlk * NW;
    AttnArgs a = a0;
    a.n_rt = (int32_t)((p.S + BM - 1) / BM);
    int gcd = 1;
    for (int d = 1; d <= kXcds; ++d)
        if (a.KVH % d == 0 && kXcds % d == 0) gcd = d;
    a.s_split = kXcds / gcd;
    a.M = a.KVH / gcd;
    const int64_t per_stream = (a.n_rt + a.s_split - 1) / a.s_split;
    a.per_xcd = (int32_t)(per_stream * a.M * a.G);
    const int64_t grid = (int64_t)a.per_xcd * kXcds;
    const int lds_bytes = 2 * NS * (2 * kBlk * D * (int)sizeof(T));   // K and V rings of NS tiles
    auto kern = dca_attention_kernel<T, D, NW, NS>;
    if (lds_bytes > 65536) {
        const hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 lds_bytes);
        if (e != hipSuccess) return (int)e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), lds_bytes, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

int launch_attention(const Problem &p, float yarn_scale, void *out, float *lse, const void *ws,
                     const Layout &L, void *stream) {
    AttnArgs a{};
    for (int i = 0; i < 3; ++i) a.qf[i] = (const char *)ws + L.q[i];
    a.kf = (const char *)ws + L.k;
    a.vf = (const char *)ws + L.v;
    a.out = out;
    a.lse = lse;
    a.S = p.S;
    a.C = p.C;
    a.Hq = (int32_t)p.Hq;
    a.Hkv = (int32_t)p.Hkv;
    a.G = (int32_t)p.G;
    a.nblk = (int32_t)(p.S_pad / kBlk);
    a.ks = yarn_scale * p.softmax_scale * 1.4426950408889634f;
    a.KVH = (int32_t)(p.B * p.Hkv);
    a.sparse = p.sparse ? 1 : 0;
    if (p.sparse) {
        a.vt = (const int32_t *)((const char *)ws + L.vs_vt);
        a.vt_n = (const int32_t *)((const char *)ws + L.vs_vt_n);
        a.dl = (const int32_t *)((const char *)ws + L.vs_dl);
        a.dl_n = (const int32_t *)((const char *)ws + L.vs_dl_n);
        a.list_stride = (int32_t)p.n_tiles;
    }
    if (p.dtype == DCA_BF16)
        return p.D == 128 ? launch_attn_t<__bf16, 128, 8, 3>(p, a, stream)
                          : launch_attn_t<__bf16, 64, 8, 3>(p, a, stream);
    return p.D == 128 ? launch_attn_t<float, 128, 2, 2>(p, a, stream)
                      : launch_attn_t<float, 64, 4, 3>(p, a, stream);
}

}  // namespace dca
