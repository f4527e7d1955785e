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
// tiles staged through an LDS ring, two tiles per barrier, the next two in
// flight; half the waves run half a tile behind the others, so the two waves
// of a SIMD are in different phases. Per wave and tile:
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
// tiles inactive for its own query tile. Its scattered tiles come through
// separate LDS rings (SPLIT): K two tiles ahead, V one.
//
// Grid order: heaviest row tiles first; the work list is cut into per-XCD
// streams so that the workgroups resident on one XCD (workgroup i lands on
// XCD i mod 8) share one KV head and sweep the same keys through that XCD's
// L2. Vertical-slash launches are ordered differently (kSparseGeneration).
//
// A launch computes the rows [q0, q0 + NQ) of the sequence (a whole-sequence
// prefill, or one block of a chunked prefill [mizuki, Chunked Prefill]) with
// the keys kept at their sequence positions. With FUSED, each wave reads its
// rows of the caller's queries and rotates them itself when it enters a
// region, instead of reading the pre-pass's rotated variants.
#include <hip/hip_runtime.h>

#include "dca_internal.h"
#include "frag.h"
#include "tile_math.h"

namespace dca {

struct AttnArgs {
    const void *qf[3];
    const void *q_nat;           // fused rotation: the call's queries [B][Hq][NQ][D], rotated here
    const float2 *table;         // fused rotation: cos/sin table [C + W][D/2]
    const void *kf;
    const void *vf;
    void *out;
    float *lse;
    int64_t S, C, W;             // S: end of the call's rows (= keys visible to the last row)
    int64_t q0, NQ;              // the call's rows are [q0, q0 + NQ); out and lse hold NQ rows
    int32_t Hq, Hkv, G;
    int32_t nblk_q, nblk_kv;     // 32-row blocks per head in the query / key-value sections
    // work decode
    int32_t n_rt, KVH, s_split, M, per_xcd, rgen;
    // vertical-slash lists
    const int32_t *vt, *vt_n, *dl, *dl_n;
    int32_t list_stride;
    int32_t sparse;
};

constexpr int kNone = 0x7fffffff;

// Vertical-slash grid order. The work is cut into units of this many
// adjacent row tiles of one query head (about the workgroups one XCD holds at
// once); units are dealt round-robin to the XCDs, KV group by KV group. The
// workgroups running together on an XCD then share their head's vertical
// tiles and many slash tiles through its L2, and all XCDs read the keys of
// one KV group, whose recently used tiles the memory-side cache keeps. Dense
// launches keep the query heads of a KV group together on an XCD instead
// (every workgroup reads every key).
constexpr int kSparseGeneration = 64;

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
struct WaveCtx {
    int lane, x, gsel, wave, r0, tb_succ, tb_intra, wave_qt;
    bool active_rows;
    int64_t bh;                  // batch * n_q_heads + head
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
// Two address forms, the same addresses: SADDR takes the piece's wave-uniform
// base in an SGPR pair plus the lane's 16-byte offset in one VGPR, shared by
// every piece and both tensors; otherwise each piece's 64-bit per-lane
// address is formed in VGPRs. SADDR frees VGPRs at the cost of SGPRs: the
// bf16 kernels take it (they need the registers for their score start tuple
// and, fused, the rotation); the fp32 ones keep the VGPR form.
template <typename T, int D, int NW, bool SADDR>
__device__ __forceinline__ void dma_tile(const WaveCtx &c, const char *base, int kt, uint32_t dst) {
    constexpr int TILE_BYTES = 2 * kBlk * D * (int)sizeof(T);
    constexpr int WAVE_CHUNKS = TILE_BYTES / 1024 / NW;
    static_assert(TILE_BYTES % (1024 * NW) == 0, "tile split");
#pragma unroll
    for (int i = 0; i < WAVE_CHUNKS; ++i) {
        const int chunk = c.wave * WAVE_CHUNKS + i;
        const char *src = base + (int64_t)kt * TILE_BYTES + chunk * 1024;
        const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(dst + chunk * 1024);
        if constexpr (SADDR)
            asm volatile(
                "s_mov_b32 m0, %2\n\t"
                "s_nop 0\n\t"
                "global_load_lds_dwordx4 %0, %1"
                :
                : "v"(c.lane * 16), "s"(src), "s"(lds_addr)
                : "memory", "m0");
        else
            asm volatile(
                "s_mov_b32 m0, %1\n\t"
                "s_nop 0\n\t"
                "global_load_lds_dwordx4 %0, off"
                :
                : "v"(src + c.lane * 16), "s"(lds_addr)
                : "memory", "m0");
    }
}

// s_waitcnt vmcnt(N) (expcnt, lgkmcnt not waited), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `pending` (<= MAXP) tiles of SL loads each are in flight.
template <int SL, int MAXP>
__device__ __forceinline__ void wait_tiles(int pending) {
    if constexpr (MAXP >= 3) if (pending == 3) { wait_vmcnt<3 * SL>(); return; }
    if constexpr (MAXP >= 2) if (pending == 2) { wait_vmcnt<2 * SL>(); return; }
    if constexpr (MAXP >= 1) if (pending == 1) { wait_vmcnt<SL>(); return; }
    __builtin_amdgcn_s_waitcnt(0);
}

__device__ __forceinline__ bool active(const WaveCtx &c, int kt, unsigned m) {
    return c.active_rows && kt * kTile <= c.r0 + kBlk - 1 && ((m >> c.wave_qt) & 1u);
}
__device__ __forceinline__ int region_of_tile(const WaveCtx &c, int kt) {
    return kt < c.tb_succ ? 2 : (kt < c.tb_intra ? 1 : 0);
}
// the one tile of a wave that can hold keys past its rows
__device__ __forceinline__ bool is_diag(const WaveCtx &c, int kt) { return kt * kTile + kTile - 1 > c.r0; }

// The lane's index within its wave, formed afresh where it is used: asm, so
// that the compiler neither hoists it nor keeps values derived from it live
// across the tile loop (the rare paths that use it recompute theirs).
__device__ __forceinline__ int fresh_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Causal mask of the tile that holds this wave's diagonal (keys past the row).
// FRESH: the lane terms come from fresh_lane(), not from registers kept live.
template <bool FRESH>
__device__ __forceinline__ void mask_diag(const WaveCtx &c, int j0, f32x16 (&s)[2]) {
    int lim;                                          // key offset k is kept iff k <= lim
    if constexpr (FRESH) {
        const int ln = fresh_lane();
        lim = c.r0 + ln % 32 - j0 - 4 * (ln / 32);
    } else {
        lim = c.r0 + c.x - j0 - 4 * c.gsel;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            if (kBlk * kb + 8 * (v / 4) + (v % 4) > lim) s[kb][v] = -INFINITY;
}

// The query fragments of the wave's rows for a region: read from the
// rotated variant the pre-pass wrote, or (FUSED) read from the caller's
// queries and turned here, with the same table entries and arithmetic as the
// pre-pass, so both give the same bits. In a lane, fragment u and u + NU/2
// hold the two halves (m, m + d/2) of the same rotation pairs.
template <typename T, int D, bool FUSED>
__device__ __forceinline__ void load_q(const AttnArgs &a, const WaveCtx &c, WaveState<T, D> &st, int region) {
    using F = Frag<T>;
    using vec = typename F::vec;
    constexpr int E = F::E;
    constexpr int NU = WaveState<T, D>::NU;
    if (region == st.region) return;
    if constexpr (FUSED) {
        const int ln = fresh_lane();
        const int row = c.r0 + ln % 32, gsel = ln / 32;
        const bool valid = row < (int)a.S;
        const T *src = (const T *)a.q_nat + ((c.bh * a.NQ) + (row - a.q0)) * D + E * gsel;
#pragma unroll
        for (int u = 0; u < NU; ++u) st.qfrag[u] = valid ? *(const vec *)(src + 2 * E * u) : F::zero();
        const int64_t p = region == 0 ? pos_intra(row, a.C) : (region == 1 ? pos_succ(row, a.C, a.W) : pos_inter(a.C, a.W));
        const float2 *tab = a.table + p * (D / 2) + E * gsel;
#pragma unroll
        for (int u = 0; u < NU / 2; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float2 cs = tab[2 * E * u + e];
                const float2 r = rope_pair((float)F::get(st.qfrag[u], e), (float)F::get(st.qfrag[u + NU / 2], e),
                                           cs.x, cs.y);
                F::set(st.qfrag[u], e, F::from_float(r.x));
                F::set(st.qfrag[u + NU / 2], e, F::from_float(r.y));
            }
    } else {
        const vec *qs = (const vec *)a.qf[region] + c.qbase / E;
#pragma unroll
        for (int u = 0; u < NU; ++u) st.qfrag[u] = qs[u * 64 + c.lane];
    }
    st.region = region;
    // land them here (twice per row block at most): no compiler-counted load
    // is then outstanding while tile loads are in flight
    __builtin_amdgcn_s_waitcnt(0);
}

// Waves per SIMD the register budget is sized for: two (256 registers per
// wave), except fp32 with d = 128, whose V fragments alone take 128 registers
// per lane: one (512), so that nothing spills.
template <typename T, int D>
constexpr int kMinWavesPerSimd = (sizeof(T) == 4 && D == 128) ? 1 : 2;

template <typename T, int D, int NW, int NS, int TPS, bool FUSED, bool SPLIT = false>
__global__ __launch_bounds__(NW * 64, (kMinWavesPerSimd<T, D>)) void dca_attention_kernel(AttnArgs a) {
    using F = Frag<T>;
    using vec = typename F::vec;
    constexpr int E = F::E;
    constexpr int NUV = kBlk / (2 * E);
    constexpr int NDB = D / 32;
    constexpr int BM = kBlk * NW;              // rows per workgroup
    constexpr int NT = BM / kTile;             // 64-row query tiles per workgroup
    constexpr int BLK_ELEMS = kBlk * D;
    constexpr int TILE_BYTES = 2 * BLK_ELEMS * (int)sizeof(T);   // one 64-key tile of K (or V)
    constexpr int STEP_LOADS = 2 * (TILE_BYTES / 1024 / NW);     // per wave and step: its share of K and V
    static_assert(NT >= 1 && BM % kTile == 0, "workgroup rows must cover whole 64-row tiles");

    extern __shared__ __attribute__((aligned(1024))) char lds_dyn[];
    char *lds = lds_dyn;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void *)lds;

    // ---- decode the work item -------------------------------------------
    const int bid = blockIdx.x;
    const int xcd = bid % kXcds;
    const int slot = bid / kXcds;
    int gg, kvg, rt_desc;
    if (a.sparse) {
        // generation units u = (kv group, row-tile block, query head), dealt
        // round-robin to the XCDs so that all XCDs work on one KV group
        const int inner = slot % a.rgen;
        const int u = (slot / a.rgen) * kXcds + xcd;
        const int nrblk = (a.n_rt + a.rgen - 1) / a.rgen;
        kvg = u / (nrblk * a.G);
        const int rem = u % (nrblk * a.G);
        gg = rem % a.G;
        rt_desc = (rem / a.G) * a.rgen + inner;
        if (slot >= a.per_xcd || kvg >= a.KVH || rt_desc >= a.n_rt) return;
    } else {
        gg = slot % a.G;
        const int mm = (slot / a.G) % a.M;
        const int tt = slot / (a.G * a.M);
        const int sigma = xcd + kXcds * mm;
        kvg = sigma % a.KVH;
        const int kres = sigma / a.KVH;
        rt_desc = kres + a.s_split * tt;
        if (slot >= a.per_xcd || rt_desc >= a.n_rt) return;
    }
    const int rt = a.n_rt - 1 - rt_desc;
    const int b = kvg / a.Hkv;
    const int kvh = kvg % a.Hkv;
    const int h = kvh * a.G + gg;
    const int64_t bh = (int64_t)b * a.Hq + h;
    const int64_t bkv = (int64_t)b * a.Hkv + kvh;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64;
    const int S = (int)a.S;
    const int q0 = (int)a.q0;
    const int i0 = q0 + rt * BM;
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
    c.bh = bh;
    c.qbase = (bh * a.nblk_q + (c.r0 - q0) / kBlk) * (int64_t)BLK_ELEMS;
    c.kbytes = (const char *)a.kf + bkv * a.nblk_kv * (int64_t)BLK_ELEMS * (int64_t)sizeof(T);
    c.vbytes = (const char *)a.vf + bkv * a.nblk_kv * (int64_t)BLK_ELEMS * (int64_t)sizeof(T);

    WaveState<T, D> st;
    st.region = -1;
    st.first = true;
#pragma unroll
    for (int db = 0; db < NDB; ++db) st.oacc[db] = f32x16{};
    st.mref = 0.f;
    st.l_run = 0.f;
    // start of the score accumulators, -mref (0 before the first tile), kept
    // in registers where they fit: bf16
    constexpr bool C0 = sizeof(T) == 2;
    // bf16 kernels take the SGPR-based tile loads and the recomputed mask
    // terms, which free the registers that tuple (and, in the fused kernel,
    // the rotation) needs
    constexpr bool LEAN = sizeof(T) == 2;
    f32x16 c0 = {};

    // The per-tile work (QK, mask, softmax step, PV) is written out in each of
    // the loops below: moved into a shared function or lambda, it changes the
    // register allocation and spills.
    if constexpr (SPLIT) {
        // separate rings: K in 3 slots (two tiles ahead), V in 2 (one ahead).
        // Per step: V(n+1), then K(n+2); at the next step's top every load but
        // that K has landed (loads complete in issue order).
        constexpr int KL = TILE_BYTES / 1024 / NW;       // loads per wave and tile
        const uint32_t vbase_lds = lds_base + 3u * TILE_BYTES;
        TileIter<NT> it;
        it.init(a, h, i0, S, last_row / kTile);
        int t[3];
        unsigned m[3] = {0, 0, 0};
        t[0] = it.next(m[0]);
        t[1] = t[0] >= 0 ? it.next(m[1]) : -1;
        t[2] = t[1] >= 0 ? it.next(m[2]) : -1;
        if (t[0] >= 0) {
            dma_tile<T, D, NW, true>(c, c.kbytes, t[0], lds_base);
            dma_tile<T, D, NW, true>(c, c.vbytes, t[0], vbase_lds);
        }
        if (t[1] >= 0) dma_tile<T, D, NW, true>(c, c.kbytes, t[1], lds_base + 1u * TILE_BYTES);
        for (int n = 0; t[0] >= 0; ++n) {
            if (t[1] >= 0) wait_vmcnt<KL>(); else __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();                 // K(n), V(n) landed; V slot (n+1)%2 and K slot (n+2)%3 are free
            if (t[1] >= 0) dma_tile<T, D, NW, true>(c, c.vbytes, t[1], vbase_lds + (uint32_t)((n + 1) & 1) * TILE_BYTES);
            if (t[2] >= 0) dma_tile<T, D, NW, true>(c, c.kbytes, t[2], lds_base + (uint32_t)((n + 2) % 3) * TILE_BYTES);
            const int kt = t[0];
            if (active(c, kt, m[0])) {
                load_q<T, D, FUSED>(a, c, st, region_of_tile(c, kt));
                const char *kcur = lds + (n % 3) * TILE_BYTES;
                const char *vcur = lds + 3 * TILE_BYTES + (n & 1) * TILE_BYTES;
                f32x16 s[2];
                if constexpr (C0)
                    tile_scores_from<T, D, true>(c.lane, st, c0, kcur, s);
                else
                    tile_scores<T, D, true>(c.lane, st, kcur, s);
                if (is_diag(c, kt)) mask_diag<true>(c, kt * kTile, s);
                VFrags<T, D> vf;
                load_v<T, D>(c.lane, vcur, vf);
                __builtin_amdgcn_sched_barrier(0);
                vec p[2][NUV];
                float psum = tile_p<T>(s, p);
                const bool ok = psum <= kPsumLimit;          // false for inf and NaN too
                if (__builtin_amdgcn_ballot_w64(!ok || st.first) != 0) {
                    raise_ref<T, D>(st, s);
                    psum = tile_p<T>(s, p);
                    if constexpr (C0) {
#pragma unroll
                        for (int v = 0; v < 16; ++v) c0[v] = -st.mref;
                    }
                }
                st.l_run += psum;
                __builtin_amdgcn_sched_barrier(0);
                tile_pv<T, D>(st, vf, p);
            }
            t[0] = t[1]; m[0] = m[1];
            t[1] = t[2]; m[1] = m[2];
            t[2] = t[1] >= 0 ? it.next(m[2]) : -1;
        }
    } else if constexpr (TPS == 2) {
        // Two key tiles per step, lagged pairs. LDS holds a ring of NS = 4
        // slots of [K tile | V tile]; tile j (in visiting order) lives in slot
        // j mod 4. Step n computes tiles 2n and 2n+1 and, right after its
        // barrier, starts the loads of tiles 2n+2 and 2n+3 into the slots of
        // tiles 2n-2 and 2n-1, which every wave has finished reading: a tile's
        // K and V are read from LDS only within its own step.
        // The second half of the waves (one of the two waves on each SIMD) runs
        // half a tile behind: it leaves the PV product of its step's second
        // tile, with that tile's V fragments and P in registers, for after the
        // next barrier. The barrier then no longer lines the two waves of a
        // SIMD up in the same phase: one's softmax runs under the other's
        // matrix work. Every row still sees its tiles' QK, softmax and PV in
        // the same order, so the results are unchanged.
        static_assert(NS == 4, "lagged ring size");
        const bool lag = wave >= NW / 2;
        TileIter<NT> it;
        it.init(a, h, i0, S, last_row / kTile);
        int t[4];                        // tiles 2n .. 2n+3 (-1 past the end)
        unsigned m[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m[i] = 0;
            t[i] = (i == 0 || t[i - 1] >= 0) ? it.next(m[i]) : -1;
        }
        auto issue = [&](int kt, int j) __attribute__((always_inline)) {
            const uint32_t slot_addr = lds_base + (uint32_t)(j % NS) * 2 * TILE_BYTES;
            dma_tile<T, D, NW, LEAN>(c, c.kbytes, kt, slot_addr);
            dma_tile<T, D, NW, LEAN>(c, c.vbytes, kt, slot_addr + TILE_BYTES);
        };
        if (t[0] >= 0) issue(t[0], 0);
        if (t[1] >= 0) issue(t[1], 1);
        VFrags<T, D> vf;                 // a lagging wave's pending tile: its V and P
        vec p[2][NUV];
        bool pend = false;
        for (int n = 0; t[0] >= 0; ++n) {
            __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of tiles 2n, 2n+1
            __syncthreads();                 // ... and everyone's; slots of 2n-2, 2n-1 free
            // The leading waves start their share of the next step's loads right
            // away; the lagging ones after their deferred PV. Issued by all eight
            // at once, the loads queue in the vector-memory path and hold up the
            // waves behind them (a timestamp probe put that at 460-920 cycles of
            // a 6800-cycle step; split this way, 1.5-2% faster at 1M).
            if (!lag) {
                if (t[2] >= 0) issue(t[2], 2 * n + 2);
                if (t[3] >= 0) issue(t[3], 2 * n + 3);
            }
            if (pend) {
                tile_pv<T, D>(st, vf, p);
                pend = false;
            }
            if (lag) {
                if (t[2] >= 0) issue(t[2], 2 * n + 2);
                if (t[3] >= 0) issue(t[3], 2 * n + 3);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int kt = t[i];
                if (kt >= 0 && active(c, kt, m[i])) {
                    load_q<T, D, FUSED>(a, c, st, region_of_tile(c, kt));
                    const char *cur = lds + ((2 * n + i) % NS) * 2 * TILE_BYTES;
                    f32x16 s[2];
                    // the raised issue priority is held through the softmax here
                    if constexpr (C0)
                        tile_scores_from<T, D, true, true>(c.lane, st, c0, cur, s);
                    else
                        tile_scores<T, D, true>(c.lane, st, cur, s);
                    if (is_diag(c, kt)) mask_diag<LEAN>(c, kt * kTile, s);
                    load_v<T, D>(c.lane, cur + TILE_BYTES, vf);
                    __builtin_amdgcn_sched_barrier(0);
                    float psum = tile_p<T>(s, p);
                    const bool ok = psum <= kPsumLimit;          // false for inf and NaN too
                    if (__builtin_amdgcn_ballot_w64(!ok || st.first) != 0) {
                        raise_ref<T, D>(st, s);
                        psum = tile_p<T>(s, p);
                        if constexpr (C0) {
#pragma unroll
                            for (int v = 0; v < 16; ++v) c0[v] = -st.mref;
                        }
                    }
                    st.l_run += psum;
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_setprio(0);
                    if (lag && i == 1)
                        pend = true;
                    else
                        tile_pv<T, D>(st, vf, p);
                }
            }
            t[0] = t[2]; m[0] = m[2];
            t[1] = t[3]; m[1] = m[3];
            t[2] = t[1] >= 0 ? it.next(m[2]) : -1;
            t[3] = t[2] >= 0 ? it.next(m[3]) : -1;
        }
        if (pend) tile_pv<T, D>(st, vf, p);
    } else {
    // ---- other step sizes (fp32 with d = 128: one tile per step) --------------
    // A step handles TPS key tiles between two barriers. LDS holds a ring of NS
    // slots of [K tile | V tile]; tile j (in visiting order) lives in slot
    // j mod NS. Step n uses tiles nTPS .. nTPS+TPS-1 and, once every wave is
    // past the barrier that frees the slots of step n-1, starts the loads of
    // tiles nTPS+NS-TPS .. nTPS+NS-1 into them.
    static_assert(NS >= 2 * TPS && NS - 2 * TPS <= 3, "ring size");
    TileIter<NT> it;
    it.init(a, h, i0, S, last_row / kTile);
    int t[NS];                       // tiles nTPS .. nTPS+NS-1 (-1 past the end)
    unsigned m[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        m[i] = 0;
        t[i] = (i == 0 || t[i - 1] >= 0) ? it.next(m[i]) : -1;
    }
    auto issue = [&](int kt, int j) __attribute__((always_inline)) {
        const uint32_t slot_addr = lds_base + (uint32_t)(j % NS) * 2 * TILE_BYTES;
        dma_tile<T, D, NW, LEAN>(c, c.kbytes, kt, slot_addr);
        dma_tile<T, D, NW, LEAN>(c, c.vbytes, kt, slot_addr + TILE_BYTES);
    };
#pragma unroll
    for (int i = 0; i < NS - TPS; ++i)
        if (t[i] >= 0) issue(t[i], i);

    // ---- main loop: TPS key tiles per step -------------------------------------
    for (int n = 0; t[0] >= 0; ++n) {
        // tiles at window positions TPS .. NS-TPS-1 may stay in flight
        int pending = 0;
#pragma unroll
        for (int i = TPS; i < NS - TPS; ++i) pending += t[i] >= 0;
        wait_tiles<STEP_LOADS, NS - 2 * TPS>(pending);
        __syncthreads();                     // step n's tiles landed; the slots of step n-1 are free
        if (active(c, t[0], m[0])) load_q<T, D, FUSED>(a, c, st, region_of_tile(c, t[0]));
#pragma unroll
        for (int i = 0; i < TPS; ++i)
            if (t[NS - TPS + i] >= 0) issue(t[NS - TPS + i], n * TPS + NS - TPS + i);
#pragma unroll
        for (int i = 0; i < TPS; ++i) {
            const int kt = t[i];
            if (kt >= 0 && active(c, kt, m[i])) {
                if (i > 0) load_q<T, D, FUSED>(a, c, st, region_of_tile(c, kt));
                const char *cur = lds + ((n * TPS + i) % NS) * 2 * TILE_BYTES;
                f32x16 s[2];
                if constexpr (C0)
                    tile_scores_from<T, D, true>(c.lane, st, c0, cur, s);
                else
                    tile_scores<T, D, true>(c.lane, st, cur, s);
                if (is_diag(c, kt)) mask_diag<LEAN>(c, kt * kTile, s);
                VFrags<T, D> vf;
                load_v<T, D>(c.lane, cur + TILE_BYTES, vf);
                __builtin_amdgcn_sched_barrier(0);
                vec p[2][NUV];
                float psum = tile_p<T>(s, p);
                const bool ok = psum <= kPsumLimit;          // false for inf and NaN too
                if (__builtin_amdgcn_ballot_w64(!ok || st.first) != 0) {
                    raise_ref<T, D>(st, s);
                    psum = tile_p<T>(s, p);
                    if constexpr (C0) {
#pragma unroll
                        for (int v = 0; v < 16; ++v) c0[v] = -st.mref;
                    }
                }
                st.l_run += psum;
                __builtin_amdgcn_sched_barrier(0);
                tile_pv<T, D>(st, vf, p);
            }
        }
#pragma unroll
        for (int i = 0; i < NS - TPS; ++i) {
            t[i] = t[i + TPS];
            m[i] = m[i + TPS];
        }
#pragma unroll
        for (int i = NS - TPS; i < NS; ++i) t[i] = t[i - 1] >= 0 ? it.next(m[i]) : -1;
    }

    }
    // ---- epilogue -----------------------------------------------------------
    const int row = c.r0 + c.x;
    if (!c.active_rows || row >= S) return;
    const float l_tot = st.l_run + lane_swap32(st.l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T *orow = (T *)a.out + (bh * a.NQ + (row - q0)) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
            const int d0 = 32 * db + 8 * vq + 4 * c.gsel;
#pragma unroll
            for (int e = 0; e < 4; ++e) orow[d0 + e] = F::from_float(st.oacc[db][4 * vq + e] * inv);
        }
    if (a.lse != nullptr && c.gsel == 0) {
        // natural log: (mref + log2 l) ln 2
        a.lse[bh * a.NQ + (row - q0)] = l_tot > 0.f ? (st.mref + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
}

template <typename T, int D, int NW, int NS, int TPS, bool SPLIT = false>
static int launch_attn_t(const Problem &p, const AttnArgs &a0, void *stream) {
    constexpr int BM = kBlk * NW;
    AttnArgs a = a0;
    a.n_rt = (int32_t)((p.NQ + BM - 1) / BM);
    int gcd = 1;
    for (int d = 1; d <= kXcds; ++d)
        if (a.KVH % d == 0 && kXcds % d == 0) gcd = d;
    a.s_split = kXcds / gcd;
    a.M = a.KVH / gcd;
    const int64_t per_stream = (a.n_rt + a.s_split - 1) / a.s_split;
    a.rgen = a.sparse ? kSparseGeneration : 1;
    if (a.sparse) {
        const int64_t units = (int64_t)a.KVH * a.G * ((a.n_rt + a.rgen - 1) / a.rgen);
        a.per_xcd = (int32_t)((units + kXcds - 1) / kXcds * a.rgen);
    } else {
        a.per_xcd = (int32_t)(per_stream * a.M * a.G);
    }
    const int64_t grid = (int64_t)a.per_xcd * kXcds;
    // NS slots of [K tile | V tile], or 3 K slots and 2 V slots (SPLIT)
    const int lds_bytes = (SPLIT ? 5 : 2 * NS) * (2 * kBlk * D * (int)sizeof(T));
    auto kern = a.q_nat != nullptr ? dca_attention_kernel<T, D, NW, NS, TPS, true, SPLIT>
                                   : dca_attention_kernel<T, D, NW, NS, TPS, false, SPLIT>;
    if (lds_bytes > 65536) {
        const hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 lds_bytes);
        if (e != hipSuccess) return (int)e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), lds_bytes, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

int launch_attention(const Problem &p, void *out, float *lse, const void *ws, const Layout &L, void *stream,
                     const void *q_nat) {
    AttnArgs a{};
    a.q_nat = q_nat;
    a.table = (const float2 *)((const char *)ws + L.table);
    a.W = p.W;
    for (int i = 0; i < 3; ++i) a.qf[i] = (const char *)ws + L.q[i];
    a.kf = (const char *)ws + L.k;
    a.vf = (const char *)ws + L.v;
    a.out = out;
    a.lse = lse;
    a.S = p.q0 + p.NQ;
    a.q0 = p.q0;
    a.NQ = p.NQ;
    a.C = p.C;
    a.Hq = (int32_t)p.Hq;
    a.Hkv = (int32_t)p.Hkv;
    a.G = (int32_t)p.G;
    a.nblk_q = (int32_t)(p.NQ_pad / kBlk);
    a.nblk_kv = (int32_t)(p.S_pad / kBlk);
    a.KVH = (int32_t)(p.B * p.Hkv);
    a.sparse = p.sparse ? 1 : 0;
    if (p.sparse) {
        a.vt = (const int32_t *)((const char *)ws + L.vs_vt);
        a.vt_n = (const int32_t *)((const char *)ws + L.vs_vt_n);
        a.dl = (const int32_t *)((const char *)ws + L.vs_dl);
        a.dl_n = (const int32_t *)((const char *)ws + L.vs_dl_n);
        a.list_stride = (int32_t)p.n_tiles;
    }
    // Sparse: 128-row workgroups, two per CU. A workgroup visits the union of
    // its query tiles' active key tiles, so fewer query tiles per workgroup
    // leave fewer waves idle on each visited tile.
    if (p.dtype == DCA_BF16 && p.sparse && p.D == 128) return launch_attn_t<__bf16, 128, 4, 2, 1, true>(p, a, stream);
    if (p.dtype == DCA_BF16)
        return p.D == 128 ? launch_attn_t<__bf16, 128, 8, 4, 2>(p, a, stream)
                          : launch_attn_t<__bf16, 64, 8, 4, 2>(p, a, stream);
    return p.D == 128 ? launch_attn_t<float, 128, 2, 2, 1>(p, a, stream)
                      : launch_attn_t<float, 64, 4, 4, 2>(p, a, stream);
}

// Read-back of the visiting order: the key tiles that one group of NT query
// tiles, starting at query tile t0, visits for head h -- the same iterator the
// attention kernel runs -- each with the bits of the group's query tiles it is
// active for. One lane; writes at most cap entries and the full count.
template <int NT>
__global__ __launch_bounds__(64) void debug_vs_tiles_kernel(AttnArgs a, int h, int t0, int cap, int32_t *kt_out,
                                                            uint32_t *m_out, int32_t *n_out) {
    if (threadIdx.x != 0) return;
    const int S = (int)a.S;
    const int i0 = t0 * kTile;
    const int last_row = (i0 + NT * kTile < S ? i0 + NT * kTile : S) - 1;
    TileIter<NT> it;
    it.init(a, h, i0, S, last_row / kTile);
    int n = 0;
    unsigned m = 0;
    for (int kt = it.next(m); kt >= 0; kt = it.next(m), ++n) {
        if (n < cap) {
            kt_out[n] = kt;
            m_out[n] = m;
        }
    }
    *n_out = n;
}

int launch_debug_vs_tiles(const Problem &p, const void *ws, const Layout &L, int head, int64_t q_tile, int group,
                          int32_t *kt_out, uint32_t *m_out, int32_t cap, int32_t *n_out, void *stream) {
    AttnArgs a{};
    a.S = p.q0 + p.NQ;
    a.sparse = 1;
    a.vt = (const int32_t *)((const char *)ws + L.vs_vt);
    a.vt_n = (const int32_t *)((const char *)ws + L.vs_vt_n);
    a.dl = (const int32_t *)((const char *)ws + L.vs_dl);
    a.dl_n = (const int32_t *)((const char *)ws + L.vs_dl_n);
    a.list_stride = (int32_t)p.n_tiles;
    if (group == 1)
        hipLaunchKernelGGL(debug_vs_tiles_kernel<1>, dim3(1), dim3(64), 0, (hipStream_t)stream, a, head,
                           (int)q_tile, (int)cap, kt_out, m_out, n_out);
    else
        hipLaunchKernelGGL(debug_vs_tiles_kernel<2>, dim3(1), dim3(64), 0, (hipStream_t)stream, a, head,
                           (int)q_tile, (int)cap, kt_out, m_out, n_out);
    return (int)hipGetLastError();
}

}  // namespace dca
