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
    int32_t pv[NT], pd[NT], tq[NT];
    const int32_t *vt, *dl;
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
        vt = a.vt + (int64_t)h * a.list_stride;
        dl = a.dl + (int64_t)h * a.list_stride;
        nv = a.vt_n[h];
        const int32_t nd = a.dl_n[h];
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
    float ks;
    int64_t qbase;               // element offset of this wave's 32-row block in a Q variant
    const char *kbytes, *vbytes; // this KV head's fragment-ordered K and V
};

// K and V of key tile kt -> one LDS buffer, straight from global memory: each
// wave moves its share of contiguous 1 KB pieces (16 bytes per lane, written to
// LDS at M0 + 16 * lane). Issued as inline asm so that the compiler does not
// make every later LDS read wait for these loads: the loop waits for them
// explicitly (s_waitcnt vmcnt(0) + barrier) before any wave reads the buffer.
// The asm has no register outputs; M0 is set inside the block with the one
// wait state an SALU write of M0 needs before an LDS DMA reads it.
template <typename T, int D, int NW>
__device__ __forceinline__ void issue_tile_dma(const WaveCtx &c, int kt, uint32_t dst) {
    constexpr int TILE_BYTES = 2 * kBlk * D * (int)sizeof(T);
    constexpr int WAVE_CHUNKS = 2 * TILE_BYTES / 1024 / NW;
#pragma unroll
    for (int i = 0; i < WAVE_CHUNKS; ++i) {
        const int chunk = c.wave * WAVE_CHUNKS + i;
        const bool is_v = chunk * 1024 >= TILE_BYTES;
        const int off = chunk * 1024 - (is_v ? TILE_BYTES : 0);
        const char *src = (is_v ? c.vbytes : c.kbytes) + (int64_t)kt * TILE_BYTES + off + c.lane * 16;
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

// One key tile for one wave: start the next tile's loads into the LDS buffer
// at byte address `next`, then scores, online softmax and PV on the tile in
// `cur`.
template <typename T, int D, int NW>
__device__ __forceinline__ void tile_step(const AttnArgs &a, const WaveCtx &c, const char *__restrict__ cur,
                                          uint32_t next, int kt, unsigned mask, int kt_next,
                                          typename Frag<T>::vec (&qfrag)[D / (2 * Frag<T>::E)],
                                          int &cur_region, f32x16 (&oacc)[D / 32], float &m_run,
                                          float &l_run) {
    using F = Frag<T>;
    using vec = typename F::vec;
    constexpr int E = F::E;
    constexpr int NU = D / (2 * E);
    constexpr int NDB = D / 32;
    constexpr int NUV = kBlk / (2 * E);
    constexpr int TILE_BYTES = 2 * kBlk * D * (int)sizeof(T);

    const int j0 = kt * kTile;
    const bool active = c.active_rows && j0 <= c.r0 + kBlk - 1 && ((mask >> c.wave_qt) & 1u);
    // query fragments of a new region are fetched before the next tile's
    // loads, so waiting for them does not wait for the tile (loads retire in order)
    const int region = kt < c.tb_succ ? 2 : (kt < c.tb_intra ? 1 : 0);
    if (active && region != cur_region) {
        const vec *qs = (const vec *)a.qf[region] + c.qbase / E;
#pragma unroll
        for (int u = 0; u < NU; ++u) qfrag[u] = qs[u * 64 + c.lane];
        cur_region = region;
        // land them here (twice per row block at most): no compiler-counted
        // load is then outstanding while the tile loads below are in flight
        __builtin_amdgcn_s_waitcnt(0);
    }
    if (kt_next >= 0) issue_tile_dma<T, D, NW>(c, kt_next, next);
    if (!active) return;
    const vec *kl = (const vec *)cur;
    const vec *vl = (const vec *)(cur + TILE_BYTES);

    // S^T = K_rot Q^T for the two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
#pragma unroll
        for (int u = 0; u < NU; ++u) F::mma(kl[(kb * NU + u) * 64 + c.lane], qfrag[u], sacc[kb]);
    }
    // causal mask on the diagonal tile (also masks keys >= S for rows < S)
    if (j0 + kTile - 1 > c.r0) {
        const int lim = c.r0 + c.x - j0 - 4 * c.gsel;     // key offset k is kept iff k <= lim
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if (kBlk * kb + 8 * (v / 4) + (v % 4) > lim) sacc[kb][v] = -INFINITY;
    }
    // online softmax with a lazily raised reference max
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    mx = fmaxf(mx, lane_swap32(mx));
    const bool raise = (mx - m_run) * c.ks > kLazyRescale;   // true while m_run = -inf
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * c.ks);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        m_run = m_new;
    }
    const float neg = m_run == -INFINITY ? 0.f : -m_run * c.ks;
    vec pfrag[2][NUV];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            F::set(pfrag[kb][v / E], v % E, F::from_float(__builtin_amdgcn_exp2f(fmaf(sacc[kb][v], c.ks, neg))));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < NUV; ++u) l_run = F::sum_into(pfrag[kb][u], l_run);
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < NUV; ++u)
                F::mma(vl[((kb * NDB + db) * NUV + u) * 64 + c.lane], pfrag[kb][u], oacc[db]);
}

template <typename T, int D, int NW, int NBUF>
__global__ __launch_bounds__(NW * 64, 2) void dca_attention_kernel(AttnArgs a) {
    using F = Frag<T>;
    using vec = typename F::vec;
    constexpr int E = F::E;
    constexpr int NU = D / (2 * E);            // QK fragments per 32-key block
    constexpr int NDB = D / 32;                // output d-blocks
    constexpr int NUV = kBlk / (2 * E);        // PV fragments per (32-key block, d-block)
    constexpr int BM = kBlk * NW;              // rows per workgroup
    constexpr int NT = BM / kTile;             // 64-row query tiles per workgroup
    constexpr int BLK_ELEMS = kBlk * D;
    constexpr int TILE_ELEMS = 2 * BLK_ELEMS;  // one 64-key tile of K (or V)
    constexpr int TILE_BYTES = TILE_ELEMS * (int)sizeof(T);
    constexpr int WAVE_CHUNKS = 2 * TILE_BYTES / 1024 / NW;   // 1 KB wave loads per wave per tile
    static_assert(NT >= 1 && BM % kTile == 0, "workgroup rows must cover whole 64-row tiles");
    static_assert((2 * TILE_BYTES) % (1024 * NW) == 0, "tile split");
    static_assert(NBUF == 2, "double-buffered LDS");

    extern __shared__ __attribute__((aligned(1024))) char lds_dyn[];
    char *lds = lds_dyn;             // NBUF buffers of [K tile | V tile]

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
    const int x = lane % 32;
    const int gsel = lane / 32;
    const int S = (int)a.S;
    const int i0 = rt * BM;
    const int r0 = i0 + kBlk * wave;               // this wave's first row
    const bool wave_rows = r0 < S;
    const int last_row = (i0 + BM < S ? i0 + BM : S) - 1;
    const int kt_last = last_row / kTile;
    // key-tile boundaries of this wave's regions: tiles [0, tb_succ) are
    // inter-chunk, [tb_succ, tb_intra) successive, [tb_intra, ...) intra
    const int tiles_per_chunk = (int)(a.C / kTile);
    const int cq = r0 / (int)a.C;
    const int tb_intra = cq * tiles_per_chunk;
    const int tb_succ = cq >= 1 ? tb_intra - tiles_per_chunk : 0;
    const int wave_qt = (kBlk * wave) / kTile;     // this wave's query tile in the workgroup

    const char *kbytes = (const char *)a.kf + bkv * a.nblk * (int64_t)BLK_ELEMS * (int64_t)sizeof(T);
    const char *vbytes = (const char *)a.vf + bkv * a.nblk * (int64_t)BLK_ELEMS * (int64_t)sizeof(T);

    // ---- key-tile visit order ---------------------------------------------
    TileIter<NT> it;
    it.init(a, h, i0, S, kt_last);
    unsigned mask = 0, next_mask = 0;

    // ---- state ----------------------------------------------------------
    vec qfrag[NU];
    int cur_region = -1;
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;   // reference max of raw scores (this row)
    float l_run = 0.f;         // sum of 2^(s ks - m_run ks) over this lane's keys

    WaveCtx c;
    c.lane = lane;
    c.x = x;
    c.gsel = gsel;
    c.wave = wave;
    c.r0 = r0;
    c.tb_succ = tb_succ;
    c.tb_intra = tb_intra;
    c.active_rows = wave_rows;
    c.wave_qt = wave_qt;
    c.ks = a.ks;
    c.qbase = (bh * a.nblk + r0 / kBlk) * (int64_t)BLK_ELEMS;
    c.kbytes = kbytes;
    c.vbytes = vbytes;

    int kt = it.next(mask);
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void *)lds;
    if (kt >= 0) issue_tile_dma<T, D, NW>(c, kt, lds_base);
    int buf = 0;
    while (kt >= 0) {
        __builtin_amdgcn_s_waitcnt(0);      // this wave's tile loads have landed
        __syncthreads();                    // ... and every wave's; buf^1 is free
        const int kt_next = it.next(next_mask);
        tile_step<T, D, NW>(a, c, (const char *)(lds + buf * 2 * TILE_BYTES),
                            lds_base + (buf ^ 1) * 2 * TILE_BYTES, kt, mask, kt_next, qfrag,
                            cur_region, oacc, m_run, l_run);
        kt = kt_next;
        mask = next_mask;
        buf ^= 1;
    }

    // ---- epilogue -----------------------------------------------------------
    const int row = r0 + x;
    if (!wave_rows || row >= S) return;
    const float l_tot = l_run + lane_swap32(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T *orow = (T *)a.out + (bh * a.S + row) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
            const int d0 = 32 * db + 8 * vq + 4 * gsel;
#pragma unroll
            for (int e = 0; e < 4; ++e) orow[d0 + e] = F::from_float(oacc[db][4 * vq + e] * inv);
        }
    if (a.lse != nullptr && gsel == 0) {
        a.lse[bh * a.S + row] = l_tot > 0.f ? (m_run * a.ks + log2f(l_tot)) * 0.69314718055994531f
                                            : -INFINITY;
    }
}

template <typename T, int D, int NW, int NBUF>
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
    const int lds_bytes = NBUF * 2 * (2 * kBlk * D * (int)sizeof(T));
    auto kern = dca_attention_kernel<T, D, NW, NBUF>;
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
        return p.D == 128 ? launch_attn_t<__bf16, 128, 4, 2>(p, a, stream)
                          : launch_attn_t<__bf16, 64, 4, 2>(p, a, stream);
    return p.D == 128 ? launch_attn_t<float, 128, 2, 2>(p, a, stream)
                      : launch_attn_t<float, 64, 4, 2>(p, a, stream);
}

}  // namespace dca
