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

__device__ inline float lane_swap32(float x) { return __shfl_xor(x, 32, 64); }

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
    constexpr int TILE_CHUNKS = TILE_ELEMS * (int)sizeof(T) / 16;
    constexpr int THREADS = NW * 64;
    constexpr int CPT = 2 * TILE_CHUNKS / THREADS;  // 16-byte chunks per thread (K then V)
    static_assert(NT >= 1 && BM % kTile == 0, "workgroup rows must cover whole 64-row tiles");
    static_assert((2 * TILE_CHUNKS) % THREADS == 0 && TILE_CHUNKS % THREADS == 0, "tile split");

    __shared__ __attribute__((aligned(16))) vec lds[NBUF][2 * TILE_ELEMS / E];

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

    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int x = lane % 32;
    const int gsel = lane / 32;
    const int64_t i0 = (int64_t)rt * BM;
    const int64_t r0 = i0 + kBlk * wave;          // this wave's first row
    const bool wave_rows = r0 < a.S;
    const int64_t cq = r0 / a.C;                  // chunk of this wave's rows
    const int64_t last_row = (i0 + BM < a.S ? i0 + BM : a.S) - 1;
    const int64_t kt_last = last_row / kTile;

    const T *kbase = (const T *)a.kf + bkv * a.nblk * BLK_ELEMS;
    const T *vbase = (const T *)a.vf + bkv * a.nblk * BLK_ELEMS;

    // ---- key-tile visit order ---------------------------------------------
    // dense: 0 .. kt_last. sparse: union over this workgroup's query tiles of
    // {kt in VT : kt <= t} and {t - delta : delta in D, delta <= t}.
    int32_t pv[NT], pd[NT], tq[NT];
    const int32_t *vt = nullptr, *dl = nullptr;
    int32_t nv = 0;
    if (a.sparse) {
        vt = a.vt + (int64_t)h * a.list_stride;
        dl = a.dl + (int64_t)h * a.list_stride;
        nv = a.vt_n[h];
        const int32_t nd = a.dl_n[h];
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            tq[q] = (int32_t)(i0 / kTile) + q;
            pv[q] = 0;
            // pd = index of the last D entry <= t (D ascending)
            int lo = 0, hi = nd;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (dl[mid] <= tq[q]) lo = mid + 1; else hi = mid;
            }
            pd[q] = lo - 1;
            if ((int64_t)tq[q] * kTile >= a.S) { pv[q] = nv; pd[q] = -1; }
        }
    }
    int64_t kt_dense = 0;
    // next active tile; *mask gets one bit per query tile of the workgroup
    auto next_tile = [&](unsigned *mask) -> int64_t {
        if (!a.sparse) {
            if (kt_dense > kt_last) return -1;
            *mask = (1u << NT) - 1;
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
        *mask = m;
        return best;
    };

    // ---- state ----------------------------------------------------------
    vec qfrag[NU];
    int cur_region = -1;
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;   // running max of raw scores (this row)
    float l_run = 0.f;         // running sum of 2^(s ks - m ks), this lane's keys only

    uint4 pre[CPT];
    auto load_tile = [&](int64_t kt) {
        const uint4 *ks_ = (const uint4 *)(kbase + kt * TILE_ELEMS);
        const uint4 *vs_ = (const uint4 *)(vbase + kt * TILE_ELEMS);
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int idx = threadIdx.x + c * THREADS;
            pre[c] = (c < CPT / 2) ? ks_[idx] : vs_[idx - TILE_CHUNKS];
        }
    };
    auto store_tile = [&](int buf) {
        uint4 *dst = (uint4 *)&lds[buf][0];
#pragma unroll
        for (int c = 0; c < CPT; ++c) dst[threadIdx.x + c * THREADS] = pre[c];
    };

    unsigned mask = 0;
    int64_t kt = next_tile(&mask);
    if (kt >= 0) load_tile(kt);
    int buf = 0;
    bool first = true;
    while (kt >= 0) {
        if (NBUF == 1 && !first) __syncthreads();
        store_tile(buf);
        __syncthreads();
        first = false;
        unsigned next_mask = 0;
        const int64_t kt_next = next_tile(&next_mask);
        if (kt_next >= 0) load_tile(kt_next);

        const int64_t j0 = kt * kTile;
        const bool active = wave_rows && j0 <= r0 + kBlk - 1 && ((mask >> (wave * kBlk / kTile)) & 1u);
        if (active) {
            const int region = region_of(cq, j0 / a.C);
            if (region != cur_region) {
                const vec *qs = (const vec *)a.qf[region] + (bh * a.nblk + r0 / kBlk) * (BLK_ELEMS / E);
#pragma unroll
                for (int u = 0; u < NU; ++u) qfrag[u] = qs[u * 64 + lane];
                cur_region = region;
            }
            const vec *kl = &lds[buf][0];
            const vec *vl = &lds[buf][TILE_ELEMS / E];

            // S^T = K_rot Q^T for the two 32-key blocks
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sacc[kb] = f32x16{};
#pragma unroll
                for (int u = 0; u < NU; ++u) F::mma(kl[(kb * NU + u) * 64 + lane], qfrag[u], sacc[kb]);
            }
            // causal mask on the diagonal tile (also masks keys >= S for rows < S)
            if (j0 + kTile - 1 > r0) {
                const int64_t row = r0 + x;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int64_t key = j0 + kBlk * kb + 8 * (v / 4) + 4 * gsel + (v % 4);
                        if (key > row) sacc[kb][v] = -INFINITY;
                    }
            }
            // online softmax
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
            mx = fmaxf(mx, lane_swap32(mx));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * a.ks);
            const float neg = -m_use * a.ks;
            float psum = 0.f;
            vec pfrag[2][NUV];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float pval = __builtin_amdgcn_exp2f(fmaf(sacc[kb][v], a.ks, neg));
                    psum += pval;
                    F::set(pfrag[kb][v / E], v % E, F::from_float(pval));
                }
            l_run = l_run * alpha + psum;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
            // O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int u = 0; u < NUV; ++u)
                        F::mma(vl[((kb * NDB + db) * NUV + u) * 64 + lane], pfrag[kb][u], oacc[db]);
        }
        kt = kt_next;
        mask = next_mask;
        if (NBUF == 2) buf ^= 1;
    }

    // ---- epilogue -----------------------------------------------------------
    const int64_t row = r0 + x;
    if (!wave_rows || row >= a.S) return;
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
        a.lse[bh * a.S + row] = l_tot > 0.f ? (m_run * a.ks + __log2f(l_tot)) * 0.69314718055994531f
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
    hipLaunchKernelGGL((dca_attention_kernel<T, D, NW, NBUF>), dim3((unsigned)grid), dim3(NW * 64), 0,
                       (hipStream_t)stream, a);
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
    return p.D == 128 ? launch_attn_t<float, 128, 4, 1>(p, a, stream)
                      : launch_attn_t<float, 64, 4, 2>(p, a, stream);
}

}  // namespace dca
