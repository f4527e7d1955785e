// Online vertical-slash estimation for gfx950 [mizuki, 稀疏注意力 + 核优化:
// key tokens are selected with continuous relative positions restored;
// 跟 NSA / 其他稀疏注意力的区别: a few key columns and diagonals draw most of
// the attention].
//
// The last n (<= 64) query rows of the sequence attend to every key with RoPE
// at the true indices i and j (not the DCA map) and the attention's logit
// scale. Per query head, a key column scores the sum of its softmax weights
// over those rows and a diagonal o = i - j the sum along it; the head keeps
// the first `forced` columns and offsets and the highest-scoring others up to
// its budgets (ties to the smaller index), as sorted lists that feed the
// vertical-slash tile index directly.
//
// Launches (after the shared pre-pass has written the keys rotated at their
// own index j and scaled by yarn * sigma * log2 e, so scores leave the matrix
// cores in base-2 exponent units):
//   est_rowstat_kernel   one wave per (split of the key tiles, head, 32-row
//                        block): S^T = K Q^T, running max and sum per row;
//                        the waves of one KV head and split run together on
//                        one XCD (est_decode) and share the key tiles in L2;
//   est_rowcombine_kernel  row max M and 1 / sum per row over the splits;
//   est_clear_kernel     zeroes the diagonal scores;
//   est_sums_kernel      one wave per (split, head): S = Q K^T for all rows,
//                        so that a lane holds one key column and the column
//                        sum is a lane reduction; the 64 x 64 weight tile goes
//                        through LDS for the diagonal sums. A diagonal gets at
//                        most two contributions (two key tiles), added
//                        atomically to zero: the result does not depend on
//                        their order;
//   est_topk_*           per (head, list), 16 workgroups each: radix select
//                        of the budget's threshold on the scores' bits (four
//                        8-bit passes; histogram adds grouped per wave and
//                        bin), then an index-ordered compaction placed by the
//                        ranges' counts (ties to the smaller index).
#include <hip/hip_runtime.h>

#include "dca_internal.h"
#include "frag.h"

namespace dca {

constexpr int64_t kEstRowstatWaves = 8192;   // targets for the two score passes
constexpr int64_t kEstSumsWaves = 4096;

struct EstArgs {
    const void *q;                   // [Hq][S][D], batch 1
    const void *kf;                  // keys at their own index, fragment order, scaled
    const float2 *table;             // cos/sin [>= S positions][D/2]
    float *rstat;                    // [Hq][64][kEstMaxSplits][2]: running max (log2), sum
    float *ml;                       // [Hq][64][2]: row max M (log2), 1 / row sum
    float *vscore, *sscore;          // [Hq][S]
    int64_t S;
    int32_t Hq, Hkv, G, nblk_kv;
    int32_t r0;                      // first scored row, S - n
    int32_t n_split, tiles_per_split, n_tiles;
    int32_t n_sets;                  // (KV head, split) pairs: the waves of a set read the same key tiles
};

// 1D grids: the waves that read the same key tiles -- one (KV head, split)
// set, `members` waves -- are consecutive workgroups of one XCD (workgroup i
// runs on XCD i mod 8), so the tiles come from HBM once per set and then
// from that XCD's L2. Returns false for the padding workgroups of the grid.
__device__ __forceinline__ bool est_decode(const EstArgs &a, int members, int &kvh, int &split, int &member) {
    const int bid = blockIdx.x;
    const int xcd = bid % kXcds, slot = bid / kXcds;
    member = slot % members;
    const int set = (slot / members) * kXcds + xcd;
    if (set >= a.n_sets) return false;
    kvh = set / a.n_split;
    split = set % a.n_split;
    return true;
}

__device__ inline float est_swap32(float x) { return __shfl_xor(x, 32, 64); }

// Query fragments of head h, scored rows [r0 + 32 rb, + 32), rotated to their
// own index; rows past the sequence are zero. The same registers serve as the
// B operand of S^T = K Q^T and the A operand of S = Q K^T.
template <typename T, int D>
__device__ __forceinline__ void est_load_q(const EstArgs &a, int h, int rb, int lane,
                                           typename Frag<T>::vec (&qf)[D / (2 * Frag<T>::E)]) {
    using F = Frag<T>;
    using vec = typename F::vec;
    constexpr int E = F::E;
    constexpr int NU = D / (2 * E);
    const int x = lane % 32, g = lane / 32;
    const int64_t row = (int64_t)a.r0 + kBlk * rb + x;
    const bool valid = row < a.S;
    const T *src = (const T *)a.q + ((int64_t)h * a.S + (valid ? row : 0)) * D + E * g;
#pragma unroll
    for (int u = 0; u < NU; ++u) qf[u] = valid ? *(const vec *)(src + 2 * E * u) : F::zero();
    const float2 *tab = a.table + (valid ? row : 0) * (D / 2) + E * g;
#pragma unroll
    for (int u = 0; u < NU / 2; ++u)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float2 cs = tab[2 * E * u + e];
            const float2 r = rope_pair((float)F::get(qf[u], e), (float)F::get(qf[u + NU / 2], e), cs.x, cs.y);
            F::set(qf[u], e, F::from_float(r.x));
            F::set(qf[u + NU / 2], e, F::from_float(r.y));
        }
}

// ---------------------------------------------------------------------------
// row statistics: grid (n_split, Hq * 2) waves
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void est_rowstat_kernel(EstArgs a) {
    using F = Frag<T>;
    using vec = typename F::vec;
    constexpr int NU = D / (2 * F::E);
    constexpr int BLK_ELEMS = kBlk * D;
    constexpr int TILE_BYTES = 2 * BLK_ELEMS * (int)sizeof(T);
    int kvh, split, member;
    if (!est_decode(a, 2 * a.G, kvh, split, member)) return;
    const int h = kvh * a.G + member / 2, rb = member % 2;
    const int lane = threadIdx.x, x = lane % 32, g = lane / 32;
    const int64_t row = (int64_t)a.r0 + kBlk * rb + x;
    const int64_t row_lo = (int64_t)a.r0 + kBlk * rb;          // the wave's first row
    const bool rows_in = row_lo + kBlk - 1 < a.S;               // all 32 rows inside the sequence
    vec qf[NU];
    est_load_q<T, D>(a, h, rb, lane, qf);
    const char *kbase = (const char *)a.kf + (int64_t)kvh * a.nblk_kv * BLK_ELEMS * (int64_t)sizeof(T);
    const int kt0 = split * a.tiles_per_split;
    const int kt1 = min(kt0 + a.tiles_per_split, a.n_tiles);
    float m_run = -INFINITY, l_run = 0.f;
    // the next tile's key fragments load while the current tile is scored
    auto load_tile = [&](int kt, vec (&dst)[2 * NU]) __attribute__((always_inline)) {
        const vec *k = (const vec *)(kbase + (int64_t)kt * TILE_BYTES);
#pragma unroll
        for (int i = 0; i < 2 * NU; ++i) dst[i] = k[i * 64 + lane];
    };
    auto score_tile = [&](int kt, const vec (&kf)[2 * NU]) __attribute__((always_inline)) {
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) F::mma(kf[kb * NU + u], qf[u], s[kb]);
        // S^T: value v of block kb is key j0 + 32 kb + 8 (v / 4) + 4 g + v % 4 of row `row`
        const int64_t j0 = (int64_t)kt * kTile;
        float mx = -INFINITY;
        if (j0 + kTile - 1 <= row_lo && rows_in) {      // every key visible to every row: no mask
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t j = j0 + kBlk * kb + 8 * (v / 4) + 4 * g + (v % 4);
                    if (j > row || row >= a.S) s[kb][v] = -INFINITY;
                    mx = fmaxf(mx, s[kb][v]);
                }
        }
        mx = fmaxf(mx, est_swap32(mx));
        if (mx == -INFINITY) return;                   // no key of this tile is visible to the row
        const float m_new = fmaxf(m_run, mx);
        float sum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) sum += __builtin_amdgcn_exp2f(s[kb][v] - m_new);
        l_run = l_run * __builtin_amdgcn_exp2f(m_run - m_new) + sum;
        m_run = m_new;
    };
    vec ka[2 * NU], kn[2 * NU];
    if (kt0 < kt1) load_tile(kt0, ka);
    for (int kt = kt0; kt < kt1; kt += 2) {
        if (kt + 1 < kt1) load_tile(kt + 1, kn);
        score_tile(kt, ka);
        if (kt + 1 >= kt1) break;
        if (kt + 2 < kt1) load_tile(kt + 2, ka);
        score_tile(kt + 1, kn);
    }
    const float l_tot = l_run + est_swap32(l_run);
    if (g == 0) {
        float *dst = a.rstat + (((int64_t)h * kEstRows + kBlk * rb + x) * kEstMaxSplits + split) * 2;
        dst[0] = m_run;
        dst[1] = l_tot;
    }
}

// grid Hq blocks of 64 threads (one per scored row)
__global__ __launch_bounds__(64) void est_rowcombine_kernel(EstArgs a) {
    const int h = blockIdx.x, r = threadIdx.x;
    const float *src = a.rstat + ((int64_t)h * kEstRows + r) * kEstMaxSplits * 2;
    float M = -INFINITY;
    for (int s = 0; s < a.n_split; ++s)
        if (src[2 * s + 1] > 0.f) M = fmaxf(M, src[2 * s]);
    float L = 0.f;
    for (int s = 0; s < a.n_split; ++s)
        if (src[2 * s + 1] > 0.f) L += src[2 * s + 1] * __builtin_amdgcn_exp2f(src[2 * s] - M);
    float *dst = a.ml + ((int64_t)h * kEstRows + r) * 2;
    dst[0] = L > 0.f ? M : 0.f;
    dst[1] = L > 0.f ? 1.f / L : 0.f;                  // rows past the sequence weigh nothing
}

__global__ void est_clear_kernel(float *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// ---------------------------------------------------------------------------
// column and diagonal sums: grid (n_split, Hq) waves
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void est_sums_kernel(EstArgs a) {
    using F = Frag<T>;
    using vec = typename F::vec;
    constexpr int NU = D / (2 * F::E);
    constexpr int BLK_ELEMS = kBlk * D;
    constexpr int TILE_BYTES = 2 * BLK_ELEMS * (int)sizeof(T);
    constexpr int LD = kTile + 1;                      // padded LDS row
    __shared__ float P[kEstRows * LD];                 // weights: [row - r0][key - j0]
    int kvh, split, member;
    if (!est_decode(a, a.G, kvh, split, member)) return;
    const int h = kvh * a.G + member;
    const int lane = threadIdx.x, x = lane % 32, g = lane / 32;
    vec qf[2][NU];
    est_load_q<T, D>(a, h, 0, lane, qf[0]);
    est_load_q<T, D>(a, h, 1, lane, qf[1]);
    // S = Q K^T: value v of row block rb is row 32 rb + 8 (v / 4) + 4 g + v % 4
    float rm[2][16], ril[2][16];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float *ml = a.ml + ((int64_t)h * kEstRows + kBlk * rb + 8 * (v / 4) + 4 * g + (v % 4)) * 2;
            rm[rb][v] = ml[0];
            ril[rb][v] = ml[1];
        }
    const char *kbase = (const char *)a.kf + (int64_t)kvh * a.nblk_kv * BLK_ELEMS * (int64_t)sizeof(T);
    const int kt0 = split * a.tiles_per_split;
    const int kt1 = min(kt0 + a.tiles_per_split, a.n_tiles);
    float *vs = a.vscore + (int64_t)h * a.S;
    float *ss = a.sscore + (int64_t)h * a.S;
    // one 32-key half of key fragments is always in flight: the second half
    // of the tile while the first is summed, the next tile's first half
    // while the second is
    auto load_half = [&](int kt, int kb, vec (&dst)[NU]) __attribute__((always_inline)) {
        const vec *k = (const vec *)(kbase + (int64_t)kt * TILE_BYTES);
#pragma unroll
        for (int u = 0; u < NU; ++u) dst[u] = k[(kb * NU + u) * 64 + lane];
    };
    auto sum_half = [&](int64_t j0, int kb, const vec (&kfr)[NU]) __attribute__((always_inline)) {
        const int64_t j = j0 + kBlk * kb + x;          // this lane's key
        float col = 0.f;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            f32x16 acc = {};
#pragma unroll
            for (int u = 0; u < NU; ++u) F::mma(qf[rb][u], kfr[u], acc);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int rl = kBlk * rb + 8 * (v / 4) + 4 * g + (v % 4);
                const int64_t row = (int64_t)a.r0 + rl;
                const float p = j <= row ? __builtin_amdgcn_exp2f(acc[v] - rm[rb][v]) * ril[rb][v] : 0.f;
                col += p;
                P[rl * LD + kBlk * kb + x] = p;
            }
        }
        col += est_swap32(col);
        if (g == 0 && j < a.S) vs[j] = col;
    };
    vec k0[NU], k1[NU];
    if (kt0 < kt1) load_half(kt0, 0, k0);
    for (int kt = kt0; kt < kt1; ++kt) {
        const int64_t j0 = (int64_t)kt * kTile;
        load_half(kt, 1, k1);
        sum_half(j0, 0, k0);
        if (kt + 1 < kt1) load_half(kt + 1, 0, k0);
        sum_half(j0, 1, k1);
        __syncthreads();
        // diagonal sums of the tile (a = row - r0, b = key - j0): lane t reads
        // P[r][(r - t) mod 64] for every r, which is diagonal a - b = t for
        // r >= t and a - b = t - 64 for r < t; the diagonal offset of a - b = d
        // is (r0 - j0) + d
        const int t = lane;
        float dp = 0.f, dm = 0.f;
#pragma unroll
        for (int r = 0; r < kEstRows; ++r) {
            const float w = P[r * LD + ((r - t) & (kTile - 1))];
            if (r >= t) dp += w; else dm += w;
        }
        const int64_t base = (int64_t)a.r0 - j0;
        if (base + t >= 0 && base + t < a.S && dp != 0.f) atomicAdd(&ss[base + t], dp);
        const int64_t om = base + t - kTile;
        if (t > 0 && om >= 0 && om < a.S && dm != 0.f) atomicAdd(&ss[om], dm);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// top-k with forced head. Per (head, list) the candidates [f, n) are cut into
// kTopkParts ranges, one workgroup each:
//   est_topk_init    forced head, the take-everything cases, selection state
//   est_topk_hist    per pass: the range's histogram of the next 8 bits of the
//                    scores matching the prefix so far, added to the list's
//                    global histogram
//   est_topk_select  per pass: picks the bin holding the budget's edge, extends
//                    the prefix, clears the histogram
//   est_topk_count   per range: scores above the final prefix and equal to it
//   est_topk_write   per range: its picks in index order, at the offset the
//                    earlier ranges' counts give; ties go to the smaller index
// ---------------------------------------------------------------------------
constexpr int kTopkBlock = 256;         // threads per workgroup
constexpr int kTopkPer = 8;             // elements per thread and step
constexpr int kTopkStep = kTopkBlock * kTopkPer;

// inclusive prefix sum of one value per thread over the block; returns it and
// the block total in *total
template <int NT>
__device__ int block_scan(int val, int *total, int *wsum) {
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    constexpr int NWAVES = NT / 64;
    int x = val;
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int w = lane < NWAVES ? wsum[lane] : 0;
#pragma unroll
        for (int d = 1; d < NWAVES; d *= 2) {
            const int y = __shfl_up(w, d, 64);
            if (lane >= d) w += y;
        }
        if (lane < NWAVES) wsum[lane] = w;
    }
    __syncthreads();
    const int res = x + (wave > 0 ? wsum[wave - 1] : 0);
    *total = wsum[NWAVES - 1];
    __syncthreads();
    return res;
}

struct TopkArgs {
    const float *score[2];          // vertical, slash scores [Hq][S]
    int32_t *out[2];                // [Hq][budget]
    int32_t budget[2];
    int32_t forced;
    int64_t S;
    unsigned *hist;                 // [Hq][2][256] histogram of the current pass
    unsigned *state;                // [Hq][2][4]: prefix, prefix mask, equal bits still to take, active
    int32_t *counts;                // [Hq][2][kTopkParts][2]: above, equal
};

// hist[bin] += 1 for the valid lanes. The scores crowd into a few bins, so
// the lanes of a wave that share a bin add once, with their count (up to four
// distinct bins per call; the remaining lanes add one by one).
__device__ __forceinline__ void hist_add(unsigned *hist, unsigned bin, bool valid) {
    const int lane = threadIdx.x % 64;
    uint64_t pending = __builtin_amdgcn_ballot_w64(valid);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        if (pending == 0) break;
        const int leader = __builtin_ctzll(pending);
        const unsigned lb = (unsigned)__builtin_amdgcn_readlane((int)bin, leader);
        const uint64_t same = __builtin_amdgcn_ballot_w64(valid && bin == lb) & pending;
        if (lane == leader) atomicAdd(&hist[lb], (unsigned)__builtin_popcountll(same));
        pending &= ~same;
    }
    if ((pending >> lane) & 1ull) atomicAdd(&hist[bin], 1u);
}

// the list of (head, list) workgroup index `lid`, and this workgroup's range
struct TopkList {
    const unsigned *bits;           // scores >= 0: bit order = value order
    int32_t *out;
    int64_t n, f, k;                // candidates [f, n), k of them to pick
    int64_t lo, hi;                 // this workgroup's range of candidates
    unsigned *st;
};
__device__ __forceinline__ TopkList topk_list(const TopkArgs &a, int lid, int part) {
    TopkList L;
    const int h = lid / 2, list = lid % 2;
    L.n = a.S;
    const int budget = a.budget[list];
    L.bits = (const unsigned *)(a.score[list] + (int64_t)h * L.n);
    L.out = a.out[list] + (int64_t)h * budget;
    L.f = min((int64_t)min(a.forced, budget), L.n);
    L.k = budget - L.f;
    const int64_t len = (L.n - L.f + kTopkParts - 1) / kTopkParts;
    L.lo = min(L.n, L.f + part * len);
    L.hi = min(L.n, L.lo + len);
    L.st = a.state + lid * 4;
    return L;
}

// grid (Hq * 2) blocks of kTopkBlock threads
__global__ __launch_bounds__(kTopkBlock) void est_topk_init(TopkArgs a) {
    const int lid = blockIdx.x, tid = threadIdx.x;
    const TopkList L = topk_list(a, lid, 0);
    for (int64_t i = tid; i < L.f; i += kTopkBlock) L.out[i] = (int32_t)i;
    a.hist[lid * 256 + tid] = 0u;                       // kTopkBlock == 256 bins
    bool active = L.k > 0;
    if (active && L.n - L.f <= L.k) {                   // every candidate
        for (int64_t i = L.f + tid; i < L.n; i += kTopkBlock) L.out[i] = (int32_t)i;
        active = false;
    }
    if (tid == 0) {
        L.st[0] = 0u;
        L.st[1] = 0u;
        L.st[2] = L.k > 0 ? (unsigned)L.k : 0u;
        L.st[3] = active ? 1u : 0u;
    }
}

// grid (kTopkParts, Hq * 2)
__global__ __launch_bounds__(kTopkBlock) void est_topk_hist(TopkArgs a, int shift) {
    __shared__ unsigned lh[256];
    const int lid = blockIdx.y, tid = threadIdx.x;
    const TopkList L = topk_list(a, lid, blockIdx.x);
    if (L.st[3] == 0u) return;
    const unsigned prefix = L.st[0], pmask = L.st[1];
    lh[tid] = 0u;
    __syncthreads();
    for (int64_t b0 = L.lo; b0 < L.hi; b0 += kTopkStep) {
        unsigned v[kTopkPer];
#pragma unroll
        for (int e = 0; e < kTopkPer; ++e) {
            const int64_t i = b0 + (int64_t)e * kTopkBlock + tid;
            v[e] = i < L.hi ? L.bits[i] : 0u;
        }
#pragma unroll
        for (int e = 0; e < kTopkPer; ++e) {
            const int64_t i = b0 + (int64_t)e * kTopkBlock + tid;
            hist_add(lh, (v[e] >> shift) & 255u, i < L.hi && (v[e] & pmask) == prefix);
        }
    }
    __syncthreads();
    if (lh[tid] != 0u) atomicAdd(&a.hist[lid * 256 + tid], lh[tid]);
}

// grid (Hq * 2)
__global__ __launch_bounds__(kTopkBlock) void est_topk_select(TopkArgs a, int shift) {
    __shared__ unsigned gh[256];
    const int lid = blockIdx.x, tid = threadIdx.x;
    unsigned *st = a.state + lid * 4;
    if (st[3] == 0u) return;
    gh[tid] = a.hist[lid * 256 + tid];
    __syncthreads();
    if (tid == 0) {
        const unsigned remaining = st[2];
        unsigned above = 0;
        int bin = 255;
        for (; bin > 0; --bin) {
            if (above + gh[bin] >= remaining) break;
            above += gh[bin];
        }
        st[0] |= (unsigned)bin << shift;
        st[1] |= 255u << shift;
        st[2] = remaining - above;
    }
    a.hist[lid * 256 + tid] = 0u;                       // for the next pass
}

// grid (kTopkParts, Hq * 2)
__global__ __launch_bounds__(kTopkBlock) void est_topk_count(TopkArgs a) {
    __shared__ int wsum[kTopkBlock / 64];
    const int lid = blockIdx.y, part = blockIdx.x, tid = threadIdx.x;
    const TopkList L = topk_list(a, lid, part);
    if (L.st[3] == 0u) return;
    const unsigned prefix = L.st[0];
    int gt = 0, eq = 0;
    for (int64_t i = L.lo + tid; i < L.hi; i += kTopkBlock) {
        const unsigned b = L.bits[i];
        gt += b > prefix;
        eq += b == prefix;
    }
    int tg, te;
    block_scan<kTopkBlock>(gt, &tg, wsum);
    block_scan<kTopkBlock>(eq, &te, wsum);
    if (tid == 0) {
        a.counts[(lid * kTopkParts + part) * 2] = tg;
        a.counts[(lid * kTopkParts + part) * 2 + 1] = te;
    }
}

// grid (kTopkParts, Hq * 2)
__global__ __launch_bounds__(kTopkBlock) void est_topk_write(TopkArgs a) {
    __shared__ int wsum[kTopkBlock / 64];
    __shared__ unsigned stage[kTopkStep];
    const int lid = blockIdx.y, part = blockIdx.x, tid = threadIdx.x;
    const TopkList L = topk_list(a, lid, part);
    if (L.st[3] == 0u) return;
    const unsigned prefix = L.st[0];
    const int R = (int)L.st[2];                        // equal bits to take, smallest indices first
    int gt_before = 0, eq_before = 0;                  // in the earlier ranges
    for (int b = 0; b < part; ++b) {
        gt_before += a.counts[(lid * kTopkParts + b) * 2];
        eq_before += a.counts[(lid * kTopkParts + b) * 2 + 1];
    }
    int64_t pos = L.f + gt_before + min(eq_before, R);
    int ties = eq_before;                              // equal bits seen before this step
    // per step, thread t owns the kTopkPer consecutive indices b0 + 8t ..; one
    // scan of its packed (above, equal) counts places all of its picks
    for (int64_t b0 = L.lo; b0 < L.hi; b0 += kTopkStep) {
#pragma unroll
        for (int e = 0; e < kTopkPer; ++e) {
            const int64_t i = b0 + (int64_t)e * kTopkBlock + tid;
            stage[e * kTopkBlock + tid] = i < L.hi ? L.bits[i] : 0u;
        }
        __syncthreads();
        unsigned w[kTopkPer];
        int gt = 0, eq = 0;
#pragma unroll
        for (int e = 0; e < kTopkPer; ++e) {
            w[e] = stage[kTopkPer * tid + e];
            const bool valid = b0 + kTopkPer * tid + e < L.hi;
            gt += valid && w[e] > prefix;
            eq += valid && w[e] == prefix;
        }
        const int packed = gt | (eq << 16);            // both < 2^16: no carry between the halves
        int total;
        const int excl = block_scan<kTopkBlock>(packed, &total, wsum) - packed;
        const int r_left = max(R - ties, 0);           // equal bits still to take
        int eq_seen = excl >> 16;
        int64_t o = pos + (excl & 0xffff) + min(eq_seen, r_left);
#pragma unroll
        for (int e = 0; e < kTopkPer; ++e) {
            const int64_t i = b0 + kTopkPer * tid + e;
            if (i >= L.hi) break;
            bool take = w[e] > prefix;
            if (w[e] == prefix) {
                take = eq_seen < r_left;
                ++eq_seen;
            }
            if (take) L.out[o++] = (int32_t)i;
        }
        const int tot_gt = total & 0xffff, tot_eq = total >> 16;
        pos += tot_gt + min(tot_eq, r_left);
        ties += tot_eq;
        __syncthreads();                               // stage is rewritten next step
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <typename T, int D>
static int launch_est_t(const Problem &p, int n_last, const void *q, const void *ws, const Layout &L,
                        size_t scratch, float *vscore, float *sscore, void *stream) {
    EstArgs a{};
    a.q = q;
    a.kf = (const char *)ws + L.k;
    a.table = (const float2 *)((const char *)ws + L.table);
    a.rstat = (float *)((char *)ws + scratch);
    a.ml = a.rstat + (size_t)p.Hq * kEstRows * kEstMaxSplits * 2;
    a.vscore = vscore;
    a.sscore = sscore;
    a.S = p.S;
    a.Hq = (int32_t)p.Hq;
    a.Hkv = (int32_t)p.Hkv;
    a.G = (int32_t)p.G;
    a.nblk_kv = (int32_t)(p.S_pad / kBlk);
    a.r0 = (int32_t)(p.S - n_last);
    a.n_tiles = (int32_t)((p.S + kTile - 1) / kTile);
    auto set_splits = [&](EstArgs &e, int64_t waves_target, int members_per_set) {
        int64_t want = waves_target / (p.Hkv * members_per_set);
        want = want < 1 ? 1 : want;
        want = want < kEstMaxSplits ? want : kEstMaxSplits;
        want = want < e.n_tiles ? want : e.n_tiles;
        e.tiles_per_split = (int32_t)((e.n_tiles + want - 1) / want);
        e.n_split = (e.n_tiles + e.tiles_per_split - 1) / e.tiles_per_split;
        e.n_sets = (int32_t)(p.Hkv * e.n_split);
    };
    // many more waves than fit at once, so that no pass ends with a thinly
    // occupied last batch of workgroups
    EstArgs ar = a;
    set_splits(ar, kEstRowstatWaves, 2 * (int)p.G);
    set_splits(a, kEstSumsWaves, (int)p.G);
    hipStream_t s = (hipStream_t)stream;
    const int64_t rows_r = (ar.n_sets + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((est_rowstat_kernel<T, D>), dim3((unsigned)(rows_r * 2 * p.G)), dim3(64), 0, s, ar);
    int err = (int)hipGetLastError();
    if (err) return err;
    const int64_t set_rows = (a.n_sets + kXcds - 1) / kXcds * kXcds;
    a.n_split = ar.n_split;      // the row combine reads the row-statistics splits
    hipLaunchKernelGGL(est_rowcombine_kernel, dim3((unsigned)p.Hq), dim3(kEstRows), 0, s, a);
    if ((err = (int)hipGetLastError())) return err;
    const int64_t n = p.Hq * p.S;
    hipLaunchKernelGGL(est_clear_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, sscore, n);
    if ((err = (int)hipGetLastError())) return err;
    {
        EstArgs as = a;
        set_splits(as, kEstSumsWaves, (int)p.G);
        hipLaunchKernelGGL((est_sums_kernel<T, D>), dim3((unsigned)(set_rows * p.G)), dim3(64), 0, s, as);
    }
    return (int)hipGetLastError();
}

int launch_vs_estimate(const Problem &p, int n_last, int n_vertical, int n_slash, int n_forced, const void *q,
                       const void *ws, const Layout &L, size_t scratch, float *vscore, float *sscore,
                       int32_t *vertical, int32_t *slash, void *stream) {
    int err;
    if (p.dtype == DCA_BF16)
        err = p.D == 128 ? launch_est_t<__bf16, 128>(p, n_last, q, ws, L, scratch, vscore, sscore, stream)
                         : launch_est_t<__bf16, 64>(p, n_last, q, ws, L, scratch, vscore, sscore, stream);
    else
        err = p.D == 128 ? launch_est_t<float, 128>(p, n_last, q, ws, L, scratch, vscore, sscore, stream)
                         : launch_est_t<float, 64>(p, n_last, q, ws, L, scratch, vscore, sscore, stream);
    if (err) return err;
    TopkArgs t{};
    t.score[0] = vscore;
    t.score[1] = sscore;
    t.out[0] = vertical;
    t.out[1] = slash;
    t.budget[0] = n_vertical;
    t.budget[1] = n_slash;
    t.forced = n_forced;
    t.S = p.S;
    char *sel = (char *)ws + scratch + est_rows_bytes(p);
    t.hist = (unsigned *)sel;
    t.state = t.hist + (size_t)p.Hq * 2 * 256;
    t.counts = (int32_t *)(t.state + (size_t)p.Hq * 2 * 4);
    hipStream_t s = (hipStream_t)stream;
    const unsigned lists = (unsigned)(p.Hq * 2);
    hipLaunchKernelGGL(est_topk_init, dim3(lists), dim3(kTopkBlock), 0, s, t);
    if ((err = (int)hipGetLastError())) return err;
    for (int shift = 24; shift >= 0; shift -= 8) {
        hipLaunchKernelGGL(est_topk_hist, dim3(kTopkParts, lists), dim3(kTopkBlock), 0, s, t, shift);
        if ((err = (int)hipGetLastError())) return err;
        hipLaunchKernelGGL(est_topk_select, dim3(lists), dim3(kTopkBlock), 0, s, t, shift);
        if ((err = (int)hipGetLastError())) return err;
    }
    hipLaunchKernelGGL(est_topk_count, dim3(kTopkParts, lists), dim3(kTopkBlock), 0, s, t);
    if ((err = (int)hipGetLastError())) return err;
    hipLaunchKernelGGL(est_topk_write, dim3(kTopkParts, lists), dim3(kTopkBlock), 0, s, t);
    return (int)hipGetLastError();
}

}  // namespace dca
