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
//   est_rowcombine_kernel  row max M and 1 / sum per row over the splits;
//   est_clear_kernel     zeroes the diagonal scores;
//   est_sums_kernel      one wave per (split, head): S = Q K^T for all rows,
//                        so that a lane holds one key column and the column
//                        sum is a lane reduction; the 64 x 64 weight tile goes
//                        through LDS for the diagonal sums. A diagonal gets at
//                        most two contributions (two key tiles), added
//                        atomically to zero: the result does not depend on
//                        their order;
//   est_topk_kernel      per (head, list): radix select of the budget's
//                        threshold on the scores' bits, then an index-ordered
//                        compaction (ties to the smaller index).
#include <hip/hip_runtime.h>

#include "dca_internal.h"
#include "frag.h"

namespace dca {

constexpr int kEstRows = 64;          // query rows scored: the last n <= 64
constexpr int kEstMaxSplits = 256;

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
};

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
    const int split = blockIdx.x;
    const int h = blockIdx.y / 2, rb = blockIdx.y % 2;
    const int lane = threadIdx.x, x = lane % 32, g = lane / 32;
    const int64_t row = (int64_t)a.r0 + kBlk * rb + x;
    const int kvh = h / a.G;
    vec qf[NU];
    est_load_q<T, D>(a, h, rb, lane, qf);
    const char *kbase = (const char *)a.kf + (int64_t)kvh * a.nblk_kv * BLK_ELEMS * (int64_t)sizeof(T);
    const int kt0 = split * a.tiles_per_split;
    const int kt1 = min(kt0 + a.tiles_per_split, a.n_tiles);
    float m_run = -INFINITY, l_run = 0.f;
    for (int kt = kt0; kt < kt1; ++kt) {
        const vec *k = (const vec *)(kbase + (int64_t)kt * TILE_BYTES);
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) F::mma(k[(kb * NU + u) * 64 + lane], qf[u], s[kb]);
        // S^T: value v of block kb is key j0 + 32 kb + 8 (v / 4) + 4 g + v % 4 of row `row`
        const int64_t j0 = (int64_t)kt * kTile;
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t j = j0 + kBlk * kb + 8 * (v / 4) + 4 * g + (v % 4);
                if (j > row || row >= a.S) s[kb][v] = -INFINITY;
                mx = fmaxf(mx, s[kb][v]);
            }
        mx = fmaxf(mx, est_swap32(mx));
        if (mx == -INFINITY) continue;                 // no key of this tile is visible to the row
        const float m_new = fmaxf(m_run, mx);
        float sum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) sum += __builtin_amdgcn_exp2f(s[kb][v] - m_new);
        l_run = l_run * __builtin_amdgcn_exp2f(m_run - m_new) + sum;
        m_run = m_new;
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
    const int split = blockIdx.x, h = blockIdx.y;
    const int lane = threadIdx.x, x = lane % 32, g = lane / 32;
    const int kvh = h / a.G;
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
    for (int kt = kt0; kt < kt1; ++kt) {
        const vec *k = (const vec *)(kbase + (int64_t)kt * TILE_BYTES);
        const int64_t j0 = (int64_t)kt * kTile;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            vec kfr[NU];
#pragma unroll
            for (int u = 0; u < NU; ++u) kfr[u] = k[(kb * NU + u) * 64 + lane];
            const int64_t j = j0 + kBlk * kb + x;      // this lane's key
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
        }
        __syncthreads();
        // diagonal sums of the tile: lane t takes a - b = t and a - b = -t
        // (a = row - r0, b = key - j0), i.e. offsets (r0 - j0) + t and (r0 - j0) - t
        const int t = lane;
        float dp = 0.f, dm = 0.f;
        for (int r = t; r < kEstRows; ++r) dp += P[r * LD + (r - t)];
        for (int r = 0; r + t < kTile; ++r) dm += P[r * LD + (r + t)];
        const int64_t base = (int64_t)a.r0 - j0;
        if (base + t >= 0 && base + t < a.S && dp != 0.f) atomicAdd(&ss[base + t], dp);
        if (t > 0 && base - t >= 0 && base - t < a.S && dm != 0.f) atomicAdd(&ss[base - t], dm);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// top-k with forced head: grid (Hq, 2 lists) blocks of 1024 threads
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;

// inclusive prefix sum of one value per thread over the block; returns it and
// the block total in *total
__device__ int block_scan(int val, int *total, int *wsum) {
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    constexpr int NWAVES = kTopkThreads / 64;
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
};

__global__ __launch_bounds__(kTopkThreads) void est_topk_kernel(TopkArgs a) {
    __shared__ unsigned hist[256];
    __shared__ int wsum[kTopkThreads / 64];
    __shared__ unsigned sel_bin, sel_above;
    const int h = blockIdx.x, list = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t n = a.S;
    const int budget = a.budget[list];
    const unsigned *bits = (const unsigned *)(a.score[list] + (int64_t)h * n);   // scores >= 0: bit order = value order
    int32_t *out = a.out[list] + (int64_t)h * budget;
    const int f = min((int64_t)min(a.forced, budget), n);
    for (int i = tid; i < f; i += kTopkThreads) out[i] = i;
    const int64_t k = budget - f;                        // to pick from [f, n)
    if (k <= 0) return;
    if (n - f <= k) {                                  // every candidate
        for (int64_t i = f + tid; i < n; i += kTopkThreads) out[i] = (int32_t)i;
        return;
    }
    // radix select, 8 bits per pass from the top: the k-th largest bit pattern
    unsigned prefix = 0, pmask = 0;
    unsigned remaining = (unsigned)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
        __syncthreads();
        for (int64_t i = f + tid; i < n; i += kTopkThreads) {
            const unsigned b = bits[i];
            if ((b & pmask) == prefix) atomicAdd(&hist[(b >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            unsigned above = 0;
            int bin = 255;
            for (; bin > 0; --bin) {
                if (above + hist[bin] >= remaining) break;
                above += hist[bin];
            }
            sel_bin = (unsigned)bin;
            sel_above = above;
        }
        __syncthreads();
        prefix |= sel_bin << shift;
        pmask |= 255u << shift;
        remaining -= sel_above;
        __syncthreads();
    }
    // bits > prefix are all taken; `remaining` of the bits == prefix, the
    // smallest indices first; written in index order after the forced head
    int pos = f;
    int ties = 0;
    for (int64_t base = f; base < n; base += kTopkThreads) {
        const int64_t i = base + tid;
        const unsigned b = i < n ? bits[i] : 0u;
        const bool gt = i < n && b > prefix;
        const bool eq = i < n && b == prefix;
        int eq_total;
        const int eq_rank = block_scan(eq ? 1 : 0, &eq_total, wsum) - (eq ? 1 : 0);
        const bool take = gt || (eq && ties + eq_rank < (int)remaining);
        int tot;
        const int rank = block_scan(take ? 1 : 0, &tot, wsum) - (take ? 1 : 0);
        if (take) out[pos + rank] = (int32_t)i;
        pos += tot;
        ties += eq_total;
        if (pos >= budget) break;
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
    int64_t want = (2048 + p.Hq - 1) / p.Hq;
    want = want < kEstMaxSplits ? want : kEstMaxSplits;
    want = want < a.n_tiles ? want : a.n_tiles;
    a.tiles_per_split = (int32_t)((a.n_tiles + want - 1) / want);
    a.n_split = (a.n_tiles + a.tiles_per_split - 1) / a.tiles_per_split;
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL((est_rowstat_kernel<T, D>), dim3((unsigned)a.n_split, (unsigned)(2 * p.Hq)), dim3(64), 0, s, a);
    int err = (int)hipGetLastError();
    if (err) return err;
    hipLaunchKernelGGL(est_rowcombine_kernel, dim3((unsigned)p.Hq), dim3(kEstRows), 0, s, a);
    if ((err = (int)hipGetLastError())) return err;
    const int64_t n = p.Hq * p.S;
    hipLaunchKernelGGL(est_clear_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, sscore, n);
    if ((err = (int)hipGetLastError())) return err;
    hipLaunchKernelGGL((est_sums_kernel<T, D>), dim3((unsigned)a.n_split, (unsigned)p.Hq), dim3(64), 0, s, a);
    return (int)hipGetLastError();
}

size_t est_scratch_bytes(const Problem &p) {
    return ((size_t)p.Hq * kEstRows * kEstMaxSplits * 2 + (size_t)p.Hq * kEstRows * 2) * sizeof(float);
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
    hipLaunchKernelGGL(est_topk_kernel, dim3((unsigned)p.Hq, 2), dim3(kTopkThreads), 0, (hipStream_t)stream, t);
    return (int)hipGetLastError();
}

}  // namespace dca
