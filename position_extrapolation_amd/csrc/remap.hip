// RoPE / DCA remap pre-pass for gfx950.
//
// [mizuki, Inter-Chunk Attention]: DCA only changes position indices -- keys
// sit at j mod C, each query gets three positions (intra r(i), successive
// min(C + r(i), C + W - 1), inter C + W - 1). This pass rotates every key once
// and every query three times and writes the results, plus a re-laid-out copy
// of V, in the attention kernel's fragment order (see dca_internal.h); the
// rotated keys are scaled by yarn * softmax_scale * log2(e) so that scores
// leave the matrix cores in base-2 exponent units [mizuki, DCA + YaRN]. It is
// bound by HBM bandwidth: per token it reads (Hq + 2 Hkv) d elements and
// writes (3 Hq + 2 Hkv) d elements.
//
// Half-split RoPE [yudong §3]: pairs (m, m + d/2) turn by p * theta_m with
// theta_m = base^(-2m/d). cos and sin come from a float32 table built here
// from float64 angles (an fp32 angle p * theta at p ~ 3e5 would carry 0.03 rad
// of error).
#include <hip/hip_runtime.h>

#include "dca_internal.h"
#include "frag.h"

namespace dca {

// ---------------------------------------------------------------------------
// cos/sin table: table[p * (D/2) + m] = (cos(p theta_m), sin(p theta_m))
// ---------------------------------------------------------------------------
__global__ void rope_table_kernel(float2 *__restrict__ table, int64_t n, int half, RopeTheta th) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n) return;
    const int64_t p = idx / half;
    const int m = (int)(idx % half);
    const double ang = (double)p * th.theta[m];
    table[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

int launch_rope_table(const Problem &p, double rope_base, void *ws, const Layout &L, void *stream) {
    RopeTheta th{};
    const int half = (int)(p.D / 2);
    for (int m = 0; m < half; ++m) th.theta[m] = pow(rope_base, -2.0 * m / (double)p.D);
    const int64_t n = p.n_pos * half;
    const int threads = 256;
    const int64_t blocks = (n + threads - 1) / threads;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(threads), 0, (hipStream_t)stream,
                       (float2 *)((char *)ws + L.table), n, half, th);
    return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// remap kernel
// The inputs hold the n rows [q0, q0 + n) of the sequence (q0 = 0, n = S for a
// whole-sequence call). grid.x = B * (Hq + Hkv + Hkv): query heads, then key
// heads (rotated), then value heads (re-laid out); grid.y = ceil(n / 256) * 8
// row blocks of 32. Query variants are written at the call's own row
// blocks; keys and values at their blocks in the sequence, up to the end of
// the last 64-key tile the call's rows can see (rows past n as zeros).
// ---------------------------------------------------------------------------
struct RemapArgs {
    const void *q, *k, *v;
    void *qf[3];
    void *kf, *vf;
    const float2 *table;
    float k_scale;               // multiplies the rotated keys
    int64_t n, q0, C, W;         // input rows per head, their first sequence index
    int32_t Hq, Hkv, Hv;         // query, key and value heads handled (Hv = 0: keys only)
    int32_t nblk_q, nblk_kv;     // 32-row blocks per head in the query / key-value sections
    int32_t kv_blk_end;          // key-value blocks [q0 / 32, kv_blk_end) are written
};

template <typename T, int D>
__global__ __launch_bounds__(256) void remap_kernel(RemapArgs a) {
    using F = Frag<T>;
    constexpr int E = F::E;
    constexpr int NP = D / (2 * E);        // 16-byte chunk pairs (c, c + NP) per row
    constexpr int NU = D / (2 * E);        // fragment slices per 32-row block
    constexpr int HALF = D / 2;
    constexpr int BLK_ELEMS = kBlk * D;

    // heads vary fastest: the workgroups of one row block, which read the
    // same table rows, run together and share them through L2
    const int64_t blk = blockIdx.y;
    const int y = blockIdx.x;
    const int per_b = a.Hq + a.Hkv + a.Hv;
    const int b = y / per_b;
    const int hh = y % per_b;
    const int64_t kv_blk = a.q0 / kBlk + blk;     // the block's place in the key-value sections
    if (hh >= a.Hq && kv_blk >= a.kv_blk_end) return;

    if (hh >= a.Hq + a.Hkv) {
        // ---- V re-layout through LDS -------------------------------------
        const int h = hh - a.Hq - a.Hkv;
        const int64_t bh = (int64_t)b * a.Hkv + h;
        __shared__ T tile[kBlk][D + 2 * E];
        const T *src = (const T *)a.v + (bh * a.n + blk * kBlk) * D;
        for (int c = threadIdx.x; c < kBlk * D / E; c += blockDim.x) {
            const int r = c / (D / E), col = (c % (D / E)) * E;
            typename F::vec val;
            if (blk * kBlk + r < a.n) {
                val = *(const typename F::vec *)(src + (int64_t)r * D + col);
            } else {
                val = F::zero();
            }
#pragma unroll
            for (int e = 0; e < E; ++e) tile[r][col + e] = F::get(val, e);
        }
        __syncthreads();
        // fragment (db, u, lane): element e = V[2E u + 8 (e/4) + 4 g + e%4][32 db + x]
        constexpr int NUV = kBlk / (2 * E);
        T *dst = (T *)a.vf + (bh * a.nblk_kv + kv_blk) * BLK_ELEMS;
        for (int f = threadIdx.x; f < (D / 32) * NUV * 64; f += blockDim.x) {
            const int lane = f % 64, u = (f / 64) % NUV, db = f / (64 * NUV);
            const int x = lane % 32, g = lane / 32;
            typename F::vec val;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int key = 2 * E * u + 8 * (e / 4) + 4 * g + (e % 4);
                F::set(val, e, tile[key][32 * db + x]);
            }
            *(typename F::vec *)(dst + (int64_t)f * E) = val;
        }
        return;
    }

    // ---- Q (three variants) or K: rotate -----------------------------------
    const bool is_q = hh < a.Hq;
    const int h = is_q ? hh : hh - a.Hq;
    const int H = is_q ? a.Hq : a.Hkv;
    const int64_t bh = (int64_t)b * H + h;
    const T *src = (const T *)(is_q ? a.q : a.k) + bh * a.n * D;
    const int nvar = is_q ? 3 : 1;

    for (int item = threadIdx.x; item < kBlk * NP; item += blockDim.x) {
        const int ri = item / NP, c = item % NP;
        const int64_t il = blk * kBlk + ri;       // input row
        const int64_t i = a.q0 + il;              // sequence index
        const bool valid = il < a.n;
        typename F::vec x1 = F::zero(), x2 = F::zero();
        if (valid) {
            x1 = *(const typename F::vec *)(src + il * D + c * E);
            x2 = *(const typename F::vec *)(src + il * D + HALF + c * E);
        }
        float f1[E], f2[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            f1[e] = (float)F::get(x1, e);
            f2[e] = (float)F::get(x2, e);
        }
        // fragment slots of the two chunks
        const int c2 = NP + c;
        const int64_t off1 = ((int64_t)(c / 2) * 64 + (c % 2) * 32 + ri) * E;
        const int64_t off2 = ((int64_t)(c2 / 2) * 64 + (c2 % 2) * 32 + ri) * E;
        for (int var = 0; var < nvar; ++var) {
            int64_t pos;
            if (!is_q) pos = pos_key(i, a.C);
            else if (var == 0) pos = pos_intra(i, a.C);
            else if (var == 1) pos = pos_succ(i, a.C, a.W);
            else pos = pos_inter(a.C, a.W);
            typename F::vec y1 = F::zero(), y2 = F::zero();
            if (valid) {
                const float2 *cs = a.table + pos * HALF + c * E;
                const float sc = is_q ? 1.f : a.k_scale;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float2 t = cs[e];
                    const float2 r = rope_pair(f1[e], f2[e], t.x, t.y);
                    F::set(y1, e, F::from_float(r.x * sc));
                    F::set(y2, e, F::from_float(r.y * sc));
                }
            }
            T *dst = is_q ? (T *)a.qf[var] + (bh * a.nblk_q + blk) * BLK_ELEMS
                          : (T *)a.kf + (bh * a.nblk_kv + kv_blk) * BLK_ELEMS;
            *(typename F::vec *)(dst + off1) = y1;
            *(typename F::vec *)(dst + off2) = y2;
        }
    }
    (void)NU;
}

template <typename T, int D>
static int launch_remap_t(const Problem &p, const void *q, const void *k, const void *v, float k_scale, void *ws,
                          const Layout &L, void *stream) {
    RemapArgs a{};
    a.k_scale = k_scale;
    a.q = q;
    a.k = k;
    a.v = v;
    for (int i = 0; i < 3; ++i) a.qf[i] = (char *)ws + L.q[i];
    a.kf = (char *)ws + L.k;
    a.vf = (char *)ws + L.v;
    a.table = (const float2 *)((char *)ws + L.table);
    a.n = p.NQ;
    a.q0 = p.q0;
    a.C = p.C;
    a.W = p.W;
    a.Hq = p.fused ? 0 : (int32_t)p.Hq;          // fused rotation: keys and values only
    a.Hkv = (int32_t)p.Hkv;
    a.Hv = p.keys_only ? 0 : (int32_t)p.Hkv;
    a.nblk_q = (int32_t)(p.NQ_pad / kBlk);
    a.nblk_kv = (int32_t)(p.S_pad / kBlk);
    a.kv_blk_end = (int32_t)((p.q0 + p.NQ + kTile - 1) / kTile * (kTile / kBlk));
    dim3 grid((unsigned)(p.B * (a.Hq + a.Hkv + a.Hv)), (unsigned)(p.NQ_pad / kBlk));
    hipLaunchKernelGGL((remap_kernel<T, D>), grid, dim3(256), 0, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

int launch_remap(const Problem &p, const void *q, const void *k, const void *v, float k_scale, void *ws,
                 const Layout &L, void *stream) {
    if (p.dtype == DCA_BF16)
        return p.D == 128 ? launch_remap_t<__bf16, 128>(p, q, k, v, k_scale, ws, L, stream)
                          : launch_remap_t<__bf16, 64>(p, q, k, v, k_scale, ws, L, stream);
    return p.D == 128 ? launch_remap_t<float, 128>(p, q, k, v, k_scale, ws, L, stream)
                      : launch_remap_t<float, 64>(p, q, k, v, k_scale, ws, L, stream);
}

// ---------------------------------------------------------------------------
// checks: device position map, tile regions, workspace unpacking
// ---------------------------------------------------------------------------
__global__ void debug_positions_kernel(int64_t S, int64_t C, int64_t W, int32_t *pq_intra,
                                       int32_t *pq_succ, int32_t *pq_inter, int32_t *pk) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= S) return;
    pq_intra[i] = (int32_t)pos_intra(i, C);
    pq_succ[i] = (int32_t)pos_succ(i, C, W);
    pk[i] = (int32_t)pos_key(i, C);
    if (i == 0) *pq_inter = (int32_t)pos_inter(C, W);
}

int launch_debug_positions(int64_t S, int64_t C, int64_t W, int32_t *pq_intra, int32_t *pq_succ,
                           int32_t *pq_inter, int32_t *pk, void *stream) {
    const int threads = 256;
    hipLaunchKernelGGL(debug_positions_kernel, dim3((unsigned)((S + threads - 1) / threads)),
                       dim3(threads), 0, (hipStream_t)stream, S, C, W, pq_intra, pq_succ, pq_inter,
                       pk);
    return (int)hipGetLastError();
}

__global__ void debug_tile_regions_kernel(int64_t n, int64_t C, uint8_t *out) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n * n) return;
    const int64_t t = idx / n, kt = idx % n;
    out[idx] = kt > t ? (uint8_t)255
                      : (uint8_t)region_of((t * kTile) / C, (kt * kTile) / C);
}

int launch_debug_tile_regions(int64_t S, int64_t C, uint8_t *out, void *stream) {
    const int64_t n = (S + kTile - 1) / kTile;
    const int threads = 256;
    hipLaunchKernelGGL(debug_tile_regions_kernel, dim3((unsigned)((n * n + threads - 1) / threads)),
                       dim3(threads), 0, (hipStream_t)stream, n, C, out);
    return (int)hipGetLastError();
}

template <typename T, int D>
__global__ void debug_unpack_kernel(const T *__restrict__ src, T *__restrict__ dst, int64_t S,
                                    int64_t nblk, int64_t n, int vlayout) {
    constexpr int E = Frag<T>::E;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n) return;
    const int d = (int)(idx % D);
    const int64_t i = (idx / D) % S;
    const int64_t bh = idx / ((int64_t)D * S);
    const int64_t blk = i / kBlk;
    const int r = (int)(i % kBlk);
    int64_t off;
    if (!vlayout) {
        const int u = d / (2 * E), g = (d % (2 * E)) / E, e = d % E;
        off = (bh * nblk + blk) * (kBlk * D) + ((int64_t)u * 64 + 32 * g + r) * E + e;
    } else {
        constexpr int NUV = kBlk / (2 * E);
        const int u = r / (2 * E), rem = r % (2 * E);
        const int g = (rem % 8) / 4, e = 4 * (rem / 8) + rem % 4;
        const int db = d / 32, x = d % 32;
        off = (bh * nblk + blk) * (kBlk * D) + (((int64_t)db * NUV + u) * 64 + 32 * g + x) * E + e;
    }
    dst[idx] = src[off];
}

template <typename T, int D>
static int launch_unpack_t(const Problem &p, const void *ws, const Layout &L, int which, void *dst,
                           void *stream) {
    const size_t base = which < 3 ? L.q[which] : (which == 3 ? L.k : L.v);
    const int64_t H = which < 3 ? p.Hq : p.Hkv;
    const int64_t n = p.B * H * p.S * p.D;
    const int threads = 256;
    hipLaunchKernelGGL((debug_unpack_kernel<T, D>), dim3((unsigned)((n + threads - 1) / threads)),
                       dim3(threads), 0, (hipStream_t)stream, (const T *)((const char *)ws + base),
                       (T *)dst, p.S, (which < 3 ? p.NQ_pad : p.S_pad) / kBlk, n, which == 4 ? 1 : 0);
    return (int)hipGetLastError();
}

int launch_debug_unpack(const Problem &p, const void *ws, const Layout &L, int which, void *dst,
                        void *stream) {
    if (p.dtype == DCA_BF16)
        return p.D == 128 ? launch_unpack_t<__bf16, 128>(p, ws, L, which, dst, stream)
                          : launch_unpack_t<__bf16, 64>(p, ws, L, which, dst, stream);
    return p.D == 128 ? launch_unpack_t<float, 128>(p, ws, L, which, dst, stream)
                      : launch_unpack_t<float, 64>(p, ws, L, which, dst, stream);
}

}  // namespace dca
