// Vertical-slash mask -> per-head 64x64 tile lists, for gfx950.
//
// [mizuki, MInference sections]: a few key columns (vertical) and diagonals
// (slash) carry most of the attention; only those are computed. Read on
// 64 x 64 tiles, tile (t, kt) is active iff
//   kt in VT_h = { v / 64 : v a vertical column of head h }          or
//   t - kt in D_h = { delta : some slash offset o of head h has
//                     max(0, 64 delta - 63) <= o <= 64 delta + 63 }.
// An offset o = 64 a + b (0 <= b < 64) meets exactly delta = a and, when
// b > 0, delta = a + 1.
//
// Three small launches: clear per-head flag rows, mark flags (any order,
// duplicates allowed, out-of-range entries ignored), then compact each flag
// row into an ascending list with one block-wide scan per (head, list).
#include <hip/hip_runtime.h>

#include "dca_internal.h"

namespace dca {

__global__ void vs_clear_kernel(uint8_t *flags, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) flags[i] = 0;
}

__global__ void vs_mark_kernel(const int32_t *__restrict__ vertical, const int32_t *__restrict__ slash,
                               int32_t n_vertical, int32_t n_slash, int32_t Hq, int64_t S,
                               int64_t n_tiles, uint8_t *flags) {
    const int64_t per_head = (int64_t)n_vertical + n_slash;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= per_head * Hq) return;
    const int64_t h = idx / per_head;
    const int64_t e = idx % per_head;
    uint8_t *fv = flags + h * n_tiles;
    uint8_t *fd = flags + ((int64_t)Hq + h) * n_tiles;
    if (e < n_vertical) {
        const int64_t val = vertical[h * n_vertical + e];
        if (val >= 0 && val < S) fv[val / kTile] = 1;
    } else {
        const int64_t val = slash[h * n_slash + (e - n_vertical)];
        if (val >= 0 && val < S) {
            const int64_t a = val / kTile;
            fd[a] = 1;
            if (val % kTile != 0 && a + 1 < n_tiles) fd[a + 1] = 1;
        }
    }
}

// one block per (list, head): ascending indices of set flags
__global__ __launch_bounds__(1024) void vs_compact_kernel(const uint8_t *flags, int64_t n_tiles,
                                                          int32_t Hq, int32_t *vt, int32_t *vt_n,
                                                          int32_t *dl, int32_t *dl_n) {
    const int list = blockIdx.x / Hq;       // 0 = VT, 1 = D
    const int h = blockIdx.x % Hq;
    const uint8_t *f = flags + ((int64_t)list * Hq + h) * n_tiles;
    int32_t *out = (list == 0 ? vt : dl) + (int64_t)h * n_tiles;
    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const int64_t per = (n_tiles + nth - 1) / nth;
    const int64_t lo = tid * per;
    const int64_t hi = lo + per < n_tiles ? lo + per : n_tiles;
    int32_t cnt = 0;
    for (int64_t i = lo; i < hi; ++i) cnt += f[i] ? 1 : 0;

    __shared__ int32_t scan[1024];
    scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < nth; off <<= 1) {     // inclusive Hillis-Steele scan
        const int32_t add = tid >= off ? scan[tid - off] : 0;
        __syncthreads();
        scan[tid] += add;
        __syncthreads();
    }
    int32_t pos = scan[tid] - cnt;
    for (int64_t i = lo; i < hi; ++i)
        if (f[i]) out[pos++] = (int32_t)i;
    if (tid == nth - 1) (list == 0 ? vt_n : dl_n)[h] = scan[tid];
}

int launch_vs_index(const Problem &p, const dca_vs_mask &m, void *ws, const Layout &L, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    uint8_t *flags = (uint8_t *)ws + L.vs_flags;
    const int64_t nflags = 2 * p.Hq * p.n_tiles;
    hipLaunchKernelGGL(vs_clear_kernel, dim3((unsigned)((nflags + 255) / 256)), dim3(256), 0, s, flags,
                       nflags);
    int err = (int)hipGetLastError();
    if (err) return err;
    const int64_t nmark = ((int64_t)m.n_vertical + m.n_slash) * p.Hq;
    if (nmark > 0) {
        hipLaunchKernelGGL(vs_mark_kernel, dim3((unsigned)((nmark + 255) / 256)), dim3(256), 0, s,
                           m.vertical, m.slash, m.n_vertical, m.n_slash, (int32_t)p.Hq, p.S, p.n_tiles,
                           flags);
        err = (int)hipGetLastError();
        if (err) return err;
    }
    hipLaunchKernelGGL(vs_compact_kernel, dim3((unsigned)(2 * p.Hq)), dim3(1024), 0, s, flags, p.n_tiles,
                       (int32_t)p.Hq, (int32_t *)((char *)ws + L.vs_vt), (int32_t *)((char *)ws + L.vs_vt_n),
                       (int32_t *)((char *)ws + L.vs_dl), (int32_t *)((char *)ws + L.vs_dl_n));
    return (int)hipGetLastError();
}

__global__ void vs_copy_kernel(const int32_t *src, int32_t *dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

int launch_debug_vs_lists(const Problem &p, const void *ws, const Layout &L, int32_t *vt, int32_t *vt_n,
                          int32_t *dl, int32_t *dl_n, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    const int64_t nl = p.Hq * p.n_tiles;
    const char *w = (const char *)ws;
    struct { const int32_t *src; int32_t *dst; int64_t n; } jobs[4] = {
        {(const int32_t *)(w + L.vs_vt), vt, nl},
        {(const int32_t *)(w + L.vs_vt_n), vt_n, p.Hq},
        {(const int32_t *)(w + L.vs_dl), dl, nl},
        {(const int32_t *)(w + L.vs_dl_n), dl_n, p.Hq},
    };
    for (auto &j : jobs) {
        hipLaunchKernelGGL(vs_copy_kernel, dim3((unsigned)((j.n + 255) / 256)), dim3(256), 0, s, j.src,
                           j.dst, j.n);
        const int err = (int)hipGetLastError();
        if (err) return err;
    }
    return 0;
}

}  // namespace dca
