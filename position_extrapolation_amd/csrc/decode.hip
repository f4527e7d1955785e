// DCA decode for gfx950: one new token per sequence against the key/value
// cache that a prefill left in the workspace.
//
// The new token sits at sequence index pos. Its query takes the three DCA
// positions of row pos -- intra pos mod C, successive min(C + pos mod C,
// C + W - 1), inter C + W - 1 [mizuki, Intra-/Successive-/Inter-Chunk
// Attention] -- and attends to the keys [0, pos], each key at j mod C, with
// the variant picked by the chunk distance of the key tile; the logits carry
// the YaRN temperature through the pre-scaled keys [mizuki, DCA + YaRN]. The
// result equals row pos of a prefill over the first pos + 1 tokens.
//
// Three launches:
//   decode_prep_kernel    rotates the new key (at pos mod C, scaled) and
//                         writes it and the new value into the cache at index
//                         pos (zero-filling the rest of a fresh 64-key tile),
//                         and rotates the new query three ways;
//   decode_attn_kernel    split-K flash decoding: one wave per (KV group,
//                         split of the key tiles). The wave's 32 score
//                         columns are the query heads of the KV group, so
//                         every K and V fragment read from HBM feeds all G
//                         heads through the same 64-key tile step as the
//                         prefill; it writes a partial (max, sum, O) per head;
//   decode_combine_kernel merges the splits per head.
// The attention launch is bound by HBM: it reads the cache once.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dca_internal.h"
#include "frag.h"
#include "tile_math.h"

namespace dca {

constexpr int kMaxSplits = kDecodeMaxSplits;

struct DecodeArgs {
    const void *q, *k, *v;       // new token: q [B][Hq][D], k and v [B][Hkv][D]
    void *kf, *vf;               // cache sections of the workspace
    void *qv;                    // rotated query variants [B][Hq][3][D]
    float *part;                 // partials [B][Hq][kMaxSplits][D + 2]: O, max (log2 units), sum
    void *out;                   // [B][Hq][D]
    float *lse;                  // [B][Hq] or null
    RopeTheta th;
    float k_scale;               // yarn * softmax scale * log2 e
    int64_t pos, C, W;
    int32_t Hq, Hkv, G, nblk_kv;
    int32_t n_split, tiles_per_split;
};

// cos and sin of p * theta_m, the same float64 formula as the prefill table
__device__ __forceinline__ float2 rope_cs(const DecodeArgs &a, int64_t p, int m) {
    const double ang = (double)p * a.th.theta[m];
    return make_float2((float)cos(ang), (float)sin(ang));
}

// ---------------------------------------------------------------------------
// prep: grid B * (Hq + Hkv + Hkv) blocks of 128 threads
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(128) void decode_prep_kernel(DecodeArgs a) {
    using F = Frag<T>;
    constexpr int E = F::E;
    constexpr int HALF = D / 2;
    constexpr int BLK_ELEMS = kBlk * D;
    constexpr int NUV = kBlk / (2 * E);
    const int per_b = a.Hq + 2 * a.Hkv;
    const int b = blockIdx.x / per_b;
    const int hh = blockIdx.x % per_b;
    const int t = threadIdx.x;

    if (hh < a.Hq) {
        // query: three rotated variants, rounded to the operand type
        if (t >= HALF) return;
        const int64_t bh = (int64_t)b * a.Hq + hh;
        const T *x = (const T *)a.q + bh * D;
        const float x1 = (float)x[t], x2 = (float)x[t + HALF];
        T *dst = (T *)a.qv + bh * 3 * D;
        for (int var = 0; var < 3; ++var) {
            const int64_t p = var == 0 ? pos_intra(a.pos, a.C)
                                       : (var == 1 ? pos_succ(a.pos, a.C, a.W) : pos_inter(a.C, a.W));
            const float2 cs = rope_cs(a, p, t);
            const float2 r = rope_pair(x1, x2, cs.x, cs.y);
            dst[var * D + t] = F::from_float(r.x);
            dst[var * D + t + HALF] = F::from_float(r.y);
        }
        return;
    }
    const bool is_k = hh < a.Hq + a.Hkv;
    const int h = is_k ? hh - a.Hq : hh - a.Hq - a.Hkv;
    const int64_t bh = (int64_t)b * a.Hkv + h;
    // rows pos .. row_end - 1 are written: the new token, then zeros to the
    // end of its 64-key tile when the token opens that tile
    const int64_t row_end = (a.pos % kTile == 0) ? a.pos + kTile : a.pos + 1;
    if (is_k) {
        const T *x = (const T *)a.k + bh * D;
        for (int64_t r = a.pos; r < row_end; ++r) {
            T *blk = (T *)a.kf + (bh * a.nblk_kv + r / kBlk) * BLK_ELEMS;
            const int ri = (int)(r % kBlk);
            for (int d = t; d < D; d += blockDim.x) {
                float y = 0.f;
                if (r == a.pos) {
                    const int m = d % HALF;
                    const float x1 = (float)x[m], x2 = (float)x[m + HALF];
                    const float2 cs = rope_cs(a, pos_key(a.pos, a.C), m);
                    const float2 rr = rope_pair(x1, x2, cs.x, cs.y);
                    y = (d < HALF ? rr.x : rr.y) * a.k_scale;
                }
                // fragment slot of element d of row ri (operand order of dca_internal.h)
                const int c = d / E, e = d % E;
                blk[((int64_t)(c / 2) * 64 + (c % 2) * 32 + ri) * E + e] = F::from_float(y);
            }
        }
    } else {
        const T *x = (const T *)a.v + bh * D;
        for (int64_t r = a.pos; r < row_end; ++r) {
            T *blk = (T *)a.vf + (bh * a.nblk_kv + r / kBlk) * BLK_ELEMS;
            const int ri = (int)(r % kBlk);
            // key ri = key(u, g, e) = 2E u + 8 (e / 4) + 4 g + e % 4
            const int u = ri / (2 * E), rem = ri % (2 * E);
            const int g = (rem % 8) / 4, e = 4 * (rem / 8) + rem % 4;
            for (int d = t; d < D; d += blockDim.x) {
                const T val = r == a.pos ? x[d] : F::from_float(0.f);
                const int db = d / 32, lane = 32 * g + d % 32;
                blk[(((int64_t)db * NUV + u) * 64 + lane) * E + e] = val;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// attention: grid (n_split, B * Hkv) waves
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64, sizeof(T) == 2 ? 2 : 1) void decode_attn_kernel(DecodeArgs a) {
    using F = Frag<T>;
    using vec = typename F::vec;
    constexpr int E = F::E;
    constexpr int NU = D / (2 * E);
    constexpr int NUV = kBlk / (2 * E);
    constexpr int NDB = D / 32;
    constexpr int BLK_ELEMS = kBlk * D;
    constexpr int TILE_BYTES = 2 * BLK_ELEMS * (int)sizeof(T);

    const int split = blockIdx.x;
    const int bkv_i = blockIdx.y;
    const int b = bkv_i / a.Hkv;
    const int kvh = bkv_i % a.Hkv;
    const int64_t bkv = (int64_t)b * a.Hkv + kvh;
    const int lane = threadIdx.x;
    const int x = lane % 32, g = lane / 32;
    const bool col_ok = x < a.G;                       // column x = query head kvh * G + x
    const int64_t bh = (int64_t)b * a.Hq + (int64_t)kvh * a.G + (col_ok ? x : 0);

    const int n_tiles = (int)(a.pos / kTile) + 1;
    const int kt0 = split * a.tiles_per_split;
    const int kt1 = min(kt0 + a.tiles_per_split, n_tiles);
    const int cq = (int)(a.pos / a.C);
    const char *kbase = (const char *)a.kf + bkv * a.nblk_kv * (int64_t)BLK_ELEMS * (int64_t)sizeof(T);
    const char *vbase = (const char *)a.vf + bkv * a.nblk_kv * (int64_t)BLK_ELEMS * (int64_t)sizeof(T);

    WaveState<T, D> st;
    st.region = -1;
    st.first = true;
#pragma unroll
    for (int db = 0; db < NDB; ++db) st.oacc[db] = f32x16{};
    st.mref = 0.f;
    st.l_run = 0.f;

    for (int kt = kt0; kt < kt1; ++kt) {
        const int region = region_of(cq, (int64_t)kt * kTile / a.C);
        if (region != st.region) {
            const vec *qs = (const vec *)((const T *)a.qv + (bh * 3 + region) * D);
#pragma unroll
            for (int u = 0; u < NU; ++u) st.qfrag[u] = col_ok ? qs[2 * u + g] : F::zero();
            st.region = region;
        }
        const char *kl = kbase + (int64_t)kt * TILE_BYTES;
        // the tile's V fragments are requested together with its K fragments
        VFrags<T, D> vf;
        load_v<T, D>(lane, vbase + (int64_t)kt * TILE_BYTES, vf);
        f32x16 s[2];
        tile_scores<T, D, false>(lane, st, kl, s);
        const int lim = (int)(a.pos - (int64_t)kt * kTile);   // key offset k is kept iff k <= lim
        if (lim < kTile - 1) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (kBlk * kb + 8 * (v / 4) + 4 * g + (v % 4) > lim) s[kb][v] = -INFINITY;
        }
        vec p[2][NUV];
        float psum = tile_p<T>(s, p);
        const bool ok = psum <= kPsumLimit;          // false for inf and NaN too
        if (__builtin_amdgcn_ballot_w64(!ok || st.first) != 0) {
            raise_ref<T, D>(st, s);
            psum = tile_p<T>(s, p);
        }
        st.l_run += psum;
        tile_pv<T, D>(st, vf, p);
    }

    if (!col_ok) return;
    float *part = a.part + (bh * kMaxSplits + split) * (D + 2);
    const float l_tot = st.l_run + lane_swap32(st.l_run);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) part[32 * db + 8 * (v / 4) + 4 * g + (v % 4)] = st.oacc[db][v];
    if (g == 0) {
        part[D] = st.first ? -INFINITY : st.mref;
        part[D + 1] = st.first ? 0.f : l_tot;
    }
}

// ---------------------------------------------------------------------------
// combine: grid B * Hq blocks of 1024 threads
// ---------------------------------------------------------------------------
constexpr int kCombineThreads = 1024;

// block-wide max / sum of one value per thread: a wave reduction, then one
// pass over the 16 wave results
template <bool MAX>
__device__ __forceinline__ float block_reduce(float x, float *wred) {
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float y = __shfl_xor(x, off, 64);
        x = MAX ? fmaxf(x, y) : x + y;
    }
    if (lane == 0) wred[wave] = x;
    __syncthreads();
    float r = wred[0];
#pragma unroll
    for (int w = 1; w < kCombineThreads / 64; ++w) r = MAX ? fmaxf(r, wred[w]) : r + wred[w];
    __syncthreads();                             // wred is reused by the next reduction
    return r;
}

template <typename T, int D>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecodeArgs a) {
    constexpr int RPT = kCombineThreads / D;     // threads sharing one output element
    static_assert(kMaxSplits <= kCombineThreads, "one thread per split for the reductions");
    __shared__ float wgt[kMaxSplits];            // 2^(m_s - M), 0 for empty splits
    __shared__ float red[kCombineThreads];
    __shared__ float wred[kCombineThreads / 64];
    const int64_t bh = blockIdx.x;
    const int t = threadIdx.x;
    const float *part = a.part + bh * kMaxSplits * (D + 2);
    const bool live = t < a.n_split && part[t * (D + 2) + D + 1] > 0.f;
    const float m = live ? part[t * (D + 2) + D] : -INFINITY;
    const float mx = block_reduce<true>(m, wred);                   // M over the live splits
    const float wt = live ? __builtin_amdgcn_exp2f(m - mx) : 0.f;
    if (t < kMaxSplits) wgt[t] = wt;
    const float den = block_reduce<false>(live ? wt * part[t * (D + 2) + D + 1] : 0.f, wred);   // also orders wgt
    // O[d] = sum_s w_s O_s[d] / den: thread t sums every RPT-th split of
    // element t % D, four independent partial sums so the loads overlap
    const int d = t % D, r = t / D;
    float n0 = 0.f, n1 = 0.f, n2 = 0.f, n3 = 0.f;
    int s = r;
    for (; s + 3 * RPT < a.n_split; s += 4 * RPT) {
        n0 += wgt[s] * part[s * (D + 2) + d];
        n1 += wgt[s + RPT] * part[(s + RPT) * (D + 2) + d];
        n2 += wgt[s + 2 * RPT] * part[(s + 2 * RPT) * (D + 2) + d];
        n3 += wgt[s + 3 * RPT] * part[(s + 3 * RPT) * (D + 2) + d];
    }
    for (; s < a.n_split; s += RPT) n0 += wgt[s] * part[s * (D + 2) + d];
    red[t] = (n0 + n1) + (n2 + n3);
    __syncthreads();
    for (int w = RPT / 2; w > 0; w /= 2) {
        if (r < w) red[t] += red[t + w * D];
        __syncthreads();
    }
    if (r == 0) {
        ((T *)a.out)[bh * D + d] = Frag<T>::from_float(den > 0.f ? red[d] / den : 0.f);
        if (a.lse != nullptr && d == 0)
            a.lse[bh] = den > 0.f ? (mx + log2f(den)) * 0.69314718055994531f : -INFINITY;
    }
}

template <typename T, int D>
static int launch_decode_t(const Problem &p, const void *q, const void *k, const void *v, void *out, float *lse,
                           double rope_base, float k_scale, void *ws, const Layout &L, void *scratch_base,
                           void *stream) {
    DecodeArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.kf = (char *)ws + L.k;
    a.vf = (char *)ws + L.v;
    char *sbase = scratch_base != nullptr ? (char *)scratch_base : (char *)ws + L.q[0];
    a.qv = sbase;
    const size_t qv_bytes = ((size_t)p.B * p.Hq * 3 * D * sizeof(T) + 255) & ~(size_t)255;
    a.part = (float *)(sbase + qv_bytes);
    a.out = out;
    a.lse = lse;
    for (int m = 0; m < D / 2; ++m) a.th.theta[m] = pow(rope_base, -2.0 * m / (double)D);
    a.k_scale = k_scale;
    a.pos = p.q0;
    a.C = p.C;
    a.W = p.W;
    a.Hq = (int32_t)p.Hq;
    a.Hkv = (int32_t)p.Hkv;
    a.G = (int32_t)p.G;
    a.nblk_kv = (int32_t)(p.S_pad / kBlk);
    // about 2048 waves in flight over the cache, at most kMaxSplits per KV group
    const int64_t n_tiles = p.q0 / kTile + 1;
    const int64_t groups = p.B * p.Hkv;
    int64_t want = (2048 + groups - 1) / groups;
    want = want < kMaxSplits ? want : kMaxSplits;
    want = want < n_tiles ? want : n_tiles;
    a.tiles_per_split = (int32_t)((n_tiles + want - 1) / want);
    a.n_split = (int32_t)((n_tiles + a.tiles_per_split - 1) / a.tiles_per_split);
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL((decode_prep_kernel<T, D>), dim3((unsigned)(p.B * (p.Hq + 2 * p.Hkv))), dim3(128), 0, s, a);
    int err = (int)hipGetLastError();
    if (err) return err;
    hipLaunchKernelGGL((decode_attn_kernel<T, D>), dim3((unsigned)a.n_split, (unsigned)groups), dim3(64), 0, s, a);
    err = (int)hipGetLastError();
    if (err) return err;
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((unsigned)(p.B * p.Hq)), dim3(kCombineThreads), 0, s, a);
    return (int)hipGetLastError();
}

int launch_decode(const Problem &p, const void *q, const void *k, const void *v, void *out, float *lse,
                  double rope_base, float k_scale, void *ws, const Layout &L, void *stream, void *scratch_base) {
    if (p.dtype == DCA_BF16)
        return p.D == 128
                   ? launch_decode_t<__bf16, 128>(p, q, k, v, out, lse, rope_base, k_scale, ws, L, scratch_base, stream)
                   : launch_decode_t<__bf16, 64>(p, q, k, v, out, lse, rope_base, k_scale, ws, L, scratch_base, stream);
    return p.D == 128
               ? launch_decode_t<float, 128>(p, q, k, v, out, lse, rope_base, k_scale, ws, L, scratch_base, stream)
               : launch_decode_t<float, 64>(p, q, k, v, out, lse, rope_base, k_scale, ws, L, scratch_base, stream);
}

// ---------------------------------------------------------------------------
// the decode scratch in a static device array (dca_decode_static)
// ---------------------------------------------------------------------------
// For callers that cannot allocate: the rotated query variants and the
// split partials live here instead of in the workspace's query section.
// Every GPU the library runs on holds its own copy, at its own address, until
// the process ends. In host code `scratch` names a host-side stand-in, not
// device memory: only the address hipGetSymbolAddress returns for the
// current device may reach a kernel.
static __device__ __align__(256) char scratch[kDecodeStaticScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];

int decode_static_scratch(void *stream, void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    if (stream != nullptr) {
        // the kernels run on the stream's device: its copy of the array is
        // the one they may touch, and it is looked up with that device current
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice((hipStream_t)stream, &sdev);
        if (e != hipSuccess) return (int)e;
        if (sdev != dev) return kStaticScratchWrongDevice;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        // once per device, with that device current
        void *addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        if (addr == nullptr) return (int)hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = addr;
    }
    *ptr = g_scratch_ptr[dev];
    return 0;
}

}  // namespace dca
