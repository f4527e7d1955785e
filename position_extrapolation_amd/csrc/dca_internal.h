// Internal declarations shared by the host code and the HIP kernels of libdca.
//
// Operand layout ("fragment order").  The attention kernel contracts on
// gfx950 matrix cores with 32x32 output blocks:
//   bf16: v_mfma_f32_32x32x16_bf16, each lane feeds 8 bf16 (16 bytes) per op;
//   f32 : v_mfma_f32_32x32x2_f32,   each lane feeds 1 float per op, and four
//         ops share one 16-byte fragment.
// A 16-byte fragment holds E elements (E = 8 bf16 or 4 f32) of one lane. A
// wave's 64 lanes split as lane = 32 g + x, x in [0, 32), g in {0, 1}: x picks
// the row (A operand) or column (B operand), g picks which half of a 2E-wide
// slice of the contraction index the lane holds.
//
// The pre-pass writes every operand straight into this order, so the kernel
// moves 16 contiguous bytes per lane from HBM to LDS to registers and never
// shuffles:
//   Q variants, rotated K (contraction over head dims):
//     [bh][blk32][u = D/2E][lane 64][E]   element = X[32 blk + x][2E u + E g + e]
//   V (contraction over keys, the kernel computes O^T = V^T P^T):
//     [bkv][blk32][db = D/32][u = 32/2E][lane 64][E]
//        element = V[32 blk + key(u, g, e)][32 db + x]
//        key(u, g, e) = 2E u + 8 (e / 4) + 4 g + e % 4
//   key(u, g, e) is the order in which the 32x32 accumulator of S^T = K Q^T
//   leaves scores in a lane (key 8 (v / 4) + 4 g + v % 4 for value v), so the
//   softmax output P^T feeds the PV contraction as-is.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dca.h"

namespace dca {

constexpr int kTile = 64;            // key-tile and vertical-slash tile size
constexpr int kBlk = 32;             // rows per MFMA block / wave
constexpr int kSeqPad = 256;         // sequences are padded to this in the workspace
constexpr int kMaxHalfDim = 64;      // head_dim <= 128
constexpr int kXcds = 8;             // MI355X: 8 XCDs, workgroups dispatched round-robin

struct RopeTheta {
    double theta[kMaxHalfDim];       // base^(-2m/d), m < d/2
};

// Validated problem description plus derived constants. A call computes the
// query rows [q0, q0 + NQ) of a sequence of S tokens against the keys
// [0, q0 + NQ); a whole-sequence prefill has q0 = 0 and NQ = S.
struct Problem {
    int64_t B, Hq, Hkv, G, D, S, S_pad, C, W;
    int64_t q0, NQ, NQ_pad;          // first row, rows, rows padded to 256
    int64_t p_inter;                 // C + W - 1
    int64_t n_pos;                   // C + W positions in the cos/sin table
    int64_t n_tiles;                 // ceil(S / 64)
    int dtype;                       // dca_dtype
    int esize;                       // bytes per element
    float softmax_scale;
    bool sparse;
    bool fused;                      // queries rotated inside the attention kernel: no query section
    bool keys_only;                  // no value section (rotated keys for the vertical-slash estimate)
    int32_t n_vertical, n_slash;
};

// Byte offsets inside the workspace (each 256-byte aligned). Everything but
// the query variants depends on the sequence alone, so one workspace serves
// every chunk of a chunked prefill; the query variants come last and hold the
// rows of one call.
struct Layout {
    size_t table;                    // float2 [n_pos][D/2]
    size_t k;                        // rotated K               [B*Hkv][S_pad*D]
    size_t v;                        // V re-layout             [B*Hkv][S_pad*D]
    size_t vs_flags;                 // uint8 [2][Hq][n_tiles] (sparse only)
    size_t vs_vt, vs_vt_n, vs_dl, vs_dl_n;  // int32 lists and counts (sparse only)
    size_t q[3];                     // Q intra / succ / inter  [B*Hq][NQ_pad*D]
    size_t total;
};

Layout layout_for(const Problem &p);

// Integer position map, the same code on host and device.
__host__ __device__ inline int64_t pos_key(int64_t j, int64_t C) { return j % C; }
__host__ __device__ inline int64_t pos_intra(int64_t i, int64_t C) { return i % C; }
__host__ __device__ inline int64_t pos_succ(int64_t i, int64_t C, int64_t W) {
    const int64_t a = C + i % C, b = C + W - 1;
    return a < b ? a : b;
}
__host__ __device__ inline int64_t pos_inter(int64_t C, int64_t W) { return C + W - 1; }
// Region of rows in chunk cq against keys in chunk ck (ck <= cq): 0 intra,
// 1 successive, 2 inter.
__host__ __device__ inline int region_of(int64_t cq, int64_t ck) {
    const int64_t d = cq - ck;
    return d >= 2 ? 2 : (int)d;
}

// Half-split RoPE turn of the pair (x1, x2) = (x[m], x[m + d/2]) by the
// angle with cosine c and sine s, in fp32: (x1 c - x2 s, x2 c + x1 s), each
// with one explicit fused multiply-add, so that every kernel that rotates a
// vector produces the same bits.
__device__ inline float2 rope_pair(float x1, float x2, float c, float s) {
    return make_float2(fmaf(x1, c, -(x2 * s)), fmaf(x2, c, x1 * s));
}

// Launchers (return hipError_t as int; 0 = success).
int launch_rope_table(const Problem &p, double rope_base, void *ws, const Layout &L, void *stream);
// k_scale multiplies the rotated keys (yarn * softmax scale * log2 e)
int launch_remap(const Problem &p, const void *q, const void *k, const void *v, float k_scale, void *ws,
                 const Layout &L, void *stream);
int launch_vs_index(const Problem &p, const dca_vs_mask &m, void *ws, const Layout &L, void *stream);
// q_nat != null: fused rotation, the kernel turns the caller's queries itself
int launch_attention(const Problem &p, void *out, float *lse, const void *ws, const Layout &L, void *stream,
                     const void *q_nat = nullptr);
// decode of the token at index p.q0 (p.NQ = 1); its scratch (query variants and
// split partials, decode_scratch_bytes) lives in the workspace's query section,
// or at scratch_base when that is not null
int launch_decode(const Problem &p, const void *q, const void *k, const void *v, void *out, float *lse,
                  double rope_base, float k_scale, void *ws, const Layout &L, void *stream,
                  void *scratch_base = nullptr);
// splits of the decode's key range per KV group (its partials are sized for this many)
constexpr int kDecodeMaxSplits = 256;
size_t decode_scratch_bytes(const Problem &p);
// the static device array that holds the decode scratch for dca_decode_static:
// its size, and its address on the current device (looked up once per
// device); kStaticScratchWrongDevice when a non-null stream belongs to
// another device than the current one
constexpr size_t kDecodeStaticScratchBytes = DCA_DECODE_STATIC_SCRATCH_BYTES;
constexpr int kStaticScratchWrongDevice = -1;
int decode_static_scratch(void *stream, void **ptr);
// online vertical-slash estimation over the keys rotated at their own index
// (the pre-pass run with C >= S, W = 0, keys only)
// query rows it scores (the last n <= 64), the splits of the row statistics
// per row, and the workgroups of the selection per (head, list)
constexpr int kEstRows = 64;
constexpr int kEstMaxSplits = 256;
constexpr int kTopkParts = 16;
// scratch bytes: the row statistics and combined rows, then the selection's
// histograms, state and counts (host arithmetic in api.cpp)
size_t est_rows_bytes(const Problem &p);
size_t est_scratch_bytes(const Problem &p);
int launch_vs_estimate(const Problem &p, int n_last, int n_vertical, int n_slash, int n_forced, const void *q,
                       const void *ws, const Layout &L, size_t scratch, float *vscore, float *sscore,
                       int32_t *vertical, int32_t *slash, void *stream);
int launch_debug_positions(int64_t S, int64_t C, int64_t W, int32_t *pq_intra, int32_t *pq_succ,
                           int32_t *pq_inter, int32_t *pk, void *stream);
int launch_debug_tile_regions(int64_t S, int64_t C, uint8_t *out, void *stream);
int launch_debug_unpack(const Problem &p, const void *ws, const Layout &L, int which, void *dst,
                        void *stream);
int launch_debug_vs_lists(const Problem &p, const void *ws, const Layout &L, int32_t *vt,
                          int32_t *vt_n, int32_t *dl, int32_t *dl_n, void *stream);
int launch_debug_vs_tiles(const Problem &p, const void *ws, const Layout &L, int head, int64_t q_tile, int group,
                          int32_t *kt_out, uint32_t *m_out, int32_t cap, int32_t *n_out, void *stream);
const char *hip_error_text(int err);

}  // namespace dca
