// libdca C ABI: argument validation, derived constants, workspace layout and
// stage sequencing. Every argument is checked before the first HIP call; a
// rejected call enqueues nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "dca_internal.h"

namespace dca {

static thread_local std::string g_last_error;

static int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
static int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

static int ok() {
    g_last_error.clear();
    return DCA_OK;
}

static int device_fail(int err, const char *what) {
    return fail(DCA_E_DEVICE, "%s: HIP error %d (%s)", what, err, hip_error_text(err));
}

const char *hip_error_text(int err) { return hipGetErrorString((hipError_t)err); }

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Scratch sizes of the decode and the vertical-slash estimate (host
// arithmetic; the kernels take the same offsets).
size_t decode_scratch_bytes(const Problem &p) {
    const size_t qv = align256((size_t)p.B * p.Hq * 3 * p.D * p.esize);
    return qv + (size_t)p.B * p.Hq * kDecodeMaxSplits * (p.D + 2) * sizeof(float);
}

size_t est_rows_bytes(const Problem &p) {
    return ((size_t)p.Hq * kEstRows * kEstMaxSplits * 2 + (size_t)p.Hq * kEstRows * 2) * sizeof(float);
}

size_t est_scratch_bytes(const Problem &p) {
    return est_rows_bytes(p) + (size_t)p.Hq * 2 * (256 + 4 + kTopkParts * 2) * 4;
}

static bool misaligned(const void *ptr, uintptr_t a) { return ptr != nullptr && ((uintptr_t)ptr & (a - 1)) != 0; }

Layout layout_for(const Problem &p) {
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    L.table = take((size_t)p.n_pos * (size_t)(p.D / 2) * 8);
    const size_t kvbytes = (size_t)p.B * p.Hkv * p.S_pad * p.D * p.esize;
    L.k = take(kvbytes);
    L.v = take(p.keys_only ? 0 : kvbytes);
    if (p.sparse) {
        L.vs_flags = take((size_t)2 * p.Hq * p.n_tiles);
        L.vs_vt = take((size_t)p.Hq * p.n_tiles * 4);
        L.vs_vt_n = take((size_t)p.Hq * 4);
        L.vs_dl = take((size_t)p.Hq * p.n_tiles * 4);
        L.vs_dl_n = take((size_t)p.Hq * 4);
    }
    const size_t qbytes = p.fused ? 0 : (size_t)p.B * p.Hq * p.NQ_pad * p.D * p.esize;
    for (int i = 0; i < 3; ++i) L.q[i] = take(qbytes);
    L.total = off;
    return L;
}

// Validate sizes and the shape; fill p. Pointers are checked by callers.
static int make_problem(int64_t seq, int64_t C, int64_t W, const dca_shape *shape,
                        const dca_vs_mask *mask, Problem *p) {
    if (shape == nullptr) return fail(DCA_E_INVALID, "shape is NULL");
    if (seq < 1) return fail(DCA_E_INVALID, "seq must be >= 1 (got %lld)", (long long)seq);
    if (seq >= ((int64_t)1 << 31)) return fail(DCA_E_UNSUPPORTED, "seq must be < 2^31");
    if (C < 1 || W < 0) return fail(DCA_E_INVALID, "need C >= 1 and W >= 0 (got C=%lld W=%lld)",
                                    (long long)C, (long long)W);
    if (C < kTile || C % kTile != 0)
        return fail(DCA_E_UNSUPPORTED, "C must be a positive multiple of %d (got %lld)", kTile, (long long)C);
    if (W > C) return fail(DCA_E_UNSUPPORTED, "W must be <= C (got W=%lld C=%lld)", (long long)W, (long long)C);
    if (C + W >= ((int64_t)1 << 31)) return fail(DCA_E_UNSUPPORTED, "C + W must be < 2^31");
    if (shape->batch < 1 || shape->n_q_heads < 1 || shape->n_kv_heads < 1)
        return fail(DCA_E_INVALID, "batch and head counts must be >= 1");
    if (shape->n_q_heads % shape->n_kv_heads != 0)
        return fail(DCA_E_INVALID, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                    shape->n_q_heads, shape->n_kv_heads);
    if (shape->head_dim != 64 && shape->head_dim != 128)
        return fail(DCA_E_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", shape->head_dim);
    if (shape->dtype != DCA_F32 && shape->dtype != DCA_BF16)
        return fail(DCA_E_INVALID, "dtype must be DCA_F32 or DCA_BF16 (got %d)", shape->dtype);
    if (!(shape->softmax_scale >= 0.f) || !isfinite(shape->softmax_scale))
        return fail(DCA_E_INVALID, "softmax_scale must be finite and >= 0");
    Problem q{};
    q.B = shape->batch;
    q.Hq = shape->n_q_heads;
    q.Hkv = shape->n_kv_heads;
    q.G = q.Hq / q.Hkv;
    q.D = shape->head_dim;
    q.S = seq;
    q.S_pad = (seq + kSeqPad - 1) / kSeqPad * kSeqPad;
    q.q0 = 0;
    q.NQ = seq;
    q.NQ_pad = q.S_pad;
    q.C = C;
    q.W = W;
    q.p_inter = C + W - 1;
    q.n_pos = C + W;
    q.n_tiles = (seq + kTile - 1) / kTile;
    q.dtype = shape->dtype;
    q.esize = shape->dtype == DCA_BF16 ? 2 : 4;
    q.softmax_scale = shape->softmax_scale > 0.f ? shape->softmax_scale : 1.f / sqrtf((float)q.D);
    if (q.B * q.Hq * q.S_pad * q.D >= ((int64_t)1 << 40))
        return fail(DCA_E_UNSUPPORTED, "problem too large");
    if (mask != nullptr) {
        if (mask->n_vertical < 0 || mask->n_slash < 0)
            return fail(DCA_E_INVALID, "mask counts must be >= 0");
        if (mask->n_vertical > 0 && mask->vertical == nullptr)
            return fail(DCA_E_INVALID, "mask->vertical is NULL");
        if (mask->n_slash > 0 && mask->slash == nullptr)
            return fail(DCA_E_INVALID, "mask->slash is NULL");
        if (misaligned(mask->vertical, 4) || misaligned(mask->slash, 4))
            return fail(DCA_E_INVALID, "mask lists must be 4-byte aligned");
        q.sparse = true;
        q.n_vertical = mask->n_vertical;
        q.n_slash = mask->n_slash;
    }
    *p = q;
    return DCA_OK;
}

// Restrict p to the query rows [q_offset, q_offset + n_rows) of its sequence.
static int set_chunk(int64_t q_offset, int64_t n_rows, Problem *p) {
    if (n_rows < 1) return fail(DCA_E_INVALID, "n_rows must be >= 1 (got %lld)", (long long)n_rows);
    if (q_offset < 0 || q_offset > p->S - n_rows)
        return fail(DCA_E_INVALID, "rows [%lld, %lld) are not inside the sequence of %lld tokens",
                    (long long)q_offset, (long long)(q_offset + n_rows), (long long)p->S);
    if (q_offset % kTile != 0)
        return fail(DCA_E_UNSUPPORTED, "q_offset must be a multiple of %d (got %lld)", kTile, (long long)q_offset);
    p->q0 = q_offset;
    p->NQ = n_rows;
    p->NQ_pad = (n_rows + kSeqPad - 1) / kSeqPad * kSeqPad;
    return DCA_OK;
}

static bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

static int check_workspace(const Problem &p, const void *ws, size_t bytes, Layout *L) {
    *L = layout_for(p);
    if (ws == nullptr) return fail(DCA_E_INVALID, "workspace is NULL");
    if (((uintptr_t)ws & 255) != 0) return fail(DCA_E_INVALID, "workspace must be 256-byte aligned");
    if (bytes < L->total)
        return fail(DCA_E_WORKSPACE, "workspace has %zu bytes, needs %zu", bytes, L->total);
    return DCA_OK;
}

// The pre-pass writes the workspace while it reads the inputs (and the
// fused-rotation kernel reads q beside the workspace): an input inside the
// workspace would be overwritten mid-read. q is [B][Hq][NQ][D], k and v
// [B][Hkv][NQ][D] for the call's rows.
static int check_inputs_vs_workspace(const Problem &p, const void *const *inputs, int n_inputs, const void *ws,
                                     size_t ws_bytes) {
    static const char *const names[3] = {"q", "k", "v"};
    for (int i = 0; i < n_inputs; ++i) {
        const size_t ib = (size_t)p.B * (i == 0 ? p.Hq : p.Hkv) * p.NQ * p.D * p.esize;
        if (overlaps(ws, ws_bytes, inputs[i], ib))
            return fail(DCA_E_INVALID, "%s overlaps the workspace", names[i]);
    }
    return DCA_OK;
}

// The mask lists are read by the index pass, which writes the workspace; in
// a chunked prefill they are read again after earlier blocks wrote out and
// lse. Lists that share memory with the workspace or the outputs would be
// overwritten before (or while) they are read.
static int check_mask_overlaps(const Problem &p, const dca_vs_mask *mask, const void *ws, size_t ws_bytes,
                               const void *out, const float *lse) {
    if (!p.sparse) return DCA_OK;
    const size_t vb = (size_t)p.Hq * mask->n_vertical * 4, sb = (size_t)p.Hq * mask->n_slash * 4;
    const size_t obytes = out ? (size_t)p.B * p.Hq * p.NQ * p.D * p.esize : 0;
    const size_t lbytes = lse ? (size_t)p.B * p.Hq * p.NQ * 4 : 0;
    if (overlaps(mask->vertical, vb, ws, ws_bytes) || overlaps(mask->slash, sb, ws, ws_bytes))
        return fail(DCA_E_INVALID, "a mask list overlaps the workspace");
    if (overlaps(mask->vertical, vb, out, obytes) || overlaps(mask->slash, sb, out, obytes) ||
        overlaps(mask->vertical, vb, lse, lbytes) || overlaps(mask->slash, sb, lse, lbytes))
        return fail(DCA_E_INVALID, "a mask list overlaps out or lse");
    return DCA_OK;
}

}  // namespace dca

using namespace dca;

extern "C" {

const char *dca_status_str(int status) {
    switch (status) {
        case DCA_OK: return "DCA_OK";
        case DCA_E_INVALID: return "DCA_E_INVALID: invalid argument";
        case DCA_E_UNSUPPORTED: return "DCA_E_UNSUPPORTED: outside the supported domain";
        case DCA_E_WORKSPACE: return "DCA_E_WORKSPACE: workspace too small";
        case DCA_E_DEVICE: return "DCA_E_DEVICE: HIP runtime or launch failure";
        default: return "unknown dca_status";
    }
}

const char *dca_last_error(void) { return g_last_error.c_str(); }

int dca_remap_positions(int64_t seq, int64_t C, int64_t W, int32_t *pq_intra, int32_t *pq_succ,
                        int32_t *pq_inter, int32_t *pk) {
    if (seq < 1 || seq >= ((int64_t)1 << 31)) return fail(DCA_E_INVALID, "seq out of range");
    if (C < 1 || W < 0 || C + W >= ((int64_t)1 << 31)) return fail(DCA_E_INVALID, "C or W out of range");
    for (int64_t i = 0; i < seq; ++i) {
        if (pq_intra) pq_intra[i] = (int32_t)pos_intra(i, C);
        if (pq_succ) pq_succ[i] = (int32_t)pos_succ(i, C, W);
        if (pk) pk[i] = (int32_t)pos_key(i, C);
    }
    if (pq_inter) *pq_inter = (int32_t)pos_inter(C, W);
    return ok();
}

int dca_workspace_size(int64_t seq, int64_t C, int64_t W, const dca_shape *shape, const dca_vs_mask *mask,
                       size_t *bytes) {
    if (bytes == nullptr) return fail(DCA_E_INVALID, "bytes is NULL");
    Problem p;
    int st = make_problem(seq, C, W, shape, mask, &p);
    if (st) return st;
    *bytes = layout_for(p).total;
    return ok();
}

static int check_rope(double rope_base) {
    if (!(rope_base > 1.0) || !isfinite(rope_base)) return fail(DCA_E_INVALID, "rope_base must be finite and > 1");
    return DCA_OK;
}

static int check_yarn(float yarn_scale) {
    if (!(yarn_scale > 0.f) || !isfinite(yarn_scale)) return fail(DCA_E_INVALID, "yarn_scale must be finite and > 0");
    return DCA_OK;
}

static int do_remap(const Problem &p, const void *q, const void *k, const void *v, double rope_base,
                    float yarn_scale, void *ws, const Layout &L, void *stream) {
    int err = launch_rope_table(p, rope_base, ws, L, stream);
    if (err) return device_fail(err, "rope table launch");
    const float k_scale = yarn_scale * p.softmax_scale * 1.4426950408889634f;
    err = launch_remap(p, q, k, v, k_scale, ws, L, stream);
    if (err) return device_fail(err, "remap launch");
    return DCA_OK;
}

int dca_remap(const void *q, const void *k, const void *v, int64_t seq, int64_t C, int64_t W, double rope_base,
              float yarn_scale, const dca_shape *shape, void *workspace, size_t workspace_bytes, void *stream) {
    Problem p;
    Layout L;
    int st = make_problem(seq, C, W, shape, nullptr, &p);
    if (st) return st;
    if (q == nullptr || k == nullptr || v == nullptr) return fail(DCA_E_INVALID, "q, k and v must be non-NULL");
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16))
        return fail(DCA_E_INVALID, "q, k and v must be 16-byte aligned");
    if ((st = check_rope(rope_base))) return st;
    if ((st = check_yarn(yarn_scale))) return st;
    if ((st = check_workspace(p, workspace, workspace_bytes, &L))) return st;
    const void *inputs[3] = {q, k, v};
    if ((st = check_inputs_vs_workspace(p, inputs, 3, workspace, workspace_bytes))) return st;
    if ((st = do_remap(p, q, k, v, rope_base, yarn_scale, workspace, L, stream))) return st;
    return ok();
}

int dca_vs_index(int64_t seq, int64_t C, int64_t W, const dca_vs_mask *mask, const dca_shape *shape,
                 void *workspace, size_t workspace_bytes, void *stream) {
    Problem p;
    Layout L;
    if (mask == nullptr) return fail(DCA_E_INVALID, "mask is NULL");
    int st = make_problem(seq, C, W, shape, mask, &p);
    if (st) return st;
    if ((st = check_workspace(p, workspace, workspace_bytes, &L))) return st;
    if ((st = check_mask_overlaps(p, mask, workspace, workspace_bytes, nullptr, nullptr))) return st;
    const int err = launch_vs_index(p, *mask, workspace, L, stream);
    if (err) return device_fail(err, "vertical-slash index launch");
    return ok();
}

static int check_outputs(const Problem &p, const void *out, const float *lse, const void *const *inputs,
                         int n_inputs, const void *ws, size_t ws_bytes) {
    if (out == nullptr) return fail(DCA_E_INVALID, "out is NULL");
    if (misaligned(out, 16) || misaligned(lse, 4)) return fail(DCA_E_INVALID, "out must be 16-byte and lse 4-byte aligned");
    const size_t obytes = (size_t)p.B * p.Hq * p.NQ * p.D * p.esize;
    const size_t kvbytes = (size_t)p.B * p.Hkv * p.NQ * p.D * p.esize;
    const size_t lbytes = lse ? (size_t)p.B * p.Hq * p.NQ * 4 : 0;
    for (int i = 0; i < n_inputs; ++i) {
        const size_t ib = i == 0 ? obytes : kvbytes;   // q first, then k, v
        if (overlaps(out, obytes, inputs[i], ib)) return fail(DCA_E_INVALID, "out overlaps an input");
        if (overlaps(lse, lbytes, inputs[i], ib)) return fail(DCA_E_INVALID, "lse overlaps an input");
    }
    if (int st = check_inputs_vs_workspace(p, inputs, n_inputs, ws, ws_bytes)) return st;
    if (overlaps(out, obytes, ws, ws_bytes)) return fail(DCA_E_INVALID, "out overlaps the workspace");
    if (overlaps(lse, lbytes, ws, ws_bytes)) return fail(DCA_E_INVALID, "lse overlaps the workspace");
    if (overlaps(lse, lbytes, out, obytes)) return fail(DCA_E_INVALID, "lse overlaps out");
    return DCA_OK;
}

int dca_attention(void *out, float *lse, int64_t seq, int64_t C, int64_t W, const dca_vs_mask *mask,
                  const dca_shape *shape, const void *workspace, size_t workspace_bytes, void *stream) {
    Problem p;
    Layout L;
    int st = make_problem(seq, C, W, shape, mask, &p);
    if (st) return st;
    if ((st = check_workspace(p, workspace, workspace_bytes, &L))) return st;
    if ((st = check_outputs(p, out, lse, nullptr, 0, workspace, workspace_bytes))) return st;
    const int err = launch_attention(p, out, lse, workspace, L, stream);
    if (err) return device_fail(err, "attention launch");
    return ok();
}

int dca_prefill(const void *q, const void *k, const void *v, void *out, float *lse, int64_t seq, int64_t C,
                int64_t W, double rope_base, float yarn_scale, const dca_vs_mask *mask, const dca_shape *shape,
                void *workspace, size_t workspace_bytes, void *stream) {
    Problem p;
    Layout L;
    int st = make_problem(seq, C, W, shape, mask, &p);
    if (st) return st;
    if (q == nullptr || k == nullptr || v == nullptr) return fail(DCA_E_INVALID, "q, k and v must be non-NULL");
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16))
        return fail(DCA_E_INVALID, "q, k and v must be 16-byte aligned");
    if ((st = check_rope(rope_base))) return st;
    if ((st = check_yarn(yarn_scale))) return st;
    if ((st = check_workspace(p, workspace, workspace_bytes, &L))) return st;
    const void *inputs[3] = {q, k, v};
    if ((st = check_outputs(p, out, lse, inputs, 3, workspace, workspace_bytes))) return st;
    if ((st = check_mask_overlaps(p, mask, workspace, workspace_bytes, out, lse))) return st;
    if ((st = do_remap(p, q, k, v, rope_base, yarn_scale, workspace, L, stream))) return st;
    if (p.sparse) {
        const int err = launch_vs_index(p, *mask, workspace, L, stream);
        if (err) return device_fail(err, "vertical-slash index launch");
    }
    const int err = launch_attention(p, out, lse, workspace, L, stream);
    if (err) return device_fail(err, "attention launch");
    return ok();
}

int dca_chunk_workspace_size(int64_t seq, int64_t max_rows, int64_t C, int64_t W, const dca_shape *shape,
                             const dca_vs_mask *mask, size_t *bytes) {
    if (bytes == nullptr) return fail(DCA_E_INVALID, "bytes is NULL");
    Problem p;
    int st = make_problem(seq, C, W, shape, mask, &p);
    if (st) return st;
    if (max_rows < 1 || max_rows > seq)
        return fail(DCA_E_INVALID, "max_rows must be in [1, seq] (got %lld)", (long long)max_rows);
    if ((st = set_chunk(0, max_rows, &p))) return st;
    *bytes = layout_for(p).total;
    return ok();
}

int dca_prefill_chunk(const void *q, const void *k, const void *v, void *out, float *lse, int64_t q_offset,
                      int64_t n_rows, int64_t seq, int64_t C, int64_t W, double rope_base, float yarn_scale,
                      const dca_vs_mask *mask, const dca_shape *shape, void *workspace, size_t workspace_bytes,
                      void *stream) {
    Problem p;
    Layout L;
    int st = make_problem(seq, C, W, shape, mask, &p);
    if (st) return st;
    if ((st = set_chunk(q_offset, n_rows, &p))) return st;
    if (q == nullptr || k == nullptr || v == nullptr) return fail(DCA_E_INVALID, "q, k and v must be non-NULL");
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16))
        return fail(DCA_E_INVALID, "q, k and v must be 16-byte aligned");
    if ((st = check_rope(rope_base))) return st;
    if ((st = check_yarn(yarn_scale))) return st;
    if ((st = check_workspace(p, workspace, workspace_bytes, &L))) return st;
    const void *inputs[3] = {q, k, v};
    if ((st = check_outputs(p, out, lse, inputs, 3, workspace, workspace_bytes))) return st;
    if ((st = check_mask_overlaps(p, mask, workspace, workspace_bytes, out, lse))) return st;
    if ((st = do_remap(p, q, k, v, rope_base, yarn_scale, workspace, L, stream))) return st;
    if (p.sparse) {
        const int err = launch_vs_index(p, *mask, workspace, L, stream);
        if (err) return device_fail(err, "vertical-slash index launch");
    }
    const int err = launch_attention(p, out, lse, workspace, L, stream);
    if (err) return device_fail(err, "attention launch");
    return ok();
}

int dca_fused_workspace_size(int64_t seq, int64_t C, int64_t W, const dca_shape *shape, const dca_vs_mask *mask,
                             size_t *bytes) {
    if (bytes == nullptr) return fail(DCA_E_INVALID, "bytes is NULL");
    Problem p;
    int st = make_problem(seq, C, W, shape, mask, &p);
    if (st) return st;
    p.fused = true;
    *bytes = layout_for(p).total;
    return ok();
}

int dca_prefill_fused(const void *q, const void *k, const void *v, void *out, float *lse, int64_t seq, int64_t C,
                      int64_t W, double rope_base, float yarn_scale, const dca_vs_mask *mask,
                      const dca_shape *shape, void *workspace, size_t workspace_bytes, void *stream) {
    Problem p;
    Layout L;
    int st = make_problem(seq, C, W, shape, mask, &p);
    if (st) return st;
    p.fused = true;
    if (q == nullptr || k == nullptr || v == nullptr) return fail(DCA_E_INVALID, "q, k and v must be non-NULL");
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16))
        return fail(DCA_E_INVALID, "q, k and v must be 16-byte aligned");
    if ((st = check_rope(rope_base))) return st;
    if ((st = check_yarn(yarn_scale))) return st;
    if ((st = check_workspace(p, workspace, workspace_bytes, &L))) return st;
    const void *inputs[3] = {q, k, v};
    if ((st = check_outputs(p, out, lse, inputs, 3, workspace, workspace_bytes))) return st;
    if ((st = check_mask_overlaps(p, mask, workspace, workspace_bytes, out, lse))) return st;
    if ((st = do_remap(p, nullptr, k, v, rope_base, yarn_scale, workspace, L, stream))) return st;
    if (p.sparse) {
        const int err = launch_vs_index(p, *mask, workspace, L, stream);
        if (err) return device_fail(err, "vertical-slash index launch");
    }
    const int err = launch_attention(p, out, lse, workspace, L, stream, q);
    if (err) return device_fail(err, "attention launch");
    return ok();
}

// The estimate's workspace: the pre-pass layout for the keys rotated at their
// own index (chunk length ceil(seq / 64) * 64 >= seq, window 0, keys only),
// then the row statistics, then the two score arrays.
static int est_problem(int64_t seq, const dca_shape *shape, Problem *p, size_t *scratch, size_t *scores,
                       size_t *total) {
    const int64_t C = (seq + kTile - 1) / kTile * kTile;
    int st = make_problem(seq, C, 0, shape, nullptr, p);
    if (st) return st;
    if (p->B != 1) return fail(DCA_E_UNSUPPORTED, "the estimate takes batch 1 (got %lld)", (long long)p->B);
    p->fused = true;
    p->keys_only = true;
    const size_t base = layout_for(*p).total;
    *scratch = base;
    *scores = align256(base + est_scratch_bytes(*p));
    *total = align256(*scores + (size_t)2 * p->Hq * p->S * sizeof(float));
    return DCA_OK;
}

int dca_vs_estimate_workspace_size(int64_t seq, const dca_shape *shape, size_t *bytes) {
    if (bytes == nullptr) return fail(DCA_E_INVALID, "bytes is NULL");
    Problem p;
    size_t scratch, scores, total;
    int st = est_problem(seq, shape, &p, &scratch, &scores, &total);
    if (st) return st;
    *bytes = total;
    return ok();
}

int dca_vs_estimate(const void *q, const void *k, int64_t seq, int32_t n_last, double rope_base, float yarn_scale,
                    int32_t n_vertical, int32_t n_slash, int32_t n_forced, const dca_shape *shape,
                    int32_t *vertical, int32_t *slash, float *vertical_score, float *slash_score,
                    void *workspace, size_t workspace_bytes, void *stream) {
    Problem p;
    size_t scratch, scores, total;
    int st = est_problem(seq, shape, &p, &scratch, &scores, &total);
    if (st) return st;
    if (q == nullptr || k == nullptr) return fail(DCA_E_INVALID, "q and k must be non-NULL");
    if (misaligned(q, 16) || misaligned(k, 16)) return fail(DCA_E_INVALID, "q and k must be 16-byte aligned");
    if (vertical == nullptr || slash == nullptr) return fail(DCA_E_INVALID, "vertical and slash must be non-NULL");
    if (misaligned(vertical, 4) || misaligned(slash, 4) || misaligned(vertical_score, 4) || misaligned(slash_score, 4))
        return fail(DCA_E_INVALID, "output lists and scores must be 4-byte aligned");
    if (n_last < 1 || n_last > 64 || n_last > seq)
        return fail(DCA_E_INVALID, "n_last must be in [1, min(64, seq)] (got %d)", n_last);
    if (n_vertical < 1 || n_vertical > seq || n_slash < 1 || n_slash > seq)
        return fail(DCA_E_INVALID, "budgets must be in [1, seq] (got %d, %d)", n_vertical, n_slash);
    if (n_forced < 0 || n_forced > n_vertical || n_forced > n_slash)
        return fail(DCA_E_INVALID, "n_forced must be in [0, min(budgets)] (got %d)", n_forced);
    if ((st = check_rope(rope_base))) return st;
    if ((st = check_yarn(yarn_scale))) return st;
    if (workspace == nullptr) return fail(DCA_E_INVALID, "workspace is NULL");
    if (((uintptr_t)workspace & 255) != 0) return fail(DCA_E_INVALID, "workspace must be 256-byte aligned");
    if (workspace_bytes < total)
        return fail(DCA_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, total);
    const void *inputs[2] = {q, k};
    if ((st = check_inputs_vs_workspace(p, inputs, 2, workspace, workspace_bytes))) return st;
    const Layout L = layout_for(p);
    float *ws_scores = (float *)((char *)workspace + scores);   // [2][Hq][seq], used for absent outputs
    float *vs = vertical_score ? vertical_score : ws_scores;
    float *ss = slash_score ? slash_score : ws_scores + p.Hq * p.S;
    // the four outputs against each other, the workspace and the inputs (q is
    // [1][Hq][seq][D], k [1][Hkv][seq][D])
    const size_t vb = (size_t)p.Hq * n_vertical * 4, sb = (size_t)p.Hq * n_slash * 4, cb = (size_t)p.Hq * p.S * 4;
    const void *outs[4] = {vertical, slash, vertical_score, slash_score};
    const size_t ob[4] = {vb, sb, cb, cb};
    const size_t qb = (size_t)p.Hq * p.S * p.D * p.esize, kb = (size_t)p.Hkv * p.S * p.D * p.esize;
    for (int i = 0; i < 4; ++i) {
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], ob[i], outs[j], ob[j])) return fail(DCA_E_INVALID, "outputs overlap each other");
        if (overlaps(outs[i], ob[i], workspace, workspace_bytes))
            return fail(DCA_E_INVALID, "an output overlaps the workspace");
        if (overlaps(outs[i], ob[i], q, qb) || overlaps(outs[i], ob[i], k, kb))
            return fail(DCA_E_INVALID, "an output overlaps q or k");
    }
    // keys rotated at their own index, scaled like the attention's
    int err = launch_rope_table(p, rope_base, workspace, L, stream);
    if (err) return device_fail(err, "rope table launch");
    const float k_scale = yarn_scale * p.softmax_scale * 1.4426950408889634f;
    err = launch_remap(p, nullptr, k, nullptr, k_scale, workspace, L, stream);
    if (err) return device_fail(err, "key rotation launch");
    err = launch_vs_estimate(p, n_last, n_vertical, n_slash, n_forced, q, workspace, L, scratch, vs, ss, vertical,
                             slash, stream);
    if (err) return device_fail(err, "vertical-slash estimate launch");
    return ok();
}

}  // extern "C"

// dca_decode and dca_decode_static: the same checks and launches; the scratch
// of the split-key reduction lives in the workspace's query section, or
// (static_scratch) in the library's static device array.
static int decode_call(const void *q, const void *k, const void *v, void *out, float *lse, int64_t pos,
                       int64_t seq, int64_t C, int64_t W, double rope_base, float yarn_scale, const dca_shape *shape,
                       void *workspace, size_t workspace_bytes, void *stream, bool static_scratch) {
    Problem p;
    Layout L;
    int st = make_problem(seq, C, W, shape, nullptr, &p);
    if (st) return st;
    if (pos < 0 || pos >= seq)
        return fail(DCA_E_INVALID, "pos must be in [0, seq) (got %lld, seq %lld)", (long long)pos, (long long)seq);
    if (p.G > kBlk)
        return fail(DCA_E_UNSUPPORTED, "decode needs n_q_heads / n_kv_heads <= %d (got %lld)", kBlk, (long long)p.G);
    p.q0 = pos;
    p.NQ = 1;
    p.NQ_pad = kSeqPad;
    // with the static scratch the workspace needs the key/value cache only
    p.fused = static_scratch;
    if (q == nullptr || k == nullptr || v == nullptr) return fail(DCA_E_INVALID, "q, k and v must be non-NULL");
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16))
        return fail(DCA_E_INVALID, "q, k and v must be 16-byte aligned");
    if ((st = check_rope(rope_base))) return st;
    if ((st = check_yarn(yarn_scale))) return st;
    if ((st = check_workspace(p, workspace, workspace_bytes, &L))) return st;
    if (static_scratch) {
        if (decode_scratch_bytes(p) > kDecodeStaticScratchBytes)
            return fail(DCA_E_UNSUPPORTED,
                        "the decode scratch of batch %lld x %lld query heads (d = %lld) needs %zu bytes; the static "
                        "array holds %zu (use dca_decode with a workspace)",
                        (long long)p.B, (long long)p.Hq, (long long)p.D, decode_scratch_bytes(p),
                        kDecodeStaticScratchBytes);
    } else if (decode_scratch_bytes(p) > L.total - L.q[0]) {
        return fail(DCA_E_WORKSPACE, "query section too small for the decode scratch");
    }
    const void *inputs[3] = {q, k, v};
    if ((st = check_outputs(p, out, lse, inputs, 3, workspace, workspace_bytes))) return st;
    void *scratch_base = nullptr;
    if (static_scratch) {
        const int err = decode_static_scratch(stream, &scratch_base);
        if (err == kStaticScratchWrongDevice)
            return fail(DCA_E_INVALID, "the stream belongs to another device than the current one; make the "
                                       "stream's device current before the call");
        if (err) return device_fail(err, "static scratch lookup");
    }
    const float k_scale = yarn_scale * p.softmax_scale * 1.4426950408889634f;
    const int err = launch_decode(p, q, k, v, out, lse, rope_base, k_scale, workspace, L, stream, scratch_base);
    if (err) return device_fail(err, "decode launch");
    return ok();
}

extern "C" {

int dca_decode(const void *q, const void *k, const void *v, void *out, float *lse, int64_t pos, int64_t seq,
               int64_t C, int64_t W, double rope_base, float yarn_scale, const dca_shape *shape, void *workspace,
               size_t workspace_bytes, void *stream) {
    return decode_call(q, k, v, out, lse, pos, seq, C, W, rope_base, yarn_scale, shape, workspace, workspace_bytes,
                       stream, false);
}

int dca_decode_static(const void *q, const void *k, const void *v, void *out, float *lse, int64_t pos, int64_t seq,
                      int64_t C, int64_t W, double rope_base, float yarn_scale, const dca_shape *shape,
                      void *workspace, size_t workspace_bytes, void *stream) {
    return decode_call(q, k, v, out, lse, pos, seq, C, W, rope_base, yarn_scale, shape, workspace, workspace_bytes,
                       stream, true);
}

int dca_debug_positions(int64_t seq, int64_t C, int64_t W, int32_t *pq_intra, int32_t *pq_succ,
                        int32_t *pq_inter, int32_t *pk, void *stream) {
    if (seq < 1 || seq >= ((int64_t)1 << 31)) return fail(DCA_E_INVALID, "seq out of range");
    if (C < 1 || W < 0 || C + W >= ((int64_t)1 << 31)) return fail(DCA_E_INVALID, "C or W out of range");
    if (!pq_intra || !pq_succ || !pq_inter || !pk) return fail(DCA_E_INVALID, "output arrays must be non-NULL");
    const int err = launch_debug_positions(seq, C, W, pq_intra, pq_succ, pq_inter, pk, stream);
    if (err) return device_fail(err, "positions launch");
    return ok();
}

int dca_debug_tile_regions(int64_t seq, int64_t C, uint8_t *out, void *stream) {
    if (seq < 1 || seq > ((int64_t)1 << 22)) return fail(DCA_E_INVALID, "seq out of range for a region table");
    if (C < kTile || C % kTile != 0) return fail(DCA_E_UNSUPPORTED, "C must be a positive multiple of 64");
    if (out == nullptr) return fail(DCA_E_INVALID, "out is NULL");
    const int err = launch_debug_tile_regions(seq, C, out, stream);
    if (err) return device_fail(err, "tile-region launch");
    return ok();
}

int dca_debug_unpack(const void *workspace, size_t workspace_bytes, int which, int64_t seq, int64_t C, int64_t W,
                     const dca_shape *shape, void *dst, void *stream) {
    Problem p;
    Layout L;
    int st = make_problem(seq, C, W, shape, nullptr, &p);
    if (st) return st;
    if (which < 0 || which > 4) return fail(DCA_E_INVALID, "which must be 0..4");
    if (dst == nullptr) return fail(DCA_E_INVALID, "dst is NULL");
    if ((st = check_workspace(p, workspace, workspace_bytes, &L))) return st;
    const int err = launch_debug_unpack(p, workspace, L, which, dst, stream);
    if (err) return device_fail(err, "unpack launch");
    return ok();
}

int dca_debug_vs_lists(const void *workspace, size_t workspace_bytes, int64_t seq, int64_t C, int64_t W,
                       const dca_vs_mask *mask, const dca_shape *shape, int32_t *vt, int32_t *vt_count,
                       int32_t *dl, int32_t *dl_count, void *stream) {
    Problem p;
    Layout L;
    if (mask == nullptr) return fail(DCA_E_INVALID, "mask is NULL");
    int st = make_problem(seq, C, W, shape, mask, &p);
    if (st) return st;
    if (!vt || !vt_count || !dl || !dl_count) return fail(DCA_E_INVALID, "output arrays must be non-NULL");
    if ((st = check_workspace(p, workspace, workspace_bytes, &L))) return st;
    const int err = launch_debug_vs_lists(p, workspace, L, vt, vt_count, dl, dl_count, stream);
    if (err) return device_fail(err, "list copy launch");
    return ok();
}

int dca_debug_vs_tiles(const void *workspace, size_t workspace_bytes, int64_t seq, int64_t C, int64_t W,
                       const dca_vs_mask *mask, const dca_shape *shape, int32_t head, int64_t q_tile,
                       int32_t group, int32_t *kt_out, uint32_t *mask_out, int32_t cap, int32_t *n_out,
                       void *stream) {
    Problem p;
    Layout L;
    if (mask == nullptr) return fail(DCA_E_INVALID, "mask is NULL");
    int st = make_problem(seq, C, W, shape, mask, &p);
    if (st) return st;
    if (head < 0 || head >= p.Hq) return fail(DCA_E_INVALID, "head out of range");
    if (group != 1 && group != 2) return fail(DCA_E_INVALID, "group must be 1 or 2");
    if (q_tile < 0 || q_tile >= p.n_tiles || q_tile % group != 0)
        return fail(DCA_E_INVALID, "q_tile must be a multiple of group below ceil(seq / 64)");
    if (cap < 1) return fail(DCA_E_INVALID, "cap must be positive");
    if (!kt_out || !mask_out || !n_out) return fail(DCA_E_INVALID, "output arrays must be non-NULL");
    if ((st = check_workspace(p, workspace, workspace_bytes, &L))) return st;
    const int err = launch_debug_vs_tiles(p, workspace, L, head, q_tile, group, kt_out, mask_out, cap, n_out, stream);
    if (err) return device_fail(err, "tile-order launch");
    return ok();
}

}  // extern "C"
