// 16-byte per-lane operand fragments and the gfx950 matrix-core ops that
// consume them (see the layout notes in dca_internal.h).
#pragma once

#include <hip/hip_runtime.h>

namespace dca {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T>
struct Frag;

// bf16: one v_mfma_f32_32x32x16_bf16 per fragment (8 contraction slots/lane).
template <>
struct Frag<__bf16> {
    static constexpr int E = 8;
    using vec = bf16x8;
    __device__ __host__ static inline vec zero() { return vec{}; }
    __device__ static inline __bf16 get(const vec &v, int e) { return v[e]; }
    __device__ static inline void set(vec &v, int e, __bf16 x) { v[e] = x; }
    __device__ static inline __bf16 from_float(float x) { return (__bf16)x; }
    // c += A(32 x 16) * B(16 x 32)
    __device__ static inline void mma(const vec &a, const vec &b, f32x16 &c) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // c0 + A * B as a new value (c0 stays live)
    __device__ static inline f32x16 mma_from(const vec &a, const vec &b, const f32x16 &c0) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    }
    // acc + sum of the 8 elements (two-element dot products with ones)
    __device__ static inline float sum_into(const vec &v, float acc) {
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x2 pr = {v[2 * i], v[2 * i + 1]};
            acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
        }
        return acc;
    }
};

// f32: four v_mfma_f32_32x32x2_f32 per fragment; op t takes element t of
// every lane (contraction slot g of op t is element t of lane group g).
template <>
struct Frag<float> {
    static constexpr int E = 4;
    using vec = f32x4;
    __device__ __host__ static inline vec zero() { return vec{}; }
    __device__ static inline float get(const vec &v, int e) { return v[e]; }
    __device__ static inline void set(vec &v, int e, float x) { v[e] = x; }
    __device__ static inline float from_float(float x) { return x; }
    __device__ static inline void mma(const vec &a, const vec &b, f32x16 &c) {
#pragma unroll
        for (int t = 0; t < 4; ++t) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], b[t], c, 0, 0, 0);
    }
    __device__ static inline f32x16 mma_from(const vec &a, const vec &b, const f32x16 &c0) {
        f32x16 c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c0, 0, 0, 0);
#pragma unroll
        for (int t = 1; t < 4; ++t) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], b[t], c, 0, 0, 0);
        return c;
    }
    __device__ static inline float sum_into(const vec &v, float acc) { return acc + ((v[0] + v[1]) + (v[2] + v[3])); }
};

}  // namespace dca
