// rope.h -- the rotary prologue's arithmetic, shared by the prefill
// (diffattn_fwd.hip), the cache path and its append kernel
// (diffattn_kv.hip).  Internal to the library.
//
// The rotation is the one the FlashDiffAttention pull request's test applies
// (apply_rotary_emb with interleaved=True on every d-wide half-head of q and
// k): the pair (x[2j], x[2j+1]) of a row at position p becomes
// (x0 c - x1 s, x0 s + x1 c) with c = cos[p, j], s = sin[p, j].  The tables
// are [len, d/2], fp32 or bf16 (the pull request caches them in bf16); a
// bf16 entry is widened to fp32 exactly, so both kinds rotate the same way
// given the same values.  The arithmetic is fp32, rounded once to the
// storage type.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diffattn_rope {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Table kinds, a template argument of the kernels that rotate: no tables,
// fp32 tables, bf16 tables.
enum { kOff = 0, kF32 = 1, kBF16 = 2 };

// N consecutive entries of a table row (N = 2 or 4; the offset is a
// multiple of N, so the load is N entries wide and aligned).
template <int RT, int N> struct Entries;
template <> struct Entries<kF32, 4> {
    __device__ static inline float4 load(const void *t, int64_t o)
    {
        return *((const float4 *)t + o / 4);
    }
};
template <> struct Entries<kF32, 2> {
    __device__ static inline float2 load(const void *t, int64_t o)
    {
        return *((const float2 *)t + o / 2);
    }
};
template <> struct Entries<kBF16, 4> {
    __device__ static inline float4 load(const void *t, int64_t o)
    {
        const bf16x4 v = *((const bf16x4 *)t + o / 4);
        return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
    }
};
template <> struct Entries<kBF16, 2> {
    __device__ static inline float2 load(const void *t, int64_t o)
    {
        const bf16x2 v = *((const bf16x2 *)t + o / 2);
        return make_float2((float)v[0], (float)v[1]);
    }
};

// Rotation of one 16-byte chunk of a half-head row: 8 bf16 values (pairs
// j .. j+3) or 4 fp32 values (pairs j, j+1).
template <typename E, int RT> struct Rope;

template <int RT> struct Rope<bf16, RT> {
    struct Coef { float4 c, s; };
    __device__ static inline Coef coef(const void *rc, const void *rs, int pos, int j, int D)
    {
        const int64_t o = (int64_t)pos * (D / 2) + j;
        return Coef{Entries<RT, 4>::load(rc, o), Entries<RT, 4>::load(rs, o)};
    }
    __device__ static inline u32x4 rotate(u32x4 x, const Coef &k)
    {
        const bf16x8 v = __builtin_bit_cast(bf16x8, x);
        const float cc[4] = {k.c.x, k.c.y, k.c.z, k.c.w};
        const float ss[4] = {k.s.x, k.s.y, k.s.z, k.s.w};
        bf16x8 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x0 = (float)v[2 * i], x1 = (float)v[2 * i + 1];
            r[2 * i] = (bf16)(x0 * cc[i] - x1 * ss[i]);
            r[2 * i + 1] = (bf16)(x0 * ss[i] + x1 * cc[i]);
        }
        return __builtin_bit_cast(u32x4, r);
    }
};

template <int RT> struct Rope<float, RT> {
    struct Coef { float2 c, s; };
    __device__ static inline Coef coef(const void *rc, const void *rs, int pos, int j, int D)
    {
        const int64_t o = (int64_t)pos * (D / 2) + j;
        return Coef{Entries<RT, 2>::load(rc, o), Entries<RT, 2>::load(rs, o)};
    }
    __device__ static inline u32x4 rotate(u32x4 x, const Coef &k)
    {
        const float4 v = __builtin_bit_cast(float4, x);
        float4 r;
        r.x = v.x * k.c.x - v.y * k.s.x;
        r.y = v.x * k.s.x + v.y * k.c.x;
        r.z = v.z * k.c.y - v.w * k.s.y;
        r.w = v.z * k.s.y + v.w * k.c.y;
        return __builtin_bit_cast(u32x4, r);
    }
    // one element (dim d0 = 2j + half) of a row, rotated: the lane reads
    // both elements of its pair
    __device__ static inline float element(const float *row, int d0, int half, const void *rc,
                                           const void *rs, int pos, int D)
    {
        const float2 x = *(const float2 *)(row + (d0 & ~1));
        const int64_t o = (int64_t)pos * (D / 2) + d0 / 2;
        float c, sn;
        if constexpr (RT == kBF16) {
            c = (float)((const bf16 *)rc)[o];
            sn = (float)((const bf16 *)rs)[o];
        } else {
            c = ((const float *)rc)[o];
            sn = ((const float *)rs)[o];
        }
        return half ? x.x * sn + x.y * c : x.x * c - x.y * sn;
    }
};

} // namespace diffattn_rope
