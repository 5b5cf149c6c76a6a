// diffattn_fwd.hip -- differential-attention forward for CDNA4 (gfx950).
//
// The operation is the one defined in include/diffattn.h (DiffTransformer.py,
// MultiHeadDifferentialAttention.forward; LlamaDiffSdpaAttention.py, forward;
// unilm pull request "Add an isolated implementation of FlashDiffAttention").
//
// Kernel design
// -------------
// One workgroup = 4 waves (one per SIMD) = one KV head g, a block of heads of
// that group and a block of query tokens of one packed sequence:
//   G % 4 == 0 : 4 heads  x 32 queries (each wave one head)
//   G % 2 == 0 : 2 heads  x 64 queries
//   otherwise  : 1 head   x 128 queries
// Every wave owns 32 query rows of one head and keeps, for both maps, the
// running row maximum, the running sum and a 32 x 2d fp32 accumulator, so
// the two softmax recurrences are fully independent.  The register budget
// is 256 per lane, so two workgroups share a CU: while one wave of a SIMD
// runs its MFMAs the other runs its softmax.
//
// The workgroup streams the KV range of its sequence in tiles of 64 keys.
// K (both halves) and V of a tile are copied global -> LDS directly
// (global_load_lds, 16 bytes per lane, no registers), row-major with an XOR
// swizzle of the 16-byte chunks, double-buffered: the copy of tile t+1 is in
// flight while tile t is computed; one barrier per tile.  K/V of a GQA group
// enter LDS once per 32..128 query rows and are never copied per head.
//
// All four contractions run on MFMA (v_mfma_f32_32x32x16_bf16 for bf16,
// v_mfma_f32_32x32x2_f32 for fp32), in transposed form:
//   S_m^T [keys x queries] = K_m [keys x d] * Q_m^T      (m = 1, 2)
//   O_m^T [2d  x queries] += V^T [2d x keys] * P_m^T
// With S^T each lane owns one query column and 16 keys of every 32-key
// block: row maxima and sums are in-lane plus one cross-half exchange, and
// the accumulator layout of S^T is directly the B-operand layout of the PV
// product.  V^T operands come from the row-major V tile through the
// transposing LDS read ds_read_b64_tr_b16 (bf16) or plain 4-byte reads
// (fp32).
//
// Softmax uses a lazily updated running maximum: probabilities are taken
// against the stored maximum as long as no score of the tile exceeds it by
// more than 2^8 in probability; only then (in practice on the first tile)
// the maximum, the sums and the accumulators are rescaled.  The result O/l
// does not depend on which maximum was used.
//
// The epilogue is fused: lambda (computed per wave from the four vectors),
// O_1/l_1 - lambda O_2/l_2, the RMSNorm over 2d (in-lane sums plus one
// cross-half exchange), the weight, the (1 - lambda_init) scale and the
// rounding store.  Causal tiles above the diagonal are never visited; on the
// diagonal, 32-key blocks a wave cannot see are skipped and the rest are
// masked by index.  Workgroups are numbered longest-first (largest query
// tile index first) so the causal tail is short.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "diffattn.h"

namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;   // keys per KV tile
constexpr int kQW = 32;   // query rows per wave
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.0f;   // lazy-max threshold, log2 units

// ---------------------------------------------------------------------------
// LDS tile geometry.  A K tile is [64 keys][2d] (K1 then K2 of each key), a
// V tile [64 keys][2d]; both row-major with padded rows so that every
// operand read is a per-lane base plus a compile-time offset and hits
// distinct banks:
//   K rows are ROWB + 16 bytes apart: the 16 rows one 16-lane group reads at
//     one column start 16 bytes apart modulo 256;
//   V rows (bf16) are ROWB + 64 bytes apart: the 4 rows x 64 bytes one
//     half-wave of a transposing read touches tile all 256 bytes of banks.
// The tiles are filled by direct global->LDS copies of 64 lanes x 16 bytes
// (1 KiB contiguous per copy); padding slots receive a harmless duplicate.
template <typename E, int D> struct Geo {
    static constexpr int ES = (int)sizeof(E);
    static constexpr int ROWB = 2 * D * ES;                 // data bytes per row
    static constexpr int CPR = ROWB / 16;                   // data chunks per row
    static constexpr int KROWB = ROWB + 16;
    static constexpr int VROWB = ROWB + (ES == 2 ? 64 : 16);
    static constexpr int KSPR = KROWB / 16;                 // slots per K row
    static constexpr int VSPR = VROWB / 16;
    static constexpr int KTILEB = kBN * KROWB;
    static constexpr int VTILEB = kBN * VROWB;
    static constexpr int KCOPIES = KTILEB / 1024;           // 1 KiB copies
    static constexpr int VCOPIES = VTILEB / 1024;
    static constexpr int STAGEB = KTILEB + VTILEB;
    static constexpr int MAXC = (KCOPIES > VCOPIES ? KCOPIES : VCOPIES);
    static constexpr int CPW = (MAXC + kWaves - 1) / kWaves; // copies per wave
    static_assert(KCOPIES * 1024 == KTILEB && VCOPIES * 1024 == VTILEB, "copy tiling");
};

// ---------------------------------------------------------------------------
// MFMA flavours.  VEC = operand elements per lane; one MFMA contracts 2*VEC.
template <typename E> struct Mfma;

template <> struct Mfma<bf16> {
    static constexpr int VEC = 8;
    typedef bf16x8 Frag;
    __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline Frag pack(const f32x16 &s, int a0)
    {
        Frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            f[e] = (bf16)s[a0 + e];
        return f;
    }
};

template <> struct Mfma<float> {
    static constexpr int VEC = 1;
    typedef float Frag;
    __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ static inline Frag pack(const f32x16 &s, int a0) { return s[a0]; }
};

// Row (key offset inside a 32-key block) of accumulator element a of a lane
// in half h of a 32x32 MFMA result.
__device__ __host__ constexpr int acc_row(int a, int h) { return 8 * (a / 4) + 4 * h + (a % 4); }

// Value of x in the lane 32 apart, and the two combined (lower lane first,
// so both halves compute bitwise the same result).
__device__ inline float pair_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// V^T operand of the PV product for one 16-key step (keys base .. base+15
// of the tile, in MFMA k order) and one 32-dim block.
template <typename E, int D> struct VOperand;

template <int D> struct VOperand<bf16, D> {
    // lane l: group G = l/16, j = l%16; for the transposing read, lane j of
    // the group addresses key row (4*(l/32) + j/4) and dims 4*(j%4)..+3 of
    // the group's 16 dims; the hardware hands lane j dim (16*(G%2) + j) of
    // all four rows.  Two reads (t = 0, 1) give keys 8t + 4h + 0..3 of the
    // 16-key step, i.e. MFMA k = 8h + 4t + e.
    __device__ static inline int lane_base(int lane)
    {
        typedef Geo<bf16, D> G;
        const int j = lane & 15;
        return (4 * (lane >> 5) + (j >> 2)) * G::VROWB + 32 * ((lane >> 4) & 1) + 8 * (j & 3);
    }
    __device__ static inline bf16x8 load(const char *vt, int step_row, int db)
    {
        typedef Geo<bf16, D> G;
        bf16x8 f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const char *addr = vt + (step_row + 8 * t) * G::VROWB + 64 * db;
            const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4 *)addr);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                f[4 * t + e] = x[e];
        }
        return f;
    }
};

template <int D> struct VOperand<float, D> {
    // lane (m = l%32, h = l/32) reads dim 32*db + m of key row step_row + 4h
    __device__ static inline int lane_base(int lane)
    {
        typedef Geo<float, D> G;
        return 4 * (lane >> 5) * G::VROWB + 4 * (lane & 31);
    }
    __device__ static inline float load(const char *vt, int step_row, int db)
    {
        typedef Geo<float, D> G;
        return *(const float *)(vt + step_row * G::VROWB + 128 * db);
    }
};

struct Params {
    const void *q;
    const void *k;
    const void *v;
    void *out;
    const float *lq1, *lk1, *lq2, *lk2;
    const float *w;
    const int32_t *cu;
    float lambda_init;
    float eps;
    int32_t T, H, Hkv, nseq, seqlen_uniform;
    int32_t causal;
    int32_t ntile_q;   // query tiles per sequence (of the longest one)
    int32_t hpw;       // heads per workgroup (1, 2 or 4)
    int32_t hblocks;   // head blocks per KV group: G / hpw
};

// Waves per SIMD the register budget is cut for: two (two workgroups per CU)
// wherever the double-buffered tiles leave room for a second workgroup in LDS.
template <typename E, int D> struct Occupancy {
    static constexpr int value = 2 * Geo<E, D>::STAGEB * 2 <= 160 * 1024 ? 2 : 1;
};

template <typename E, int D>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(Occupancy<E, D>::value, Occupancy<E, D>::value)))
void diffattn_fwd_kernel(Params p)
{
    typedef Geo<E, D> GEO;
    typedef Mfma<E> M;
    typedef typename M::Frag Frag;
    constexpr int VEC = M::VEC;
    constexpr int KSTEP = 2 * VEC;      // contraction depth of one MFMA
    constexpr int NKS = D / KSTEP;      // MFMAs per 32x32 score block
    constexpr int NDB = 2 * D / 32;     // 32-wide blocks of the output
    constexpr int NPS = 32 / KSTEP;     // PV steps per 32-key block
    static_assert(D % KSTEP == 0 && (2 * D) % 32 == 0, "unsupported d");

    __shared__ __attribute__((aligned(1024))) char smem[2 * GEO::STAGEB];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int n = lane & 31;   // query column owned by this lane
    const int h = lane >> 5;   // lane half

    // ---- tile scheduler: longest query tiles first ------------------------
    const int pairs = p.nseq * p.Hkv * p.hblocks;
    const int id = blockIdx.x;
    const int t = p.ntile_q - 1 - id / pairs;
    const int rem = id % pairs;
    const int seq = rem / (p.Hkv * p.hblocks);
    const int grp = rem % (p.Hkv * p.hblocks);
    const int g = grp / p.hblocks;
    const int hb = grp % p.hblocks;

    int s0, s1;
    if (p.cu) {
        s0 = p.cu[seq];
        s1 = p.cu[seq + 1];
    } else {
        s0 = seq * p.seqlen_uniform;
        s1 = s0 + p.seqlen_uniform;
    }
    const int qpw = kWaves / p.hpw;     // query blocks per workgroup
    const int bm = kQW * qpw;           // query rows per workgroup
    const int q0 = s0 + t * bm;
    if (q0 >= s1)
        return;
    const int qhi = min(s1, q0 + bm);

    const int head = g * (p.H / p.Hkv) + hb * p.hpw + wave / qpw;
    const int wq0 = q0 + (wave % qpw) * kQW;   // first query row of this wave
    const int wq_last = min(wq0 + kQW, s1) - 1;
    const int tq = wq0 + n;                    // this lane's query token

    const E *__restrict__ qg = (const E *)p.q;

    // ---- lambda (every wave computes the same scalar) ---------------------
    float lam;
    {
        float a = 0.f, b = 0.f;
        for (int c = lane; c < D; c += 64) {
            a += p.lq1[c] * p.lk1[c];
            b += p.lq2[c] * p.lk2[c];
        }
#pragma unroll
        for (int off = 32; off >= 1; off /= 2) {
            a += __shfl_xor(a, off, 64);
            b += __shfl_xor(b, off, 64);
        }
        lam = expf(a) - expf(b) + p.lambda_init;
    }

    // ---- Q fragments (B operand of S^T = K Q^T), kept in registers --------
    Frag qf[2][NKS];
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if (tq < s1) {
                const E *src = qg + (((int64_t)tq * p.H + head) * 2 + mp) * D + ks * KSTEP + h * VEC;
                qf[mp][ks] = *(const Frag *)src;
            } else {
                qf[mp][ks] = Frag{};
            }
        }

    // ---- KV tile copies: per-lane source offsets (bytes) -------------------
    // Copy i fills LDS slots [64 i, 64 i + 64) of 16 bytes of a tile; slot s
    // holds chunk s % SPR of row s / SPR (chunks past the row's data are
    // padding and get chunk 0 again).  Wave w issues copies w, w + 4, ...
    const int rowstride = p.Hkv * GEO::ROWB;   // bytes between keys
    // slot -> (row, byte offset inside the row's data); padding slots take
    // chunk 0 of their row
    auto slot_row = [&](int slot, int spr) { return slot / spr; };
    auto slot_col = [&](int slot, int spr) {
        const int ch = slot % spr;
        return (ch < GEO::CPR ? ch : 0) * 16 + g * GEO::ROWB;
    };
    int kc_off[GEO::CPW], vc_off[GEO::CPW];   // source offsets of full tiles
#pragma unroll
    for (int j = 0; j < GEO::CPW; ++j) {
        const int slot = (wave + kWaves * j) * 64 + lane;
        kc_off[j] = slot_row(slot, GEO::KSPR) * rowstride + slot_col(slot, GEO::KSPR);
        vc_off[j] = slot_row(slot, GEO::VSPR) * rowstride + slot_col(slot, GEO::VSPR);
    }
    const char *kbytes = (const char *)p.k;
    const char *vbytes = (const char *)p.v;
    auto issue_copy = [&](int k0, char *stage) {
        // rows past the end of the sequence are clamped to its last row
        const bool tail = k0 + kBN > s1;
        const char *kb = kbytes + (int64_t)k0 * rowstride;
        const char *vb = vbytes + (int64_t)k0 * rowstride;
#pragma unroll
        for (int j = 0; j < GEO::CPW; ++j) {
            const int i = wave + kWaves * j;
            const int slot = i * 64 + lane;
            if (i < GEO::KCOPIES) {
                int off = kc_off[j];
                if (tail)
                    off = min(slot_row(slot, GEO::KSPR), s1 - 1 - k0) * rowstride +
                          slot_col(slot, GEO::KSPR);
                __builtin_amdgcn_global_load_lds((gbl_void *)(kb + off),
                                                 (lds_void *)(stage + 1024 * i), 16, 0, 0);
            }
            if (i < GEO::VCOPIES) {
                int off = vc_off[j];
                if (tail)
                    off = min(slot_row(slot, GEO::VSPR), s1 - 1 - k0) * rowstride +
                          slot_col(slot, GEO::VSPR);
                __builtin_amdgcn_global_load_lds((gbl_void *)(vb + off),
                                                 (lds_void *)(stage + GEO::KTILEB + 1024 * i),
                                                 16, 0, 0);
            }
        }
    };
    const int k_lane = n * GEO::KROWB + h * VEC * (int)sizeof(E);
    const int v_lane = VOperand<E, D>::lane_base(lane);

    // ---- running state ----------------------------------------------------
    const float c = kLog2e / sqrtf((float)D);   // softmax scale in log2 units
    float m_run[2] = {-INFINITY, -INFINITY};    // raw-score units
    float l_run[2] = {0.f, 0.f};                // this lane's partial sums
    f32x16 o[2][NDB];
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            o[mp][db] = f32x16{};

    const int kv_end = p.causal ? qhi : s1;
    const int ntiles = (kv_end - s0 + kBN - 1) / kBN;

    issue_copy(s0, smem);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int k0 = s0 + it * kBN;
        const char *kt = smem + (it & 1) * GEO::STAGEB + k_lane;
        const char *vt = smem + (it & 1) * GEO::STAGEB + GEO::KTILEB + v_lane;
        if (it + 1 < ntiles)
            issue_copy(k0 + kBN, smem + ((it + 1) & 1) * GEO::STAGEB);

        // The tile is consumed one 32-key block at a time: both maps' scores
        // of the block, their softmax update, then both PV products sharing
        // each V operand read.
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int kb0 = k0 + 32 * b;
            // wave-uniform: can this wave see any key of the block, and does
            // any key need the index mask?
            if (kb0 >= s1 || (p.causal && kb0 > wq_last))
                continue;
            const bool masked = kb0 + 32 > s1 || (p.causal && kb0 + 31 > wq0);

            // ---- S^T = K Q^T for both maps -------------------------------
            f32x16 s[2];
#pragma unroll
            for (int mp = 0; mp < 2; ++mp) {
                s[mp] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int off = 32 * b * GEO::KROWB + (mp * D + ks * KSTEP) * (int)sizeof(E);
                    const Frag a = *(const Frag *)(kt + off);
                    s[mp] = M::mma(a, qf[mp][ks], s[mp]);
                }
            }

            if (masked) {
#pragma unroll
                for (int a = 0; a < 16; ++a) {
                    const int key = kb0 + acc_row(a, h);
                    if (key >= s1 || (p.causal && key > tq)) {
                        s[0][a] = -INFINITY;
                        s[1][a] = -INFINITY;
                    }
                }
            }

            // ---- two independent online-softmax updates (lazy maximum) ----
#pragma unroll
            for (int mp = 0; mp < 2; ++mp) {
                float pm = -INFINITY;
#pragma unroll
                for (int a = 0; a < 16; ++a)
                    pm = fmaxf(pm, s[mp][a]);
                const bool grow = (pm - m_run[mp]) * c > kRescaleLog2;
                if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                    const float mold = m_run[mp];
                    const float mnew = fmaxf(mold, pair_max(pm));
                    float alpha;
                    if (mold == -INFINITY)
                        alpha = 0.f;          // nothing accumulated yet
                    else
                        alpha = __builtin_amdgcn_exp2f((mold - mnew) * c);
                    m_run[mp] = mnew;
                    l_run[mp] *= alpha;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        o[mp][db] *= alpha;
                }
                // every row has a visible key in its first block, so m_run is
                // finite from here on
                const float mc = m_run[mp] * c;
                float rs = 0.f;
#pragma unroll
                for (int a = 0; a < 16; ++a) {
                    const float pv = __builtin_amdgcn_exp2f(fmaf(s[mp][a], c, -mc));
                    s[mp][a] = pv;
                    rs += pv;
                }
                l_run[mp] += rs;
            }

            // ---- O^T += V^T P^T ------------------------------------------
#pragma unroll
            for (int ps = 0; ps < NPS; ++ps) {
                const Frag p1 = M::pack(s[0], ps * VEC);
                const Frag p2 = M::pack(s[1], ps * VEC);
                // first key row of this step (the lane part is in v_lane)
                const int row = VEC == 8 ? 32 * b + 16 * ps
                                         : 32 * b + 8 * (ps / 4) + (ps % 4);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const Frag vf = VOperand<E, D>::load(vt, row, db);
                    o[0][db] = M::mma(vf, p1, o[0][db]);
                    o[1][db] = M::mma(vf, p2, o[1][db]);
                }
            }
        }

        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- epilogue: combine, RMSNorm, scale, store --------------------------
    const float l1 = pair_sum(l_run[0]);
    const float l2 = pair_sum(l_run[1]);
    const float i1 = 1.f / l1;
    const float i2 = lam / l2;
    float ss = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
            const float pre = o[0][db][a] * i1 - o[1][db][a] * i2;
            o[0][db][a] = pre;
            ss += pre * pre;
        }
    ss = pair_sum(ss);
    const float r = (1.f - p.lambda_init) / sqrtf(ss / (float)(2 * D) + p.eps);
    if (tq < s1) {
        E *dst = (E *)p.out + ((int64_t)tq * p.H + head) * (2 * D);
        // weight: one wave-uniform branch, not one per element
        float wv[NDB][16];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int a = 0; a < 16; ++a)
                wv[db][a] = r;
        if (p.w) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 w4 = *(const float4 *)(p.w + 32 * db + 8 * i + 4 * h);
                    wv[db][4 * i + 0] *= w4.x;
                    wv[db][4 * i + 1] *= w4.y;
                    wv[db][4 * i + 2] *= w4.z;
                    wv[db][4 * i + 3] *= w4.w;
                }
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int dim = 32 * db + 8 * i + 4 * h;
                E vals[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    vals[j] = (E)(o[0][db][4 * i + j] * wv[db][4 * i + j]);
                __builtin_memcpy(dst + dim, vals, sizeof(vals));
            }
    }
}

template <typename E, int D>
int launch(const Params &p, int nblocks, hipStream_t stream)
{
    hipLaunchKernelGGL((diffattn_fwd_kernel<E, D>), dim3(nblocks), dim3(kThreads), 0,
                       stream, p);
    return hipGetLastError() == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}

typedef int (*launch_fn)(const Params &, int, hipStream_t);

launch_fn find_launcher(int dtype, int d)
{
    if (dtype == DIFFATTN_BF16) {
        if (d == 64) return launch<bf16, 64>;
        if (d == 32) return launch<bf16, 32>;
        if (d == 16) return launch<bf16, 16>;
    } else if (dtype == DIFFATTN_F32) {
        if (d == 64) return launch<float, 64>;
        if (d == 16) return launch<float, 16>;
    }
    return nullptr;
}

} // namespace

extern "C" {

int diffattn_abi_version(void) { return DIFFATTN_ABI_VERSION; }

const char *diffattn_strerror(int status)
{
    switch (status) {
    case DIFFATTN_OK: return "success";
    case DIFFATTN_EINVAL: return "invalid argument";
    case DIFFATTN_EUNSUPPORTED: return "unsupported (dtype, d) combination";
    case DIFFATTN_EHIP: return "HIP runtime error (no device or launch failure)";
    default: return "unknown status";
    }
}

double diffattn_lambda_init(int depth) { return 0.8 - 0.6 * exp(-0.3 * (double)(depth - 1)); }

int diffattn_supported(int dtype, int d) { return find_launcher(dtype, d) != nullptr; }

int diffattn_check_cu_seqlens(const int32_t *host_cu, int32_t nseq, int32_t T,
                              int32_t max_seqlen)
{
    if (!host_cu || nseq < 0 || T < 0)
        return DIFFATTN_EINVAL;
    if (host_cu[0] != 0 || host_cu[nseq] != T)
        return DIFFATTN_EINVAL;
    for (int32_t s = 0; s < nseq; ++s) {
        const int64_t len = (int64_t)host_cu[s + 1] - host_cu[s];
        if (len < 0 || len > max_seqlen)
            return DIFFATTN_EINVAL;
    }
    return DIFFATTN_OK;
}

int diffattn_fwd(int dtype, const void *q, const void *k, const void *v,
                 const float *lambda_q1, const float *lambda_k1,
                 const float *lambda_q2, const float *lambda_k2,
                 float lambda_init, const float *subln_weight, float eps,
                 int causal, const int32_t *cu_seqlens, int32_t nseq,
                 int32_t max_seqlen, int32_t T, int32_t H, int32_t Hkv,
                 int32_t d, void *out, void *stream)
{
    if (dtype != DIFFATTN_BF16 && dtype != DIFFATTN_F32)
        return DIFFATTN_EINVAL;
    if (T < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || d < 1)
        return DIFFATTN_EINVAL;
    if (causal != 0 && causal != 1)
        return DIFFATTN_EINVAL;
    if (!(eps >= 0.f) || isinf(eps) || !isfinite(lambda_init))
        return DIFFATTN_EINVAL;
    const launch_fn fn = find_launcher(dtype, d);
    if (!fn)
        return DIFFATTN_EUNSUPPORTED;
    if (T == 0)
        return DIFFATTN_OK;
    if (!q || !k || !v || !out || !lambda_q1 || !lambda_k1 || !lambda_q2 || !lambda_k2)
        return DIFFATTN_EINVAL;
    // q, k, v and out are read and written in 16-byte vectors
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out |
         (uintptr_t)subln_weight) % 16 != 0)
        return DIFFATTN_EINVAL;
    if (nseq < 1)
        return DIFFATTN_EINVAL;
    int32_t uniform = 0;
    if (!cu_seqlens) {
        if (T % nseq != 0)
            return DIFFATTN_EINVAL;
        uniform = T / nseq;
        if (max_seqlen <= 0)
            max_seqlen = uniform;
        if (max_seqlen != uniform)
            return DIFFATTN_EINVAL;
    } else if (max_seqlen < 1 || max_seqlen > T) {
        return DIFFATTN_EINVAL;
    }
    // byte offsets of K/V rows are formed in 64 bits; the grid in 32 bits
    const int G = H / Hkv;
    const int hpw = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);
    const int bm = kQW * (kWaves / hpw);
    const int64_t ntile_q = ((int64_t)max_seqlen + bm - 1) / bm;
    const int64_t nblocks = ntile_q * nseq * Hkv * (G / hpw);
    if (nblocks > INT32_MAX)
        return DIFFATTN_EINVAL;

    Params p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.lq1 = lambda_q1;
    p.lk1 = lambda_k1;
    p.lq2 = lambda_q2;
    p.lk2 = lambda_k2;
    p.w = subln_weight;
    p.cu = cu_seqlens;
    p.lambda_init = lambda_init;
    p.eps = eps;
    p.T = T;
    p.H = H;
    p.Hkv = Hkv;
    p.nseq = nseq;
    p.seqlen_uniform = uniform;
    p.causal = causal;
    p.ntile_q = (int32_t)ntile_q;
    p.hpw = hpw;
    p.hblocks = G / hpw;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return DIFFATTN_EHIP;
    return fn(p, (int)nblocks, (hipStream_t)stream);
}

} // extern "C"
