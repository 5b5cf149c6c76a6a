// diffattn_fwd.hip -- differential-attention forward for CDNA4 (gfx950).
//
// The operation is the one defined in include/diffattn.h (DiffTransformer.py,
// MultiHeadDifferentialAttention.forward; LlamaDiffSdpaAttention.py, forward;
// unilm pull request "Add an isolated implementation of FlashDiffAttention").
//
// Kernel design
// -------------
// One workgroup = 8 waves = one KV head g, a block of heads of that group
// and a block of query tokens of one packed sequence.  The four "slots" of
// a workgroup are (head, 64 queries) pairs:
//   G % 4 == 0 : 4 heads  x  64 queries
//   G % 2 == 0 : 2 heads  x 128 queries
//   otherwise  : 1 head   x 256 queries
// and every slot is served by two waves, one per attention map: wave w
// computes map (w / 4) of slot (w % 4) for its 64 queries, as two 32-query
// sub-blocks.  (Grids that would leave fewer than two workgroups per CU run
// an instantiation with one 32-query sub-block per wave, so twice the
// workgroups share the work; everything below then holds with 32 queries
// per slot.)  Each K operand read and each V operand read of a wave feeds
// two MFMAs (one per sub-block), and each K/V tile staged in LDS serves 256
// query rows of the GQA group, which keeps LDS traffic per MFMA low (the
// transposing V read runs at half the LDS read rate, 16-byte LDS writes at a
// third of it).  A wave keeps, per sub-block, one running row maximum, one
// running sum and a 32 x 2d fp32 accumulator of its map; the combine
// O_1/l_1 - lambda O_2/l_2 happens once, in the epilogue, through LDS.  Two
// waves per SIMD (256 registers each, waves s and s + 4: the two maps of a
// slot) interleave their MFMA and softmax phases; the map-2 wave runs each
// block's PV product at the start of the next block, which keeps the pair
// about half a block apart.
//
// The workgroup streams the KV range of its sequence in tiles of 128 keys
// (64 where two stages of 128 would not fit LDS).  K (both halves) and V of
// a tile are staged into padded row-major LDS tiles, double-buffered: tile
// t+1 moves global -> registers -> LDS in slices, one per 32-key block of
// tile t, so its loads are in flight while tile t is computed; two barriers
// per tile (after its first block, for the late PV of the map-2 waves, and
// at its end).  (Direct global -> LDS copies were measured slower on this
// part: their transfer path costs more than 16-byte LDS writes.)
//
// All contractions run on MFMA (v_mfma_f32_32x32x16_bf16 for bf16,
// v_mfma_f32_32x32x2_f32 for fp32), in transposed form:
//   S_m^T [keys x queries] = K_m [keys x d] * Q_m^T
//   O_m^T [2d  x queries] += V^T [2d x keys] * P_m^T
// With S^T each lane owns one query column and 16 keys of every 32-key
// block: row maxima and sums are in-lane plus one cross-half exchange, and
// the accumulator layout of S^T is directly the B-operand layout of the PV
// product.  V^T operands come from the row-major V tile through the
// transposing LDS read ds_read_b64_tr_b16 (bf16) or plain 4-byte reads
// (fp32).
//
// Softmax uses a lazily updated running maximum: probabilities are taken
// against the stored maximum as long as none of the block exceeds 2^8; only
// then (in practice on the first block) the maximum, the sum and the
// accumulator are rescaled.  The result O/l does not depend on which maximum
// was used.  For bf16 the block's probabilities are computed first and their
// sum serves both as the row-sum update and as the test: every probability
// is at most the sum, so no per-block row maximum is needed on the common
// path.
//
// The epilogue is fused: lambda (from the four vectors), O_1/l_1 -
// lambda O_2/l_2, the RMSNorm over 2d (in-lane sums plus one cross-half
// exchange), the weight, the (1 - lambda_init) scale and the rounding
// store.  The two waves of a slot share it, one 32-query sub-block each,
// and bf16 rows leave through LDS as whole 256-byte rows.
//
// Causal tiles above the diagonal are never visited; on the diagonal,
// 32-key blocks a wave cannot see are skipped and the rest are masked by
// index.  Workgroups are numbered longest-first (largest query tile index
// first) so the causal tail is short; for packed sequences of mixed
// lengths the grid lists only the tiles that exist, in that order, each
// workgroup finding its tile from cu_seqlens in its prologue.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <math.h>
#include <stdint.h>

#include "chunk.h"
#include "diffattn.h"
#include "rope.h"
#include "splits.h"

namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;    // two maps x four slots
constexpr int kCUs = 256;    // compute units of the part
constexpr float kUnseen = 1e30f;   // floor of a key split's running maximum
constexpr int kSlots = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.0f;   // lazy-max threshold, log2 units
constexpr float kRescaleSum = 256.0f;  // the same threshold as a probability

// ---------------------------------------------------------------------------
// LDS tile geometry.  A K tile is [64 keys][2d] (K1 then K2 of each key), a
// V tile [64 keys][2d]; both row-major with padded rows so that every
// operand read is a per-lane base plus a compile-time offset and hits
// distinct banks:
//   K rows are ROWB + 16 bytes apart: the 16 rows one 16-lane group reads at
//     one column start 16 bytes apart modulo 256;
//   V rows (bf16) are ROWB + 64 bytes apart: the 4 rows x 64 bytes one
//     half-wave of a transposing read touches tile all 256 bytes of banks.
// The tiles are filled through registers (16-byte global loads, 16-byte LDS
// writes), so the padding is never transferred.
template <typename E, int D> struct Geo {
    static constexpr int ES = (int)sizeof(E);
    static constexpr int ROWB = 2 * D * ES;                 // data bytes per row
    static constexpr int CPR = ROWB / 16;                   // data chunks per row
    static constexpr int KROWB = ROWB + 16;
    static constexpr int VROWB = ROWB + (ES == 2 ? 64 : 16);
    // keys per tile: 128 when two stages of that size fit the 160 KiB LDS
    static constexpr int BN = 2 * 128 * (KROWB + VROWB) <= 160 * 1024 ? 128 : 64;
    static constexpr int NB = BN / 32;                      // 32-key blocks per tile
    static constexpr int KTILEB = BN * KROWB;
    static constexpr int VTILEB = BN * VROWB;
    static constexpr int STAGEB = KTILEB + VTILEB;          // K tile, then V tile
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
    __device__ static inline Frag pack(const float *s, int a0)
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
    __device__ static inline Frag pack(const float *s, int a0) { return s[a0]; }
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

// ---------------------------------------------------------------------------
// Rotary prologue (the pull request's apply_rotary_emb with interleaved=True
// on every d-wide half-head): the pair (x[2j], x[2j+1]) of a row at
// sequence position pos becomes (x0 c - x1 s, x0 s + x1 c) with c, s the
// table entries at row pos, column j.  Tables are fp32 [len][d/2]; the
// rotation runs in fp32 and rounds once to the storage type.  A 16-byte
// chunk of a row holds whole pairs (4 for bf16, 2 for fp32).  K is rotated
// once per call into the caller's workspace (every query tile of a group
// reads each K row, so rotating it while staging would repeat the work
// per tile); Q fragments are rotated when each wave loads them.
using diffattn_rope::Rope;

// Rotates every K row once, into a copy.  Thread = one 16-byte chunk
// position (whole pairs) of one token, taken through all 2 Hkv half-heads
// of that token: the coefficients depend only on the position and the pair
// index, so each thread reads them once and keeps up to eight chunk loads
// in flight.  The token's position is its offset in its sequence, found by
// binary search over cu_seqlens.  The prefill kernel then stages the
// rotated copy.
template <typename E, int D, int RT>
__global__ __launch_bounds__(256) void rope_rotate_k(const char *k, char *kr, const int32_t *cu,
                                                     int32_t nseq, int32_t uniform, int32_t T,
                                                     int32_t Hkv, const void *rc, const void *rs)
{
    constexpr int HB = D * (int)sizeof(E);   // bytes per d-wide half-head
    constexpr int CPH = HB / 16;             // chunks per half-head
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int t = (int)(idx / CPH);
    if (t >= T)
        return;
    int s0;
    if (cu) {
        int lo = 0, hi = nseq;   // last sequence with cu[s] <= t
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (cu[mid] <= t)
                lo = mid;
            else
                hi = mid;
        }
        s0 = cu[lo];
    } else {
        s0 = (t / uniform) * uniform;
    }
    const int c = (int)(idx % CPH);
    // pair index of the chunk's first element within its half-head
    const int j = c * (16 / (int)sizeof(E)) / 2;
    const auto coef = Rope<E, RT>::coef(rc, rs, t - s0, j, D);
    const int nh = 2 * Hkv;
    const int64_t base = (int64_t)t * nh * HB + c * 16;
    for (int h0 = 0; h0 < nh; h0 += 8) {
        u32x4 x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (h0 + i < nh)
                x[i] = *(const u32x4 *)(k + base + (int64_t)(h0 + i) * HB);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (h0 + i < nh)
                *(u32x4 *)(kr + base + (int64_t)(h0 + i) * HB) = Rope<E, RT>::rotate(x[i], coef);
    }
}

struct Params {
    const void *q;
    const void *k;
    const void *v;
    void *out;
    const float *lq1, *lk1, *lq2, *lk2;
    int64_t lstride;   // elements between heads' lambda vectors (0: shared)
    const float *w;
    const int32_t *cu;
    // query chunks against a longer key range (the CHUNK instantiation):
    // the keys' own boundaries, or NULL with klen_uniform keys per sequence
    const int32_t *cuk;
    int32_t klen_uniform;
    // key splits of a chunk (ck > 0): the grid's first index runs over
    // nslots split slots (sequence s owns ceil(nk_s / ck) consecutive ones),
    // and each workgroup writes its rows' partial (maximum in log2 units,
    // sum, unnormalised O) per map to ws_ml [slot][Hkv][rmax][4] and ws_o
    // [slot][Hkv][rmax][2][2d] for a merge kernel, row r = i G + gh
    float *ws_o, *ws_ml;
    int32_t ck, nslots, rmax;
    const void *rcos, *rsin;    // rotary tables [len][d/2] (fp32 or bf16), or NULL
    int32_t rope_dtype;         // element type of the tables
    const void *k_orig;         // unrotated K when rcos is set (k is then its rotated copy)
    int32_t max_seqlen;
    float *lse;                 // training forward: [T][H][2] log2-sum-exp, or NULL
    float *o12;                 // training forward: [T][H][2][2d] normalised O_m
    float lambda_init;
    float eps;
    int32_t T, H, Hkv, nseq, seqlen_uniform;
    int32_t causal;
    int32_t ntile_q;   // query tiles per sequence (of the longest one)
    int32_t hpw;       // heads per workgroup (1, 2 or 4)
    int32_t hblocks;   // head blocks per KV group: G / hpw
    int32_t sub;       // 32-query sub-blocks per wave (the kernel's SUB)
    // packed sequences (cu given, nseq <= 64): the grid is the compact list
    // of the tiles that exist, level t = ntile_q - 1 down to 0, found by
    // each workgroup from cu; 0: the padded grid of ntile_q tiles for
    // every sequence
    int32_t compact;
};

// Every CU runs one workgroup of 8 waves (two per SIMD); the register
// budget per lane is the 256 that two waves per SIMD leave.  SUB: 32-query
// sub-blocks per wave -- 2 (each K/V operand read feeds two MFMAs), or 1 for
// grids too small to fill the chip, which doubles the workgroups.  CHUNK:
// each sequence's queries are the last nq of its nk keys (a chunk of new
// queries against a key/value cache that already holds their keys, aligned
// bottom-right as in the cache path), packed by their own boundaries; the
// keys are used as given (a rotary chunk turns only its queries).
template <typename E, int D, int RT, int SUB, bool CHUNK = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void diffattn_fwd_kernel(Params p)
{
    constexpr int kSub = SUB;
    constexpr int kQB = 32 * kSub;   // query rows per slot
    static_assert(SUB == 1 || SUB == 2, "one or two sub-blocks per wave");
    constexpr bool ROPE = RT != diffattn_rope::kOff;   // rotary tables given
    typedef Geo<E, D> GEO;
    typedef Mfma<E> M;
    typedef typename M::Frag Frag;
    constexpr int VEC = M::VEC;
    constexpr int KSTEP = 2 * VEC;      // contraction depth of one MFMA
    constexpr int NKS = D / KSTEP;      // MFMAs per 32x32 score block
    constexpr int NDB = 2 * D / 32;     // 32-wide blocks of the output
    constexpr int NPS = 32 / KSTEP;     // PV steps per 32-key block
    static_assert(D % KSTEP == 0 && (2 * D) % 32 == 0, "unsupported d");
    // epilogue exchange: two slots per stage object, kSub x NDB x 16 x 64
    // floats each
    constexpr int XCH = kSub * NDB * 16 * 64;
    static_assert(2 * XCH * 4 <= GEO::STAGEB, "exchange must fit a stage");

    // two distinct LDS objects for the two stages, so the compiler can see
    // that reads of one never alias writes into the other
    __shared__ __attribute__((aligned(1024))) char stage0[GEO::STAGEB];
    __shared__ __attribute__((aligned(1024))) char stage1[GEO::STAGEB];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lane = tid & 63;
    const int n = lane & 31;           // query column owned by this lane
    const int h = lane >> 5;           // lane half
    const int slot = wave % kSlots;    // (head, query block) served
    const int map = wave / kSlots;     // 0: map 1 (Q1, K1), 1: map 2 (Q2, K2)

    // ---- tile scheduler: longest query tiles first ------------------------
    // (units: sequences, or a chunk's key splits)
    const int units = CHUNK ? p.nslots : p.nseq;
    const int GH = p.Hkv * p.hblocks;   // (KV group, head block) pairs
    const int id = blockIdx.x;
    int t, unit, grp;
    if (!CHUNK && p.compact) {
        // Compact list: the tiles of level t (query tile t of every
        // sequence that has one, in sequence order, each for all GH pairs)
        // come before those of level t - 1.  Lane l holds sequence l's tile
        // count; cnt(t) = sum over sequences of max(0, nt - t) is the number
        // of list entries at level t or above, so this workgroup's level is
        // the largest t with cnt(t) > qi, and its sequence the
        // (qi - cnt(t + 1))-th of those with a tile at that level.
        const int qi = id / GH;
        grp = id % GH;
        const int bmt = kQB * (kSlots / p.hpw);   // query rows per tile
        int nt = 0;   // (clamped: a sequence past max_seqlen keeps the list in range)
        if (lane < p.nseq)
            nt = min(max(0, (p.cu[lane + 1] - p.cu[lane] + bmt - 1) / bmt), p.ntile_q);
        int lvl = -1;
        for (int t0 = 0; t0 < p.ntile_q; t0 += 64) {
            const int tl = t0 + lane;
            int cnt = 0;
            for (int s = 0; s < p.nseq; ++s)
                cnt += max(0, __builtin_amdgcn_readlane(nt, s) - tl);
            const uint64_t hit = __builtin_amdgcn_ballot_w64(tl < p.ntile_q && cnt > qi);
            if (hit)
                lvl = t0 + 63 - __builtin_clzll(hit);
        }
        if (lvl < 0)
            return;   // past the last tile (the grid is an upper bound)
        int below = 0;   // cnt(lvl + 1)
        for (int s = 0; s < p.nseq; ++s)
            below += max(0, __builtin_amdgcn_readlane(nt, s) - (lvl + 1));
        const int k = qi - below;
        const uint64_t has = __builtin_amdgcn_ballot_w64(nt > lvl);
        const int rank = (int)__builtin_amdgcn_mbcnt_hi(
            (uint32_t)(has >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)has, 0u));
        const uint64_t pick = __builtin_amdgcn_ballot_w64(nt > lvl && rank == k);
        t = lvl;
        unit = __builtin_ctzll(pick);
    } else {
        const int pairs = units * GH;
        t = p.ntile_q - 1 - id / pairs;
        const int rem = id % pairs;
        unit = rem / GH;
        grp = rem % GH;
    }
    const int g = grp / p.hblocks;
    const int hb = grp % p.hblocks;
    int seq = unit, split = 0;
    if constexpr (CHUNK) {
        if (p.ck > 0) {
            int base = 0;
            if (!diffattn_splits::split_owner(p, unit, lane, seq, base))
                return;   // past the last split
            split = unit - base;
        }
    }

    int s0, s1;                          // the sequence's query rows
    if (p.cu) {
        s0 = p.cu[seq];
        s1 = p.cu[seq + 1];
    } else {
        s0 = seq * p.seqlen_uniform;
        s1 = s0 + p.seqlen_uniform;
    }
    // its key rows [ks0, ks1), and dk: the key index of query row tq (its
    // own key) is tq + dk; without CHUNK the same rows, dk = 0
    int ks0 = s0, ks1 = s1;
    if constexpr (CHUNK) {
        if (p.cuk) {
            ks0 = p.cuk[seq];
            ks1 = p.cuk[seq + 1];
        } else {
            ks0 = seq * p.klen_uniform;
            ks1 = ks0 + p.klen_uniform;
        }
        if (ks1 <= ks0)
            return;   // queries without keys: a broken precondition
    }
    const int dk = CHUNK ? ks1 - s1 : 0;
    // this workgroup's keys [kr0, kr1): the sequence's, or one split of them
    int kr0 = ks0, kr1 = ks1;
    if constexpr (CHUNK) {
        if (p.ck > 0) {
            kr0 = ks0 + split * p.ck;
            kr1 = min(kr0 + p.ck, ks1);
            if (kr0 >= ks1)
                return;
        }
    }
    // rotary position of query row tq: its key's index in the sequence
    // (clamped at 0 for chunks longer than their keys, a broken precondition
    // of rotary chunks that must still read inside the tables)
    auto rope_pos = [&](int tq) __attribute__((always_inline)) {
        return CHUNK ? max(tq + dk - ks0, 0) : tq - ks0;
    };
    const int qpw = kSlots / p.hpw;     // query blocks per workgroup
    const int bm = kQB * qpw;           // query rows per workgroup
    const int q0 = s0 + t * bm;
    if (q0 >= s1)
        return;
    const int qhi = min(s1, q0 + bm);

    const int head = g * (p.H / p.Hkv) + hb * p.hpw + slot / qpw;
    const int wq0 = q0 + (slot % qpw) * kQB;   // first query row of this slot
    const int wq_last = min(wq0 + kQB, s1) - 1;

    // ---- Q fragments of this wave's map (B operand of S^T = K Q^T) --------
    // sub-block u holds queries wq0 + 32 u + n
    Frag qf[kSub][NKS];
    if constexpr (sizeof(E) == 2) {
        // The wave's Q rows (its map's half) arrive as whole rows, CPQ lanes
        // per row and 16 bytes per lane, pass through the wave's own region
        // of stage 1 (idle until the first tile is computed) and are read
        // back as fragments.  Loaded as fragments, every load instruction
        // would touch 32 rows in 32-byte pieces.
        constexpr int QROWB = D * 2 + 16;   // padded LDS row
        constexpr int CPQ = D * 2 / 16;     // 16-byte chunks per row
        constexpr int RPQ = 64 / CPQ;       // rows per load
        static_assert(kWaves * kQB * QROWB <= GEO::STAGEB, "Q rows must fit a stage");
        char *qst = stage1 + wave * kQB * QROWB;
        const int qr = lane / CPQ, qc = lane % CPQ;
        u32x4 qv[kQB / RPQ];
#pragma unroll
        for (int i = 0; i < kQB / RPQ; ++i) {
            const int tq = wq0 + i * RPQ + qr;
            if (tq < s1) {
                const char *src = (const char *)p.q +
                                  (((int64_t)tq * p.H + head) * 2 + map) * (D * 2) + qc * 16;
                qv[i] = *(const u32x4 *)src;
                if constexpr (ROPE)   // pairs 4 qc .. 4 qc + 3 of the half-head
                    qv[i] = Rope<E, RT>::rotate(qv[i], Rope<E, RT>::coef(p.rcos, p.rsin, rope_pos(tq),
                                                                 4 * qc, D));
            } else {
                qv[i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < kQB / RPQ; ++i)
            *(u32x4 *)(qst + (i * RPQ + qr) * QROWB + qc * 16) = qv[i];
        // (same wave, same bytes: LDS operations of a wave complete in order)
#pragma unroll
        for (int u = 0; u < kSub; ++u)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                qf[u][ks] = *(const Frag *)(qst + (32 * u + n) * QROWB +
                                            (ks * KSTEP + h * VEC) * 2);
    } else {
        const E *__restrict__ qg = (const E *)p.q;
#pragma unroll
        for (int u = 0; u < kSub; ++u)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int tq = wq0 + 32 * u + n;
                if (tq < s1) {
                    const E *row = qg + (((int64_t)tq * p.H + head) * 2 + map) * D;
                    if constexpr (ROPE)
                        qf[u][ks] = Rope<E, RT>::element(row, ks * KSTEP + h * VEC, h,
                                                         p.rcos, p.rsin, rope_pos(tq), D);
                    else
                        qf[u][ks] = *(const Frag *)(row + ks * KSTEP + h * VEC);
                } else {
                    qf[u][ks] = Frag{};
                }
            }
    }

    // ---- KV tile staging ---------------------------------------------------
    // A tile's K rows (and V rows) move in loads of 64 lanes x 16 bytes = RPL
    // consecutive rows: load L covers rows [L RPL, L RPL + RPL), lane l row
    // L RPL + l / CPR and 16-byte chunk l % CPR.  Wave w moves loads w,
    // w + 8, ...: LPW per tensor and tile.  While 32-key block b of tile t is
    // computed, the slice of loads assigned to block b of tile t + 1 travels
    // global -> registers; it is written registers -> LDS (into the padded
    // rows) during block b + 1, so each load has a block's time to arrive.
    constexpr int RPL = 1024 / GEO::ROWB;          // rows per load
    constexpr int NLT = GEO::BN / RPL;             // loads per tensor per tile
    constexpr int LPW = NLT / kWaves;              // loads per wave
    constexpr int MAXL = (LPW + GEO::NB - 1) / GEO::NB;
    static_assert(RPL * GEO::ROWB == 1024 && LPW * kWaves == NLT, "staging tiling");
    const int rowstride = p.Hkv * GEO::ROWB;       // bytes between keys
    const int lrow = wave * RPL + lane / GEO::CPR; // row of load 0
    const int lcol = (lane % GEO::CPR) * 16;
    const char *kbytes = (const char *)p.k + g * GEO::ROWB + lcol;
    const char *vbytes = (const char *)p.v + g * GEO::ROWB + lcol;
    const int kdst = lrow * GEO::KROWB + lcol;
    const int vdst = GEO::KTILEB + lrow * GEO::VROWB + lcol;
    u32x4 kst[MAXL], vst[MAXL];
    // global -> registers: this wave's loads of block slice b of the tile at k0
    auto stage_load = [&](int k0, int b) __attribute__((always_inline)) {
        const bool tail = k0 + GEO::BN > kr1;
#pragma unroll
        for (int i = b * LPW / GEO::NB; i < (b + 1) * LPW / GEO::NB; ++i) {
            int key = k0 + lrow + i * kWaves * RPL;
            if (tail)   // rows past the key range repeat its last row
                key = min(key, kr1 - 1);
            const int64_t off = (int64_t)key * rowstride;
            kst[i - b * LPW / GEO::NB] = *(const u32x4 *)(kbytes + off);
            vst[i - b * LPW / GEO::NB] = *(const u32x4 *)(vbytes + off);
        }
    };
    // registers -> LDS stage
    auto stage_store = [&](char *stage, int b) __attribute__((always_inline)) {
#pragma unroll
        for (int i = b * LPW / GEO::NB; i < (b + 1) * LPW / GEO::NB; ++i) {
            *(u32x4 *)(stage + kdst + i * kWaves * RPL * GEO::KROWB) = kst[i - b * LPW / GEO::NB];
            *(u32x4 *)(stage + vdst + i * kWaves * RPL * GEO::VROWB) = vst[i - b * LPW / GEO::NB];
        }
    };
    // this lane's part of its K operand address (row n, map half, lane half)
    const int k_lane = n * GEO::KROWB + (map * D + h * VEC) * (int)sizeof(E);
    const int v_lane = VOperand<E, D>::lane_base(lane);

    // ---- running state of this wave's map, per query sub-block ------------
    const float c = kLog2e / sqrtf((float)D);   // softmax scale in log2 units
    float m_run[kSub], l_run[kSub];             // raw-score units; partial sums
    f32x16 o[kSub][NDB];
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
        // (a key split can hold no key of a row: a finite floor keeps its
        // probabilities 0 instead of exp2(-inf + inf), and the first visible
        // key still overflows the lazy test and raises the maximum)
        m_run[u] = CHUNK ? -kUnseen : -INFINITY;
        l_run[u] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            o[u][db] = f32x16{};
    }

    const int kv_end = p.causal ? (CHUNK ? min(qhi + dk, kr1) : qhi) : kr1;
    const int ntiles = (kv_end - kr0 + GEO::BN - 1) / GEO::BN;   // (<= 0: none visible)

    // lambda of this head (needed by the map-2 waves in the epilogue); its
    // loads travel with the first tile's.  The butterfly leaves every lane
    // with the same bits, so the value is kept in a scalar register.
    float lam = 0.f;
    if (map == 1) {
        float a = 0.f, b = 0.f;
        const int64_t lo = head * p.lstride;   // this head's lambda vectors
        for (int cc = lane; cc < D; cc += 64) {
            a += p.lq1[lo + cc] * p.lk1[lo + cc];
            b += p.lq2[lo + cc] * p.lk2[lo + cc];
        }
#pragma unroll
        for (int off = 32; off >= 1; off /= 2) {
            a += __shfl_xor(a, off, 64);
            b += __shfl_xor(b, off, 64);
        }
        lam = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                             __builtin_bit_cast(int, expf(a) - expf(b) + p.lambda_init)));
    }

    // first tile: every load of this wave in flight before the first LDS
    // write (slice by slice, each write would wait for its own load)
    {
        u32x4 k0v[LPW], v0v[LPW];
        const bool tail = kr0 + GEO::BN > kr1;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            int key = kr0 + lrow + i * kWaves * RPL;
            if (tail)   // rows past the key range repeat its last row
                key = min(key, kr1 - 1);
            const int64_t off = (int64_t)key * rowstride;
            k0v[i] = *(const u32x4 *)(kbytes + off);
            v0v[i] = *(const u32x4 *)(vbytes + off);
        }
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            *(u32x4 *)(stage0 + kdst + i * kWaves * RPL * GEO::KROWB) = k0v[i];
            *(u32x4 *)(stage0 + vdst + i * kWaves * RPL * GEO::VROWB) = v0v[i];
        }
    }
    __syncthreads();

    // Map-2 waves run the PV product of each block at the start of the next
    // one (its probabilities wait in registers), so the two waves of a SIMD
    // are offset by about half a block: one issues MFMAs while the other
    // runs its exponentials.  A barrier after the first block of every tile
    // keeps the previous tile's V in place until the late PV has read it.
    const bool lag = map == 1;
    Frag pf[kSub][NPS];
    bool pend = false;   // lagging wave: PV of the previous block pending
    auto pv_block = [&](const char *stage, int b) __attribute__((always_inline)) {
        const char *vt = stage + GEO::KTILEB + v_lane;
#pragma unroll
            for (int ps = 0; ps < NPS; ++ps) {
                // first key row of this step (the lane part is in v_lane)
                const int row = VEC == 8 ? 32 * b + 16 * ps
                                         : 32 * b + 8 * (ps / 4) + (ps % 4);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const Frag vf = VOperand<E, D>::load(vt, row, db);
#pragma unroll
                    for (int u = 0; u < kSub; ++u)
                        o[u][db] = M::mma(vf, pf[u][ps], o[u][db]);
                }
            }
    };
    // One tile: compute from `cur` while the next tile is staged into `nxt`.
    auto tile = [&](int it, const char *cur, char *nxt) __attribute__((always_inline)) {
        const int k0 = kr0 + it * GEO::BN;
        const char *kt = cur + k_lane;
        const bool more = it + 1 < ntiles;
#pragma unroll
        for (int b = 0; b < GEO::NB; ++b) {
            // staging of the next tile, one slice per block
            if (more) {
                if (b > 0)
                    stage_store(nxt, b - 1);
                stage_load(k0 + GEO::BN, b);
            }
            if (lag && pend) {
                pv_block(b == 0 ? nxt : cur, (b + GEO::NB - 1) % GEO::NB);
                pend = false;
            }
            const int kb0 = k0 + 32 * b;
            // wave-uniform: can this wave see any key of the block, and does
            // any key need the index mask?
            if (!(kb0 >= kr1 || (p.causal && kb0 > wq_last + dk))) {
            const bool masked = kb0 + 32 > kr1 || (p.causal && kb0 + 31 > wq0 + dk);
            // ---- S^T = K Q^T ------------------------------------------------
            Frag ka[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                ka[ks] = *(const Frag *)(kt + 32 * b * GEO::KROWB + ks * KSTEP * (int)sizeof(E));
            f32x16 sc[kSub];
#pragma unroll
            for (int u = 0; u < kSub; ++u) {
                sc[u] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    sc[u] = M::mma(ka[ks], qf[u][ks], sc[u]);
            }

            if (masked) {
#pragma unroll
                for (int u = 0; u < kSub; ++u) {
                    // wave-uniform: does this sub-block straddle the diagonal
                    // or the end of the sequence?
                    if (kb0 + 32 > kr1 || (p.causal && kb0 + 31 > wq0 + dk + 32 * u)) {
                        // key kb0 + acc_row(a, h) is visible iff its offset
                        // acc_row(a, 0) is at most lim (one compare per key)
                        int lim = kr1 - 1 - kb0;
                        if (p.causal)
                            lim = min(lim, wq0 + dk + 32 * u + n - kb0);
                        lim -= 4 * h;
#pragma unroll
                        for (int a = 0; a < 16; ++a)
                            if (acc_row(a, 0) > lim)
                                sc[u][a] = -INFINITY;
                    }
                }
            }

            // ---- online softmax with a lazily raised maximum ---------------
            // (a query row whose keys of this block are all masked keeps its
            // maximum: its first block always has a visible key, except in a
            // key split, where the maximum starts at the finite floor)
#pragma unroll
            for (int u = 0; u < kSub; ++u) {
                // the row maximum of the block, then a raised running maximum
                // with the sum and accumulator rescaled to it
                auto raise = [&]() __attribute__((always_inline)) {
                    float pm = -INFINITY;
#pragma unroll
                    for (int a = 0; a < 16; ++a)
                        pm = fmaxf(pm, sc[u][a]);
                    const float mnew = fmaxf(m_run[u], pair_max(pm));
                    // nothing accumulated yet when m_run is still -inf
                    const float alpha = m_run[u] == -INFINITY
                                            ? 0.f
                                            : __builtin_amdgcn_exp2f((m_run[u] - mnew) * c);
                    m_run[u] = mnew;
                    l_run[u] *= alpha;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        o[u][db] *= alpha;
                };
                // probabilities against the stored maximum, packed as the
                // B operand of the PV product; returns their fp32 sum
                auto probs = [&]() __attribute__((always_inline)) {
                    const float mc = m_run[u] * c;
                    float pv[16];
#pragma unroll
                    for (int a = 0; a < 16; ++a)
                        pv[a] = __builtin_amdgcn_exp2f(fmaf(sc[u][a], c, -mc));
#pragma unroll
                    for (int ps = 0; ps < NPS; ++ps)
                        pf[u][ps] = M::pack(pv, ps * VEC);
                    float s4[4] = {pv[0], pv[1], pv[2], pv[3]};
#pragma unroll
                    for (int a = 4; a < 16; ++a)
                        s4[a & 3] += pv[a];
                    return (s4[0] + s4[1]) + (s4[2] + s4[3]);
                };
                if constexpr (VEC == 8) {
                    // Probabilities against the stored maximum first; their
                    // sum bounds each of them, so a sum within 2^8 means none
                    // exceeded the lazy threshold.  A larger, infinite or NaN
                    // sum (a raised maximum, or the first block against -inf)
                    // takes the slow path: raise the maximum and recompute.
                    // (The sum is of the fp32 probabilities: a row sum of
                    // their bf16 roundings is measurably less accurate.)
                    float bsum = probs();
                    if (__builtin_amdgcn_ballot_w64(!(bsum <= kRescaleSum)) != 0) {
                        raise();
                        bsum = probs();
                    }
                    l_run[u] += bsum;
                } else {
                    float pm = -INFINITY;
#pragma unroll
                    for (int a = 0; a < 16; ++a)
                        pm = fmaxf(pm, sc[u][a]);
                    const bool grow = (pm - m_run[u]) * c > kRescaleLog2;
                    if (__builtin_amdgcn_ballot_w64(grow) != 0)
                        raise();
                    const float mc = m_run[u] * c;
                    float ps_sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int a = 0; a < 16; ++a) {
                        const float pv = __builtin_amdgcn_exp2f(fmaf(sc[u][a], c, -mc));
                        sc[u][a] = pv;
                        ps_sum[a & 3] += pv;
                    }
                    l_run[u] += (ps_sum[0] + ps_sum[1]) + (ps_sum[2] + ps_sum[3]);
#pragma unroll
                    for (int ps = 0; ps < NPS; ++ps)
                        pf[u][ps] = M::pack(sc[u], ps * VEC);
                }
            }

            if (lag)
                pend = true;
            else
                pv_block(cur, b);
            }
            if (b == 0)
                __syncthreads();
        }

        if (more)
            stage_store(nxt, GEO::NB - 1);
        __syncthreads();
    };
    for (int it = 0; it < ntiles; it += 2) {
        tile(it, stage0, stage1);
        if (it + 1 < ntiles)
            tile(it + 1, stage1, stage0);
    }
    if (lag && pend)
        pv_block((ntiles & 1) ? stage0 : stage1, GEO::NB - 1);
    __syncthreads();

    // ---- epilogue: combine through LDS, RMSNorm, scale, store -------------
    // With two sub-blocks the two waves of a slot split the epilogue by
    // query sub-block: the map-1 wave finishes sub-block 0, the map-2 wave
    // sub-block 1.  Each publishes the term the other needs (map 1: O_1/l_1
    // of sub-block 1; map 2: lambda O_2/l_2 of sub-block 0) in its
    // accumulator layout (four consecutive elements of a lane as one 16-byte
    // entry, lanes adjacent); the partner's lanes hold the same (query, dim)
    // elements.  With one sub-block the map-2 wave publishes and the map-1
    // wave finishes.
    float *xch = (float *)((slot < 2 ? stage0 : stage1)) + (slot & 1) * XCH;
    constexpr int XHALF = XCH / kSub;   // floats per published sub-block
    float lsum[kSub];
#pragma unroll
    for (int u = 0; u < kSub; ++u)
        lsum[u] = pair_sum(l_run[u]);
    if constexpr (CHUNK) {
        if (p.ws_o) {
            // key split: this map's partial per row for the merge (a row that
            // saw no key of the split leaves the floor, a zero sum and zeros)
            const int G = p.H / p.Hkv;
#pragma unroll
            for (int u = 0; u < kSub; ++u) {
                const int tq = wq0 + 32 * u + n;
                if (tq >= s1 || tq - s0 >= p.max_seqlen)
                    continue;
                const int64_t r = (int64_t)(tq - s0) * G + (head - g * G);
                const int64_t row = ((int64_t)unit * p.Hkv + g) * p.rmax + r;
                float *dst = p.ws_o + (row * 2 + map) * (2 * D);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        *(float4 *)(dst + 32 * db + 8 * i + 4 * h) =
                            make_float4(o[u][db][4 * i], o[u][db][4 * i + 1], o[u][db][4 * i + 2],
                                        o[u][db][4 * i + 3]);
                if (h == 0)
                    *(float2 *)(p.ws_ml + row * 4 + 2 * map) = make_float2(m_run[u] * c, lsum[u]);
            }
            return;
        }
    }
    if (p.lse) {
        // training forward: each map's log2-sum-exp of the scaled scores and
        // its normalised output, for the backward pass
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
            const int tq = wq0 + 32 * u + n;
            if (tq >= s1)
                continue;
            const int64_t row = (int64_t)tq * p.H + head;
            if (h == 0)
                p.lse[row * 2 + map] = m_run[u] * c + log2f(lsum[u]);
            float *dst = p.o12 + (row * 2 + map) * (2 * D);
            const float il = 1.f / lsum[u];
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *(float4 *)(dst + 32 * db + 8 * i + 4 * h) =
                        make_float4(o[u][db][4 * i] * il, o[u][db][4 * i + 1] * il,
                                    o[u][db][4 * i + 2] * il, o[u][db][4 * i + 3] * il);
        }
    }
    // this wave's scale of its own map (1/l_1, or lambda/l_2) per sub-block
    float own[kSub];
#pragma unroll
    for (int u = 0; u < kSub; ++u)
        own[u] = (map == 0 ? 1.f : lam) / lsum[u];
    // (the accumulators are indexed by compile-time sub-block only: one
    // branch per map, so they stay in registers)
    auto publish = [&](const f32x16 (&acc)[NDB], float scale, float *dst)
        __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *(float4 *)(dst + ((db * 4 + i) * 64 + lane) * 4) =
                    make_float4(acc[db][4 * i] * scale, acc[db][4 * i + 1] * scale,
                                acc[db][4 * i + 2] * scale, acc[db][4 * i + 3] * scale);
    };
    if constexpr (kSub == 2) {
        if (map == 0)
            publish(o[1], own[1], xch + XHALF);
        else
            publish(o[0], own[0], xch);
    } else {
        if (map == 1)
            publish(o[0], own[0], xch);
    }
    // weights of this lane's output dims (loads in flight across the barrier)
    float wv[NDB][16];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int a = 0; a < 16; ++a)
            wv[db][a] = 1.f;
    if (p.w) {   // one wave-uniform branch, not one per element
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 w4 = *(const float4 *)(p.w + 32 * db + 8 * i + 4 * h);
                wv[db][4 * i + 0] = w4.x;
                wv[db][4 * i + 1] = w4.y;
                wv[db][4 * i + 2] = w4.z;
                wv[db][4 * i + 3] = w4.w;
            }
    }
    __syncthreads();

    // pre = O_1/l_1 - lambda O_2/l_2 of this wave's sub-block u = map, its
    // RMSNorm, weight, scale and store
    auto finish = [&](const f32x16 (&acc)[NDB], float scale, int u) __attribute__((always_inline)) {
        const float *src = xch + u * XHALF;
        float pre[NDB][16];
        float ss = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 x4 = *(const float4 *)(src + ((db * 4 + i) * 64 + lane) * 4);
                const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float mine = acc[db][4 * i + e] * scale;
                    const float v = u == 0 ? mine - xs[e] : xs[e] - mine;
                    pre[db][4 * i + e] = v;
                    ss += v * v;
                }
            }
        ss = pair_sum(ss);
        const float r = (1.f - p.lambda_init) / sqrtf(ss / (float)(2 * D) + p.eps);
        const int qbase = wq0 + 32 * u;   // query of row 0 of this sub-block
        if constexpr (sizeof(E) == 2) {
            // Rounded rows go through the wave's own LDS (the half of the
            // exchange it has just read, so no other wave touches it) and out
            // as whole rows: 16 bytes per lane, each store covers 64 / CPR
            // consecutive rows instead of 32 scattered 16-byte pieces.
            constexpr int ROW = 2 * D * 2;        // bytes per output row
            constexpr int PITCH = ROW + 8;        // 8-byte writes of 32 rows hit distinct banks
            constexpr int CPR = ROW / 16;         // 16-byte chunks per row
            constexpr int RPS = 64 / CPR;         // rows per store
            static_assert(32 * PITCH <= XHALF * 4, "staged rows must fit the read half");
            char *stg = (char *)src;
            // ordered after this wave's reads of the same bytes (LDS operations
            // of one wave complete in order)
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bf16x4 vals;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        vals[j] = (bf16)(pre[db][4 * i + j] * r * wv[db][4 * i + j]);
                    *(bf16x4 *)(stg + n * PITCH + (32 * db + 8 * i + 4 * h) * 2) = vals;
                }
            __builtin_amdgcn_wave_barrier();
            const int rr = lane / CPR, cc = (lane % CPR) * 16;
#pragma unroll
            for (int k = 0; k < 32 / RPS; ++k) {
                const int row = k * RPS + rr;
                const char *a = stg + row * PITCH + cc;
                const uint2 lo = *(const uint2 *)a, hi = *(const uint2 *)(a + 8);
                const int tq = qbase + row;
                // (nontemporal: the output is not read again here, and
                // keeping it out of L2 leaves room for the K/V tiles that
                // other workgroups re-read; 0.9% on 8 x 4096 tokens)
                if (tq < s1)
                    __builtin_nontemporal_store(
                        u32x4{lo.x, lo.y, hi.x, hi.y},
                        (u32x4 *)((char *)p.out + ((int64_t)tq * p.H + head) * ROW + cc));
            }
        } else {
            const int tq = qbase + n;
            if (tq < s1) {
                E *dst = (E *)p.out + ((int64_t)tq * p.H + head) * (2 * D);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int dim = 32 * db + 8 * i + 4 * h;
                        E vals[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            vals[j] = (E)(pre[db][4 * i + j] * r * wv[db][4 * i + j]);
                        __builtin_memcpy(dst + dim, vals, sizeof(vals));
                    }
            }
        }
    };
    if (map == 0)
        finish(o[0], own[0], 0);
    else if constexpr (kSub == 2)
        finish(o[kSub - 1], own[kSub - 1], 1);
}

template <typename E, int D, int RT>
void launch_rt(const Params &p, int nblocks, hipStream_t stream)
{
    if constexpr (RT != diffattn_rope::kOff) {
        // K rotated once into the workspace, which the kernel then reads as K
        const int64_t threads = (int64_t)p.T * (D * (int)sizeof(E) / 16);
        hipLaunchKernelGGL((rope_rotate_k<E, D, RT>), dim3((unsigned)((threads + 255) / 256)),
                           dim3(256), 0, stream, (const char *)p.k_orig, (char *)p.k, p.cu,
                           p.nseq, p.seqlen_uniform, p.T, p.Hkv, p.rcos, p.rsin);
    }
    if (p.sub == 2)
        hipLaunchKernelGGL((diffattn_fwd_kernel<E, D, RT, 2>), dim3(nblocks), dim3(kThreads), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((diffattn_fwd_kernel<E, D, RT, 1>), dim3(nblocks), dim3(kThreads), 0,
                           stream, p);
}

template <typename E, int D>
int launch(const Params &p, int nblocks, hipStream_t stream)
{
    if (!p.rcos)
        launch_rt<E, D, diffattn_rope::kOff>(p, nblocks, stream);
    else if (p.rope_dtype == DIFFATTN_BF16)
        launch_rt<E, D, diffattn_rope::kBF16>(p, nblocks, stream);
    else
        launch_rt<E, D, diffattn_rope::kF32>(p, nblocks, stream);
    return hipGetLastError() == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}

// Query chunks against a key/value cache: the keys are used as given, so a
// rotary chunk turns only its queries (no K rotation).
template <typename E, int D, int RT>
void launch_chunk_rt(const Params &p, int nblocks, hipStream_t stream)
{
    if (p.sub == 2)
        hipLaunchKernelGGL((diffattn_fwd_kernel<E, D, RT, 2, true>), dim3(nblocks), dim3(kThreads),
                           0, stream, p);
    else
        hipLaunchKernelGGL((diffattn_fwd_kernel<E, D, RT, 1, true>), dim3(nblocks), dim3(kThreads),
                           0, stream, p);
}

template <typename E, int D>
int launch_chunk(const Params &p, int nblocks, hipStream_t stream)
{
    if (!p.rcos)
        launch_chunk_rt<E, D, diffattn_rope::kOff>(p, nblocks, stream);
    else if (p.rope_dtype == DIFFATTN_BF16)
        launch_chunk_rt<E, D, diffattn_rope::kBF16>(p, nblocks, stream);
    else
        launch_chunk_rt<E, D, diffattn_rope::kF32>(p, nblocks, stream);
    return hipGetLastError() == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}

// Grid of a launch: 64 queries per wave, or 32 when that leaves fewer than
// two workgroups per CU (256 CUs), so small problems spread over twice the
// workgroups.  Returns false when the grid would not fit 32 bits.
// Grid with `sub` 32-query sub-blocks per wave.
// With T >= 0 (packed sequences whose tile list the kernel can build) the
// grid may be the compact list: at most T / bm + nseq tiles (the sum of
// ceil(n_s / bm) over the sequences), whatever the lengths, so the host
// needs no look at cu_seqlens.  It is taken only where that bound is below
// the padded grid's ntile_q * nseq tiles: the list costs each workgroup a
// few dozen instructions more in its prologue (1% on eight 4096-token
// sequences, whose padded grid has no empty tile), and saves the empty
// workgroups of a length mix (about 3% on 30 sequences of 128 to 4096
// tokens).
void grid_of(int max_seqlen, int nseq, int H, int Hkv, int sub, int &hpw, int64_t &ntile_q,
             int64_t &nblocks, int64_t T = -1, bool *compact = nullptr)
{
    const int G = H / Hkv;
    hpw = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);
    const int bm = 32 * sub * (kSlots / hpw);
    ntile_q = ((int64_t)max_seqlen + bm - 1) / bm;
    int64_t tiles = ntile_q * nseq;
    const bool cpt = T >= 0 && T / bm + nseq < tiles;
    if (cpt)
        tiles = T / bm + nseq;
    if (compact)
        *compact = cpt;
    nblocks = tiles * Hkv * (G / hpw);
}

bool grid_shape(int max_seqlen, int nseq, int H, int Hkv, int &hpw, int &sub, int64_t &ntile_q,
                int64_t &nblocks, int64_t T = -1, bool *compact = nullptr)
{
    sub = 2;
    grid_of(max_seqlen, nseq, H, Hkv, sub, hpw, ntile_q, nblocks, T, compact);
    if (nblocks < 2 * kCUs) {
        sub = 1;
        grid_of(max_seqlen, nseq, H, Hkv, sub, hpw, ntile_q, nblocks, T, compact);
    }
    return nblocks <= INT32_MAX;
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
        if (d == 32) return launch<float, 32>;
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
    case DIFFATTN_ETOOLARGE:
        return "sizes need more device scratch than the library's static array holds";
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

} // extern "C"

namespace {

int fwd_impl(int dtype, const void *q, const void *k, const void *v,
             const float *lambda_q1, const float *lambda_k1,
             const float *lambda_q2, const float *lambda_k2,
             int32_t lambda_stride, float lambda_init,
             const float *subln_weight, float eps,
             int causal, const int32_t *cu_seqlens, int32_t nseq,
             int32_t max_seqlen, int32_t T, int32_t H, int32_t Hkv,
             int32_t d, const void *rope_cos, const void *rope_sin,
             int32_t rope_len, int rope_dtype, void *workspace, size_t workspace_bytes,
             float *lse, float *o12, void *out, void *stream)
{
    if (dtype != DIFFATTN_BF16 && dtype != DIFFATTN_F32)
        return DIFFATTN_EINVAL;
    if (T < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || d < 1)
        return DIFFATTN_EINVAL;
    if (causal != 0 && causal != 1)
        return DIFFATTN_EINVAL;
    if (!(eps >= 0.f) || isinf(eps) || !isfinite(lambda_init))
        return DIFFATTN_EINVAL;
    if (lambda_stride != 0 && lambda_stride < d)
        return DIFFATTN_EINVAL;
    if ((rope_cos == nullptr) != (rope_sin == nullptr))
        return DIFFATTN_EINVAL;
    if (rope_cos && rope_dtype != DIFFATTN_F32 && rope_dtype != DIFFATTN_BF16)
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
    // rotary tables cover every position and are read in aligned vectors
    // of 2 or 4 entries; the workspace holds the rotated copy of K
    if (rope_cos && (rope_len < max_seqlen ||
                     ((uintptr_t)rope_cos | (uintptr_t)rope_sin) % 16 != 0))
        return DIFFATTN_EINVAL;
    if (rope_cos && (!workspace || (uintptr_t)workspace % 16 != 0 ||
                     workspace_bytes < diffattn_fwd_workspace_size(dtype, T, Hkv, d, 1)))
        return DIFFATTN_EINVAL;
    // byte offsets of K/V rows are formed in 64 bits; the grid in 32 bits
    const int G = H / Hkv;
    int hpw = 0, sub = 0;
    int64_t ntile_q = 0, nblocks = 0;
    // packed sequences, up to one per lane: the compact tile list where it
    // is the smaller grid
    bool compact = false;
    if (!grid_shape(max_seqlen, nseq, H, Hkv, hpw, sub, ntile_q, nblocks,
                    cu_seqlens && nseq <= 64 ? T : -1, &compact))
        return DIFFATTN_EINVAL;

    Params p;
    p.q = q;
    p.k = rope_cos ? workspace : k;
    p.k_orig = k;
    p.v = v;
    p.out = out;
    p.lq1 = lambda_q1;
    p.lk1 = lambda_k1;
    p.lq2 = lambda_q2;
    p.lk2 = lambda_k2;
    p.lstride = lambda_stride;
    p.w = subln_weight;
    p.cu = cu_seqlens;
    p.cuk = nullptr;
    p.klen_uniform = 0;
    p.ws_o = p.ws_ml = nullptr;
    p.ck = 0;
    p.nslots = nseq;
    p.rmax = 0;
    p.rcos = rope_cos;
    p.rsin = rope_sin;
    p.rope_dtype = rope_dtype;
    p.lse = lse;
    p.o12 = o12;
    p.lambda_init = lambda_init;
    p.eps = eps;
    p.T = T;
    p.H = H;
    p.Hkv = Hkv;
    p.nseq = nseq;
    p.seqlen_uniform = uniform;
    p.causal = causal;
    p.ntile_q = (int32_t)ntile_q;
    p.max_seqlen = max_seqlen;
    p.hpw = hpw;
    p.hblocks = G / hpw;
    p.sub = sub;
    p.compact = compact ? 1 : 0;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return DIFFATTN_EHIP;
    return fn(p, (int)nblocks, (hipStream_t)stream);
}

} // namespace

int diffattn_chunk_plan(int32_t nseq, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t H,
                        int32_t Hkv, int32_t d, int splits, size_t ws_cap,
                        DiffattnChunkPlan *plan)
{
    int hpw = 0, sub0 = 0;
    int64_t ntile_q = 0, nblocks = 0;
    if (nseq < 1 || max_seqlen_q < 1 || max_seqlen_k < 1 ||
        !grid_shape(max_seqlen_q, nseq, H, Hkv, hpw, sub0, ntile_q, nblocks))
        return 0;
    const int64_t rmax = (int64_t)(H / Hkv) * max_seqlen_q;
    // Estimated duration with units of ck keys each (sequences, or splits):
    // rounds of at most one workgroup per CU, each as long as a workgroup
    // streaming ck keys, plus, for splits, the merge kernel.  The constants
    // are fitted to 300 measured calls on this part (d = 64; d = 32 about
    // 0.72 of the per-key time; an 11.5% RMS fit of log time): per key 20.7
    // ns with 32-query sub-blocks and 33.2 with 64, 45% more when every CU
    // is busy (the clock under load), 9.8 us per round; the merge 0.28 us
    // per MB of partials, 0.65 ns per output row and 5.7 us.
    const double fd = d == 32 ? 0.72 : 1.0;
    const double out_rows = (double)nseq * max_seqlen_q * H;
    auto estimate = [&](int sub, int64_t blocks, int64_t keys, size_t ws_bytes) {
        const double ns_per_key = (sub == 2 ? 33.2 : 20.7) * fd;
        const double occ = (double)std::min<int64_t>(blocks, kCUs) / kCUs;
        double us = (double)((blocks + kCUs - 1) / kCUs) *
                    (1e-3 * ns_per_key * (double)keys * (1.0 + 0.455 * occ) + 9.8);
        if (ws_bytes)
            us += 0.275e-6 * (double)ws_bytes + 0.647e-3 * out_rows + 5.7;
        return us;
    };
    // unsplit: the prefill's own choice of sub-blocks
    DiffattnChunkPlan pl{};
    pl.rmax = (int32_t)std::min<int64_t>(rmax, INT32_MAX);
    pl.nslots = nseq;
    pl.sub = sub0;
    pl.est_us = splits == 2 ? INFINITY : estimate(sub0, nblocks, max_seqlen_k, 0);
    // key splits of 256, 512, 1024, ... keys (whole 128-key tiles), with 64-
    // or 32-query sub-blocks, the cheapest estimate among those that fit the
    // workspace winning
    for (int sub = 2; splits && sub >= 1; --sub) {
        int64_t nb = 0;
        grid_of(max_seqlen_q, nseq, H, Hkv, sub, hpw, ntile_q, nb);
        const int64_t per_unit = nb / nseq;   // workgroups per sequence or split
        for (int64_t ck = 256; ck < max_seqlen_k; ck *= 2) {
            const int64_t slots = (int64_t)nseq * ((max_seqlen_k + ck - 1) / ck);
            const int64_t rows = slots * Hkv * rmax;
            if (slots > INT32_MAX || per_unit * slots > INT32_MAX || rmax > (1 << 24) ||
                rows > ((int64_t)1 << 36))
                continue;
            const size_t ws_o = (size_t)rows * 2 * (2 * d) * 4, ws_ml = (size_t)rows * 4 * 4;
            if (ws_o + ws_ml > ws_cap)
                continue;   // (the partials would not fit the workspace)
            const double us = estimate(sub, per_unit * slots, ck, ws_o + ws_ml);
            if (us < pl.est_us) {
                pl.ck = (int32_t)ck;
                pl.nslots = (int32_t)slots;
                pl.sub = sub;
                pl.ws_o_bytes = ws_o;
                pl.ws_ml_bytes = ws_ml;
                pl.est_us = us;
            }
        }
    }
    if (splits == 2 && pl.ck == 0)
        return 0;   // no split fits
    *plan = pl;
    return 1;
}

int diffattn_chunk_prefill(const void *q, const void *k, const void *v, const float *lambda_q1,
                           const float *lambda_k1, const float *lambda_q2,
                           const float *lambda_k2, int32_t lambda_stride, float lambda_init,
                           const float *subln_weight, float eps, int causal,
                           const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                           int32_t nseq, int32_t max_seqlen_q, int32_t Tq, int32_t Tk, int32_t H,
                           int32_t Hkv, int32_t d, const void *rope_cos, const void *rope_sin,
                           int rope_dtype, const DiffattnChunkPlan *plan, float *ws_o,
                           float *ws_ml, void *out, void *stream)
{
    if (d != 64 && d != 32)
        return DIFFATTN_EUNSUPPORTED;
    // (the grid's first index runs over the split slots, or the sequences)
    const int units = plan->ck > 0 ? plan->nslots : nseq;
    const int sub = plan->sub;
    if (sub != 1 && sub != 2)
        return DIFFATTN_EINVAL;
    int hpw = 0;
    int64_t ntile_q = 0, nblocks = 0;
    grid_of(max_seqlen_q, nseq, H, Hkv, sub, hpw, ntile_q, nblocks);
    nblocks = nblocks / nseq * units;
    if (nblocks > INT32_MAX)
        return DIFFATTN_EINVAL;
    Params p;
    p.q = q;
    p.k = k;
    p.k_orig = k;
    p.v = v;
    p.out = out;
    p.lq1 = lambda_q1;
    p.lk1 = lambda_k1;
    p.lq2 = lambda_q2;
    p.lk2 = lambda_k2;
    p.lstride = lambda_stride;
    p.w = subln_weight;
    p.cu = cu_seqlens_q;
    p.cuk = cu_seqlens_k;
    p.klen_uniform = cu_seqlens_q ? 0 : Tk / nseq;
    p.ck = plan->ck;
    p.nslots = units;
    p.rmax = plan->rmax;
    p.ws_o = plan->ck > 0 ? ws_o : nullptr;
    p.ws_ml = plan->ck > 0 ? ws_ml : nullptr;
    p.rcos = rope_cos;
    p.rsin = rope_sin;
    p.rope_dtype = rope_dtype;
    p.lse = nullptr;
    p.o12 = nullptr;
    p.lambda_init = lambda_init;
    p.eps = eps;
    p.T = Tq;
    p.H = H;
    p.Hkv = Hkv;
    p.nseq = nseq;
    p.seqlen_uniform = cu_seqlens_q ? 0 : Tq / nseq;
    p.causal = causal;
    p.ntile_q = (int32_t)ntile_q;
    p.max_seqlen = max_seqlen_q;
    p.hpw = hpw;
    p.hblocks = H / Hkv / hpw;
    p.sub = sub;
    p.compact = 0;
    hipStream_t st = (hipStream_t)stream;
    return d == 64 ? launch_chunk<bf16, 64>(p, (int)nblocks, st)
                   : launch_chunk<bf16, 32>(p, (int)nblocks, st);
}

extern "C" {

int diffattn_fwd(int dtype, const void *q, const void *k, const void *v,
                 const float *lambda_q1, const float *lambda_k1,
                 const float *lambda_q2, const float *lambda_k2,
                 int32_t lambda_stride, float lambda_init,
                 const float *subln_weight, float eps,
                 int causal, const int32_t *cu_seqlens, int32_t nseq,
                 int32_t max_seqlen, int32_t T, int32_t H, int32_t Hkv,
                 int32_t d, const void *rope_cos, const void *rope_sin,
                 int32_t rope_len, int rope_dtype, void *workspace, size_t workspace_bytes,
                 void *out, void *stream)
{
    return fwd_impl(dtype, q, k, v, lambda_q1, lambda_k1, lambda_q2, lambda_k2,
                    lambda_stride, lambda_init, subln_weight, eps, causal, cu_seqlens,
                    nseq, max_seqlen, T, H, Hkv, d, rope_cos, rope_sin, rope_len, rope_dtype,
                    workspace, workspace_bytes, nullptr, nullptr, out, stream);
}

size_t diffattn_fwd_workspace_size(int dtype, int32_t T, int32_t Hkv, int32_t d, int rope)
{
    if (!rope || T <= 0 || Hkv < 1 || d < 1)
        return 0;
    const size_t es = dtype == DIFFATTN_F32 ? 4 : 2;
    return ((size_t)T * Hkv * 2 * d * es + 255) & ~(size_t)255;
}

int diffattn_fwd_train(int dtype, const void *q, const void *k, const void *v,
                       const float *lambda_q1, const float *lambda_k1,
                       const float *lambda_q2, const float *lambda_k2,
                       int32_t lambda_stride, float lambda_init,
                       const float *subln_weight, float eps, int causal,
                       const int32_t *cu_seqlens, int32_t nseq, int32_t max_seqlen,
                       int32_t T, int32_t H, int32_t Hkv, int32_t d, void *out,
                       float *lse, float *o12, void *stream)
{
    if (T > 0 && (!lse || !o12 || ((uintptr_t)o12 % 16) != 0 || ((uintptr_t)lse % 4) != 0))
        return DIFFATTN_EINVAL;
    return fwd_impl(dtype, q, k, v, lambda_q1, lambda_k1, lambda_q2, lambda_k2,
                    lambda_stride, lambda_init, subln_weight, eps, causal, cu_seqlens,
                    nseq, max_seqlen, T, H, Hkv, d, nullptr, nullptr, 0, 0, nullptr, 0, lse,
                    o12, out, stream);
}

} // extern "C"
