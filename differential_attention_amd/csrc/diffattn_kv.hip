// diffattn_kv.hip -- differential attention of new queries against a
// key/value cache, for CDNA4 (gfx950).
//
// The operation is the one defined for diffattn_fwd_kv in include/diffattn.h:
// the LlamaDiffSdpaAttention.py gist's forward appends the step's keys and
// values to the cache and then attends with both maps; the causal mask is
// aligned bottom-right, as the FlashDiffAttention pull request's
// alternative_forward builds it (-inf above diagonal 1 + src_len - tgt_len),
// so query i of nq sees cache keys 0 .. nk - nq + i.
//
// Why a second kernel
// -------------------
// A decode step has a handful of query rows per KV head (G heads x nq
// queries) against thousands of keys: every K/V byte feeds only G * nq rows,
// so the work is bound by reading the cache from HBM, not by MFMA.  The
// design goal is to stream K and V once, with enough bytes in flight on
// every CU, and to keep the GQA sharing (one K/V read serves all G heads of
// a group).
//
// Split-KV partial kernel
// -----------------------
// One wave = (sequence s, KV head g, block of 16 query rows, split of Ck
// keys).  A row is (query i, head gh of the group), row r = i * G + gh.
// Waves are independent: each has a private LDS slice for its K and V tiles
// and no barrier is ever taken.  Per 32-key block:
//   * K and V go global -> registers one block ahead of use, in whole rows
//     (one load instruction covers consecutive rows) and with nontemporal
//     loads, then into the wave's padded LDS tiles.  Loading K straight
//     into the MFMA operand layout instead (16 keys x 64 bytes per load
//     instruction) read the cache about 7% slower;
//   * K comes back from LDS in the A-operand layout of
//     v_mfma_f32_16x16x32_bf16 (lane (key n, quarter q) holds 8 consecutive
//     dims), V through the transposing read ds_read_b64_tr_b16 as the V^T
//     operand;
//   * S^T [16 keys x 16 rows] = K Q^T per map and 16-key half: each lane
//     owns one row and 4 keys of each half, so the accumulator is directly
//     the P^T operand of the PV product when the contraction runs over keys
//     {4q..4q+3} U {16+4q..16+4q+3} -- the order the transposing read
//     produces;
//   * O_m^T [2d x 16 rows] += V^T P_m^T; one V^T operand feeds both maps.
// The softmax keeps, per map and row, a lazily raised maximum (log2 units)
// and a running sum; the partial (m, l, O) of the split is written to the
// caller's workspace in fp32.
//
// Combine kernel
// --------------
// One or more thread groups per output row (token, head), as many as the
// longest row's split count asks for: merges the splits' partials of both
// maps by log-sum-exp, then applies the epilogue that the prefill kernel
// fuses -- lambda from the four vectors, O_1/l_1 - lambda O_2/l_2,
// RMSNorm over 2d, the weight and the (1 - lambda_init) scale -- and stores
// in the input dtype.  Partial outputs cannot simply be summed: the
// combination is nonlinear in the two maps' normalisers.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>
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
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = 64 * kWavesPerBlock;
constexpr int kRows = 16;      // query rows per wave
constexpr int kBlockKeys = 32; // keys per inner block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.0f;

struct KvParams {
    const void *q;
    const void *k;
    const void *v;
    void *out;
    const float *lq1, *lk1, *lq2, *lk2;
    int64_t lstride;
    const float *w;
    const int32_t *cuq;   // NULL: uniform lengths qlen_uniform
    const int32_t *cuk;   // NULL: uniform lengths klen_uniform
    float *ws_o;          // [split slot][Hkv][rmax][2][2d]
    float *ws_ml;         // [split slot][Hkv][rmax][4]: m, l of map 1, m, l of map 2
    const void *rcos, *rsin;   // rotary tables of the new queries, or NULL
    int32_t rope_len;
    float lambda_init;
    float eps;
    int32_t H, Hkv, G, nseq, causal;
    int32_t qlen_uniform, klen_uniform;
    int32_t max_q;        // queries per sequence at most
    int32_t rmax;         // G * max_q rows per (sequence, group)
    int32_t nrb;          // 16-row blocks per (sequence, group)
    int32_t nslots;       // split slots of the workspace (bound on all sequences' splits)
    int32_t ck;           // keys per split (multiple of 32)
};

__device__ inline void seq_bounds(const int32_t *cu, int uniform, int s, int &a, int &n)
{
    if (cu) {
        a = cu[s];
        n = cu[s + 1] - a;
    } else {
        a = s * uniform;
        n = uniform;
    }
}

using diffattn_splits::split_count;
using diffattn_splits::split_owner;

// Combined value over the four lanes l, l^16, l^32, l^48 (the quarter-waves
// of one row); the order of combination is fixed, so all four lanes get
// bitwise the same result.
__device__ inline float quad_max(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y),
                                                    false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float quad_sum(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y),
                                                    false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ inline f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// RT: rotary tables of the new queries (diffattn_rope::kOff, kF32, kBF16).
template <int D, int RT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void diffattn_kv_partial(KvParams p)
{
    constexpr int NKS = D / 32;              // QK MFMAs per map and 16-key half
    constexpr int NDT = 2 * D / 16;          // 16-wide tiles of the 2d output
    constexpr int ROWB = 2 * D * 2;          // bytes of one K (or V) row
    constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
    constexpr int RPL = 64 / CPR;            // rows per 64-lane V load
    constexpr int NVL = kBlockKeys / RPL;    // V loads per lane per block
    // padded V row: the 8 rows one half-wave reads per transposing read
    // start 32 bytes apart modulo 256 and cover all banks once
    constexpr int VROWB = ROWB + 32;
    // padded K row: the 16 rows of one operand read start 16 bytes apart
    // modulo 256 (d = 64; d = 32: distinct multiples of 16)
    constexpr int KROWB = ROWB + 16;
    static_assert(D % 32 == 0 && NVL * RPL == kBlockKeys, "unsupported d");

    __shared__ __attribute__((aligned(16))) char klds[kWavesPerBlock][kBlockKeys * KROWB];
    __shared__ __attribute__((aligned(16))) char vlds[kWavesPerBlock][kBlockKeys * VROWB];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;      // row (S^T column) owned by this lane; key row for K loads
    const int qq = lane >> 4;     // quarter of the wave

    // ---- work item ---------------------------------------------------------
    // KV head fastest: the waves of a workgroup (and neighbouring
    // workgroups) read the other heads' slices of the same key rows at the
    // same time, so every DRAM page they open is read whole
    int64_t wid = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    const int g = (int)(wid % p.Hkv);
    wid /= p.Hkv;
    const int rb = (int)(wid % p.nrb);
    const int j = (int)(wid / p.nrb);   // split slot
    if (j >= p.nslots)
        return;
    int s, sbase;
    if (!split_owner(p, j, lane, s, sbase))
        return;   // past the last split
    int qa, nq, ka, nk;
    seq_bounds(p.cuq, p.qlen_uniform, s, qa, nq);
    seq_bounds(p.cuk, p.klen_uniform, s, ka, nk);
    const int nrows = p.G * min(nq, p.max_q);   // rows of this (sequence, group)
    const int r0 = rb * kRows;
    const int kstart = (j - sbase) * p.ck;
    if (r0 >= nrows || kstart >= nk)
        return;   // nothing to compute; the combine reads no partial here

    // rows of this wave: r = r0 + n (valid if r < nrows), query i = r / G
    const int r = r0 + n;
    const bool row_ok = r < nrows;
    const int qi = r / p.G;
    const int i_lo = r0 / p.G;
    const int i_hi = min(nrows - 1, r0 + kRows - 1) / p.G;
    // keys this wave can see: [kstart, kend)
    int kend = min(nk, kstart + p.ck);
    if (p.causal)
        kend = min(kend, nk - nq + i_hi + 1);
    // keys below kvis are visible to every row of the wave
    const int kvis = p.causal ? min(nk, nk - nq + i_lo + 1) : nk;
    const int row_lim = p.causal ? min(nk - 1, nk - nq + qi) : nk - 1;

    // ---- Q fragments (B operand of S^T = K Q^T) ----------------------------
    // With rotary tables each fragment (pairs 16 ks + 4 qq .. + 3 of the
    // half-head) is rotated at the query's absolute position nk - nq + i
    // (clamped into the tables, which only matters when the preconditions
    // nq <= nk and rope_len >= nk are broken)
    bf16x8 qf[2][NKS];
    {
        const bf16 *qg = (const bf16 *)p.q;
        const int head = g * p.G + r % p.G;
        const int64_t tok = (int64_t)qa + qi;
        const int pos = min(max(nk - nq + qi, 0), p.rope_len - 1);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                if (row_ok) {
                    qf[m][ks] = *(const bf16x8 *)(qg + ((tok * p.H + head) * 2 + m) * D + 32 * ks + 8 * qq);
                    if constexpr (RT != diffattn_rope::kOff) {
                        typedef diffattn_rope::Rope<bf16, RT> R;
                        qf[m][ks] = __builtin_bit_cast(
                            bf16x8, R::rotate(__builtin_bit_cast(u32x4, qf[m][ks]),
                                              R::coef(p.rcos, p.rsin, pos, 16 * ks + 4 * qq, D)));
                    }
                } else {
                    qf[m][ks] = bf16x8{};
                }
            }
    }

    // ---- accumulators --------------------------------------------------------
    f32x4 o[2][NDT];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < NDT; ++t)
            o[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrun[2] = {-INFINITY, -INFINITY};
    float lsum[2] = {0.f, 0.f};
    const float c = kLog2e * rsqrtf((float)D);

    // ---- K/V streaming -------------------------------------------------------
    const int64_t rowstride = (int64_t)p.Hkv * ROWB;    // bytes between keys
    const char *kbase = (const char *)p.k + (int64_t)ka * rowstride + (int64_t)g * ROWB;
    const char *vbase = (const char *)p.v + (int64_t)ka * rowstride + (int64_t)g * ROWB;
    char *kl = klds[wave];
    char *vl = vlds[wave];
    // K and V of the next block travel through registers in whole rows (a
    // load instruction covers RPL consecutive rows), with nontemporal loads:
    // the cache is read once
    u32x4 kn[NVL], vn[NVL];
    const int vrow = lane / CPR;
    const int vcol = (lane % CPR) * 16;
    auto load_block = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const int64_t off = (int64_t)min(kb + vrow + RPL * i, nk - 1) * rowstride + vcol;
            kn[i] = __builtin_nontemporal_load((const u32x4 *)(kbase + off));
            vn[i] = __builtin_nontemporal_load((const u32x4 *)(vbase + off));
        }
    };
    auto store_kv = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            *(u32x4 *)(kl + (vrow + RPL * i) * KROWB + vcol) = kn[i];
            *(u32x4 *)(vl + (vrow + RPL * i) * VROWB + vcol) = vn[i];
        }
    };
    // K operand read of this lane: key 16 half + n, dims 32 ks + 8 qq .. + 7
    // of map m
    const char *krd = kl + n * KROWB + 16 * qq;
    // transposing-read base of this lane: row 4 qq + (n / 4), dims 4 (n % 4)
    const int trbase = (4 * qq + (n >> 2)) * VROWB + 8 * (n & 3);

    if (kstart < kend) {
        load_block(kstart);
        store_kv();
    }
    for (int kb = kstart; kb < kend; kb += kBlockKeys) {
        const bool more = kb + kBlockKeys < kend;
        if (more)
            load_block(kb + kBlockKeys);

        // S^T for both maps and both 16-key halves, in log2 units
        f32x4 sc[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    acc = mma(*(const bf16x8 *)(krd + 16 * hf * KROWB + m * (ROWB / 2) + 64 * ks),
                              qf[m][ks], acc);
                sc[m][hf] = acc * c;
            }
        // keys past the sequence end or above the row's causal limit
        if (kb + kBlockKeys > kvis) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (kb + 16 * hf + 4 * qq + e > row_lim) {
                        sc[0][hf][e] = -INFINITY;
                        sc[1][hf][e] = -INFINITY;
                    }
        }
        // lazily raised maximum; rescale only when a score outgrows it by 2^8
        float bmax[2];
        bool grow = false;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            float x = fmaxf(fmaxf(sc[m][0][0], sc[m][0][1]), fmaxf(sc[m][0][2], sc[m][0][3]));
            x = fmaxf(x, fmaxf(fmaxf(sc[m][1][0], sc[m][1][1]), fmaxf(sc[m][1][2], sc[m][1][3])));
            bmax[m] = quad_max(x);
            grow |= bmax[m] > mrun[m] + kRescaleLog2;
        }
        if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const float mn = fmaxf(mrun[m], bmax[m]);
                const float a = mn == -INFINITY ? 1.f : exp2f(mrun[m] - mn);
                lsum[m] *= a;
#pragma unroll
                for (int t = 0; t < NDT; ++t)
                    o[m][t] *= a;
                mrun[m] = mn;
            }
        }
        // probabilities, packed as the P^T operand: k = 8 qq + 4 hf + e
        bf16x8 pf[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const float mref = mrun[m] == -INFINITY ? 0.f : mrun[m];
            float ps = 0.f;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float pv = exp2f(sc[m][hf][e] - mref);
                    ps += pv;
                    pf[m][4 * hf + e] = (bf16)pv;
                }
            lsum[m] += ps;
        }
        // O^T += V^T P^T, one V^T operand per 16-wide tile for both maps
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
            bf16x8 va;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (__attribute__((address_space(3))) bf16x4 *)(vl + trbase + 16 * hf * VROWB + 32 * t));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    va[4 * hf + e] = x[e];
            }
            o[0][t] = mma(va, pf[0], o[0][t]);
            o[1][t] = mma(va, pf[1], o[1][t]);
        }
        if (more)
            store_kv();
    }

    // ---- partial of this split -------------------------------------------
    if (!row_ok)
        return;
    const int64_t slot = ((int64_t)j * p.Hkv + g) * p.rmax + r;
    const float l0 = quad_sum(lsum[0]);
    const float l1 = quad_sum(lsum[1]);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        float *dst = p.ws_o + (slot * 2 + m) * (2 * D);
#pragma unroll
        for (int t = 0; t < NDT; ++t)
            *(f32x4 *)(dst + 16 * t + 4 * qq) = o[m][t];
    }
    if (qq == 0)
        *(f32x4 *)(p.ws_ml + slot * 4) = f32x4{mrun[0], l0, mrun[1], l1};
}


// Combine kernel: NG thread groups per output row.  A row's columns are
// NCH chunks of 16 bytes per map; thread (row, j, c) owns chunk c and the
// splits j, j + NG, j + 2 NG, ... of its row, four per round, and issues
// their (m, l) and O loads together, then merges them by log-sum-exp.  The
// NG groups of a row meet in LDS, where the row's first NCH threads merge
// them, combine the two maps, normalise and store.  NG grows with the
// longest row's split count (one round of loads per thread where it can):
// rows with few splits pack 256 / (NCH NG) rows into a workgroup, rows with
// many spread one row over more threads, so a small step's few rows still
// reach their partials in one memory round trip.
template <int D, int NG>
__global__ __launch_bounds__(256)
void diffattn_kv_combine(KvParams p)
{
    constexpr int W = 2 * D;          // columns of one map's row
    constexpr int NCH = W / 4;        // 16-byte chunks per row
    constexpr int TPR = NCH * NG;     // threads per row
    constexpr int RW = 256 / TPR;     // rows per workgroup
    constexpr int SW = TPR < 64 ? TPR : 64;   // lanes of one row in a wave
    constexpr int U = 4;              // splits per thread per round
    constexpr int LPC = D / NCH;      // lambda-vector elements per merging thread
    static_assert(RW * TPR == 256 && NCH <= 32 && LPC >= 1 && D % NCH == 0, "chunking");
    __shared__ f32x4 s_ml[RW][NG];
    __shared__ f32x4 s_o[RW][2][NG][NCH];
    const int t = threadIdx.x;
    const int rw = t / TPR, j = (t / NCH) % NG, c = t % NCH, sl = t % SW;
    int64_t wid = (int64_t)blockIdx.x * RW + rw;
    const int h = (int)(wid % p.H);
    wid /= p.H;
    const int i = (int)(wid % p.max_q);
    const int s_raw = (int)(wid / p.max_q);
    const int s = min(s_raw, p.nseq - 1);   // (clamped: loads stay in bounds)
    // everything that does not depend on the partials, loaded before any of
    // it is used (clamped indices, no loads under lane masks)
    const int64_t lo = (int64_t)h * p.lstride + c * LPC;
    float lq1[LPC], lk1[LPC], lq2[LPC], lk2[LPC];
#pragma unroll
    for (int e = 0; e < LPC; ++e) {
        lq1[e] = p.lq1[lo + e];
        lk1[e] = p.lk1[lo + e];
        lq2[e] = p.lq2[lo + e];
        lk2[e] = p.lk2[lo + e];
    }
    const f32x4 wc = p.w ? *(const f32x4 *)(p.w + 4 * c) : f32x4{1.f, 1.f, 1.f, 1.f};
    int qa, qe, ka, ke;
    if (p.cuq) {
        qa = p.cuq[s];
        qe = p.cuq[s + 1];
        ka = p.cuk[s];
        ke = p.cuk[s + 1];
    } else {
        qa = s * p.qlen_uniform;
        qe = qa + p.qlen_uniform;
        ka = s * p.klen_uniform;
        ke = ka + p.klen_uniform;
    }
    const int nq = qe - qa, nk = ke - ka;
    const bool live = s_raw < p.nseq && i < nq;
    const int g = h / p.G;
    const int r = i * p.G + h % p.G;
    // base of this sequence's splits: the split counts of the sequences
    // before it, summed over the SW lanes of the row in this wave
    int sbase;
    if (!p.cuk) {
        sbase = s * split_count(p.klen_uniform, p.ck);
    } else {
        int cnt = 0;
        for (int si = sl; si < s; si += SW)
            cnt += split_count(p.cuk[si + 1] - p.cuk[si], p.ck);
#pragma unroll
        for (int off = SW / 2; off >= 1; off >>= 1)
            cnt += __shfl_xor(cnt, off, 64);
        sbase = cnt;
    }
    // (the clamp only matters when cu_seqlens_k breaks its preconditions:
    // no read past the workspace)
    const int nsp = live ? max(0, min(split_count(nk, p.ck), p.nslots - sbase)) : 0;
    const int64_t slot0 = ((int64_t)sbase * p.Hkv + g) * p.rmax + r;
    const int64_t sstride = (int64_t)p.Hkv * p.rmax;   // between a row's splits

    // this thread's splits, U per round, merged online per map
    float M[2] = {-INFINITY, -INFINITY}, L[2] = {0.f, 0.f};
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int j0 = j; j0 < nsp; j0 += U * NG) {
        f32x4 ml[U], ob[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // past the row's last split: re-read split j0 (weight 0 below)
            const int js = j0 + u * NG < nsp ? j0 + u * NG : j0;
            const int64_t slot = slot0 + (int64_t)js * sstride;
            ml[u] = *(const f32x4 *)(p.ws_ml + slot * 4);
            const float *op = p.ws_o + slot * 2 * W + 4 * c;
            ob[u][0] = *(const f32x4 *)op;
            ob[u][1] = *(const f32x4 *)(op + W);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool in = j0 + u * NG < nsp;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const float mj = in ? ml[u][2 * m] : -INFINITY;
                const float mn = fmaxf(M[m], mj);
                // (0 for what is not there yet, and for splits no key of
                // the row reached)
                const float fa = M[m] == -INFINITY ? 0.f : exp2f(M[m] - mn);
                const float wj = mj == -INFINITY ? 0.f : exp2f(mj - mn);
                L[m] = L[m] * fa + ml[u][2 * m + 1] * wj;
                acc[m] = acc[m] * fa + ob[u][m] * wj;
                M[m] = mn;
            }
        }
    }
    if (c == 0)
        s_ml[rw][j] = f32x4{M[0], L[0], M[1], L[1]};
    s_o[rw][0][j][c] = acc[0];
    s_o[rw][1][j][c] = acc[1];
    __syncthreads();
    if (j != 0 || !live)
        return;

    // the row's first NCH threads: merge the groups, lambda, combine the
    // maps, RMSNorm over 2d, weight, (1 - lambda_init), store
    float Mg[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int q = 0; q < NG; ++q) {
        const f32x4 mlq = s_ml[rw][q];
        Mg[0] = fmaxf(Mg[0], mlq[0]);
        Mg[1] = fmaxf(Mg[1], mlq[2]);
    }
    float Lg[2] = {0.f, 0.f};
    f32x4 og[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int q = 0; q < NG; ++q) {
        const f32x4 mlq = s_ml[rw][q];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const float wq = mlq[2 * m] == -INFINITY ? 0.f : exp2f(mlq[2 * m] - Mg[m]);
            Lg[m] += mlq[2 * m + 1] * wq;
            og[m] += s_o[rw][m][q][c] * wq;
        }
    }
    float d1 = 0.f, d2 = 0.f;
#pragma unroll
    for (int e = 0; e < LPC; ++e) {
        d1 += lq1[e] * lk1[e];
        d2 += lq2[e] * lk2[e];
    }
#pragma unroll
    for (int off = NCH / 2; off >= 1; off >>= 1) {
        d1 += __shfl_xor(d1, off, 64);
        d2 += __shfl_xor(d2, off, 64);
    }
    const float lam = expf(d1) - expf(d2) + p.lambda_init;
    const float i1 = 1.f / Lg[0], i2 = lam / Lg[1];
    const f32x4 pre = og[0] * i1 - og[1] * i2;
    float ss = (pre[0] * pre[0] + pre[1] * pre[1]) + (pre[2] * pre[2] + pre[3] * pre[3]);
#pragma unroll
    for (int off = NCH / 2; off >= 1; off >>= 1)
        ss += __shfl_xor(ss, off, 64);
    const float scale = rsqrtf(ss / (float)W + p.eps) * (1.f - p.lambda_init);
    bf16x4 o4;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o4[e] = (bf16)(pre[e] * scale * wc[e]);
    *(bf16x4 *)((bf16 *)p.out + ((int64_t)(qa + i) * p.H + h) * W + 4 * c) = o4;
}

// Split policy: keys per split ck chosen from the total number of cache
// keys Tk so that all sequences together have at most kTargetWaves busy
// waves (one per SIMD), every one with the same ck keys whatever the length
// mix: with U waves per split (KV heads x 16-row blocks) and
// ck >= Tk / (kTargetWaves / U - nseq), the splits of all sequences number
// at most Tk / ck + nseq <= kTargetWaves / U (each sequence's last split may
// be short), so no launch spills a few waves into a second round.  When the
// sequences alone exceed that, every sequence is one split.  At least 128
// keys per split keep the partial traffic small against the cache bytes each
// wave reads.  Measured on 64 x 8192, 32 x [1024, 32768] (4 queries) and
// 8 x 4097 caches: this rule at 1024 waves beat 512, 768 and 2048 waves, and
// the earlier rule ck = Tk U / W at W = 1024 ... 8192 waves.  The bound
// nseq + kTargetWaves / U on the splits, which does not depend on Tk, sizes
// the workspace (with nseq * ceil(max_k / 128), whichever is smaller).
struct KvPlan {
    int nrb, nslots, ck, rmax;
    size_t ws_o_bytes, ws_ml_bytes;
};

constexpr int64_t kTargetWaves = 1024;

// Long query chunks (chunked prefill, a context-parallel shard, many
// speculative tokens) run on the prefill kernel, which reads each key tile
// once for 32 or 64 query rows of up to four heads -- over the sequences'
// whole key ranges, or over key splits whose partials the combine kernel
// below merges -- when its estimated time beats the split-KV pair's.  The
// prefill plan (split size and estimate) depends on the bounds alone,
// taken as uniform sequences; the pair's estimate uses the totals Tq and Tk
// too, since its time follows the keys actually cached: about 3.6 ps per
// (query row x head x key) at d = 64, 0.26 us per MB of K/V, 0.12 us per
// split of a row and 6.3 us (fitted to measured calls on this part).
// Below kChunkMinRows query rows per sequence the pair always runs.
constexpr int kChunkMinRows = 4;

enum KvPath { kPathSplitKv = 0, kPathChunk = 1, kPathChunkSplit = 2 };

// Tk < 0: the workspace bound only (ck left 0)
bool make_plan(int nseq, int max_q, int max_k, int G, int Hkv, int d, int64_t Tk, KvPlan &pl);

double split_kv_us(int nseq, int max_q, int max_k, int64_t Tq, int64_t Tk, int H, int Hkv,
                   int d)
{
    KvPlan pl;
    if (!make_plan(nseq, max_q, max_k, H / Hkv, Hkv, d, Tk, pl))
        return INFINITY;
    const double rowkeys = (double)H * std::min((double)max_q * Tk, (double)Tq * max_k);
    const double kv_mb = (double)Tk * Hkv * 4 * d * 2 / 1e6;
    const int splits = (max_k + pl.ck - 1) / pl.ck;
    return 3.62e-6 * rowkeys * d / 64 + 0.262 * kv_mb + 0.119 * splits + 6.3;
}

// The path of a call with these bounds and totals (Tq, Tk < 0: taken as
// uniform) and a workspace of ws_cap bytes: the lowest estimate among the
// paths whose partials fit, the split-KV path when none does (the call then
// refuses the workspace).  cp receives the prefill plan when a prefill path
// wins; need, when given, the workspace bytes of the chosen plan.
int kv_path(int nseq, int max_q, int max_k, int64_t Tq, int64_t Tk, int H, int Hkv, int d,
            size_t ws_cap, DiffattnChunkPlan *cp, size_t *need)
{
    KvPlan sk;
    const bool sk_ok = nseq >= 1 && H >= 1 && Hkv >= 1 && H % Hkv == 0 &&
                       make_plan(nseq, max_q, max_k, H / Hkv, Hkv, d, -1, sk);
    const size_t sk_need = sk_ok ? sk.ws_o_bytes + sk.ws_ml_bytes : SIZE_MAX;
    auto split_kv = [&]() {
        if (need)
            *need = sk_need;
        return (int)kPathSplitKv;
    };
    if (max_q < kChunkMinRows || nseq < 1 || max_k < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 ||
        !diffattn_supported_kv(DIFFATTN_BF16, d))
        return split_kv();
    DiffattnChunkPlan pl;
    if (!diffattn_chunk_plan(nseq, max_q, max_k, H, Hkv, d, 1, ws_cap, &pl))
        return split_kv();
    if (Tq < 0 || Tk < 0) {
        Tq = (int64_t)nseq * max_q;
        Tk = (int64_t)nseq * max_k;
    }
    if (sk_need <= ws_cap && !(pl.est_us < split_kv_us(nseq, max_q, max_k, Tq, Tk, H, Hkv, d)))
        return split_kv();
    if (cp)
        *cp = pl;
    if (need)
        *need = pl.ck > 0 ? pl.ws_o_bytes + pl.ws_ml_bytes : 0;
    return pl.ck > 0 ? kPathChunkSplit : kPathChunk;
}

// Tk < 0: the workspace bound only (ck left 0)
bool make_plan(int nseq, int max_q, int max_k, int G, int Hkv, int d, int64_t Tk, KvPlan &pl)
{
    if (nseq < 1 || max_q < 1 || max_k < 1 || G < 1 || Hkv < 1)
        return false;
    const int64_t rmax = (int64_t)G * max_q;
    if (rmax > (1 << 24))
        return false;
    pl.rmax = (int)rmax;
    pl.nrb = (int)((rmax + kRows - 1) / kRows);
    const int64_t per_split = (int64_t)Hkv * pl.nrb;
    // (also at most ceil(max_k / 128) splits per sequence, as ck >= 128)
    const int64_t nslots = std::min((kTargetWaves + per_split - 1) / per_split + nseq,
                                    (int64_t)nseq * ((max_k + 127) / 128));
    if (nslots > (1 << 30))
        return false;
    pl.nslots = (int)nslots;
    pl.ck = 0;
    if (Tk >= 0) {
        const int64_t fit = kTargetWaves / per_split - nseq;   // splits beyond one per sequence
        int64_t ck = fit > 0 ? (Tk + fit - 1) / fit : max_k;
        if (ck < 128)
            ck = 128;
        ck = (ck + kBlockKeys - 1) / kBlockKeys * kBlockKeys;
        if (ck > (1 << 30))
            return false;
        pl.ck = (int)ck;
    }
    const int64_t slots = nslots * Hkv * rmax * 2;
    pl.ws_o_bytes = (size_t)(slots * 2 * d * 4);
    pl.ws_ml_bytes = (size_t)(slots * 2 * 4);
    return true;
}

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

} // namespace

extern "C" int diffattn_supported_kv(int dtype, int d)
{
    return dtype == DIFFATTN_BF16 && (d == 32 || d == 64);
}

extern "C" int diffattn_check_cu_seqlens_kv(const int32_t *host_cu_q, const int32_t *host_cu_k,
                                            int32_t nseq, int32_t Tq, int32_t Tk,
                                            int32_t max_seqlen_q, int32_t max_seqlen_k,
                                            int causal)
{
    if (!host_cu_q || !host_cu_k || nseq < 0 || Tq < 0 || Tk < 0)
        return DIFFATTN_EINVAL;
    if (host_cu_q[0] != 0 || host_cu_k[0] != 0 || host_cu_q[nseq] != Tq ||
        host_cu_k[nseq] != Tk)
        return DIFFATTN_EINVAL;
    for (int32_t s = 0; s < nseq; ++s) {
        const int64_t nq = (int64_t)host_cu_q[s + 1] - host_cu_q[s];
        const int64_t nk = (int64_t)host_cu_k[s + 1] - host_cu_k[s];
        if (nq < 0 || nk < 0 || nq > max_seqlen_q || nk > max_seqlen_k)
            return DIFFATTN_EINVAL;
        if ((nq > 0 && nk == 0) || (causal && nq > nk))
            return DIFFATTN_EINVAL;
    }
    return DIFFATTN_OK;
}

extern "C" int diffattn_fwd_kv_path(int32_t nseq, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t Tq, int32_t Tk, int32_t H, int32_t Hkv, int32_t d,
                                    size_t workspace_bytes, size_t *workspace_needed)
{
    if (nseq < 1 || max_seqlen_q < 1 || max_seqlen_k < 1 || Tq < 1 || Tk < 1 || H < 1 ||
        Hkv < 1 || H % Hkv != 0 || !diffattn_supported_kv(DIFFATTN_BF16, d))
        return -1;
    return kv_path(nseq, max_seqlen_q, max_seqlen_k, Tq, Tk, H, Hkv, d, workspace_bytes, nullptr,
                   workspace_needed);
}

extern "C" size_t diffattn_fwd_kv_workspace_size(int32_t nseq, int32_t max_seqlen_q,
                                                 int32_t max_seqlen_k, int32_t H, int32_t Hkv,
                                                 int32_t d)
{
    if (H < 1 || Hkv < 1 || H % Hkv != 0 || d < 1)
        return 0;
    KvPlan pl;
    if (!make_plan(nseq, max_seqlen_q, max_seqlen_k, H / Hkv, Hkv, d, -1, pl))
        return 0;
    size_t need = pl.ws_o_bytes + pl.ws_ml_bytes;
    // (a call within these bounds may take the prefill kernel on key splits
    // instead, whose plan depends on the bounds alone)
    DiffattnChunkPlan cp;
    if (max_seqlen_q >= kChunkMinRows && diffattn_supported_kv(DIFFATTN_BF16, d) &&
        diffattn_chunk_plan(nseq, max_seqlen_q, max_seqlen_k, H, Hkv, d, 1, SIZE_MAX, &cp) &&
        cp.ck > 0)
        need = std::max(need, cp.ws_o_bytes + cp.ws_ml_bytes);
    return need;
}

namespace {

template <int D>
void launch_partial(int rt, unsigned blocks, hipStream_t st, const KvParams &p)
{
    if (rt == diffattn_rope::kBF16)
        hipLaunchKernelGGL((diffattn_kv_partial<D, diffattn_rope::kBF16>), dim3(blocks),
                           dim3(kThreads), 0, st, p);
    else if (rt == diffattn_rope::kF32)
        hipLaunchKernelGGL((diffattn_kv_partial<D, diffattn_rope::kF32>), dim3(blocks),
                           dim3(kThreads), 0, st, p);
    else
        hipLaunchKernelGGL((diffattn_kv_partial<D, diffattn_rope::kOff>), dim3(blocks),
                           dim3(kThreads), 0, st, p);
}

// The merge of up to `splits` splits per row: as many per memory round as
// the longest row has, in steps of 4, 8, 16 or 32 (a round of the longest
// row's width, where fewer would take two; narrower rounds hold fewer
// registers and issue fewer loads).
template <int D>
void launch_combine(int64_t splits, int64_t rows, hipStream_t st, const KvParams &p)
{
    constexpr int NCH = D / 2;   // 16-byte chunks of a 2d-wide fp32 row
    auto go = [&](auto ng) {
        constexpr int NG = decltype(ng)::value;
        const int64_t rw = 256 / (NCH * NG);
        hipLaunchKernelGGL((diffattn_kv_combine<D, NG>), dim3((unsigned)((rows + rw - 1) / rw)),
                           dim3(256), 0, st, p);
    };
    if (splits <= 4)
        go(std::integral_constant<int, 1>{});
    else if (splits <= 8)
        go(std::integral_constant<int, 2>{});
    else if (splits <= 16)
        go(std::integral_constant<int, 4>{});
    else
        go(std::integral_constant<int, 8>{});
}

// Validates the arguments, makes the split plan and launches both kernels
// with the workspace that `get_ws` returns for the plan's size (it returns
// a status and sets the pointer, or refuses the size).  ws_cap is the
// workspace's size: the path and plan are chosen among those that fit it.
template <typename GetWs>
int kv_impl(int dtype, const void *q, const void *k, const void *v,
            const float *lambda_q1, const float *lambda_k1, const float *lambda_q2,
            const float *lambda_k2, int32_t lambda_stride, float lambda_init,
            const float *subln_weight, float eps, int causal, const int32_t *cu_seqlens_q,
            const int32_t *cu_seqlens_k, int32_t nseq, int32_t max_seqlen_q,
            int32_t max_seqlen_k, int32_t Tq, int32_t Tk, int32_t H, int32_t Hkv, int32_t d,
            const void *rope_cos, const void *rope_sin, int32_t rope_len, int rope_dtype,
            int force_path, size_t ws_cap, GetWs get_ws, void *out, void *stream)
{
    if (force_path < -1 || force_path > kPathChunkSplit)
        return DIFFATTN_EINVAL;
    if (dtype != DIFFATTN_BF16 && dtype != DIFFATTN_F32)
        return DIFFATTN_EINVAL;
    if (Tq < 0 || Tk < 0 || H < 1 || Hkv < 1 || d < 1 || H % Hkv != 0 || nseq < 1)
        return DIFFATTN_EINVAL;
    if (causal != 0 && causal != 1)
        return DIFFATTN_EINVAL;
    if (!(eps >= 0.f) || !isfinite(eps) || !isfinite(lambda_init))
        return DIFFATTN_EINVAL;
    if (lambda_stride != 0 && lambda_stride < d)
        return DIFFATTN_EINVAL;
    if ((cu_seqlens_q == nullptr) != (cu_seqlens_k == nullptr))
        return DIFFATTN_EINVAL;
    if ((rope_cos == nullptr) != (rope_sin == nullptr))
        return DIFFATTN_EINVAL;
    if (rope_cos && rope_dtype != DIFFATTN_F32 && rope_dtype != DIFFATTN_BF16)
        return DIFFATTN_EINVAL;
    if (!cu_seqlens_q) {
        if (Tq % nseq != 0 || Tk % nseq != 0)
            return DIFFATTN_EINVAL;
        max_seqlen_q = Tq / nseq;
        max_seqlen_k = Tk / nseq;
        if (causal && max_seqlen_q > max_seqlen_k)
            return DIFFATTN_EINVAL;
        if (max_seqlen_q > 0 && max_seqlen_k == 0)
            return DIFFATTN_EINVAL;
    } else if (max_seqlen_q < 0 || max_seqlen_k < 0 || max_seqlen_q > Tq || max_seqlen_k > Tk) {
        return DIFFATTN_EINVAL;
    }
    if (!diffattn_supported_kv(dtype, d))
        return DIFFATTN_EUNSUPPORTED;
    if (Tq == 0 || max_seqlen_q == 0)
        return DIFFATTN_OK;   // no query rows: nothing to write
    if (max_seqlen_k == 0)
        return DIFFATTN_EINVAL;   // queries with no key at all
    if (!q || !k || !v || !out || !lambda_q1 || !lambda_k1 || !lambda_q2 || !lambda_k2)
        return DIFFATTN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (subln_weight && !aligned16(subln_weight)))
        return DIFFATTN_EINVAL;
    // the tables cover every position a new query can have (< nk)
    if (rope_cos && (rope_len < max_seqlen_k || !aligned16(rope_cos) || !aligned16(rope_sin)))
        return DIFFATTN_EINVAL;
    const int G = H / Hkv;
    KvParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.lq1 = lambda_q1;
    p.lk1 = lambda_k1;
    p.lq2 = lambda_q2;
    p.lk2 = lambda_k2;
    p.lstride = lambda_stride;
    p.w = subln_weight;
    p.cuq = cu_seqlens_q;
    p.cuk = cu_seqlens_k;
    p.rcos = rope_cos;
    p.rsin = rope_sin;
    p.rope_len = rope_cos ? rope_len : 1;
    p.lambda_init = lambda_init;
    p.eps = eps;
    p.H = H;
    p.Hkv = Hkv;
    p.G = G;
    p.nseq = nseq;
    p.causal = causal;
    p.qlen_uniform = cu_seqlens_q ? 0 : Tq / nseq;
    p.klen_uniform = cu_seqlens_q ? 0 : Tk / nseq;
    p.max_q = max_seqlen_q;
    hipStream_t st = (hipStream_t)stream;
    const int64_t rows2 = (int64_t)nseq * max_seqlen_q * H;   // output rows of the combine
    if (rows2 > 0x7fffffff)
        return DIFFATTN_EINVAL;
    // merge the splits of every row (at most those of ck keys of the
    // longest cache)
    auto combine = [&](int ck) {
        const int64_t kmax = cu_seqlens_q ? max_seqlen_k : Tk / nseq;
        const int64_t splits = (kmax + ck - 1) / ck;
        if (d == 64)
            launch_combine<64>(splits, rows2, st, p);
        else
            launch_combine<32>(splits, rows2, st, p);
    };

    // long query chunks: the prefill kernel, on whole key ranges (no
    // workspace) or on key splits merged by the combine kernel
    DiffattnChunkPlan cp;
    int path = force_path;
    if (path == -1) {
        path = kv_path(nseq, max_seqlen_q, max_seqlen_k, Tq, Tk, H, Hkv, d, ws_cap, &cp,
                       nullptr);
    } else if (path != kPathSplitKv) {
        // (the grid of the prefill kernel must fit, and for splits, a split
        // size whose partials fit the workspace must)
        if (!diffattn_chunk_plan(nseq, max_seqlen_q, max_seqlen_k, H, Hkv, d,
                                 path == kPathChunkSplit ? 2 : 0, ws_cap, &cp))
            return DIFFATTN_EINVAL;
    }
    if (path != kPathSplitKv) {
        void *workspace = nullptr;
        if (cp.ck > 0) {
            const int wst = get_ws(cp.ws_o_bytes + cp.ws_ml_bytes, workspace);
            if (wst != DIFFATTN_OK)
                return wst;
        }
        float *ws_o = (float *)workspace;
        float *ws_ml = cp.ck > 0 ? (float *)((char *)workspace + cp.ws_o_bytes) : nullptr;
        const int cst = diffattn_chunk_prefill(
            q, k, v, lambda_q1, lambda_k1, lambda_q2, lambda_k2, lambda_stride, lambda_init,
            subln_weight, eps, causal, cu_seqlens_q, cu_seqlens_k, nseq, max_seqlen_q, Tq, Tk,
            H, Hkv, d, rope_cos, rope_sin, rope_dtype, &cp, ws_o, ws_ml, out, stream);
        if (cst != DIFFATTN_OK || cp.ck == 0)
            return cst;
        p.ws_o = ws_o;
        p.ws_ml = ws_ml;
        p.rmax = cp.rmax;
        p.nslots = cp.nslots;
        p.ck = cp.ck;
        p.nrb = 0;   // (the partial kernel's; unused by the combine)
        combine(cp.ck);
        return hipGetLastError() == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
    }

    KvPlan pl;
    if (!make_plan(nseq, max_seqlen_q, max_seqlen_k, G, Hkv, d, Tk, pl))
        return DIFFATTN_EINVAL;
    void *workspace = nullptr;
    const int wst = get_ws(pl.ws_o_bytes + pl.ws_ml_bytes, workspace);
    if (wst != DIFFATTN_OK)
        return wst;
    p.ws_o = (float *)workspace;
    p.ws_ml = (float *)((char *)workspace + pl.ws_o_bytes);
    p.rmax = pl.rmax;
    p.nrb = pl.nrb;
    p.nslots = pl.nslots;
    p.ck = pl.ck;
    const int64_t waves1 = (int64_t)pl.nslots * Hkv * pl.nrb;
    const int64_t blocks1 = (waves1 + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks1 > 0x7fffffff)
        return DIFFATTN_EINVAL;
    const int rt = !rope_cos ? diffattn_rope::kOff
                             : (rope_dtype == DIFFATTN_BF16 ? diffattn_rope::kBF16 : diffattn_rope::kF32);
    if (d == 64)
        launch_partial<64>(rt, (unsigned)blocks1, st, p);
    else
        launch_partial<32>(rt, (unsigned)blocks1, st, p);
    combine(pl.ck);
    return hipGetLastError() == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}

// ---------------------------------------------------------------------------
// Static scratch of diffattn_fwd_kv_noalloc: the split partials live in this
// array instead of a caller's workspace.  Every GPU the library runs on holds
// its own copy (at its own address) until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: the device
// address is taken once per device with hipGetSymbolAddress (that device
// current) and only that address is handed to kernels.
static __device__ __align__(256) char scratch[DIFFATTN_KV_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::atomic<void *> g_scratch_dev[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch, looked up on the first
// call on that device.
int scratch_address(void *&ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return DIFFATTN_EHIP;
    ptr = g_scratch_dev[dev].load(std::memory_order_acquire);
    if (ptr)
        return DIFFATTN_OK;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_dev[dev].load(std::memory_order_relaxed);
    if (!ptr) {
        void *addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr)
            return DIFFATTN_EHIP;
        g_scratch_dev[dev].store(addr, std::memory_order_release);
        ptr = addr;
    }
    return DIFFATTN_OK;
}

} // namespace

extern "C" int diffattn_fwd_kv(int dtype, const void *q, const void *k, const void *v,
                               const float *lambda_q1, const float *lambda_k1,
                               const float *lambda_q2, const float *lambda_k2,
                               int32_t lambda_stride, float lambda_init,
                               const float *subln_weight, float eps, int causal,
                               const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                               int32_t nseq, int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t Tq, int32_t Tk, int32_t H, int32_t Hkv, int32_t d,
                               const void *rope_cos, const void *rope_sin, int32_t rope_len,
                               int rope_dtype, void *workspace, size_t workspace_bytes,
                               void *out, void *stream)
{
    if (workspace && !aligned16(workspace))
        return DIFFATTN_EINVAL;
    auto caller_ws = [&](size_t need, void *&ws) {
        if (!workspace || workspace_bytes < need)
            return (int)DIFFATTN_EINVAL;
        ws = workspace;
        return (int)DIFFATTN_OK;
    };
    return kv_impl(dtype, q, k, v, lambda_q1, lambda_k1, lambda_q2, lambda_k2, lambda_stride,
                   lambda_init, subln_weight, eps, causal, cu_seqlens_q, cu_seqlens_k, nseq,
                   max_seqlen_q, max_seqlen_k, Tq, Tk, H, Hkv, d, rope_cos, rope_sin, rope_len,
                   rope_dtype, -1, workspace ? workspace_bytes : 0, caller_ws, out, stream);
}

extern "C" int diffattn_fwd_kv_noalloc(int dtype, const void *q, const void *k, const void *v,
                                       const float *lambda_q1, const float *lambda_k1,
                                       const float *lambda_q2, const float *lambda_k2,
                                       int32_t lambda_stride, float lambda_init,
                                       const float *subln_weight, float eps, int causal,
                                       const int32_t *cu_seqlens_q,
                                       const int32_t *cu_seqlens_k, int32_t nseq,
                                       int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Tq,
                                       int32_t Tk, int32_t H, int32_t Hkv, int32_t d,
                                       const void *rope_cos, const void *rope_sin,
                                       int32_t rope_len, int rope_dtype, void *out,
                                       void *stream)
{
    // the size check comes first, so an oversized call touches no device
    auto static_ws = [&](size_t need, void *&ws) {
        if (need > (size_t)DIFFATTN_KV_SCRATCH_BYTES)
            return (int)DIFFATTN_ETOOLARGE;
        return scratch_address(ws);
    };
    return kv_impl(dtype, q, k, v, lambda_q1, lambda_k1, lambda_q2, lambda_k2, lambda_stride,
                   lambda_init, subln_weight, eps, causal, cu_seqlens_q, cu_seqlens_k, nseq,
                   max_seqlen_q, max_seqlen_k, Tq, Tk, H, Hkv, d, rope_cos, rope_sin, rope_len,
                   rope_dtype, -1, (size_t)DIFFATTN_KV_SCRATCH_BYTES, static_ws, out, stream);
}

extern "C" int diffattn_fwd_kv_on_path(int path, int dtype, const void *q, const void *k,
                                       const void *v, const float *lambda_q1,
                                       const float *lambda_k1, const float *lambda_q2,
                                       const float *lambda_k2, int32_t lambda_stride,
                                       float lambda_init, const float *subln_weight, float eps,
                                       int causal, const int32_t *cu_seqlens_q,
                                       const int32_t *cu_seqlens_k, int32_t nseq,
                                       int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Tq,
                                       int32_t Tk, int32_t H, int32_t Hkv, int32_t d,
                                       const void *rope_cos, const void *rope_sin,
                                       int32_t rope_len, int rope_dtype, void *workspace,
                                       size_t workspace_bytes, void *out, void *stream)
{
    if (path < 0 || (workspace && !aligned16(workspace)))
        return DIFFATTN_EINVAL;
    auto caller_ws = [&](size_t need, void *&ws) {
        if (!workspace || workspace_bytes < need)
            return (int)DIFFATTN_EINVAL;
        ws = workspace;
        return (int)DIFFATTN_OK;
    };
    return kv_impl(dtype, q, k, v, lambda_q1, lambda_k1, lambda_q2, lambda_k2, lambda_stride,
                   lambda_init, subln_weight, eps, causal, cu_seqlens_q, cu_seqlens_k, nseq,
                   max_seqlen_q, max_seqlen_k, Tq, Tk, H, Hkv, d, rope_cos, rope_sin, rope_len,
                   rope_dtype, path, workspace ? workspace_bytes : 0, caller_ws, out, stream);
}

extern "C" size_t diffattn_fwd_kv_path_workspace_size(int path, int32_t nseq,
                                                      int32_t max_seqlen_q,
                                                      int32_t max_seqlen_k, int32_t H,
                                                      int32_t Hkv, int32_t d)
{
    if (nseq < 1 || max_seqlen_q < 1 || max_seqlen_k < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 ||
        !diffattn_supported_kv(DIFFATTN_BF16, d))
        return 0;
    if (path == kPathSplitKv) {
        KvPlan pl;
        if (!make_plan(nseq, max_seqlen_q, max_seqlen_k, H / Hkv, Hkv, d, -1, pl))
            return 0;
        return pl.ws_o_bytes + pl.ws_ml_bytes;
    }
    DiffattnChunkPlan cp;
    if (path == kPathChunkSplit &&
        diffattn_chunk_plan(nseq, max_seqlen_q, max_seqlen_k, H, Hkv, d, 2, SIZE_MAX, &cp))
        return cp.ws_o_bytes + cp.ws_ml_bytes;
    return 0;
}

// ---------------------------------------------------------------------------
// Cache update of a decode step.  Thread = one 16-byte chunk of one new
// token's key row (the first half of the grid) or value row (the second
// half; both rows are Hkv x 2d elements).  The token's sequence comes from
// a binary search of cu_seqlens_q; its cache row and position from the
// sequence's bounds.
namespace {

struct AppendParams {
    const char *k_new, *v_new;
    char *k_cache, *v_cache;
    const int32_t *cuq, *cuk;
    const void *rcos, *rsin;
    int32_t nseq, Tq, Hkv, rope_len;
    int32_t qlen_uniform, klen_uniform;
};

template <typename E, int D, int RT>
__global__ __launch_bounds__(256) void diffattn_kv_append_kernel(AppendParams p)
{
    constexpr int ES = (int)sizeof(E);
    constexpr int CPH = D * ES / 16;   // 16-byte chunks per d-wide half-head
    const int cpt = 2 * p.Hkv * CPH;   // chunks per token row
    const int64_t per = (int64_t)p.Tq * cpt;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= 2 * per)
        return;
    const bool is_v = idx >= per;
    const int64_t e = is_v ? idx - per : idx;
    const int t = (int)(e / cpt), c = (int)(e % cpt);
    int qa, nq, ka, nk;
    if (p.cuq) {
        int lo = 0, hi = p.nseq;   // last sequence with cu_q[s] <= t
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.cuq[mid] <= t)
                lo = mid;
            else
                hi = mid;
        }
        qa = p.cuq[lo];
        nq = p.cuq[lo + 1] - qa;
        ka = p.cuk[lo];
        nk = p.cuk[lo + 1] - ka;
    } else {
        const int s = t / p.qlen_uniform;
        qa = s * p.qlen_uniform;
        nq = p.qlen_uniform;
        ka = s * p.klen_uniform;
        nk = p.klen_uniform;
    }
    if (nq > nk)
        return;   // broken precondition: the new rows would leave the sequence
    const int i = t - qa;
    const int64_t rowb = (int64_t)2 * p.Hkv * D * ES;   // bytes per token row
    const int64_t row = (int64_t)ka + nk - nq + i;
    u32x4 x = *(const u32x4 *)((is_v ? p.v_new : p.k_new) + (int64_t)t * rowb + c * 16);
    if constexpr (RT != diffattn_rope::kOff) {
        if (!is_v) {
            typedef diffattn_rope::Rope<E, RT> R;
            const int pos = min(nk - nq + i, p.rope_len - 1);
            const int j = (c % CPH) * (16 / ES) / 2;   // first pair of the chunk
            x = R::rotate(x, R::coef(p.rcos, p.rsin, pos, j, D));
        }
    }
    *(u32x4 *)((is_v ? p.v_cache : p.k_cache) + row * rowb + c * 16) = x;
}

template <typename E, int D>
void launch_append(int rt, unsigned blocks, hipStream_t st, const AppendParams &p)
{
    if (rt == diffattn_rope::kBF16)
        hipLaunchKernelGGL((diffattn_kv_append_kernel<E, D, diffattn_rope::kBF16>), dim3(blocks),
                           dim3(256), 0, st, p);
    else if (rt == diffattn_rope::kF32)
        hipLaunchKernelGGL((diffattn_kv_append_kernel<E, D, diffattn_rope::kF32>), dim3(blocks),
                           dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL((diffattn_kv_append_kernel<E, D, diffattn_rope::kOff>), dim3(blocks),
                           dim3(256), 0, st, p);
}

} // namespace

extern "C" int diffattn_kv_append(int dtype, const void *k_new, const void *v_new,
                                  const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                  int32_t nseq, int32_t max_seqlen_k, int32_t Tq, int32_t Tk,
                                  int32_t Hkv, int32_t d, const void *rope_cos,
                                  const void *rope_sin, int32_t rope_len, int rope_dtype,
                                  void *k_cache, void *v_cache, void *stream)
{
    if (dtype != DIFFATTN_BF16 && dtype != DIFFATTN_F32)
        return DIFFATTN_EINVAL;
    if (Tq < 0 || Tk < 0 || Hkv < 1 || d < 1 || nseq < 1)
        return DIFFATTN_EINVAL;
    if ((cu_seqlens_q == nullptr) != (cu_seqlens_k == nullptr))
        return DIFFATTN_EINVAL;
    if ((rope_cos == nullptr) != (rope_sin == nullptr))
        return DIFFATTN_EINVAL;
    if (rope_cos && rope_dtype != DIFFATTN_F32 && rope_dtype != DIFFATTN_BF16)
        return DIFFATTN_EINVAL;
    if (!cu_seqlens_q) {
        if (Tq % nseq != 0 || Tk % nseq != 0 || Tq / nseq > Tk / nseq)
            return DIFFATTN_EINVAL;
        max_seqlen_k = Tk / nseq;
    } else if (max_seqlen_k < 0 || max_seqlen_k > Tk) {
        return DIFFATTN_EINVAL;
    }
    if (d != 16 && d != 32 && d != 64)
        return DIFFATTN_EUNSUPPORTED;
    if (Tq == 0)
        return DIFFATTN_OK;
    if (!k_new || !v_new || !k_cache || !v_cache)
        return DIFFATTN_EINVAL;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
        return DIFFATTN_EINVAL;
    if (rope_cos && (rope_len < max_seqlen_k || rope_len < 1 || !aligned16(rope_cos) ||
                     !aligned16(rope_sin)))
        return DIFFATTN_EINVAL;
    const int es = dtype == DIFFATTN_F32 ? 4 : 2;
    const int64_t threads = (int64_t)2 * Tq * (2 * Hkv * d * es / 16);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffff)
        return DIFFATTN_EINVAL;
    AppendParams p;
    p.k_new = (const char *)k_new;
    p.v_new = (const char *)v_new;
    p.k_cache = (char *)k_cache;
    p.v_cache = (char *)v_cache;
    p.cuq = cu_seqlens_q;
    p.cuk = cu_seqlens_k;
    p.rcos = rope_cos;
    p.rsin = rope_sin;
    p.nseq = nseq;
    p.Tq = Tq;
    p.Hkv = Hkv;
    p.rope_len = rope_cos ? rope_len : 1;
    p.qlen_uniform = cu_seqlens_q ? 0 : Tq / nseq;
    p.klen_uniform = cu_seqlens_q ? 0 : Tk / nseq;
    const int rt = !rope_cos ? diffattn_rope::kOff
                             : (rope_dtype == DIFFATTN_BF16 ? diffattn_rope::kBF16 : diffattn_rope::kF32);
    hipStream_t st = (hipStream_t)stream;
    const unsigned nb = (unsigned)blocks;
    if (dtype == DIFFATTN_BF16) {
        if (d == 64)
            launch_append<bf16, 64>(rt, nb, st, p);
        else if (d == 32)
            launch_append<bf16, 32>(rt, nb, st, p);
        else
            launch_append<bf16, 16>(rt, nb, st, p);
    } else {
        if (d == 64)
            launch_append<float, 64>(rt, nb, st, p);
        else if (d == 32)
            launch_append<float, 32>(rt, nb, st, p);
        else
            launch_append<float, 16>(rt, nb, st, p);
    }
    return hipGetLastError() == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}
