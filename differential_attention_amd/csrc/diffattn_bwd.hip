// diffattn_bwd.hip -- backward pass of the differential-attention prefill
// for CDNA4 (gfx950).
//
// The gradients are those of diffattn_bwd in include/diffattn.h: the
// DiffTransformer page's MultiHeadDifferentialAttention.forward (and the
// gist's two-SDPA form) differentiated through the RMSNorm, the
// lambda-weighted difference of the two softmax maps and the lambda
// re-parameterisation.  The training forward (diffattn_fwd_train) saved,
// per row and map, the log2-sum-exp of the scaled scores and the
// normalised output O_m.
//
// Four kernels, no atomics (the result is bitwise reproducible):
//
//  prep     workgroups of four waves per head, each wave striding over the
//           tokens: pre = O_1 - lambda O_2 and its RMSNorm backward dpre
//           (stored bf16 as the MFMA operand; the maps' output gradients
//           are dO_1 = dpre and dO_2 = -lambda dpre, and -lambda is applied
//           in fp32 where map 2 uses it), D'_m = <dpre, O_m> from the
//           rounded dpre (so that the softmax gradients of a row sum to
//           zero; stored as D'_1 and lambda D'_2), lambda per head, and
//           per-workgroup partial sums of the weight and lambda gradients.
//  reduce   one workgroup: the partial sums in a fixed order, and the
//           lambda-vector gradients by the chain rule.
//  dq       query-outer, as the forward: one workgroup = (sequence, head,
//           128 queries), wave = (map, 32 queries).  Over K/V tiles
//           double-buffered in LDS (the next tile travels through registers
//           while the current one is used): S^T = K Q^T,
//           P^T = exp2(S^T c - lse), dP'^T = V dpre^T,
//           dS_1^T = P_1^T (dP'^T - D'_1) or
//           dS_2^T = P_2^T (-lambda dP'^T + lambda D'_2), dQ^T += K^T dS^T
//           (K^T through the transposing LDS read, dS^T straight from the
//           accumulator).
//  dkdv     key-outer: one workgroup = (sequence, KV head, 128 keys).  Four
//           waves (32 keys each, both maps) compute S_m = Q_m K_m^T, P_m,
//           dS_1 = P_1 (dP - D'_1), dS_2 = P_2 (-lambda dP + lambda D'_2)
//           and dK_m^T += Q_m^T dS_m, and form W = P_1 - lambda P_2 in fp32
//           (then rounded); the other four waves (same keys) compute
//           dP = dpre V^T once for both maps one query tile ahead (handed
//           over as dP - D'_1, with lambda D'_2 - lambda D'_1 per row, so
//           that map 2's factor is one FMA) and add
//           dV^T += dpre^T W one query tile behind, dP and W travelling
//           through LDS.  Query tiles (Q, dpre, lse, D) of all G heads of
//           the group rotate through four LDS stages.
//
// All contractions run on v_mfma_f32_32x32x16_bf16 with fp32 accumulators;
// P, W and dS are rounded to bf16 as operands, as is dpre.
//
// The exact path serves the (storage, d) pairs the MFMA kernels do not
// (fp32 storage at d = 16, 32, 64; bf16 at d = 16): the same prep and
// reduce with dpre kept in fp32, then a dq kernel with one wave per query
// row and a dk/dv kernel with one wave per key row, lanes over the row's
// dimensions, every score and dot product a 64-lane fp32 sum.  Nothing is
// rounded below fp32 before the final store; it is built for correctness at
// the small scales fp32 training runs at, not for speed.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "diffattn.h"

namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 512;   // 8 waves: 2 maps x 4 blocks of 32 rows
constexpr int kSubs = 4;        // blocks of 32 rows per map
constexpr int kTile = 32 * kSubs;   // queries (dq) or keys (dkdv) per workgroup
constexpr int kInner = 64;      // keys per staged K/V tile of dq
constexpr int kPrepPerHead = 256;  // prep waves per head (4 per workgroup)

__device__ inline f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (offset inside a 32-row block) of accumulator element a of a lane in
// half h of a 32x32 MFMA result.
__device__ constexpr int acc_row(int a, int h) { return 8 * (a / 4) + 4 * h + (a % 4); }

// Accumulator elements a0 .. a0+7 as a bf16 operand: rows 16 (a0/8) + 8t +
// 4h + e (t = 0, 1), the contraction order of tr_operand below.
__device__ inline bf16x8 pack8(const f32x16 &s, int a0)
{
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        f[e] = (bf16)s[a0 + e];
    return f;
}

// A operand X^T for a contraction over 16 rows of a row-major bf16 LDS tile
// X: lane (column i, half h) gets X[step_row + 8t + 4h + e][i] for t, e in
// 0..3 (two transposing reads).  col_byte selects the 32 columns.
// Swizzled tiles (swz): the 16-byte chunk c of tile row r is stored at
// chunk c ^ ((r >> 2) & 3).  LDS serves 256 bytes per cycle: a plain
// 16-byte read by 16 lanes (here 16 consecutive rows at one chunk), a
// transposing 8-byte read by 32 lanes (4 consecutive rows x 64 bytes).
// With a row pitch of 64 mod 256 bytes the 4 rows of a transposing read
// tile the 256 bytes (the swizzle only permutes chunks inside each row's
// aligned group of 4), and the 16 rows of a plain read at one chunk land on
// 16 distinct 16-byte slots (rows 4 apart share a 64-byte window and the
// swizzle spreads them across it).  Every reader's swizzle is a lane
// constant, folded into its base addresses.
struct TrOperand {
    int base[2];   // for the two 8-row halves of a 16-row step
    __device__ TrOperand(int lane, int rowb, bool swz = false)
    {
        const int j = lane & 15;
        // this lane's 8 bytes: row 8 t + 4 (lane >> 5) + j / 4 of the step,
        // chunk 2 ((lane >> 4) & 1) + (j & 3) / 2 of the column block (a
        // multiple of 4 chunks), half j & 1; steps start at multiples of 16
        // rows, so the row's swizzle bits are (2 t + (lane >> 5)) & 3
        const int ch = 2 * ((lane >> 4) & 1) + ((j & 3) >> 1);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int sw = swz ? (2 * t + (lane >> 5)) & 3 : 0;
            base[t] = (8 * t + 4 * (lane >> 5) + (j >> 2)) * rowb + 16 * (ch ^ sw) + 8 * (j & 1);
        }
    }
    __device__ inline bf16x8 load(const char *tile, int rowb, int step_row, int col_byte) const
    {
        bf16x8 f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const char *addr = tile + base[t] + step_row * rowb + col_byte;
            const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4 *)addr);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                f[4 * t + e] = x[e];
        }
        return f;
    }
};

__device__ inline float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

struct BwdParams {
    const bf16 *q, *k, *v, *dy;
    const float *lse;    // [T][H][2]
    const float *o12;    // [T][H][2][2d]
    const float *lq1, *lk1, *lq2, *lk2;
    int64_t lstride;
    const float *w;
    const int32_t *cu;
    bf16 *dq, *dk, *dv;
    float *dlq1, *dlk1, *dlq2, *dlk2, *dw;
    // workspace
    bf16 *dpre;          // [T][H][2d]: dO_1 = dpre, dO_2 = -lambda dpre
    float *dd;           // [T][H][2]: <dpre, O_1>, lambda <dpre, O_2>
    float *lam;          // [H]
    float *part_dw;      // [nprep][2d]
    float *part_dl;      // [nprep]
    float lambda_init, eps;
    int32_t T, H, Hkv, G, nseq, seqlen_uniform, causal, ntile;
};

__device__ inline void seq_bounds(const BwdParams &p, int s, int &s0, int &s1)
{
    if (p.cu) {
        s0 = p.cu[s];
        s1 = p.cu[s + 1];
    } else {
        s0 = s * p.seqlen_uniform;
        s1 = s0 + p.seqlen_uniform;
    }
}

__device__ inline float head_lambda(const BwdParams &p, int h, int lane, int D)
{
    const int64_t lo = (int64_t)h * p.lstride;
    float a = 0.f, b = 0.f;
    for (int cc = lane; cc < D; cc += 64) {
        a += p.lq1[lo + cc] * p.lk1[lo + cc];
        b += p.lq2[lo + cc] * p.lk2[lo + cc];
    }
    return expf(wave_sum(a)) - expf(wave_sum(b)) + p.lambda_init;
}

// ---------------------------------------------------------------------------
// prep: RMSNorm / combine backward per row, D_m, partial weight and lambda
// gradients.  Wave w serves head w % H and tokens w / H, w / H + nper, ...
// Sum over the 16 lanes of a row group (lanes 16 r .. 16 r + 15).
__device__ inline float seg16_sum(float x)
{
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

// N consecutive floats / bf16 values of a row, in 16-, 8- or 4-byte pieces.
template <int N> __device__ inline void load_f32(float (&x)[N], const float *src)
{
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int k = 0; k < N / 4; ++k) {
            const float4 v = *(const float4 *)(src + 4 * k);
            x[4 * k] = v.x, x[4 * k + 1] = v.y, x[4 * k + 2] = v.z, x[4 * k + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
            const float2 v = *(const float2 *)(src + 2 * k);
            x[2 * k] = v.x, x[2 * k + 1] = v.y;
        }
    }
}
template <int N> __device__ inline void load_f32_nt(float (&x)[N], const float *src)
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int k = 0; k < N / 4; ++k) {
            const f4 v = __builtin_nontemporal_load((const f4 *)(src + 4 * k));
            x[4 * k] = v.x, x[4 * k + 1] = v.y, x[4 * k + 2] = v.z, x[4 * k + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
            const f2 v = __builtin_nontemporal_load((const f2 *)(src + 2 * k));
            x[2 * k] = v.x, x[2 * k + 1] = v.y;
        }
    }
}
template <int N> __device__ inline void load_bf16(float (&x)[N], const bf16 *src)
{
    typedef __bf16 bv __attribute__((ext_vector_type(N)));
    const bv v = *(const bv *)src;
#pragma unroll
    for (int k = 0; k < N; ++k)
        x[k] = (float)v[k];
}
template <int N> __device__ inline void store_bf16(bf16 *dst, const bf16 (&x)[N])
{
    typedef __bf16 bv __attribute__((ext_vector_type(N)));
    bv v;
#pragma unroll
    for (int k = 0; k < N; ++k)
        v[k] = x[k];
    *(bv *)dst = v;
}
template <int N> __device__ inline void store_f32(float *dst, const float (&x)[N])
{
    typedef float fv __attribute__((ext_vector_type(N)));
    fv v;
#pragma unroll
    for (int k = 0; k < N; ++k)
        v[k] = x[k];
    *(fv *)dst = v;
}
// a row of storage-type values as floats / floats stored in a row of the
// storage or dpre type
template <int N> __device__ inline void load_row(float (&x)[N], const bf16 *src) { load_bf16(x, src); }
template <int N> __device__ inline void load_row(float (&x)[N], const float *src) { load_f32(x, src); }
template <int N> __device__ inline void store_row(bf16 *dst, const bf16 (&x)[N]) { store_bf16(dst, x); }
template <int N> __device__ inline void store_row(float *dst, const float (&x)[N]) { store_f32(dst, x); }

// E: storage type of dout; DP: type of the stored dpre (bf16 as the MFMA
// operand, whose rounded value then also enters D'_m; fp32 on the exact
// path)
template <typename E, typename DP, int D>
__global__ __launch_bounds__(256) void bwd_prep(BwdParams p)
{
    // a wave takes four (token, head) rows at a time, 16 lanes per row and
    // CPL consecutive columns per lane, so every load and store is 8 to 32
    // bytes wide and the row sums are 16-lane reductions
    constexpr int CPL = 2 * D / 16;   // columns per lane
    __shared__ float red_dw[4][2 * D];
    __shared__ float red_dl[4];
    const int lane = threadIdx.x & 63, wv4 = threadIdx.x >> 6;
    const int sub = lane >> 4, l16 = lane & 15;
    // the four waves of a workgroup serve one head: wave w of the head takes
    // the row groups w, w + kPrepPerHead, ... (tokens 4 g .. 4 g + 3)
    const int h = blockIdx.x % p.H;
    const int wid = (blockIdx.x / p.H) * 4 + wv4;   // wave index within the head
    const float lam = head_lambda(p, h, lane, D);
    if (blockIdx.x < p.H && threadIdx.x == 0)
        p.lam[h] = lam;
    const float sc = 1.f - p.lambda_init;
    float wv[CPL], dwp[CPL];
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
        wv[cc] = p.w ? p.w[CPL * l16 + cc] : 1.f;
        dwp[cc] = 0.f;
    }
    float dlp = 0.f;
    for (int g0 = 4 * wid; g0 < p.T; g0 += 4 * kPrepPerHead) {
        const int t = g0 + sub;
        const bool ok = t < p.T;
        const int64_t row = (int64_t)(ok ? t : 0) * p.H + h;
        float a1[CPL], a2[CPL], dyv[CPL];
        if (ok) {
            // (the saved maps are read once: nontemporal loads)
            const float *o1 = p.o12 + row * 2 * (2 * D) + CPL * l16;
            load_f32_nt(a1, o1);
            load_f32_nt(a2, o1 + 2 * D);
            load_row(dyv, (const E *)p.dy + row * (2 * D) + CPL * l16);
        } else {
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc)
                a1[cc] = a2[cc] = dyv[cc] = 0.f;
        }
        float pre[CPL], g[CPL];
        float ss = 0.f, gp = 0.f;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            pre[cc] = a1[cc] - lam * a2[cc];
            ss += pre[cc] * pre[cc];
            g[cc] = dyv[cc] * wv[cc] * sc;
            gp += g[cc] * pre[cc];
        }
        ss = seg16_sum(ss);
        gp = seg16_sum(gp);
        const float r = rsqrtf(ss / (float)(2 * D) + p.eps);
        const float r3 = r * r * r * gp / (float)(2 * D);
        float d1 = 0.f, d2 = 0.f;
        DP b1[CPL];
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const float dpre = r * g[cc] - r3 * pre[cc];
            b1[cc] = (DP)dpre;
            d1 += (float)b1[cc] * a1[cc];
            d2 += (float)b1[cc] * a2[cc];
            dlp -= dpre * a2[cc];
            dwp[cc] += dyv[cc] * pre[cc] * r * sc;
        }
        d1 = seg16_sum(d1);
        d2 = seg16_sum(d2);
        if (ok) {
            store_row((DP *)p.dpre + row * (2 * D) + CPL * l16, b1);
            if (l16 == 0) {
                p.dd[row * 2] = d1;
                p.dd[row * 2 + 1] = lam * d2;
            }
        }
    }
    // the wave's four row groups, then the workgroup's four waves, summed in
    // a fixed order: one partial per workgroup, part[blockIdx.x] (head h =
    // blockIdx.x % H)
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
        dwp[cc] += __shfl_xor(dwp[cc], 16, 64);
        dwp[cc] += __shfl_xor(dwp[cc], 32, 64);
    }
    if (sub == 0) {
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
            red_dw[wv4][CPL * l16 + cc] = dwp[cc];
    }
    dlp = wave_sum(dlp);
    if (lane == 0)
        red_dl[wv4] = dlp;
    __syncthreads();
    for (int c = threadIdx.x; c < 2 * D; c += 256)
        p.part_dw[(int64_t)blockIdx.x * 2 * D + c] =
            (red_dw[0][c] + red_dw[1][c]) + (red_dw[2][c] + red_dw[3][c]);
    if (threadIdx.x == 0)
        p.part_dl[blockIdx.x] = (red_dl[0] + red_dl[1]) + (red_dl[2] + red_dl[3]);
}

// ---------------------------------------------------------------------------
// reduce: fixed-order sums of the partials, lambda-vector gradients.
constexpr int kPrepBlocksPerHead = kPrepPerHead / 4;

template <int D>
__global__ __launch_bounds__(1024) void bwd_reduce(BwdParams p)
{
    // 1024 threads: (column c, part j) sums partials j, j + 8, ... of its
    // column, then the 8 parts are added in a fixed order
    constexpr int NPART = 1024 / (2 * D);
    __shared__ float red[1024];
    __shared__ float dlh[256];   // per head (H <= 256)
    const int tid = threadIdx.x;
    const int nblk = p.H * kPrepBlocksPerHead;
    {
        const int c = tid % (2 * D), j = tid / (2 * D);
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        int w = j;
        for (; w + 3 * NPART < nblk; w += 4 * NPART)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                acc[u] += p.part_dw[(int64_t)(w + u * NPART) * 2 * D + c];
        for (; w < nblk; w += NPART)
            acc[0] += p.part_dw[(int64_t)w * 2 * D + c];
        red[tid] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
    for (int h = tid; h < p.H; h += 1024) {
        float acc = 0.f;
        for (int k = 0; k < kPrepBlocksPerHead; ++k)
            acc += p.part_dl[k * p.H + h];
        dlh[h] = acc;
    }
    __syncthreads();
    if (p.dw && tid < 2 * D) {
        float acc = 0.f;
        for (int j = 0; j < NPART; ++j)
            acc += red[j * 2 * D + tid];
        p.dw[tid] = acc;
    }
    const int nsets = p.lstride ? p.H : 1;
    for (int idx = tid; idx < nsets * D; idx += 1024) {
        const int st = idx / D, c = idx % D;
        float dlam = 0.f;
        if (p.lstride) {
            dlam = dlh[st];
        } else {
            for (int h = 0; h < p.H; ++h)
                dlam += dlh[h];
        }
        const int64_t off = (int64_t)st * p.lstride;
        float a = 0.f, b = 0.f;
        for (int j = 0; j < D; ++j) {
            a += p.lq1[off + j] * p.lk1[off + j];
            b += p.lq2[off + j] * p.lk2[off + j];
        }
        const float ea = expf(a), eb = expf(b);
        p.dlq1[off + c] = dlam * ea * p.lk1[off + c];
        p.dlk1[off + c] = dlam * ea * p.lq1[off + c];
        p.dlq2[off + c] = -dlam * eb * p.lk2[off + c];
        p.dlk2[off + c] = -dlam * eb * p.lq2[off + c];
    }
}

// ---------------------------------------------------------------------------
// Staging of row tiles: `rows` rows of ROWB bytes from global rows `stride`
// bytes apart into an LDS tile with rows LROW bytes apart, in 16-byte
// chunks spread over the workgroup; rows at or past `valid` read as zero.
// load() fills this thread's registers (the loads stay in flight), store()
// writes them to LDS, so a tile can travel while the previous one is used.
template <int ROWB, int LROW, int ROWS, bool SWZ = false>
struct Stager {
    static constexpr int CPR = ROWB / 16;
    static constexpr int N = (ROWS * CPR + kThreads - 1) / kThreads;   // chunks per thread
    u32x4 r[N];
    __device__ inline void load(const char *src, int64_t stride, int valid)
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = threadIdx.x + i * kThreads;
            const int row = idx / CPR, c = (idx % CPR) * 16;
            r[i] = u32x4{0u, 0u, 0u, 0u};
            if (idx < ROWS * CPR && row < valid)
                r[i] = *(const u32x4 *)(src + row * stride + c);
        }
    }
    __device__ inline void store(char *lds) const
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = threadIdx.x + i * kThreads;
            const int row = idx / CPR, c = ((idx % CPR) ^ (SWZ ? (row >> 2) & 3 : 0)) * 16;
            if (idx < ROWS * CPR)
                *(u32x4 *)(lds + row * LROW + c) = r[i];
        }
    }
};

// ---------------------------------------------------------------------------
// dq: query-outer; K/V tiles of kInner keys double-buffered in LDS.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq(BwdParams p)
{
    constexpr int ROWB = 2 * D * 2;        // K or V row bytes
    // K rows are read both as plain 16-byte rows and through the transposing
    // read, V rows plainly: swizzled tiles with a pitch of 64 mod 256 bytes
    // (TrOperand) keep both on distinct banks (d = 32: 192 = -64 mod 256)
    constexpr int LROW = ROWB + 64;
    constexpr int NKS = D / 16;            // QK contraction steps
    constexpr int NVS = 2 * D / 16;        // dO V contraction steps
    constexpr int NDB = D / 32;            // 32-dim blocks of dQ
    constexpr int TILEB = kInner * LROW;
    // two stages, each a K tile then a V tile; separate objects so that the
    // compiler can see stores to one never alias loads from the other
    __shared__ __attribute__((aligned(16))) char st0[2 * TILEB];
    __shared__ __attribute__((aligned(16))) char st1[2 * TILEB];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = lane & 31, h = lane >> 5;
    const int map = wave / kSubs, sub = wave % kSubs;

    // longest query tiles first
    const int pairs = p.nseq * p.H;
    const int tile = p.ntile - 1 - blockIdx.x / pairs;
    const int rem = blockIdx.x % pairs;
    const int s = rem / p.H, head = rem % p.H;
    const int g = head / p.G;
    int s0, s1;
    seq_bounds(p, s, s0, s1);
    const int q0 = s0 + tile * kTile;
    if (q0 >= s1)
        return;
    const int wq = q0 + 32 * sub + n;      // this lane's query
    const bool qok = wq < s1;
    const int64_t qrow = (int64_t)wq * p.H + head;

    bf16x8 qf[NKS], df[NVS];
    // dS = P (dpf dP' - dval) with dP' = dpre V^T: map 1 dpf = 1, dval = D'_1;
    // map 2 dpf = -lambda, dval = -lambda D'_2 (dO_2 = -lambda dpre)
    const float dpf = map ? -p.lam[head] : 1.f;
    float lse = INFINITY, dval = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        qf[ks] = qok ? *(const bf16x8 *)(p.q + (qrow * 2 + map) * D + 16 * ks + 8 * h) : bf16x8{};
#pragma unroll
    for (int ks = 0; ks < NVS; ++ks)
        df[ks] = qok ? *(const bf16x8 *)(p.dpre + qrow * (2 * D) + 16 * ks + 8 * h) : bf16x8{};
    if (qok) {
        lse = p.lse[qrow * 2 + map];
        dval = map ? -p.dd[qrow * 2 + 1] : p.dd[qrow * 2];
    }
    f32x16 dqa[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
        dqa[db] = f32x16{};
    const float c = kLog2e * rsqrtf((float)D);
    const TrOperand tr(lane, LROW, true);
    // plain reads of row 32 b + n of a swizzled tile: chunk 2 ks + h lies at
    // (2 ks + h) ^ a, a = (n >> 2) & 3: bases for even and odd ks
    const int sa_ = (n >> 2) & 3;
    const int plain_e = n * LROW + 16 * (h ^ (sa_ & 1)) + 32 * (sa_ >> 1);
    const int plain_o = n * LROW + 16 * (h ^ (sa_ & 1)) - 32 * (sa_ >> 1);
    const int qhi = min(s1, q0 + kTile);
    const int kend = p.causal ? qhi : s1;
    const int ntiles = (kend - s0 + kInner - 1) / kInner;
    const int64_t kstride = (int64_t)p.Hkv * ROWB;
    const char *kg = (const char *)p.k + (int64_t)g * ROWB;
    const char *vg = (const char *)p.v + (int64_t)g * ROWB;
    Stager<ROWB, LROW, kInner, true> sk, sv;
    auto fetch = [&](int it) __attribute__((always_inline)) {
        const int k0 = s0 + it * kInner;
        sk.load(kg + (int64_t)k0 * kstride, kstride, min(kInner, s1 - k0));
        sv.load(vg + (int64_t)k0 * kstride, kstride, min(kInner, s1 - k0));
    };
    auto put = [&](char *stage) __attribute__((always_inline)) {
        sk.store(stage);
        sv.store(stage + TILEB);
    };

    // NB consecutive 32-key blocks from block b0 of the tile, their S, dP,
    // softmax and dS interleaved in one straight-line region (independent
    // chains for the scheduler), then their dQ products; masked: apply the
    // index mask (blocks reaching the diagonal or the sequence end)
    auto blocks = [&](auto nb, int k0, int b0, bool masked, const char *stage)
        __attribute__((always_inline)) {
        constexpr int NB = decltype(nb)::value;
        const char *kt = stage, *vt = stage + TILEB;
        f32x16 sa[NB], dp[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int b = b0 + j;
            // S^T = K Q^T (keys x queries)
            sa[j] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 ka = *(const bf16x8 *)(kt + 32 * b * LROW + map * D * 2 +
                                                    ((ks & 1) ? plain_o : plain_e) + 32 * ks);
                sa[j] = mma(ka, qf[ks], sa[j]);
            }
            // dP^T = V dO^T
            dp[j] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < NVS; ++ks) {
                const bf16x8 va = *(const bf16x8 *)(vt + 32 * b * LROW +
                                                    ((ks & 1) ? plain_o : plain_e) + 32 * ks);
                dp[j] = mma(va, df[ks], dp[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            // P^T and dS^T; lane owns query wq, element a is key kb0 +
            // acc_row(a, h).  Keys past the sequence or after the query get
            // a score of -inf (probability 0).
            const int kb0 = k0 + 32 * (b0 + j);
            if (masked) {
#pragma unroll
                for (int a = 0; a < 16; ++a) {
                    const int key = kb0 + acc_row(a, h);
                    if (!(key < s1 && (!p.causal || key <= wq)))
                        sa[j][a] = -INFINITY;
                }
            }
#pragma unroll
            for (int a = 0; a < 16; ++a) {
                const float pv = __builtin_amdgcn_exp2f(fmaf(sa[j][a], c, -lse));
                sa[j][a] = pv * fmaf(dpf, dp[j][a], -dval);
            }
        }
        // dQ^T += K^T dS^T
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int ps = 0; ps < 2; ++ps) {
                const bf16x8 bs = pack8(sa[j], 8 * ps);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    dqa[db] = mma(tr.load(kt, LROW, 32 * (b0 + j) + 16 * ps,
                                          (map * D + 32 * db) * 2),
                                  bs, dqa[db]);
            }
    };
    auto compute = [&](int it, const char *stage) __attribute__((always_inline)) {
        const int k0 = s0 + it * kInner;
        static_assert(kInner == 64, "two 32-key blocks per tile");
        // wave-uniform: both blocks visible and unmasked (the common case:
        // one region for both), else block by block
        const int klast = k0 + 32;   // first key of the tile's second block
        if (klast + 32 <= s1 && (!p.causal || klast + 31 <= q0 + 32 * sub)) {
            blocks(std::integral_constant<int, 2>{}, k0, 0, false, stage);
            return;
        }
#pragma unroll
        for (int b = 0; b < kInner / 32; ++b) {
            const int kb0 = k0 + 32 * b;
            // wave-uniform: keys of the block this wave's queries can see
            if (kb0 >= s1 || (p.causal && kb0 > q0 + 32 * sub + 31))
                continue;
            const bool masked = kb0 + 32 > s1 || (p.causal && kb0 + 31 > q0 + 32 * sub);
            blocks(std::integral_constant<int, 1>{}, k0, b, masked, stage);
        }
    };
    auto step = [&](int it, const char *cur, char *nxt) __attribute__((always_inline)) {
        const bool more = it + 1 < ntiles;
        if (more)
            fetch(it + 1);
        compute(it, cur);
        if (more)
            put(nxt);
        __syncthreads();
    };

    fetch(0);
    put(st0);
    __syncthreads();
    for (int it = 0; it < ntiles; it += 2) {
        step(it, st0, st1);
        if (it + 1 < ntiles)
            step(it + 1, st1, st0);
    }
    if (!qok)
        return;
    const float scale = rsqrtf((float)D);
    bf16 *dst = p.dq + (qrow * 2 + map) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16 vals[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                vals[e] = (bf16)(dqa[db][4 * i + e] * scale);
            __builtin_memcpy(dst + 32 * db + 8 * i + 4 * h, vals, sizeof(vals));
        }
}

// ---------------------------------------------------------------------------
// dkdv: key-outer.  Waves 0..3 (the S role) take 32 keys each and both
// maps: S_m = Q_m K_m^T, P_m, dS_1 = P_1 (dP - D'_1),
// dS_2 = -lambda P_2 (dP - D'_2), dK_m^T += Q_m^T dS_m, and
// W = P_1 - lambda P_2 rounded to bf16.  Waves 4..7 (the V role, same
// keys) compute dP = dpre V^T one query tile ahead (one product serves
// both maps: dO_2 = -lambda dO_1) and add dV^T += dpre^T W one query tile
// behind; dP and W travel through LDS.  Forming P_1 - lambda P_2 in fp32
// before rounding keeps dV accurate where the two maps nearly cancel (the
// first key of a sequence when lambda is near 1, where both maps put all
// weight on that key).  K rows (S role) and V rows (V role) live in
// registers; 32-row query tiles (Q, dpre, lse, D') rotate through four LDS
// stages: at step i the S role computes on tile i, the V role reads tiles
// i + 1 and i - 1, and tile i + 2 is written.
constexpr int kQT = 32;

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv(BwdParams p)
{
    constexpr int ROWB = 2 * D * 2;          // K, V, Q (both maps) or dpre row bytes
    // Q and dpre rows are read both ways, plain 16-byte reads and
    // transposing reads: swizzled tiles with a pitch of 64 mod 256 bytes
    // (TrOperand) keep both on distinct banks
    // (d = 64: 320 bytes; d = 32: 192, which is -64 mod 256 and works alike)
    constexpr int LQROW = ROWB + 64;
    constexpr int NKS = D / 16;
    constexpr int NVS = 2 * D / 16;
    constexpr int NKB = D / 32;              // 32-dim blocks of dK (per map)
    constexpr int NVB = 2 * D / 32;          // 32-dim blocks of dV
    static_assert(2 * NKB == NVB && 2 * NKS == NVS, "both roles share registers");
    constexpr int QB = kQT * LQROW;          // Q tile bytes
    constexpr int STB = 2 * QB + kQT * 4 * 4;   // one stage: Q, dpre, lse[2], D[2]
    constexpr int WXB = kSubs * 2 * 64 * 16;    // one W hand-over buffer (bf16)
    constexpr int PXB = kSubs * 4 * 64 * 16;    // one dP - D'_1 hand-over buffer (fp32)
    __shared__ __attribute__((aligned(16))) char stg[4 * STB];
    __shared__ __attribute__((aligned(16))) char wx[2 * WXB];
    __shared__ __attribute__((aligned(16))) char px[2 * PXB];
    // per query row of a tile: lambda D'_2 - lambda D'_1, so that the S role
    // forms map 2's factor from map 1's hand-over in one FMA
    __shared__ __attribute__((aligned(16))) float cx[2][kQT];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = lane & 31, h = lane >> 5;
    const int role = wave / kSubs, sub = wave % kSubs;   // role 0: S, 1: V

    const int pairs = p.nseq * p.Hkv;
    const int tile = blockIdx.x / pairs;
    const int rem = blockIdx.x % pairs;
    const int s = rem / p.Hkv, g = rem % p.Hkv;
    int s0, s1;
    seq_bounds(p, s, s0, s1);
    const int k0 = s0 + tile * kTile;
    if (k0 >= s1)
        return;
    const int wk = k0 + 32 * sub + n;   // this lane's key
    const bool kok = wk < s1;
    const int64_t kvrow = (int64_t)wk * p.Hkv + g;
    // B operands from this wave's key rows: S role K_1, K_2 (of S_m =
    // Q_m K_m^T), V role V (of dP = dpre V^T)
    bf16x8 kv[NVS];
#pragma unroll
    for (int i = 0; i < NVS; ++i) {
        const bf16 *src = role == 0 ? p.k : p.v;
        kv[i] = kok ? *(const bf16x8 *)(src + kvrow * 2 * D + 16 * i + 8 * h) : bf16x8{};
    }
    // S role: dK of map m in acc[m * NKB + db]; V role: dV in acc[db]
    f32x16 acc[NVB];
#pragma unroll
    for (int db = 0; db < NVB; ++db)
        acc[db] = f32x16{};
    const float c = kLog2e * rsqrtf((float)D);
    const TrOperand tr(lane, LQROW, true);
    // this lane's plain reads of its row n of a swizzled tile: chunk
    // 2 ks + h lies at (2 ks + h) ^ a, a = (n >> 2) & 3, that is at
    // 2 (ks ^ (a >> 1)) + (h ^ (a & 1)): two bases, for even and odd ks
    const int sa = (n >> 2) & 3;
    const int plain_e = n * LQROW + 16 * (h ^ (sa & 1)) + 32 * (sa >> 1);
    const int plain_o = n * LQROW + 16 * (h ^ (sa & 1)) - 32 * (sa >> 1);
    const int wk_first = k0 + 32 * sub;   // first key of this wave
    // queries before the tile's first key cannot see any of its keys
    const int qstart = p.causal ? k0 : s0;
    const int nqt = (s1 - qstart + kQT - 1) / kQT;   // query tiles per head
    const int total = p.G * nqt;                     // (head, query tile) steps

    Stager<ROWB, LQROW, kQT, true> sq, sd;
    // lse, and D'_1 or lambda D'_2, of the tile as [lse, D][map][row], so
    // that the four rows a lane's accumulator elements cover are one 16-byte
    // read
    float lv = 0.f;   // one lse or D' value per thread of the first 4 kQT
    auto fetch = [&](int stp) __attribute__((always_inline)) {
        const int head = g * p.G + stp / nqt;
        const int q0 = qstart + (stp % nqt) * kQT;
        const int valid = min(kQT, s1 - q0);
        const int64_t qrow0 = (int64_t)q0 * p.H + head;
        sq.load((const char *)(p.q + qrow0 * 2 * D), (int64_t)p.H * ROWB, valid);
        sd.load((const char *)(p.dpre + qrow0 * 2 * D), (int64_t)p.H * ROWB, valid);
        const int i = threadIdx.x;
        if (i < kQT * 4) {
            // i = (which * 2 + map) * kQT + row; which 0: lse, 1: D'
            const int which = i / (kQT * 2), mp = (i / kQT) & 1, r = i % kQT;
            const float *src = which ? p.dd : p.lse;
            lv = r < valid ? src[(qrow0 + (int64_t)r * p.H) * 2 + mp]
                           : (which ? 0.f : INFINITY);
        }
    };
    auto put = [&](char *stage) __attribute__((always_inline)) {
        sq.store(stage);
        sd.store(stage + QB);
        if (threadIdx.x < kQT * 4)
            ((float *)(stage + 2 * QB))[threadIdx.x] = lv;
    };
    auto stage_of = [&](int stp) __attribute__((always_inline)) { return stg + (stp & 3) * STB; };
    // wave-uniform: can any query of step stp's tile see a key of the wave?
    auto visible = [&](int stp) __attribute__((always_inline)) {
        const int q0 = qstart + (stp % nqt) * kQT;
        return !(q0 >= s1 || (p.causal && q0 + kQT - 1 < wk_first));
    };
    // V role: dP = dpre V^T of step stp (queries x keys; lane owns key wk),
    // handed over as dP - D'_1 (the factor of map 1's dS), 16 floats per
    // lane; the first V wave also tabulates the tile's lambda D'_2 - lambda
    // D'_1 (map 2's factor is -lambda (dP - D'_1) plus that)
    auto compute_dp = [&](int stp) __attribute__((always_inline)) {
        if (!visible(stp))
            return;
        const char *dt = stage_of(stp) + QB;
        const float *tab = (const float *)(stage_of(stp) + 2 * QB);
        f32x16 dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NVS; ++ks)
            dp = mma(*(const bf16x8 *)(dt + ((ks & 1) ? plain_o : plain_e) + 32 * ks), kv[ks], dp);
        if (sub == 0 && lane < kQT) {
            const float nlam = -p.lam[g * p.G + stp / nqt];
            cx[stp & 1][lane] = fmaf(nlam, tab[2 * kQT + lane], tab[3 * kQT + lane]);
        }
        char *out = px + (stp & 1) * PXB + sub * 4 * 1024 + lane * 16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 e1 = *(const float4 *)(tab + 2 * kQT + 8 * j + 4 * h);
            *(float4 *)(out + j * 1024) = float4{dp[4 * j] - e1.x, dp[4 * j + 1] - e1.y,
                                                 dp[4 * j + 2] - e1.z, dp[4 * j + 3] - e1.w};
        }
    };
    auto compute_s = [&](int stp) __attribute__((always_inline)) {
        if (!visible(stp))
            return;
        const char *qt = stage_of(stp);
        const float *tab = (const float *)(qt + 2 * QB);
        const int q0 = qstart + (stp % nqt) * kQT;
        const float nlam = -p.lam[g * p.G + stp / nqt];
        // S_m = Q_m K_m^T (queries x keys); lane owns key wk
        f32x16 s1a = f32x16{}, s2a = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const char *qa = qt + ((ks & 1) ? plain_o : plain_e) + 32 * ks;
            s1a = mma(*(const bf16x8 *)qa, kv[ks], s1a);
            s2a = mma(*(const bf16x8 *)(qa + D * 2), kv[NKS + ks], s2a);
        }
        // queries before the wave's key get a score of -inf (probability 0);
        // wave-uniform: only tiles that reach the diagonal need the test
        if (p.causal && q0 < wk_first + 31) {
#pragma unroll
            for (int a = 0; a < 16; ++a)
                if (wk > q0 + acc_row(a, h)) {
                    s1a[a] = -INFINITY;
                    s2a[a] = -INFINITY;
                }
        }
        const char *pin = px + (stp & 1) * PXB + sub * 4 * 1024 + lane * 16;
        bf16x8 wpk[2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // rows 8 j + 4 h .. + 3 of the tile
            const int r0 = 8 * j + 4 * h;
            const float4 l1 = *(const float4 *)(tab + r0);
            const float4 l2 = *(const float4 *)(tab + kQT + r0);
            const float4 c4 = *(const float4 *)(&cx[stp & 1][r0]);
            const float4 d4 = *(const float4 *)(pin + j * 1024);
            const float lr1[4] = {l1.x, l1.y, l1.z, l1.w}, lr2[4] = {l2.x, l2.y, l2.z, l2.w};
            const float cr[4] = {c4.x, c4.y, c4.z, c4.w};
            const float x1[4] = {d4.x, d4.y, d4.z, d4.w};   // dP - D'_1
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int a = 4 * j + e;
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s1a[a], c, -lr1[e]));
                const float p2 = __builtin_amdgcn_exp2f(fmaf(s2a[a], c, -lr2[e]));
                // W = P_1 - lambda P_2; dS_1 = P_1 (dP - D'_1);
                // dS_2 = P_2 (-lambda dP + lambda D'_2)
                //      = P_2 (-lambda (dP - D'_1) + lambda D'_2 - lambda D'_1)
                wpk[a / 8][a % 8] = (bf16)fmaf(nlam, p2, p1);
                s1a[a] = p1 * x1[e];
                s2a[a] = p2 * fmaf(nlam, x1[e], cr[e]);
            }
        }
        char *wout = wx + (stp & 1) * WXB;
#pragma unroll
        for (int ps = 0; ps < 2; ++ps)
            *(bf16x8 *)(wout + ((sub * 2 + ps) * 64 + lane) * 16) = wpk[ps];
        // dK_m^T += Q_m^T dS_m
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            const bf16x8 b1 = pack8(s1a, 8 * ps), b2 = pack8(s2a, 8 * ps);
#pragma unroll
            for (int db = 0; db < NKB; ++db) {
                acc[db] = mma(tr.load(qt, LQROW, 16 * ps, 32 * db * 2), b1, acc[db]);
                acc[NKB + db] =
                    mma(tr.load(qt, LQROW, 16 * ps, (D + 32 * db) * 2), b2, acc[NKB + db]);
            }
        }
    };
    // V role: dV^T += dpre^T W of step stp
    auto compute_v = [&](int stp) __attribute__((always_inline)) {
        if (!visible(stp))
            return;
        const char *dt = stage_of(stp) + QB;
        const char *win = wx + (stp & 1) * WXB;
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            const bf16x8 w = *(const bf16x8 *)(win + ((sub * 2 + ps) * 64 + lane) * 16);
#pragma unroll
            for (int db = 0; db < NVB; ++db)
                acc[db] = mma(tr.load(dt, LQROW, 16 * ps, 32 * db * 2), w, acc[db]);
        }
    };

    // prologue: tiles 0 and 1 staged, dP of tile 0 handed over
    fetch(0);
    put(stage_of(0));
    if (total > 1)
        fetch(1);
    __syncthreads();
    if (role == 1)
        compute_dp(0);
    if (total > 1)
        put(stage_of(1));
    __syncthreads();
    // step i: the S role on tile i (dP from the V role's step i - 1); the V
    // role's dP of tile i + 1 and dV of tile i - 1; tile i + 2 written into
    // the stage of tile i - 2, which no wave reads after the barrier that
    // ended step i - 1
    for (int stp = 0; stp < total; ++stp) {
        const bool more = stp + 2 < total;
        if (more)
            fetch(stp + 2);
        if (role == 0) {
            compute_s(stp);
        } else {
            if (stp + 1 < total)
                compute_dp(stp + 1);
            if (stp > 0)
                compute_v(stp - 1);
        }
        if (more)
            put(stage_of(stp + 2));
        __syncthreads();
    }
    if (role == 1)
        compute_v(total - 1);

    if (!kok)
        return;
    if (role == 0) {
        const float scale = rsqrtf((float)D);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            bf16 *dst = p.dk + (kvrow * 2 + m) * D;
#pragma unroll
            for (int db = 0; db < NKB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bf16 vals[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        vals[e] = (bf16)(acc[m * NKB + db][4 * i + e] * scale);
                    __builtin_memcpy(dst + 32 * db + 8 * i + 4 * h, vals, sizeof(vals));
                }
        }
    } else {
        bf16 *dst = p.dv + kvrow * (2 * D);
#pragma unroll
        for (int db = 0; db < NVB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf16 vals[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    vals[e] = (bf16)acc[db][4 * i + e];
                __builtin_memcpy(dst + 32 * db + 8 * i + 4 * h, vals, sizeof(vals));
            }
    }
}

// ---------------------------------------------------------------------------
// Exact path.  The sequence of token t: the last s with cu[s] <= t (zero-
// length sequences are skipped over).
__device__ inline void seq_of(const BwdParams &p, int t, int &s0, int &s1)
{
    if (p.cu) {
        int lo = 0, hi = p.nseq;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.cu[mid] <= t)
                lo = mid;
            else
                hi = mid;
        }
        s0 = p.cu[lo];
        s1 = p.cu[lo + 1];
    } else {
        s0 = (t / p.seqlen_uniform) * p.seqlen_uniform;
        s1 = s0 + p.seqlen_uniform;
    }
}

// lane's elements of a d-wide half (dim lane, if lane < D) and of a 2d-wide
// row (dims lane + 64 i)
template <int D> struct Lanes {
    static constexpr int NV = (2 * D + 63) / 64;   // 2d-row elements per lane
};

// dq: one wave per (token t, head h): over the keys j the row sees,
//   P_m = 2^(<Q_m, K_m[j]> log2(e) / sqrt(d) - lse_m), dP' = <dpre, V[j]>,
//   dS_1 = P_1 (dP' - D'_1), dS_2 = P_2 (lambda D'_2 - lambda dP'),
//   dQ_m += dS_m K_m[j] / sqrt(d).
template <typename E, int D>
__global__ __launch_bounds__(256) void bwdx_dq(BwdParams p)
{
    constexpr int NV = Lanes<D>::NV;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // t H + h
    if (row >= (int64_t)p.T * p.H)
        return;
    const int t = (int)(row / p.H), h = (int)(row % p.H), g = h / p.G;
    int s0, s1;
    seq_of(p, t, s0, s1);
    const int jend = p.causal ? t + 1 : s1;
    const float c = kLog2e * rsqrtf((float)D);
    const E *q = (const E *)p.q, *k = (const E *)p.k, *v = (const E *)p.v;
    const float *dpre = (const float *)p.dpre;
    const bool cd = lane < D;
    const float q1 = cd ? (float)q[(row * 2) * D + lane] : 0.f;
    const float q2 = cd ? (float)q[(row * 2 + 1) * D + lane] : 0.f;
    float dp[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i)
        dp[i] = lane + 64 * i < 2 * D ? dpre[row * (2 * D) + lane + 64 * i] : 0.f;
    const float lse1 = p.lse[row * 2], lse2 = p.lse[row * 2 + 1];
    const float dd1 = p.dd[row * 2], dd2 = p.dd[row * 2 + 1];   // D'_1, lambda D'_2
    const float lam = p.lam[h];
    float a1 = 0.f, a2 = 0.f;
    for (int j = s0; j < jend; ++j) {
        const int64_t kr = (int64_t)j * p.Hkv + g;
        const float k1 = cd ? (float)k[(kr * 2) * D + lane] : 0.f;
        const float k2 = cd ? (float)k[(kr * 2 + 1) * D + lane] : 0.f;
        float vd = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (lane + 64 * i < 2 * D)
                vd += dp[i] * (float)v[kr * (2 * D) + lane + 64 * i];
        const float sa = wave_sum(q1 * k1), sb = wave_sum(q2 * k2), dpv = wave_sum(vd);
        const float P1 = exp2f(sa * c - lse1), P2 = exp2f(sb * c - lse2);
        a1 += P1 * (dpv - dd1) * k1;
        a2 += P2 * (dd2 - lam * dpv) * k2;
    }
    if (cd) {
        const float isd = rsqrtf((float)D);
        ((E *)p.dq)[(row * 2) * D + lane] = (E)(a1 * isd);
        ((E *)p.dq)[(row * 2 + 1) * D + lane] = (E)(a2 * isd);
    }
}

// dk, dv: one wave per (key token j, KV head g): over the rows (t, h) of the
// group that see key j, with P_m, dP', dS_m as in bwdx_dq,
//   dK_m += dS_m Q_m[t, h] / sqrt(d),  dV += (P_1 - lambda_h P_2) dpre[t, h].
template <typename E, int D>
__global__ __launch_bounds__(256) void bwdx_dkdv(BwdParams p)
{
    constexpr int NV = Lanes<D>::NV;
    const int lane = threadIdx.x & 63;
    const int64_t kr = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // j Hkv + g
    if (kr >= (int64_t)p.T * p.Hkv)
        return;
    const int j = (int)(kr / p.Hkv), g = (int)(kr % p.Hkv);
    int s0, s1;
    seq_of(p, j, s0, s1);
    const int tbeg = p.causal ? j : s0;
    const float c = kLog2e * rsqrtf((float)D);
    const E *q = (const E *)p.q, *k = (const E *)p.k, *v = (const E *)p.v;
    const float *dpre = (const float *)p.dpre;
    const bool cd = lane < D;
    const float k1 = cd ? (float)k[(kr * 2) * D + lane] : 0.f;
    const float k2 = cd ? (float)k[(kr * 2 + 1) * D + lane] : 0.f;
    float vv[NV], dv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        vv[i] = lane + 64 * i < 2 * D ? (float)v[kr * (2 * D) + lane + 64 * i] : 0.f;
        dv[i] = 0.f;
    }
    float a1 = 0.f, a2 = 0.f;
    for (int hh = 0; hh < p.G; ++hh) {
        const int h = g * p.G + hh;
        const float lam = p.lam[h];
        for (int t = tbeg; t < s1; ++t) {
            const int64_t row = (int64_t)t * p.H + h;
            const float q1 = cd ? (float)q[(row * 2) * D + lane] : 0.f;
            const float q2 = cd ? (float)q[(row * 2 + 1) * D + lane] : 0.f;
            float dp[NV], vd = 0.f;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                dp[i] = lane + 64 * i < 2 * D ? dpre[row * (2 * D) + lane + 64 * i] : 0.f;
                vd += dp[i] * vv[i];
            }
            const float sa = wave_sum(q1 * k1), sb = wave_sum(q2 * k2), dpv = wave_sum(vd);
            const float P1 = exp2f(sa * c - p.lse[row * 2]);
            const float P2 = exp2f(sb * c - p.lse[row * 2 + 1]);
            a1 += P1 * (dpv - p.dd[row * 2]) * q1;
            a2 += P2 * (p.dd[row * 2 + 1] - lam * dpv) * q2;
            const float W = P1 - lam * P2;
#pragma unroll
            for (int i = 0; i < NV; ++i)
                dv[i] += W * dp[i];
        }
    }
    const float isd = rsqrtf((float)D);
    if (cd) {
        ((E *)p.dk)[(kr * 2) * D + lane] = (E)(a1 * isd);
        ((E *)p.dk)[(kr * 2 + 1) * D + lane] = (E)(a2 * isd);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
        if (lane + 64 * i < 2 * D)
            ((E *)p.dv)[kr * (2 * D) + lane + 64 * i] = (E)dv[i];
}

struct BwdPlan {
    size_t dpre, dd, lam, part_dw, part_dl, total;
};

// dpre_bytes: 2 on the MFMA path (bf16 operand), 4 on the exact path
BwdPlan bwd_plan(int64_t T, int H, int d, int dpre_bytes)
{
    BwdPlan pl;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    pl.dpre = up((size_t)T * H * (2 * d) * dpre_bytes);
    pl.dd = up((size_t)T * H * 2 * 4);
    pl.lam = up((size_t)H * 4);
    pl.part_dw = up((size_t)H * (kPrepPerHead / 4) * 2 * d * 4);
    pl.part_dl = up((size_t)H * (kPrepPerHead / 4) * 4);
    pl.total = pl.dpre + pl.dd + pl.lam + pl.part_dw + pl.part_dl;
    return pl;
}

template <int D>
void launch_bwd(const BwdParams &p, int nseq, int Hkv, hipStream_t st)
{
    hipLaunchKernelGGL((bwd_prep<bf16, bf16, D>), dim3(p.H * kPrepBlocksPerHead), dim3(256), 0,
                       st, p);
    hipLaunchKernelGGL(bwd_reduce<D>, dim3(1), dim3(1024), 0, st, p);
    hipLaunchKernelGGL(bwd_dq<D>, dim3(p.ntile * nseq * p.H), dim3(kThreads), 0, st, p);
    hipLaunchKernelGGL(bwd_dkdv<D>, dim3(p.ntile * nseq * Hkv), dim3(kThreads), 0, st, p);
}

template <typename E, int D>
void launch_bwd_exact(const BwdParams &p, hipStream_t st)
{
    hipLaunchKernelGGL((bwd_prep<E, float, D>), dim3(p.H * kPrepBlocksPerHead), dim3(256), 0,
                       st, p);
    hipLaunchKernelGGL(bwd_reduce<D>, dim3(1), dim3(1024), 0, st, p);
    const int64_t rq = ((int64_t)p.T * p.H + 3) / 4, rk = ((int64_t)p.T * p.Hkv + 3) / 4;
    hipLaunchKernelGGL((bwdx_dq<E, D>), dim3((unsigned)rq), dim3(256), 0, st, p);
    hipLaunchKernelGGL((bwdx_dkdv<E, D>), dim3((unsigned)rk), dim3(256), 0, st, p);
}

// the MFMA kernels serve bf16 at d = 32 and 64; the exact path the rest
bool mfma_path(int dtype, int d) { return dtype == DIFFATTN_BF16 && (d == 32 || d == 64); }

bool a16(const void *x) { return ((uintptr_t)x & 15u) == 0; }

} // namespace

extern "C" int diffattn_supported_bwd(int dtype, int d)
{
    return (dtype == DIFFATTN_BF16 || dtype == DIFFATTN_F32) && (d == 16 || d == 32 || d == 64);
}

extern "C" size_t diffattn_bwd_workspace_size(int dtype, int32_t T, int32_t H, int32_t d)
{
    if (T < 0 || H < 1 || d < 1 || !diffattn_supported_bwd(dtype, d))
        return 0;
    return bwd_plan(T, H, d, mfma_path(dtype, d) ? 2 : 4).total;
}

extern "C" int diffattn_bwd(int dtype, const void *q, const void *k, const void *v,
                            const float *lambda_q1, const float *lambda_k1,
                            const float *lambda_q2, const float *lambda_k2,
                            int32_t lambda_stride, float lambda_init,
                            const float *subln_weight, float eps, int causal,
                            const int32_t *cu_seqlens, int32_t nseq, int32_t max_seqlen,
                            int32_t T, int32_t H, int32_t Hkv, int32_t d, const void *dout,
                            const float *lse, const float *o12, void *dq, void *dk, void *dv,
                            float *dlambda_q1, float *dlambda_k1, float *dlambda_q2,
                            float *dlambda_k2, float *dsubln_weight, void *workspace,
                            size_t workspace_bytes, void *stream)
{
    if (dtype != DIFFATTN_BF16 && dtype != DIFFATTN_F32)
        return DIFFATTN_EINVAL;
    if (T < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || d < 1 || nseq < 1 || H > 256)
        return DIFFATTN_EINVAL;
    if (causal != 0 && causal != 1)
        return DIFFATTN_EINVAL;
    if (!(eps >= 0.f) || !isfinite(eps) || !isfinite(lambda_init))
        return DIFFATTN_EINVAL;
    if (lambda_stride != 0 && lambda_stride < d)
        return DIFFATTN_EINVAL;
    if (!diffattn_supported_bwd(dtype, d))
        return DIFFATTN_EUNSUPPORTED;
    if (!lambda_q1 || !lambda_k1 || !lambda_q2 || !lambda_k2 || !dlambda_q1 || !dlambda_k1 ||
        !dlambda_q2 || !dlambda_k2)
        return DIFFATTN_EINVAL;
    int32_t uniform = 0;
    if (!cu_seqlens) {
        if (T % nseq != 0)
            return DIFFATTN_EINVAL;
        uniform = T / nseq;
        max_seqlen = uniform;
    } else if (max_seqlen < 0 || max_seqlen > T) {
        return DIFFATTN_EINVAL;
    }
    const bool mfma = mfma_path(dtype, d);
    const BwdPlan pl = bwd_plan(T, H, d, mfma ? 2 : 4);
    if (T > 0) {
        if (!q || !k || !v || !dout || !lse || !o12 || !dq || !dk || !dv || !workspace)
            return DIFFATTN_EINVAL;
        if (!a16(q) || !a16(k) || !a16(v) || !a16(dout) || !a16(o12) || !a16(dq) || !a16(dk) ||
            !a16(dv) || !a16(workspace) || (subln_weight && !a16(subln_weight)))
            return DIFFATTN_EINVAL;
        if (workspace_bytes < pl.total)
            return DIFFATTN_EINVAL;
        if (max_seqlen < 1)
            return DIFFATTN_EINVAL;
    }
    BwdParams p;
    p.q = (const bf16 *)q;
    p.k = (const bf16 *)k;
    p.v = (const bf16 *)v;
    p.dy = (const bf16 *)dout;
    p.lse = lse;
    p.o12 = o12;
    p.lq1 = lambda_q1;
    p.lk1 = lambda_k1;
    p.lq2 = lambda_q2;
    p.lk2 = lambda_k2;
    p.lstride = lambda_stride;
    p.w = subln_weight;
    p.cu = cu_seqlens;
    p.dq = (bf16 *)dq;
    p.dk = (bf16 *)dk;
    p.dv = (bf16 *)dv;
    p.dlq1 = dlambda_q1;
    p.dlk1 = dlambda_k1;
    p.dlq2 = dlambda_q2;
    p.dlk2 = dlambda_k2;
    p.dw = dsubln_weight;
    char *ws = (char *)workspace;
    p.dpre = (bf16 *)ws;
    ws += pl.dpre;
    p.dd = (float *)ws;
    ws += pl.dd;
    p.lam = (float *)ws;
    ws += pl.lam;
    p.part_dw = (float *)ws;
    ws += pl.part_dw;
    p.part_dl = (float *)ws;
    p.lambda_init = lambda_init;
    p.eps = eps;
    p.T = T;
    p.H = H;
    p.Hkv = Hkv;
    p.G = H / Hkv;
    p.nseq = nseq;
    p.seqlen_uniform = uniform;
    p.causal = causal;
    p.ntile = T > 0 ? (max_seqlen + kTile - 1) / kTile : 0;
    const int64_t blocks = (int64_t)p.ntile * nseq * H;
    if (blocks > INT32_MAX)
        return DIFFATTN_EINVAL;
    if (!mfma && ((int64_t)T * H + 3) / 4 > INT32_MAX)   // exact path: a wave per row
        return DIFFATTN_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    if (T == 0)
        return DIFFATTN_OK;   // no rows: nothing is launched or written
    if (mfma) {
        if (d == 64)
            launch_bwd<64>(p, nseq, Hkv, st);
        else
            launch_bwd<32>(p, nseq, Hkv, st);
    } else if (dtype == DIFFATTN_BF16) {
        launch_bwd_exact<bf16, 16>(p, st);
    } else if (d == 64) {
        launch_bwd_exact<float, 64>(p, st);
    } else if (d == 32) {
        launch_bwd_exact<float, 32>(p, st);
    } else {
        launch_bwd_exact<float, 16>(p, st);
    }
    return hipGetLastError() == hipSuccess ? DIFFATTN_OK : DIFFATTN_EHIP;
}
