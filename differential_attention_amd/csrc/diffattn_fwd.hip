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
// the two softmax recurrences are fully independent.
//
// The workgroup streams the KV range of its sequence in tiles of 64 keys.
// Each tile's K (both halves, 64 x 2d) and V (transposed, 2d x 64) is staged
// once in LDS and read by all four waves: K/V of a GQA group enter the chip
// once per 32..128 query rows and are never copied per head.  Tiles are
// double-buffered: global loads of tile t+1 are in flight (in registers)
// while tile t is computed, then written to the other LDS buffer; one
// barrier per tile.
//
// All four contractions run on MFMA (v_mfma_f32_32x32x16_bf16 for bf16,
// v_mfma_f32_32x32x2_f32 for fp32), in transposed form:
//   S_m^T [keys x queries] = K_m [keys x d] * Q_m^T      (m = 1, 2)
//   O_m^T [2d  x queries] += V^T [2d x keys] * P_m^T
// With S^T, each lane owns one query column and 16 keys of every 32-key
// block, so row maxima and sums need one cross-half exchange only, and the
// accumulator layout of S^T is directly the B-operand layout of the PV
// product.  The key order inside a 32-key block is permuted (K rows are
// gathered in order sigma) so that the 8 keys one lane contributes to a PV
// step are consecutive, which makes every V^T operand a single 16-byte LDS
// read.
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
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;   // keys per KV tile
constexpr int kQW = 32;   // query rows per wave
constexpr float kLog2e = 1.4426950408889634f;

template <typename E> struct Mfma;

template <> struct Mfma<bf16> {
    static constexpr int VEC = 8;   // operand elements per lane
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

// Key offset, inside a 32-key block, of accumulator element a of a lane in
// half h (= lane / 32).  The 32x32 MFMA accumulator puts element a of lane
// (n, h) at row 8*(a/4) + 4*h + a%4; K rows are gathered so that this row
// holds key 16*(a/8) + 8*h + a%8.
__device__ __host__ constexpr int key_of_acc(int a, int h)
{
    return 16 * (a / 8) + 8 * h + (a % 8);
}

// The K row that MFMA row m (= lane % 32 of the A operand) must hold.
__device__ __host__ constexpr int key_of_row(int m)
{
    return key_of_acc(4 * (m / 8) + (m % 4), (m / 4) % 2);
}

__device__ inline float xor32(float x) { return __shfl_xor(x, 32, 64); }

template <typename E, int D> struct Layout {
    static constexpr int CH = 16 / (int)sizeof(E);        // elements per 16 B
    static constexpr int KROW = 2 * D + CH;               // K row stride
    static constexpr int VROW = kBN + CH;                 // V^T row stride
    static constexpr int K_ELEMS = kBN * KROW;
    static constexpr int V_ELEMS = 2 * D * VROW;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int CPR = 2 * D / CH;                // 16 B chunks per row
    static constexpr int KC = kBN * CPR / kThreads;       // K chunks per thread
    static constexpr int KG = kThreads / CPR;             // V key groups
    static constexpr int R = kBN / KG;                    // keys per V group
    static_assert(KC * kThreads == kBN * CPR, "K staging must tile evenly");
    static_assert(KG * R == kBN && KG * CPR == kThreads, "V staging tiling");
    static_assert(D % (2 * Mfma<E>::VEC) == 0, "d must be a multiple of the MFMA depth");
    static_assert((2 * D) % 32 == 0, "2d must be a multiple of 32");
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Global -> registers part of staging one KV tile (keys [k0, k0 + 64) of KV
// head g).  Keys at or beyond `kend` are replaced by zeros.
template <typename E, int D> struct Stage {
    typedef Layout<E, D> L;
    u32x4 kr[L::KC];
    u32x4 vr[L::R];

    __device__ inline void load(const E *__restrict__ k, const E *__restrict__ v,
                                int Hkv, int g, int k0, int kend, int tid)
    {
#pragma unroll
        for (int c = 0; c < L::KC; ++c) {
            const int idx = tid + c * kThreads;
            const int row = idx / L::CPR, col = idx % L::CPR;
            const int key = k0 + row;
            if (key < kend) {
                const E *src = k + ((int64_t)key * Hkv + g) * (2 * D) + col * L::CH;
                kr[c] = *(const u32x4 *)src;
            } else {
                kr[c] = u32x4{0, 0, 0, 0};
            }
        }
        const int kg = tid % L::KG, dc = tid / L::KG;
#pragma unroll
        for (int r = 0; r < L::R; ++r) {
            const int key = k0 + kg * L::R + r;
            if (key < kend) {
                const E *src = v + ((int64_t)key * Hkv + g) * (2 * D) + dc * L::CH;
                vr[r] = *(const u32x4 *)src;
            } else {
                vr[r] = u32x4{0, 0, 0, 0};
            }
        }
    }

    __device__ inline void store(E *__restrict__ ks, E *__restrict__ vts, int tid) const
    {
#pragma unroll
        for (int c = 0; c < L::KC; ++c) {
            const int idx = tid + c * kThreads;
            const int row = idx / L::CPR, col = idx % L::CPR;
            *(u32x4 *)(ks + row * L::KROW + col * L::CH) = kr[c];
        }
        // transpose: V rows (keys) -> V^T rows (dims)
        const int kg = tid % L::KG, dc = tid / L::KG;
        E vals[L::R][L::CH];
#pragma unroll
        for (int r = 0; r < L::R; ++r)
            __builtin_memcpy(&vals[r][0], &vr[r], 16);
#pragma unroll
        for (int e = 0; e < L::CH; ++e) {
            E col[L::R];
#pragma unroll
            for (int r = 0; r < L::R; ++r)
                col[r] = vals[r][e];
            __builtin_memcpy(vts + (dc * L::CH + e) * L::VROW + kg * L::R, col,
                             sizeof(col));
        }
    }
};

template <typename E, int D>
__global__ __launch_bounds__(kThreads, 1) void diffattn_fwd_kernel(Params p)
{
    typedef Layout<E, D> L;
    typedef Mfma<E> M;
    typedef typename M::Frag Frag;
    constexpr int VEC = M::VEC;
    constexpr int KSTEP = 2 * VEC;         // contraction depth of one MFMA
    constexpr int NKS = D / KSTEP;         // MFMAs per 32x32 score block
    constexpr int NDB = 2 * D / 32;        // 32-wide blocks of the output
    constexpr int NPS = 32 / KSTEP;        // PV steps per 32-key block

    __shared__ __attribute__((aligned(16))) E smem[2 * L::STAGE];

    const int tid = threadIdx.x;
    const int wave = tid / 64;
    const int lane = tid % 64;
    const int n = lane % 32;   // query column owned by this lane
    const int h = lane / 32;   // lane half

    // ---- tile scheduler: longest query tiles first ----------------------
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
    const int qpw = kWaves / p.hpw;           // query blocks per workgroup
    const int bm = kQW * qpw;                 // query rows per workgroup
    const int q0 = s0 + t * bm;
    if (q0 >= s1)
        return;
    const int qhi = min(s1, q0 + bm);

    const int head = g * (p.H / p.Hkv) + hb * p.hpw + wave / qpw;
    const int wq0 = q0 + (wave % qpw) * kQW;  // first query row of this wave
    const int wq_last = min(wq0 + kQW, s1) - 1;
    const int tq = wq0 + n;                   // this lane's query token

    const E *__restrict__ qg = (const E *)p.q;
    const E *__restrict__ kg = (const E *)p.k;
    const E *__restrict__ vg = (const E *)p.v;

    // ---- lambda (every wave computes the same scalar) --------------------
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

    // ---- running state ---------------------------------------------------
    const float c = kLog2e / sqrtf((float)D);   // softmax scale in log2 units
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};
    f32x16 o[2][NDB];
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            o[mp][db] = f32x16{};

    const int kv_end = p.causal ? qhi : s1;
    const int ntiles = (kv_end - s0 + kBN - 1) / kBN;

    Stage<E, D> st;
    st.load(kg, vg, p.Hkv, g, s0, s1, tid);
    st.store(smem, smem + L::K_ELEMS, tid);
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int k0 = s0 + it * kBN;
        E *ks_lds = smem + (it & 1) * L::STAGE;
        E *vt_lds = ks_lds + L::K_ELEMS;
        if (it + 1 < ntiles)
            st.load(kg, vg, p.Hkv, g, k0 + kBN, s1, tid);

        // ---- S^T = K Q^T for both maps and both 32-key blocks -------------
        f32x16 s[2][2];
        bool live[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int kb0 = k0 + 32 * b;
            live[b] = kb0 < s1 && (!p.causal || kb0 <= wq_last);
#pragma unroll
            for (int mp = 0; mp < 2; ++mp) {
                s[mp][b] = f32x16{};
                if (live[b]) {
                    const E *arow = ks_lds + (32 * b + key_of_row(n)) * L::KROW + mp * D + h * VEC;
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        Frag a = *(const Frag *)(arow + ks * KSTEP);
                        s[mp][b] = M::mma(a, qf[mp][ks], s[mp][b]);
                    }
                }
            }
        }

        // ---- mask: keys beyond the sequence, or after the query ----------
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int kb0 = k0 + 32 * b;
            const bool need = !live[b] || kb0 + 31 >= s1 || (p.causal && kb0 + 31 > wq0);
            if (need) {
#pragma unroll
                for (int a = 0; a < 16; ++a) {
                    const int key = kb0 + key_of_acc(a, h);
                    const bool ok = live[b] && key < s1 && (!p.causal || key <= tq);
                    if (!ok) {
                        s[0][b][a] = -INFINITY;
                        s[1][b][a] = -INFINITY;
                    }
                }
            }
        }

        // ---- two independent online-softmax updates ----------------------
#pragma unroll
        for (int mp = 0; mp < 2; ++mp) {
            float mt = -INFINITY;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int a = 0; a < 16; ++a)
                    mt = fmaxf(mt, s[mp][b][a]);
            mt = fmaxf(mt, xor32(mt));
            const float mnew = fmaxf(m_run[mp], mt);
            const bool fin = mnew != -INFINITY;
            const float alpha = fin ? __builtin_amdgcn_exp2f((m_run[mp] - mnew) * c) : 1.f;
            const float mc = fin ? mnew * c : 0.f;
            m_run[mp] = mnew;
            float rs = 0.f;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int a = 0; a < 16; ++a) {
                    const float pv = __builtin_amdgcn_exp2f(s[mp][b][a] * c - mc);
                    s[mp][b][a] = pv;
                    rs += pv;
                }
            l_run[mp] = l_run[mp] * alpha + rs;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                o[mp][db] *= alpha;
        }

        // ---- O^T += V^T P^T ---------------------------------------------
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            if (!live[b])
                continue;
#pragma unroll
            for (int ps = 0; ps < NPS; ++ps) {
                const int a0 = ps * VEC;
                const Frag p1 = M::pack(s[0][b], a0);
                const Frag p2 = M::pack(s[1][b], a0);
                const E *vcol = vt_lds + 32 * b + key_of_acc(a0, h);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const Frag vf = *(const Frag *)(vcol + (32 * db + n) * L::VROW);
                    o[0][db] = M::mma(vf, p1, o[0][db]);
                    o[1][db] = M::mma(vf, p2, o[1][db]);
                }
            }
        }

        if (it + 1 < ntiles)
            st.store(smem + ((it + 1) & 1) * L::STAGE,
                     smem + ((it + 1) & 1) * L::STAGE + L::K_ELEMS, tid);
        __syncthreads();
    }

    // ---- epilogue: combine, RMSNorm, scale, store -------------------------
    const float l1 = l_run[0] + xor32(l_run[0]);
    const float l2 = l_run[1] + xor32(l_run[1]);
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
    ss += xor32(ss);
    const float r = (1.f - p.lambda_init) / sqrtf(ss / (float)(2 * D) + p.eps);
    if (tq < s1) {
        E *dst = (E *)p.out + ((int64_t)tq * p.H + head) * (2 * D);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int dim = 32 * db + 8 * i + 4 * h;
                E vals[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float wv = p.w ? p.w[dim + j] : 1.f;
                    vals[j] = (E)(o[0][db][4 * i + j] * r * wv);
                }
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
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) % 16 != 0)
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
    // element offsets of q/out rows stay within int64; the grid within int32
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
