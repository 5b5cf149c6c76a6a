// splits.h -- key splits shared by the cache path's kernels and the prefill
// kernel's key-split mode (device helpers; internal to the library).
//
// The splits of all sequences share one index space: sequence s owns the
// ceil(nk_s / ck) consecutive slots starting at base(s), the sum of the
// earlier sequences' split counts.  The merge kernel reads a row's splits
// from that layout, so every kernel that writes partials uses these
// helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diffattn_splits {

__device__ inline int split_count(int nk, int ck) { return (nk + ck - 1) / ck; }

// Sequence owning slot j and its first slot, or false past the last split.
// P has nseq, ck, klen_uniform (keys per sequence without boundaries) and
// cuk (the keys' boundaries, or NULL).  A wave-wide scan of the boundaries,
// 64 sequences per step; every lane gets the same (wave-uniform) answer.
template <class P>
__device__ inline bool split_owner(const P &p, int j, int lane, int &s, int &base)
{
    if (!p.cuk) {
        const int cnt = split_count(p.klen_uniform, p.ck);
        if (cnt == 0 || j >= cnt * p.nseq)
            return false;
        s = j / cnt;
        base = s * cnt;
        return true;
    }
    int run = 0;
    for (int s0 = 0; s0 < p.nseq; s0 += 64) {
        const int si = s0 + lane;
        const int cnt = si < p.nseq ? split_count(p.cuk[si + 1] - p.cuk[si], p.ck) : 0;
        int incl = cnt;   // inclusive prefix over the lanes
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off, 64);
            if (lane >= off)
                incl += t;
        }
        const uint64_t hit = __builtin_amdgcn_ballot_w64(j >= run + incl - cnt && j < run + incl);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            s = s0 + l;
            base = run + __builtin_amdgcn_readlane(incl - cnt, l);
            return true;
        }
        run += __builtin_amdgcn_readlane(incl, 63);
    }
    return false;
}

} // namespace diffattn_splits
