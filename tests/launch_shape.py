"""Which instantiation of the prefill kernel a launch takes, restated from
the library's host rule so that tests can pick shapes for each: a
workgroup serves four (head, query block) slots of one KV group, with 64
queries per slot, or 32 when 64 would leave fewer than two workgroups per
compute unit (256 of them).  Packed sequences (cu_seqlens given, at most
64 of them) run on the compact tile list when its bound, T / bm + nseq
tiles, is below the padded grid's ceil(max_seqlen / bm) * nseq."""

CUS = 256


def workgroups(H, Hkv, nseq, max_seqlen, sub, T=None):
    """Workgroups of the launch; T: total tokens of packed sequences (None
    without cu_seqlens)."""
    G = H // Hkv
    hpw = 4 if G % 4 == 0 else (2 if G % 2 == 0 else 1)
    bm = 32 * sub * (4 // hpw)
    tiles = -(-max_seqlen // bm) * nseq
    if T is not None and nseq <= 64:
        tiles = min(tiles, T // bm + nseq)
    return tiles * Hkv * (G // hpw)


def compact_list(H, Hkv, nseq, max_seqlen, T):
    """Whether packed sequences run on the compact tile list."""
    sub = prefill_sub_blocks(H, Hkv, nseq, max_seqlen, T)
    G = H // Hkv
    hpw = 4 if G % 4 == 0 else (2 if G % 2 == 0 else 1)
    bm = 32 * sub * (4 // hpw)
    return nseq <= 64 and T // bm + nseq < -(-max_seqlen // bm) * nseq


def prefill_sub_blocks(H, Hkv, nseq, max_seqlen, T=None):
    """32-query sub-blocks per wave (2 or 1) of the launch."""
    return 2 if workgroups(H, Hkv, nseq, max_seqlen, 2, T) >= 2 * CUS else 1
