"""Which instantiation of the prefill kernel a launch takes, restated from
the library's host rule so that tests can pick shapes for each: a
workgroup serves four (head, query block) slots of one KV group, with 64
queries per slot, or 32 when 64 would leave fewer than two workgroups per
compute unit (256 of them)."""

CUS = 256


def workgroups(H, Hkv, nseq, max_seqlen, sub):
    G = H // Hkv
    hpw = 4 if G % 4 == 0 else (2 if G % 2 == 0 else 1)
    bm = 32 * sub * (4 // hpw)
    return -(-max_seqlen // bm) * nseq * Hkv * (G // hpw)


def prefill_sub_blocks(H, Hkv, nseq, max_seqlen):
    """32-query sub-blocks per wave (2 or 1) of the launch."""
    return 2 if workgroups(H, Hkv, nseq, max_seqlen, 2) >= 2 * CUS else 1
