"""Brute-force MLA decode for tiny inputs: pure Python, element by element.

Independent of the oracle: the page walk, the element decoders and the softmax
are written again from their definitions (loops, math.fsum), so a slip in the
oracle's vectorised code shows up as a disagreement. An mpmath variant runs the
same loops at 50 significant digits.
"""

import math
import struct


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def e4m3fn_value(byte: int) -> float:
    byte = int(byte) & 0xFF
    s = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * math.ldexp(m, -9)
    return s * math.ldexp(8 + m, e - 10)


def logical_rows(page_list, page_size, n):
    """Physical slots of the first n logical rows, by walking the pages in order."""
    slots = []
    for page in page_list:
        for off in range(page_size):
            slots.append(int(page) * page_size + off)
    return slots[:n]


def brute_decode(case, use_mpmath=False):
    """Returns (out[b][s][h] -> list of 512 floats, lse[b][s][h] -> float)."""
    if use_mpmath:
        import mpmath as mp
        mp.mp.dps = 50
        exp, log, fsum, num = mp.exp, mp.log, mp.fsum, mp.mpf
    else:
        exp, log, fsum, num = math.exp, math.log, math.fsum, float
    B, S, H = case.batch, case.seqlen_qo, case.num_heads
    P = case.page_size
    scale = num(case.softmax_scale)
    kv_scale = num(case.kv_scale)
    out, lse = {}, {}
    for b in range(B):
        ctx = int(case.context_lens[b])
        plist = case.kv_page_indices[case.kv_indptr[b]:case.kv_indptr[b + 1]]
        slots = logical_rows(plist, P, ctx)
        rows = []
        for slot in slots:
            raw = case.cache_raw[slot]
            if case.kv_dtype == "bf16":
                rows.append([num(bf16_value(x)) for x in raw])
            else:
                rows.append([num(e4m3fn_value(x)) * kv_scale for x in raw])
        for s in range(S):
            n = ctx - S + 1 + s if case.causal else ctx
            for h in range(H):
                if getattr(case, "q_dtype", "bf16") == "fp8_e4m3fn":
                    q = [num(e4m3fn_value(x)) * num(case.q_scale) for x in case.q_bits[b, s, h]]
                else:
                    q = [num(bf16_value(x)) for x in case.q_bits[b, s, h]]
                z = [scale * fsum([q[d] * rows[r][d] for d in range(576)]) for r in range(n)]
                mu = max(z)
                w = [exp(zr - mu) for zr in z]
                den = fsum(w)
                out[(b, s, h)] = [fsum([w[r] * rows[r][d] for r in range(n)]) / den for d in range(512)]
                lse[(b, s, h)] = mu + log(den)
    return out, lse
