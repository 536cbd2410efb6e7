"""Pure-Python brute force of segment-causal, action-aware attention.

Used only to pin the numpy oracle on tiny inputs.  It is written separately
from the oracle: tokens are enumerated by nested loops, visibility is a chain
of if-statements that follows the rule table key kind by key kind, history
values come from the exact-rational quantizer, and sums are plain Python
loops with math.exp.
"""
import math

from _exact_quant import quantize_row_exact, bf16_to_fraction

TILE = 128


def _tokens(w):
    """Yield (seg, kind, tail, local frame, global frame, where, row, pos_in_frame)."""
    out = []
    gstart = 0
    for s, seg in enumerate(w.segments):
        for i in range(seg.head_len):
            out.append((s, "head", None, None, None, "txt", i, None))
        r = seg.head_len
        for j, a in enumerate(seg.action_len):
            for i in range(a):
                out.append((s, "tail", j, None, None, "txt", r, None))
                r += 1
        for f in range(seg.frames):
            for p in range(seg.tokens_per_frame):
                out.append((s, "video", None, f, gstart + f, "vid",
                            f * seg.tokens_per_frame + p, p))
        gstart += seg.frames
    return out


def brute_visible(w, tok, q_frame, q_row, csr=None):
    S = w.query_segment
    s, kind, tail, lf, gf, where, row, p = tok
    g0 = sum(seg.frames for seg in w.segments[:S])
    if s > S:
        return False
    if s < S:
        if kind == "head":
            ok = True
        elif kind == "tail":
            return False
        else:
            if w.window is not None and gf < g0 - w.window:
                return False
            ok = True
    else:
        if kind == "head":
            ok = True
        elif kind == "tail":
            seg = w.segments[S]
            ok = seg.action_f0[tail] <= q_frame < seg.action_f1[tail]
        else:
            ok = True
    if not ok:
        return False
    if csr is not None and kind == "video":
        P = w.segments[S].tokens_per_frame
        kept_frames = g0 if w.window is None else min(g0, w.window)
        n_hist_tiles = (kept_frames * P + TILE - 1) // TILE
        if s < S:
            oldest = g0 - kept_frames
            tile = ((gf - oldest) * P + p) // TILE
        else:
            tile = n_hist_tiles + row // TILE
        qt = q_row // TILE
        if tile not in list(csr["col"][csr["row_ptr"][qt]:csr["row_ptr"][qt + 1]]):
            return False
    return True


def brute_visible_text(w, tok, q_tail):
    """Visibility for a text-stream query of the query segment; q_tail is the
    query's tail index, or None for a description-head token."""
    S = w.query_segment
    s, kind, tail, lf, gf, where, row, p = tok
    g0 = sum(seg.frames for seg in w.segments[:S])
    if s > S:
        return False
    if s < S:
        if kind == "head":
            return True
        if kind == "tail":
            return False
        return w.window is None or gf >= g0 - w.window
    if kind == "head":
        return True
    if kind == "tail":
        return q_tail is not None and tail == q_tail
    return True


def text_query_tail(seg, r):
    """Tail index of text row r of a segment (None for head rows)."""
    if r < seg.head_len:
        return None
    r -= seg.head_len
    for j, a in enumerate(seg.action_len):
        if r < a:
            return j
        r -= a
    raise IndexError(r)


def _value_row(w, data, tok, h, which):
    S = w.query_segment
    s, kind, tail, lf, gf, where, row, p = tok
    bits = data["segments"][s][which + "_" + where][row, h, :]
    if s < S:
        q, scale = quantize_row_exact([int(b) for b in bits])
        return [float(qi * scale) for qi in q]
    return [float(bf16_to_fraction(int(b))) for b in bits]


def brute_attention(w, data, rows=None, sm_scale=None, queries="video"):
    """Returns (O[r][h][d], lse[h][r]) as nested Python lists; queries is
    "video" or "text" (the query segment's head and tail tokens)."""
    S = w.query_segment
    cur = w.segments[S]
    D = w.head_dim
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    toks = _tokens(w)
    csr = data.get("csr") if w.sparse_keep is not None else None
    nq = cur.frames * cur.tokens_per_frame if queries == "video" else cur.text_len
    rows = list(range(nq)) if rows is None else list(rows)
    cache = {}

    def val(i, h, which):
        key = (i, h, which)
        if key not in cache:
            cache[key] = _value_row(w, data, toks[i], h, which)
        return cache[key]

    O = [[None] * w.heads for _ in rows]
    lse = [[None] * len(rows) for _ in range(w.heads)]
    for ri, r in enumerate(rows):
        if queries == "video":
            f = r // cur.tokens_per_frame
            vis = [i for i, t in enumerate(toks) if brute_visible(w, t, f, r, csr)]
        else:
            qj = text_query_tail(cur, r)
            vis = [i for i, t in enumerate(toks) if brute_visible_text(w, t, qj)]
        qname = "q_vid" if queries == "video" else "q_txt"
        for h in range(w.heads):
            q = [float(bf16_to_fraction(int(b))) for b in data[qname][r, h, :]]
            scores = []
            for i in vis:
                k = val(i, h, "k")
                acc = 0.0
                for d in range(D):
                    acc += q[d] * k[d]
                scores.append(acc * sm_scale)
            m = max(scores)
            e = [math.exp(x - m) for x in scores]
            l = sum(e)
            o = [0.0] * D
            for wgt, i in zip(e, vis):
                v = val(i, h, "v")
                for d in range(D):
                    o[d] += wgt * v[d]
            O[ri][h] = [x / l for x in o]
            lse[h][ri] = m + math.log(l)
    return O, lse
