"""The MoE layer as plain Python loops, for tiny inputs only.

Test infrastructure only.  Independent of `moe` and of the tables in `nvfp4`:
codes are decoded here by their bit-field formulas, top-k is found by repeated
arg-max scans, dot products are explicit sums, and the combine walks tokens and
their k slots directly (no permutation).  Used to pin the vectorised oracle.
Follows the same passages as `oracle.moe` (page "Serving Solar Open 2 on DGX
Spark": top-k routing with one shared expert; contiguous expert shard with
shard-relative ids and dropped out-of-range pairs; per-shard partial sums).
"""
import math


def e2m1_by_formula(nib):
    s, e, m = (nib >> 3) & 1, (nib >> 1) & 3, nib & 1
    mag = m * 0.5 if e == 0 else math.ldexp(1.0 + m / 2.0, e - 1)
    return -mag if s else mag


def e4m3_by_formula(b):
    s, e, m = (b >> 7) & 1, (b >> 3) & 15, b & 7
    mag = math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7)
    return -mag if s else mag


def dequant_matrix(packed, scales, g):
    """packed: rows of bytes (list/array [R][C/2]); scales: [R][C/16] bytes."""
    R = len(packed)
    C = 2 * len(packed[0])
    W = [[0.0] * C for _ in range(R)]
    for r in range(R):
        for c in range(C):
            byte = int(packed[r][c // 2])
            nib = (byte & 15) if c % 2 == 0 else (byte >> 4)
            W[r][c] = e2m1_by_formula(nib) * e4m3_by_formula(int(scales[r][c // 16])) * float(g)
    return W


def fake_quant_row(v, g=1.0):
    """W4A4 activation quantize-dequantize of one row, by explicit loops; g is
    the static activation global (1: dynamic W4A4).  Decisions in fp32 (via
    struct round trips) like the vectorised oracle."""
    import struct

    def f32(z):
        return struct.unpack("f", struct.pack("f", z))[0]

    e2m1_vals = sorted({abs(e2m1_by_formula(n)) for n in range(8)})
    e4m3_vals = [e4m3_by_formula(b) for b in range(127)]

    def rne(val, grid):  # grid ascending, index = code
        if val >= grid[-1]:
            return len(grid) - 1
        best = 0
        for i in range(len(grid) - 1):
            if grid[i] <= val < grid[i + 1]:
                mid = (grid[i] + grid[i + 1]) / 2
                if val < mid:
                    best = i
                elif val > mid:
                    best = i + 1
                else:
                    best = i if i % 2 == 0 else i + 1
                break
        return best

    g = f32(g)
    out = []
    for b0 in range(0, len(v), 16):
        blk = [f32(z) for z in v[b0:b0 + 16]]
        amax = max(abs(z) for z in blk)
        s = e4m3_vals[rne(f32(amax / f32(6.0 * g)), e4m3_vals)]
        sg = f32(s * g)
        for z in blk:
            if sg == 0:
                out.append(0.0)
                continue
            r = f32(z / sg)
            mag = e2m1_vals[rne(abs(r), e2m1_vals)]
            out.append(-mag * s * g if (r < 0 and mag != 0) else mag * s * g)
    return out


def layer(x, gate, experts_q, shared_q, top_k, offset, num_local, w4a4=False, act_global=None):
    """x: [T][d] floats; gate: [d][E]; experts_q[l] / shared_q: dicts of
    packed codes, scales and g for w13 ([2F][d]) and w2 ([d][F]).
    act_global = (g of h, g of the SwiGLU output) selects static W4A4."""
    if act_global is not None:
        w4a4 = True
    ga = act_global if act_global is not None else (1.0, 1.0)
    T, d, E = len(x), len(x[0]), len(gate[0])

    def mlp(h, q):
        W13 = dequant_matrix(q["w13"], q["w13_scale"], q["g13"])
        W2 = dequant_matrix(q["w2"], q["w2_scale"], q["g2"])
        F = len(W13) // 2
        a = []
        for f in range(F):
            gsum = sum(W13[f][c] * h[c] for c in range(d))
            usum = sum(W13[F + f][c] * h[c] for c in range(d))
            a.append(gsum / (1.0 + math.exp(-gsum)) * usum if gsum > -700 else 0.0 * usum)
        if w4a4:
            a = fake_quant_row(a, ga[1])
        return [sum(W2[c][f] * a[f] for f in range(F)) for c in range(d)]

    out = [[0.0] * d for _ in range(T)]
    for t in range(T):
        logits = [sum(x[t][c] * gate[c][e] for c in range(d)) for e in range(E)]
        chosen = []
        for _ in range(top_k):                      # repeated arg-max, lower id on ties
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or logits[e] > logits[best]:
                    best = e
            chosen.append(best)
        zmax = logits[chosen[0]]
        den = sum(math.exp(logits[e] - zmax) for e in chosen)
        h = fake_quant_row(x[t], ga[0]) if w4a4 else list(x[t])
        for e in chosen:
            lam = e - offset
            if 0 <= lam < num_local:
                w = math.exp(logits[e] - zmax) / den
                y = mlp(h, experts_q[lam])
                for c in range(d):
                    out[t][c] += w * y[c]
        if shared_q is not None:
            y = mlp(h, shared_q)
            for c in range(d):
                out[t][c] += y[c]
    return out
