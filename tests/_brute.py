"""Pure-Python brute-force references used to pin the oracle on tiny inputs.

These are independent of ``oracle/``: element-by-element loops over Python
ints and floats, no numpy vectorisation, no matmul. They exist only to check
the oracle, and are far too slow for anything but tiny shapes.
"""
import math
import struct


def brute_align(topk_ids, E, b, capacity, base=0):
    """Sort-based alignment: valid routes (expert ID in [base, base + E))
    sorted by (expert ID, route ID); block entries are local indices."""
    flat = [int(e) for row in topk_ids for e in row]
    mk = len(flat)
    valid = [r for r in range(mk) if base <= flat[r] < base + E]
    order = sorted(valid, key=lambda r: (flat[r], r))
    rows, blocks = [], []
    i = 0
    while i < len(order):
        e = flat[order[i]]
        j = i
        while j < len(order) and flat[order[j]] == e:
            j += 1
        seg = order[i:j]
        while len(seg) % b:
            seg = seg + [mk]
        rows.extend(seg)
        blocks.extend([e - base] * (len(seg) // b))
        i = j
    n = len(rows)
    rows += [mk] * (capacity - n)
    blocks += [-1] * (capacity // b - len(blocks))
    return rows, blocks, n


def bf16_bits_to_float(bits):
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def deq_elem(q, s, z, g, e, n, kk):
    word = int(q[e][n][kk // 8])
    j = kk % 8
    # even element 2m in nibble slot m, odd element 2m+1 in slot m+4
    nib = (word >> (4 * (j >> 1) + 16 * (j & 1))) & 0xF
    return (nib - int(z[e][n][kk // g])) * float(s[e][n][kk // g])


def brute_ffn(x_bits, topk_ids, topk_w, w13, w2, E, base=0):
    """y[t][h] by explicit loops over tokens, routes, neurons and elements;
    expert ID e is valid in [base, base + E) and uses weight index e - base."""
    M = len(topk_ids)
    k = len(topk_ids[0])
    H = len(x_bits[0])
    I = w13.N // 2
    q13, s13, z13, g13 = w13.q.tolist(), w13.s.astype(float).tolist(), w13.z.tolist(), w13.g
    q2, s2, z2, g2 = w2.q.tolist(), w2.s.astype(float).tolist(), w2.z.tolist(), w2.g
    y = [[0.0] * H for _ in range(M)]
    for t in range(M):
        x = [bf16_bits_to_float(v) for v in x_bits[t]]
        for j in range(k):
            e = int(topk_ids[t][j]) - base
            if not (0 <= e < E):
                continue
            wt = float(topk_w[t][j])
            a = []
            for i in range(I):
                gate = 0.0
                up = 0.0
                for h in range(H):
                    gate += x[h] * deq_elem(q13, s13, z13, g13, e, i, h)
                    up += x[h] * deq_elem(q13, s13, z13, g13, e, I + i, h)
                a.append(gate / (1.0 + math.exp(-gate)) * up)
            for h in range(H):
                acc = 0.0
                for i in range(I):
                    acc += a[i] * deq_elem(q2, s2, z2, g2, e, h, i)
                y[t][h] += wt * acc
    return y


def brute_batched(x_bits, counts, w13, w2):
    """Per expert e and row n < clamp(counts[e]): the gate/up product a and the
    down product yhat by explicit loops (lists of lists)."""
    E, cap, H = len(x_bits), len(x_bits[0]), len(x_bits[0][0])
    I = w13.N // 2
    q13, s13, z13, g13 = w13.q.tolist(), w13.s.astype(float).tolist(), w13.z.tolist(), w13.g
    q2, s2, z2, g2 = w2.q.tolist(), w2.s.astype(float).tolist(), w2.z.tolist(), w2.g
    a = [[[0.0] * I for _ in range(cap)] for _ in range(E)]
    y = [[[0.0] * H for _ in range(cap)] for _ in range(E)]
    for e in range(E):
        n_e = min(max(int(counts[e]), 0), cap)
        for n in range(n_e):
            x = [bf16_bits_to_float(v) for v in x_bits[e][n]]
            for i in range(I):
                gate = sum(x[h] * deq_elem(q13, s13, z13, g13, e, i, h) for h in range(H))
                up = sum(x[h] * deq_elem(q13, s13, z13, g13, e, I + i, h) for h in range(H))
                a[e][n][i] = gate / (1.0 + math.exp(-gate)) * up
            for h in range(H):
                y[e][n][h] = sum(a[e][n][i] * deq_elem(q2, s2, z2, g2, e, h, i) for i in range(I))
    return a, y
