"""Host model of the split-KV schedule the device computes.

Rule (also stated in the scheduler source): sequence b has n_b = max(1,
ceil(L_b/64)) page slots and costs c0 + n_b units; the units of all
sequences are laid end to end and partition p starts at unit p*q with
q = ceil(T / num_parts).  A start inside b's c0 overhead units maps to page 0
of b, inside its page units to page (p*q - U_b - c0).
"""

PAGE = 64


def schedule(seqlens, num_parts, c0):
    batch = len(seqlens)
    n = [max(1, (int(L) + PAGE - 1) // PAGE) for L in seqlens]
    cost = [c0 + nb for nb in n]
    U = [0] * batch
    acc = 0
    for b in range(batch):
        U[b] = acc
        acc += cost[b]
    T = acc
    q = -(-T // num_parts)
    begins = [(batch, 0, 0)] * (num_parts + 1)
    nsplit = [0] * batch
    for b in range(batch):
        A = U[b] + c0
        nsplit[b] = 1 + (A + n[b] - 1) // q - A // q
        p_lo = -(-U[b] // q)
        p_hi = (U[b] + cost[b] - 1) // q
        for p in range(p_lo, min(p_hi, num_parts - 1) + 1):
            u = p * q
            if u > A:
                begins[p] = (b, u - A, p - A // q)
            else:
                begins[p] = (b, 0, 0)
    splits = [0] * (batch + 1)
    for b in range(batch):
        splits[b + 1] = splits[b] + nsplit[b]
    meta = []
    for p in range(num_parts):
        bb, bj, first = begins[p]
        eb, ej, _ = begins[p + 1]
        meta.append([bb, bj, eb, ej, first, q, c0, min(T, 2**31 - 1)])
    return meta, splits, n


def partition_items(meta_row, n):
    """(b, j) items of one partition, in order."""
    bb, bj, eb, ej = meta_row[:4]
    items = []
    b, j = bb, bj
    while (b, j) < (eb, ej):
        items.append((b, j))
        if j + 1 < n[b]:
            j += 1
        else:
            b, j = b + 1, 0
    return items
