"""Host mirror of the split plan that the decode's prep kernel computes on the
GPU (csrc/plan.h, plan_block), step for step, and of the workspace layout
it is written into (csrc/common.h, make_layout). Host logic for the tests: the
CPU test checks the plan's invariants on random batches, the GPU test checks
that the device writes exactly this plan. Not part of the oracle: the plan
decides only how the exact softmax sum is regrouped.
"""
import math, numpy as np
KW, SORTMAX, MINC, COST, TILE = 4, 1024, 64, 6, 32

def layout(B, sq, max_seq_len, P):
    """(positions, depth, partial-slot capacity) of the workspace."""
    max_blocks = -(-max_seq_len // 64)
    positions = -(-P // 8) * 8
    depth = max(KW, 1 + -(-B // P))   # searched plan: <= KW rounds; simple plan: <= 1 + ceil(B / P)
    cap = depth * P
    max_chunks = max(1, min(cap, B * max_blocks))
    return positions, depth, max_chunks

def up64(x): return -(-x // MINC) * MINC

def plan(lens, max_len, P, positions, depth, max_chunks):
    B = len(lens)
    L = [min(max(int(x), 0), max_len) for x in lens]
    total = sum(L); n_ne = sum(1 for x in L if x > 0); max_l = max(L) if L else 0
    search = total > 0 and B <= SORTMAX and n_ne <= KW * P
    if search:
        lo, hi, feas = [], [], []
        for k in range(KW):
            cap = (k + 1) * P
            feas.append(cap >= n_ne)
            l = max(up64(-(-total // cap)), MINC); h = max(up64(max_l), MINC)
            if cap > n_ne: h = min(h, max(up64(-(-total // (cap - n_ne))), MINC))
            lo.append(min(l, h)); hi.append(h)
        while True:
            opn = [feas[k] and lo[k] < hi[k] for k in range(KW)]
            if not any(opn): break
            mid = [lo[k] + (hi[k] - lo[k]) // (2 * MINC) * MINC if opn[k] else hi[k] for k in range(KW)]
            for k in range(KW):
                if opn[k]:
                    n = sum(-(-x // mid[k]) for x in L)
                    if n <= (k + 1) * P: hi[k] = mid[k]
                    else: lo[k] = mid[k] + MINC
        best = None; C = hi[KW - 1]
        for k in range(KW):
            if not feas[k]: continue
            cost = (k + 1) * (-(-lo[k] // TILE) + COST)
            if best is None or cost < best: best, C = cost, lo[k]
    else:
        C = max(up64(-(-total // P)), MINC)
        C = min(C, max(up64(max_l), MINC))   # no longer than the longest sequence needs
    def pieces(x):
        if x <= 0: return 0, MINC
        nb = -(-x // C)
        if search:
            base = up64(-(-x // nb)); return -(-x // base), base
        return nb, C
    per_xcd = positions // 8
    def entry(k):
        i = k % P
        return (k // P) * positions + (i % per_xcd) * 8 + i // per_xcd
    work = {}; seqinfo = []
    slot = 0; items = []   # (k, b, t0, t1, slot)
    n_all = [pieces(x)[0] for x in L]
    if not search:
        tot_full = sum(x // C for x in L)
        full_idx, tail_idx = 0, tot_full
        for b, x in enumerate(L):
            n, base = pieces(x); nf = x // C
            seqinfo.append((slot, n, x))
            for q in range(nf): items.append((full_idx, b, q * C, (q + 1) * C, slot + q)); full_idx += 1
            if n > nf: items.append((tail_idx, b, nf * C, x, slot + nf)); tail_idx += 1
            slot += n
    else:
        info = []
        for b, x in enumerate(L):
            n, base = pieces(x); seqinfo.append((slot, n, x)); info.append((n, base, slot)); slot += n
        n_items_ = sum(x[0] for x in info)
        if n_items_ <= P:   # one round: sequence order, no sort
            keys = list(range(B))
        else:
            keys = sorted(((4095 - min(info[b][1] // 64, 4095)) << 20) | b for b in range(B))
        start = 0
        for kk in keys:
            b = kk & 0xfffff; n, base, sl = info[b]
            for q in range(n): items.append((start + q, b, q * base, min((q + 1) * base, L[b]), sl + q))
            start += n
    n_items = sum(n_all)
    for k, b, t0, t1, sl in items:
        if sl < max_chunks and k // P < depth:
            e = entry(k); assert e not in work, 'entry written twice'; work[e] = (b, t0, t1, sl)
    return dict(C=C, search=search, n_items=n_items, work=work, seqinfo=seqinfo, L=L)

def check(lens, max_seq_len, P):
    """Plans the batch and asserts every invariant the attention and merge
    passes rely on; returns the plan."""
    positions, depth, max_chunks = layout(len(lens), 1, max_seq_len, P)
    r = plan(lens, max_seq_len, P, positions, depth, max_chunks)
    L = r['L']; work = r['work']
    assert r['n_items'] <= max_chunks and r['n_items'] <= depth * P, (r['n_items'], max_chunks, depth * P)
    assert len(work) == r['n_items']
    cov = {}
    for e, (b, t0, t1, sl) in work.items():
        assert 0 <= e < depth * positions
        assert t0 % 64 == 0 and t0 < t1 <= L[b] and (t1 % 64 == 0 or t1 == L[b])
        cov.setdefault(b, []).append((t0, t1, sl))
    for b, x in enumerate(L):
        segs = sorted(cov.get(b, []))
        base, n, _ = r['seqinfo'][b]
        assert len(segs) == n
        pos = 0
        for i, (t0, t1, sl) in enumerate(segs):
            assert t0 == pos and sl == base + i; pos = t1
        assert pos == x
    # each position's entries are dense from depth 0
    for p in range(positions):
        used = [j for j in range(depth) if j * positions + p in work]
        assert used == list(range(len(used)))
    return r

