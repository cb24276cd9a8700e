"""Independent numpy brute force used to pin the oracle on small inputs.

These routines compute the same definitions as the oracle by different
means (library sorts, bincount, unique), so that a slip in the oracle's C++
shows up as a mismatch.
"""
import numpy as np


def keys(a):
    """Magnitude keys: IEEE bits of a float32 with the sign bit cleared."""
    return (np.asarray(a, np.float32).view(np.uint32) & np.uint32(0x7FFFFFFF)).astype(np.int64)


def topk_ef(g, r, k):
    g = np.asarray(g, np.float32)
    r = np.asarray(r, np.float32)
    a = (g + r).astype(np.float32)
    P, N = a.shape
    idx = np.zeros((P, k), np.uint32)
    val = np.zeros((P, k), np.float32)
    r_new = a.copy()
    for p in range(P):
        kk = keys(a[p])
        # lexsort: last key is primary -> sort by -key, then by index
        order = np.lexsort((np.arange(N), -kk))
        sel = np.sort(order[:k])
        idx[p] = sel
        val[p] = a[p, sel]
        r_new[p, sel] = 0.0
    return idx, val, r_new


def characterise(a_row, sel, k):
    """True iff `sel` is exactly the k first positions under (key desc, index asc)."""
    N = len(a_row)
    kk = keys(a_row)
    s = set(int(i) for i in sel)
    if len(s) != k or len(sel) != k:
        return False
    for i in s:
        for j in range(N):
            if j in s:
                continue
            if not (kk[i] > kk[j] or (kk[i] == kk[j] and i < j)):
                return False
    return True


def reduce(offsets, idx, val, N, delta):
    idx = np.asarray(idx, np.int64)
    val = np.asarray(val, np.float32)
    sums = np.bincount(idx, weights=val.astype(np.float64), minlength=N)[:N]
    union = np.unique(idx)
    K = int(union.size)
    T = np.ceil(np.float64(delta) * np.float64(N))
    if K >= T:
        return K, True, np.zeros(0, np.uint32), sums.astype(np.float32)
    return K, False, union.astype(np.uint32), sums[union].astype(np.float32)


def topk_ef_bucketed(g, r, bucket, kb):
    """Per bucket of `bucket` positions: the min(kb, len) first under (key
    desc, index asc) by a library lexsort; output rows concatenate buckets."""
    a = (np.asarray(g, np.float32) + np.asarray(r, np.float32)).astype(np.float32)
    P, N = a.shape
    idx_rows, val_rows = [], []
    r_new = a.copy()
    for p in range(P):
        ii, vv = [], []
        for lo in range(0, N, bucket):
            hi = min(lo + bucket, N)
            kk = keys(a[p, lo:hi])
            order = np.lexsort((np.arange(hi - lo), -kk))
            sel = np.sort(order[:min(kb, hi - lo)]) + lo
            ii.append(sel)
            vv.append(a[p, sel])
            r_new[p, sel] = 0.0
        idx_rows.append(np.concatenate(ii).astype(np.uint32) if ii else np.zeros(0, np.uint32))
        val_rows.append(np.concatenate(vv).astype(np.float32) if vv else np.zeros(0, np.float32))
    return np.stack(idx_rows), np.stack(val_rows), r_new


def topk_ef_layers(g, r, off, ks):
    """Per layer [off[l], off[l+1]): the k[l] first under (key desc, index asc)
    by a library lexsort; rows concatenate the layers."""
    a = (np.asarray(g, np.float32) + np.asarray(r, np.float32)).astype(np.float32)
    P, N = a.shape
    r_new = a.copy()
    idx_rows, val_rows = [], []
    for p in range(P):
        ii = []
        for l in range(len(ks)):
            lo, hi = int(off[l]), int(off[l + 1])
            kk = keys(a[p, lo:hi])
            order = np.lexsort((np.arange(hi - lo), -kk))
            ii.append(np.sort(order[:int(ks[l])]) + lo)
        sel = np.concatenate(ii).astype(np.int64) if ii else np.zeros(0, np.int64)
        idx_rows.append(sel.astype(np.uint32))
        val_rows.append(a[p, sel])
        r_new[p, sel] = 0.0
    return np.stack(idx_rows), np.stack(val_rows), r_new
