"""Mask definitions, materialised as dense bool arrays (oracle; test-only).

The splash page names three "computable" masks -- CausalMask, LocalMask and
ChunkedCausalMask -- whose blocks the kernel recomputes instead of loading,
and dense masks given as arrays (the random-mask answer).  The pages never
write the predicates out, so the plainest readings are used:

  causal          key j allowed for query i  iff  j <= i
  local(L, R)     i - L <= j <= i + R, both ends inclusive; a side given as
                  None (or a negative number) is unbounded
  chunked(C)      i // C == j // C  and  j <= i  (chunks start at position 0)
  dense           the given [Hm, Sq, Skv] array, nonzero = allowed

Query and key positions are plain indices 0..Sq-1 and 0..Skv-1 (top-left
alignment).
"""
import numpy as np

COMPUTABLE = ("causal", "local", "chunked")


def _bound(x):
    return None if x is None or x < 0 else int(x)


def allowed_block(kind, rows, cols, left=None, right=None, chunk=None, dense=None, head=0):
    """Bool matrix allowed[i, j] for query positions `rows` and key positions `cols`."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    if kind == "causal":
        return j <= i
    if kind == "local":
        lo, hi = _bound(left), _bound(right)
        ok = np.ones((i.shape[0], j.shape[1]), dtype=bool)
        if lo is not None:
            ok &= j >= i - lo
        if hi is not None:
            ok &= j <= i + hi
        return ok
    if kind == "chunked":
        if chunk is None or chunk <= 0:
            raise ValueError("chunked mask needs a positive chunk size")
        return (i // chunk == j // chunk) & (j <= i)
    if kind == "dense":
        d = np.asarray(dense)
        return d[head][np.ix_(np.asarray(rows), np.asarray(cols))] != 0
    raise ValueError(f"unknown mask kind {kind!r}")


def materialize(kind, q_len, kv_len, left=None, right=None, chunk=None, dense=None):
    """Full mask as a bool array [Hm, q_len, kv_len] (Hm = 1 for computable masks)."""
    if kind == "dense":
        d = np.asarray(dense)
        if d.ndim == 2:
            d = d[None]
        if d.shape[1:] != (q_len, kv_len):
            raise ValueError("dense mask shape does not match (q_len, kv_len)")
        return d != 0
    m = allowed_block(kind, np.arange(q_len), np.arange(kv_len), left, right, chunk)
    return m[None]
