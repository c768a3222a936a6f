"""MaskInfo built by the plain definition (oracle; test-only).

Follows the splash page ("What is MaskInfo in splash attention?", "Does
splash attention make every sparse mask faster?", "What does grid shrinking
do in splash attention?") step by step, in the order the page gives:

  1. cut the mask into bq x bk grid-step blocks and label each one with the
     two questions chunk.any() / chunk.all(): 0 = all zeros, 1 = mixed,
     2 = all ones;
  2. dense (non-computable) masks only: store each distinct mixed block once
     (the "deduplicated stack" partial_mask_blocks, one byte per element) and
     remember, per grid position, which stored block it uses;
  3. grid shrink: per block row keep the non-empty columns in ascending
     order and pad every row to the longest row's count;
  4. data_next: per grid position, the key/value block to fetch there, so no
     block is fetched again across a skipped one;
  5. mask_next: per grid position, an index into partial_mask_blocks;
  6. downcast the three integer arrays to int8 / int16 when their largest
     value fits;
  7. q_sequence: the query indices (computable masks), used to recompute the
     mask in-kernel; for a single computable mask mask_next and
     partial_mask_blocks are None.

Readings taken where the page is silent (each also listed in the design
notes):
  * W = max(1, longest row); padding slots sit at the row end with label 0.
  * Empty / padding slots: data_next = column of the next non-empty slot in
    the row, else of the previous one, else 0.  mask_next at a non-partial
    slot: the index of the next partial slot, else the previous one, else 0.
    These fill values are a convention -- parity unpinned by the pages.
  * Deduplication order: first appearance in (head, row, column) row-major
    order over the unshrunk grid, across heads; equality is byte-wise.
  * Downcast: each array independently signed int8 if max <= 127, else
    int16 if max <= 32767, else int32; with downcast off all are int32.
    q_sequence always stays int32.
  * Shrink off: W = nk and every column is listed.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass
class MaskInfo:
    block_mask: np.ndarray                       # [Hm, nq, W] labels 0/1/2
    data_next: np.ndarray                        # [Hm, nq, W] key-block column
    mask_next: Optional[np.ndarray]              # [Hm, nq, W] index into partial blocks, or None
    partial_mask_blocks: Optional[np.ndarray]    # [P, bq, bk] uint8, or None
    q_sequence: Optional[np.ndarray]             # [Sq] int32, or None


def classify(mask, bq, bk):
    """Step 1: labels [Hm, nq, nk] by any/all over each bq x bk block."""
    hm, sq, skv = mask.shape
    if sq % bq or skv % bk:
        raise ValueError("block sizes must divide the sequence lengths")
    nq, nk = sq // bq, skv // bk
    labels = np.zeros((hm, nq, nk), dtype=np.int64)
    for h in range(hm):
        for r in range(nq):
            for c in range(nk):
                chunk = mask[h, r * bq:(r + 1) * bq, c * bk:(c + 1) * bk]
                if chunk.all():
                    labels[h, r, c] = 2
                elif chunk.any():
                    labels[h, r, c] = 1
    return labels


def classify_fast(mask, bq, bk):
    """Step 1 with numpy reductions instead of Python loops (same definition).

    Used for the large page workloads; tests check it equals classify() on
    small masks.
    """
    hm, sq, skv = mask.shape
    if sq % bq or skv % bk:
        raise ValueError("block sizes must divide the sequence lengths")
    nq, nk = sq // bq, skv // bk
    blocks = mask.reshape(hm, nq, bq, nk, bk)
    any_ = blocks.any(axis=(2, 4))
    all_ = blocks.all(axis=(2, 4))
    return np.where(all_, 2, np.where(any_, 1, 0)).astype(np.int64)


def _smallest_int(a):
    m = int(a.max()) if a.size else 0
    if m <= 127:
        return a.astype(np.int8)
    if m <= 32767:
        return a.astype(np.int16)
    return a.astype(np.int32)


def build(mask, bq, bk, computable, shrink=True, downcast=True, labels=None):
    """MaskInfo for a bool mask [Hm, Sq, Skv]; `computable` marks a single
    causal / local / chunked mask (no mask data is stored for it)."""
    mask = np.asarray(mask, dtype=bool)
    hm, sq, skv = mask.shape
    if labels is None:
        labels = classify_fast(mask, bq, bk)
    nq, nk = labels.shape[1], labels.shape[2]

    # Step 2: deduplicated stack of mixed blocks (dense masks only).
    pm = np.zeros((hm, nq, nk), dtype=np.int64)
    stack = []
    if not computable:
        seen = {}
        for h in range(hm):
            for r in range(nq):
                for c in range(nk):
                    if labels[h, r, c] != 1:
                        continue
                    blk = mask[h, r * bq:(r + 1) * bq, c * bk:(c + 1) * bk].astype(np.uint8)
                    key = blk.tobytes()
                    if key not in seen:
                        seen[key] = len(stack)
                        stack.append(blk)
                    pm[h, r, c] = seen[key]

    # Step 3: grid shrink -- the columns each block row keeps.
    rows = {}
    for h in range(hm):
        for r in range(nq):
            if shrink:
                rows[h, r] = [c for c in range(nk) if labels[h, r, c] > 0]
            else:
                rows[h, r] = list(range(nk))
    if shrink:
        width = max([1] + [len(v) for v in rows.values()])
    else:
        width = max(nk, 1)

    block_mask = np.zeros((hm, nq, width), dtype=np.int64)
    data_next = np.zeros((hm, nq, width), dtype=np.int64)
    mask_next = np.zeros((hm, nq, width), dtype=np.int64)
    for h in range(hm):
        for r in range(nq):
            cols = rows[h, r]
            lab = [labels[h, r, cols[s]] if s < len(cols) else 0 for s in range(width)]
            block_mask[h, r] = lab
            # Step 4: data_next -- own column if non-empty, else the next
            # non-empty slot's column, else the previous one's, else 0.
            nonempty = [s for s in range(width) if lab[s] > 0]
            for s in range(width):
                after = [t for t in nonempty if t >= s]
                before = [t for t in nonempty if t < s]
                if after:
                    data_next[h, r, s] = cols[after[0]]
                elif before:
                    data_next[h, r, s] = cols[before[-1]]
            # Step 5: mask_next -- the same rule over the partial slots.
            if not computable:
                partial = [s for s in range(width) if lab[s] == 1]
                for s in range(width):
                    after = [t for t in partial if t >= s]
                    before = [t for t in partial if t < s]
                    if after:
                        mask_next[h, r, s] = pm[h, r, cols[after[0]]]
                    elif before:
                        mask_next[h, r, s] = pm[h, r, cols[before[-1]]]

    # Step 6: downcast.
    conv = _smallest_int if downcast else (lambda a: a.astype(np.int32))
    bm = conv(block_mask)
    dn = conv(data_next)
    if computable:
        return MaskInfo(bm, dn, None, None, np.arange(sq, dtype=np.int32))
    if stack:
        pmb = np.stack(stack).astype(np.uint8)
    else:
        pmb = np.zeros((0, bq, bk), dtype=np.uint8)
    return MaskInfo(bm, dn, conv(mask_next), pmb, None)


def reconstruct(mi, q_len, kv_len, bq, bk, mask_fn=None):
    """Rebuild the dense mask a kernel would see from a MaskInfo.

    Label 0 -> nothing allowed; label 2 -> everything; label 1 -> the stored
    partial block mask_next points at (dense) or the mask function evaluated
    on (q_sequence rows, data_next columns) (computable).  Used as an
    invariant: it must give back the original mask exactly.
    """
    hm, nq, width = mi.block_mask.shape
    out = np.zeros((hm, q_len, kv_len), dtype=bool)
    for h in range(hm):
        for r in range(nq):
            for s in range(width):
                lab = int(mi.block_mask[h, r, s])
                if lab == 0:
                    continue
                c = int(mi.data_next[h, r, s])
                rs, cs = slice(r * bq, (r + 1) * bq), slice(c * bk, (c + 1) * bk)
                if lab == 2:
                    out[h, rs, cs] = True
                elif mi.partial_mask_blocks is not None:
                    out[h, rs, cs] = mi.partial_mask_blocks[int(mi.mask_next[h, r, s])] != 0
                else:
                    qpos = mi.q_sequence[r * bq:(r + 1) * bq]
                    out[h, rs, cs] = mask_fn(qpos, np.arange(c * bk, (c + 1) * bk))
    return out
