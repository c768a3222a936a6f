"""Dense fp64 masked softmax attention (oracle; test-only).

Splash and flash attention compute the same masked softmax attention and
differ only in which work they skip (splash page, "What is splash attention
and how is it different from flash attention?").  So this oracle is the
plain definition, in float64, with no tiling and no online softmax:

  s_ij  = scale * <q_i, k_j>           scale defaults to head_dim ** -0.5
                                       (EasyDeL BlockSparseAttn.forward_native)
  s_ij <- c * tanh(s_ij / c)           only if a logits soft cap c is given;
                                       the pages name the parameter but not the
                                       formula -- the usual tanh cap on the
                                       scaled logits, before masking, is taken
  over allowed j:  M_i = max s_ij,  lse_i = M_i + ln sum_j exp(s_ij - M_i),
                   o_i = sum_j exp(s_ij - lse_i) v_j
  no allowed j:    o_i = 0, lse_i = -inf

lse is the natural-log residual the flash kernel keeps for its backward pass
(pallas-flash-attention-tpu page, "What does the TPU flash attention kernel
save for the backward pass?": the running max and the running sum; here
combined as max + log(sum)).

GQA/MQA: query head h reads key/value head h // (Hq // Hkv).
Mask heads: Hm == 1 is shared by every query head; Hm == Hq is per head.

Attention sinks (softmax_aux of the EasyDeL BlockSparseAttn.forward_native
signature, typed [num_kv_heads, num_sinks] or [num_sinks]): the pages give
the argument, not its arithmetic.  The reading taken is the usual one: each
sink logit a_k is one more column of the softmax that carries no value, so

  lse_i = ln( sum_{allowed j} exp(s_ij) + sum_k exp(a_k) ),
  o_i   = sum_{allowed j} exp(s_ij - lse_i) v_j,

unscaled and uncapped (the logits are given as they enter the softmax).  A
[num_kv_heads, ns] array gives query head h the row of its key/value head
h // (Hq // Hkv); a [Hq, ns] array one row per query head; [ns] is shared.
A row with no allowed key then has o_i = 0 and lse_i = ln sum_k exp(a_k).
"""
import numpy as np


def attention_rows(q, k, v, allowed, scale=None, soft_cap=None, sinks=None):
    """One (batch, head): q [n, D], k [Skv, D], v [Skv, Dv], allowed [n, Skv] bool;
    sinks: this head's sink logits [ns] or None.

    Returns (o [n, Dv] float64, lse [n] float64).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = q.shape[-1] ** -0.5
    s = scale * (q @ k.T)
    if soft_cap is not None:
        s = soft_cap * np.tanh(s / soft_cap)
    s = np.where(allowed, s, -np.inf)
    if sinks is not None and len(sinks):
        # the sinks are extra softmax columns whose value rows are zero
        a = np.broadcast_to(np.asarray(sinks, dtype=np.float64), (s.shape[0], len(sinks)))
        s = np.concatenate([s, a], axis=1)
        v = np.concatenate([v, np.zeros((len(sinks), v.shape[1]))], axis=0)
    m = s.max(axis=1)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    e = np.exp(s - m_safe[:, None])            # exp(-inf) = 0 at masked entries
    total = e.sum(axis=1)
    lse = np.where(has, m_safe + np.log(np.where(has, total, 1.0)), -np.inf)
    w = np.where(has[:, None], e / np.where(has, total, 1.0)[:, None], 0.0)
    o = w @ v
    return o, lse


def sink_row(softmax_aux, h, hq, hkv):
    """Sink logits of query head h, or None (see the module docstring)."""
    if softmax_aux is None:
        return None
    a = np.asarray(softmax_aux, dtype=np.float64)
    if a.ndim == 1:
        return a
    if a.shape[0] == hkv:
        return a[h // (hq // hkv)]
    if a.shape[0] == hq:
        return a[h]
    raise ValueError("softmax_aux must be [ns], [Hkv, ns] or [Hq, ns]")


def attention(q, k, v, mask_rows, scale=None, soft_cap=None, row_chunk=512, softmax_aux=None):
    """Full attention.

    q [B, Hq, Sq, D], k [B, Hkv, Skv, D], v [B, Hkv, Skv, Dv] (any float type,
    upcast to float64); mask_rows(head, rows) -> bool [len(rows), Skv] gives
    the allowed keys for the query positions `rows` of mask head `head`
    (callers pass head = 0 for a shared mask).

    Returns (o [B, Hq, Sq, Dv], lse [B, Hq, Sq]) in float64.  Rows are done
    in chunks so no Sq x Skv float64 slab is held whole.
    """
    b_, hq, sq, _ = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    o = np.zeros((b_, hq, sq, v.shape[-1]), dtype=np.float64)
    lse = np.zeros((b_, hq, sq), dtype=np.float64)
    for b in range(b_):
        for h in range(hq):
            kk = np.asarray(k[b, h // group], dtype=np.float64)
            vv = np.asarray(v[b, h // group], dtype=np.float64)
            for i0 in range(0, sq, row_chunk):
                rows = np.arange(i0, min(sq, i0 + row_chunk))
                ob, lb = attention_rows(q[b, h, rows], kk, vv, mask_rows(h, rows), scale, soft_cap,
                                        sink_row(softmax_aux, h, hq, hkv))
                o[b, h, rows] = ob
                lse[b, h, rows] = lb
    return o, lse


def attention_sampled(q, k, v, mask_rows, samples, scale=None, soft_cap=None, softmax_aux=None):
    """Selected output rows only: samples = iterable of (b, h, i).

    Returns (o [n, Dv], lse [n]) in the order given.  Used at full workload
    sizes, where the whole output is too costly to compute in float64.
    """
    hq, hkv = q.shape[1], k.shape[1]
    group = hq // hkv
    outs, lses = [], []
    for b, h, i in samples:
        ob, lb = attention_rows(q[b, h, [i]], k[b, h // group], v[b, h // group],
                                mask_rows(h, np.array([i])), scale, soft_cap,
                                sink_row(softmax_aux, h, hq, hkv))
        outs.append(ob[0])
        lses.append(lb[0])
    return np.stack(outs), np.array(lses)


def merge(o_a, lse_a, o_b, lse_b):
    """Combine two attention results over disjoint key sets into the result
    over their union (ring attention on the splash page: each shard's
    partial result carries its own max and normaliser, and the partials are
    rescaled the way flash attention rescales inside one kernel).  With
    lse = ln(e^lse_a + e^lse_b), the union's output is
    e^(lse_a - lse) o_a + e^(lse_b - lse) o_b.  A part whose lse is -inf (no
    allowed key in that shard) contributes nothing, whatever its output
    holds -- the tokamax variant's rule of zeroing inactive shards.

    o_* [..., Dv], lse_* [...]; returns (o, lse) in float64."""
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    has = np.isfinite(lse)
    ref = np.where(has, lse, 0.0)
    wa = np.where(np.isfinite(lse_a), np.exp(np.where(np.isfinite(lse_a), lse_a, 0.0) - ref), 0.0)
    wb = np.where(np.isfinite(lse_b), np.exp(np.where(np.isfinite(lse_b), lse_b, 0.0) - ref), 0.0)
    pa = np.where(np.isfinite(lse_a)[..., None], o_a, 0.0)
    pb = np.where(np.isfinite(lse_b)[..., None], o_b, 0.0)
    o = wa[..., None] * pa + wb[..., None] * pb
    return o, lse


def attention_bwd_rows(q, k, v, do, allowed, scale=None, soft_cap=None):
    """Gradients of one (batch, head): q [n, D], k [Skv, D], v [Skv, Dv],
    do [n, Dv] (the gradient of the output), allowed [n, Skv] bool.

    The backward the pages describe for flash attention (pallas flash
    attention page, "What does the TPU flash attention kernel save for the
    backward pass?" and "Why does the TPU flash attention backward pass run
    two kernels instead of one?"): the weights are rebuilt from q, k and the
    forward's log-sum-exp, and the row-wise dot product di = <do_i, o_i> is
    formed once.  With p_ij = exp(s'_ij - lse_i) on allowed pairs (0
    elsewhere), s' the capped or plain scaled logit:

      dv_j  = sum_i p_ij do_i
      dp_ij = <do_i, v_j>
      ds'_ij = p_ij (dp_ij - di_i)
      ds_ij = ds'_ij * (1 - tanh^2(s_ij / c))     (soft cap c; else ds = ds')
      dq_i  = scale * sum_j ds_ij k_j
      dk_j  = scale * sum_i ds_ij q_i

    Returns (dq [n, D], dk [Skv, D], dv [Skv, Dv]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    if scale is None:
        scale = q.shape[-1] ** -0.5
    o, lse = attention_rows(q, k, v, allowed, scale, soft_cap)
    s = scale * (q @ k.T)
    if soft_cap is not None:
        t = np.tanh(s / soft_cap)
        sc = soft_cap * t
    else:
        sc = s
    has = np.isfinite(lse)
    p = np.where(allowed & has[:, None], np.exp(sc - np.where(has, lse, 0.0)[:, None]), 0.0)
    di = (do * o).sum(axis=1)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - di[:, None])
    if soft_cap is not None:
        ds = ds * (1.0 - t * t)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_bwd(q, k, v, do, mask_rows, scale=None, soft_cap=None, row_chunk=512):
    """Gradients of attention(...) for the output gradient do [B, Hq, Sq, Dv].
    Key/value gradients of a GQA group sum over its query heads.
    Returns (dq, dk, dv) in float64, shaped like q, k, v."""
    b_, hq, sq, _ = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(b_):
        for h in range(hq):
            g = h // group
            for i0 in range(0, sq, row_chunk):
                rows = np.arange(i0, min(sq, i0 + row_chunk))
                a, bk_, bv = attention_bwd_rows(q[b, h, rows], k[b, g], v[b, g], do[b, h, rows],
                                                mask_rows(h, rows), scale, soft_cap)
                dq[b, h, rows] = a
                dk[b, g] += bk_
                dv[b, g] += bv
    return dq, dk, dv
