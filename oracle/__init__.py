"""Plain fp64 CPU oracle for the fused linear log-prob operator.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg do. It shares no code
with the HIP library (no kernels, headers, helpers or constants) and imports nothing from it.

Every function is the plain definition of what the operator computes, written out in fp64
NumPy on the exact fp64 values of the bf16 inputs. The only blocking is over rows, which are
independent by definition. Library primitives used as steps: matrix product, exp, log, sort.

Sources (cited by page title and section; the pages are three pull-request descriptions):
  [CUDA provider]  "feat(rl-kernel): add CUDA linear logp provider integration"
  [ROCm provider]  "feat(rl-kernel): add ROCm linear logp provider integration"
  [top-p replay]   "Perf/cuda compact top p replay"

Readings where the pages are silent (each is listed with its reason in the design notes):
  * logits are z = (h W^T + b) / tau with tau applied exactly once, after the bias;
  * padded vocabulary columns (global id >= real_vocab) are not part of the distribution;
  * entropy is that of softmax(z) over the real vocabulary, in nats;
  * loss-masked rows produce 0 for every output and a zero gradient;
  * an empty shard gives lse = -inf, target logit 0, in_range 0, entropy 0, local logp -inf;
  * a row whose target no shard holds gets logp = -inf (and a status bit on the device).

Status bits mirror the C header: 1 target outside [0, real_vocab), 2 target not found after
the merge, 4 replay id outside [-1, real_vocab).

Parity status: every function here is pinned by tests that do not reuse its formulas
(mpmath brute force, torch library routines, closed forms, finite differences, invariants).
"""
from __future__ import annotations

import numpy as np

ST_TARGET_OUT_OF_RANGE = 1
ST_TARGET_NOT_FOUND = 2
ST_REPLAY_ID_INVALID = 4

NEG_INF = -np.inf


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact fp64 value of bf16 bit patterns (a bf16 is the top half of an fp32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_f64(x) -> np.ndarray | None:
    """uint16 arrays are bf16 bit patterns; anything else is converted as a number."""
    if x is None:
        return None
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    return x if x.dtype == np.float64 else x.astype(np.float64)


def logits(h: np.ndarray, w_rows: np.ndarray, bias_rows, temperature: float) -> np.ndarray:
    """z = (h . W^T + b) / tau for the given weight rows.

    [CUDA provider, "Megatron integration"]: the request carries the output-layer hidden
    states and the local projection weight and bias. [ROCm provider, "Megatron integration"]
    and [top-p replay, "Summary"]: temperature scaling happens exactly once.
    """
    z = h @ w_rows.T
    if bias_rows is not None:
        z = z + bias_rows[None, :]
    return z / temperature


def softmax_stats(z: np.ndarray):
    """Per row: lse = log sum_v exp(z_v); entropy = -sum_v p_v log p_v with p = softmax(z).

    A row with no columns is the empty-shard case of [top-p replay, "Changes" table, CUDA
    kernel and empty-shard handling]: lse = -inf and entropy 0 (zero probabilities).
    """
    n = z.shape[0]
    if z.shape[1] == 0:
        return np.full(n, NEG_INF), np.zeros(n)
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    s = e.sum(axis=1)
    lse = m + np.log(s)
    p = e / s[:, None]
    entropy = lse - (p * z).sum(axis=1)  # -sum p (z - lse), sum p = 1
    return lse, entropy


def shard_forward(hidden, weight, bias, temperature: float, targets, mask, offset: int,
                  local_size: int, real_vocab: int, row_block: int = 256) -> dict:
    """Per-shard partials of one vocabulary shard.

    The shard owns global ids [offset, offset + local_size) of the padded vocabulary
    ([CUDA provider, "Megatron integration"]: tensor-parallel vocabulary range and real/padded
    vocabulary sizes); its real columns are the first clamp(real_vocab - offset, 0, local_size).
    Returns, per row, target_logit, in_range, lse, entropy and the local logp
    (target_logit - lse when the target lies in the shard, else -inf).
    ``weight`` holds the shard's local rows (bf16 bits or numbers), ``bias`` its local bias.
    """
    h = as_f64(hidden)
    T = h.shape[0]
    targets = np.asarray(targets, dtype=np.int64)
    mask = np.ones(T, dtype=bool) if mask is None else np.asarray(mask).astype(bool)
    n_real = int(min(max(real_vocab - offset, 0), local_size))
    w = as_f64(np.asarray(weight)[:n_real]) if n_real > 0 else np.zeros((0, h.shape[1]))
    b = as_f64(np.asarray(bias)[:n_real]) if bias is not None else None

    out = dict(target_logit=np.zeros(T), in_range=np.zeros(T, dtype=np.uint8),
               lse=np.zeros(T), entropy=np.zeros(T), logp=np.zeros(T), status=0)
    rows = np.nonzero(mask)[0]
    bad = rows[(targets[rows] < 0) | (targets[rows] >= real_vocab)]
    if bad.size:
        out["status"] |= ST_TARGET_OUT_OF_RANGE
    for i in range(0, rows.size, row_block):
        r = rows[i:i + row_block]
        z = logits(h[r], w, b, temperature)
        lse, ent = softmax_stats(z)
        loc = targets[r] - offset
        hit = (loc >= 0) & (loc < n_real) & (targets[r] < real_vocab)
        t = np.zeros(r.size)
        t[hit] = z[np.nonzero(hit)[0], loc[hit]]
        out["target_logit"][r] = t
        out["in_range"][r] = hit.astype(np.uint8)
        out["lse"][r] = lse
        out["entropy"][r] = ent
        out["logp"][r] = np.where(hit, t - lse, NEG_INF)
    return out


def forward(hidden, weight, bias, temperature: float, targets, mask, real_vocab: int,
            row_block: int = 256) -> dict:
    """Unsharded forward: the full vocabulary is one shard at offset 0.

    [CUDA provider, "Motivation"]: the provider returns log probabilities of the selected
    tokens and optional entropy. logp = z[target] - lse over the real vocabulary.
    """
    w = np.asarray(weight)
    out = shard_forward(hidden, w, bias, temperature, targets, mask, 0, w.shape[0], real_vocab,
                        row_block)
    hit = out["in_range"].astype(bool)
    scored = np.ones(len(out["lse"]), bool) if mask is None else np.asarray(mask).astype(bool)
    if np.any(scored & ~hit):
        out["status"] |= ST_TARGET_NOT_FOUND
    return out


def merge(parts: list, mask=None) -> dict:
    """Rank-ordered merge of per-shard partials ([top-p replay, "Summary"]: rank-ordered
    reductions, including shards with no candidates).

    For shards r = 0..R-1 in order: M = max_r lse_r; lse = M + log sum_r exp(lse_r - M)
    (empty shards, lse_r = -inf, contribute nothing; all empty gives -inf). The target logit
    is the one from the shard holding the target; logp = target - lse, or -inf if no shard
    holds it. Entropy: with w_r = exp(lse_r - lse), H = sum_r w_r (H_r + lse - lse_r), which
    is -sum_v p_v log p_v over the union of the shards' columns.
    """
    R = len(parts)
    T = len(parts[0]["lse"])
    L = np.stack([np.asarray(p["lse"], dtype=np.float64) for p in parts])       # [R, T]
    tl = np.stack([np.asarray(p["target_logit"], dtype=np.float64) for p in parts])
    fl = np.stack([np.asarray(p["in_range"]).astype(bool) for p in parts])
    have_ent = all(p.get("entropy") is not None for p in parts)
    Hs = np.stack([np.asarray(p["entropy"], dtype=np.float64) for p in parts]) if have_ent else None
    scored = np.ones(T, bool) if mask is None else np.asarray(mask).astype(bool)

    out = dict(logp=np.zeros(T), lse=np.zeros(T), entropy=np.zeros(T), status=0)
    for t in np.nonzero(scored)[0]:
        live = [r for r in range(R) if L[r, t] != NEG_INF]
        if not live:
            lse = NEG_INF
        else:
            M = max(L[r, t] for r in live)
            S = 0.0
            for r in live:
                S += np.exp(L[r, t] - M)
            lse = M + np.log(S)
        found = [r for r in range(R) if fl[r, t]]
        if found:
            out["logp"][t] = tl[found[0], t] - lse
        else:
            out["logp"][t] = NEG_INF
            out["status"] |= ST_TARGET_NOT_FOUND
        out["lse"][t] = lse
        if have_ent and live:
            ent = 0.0
            for r in live:
                ent += np.exp(L[r, t] - lse) * (Hs[r, t] + lse - L[r, t])
            out["entropy"][t] = ent
    return out


def backward(hidden, weight, bias, temperature: float, targets, mask, offset: int,
             local_size: int, real_vocab: int, lse, dlogp, dentropy=None, entropy=None,
             want_g: bool = False) -> dict:
    """Gradients of sum_t dlogp_t * logp_t (+ sum_t dentropy_t * entropy_t) for one shard.

    The pages require gradients to flow ([CUDA provider, "Motivation"]: strict mode rejects
    detached gradients) but print no formula; this is the derivative of the definitions above.
    With p = exp(z - lse) (lse = the merged, global log-sum-exp):
      dlogp_t/dz_v   = 1[v = target_t] - p_v
      dentropy_t/dz_v = -p_v (z_v - E_p[z]),  E_p[z] = lse - entropy
    and z = (h W^T + b)/tau, so G = dL/dz / tau, dH = G W, dW = G^T h, db = sum_t G.
    Padded columns and masked rows get no gradient; padded dW / db rows are zero.
    """
    h = as_f64(hidden)
    T, Hd = h.shape
    n_real = int(min(max(real_vocab - offset, 0), local_size))
    w_all = as_f64(weight)
    w = w_all[:n_real]
    b = as_f64(np.asarray(bias)[:n_real]) if bias is not None else None
    mask = np.ones(T, bool) if mask is None else np.asarray(mask).astype(bool)
    targets = np.asarray(targets, dtype=np.int64)
    z = logits(h, w, b, temperature)
    lse = np.asarray(lse, dtype=np.float64)
    p = np.exp(z - lse[:, None])
    loc = targets - offset
    onehot = np.zeros_like(z)
    ok = (loc >= 0) & (loc < n_real)
    onehot[np.nonzero(ok)[0], loc[ok]] = 1.0
    g = np.asarray(dlogp, dtype=np.float64)[:, None] * (onehot - p)
    if dentropy is not None:
        ez = lse - np.asarray(entropy, dtype=np.float64)
        g = g + np.asarray(dentropy, dtype=np.float64)[:, None] * (-p * (z - ez[:, None]))
    g = g / temperature
    g[~mask] = 0.0
    dH = g @ w
    dW = np.zeros((local_size, Hd))
    dW[:n_real] = g.T @ h
    db = np.zeros(local_size)
    db[:n_real] = g.sum(axis=0)
    out = dict(dhidden=dH, dweight=dW, dbias=db)
    if want_g:
        out["G"] = g
    return out


def top_p_replay(logits_rows, replay_ids, targets, temperature: float, offset: int,
                 local_size: int, real_vocab: int, mask=None) -> dict:
    """Compact top-p replay scoring of one vocabulary shard.

    [top-p replay, "Summary"]: replay the native finite nucleus and score the compact replay
    ids directly; [top-p replay, "Changes" table]: up to 64 ids are sorted and deduplicated
    and temperature is applied. Per row, U = the distinct listed ids that fall in the shard's
    real range (-1 marks an empty slot); lse_N = log sum_{v in U} exp(x_v / tau); the target
    logit is x_tgt / tau when the target is in U. The shard's partials merge like
    ``merge``. ``logits_rows`` is the shard's local logits [T, local_size].
    """
    x = np.asarray(logits_rows, dtype=np.float64)
    ids = np.asarray(replay_ids, dtype=np.int64)
    T = ids.shape[0]
    targets = np.asarray(targets, dtype=np.int64)
    mask = np.ones(T, bool) if mask is None else np.asarray(mask).astype(bool)
    n_real = int(min(max(real_vocab - offset, 0), local_size))
    out = dict(target_logit=np.zeros(T), in_range=np.zeros(T, dtype=np.uint8),
               lse=np.zeros(T), logp=np.zeros(T), status=0)
    for t in range(T):
        row = ids[t]
        if np.any((row < -1) | (row >= real_vocab)):
            out["status"] |= ST_REPLAY_ID_INVALID
        if not mask[t]:
            continue
        if targets[t] < 0 or targets[t] >= real_vocab:
            out["status"] |= ST_TARGET_OUT_OF_RANGE
        U = sorted({int(v) for v in row if offset <= v < offset + n_real})
        if not U:
            out["lse"][t] = NEG_INF
            out["logp"][t] = NEG_INF
            continue
        z = x[t, np.array(U) - offset] / temperature
        m = z.max()
        lse = m + np.log(np.exp(z - m).sum())
        out["lse"][t] = lse
        if int(targets[t]) in U:
            tz = z[U.index(int(targets[t]))]
            out["target_logit"][t] = tz
            out["in_range"][t] = 1
            out["logp"][t] = tz - lse
        else:
            out["logp"][t] = NEG_INF
    return out


def logits_forward(logits_rows, targets, temperature: float, offset: int, local_size: int,
                   real_vocab: int, mask=None, world: int = 1) -> dict:
    """Per-shard partials from the shard's precomputed local logits.

    [CUDA provider, "Megatron integration"]: strict LM-head local logits are reused when
    available, with no second projection. [top-p replay, "Summary"]: temperature scaling
    happens once, so the given logits are the unscaled h . W^T + b and z = x / tau here.
    ``logits_rows`` is [T, local_size] (fp32 numbers or bf16 bit patterns); only the first
    clamp(real_vocab - offset, 0, local_size) columns are part of the distribution. The
    outputs are those of ``shard_forward``; with world == 1 a target outside the real range
    also sets the not-found bit, as there is no other shard to hold it.
    """
    x = as_f64(logits_rows)
    T = x.shape[0]
    targets = np.asarray(targets, dtype=np.int64)
    mask = np.ones(T, dtype=bool) if mask is None else np.asarray(mask).astype(bool)
    n_real = int(min(max(real_vocab - offset, 0), local_size))
    out = dict(target_logit=np.zeros(T), in_range=np.zeros(T, dtype=np.uint8),
               lse=np.zeros(T), entropy=np.zeros(T), logp=np.zeros(T), status=0)
    rows = np.nonzero(mask)[0]
    if rows.size == 0:
        return out
    if np.any((targets[rows] < 0) | (targets[rows] >= real_vocab)):
        out["status"] |= ST_TARGET_OUT_OF_RANGE
    z = x[rows][:, :n_real] / temperature
    lse, ent = softmax_stats(z)
    loc = targets[rows] - offset
    hit = (loc >= 0) & (loc < n_real) & (targets[rows] < real_vocab)
    t = np.zeros(rows.size)
    t[hit] = z[np.nonzero(hit)[0], loc[hit]]
    out["target_logit"][rows] = t
    out["in_range"][rows] = hit.astype(np.uint8)
    out["lse"][rows] = lse
    out["entropy"][rows] = ent
    out["logp"][rows] = np.where(hit, t - lse, NEG_INF)
    if world == 1 and np.any(~hit):
        out["status"] |= ST_TARGET_NOT_FOUND
    return out


def keep_mask_replay(logits_rows, keep_mask, targets, temperature: float, offset: int,
                     local_size: int, real_vocab: int, mask=None) -> dict:
    """Dense keep-mask replay scoring of one shard.

    [top-p replay, "Changes" table, VIME masked replay behavior]: the local logits are reused
    with a keep mask and excluded entries are -inf, so per row U = the kept local columns
    among the shard's real ones and lse_N = log sum_{v in U} exp(x_v / tau); the target logit
    is x_tgt / tau when the target is kept. [top-p replay, "Validation"]: this dense form and
    the compact replay of the same nucleus give the same results. ``keep_mask`` is
    [T, local_size] with nonzero = kept.
    """
    x = as_f64(logits_rows)
    km = np.asarray(keep_mask)
    T = x.shape[0]
    targets = np.asarray(targets, dtype=np.int64)
    mask = np.ones(T, bool) if mask is None else np.asarray(mask).astype(bool)
    n_real = int(min(max(real_vocab - offset, 0), local_size))
    out = dict(target_logit=np.zeros(T), in_range=np.zeros(T, dtype=np.uint8),
               lse=np.zeros(T), logp=np.zeros(T), status=0)
    for t in range(T):
        if not mask[t]:
            continue
        if targets[t] < 0 or targets[t] >= real_vocab:
            out["status"] |= ST_TARGET_OUT_OF_RANGE
        cols = np.nonzero(km[t, :n_real])[0]
        if cols.size == 0:
            out["lse"][t] = NEG_INF
            out["logp"][t] = NEG_INF
            continue
        z = x[t, cols] / temperature
        m = z.max()
        lse = m + np.log(np.exp(z - m).sum())
        out["lse"][t] = lse
        loc = int(targets[t]) - offset
        if 0 <= loc < n_real and km[t, loc] and targets[t] < real_vocab:
            tz = x[t, loc] / temperature
            out["target_logit"][t] = tz
            out["in_range"][t] = 1
            out["logp"][t] = tz - lse
        else:
            out["logp"][t] = NEG_INF
    return out
