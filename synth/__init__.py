"""Seeded synthetic inputs for the fused linear log-prob operator.

This module draws inputs only. It holds none of the operator's arithmetic (no logits, no
log-sum-exp, no gradients): the HIP path and the CPU oracle both consume what it returns,
and neither is imported here. The one exception by design is the rollout-side top-p
*selection* rule used to build replay candidate lists (``topp_case``): the scorer never
selects, it only scores the ids it is given.

Shapes follow the workloads the pages describe (a Qwen3-8B language-model head: hidden size
4096, vocabulary 151669 real / 151936 padded; at most 4096 tokens per GPU; responses up to
7168 tokens; temperature 0.7 and top-p 0.95 on the compact top-p replay page). Seeds derive
from 1234, the seed the pages' ablation runs use.

bf16 tensors are returned as ``numpy.uint16`` bit patterns (round-to-nearest-even from
float32 samples); ``bf16_bits`` does that rounding.
"""
from __future__ import annotations

import numpy as np

SEED = 1234

# Qwen3-8B-shaped LM head.
H_FULL = 4096
V_REAL_FULL = 151669
V_PAD_FULL = 151936
TP_SHARDS = 4
V_SHARD = V_PAD_FULL // TP_SHARDS  # 37984

# Stream ids inside one config (spawn keys); W is shared by the full-size configs.
_S_H, _S_W, _S_T, _S_U, _S_MASK, _S_DLOGP, _S_LEN, _S_LOGITS, _S_SPIKE, _S_IDS = range(10)


def rng(config_id: int, stream: int) -> np.random.Generator:
    """Independent, platform-stable PCG64 stream for (config, stream)."""
    return np.random.default_rng(np.random.SeedSequence(entropy=SEED, spawn_key=(config_id, stream)))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    # Process in slabs to bound temporaries for the 622M-element weight.
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    step = 1 << 26
    for s in range(0, flat_u.size, step):
        v = flat_u[s:s + step]
        r = ((v >> 16) & 1) + np.uint32(0x7FFF)
        flat_o[s:s + step] = ((v + r) >> 16).astype(np.uint16)
    return out


def normal_bf16(g: np.random.Generator, shape, std: float) -> np.ndarray:
    """N(0, std^2) samples rounded to bf16 (std is the standard deviation)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 26
    for s in range(0, n, step):
        k = min(step, n - s)
        x = g.standard_normal(k, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:s + k] = bf16_bits(x)
    return out.reshape(shape)


def full_weight() -> np.ndarray:
    """W[151936, 4096] bf16 bits ~ N(0, 0.02^2); padded rows are random too."""
    return normal_bf16(rng(2, _S_W), (V_PAD_FULL, H_FULL), 0.02)


def config1(seed_offset: int = 0) -> dict:
    """Tiny forward: T=64, H=256, V_real=1000 padded to 1024, tau=1, zero bias."""
    cid = 1 + 100 * seed_offset
    T, H, Vr, Vp = 64, 256, 1000, 1024
    return dict(
        T=T, H=H, real_vocab=Vr, padded_vocab=Vp, temperature=1.0,
        hidden=normal_bf16(rng(cid, _S_H), (T, H), 1.0),
        weight=normal_bf16(rng(cid, _S_W), (Vp, H), 0.02),
        bias=np.zeros(Vp, dtype=np.uint16),
        targets=rng(cid, _S_T).integers(0, Vr, size=T, dtype=np.int64),
        mask=np.ones(T, dtype=np.uint8),
    )


def small_case(T: int, H: int, real_vocab: int, padded_vocab: int, temperature: float,
               case_id: int, mask_frac: float = 0.0, with_bias: bool = False,
               w_std: float = 0.02) -> dict:
    """Seeded case of arbitrary (small) shape; used to span tiles and ragged tails."""
    cid = 1000 + case_id
    mask = np.ones(T, dtype=np.uint8)
    if mask_frac > 0:
        mask = (rng(cid, _S_MASK).random(T) >= mask_frac).astype(np.uint8)
    bias = normal_bf16(rng(cid, _S_U), (padded_vocab,), 0.5) if with_bias else None
    return dict(
        T=T, H=H, real_vocab=real_vocab, padded_vocab=padded_vocab, temperature=temperature,
        hidden=normal_bf16(rng(cid, _S_H), (T, H), 1.0),
        weight=normal_bf16(rng(cid, _S_W), (padded_vocab, H), w_std),
        bias=bias,
        targets=rng(cid, _S_T).integers(0, real_vocab, size=T, dtype=np.int64),
        mask=mask,
    )


def config2_hidden() -> np.ndarray:
    """h[4096, 4096] bf16 bits ~ N(0, 1)."""
    return normal_bf16(rng(2, _S_H), (4096, H_FULL), 1.0)


def config2_uniforms() -> np.ndarray:
    """One U(0,1) per row, for inverse-CDF target sampling from the softmax of the logits."""
    return rng(2, _S_U).random(4096)


def inverse_cdf(probs: np.ndarray, u: float) -> int:
    """First index whose ascending-id cumulative sum reaches u (clamped to the last index)."""
    c = np.cumsum(probs)
    i = int(np.searchsorted(c, u * c[-1], side="left"))
    return min(i, probs.size - 1)


def config2_base() -> dict:
    """Qwen3-8B-shaped forward: T=4096, tau=0.7, no bias. Targets are added by the caller
    (sampled from the softmax of the oracle logits; stored once under tests/golden)."""
    return dict(T=4096, H=H_FULL, real_vocab=V_REAL_FULL, padded_vocab=V_PAD_FULL,
                temperature=0.7, hidden=config2_hidden(), weight=None, bias=None,
                mask=np.ones(4096, dtype=np.uint8))


def shard_ranges(n_shards: int = TP_SHARDS, padded: int = V_PAD_FULL):
    """Contiguous vocab ranges (offset, local_size) of an even TP split of the padded vocab."""
    loc = padded // n_shards
    return [(r * loc, loc) for r in range(n_shards)]


def config4_layout(seed_offset: int = 0) -> dict:
    """Packed variable-length layout: 16 sequences, lengths U{256..7168}, the first
    floor(f*len) rows of each masked with f ~ U[0.2, 0.4]."""
    cid = 4 + 100 * seed_offset
    g = rng(cid, _S_LEN)
    lens = g.integers(256, 7168, size=16, endpoint=True)
    fr = g.uniform(0.2, 0.4, size=16)
    cu = np.zeros(17, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    mask = np.ones(int(cu[-1]), dtype=np.uint8)
    for s in range(16):
        mask[cu[s]:cu[s] + int(np.floor(fr[s] * lens[s]))] = 0
    return dict(lens=lens, cu_seqlens=cu, mask=mask, T=int(cu[-1]))


def config4_case(seed_offset: int = 0) -> dict:
    """Config-4 data except W (shared full weight): hidden, uniform targets, dlogp."""
    cid = 4 + 100 * seed_offset
    lay = config4_layout(seed_offset)
    T = lay["T"]
    dlogp = rng(cid, _S_DLOGP).standard_normal(T).astype(np.float32)
    dlogp[lay["mask"] == 0] = 0.0
    return dict(lay, H=H_FULL, real_vocab=V_REAL_FULL, padded_vocab=V_PAD_FULL,
                temperature=0.7, hidden=normal_bf16(rng(cid, _S_H), (T, H_FULL), 1.0),
                targets=rng(cid, _S_T).integers(0, V_REAL_FULL, size=T, dtype=np.int64),
                dlogp=dlogp)


def repack_order(n_seqs: int = 16, seed_offset: int = 0) -> np.ndarray:
    """Seeded permutation of sequences for the batch-packing invariance check."""
    return rng(4 + 100 * seed_offset, _S_IDS).permutation(n_seqs)


def _nucleus_rows(x_blk: np.ndarray, temperature: float, top_p: float,
                  real_vocab: int) -> list:
    """Rollout-side top-p selection for a block of rows: probabilities of x/tau in fp64,
    sorted descending (ties by ascending id); each row keeps the shortest prefix whose mass
    reaches top_p (at least one id)."""
    z = x_blk[:, :real_vocab].astype(np.float64) / temperature
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    out = []
    for row in p:
        top = np.argpartition(-row, 64)[:64]
        order = top[np.lexsort((top, -row[top]))]
        c = np.cumsum(row[order])
        if c[-1] < top_p:  # nucleus wider than 64: fall back to the full sort
            order = np.lexsort((np.arange(real_vocab), -row))
            c = np.cumsum(row[order])
        k = int(np.searchsorted(c, top_p, side="left")) + 1
        out.append(order[:max(1, min(k, order.size))])
    return out


def topp_case(T: int = 4096, V_pad: int = V_PAD_FULL, V_real: int = V_REAL_FULL,
              K: int = 64, temperature: float = 0.7, top_p: float = 0.95,
              dup_prob: float = 0.1, case_id: int = 5, big_nucleus: int = 0) -> dict:
    """Compact top-p replay case: fp32 logits ~ N(0, 2^2) with 1..10 spikes of height
    18 + U(0,3) per row (padded columns at -1e30), the native nucleus of each row, shuffled,
    with ~10% duplicates, padded with -1 to K slots, and a target drawn inside the nucleus.
    With ``big_nucleus`` > 0 each row's list instead holds that many nucleus-ordered ids plus
    duplicates up to K (capacity case)."""
    g = rng(case_id, _S_LOGITS)
    logits = np.empty((T, V_pad), dtype=np.float32)
    for r0 in range(0, T, 256):
        r1 = min(T, r0 + 256)
        logits[r0:r1] = g.standard_normal((r1 - r0, V_pad), dtype=np.float32) * np.float32(2.0)
    logits[:, V_real:] = np.float32(-1e30)
    gs = rng(case_id, _S_SPIKE)
    for r in range(T):
        k = int(gs.integers(1, 10, endpoint=True))
        ids = gs.choice(V_real, size=k, replace=False)
        logits[r, ids] = (18.0 + 3.0 * gs.random(k)).astype(np.float32)
    gi = rng(case_id, _S_IDS)
    gu = rng(case_id, _S_U)
    replay = np.full((T, K), -1, dtype=np.int64)
    targets = np.empty(T, dtype=np.int64)
    nuclei = []
    for r0 in range(0, T, 256):
        blk = logits[r0:min(T, r0 + 256)]
        if big_nucleus:
            nuclei += [np.argsort(-row[:V_real], kind="stable")[:big_nucleus] for row in blk]
        else:
            nuclei += _nucleus_rows(blk, temperature, top_p, V_real)
    for r in range(T):
        nuc = nuclei[r]
        lst = list(nuc)
        for i in nuc:
            if len(lst) < K and gi.random() < dup_prob:
                lst.append(i)
        if big_nucleus:
            while len(lst) < K:
                lst.append(nuc[int(gi.integers(0, len(nuc)))])
        lst = np.array(lst[:K], dtype=np.int64)
        gi.shuffle(lst)
        replay[r, :lst.size] = lst
        # Target ~ nucleus-restricted softmax (inverse CDF in ascending-id order).
        ids_sorted = np.sort(nuc)
        zz = logits[r, ids_sorted].astype(np.float64) / temperature
        w = np.exp(zz - zz.max())
        targets[r] = ids_sorted[inverse_cdf(w, gu.random())]
    return dict(T=T, padded_vocab=V_pad, real_vocab=V_real, temperature=temperature,
                top_p=top_p, logits=logits, replay_ids=replay, targets=targets,
                mask=np.ones(T, dtype=np.uint8))
