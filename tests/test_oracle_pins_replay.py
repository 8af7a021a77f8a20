"""Pins of the replay scorers' range filter in the oracle: ids (top-p) and kept columns (dense
keep mask) that fall in a shard's padded columns, [real_vocab, offset + local_size), are not
part of the nucleus.

[top-p replay, "Changes" table]: the scorer validates its replay inputs before it sorts and
deduplicates the ids, and the padded vocabulary is not part of the distribution ([CUDA
provider, "Megatron integration"]: real and padded vocabulary sizes). Each pin gives the padded
columns a logit of +1e4, so that an id let through would dominate the row, and checks the row
two ways: bitwise against the same row with those ids left out, and against torch.logsumexp /
log_softmax in fp64 over the row's distinct real ids only (a masked dense row, another route
than the oracle's sort and gather). Planted mistakes that widen the range to the shard's local
size must fail a pin.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

V, VP, T = 50, 64, 16
BIG = 1e4


def _case(seed=31):
    """Rows of <= 40 listed real ids (shuffled, with duplicates and -1 slots), each row also
    listing 1..6 padded ids; logits ~ N(0, 2^2) with +1e4 in the padded columns."""
    g = synth.rng(seed, 5)
    x = g.standard_normal((T, VP)) * 2.0
    x[:, V:] = BIG
    ids_real = np.full((T, 64), -1, dtype=np.int64)
    ids_pad = np.full((T, 64), -1, dtype=np.int64)
    tg = np.empty(T, dtype=np.int64)
    for t in range(T):
        k = int(g.integers(1, 30))
        u = g.choice(V, size=k, replace=False)
        dup = u[: int(g.integers(0, min(k, 10) + 1))]
        pad = g.choice(np.arange(V, VP), size=int(g.integers(1, 7)), replace=False)
        real = np.concatenate([u, dup])
        g.shuffle(real)
        ids_real[t, :real.size] = real
        both = np.concatenate([real, pad])
        g.shuffle(both)
        ids_pad[t, :both.size] = both
        # Target: mostly a listed real id; some rows a padded id (never in the nucleus).
        r = g.random()
        tg[t] = u[0] if r < 0.7 else (pad[0] if r < 0.85 else int(g.integers(0, V)))
    return x, ids_real, ids_pad, tg


def _torch_reference(x, ids_real, tg, lo, hi, tau):
    """lse and logp over the distinct listed real ids in [lo, min(hi, V)) by masked
    torch.logsumexp / log_softmax (fp64); -inf where the row has no such id or the target is
    not one of them."""
    z = torch.from_numpy(x / tau).clone()
    keep = torch.zeros((T, VP), dtype=torch.bool)
    for t in range(T):
        for v in ids_real[t]:
            if lo <= v < min(hi, V):
                keep[t, v] = True
    z = z.masked_fill(~keep, -torch.inf)
    lse = torch.logsumexp(z, -1)
    ls = torch.log_softmax(z, -1)
    lp = torch.full((T,), -torch.inf, dtype=torch.float64)
    for t in range(T):
        if keep[t].any() and 0 <= tg[t] < VP and keep[t, tg[t]]:
            lp[t] = ls[t, tg[t]]
    return lse.numpy(), lp.numpy(), keep.numpy()


SHARDS = ((0, 64), (32, 64), (48, 64), (0, 32))


def pin_topp_padded_ids_excluded(fn):
    x, ids_real, ids_pad, tg = _case()
    for lo, hi in SHARDS:
        a = fn(x[:, lo:hi], ids_pad, tg, 0.7, lo, hi - lo, V)
        b = fn(x[:, lo:hi], ids_real, tg, 0.7, lo, hi - lo, V)
        for k in ("lse", "logp", "target_logit", "in_range"):
            np.testing.assert_array_equal(a[k], b[k], err_msg=f"{k} shard [{lo},{hi})")
        lse, lp, _ = _torch_reference(x, ids_real, tg, lo, hi, 0.7)
        np.testing.assert_allclose(a["lse"], lse, rtol=1e-14, atol=0)
        fin = np.isfinite(lp)
        np.testing.assert_array_equal(np.isneginf(a["logp"]), ~fin)
        np.testing.assert_allclose(a["logp"][fin], lp[fin], atol=1e-12)
        assert np.all(a["logp"] <= 0)
        assert np.all(a["target_logit"][~fin] == 0) and np.all(a["in_range"][~fin] == 0)


def pin_keep_padded_columns_excluded(fn):
    x, ids_real, ids_pad, tg = _case(seed=32)
    keep_real = np.zeros((T, VP), dtype=np.uint8)
    keep_pad = np.zeros((T, VP), dtype=np.uint8)
    for t in range(T):
        keep_real[t, ids_real[t][ids_real[t] >= 0]] = 1
        keep_pad[t, ids_pad[t][ids_pad[t] >= 0]] = 1
    for lo, hi in SHARDS:
        a = fn(x[:, lo:hi], keep_pad[:, lo:hi], tg, 0.7, lo, hi - lo, V)
        b = fn(x[:, lo:hi], keep_real[:, lo:hi], tg, 0.7, lo, hi - lo, V)
        for k in ("lse", "logp", "target_logit", "in_range"):
            np.testing.assert_array_equal(a[k], b[k], err_msg=f"{k} shard [{lo},{hi})")
        lse, lp, _ = _torch_reference(x, ids_real, tg, lo, hi, 0.7)
        np.testing.assert_allclose(a["lse"], lse, rtol=1e-14, atol=0)
        fin = np.isfinite(lp)
        np.testing.assert_array_equal(np.isneginf(a["logp"]), ~fin)
        np.testing.assert_allclose(a["logp"][fin], lp[fin], atol=1e-12)


def test_topp_padded_ids_excluded():
    pin_topp_padded_ids_excluded(oracle.top_p_replay)


def test_topp_padded_ids_set_status_bit():
    x, _, ids_pad, tg = _case()
    out = oracle.top_p_replay(x, ids_pad, tg, 0.7, 0, VP, V)
    assert out["status"] & oracle.ST_REPLAY_ID_INVALID
    # A padded target is out of range for the real vocabulary.
    assert (out["status"] & oracle.ST_TARGET_OUT_OF_RANGE) == (
        oracle.ST_TARGET_OUT_OF_RANGE if np.any(tg >= V) else 0)


def test_keep_mask_padded_columns_excluded():
    pin_keep_padded_columns_excluded(oracle.keep_mask_replay)


def test_shard_with_only_padded_ids_is_empty():
    """A shard whose listed ids are all padding has no candidates: -inf / 0 / 0."""
    x, _, ids_pad, tg = _case(seed=33)
    only_pad = np.where(ids_pad >= V, ids_pad, -1)
    out = oracle.top_p_replay(x[:, V:], only_pad, tg, 0.7, V, VP - V, V)
    assert np.all(out["lse"] == -np.inf) and np.all(out["logp"] == -np.inf)
    assert np.all(out["target_logit"] == 0) and np.all(out["in_range"] == 0)


# --------------------------------------------------------------------- planted mistakes

def _topp_range_local_size(x, ids, tg, tau, offset, local, real, mask=None):
    # The range filter bounded by offset + local_size instead of the shard's real columns.
    return oracle.top_p_replay(x, ids, tg, tau, offset, local, offset + local, mask)


def _topp_tau_twice(x, ids, tg, tau, *a, **k):
    return oracle.top_p_replay(np.asarray(x) / tau, ids, tg, tau, *a, **k)


def _keep_range_local_size(x, km, tg, tau, offset, local, real, mask=None):
    return oracle.keep_mask_replay(x, km, tg, tau, offset, local, offset + local, mask)


@pytest.mark.parametrize("name,fn,pin", [
    ("top-p range bounded by local_size", _topp_range_local_size, pin_topp_padded_ids_excluded),
    ("top-p tau applied twice", _topp_tau_twice, pin_topp_padded_ids_excluded),
    ("keep-mask range bounded by local_size", _keep_range_local_size,
     pin_keep_padded_columns_excluded),
])
def test_replay_planted_mistakes_are_caught(name, fn, pin):
    with pytest.raises(AssertionError):
        pin(fn)
