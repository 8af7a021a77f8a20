"""Pins of the logits-input forward and the dense keep-mask replay in the oracle.

Each check ties an oracle function to something other than its own formula: torch library
routines (log_softmax, logsumexp, Categorical entropy) in fp64, closed forms, invariants the
definition fixes (exclusion of padded columns, temperature applied once, shard merge identity,
empty shards), and planted mistakes that each of these checks must catch.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _logits_case(T=24, V=90, Vp=96, seed=3):
    g = synth.rng(seed, 40)
    x = g.standard_normal((T, Vp)) * 2.0
    tg = g.integers(0, V, size=T)
    mask = g.random(T) > 0.25
    return x, tg, mask, V, Vp


def pin_logits_library(fn, x, tg, mask, V, tau):
    out = fn(x, tg, tau, 0, x.shape[1], V, mask)
    z = torch.from_numpy(x[:, :V] / tau)
    lp = torch.log_softmax(z, -1).gather(1, torch.from_numpy(tg)[:, None])[:, 0].numpy()
    ent = torch.distributions.Categorical(logits=z).entropy().numpy()
    lse = torch.logsumexp(z, -1).numpy()
    m = mask
    np.testing.assert_allclose(out["logp"][m], lp[m], atol=1e-12)
    np.testing.assert_allclose(out["entropy"][m], ent[m], atol=1e-12)
    np.testing.assert_allclose(out["lse"][m], lse[m], rtol=1e-14)
    assert np.all(out["logp"][~m] == 0) and np.all(out["lse"][~m] == 0)
    assert np.all(out["entropy"][~m] == 0) and np.all(out["in_range"][~m] == 0)


def pin_logits_temperature_once(fn, x, tg, V):
    a = fn(x, tg, 2.0, 0, x.shape[1], V)
    b = fn(x / 2.0, tg, 1.0, 0, x.shape[1], V)       # exact: division by a power of two
    for k in ("lse", "logp", "entropy", "target_logit"):
        np.testing.assert_array_equal(a[k], b[k])


def pin_logits_merge(fn, x, tg, V, cuts):
    full = fn(x, tg, 0.7, 0, x.shape[1], V)
    parts = [fn(x[:, lo:hi], tg, 0.7, lo, hi - lo, V, world=len(cuts) - 1)
             for lo, hi in zip(cuts[:-1], cuts[1:])]
    mg = oracle.merge(parts)
    np.testing.assert_allclose(mg["lse"], full["lse"], rtol=1e-14)
    np.testing.assert_allclose(mg["logp"], full["logp"], atol=1e-13)
    np.testing.assert_allclose(mg["entropy"], full["entropy"], atol=1e-12)


def test_logits_forward_vs_torch_library():
    x, tg, mask, V, _ = _logits_case()
    pin_logits_library(oracle.logits_forward, x, tg, mask, V, 0.7)


def test_logits_forward_bf16_bits_are_exact_values():
    x, tg, mask, V, _ = _logits_case(seed=4)
    bits = synth.bf16_bits(x.astype(np.float32))
    a = oracle.logits_forward(bits, tg, 0.7, 0, x.shape[1], V, mask)
    b = oracle.logits_forward(oracle.bf16_to_f64(bits), tg, 0.7, 0, x.shape[1], V, mask)
    for k in ("lse", "logp", "entropy"):
        np.testing.assert_array_equal(a[k], b[k])


def test_logits_forward_closed_forms():
    T, V = 4, 37
    x = np.full((T, 40), 3.0)
    out = oracle.logits_forward(x, np.arange(T), 0.5, 0, 40, V)
    np.testing.assert_allclose(out["lse"], np.log(V) + 6.0, rtol=1e-15)
    np.testing.assert_allclose(out["entropy"], np.log(V), rtol=1e-14)
    np.testing.assert_allclose(out["logp"], -np.log(V), rtol=1e-14)
    x[:, 5] = 1e3                                           # one dominant logit
    out = oracle.logits_forward(x, np.full(T, 5), 1.0, 0, 40, V)
    assert np.all(np.abs(out["logp"]) < 1e-12) and np.all(np.abs(out["entropy"]) < 1e-12)


def test_logits_forward_excludes_padded_columns():
    x, tg, mask, V, Vp = _logits_case(seed=5)
    a = oracle.logits_forward(x, tg, 0.7, 0, Vp, V, mask)
    y = x.copy()
    y[:, V:] = 1e30
    b = oracle.logits_forward(y, tg, 0.7, 0, Vp, V, mask)
    for k in ("lse", "logp", "entropy"):
        np.testing.assert_array_equal(a[k], b[k])


def test_logits_forward_temperature_once_and_merge():
    x, tg, _, V, _ = _logits_case(seed=6)
    pin_logits_temperature_once(oracle.logits_forward, x, tg, V)
    pin_logits_merge(oracle.logits_forward, x, tg, V, [0, 30, 60, 96])


def test_logits_forward_matches_projection_oracle():
    """Given the exact logits h W^T + b, the logits-input path is the fused path."""
    case = synth.small_case(T=16, H=32, real_vocab=60, padded_vocab=64, temperature=0.7,
                            case_id=41, with_bias=True, w_std=0.3)
    h, W, b = (oracle.as_f64(case[k]) for k in ("hidden", "weight", "bias"))
    x = h @ W.T + b[None, :]
    a = oracle.logits_forward(x, case["targets"], 0.7, 0, 64, 60, case["mask"])
    f = oracle.forward(case["hidden"], case["weight"], case["bias"], 0.7, case["targets"],
                       case["mask"], 60)
    for k in ("lse", "logp", "entropy"):
        np.testing.assert_allclose(a[k], f[k], atol=1e-12)


def test_logits_forward_empty_shard_and_status():
    x, tg, _, V, _ = _logits_case(T=5, seed=7)
    out = oracle.logits_forward(x[:, :0], tg, 0.7, V, 0, V, world=2)
    assert np.all(out["lse"] == -np.inf) and np.all(out["logp"] == -np.inf)
    assert np.all(out["entropy"] == 0) and np.all(out["target_logit"] == 0)
    assert not np.any(np.isnan(out["lse"]))
    tg2 = tg.copy()
    tg2[0] = V                                              # a padded id: out of range
    out = oracle.logits_forward(x, tg2, 0.7, 0, x.shape[1], V)
    assert out["status"] & oracle.ST_TARGET_OUT_OF_RANGE
    assert out["status"] & oracle.ST_TARGET_NOT_FOUND
    assert out["logp"][0] == -np.inf and out["in_range"][0] == 0


# ------------------------------------------------------------------ dense keep-mask replay

def _nucleus_case(T=20, V=50, Vp=64, seed=21):
    g = synth.rng(seed, 41)
    x = g.standard_normal((T, Vp)) * 2.0
    ids = np.full((T, 64), -1, dtype=np.int64)
    keep = np.zeros((T, Vp), dtype=np.uint8)
    tg = np.zeros(T, dtype=np.int64)
    for t in range(T):
        k = int(g.integers(1, 12))
        u = g.choice(V, size=k, replace=False)
        lst = np.concatenate([u, u[: int(g.integers(0, k + 1))]])   # duplicates
        g.shuffle(lst)
        ids[t, :lst.size] = lst
        keep[t, u] = 1
        tg[t] = u[0] if g.random() < 0.8 else int(g.integers(0, V))
    return x, ids, keep, tg, V, Vp


def test_keep_mask_replay_vs_torch_library():
    x, _, keep, tg, V, Vp = _nucleus_case()
    out = oracle.keep_mask_replay(x, keep, tg, 0.7, 0, Vp, V)
    z = torch.from_numpy(x / 0.7).masked_fill(torch.from_numpy(keep == 0), -torch.inf)
    z[:, V:] = -torch.inf
    lse = torch.logsumexp(z, -1).numpy()
    lp = torch.log_softmax(z, -1).gather(1, torch.from_numpy(tg)[:, None])[:, 0].numpy()
    np.testing.assert_allclose(out["lse"], lse, rtol=1e-14)
    np.testing.assert_allclose(out["logp"], lp, atol=1e-12)   # -inf where the target is dropped


def test_keep_mask_replay_equals_compact_replay():
    """[top-p replay, "Validation"]: dense keep mask and compact ids of one nucleus agree."""
    x, ids, keep, tg, V, Vp = _nucleus_case(seed=22)
    for lo, hi in ((0, 64), (0, 20), (20, 40), (40, 64), (50, 64)):
        a = oracle.keep_mask_replay(x[:, lo:hi], keep[:, lo:hi], tg, 0.7, lo, hi - lo, V)
        b = oracle.top_p_replay(x[:, lo:hi], ids, tg, 0.7, lo, hi - lo, V)
        for k in ("lse", "logp", "target_logit", "in_range"):
            np.testing.assert_array_equal(a[k], b[k])


def test_keep_mask_replay_special_cases():
    x, _, keep, tg, V, Vp = _nucleus_case(T=4, seed=23)
    one = np.zeros_like(keep)
    one[:, 7] = 1
    out = oracle.keep_mask_replay(x, one, np.full(4, 7), 0.7, 0, Vp, V)
    np.testing.assert_array_equal(out["logp"], np.zeros(4))      # a single kept id: log 1
    np.testing.assert_allclose(out["lse"], x[:, 7] / 0.7, rtol=1e-15)
    allk = np.ones_like(keep)                                     # everything kept = full vocab
    out = oracle.keep_mask_replay(x, allk, tg, 0.7, 0, Vp, V)
    full = oracle.logits_forward(x, tg, 0.7, 0, Vp, V)
    np.testing.assert_allclose(out["lse"], full["lse"], rtol=1e-14)
    out = oracle.keep_mask_replay(x, np.zeros_like(keep), tg, 0.7, 0, Vp, V)
    assert np.all(out["lse"] == -np.inf) and np.all(out["logp"] == -np.inf)


# --------------------------------------------------------------------- planted mistakes

def _lf_tau_twice(x, tg, tau, *a, **k):
    return oracle.logits_forward(np.asarray(oracle.as_f64(x)) / tau, tg, tau, *a, **k)


def _lf_padded_included(x, tg, tau, offset, local, real, *a, **k):
    return oracle.logits_forward(x, tg, tau, offset, local, real + 3, *a, **k)


def _lf_entropy_sign(*a, **k):
    out = oracle.logits_forward(*a, **k)
    out["entropy"] = -out["entropy"]
    return out


@pytest.mark.parametrize("name,fn", [
    ("tau applied twice", _lf_tau_twice),
    ("padded columns included", _lf_padded_included),
    ("entropy sign", _lf_entropy_sign),
])
def test_logits_planted_mistakes_are_caught(name, fn):
    x, tg, mask, V, _ = _logits_case(seed=8)
    caught = 0
    for pin in (lambda: pin_logits_library(fn, x, tg, mask, V, 0.7),
                lambda: pin_logits_temperature_once(fn, x, tg, V),
                lambda: pin_logits_merge(fn, x, tg, V, [0, 30, 60, 96])):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, name
