"""Pins for the fp64 oracle, independent of its own formulas.

Each check reaches the expected value by another route: mpmath brute force on exactly
summed logits, torch library routines (log_softmax, Categorical entropy, autograd), closed
forms, central finite differences and invariants. ``test_planted_mistakes_are_caught``
plants plausible mistakes in copies of the oracle and checks that some pin fails.
"""
import math
import types

import numpy as np
import pytest
import torch

import oracle
import synth

mpmath = pytest.importorskip("mpmath")


def _f64(bits):
    return oracle.bf16_to_f64(bits)


# ----------------------------------------------------------------------------- pin bodies
# Each pin takes an oracle-like namespace so that planted mistakes can be run through it.

def pin_mpmath(orc, case, rows):
    """lse/logp/entropy of a few rows vs 50-digit mpmath on exactly summed logits."""
    h, W = _f64(case["hidden"]), _f64(case["weight"])
    b = _f64(case["bias"]) if case["bias"] is not None else None
    Vr, tau = case["real_vocab"], case["temperature"]
    out = orc.forward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                      case["mask"], Vr)
    mpmath.mp.dps = 50
    for r in rows:
        # bf16 x bf16 products are exact in fp64; fsum gives the correctly rounded sum.
        zs = []
        for v in range(Vr):
            acc = math.fsum(list(h[r] * W[v]) + ([b[v]] if b is not None else []))
            zs.append(mpmath.mpf(acc) / mpmath.mpf(tau))
        lse = mpmath.log(mpmath.fsum([mpmath.exp(z) for z in zs]))
        ps = [mpmath.exp(z - lse) for z in zs]
        ent = -mpmath.fsum([p * mpmath.log(p) for p in ps if p > 0])
        tgt = int(case["targets"][r])
        assert abs(float(lse) - out["lse"][r]) <= 1e-11 * max(1.0, abs(float(lse)))
        assert abs(float(zs[tgt] - lse) - out["logp"][r]) <= 1e-11
        assert abs(float(ent) - out["entropy"][r]) <= 1e-11


def pin_torch_library(orc, case):
    """vs torch.log_softmax / Categorical.entropy in fp64 on the same exact inputs."""
    h = torch.from_numpy(_f64(case["hidden"]))
    Vr = case["real_vocab"]
    W = torch.from_numpy(_f64(case["weight"][:Vr]))
    z = h @ W.T
    if case["bias"] is not None:
        z = z + torch.from_numpy(_f64(case["bias"][:Vr]))
    z = z / case["temperature"]
    ls = torch.log_softmax(z, dim=-1)
    tg = torch.from_numpy(case["targets"])
    logp = ls.gather(1, tg[:, None])[:, 0].numpy()
    ent = torch.distributions.Categorical(logits=z).entropy().numpy()
    lse = torch.logsumexp(z, dim=-1).numpy()
    out = orc.forward(case["hidden"], case["weight"], case["bias"], case["temperature"],
                      case["targets"], case["mask"], Vr)
    m = case["mask"].astype(bool)
    np.testing.assert_allclose(out["logp"][m], logp[m], rtol=0, atol=1e-11)
    np.testing.assert_allclose(out["entropy"][m], ent[m], rtol=0, atol=1e-11)
    np.testing.assert_allclose(out["lse"][m], lse[m], rtol=1e-13, atol=1e-11)
    assert np.all(out["logp"][~m] == 0) and np.all(out["entropy"][~m] == 0)
    assert np.all(out["lse"][~m] == 0)


def pin_temperature_once(orc, case):
    """tau = 2 with W equals tau = 1 with W/2 (exact in bf16): tau enters exactly once."""
    W2 = (_f64(case["weight"]) / 2.0)
    a = orc.forward(case["hidden"], case["weight"], None, 2.0, case["targets"], None,
                    case["real_vocab"])
    b = orc.forward(case["hidden"], W2, None, 1.0, case["targets"], None, case["real_vocab"])
    for k in ("logp", "lse", "entropy"):
        np.testing.assert_allclose(a[k], b[k], rtol=1e-14, atol=1e-14)


def pin_merge_identity(orc, case, cuts):
    """Merged shard partials equal the unsharded result, for any contiguous partition."""
    Vp, Vr, tau = case["padded_vocab"], case["real_vocab"], case["temperature"]
    full = orc.forward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                       case["mask"], Vr)
    parts = []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        parts.append(orc.shard_forward(case["hidden"], case["weight"][lo:hi],
                                       None if case["bias"] is None else case["bias"][lo:hi],
                                       tau, case["targets"], case["mask"], lo, hi - lo, Vr))
    mg = orc.merge(parts, case["mask"])
    np.testing.assert_allclose(mg["lse"], full["lse"], rtol=1e-13, atol=1e-12)
    np.testing.assert_allclose(mg["logp"], full["logp"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(mg["entropy"], full["entropy"], rtol=0, atol=1e-12)


def _torch_loss_grads(case, dlogp, dent):
    h = torch.from_numpy(_f64(case["hidden"])).requires_grad_(True)
    Vr, Vp = case["real_vocab"], case["padded_vocab"]
    Wf = torch.from_numpy(_f64(case["weight"])).requires_grad_(True)
    bf = torch.from_numpy(_f64(case["bias"]) if case["bias"] is not None
                          else np.zeros(Vp)).requires_grad_(True)
    z = (h @ Wf[:Vr].T + bf[:Vr]) / case["temperature"]
    ls = torch.log_softmax(z, dim=-1)
    logp = ls.gather(1, torch.from_numpy(case["targets"])[:, None])[:, 0]
    ent = -(ls.exp() * ls).sum(-1)
    m = torch.from_numpy(case["mask"].astype(bool))
    loss = (torch.from_numpy(dlogp) * logp * m).sum()
    if dent is not None:
        loss = loss + (torch.from_numpy(dent) * ent * m).sum()
    loss.backward()
    return h.grad.numpy(), Wf.grad.numpy(), bf.grad.numpy(), logp.detach().numpy(), \
        torch.logsumexp(z, -1).detach().numpy(), ent.detach().numpy()


def pin_backward_autograd(orc, case, with_dent):
    g = synth.rng(77, 1)
    T = case["T"]
    dlogp = g.standard_normal(T)
    dent = g.standard_normal(T) if with_dent else None
    gh, gW, gb, _, lse, ent = _torch_loss_grads(case, dlogp, dent)
    out = orc.backward(case["hidden"], case["weight"], case["bias"], case["temperature"],
                       case["targets"], case["mask"], 0, case["padded_vocab"],
                       case["real_vocab"], lse, dlogp, dent, ent if with_dent else None)
    for a, b in ((out["dhidden"], gh), (out["dweight"], gW), (out["dbias"], gb)):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-12)


# ----------------------------------------------------------------------------- the pins

def test_bf16_conversion_exact():
    x = np.array([1.0, -2.5, 3.140625, 65280.0, 2.0 ** -133, 0.0], dtype=np.float32)
    bits = synth.bf16_bits(x)
    np.testing.assert_array_equal(oracle.bf16_to_f64(bits), x.astype(np.float64))
    # round to nearest even: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> 1
    assert oracle.bf16_to_f64(synth.bf16_bits(np.float32([1 + 2 ** -8])))[0] == 1.0
    assert oracle.bf16_to_f64(synth.bf16_bits(np.float32([1 + 3 * 2 ** -8])))[0] == 1 + 2 ** -6


def test_forward_vs_mpmath_config1():
    pin_mpmath(oracle, synth.config1(), rows=[0, 17, 63])


def test_forward_vs_mpmath_bias_temperature():
    case = synth.small_case(T=8, H=64, real_vocab=97, padded_vocab=128, temperature=0.7,
                            case_id=3, with_bias=True, w_std=0.3)
    pin_mpmath(oracle, case, rows=[0, 5])


def test_forward_vs_torch_library():
    pin_torch_library(oracle, synth.config1())
    pin_torch_library(oracle, synth.small_case(T=40, H=128, real_vocab=300, padded_vocab=320,
                                               temperature=0.7, case_id=4, mask_frac=0.3,
                                               with_bias=True, w_std=0.2))


def test_closed_form_uniform_logits():
    """W = 0, b = 0: softmax is uniform over the real vocabulary."""
    T, H, Vr, Vp = 5, 32, 1000, 1024
    h = synth.normal_bf16(synth.rng(9, 0), (T, H), 1.0)
    W = np.zeros((Vp, H), dtype=np.uint16)
    tg = np.array([0, 1, 500, 998, 999])
    out = oracle.forward(h, W, None, 0.7, tg, None, Vr)
    np.testing.assert_allclose(out["lse"], np.log(Vr), rtol=1e-15)
    np.testing.assert_allclose(out["logp"], -np.log(Vr), rtol=1e-15)
    np.testing.assert_allclose(out["entropy"], np.log(Vr), rtol=1e-14)


def test_closed_form_dominant_logit():
    """One logit 1000 above the rest: logp of it -> 0, entropy -> 0, others -> -1000/tau."""
    T, H, Vr, Vp = 3, 16, 50, 64
    h = np.zeros((T, H)); h[:, 0] = 1.0
    W = np.zeros((Vp, H)); W[7, 0] = 1000.0
    out = oracle.forward(h, W, None, 1.0, np.array([7, 7, 3]), None, Vr)
    assert abs(out["logp"][0]) <= 1e-12 and abs(out["entropy"][0]) <= 1e-12
    np.testing.assert_allclose(out["logp"][2], -1000.0, rtol=1e-12)


def test_invariants_config1():
    case = synth.config1()
    out = oracle.forward(case["hidden"], case["weight"], case["bias"], 1.0, case["targets"],
                         None, case["real_vocab"])
    assert np.all(out["logp"] <= 0)
    assert np.all(out["entropy"] >= 0) and np.all(out["entropy"] <= np.log(1000) + 1e-12)
    z = _f64(case["hidden"]) @ _f64(case["weight"][:1000]).T
    assert np.all(out["lse"] >= z.max(axis=1))
    np.testing.assert_allclose(np.exp(z - out["lse"][:, None]).sum(1), 1.0, atol=1e-12)


def test_padded_columns_excluded():
    """Padded weight rows set to +-1e4 change nothing (bitwise)."""
    case = synth.config1()
    a = oracle.forward(case["hidden"], case["weight"], case["bias"], 1.0, case["targets"],
                       None, 1000)
    W = case["weight"].copy()
    W[1000:] = synth.bf16_bits(np.where(np.arange(W[1000:].size).reshape(W[1000:].shape) % 2,
                                        1e4, -1e4).astype(np.float32))
    b = oracle.forward(case["hidden"], W, case["bias"], 1.0, case["targets"], None, 1000)
    for k in ("logp", "lse", "entropy"):
        np.testing.assert_array_equal(a[k], b[k])


def test_temperature_applied_once():
    pin_temperature_once(oracle, synth.config1())


def test_merge_identity_and_empty_shards():
    case = synth.small_case(T=24, H=64, real_vocab=300, padded_vocab=320, temperature=0.7,
                            case_id=5, mask_frac=0.25, with_bias=True, w_std=0.3)
    pin_merge_identity(oracle, case, [0, 80, 160, 240, 320])   # last shard partly padded
    pin_merge_identity(oracle, case, [0, 1, 150, 150, 299, 320])  # empty + 1-col shards
    pin_merge_identity(oracle, case, [0, 300, 320])             # a shard of padding only


def test_empty_shard_partials():
    case = synth.small_case(T=6, H=32, real_vocab=100, padded_vocab=128, temperature=1.0,
                            case_id=6)
    for lo, n in ((40, 0), (100, 28)):   # zero columns; only padded columns
        p = oracle.shard_forward(case["hidden"], case["weight"][lo:lo + n], None, 1.0,
                                 case["targets"], None, lo, n, 100)
        assert np.all(p["lse"] == -np.inf) and np.all(p["logp"] == -np.inf)
        assert np.all(p["target_logit"] == 0) and np.all(p["in_range"] == 0)
        assert np.all(p["entropy"] == 0)
    # Adding an empty shard anywhere leaves the merge bitwise unchanged.
    ps = [oracle.shard_forward(case["hidden"], case["weight"][lo:hi], None, 1.0,
                               case["targets"], None, lo, hi - lo, 100)
          for lo, hi in ((0, 64), (64, 128))]
    empty = oracle.shard_forward(case["hidden"], case["weight"][:0], None, 1.0,
                                 case["targets"], None, 64, 0, 100)
    a, b = oracle.merge(ps), oracle.merge([ps[0], empty, ps[1]])
    for k in ("logp", "lse", "entropy"):
        np.testing.assert_array_equal(a[k], b[k])


def test_target_not_found_and_out_of_range():
    case = synth.small_case(T=4, H=32, real_vocab=100, padded_vocab=128, temperature=1.0,
                            case_id=7)
    tg = np.array([5, 99, 100, -1])
    out = oracle.forward(case["hidden"], case["weight"], None, 1.0, tg, None, 100)
    assert np.isfinite(out["logp"][:2]).all() and np.all(out["logp"][2:] == -np.inf)
    assert out["status"] & oracle.ST_TARGET_OUT_OF_RANGE
    assert out["status"] & oracle.ST_TARGET_NOT_FOUND


def test_backward_vs_autograd():
    case = synth.small_case(T=24, H=48, real_vocab=90, padded_vocab=96, temperature=0.7,
                            case_id=8, mask_frac=0.3, with_bias=True, w_std=0.3)
    pin_backward_autograd(oracle, case, with_dent=False)
    pin_backward_autograd(oracle, case, with_dent=True)


def test_backward_finite_differences():
    """Central differences of the oracle's own forward at a few coordinates (fp64 inputs)."""
    case = synth.small_case(T=6, H=16, real_vocab=40, padded_vocab=48, temperature=0.7,
                            case_id=9, with_bias=True, w_std=0.5)
    h, W, b = _f64(case["hidden"]), _f64(case["weight"]), _f64(case["bias"])
    g = synth.rng(78, 1)
    dlogp, dent = g.standard_normal(6), g.standard_normal(6)

    def loss(h_, W_, b_):
        o = oracle.forward(h_, W_, b_, 0.7, case["targets"], None, 40)
        return float(dlogp @ o["logp"] + dent @ o["entropy"])

    f = oracle.forward(h, W, b, 0.7, case["targets"], None, 40)
    bw = oracle.backward(h, W, b, 0.7, case["targets"], None, 0, 48, 40, f["lse"], dlogp,
                         dent, f["entropy"])
    eps = 1e-6
    for (t, k) in ((0, 3), (5, 15)):
        hp, hm = h.copy(), h.copy(); hp[t, k] += eps; hm[t, k] -= eps
        fd = (loss(hp, W, b) - loss(hm, W, b)) / (2 * eps)
        assert abs(fd - bw["dhidden"][t, k]) < 1e-6 * max(1, abs(fd))
    for (v, k) in ((int(case["targets"][0]), 2), (11, 7), (45, 1)):   # 45 is padded: 0
        Wp, Wm = W.copy(), W.copy(); Wp[v, k] += eps; Wm[v, k] -= eps
        fd = (loss(h, Wp, b) - loss(h, Wm, b)) / (2 * eps)
        assert abs(fd - bw["dweight"][v, k]) < 1e-6 * max(1, abs(fd))
    for v in (int(case["targets"][1]), 30):
        bp, bm = b.copy(), b.copy(); bp[v] += eps; bm[v] -= eps
        fd = (loss(h, W, bp) - loss(h, W, bm)) / (2 * eps)
        assert abs(fd - bw["dbias"][v]) < 1e-6 * max(1, abs(fd))


def test_backward_invariants():
    case = synth.small_case(T=20, H=32, real_vocab=70, padded_vocab=80, temperature=0.7,
                            case_id=10, mask_frac=0.4)
    f = oracle.forward(case["hidden"], case["weight"], None, 0.7, case["targets"],
                       case["mask"], 70)
    dlogp = synth.rng(79, 1).standard_normal(20)
    bw = oracle.backward(case["hidden"], case["weight"], None, 0.7, case["targets"],
                         case["mask"], 0, 80, 70, f["lse"], dlogp, want_g=True)
    np.testing.assert_allclose(bw["G"].sum(axis=1), 0.0, atol=1e-13)   # sum_v (1[v=t]-p) = 0
    m = case["mask"].astype(bool)
    assert np.all(bw["G"][~m] == 0) and np.all(bw["dhidden"][~m] == 0)
    assert np.all(bw["dweight"][70:] == 0) and np.all(bw["dbias"][70:] == 0)
    # Sharded backward: dW rows are the shard's, dH sums over shards.
    parts = [oracle.backward(case["hidden"], case["weight"][lo:hi], None, 0.7,
                             case["targets"], case["mask"], lo, hi - lo, 70, f["lse"], dlogp)
             for lo, hi in ((0, 33), (33, 80))]
    np.testing.assert_allclose(parts[0]["dhidden"] + parts[1]["dhidden"], bw["dhidden"],
                               atol=1e-12)
    np.testing.assert_allclose(np.concatenate([parts[0]["dweight"], parts[1]["dweight"]]),
                               bw["dweight"], atol=1e-12)


def _topp_small(V=50, Vp=64, T=12, seed=11):
    g = synth.rng(seed, 1)
    x = (g.standard_normal((T, Vp)) * 2.0)
    ids = np.full((T, 64), -1, dtype=np.int64)
    for t in range(T):
        lst = np.concatenate([np.arange(V), g.integers(0, V, size=64 - V)])
        g.shuffle(lst)
        ids[t] = lst
    tg = g.integers(0, V, size=T)
    return x, ids, tg


def test_topp_full_nucleus_equals_full_vocab():
    """With every real id listed (top_p = 1) the replay score is the full-vocab log-softmax."""
    x, ids, tg = _topp_small()
    out = oracle.top_p_replay(x, ids, tg, 0.7, 0, 64, 50)
    z = torch.from_numpy(x[:, :50] / 0.7)
    ref = torch.log_softmax(z, -1).gather(1, torch.from_numpy(tg)[:, None])[:, 0].numpy()
    np.testing.assert_allclose(out["logp"], ref, atol=1e-12)
    np.testing.assert_allclose(out["lse"], torch.logsumexp(z, -1).numpy(), rtol=1e-14)


def test_topp_invariants_and_shards():
    x, ids, tg = _topp_small(seed=12)
    g = synth.rng(12, 2)
    ids_n = ids.copy()
    ids_n[:, 20:] = -1                                      # a nucleus of <= 20 slots
    a = oracle.top_p_replay(x, ids_n, tg, 0.7, 0, 64, 50)
    perm = ids_n.copy()
    for r in perm:
        g.shuffle(r)
    dup = np.where(ids_n >= 0, ids_n, np.roll(ids_n, 3, axis=1))  # duplicates into empty slots
    for other in (perm, dup):
        b = oracle.top_p_replay(x, other, tg, 0.7, 0, 64, 50)
        for k in ("lse", "logp", "target_logit"):
            np.testing.assert_array_equal(a[k], b[k])
    full = oracle.top_p_replay(x, ids, tg, 0.7, 0, 64, 50)
    assert np.all(a["lse"] <= full["lse"] + 1e-15)
    fin = np.isfinite(a["logp"])
    assert np.all(a["logp"][fin] >= full["logp"][fin] - 1e-15)
    # Shards (one with no candidates in some rows) merge to the unsharded result.
    parts = [oracle.top_p_replay(x[:, lo:hi], ids_n, tg, 0.7, lo, hi - lo, 50)
             for lo, hi in ((0, 16), (16, 32), (32, 48), (48, 64))]
    for p in parts:
        p["entropy"] = None
    mg = oracle.merge(parts)
    np.testing.assert_allclose(mg["lse"], a["lse"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(mg["logp"][fin], a["logp"][fin], atol=1e-13)
    assert np.all(mg["logp"][~fin] == -np.inf)


def test_topp_empty_and_invalid():
    x, ids, tg = _topp_small(T=3, seed=13)
    ids[0] = -1                                   # empty row
    ids[1, 0] = 50                                # padded id: invalid for the real vocab
    out = oracle.top_p_replay(x, ids, tg, 0.7, 0, 64, 50)
    assert out["lse"][0] == -np.inf and out["logp"][0] == -np.inf
    assert out["target_logit"][0] == 0 and out["in_range"][0] == 0
    assert out["status"] & oracle.ST_REPLAY_ID_INVALID


# ----------------------------------------------------------------------------- planted mistakes

def _mutant(**overrides):
    ns = types.SimpleNamespace(**{k: getattr(oracle, k) for k in dir(oracle) if not k.startswith("__")})
    for k, v in overrides.items():
        setattr(ns, k, v)

    # Rebind the module-level helpers the entry points use, so a mutation propagates.
    def shard_forward(*a, **k):
        saved = (oracle.logits, oracle.softmax_stats)
        oracle.logits, oracle.softmax_stats = ns.logits, ns.softmax_stats
        try:
            return _orig_shard_forward(*a, **k)
        finally:
            oracle.logits, oracle.softmax_stats = saved

    def forward(*a, **k):
        saved = (oracle.logits, oracle.softmax_stats)
        oracle.logits, oracle.softmax_stats = ns.logits, ns.softmax_stats
        try:
            return _orig_forward(*a, **k)
        finally:
            oracle.logits, oracle.softmax_stats = saved

    def backward(*a, **k):
        saved = oracle.logits
        oracle.logits = ns.logits
        try:
            return overrides.get("backward_impl", _orig_backward)(*a, **k)
        finally:
            oracle.logits = saved

    ns.shard_forward = overrides.get("shard_forward", shard_forward)
    ns.forward = overrides.get("forward", forward)
    ns.backward = backward
    if "merge" in overrides:
        ns.merge = overrides["merge"]
    return ns


_orig_shard_forward = oracle.shard_forward
_orig_forward = oracle.forward
_orig_backward = oracle.backward


def _tau_twice(h, w, b, tau):
    return _orig_logits_fn(h, w, b, tau) / tau


def _no_bias(h, w, b, tau):
    return _orig_logits_fn(h, w, None, tau)


def _entropy_sign(z):
    lse, ent = _orig_stats_fn(z)
    return lse, -ent


def _lse_without_max(z):
    m = z.max(axis=1)
    lse, ent = _orig_stats_fn(z)
    return lse - m, ent


def _target_off_by_one(h, W, b, tau, targets, *a, **k):
    return _orig_forward(h, W, b, tau, np.minimum(np.asarray(targets) + 1, 10 ** 9), *a, **k)


def _merge_drop_last(parts, mask=None):
    return oracle.merge(parts[:-1], mask) if len(parts) > 1 else oracle.merge(parts, mask)


def _backward_sign(*a, **k):
    out = _orig_backward(*a, **k)
    out["dhidden"] = -out["dhidden"]
    return out


_orig_logits_fn = oracle.logits
_orig_stats_fn = oracle.softmax_stats


@pytest.mark.parametrize("name,mut", [
    ("tau applied twice", dict(logits=_tau_twice)),
    ("bias dropped", dict(logits=_no_bias)),
    ("entropy sign", dict(softmax_stats=_entropy_sign)),
    ("lse without its max", dict(softmax_stats=_lse_without_max)),
    ("target index off by one", dict(forward=_target_off_by_one)),
    ("merge drops a shard", dict(merge=_merge_drop_last)),
    ("dH sign", dict(backward_impl=_backward_sign)),
])
def test_planted_mistakes_are_caught(name, mut):
    ns = _mutant(**mut)
    bias_case = synth.small_case(T=8, H=32, real_vocab=60, padded_vocab=64, temperature=0.7,
                                 case_id=14, with_bias=True, w_std=0.3)
    pins = [
        lambda: pin_mpmath(ns, bias_case, rows=[0]),
        lambda: pin_torch_library(ns, bias_case),
        lambda: pin_temperature_once(ns, synth.config1()),
        lambda: pin_merge_identity(ns, bias_case, [0, 20, 40, 64]),
        lambda: pin_backward_autograd(ns, bias_case, with_dent=False),
    ]
    failed = 0
    for p in pins:
        try:
            p()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"planted mistake '{name}' passed every pin"


def test_backward_vocab_subset_shard_equals_full_rows():
    """The full-size dweight check evaluates the oracle on a gathered set of vocabulary rows
    (every target plus others) as one shard, with targets renumbered to their position in the
    set. That reproduces the full backward's dweight rows: G[t, v] depends on z[t, v], the
    row's (global) lse and whether v is the row's target only."""
    case = synth.small_case(T=40, H=64, real_vocab=300, padded_vocab=320, temperature=0.7,
                            case_id=16, mask_frac=0.3, w_std=0.2)
    m = case["mask"].astype(bool)
    f = oracle.forward(case["hidden"], case["weight"], None, 0.7, case["targets"], case["mask"],
                       300)
    dlogp = synth.rng(16, 9).standard_normal(40) * m
    full = oracle.backward(case["hidden"], case["weight"], None, 0.7, case["targets"],
                           case["mask"], 0, 320, 300, f["lse"], dlogp)
    vs = np.unique(np.concatenate([case["targets"][m], [0, 7, 150, 299]]))
    pos = np.full(320, -1, dtype=np.int64)
    pos[vs] = np.arange(vs.size)
    rows = np.nonzero(m)[0]
    sub = oracle.backward(case["hidden"][rows], case["weight"][vs], None, 0.7,
                          pos[case["targets"][rows]], None, 0, vs.size, vs.size, f["lse"][rows],
                          dlogp[rows])
    np.testing.assert_allclose(sub["dweight"], full["dweight"][vs], rtol=1e-12, atol=1e-14)
