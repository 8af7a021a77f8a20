"""GPU parity at the full workload shapes (H=4096, V=151669 real / 151936 padded).

Every row is compared with the fp64 oracle on the same seeded inputs:
  * config 2: logp, entropy and lse of all 4096 rows, and 10 bitwise-equal repeats;
  * config 3: each of the four shards' partials and the rank-ordered merge, all rows;
  * config 4: logp of every scored row of the 16 packed sequences (14 chunks of 4096 rows),
    dhidden on two whole chunks plus a seeded 512-row sample of the others, and the dweight
    accumulated over all 14 chunks on a vocabulary subset holding every target, the
    real/padded boundary and 2048 seeded other rows; the repack (shuffled sequences, chunks of
    3000) is bitwise per row for logp and dhidden, and dweight is bitwise run to run; one
    backward call over the whole pack gives the chunked dhidden bitwise and its dweight to
    rounding;
  * config 5: the top-p replay of all rows, unsharded, per shard and merged.
Observed errors are printed (and logged when LLP_PARITY_LOG is set) and held to regression
guards far below the parity bounds.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import (GRAD_GUARD, GRAD_RTOL, LOGP_ATOL, LOGP_GUARD, assert_rows_close,
                        bytes_equal, dev, dev_bf16, host, need_gpu, normwise_rel, record, say)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "config2_targets.txt")
VR, VP, H = synth.V_REAL_FULL, synth.V_PAD_FULL, synth.H_FULL
TAU = 0.7
ORACLE_BLOCK = 512      # rows per oracle call where a call materialises [rows, V] arrays


def config2_targets():
    return np.loadtxt(GOLDEN, dtype=np.int64, comments="#")


def check_rows(gpu, ref, name, atol=LOGP_ATOL, guard=LOGP_GUARD):
    e = assert_rows_close(gpu, ref, atol, name)
    record(name, e)
    assert e <= guard, f"{name}: max error {e:.3g} above the regression guard {guard}"
    return e


def check_grad(gpu, ref, name):
    r = normwise_rel(gpu, ref)
    record(name, r)
    assert r <= GRAD_RTOL, f"{name}: normwise relative error {r:.3g} > {GRAD_RTOL}"
    assert r <= GRAD_GUARD, f"{name}: {r:.3g} above the regression guard {GRAD_GUARD}"
    return r


@pytest.fixture(scope="module")
def llp():
    need_gpu()
    import lm_head_linear_logp_amd as m
    m.open(0)
    return m


@pytest.fixture(scope="module")
def weight():
    say("generating W [151936, 4096] bf16")
    w = synth.full_weight()
    return dict(bits=w, dev=dev_bf16(w), f64=None)


def w64(weight):
    if weight["f64"] is None:
        weight["f64"] = oracle.bf16_to_f64(weight["bits"][:VR])
    return weight["f64"]


@pytest.fixture(scope="module")
def config2(weight):
    base = synth.config2_base()
    base["targets"] = config2_targets()
    base["hidden_dev"] = dev_bf16(base["hidden"])
    return base


@pytest.fixture(scope="module")
def config2_oracle(weight, config2):
    say("oracle: config-2 forward over all 4096 rows")
    return oracle.forward(config2["hidden"], w64(weight), None, TAU, config2["targets"], None, VR)


def fwd_full(llp, c, W, **kw):
    return llp.forward(c["hidden_dev"], W, dev(c["targets"]), temperature=TAU,
                       real_vocab=VR, padded_vocab=VP, **kw)


@pytest.mark.timeout(900)
def test_config2_every_row_and_repeats(llp, weight, config2, config2_oracle):
    say("config2 forward T=4096 H=4096 V=151669/151936 tau=0.7: 10 repeats, every row")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = [fwd_full(llp, config2, weight["dev"], status=st) for _ in range(10)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        for k in ("logp", "entropy", "lse", "target_logit", "in_range"):
            assert bytes_equal(outs[0][k], o[k]), k
    assert int(st.item()) == 0
    o = outs[0]
    assert np.all(host(o["in_range"]) == 1) and np.all(host(o["logp"]) <= 0)
    ref = config2_oracle
    check_rows(host(o["logp"]), ref["logp"], "config2 logp (4096 rows)")
    check_rows(host(o["entropy"]), ref["entropy"], "config2 entropy (4096 rows)")
    check_rows(host(o["lse"]), ref["lse"], "config2 lse (4096 rows)")
    check_rows(host(o["target_logit"]), ref["target_logit"], "config2 target logit (4096 rows)")


@pytest.mark.timeout(900)
def test_config3_four_shards_every_row(llp, weight, config2, config2_oracle):
    say("config3: 4 shards of 37984 + an empty shard, merged in rank order, every row")
    W = weight["dev"]
    tg = dev(config2["targets"])
    parts = []
    for r, (off, n) in enumerate(synth.shard_ranges()):
        parts.append(llp.forward(config2["hidden_dev"], W[off:off + n], tg, temperature=TAU,
                                 offset=off, real_vocab=VR, padded_vocab=VP, rank=r, world=4))
    empty = llp.forward(config2["hidden_dev"], W[:0], tg, temperature=TAU, offset=VP,
                        real_vocab=VR, padded_vocab=VP, rank=4, world=5)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    mg = llp.merge(parts, status=st)
    mg2 = llp.merge(parts[:2] + [empty] + parts[2:])
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.all(np.isneginf(host(empty["lse"]))) and np.all(host(empty["entropy"]) == 0)
    assert np.all(host(empty["target_logit"]) == 0) and np.all(host(empty["in_range"]) == 0)
    assert np.all(np.isneginf(host(empty["logp"])))
    for k in ("logp", "lse", "entropy"):
        assert bytes_equal(mg[k], mg2[k]), k            # an empty shard is bitwise neutral
    inr = np.stack([host(p["in_range"]) for p in parts])
    assert np.all(inr.sum(0) == 1)
    # Each shard's partials against the oracle's shard partials, every row (the last shard
    # has 37717 real columns and 267 padded ones).
    W64 = w64(weight)
    for r, (off, n) in enumerate(synth.shard_ranges()):
        say(f"oracle: shard {r} [{off}, {off + n})")
        nr = min(n, VR - off)
        ref = oracle.shard_forward(config2["hidden"], W64[off:off + nr], None, TAU,
                                   config2["targets"], None, off, n, VR)
        p = parts[r]
        np.testing.assert_array_equal(host(p["in_range"]), ref["in_range"])
        check_rows(host(p["lse"]), ref["lse"], f"config3 shard {r} lse")
        check_rows(host(p["entropy"]), ref["entropy"], f"config3 shard {r} entropy")
        check_rows(host(p["target_logit"]), ref["target_logit"], f"config3 shard {r} target logit")
        check_rows(host(p["logp"]), ref["logp"], f"config3 shard {r} local logp")
    ref = config2_oracle
    for k in ("logp", "lse", "entropy"):
        check_rows(host(mg[k]), ref[k], f"config3 merged {k} (4096 rows)")


# ----------------------------------------------------------------------------- config 4

def repack_index(order, lens):
    """Row indices of the packed stream after concatenating sequences in `order`."""
    cu = np.concatenate([[0], np.cumsum(lens)])
    return np.concatenate([np.arange(cu[s], cu[s + 1]) for s in order])


def run_forward_chunks(llp, W, hd, tg, mk, chunk):
    T = hd.shape[0]
    logp, lse = torch.empty(T, device="cuda"), torch.empty(T, device="cuda")
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        o = llp.forward(hd[c0:c1], W, tg[c0:c1], temperature=TAU, loss_mask=mk[c0:c1],
                        real_vocab=VR, padded_vocab=VP, want_entropy=False)
        logp[c0:c1] = o["logp"]
        lse[c0:c1] = o["lse"]
    return logp, lse


def run_backward_chunks(llp, W, hd, tg, mk, dl, lse, chunk):
    """One step's gradient: dhidden per chunk; dweight overwritten by the first chunk
    (LLP_FLAG_OVERWRITE_GRADS) and accumulated by the others, in chunk order."""
    T = hd.shape[0]
    dH = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    dW = torch.full((VP, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = None
    for i, c0 in enumerate(range(0, T, chunk)):
        c1 = min(T, c0 + chunk)
        llp.backward(hd[c0:c1], W, tg[c0:c1], lse[c0:c1], dl[c0:c1], temperature=TAU,
                     loss_mask=mk[c0:c1], real_vocab=VR, padded_vocab=VP, dweight=dW,
                     dhidden=dH[c0:c1], workspace=ws, overwrite=(i == 0))
    return dH, dW


@pytest.fixture(scope="module")
def config4(llp, weight):
    case = synth.config4_case()
    T = case["T"]
    m = case["mask"].astype(bool)
    say(f"config4: {T} packed tokens, {int(m.sum())} scored, chunks of 4096 (GPU runs)")
    W = weight["dev"]
    hd, tg, mk = dev_bf16(case["hidden"]), dev(case["targets"]), dev(case["mask"])
    dl = dev(case["dlogp"])
    logp, lse = run_forward_chunks(llp, W, hd, tg, mk, 4096)
    dH, dW = run_backward_chunks(llp, W, hd, tg, mk, dl, lse, 4096)
    dH2, dW2 = run_backward_chunks(llp, W, hd, tg, mk, dl, lse, 4096)
    torch.cuda.synchronize()
    same_dw = bytes_equal(dW, dW2) and bytes_equal(dH, dH2)
    del dH2, dW2
    # One backward call over the whole pack (T = 56583; G for all scored rows, ~17 GB).
    whole = run_backward_chunks(llp, W, hd, tg, mk, dl, lse, T)
    torch.cuda.synchronize()
    whole_dH_same = bytes_equal(whole[0], dH)
    whole_dW_rel = normwise_rel(host(whole[1])[:VR], host(dW)[:VR])
    whole_dW_pad = bool(np.all(host(whole[1])[VR:] == 0))
    del whole
    torch.cuda.empty_cache()
    idx = repack_index(synth.repack_order(), case["lens"])
    ix = dev(idx)
    logp_b, lse_b = run_forward_chunks(llp, W, hd[ix], tg[ix], mk[ix], 3000)
    dH_b, dW_b = run_backward_chunks(llp, W, hd[ix], tg[ix], mk[ix], dl[ix], lse_b, 3000)
    torch.cuda.synchronize()
    out = dict(case=case, idx=idx, logp=host(logp), lse=host(lse), dH=host(dH),
               dW=host(dW), same_dw=same_dw, logp_b=host(logp_b), dH_b=host(dH_b),
               dW_b=host(dW_b), whole_dH_same=whole_dH_same, whole_dW_rel=whole_dW_rel,
               whole_dW_pad=whole_dW_pad)
    del hd, dW, dW_b, dH, dH_b
    torch.cuda.empty_cache()
    return out


@pytest.fixture(scope="module")
def config4_oracle_fwd(weight, config4):
    case = config4["case"]
    m = case["mask"].astype(bool)
    say(f"oracle: config-4 forward over all {int(m.sum())} scored rows")
    return oracle.forward(case["hidden"], w64(weight), None, TAU, case["targets"], case["mask"],
                          VR)


@pytest.mark.timeout(900)
def test_config4_logp_every_scored_row(config4, config4_oracle_fwd):
    case = config4["case"]
    m = case["mask"].astype(bool)
    la = config4["logp"]
    assert np.all(la[~m] == 0) and not np.isnan(la).any()
    check_rows(la[m], config4_oracle_fwd["logp"][m], f"config4 logp ({int(m.sum())} scored rows)")
    check_rows(config4["lse"][m], config4_oracle_fwd["lse"][m], "config4 lse (scored rows)")


def test_config4_repack_bitwise(config4):
    """Shuffled sequences chunked at 3000 rows: logp and dhidden bitwise per row; dweight is a
    sum over rows in another order, equal to rounding."""
    idx = config4["idx"]
    np.testing.assert_array_equal(config4["logp"][idx].view(np.uint32),
                                  config4["logp_b"].view(np.uint32))
    np.testing.assert_array_equal(config4["dH"][idx], config4["dH_b"])
    r = normwise_rel(config4["dW_b"][:VR], config4["dW"][:VR])
    record("config4 dweight repacked vs chunked (normwise)", r)
    assert r <= 1e-5
    assert config4["same_dw"], "dweight / dhidden differ between two runs of the same chunks"


def test_config4_whole_pack_backward(config4):
    """One backward call over all 56583 rows: dhidden rows bitwise those of the 14 chunked
    calls (row-local arithmetic), dweight equal to rounding (one sum over the tokens instead of
    14 chunk sums added in order), padded dweight rows zero."""
    assert config4["whole_dH_same"], "whole-pack dhidden differs from the chunked dhidden"
    record("config4 dweight whole-pack vs chunked (normwise)", config4["whole_dW_rel"])
    assert config4["whole_dW_rel"] <= 1e-5
    assert config4["whole_dW_pad"]


@pytest.mark.timeout(900)
def test_config4_dhidden_two_chunks_and_sample(weight, config4, config4_oracle_fwd):
    case = config4["case"]
    T = case["T"]
    m = case["mask"].astype(bool)
    dH = oracle.bf16_to_f64(config4["dH"])
    assert not np.isnan(dH).any() and np.all(dH[~m] == 0)
    nchunk = (T + 4095) // 4096
    whole = [0, nchunk // 2]
    rows_whole = np.concatenate([np.arange(c * 4096, min(T, c * 4096 + 4096)) for c in whole])
    others = np.setdiff1d(np.nonzero(m)[0], rows_whole)
    sample = np.sort(synth.rng(4, 51).choice(others, 512, replace=False))
    W64 = w64(weight)
    for name, rows in ((f"chunks {whole}", rows_whole), ("512 sampled rows", sample)):
        ref = np.empty((rows.size, H))
        for b0 in range(0, rows.size, ORACLE_BLOCK):
            r = rows[b0:b0 + ORACLE_BLOCK]
            say(f"oracle: config-4 dhidden rows {b0}..{b0 + r.size} of {rows.size} ({name})")
            ref[b0:b0 + r.size] = oracle.backward(
                case["hidden"][r], W64, None, TAU, case["targets"][r], case["mask"][r], 0, VP,
                VR, config4_oracle_fwd["lse"][r], case["dlogp"][r].astype(np.float64))["dhidden"]
        check_grad(dH[rows], ref, f"config4 dhidden ({name})")


@pytest.mark.timeout(900)
def test_config4_dweight_accumulated_subset(weight, config4, config4_oracle_fwd):
    """dweight after all 14 chunks (the first overwriting, the rest accumulating) on the rows
    of every scored target, the last 300 real rows and 2048 seeded others. The oracle's
    dweight rows for a set of vocabulary ids are the backward of the shard made of those
    weight rows (G[t, v] depends on z[t, v], the row's lse and whether v is its target only);
    summed over the chunks in fp64."""
    case = config4["case"]
    m = case["mask"].astype(bool)
    dW = config4["dW"]
    assert not np.isnan(dW).any()
    assert np.all(dW[VR:] == 0), "padded dweight rows must be 0"
    g = synth.rng(4, 52)
    tg = case["targets"]
    vs = np.unique(np.concatenate([tg[m], np.arange(VR - 300, VR), g.choice(VR, 2048, replace=False)]))
    say(f"oracle: config-4 dweight on {vs.size} vocabulary rows over {int(m.sum())} scored rows")
    pos = np.full(VP, -1, dtype=np.int64)
    pos[vs] = np.arange(vs.size)
    Wsub = weight["bits"][vs]
    acc = np.zeros((vs.size, H))
    T = case["T"]
    for c0 in range(0, T, 4096):
        rows = np.arange(c0, min(T, c0 + 4096))
        rows = rows[m[rows]]
        for b0 in range(0, rows.size, 2048):
            r = rows[b0:b0 + 2048]
            # Every scored target is in vs, so its position is its column in the subset shard.
            rb = oracle.backward(case["hidden"][r], Wsub, None, TAU, pos[tg[r]], None, 0,
                                 vs.size, vs.size, config4_oracle_fwd["lse"][r],
                                 case["dlogp"][r].astype(np.float64))
            acc += rb["dweight"]
    check_grad(dW[vs], acc, f"config4 dweight accumulated over 14 chunks ({vs.size} rows)")


@pytest.mark.timeout(900)
def test_full_vocab_dweight_subset(llp, weight):
    """dW at full H and V over one 1024-row chunk accumulated into zeros, checked on a vocabulary
    subset that holds every target and the real/padded boundary; dhidden on every row."""
    g = synth.rng(4, 60)
    T = 1024
    hb = synth.normal_bf16(g, (T, H), 1.0)
    tg = g.integers(0, VR, T)
    mask = (g.random(T) > 0.25).astype(np.uint8)
    dlogp = g.standard_normal(T) * mask
    W = weight["dev"]
    f = llp.forward(dev_bf16(hb), W, dev(tg), temperature=TAU, loss_mask=dev(mask),
                    real_vocab=VR, padded_vocab=VP)
    ref = oracle.forward(hb, w64(weight), None, TAU, tg, mask, VR)
    check_rows(host(f["logp"]), ref["logp"], "1024-row logp")
    out = llp.backward(dev_bf16(hb), W, dev(tg), dev(ref["lse"], torch.float32),
                       dev(dlogp, torch.float32), temperature=TAU, loss_mask=dev(mask),
                       real_vocab=VR, padded_vocab=VP)
    torch.cuda.synchronize()
    rb = oracle.backward(hb, w64(weight), None, TAU, tg, mask, 0, VP, VR, ref["lse"], dlogp)
    vs = np.unique(np.concatenate([tg[mask.astype(bool)], np.arange(VR - 300, VP),
                                   g.choice(VR, 1500, replace=False)]))
    check_grad(host(out["dweight"])[vs], rb["dweight"][vs], f"1024-row dweight ({vs.size} rows)")
    assert np.all(host(out["dweight"])[VR:] == 0)
    check_grad(oracle.bf16_to_f64(host(out["dhidden"])), rb["dhidden"], "1024-row dhidden")
    # G held one vocabulary slab at a time (5 slabs): dweight bitwise the same, dhidden summed
    # slab by slab.
    sl = llp.backward(dev_bf16(hb), W, dev(tg), dev(ref["lse"], torch.float32),
                      dev(dlogp, torch.float32), temperature=TAU, loss_mask=dev(mask),
                      real_vocab=VR, padded_vocab=VP, g_slabs=True)
    torch.cuda.synchronize()
    assert bytes_equal(sl["dweight"], out["dweight"])
    check_grad(oracle.bf16_to_f64(host(sl["dhidden"])), rb["dhidden"],
               "1024-row dhidden, G in slabs")


# ----------------------------------------------------------------------------- config 5

@pytest.mark.timeout(900)
def test_config5_topp_every_row(llp):
    say("config5: top-p replay T=4096 V=151936 fp32 logits, unsharded and 4 shards")
    c = synth.topp_case()
    x = dev(c["logits"])
    ids, tg = dev(c["replay_ids"]), dev(c["targets"])
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    full = llp.top_p_replay(x, ids, tg, temperature=TAU, real_vocab=VR, padded_vocab=VP, status=st)
    parts = [llp.top_p_replay(x[:, off:off + n], ids, tg, temperature=TAU, offset=off,
                              real_vocab=VR, padded_vocab=VP, rank=r, world=4, status=st)
             for r, (off, n) in enumerate(synth.shard_ranges())]
    mg = llp.merge(parts, want_entropy=False, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref = oracle.top_p_replay(c["logits"], c["replay_ids"], c["targets"], TAU, 0, VP, VR)
    check_rows(host(full["logp"]), ref["logp"], "config5 logp (4096 rows)")
    check_rows(host(full["lse"]), ref["lse"], "config5 lse (4096 rows)")
    check_rows(host(mg["logp"]), ref["logp"], "config5 merged logp (4096 rows)")
    check_rows(host(mg["lse"]), ref["lse"], "config5 merged lse (4096 rows)")
    assert np.all(host(full["in_range"]) == 1)
    no_cand = 0
    for r, (off, n) in enumerate(synth.shard_ranges()):
        rs = oracle.top_p_replay(c["logits"][:, off:off + n], c["replay_ids"], c["targets"], TAU,
                                 off, n, VR)
        p = parts[r]
        np.testing.assert_array_equal(host(p["in_range"]), rs["in_range"])
        check_rows(host(p["lse"]), rs["lse"], f"config5 shard {r} lse")
        check_rows(host(p["target_logit"]), rs["target_logit"], f"config5 shard {r} target logit")
        no_cand += int(np.isneginf(rs["lse"]).sum())
    say(f"config5: shard rows without candidates: {no_cand}")
    assert no_cand > 0


def test_topp_capacity_56_ids(llp):
    c = synth.topp_case(T=256, big_nucleus=56, case_id=55)
    n = (c["replay_ids"] >= 0).sum(1)
    assert n.max() == 64
    out = llp.top_p_replay(dev(c["logits"]), dev(c["replay_ids"]), dev(c["targets"]),
                           temperature=TAU, real_vocab=VR, padded_vocab=VP)
    torch.cuda.synchronize()
    ref = oracle.top_p_replay(c["logits"], c["replay_ids"], c["targets"], TAU, 0, VP, VR)
    check_rows(host(out["logp"]), ref["logp"], "top-p capacity (56 ids + duplicates) logp")
