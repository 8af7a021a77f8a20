"""GPU parity at sizes the oracle finishes in seconds (several tiles, ragged tails), plus
bitwise determinism, batch-packing invariance, edge cases and status bits. Every call goes
through the C ABI (the Python binding only marshals arguments)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import (GRAD_RTOL, LOGP_ATOL, assert_rows_close, bytes_equal, dev, dev_bf16,
                        host, need_gpu, normwise_rel, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def llp():
    need_gpu()
    import lm_head_linear_logp_amd as m
    info = m.open(0)
    say(f"opened {info}")
    return m


def run_forward(llp, case, bias_dtype=torch.bfloat16, **kw):
    bias = None
    if case.get("bias") is not None:
        bias = dev_bf16(case["bias"])
        if bias_dtype == torch.float32:
            bias = bias.float()
    out = llp.forward(dev_bf16(case["hidden"]), dev_bf16(case["weight"]), dev(case["targets"]),
                      temperature=case["temperature"], bias=bias,
                      loss_mask=dev(case["mask"]), real_vocab=case["real_vocab"],
                      padded_vocab=case["padded_vocab"], **kw)
    torch.cuda.synchronize()
    return out


def check_forward(out, ref, mask, tag):
    m = mask.astype(bool)
    e1 = assert_rows_close(host(out["logp"]), ref["logp"], LOGP_ATOL, f"{tag} logp")
    e2 = assert_rows_close(host(out["entropy"]), ref["entropy"], LOGP_ATOL, f"{tag} entropy")
    e3 = assert_rows_close(host(out["lse"]), ref["lse"], LOGP_ATOL, f"{tag} lse")
    np.testing.assert_array_equal(host(out["in_range"]), ref["in_range"])
    assert np.all(host(out["logp"])[~m] == 0) and np.all(host(out["lse"])[~m] == 0)
    say(f"{tag}: max err logp {e1:.2e} entropy {e2:.2e} lse {e3:.2e}")
    return max(e1, e2)


def test_config1(llp):
    case = synth.config1()
    say("config1 forward T=64 H=256 V=1000/1024")
    out = run_forward(llp, case)
    ref = oracle.forward(case["hidden"], case["weight"], case["bias"], 1.0, case["targets"],
                         case["mask"], 1000)
    check_forward(out, ref, case["mask"], "config1")
    assert np.all(host(out["logp"]) <= 0)


SHAPES = [  # T, H, V_real, V_pad, tau, mask_frac, bias
    (600, 512, 1000, 1100, 0.7, 0.3, True),
    (257, 256, 513, 520, 1.3, 0.0, False),
    (1, 64, 1, 8, 0.5, 0.0, True),
    (300, 320, 2049, 2304, 0.7, 0.5, False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"T{s[0]}_H{s[1]}_V{s[2]}" for s in SHAPES])
def test_tiles_and_ragged_tails(llp, shape):
    T, H, Vr, Vp, tau, mf, hb = shape
    case = synth.small_case(T, H, Vr, Vp, tau, case_id=20 + T, mask_frac=mf, with_bias=hb,
                            w_std=0.05)
    say(f"small forward {shape}")
    ref = oracle.forward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                         case["mask"], Vr)
    out = run_forward(llp, case)
    check_forward(out, ref, case["mask"], f"shape{shape}")
    if hb:
        out32 = run_forward(llp, case, bias_dtype=torch.float32)
        # bf16 bias widened to fp32 is the same number: bitwise equal results.
        for k in ("logp", "entropy", "lse"):
            assert bytes_equal(out[k], out32[k]), k


# Over 256 tiles: the persistent forward workers (one per compute unit) run several tiles each,
# chaining each tile's last K steps into the next tile's first loads. Two K steps (H = 128) is
# the shortest chain; the masked case skips whole token blocks past the scored rows.
MANY_TILES = [  # T, H, V_real, V_pad, tau, mask_frac, bias
    (512, 128, 131000, 131072, 0.7, 0.0, False),
    (700, 256, 99990, 100096, 0.9, 0.4, True),
]


@pytest.mark.parametrize("shape", MANY_TILES, ids=[f"T{s[0]}_H{s[1]}_V{s[2]}" for s in MANY_TILES])
def test_several_tiles_per_worker(llp, shape):
    T, H, Vr, Vp, tau, mf, hb = shape
    case = synth.small_case(T, H, Vr, Vp, tau, case_id=90 + H, mask_frac=mf, with_bias=hb,
                            w_std=0.05)
    say(f"many-tile forward {shape}")
    ref = oracle.forward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                         case["mask"], Vr)
    out = run_forward(llp, case)
    check_forward(out, ref, case["mask"], f"many{shape}")
    again = run_forward(llp, case)
    for k in ("logp", "entropy", "lse", "target_logit", "in_range"):
        assert bytes_equal(out[k], again[k]), k


def test_padded_columns_excluded_bitwise(llp):
    case = synth.small_case(200, 256, 700, 768, 0.7, case_id=40, w_std=0.05)
    a = run_forward(llp, case)
    W = case["weight"].copy()
    big = np.where(np.arange(W[700:].size).reshape(W[700:].shape) % 2, 1e4, -1e4)
    W[700:] = synth.bf16_bits(big.astype(np.float32))
    b = run_forward(llp, dict(case, weight=W))
    for k in ("logp", "entropy", "lse", "target_logit"):
        assert bytes_equal(a[k], b[k]), k


def test_repeat_runs_bitwise(llp):
    case = synth.small_case(700, 512, 3000, 3072, 0.7, case_id=41, mask_frac=0.2, w_std=0.05)
    outs = [run_forward(llp, case) for _ in range(4)]
    for o in outs[1:]:
        for k in ("logp", "entropy", "lse", "target_logit", "in_range"):
            assert bytes_equal(outs[0][k], o[k]), k


def test_batch_packing_invariance_bitwise(llp):
    """The same rows, permuted and embedded among extra masked rows, give identical bytes."""
    case = synth.small_case(500, 512, 3000, 3072, 0.7, case_id=42, mask_frac=0.3, w_std=0.05)
    a = run_forward(llp, case)
    g = synth.rng(42, 9)
    perm = g.permutation(500)
    extra = 77
    hid = np.concatenate([case["hidden"][perm], synth.normal_bf16(g, (extra, 512), 1.0)])
    tg = np.concatenate([case["targets"][perm], g.integers(0, 3000, extra)])
    mk = np.concatenate([case["mask"][perm], np.zeros(extra, np.uint8)])
    order = g.permutation(500 + extra)
    case2 = dict(case, T=500 + extra, hidden=hid[order], targets=tg[order], mask=mk[order])
    b = run_forward(llp, case2)
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    rows_b = inv[np.arange(500)]          # position of original permuted row i in case2
    for k in ("logp", "entropy", "lse", "target_logit"):
        ha, hb = host(a[k]), host(b[k])
        np.testing.assert_array_equal(ha[perm].view(np.uint32), hb[rows_b].view(np.uint32))


def test_temperature_power_of_two_bitwise(llp):
    """tau = 2 with W equals tau = 1 with W/2 bit for bit: tau is applied exactly once."""
    case = synth.small_case(300, 256, 1000, 1024, 2.0, case_id=43, w_std=0.05)
    a = run_forward(llp, case)
    W2 = synth.bf16_bits((oracle.bf16_to_f64(case["weight"]) / 2).astype(np.float32))
    b = run_forward(llp, dict(case, weight=W2, temperature=1.0))
    for k in ("logp", "entropy", "lse", "target_logit"):
        assert bytes_equal(a[k], b[k]), k


def shard_run(llp, case, cuts, want_entropy=True):
    parts = []
    Vp, Vr = case["padded_vocab"], case["real_vocab"]
    hid, tg, mk = dev_bf16(case["hidden"]), dev(case["targets"]), dev(case["mask"])
    W = dev_bf16(case["weight"])
    for r, (lo, hi) in enumerate(zip(cuts[:-1], cuts[1:])):
        parts.append(llp.forward(hid, W[lo:hi], tg, temperature=case["temperature"], loss_mask=mk,
                                 offset=lo, real_vocab=Vr, padded_vocab=Vp, rank=r,
                                 world=len(cuts) - 1, want_entropy=want_entropy))
    torch.cuda.synchronize()
    return parts


def test_shards_and_empty_shard(llp):
    case = synth.small_case(400, 256, 1900, 2048, 0.7, case_id=44, mask_frac=0.2, w_std=0.05)
    ref = oracle.forward(case["hidden"], case["weight"], None, 0.7, case["targets"],
                         case["mask"], 1900)
    for cuts in ([0, 512, 1024, 1536, 2048], [0, 700, 700, 1900, 2048], [0, 1, 999, 2048]):
        say(f"shards {cuts}")
        parts = shard_run(llp, case, cuts)
        for r, (lo, hi) in enumerate(zip(cuts[:-1], cuts[1:])):
            pr = oracle.shard_forward(case["hidden"], case["weight"][lo:hi], None, 0.7,
                                      case["targets"], case["mask"], lo, hi - lo, 1900)
            for k in ("lse", "entropy", "logp"):
                assert_rows_close(host(parts[r][k]), pr[k], LOGP_ATOL, f"shard{r} {k}")
            np.testing.assert_array_equal(host(parts[r]["in_range"]), pr["in_range"])
            if hi - lo == 0 or lo >= 1900:   # empty shard: exact empty values, no NaN
                m = case["mask"].astype(bool)
                assert np.all(np.isneginf(host(parts[r]["lse"])[m]))
                assert np.all(host(parts[r]["target_logit"]) == 0)
                assert np.all(host(parts[r]["entropy"]) == 0)
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        mg = llp.merge(parts, loss_mask=dev(case["mask"]), status=st)
        torch.cuda.synchronize()
        for k in ("logp", "lse", "entropy"):
            assert_rows_close(host(mg[k]), ref[k], LOGP_ATOL, f"merged {k}")
        assert int(st.item()) == 0


def test_merge_empty_shard_inserted_bitwise(llp):
    case = synth.small_case(256, 256, 1000, 1024, 0.7, case_id=45, w_std=0.05)
    p = shard_run(llp, case, [0, 512, 1024])
    e = shard_run(llp, case, [0, 512, 512, 1024])
    a = llp.merge(p)
    b = llp.merge([e[0], e[1], e[2]])
    torch.cuda.synchronize()
    for k in ("logp", "lse", "entropy"):
        assert bytes_equal(a[k], b[k]), k


def test_status_bits_and_no_nan(llp):
    case = synth.small_case(64, 128, 500, 512, 0.7, case_id=46, w_std=0.05)
    tg = case["targets"].copy()
    tg[3], tg[10] = 500, -1            # padded id and negative id: out of range
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = run_forward(llp, dict(case, targets=tg), status=st)
    lp = host(out["logp"])
    assert np.isneginf(lp[3]) and np.isneginf(lp[10]) and np.isfinite(np.delete(lp, [3, 10])).all()
    assert int(st.item()) & llp.STATUS_BITS["TARGET_OUT_OF_RANGE"]
    assert not np.isnan(host(out["entropy"])).any()
    # Malformed cu_seqlens -> layout bit; results unaffected.
    st.zero_()
    cu = torch.tensor([0, 40, 30, 64], dtype=torch.int32, device="cuda")
    out2 = run_forward(llp, case, status=st, cu_seqlens=cu)
    assert int(st.item()) == llp.STATUS_BITS["LAYOUT_INVALID"]
    ref = run_forward(llp, case)
    assert bytes_equal(out2["logp"], ref["logp"])


def test_all_rows_masked_and_zero_rows(llp):
    case = synth.small_case(50, 64, 100, 128, 0.7, case_id=47)
    out = run_forward(llp, dict(case, mask=np.zeros(50, np.uint8)))
    for k in ("logp", "lse", "entropy", "target_logit"):
        assert np.all(host(out[k]) == 0)
    e = dict(case, T=0, hidden=case["hidden"][:0], targets=case["targets"][:0],
             mask=case["mask"][:0])
    out0 = run_forward(llp, e)
    assert out0["logp"].numel() == 0


# ------------------------------------------------------------------------------ top-p

def topp_inputs(T=300, V=600, Vp=640, seed=50):
    g = synth.rng(seed, 1)
    x = (g.standard_normal((T, Vp)) * 2.0).astype(np.float32)
    x[:, V:] = -1e30
    ids = np.full((T, 64), -1, dtype=np.int64)
    for t in range(T):
        n = int(g.integers(0, 40))
        lst = g.choice(V, size=n, replace=False) if n else np.zeros(0, np.int64)
        lst = np.concatenate([lst, lst[: int(g.integers(0, n + 1))]])[:64] if n else lst
        g.shuffle(lst)
        ids[t, :lst.size] = lst
    tg = np.where(g.random(T) < 0.8, ids[:, 0], g.integers(0, V, T))
    tg = np.where(tg < 0, 0, tg)
    return x, ids, tg


def test_topp_small_parity_and_invariance(llp):
    x, ids, tg = topp_inputs()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = llp.top_p_replay(dev(x), dev(ids), dev(tg), temperature=0.7, real_vocab=600,
                           padded_vocab=640, status=st)
    torch.cuda.synchronize()
    ref = oracle.top_p_replay(x, ids, tg, 0.7, 0, 640, 600)
    for k in ("lse", "logp"):
        assert_rows_close(host(out[k]), ref[k], LOGP_ATOL, f"topp {k}")
    np.testing.assert_array_equal(host(out["in_range"]), ref["in_range"])
    # permuted + duplicated ids: bitwise identical
    g = synth.rng(51, 1)
    ids2 = ids.copy()
    for r in ids2:
        g.shuffle(r)
    out2 = llp.top_p_replay(dev(x), dev(ids2), dev(tg), temperature=0.7, real_vocab=600,
                            padded_vocab=640)
    torch.cuda.synchronize()
    for k in ("lse", "logp", "target_logit"):
        assert bytes_equal(out[k], out2[k]), k
    assert int(st.item()) == 0


def test_topp_full_nucleus_matches_fused_forward(llp):
    """V <= 64 with every real id listed: replay logp == full-vocab logp (top_p = 1)."""
    case = synth.small_case(128, 256, 50, 64, 0.7, case_id=52, w_std=0.2)
    fwd = run_forward(llp, case)
    z = (oracle.bf16_to_f64(case["hidden"]) @ oracle.bf16_to_f64(case["weight"]).T).astype(np.float32)
    ids = np.tile(np.concatenate([np.arange(50), np.arange(14)]), (128, 1)).astype(np.int64)
    out = llp.top_p_replay(dev(z), dev(ids), dev(case["targets"]), temperature=0.7,
                           real_vocab=50, padded_vocab=64)
    torch.cuda.synchronize()
    assert_rows_close(host(out["logp"]), host(fwd["logp"]), LOGP_ATOL, "topp vs fused")


def test_topp_shards_empty_and_status(llp):
    x, ids, tg = topp_inputs(seed=53)
    ids[5] = -1                    # empty row
    ids[7, 3] = 600                # padded id: invalid
    ids[8, 0] = -5                 # negative: invalid
    parts = []
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    xd = dev(x)
    for r, (lo, hi) in enumerate([(0, 160), (160, 320), (320, 480), (480, 640)]):
        parts.append(llp.top_p_replay(xd[:, lo:hi], dev(ids), dev(tg), temperature=0.7, offset=lo,
                                      real_vocab=600, padded_vocab=640, rank=r, world=4,
                                      status=st))
    mg = llp.merge(parts, want_entropy=False, status=st)
    torch.cuda.synchronize()
    ref = oracle.top_p_replay(x, ids, tg, 0.7, 0, 640, 600)
    for k in ("lse", "logp"):
        assert_rows_close(host(mg[k]), ref[k], LOGP_ATOL, f"topp merged {k}")
    assert np.isneginf(host(mg["lse"])[5])
    s = int(st.item())
    assert s & llp.STATUS_BITS["REPLAY_ID_INVALID"] and s & llp.STATUS_BITS["TARGET_NOT_FOUND"]
    with pytest.raises(llp.LLPError):
        llp.top_p_replay(xd, dev(ids), dev(tg), temperature=0.7, real_vocab=600,
                         padded_vocab=640, processed_logprobs=False)


def test_topp_bf16_logits(llp):
    x, ids, tg = topp_inputs(seed=54)
    xb = synth.bf16_bits(np.maximum(x, -1e30))
    out = llp.top_p_replay(dev_bf16(xb), dev(ids), dev(tg), temperature=0.7, real_vocab=600,
                           padded_vocab=640)
    torch.cuda.synchronize()
    ref = oracle.top_p_replay(oracle.bf16_to_f64(xb), ids, tg, 0.7, 0, 640, 600)
    assert_rows_close(host(out["logp"]), ref["logp"], LOGP_ATOL, "topp bf16 logp")


# ------------------------------------------------------------------------------ backward

def run_backward(llp, case, lse, dlogp, dent=None, ent=None, bias_dtype=torch.bfloat16, **kw):
    bias = None
    if case.get("bias") is not None:
        bias = dev_bf16(case["bias"])
        if bias_dtype == torch.float32:
            bias = bias.float()
    out = llp.backward(dev_bf16(case["hidden"]), dev_bf16(case["weight"]), dev(case["targets"]),
                       dev(lse, torch.float32), dev(dlogp, torch.float32),
                       temperature=case["temperature"], bias=bias, loss_mask=dev(case["mask"]),
                       real_vocab=case["real_vocab"], padded_vocab=case["padded_vocab"],
                       dentropy=None if dent is None else dev(dent, torch.float32),
                       entropy=None if ent is None else dev(ent, torch.float32), **kw)
    torch.cuda.synchronize()
    return out


BWD = [  # T, H, V_real, V_pad, tau, mask_frac, bias, dentropy
    (300, 256, 1000, 1024, 0.7, 0.3, True, False),
    (513, 320, 700, 768, 1.0, 0.0, False, True),
    (64, 256, 1000, 1024, 0.7, 0.0, False, False),
]


@pytest.mark.parametrize("shape", BWD, ids=[f"T{s[0]}_H{s[1]}_V{s[2]}_ent{int(s[7])}" for s in BWD])
def test_backward_parity(llp, shape):
    T, H, Vr, Vp, tau, mf, hb, went = shape
    case = synth.small_case(T, H, Vr, Vp, tau, case_id=60 + T, mask_frac=mf, with_bias=hb,
                            w_std=0.1)
    say(f"backward {shape}")
    f = oracle.forward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                       case["mask"], Vr)
    g = synth.rng(60 + T, 7)
    dlogp = g.standard_normal(T) * case["mask"]
    dent = g.standard_normal(T) * case["mask"] if went else None
    ref = oracle.backward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                          case["mask"], 0, Vp, Vr, f["lse"], dlogp, dent,
                          f["entropy"] if went else None)
    out = run_backward(llp, case, f["lse"], dlogp, dent, f["entropy"] if went else None)
    dH = oracle.bf16_to_f64(host(out["dhidden"]))
    r1 = normwise_rel(dH, ref["dhidden"])
    r2 = normwise_rel(host(out["dweight"]), ref["dweight"])
    say(f"  rel dH {r1:.2e} dW {r2:.2e}")
    assert r1 <= GRAD_RTOL and r2 <= GRAD_RTOL
    m = case["mask"].astype(bool)
    assert np.all(dH[~m] == 0)
    assert np.all(host(out["dweight"])[Vr:] == 0)
    if hb:
        r3 = normwise_rel(host(out["dbias"]), ref["dbias"])
        say(f"  rel db {r3:.2e}")
        assert r3 <= GRAD_RTOL


def test_backward_bitwise_and_dh_row_invariance(llp):
    case = synth.small_case(400, 256, 1500, 1536, 0.7, case_id=70, mask_frac=0.25, w_std=0.1)
    f = oracle.forward(case["hidden"], case["weight"], None, 0.7, case["targets"], case["mask"],
                       1500)
    dlogp = synth.rng(70, 3).standard_normal(400) * case["mask"]
    a = run_backward(llp, case, f["lse"], dlogp)
    b = run_backward(llp, case, f["lse"], dlogp)
    assert bytes_equal(a["dhidden"], b["dhidden"]) and bytes_equal(a["dweight"], b["dweight"])
    perm = synth.rng(70, 4).permutation(400)
    c2 = dict(case, hidden=case["hidden"][perm], targets=case["targets"][perm],
              mask=case["mask"][perm])
    c = run_backward(llp, c2, f["lse"][perm], dlogp[perm])
    np.testing.assert_array_equal(host(a["dhidden"])[perm], host(c["dhidden"]))


def test_backward_accumulates_dweight(llp):
    case = synth.small_case(128, 256, 500, 512, 0.7, case_id=71, w_std=0.1)
    f = oracle.forward(case["hidden"], case["weight"], None, 0.7, case["targets"], None, 500)
    dlogp = synth.rng(71, 3).standard_normal(128)
    one = run_backward(llp, case, f["lse"], dlogp)
    two = run_backward(llp, case, f["lse"], dlogp, dweight=one["dweight"].clone())
    np.testing.assert_allclose(host(two["dweight"]), 2 * host(one["dweight"]), rtol=1e-6, atol=1e-9)


def test_backward_vocab_shards_sum_to_unsharded(llp):
    """Per-shard backward with the merged lse: each shard matches the oracle's shard backward,
    dhidden summed over the shards and dweight assembled from them match the unsharded
    gradients. Cuts include an empty shard, one that ends at the last real column and one that
    holds padding only (zero dhidden, dweight rows untouched)."""
    T, H, Vr, Vp, tau = 300, 256, 900, 1024, 0.7
    case = synth.small_case(T, H, Vr, Vp, tau, case_id=72, mask_frac=0.2, w_std=0.1)
    f = oracle.forward(case["hidden"], case["weight"], None, tau, case["targets"], case["mask"],
                       Vr)
    g = synth.rng(72, 3)
    dlogp = g.standard_normal(T) * case["mask"]
    dent = g.standard_normal(T) * case["mask"]
    full = oracle.backward(case["hidden"], case["weight"], None, tau, case["targets"],
                           case["mask"], 0, Vp, Vr, f["lse"], dlogp, dent, f["entropy"])
    cuts = [0, 256, 520, 520, 900, 1024]
    dW = torch.zeros((Vp, H), dtype=torch.float32, device="cuda")
    dH_sum = np.zeros((T, H))
    for r, (lo, hi) in enumerate(zip(cuts[:-1], cuts[1:])):
        say(f"backward shard {r} [{lo}, {hi})")
        out = run_backward(llp, dict(case, weight=case["weight"][lo:hi]), f["lse"], dlogp, dent,
                           f["entropy"], offset=lo, rank=r, world=len(cuts) - 1,
                           dweight=dW[lo:hi])
        dH = oracle.bf16_to_f64(host(out["dhidden"]))
        ref = oracle.backward(case["hidden"], case["weight"][lo:hi], None, tau, case["targets"],
                              case["mask"], lo, hi - lo, Vr, f["lse"], dlogp, dent,
                              f["entropy"])
        if lo >= Vr or hi == lo:
            assert np.all(dH == 0)
        else:
            r1 = normwise_rel(dH, ref["dhidden"])
            say(f"  rel dH {r1:.2e}")
            assert r1 <= GRAD_RTOL
        dH_sum += dH
    r1 = normwise_rel(dH_sum, full["dhidden"])
    r2 = normwise_rel(host(dW), full["dweight"])
    say(f"summed shards: rel dH {r1:.2e} dW {r2:.2e}")
    assert r1 <= GRAD_RTOL and r2 <= GRAD_RTOL
    assert np.all(host(dW)[Vr:] == 0)


def test_backward_f32_bias_masked_and_empty(llp):
    """fp32 bias: dH, dW, db against the oracle. All rows masked: dhidden zero, dweight and
    dbias unchanged. No rows at all: nothing written."""
    T, H, Vr, Vp, tau = 200, 128, 500, 512, 0.9
    case = synth.small_case(T, H, Vr, Vp, tau, case_id=73, mask_frac=0.3, with_bias=True,
                            w_std=0.1)
    f = oracle.forward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                       case["mask"], Vr)
    dlogp = synth.rng(73, 3).standard_normal(T) * case["mask"]
    ref = oracle.backward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                          case["mask"], 0, Vp, Vr, f["lse"], dlogp)
    out = run_backward(llp, case, f["lse"], dlogp, bias_dtype=torch.float32)
    r1 = normwise_rel(oracle.bf16_to_f64(host(out["dhidden"])), ref["dhidden"])
    r2 = normwise_rel(host(out["dweight"]), ref["dweight"])
    r3 = normwise_rel(host(out["dbias"]), ref["dbias"])
    say(f"f32 bias: rel dH {r1:.2e} dW {r2:.2e} db {r3:.2e}")
    assert r1 <= GRAD_RTOL and r2 <= GRAD_RTOL and r3 <= GRAD_RTOL

    ones_w = torch.ones((Vp, H), dtype=torch.float32, device="cuda")
    ones_b = torch.ones(Vp, dtype=torch.float32, device="cuda")
    masked = run_backward(llp, dict(case, mask=np.zeros(T, np.uint8)), f["lse"], dlogp,
                          bias_dtype=torch.float32, dweight=ones_w, dbias=ones_b)
    assert np.all(host(masked["dhidden"]) == 0)
    assert np.all(host(ones_w) == 1) and np.all(host(ones_b) == 1)

    empty = dict(case, T=0, hidden=case["hidden"][:0], targets=case["targets"][:0],
                 mask=case["mask"][:0])
    out0 = run_backward(llp, empty, f["lse"][:0], dlogp[:0], bias_dtype=torch.float32,
                        dweight=ones_w, dbias=ones_b)
    assert out0["dhidden"].numel() == 0
    assert np.all(host(ones_w) == 1) and np.all(host(ones_b) == 1)


def test_backward_overwrite_mode(llp):
    """LLP_FLAG_OVERWRITE_GRADS: dweight and dbias are bitwise the accumulate form applied to
    zeroed buffers, whatever the buffers held (NaN here), and match the oracle; padding rows
    are written as 0. All rows masked, no rows at all, and a shard of padding only: every row
    of dweight and dbias is written as 0."""
    T, H, Vr, Vp, tau = 300, 320, 1300, 1536, 0.8
    case = synth.small_case(T, H, Vr, Vp, tau, case_id=74, mask_frac=0.25, with_bias=True,
                            w_std=0.1)
    f = oracle.forward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                       case["mask"], Vr)
    dlogp = synth.rng(74, 3).standard_normal(T) * case["mask"]
    ref = oracle.backward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                          case["mask"], 0, Vp, Vr, f["lse"], dlogp)
    acc = run_backward(llp, case, f["lse"], dlogp, bias_dtype=torch.float32)
    nan_w = torch.full((Vp, H), float("nan"), dtype=torch.float32, device="cuda")
    nan_b = torch.full((Vp,), float("nan"), dtype=torch.float32, device="cuda")
    ow = run_backward(llp, case, f["lse"], dlogp, bias_dtype=torch.float32, dweight=nan_w,
                      dbias=nan_b, overwrite=True)
    assert bytes_equal(ow["dweight"], acc["dweight"]) and bytes_equal(ow["dbias"], acc["dbias"])
    assert bytes_equal(ow["dhidden"], acc["dhidden"])
    r2 = normwise_rel(host(nan_w), ref["dweight"])
    r3 = normwise_rel(host(nan_b), ref["dbias"])
    say(f"overwrite: rel dW {r2:.2e} db {r3:.2e}")
    assert r2 <= GRAD_RTOL and r3 <= GRAD_RTOL
    assert np.all(host(nan_w)[Vr:] == 0) and np.all(host(nan_b)[Vr:] == 0)

    def all_zero(*ts):
        return all(np.all(host(t) == 0) for t in ts)

    for name, c, lse, dl in (
            ("all rows masked", dict(case, mask=np.zeros(T, np.uint8)), f["lse"], dlogp),
            ("no rows", dict(case, hidden=case["hidden"][:0], targets=case["targets"][:0],
                             mask=case["mask"][:0]), f["lse"][:0], dlogp[:0])):
        say(f"overwrite: {name}")
        nan_w.fill_(float("nan"))
        nan_b.fill_(float("nan"))
        run_backward(llp, c, lse, dl, bias_dtype=torch.float32, dweight=nan_w, dbias=nan_b,
                     overwrite=True)
        assert all_zero(nan_w, nan_b), name
    say("overwrite: padding-only shard")
    lo = Vr
    sw = torch.full((Vp - lo, H), float("nan"), dtype=torch.float32, device="cuda")
    sb = torch.full((Vp - lo,), float("nan"), dtype=torch.float32, device="cuda")
    out = run_backward(llp, dict(case, weight=case["weight"][lo:], bias=case["bias"][lo:]),
                       f["lse"], dlogp, bias_dtype=torch.float32, offset=lo, rank=1, world=2,
                       dweight=sw, dbias=sb, overwrite=True)
    assert all_zero(sw, sb, out["dhidden"])


def test_backward_g_slabs(llp):
    """LLP_FLAG_G_SLABS: G held one vocabulary slab of 32768 columns at a time. 70144 columns
    make three slabs (the last one ragged, with the padded columns). dweight and dbias are
    bitwise those of the default mode (each tile's arithmetic is the same); dhidden, summed
    slab by slab, matches the oracle, repeats bitwise and keeps each row's bits under a
    permutation of the rows; accumulation into an existing dweight and two vocabulary shards
    agree with the default mode."""
    T, H, Vr, Vp, tau = 300, 256, 70000, 70144, 0.7
    case = synth.small_case(T, H, Vr, Vp, tau, case_id=85, mask_frac=0.2, with_bias=True,
                            w_std=0.05)
    f = oracle.forward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                       case["mask"], Vr)
    g = synth.rng(85, 7)
    dlogp = g.standard_normal(T) * case["mask"]
    dent = g.standard_normal(T) * case["mask"]
    ref = oracle.backward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                          case["mask"], 0, Vp, Vr, f["lse"], dlogp, dent, f["entropy"])
    args = (llp, case, f["lse"], dlogp, dent, f["entropy"], torch.float32)
    base = run_backward(*args, overwrite=True)
    sl = run_backward(*args, overwrite=True, g_slabs=True)
    assert bytes_equal(sl["dweight"], base["dweight"]) and bytes_equal(sl["dbias"], base["dbias"])
    dH = oracle.bf16_to_f64(host(sl["dhidden"]))
    r1 = normwise_rel(dH, ref["dhidden"])
    say(f"  G in slabs: rel dH {r1:.2e}")
    assert r1 <= GRAD_RTOL
    assert np.all(dH[case["mask"] == 0] == 0)
    again = run_backward(*args, overwrite=True, g_slabs=True)
    assert bytes_equal(again["dhidden"], sl["dhidden"])
    perm = synth.rng(85, 8).permutation(T)
    c2 = dict(case, hidden=case["hidden"][perm], targets=case["targets"][perm],
              mask=case["mask"][perm])
    p = run_backward(llp, c2, f["lse"][perm], dlogp[perm], dent[perm], f["entropy"][perm],
                     torch.float32, overwrite=True, g_slabs=True)
    np.testing.assert_array_equal(host(sl["dhidden"])[perm], host(p["dhidden"]))
    # Accumulating into an existing dweight: bitwise the default mode's accumulation.
    start = torch.randn((Vp, H), device="cuda")
    acc_base = run_backward(*args, dweight=start.clone())
    acc_sl = run_backward(*args, dweight=start.clone(), g_slabs=True)
    assert bytes_equal(acc_sl["dweight"], acc_base["dweight"])
    # Two shards of 137 tiles (two slabs each; the second holds the real/padded boundary).
    hid, tg, mk = dev_bf16(case["hidden"]), dev(case["targets"]), dev(case["mask"])
    W, bias = dev_bf16(case["weight"]), dev_bf16(case["bias"]).float()
    dH2 = np.zeros((T, H))
    for r, (lo, hi) in enumerate(((0, 35072), (35072, Vp))):
        kw = dict(temperature=tau, bias=bias[lo:hi], loss_mask=mk, offset=lo, real_vocab=Vr,
                  padded_vocab=Vp, rank=r, world=2, dentropy=dev(dent, torch.float32),
                  entropy=dev(f["entropy"], torch.float32), overwrite=True)
        a = llp.backward(hid, W[lo:hi], tg, dev(f["lse"], torch.float32),
                         dev(dlogp, torch.float32), **kw)
        b = llp.backward(hid, W[lo:hi], tg, dev(f["lse"], torch.float32),
                         dev(dlogp, torch.float32), g_slabs=True, **kw)
        torch.cuda.synchronize()
        assert bytes_equal(a["dweight"], b["dweight"]) and bytes_equal(a["dbias"], b["dbias"])
        assert bytes_equal(b["dweight"], base["dweight"][lo:hi])
        dH2 += oracle.bf16_to_f64(host(b["dhidden"]))
    r2 = normwise_rel(dH2, ref["dhidden"])
    say(f"  two shards, G in slabs: rel summed dH {r2:.2e}")
    assert r2 <= GRAD_RTOL


def test_backward_g_slabs_bf16_bias_odd_k_steps(llp):
    # H = 320 (5 K steps), a bf16 bias, 258 vocabulary tiles: slabs of 128, 128 and 2 tiles.
    T, H, Vr, Vp, tau = 129, 320, 66000, 66048, 1.3
    case = synth.small_case(T, H, Vr, Vp, tau, case_id=86, with_bias=True, w_std=0.05)
    f = oracle.forward(case["hidden"], case["weight"], case["bias"], tau, case["targets"], None,
                       Vr)
    dlogp = synth.rng(86, 7).standard_normal(T)
    ref = oracle.backward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                          None, 0, Vp, Vr, f["lse"], dlogp)
    base = run_backward(llp, case, f["lse"], dlogp, overwrite=True)
    sl = run_backward(llp, case, f["lse"], dlogp, overwrite=True, g_slabs=True)
    assert bytes_equal(sl["dweight"], base["dweight"]) and bytes_equal(sl["dbias"], base["dbias"])
    r = normwise_rel(oracle.bf16_to_f64(host(sl["dhidden"])), ref["dhidden"])
    say(f"  G in slabs, H=320, bf16 bias: rel dH {r:.2e}")
    assert r <= GRAD_RTOL


def test_forward_batch_size_invariance_bitwise(llp):
    """The same rows in batches of different size get the same bits: 5700 rows over 12
    vocabulary tiles make 276 tiles (more than one round on a 256-CU device); 700 of those rows
    (token blocks 0-1 and 19-20 of the large batch) make 36 tiles in another order. Sampled
    rows match the oracle."""
    T, H, Vr, Vp, tau = 5700, 512, 3000, 3072, 0.7
    case = synth.small_case(T, H, Vr, Vp, tau, case_id=75, mask_frac=0.1, with_bias=True,
                            w_std=0.05)
    say("forward batch size: T=5700 V=3000 vs 700 of its rows")
    a = run_forward(llp, case)
    rows = np.concatenate([np.arange(0, 350), np.arange(5000, 5350)])
    sub = dict(case, T=rows.size, hidden=case["hidden"][rows], targets=case["targets"][rows],
               mask=case["mask"][rows])
    b = run_forward(llp, sub)
    for k in ("logp", "entropy", "lse", "target_logit", "in_range"):
        np.testing.assert_array_equal(host(a[k])[rows].view(np.uint8), host(b[k]).view(np.uint8),
                                      err_msg=k)
    pick = np.unique(np.concatenate([rows[::37], np.arange(4608, 5700, 97)]))
    ref = oracle.forward(case["hidden"][pick], case["weight"], case["bias"], tau,
                         case["targets"][pick], case["mask"][pick], Vr)
    check_forward({k: a[k][torch.from_numpy(pick).cuda()] for k in ("logp", "entropy", "lse",
                                                                    "in_range")},
                  ref, case["mask"][pick], "batch size")


@pytest.mark.parametrize("T", [16385, 3 * 16384 + 1234])
def test_layout_scan_over_several_blocks_bitwise(llp, T):
    """Beyond 16384 rows the layout scan takes one workgroup per 16384-row block, each block's
    compact indices following the scored rows counted in the blocks before it. With masked
    and scored runs that cross the block edges, the forward outputs and the dhidden rows are
    bitwise those of the same rows in calls of at most 16384 rows (one workgroup), the status
    word stays clear, and rows at the block edges match the oracle."""
    H, Vr, Vp, tau = 64, 700, 768, 0.7
    case = synth.small_case(T, H, Vr, Vp, tau, case_id=90 + T % 7, mask_frac=0.3, w_std=0.05)
    mask = case["mask"].copy()
    mask[16000:16384 + 300] = 0                  # masked across the first block edge
    mask[min(T, 32000):min(T, 33500)] = 1        # scored across the second
    case = dict(case, mask=mask)
    say(f"layout scan: T={T} ({-(-T // 16384)} blocks), {int(mask.sum())} scored rows")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    a = run_forward(llp, case, status=st)
    assert int(st.item()) == 0
    cuts = sorted({c for c in (0, 7000, 16384, 16385, 30000, 40000) if c < T} | {T})
    dl = synth.rng(90, 1).standard_normal(T).astype(np.float32) * mask
    dH = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    dW = torch.empty((Vp, H), dtype=torch.float32, device="cuda")
    run_backward(llp, case, host(a["lse"]), dl, dhidden=dH, dweight=dW, overwrite=True)
    dH_all = host(dH.float())
    for c0, c1 in zip(cuts[:-1], cuts[1:]):
        sub = dict(case, T=c1 - c0, hidden=case["hidden"][c0:c1], targets=case["targets"][c0:c1],
                   mask=case["mask"][c0:c1])
        b = run_forward(llp, sub)
        for k in ("logp", "entropy", "lse", "target_logit", "in_range"):
            np.testing.assert_array_equal(host(a[k])[c0:c1].view(np.uint8),
                                          host(b[k]).view(np.uint8), err_msg=f"{k} rows {c0}:{c1}")
        dHs = torch.empty((c1 - c0, H), dtype=torch.bfloat16, device="cuda")
        run_backward(llp, sub, host(b["lse"]), dl[c0:c1], dhidden=dHs, dweight=dW, overwrite=True)
        np.testing.assert_array_equal(dH_all[c0:c1], host(dHs.float()), err_msg=f"dH {c0}:{c1}")
    pick = np.unique([r for r in (0, 16383, 16384, 16385, 32767, 32768, 49151, 49152, T - 1)
                      if r < T])
    ref = oracle.forward(case["hidden"][pick], case["weight"], None, tau, case["targets"][pick],
                         mask[pick], Vr)
    check_forward({k: a[k][torch.from_numpy(pick).cuda()] for k in ("logp", "entropy", "lse",
                                                                    "in_range")},
                  ref, mask[pick], f"layout T={T}")


def test_row_strides_wider_than_H_bitwise(llp):
    """hidden, weight, dhidden and dweight given as views into wider row-major buffers (row
    strides H + 72, H + 136, H + 40 and H + 12 elements). The padding columns of the inputs
    hold 1e4, so reading any of them would change every result; the outputs' padding holds a
    sentinel that must come back untouched. Forward outputs, dhidden and dweight are bitwise
    those of contiguous tensors."""
    T, H, Vr, Vp, tau = 300, 256, 1000, 1024, 0.7
    case = synth.small_case(T, H, Vr, Vp, tau, case_id=77, mask_frac=0.2, with_bias=True,
                            w_std=0.05)
    say("row strides wider than H: forward and backward on views")
    h, W = dev_bf16(case["hidden"]), dev_bf16(case["weight"])
    hw = torch.full((T, H + 72), 1e4, dtype=torch.bfloat16, device="cuda")
    ww = torch.full((Vp, H + 136), 1e4, dtype=torch.bfloat16, device="cuda")
    hw[:, :H] = h
    ww[:, :H] = W
    hv, wv = hw[:, :H], ww[:, :H]
    assert hv.stride(0) == H + 72 and wv.stride(0) == H + 136
    kw = dict(temperature=tau, bias=dev_bf16(case["bias"]), loss_mask=dev(case["mask"]),
              real_vocab=Vr, padded_vocab=Vp)
    tg = dev(case["targets"])
    a = llp.forward(h, W, tg, **kw)
    b = llp.forward(hv, wv, tg, **kw)
    torch.cuda.synchronize()
    for k in ("logp", "entropy", "lse", "target_logit", "in_range"):
        assert bytes_equal(a[k], b[k]), k
    dl = dev(synth.rng(77, 3).standard_normal(T).astype(np.float32), torch.float32)
    dH = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    dW = torch.empty((Vp, H), dtype=torch.float32, device="cuda")
    llp.backward(h, W, tg, a["lse"], dl, dhidden=dH, dweight=dW, overwrite=True, **kw)
    dHw = torch.full((T, H + 40), -7.0, dtype=torch.bfloat16, device="cuda")
    dWw = torch.full((Vp, H + 12), float("nan"), dtype=torch.float32, device="cuda")
    llp.backward(hv, wv, tg, b["lse"], dl, dhidden=dHw[:, :H], dweight=dWw[:, :H],
                 overwrite=True, **kw)
    torch.cuda.synchronize()
    assert bytes_equal(dH, dHw[:, :H].contiguous()) and bytes_equal(dW, dWw[:, :H].contiguous())
    assert torch.all(dHw[:, H:] == -7.0) and torch.all(torch.isnan(dWw[:, H:]))
    ref = oracle.forward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                         case["mask"], Vr)
    check_forward(b, ref, case["mask"], "strided views")


def test_layout_scan_past_64_blocks_bitwise(llp):
    """Past 64 layout blocks (T > 64 * 16384 rows) each workgroup's count of the scored rows
    before it is summed by the 64 lanes of a wave in strides. 1,065,037 rows (66 blocks) with
    a small projection: the forward outputs are bitwise those of separate calls over row
    ranges around the 64-block edge and at the tail, and the status word stays clear."""
    T, H, Vr, Vp, tau = 65 * 16384 + 77, 64, 200, 256, 0.7
    case = synth.small_case(T, H, Vr, Vp, tau, case_id=95, mask_frac=0.4, w_std=0.05)
    say(f"layout scan past 64 blocks: T={T}, {int(case['mask'].sum())} scored rows")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    a = run_forward(llp, case, status=st)
    assert int(st.item()) == 0
    for c0, c1 in ((0, 9000), (64 * 16384 - 5000, 64 * 16384 + 5000), (T - 12000, T)):
        sub = dict(case, T=c1 - c0, hidden=case["hidden"][c0:c1], targets=case["targets"][c0:c1],
                   mask=case["mask"][c0:c1])
        b = run_forward(llp, sub)
        for k in ("logp", "entropy", "lse", "target_logit", "in_range"):
            np.testing.assert_array_equal(host(a[k])[c0:c1].view(np.uint8),
                                          host(b[k]).view(np.uint8), err_msg=f"{k} rows {c0}:{c1}")
    m = case["mask"].astype(bool)
    assert np.all(host(a["logp"])[~m] == 0) and np.all(host(a["in_range"])[m] == 1)
