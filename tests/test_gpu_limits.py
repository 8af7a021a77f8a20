"""GPU parity at the largest sizes the C ABI accepts, where 32-bit address arithmetic would
break first.

- The fused forward and backward gather scored hidden rows through one buffer resource per tile
  with 32-bit byte offsets from the tile's first scored row, so the host refuses hidden rows
  that span 2^31 bytes or more. Here T * H * 2 is one row short of 2^31 bytes (T = 2^22 - 1,
  H = 256). 300 rows are scored, including the first and the last row. The first token block
  therefore spans almost the whole range, and the last one ends at the final row. Every
  unscored row holds NaN, so a load of a wrong row would show in the results.
- A shard's local vocabulary may hold up to 2^23 - 256 columns. At that width the dhidden
  product's buffer resource over 256 rows of G (all of its K range) just fits in 32 bits: it
  ends 131088 bytes short of 2^32. Here the shard has exactly that width (H = 128, an fp32 bias,
  the last 100 columns padding), and it is checked against the oracle evaluated window by
  window.
- The hidden size may be up to 2^20. At that size a tile's K loop runs 16384 steps, the
  dhidden and dweight products span 4096 column tiles, and a dweight tile's rows are 4 MiB
  apart. Here H = 2^20, with a bf16 bias and a ragged second vocabulary tile.
- The merge takes up to 64 shards. Here 64 shards of seeded, uneven widths (some empty, some
  padding only) are merged and compared with the unsharded oracle. Their backward calls with
  the merged lse assemble the unsharded gradients.
- The logits-input forward, the compact top-p replay and the dense keep-mask replay address a
  row of logits with 64-bit arithmetic. Here the logits exceed 2^32 bytes (fp32 and bf16), so
  the last rows lie past any 32-bit byte offset.

Inputs come from the seeded generators and are tiled on the device. Sampled rows, including the
first and the last ones, are compared with the oracle; the rest are checked through properties
that hold at any size (zero outputs of unscored rows; dense replay bitwise equal to compact)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from lm_head_linear_logp_amd import _capi as A
from tests._gpu import (GRAD_GUARD, GRAD_RTOL, LOGP_ATOL, LOGP_GUARD, assert_rows_close, dev,
                        dev_bf16, host, need_gpu, normwise_rel, record, say)

pytestmark = pytest.mark.gpu

BF16_NAN = 0x7FC0


@pytest.fixture(scope="module")
def llp():
    need_gpu()
    import lm_head_linear_logp_amd as m
    m.open(0)
    return m


def test_fused_forward_backward_at_the_hidden_span_limit(llp):
    H, Vr, Vp, tau, NS = 256, 1000, 1024, 0.7, 300
    T = (1 << 31) // (2 * H) - 1                      # T * H * 2 = 2^31 - 512 bytes
    case = synth.small_case(NS, H, Vr, Vp, tau, case_id=80, w_std=0.1)
    g = synth.rng(1080, 9)
    rows = np.sort(np.concatenate([[0, T - 1], g.choice(np.arange(1, T - 1), NS - 2,
                                                         replace=False)]))
    say(f"hidden span limit: T={T} H={H} ({T * H * 2} bytes), {NS} scored rows")
    rows_d = dev(rows)
    hidden = torch.full((T, H), BF16_NAN, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    hidden[rows_d] = dev_bf16(case["hidden"])
    weight = dev_bf16(case["weight"])
    tg = torch.zeros(T, dtype=torch.int64, device="cuda")
    tg[rows_d] = dev(case["targets"])
    mask = torch.zeros(T, dtype=torch.uint8, device="cuda")
    mask[rows_d] = 1
    unscored = mask == 0

    out = llp.forward(hidden, weight, tg, temperature=tau, loss_mask=mask, real_vocab=Vr,
                      padded_vocab=Vp)
    torch.cuda.synchronize()
    f = oracle.forward(case["hidden"], case["weight"], None, tau, case["targets"], None, Vr)
    err = 0.0
    for k in ("logp", "entropy", "lse"):
        err = max(err, assert_rows_close(host(out[k][rows_d]), f[k], LOGP_ATOL, f"limit {k}"))
        assert not bool(torch.any(out[k][unscored] != 0)), f"unscored rows of {k} are not 0"
    np.testing.assert_array_equal(host(out["in_range"][rows_d]), f["in_range"])
    record("hidden span limit: forward max |d|", err)
    assert err <= LOGP_GUARD

    dlogp = g.standard_normal(NS)
    lse = torch.zeros(T, dtype=torch.float32, device="cuda")
    lse[rows_d] = dev(f["lse"], torch.float32)
    dl = torch.zeros(T, dtype=torch.float32, device="cuda")
    dl[rows_d] = dev(dlogp, torch.float32)
    b = llp.backward(hidden, weight, tg, lse, dl, temperature=tau, loss_mask=mask,
                     real_vocab=Vr, padded_vocab=Vp, overwrite=True)
    torch.cuda.synchronize()
    ref = oracle.backward(case["hidden"], case["weight"], None, tau, case["targets"], None, 0,
                          Vp, Vr, f["lse"], dlogp)
    r1 = normwise_rel(oracle.bf16_to_f64(host(b["dhidden"][rows_d])), ref["dhidden"])
    r2 = normwise_rel(host(b["dweight"]), ref["dweight"])
    record("hidden span limit: dhidden normwise", r1)
    record("hidden span limit: dweight normwise", r2)
    assert r1 <= GRAD_RTOL and r2 <= GRAD_RTOL
    assert r1 <= GRAD_GUARD and r2 <= GRAD_GUARD
    dh_bits = b["dhidden"].view(torch.int16)
    assert not bool(torch.any(dh_bits[unscored] != 0)), "unscored dhidden rows are not 0"
    assert not bool(torch.any(b["dweight"][Vr:] != 0)), "padded dweight rows are not 0"


def test_vocabulary_at_the_local_size_limit(llp):
    Vp = (1 << 23) - 256                               # local_size = padded vocabulary
    Vr, H, T, tau, P = Vp - 100, 128, 8, 0.7, 65521
    # Weight and bias rows repeat with a prime period: a row read from a wrapped 32-bit
    # offset (a multiple of 2^24 rows away) would hold other values.
    g = synth.rng(1082, 1)
    wb = synth.normal_bf16(g, (P, H), 0.1)
    bb = (g.standard_normal(P) * 0.5).astype(np.float32)
    hid = synth.normal_bf16(g, (T, H), 1.0)
    tg = np.concatenate([[0, Vr - 1, Vp - 101 - 7, P, 2 * P + 5],
                         g.integers(0, Vr, T - 5)]).astype(np.int64)
    say(f"local size limit: V={Vp} ({Vr} real) H={H} T={T}")
    idx_d = dev(np.arange(Vp, dtype=np.int64) % P)
    W = dev_bf16(wb)[idx_d]
    bias = dev(bb)[idx_d]
    out = llp.forward(dev_bf16(hid), W, dev(tg), temperature=tau, bias=bias, real_vocab=Vr,
                      padded_vocab=Vp)
    torch.cuda.synchronize()

    # The oracle over windows of the vocabulary (shards of one call), merged in order.
    step = 1 << 20
    wins = [(lo, min(lo + step, Vp)) for lo in range(0, Vp, step)]
    rows_of = lambda lo, hi: np.arange(lo, hi) % P
    parts = [oracle.shard_forward(hid, wb[rows_of(lo, hi)], bb[rows_of(lo, hi)], tau, tg, None,
                                  lo, hi - lo, Vr) for lo, hi in wins]
    f = oracle.merge(parts)
    err = 0.0
    for k in ("logp", "entropy", "lse"):
        err = max(err, assert_rows_close(host(out[k]), f[k], LOGP_ATOL, f"local size limit {k}"))
    record("local size limit: forward max |d|", err)
    assert err <= LOGP_GUARD

    dlogp = g.standard_normal(T)
    b = llp.backward(dev_bf16(hid), W, dev(tg), dev(f["lse"], torch.float32),
                     dev(dlogp, torch.float32), temperature=tau, bias=bias, real_vocab=Vr,
                     padded_vocab=Vp, overwrite=True)
    torch.cuda.synchronize()
    dH = np.zeros((T, H))
    checked = {0, len(wins) // 2, len(wins) - 1}
    for i, (lo, hi) in enumerate(wins):
        r = rows_of(lo, hi)
        ref = oracle.backward(hid, wb[r], bb[r], tau, tg, None, lo, hi - lo, Vr, f["lse"], dlogp)
        dH += ref["dhidden"]
        if i in checked:
            rw = normwise_rel(host(b["dweight"][lo:hi]), ref["dweight"])
            rb = normwise_rel(host(b["dbias"][lo:hi]), ref["dbias"])
            record(f"local size limit: dweight rows [{lo}, {hi}) normwise", rw)
            record(f"local size limit: dbias [{lo}, {hi}) normwise", rb)
            assert rw <= GRAD_GUARD and rb <= GRAD_GUARD
    rh = normwise_rel(oracle.bf16_to_f64(host(b["dhidden"])), dH)
    record("local size limit: dhidden normwise", rh)
    assert rh <= GRAD_GUARD
    assert not bool(torch.any(b["dweight"][Vr:] != 0)), "padded dweight rows are not 0"
    assert not bool(torch.any(b["dbias"][Vr:] != 0)), "padded dbias entries are not 0"


def test_hidden_size_at_its_limit(llp):
    H, T, Vr, Vp, tau = 1 << 20, 8, 300, 320, 0.7
    case = synth.small_case(T, H, Vr, Vp, tau, case_id=83, mask_frac=0.2, with_bias=True,
                            w_std=0.002)
    say(f"hidden size limit: H={H} T={T} V={Vr}/{Vp}")
    hid, W, bias = dev_bf16(case["hidden"]), dev_bf16(case["weight"]), dev_bf16(case["bias"])
    tg, mask = dev(case["targets"]), dev(case["mask"])
    out = llp.forward(hid, W, tg, temperature=tau, bias=bias, loss_mask=mask, real_vocab=Vr,
                      padded_vocab=Vp)
    torch.cuda.synchronize()
    f = oracle.forward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                       case["mask"], Vr)
    err = 0.0
    for k in ("logp", "entropy", "lse"):
        err = max(err, assert_rows_close(host(out[k]), f[k], LOGP_ATOL, f"hidden size limit {k}"))
    record("hidden size limit: forward max |d|", err)
    assert err <= LOGP_GUARD        # observed 5.5e-5: fp32 sums of 2^20 products

    dlogp = synth.rng(1083, 5).standard_normal(T) * case["mask"]
    b = llp.backward(hid, W, tg, dev(f["lse"], torch.float32), dev(dlogp, torch.float32),
                     temperature=tau, bias=bias, loss_mask=mask, real_vocab=Vr, padded_vocab=Vp,
                     overwrite=True)
    torch.cuda.synchronize()
    ref = oracle.backward(case["hidden"], case["weight"], case["bias"], tau, case["targets"],
                          case["mask"], 0, Vp, Vr, f["lse"], dlogp)
    dH = oracle.bf16_to_f64(host(b["dhidden"]))
    r1 = normwise_rel(dH, ref["dhidden"])
    r2 = normwise_rel(host(b["dweight"]), ref["dweight"])
    r3 = normwise_rel(host(b["dbias"]), ref["dbias"])
    for name, v in (("dhidden", r1), ("dweight", r2), ("dbias", r3)):
        record(f"hidden size limit: {name} normwise", v)
        assert v <= GRAD_GUARD
    assert np.all(dH[case["mask"] == 0] == 0)
    assert not bool(torch.any(b["dweight"][Vr:] != 0)), "padded dweight rows are not 0"


def test_merge_of_the_largest_world(llp):
    world = A.LLP_MAX_WORLD
    T, H, Vr, Vp, tau = 300, 128, 16000, 16384, 0.7
    case = synth.small_case(T, H, Vr, Vp, tau, case_id=84, mask_frac=0.2, w_std=0.1)
    g = synth.rng(1084, 1)
    # Seeded cut points, plus an empty shard at 5000 and a shard of padding only.
    cuts = np.concatenate([[0], g.choice(Vp + 1, world - 5, replace=True),
                           [5000, 5000, Vr, Vr + 100, Vp]])
    cuts.sort()
    widths = np.diff(cuts)
    say(f"merge of {world} shards: {int((widths == 0).sum())} empty, widths up to {widths.max()}")
    hid, tg, mk = dev_bf16(case["hidden"]), dev(case["targets"]), dev(case["mask"])
    W = dev_bf16(case["weight"])
    kw = dict(temperature=tau, loss_mask=mk, real_vocab=Vr, padded_vocab=Vp, world=world)
    parts = [llp.forward(hid, W[lo:hi], tg, offset=int(lo), rank=r, **kw)
             for r, (lo, hi) in enumerate(zip(cuts[:-1], cuts[1:]))]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    mg = llp.merge(parts, loss_mask=mk, status=st)
    torch.cuda.synchronize()
    ref = oracle.forward(case["hidden"], case["weight"], None, tau, case["targets"], case["mask"],
                         Vr)
    err = 0.0
    for k in ("logp", "lse", "entropy"):
        err = max(err, assert_rows_close(host(mg[k]), ref[k], LOGP_ATOL, f"merged {k}"))
    assert int(st.item()) == 0
    record(f"merge of {world} shards: max |d|", err)
    assert err <= LOGP_GUARD

    dlogp = g.standard_normal(T) * case["mask"]
    lse_d, dl_d = dev(ref["lse"], torch.float32), dev(dlogp, torch.float32)
    dW = torch.empty((Vp, H), dtype=torch.float32, device="cuda")
    dH = np.zeros((T, H))
    for r, (lo, hi) in enumerate(zip(cuts[:-1], cuts[1:])):
        b = llp.backward(hid, W[lo:hi], tg, lse_d, dl_d, offset=int(lo), rank=r,
                         dweight=dW[lo:hi], overwrite=True, **kw)
        dH += oracle.bf16_to_f64(host(b["dhidden"]))
    torch.cuda.synchronize()
    gref = oracle.backward(case["hidden"], case["weight"], None, tau, case["targets"],
                           case["mask"], 0, Vp, Vr, ref["lse"], dlogp)
    r1 = normwise_rel(dH, gref["dhidden"])
    r2 = normwise_rel(host(dW), gref["dweight"])
    record(f"{world} shards: summed dhidden normwise", r1)
    record(f"{world} shards: assembled dweight normwise", r2)
    assert r1 <= GRAD_RTOL and r2 <= GRAD_GUARD


REPLAY_LIMIT = [  # logits dtype, rows (T * 151936 * element size > 2^32 bytes)
    (torch.float32, 8197),
    (torch.bfloat16, 16389),
]


@pytest.mark.parametrize("dtype,T", REPLAY_LIMIT, ids=["f32", "bf16"])
def test_logits_input_paths_past_4gib(llp, dtype, T):
    Vr, Vp, tau, NB = synth.V_REAL_FULL, synth.V_PAD_FULL, 0.7, 16
    esize = 4 if dtype == torch.float32 else 2
    assert (T - 1) * Vp * esize > (1 << 32)
    g = synth.rng(1081, 1 if dtype == torch.float32 else 2)
    base = (g.standard_normal((NB, Vp)) * 2.0).astype(np.float32)
    base[:, Vr:] = np.float32(1e30)                    # padded columns: never part of a row
    ids = np.full((NB, 64), -1, dtype=np.int64)
    keep = np.zeros((NB, Vp), dtype=np.uint8)
    member = np.zeros(NB, dtype=np.int64)
    for r in range(NB):
        u = g.choice(Vr, 1 + r, replace=False)          # 1..16 distinct ids per row
        ids[r, g.choice(64, u.size, replace=False)] = u
        keep[r, u] = 1
        member[r] = u[0]
    idx = np.arange(T) % NB
    # Half the targets lie in their row's nucleus, the others anywhere in the real vocabulary.
    tg = np.where(g.random(T) < 0.5, member[idx], g.integers(0, Vr, T)).astype(np.int64)
    mask = (g.random(T) >= 0.1).astype(np.uint8)
    mask[[0, T - 1]] = 1
    say(f"logits past 4 GiB: T={T} {dtype} ({T * Vp * esize} bytes)")

    bd = dev(base)
    if dtype == torch.bfloat16:
        bd = bd.to(torch.bfloat16)
    vals = bd.float().cpu().numpy().astype(np.float64)  # the exact values the kernels read
    idx_d = dev(idx)
    X = bd[idx_d]
    K = dev(keep)[idx_d]
    I, G, M = dev(ids[idx]), dev(tg), dev(mask)
    kw = dict(temperature=tau, real_vocab=Vr, padded_vocab=Vp, loss_mask=M)
    fl = llp.forward_logits(X, G, want_entropy=True, **kw)
    tp = llp.top_p_replay(X, I, G, **kw)
    km = llp.keep_mask_replay(X, K, G, **kw)
    torch.cuda.synchronize()

    for k in ("target_logit", "in_range", "lse", "logp"):
        assert torch.equal(tp[k], km[k]), f"dense and compact replay differ in {k}"
    rows = np.unique(np.concatenate([[0, 1, 2, T - 3, T - 2, T - 1],
                                     g.integers(0, T, 20)]))
    rf = oracle.logits_forward(vals[idx[rows]], tg[rows], tau, 0, Vp, Vr, mask[rows])
    rt = oracle.top_p_replay(vals[idx[rows]], ids[idx[rows]], tg[rows], tau, 0, Vp, Vr,
                             mask[rows])
    err = 0.0
    for k in ("lse", "logp", "entropy"):
        err = max(err, assert_rows_close(host(fl[k])[rows], rf[k], LOGP_ATOL, f"logits {k}"))
    for k in ("lse", "logp"):
        err = max(err, assert_rows_close(host(tp[k])[rows], rt[k], LOGP_ATOL, f"top-p {k}"))
    np.testing.assert_array_equal(host(fl["in_range"])[rows], rf["in_range"])
    np.testing.assert_array_equal(host(tp["in_range"])[rows], rt["in_range"])
    record(f"logits past 4 GiB ({str(dtype)[6:]}): max |d|", err)
    assert err <= LOGP_GUARD
