"""GPU parity of the logits-input forward and the dense keep-mask replay, through the C ABI:
against the oracle at small and full sizes, bitwise determinism and row invariance, shards and
empty shards, and bitwise equality of the dense keep-mask and compact replay scorers."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import LOGP_ATOL, assert_rows_close, bytes_equal, dev, host, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def llp():
    need_gpu()
    import lm_head_linear_logp_amd as m
    m.open(0)
    return m


def logits_case(T, V, Vp, seed, mask_frac=0.0):
    g = synth.rng(seed, 60)
    x = (g.standard_normal((T, Vp)) * 2.0).astype(np.float32)
    x[:, V:] = np.float32(1e30)                      # padded columns: must never be read in
    spikes = g.integers(0, V, size=(T, 3))
    for r in range(T):
        x[r, spikes[r]] = 14.0 + 4.0 * g.random(3)
    tg = np.where(g.random(T) < 0.6, spikes[:, 0], g.integers(0, V, T)).astype(np.int64)
    mask = (g.random(T) >= mask_frac).astype(np.uint8)
    return x, tg, mask


def as_dtype(x, dtype):
    """The device tensor and the exact values the kernel sees."""
    t = dev(x)
    if dtype == torch.bfloat16:
        t = t.to(torch.bfloat16)
        return t, t.float().cpu().numpy().astype(np.float64)
    return t, x.astype(np.float64)


SHAPES = [  # T, V_real, V_pad, tau, mask_frac, dtype, entropy
    (300, 1000, 1024, 0.7, 0.3, torch.float32, True),
    (257, 513, 520, 1.3, 0.0, torch.bfloat16, True),
    (1, 7, 8, 0.5, 0.0, torch.float32, False),
    (64, 2049, 2304, 0.7, 0.5, torch.bfloat16, False),
    (33, 8200, 8200, 1.0, 0.0, torch.float32, True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"T{s[0]}_V{s[1]}_{str(s[5])[6:]}" for s in SHAPES])
def test_logits_forward_parity(llp, shape):
    T, V, Vp, tau, mf, dt, ent = shape
    x, tg, mask = logits_case(T, V, Vp, seed=70 + T, mask_frac=mf)
    xt, xv = as_dtype(x, dt)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = llp.forward_logits(xt, dev(tg), temperature=tau, loss_mask=dev(mask), real_vocab=V,
                             padded_vocab=Vp, want_entropy=ent, status=st)
    torch.cuda.synchronize()
    ref = oracle.logits_forward(xv, tg, tau, 0, Vp, V, mask)
    e = assert_rows_close(host(out["logp"]), ref["logp"], LOGP_ATOL, "logp")
    assert_rows_close(host(out["lse"]), ref["lse"], LOGP_ATOL, "lse")
    if ent:
        assert_rows_close(host(out["entropy"]), ref["entropy"], LOGP_ATOL, "entropy")
    np.testing.assert_array_equal(host(out["in_range"]), ref["in_range"])
    m = mask.astype(bool)
    assert np.all(host(out["logp"])[~m] == 0) and np.all(host(out["lse"])[~m] == 0)
    assert int(st.item()) == ref["status"]
    say(f"logits forward {shape}: max err logp {e:.2e}")


def test_logits_forward_shards_merge_and_empty(llp):
    T, V, Vp = 200, 3000, 3072
    x, tg, mask = logits_case(T, V, Vp, seed=81, mask_frac=0.2)
    xt = dev(x)
    cuts = [0, 1024, 2048, 3072]
    parts = []
    for r, (lo, hi) in enumerate(zip(cuts[:-1], cuts[1:])):
        parts.append(llp.forward_logits(xt[:, lo:hi], dev(tg), temperature=0.7,
                                        loss_mask=dev(mask), offset=lo, real_vocab=V,
                                        padded_vocab=4096, rank=r, world=4, local_size=hi - lo))
    empty = llp.forward_logits(xt[:, :0], dev(tg), temperature=0.7, loss_mask=dev(mask),
                               offset=3072, real_vocab=V, padded_vocab=4096, rank=3, world=4,
                               local_size=1024)
    torch.cuda.synchronize()
    m = mask.astype(bool)
    assert np.all(host(empty["lse"])[m] == -np.inf) and np.all(host(empty["entropy"]) == 0)
    assert np.all(host(empty["logp"])[m] == -np.inf) and not np.any(host(empty["in_range"]))
    mg = llp.merge(parts + [empty], loss_mask=dev(mask))
    torch.cuda.synchronize()
    ref = oracle.logits_forward(x, tg, 0.7, 0, Vp, V, mask)
    assert_rows_close(host(mg["logp"]), ref["logp"], LOGP_ATOL, "merged logp")
    assert_rows_close(host(mg["entropy"]), ref["entropy"], LOGP_ATOL, "merged entropy")


def test_logits_forward_bitwise_repeat_and_row_invariance(llp):
    T, V = 96, 5000
    x, tg, _ = logits_case(T, V, V, seed=82)
    xt, tgt = dev(x), dev(tg)
    a = llp.forward_logits(xt, tgt, temperature=0.7)
    b = llp.forward_logits(xt, tgt, temperature=0.7)
    sub = torch.arange(T - 1, -1, -3, device="cuda")            # other rows, other order
    c = llp.forward_logits(xt[sub].contiguous(), tgt[sub].contiguous(), temperature=0.7)
    torch.cuda.synchronize()
    for k in ("lse", "logp", "entropy", "target_logit"):
        assert bytes_equal(a[k], b[k]), k
        assert torch.equal(a[k][sub], c[k]), k


def test_logits_forward_matches_fused_forward(llp):
    """The projection's logits fed back through the logits path give the fused result."""
    case = synth.small_case(T=128, H=256, real_vocab=1000, padded_vocab=1024, temperature=0.7,
                            case_id=83)
    from tests._gpu import dev_bf16
    h, W = dev_bf16(case["hidden"]), dev_bf16(case["weight"])
    fused = llp.forward(h, W, dev(case["targets"]), temperature=0.7, real_vocab=1000,
                        padded_vocab=1024)
    logits = (h.float() @ W.float().t()).contiguous()
    lo = llp.forward_logits(logits, dev(case["targets"]), temperature=0.7, real_vocab=1000,
                            padded_vocab=1024)
    torch.cuda.synchronize()
    for k in ("lse", "logp", "entropy"):
        assert_rows_close(host(lo[k]), host(fused[k]), 1e-4, k)


def test_logits_forward_status_bits(llp):
    x, tg, _ = logits_case(8, 100, 128, seed=84)
    tg[1] = 100                          # a padded id
    tg[2] = -5
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = llp.forward_logits(dev(x), dev(tg), temperature=1.0, real_vocab=100, padded_vocab=128,
                             status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == (llp.STATUS_BITS["TARGET_OUT_OF_RANGE"] |
                              llp.STATUS_BITS["TARGET_NOT_FOUND"])
    lp = host(out["logp"])
    assert lp[1] == -np.inf and lp[2] == -np.inf and np.all(np.isfinite(lp[3:]))


# ------------------------------------------------------------------ dense keep-mask replay

def dense_mask(ids, Vp):
    T = ids.shape[0]
    km = np.zeros((T, Vp), dtype=np.uint8)
    for t in range(T):
        v = ids[t][ids[t] >= 0]
        km[t, v] = 1
    return km


def topp_small(T=300, V=600, Vp=640, seed=90):
    g = synth.rng(seed, 61)
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


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_keep_mask_equals_compact_bitwise(llp, dtype):
    """[top-p replay, "Validation"]: dense mask vs compact ids, bitwise, across shard offsets
    (including a shard with no candidates in many rows and an empty shard)."""
    x, ids, tg = topp_small()
    km = dense_mask(ids, 640)
    xt, kt = dev(x).to(dtype), dev(km)
    mask = (synth.rng(91, 1).random(x.shape[0]) > 0.1).astype(np.uint8)
    for lo, hi in ((0, 640), (0, 160), (160, 320), (320, 480), (480, 640), (608, 640)):
        kw = dict(temperature=0.7, offset=lo, real_vocab=600, padded_vocab=640,
                  world=1 if (lo, hi) == (0, 640) else 4, local_size=hi - lo,
                  loss_mask=dev(mask))
        a = llp.keep_mask_replay(xt[:, lo:hi], kt[:, lo:hi], dev(tg), **kw)
        b = llp.top_p_replay(xt[:, lo:hi], dev(ids), dev(tg), **kw)
        torch.cuda.synchronize()
        for k in ("target_logit", "in_range", "lse", "logp"):
            assert torch.equal(a[k], b[k]), (lo, hi, k)
    ref = oracle.keep_mask_replay(x.astype(np.float64) if dtype == torch.float32 else
                                  xt.float().cpu().numpy().astype(np.float64), km, tg, 0.7, 0,
                                  640, 600, mask)
    out = llp.keep_mask_replay(xt, kt, dev(tg), temperature=0.7, real_vocab=600,
                               padded_vocab=640, loss_mask=dev(mask))
    torch.cuda.synchronize()
    assert_rows_close(host(out["lse"]), ref["lse"], LOGP_ATOL, "keep lse")
    assert_rows_close(host(out["logp"]), ref["logp"], LOGP_ATOL, "keep logp")


def test_keep_mask_large_nucleus_and_edges(llp):
    """Kept sets beyond 64 ids (no compact form), empty rows and masked rows."""
    T, V, Vp = 64, 3000, 3072
    g = synth.rng(92, 1)
    x = (g.standard_normal((T, Vp)) * 2.0).astype(np.float32)
    km = (g.random((T, Vp)) < np.linspace(0.0, 0.9, T)[:, None]).astype(np.uint8)
    km[:, V:] = 1                         # padded columns are ignored even when kept
    tg = g.integers(0, V, T)
    mask = np.ones(T, np.uint8)
    mask[5] = 0
    out = llp.keep_mask_replay(dev(x), dev(km), dev(tg), temperature=0.7, real_vocab=V,
                               padded_vocab=Vp, loss_mask=dev(mask))
    torch.cuda.synchronize()
    ref = oracle.keep_mask_replay(x, km, tg, 0.7, 0, Vp, V, mask)
    assert_rows_close(host(out["lse"]), ref["lse"], LOGP_ATOL, "lse")
    assert_rows_close(host(out["logp"]), ref["logp"], LOGP_ATOL, "logp")
    np.testing.assert_array_equal(host(out["in_range"]), ref["in_range"])
    assert host(out["lse"])[0] == -np.inf          # row 0 keeps nothing
    assert host(out["lse"])[5] == 0 and host(out["logp"])[5] == 0


@pytest.mark.slow
def test_config5_logits_forward_and_keep_mask_full(llp):
    """Full size: config-5 logits [4096, 151936] fp32 (2.49 GB): the logits-input forward on
    sampled rows against the oracle, and the dense keep mask against the compact scorer,
    bitwise, over the four shards."""
    say("config5 full: logits forward + dense keep mask, T=4096 V=151936")
    c = synth.topp_case()
    x = c["logits"]
    xt = dev(x)
    tg, ids = dev(c["targets"]), dev(c["replay_ids"])
    out = llp.forward_logits(xt, tg, temperature=0.7, real_vocab=151669, padded_vocab=151936)
    torch.cuda.synchronize()
    rows = synth.rng(93, 1).choice(4096, size=48, replace=False)
    ref = oracle.logits_forward(x[rows], c["targets"][rows], 0.7, 0, 151936, 151669)
    for k in ("lse", "logp", "entropy"):
        assert_rows_close(host(out[k])[rows], ref[k], LOGP_ATOL, f"config5 logits {k}")
    km = torch.zeros((4096, 151936), dtype=torch.uint8, device="cuda")
    valid = ids >= 0
    km[torch.arange(4096, device="cuda")[:, None].expand_as(ids)[valid], ids[valid]] = 1
    for r in range(4):
        lo, hi = 37984 * r, 37984 * (r + 1)
        kw = dict(temperature=0.7, offset=lo, real_vocab=151669, padded_vocab=151936, rank=r,
                  world=4, local_size=hi - lo)
        a = llp.keep_mask_replay(xt[:, lo:hi], km[:, lo:hi], tg, **kw)
        b = llp.top_p_replay(xt[:, lo:hi], ids, tg, **kw)
        torch.cuda.synchronize()
        for k in ("target_logit", "in_range", "lse", "logp"):
            assert torch.equal(a[k], b[k]), (r, k)
    say("config5 full: dense keep mask == compact scorer bitwise on 4 shards")


def test_topp_row_position_invariance_bitwise(llp):
    """A wave scores 4 rows at once, 16 lanes each, and falls back to the whole wave for a
    row whose shard holds more than 16 of its ids. Every row gets the same bits wherever it
    lands: the same rows scored in calls that start at other rows (so each row sits in another
    lane group and wave), with a ragged T, equal the dense keep-mask scorer bit for bit, and
    sampled rows match the oracle. Rows of up to 40 distinct ids (the full-vocabulary call
    takes the fallback), masked rows, empty rows and an invalid id are included, over a
    full-vocabulary call and a shard."""
    x, ids, tg = topp_small()
    T = 65536 + 13
    idx = np.arange(T) % x.shape[0]
    X, I, G = dev(x[idx]), ids[idx].copy(), tg[idx]
    I[7, 2] = 640                          # padded id: invalid, ignored
    I[11] = -1                             # empty row
    km = dense_mask(np.where(I >= 600, -1, I), 640)
    mask = (synth.rng(93, 1).random(T) > 0.1).astype(np.uint8)
    Id, Gd, Md, Kd = dev(I), dev(G), dev(mask), dev(km)
    for lo, hi in ((0, 640), (160, 320)):
        say(f"topp rows-per-wave paths, columns [{lo}, {hi})")
        kw = dict(temperature=0.7, offset=lo, real_vocab=600, padded_vocab=640,
                  world=1 if (lo, hi) == (0, 640) else 4, local_size=hi - lo)
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        big = llp.top_p_replay(X[:, lo:hi], Id, Gd, loss_mask=Md, status=st, **kw)
        cuts = [0, 5, 16387, 16390, 50000, T]
        parts = [llp.top_p_replay(X[s:e, lo:hi], Id[s:e], Gd[s:e], loss_mask=Md[s:e], **kw)
                 for s, e in zip(cuts[:-1], cuts[1:])]
        dense = llp.keep_mask_replay(X[:, lo:hi], Kd[:, lo:hi], Gd, loss_mask=Md, **kw)
        torch.cuda.synchronize()
        assert int(st.item()) & llp.STATUS_BITS["REPLAY_ID_INVALID"]
        for k in ("target_logit", "in_range", "lse", "logp"):
            one = torch.cat([p[k] for p in parts])
            assert torch.equal(big[k], one), (lo, hi, k)
            assert torch.equal(big[k], dense[k]), (lo, hi, k)
        rows = np.unique(np.concatenate([np.arange(16), np.arange(T - 29, T),
                                         synth.rng(93, 2).integers(0, T, 200)]))
        ref = oracle.top_p_replay(x[idx[rows]][:, lo:hi], I[rows], G[rows], 0.7, lo, hi - lo,
                                  600, mask[rows])
        for k in ("lse", "logp"):
            assert_rows_close(host(big[k])[rows], ref[k], LOGP_ATOL, f"topp {k} [{lo},{hi})")
        np.testing.assert_array_equal(host(big["in_range"])[rows], ref["in_range"])
