"""The execution calls under HIP graph capture ([CUDA provider, "Changes"]: the provider calls
must be capturable into CUDA/HIP graphs). Forward + backward with caller-allocated outputs and
workspace (G whole, and G in vocabulary slabs), the forward in the library's static scratch, and the replay-side calls (compact
replay over 4 shards and their merge, the logits-input forward, the dense keep-mask replay;
their outputs allocated from the graph's pool during capture) are captured once and replayed
several times. Between replays the program does its own eager work, overwrites the graph's
outputs with NaN and synchronizes. Every replay must give bitwise the eager results (the
workspace's tile-queue counters are zeroed by a kernel of the call, not by a memset node).
The shape runs more tiles than there are compute units, so the forward's persistent workers
chain tiles and claim dynamic ones inside the graph."""
import numpy as np
import pytest
import torch

import synth
from tests._gpu import bytes_equal, dev, dev_bf16, need_gpu, say

pytestmark = pytest.mark.gpu

T, H, VR, VP, TAU = 512, 256, 70000, 70144, 0.8


@pytest.fixture(scope="module")
def llp():
    need_gpu()
    import lm_head_linear_logp_amd as m
    m.open(0)
    return m


def _case():
    c = synth.small_case(T, H, VR, VP, TAU, case_id=81, mask_frac=0.2, with_bias=True,
                         w_std=0.05)
    g = np.random.default_rng(81)
    return dict(h=dev_bf16(c["hidden"]), W=dev_bf16(c["weight"]), b=dev_bf16(c["bias"]),
                tg=dev(c["targets"]), mask=dev(c["mask"]),
                dl=torch.from_numpy(g.standard_normal(T).astype(np.float32)).cuda())


def _buffers(llp, x):
    fo = dict(target_logit=torch.empty(T, device="cuda"),
              in_range=torch.empty(T, dtype=torch.uint8, device="cuda"),
              lse=torch.empty(T, device="cuda"), entropy=torch.empty(T, device="cuda"),
              logp=torch.empty(T, device="cuda"))
    req = dict(temperature=TAU, bias=x["b"], loss_mask=x["mask"], real_vocab=VR, padded_vocab=VP)
    fws = torch.empty(1 << 26, dtype=torch.uint8, device="cuda")
    bws = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
    go = dict(dhidden=torch.empty((T, H), dtype=torch.bfloat16, device="cuda"),
              dweight=torch.empty((VP, H), device="cuda"), dbias=torch.empty(VP, device="cuda"))
    return fo, req, fws, bws, go


def _step(llp, x, fo, req, fws, bws, go, g_slabs=False):
    llp.forward(x["h"], x["W"], x["tg"], workspace=fws, out=fo, **req)
    llp.backward(x["h"], x["W"], x["tg"], fo["lse"], x["dl"], overwrite=True, workspace=bws,
                 dhidden=go["dhidden"], dweight=go["dweight"], dbias=go["dbias"],
                 g_slabs=g_slabs, **req)


def _snapshot(fo, go):
    return {k: v.clone() for k, v in list(fo.items()) + list(go.items())}


def _poison(fo, go):
    for t in list(fo.values()) + list(go.values()):
        if t.dtype == torch.uint8:
            t.fill_(7)
        else:
            t.fill_(float("nan"))


@pytest.mark.parametrize("g_slabs", [False, True], ids=["g_whole", "g_slabs"])
def test_forward_backward_replays_match_eager(llp, g_slabs):
    # With g_slabs the backward runs its kernels once per vocabulary slab (three here).
    x = _case()
    fo, req, fws, bws, go = _buffers(llp, x)
    say(f"graph: eager forward + backward T={T} H={H} V={VR}/{VP} g_slabs={g_slabs}")
    _step(llp, x, fo, req, fws, bws, go, g_slabs)
    torch.cuda.synchronize()
    ref = _snapshot(fo, go)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(llp, x, fo, req, fws, bws, go, g_slabs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph: capture")
    with torch.cuda.graph(g):
        _step(llp, x, fo, req, fws, bws, go, g_slabs)
    torch.cuda.synchronize()
    other = _case()
    other["dl"] = other["dl"] * 2
    ob = _buffers(llp, other)
    for rep in range(4):
        say(f"graph: replay {rep}")
        _step(llp, other, *ob, g_slabs)          # the program's own eager work between replays
        _poison(fo, go)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert bytes_equal(fo.get(k, go.get(k)), v), (rep, k)


def test_noalloc_forward_replays_match_eager(llp):
    x = _case()
    fo, req, _, _, _ = _buffers(llp, x)
    say("graph: eager noalloc forward")
    llp.forward_noalloc(x["h"], x["W"], x["tg"], out=fo, **req)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in fo.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        llp.forward_noalloc(x["h"], x["W"], x["tg"], out=fo, **req)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph: capture noalloc")
    with torch.cuda.graph(g):
        llp.forward_noalloc(x["h"], x["W"], x["tg"], out=fo, **req)
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"graph: noalloc replay {rep}")
        # eager work on the same static scratch between replays (a smaller call)
        y = _case()
        fo2 = {k: torch.empty(T // 2, dtype=v.dtype, device="cuda") for k, v in fo.items()}
        llp.forward_noalloc(y["h"][: T // 2], y["W"], y["tg"][: T // 2], out=fo2,
                            temperature=TAU, bias=y["b"], loss_mask=y["mask"][: T // 2],
                            real_vocab=VR, padded_vocab=VP)
        for v in fo.values():
            v.fill_(7) if v.dtype == torch.uint8 else v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert bytes_equal(fo[k], v), (rep, k)


def _replay_inputs(seed):
    g = np.random.default_rng(seed)
    Tr, V, Vp = 300, 600, 640
    x = (g.standard_normal((Tr, Vp)) * 2.0).astype(np.float32)
    x[:, V:] = -1e30
    ids = np.full((Tr, 64), -1, dtype=np.int64)
    for t in range(Tr):
        n = int(g.integers(0, 40))
        lst = g.choice(V, size=n, replace=False)
        lst = np.concatenate([lst, lst[: int(g.integers(0, n + 1))]])[:64]
        g.shuffle(lst)
        ids[t, :lst.size] = lst
    tg = np.where(g.random(Tr) < 0.8, np.maximum(ids[:, 0], 0), g.integers(0, V, Tr))
    keep = np.zeros((Tr, Vp), dtype=np.uint8)
    for t in range(Tr):
        keep[t, ids[t][ids[t] >= 0]] = 1
    mask = (g.random(Tr) > 0.1).astype(np.uint8)
    return dict(x=dev(x), ids=dev(ids), tg=dev(tg.astype(np.int64)), keep=dev(keep),
                mask=dev(mask), V=V, Vp=Vp)


def _replay_calls(llp, d):
    """The replay-side execution calls: compact replay over 4 shards and their merge, the
    logits-input forward and the dense keep-mask replay. Outputs come from the calls."""
    V, Vp = d["V"], d["Vp"]
    parts = []
    for r, lo in enumerate(range(0, Vp, Vp // 4)):
        hi = lo + Vp // 4
        parts.append(llp.top_p_replay(d["x"][:, lo:hi], d["ids"], d["tg"], temperature=0.7,
                                      offset=lo, real_vocab=V, padded_vocab=Vp, rank=r,
                                      world=4, local_size=hi - lo, loss_mask=d["mask"]))
    mg = llp.merge(parts, loss_mask=d["mask"], want_entropy=False)
    fl = llp.forward_logits(d["x"], d["tg"], temperature=0.7, real_vocab=V, padded_vocab=Vp,
                            loss_mask=d["mask"])
    km = llp.keep_mask_replay(d["x"], d["keep"], d["tg"], temperature=0.7, real_vocab=V,
                              padded_vocab=Vp, loss_mask=d["mask"])
    outs = {f"merge.{k}": v for k, v in mg.items() if v is not None}
    outs.update({f"logits.{k}": v for k, v in fl.items() if v is not None})
    outs.update({f"keep.{k}": v for k, v in km.items() if v is not None})
    return outs


def test_replay_paths_replays_match_eager(llp):
    d = _replay_inputs(7)
    say("graph: eager replay paths")
    ref = {k: v.clone() for k, v in _replay_calls(llp, d).items()}
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _replay_calls(llp, d)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph: capture replay paths")
    with torch.cuda.graph(g):
        outs = _replay_calls(llp, d)
    torch.cuda.synchronize()
    other = _replay_inputs(8)
    for rep in range(4):
        say(f"graph: replay-path replay {rep}")
        _replay_calls(llp, other)
        for v in outs.values():
            v.fill_(7) if v.dtype == torch.uint8 else v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert bytes_equal(outs[k], v), (rep, k)
