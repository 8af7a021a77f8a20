"""The execution calls under HIP graph capture ([CUDA provider, "Changes"]: the provider calls
must be capturable into CUDA/HIP graphs). Forward + backward with caller-allocated outputs and
workspace, and the forward in the library's static scratch, are captured once and replayed
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


def _step(llp, x, fo, req, fws, bws, go):
    llp.forward(x["h"], x["W"], x["tg"], workspace=fws, out=fo, **req)
    llp.backward(x["h"], x["W"], x["tg"], fo["lse"], x["dl"], overwrite=True, workspace=bws,
                 dhidden=go["dhidden"], dweight=go["dweight"], dbias=go["dbias"], **req)


def _snapshot(fo, go):
    return {k: v.clone() for k, v in list(fo.items()) + list(go.items())}


def _poison(fo, go):
    for t in list(fo.values()) + list(go.values()):
        if t.dtype == torch.uint8:
            t.fill_(7)
        else:
            t.fill_(float("nan"))


def test_forward_backward_replays_match_eager(llp):
    x = _case()
    fo, req, fws, bws, go = _buffers(llp, x)
    say(f"graph: eager forward + backward T={T} H={H} V={VR}/{VP}")
    _step(llp, x, fo, req, fws, bws, go)
    torch.cuda.synchronize()
    ref = _snapshot(fo, go)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(llp, x, fo, req, fws, bws, go)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph: capture")
    with torch.cuda.graph(g):
        _step(llp, x, fo, req, fws, bws, go)
    torch.cuda.synchronize()
    other = _case()
    other["dl"] = other["dl"] * 2
    ob = _buffers(llp, other)
    for rep in range(4):
        say(f"graph: replay {rep}")
        _step(llp, other, *ob)          # the program's own eager work between replays
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
