"""linear_logp: the operator as an autograd node ([CUDA provider, "Motivation"]: gradients must
flow). Its forward values are bitwise those of llp.forward, and the gradients autograd hands
back for hidden, weight and bias are bitwise llp.backward's for the same upstream dlogp and
dentropy (weight and bias gradients after the cast to the parameters' dtype). llp.forward and
llp.backward are checked against the oracle elsewhere; here the composition is checked."""
import numpy as np
import pytest
import torch

import synth
from tests._gpu import bytes_equal, dev, dev_bf16, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def llp():
    need_gpu()
    import lm_head_linear_logp_amd as m
    m.open(0)
    return m


@pytest.mark.parametrize("with_entropy_grad", [True, False])
def test_autograd_matches_forward_and_backward(llp, with_entropy_grad):
    T, H, Vr, Vp, tau = 300, 256, 1900, 2048, 0.8
    c = synth.small_case(T, H, Vr, Vp, tau, case_id=85, mask_frac=0.25, with_bias=True,
                         w_std=0.05)
    h = dev_bf16(c["hidden"]).requires_grad_(True)
    W = dev_bf16(c["weight"]).requires_grad_(True)
    b = dev_bf16(c["bias"]).requires_grad_(True)
    tg, mask = dev(c["targets"]), dev(c["mask"])
    g = np.random.default_rng(85)
    w1 = torch.from_numpy(g.standard_normal(T).astype(np.float32)).cuda()
    w2 = torch.from_numpy(g.standard_normal(T).astype(np.float32)).cuda()
    say(f"autograd T={T} H={H} V={Vr}/{Vp} entropy grad {with_entropy_grad}")
    logp, ent, lse = llp.linear_logp(h, W, tg, temperature=tau, bias=b,
                                     loss_mask=mask.bool(), real_vocab=Vr, padded_vocab=Vp)
    loss = (logp * w1).sum() + ((ent * w2).sum() if with_entropy_grad else 0.0)
    loss.backward()
    torch.cuda.synchronize()

    with torch.no_grad():
        ref = llp.forward(h.detach(), W.detach(), tg, temperature=tau, bias=b.detach(),
                          loss_mask=mask, real_vocab=Vr, padded_vocab=Vp)
        for k, v in (("logp", logp), ("entropy", ent), ("lse", lse)):
            assert bytes_equal(v, ref[k]), k
        gr = llp.backward(h.detach(), W.detach(), tg, ref["lse"], w1, temperature=tau,
                          bias=b.detach(), loss_mask=mask, real_vocab=Vr, padded_vocab=Vp,
                          dentropy=w2 if with_entropy_grad else None,
                          entropy=ref["entropy"] if with_entropy_grad else None,
                          overwrite=True, want_dbias=True)
        torch.cuda.synchronize()
    assert bytes_equal(h.grad, gr["dhidden"])
    assert bytes_equal(W.grad, gr["dweight"].to(torch.bfloat16))
    assert bytes_equal(b.grad, gr["dbias"].to(torch.bfloat16))
    m = mask.bool()
    assert torch.all(h.grad[~m] == 0)
    assert torch.all(logp[~m] == 0)


def test_autograd_without_entropy_output(llp):
    T, H, Vr, Vp, tau = 128, 128, 500, 512, 0.7
    c = synth.small_case(T, H, Vr, Vp, tau, case_id=86, w_std=0.05)
    h = dev_bf16(c["hidden"]).requires_grad_(True)
    W = dev_bf16(c["weight"]).requires_grad_(True)
    tg = dev(c["targets"])
    logp, ent, _ = llp.linear_logp(h, W, tg, temperature=tau, want_entropy=False)
    assert ent.numel() == 0
    logp.sum().backward()
    torch.cuda.synchronize()
    with torch.no_grad():
        ref = llp.forward(h.detach(), W.detach(), tg, temperature=tau, want_entropy=False)
        gr = llp.backward(h.detach(), W.detach(), tg, ref["lse"], torch.ones(T, device="cuda"),
                          temperature=tau, overwrite=True)
        torch.cuda.synchronize()
    assert bytes_equal(logp, ref["logp"])
    assert bytes_equal(h.grad, gr["dhidden"])
    assert bytes_equal(W.grad, gr["dweight"].to(torch.bfloat16))


def test_autograd_with_g_slabs(llp):
    # 157 vocabulary tiles: two slabs of G in the backward.
    T, H, Vr, Vp, tau = 64, 128, 40000, 40192, 0.7
    c = synth.small_case(T, H, Vr, Vp, tau, case_id=87, w_std=0.05)
    h = dev_bf16(c["hidden"]).requires_grad_(True)
    W = dev_bf16(c["weight"]).requires_grad_(True)
    tg = dev(c["targets"])
    logp, ent, _ = llp.linear_logp(h, W, tg, temperature=tau, real_vocab=Vr, padded_vocab=Vp,
                                   g_slabs=True)
    (logp.sum() + 0.5 * ent.sum()).backward()
    torch.cuda.synchronize()
    with torch.no_grad():
        ref = llp.forward(h.detach(), W.detach(), tg, temperature=tau, real_vocab=Vr,
                          padded_vocab=Vp)
        gr = llp.backward(h.detach(), W.detach(), tg, ref["lse"], torch.ones(T, device="cuda"),
                          temperature=tau, real_vocab=Vr, padded_vocab=Vp,
                          dentropy=torch.full((T,), 0.5, device="cuda"), entropy=ref["entropy"],
                          overwrite=True, g_slabs=True)
        torch.cuda.synchronize()
    assert bytes_equal(h.grad, gr["dhidden"])
    assert bytes_equal(W.grad, gr["dweight"].to(torch.bfloat16))
