"""llp_forward_noalloc: the forward in the library's static device scratch, for callers that
cannot allocate. Its results must be bitwise those of llp_forward (same kernels), call after
call, whatever the previous call left in the shared scratch: the calls below run largest
first, then smaller ones. The size limit is checked on the CPU."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import synth
from lm_head_linear_logp_amd import _capi as A

FAKE = 1 << 20


def _request(T, H, V, Vr):
    r = A.llp_request()
    r.proj.hidden, r.proj.hidden_stride = FAKE, H
    r.proj.weight, r.proj.weight_stride = FAKE, H
    r.proj.hidden_size = H
    r.vocab.offset, r.vocab.local_size, r.vocab.real_vocab, r.vocab.padded_vocab = 0, V, Vr, V
    r.vocab.rank, r.vocab.world = 0, 1
    r.layout.num_tokens = T
    r.target_ids = FAKE
    r.temperature = 0.7
    return r


def _noalloc_status(T, H, V, Vr):
    out = A.llp_partials(FAKE, FAKE, FAKE, FAKE, FAKE)
    return A.load().llp_forward_noalloc(C.byref(_request(T, H, V, Vr)), C.byref(out), None)


def test_noalloc_size_limit():
    """4608 rows over a 151669-column vocabulary fit the 32 MiB scratch; 4609 do not and are
    refused before anything else is looked at (no device needed)."""
    assert _noalloc_status(4609, 64, 151936, 151669) == A.LLP_ERR_UNSUPPORTED
    assert b"static scratch" in A.load().llp_last_error()
    assert _noalloc_status(4608, 64, 151936, 151669) != A.LLP_ERR_UNSUPPORTED
    assert _noalloc_status(18433, 64, 37984, 37984) == A.LLP_ERR_UNSUPPORTED
    assert _noalloc_status(18432, 64, 37984, 37984) != A.LLP_ERR_UNSUPPORTED


def d16(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def _outputs(T, want_entropy):
    return dict(target_logit=torch.full((T,), np.nan, device="cuda"),
                in_range=torch.full((T,), 7, dtype=torch.uint8, device="cuda"),
                lse=torch.full((T,), np.nan, device="cuda"),
                entropy=torch.full((T,), np.nan, device="cuda") if want_entropy else None,
                logp=torch.full((T,), np.nan, device="cuda"))


def _same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.gpu
def test_noalloc_matches_forward_on_consecutive_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import lm_head_linear_logp_amd as llp
    llp.open(0)
    cases = [
        # (T, H, real V, padded V, bias, masked fraction, entropy): largest first.
        (18432, 64, 37717, 37984, None, 0.25, True),       # at the limit, 2 layout blocks
        (4608, 64, 151669, 151936, None, 0.0, True),       # at the scratch limit
        (3000, 512, 20000, 20480, "f32", 0.2, True),
        (700, 256, 3000, 3072, None, 0.3, False),
        (64, 256, 1000, 1024, "bf16", 0.0, True),
    ]
    for i, (T, H, Vr, Vp, bias, mf, ent) in enumerate(cases):
        print(f"noalloc case {i}: T={T} H={H} V={Vr}/{Vp} bias={bias} mask={mf} entropy={ent}",
              flush=True)
        c = synth.small_case(T, H, Vr, Vp, 0.7, case_id=700 + i, mask_frac=mf,
                             with_bias=bias is not None, w_std=0.05)
        h, W, tg, mk = d16(c["hidden"]), d16(c["weight"]), torch.from_numpy(c["targets"]).cuda(), \
            torch.from_numpy(c["mask"]).cuda()
        b = None
        if bias == "bf16":
            b = d16(c["bias"])
        elif bias == "f32":
            b = torch.from_numpy(oracle.bf16_to_f64(c["bias"]).astype(np.float32)).cuda()
        kw = dict(temperature=0.7, bias=b, loss_mask=mk, real_vocab=Vr, padded_vocab=Vp,
                  want_entropy=ent)
        st_a = torch.zeros(1, dtype=torch.int32, device="cuda")
        st_b = torch.zeros(1, dtype=torch.int32, device="cuda")
        ref = llp.forward(h, W, tg, status=st_a, **kw)
        got = llp.forward_noalloc(h, W, tg, out=_outputs(T, ent), status=st_b, **kw)
        again = llp.forward_noalloc(h, W, tg, out=_outputs(T, ent), **kw)
        torch.cuda.synchronize()
        keys = ["target_logit", "in_range", "lse", "logp"] + (["entropy"] if ent else [])
        for k in keys:
            assert _same(got[k], ref[k]), f"case {i}: {k} differs from llp_forward"
            assert _same(again[k], ref[k]), f"case {i}: {k} differs on the repeat"
        assert int(st_a.item()) == int(st_b.item())
        if T <= 700:
            o = oracle.forward(c["hidden"], c["weight"], c["bias"] if bias else None, 0.7,
                               c["targets"], c["mask"], Vr)
            err = float(np.max(np.abs(got["logp"].cpu().numpy() - o["logp"])))
            assert err <= 2e-3, f"case {i}: max |logp - oracle| = {err:.3g}"
