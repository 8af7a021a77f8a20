"""The Python binding refuses every tensor whose shape, dtype, device or layout does not match
the request before anything reaches the library (the kernels index by T, H and local_size, so
a short tensor would become an out-of-bounds device access). Runs on the CPU: a malformed call
raises ValueError or TypeError; the same call made well formed gets past validation and fails
only where the library is asked for a device (LLPError, or RuntimeError without a build)."""
import pytest
import torch

import lm_head_linear_logp_amd as llp

T, H, V = 8, 64, 96
BAD = (ValueError, TypeError)
REACHES_LIBRARY = RuntimeError   # LLPError (no GPU here) is a RuntimeError


def f32(*s):
    return torch.zeros(*s, dtype=torch.float32)


def base():
    return dict(hidden=torch.zeros(T, H, dtype=torch.bfloat16),
                weight=torch.zeros(V, H, dtype=torch.bfloat16),
                target_ids=torch.zeros(T, dtype=torch.int64))


def run_forward(**over):
    a = base()
    kw = dict(temperature=0.7)
    for k, v in over.items():
        (a if k in a else kw)[k] = v
    return llp.forward(a["hidden"], a["weight"], a["target_ids"], **kw)


def partials(n=T, ent=True):
    return dict(target_logit=f32(n), in_range=torch.zeros(n, dtype=torch.uint8), lse=f32(n),
                entropy=f32(n) if ent else None, logp=f32(n))


def test_forward_well_formed_reaches_library():
    with pytest.raises(REACHES_LIBRARY) as e:
        run_forward(out=partials(), loss_mask=torch.ones(T, dtype=torch.uint8),
                    bias=f32(V), status=torch.zeros(1, dtype=torch.int32))
    assert not isinstance(e.value, BAD)


@pytest.mark.parametrize("over", [
    dict(target_ids=torch.zeros(T - 1, dtype=torch.int64)),
    dict(target_ids=torch.zeros(T, dtype=torch.int32)),
    dict(weight=torch.zeros(V, H + 8, dtype=torch.bfloat16)),
    dict(hidden=torch.zeros(T, H, dtype=torch.float32)),
    dict(loss_mask=torch.ones(T + 1, dtype=torch.uint8)),
    dict(loss_mask=torch.ones(T, dtype=torch.bool)),
    dict(bias=f32(V - 1)),
    dict(bias=torch.zeros(V, dtype=torch.int32)),
    dict(bias=f32(2 * V)[::2]),
    dict(status=torch.zeros(0, dtype=torch.int32)),
    dict(status=torch.zeros(1, dtype=torch.int64)),
    dict(cu_seqlens=torch.zeros(0, dtype=torch.int32)),
    dict(out=partials(T - 1)),
    dict(out=dict(partials(), lse=f32(T + 3))),
    dict(out=dict(partials(), in_range=f32(T))),
    dict(out=partials(ent=False)),                                  # entropy wanted, not given
    dict(out=partials(), want_entropy=False),                       # entropy given, not wanted
    dict(out=dict(partials(), logp=f32(T - 2))),
    dict(workspace=torch.zeros(16, dtype=torch.float32)),
])
def test_forward_refuses(over):
    with pytest.raises(BAD):
        run_forward(**over)


def run_backward(**over):
    a = base()
    a.update(lse=f32(T), dlogp=f32(T))
    kw = dict(temperature=0.7)
    for k, v in over.items():
        (a if k in a else kw)[k] = v
    return llp.backward(a["hidden"], a["weight"], a["target_ids"], a["lse"], a["dlogp"], **kw)


def test_backward_well_formed_reaches_library():
    with pytest.raises(REACHES_LIBRARY) as e:
        run_backward(dhidden=torch.zeros(T, H, dtype=torch.bfloat16), dweight=f32(V, H),
                     dbias=f32(V), dentropy=f32(T), entropy=f32(T))
    assert not isinstance(e.value, BAD)


@pytest.mark.parametrize("over", [
    dict(lse=f32(T - 1)),
    dict(lse=torch.zeros(T, dtype=torch.float64)),
    dict(dlogp=f32(T + 1)),
    dict(dlogp=torch.zeros(T, dtype=torch.bfloat16)),
    dict(dentropy=f32(T)),                                          # without the entropy
    dict(dentropy=f32(T), entropy=f32(T - 1)),
    dict(dentropy=f32(T - 1), entropy=f32(T)),
    dict(dhidden=torch.zeros(T - 1, H, dtype=torch.bfloat16)),
    dict(dhidden=torch.zeros(T, H, dtype=torch.float32)),
    dict(dhidden=torch.zeros(H, T, dtype=torch.bfloat16).t()),
    dict(dweight=f32(V - 1, H)),
    dict(dweight=f32(V, H - 8)),
    dict(dweight=torch.zeros(V, H, dtype=torch.bfloat16)),
    dict(dbias=torch.zeros(V, dtype=torch.bfloat16)),
    dict(dbias=f32(V - 1)),
    dict(dbias=f32(V, 1)),
])
def test_backward_refuses(over):
    with pytest.raises(BAD):
        run_backward(**over)


def test_merge_refuses():
    good = [partials(), partials()]
    with pytest.raises(REACHES_LIBRARY) as e:
        llp.merge(good, loss_mask=torch.ones(T, dtype=torch.uint8))
    assert not isinstance(e.value, BAD)
    for parts, kw in [
        ([partials(), partials(T - 1)], {}),
        ([partials(), dict(partials(), lse=f32(T + 1))], {}),
        ([partials(), partials(ent=False)], {}),                    # merged entropy wanted
        ([partials(), dict(partials(), entropy=f32(T - 1))], {}),
        ([partials(), dict(partials(), in_range=f32(T))], {}),
        (good, dict(loss_mask=torch.ones(T - 1, dtype=torch.uint8))),
        (good, dict(status=torch.zeros(0, dtype=torch.int32))),
        ([partials()] * 65, {}),
    ]:
        with pytest.raises(BAD):
            llp.merge(parts, **kw)
    with pytest.raises(REACHES_LIBRARY) as e:                       # no entropy: none needed
        llp.merge([partials(ent=False)] * 2, want_entropy=False)
    assert not isinstance(e.value, BAD)


def replay_args(**over):
    a = dict(logits=f32(T, V), replay_ids=torch.full((T, 64), -1, dtype=torch.int64),
             target_ids=torch.zeros(T, dtype=torch.int64))
    kw = dict(temperature=0.7)
    for k, v in over.items():
        (a if k in a else kw)[k] = v
    return a, kw


def test_top_p_replay_refuses():
    a, kw = replay_args(local_size=V // 2)
    with pytest.raises(REACHES_LIBRARY) as e:
        llp.top_p_replay(a["logits"], a["replay_ids"], a["target_ids"], **kw)
    assert not isinstance(e.value, BAD)
    for over in [dict(logits=f32(T + 1, V)), dict(logits=f32(T - 1, V)),
                 dict(logits=torch.zeros(T, V, dtype=torch.int32)),
                 dict(logits=f32(V, T).t()), dict(local_size=V + 1),
                 dict(target_ids=torch.zeros(T - 1, dtype=torch.int64)),
                 dict(replay_ids=torch.zeros(T, 64, dtype=torch.int32)),
                 dict(loss_mask=torch.ones(T + 2, dtype=torch.uint8)),
                 dict(status=torch.zeros(1, dtype=torch.float32))]:
        a, kw = replay_args(**over)
        with pytest.raises(BAD):
            llp.top_p_replay(a["logits"], a["replay_ids"], a["target_ids"], **kw)


def test_forward_logits_refuses():
    tg = torch.zeros(T, dtype=torch.int64)
    with pytest.raises(REACHES_LIBRARY) as e:
        llp.forward_logits(f32(T, V), tg, temperature=0.7, local_size=V - 5)
    assert not isinstance(e.value, BAD)
    # A shard with no real columns reads no logits: a zero-width view of it is fine.
    with pytest.raises(REACHES_LIBRARY) as e:
        llp.forward_logits(f32(T, 4 * V)[:, :0], tg, temperature=0.7, offset=3 * V,
                           real_vocab=2 * V, padded_vocab=4 * V, rank=3, world=4, local_size=V)
    assert not isinstance(e.value, BAD)
    with pytest.raises(BAD):       # the same view for a shard that has real columns
        llp.forward_logits(f32(T, 4 * V)[:, :0], tg, temperature=0.7, offset=V,
                           real_vocab=2 * V, padded_vocab=4 * V, rank=1, world=4, local_size=V)
    for x, kw in [(f32(T + 1, V), {}), (f32(T - 1, V), {}), (f32(T, V), dict(local_size=V + 1)),
                  (f32(T, V), dict(loss_mask=torch.ones(T - 1, dtype=torch.uint8))),
                  (torch.zeros(T, V, dtype=torch.float16), {}),
                  (f32(T, V), dict(cu_seqlens=torch.zeros(0, dtype=torch.int32)))]:
        with pytest.raises(BAD):
            llp.forward_logits(x, tg, temperature=0.7, **kw)


def test_keep_mask_replay_refuses():
    tg = torch.zeros(T, dtype=torch.int64)
    km = torch.zeros(T, V, dtype=torch.uint8)
    with pytest.raises(REACHES_LIBRARY) as e:
        llp.keep_mask_replay(f32(T, V), km, tg, temperature=0.7)
    assert not isinstance(e.value, BAD)
    for x, k, kw in [(f32(T, V), torch.zeros(T - 1, V, dtype=torch.uint8), {}),
                     (f32(T, V), torch.zeros(T, V - 1, dtype=torch.uint8), {}),
                     (f32(T, V), torch.zeros(T, V, dtype=torch.bool), {}),
                     (f32(T + 1, V), km, {}),
                     (f32(T, V), km, dict(local_size=V + 1)),
                     (f32(T, V), km, dict(loss_mask=torch.ones(T + 1, dtype=torch.uint8)))]:
        with pytest.raises(BAD):
            llp.keep_mask_replay(x, k, tg, temperature=0.7, **kw)
