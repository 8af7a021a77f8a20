"""Python binding of the fused linear log-prob operator's C ABI (include/llp.h).

Argument marshalling only: every step of the operator runs in the HIP library libllp.so.
PyTorch supplies device memory (outputs, workspace) and the current HIP stream. There is no
CPU fallback: if the library is missing or the device is not a gfx950 GPU, calls raise.

Functions mirror the ABI: ``open``, ``workspace_bytes``, ``forward``, ``merge``, ``backward``,
``top_p_replay``, ``last_error``. ``linear_logp`` composes ``forward`` and ``backward`` into
one autograd node for a full-vocabulary shard.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence

import torch

from . import _capi as A

__all__ = ["LLPError", "open", "workspace_bytes", "forward", "forward_noalloc", "merge",
           "backward", "top_p_replay", "last_error", "STATUS_BITS", "forward_logits",
           "keep_mask_replay", "SCRATCH_BYTES", "linear_logp"]

# Size of the static device scratch llp_forward_noalloc works in (include/llp.h).
SCRATCH_BYTES = 32 << 20

STATUS_BITS = {"TARGET_OUT_OF_RANGE": A.LLP_STATUS_TARGET_OUT_OF_RANGE,
               "TARGET_NOT_FOUND": A.LLP_STATUS_TARGET_NOT_FOUND,
               "REPLAY_ID_INVALID": A.LLP_STATUS_REPLAY_ID_INVALID,
               "LAYOUT_INVALID": A.LLP_STATUS_LAYOUT_INVALID}


class LLPError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {A.STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_opened = {}


def last_error() -> str:
    return A.load().llp_last_error().decode()


def _check(st: int, where: str):
    if st != A.LLP_OK:
        raise LLPError(st, where, last_error())


def open(device: Optional[int] = None) -> dict:
    """Load the kernels on a gfx950 device (llp_open); returns the library identity."""
    lib = A.load()
    if device is None:
        device = torch.cuda.current_device()
    if device in _opened:
        return _opened[device]
    info = A.llp_info()
    _check(lib.llp_open(int(device), C.byref(info)), "llp_open")
    d = dict(name=info.name.decode(), version=info.version.decode(), arch=info.arch.decode(),
             route=info.route.decode(), max_replay_ids=info.max_replay_ids,
             num_cus=info.num_cus, device=info.device)
    _opened[device] = d
    return d


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, name, dtype, ndim, device, shape=None):
    """Type, rank, device and last-dimension contiguity of a tensor the library reads or
    writes through a raw pointer; with `shape`, also its exact shape (None entries are free).
    The kernels index by T, H and local_size, so a short tensor would be an out-of-bounds
    device access: every mismatch is refused here, before anything is enqueued."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None:
        for i, n in enumerate(shape):
            if n is not None and t.shape[i] != n:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected "
                                 f"{tuple('*' if x is None else x for x in shape)}")
    if ndim >= 1 and t.numel() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name} must be contiguous in its last dimension")


def _vec(t, name, dtype, n, device):
    """A contiguous 1-d tensor of exactly n elements."""
    _need(t, name, dtype, 1, device, (n,))


def _status(status, device):
    if status is not None:
        _need(status, "status", torch.int32, 1, device)
        if status.numel() < 1:
            raise ValueError("status must hold at least one int32")


def _request(hidden, weight, target_ids, temperature, bias, loss_mask, cu_seqlens, offset,
             real_vocab, padded_vocab, rank, world, want_entropy, status):
    dev = hidden.device
    _need(hidden, "hidden", torch.bfloat16, 2, dev)
    _need(weight, "weight", torch.bfloat16, 2, dev)
    T, H = hidden.shape
    _vec(target_ids, "target_ids", torch.int64, T, dev)
    if weight.shape[1] != H:
        raise ValueError(f"weight is {tuple(weight.shape)}, hidden size is {H}")
    if padded_vocab is None:
        padded_vocab = weight.shape[0] if world == 1 else None
    if real_vocab is None:
        real_vocab = padded_vocab
    if padded_vocab is None:
        raise ValueError("padded_vocab is required for a vocabulary shard (world > 1)")
    req = A.llp_request()
    req.proj.hidden = _ptr(hidden)
    req.proj.hidden_stride = hidden.stride(0) if T > 0 else H
    req.proj.weight = _ptr(weight)
    req.proj.weight_stride = weight.stride(0) if weight.shape[0] > 0 else H
    if bias is not None:
        if not isinstance(bias, torch.Tensor) or bias.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("bias must be a bf16 or fp32 tensor")
        _vec(bias, "bias", bias.dtype, weight.shape[0], dev)
        req.proj.bias = _ptr(bias)
        req.proj.bias_dtype = A.LLP_DTYPE_F32 if bias.dtype == torch.float32 else A.LLP_DTYPE_BF16
    req.proj.hidden_size = H
    req.vocab.offset = int(offset)
    req.vocab.local_size = int(weight.shape[0])
    req.vocab.real_vocab = int(real_vocab)
    req.vocab.padded_vocab = int(padded_vocab)
    req.vocab.rank = int(rank)
    req.vocab.world = int(world)
    req.layout.num_tokens = T
    if loss_mask is not None:
        _vec(loss_mask, "loss_mask", torch.uint8, T, dev)
        req.layout.loss_mask = _ptr(loss_mask)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, 1, dev)
        if cu_seqlens.shape[0] < 1:
            raise ValueError("cu_seqlens needs at least one entry")
        req.layout.cu_seqlens = _ptr(cu_seqlens)
        req.layout.num_seqs = cu_seqlens.shape[0] - 1
    req.target_ids = _ptr(target_ids)
    req.temperature = float(temperature)
    req.flags = A.LLP_FLAG_WANT_ENTROPY if want_entropy else 0
    _status(status, dev)
    req.status_word = _ptr(status)
    return req


def workspace_bytes(req: "A.llp_request", op: int) -> int:
    n = C.c_size_t(0)
    _check(A.load().llp_workspace_bytes(C.byref(req), op, C.byref(n)), "llp_workspace_bytes")
    return int(n.value)


def _workspace(req, op, dev, workspace):
    need = workspace_bytes(req, op)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    return workspace


def _partials_out(out, T, dev, want_entropy, with_logp_required=False):
    """Checks a caller-supplied partials dict (target_logit, in_range, lse, entropy, logp)."""
    _vec(out["target_logit"], "out['target_logit']", torch.float32, T, dev)
    _vec(out["in_range"], "out['in_range']", torch.uint8, T, dev)
    _vec(out["lse"], "out['lse']", torch.float32, T, dev)
    ent = out.get("entropy")
    if want_entropy:
        if ent is None:
            raise ValueError("out['entropy'] is required when the entropy is wanted")
        _vec(ent, "out['entropy']", torch.float32, T, dev)
    elif ent is not None:
        raise ValueError("out['entropy'] given but the entropy is not wanted")
    lp = out.get("logp")
    if lp is not None or with_logp_required:
        _vec(lp, "out['logp']", torch.float32, T, dev)


def forward(hidden: torch.Tensor, weight: torch.Tensor, target_ids: torch.Tensor, *,
            temperature: float, bias: Optional[torch.Tensor] = None,
            loss_mask: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
            offset: int = 0, real_vocab: Optional[int] = None,
            padded_vocab: Optional[int] = None, rank: int = 0, world: int = 1,
            want_entropy: bool = True, status: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None) -> dict:
    """llp_forward on one shard. Returns target_logit, in_range, lse, entropy, logp (device
    tensors of length T; entropy None unless want_entropy). For world == 1, logp/entropy are
    final; otherwise pass the shards' results to ``merge``."""
    req = _request(hidden, weight, target_ids, temperature, bias, loss_mask, cu_seqlens, offset,
                   real_vocab, padded_vocab, rank, world, want_entropy, status)
    dev, T = hidden.device, hidden.shape[0]
    if out is not None:
        _partials_out(out, T, dev, want_entropy)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1, dev)
    open(dev.index)
    if out is None:
        out = dict(target_logit=torch.empty(T, dtype=torch.float32, device=dev),
                   in_range=torch.empty(T, dtype=torch.uint8, device=dev),
                   lse=torch.empty(T, dtype=torch.float32, device=dev),
                   entropy=torch.empty(T, dtype=torch.float32, device=dev) if want_entropy else None,
                   logp=torch.empty(T, dtype=torch.float32, device=dev))
    o = A.llp_partials(_ptr(out["target_logit"]), _ptr(out["in_range"]), _ptr(out["lse"]),
                       _ptr(out.get("entropy")), _ptr(out.get("logp")))
    ws = _workspace(req, A.LLP_OP_FORWARD, dev, workspace)
    _check(A.load().llp_forward(C.byref(req), C.byref(o), _ptr(ws), ws.numel(),
                                _stream_ptr(dev)), "llp_forward")
    return out


def forward_noalloc(hidden: torch.Tensor, weight: torch.Tensor, target_ids: torch.Tensor, *,
                    temperature: float, out: dict, bias: Optional[torch.Tensor] = None,
                    loss_mask: Optional[torch.Tensor] = None,
                    cu_seqlens: Optional[torch.Tensor] = None, offset: int = 0,
                    real_vocab: Optional[int] = None, padded_vocab: Optional[int] = None,
                    rank: int = 0, world: int = 1, want_entropy: bool = True,
                    status: Optional[torch.Tensor] = None) -> dict:
    """llp_forward_noalloc: ``forward`` in the library's static device scratch. The caller
    passes the output tensors (``out``: target_logit, in_range, lse, entropy when wanted,
    logp optional); neither this function nor the library allocates device memory, so it
    can run where allocation is not allowed. Calls that overlap on one device race on the
    scratch."""
    req = _request(hidden, weight, target_ids, temperature, bias, loss_mask, cu_seqlens, offset,
                   real_vocab, padded_vocab, rank, world, want_entropy, status)
    dev, T = hidden.device, hidden.shape[0]
    if not isinstance(out, dict):
        raise TypeError("out must be a dict of output tensors")
    _partials_out(out, T, dev, want_entropy)
    open(dev.index)
    o = A.llp_partials(_ptr(out["target_logit"]), _ptr(out["in_range"]), _ptr(out["lse"]),
                       _ptr(out.get("entropy")), _ptr(out.get("logp")))
    _check(A.load().llp_forward_noalloc(C.byref(req), C.byref(o), _stream_ptr(dev)),
           "llp_forward_noalloc")
    return out


def merge(parts: Sequence[dict], *, loss_mask: Optional[torch.Tensor] = None,
          want_entropy: bool = True, status: Optional[torch.Tensor] = None) -> dict:
    """llp_merge of shard partials given in rank order. Returns logp, lse, entropy."""
    world = len(parts)
    if world < 1:
        raise ValueError("merge needs at least one shard")
    if world > A.LLP_MAX_WORLD:
        raise ValueError(f"merge takes at most {A.LLP_MAX_WORLD} shards")
    if not isinstance(parts[0].get("lse"), torch.Tensor):
        raise TypeError("parts[0]['lse'] must be a torch.Tensor")
    dev = parts[0]["lse"].device
    T = parts[0]["lse"].shape[0] if parts[0]["lse"].dim() == 1 else -1
    arr = (A.llp_partials * world)()
    for r, p in enumerate(parts):
        for k, dt in (("target_logit", torch.float32), ("in_range", torch.uint8),
                      ("lse", torch.float32)):
            _vec(p[k], f"parts[{r}]['{k}']", dt, T, dev)
        ent = p.get("entropy") if want_entropy else None
        if want_entropy:
            if ent is None:
                raise ValueError(f"parts[{r}]['entropy'] is required for the merged entropy")
            _vec(ent, f"parts[{r}]['entropy']", torch.float32, T, dev)
        arr[r] = A.llp_partials(_ptr(p["target_logit"]), _ptr(p["in_range"]), _ptr(p["lse"]),
                                _ptr(ent), None)
    if loss_mask is not None:
        _vec(loss_mask, "loss_mask", torch.uint8, T, dev)
    _status(status, dev)
    open(dev.index)
    out = dict(logp=torch.empty(T, dtype=torch.float32, device=dev),
               lse=torch.empty(T, dtype=torch.float32, device=dev),
               entropy=torch.empty(T, dtype=torch.float32, device=dev) if want_entropy else None)
    fo = A.llp_final_out(_ptr(out["logp"]), _ptr(out["lse"]), _ptr(out["entropy"]))
    _check(A.load().llp_merge(world, arr, T, _ptr(loss_mask), C.byref(fo), _ptr(status),
                              _stream_ptr(dev)), "llp_merge")
    return out


def backward(hidden: torch.Tensor, weight: torch.Tensor, target_ids: torch.Tensor,
             lse: torch.Tensor, dlogp: torch.Tensor, *, temperature: float,
             bias: Optional[torch.Tensor] = None, loss_mask: Optional[torch.Tensor] = None,
             cu_seqlens: Optional[torch.Tensor] = None, offset: int = 0,
             real_vocab: Optional[int] = None, padded_vocab: Optional[int] = None,
             rank: int = 0, world: int = 1, dentropy: Optional[torch.Tensor] = None,
             entropy: Optional[torch.Tensor] = None, dweight: Optional[torch.Tensor] = None,
             dbias: Optional[torch.Tensor] = None, want_dbias: Optional[bool] = None,
             dhidden: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, overwrite: bool = False,
             g_slabs: bool = False) -> dict:
    """llp_backward on one shard: dhidden (bf16, overwritten), dweight (fp32, accumulated),
    dbias (fp32, accumulated; allocated when the request has a bias or want_dbias). With
    overwrite=True (LLP_FLAG_OVERWRITE_GRADS) dweight and dbias are written instead of added
    to, and a missing dweight/dbias is allocated uninitialised. With g_slabs=True
    (LLP_FLAG_G_SLABS) the workspace holds G for one vocabulary slab of LLP_G_SLAB_COLUMNS
    columns at a time instead of the whole shard."""
    req = _request(hidden, weight, target_ids, temperature, bias, loss_mask, cu_seqlens, offset,
                   real_vocab, padded_vocab, rank, world, False, status)
    if overwrite:
        req.flags |= A.LLP_FLAG_OVERWRITE_GRADS
    if g_slabs:
        req.flags |= A.LLP_FLAG_G_SLABS
    dev = hidden.device
    T, H = hidden.shape
    V = weight.shape[0]
    _vec(lse, "lse", torch.float32, T, dev)
    _vec(dlogp, "dlogp", torch.float32, T, dev)
    if dentropy is not None:
        if entropy is None:
            raise ValueError("dentropy needs the merged entropy")
        _vec(dentropy, "dentropy", torch.float32, T, dev)
        _vec(entropy, "entropy", torch.float32, T, dev)
    if dhidden is not None:
        _need(dhidden, "dhidden", torch.bfloat16, 2, dev, (T, H))
    if dweight is not None:
        _need(dweight, "dweight", torch.float32, 2, dev, (V, H))
    if want_dbias is None:
        want_dbias = bias is not None or dbias is not None
    if dbias is not None:
        _vec(dbias, "dbias", torch.float32, V, dev)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1, dev)
    open(dev.index)
    if dhidden is None:
        dhidden = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    alloc = torch.empty if overwrite else torch.zeros
    if dweight is None:
        dweight = alloc(weight.shape, dtype=torch.float32, device=dev)
    if dbias is None and want_dbias:
        dbias = alloc(V, dtype=torch.float32, device=dev)
    bi = A.llp_bwd_in(_ptr(lse), _ptr(dlogp), _ptr(dentropy), _ptr(entropy))
    bo = A.llp_bwd_out(_ptr(dhidden), dhidden.stride(0) if T > 0 else H, _ptr(dweight),
                       dweight.stride(0) if V > 0 else H, _ptr(dbias))
    ws = _workspace(req, A.LLP_OP_BACKWARD, dev, workspace)
    _check(A.load().llp_backward(C.byref(req), C.byref(bi), C.byref(bo), _ptr(ws), ws.numel(),
                                 _stream_ptr(dev)), "llp_backward")
    return dict(dhidden=dhidden, dweight=dweight, dbias=dbias)


def _vocab(req_vocab, offset, local_size, real_vocab, padded_vocab, rank, world):
    if padded_vocab is None:
        padded_vocab = local_size if world == 1 else None
    if real_vocab is None:
        real_vocab = padded_vocab
    if padded_vocab is None:
        raise ValueError("padded_vocab is required for a vocabulary shard (world > 1)")
    req_vocab.offset = int(offset)
    req_vocab.local_size = int(local_size)
    req_vocab.real_vocab = int(real_vocab)
    req_vocab.padded_vocab = int(padded_vocab)
    req_vocab.rank = int(rank)
    req_vocab.world = int(world)


def _logits_view(logits, T, local_size, dev):
    """A shard's local logits [T, width] (fp32 or bf16, contiguous rows): returns the ABI dtype
    code, the row stride and local_size (default: the view's width). The view must cover the
    shard's real columns (checked by _covers_real once the partition is known)."""
    if not isinstance(logits, torch.Tensor) or logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("logits must be an fp32 or bf16 tensor")
    _need(logits, "logits", logits.dtype, 2, dev, (T, None))
    if local_size is None:
        local_size = logits.shape[1]
    if int(local_size) < 0:
        raise ValueError(f"local_size {local_size} < 0")
    dt = A.LLP_DTYPE_F32 if logits.dtype == torch.float32 else A.LLP_DTYPE_BF16
    return dt, (logits.stride(0) if T > 0 else int(local_size)), int(local_size)


def _covers_real(t, name, vocab):
    """The kernels read a row's columns below the shard's real ones only,
    clamp(real_vocab - offset, 0, local_size): `t` must be at least that wide."""
    n_real = min(max(vocab.real_vocab - vocab.offset, 0), vocab.local_size)
    if t.shape[1] < n_real:
        raise ValueError(f"{name} has {t.shape[1]} columns; the shard has {n_real} real columns")


def _partials_alloc(T, dev, want_entropy):
    return dict(target_logit=torch.empty(T, dtype=torch.float32, device=dev),
                in_range=torch.empty(T, dtype=torch.uint8, device=dev),
                lse=torch.empty(T, dtype=torch.float32, device=dev),
                entropy=torch.empty(T, dtype=torch.float32, device=dev) if want_entropy else None,
                logp=torch.empty(T, dtype=torch.float32, device=dev))


def top_p_replay(logits: torch.Tensor, replay_ids: torch.Tensor, target_ids: torch.Tensor, *,
                 temperature: float, offset: int = 0, real_vocab: Optional[int] = None,
                 padded_vocab: Optional[int] = None, rank: int = 0, world: int = 1,
                 loss_mask: Optional[torch.Tensor] = None, processed_logprobs: bool = True,
                 status: Optional[torch.Tensor] = None, local_size: Optional[int] = None) -> dict:
    """llp_top_p_replay on one shard's local logits [T, local_size] (fp32 or bf16; a strided
    view of a wider logits tensor is fine). Returns target_logit, in_range, lse, logp."""
    dev = logits.device
    if not isinstance(replay_ids, torch.Tensor):
        raise TypeError("replay_ids must be a torch.Tensor")
    _need(replay_ids, "replay_ids", torch.int64, 2, dev)
    T = replay_ids.shape[0]
    _vec(target_ids, "target_ids", torch.int64, T, dev)
    dt, ld, local_size = _logits_view(logits, T, local_size, dev)
    req = A.llp_topp_request()
    req.logits = _ptr(logits)
    req.logits_dtype = dt
    req.num_replay = replay_ids.shape[1]
    req.logits_stride = ld
    req.num_tokens = T
    _vocab(req.vocab, offset, local_size, real_vocab, padded_vocab, rank, world)
    _covers_real(logits, "logits", req.vocab)
    req.replay_ids = _ptr(replay_ids)
    req.replay_stride = replay_ids.stride(0) if T > 0 else replay_ids.shape[1]
    req.target_ids = _ptr(target_ids)
    if loss_mask is not None:
        _vec(loss_mask, "loss_mask", torch.uint8, T, dev)
        req.loss_mask = _ptr(loss_mask)
    req.temperature = float(temperature)
    req.processed_logprobs = 1 if processed_logprobs else 0
    _status(status, dev)
    req.status_word = _ptr(status)
    open(dev.index)
    out = _partials_alloc(T, dev, False)
    o = A.llp_partials(_ptr(out["target_logit"]), _ptr(out["in_range"]), _ptr(out["lse"]), None,
                       _ptr(out["logp"]))
    _check(A.load().llp_top_p_replay(C.byref(req), C.byref(o), _stream_ptr(dev)),
           "llp_top_p_replay")
    return out


def forward_logits(logits: torch.Tensor, target_ids: torch.Tensor, *, temperature: float,
                   loss_mask: Optional[torch.Tensor] = None,
                   cu_seqlens: Optional[torch.Tensor] = None, offset: int = 0,
                   real_vocab: Optional[int] = None, padded_vocab: Optional[int] = None,
                   rank: int = 0, world: int = 1, want_entropy: bool = True,
                   status: Optional[torch.Tensor] = None,
                   local_size: Optional[int] = None) -> dict:
    """llp_forward_logits on one shard's unscaled local logits [T, local_size] (fp32 or bf16;
    a strided view of a wider tensor is fine). Returns the partials of ``forward``."""
    dev = logits.device
    if not isinstance(target_ids, torch.Tensor):
        raise TypeError("target_ids must be a torch.Tensor")
    _need(target_ids, "target_ids", torch.int64, 1, dev)
    T = target_ids.shape[0]
    dt, ld, local_size = _logits_view(logits, T, local_size, dev)
    req = A.llp_logits_request()
    req.logits = _ptr(logits)
    req.logits_dtype, req.logits_stride = dt, ld
    _vocab(req.vocab, offset, local_size, real_vocab, padded_vocab, rank, world)
    _covers_real(logits, "logits", req.vocab)
    req.layout.num_tokens = T
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, 1, dev)
        if cu_seqlens.shape[0] < 1:
            raise ValueError("cu_seqlens needs at least one entry")
        req.layout.cu_seqlens = _ptr(cu_seqlens)
        req.layout.num_seqs = cu_seqlens.shape[0] - 1
    if loss_mask is not None:
        _vec(loss_mask, "loss_mask", torch.uint8, T, dev)
        req.layout.loss_mask = _ptr(loss_mask)
    req.target_ids = _ptr(target_ids)
    req.temperature = float(temperature)
    req.flags = A.LLP_FLAG_WANT_ENTROPY if want_entropy else 0
    _status(status, dev)
    req.status_word = _ptr(status)
    open(dev.index)
    out = _partials_alloc(T, dev, want_entropy)
    o = A.llp_partials(_ptr(out["target_logit"]), _ptr(out["in_range"]), _ptr(out["lse"]),
                       _ptr(out["entropy"]), _ptr(out["logp"]))
    _check(A.load().llp_forward_logits(C.byref(req), C.byref(o), _stream_ptr(dev)),
           "llp_forward_logits")
    return out


def keep_mask_replay(logits: torch.Tensor, keep_mask: torch.Tensor, target_ids: torch.Tensor, *,
                     temperature: float, offset: int = 0, real_vocab: Optional[int] = None,
                     padded_vocab: Optional[int] = None, rank: int = 0, world: int = 1,
                     loss_mask: Optional[torch.Tensor] = None, processed_logprobs: bool = True,
                     status: Optional[torch.Tensor] = None,
                     local_size: Optional[int] = None) -> dict:
    """llp_keep_mask_replay on one shard: local logits [T, local_size] and a uint8 keep mask of
    the same shape (views of wider tensors are fine). Returns target_logit, in_range, lse,
    logp, as ``top_p_replay``."""
    dev = logits.device
    if not isinstance(target_ids, torch.Tensor):
        raise TypeError("target_ids must be a torch.Tensor")
    _need(target_ids, "target_ids", torch.int64, 1, dev)
    T = target_ids.shape[0]
    dt, ld, local_size = _logits_view(logits, T, local_size, dev)
    _need(keep_mask, "keep_mask", torch.uint8, 2, dev, (T, None))
    req = A.llp_keep_mask_request()
    req.logits = _ptr(logits)
    req.logits_dtype, req.logits_stride = dt, ld
    req.keep_mask = _ptr(keep_mask)
    req.keep_stride = keep_mask.stride(0) if T > 0 else local_size
    req.num_tokens = T
    _vocab(req.vocab, offset, local_size, real_vocab, padded_vocab, rank, world)
    _covers_real(logits, "logits", req.vocab)
    _covers_real(keep_mask, "keep_mask", req.vocab)
    req.target_ids = _ptr(target_ids)
    if loss_mask is not None:
        _vec(loss_mask, "loss_mask", torch.uint8, T, dev)
        req.loss_mask = _ptr(loss_mask)
    req.temperature = float(temperature)
    req.processed_logprobs = 1 if processed_logprobs else 0
    _status(status, dev)
    req.status_word = _ptr(status)
    open(dev.index)
    out = _partials_alloc(T, dev, False)
    del out["entropy"]
    o = A.llp_partials(_ptr(out["target_logit"]), _ptr(out["in_range"]), _ptr(out["lse"]), None,
                       _ptr(out["logp"]))
    _check(A.load().llp_keep_mask_replay(C.byref(req), C.byref(o), _stream_ptr(dev)),
           "llp_keep_mask_replay")
    return out


class _LinearLogp(torch.autograd.Function):
    """forward + backward of one full-vocabulary shard as an autograd node (world = 1)."""

    @staticmethod
    def forward(ctx, hidden, weight, bias, target_ids, loss_mask, temperature, real_vocab,
                padded_vocab, want_entropy, g_slabs):
        out = forward(hidden, weight, target_ids, temperature=temperature, bias=bias,
                      loss_mask=loss_mask, real_vocab=real_vocab, padded_vocab=padded_vocab,
                      want_entropy=want_entropy)
        ctx.save_for_backward(hidden, weight, bias, target_ids, loss_mask, out["lse"],
                              out["entropy"])
        ctx.cfg = (temperature, real_vocab, padded_vocab, g_slabs)
        ctx.mark_non_differentiable(out["lse"])
        ent = out["entropy"] if want_entropy else out["lse"].new_zeros(0)
        return out["logp"], ent, out["lse"]

    @staticmethod
    def backward(ctx, dlogp, dentropy, _dlse):
        hidden, weight, bias, target_ids, loss_mask, lse, entropy = ctx.saved_tensors
        temperature, real_vocab, padded_vocab, g_slabs = ctx.cfg
        T = hidden.shape[0]
        if dlogp is None:
            dlogp = torch.zeros(T, dtype=torch.float32, device=hidden.device)
        use_ent = dentropy is not None and entropy is not None and dentropy.numel() == T
        g = backward(hidden, weight, target_ids, lse, dlogp.float().contiguous(),
                     temperature=temperature, bias=bias, loss_mask=loss_mask,
                     real_vocab=real_vocab, padded_vocab=padded_vocab,
                     dentropy=dentropy.float().contiguous() if use_ent else None,
                     entropy=entropy if use_ent else None, overwrite=True,
                     want_dbias=bias is not None and ctx.needs_input_grad[2], g_slabs=g_slabs)
        dW = g["dweight"].to(weight.dtype) if ctx.needs_input_grad[1] else None
        db = g["dbias"].to(bias.dtype) if bias is not None and ctx.needs_input_grad[2] else None
        dH = g["dhidden"] if ctx.needs_input_grad[0] else None
        return dH, dW, db, None, None, None, None, None, None, None


def linear_logp(hidden: torch.Tensor, weight: torch.Tensor, target_ids: torch.Tensor, *,
                temperature: float, bias: Optional[torch.Tensor] = None,
                loss_mask: Optional[torch.Tensor] = None, real_vocab: Optional[int] = None,
                padded_vocab: Optional[int] = None, want_entropy: bool = True,
                g_slabs: bool = False):
    """Per-token log-probability of target_ids (and entropy) under softmax((h W^T + b) / tau)
    over the real vocabulary, differentiable in hidden, weight and bias: the operator's
    forward, and in autograd's backward pass its backward with the incoming dlogp/dentropy
    ([CUDA provider, "Motivation"]: gradients must flow). One full-vocabulary shard (world = 1).
    Returns (logp, entropy, lse); entropy is an empty tensor when want_entropy is False, and
    lse carries no gradient. Rows with loss_mask 0 give logp = entropy = 0 and no gradient.
    The weight and bias gradients are computed in fp32 and handed to autograd in the
    parameters' dtype. g_slabs: the backward holds G one vocabulary slab at a time
    (LLP_FLAG_G_SLABS)."""
    if loss_mask is not None and loss_mask.dtype == torch.bool:
        loss_mask = loss_mask.to(torch.uint8)
    return _LinearLogp.apply(hidden, weight, bias, target_ids, loss_mask, temperature,
                             real_vocab, padded_vocab, want_entropy, g_slabs)
