"""Host-side checks of the C ABI (no GPU needed).

* the library loads and exports every function include/llp.h declares;
* the ctypes mirror has the header's struct sizes and field offsets (gcc-compiled probe);
* malformed requests are rejected with LLP_ERR_INVALID_ARGUMENT / LLP_ERR_UNSUPPORTED before
  anything touches a device; llp_open without a gfx950 device returns LLP_ERR_UNAVAILABLE;
* llp_workspace_bytes is a pure function of the shapes.
"""
import ctypes as C
import os
import re
import subprocess

import pytest

from lm_head_linear_logp_amd import _capi as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llp.h")

pytestmark = pytest.mark.skipif(not os.path.exists(A.LIB_PATH),
                                reason="libllp.so not built (python -m lm_head_linear_logp_amd.build)")

FAKE = 0x100000  # aligned, never dereferenced by validation


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"LLP_API\s+[\w\s\*]+?\b(llp_\w+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(A.SIGNATURES), names
    lib = C.CDLL(A.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


STRUCTS = ["llp_info", "llp_projection", "llp_vocab_partition", "llp_token_layout",
           "llp_request", "llp_partials", "llp_final_out", "llp_bwd_in", "llp_bwd_out",
           "llp_topp_request", "llp_logits_request", "llp_keep_mask_request"]


def test_ctypes_mirror_matches_header(tmp_path):
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "llp.h"', "int main(void){"]
    for s in STRUCTS:
        lines.append(f'printf("{s} size %zu\\n", sizeof({s}));')
        for f, _ in getattr(A, s)._fields_:
            lines.append(f'printf("{s} {f} %zu\\n", offsetof({s}, {f}));')
    lines.append("return 0;}")
    src = tmp_path / "probe.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    got = {}
    for ln in out.splitlines():
        s, f, v = ln.split()
        got[(s, f)] = int(v)
    for s in STRUCTS:
        cs = getattr(A, s)
        assert got[(s, "size")] == C.sizeof(cs), s
        for f, _ in cs._fields_:
            assert got[(s, f)] == getattr(cs, f).offset, (s, f)


def test_header_constants_match():
    src = open(HEADER).read()
    for name in ("LLP_MAX_REPLAY_IDS", "LLP_MAX_WORLD", "LLP_G_SLAB_COLUMNS"):
        assert int(re.search(rf"#define {name} (\d+)", src).group(1)) == getattr(A, name)
    for name in ("LLP_STATUS_TARGET_OUT_OF_RANGE", "LLP_STATUS_TARGET_NOT_FOUND",
                 "LLP_STATUS_REPLAY_ID_INVALID", "LLP_STATUS_LAYOUT_INVALID",
                 "LLP_ERR_UNAVAILABLE", "LLP_ERR_INVALID_ARGUMENT", "LLP_ERR_UNSUPPORTED",
                 "LLP_DTYPE_BF16", "LLP_DTYPE_F32", "LLP_OP_FORWARD", "LLP_OP_BACKWARD",
                 "LLP_FLAG_WANT_ENTROPY", "LLP_FLAG_OVERWRITE_GRADS", "LLP_FLAG_G_SLABS"):
        assert int(re.search(rf"\b{name} = (\d+)", src).group(1)) == getattr(A, name), name


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_gpu_present(), reason="a GPU is present")
def test_open_without_device_is_unavailable():
    lib = A.load()
    info = A.llp_info()
    assert lib.llp_open(0, C.byref(info)) == A.LLP_ERR_UNAVAILABLE
    assert lib.llp_last_error()


def good_request(T=4096, H=4096, V=151936, Vr=151669):
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


def good_out():
    return A.llp_partials(FAKE, FAKE, FAKE, FAKE, FAKE)


def call_forward(req, out=None, ws_bytes=1 << 40, ws=FAKE):
    lib = A.load()
    return lib.llp_forward(C.byref(req), C.byref(out or good_out()), ws, ws_bytes, None)


def _mut(fn):
    r = good_request()
    fn(r)
    return r


BAD_FORWARD = [
    ("negative T", lambda r: setattr(r.layout, "num_tokens", -1), A.LLP_ERR_INVALID_ARGUMENT),
    ("H not multiple of 64", lambda r: (setattr(r.proj, "hidden_size", 4000),
                                        setattr(r.proj, "hidden_stride", 4000),
                                        setattr(r.proj, "weight_stride", 4000)), A.LLP_ERR_UNSUPPORTED),
    ("hidden stride < H", lambda r: setattr(r.proj, "hidden_stride", 4095), A.LLP_ERR_INVALID_ARGUMENT),
    ("weight stride odd", lambda r: setattr(r.proj, "weight_stride", 4097), A.LLP_ERR_INVALID_ARGUMENT),
    ("hidden misaligned", lambda r: setattr(r.proj, "hidden", FAKE + 2), A.LLP_ERR_INVALID_ARGUMENT),
    ("weight NULL", lambda r: setattr(r.proj, "weight", None), A.LLP_ERR_INVALID_ARGUMENT),
    ("targets NULL", lambda r: setattr(r, "target_ids", None), A.LLP_ERR_INVALID_ARGUMENT),
    ("tau zero", lambda r: setattr(r, "temperature", 0.0), A.LLP_ERR_INVALID_ARGUMENT),
    ("tau negative", lambda r: setattr(r, "temperature", -1.0), A.LLP_ERR_INVALID_ARGUMENT),
    ("tau nan", lambda r: setattr(r, "temperature", float("nan")), A.LLP_ERR_INVALID_ARGUMENT),
    ("tau inf", lambda r: setattr(r, "temperature", float("inf")), A.LLP_ERR_INVALID_ARGUMENT),
    ("real > padded", lambda r: setattr(r.vocab, "real_vocab", 151937), A.LLP_ERR_INVALID_ARGUMENT),
    ("real zero", lambda r: setattr(r.vocab, "real_vocab", 0), A.LLP_ERR_INVALID_ARGUMENT),
    ("world1 partial shard", lambda r: setattr(r.vocab, "local_size", 1000), A.LLP_ERR_INVALID_ARGUMENT),
    ("shard past padded", lambda r: (setattr(r.vocab, "world", 4), setattr(r.vocab, "offset", 120000),
                                     setattr(r.vocab, "local_size", 37984)), A.LLP_ERR_INVALID_ARGUMENT),
    ("rank >= world", lambda r: (setattr(r.vocab, "world", 4), setattr(r.vocab, "rank", 4),
                                 setattr(r.vocab, "local_size", 37984)), A.LLP_ERR_INVALID_ARGUMENT),
    ("world too big", lambda r: setattr(r.vocab, "world", 65), A.LLP_ERR_INVALID_ARGUMENT),
    ("bad bias dtype", lambda r: (setattr(r.proj, "bias", FAKE), setattr(r.proj, "bias_dtype", 7)),
     A.LLP_ERR_INVALID_ARGUMENT),
    ("unknown flag", lambda r: setattr(r, "flags", 8), A.LLP_ERR_INVALID_ARGUMENT),
    ("T too large", lambda r: setattr(r.layout, "num_tokens", 1 << 23), A.LLP_ERR_UNSUPPORTED),
    ("hidden bytes > 4 GiB", lambda r: (setattr(r.layout, "num_tokens", 1 << 20),
                                        setattr(r.proj, "hidden_stride", 4096)), A.LLP_ERR_UNSUPPORTED),
    ("weight stride >= 2^23", lambda r: setattr(r.proj, "weight_stride", 1 << 23), A.LLP_ERR_UNSUPPORTED),
    ("H > 2^20", lambda r: (setattr(r.layout, "num_tokens", 8),
                            setattr(r.proj, "hidden_size", (1 << 20) + 64),
                            setattr(r.proj, "hidden_stride", (1 << 20) + 64),
                            setattr(r.proj, "weight_stride", (1 << 20) + 64)), A.LLP_ERR_UNSUPPORTED),
    ("local size 2^23 - 192", lambda r: (setattr(r.vocab, "padded_vocab", (1 << 23) - 192),
                                         setattr(r.vocab, "local_size", (1 << 23) - 192),
                                         setattr(r.vocab, "real_vocab", 1000)), A.LLP_ERR_UNSUPPORTED),
    ("shard too large", lambda r: (setattr(r.vocab, "padded_vocab", 1 << 24), setattr(r.vocab, "local_size", 1 << 24),
                                   setattr(r.vocab, "real_vocab", 1 << 24)), A.LLP_ERR_UNSUPPORTED),
    ("f32 bias misaligned", lambda r: (setattr(r.proj, "bias", FAKE + 8),
                                       setattr(r.proj, "bias_dtype", A.LLP_DTYPE_F32)),
     A.LLP_ERR_INVALID_ARGUMENT),
    ("bf16 bias misaligned", lambda r: (setattr(r.proj, "bias", FAKE + 4),
                                        setattr(r.proj, "bias_dtype", A.LLP_DTYPE_BF16)),
     A.LLP_ERR_INVALID_ARGUMENT),
]


@pytest.mark.parametrize("name,fn,code", BAD_FORWARD, ids=[b[0] for b in BAD_FORWARD])
def test_forward_rejects_malformed_request(name, fn, code):
    assert call_forward(_mut(fn)) == code
    assert A.load().llp_last_error()


def test_forward_rejects_bad_outputs_and_workspace():
    r = good_request()
    assert call_forward(r, A.llp_partials(None, FAKE, FAKE, FAKE, FAKE)) == A.LLP_ERR_INVALID_ARGUMENT
    r.flags = A.LLP_FLAG_WANT_ENTROPY
    assert call_forward(r, A.llp_partials(FAKE, FAKE, FAKE, None, FAKE)) == A.LLP_ERR_INVALID_ARGUMENT
    r.layout.num_tokens = 0          # no rows: output pointers may be NULL
    assert call_forward(r, A.llp_partials(None, None, None, None, None)) != A.LLP_ERR_INVALID_ARGUMENT
    r.layout.num_tokens = 4096
    r.flags = 0
    assert call_forward(r, ws_bytes=1000) == A.LLP_ERR_INVALID_ARGUMENT
    assert call_forward(r, ws=FAKE + 16) == A.LLP_ERR_INVALID_ARGUMENT
    lib = A.load()
    assert lib.llp_forward(None, C.byref(good_out()), FAKE, 1 << 40, None) == A.LLP_ERR_INVALID_ARGUMENT


@pytest.mark.skipif(_gpu_present(), reason="a GPU is present")
def test_valid_request_passes_validation():
    """A well-formed request gets past validation; without a device it fails afterwards."""
    st = call_forward(good_request())
    assert st not in (A.LLP_OK, A.LLP_ERR_INVALID_ARGUMENT) or "llp_open" in A.load().llp_last_error().decode()


def test_requests_at_the_limits_pass_validation():
    """H = 2^20 and a local vocabulary of 2^23 - 256 columns are inside the envelope: such
    requests get past validation (one column or one 64-column step more is refused above)."""
    def at_h_limit(r):
        r.layout.num_tokens = 8
        r.proj.hidden_size = r.proj.hidden_stride = r.proj.weight_stride = 1 << 20

    def at_local_size_limit(r):
        r.vocab.padded_vocab = r.vocab.local_size = (1 << 23) - 256
        r.vocab.real_vocab = 1000

    for fn in (at_h_limit, at_local_size_limit):
        st = call_forward(_mut(fn))
        assert st not in (A.LLP_ERR_INVALID_ARGUMENT, A.LLP_ERR_UNSUPPORTED), \
            A.load().llp_last_error()


def _ws_status(T, stride):
    r = good_request(H=256, V=1024, Vr=1000)
    r.layout.num_tokens, r.proj.hidden_stride = T, stride
    n = C.c_size_t()
    return A.load().llp_workspace_bytes(C.byref(r), A.LLP_OP_FORWARD, C.byref(n))


def test_hidden_byte_bound_is_strict():
    """The T hidden rows must span fewer than 2^31 bytes (32-bit offsets from a tile's first
    row): exactly 2^31 is refused, one row less is accepted."""
    assert _ws_status(1 << 22, 256) == A.LLP_ERR_UNSUPPORTED          # 2^22 * 256 * 2 = 2^31
    assert _ws_status((1 << 22) - 1, 256) == A.LLP_OK
    assert _ws_status(1 << 21, 512) == A.LLP_ERR_UNSUPPORTED
    assert _ws_status((1 << 21) - 1, 512) == A.LLP_OK


def test_workspace_bytes_pure_function():
    lib = A.load()
    n1, n2 = C.c_size_t(), C.c_size_t()
    r = good_request()
    assert lib.llp_workspace_bytes(C.byref(r), A.LLP_OP_FORWARD, C.byref(n1)) == A.LLP_OK
    assert lib.llp_workspace_bytes(C.byref(r), A.LLP_OP_FORWARD, C.byref(n2)) == A.LLP_OK
    assert n1.value == n2.value
    # 593 vocabulary tiles x 4096 rows x 3 fp32 partials dominate the forward workspace.
    assert 593 * 4096 * 12 <= n1.value < 593 * 4096 * 12 + (1 << 20)
    nb = C.c_size_t()
    assert lib.llp_workspace_bytes(C.byref(r), A.LLP_OP_BACKWARD, C.byref(nb)) == A.LLP_OK
    assert nb.value >= 4096 * 593 * 256 * 2          # the bf16 G buffer
    assert lib.llp_workspace_bytes(C.byref(r), 3, C.byref(nb)) == A.LLP_ERR_INVALID_ARGUMENT


def test_slab_flag_sizes_g_for_one_slab():
    """LLP_FLAG_G_SLABS: the backward workspace holds G for one slab of LLP_G_SLAB_COLUMNS
    columns; the forward's workspace does not depend on it, nor does a shard of one slab."""
    lib = A.load()

    def ws(r, op):
        n = C.c_size_t()
        assert lib.llp_workspace_bytes(C.byref(r), op, C.byref(n)) == A.LLP_OK
        return n.value
    r = good_request()
    full_b, full_f = ws(r, A.LLP_OP_BACKWARD), ws(r, A.LLP_OP_FORWARD)
    r.flags = A.LLP_FLAG_G_SLABS
    slab_b = ws(r, A.LLP_OP_BACKWARD)
    assert ws(r, A.LLP_OP_FORWARD) == full_f
    g_full, g_slab = 4096 * 594 * 256 * 2, 4096 * A.LLP_G_SLAB_COLUMNS * 2
    assert full_b - slab_b >= g_full - g_slab - (1 << 16)
    assert slab_b < full_b / 3
    small = good_request(V=A.LLP_G_SLAB_COLUMNS, Vr=A.LLP_G_SLAB_COLUMNS - 5)
    a = ws(small, A.LLP_OP_BACKWARD)
    small.flags = A.LLP_FLAG_G_SLABS
    assert ws(small, A.LLP_OP_BACKWARD) == a


def _merge(world, parts, T=16, out=None):
    lib = A.load()
    arr = (A.llp_partials * max(world, 1))(*parts) if parts else None
    fo = out or A.llp_final_out(FAKE, FAKE, None)
    return lib.llp_merge(world, arr, T, None, C.byref(fo), None, None)


def test_merge_validation():
    p = A.llp_partials(FAKE, FAKE, FAKE, None, None)
    assert _merge(0, [p]) == A.LLP_ERR_INVALID_ARGUMENT
    assert _merge(65, [p] * 65) == A.LLP_ERR_INVALID_ARGUMENT
    assert _merge(2, [p, A.llp_partials(FAKE, None, FAKE, None, None)]) == A.LLP_ERR_INVALID_ARGUMENT
    # entropy requested but a part has none
    assert _merge(2, [p, p], out=A.llp_final_out(FAKE, FAKE, FAKE)) == A.LLP_ERR_INVALID_ARGUMENT
    assert _merge(1, [p], out=A.llp_final_out(None, FAKE, None)) == A.LLP_ERR_INVALID_ARGUMENT
    # more rows than one launch grid covers
    assert _merge(1, [p], T=1 << 31) == A.LLP_ERR_INVALID_ARGUMENT


def good_topp():
    q = A.llp_topp_request()
    q.logits, q.logits_dtype, q.num_replay, q.logits_stride = FAKE, A.LLP_DTYPE_F32, 64, 151936
    q.num_tokens = 4096
    q.vocab.offset, q.vocab.local_size, q.vocab.real_vocab, q.vocab.padded_vocab = 0, 151936, 151669, 151936
    q.vocab.rank, q.vocab.world = 0, 1
    q.replay_ids, q.replay_stride, q.target_ids = FAKE, 64, FAKE
    q.temperature, q.processed_logprobs = 0.7, 1
    return q


BAD_TOPP = [
    ("raw logprobs mode", lambda q: setattr(q, "processed_logprobs", 0)),
    ("K = 65", lambda q: (setattr(q, "num_replay", 65), setattr(q, "replay_stride", 65))),
    ("K = 0", lambda q: setattr(q, "num_replay", 0)),
    ("replay stride < K", lambda q: setattr(q, "replay_stride", 32)),
    ("bad dtype", lambda q: setattr(q, "logits_dtype", 9)),
    ("logits stride < local", lambda q: setattr(q, "logits_stride", 1000)),
    ("tau zero", lambda q: setattr(q, "temperature", 0.0)),
    ("ids NULL", lambda q: setattr(q, "replay_ids", None)),
    ("bad partition", lambda q: setattr(q.vocab, "real_vocab", 200000)),
    ("T = 2^31 (grid limit)", lambda q: setattr(q, "num_tokens", 1 << 31)),
    ("T < 0", lambda q: setattr(q, "num_tokens", -1)),
]


@pytest.mark.parametrize("name,fn", BAD_TOPP, ids=[b[0] for b in BAD_TOPP])
def test_topp_rejects_malformed_request(name, fn):
    q = good_topp()
    fn(q)
    o = A.llp_partials(FAKE, FAKE, FAKE, None, FAKE)
    assert A.load().llp_top_p_replay(C.byref(q), C.byref(o), None) == A.LLP_ERR_INVALID_ARGUMENT


def test_topp_rejects_entropy_output():
    q = good_topp()
    o = A.llp_partials(FAKE, FAKE, FAKE, FAKE, FAKE)
    assert A.load().llp_top_p_replay(C.byref(q), C.byref(o), None) == A.LLP_ERR_INVALID_ARGUMENT


def test_backward_validation():
    lib = A.load()
    r = good_request()
    bi = A.llp_bwd_in(FAKE, FAKE, None, None)
    bo = A.llp_bwd_out(FAKE, 4096, FAKE, 4096, None)
    call = lambda: lib.llp_backward(C.byref(r), C.byref(bi), C.byref(bo), FAKE, 1 << 40, None)
    bi.dentropy = FAKE   # dentropy without entropy
    assert call() == A.LLP_ERR_INVALID_ARGUMENT
    bi.dentropy = None
    bo.dhidden_stride = 100
    assert call() == A.LLP_ERR_INVALID_ARGUMENT
    bo.dhidden_stride = 4096
    bo.dweight = None
    assert call() == A.LLP_ERR_INVALID_ARGUMENT
    bo.dweight = FAKE
    bi.lse = None
    assert call() == A.LLP_ERR_INVALID_ARGUMENT


@pytest.mark.skipif(_gpu_present(), reason="a GPU is present")
def test_backward_overwrite_flag_passes_validation():
    """LLP_FLAG_OVERWRITE_GRADS is a known request flag: a backward request carrying it gets
    past validation (without a device it then fails in llp_open's check); flag 4 is unknown."""
    lib = A.load()
    r = good_request()
    bi = A.llp_bwd_in(FAKE, FAKE, None, None)
    bo = A.llp_bwd_out(FAKE, 4096, FAKE, 4096, None)
    call = lambda: lib.llp_backward(C.byref(r), C.byref(bi), C.byref(bo), FAKE, 1 << 40, None)
    r.flags = A.LLP_FLAG_OVERWRITE_GRADS
    st = call()
    assert st != A.LLP_ERR_INVALID_ARGUMENT or "llp_open" in lib.llp_last_error().decode()
    r.flags = A.LLP_FLAG_OVERWRITE_GRADS | A.LLP_FLAG_G_SLABS
    st = call()
    assert st != A.LLP_ERR_INVALID_ARGUMENT or "llp_open" in lib.llp_last_error().decode()
    r.flags = 8
    assert call() == A.LLP_ERR_INVALID_ARGUMENT
    assert b"unknown flags" in lib.llp_last_error()


def test_backward_rejects_bad_dweight_layout():
    lib = A.load()
    r = good_request()
    bi = A.llp_bwd_in(FAKE, FAKE, None, None)
    call = lambda bo: lib.llp_backward(C.byref(r), C.byref(bi), C.byref(bo), FAKE, 1 << 40, None)
    # stride not a multiple of 4, misaligned base, stride beyond the 32-bit offset envelope
    assert call(A.llp_bwd_out(FAKE, 4096, FAKE, 4098, None)) == A.LLP_ERR_INVALID_ARGUMENT
    assert call(A.llp_bwd_out(FAKE, 4096, FAKE + 4, 4096, None)) == A.LLP_ERR_INVALID_ARGUMENT
    assert call(A.llp_bwd_out(FAKE, 4096, FAKE, 1 << 21, None)) == A.LLP_ERR_UNSUPPORTED


def good_logits_request(T=16, V=1000, Vp=1024):
    r = A.llp_logits_request()
    r.logits, r.logits_dtype, r.logits_stride = FAKE, A.LLP_DTYPE_F32, Vp
    r.vocab.offset, r.vocab.local_size, r.vocab.real_vocab, r.vocab.padded_vocab = 0, Vp, V, Vp
    r.vocab.rank, r.vocab.world = 0, 1
    r.layout.num_tokens = T
    r.target_ids = FAKE
    r.temperature = 0.7
    return r


def good_keep_request(T=16, V=1000, Vp=1024):
    r = A.llp_keep_mask_request()
    r.logits, r.logits_dtype, r.logits_stride = FAKE, A.LLP_DTYPE_F32, Vp
    r.keep_mask, r.keep_stride = FAKE, Vp
    r.num_tokens = T
    r.vocab.offset, r.vocab.local_size, r.vocab.real_vocab, r.vocab.padded_vocab = 0, Vp, V, Vp
    r.vocab.rank, r.vocab.world = 0, 1
    r.target_ids = FAKE
    r.temperature = 0.7
    r.processed_logprobs = 1
    return r


BAD_LOGITS = [
    ("dtype", lambda r: setattr(r, "logits_dtype", 9)),
    ("stride < local_size", lambda r: setattr(r, "logits_stride", 1000)),
    ("misaligned base", lambda r: setattr(r, "logits", FAKE + 8)),
    ("f32 stride not 16-byte rows", lambda r: setattr(r, "logits_stride", 1026)),
    ("tau zero", lambda r: setattr(r, "temperature", 0.0)),
    ("unknown flag", lambda r: setattr(r, "flags", 8)),
    ("targets NULL", lambda r: setattr(r, "target_ids", None)),
    ("real > padded", lambda r: setattr(r.vocab, "real_vocab", 2000)),
    ("T = 2^31 (grid limit)", lambda r: setattr(r.layout, "num_tokens", 1 << 31)),
]


@pytest.mark.parametrize("name,fn", BAD_LOGITS, ids=[b[0] for b in BAD_LOGITS])
def test_forward_logits_rejects_malformed_request(name, fn):
    r = good_logits_request()
    fn(r)
    o = A.llp_partials(FAKE, FAKE, FAKE, None, FAKE)
    assert A.load().llp_forward_logits(C.byref(r), C.byref(o), None) == A.LLP_ERR_INVALID_ARGUMENT
    assert A.load().llp_last_error()


def test_forward_logits_entropy_output_must_match_flag():
    r = good_logits_request()
    o = A.llp_partials(FAKE, FAKE, FAKE, FAKE, FAKE)            # entropy given, not wanted
    assert A.load().llp_forward_logits(C.byref(r), C.byref(o), None) == A.LLP_ERR_INVALID_ARGUMENT
    r.flags = A.LLP_FLAG_WANT_ENTROPY
    o = A.llp_partials(FAKE, FAKE, FAKE, None, FAKE)            # wanted, not given
    assert A.load().llp_forward_logits(C.byref(r), C.byref(o), None) == A.LLP_ERR_INVALID_ARGUMENT


def test_new_entry_points_valid_requests_pass_validation():
    """Well-formed requests get past validation; without a device they fail afterwards."""
    o = A.llp_partials(FAKE, FAKE, FAKE, None, FAKE)
    for st in (A.load().llp_forward_logits(C.byref(good_logits_request()), C.byref(o), None),
               A.load().llp_keep_mask_replay(C.byref(good_keep_request()), C.byref(o), None)):
        assert st not in (A.LLP_OK, A.LLP_ERR_INVALID_ARGUMENT) or \
            "llp_open" in A.load().llp_last_error().decode()


BAD_KEEP = [
    ("raw logprobs", lambda r: setattr(r, "processed_logprobs", 0)),
    ("keep stride < local_size", lambda r: setattr(r, "keep_stride", 1000)),
    ("keep stride not 16", lambda r: setattr(r, "keep_stride", 1032 + 4)),
    ("keep misaligned", lambda r: setattr(r, "keep_mask", FAKE + 4)),
    ("logits misaligned", lambda r: setattr(r, "logits", FAKE + 2)),
    ("dtype", lambda r: setattr(r, "logits_dtype", 0)),
    ("tau nan", lambda r: setattr(r, "temperature", float("nan"))),
    ("keep NULL", lambda r: setattr(r, "keep_mask", None)),
    ("T = 2^31 (grid limit)", lambda r: setattr(r, "num_tokens", 1 << 31)),
]


@pytest.mark.parametrize("name,fn", BAD_KEEP, ids=[b[0] for b in BAD_KEEP])
def test_keep_mask_replay_rejects_malformed_request(name, fn):
    r = good_keep_request()
    fn(r)
    o = A.llp_partials(FAKE, FAKE, FAKE, None, FAKE)
    assert A.load().llp_keep_mask_replay(C.byref(r), C.byref(o), None) == A.LLP_ERR_INVALID_ARGUMENT


def test_keep_mask_replay_rejects_entropy_output():
    r = good_keep_request()
    o = A.llp_partials(FAKE, FAKE, FAKE, FAKE, FAKE)
    assert A.load().llp_keep_mask_replay(C.byref(r), C.byref(o), None) == A.LLP_ERR_INVALID_ARGUMENT


def test_partition_offset_near_int64_max_is_refused():
    """offset + local_size past the int64 range is refused, not overflowed."""
    r = good_request()
    r.vocab.world, r.vocab.offset, r.vocab.local_size = 2, (1 << 63) - 6, 100
    n = C.c_size_t()
    assert A.load().llp_workspace_bytes(C.byref(r), A.LLP_OP_FORWARD, C.byref(n)) == \
        A.LLP_ERR_INVALID_ARGUMENT
