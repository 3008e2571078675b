"""ctypes binding of libspecdec.so with the C ABI's names.

Argument marshalling only: shape checks, output/workspace allocation when the
caller does not pass them, and the current torch stream.  Every step of the
method runs in the library's HIP kernels.
"""
import contextlib
import ctypes
import functools
import os

import torch

SPEC_F32 = 0
SPEC_BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libspecdec.so")
_lib = None


class SpecError(RuntimeError):
    pass


def library_path():
    return _LIB_PATH


def load_library():
    """Load libspecdec.so (built by __graft_entry__.build()).  Raises if it is
    missing: there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise SpecError(f"{_LIB_PATH} is missing: build the HIP library first "
                        "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, u64, u32, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                  ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t)
    lib.spec_version.restype = i32
    lib.spec_last_error.restype = ctypes.c_char_p
    lib.spec_philox_uniforms.argtypes = [u64, u32, u32, i32, i32, vp, vp]
    lib.spec_philox_uniforms.restype = i32
    lib.spec_draft_markov_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.spec_draft_markov_workspace_size.restype = sz
    lib.spec_draft_sample_markov.argtypes = [vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                             f32, vp, u64, u32, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_draft_sample_markov.restype = i32
    lib.spec_draft_rnn_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.spec_draft_rnn_workspace_size.restype = sz
    lib.spec_draft_sample_rnn.argtypes = [vp, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, i32,
                                          i32, i32, i32, i32, f32, vp, u64, u32, vp, vp, vp, vp,
                                          vp, sz, vp]
    lib.spec_draft_sample_rnn.restype = i32
    lib.spec_verify_workspace_size.argtypes = [i32, i32, i32]
    lib.spec_verify_workspace_size.restype = sz
    lib.spec_verify.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, i32, i32, i32, f32, vp, u64,
                                u32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_verify.restype = i32
    lib.spec_verify_noalloc_max_bytes.argtypes = []
    lib.spec_verify_noalloc_max_bytes.restype = sz
    lib.spec_verify_noalloc.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, i32, i32, i32, f32, vp,
                                        u64, u32, vp, vp, vp, vp, vp, vp]
    lib.spec_verify_noalloc.restype = i32
    lib.spec_pack_w2_bytes.argtypes = [i32, i32]
    lib.spec_pack_w2_bytes.restype = sz
    lib.spec_pack_w2.argtypes = [vp, vp, i32, i32, vp]
    lib.spec_pack_w2.restype = i32
    lib.spec_verify_markov_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.spec_verify_markov_workspace_size.restype = sz
    lib.spec_verify_markov.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, i32, i32, vp, vp, vp,
                                       vp, vp, i32, i32, i32, f32, vp, u64, u32, vp, vp, vp, vp,
                                       vp, sz, vp]
    lib.spec_verify_markov.restype = i32
    lib.spec_draft_set_persistent.argtypes = [i32]
    lib.spec_draft_set_persistent.restype = i32
    lib.spec_acceptance_rate.argtypes = [vp, i32, vp, i32, vp, vp, vp, i32, i32, i32, f32, vp,
                                         vp, vp]
    lib.spec_acceptance_rate.restype = i32
    lib.spec_confidence_head.argtypes = [vp, i32, i32, vp, vp, vp, i32, i32, vp, i32, i32, i32,
                                         vp, vp]
    lib.spec_confidence_head.restype = i32
    lib.spec_prefix_schedule_workspace_size.argtypes = [i32, i32]
    lib.spec_prefix_schedule_workspace_size.restype = sz
    lib.spec_prefix_schedule.argtypes = [vp, i32, i32, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.spec_prefix_schedule.restype = i32
    lib.spec_tree_select.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    lib.spec_tree_select.restype = i32
    lib.spec_draft_rnn_cond_offset.argtypes = [i32, i32, i32, i32, i32]
    lib.spec_draft_rnn_cond_offset.restype = sz
    lib.spec_verify_rnn_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.spec_verify_rnn_workspace_size.restype = sz
    lib.spec_verify_rnn.argtypes = [vp, i32, vp, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, i32,
                                    i32, i32, f32, vp, u64, u32, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_rnn.restype = i32
    lib.spec_verify_tree.argtypes = [vp, i32, vp, i32, vp, vp, vp, i32, i32, i32, f32, vp, u64,
                                     u32, vp, vp, vp, vp]
    lib.spec_verify_tree.restype = i32
    lib.spec_draft_status.argtypes = [vp, sz, i32, i32, i32, i32, vp, vp]
    lib.spec_draft_status.restype = i32
    lib.spec_draft_set_poll_limit.argtypes = [u32]
    lib.spec_draft_set_poll_limit.restype = u32
    lib.spec_profile_enable.argtypes = [ctypes.c_char_p]
    lib.spec_profile_enable.restype = i32
    lib.spec_profile_read.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_double)]
    lib.spec_profile_read.restype = i32
    _lib = lib
    return lib


def spec_version():
    return load_library().spec_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t, name):
    if t.dtype == torch.float32:
        return SPEC_F32
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    raise SpecError(f"{name} must be float32 or bfloat16, got {t.dtype}")


def _dev(t, name):
    if not (t.is_cuda and t.is_contiguous()):
        raise SpecError(f"{name} must be a contiguous device tensor")
    return t


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run a wrapper with its `stream` as torch's current stream, so that the
    outputs and the workspace it allocates belong to the stream the library
    enqueues on: torch's caching allocator then hands their memory to a later
    allocation only in that stream's order (a workspace freed when the wrapper
    returns is not reused by another stream while the kernels still run)."""
    @functools.wraps(fn)
    def wrapped(*args, stream=None, **kw):
        ctx = contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)
        with ctx:
            return fn(*args, stream=stream, **kw)
    return wrapped


def _check(st, what):
    if st != 0:
        msg = load_library().spec_last_error().decode()
        raise SpecError(f"{what} failed with status {st}: {msg}")


def workspace_bytes(kind, **dims):
    lib = load_library()
    if kind == "markov":
        return lib.spec_draft_markov_workspace_size(dims["B"], dims["gamma"], dims["V"], dims["r"])
    if kind == "rnn":
        return lib.spec_draft_rnn_workspace_size(dims["B"], dims["gamma"], dims["V"], dims["r"],
                                                 dims["d"])
    if kind == "verify":
        return lib.spec_verify_workspace_size(dims["B"], dims["gamma_max"], dims["V"])
    if kind == "verify_markov":
        return lib.spec_verify_markov_workspace_size(dims["B"], dims["gamma_max"], dims["V"],
                                                     dims["r"])
    raise ValueError(kind)


def _workspace(nbytes, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() < nbytes:
        raise SpecError(f"workspace too small: {ws.numel()} < {nbytes}")
    return ws, ws.numel()


@_on_stream
def spec_philox_uniforms(seed, offset, stream_id, B, K, device="cuda", out=None, stream=None):
    """[B, K] float32 uniforms u(seed, offset, b, k, stream_id)."""
    lib = load_library()
    out = torch.empty((B, K), dtype=torch.float32, device=device) if out is None else out
    _check(lib.spec_philox_uniforms(seed, offset, stream_id, B, K, _ptr(out), _stream(stream)),
           "spec_philox_uniforms")
    return out


def _draft_outputs(B, gamma, V, device, out, q_free=False):
    if out is not None:
        return out
    o = dict(tokens=torch.empty((B, gamma), dtype=torch.int32, device=device),
             q_logZ=torch.empty((B, gamma), dtype=torch.float32, device=device),
             q_tok_prob=torch.empty((B, gamma), dtype=torch.float32, device=device))
    if not q_free:
        o["q_logits"] = torch.empty((B, gamma, V), dtype=torch.float32, device=device)
    return o


def spec_pack_w2_bytes(r, V):
    return load_library().spec_pack_w2_bytes(r, V)


@_on_stream
def spec_pack_w2(W2, out=None, stream=None):
    """W2 [r, V] bf16 -> packed image (uint8 [spec_pack_w2_bytes(r, V)]);
    pack once per model load and pass as W2T=."""
    lib = load_library()
    _dev(W2, "W2")
    if W2.dtype != torch.bfloat16:
        raise SpecError("spec_pack_w2 packs bf16 weights")
    r, V = W2.shape
    nbytes = lib.spec_pack_w2_bytes(r, V)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=W2.device)
    elif out.numel() * out.element_size() < nbytes:
        raise SpecError(f"W2T buffer needs {nbytes} bytes")
    _check(lib.spec_pack_w2(_ptr(W2), _ptr(out), r, V, _stream(stream)), "spec_pack_w2")
    return out


def _check_w2t(W2T, r, V):
    _dev(W2T, "W2T")
    if W2T.numel() * W2T.element_size() < load_library().spec_pack_w2_bytes(r, V):
        raise SpecError("W2T must be a packed image from spec_pack_w2 (too small)")


@_on_stream
def spec_draft_sample_markov(U, x0, W1, W2, T=1.0, *, W2T=None, q_free=False, uniforms=None,
                             seed=0, offset=0, out=None, workspace=None, status=None,
                             stream=None):
    """Markov-head draft.  U [B, gamma, V], x0 [B] int32, W1 [V, r], W2 [r, V]
    (or None with W2T, the packed image from spec_pack_w2).  q_free=True writes no q
    logits (verify with spec_verify_markov).  status: optional int32 [1] device
    tensor that receives spec_draft_status right after the draft (0: every draw
    happened; 1: the persistent engine's waits gave up)."""
    lib = load_library()
    for t, n in ((U, "U"), (x0, "x0"), (W1, "W1")):
        _dev(t, n)
    B, gamma, V = U.shape
    r = W1.shape[1]
    if x0.dtype != torch.int32 or x0.shape != (B,):
        raise SpecError("x0 must be int32 [B]")
    if W2 is not None:
        _dev(W2, "W2")
        if W2.shape != (r, V) or W1.dtype != W2.dtype:
            raise SpecError("W2 must be [r, V] of W1's dtype")
    if W2T is not None:
        _check_w2t(W2T, r, V)
    if W1.shape != (V, r):
        raise SpecError("W1 must be [V, r]")
    if uniforms is not None and (uniforms.dtype != torch.float32 or uniforms.shape != (B, gamma)):
        raise SpecError("uniforms must be float32 [B, gamma]")
    o = _draft_outputs(B, gamma, V, U.device, out, q_free)
    ws, nws = _workspace(lib.spec_draft_markov_workspace_size(B, gamma, V, r), U.device, workspace)
    st = lib.spec_draft_sample_markov(
        _ptr(U), _dtype_code(U, "U"), _ptr(x0), _ptr(W1), _ptr(W2), _ptr(W2T),
        _dtype_code(W1, "W1"), r, B, gamma, V, float(T), _ptr(uniforms), seed, offset,
        _ptr(o["tokens"]), _ptr(o.get("q_logits")), _ptr(o.get("q_logZ")),
        _ptr(o.get("q_tok_prob")), _ptr(ws), nws, _stream(stream))
    _check(st, "spec_draft_sample_markov")
    if status is not None:
        _draft_status(ws, nws, B, gamma, V, r, status, stream)
    return o


def _draft_status(ws, nws, B, gamma, V, r, status, stream):
    _dev(status, "status")
    if status.dtype != torch.int32 or status.numel() < 1:
        raise SpecError("status must be an int32 device tensor with one element")
    _check(load_library().spec_draft_status(_ptr(ws), nws, B, gamma, V, r, _ptr(status),
                                            _stream(stream)), "spec_draft_status")


@_on_stream
def spec_draft_status(workspace, B, gamma, V, r, *, out=None, stream=None):
    """Completion word of the last draft made with `workspace` (a uint8 device
    tensor passed as workspace= to that draft): int32 [1], 0 when every draw
    happened, 1 when the persistent engine's waits gave up."""
    if out is None:
        out = torch.empty(1, dtype=torch.int32, device=workspace.device)
    _draft_status(workspace, workspace.numel(), B, gamma, V, r, out, stream)
    return out


@_on_stream
def spec_draft_sample_rnn(U, x0, h, W1, W2, Wg, Wc, Wo, T=1.0, *, W2T=None, q_free=False,
                          uniforms=None, seed=0, offset=0, out=None, workspace=None, stream=None):
    """RNN-head draft.  h [B, gamma, d]; Wg, Wc, Wo [r, 2r + d].  q_free=True
    writes no q logits; the result then also holds `cond`, the conditioning
    rows [B, gamma, 3, r] (bf16 bits as int16) inside the draft's workspace
    (kept alive by the result), for spec_verify_rnn."""
    lib = load_library()
    for t, n in ((U, "U"), (x0, "x0"), (h, "h"), (W1, "W1"), (Wg, "Wg"), (Wc, "Wc"), (Wo, "Wo")):
        _dev(t, n)
    if W2 is not None:
        _dev(W2, "W2")
    elif W2T is None:
        raise SpecError("W2 or W2T is required")
    B, gamma, V = U.shape
    r = W1.shape[1]
    d = h.shape[2]
    if h.shape[:2] != (B, gamma):
        raise SpecError("h must be [B, gamma, d]")
    for t, n in ((Wg, "Wg"), (Wc, "Wc"), (Wo, "Wo")):
        if t.shape != (r, 2 * r + d):
            raise SpecError(f"{n} must be [r, 2r + d]")
    if W2T is not None:
        _check_w2t(W2T, r, V)
    o = _draft_outputs(B, gamma, V, U.device, out, q_free=q_free)
    ws, nws = _workspace(lib.spec_draft_rnn_workspace_size(B, gamma, V, r, d), U.device, workspace)
    st = lib.spec_draft_sample_rnn(
        _ptr(U), _dtype_code(U, "U"), _ptr(x0), _ptr(h), _dtype_code(h, "h"), d, _ptr(W1),
        _ptr(W2), _ptr(W2T), _ptr(Wg), _ptr(Wc), _ptr(Wo), _dtype_code(W1, "W1"), r, B, gamma, V,
        float(T),
        _ptr(uniforms), seed, offset, _ptr(o["tokens"]), _ptr(o.get("q_logits")),
        _ptr(o.get("q_logZ")), _ptr(o.get("q_tok_prob")), _ptr(ws), nws, _stream(stream))
    _check(st, "spec_draft_sample_rnn")
    if q_free:
        off = lib.spec_draft_rnn_cond_offset(B, gamma, V, r, d)
        nb = B * gamma * 3 * r * 2
        o["cond"] = ws.view(torch.uint8).reshape(-1)[off:off + nb].view(torch.int16).view(
            B, gamma, 3, r)
    return o


@_on_stream
def spec_verify_rnn(P, U, cond, W2, draft, q_logZ, q_tok_prob, T=1.0, *, W2T=None,
                    gamma_max=None, lens=None, p_row_off=None, uniforms=None, seed=0, offset=0,
                    diagnostics=True, out=None, workspace=None, stream=None):
    """Verification of a q-free RNN draft: P target logits (dense [B, gamma+1, V]
    or packed with p_row_off), U and W2 (or W2T) as given to the draft, cond
    the draft's conditioning rows (the `cond` of spec_draft_sample_rnn's
    result), the draft's tokens, q_logZ and q_tok_prob [B, gamma]."""
    lib = load_library()
    for t, n in ((P, "P"), (U, "U"), (cond, "cond"), (draft, "draft"), (q_logZ, "q_logZ"),
                 (q_tok_prob, "q_tok_prob")):
        _dev(t, n)
    B = draft.shape[0]
    gamma_max = draft.shape[1] if gamma_max is None else gamma_max
    V = P.shape[-1]
    if cond.dim() != 4 or cond.shape[:3] != (B, gamma_max, 3) or cond.element_size() != 2:
        raise SpecError("cond must be [B, gamma_max, 3, r] 16-bit")
    r = cond.shape[3]
    if U.shape != (B, gamma_max, V):
        raise SpecError("U must be dense [B, gamma_max, V]")
    for t, n in ((q_logZ, "q_logZ"), (q_tok_prob, "q_tok_prob")):
        if t.dtype != torch.float32 or t.shape != (B, gamma_max):
            raise SpecError(f"{n} must be float32 [B, gamma_max]")
    if draft.dtype != torch.int32 or draft.shape != (B, gamma_max):
        raise SpecError("draft must be int32 [B, gamma_max]")
    for t, n, dt in ((lens, "lens", torch.int32), (p_row_off, "p_row_off", torch.int64)):
        if t is not None:
            _dev(t, n)
            if t.dtype != dt or t.shape != (B,):
                raise SpecError(f"{n} must be {dt} [B]")
    if W2 is not None:
        _dev(W2, "W2")
    if W2T is not None:
        _check_w2t(W2T, r, V)
    dev = P.device
    if out is None:
        out = dict(accepted=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty((B, gamma_max + 1), dtype=torch.int32, device=dev))
        if diagnostics:
            out["p_logZ"] = torch.empty((B, gamma_max + 1), dtype=torch.float32, device=dev)
            out["accept_prob"] = torch.empty((B, gamma_max), dtype=torch.float32, device=dev)
    ws, nws = _workspace(lib.spec_verify_rnn_workspace_size(B, gamma_max, V, r), dev, workspace)
    st = lib.spec_verify_rnn(
        _ptr(P), _dtype_code(P, "P"), _ptr(U), _dtype_code(U, "U"), _ptr(cond), _ptr(W2),
        _ptr(W2T), r, _ptr(draft), _ptr(q_logZ), _ptr(q_tok_prob), _ptr(lens), _ptr(p_row_off),
        B, gamma_max, V, float(T), _ptr(uniforms), seed, offset, _ptr(out["accepted"]),
        _ptr(out["out_tokens"]), _ptr(out.get("p_logZ")), _ptr(out.get("accept_prob")),
        _ptr(ws), nws, _stream(stream))
    _check(st, "spec_verify_rnn")
    return out


@_on_stream
def spec_verify(P, Q, draft, T=1.0, *, gamma_max=None, lens=None, p_row_off=None, q_row_off=None,
                uniforms=None, seed=0, offset=0, diagnostics=True, out=None, workspace=None,
                stream=None):
    """Lossless verification.  Dense: P [B, gamma+1, V], Q [B, gamma, V],
    draft [B, gamma].  Packed: P [rows, V] with p_row_off, Q [rows, V] with
    q_row_off, lens [B] int32, gamma_max given."""
    lib = load_library()
    B, gamma_max, V = _verify_shapes(P, Q, draft, gamma_max, lens, p_row_off, q_row_off, uniforms)
    dev = P.device
    if out is None:
        out = dict(accepted=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty((B, gamma_max + 1), dtype=torch.int32, device=dev))
        if diagnostics:
            out["p_logZ"] = torch.empty((B, gamma_max + 1), dtype=torch.float32, device=dev)
            out["q_logZ"] = torch.empty((B, gamma_max), dtype=torch.float32, device=dev)
            out["accept_prob"] = torch.empty((B, gamma_max), dtype=torch.float32, device=dev)
    ws, nws = _workspace(lib.spec_verify_workspace_size(B, gamma_max, V), dev, workspace)
    st = lib.spec_verify(
        _ptr(P), _dtype_code(P, "P"), _ptr(Q), _dtype_code(Q, "Q") if Q is not None else SPEC_F32,
        _ptr(draft), _ptr(lens), _ptr(p_row_off), _ptr(q_row_off), B, gamma_max, V, float(T),
        _ptr(uniforms), seed, offset, _ptr(out["accepted"]), _ptr(out["out_tokens"]),
        _ptr(out.get("p_logZ")), _ptr(out.get("q_logZ")), _ptr(out.get("accept_prob")), _ptr(ws),
        nws, _stream(stream))
    _check(st, "spec_verify")
    return out


def spec_verify_noalloc_max_bytes():
    """Scratch bytes spec_verify_noalloc holds per GPU (its size limit)."""
    return int(load_library().spec_verify_noalloc_max_bytes())


def spec_verify_noalloc(P, Q, draft, out, T=1.0, *, gamma_max=None, lens=None, p_row_off=None,
                        q_row_off=None, uniforms=None, seed=0, offset=0, stream=None):
    """spec_verify for callers that cannot allocate: the library's fixed device
    scratch stands in for the workspace, and the caller passes every output in
    `out` (accepted int32 [B], out_tokens int32 [B, gamma_max + 1], and
    optionally p_logZ, q_logZ, accept_prob).  Neither this wrapper nor the
    library allocates device memory.  Calls that overlap on one GPU share the
    scratch and race."""
    lib = load_library()
    B, gamma_max, V = _verify_shapes(P, Q, draft, gamma_max, lens, p_row_off, q_row_off, uniforms)
    for n, dt, shp in (("accepted", torch.int32, (B,)), ("out_tokens", torch.int32, (B, gamma_max + 1)),
                       ("p_logZ", torch.float32, (B, gamma_max + 1)),
                       ("q_logZ", torch.float32, (B, gamma_max)),
                       ("accept_prob", torch.float32, (B, gamma_max))):
        t = out.get(n)
        if t is None:
            if n in ("accepted", "out_tokens"):
                raise SpecError(f"out[{n!r}] is required")
            continue
        _dev(t, n)
        if t.dtype != dt or tuple(t.shape) != shp or not t.is_contiguous():
            raise SpecError(f"out[{n!r}] must be contiguous {dt} {list(shp)}")
    st = lib.spec_verify_noalloc(
        _ptr(P), _dtype_code(P, "P"), _ptr(Q), _dtype_code(Q, "Q") if Q is not None else SPEC_F32,
        _ptr(draft), _ptr(lens), _ptr(p_row_off), _ptr(q_row_off), B, gamma_max, V, float(T),
        _ptr(uniforms), seed, offset, _ptr(out["accepted"]), _ptr(out["out_tokens"]),
        _ptr(out.get("p_logZ")), _ptr(out.get("q_logZ")), _ptr(out.get("accept_prob")),
        _stream(stream))
    _check(st, "spec_verify_noalloc")
    return out


def _verify_shapes(P, Q, draft, gamma_max, lens, p_row_off, q_row_off, uniforms):
    """Shape and dtype checks of spec_verify's arguments; returns (B, gamma_max, V)."""
    _dev(P, "P")
    _dev(draft, "draft")
    B = draft.shape[0]
    if gamma_max is None:
        gamma_max = draft.shape[1]
    V = P.shape[-1]
    if draft.dtype != torch.int32 or draft.shape != (B, gamma_max):
        raise SpecError("draft must be int32 [B, gamma_max]")
    if p_row_off is None and P.dim() == 3 and P.shape != (B, gamma_max + 1, V):
        raise SpecError("dense P must be [B, gamma_max + 1, V]")
    if Q is not None:
        _dev(Q, "Q")
        if Q.shape[-1] != V:
            raise SpecError("Q and P must share V")
        if q_row_off is None and Q.dim() == 3 and Q.shape != (B, gamma_max, V):
            raise SpecError("dense Q must be [B, gamma_max, V]")
    for t, n, dt in ((lens, "lens", torch.int32), (p_row_off, "p_row_off", torch.int64),
                     (q_row_off, "q_row_off", torch.int64)):
        if t is not None:
            _dev(t, n)
            if t.dtype != dt or t.shape != (B,):
                raise SpecError(f"{n} must be {dt} [B]")
    if uniforms is not None and (uniforms.dtype != torch.float32
                                 or uniforms.shape != (B, gamma_max + 1)):
        raise SpecError("uniforms must be float32 [B, gamma_max + 1]")
    return B, gamma_max, V


@_on_stream
def spec_acceptance_rate(P, Q, T=1.0, *, gamma_max=None, lens=None, p_row_off=None,
                         q_row_off=None, want_tv=True, out=None, stream=None):
    """Acceptance rate alpha[b, k] = sum min(p_k, q_k) (and the total variation
    1/2 sum |p_k - q_k|) of every drafted position.  Dense: P [B, gamma+1, V],
    Q [B, gamma, V].  Packed: P and Q [rows, V] with p_row_off / q_row_off
    int64 [B], lens int32 [B] and gamma_max given.  NaN where a request has no
    such position."""
    lib = load_library()
    _dev(P, "P")
    _dev(Q, "Q")
    V = P.shape[-1]
    if Q.shape[-1] != V:
        raise SpecError("Q and P must share V")
    if p_row_off is None:
        if P.dim() != 3:
            raise SpecError("dense P must be [B, gamma + 1, V]")
        B = P.shape[0]
        if gamma_max is None:
            gamma_max = P.shape[1] - 1
        if P.shape != (B, gamma_max + 1, V):
            raise SpecError("dense P must be [B, gamma_max + 1, V]")
    else:
        B = p_row_off.shape[0]
        if gamma_max is None:
            raise SpecError("packed rows need gamma_max")
    if q_row_off is None and Q.shape != (B, gamma_max, V):
        raise SpecError("dense Q must be [B, gamma_max, V]")
    for t, n, dt in ((lens, "lens", torch.int32), (p_row_off, "p_row_off", torch.int64),
                     (q_row_off, "q_row_off", torch.int64)):
        if t is not None:
            _dev(t, n)
            if t.dtype != dt or t.shape != (B,):
                raise SpecError(f"{n} must be {dt} [B]")
    if out is None:
        out = dict(alpha=torch.empty((B, gamma_max), dtype=torch.float32, device=P.device))
        if want_tv:
            out["tv"] = torch.empty((B, gamma_max), dtype=torch.float32, device=P.device)
    st = lib.spec_acceptance_rate(_ptr(P), _dtype_code(P, "P"), _ptr(Q), _dtype_code(Q, "Q"),
                                  _ptr(lens), _ptr(p_row_off), _ptr(q_row_off), B, gamma_max, V,
                                  float(T), _ptr(out["alpha"]), _ptr(out.get("tv")),
                                  _stream(stream))
    _check(st, "spec_acceptance_rate")
    return out


@_on_stream
def spec_confidence_head(h, x0, draft, W1, w, *, out=None, stream=None):
    """Confidence c[b, k] = sigmoid(w[:d] . h[b, k] + w[d:] . W1[prev]) of every
    drafted position (prev = x0[b] at k = 0, else draft[b, k-1]).  h [R, gamma,
    d], x0 int32 [R], draft int32 [R, gamma], W1 [V, r], w float32 [d + r]."""
    lib = load_library()
    for t, n in ((h, "h"), (x0, "x0"), (draft, "draft"), (W1, "W1"), (w, "w")):
        _dev(t, n)
    if h.dim() != 3 or W1.dim() != 2:
        raise SpecError("h must be [R, gamma, d] and W1 [V, r]")
    R, gamma, d = h.shape
    V, r = W1.shape
    if x0.dtype != torch.int32 or x0.shape != (R,):
        raise SpecError("x0 must be int32 [R]")
    if draft.dtype != torch.int32 or draft.shape != (R, gamma):
        raise SpecError("draft must be int32 [R, gamma]")
    if w.dtype != torch.float32 or w.shape != (d + r,):
        raise SpecError("w must be float32 [d + r]")
    if out is None:
        out = torch.empty((R, gamma), dtype=torch.float32, device=h.device)
    st = lib.spec_confidence_head(_ptr(h), _dtype_code(h, "h"), d, _ptr(x0), _ptr(draft),
                                  _ptr(W1), _dtype_code(W1, "W1"), r, _ptr(w), R, gamma, V,
                                  _ptr(out), _stream(stream))
    _check(st, "spec_confidence_head")
    return out


@_on_stream
def spec_prefix_schedule(c, sps, *, out=None, workspace=None, stream=None):
    """Acceptance lengths l [R] (int32) from confidences c float32 [R, gamma]
    and the steps-per-second table sps float64 [nsps] (index = batch size).
    Returns dict(lens, B, tau) of device tensors (B int32 [1], tau float64
    [1])."""
    lib = load_library()
    _dev(c, "c")
    _dev(sps, "sps")
    if c.dtype != torch.float32 or c.dim() != 2:
        raise SpecError("c must be float32 [R, gamma]")
    if sps.dtype != torch.float64 or sps.dim() != 1:
        raise SpecError("sps must be float64 [nsps]")
    R, gamma = c.shape
    if out is None:
        out = dict(lens=torch.empty(R, dtype=torch.int32, device=c.device),
                   B=torch.empty(1, dtype=torch.int32, device=c.device),
                   tau=torch.empty(1, dtype=torch.float64, device=c.device))
    ws, nws = _workspace(lib.spec_prefix_schedule_workspace_size(R, gamma), c.device, workspace)
    st = lib.spec_prefix_schedule(_ptr(c), R, gamma, _ptr(sps), sps.numel(), _ptr(out["lens"]),
                                  _ptr(out.get("B")), _ptr(out.get("tau")), _ptr(ws), nws,
                                  _stream(stream))
    _check(st, "spec_prefix_schedule")
    return out


@_on_stream
def spec_tree_select(parent, c, n, *, out=None, stream=None):
    """Top-n nodes of R draft trees by survival probability.  parent int32
    [R, M] (parents first, -1: child of the root), c float32 [R, M].  Returns
    dict(sel int32 [R, n], score float64 [R])."""
    lib = load_library()
    _dev(parent, "parent")
    _dev(c, "c")
    if parent.dtype != torch.int32 or parent.dim() != 2:
        raise SpecError("parent must be int32 [R, M]")
    if c.dtype != torch.float32 or c.shape != parent.shape:
        raise SpecError("c must be float32 [R, M]")
    R, M = parent.shape
    if out is None:
        out = dict(sel=torch.empty((R, n), dtype=torch.int32, device=c.device),
                   score=torch.empty(R, dtype=torch.float64, device=c.device))
    st = lib.spec_tree_select(_ptr(parent), _ptr(c), R, M, int(n), _ptr(out["sel"]),
                              _ptr(out.get("score")), _stream(stream))
    _check(st, "spec_tree_select")
    return out


@_on_stream
def spec_verify_tree(P, Q, parent, tokens, T=1.0, *, n_nodes=None, uniforms=None, seed=0,
                     offset=0, want_path=True, out=None, stream=None):
    """Verification of tree drafts.  P, Q [B, M + 1, V] (row 0 the root, row
    1 + v node v), parent and tokens int32 [B, M] (parents first, -1: child of
    the root), n_nodes int32 [B] or None.  Returns dict(accepted int32 [B],
    out_tokens int32 [B, M + 1], path int32 [B, M])."""
    lib = load_library()
    _dev(P, "P")
    if P.dim() != 3:
        raise SpecError("P must be [B, M + 1, V]")
    B, M1, V = P.shape
    M = M1 - 1
    if M > 0:
        for t, n in ((Q, "Q"), (parent, "parent"), (tokens, "tokens")):
            if t is None:
                raise SpecError(f"{n} is required when M > 0")
            _dev(t, n)
        if Q.shape != P.shape:
            raise SpecError("Q must be [B, M + 1, V] like P")
        for t, n in ((parent, "parent"), (tokens, "tokens")):
            if t.dtype != torch.int32 or t.shape != (B, M):
                raise SpecError(f"{n} must be int32 [B, M]")
    if n_nodes is not None:
        _dev(n_nodes, "n_nodes")
        if n_nodes.dtype != torch.int32 or n_nodes.shape != (B,):
            raise SpecError("n_nodes must be int32 [B]")
    if uniforms is not None and (uniforms.dtype != torch.float32 or uniforms.shape != (B, M + 1)):
        raise SpecError("uniforms must be float32 [B, M + 1]")
    dev = P.device
    if out is None:
        out = dict(accepted=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty((B, M + 1), dtype=torch.int32, device=dev))
        if want_path:
            out["path"] = torch.empty((B, max(M, 1)), dtype=torch.int32, device=dev)
    st = lib.spec_verify_tree(
        _ptr(P), _dtype_code(P, "P"), _ptr(Q) if M > 0 else None,
        _dtype_code(Q, "Q") if M > 0 else SPEC_F32, _ptr(parent) if M > 0 else None,
        _ptr(tokens) if M > 0 else None, _ptr(n_nodes), B, M, V, float(T), _ptr(uniforms),
        seed, offset, _ptr(out["accepted"]), _ptr(out["out_tokens"]), _ptr(out.get("path")),
        _stream(stream))
    _check(st, "spec_verify_tree")
    return out


def spec_draft_set_poll_limit(polls):
    """Wait limit of the persistent draft in polls (0: the default); a
    testing aid.  Returns the previous limit."""
    return int(load_library().spec_draft_set_poll_limit(int(polls)))


def spec_draft_set_persistent(mode):
    """Engine of the q-free Markov draft: 1 (or True) one persistent plain
    launch for all positions where the shape allows it, 2 the same kernel
    under a cooperative launch, 0 (or False) two launches per position.
    Returns the previous mode."""
    mode = int(mode)
    was = load_library().spec_draft_set_persistent(mode)
    if was < 0:
        raise SpecError(f"spec_draft_set_persistent: no mode {mode}")
    return was


def spec_profile_enable(kernel):
    """Start timing every launch of `kernel` ("*" = all, None = stop)."""
    lib = load_library()
    _check(lib.spec_profile_enable(None if kernel is None else kernel.encode()),
           "spec_profile_enable")


def spec_profile_read():
    """(launches, total milliseconds) of the kernel being timed."""
    lib = load_library()
    n, ms = ctypes.c_int(), ctypes.c_double()
    _check(lib.spec_profile_read(ctypes.byref(n), ctypes.byref(ms)), "spec_profile_read")
    return n.value, ms.value


@_on_stream
def spec_verify_markov(P, U, x0, W1, W2, draft, q_logZ, q_tok_prob, T=1.0, *, W2T=None,
                       gamma_max=None, lens=None, p_row_off=None, uniforms=None, seed=0,
                       offset=0, diagnostics=True, out=None, workspace=None, stream=None):
    """Verification of a q-free Markov draft: P target logits (dense
    [B, gamma+1, V] or packed with p_row_off), U/x0/W1/W2 (or W2T) as given to
    the draft, draft tokens and the draft's q_logZ / q_tok_prob [B, gamma]."""
    lib = load_library()
    for t, n in ((P, "P"), (U, "U"), (x0, "x0"), (W1, "W1"), (draft, "draft"),
                 (q_logZ, "q_logZ"), (q_tok_prob, "q_tok_prob")):
        _dev(t, n)
    B = draft.shape[0]
    gamma_max = draft.shape[1] if gamma_max is None else gamma_max
    V = P.shape[-1]
    r = W1.shape[1]
    if U.shape != (B, gamma_max, V):
        raise SpecError("U must be dense [B, gamma_max, V]")
    for t, n in ((q_logZ, "q_logZ"), (q_tok_prob, "q_tok_prob")):
        if t.dtype != torch.float32 or t.shape != (B, gamma_max):
            raise SpecError(f"{n} must be float32 [B, gamma_max]")
    if draft.dtype != torch.int32 or draft.shape != (B, gamma_max):
        raise SpecError("draft must be int32 [B, gamma_max]")
    for t, n, dt in ((lens, "lens", torch.int32), (p_row_off, "p_row_off", torch.int64)):
        if t is not None:
            _dev(t, n)
            if t.dtype != dt or t.shape != (B,):
                raise SpecError(f"{n} must be {dt} [B]")
    if W2 is not None:
        _dev(W2, "W2")
    if W2T is not None:
        _check_w2t(W2T, r, V)
    dev = P.device
    if out is None:
        out = dict(accepted=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty((B, gamma_max + 1), dtype=torch.int32, device=dev))
        if diagnostics:
            out["p_logZ"] = torch.empty((B, gamma_max + 1), dtype=torch.float32, device=dev)
            out["accept_prob"] = torch.empty((B, gamma_max), dtype=torch.float32, device=dev)
    ws, nws = _workspace(lib.spec_verify_markov_workspace_size(B, gamma_max, V, r), dev, workspace)
    st = lib.spec_verify_markov(
        _ptr(P), _dtype_code(P, "P"), _ptr(U), _dtype_code(U, "U"), _ptr(x0), _ptr(W1), _ptr(W2),
        _ptr(W2T), SPEC_BF16, r, _ptr(draft), _ptr(q_logZ), _ptr(q_tok_prob), _ptr(lens),
        _ptr(p_row_off), B, gamma_max, V, float(T), _ptr(uniforms), seed, offset,
        _ptr(out["accepted"]), _ptr(out["out_tokens"]), _ptr(out.get("p_logZ")),
        _ptr(out.get("accept_prob")), _ptr(ws), nws, _stream(stream))
    _check(st, "spec_verify_markov")
    return out
