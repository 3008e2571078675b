"""CPU-side checks of the C ABI: the library loads, exports every function
include/specdec.h declares, and rejects invalid arguments before any launch
(these calls return during validation and never touch a device)."""
import ctypes
import os
import re

import pytest

import draft_sampling_lossless_head_amd as sd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specdec.h")

SPEC_OK, SPEC_ERR_INVALID, SPEC_ERR_UNSUPPORTED, SPEC_ERR_WORKSPACE = 0, 1, 2, 3


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sd.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return sd.load_library()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("spec_draft_sample_markov", "spec_draft_sample_rnn", "spec_verify",
              "spec_draft_markov_workspace_size", "spec_draft_rnn_workspace_size",
              "spec_verify_workspace_size", "spec_philox_uniforms", "spec_last_error",
              "spec_version", "spec_pack_w2", "spec_pack_w2_bytes", "spec_verify_markov",
              "spec_verify_markov_workspace_size", "spec_draft_set_persistent",
              "spec_draft_set_poll_limit", "spec_acceptance_rate", "spec_confidence_head",
              "spec_prefix_schedule", "spec_prefix_schedule_workspace_size", "spec_tree_select",
              "spec_draft_status", "spec_verify_tree", "spec_verify_noalloc",
              "spec_verify_noalloc_max_bytes", "spec_verify_rnn",
              "spec_verify_rnn_workspace_size", "spec_draft_rnn_cond_offset"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in _declared():
        assert hasattr(lib, n), n
    assert lib.spec_version() == 100


def test_workspace_sizes(lib):
    assert lib.spec_verify_workspace_size(0, 4, 100) == 0
    a = lib.spec_draft_markov_workspace_size(128, 16, 151936, 256)
    assert a > 0 and a % 256 == 0
    assert lib.spec_draft_rnn_workspace_size(64, 8, 32000, 256, 4096) > \
        lib.spec_draft_markov_workspace_size(64, 8, 32000, 256)
    # room for the summaries of 64-token segments, the 16 group sums of every
    # 128-token segment and a packed W2 copy (V = 3000: 47 and 24 segments)
    B, V, r = 40, 3000, 32
    need = B * 47 * 16 + B * 24 * 16 * 4 + lib.spec_pack_w2_bytes(r, V)
    assert lib.spec_draft_markov_workspace_size(B, 3, V, r) >= need


def _markov(lib, **kw):
    fake = ctypes.c_void_p(4096)   # never dereferenced: validation fails first
    a = dict(U=fake, U_dtype=0, x0=fake, W1=fake, W2=fake, W2T=None, w_dtype=1, r=256, B=2, gamma=3,
             V=1000, T=1.0, uniforms=None, seed=0, offset=0, tokens=fake, q_logits=fake,
             q_logZ=None, q_tok=None, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.spec_draft_sample_markov(*a.values())


def test_markov_validation(lib):
    fake = ctypes.c_void_p(4096)
    assert _markov(lib, U=None) == SPEC_ERR_INVALID
    assert _markov(lib, B=-1) == SPEC_ERR_INVALID
    assert _markov(lib, V=0) == SPEC_ERR_INVALID
    assert _markov(lib, r=0) == SPEC_ERR_INVALID
    assert _markov(lib, T=-1.0) == SPEC_ERR_INVALID
    assert _markov(lib, T=float("nan")) == SPEC_ERR_INVALID
    assert _markov(lib, U_dtype=7) == SPEC_ERR_UNSUPPORTED
    assert _markov(lib, r=40) == SPEC_ERR_UNSUPPORTED         # bf16 MFMA needs r % 16 == 0
    assert _markov(lib, r=512) == SPEC_ERR_UNSUPPORTED
    assert _markov(lib, W1=ctypes.c_void_p(4098)) == SPEC_ERR_UNSUPPORTED   # misaligned
    assert _markov(lib) == SPEC_ERR_WORKSPACE                 # no workspace given
    assert _markov(lib, ws=ctypes.c_void_p(4096 + 64), ws_bytes=1 << 30) == SPEC_ERR_WORKSPACE
    assert _markov(lib, ws=ctypes.c_void_p(4096), ws_bytes=16) == SPEC_ERR_WORKSPACE
    assert "workspace" in lib.spec_last_error().decode()
    assert _markov(lib, B=0) == SPEC_OK                        # empty batch: nothing to do
    assert _markov(lib, gamma=0) == SPEC_OK
    # q-free mode (q_logits NULL): needs q_logZ and q_tok_prob and bf16 weights
    assert _markov(lib, q_logits=None) == SPEC_ERR_INVALID
    assert _markov(lib, q_logits=None, q_logZ=fake, q_tok=fake, w_dtype=0) == SPEC_ERR_UNSUPPORTED
    assert _markov(lib, q_logits=None, q_logZ=fake, q_tok=fake) == SPEC_ERR_WORKSPACE
    # a packed W2T may stand in for W2 (bf16 only)
    assert _markov(lib, W2=None) == SPEC_ERR_INVALID
    assert _markov(lib, W2=None, W2T=fake) == SPEC_ERR_WORKSPACE
    assert _markov(lib, W2T=fake, w_dtype=0) == SPEC_ERR_UNSUPPORTED
    assert _markov(lib, W2T=ctypes.c_void_p(4104)) == SPEC_ERR_UNSUPPORTED


def _verify(lib, **kw):
    fake = ctypes.c_void_p(4096)
    a = dict(P=fake, p_dtype=1, Q=fake, q_dtype=0, draft=fake, lens=None, p_off=None, q_off=None,
             B=2, G=3, V=1000, T=1.0, uniforms=None, seed=0, offset=0, accepted=fake, out=fake,
             p_logZ=None, q_logZ=None, ap=None, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.spec_verify(*a.values())


def test_verify_validation(lib):
    assert _verify(lib, P=None) == SPEC_ERR_INVALID
    assert _verify(lib, Q=None) == SPEC_ERR_INVALID
    assert _verify(lib, G=0, Q=None, draft=None) == SPEC_ERR_WORKSPACE   # bonus-only is valid
    assert _verify(lib, G=-1) == SPEC_ERR_INVALID
    assert _verify(lib, T=-0.5) == SPEC_ERR_INVALID
    assert _verify(lib, q_dtype=3) == SPEC_ERR_UNSUPPORTED
    assert _verify(lib, P=ctypes.c_void_p(4100)) == SPEC_ERR_UNSUPPORTED
    assert _verify(lib) == SPEC_ERR_WORKSPACE
    assert _verify(lib, B=0) == SPEC_OK


def test_rnn_validation(lib):
    fake = ctypes.c_void_p(4096)
    base = dict(U=fake, U_dtype=0, x0=fake, h=fake, h_dtype=1, d=64, W1=fake, W2=fake, W2T=None, Wg=fake,
                Wc=fake, Wo=fake, w_dtype=1, r=32, B=2, gamma=2, V=500, T=1.0, uniforms=None,
                seed=0, offset=0, tokens=fake, q_logits=fake, q_logZ=None, q_tok=None, ws=None,
                ws_bytes=0, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return lib.spec_draft_sample_rnn(*a.values())

    assert call(h=None) == SPEC_ERR_INVALID
    assert call(d=-1) == SPEC_ERR_INVALID
    assert call(d=12) == SPEC_ERR_UNSUPPORTED
    assert call(w_dtype=0) == SPEC_ERR_UNSUPPORTED
    assert call(q_logits=None) == SPEC_ERR_INVALID                    # q-free needs q_logZ, q(x)
    assert call(q_logits=None, q_logZ=fake, q_tok=fake) == SPEC_ERR_WORKSPACE   # q-free RNN draft
    assert lib.spec_draft_rnn_cond_offset(2, 2, 500, 32, 64) % 256 == 0
    assert lib.spec_draft_rnn_cond_offset(2, 2, 500, 32, 64) + 2 * 2 * 3 * 32 * 2 <= \
        lib.spec_draft_rnn_workspace_size(2, 2, 500, 32, 64)
    assert call() == SPEC_ERR_WORKSPACE


def _verify_markov(lib, **kw):
    fake = ctypes.c_void_p(4096)
    a = dict(P=fake, p_dtype=1, U=fake, U_dtype=0, x0=fake, W1=fake, W2=fake, W2T=None,
             w_dtype=1, r=64, draft=fake, q_logZ=fake, q_tok=fake, lens=None, p_off=None, B=2,
             G=3, V=1000, T=1.0, uniforms=None, seed=0, offset=0, accepted=fake, out=fake,
             p_logZ=None, ap=None, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.spec_verify_markov(*a.values())


def test_verify_markov_validation(lib):
    fake = ctypes.c_void_p(4096)
    assert _verify_markov(lib, P=None) == SPEC_ERR_INVALID
    assert _verify_markov(lib, q_logZ=None) == SPEC_ERR_INVALID
    assert _verify_markov(lib, W2=None) == SPEC_ERR_INVALID
    assert _verify_markov(lib, G=-1) == SPEC_ERR_INVALID
    assert _verify_markov(lib, V=300000) == SPEC_ERR_INVALID
    assert _verify_markov(lib, w_dtype=0) == SPEC_ERR_UNSUPPORTED
    assert _verify_markov(lib, r=40) == SPEC_ERR_UNSUPPORTED
    assert _verify_markov(lib, U=ctypes.c_void_p(4100)) == SPEC_ERR_UNSUPPORTED
    assert _verify_markov(lib) == SPEC_ERR_WORKSPACE
    assert _verify_markov(lib, W2=None, W2T=fake) == SPEC_ERR_WORKSPACE
    assert _verify_markov(lib, G=0, U=None, draft=None, q_logZ=None) == SPEC_ERR_WORKSPACE
    assert _verify_markov(lib, B=0) == SPEC_OK
    assert lib.spec_verify_markov_workspace_size(4, 3, 1000, 64) > \
        lib.spec_verify_workspace_size(4, 3, 1000)


def test_pack_w2_validation(lib):
    fake = ctypes.c_void_p(4096)
    assert lib.spec_pack_w2(None, fake, 64, 1000, None) == SPEC_ERR_INVALID
    assert lib.spec_pack_w2(fake, fake, 0, 1000, None) == SPEC_ERR_INVALID
    assert lib.spec_pack_w2(fake, ctypes.c_void_p(4098), 64, 1000, None) == SPEC_ERR_UNSUPPORTED
    assert lib.spec_pack_w2(fake, fake, 40, 1000, None) == SPEC_ERR_UNSUPPORTED
    assert lib.spec_pack_w2(fake, fake, 512, 1000, None) == SPEC_ERR_UNSUPPORTED
    # whole 128-token tiles of r bf16
    assert lib.spec_pack_w2_bytes(256, 151936) == 1187 * 128 * 256 * 2
    assert lib.spec_pack_w2_bytes(16, 129) == 2 * 128 * 16 * 2
    assert lib.spec_pack_w2_bytes(0, 100) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import draft_sampling_lossless_head_amd.api as api
    monkeypatch.setattr(api, "_lib", None)
    monkeypatch.setattr(api, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(api.SpecError):
        api.load_library()


def test_acceptance_rate_validation(lib):
    """Argument checks of spec_acceptance_rate happen before any launch."""
    fake = ctypes.c_void_p(4096)
    f = lib.spec_acceptance_rate
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int

    def call(P=fake, pd=0, Q=fake, qd=0, B=2, G=3, V=100, T=1.0, alpha=fake):
        return f(P, pd, Q, qd, None, None, None, B, G, V, T, alpha, None, None)
    assert call(P=None) == SPEC_ERR_INVALID
    assert call(Q=None) == SPEC_ERR_INVALID
    assert call(alpha=None) == SPEC_ERR_INVALID
    assert call(B=-1) == SPEC_ERR_INVALID
    assert call(V=0) == SPEC_ERR_INVALID
    assert call(T=-0.5) == SPEC_ERR_INVALID
    assert call(T=float("inf")) == SPEC_ERR_INVALID
    assert call(pd=7) == SPEC_ERR_UNSUPPORTED
    assert call(B=0, P=None) == SPEC_OK        # nothing to do
    assert call(G=0, P=None) == SPEC_OK


def test_confidence_head_validation(lib):
    """Argument checks of spec_confidence_head happen before any launch."""
    fake = ctypes.c_void_p(4096)
    f = lib.spec_confidence_head
    vp, i = ctypes.c_void_p, ctypes.c_int
    f.argtypes = [vp, i, i, vp, vp, vp, i, i, vp, i, i, i, vp, vp]
    f.restype = i

    def call(h=fake, hd=1, d=64, x0=fake, draft=fake, W1=fake, wd=1, r=16, w=fake, R=2, G=3,
             V=100, c=fake):
        return f(h, hd, d, x0, draft, W1, wd, r, w, R, G, V, c, None)
    for k in ("h", "x0", "draft", "W1", "w", "c"):
        assert call(**{k: None}) == SPEC_ERR_INVALID, k
    assert call(R=-1) == SPEC_ERR_INVALID
    assert call(d=0) == SPEC_ERR_INVALID
    assert call(r=0) == SPEC_ERR_INVALID
    assert call(V=0) == SPEC_ERR_INVALID
    assert call(hd=5) == SPEC_ERR_UNSUPPORTED
    assert call(wd=5) == SPEC_ERR_UNSUPPORTED
    assert call(R=0, h=None) == SPEC_OK        # nothing to do
    assert call(G=0, h=None) == SPEC_OK


def test_prefix_schedule_validation(lib):
    """Argument checks of spec_prefix_schedule happen before any launch."""
    fake = ctypes.c_void_p(4096)
    f = lib.spec_prefix_schedule
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    f.argtypes = [vp, i, i, vp, i, vp, vp, vp, vp, sz, vp]
    f.restype = i
    lib.spec_prefix_schedule_workspace_size.argtypes = [i, i]
    lib.spec_prefix_schedule_workspace_size.restype = sz
    need = lib.spec_prefix_schedule_workspace_size(4, 3)
    assert need > 0 and lib.spec_prefix_schedule_workspace_size(0, 3) == 0

    def call(c=fake, R=4, G=3, sps=fake, nsps=10, lens=fake, ws=fake, nws=None):
        return f(c, R, G, sps, nsps, lens, None, None, ws, need if nws is None else nws, None)
    assert call(ws=None) == SPEC_ERR_WORKSPACE
    assert call(nws=need - 1) == SPEC_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(4100)) == SPEC_ERR_WORKSPACE   # unaligned
    assert call(c=None) == SPEC_ERR_INVALID
    assert call(lens=None) == SPEC_ERR_INVALID
    assert call(sps=None) == SPEC_ERR_INVALID
    assert call(R=-1) == SPEC_ERR_INVALID
    assert call(G=-1) == SPEC_ERR_INVALID
    assert call(nsps=-1) == SPEC_ERR_INVALID
    assert call(R=1025, G=8) == SPEC_ERR_UNSUPPORTED
    assert call(R=8193, G=1) == SPEC_ERR_UNSUPPORTED
    assert call(R=8193, G=0) == SPEC_ERR_UNSUPPORTED


def test_tree_select_validation(lib):
    """Argument checks of spec_tree_select happen before any launch."""
    fake = ctypes.c_void_p(4096)
    f = lib.spec_tree_select
    vp, i = ctypes.c_void_p, ctypes.c_int
    f.argtypes = [vp, vp, i, i, i, vp, vp, vp]
    f.restype = i

    def call(parent=fake, c=fake, R=2, M=10, n=4, sel=fake):
        return f(parent, c, R, M, n, sel, None, None)
    assert call(parent=None) == SPEC_ERR_INVALID
    assert call(c=None) == SPEC_ERR_INVALID
    assert call(sel=None) == SPEC_ERR_INVALID
    assert call(R=-1) == SPEC_ERR_INVALID
    assert call(M=-1) == SPEC_ERR_INVALID
    assert call(n=-1) == SPEC_ERR_INVALID
    assert call(M=4097) == SPEC_ERR_UNSUPPORTED
    assert call(R=0, parent=None) == SPEC_OK   # nothing to do


def test_draft_poll_limit(lib):
    """The wait limit is process-wide, returns the previous value, and 0
    restores the default."""
    import ctypes
    lib.spec_draft_set_poll_limit.argtypes = [ctypes.c_uint32]
    lib.spec_draft_set_poll_limit.restype = ctypes.c_uint32
    default = lib.spec_draft_set_poll_limit(0)
    assert default == 1 << 20
    assert lib.spec_draft_set_poll_limit(3) == 1 << 20
    assert lib.spec_draft_set_poll_limit(0) == 3
    assert lib.spec_draft_set_poll_limit(0) == 1 << 20


def test_draft_engine_switch(lib):
    """The draft engine setting is process-wide and returns the previous value;
    a mode outside 0..2 is refused and changes nothing."""
    was = lib.spec_draft_set_persistent(0)
    assert was in (0, 1, 2)
    assert lib.spec_draft_set_persistent(1) == 0
    assert lib.spec_draft_set_persistent(2) == 1
    assert lib.spec_draft_set_persistent(7) == -1
    assert lib.spec_draft_set_persistent(-1) == -1
    assert lib.spec_draft_set_persistent(was) == 2


def test_draft_status_validation(lib):
    fake = ctypes.c_void_p(4096)
    i32, sz = ctypes.c_int, ctypes.c_size_t
    need = lib.spec_draft_markov_workspace_size(128, 16, 151936, 256)
    # null status, bad sizes, missing or short workspace: rejected before any copy
    assert lib.spec_draft_status(fake, need, 128, 16, 151936, 256, None, None) == SPEC_ERR_INVALID
    assert lib.spec_draft_status(fake, need, 0, 16, 151936, 256, fake, None) == SPEC_ERR_INVALID
    assert lib.spec_draft_status(fake, need, 128, 16, 1 << 20, 256, fake, None) == SPEC_ERR_INVALID
    assert lib.spec_draft_status(None, need, 128, 16, 151936, 256, fake, None) == SPEC_ERR_WORKSPACE
    assert lib.spec_draft_status(fake, 64, 128, 16, 151936, 256, fake, None) == SPEC_ERR_WORKSPACE
    assert lib.spec_draft_status(ctypes.c_void_p(4096 + 16), need, 128, 16, 151936, 256, fake,
                                 None) == SPEC_ERR_WORKSPACE


def test_verify_tree_validation(lib):
    fake = ctypes.c_void_p(4096)
    base = dict(P=fake, p_dtype=1, Q=fake, q_dtype=1, parent=fake, tokens=fake, n_nodes=None,
                B=2, M=5, V=1000, T=1.0, uniforms=None, seed=0, offset=0, accepted=fake,
                out=fake, path=None, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return lib.spec_verify_tree(*a.values())

    assert call(P=None) == SPEC_ERR_INVALID
    assert call(Q=None) == SPEC_ERR_INVALID
    assert call(parent=None) == SPEC_ERR_INVALID
    assert call(tokens=None) == SPEC_ERR_INVALID
    assert call(accepted=None) == SPEC_ERR_INVALID
    assert call(B=-1) == SPEC_ERR_INVALID
    assert call(M=-1) == SPEC_ERR_INVALID
    assert call(V=0) == SPEC_ERR_INVALID
    assert call(V=(1 << 20) + 1) == SPEC_ERR_INVALID
    assert call(T=-1.0) == SPEC_ERR_INVALID
    assert call(M=1025) == SPEC_ERR_UNSUPPORTED
    assert call(p_dtype=5) == SPEC_ERR_UNSUPPORTED
    assert call(Q=ctypes.c_void_p(4100)) == SPEC_ERR_UNSUPPORTED
    assert call(B=0) == SPEC_OK


def test_verify_noalloc_validation(lib):
    fake = ctypes.c_void_p(4096)
    base = dict(P=fake, p_dtype=1, Q=fake, q_dtype=0, draft=fake, lens=None, p_off=None,
                q_off=None, B=2, G=3, V=1000, T=1.0, uniforms=None, seed=0, offset=0,
                accepted=fake, out=fake, p_logZ=None, q_logZ=None, ap=None, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return lib.spec_verify_noalloc(*a.values())

    assert lib.spec_verify_noalloc_max_bytes() == 16 << 20
    assert call(P=None) == SPEC_ERR_INVALID
    assert call(G=-1) == SPEC_ERR_INVALID
    assert call(q_dtype=3) == SPEC_ERR_UNSUPPORTED
    assert call(B=0) == SPEC_OK
    # more scratch than the fixed array: refused on the host, nothing launched
    assert call(B=65536, G=8, V=262144) == SPEC_ERR_WORKSPACE
    assert "spec_verify_noalloc" in lib.spec_last_error().decode()


def test_verify_rnn_validation(lib):
    fake = ctypes.c_void_p(4096)
    base = dict(P=fake, p_dtype=1, U=fake, U_dtype=1, cond=fake, W2=fake, W2T=None, r=64,
                draft=fake, q_logZ=fake, q_tok=fake, lens=None, p_off=None, B=2, G=3, V=1000,
                T=1.0, uniforms=None, seed=0, offset=0, accepted=fake, out=fake, p_logZ=None,
                ap=None, ws=None, ws_bytes=0, stream=None)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return lib.spec_verify_rnn(*a.values())

    assert call(cond=None) == SPEC_ERR_INVALID
    assert call(cond=ctypes.c_void_p(4100)) == SPEC_ERR_UNSUPPORTED
    assert call(q_logZ=None) == SPEC_ERR_INVALID
    assert call(r=40) == SPEC_ERR_UNSUPPORTED
    assert call() == SPEC_ERR_WORKSPACE
    assert call(B=0) == SPEC_OK
    assert lib.spec_verify_rnn_workspace_size(2, 3, 1000, 64) == \
        lib.spec_verify_markov_workspace_size(2, 3, 1000, 64)
