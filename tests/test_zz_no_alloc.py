"""GPU: spec_verify_noalloc (the library's fixed device scratch instead of a
workspace) gives exactly spec_verify's outputs, on two calls in a row with the
second smaller, and refuses a shape whose scratch exceeds the fixed size
before launching anything."""
import ctypes

import numpy as np
import pytest

import workloads
from tests.gpu_util import dev, note, require_gpu, torch

pytestmark = pytest.mark.gpu

KEYS = ("accepted", "out_tokens", "p_logZ", "q_logZ", "accept_prob")


def _outputs(B, gamma):
    return dict(accepted=torch.full((B,), -7, dtype=torch.int32, device="cuda"),
                out_tokens=torch.full((B, gamma + 1), -7, dtype=torch.int32, device="cuda"),
                p_logZ=torch.full((B, gamma + 1), np.nan, dtype=torch.float32, device="cuda"),
                q_logZ=torch.full((B, gamma), np.nan, dtype=torch.float32, device="cuda"),
                accept_prob=torch.full((B, gamma), np.nan, dtype=torch.float32, device="cuda"))


def _case(B, gamma, V, dtype, sigma, seed, ragged):
    vw = workloads.make_verify_only(B, gamma, V, seed=seed, dtype=dtype, sigma=sigma)
    P, Q = dev(vw["P"], dtype), dev(vw["Q"], dtype)
    rng = np.random.default_rng(seed)
    # draft tokens: the draft row's argmax where the rows agree often enough
    # to accept some positions, random ids elsewhere
    draft = np.argmax(vw["Q"].astype(np.float32) if dtype == "f32" else
                      workloads.as_f64(vw["Q"], dtype), axis=-1).astype(np.int32)
    flip = rng.random(draft.shape) < 0.3
    draft[flip] = rng.integers(0, V, size=int(flip.sum()), dtype=np.int32)
    lens = None
    if ragged:
        lens = torch.from_numpy(rng.integers(0, gamma + 1, size=B, dtype=np.int32)).cuda()
    return P, Q, dev(draft), lens


def _run_pair(sd, B, gamma, V, dtype, sigma, seed, ragged, T):
    note(f"noalloc B={B} gamma={gamma} V={V} dtype={dtype} ragged={ragged} T={T}")
    P, Q, draft, lens = _case(B, gamma, V, dtype, sigma, seed, ragged)
    want = sd.spec_verify(P, Q, draft, T, lens=lens, seed=seed, offset=3)
    got = sd.spec_verify_noalloc(P, Q, draft, _outputs(B, gamma), T, lens=lens, seed=seed, offset=3)
    torch.cuda.synchronize()
    for k in KEYS:
        a, b = want[k].cpu().numpy(), got[k].cpu().numpy()
        assert np.array_equal(a, b, equal_nan=True), k
    return want["accepted"].cpu().numpy()


def test_noalloc_matches_verify_two_calls():
    sd = require_gpu()
    assert sd.spec_verify_noalloc_max_bytes() == 16 << 20
    # first call: the larger shape; second: smaller, over the first's leftovers
    acc1 = _run_pair(sd, 96, 6, 32000, "f32", 0.6, 41, False, 1.0)
    acc2 = _run_pair(sd, 7, 3, 4099, "bf16", 0.3, 42, True, 0.7)
    assert acc1.max() > 0 and acc2.min() >= -1
    # a third call at T = 0 after both
    _run_pair(sd, 33, 4, 5000, "bf16", 0.6, 43, False, 0.0)


def test_noalloc_rejects_oversized_shape():
    sd = require_gpu()
    lib = sd.load_library()
    B, gamma, V = 65536, 8, 262144
    need = lib.spec_verify_workspace_size(B, gamma, V)
    assert need > sd.spec_verify_noalloc_max_bytes()
    # small real buffers: the call must refuse on the host, before any launch
    small = torch.zeros(64, dtype=torch.float32, device="cuda")
    ints = torch.zeros(64, dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(small.data_ptr())
    i = ctypes.c_void_p(ints.data_ptr())
    st = lib.spec_verify_noalloc(p, sd.SPEC_F32, p, sd.SPEC_F32, i, None, None, None, B, gamma, V,
                                 1.0, None, 0, 0, i, i, None, None, None, None)
    assert st == 3, st   # SPEC_ERR_WORKSPACE
    assert b"spec_verify_noalloc" in lib.spec_last_error()
    torch.cuda.synchronize()
