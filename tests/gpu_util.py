"""Shared helpers of the GPU tests: host -> device transfer of seeded inputs,
and running the oracle on selected requests."""
import sys

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_sampling_lossless_head_amd as sd
    sd.load_library()      # raises if the HIP library is missing
    return sd


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x, dtype_name=None):
    """numpy -> cuda tensor; bf16 inputs travel as uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype_name == "bf16":
        t = t.view(torch.bfloat16)
    return t.to("cuda")


def host(d):
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in d.items()}


def markov_to_device(wl):
    lb, wb = wl["logit_dtype"], wl["w_dtype"]
    return dict(U=dev(wl["U"], lb), P=dev(wl["P"], lb), W1=dev(wl["W1"], wb), W2=dev(wl["W2"], wb),
                x0=dev(wl["x0"]))


def request_f64(wl, i):
    """Exact float64 inputs of the i-th request of a workload."""
    return workloads.as_f64(wl["U"][i], wl["logit_dtype"])
