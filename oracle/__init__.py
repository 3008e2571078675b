"""fp64 CPU oracle for DSpark draft sampling and lossless verification.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP path, and the HIP path never imports it.

Parity status of each function is recorded in ``oracle.PINS`` below.
"""
from .binding import (  # noqa: F401
    PINS,
    build,
    philox4x32_10,
    uniform,
    draft_uniforms,
    verify_uniforms,
    softmax_weights,
    residual_weights,
    inverse_cdf,
    cdf_interval,
    argmax,
    alpha_tv,
    draft_markov,
    draft_rnn,
    verify,
    tree_uniforms,
    verify_tree,
    confidence,
    prefix_schedule,
    tree_select,
)
