"""MI355X-native DSpark draft sampling and lossless verification.

The compute path is the HIP library libspecdec.so (include/specdec.h); this
package only marshals torch device tensors into its C ABI.  Importing the
package does not load the library; the first call does, and fails loudly if
the library is missing.
"""
from .api import (  # noqa: F401
    SPEC_BF16,
    SPEC_F32,
    SpecError,
    library_path,
    load_library,
    spec_acceptance_rate,
    spec_confidence_head,
    spec_draft_sample_markov,
    spec_draft_sample_rnn,
    spec_draft_set_persistent,
    spec_draft_set_poll_limit,
    spec_draft_status,
    spec_pack_w2,
    spec_pack_w2_bytes,
    spec_philox_uniforms,
    spec_prefix_schedule,
    spec_profile_enable,
    spec_profile_read,
    spec_tree_select,
    spec_verify,
    spec_verify_markov,
    spec_verify_noalloc,
    spec_verify_rnn,
    spec_verify_noalloc_max_bytes,
    spec_verify_tree,
    spec_version,
    workspace_bytes,
)
