"""MI355X-native speculative-verify Gated DeltaNet route.

Three calls over one caller stream, each a thin binding of the C ABI in
include/gdn_verify.h (libgdnverify.so, hand-written gfx950 HIP kernels):

    conv_tree_step  -> conv_out, commit_win
    tree_verify     -> out, replay_log          (persistent state read-only)
    conv_tree_verify -> out, replay_log, commit_win  (the two above fused)
    replay_commit   -> advances state_pool / conv_hist of accepting slots
    replay_commit_layers -> the same for every layer of a round, one launch

and, for a step without a draft (plain decode), two calls that advance the slots
directly:

    conv_step       -> conv_out; writes each slot's conv history in place
    decode_step     -> out; applies one token to each slot's state in place
    conv_decode_step -> out; the two above for one token, fused in one launch

and a prompt fills a slot with conv_step over its tokens followed by

    prefill         -> out; the recurrence over the prompt, each slot's state in place
                       (prefill_workspace_size: the scratch bytes it needs;
                       prefill_noalloc: the same with the library's static scratch,
                       for callers that cannot allocate)

The library is loaded on first use and must have been built
(`python -m gated_deltanet_speculative_amd.build`); there is no fallback path.
"""

from ._lib import (  # noqa: F401
    EXPORTED,
    GdnError,
    LIB_PATH,
    MAX_CHAIN,
    MAX_LAYERS,
    Shape,
    STATUS_ACCEPT,
    STATUS_NODES,
    STATUS_PARENT,
    STATUS_SLOT_DUP,
    STATUS_SLOT_RANGE,
    SYNC_STRIDE,
    conv_decode_step,
    conv_step,
    conv_tree_step,
    conv_tree_verify,
    decode_step,
    STATIC_SCRATCH_BYTES,
    prefill,
    prefill_noalloc,
    prefill_workspace_size,
    load_library,
    replay_commit,
    replay_commit_layers,
    strerror,
    tree_verify,
)
