"""specverify: the verify step of speculative sampling on AMD Instinct MI355X.

The work runs in the HIP library libspecverify.so (C ABI in
include/specverify.h); this package holds its sources (csrc/), the build
script and a thin ctypes binding.
"""
from .binding import (  # noqa: F401
    DraftPlan,
    GreedyPlan,
    LikelihoodPlan,
    SamplePlan,
    StreamReadPlan,
    HipEvents,
    SpecVerifyError,
    load_library,
    draft_sample,
    status_string,
    token_likelihood,
    verify_argmax,
    verify_greedy,
    verify_sample,
    verify_sample_noalloc,
    workspace_bytes,
)
