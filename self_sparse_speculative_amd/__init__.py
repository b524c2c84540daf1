"""S3R (self-sparse speculative rollouts) attention-and-sampling step on MI355X.

The product is libs3r.so (HIP kernels for gfx950 behind the C ABI in
include/s3r.h); this package builds it (``build.py``) and binds it
(``s3r.py``). Importing the package does not load the library; the first
call does, and raises if it has not been built.
"""

from .s3r import (  # noqa: F401
    EXPORTED,
    SAMPLE_SCRATCH_BYTES,
    PagedKV,
    S3RError,
    Workspace,
    budget,
    commit,
    kv_append,
    length_order,
    lib_path,
    load,
    read_draft_pattern,
    read_verify_pattern,
    select,
    select_grouped,
    select_grouped_capacity,
    select_pages,
    sparse_decode_attn,
    sparse_decode_workspace_bytes,
    spec_sample,
    spec_sample_noalloc,
    spec_sample_workspace_bytes,
    status_string,
    verify_attn,
    verify_attn_deferred,
    verify_attn_pages,
    verify_pages_workspace_bytes,
    verify_scores,
    verify_workspace_bytes,
)
