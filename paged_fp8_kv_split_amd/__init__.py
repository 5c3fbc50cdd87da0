"""Split-KV verify attention over a paged fp8 KV cache, native to MI355X (gfx950).

The compute path is the HIP library ``libpfkv.so`` built from ``csrc/``; the
Python side only marshals arguments to its C ABI (see ``binding.py``). The
library is loaded on first use and a missing build raises ``RuntimeError``:
there is no CPU fallback.

A second workload, fp8 varlen prefill attention (``prefill_attn``), runs on the
same library.
"""

from .binding import (  # noqa: F401
    PfkvError,
    library_path,
    load_library,
    merge_sync_buffer,
    merge_sync_bytes,
    num_segments,
    partials_row_major,
    prefill_attn,
    set_debug,
    stream_read,
    verify_attn,
    workspace_bytes,
)
