"""MI355X-native chunked-prefill forward of the gated delta rule (Gated DeltaNet / KDA).

The computation runs in hand-written HIP kernels behind the C ABI declared in
``include/gdn.h`` (library ``libgdn.so``); ``gdn`` is the thin ctypes binding.
Importing the package does not load the native library; the first call does,
and fails loudly if it has not been built.
"""
from .gdn import GdnError, bwd, fwd, fwd_raw, fwd_recurrent, make_args, workspace_bytes  # noqa: F401
