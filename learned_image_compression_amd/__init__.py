"""MI355X (gfx950) indexed rANS64 entropy coder for learned image compression.

The coder is the hand-written HIP library ``librans_hip.so`` behind the C ABI
declared in ``include/rans_hip.h``; ``learned_image_compression_amd.binding``
marshals torch tensors into it.  Importing this package does not load the
library; the first call does, and fails loudly if it was not built.
"""
