"""MI355X-native paged decode attention: a C-ABI library (``libpa.so``, gfx950 HIP
kernels) and a thin ctypes binding with the same entry-point names.

Importing the package does not load the library; the first call does, and fails
loudly when it has not been built."""
from .binding import (BlockManager, PaError, PreparedCacheWrite,  # noqa: F401
                      PreparedCopyBlocks, PreparedDecode, PreparedMultiToken, pa_cache_write,
                      pa_cache_write_decode,
                      pa_copy_blocks, pa_decode, pa_decode_noalloc, pa_decode_workspace_bytes,
                      pa_multi_token, pa_read_probe,
                      decode_partition_used, workspace_for)
