"""MI355X (gfx950) WKV7 recurrence of RWKV-7: hand-written HIP kernels behind a
C ABI (include/rwkv7_wkv.h), with this package as its Python binding."""
from .wkv import (ALGOS, Rwkv7Error, abi_version, decode, forward, prepare_decode,  # noqa: F401
                  forward_workspace_bytes, lib)
