"""MI355X (gfx950) WKV7 recurrence of RWKV-7: hand-written HIP kernels behind a
C ABI (include/rwkv7_wkv.h), with this package as its Python binding."""
from .wkv import (ALGOS, CKPT_INTERVAL, Rwkv7Error, abi_version, backward,  # noqa: F401
                  backward_workspace_bytes,
                  decode, decode_fused, forward, forward_bidir, forward_bidir_workspace_bytes,
                  forward_fused, forward_noalloc, forward_train,
                  forward_workspace_bytes, lib, prepare_decode, stream_copy)
