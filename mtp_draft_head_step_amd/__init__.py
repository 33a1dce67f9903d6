"""MI355X-native MTP draft round: draft-head step, pending-pair flush,
speculative verification and draft-KV rollback, as hand-written HIP kernels for
gfx950 behind a C ABI (``libmtp.so``, declared in ``include/mtp.h``).

``mtp_draft_head_step_amd.abi`` is the thin ctypes binding (argument marshalling
only); importing it loads the library and fails loudly if it is not built.
``mtp_draft_head_step_amd.inputs`` holds the seeded synthetic input generators.
"""
__all__ = ["abi", "inputs"]
