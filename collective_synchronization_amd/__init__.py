"""Self-synchronizing small-message one-shot bf16 all-reduce for MI355X.

Submodules:
  abi      -- ctypes binding of libcsync_ar.so (the C ABI in include/ar.h)
  buffers  -- torch-allocated device buffers for the binding (marshalling)
  inputs   -- seeded synthetic workloads (no all-reduce arithmetic)
  configs  -- the five workloads
  selector -- fitting the cost table of the protocol selector

The HIP library is loaded by ``abi``; importing it without the built library
raises ImportError.  There is no CPU implementation in this package.
"""
__all__ = ["abi", "buffers", "inputs", "configs", "selector"]
