"""MI355X (gfx950) implementation of the Kimi Delta Attention (KDA) forward pass.

The compute lives in ``libkda.so`` (HIP kernels behind the C ABI of ``include/kda.h``);
``gated_delta_rule_60_amd.kda`` is its ctypes binding and ``gated_delta_rule_60_amd.inputs``
the seeded synthetic workloads.  Importing the package loads nothing: the library is loaded on
the first call and a missing build raises.
"""

__all__ = ["kda", "inputs", "build"]
