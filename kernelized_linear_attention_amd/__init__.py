"""Kernelized linear attention for AMD MI355X (gfx950).

The compute path is the C-ABI library ``liblinattn.so`` (hand-written HIP
kernels, declared in ``include/lin_attn.h``).  ``kernelized_linear_attention_amd.binding``
exposes its entry points to Python under the same names; importing it loads
the library and fails loudly when it has not been built.

``inputs`` and ``workloads`` are plain-data helpers (seeded random inputs and
the workload shapes) that do not need a GPU.
"""
__all__ = ["binding", "inputs", "workloads"]
