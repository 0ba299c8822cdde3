"""Kimi Delta Attention (gated delta rule) for AMD MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(`libkda.so`, declared in include/kda.h).  `gated_delta_rule_42_amd.kda` is the
thin ctypes binding with the same entry-point names; it only marshals
arguments.  `workloads` draws the seeded synthetic inputs.
"""
__all__ = ["kda", "workloads"]
