"""Sampling-transform scoring core for AMD Instinct MI355X (gfx950).

The scoring arithmetic lives in the HIP library ``libstce.so`` (built from
``csrc/``); this package only marshals arguments to its C ABI.
"""
