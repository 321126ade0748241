"""libmiattn: fused softmax-attention forward for AMD Instinct MI355X (gfx950).

The compute lives in the HIP C-ABI library ``libmiattn.so`` (sources under
``csrc/``, declarations in ``include/miattn.h``); :mod:`.miattn` is the thin
ctypes binding with the same entry-point names. :mod:`.inputs` holds the
seeded synthetic workloads.
"""
__all__ = ["miattn", "inputs"]
