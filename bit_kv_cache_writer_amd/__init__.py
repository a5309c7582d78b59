"""MI355X-native dual-path low-bit MLA cache: fused writer + decode attention.

The work runs in the HIP library ``libmla_lowbit.so`` (C ABI declared in
``include/mla_lowbit.h``); :mod:`bit_kv_cache_writer_amd.mla` is the thin
ctypes binding over it.  :mod:`bit_kv_cache_writer_amd.workloads` draws the
seeded synthetic inputs.
"""
