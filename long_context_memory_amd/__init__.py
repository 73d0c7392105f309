"""MI355X-native Memory Sparse Attention (MSA) hot path.

The compute path is the HIP library ``libmsa.so`` (built from ``csrc/`` by
``long_context_memory_amd.build``); ``long_context_memory_amd.msa`` is its
thin ctypes binding.  ``synth`` draws seeded synthetic inputs.
"""
