"""One rank of a Megatron-style tensor-parallel transformer block on MI355X (gfx950).

The compute lives in ``libtpshard.so`` (HIP kernels behind a C ABI, declared in
``include/tpshard.h``); ``tpshard`` is its thin Python binding and
``inputs`` draws the seeded synthetic workloads.
"""
