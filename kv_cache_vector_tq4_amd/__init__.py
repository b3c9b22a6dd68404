"""TurboQuant KV-cache compression and compressed paged decode for MI355X (gfx950).

The product is libfq.so (C ABI declared in include/fq.h): a host codebook /
rotation builder plus HIP kernels for compress and decode attention. ``fq``
is the thin ctypes binding; ``synth`` makes seeded synthetic workloads.
"""
