"""MI355X-native BN254 G1 multi-scalar multiplication (Pippenger, batched affine adds).

The compute path is the HIP library ``libmsm.so`` built from ``csrc/`` for gfx950;
``elliptic_curve_scalar_amd.msm`` is its thin ctypes binding and
``elliptic_curve_scalar_amd.workloads`` the seeded synthetic inputs.
"""
