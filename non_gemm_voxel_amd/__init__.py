"""MI355X-native hot path of fused non-GEMM image registration.

``non_gemm_voxel_amd.ngv`` is the thin binding over the C-ABI library
``libngv.so`` (HIP kernels for gfx950); ``non_gemm_voxel_amd.synth`` makes the
seeded synthetic volume pairs. Importing the package loads neither.
"""
