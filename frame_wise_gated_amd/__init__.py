"""Frame-wise Gated DeltaNet frame scan for AMD Instinct MI355X (gfx950).

The compute lives in the C-ABI library ``libgdn.so`` (hand-written HIP
kernels); ``frame_wise_gated_amd.gdn`` is its thin ctypes binding and
``frame_wise_gated_amd.inputs`` the seeded synthetic-input generator. This
package import is deliberately light: nothing is loaded until ``gdn`` is
imported.
"""
