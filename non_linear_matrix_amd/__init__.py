"""M²RNN forward recurrence for AMD Instinct MI355X (gfx950).

The computation runs in libm2rnn.so (hand-written HIP); ``non_linear_matrix_amd.m2rnn``
is its ctypes binding and ``non_linear_matrix_amd.inputs`` the seeded workload
generator. Importing the package does not load the library; the first call does,
and fails loudly if it has not been built.
"""

__version__ = "0.1.0"
