"""MI355X drafter block forward: HIP kernels behind a C ABI (libdbf.so).

Import ``verifier_block_forward_amd.dbf`` for the binding; it loads the built
library and raises if it is missing.
"""
