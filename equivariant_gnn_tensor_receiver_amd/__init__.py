"""MI355X-native streaming CG tensor-product convolution (HIP kernels behind a C ABI).

``equivariant_gnn_tensor_receiver_amd.tpconv`` is the thin ctypes binding over
``libtpconv.so`` (built in-tree by ``__graft_entry__.build()``); it loads the
library on first use and raises if it is missing.  ``inputs`` draws the seeded
synthetic workloads.
"""
