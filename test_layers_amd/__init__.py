"""MI355X-native LaCT fast-weight layer forward (update + apply).

The compute path is the C-ABI library `liblact.so` (hand-written gfx950 HIP
kernels); `test_layers_amd.lact` is its thin ctypes binding.  Importing this
package loads nothing: import `test_layers_amd.lact` for the binding and
`test_layers_amd.workloads` for the seeded synthetic inputs.
"""
