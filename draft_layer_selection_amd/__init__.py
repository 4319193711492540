"""MI355X-native KnapSpec layer-selection DP: HIP kernels behind a C ABI (libknapspec.so).

Import ``draft_layer_selection_amd.knapspec`` for the binding (it requires the built
library and raises otherwise).
"""
