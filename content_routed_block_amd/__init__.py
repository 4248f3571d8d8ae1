"""Content-routed block sparse attention for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``liblsa.so`` (hand-written HIP
kernels); ``content_routed_block_amd.lsa`` is its thin Python binding and
``content_routed_block_amd.workloads`` draws the seeded synthetic inputs.
"""
