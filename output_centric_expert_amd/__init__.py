"""libmoedecode: output-centric MoE decode expert layer for MI355X (gfx950).

The compute path is the C-ABI shared library ``libmoedecode.so`` (hand-written
HIP kernels); :mod:`output_centric_expert_amd.moedecode` is its ctypes binding
and :mod:`output_centric_expert_amd.synth` makes seeded synthetic inputs.
"""
