"""fp64 CPU oracle of the routed-expert MoE FFN layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg.  The GPU library never imports or links it, and
it imports nothing from the GPU package.
"""
