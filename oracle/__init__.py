"""CPU fp64 oracle of the gated delta-rule core and its gated-RMSNorm tail.

Test infrastructure only: used by tests/, the smoke check and the CPU baseline
leg of bench.py.  The library and its binding never import this package.
"""
