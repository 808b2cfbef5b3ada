"""CPU oracle of the int4-g64 grouped MoE layer: test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU baseline may import it.
"""
