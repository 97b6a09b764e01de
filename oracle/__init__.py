"""CPU oracle of the mHC pre / H-aggregate forward and backward.

Test infrastructure only: used by tests/, the smoke check and the benchmark's
CPU baseline, never by the product path.
"""
