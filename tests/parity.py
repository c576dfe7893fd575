"""Element-by-element comparison of GPU results with the CPU oracle (the
parity rule lives beside the oracle, in oracle/parity.py)."""
from oracle.parity import check_sample, compare, large_sample, merge, tile_origin  # noqa: F401
