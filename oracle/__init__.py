"""Test infrastructure: the CPU oracle of the tile-aligned W4/W8 x A8 linear
layer.  Only tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does."""
from . import aq_oracle  # noqa: F401
