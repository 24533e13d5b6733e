"""Test-only CPU oracle (fp64).  Only tests, the smoke check and the bench's
CPU-baseline leg may import this package; the product path never does."""
from .nystrom_oracle import *  # noqa: F401,F403
from .nystrom_backward import *  # noqa: F401,F403
from .nystrom_layer import *  # noqa: F401,F403
