"""CPU oracle of the draft-block forward. Test infrastructure only: imported
by the tests, the smoke check and the benchmark's CPU-baseline leg, never by
the library."""
from .dspark_oracle import *  # noqa: F401,F403
