"""CPU oracle of the decode hot path.  TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline)."""
from .oracle import *  # noqa: F401,F403
from .oracle import build, lib, OracleModel  # noqa: F401
