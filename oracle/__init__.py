"""CPU float64 oracle of the native-sparse-attention hot path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the library never does.
"""
from .nsa import *  # noqa: F401,F403
