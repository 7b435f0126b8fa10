"""CPU oracle of the routed-expert MoE FFN -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the GPU library.
"""
from . import moe_oracle  # noqa: F401
