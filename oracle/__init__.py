"""fp64 CPU oracle for Video Delta Attention (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg may import this
package.  The HIP library shares no code with it.
"""
from .vda_oracle import *  # noqa: F401,F403
from .vda_oracle import __all__  # noqa: F401
