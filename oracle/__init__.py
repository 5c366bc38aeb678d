"""fp64 CPU oracle for the cross-model KV mapper.

TEST INFRASTRUCTURE ONLY.  Nothing in the product library imports, calls or
links anything here; only the tests, the smoke check and the bench's CPU
baseline leg do.  It shares no code with the HIP path.
"""

from .kvmap_oracle import *  # noqa: F401,F403
