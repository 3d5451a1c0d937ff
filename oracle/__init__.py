"""CPU fp64 oracle of the global cross-frame attention layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this package: only the tests, the smoke check and the benchmark's CPU-baseline
leg do. It shares no code with the HIP library.

Every function here is a plain, slow, fp64 NumPy restatement of what the pages
describe; see ``oracle/layer.py`` for the citations and for the readings taken
where the pages leave a step open.
"""
from .layer import *  # noqa: F401,F403
from .layer import __all__  # noqa: F401
