"""CPU oracle for the ConvRot W4A8 codebook linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table, constant
or helper with the HIP library in ``bit_codebook_quantized_amd/``; the two meet
only through the seeded input generators in ``bit_codebook_quantized_amd/synth.py``,
which hold none of the method's arithmetic.

See ``oracle/convrot_w4a8.py`` for the functions and their citations.
"""

from .convrot_w4a8 import *  # noqa: F401,F403
from .convrot_w4a8 import __all__  # noqa: F401
