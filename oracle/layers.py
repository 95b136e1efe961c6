"""Which linear layers run in NVFP4 and which stay bf16.

Test infrastructure only (see the package docstring).

[P1] section "NVFP4量化" prints the regex the FLUX.2 integration passes as
``exclude_pattern`` and says it names the layers that are *not* quantized.
The regex itself is a negative lookahead: it matches exactly the names that
contain none of six substrings.  Reading R-12: a layer is NVFP4 iff the regex
matches its name, so layers whose name holds one of the substrings stay bf16 --
which is also what the prose says.  The oracle is Python's ``re`` applied to
the printed pattern.
"""

import re

EXCLUDE_PATTERN = r"^(?!.*(embedder|norm_out|proj_out|to_add_out|to_added_qkv|stream)).*"


def layer_is_quantized(name, pattern=EXCLUDE_PATTERN):
    """True when ``pattern`` matches ``name`` at its start (``re.match``)."""
    return re.match(pattern, name) is not None
