"""MI355X-native DSpark Markov-head draft / prefix-schedule / verify path.

The compute runs in hand-written HIP kernels for gfx950 behind the C ABI of
``libdspark.so`` (declared in ``include/dspark.h``).  This package only
marshals arguments: it passes device pointers and the current HIP stream.
Importing the functions below fails loudly if the library is not built.
"""
from .binding import markov_draft, parallel_draft, schedule, verify, workspace_bytes, library_path  # noqa: F401
