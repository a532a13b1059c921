"""MI355X-native DSpark Markov-head draft / prefix-schedule / verify path,
plus RNN-head drafting, parallel-only drafting and the sequential-temperature fit.

The compute runs in hand-written HIP kernels for gfx950 behind the C ABI of
``libdspark.so`` (declared in ``include/dspark.h``).  This package only
marshals arguments: it passes device pointers and the current HIP stream.
Importing the functions below fails loudly if the library is not built.
"""
from .binding import (markov_draft, parallel_draft, schedule, schedule_threshold, serve, sts_fit,  # noqa: F401
                      verify, workspace_bytes, library_path, set_draft_launch, get_draft_launch, rnn_draft,
                      rnn_workspace_bytes, schedule_workspace_bytes, step)
