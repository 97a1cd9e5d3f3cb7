"""CPU float64 oracle for BSR attention: test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library.
"""

from .attention import (  # noqa: F401
    attention_dense,
    bsr_attention,
    composable_attention,
    default_scale,
    gather_request_kv,
    kv_lengths,
    merge_state,
    merge_states,
)
from .append import append_paged_kv, append_slots  # noqa: F401
from .fp8 import decode_e4m3  # noqa: F401
from .quest import page_scores, page_summaries, quest_attention, quest_selection, select_pages  # noqa: F401
