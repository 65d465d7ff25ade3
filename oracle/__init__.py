"""CPU fp64 oracle for exact attention and its gradients (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library.
"""

from .exact import (  # noqa: F401
    allowed_key_mask,
    attention,
    attention_head,
    attention_rows,
    attention_samples,
)
from .gradient import (  # noqa: F401
    attention_backward,
    attention_backward_head,
    backward_samples,
)
from .gradient_kv import (  # noqa: F401
    attention_backward_kv,
    attention_backward_kv_head,
)
from .kv import (  # noqa: F401
    allowed_keys_kv,
    attention_kv,
    attention_kv_rows,
    attention_kv_samples,
)
