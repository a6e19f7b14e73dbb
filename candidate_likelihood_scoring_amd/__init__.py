"""MI355X-native teacher-forced candidate-likelihood scoring (libjet, gfx950).

The scoring path runs in hand-written HIP kernels behind the C ABI of include/jet.h; this
package is the thin Python binding (torch supplies device memory and streams).
"""
from ._lib import JetError, LIB_PATH, load  # noqa: F401
from .api import (  # noqa: F401
    Workspace,
    build_union,
    score,
    score_restricted,
    score_workspace_size,
    restricted_workspace_size,
    validate,
    validate_restricted,
)
