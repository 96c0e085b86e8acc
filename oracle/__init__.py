"""fp64 CPU oracle for LoopVQ (test infrastructure only; see loopvq_ref and tasq_ref)."""
from .loopvq_ref import *  # noqa: F401,F403
from .loopvq_ref import NEAR_TIE_REL, NearestResult  # noqa: F401
from . import tasq_ref  # noqa: F401
