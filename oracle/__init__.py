"""Plain CPU oracle of the routed-expert MoE layer (fp64, NumPy).

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously correct
definition that the GPU path is checked against.  Only the test-suite, the
package's smoke check and the benchmark's CPU-baseline leg may import it; the
product path never does, and it shares no code with the HIP kernels.

Source: "Scalable Training of Mixture-of-Experts Models with Megatron Core"
(gist.science summaries in German, French and Spanish; Spanish technical
summary, section 2.1 "Arquitectura de la capa MoE": route to the k best
experts, dispatch, grouped expert compute, combine).  Where the pages leave a
step open (softmax over the selected k, SwiGLU experts, tie-breaking, fp8 block
quantisation) the reading used is stated in each function's docstring.

Every function here is pinned by CPU tests against brute force, closed forms,
invariants, finite differences or an independent library derivation; none is
"parity unpinned".
"""
from .moe import *  # noqa: F401,F403
from .e4m3 import *  # noqa: F401,F403
from .moe_e4m3 import *  # noqa: F401,F403
from .router import *  # noqa: F401,F403
from .mx import *  # noqa: F401,F403
