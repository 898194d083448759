"""MI355X-native Levenberg-Marquardt bundle adjustment.

``libba.so`` (fp64, include/ba.h) holds one LM iteration of large-scale
bundle adjustment as hand-written gfx950 HIP kernels; ``libdba.so``
(include/dba.h) holds the fp32 dense frame-graph variant; ``libpgo.so``
(include/pgo.h) holds fp64 pose-graph optimisation.  The Python modules
here only marshal arguments.
"""

from . import ba, dba, pgo  # noqa: F401
