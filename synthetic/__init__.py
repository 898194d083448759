"""Seeded synthetic inputs for the bundle-adjustment solvers.

The generators here draw random scenes and synthesise image observations with a
forward image model written on scipy's ``Rotation`` and numpy.  They contain no
part of the solver itself (no linearisation, assembly, damping, elimination,
linear solve or parameter update).  The CPU oracle and the GPU library both take
their inputs from here and share nothing else.
"""

from .ba import CONFIGS, ba_scene, heavy_camera_scene, scene_summary  # noqa: F401
from .droid import droid_scene  # noqa: F401
from .pgo import PGO_CONFIGS, pgo_scene, pgo_summary  # noqa: F401
