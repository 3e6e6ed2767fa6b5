"""fp64 CPU oracle of the IceCache hot path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package. The library under ``ann_retrieval_amd/`` never imports it, and it
imports nothing from the library: the two share no code. The one shared
module is ``ann_retrieval_amd.synth`` (seeded input draws, no arithmetic of
the method), and the oracle does not even import that: inputs are passed in.
"""
from .icecache import *  # noqa: F401,F403
