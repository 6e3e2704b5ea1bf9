"""FP64 CPU oracle for the KDA token mixer.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it; the library never does.
"""
