"""CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct reference implementations that the HIP path is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from here; the
product library and its Python binding never do.
"""
