"""CPU oracle of the DAC-style decoder -- TEST INFRASTRUCTURE ONLY.

Imported only by tests/, ``__graft_entry__.smoke()`` and bench.py's CPU
baseline leg.  Never imported by the product package.
"""
