"""CPU oracle of the selective scan (S6) — TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import
anything here.  The GPU library (selective_state_space_34_amd) never does, and
the two share no code: only the seeded input generators in gen/ serve both.

  ss_ref  numpy float64 forward/backward (small cases, pins)
  cref    ctypes front end of ss_oracle.c, the same definition in C + OpenMP
"""
