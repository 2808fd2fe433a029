"""Issue-rate probes of the gfx950 instructions the mixer's inner loops use
(measurement infrastructure: see run_probes.py)."""
