"""KDA reference implementations -- TEST INFRASTRUCTURE ONLY.

Slow, obviously-correct CPU definitions of the Kimi Delta Attention operator (Kimi K3: Open
Frontier Intelligence, §2.1.1, eq. (1)).  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the HIP library never does and shares no code
with it.

- kda_oracle.py : float64 numpy token loop (the definition)
- kda_oracle.c  : the same token loop in plain C (float64, OpenMP over units), via c_oracle.py
- chunkwise.py  : an independent float64 chunkwise algorithm, used only to pin the token loop
"""
