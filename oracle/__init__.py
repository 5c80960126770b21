"""CPU oracle for RNS-CKKS hybrid key-switching with a ChaCha12-regenerated key half.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
restatement of what the GPU path computes.  Only the test-suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product
path (the HIP library and its Python binding) never does, and shares no code,
tables or constants with it.

Sources.  The pages describe the method only at one point: half of every
key-switching key is uniformly random, so it is regenerated inside the two
kernels that use the key by a counter-mode ChaCha12 expander, which halves key
storage, on a 32-bit RNS CKKS chain (Perseus summary on ai4snews,
"Interpretation" paragraph 2; the Perseus abstract on paperdot names the
in-kernel key regeneration at the backend level).  Everything else here is the
published textbook algorithm, named in each module: RNS-CKKS (Cheon, Han, Kim,
Kim, Song, SAC 2018), hybrid key-switching (Han and Ki, CT-RSA 2020), fast base
conversion (Bajard, Eynard, Hasan, Zucca, SAC 2016), merged-twist negacyclic
NTT (Longa and Naehrig 2016), ChaCha (Bernstein 2008; RFC 8439 state layout).
Where the pages are silent the module states the reading it adopts.

Arithmetic is numpy uint64 on canonical residues in [0, q) with q < 2**32, so
every product of two residues is exact; every product is reduced before it is
summed.  Python integers are used for the big-integer checks.

Modules:
  chain     prime chain, minimal 2N-th roots, big-integer CRT helpers
  ntt       negacyclic NTT/INTT (definition and fast merged-twist form)
  automorph Galois automorphisms in the coefficient and NTT domains
  chacha    ChaCha block function and the counter-mode rejection expander
  rns       ModUp and ModDown fast base conversion
  ks        key generation, inner product, key-switch, hoisted key-switch,
            decryption and the decrypt-after-switch noise check
"""
