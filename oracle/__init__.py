"""fp64 CPU oracle for ISPA's dual-stream attention and Layer Absorb.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package. The library's product path never calls it, and it shares no code with
the HIP path: it is plain NumPy in float64 (plus pure-Python loops and exact rationals in
`oracle.brute` for tiny cases), written from the definitions on the ISPA summary page
("Instance-Specific Parametric Absorption", gist.science, Italian and Japanese editions):

  * `oracle.attention`  section 2, stage 1 "Dual-Stream Warmup": A_full is attention over the whole
    history, A_loc attention over the sink tokens and the current chunk only. Each output is
    computed from its own key set by the plain softmax definition; there is no branch merge.
  * `oracle.absorb`     section 2, stage 2 "Layer Absorb": the ridge objective and its closed form
    (first and second display equations of that stage), and "Dynamic Layer Selection" (rank layers
    by reconstruction error, lowest first).
  * `oracle.steady`     section 2, stage 3 "Memory-Efficient Inference": the L-Layer steady state
    (updated weights W + dW at the model precision, the output projection, history eviction).
  * `oracle.tempcache`  FAST-AR summary page ("Sintesi Tecnica: FAST-AR"), section 2 part A
    "TempCache", Lemma 5.1: merging duplicate keys (mean values, log group size added to the
    merged key's logit) and softmax attention with a per-key additive logit bias.
  * `oracle.future`     Future Forcing summary page ("Riepilogo Tecnico: Future Forcing"), section
    "Componenti Algorithmiche", module 1: importance of cached keys as their mean attention weight
    under proxy queries of future frames, per-token and hybrid eviction scores.
  * `oracle.fp8`        section 4 "Experimental Results" (ISPA combined with W8A8 quantisation): the
    OCP E4M3 encoding, per-head scaling, and attention scores from dequantised e4m3 Q and K.
  * `oracle.brute`      tiny-size brute force (loops, `fractions.Fraction`) used to pin the above.

Every function is pinned by a `-m "not gpu"` test against closed forms, identities fixed by the
mathematics, textbook routines or brute force. Readings the pages leave open (Gram scaling, error
normalisation, the warmup protocol, the key distribution) are fixed by the workload definitions and
carry no pin from the pages: parity unpinned for those readings only.
"""
from . import attention, absorb, brute, fp8, future, steady, tempcache  # noqa: F401
