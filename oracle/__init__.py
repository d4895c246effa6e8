"""CPU oracle for the OCR-decoder decode step (plain numpy, float64).

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
imports, links or calls it, and it shares no code with the library: the two
meet only in the seeded inputs drawn by ``synth``.

Every function states the passage of the pages it follows.  The pages are:

* [UOCR]   "Eseguire Unlimited-OCR su Apple Silicon con C e Metal"
           (mauroscia.it gradientlab), sections "In sintesi", "Il decoder e il
           Mixture of Experts", "Quantizzazione: Q8 prima, Q4 dove conviene".
* [NCNN]   "HunyuanOCR 的 ncnn 移植" (Tencent/ncnn discussion 6880), sections
           3.2 (decoder and KV cache) and 3.4 (greedy token choice).
* [FALCON] "Nicolassuez/Falcon-OCR-int8-openvino" (Hugging Face model card),
           paragraphs on the attention sink, the KV cache as an input, the
           INT8_ASYM weights and "How it is meant to be run".

Where the pages leave a step open, the reading taken is stated at the function.
Every primitive here is pinned by a CPU test against something other than
itself (hand-built blocks, closed forms, brute force, identities); the composed
multi-layer step is pinned only through its parts and the invariants listed in
the tests (parity of the 12-layer composition as a whole is unpinned beyond the
oracle itself, since the pages print no numbers for it).
"""
from .core import *  # noqa: F401,F403
