"""FibQuant CPU oracle: plain, slow, float64 reference of the codec.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it, plus
``oracle/build_codebooks.py``, the offline script that writes the shared
codebook artifacts.  The oracle shares no code with the HIP path; the only
thing both sides read is the artifact file (the rotation and the codebook
table), whose parser each side implements on its own.

Sources, cited by short name throughout the package:

* [FQ]  "FibQuant: Universal Vector Quantization for Random-Access KV-Cache
  Compression", technical summary (gist.science, zh and fr editions), with
  the section number of that summary (1 problem statement, 2.1 canonical
  source, 2.2 codebook construction, 2.3 encoding and decoding, 3.1-3.3
  contributions, 4.1-4.3 experiments, 5 significance).
* [FQ-abs] the authors' abstract of the same paper (paper-with-me page).
* [TQ]  "TurboQuant: Online Vector Quantization with Near-optimal Distortion
  Rate", reading notes (leeon-k.github.io), with their section numbers
  (1.3 overview, 2 preliminaries / coordinate lemma, 2.1 Shannon lower bound,
  3.1 MSE-optimal TurboQuant, 3.3 lower bound).
* [BSQ] "Block Sphere Vector Quantization" (NeurIPS 2026 notes,
  papernotes.org): key design 1 (exact block marginal), key design 2
  (Cartesian LUT search), main table, ablation table.

Modules, one step each, in the pages' order:

* ``rotation``  -- the shared Haar rotation (QR of a Gaussian matrix).
* ``source``    -- the canonical spherical-Beta block source and samplers.
* ``codebook``  -- Beta-quantile radii, Fibonacci / Roberts-Kronecker
  directions, multi-restart Lloyd-Max.
* ``scalar``    -- the scalar (k = 1) Lloyd-Max comparator of TurboQuant.
* ``codec``     -- normalise, rotate, block nearest-codeword search, pack,
  unpack, decode; fp16 rounding of the norm.
* ``attend``    -- decode-step attention over a decompressed cache.
* ``artifact``  -- the codebook artifact file (writer and reader).

Readings taken where the pages are silent are listed in each function's
docstring.  "parity unpinned" marks any function with no pin in
``tests/``; at present there is none.
"""
