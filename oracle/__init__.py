"""fp64 CPU oracle for the packed in-place real FFT and block-circulant layers.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it, and this package imports nothing from the product path: the two
share no code, tables or helpers.  Inputs reach both sides from the seeded
generators in ``block_circulant_layers_amd.synthetic``, which hold none of the
method's arithmetic.

Source pages (all describe "Memory-Efficient Training with In-Place FFT
Implementation", NeurIPS 2025, arXiv 2511.01385):
  * the Paper-Notes page (zhaoyang97.github.io), section "方法详解 / 关键设计":
    packed layout ("Squeeze"), Proposition 1 four-element groups, in-place
    IFFT formulas, circulant training adaptation;
  * the scime.ai summary page, sections "Approach" and "Problem".

Modules
  rdfft_oracle     packed forward / inverse transform as the DFT definition
                   (numpy's complex FFT as the DFT primitive) plus the packing
                   rule; packed spectrum product.
  packed_stages    the pages' algorithm itself (radix-2 Cooley-Tukey on
                   four-element conjugate-symmetric groups, in place), in plain
                   Python loops, for small rows.  Pins the reading of the pages.
  circulant_oracle block-circulant layer forward / backward, once as the dense
                   matrix definition and once as the pages' FFT formula.
  rdfft2d_oracle   the 2D extension (packed along each axis where the data is
                   conjugate-symmetric), as the 2D DFT definition plus its
                   packing rule.

Every function here is pinned by ``tests/test_oracle.py`` (2D:
``tests/test_oracle2d.py``) against something
other than itself (brute-force DFT, closed forms, the pages' worked index
example, finite differences, invariants).  No function is "parity unpinned".
"""
