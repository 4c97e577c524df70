"""CPU oracle for the routed, block-quantized MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library under ``quantized_expert_ffn_top_amd/`` and imports nothing from it.

What it computes is the plain definition of the layer, slowly:

* ``formats``  -- scalar (pure Python) and vectorised (NumPy) unpackers and
  dequantisers of the two expert weight codecs, and the round-to-nearest
  quantisers used to build test data.
* ``moe``      -- router logits, exact top-k, softmax over the selected logits,
  stable counting-sort permutation, the SwiGLU expert FFN, the always-on shared
  expert, the weighted combine, and the RMSNorm + residual step between
  stacked layers; all floating point in fp64, with bf16 round-to-nearest-even
  applied exactly where the numerics contract puts it.

Sources (the web pages this layer is read from):

* "Avalon" README, opening paragraphs: the model routes every token to 10 of
  512 experts in each of 48 layers.
* "Qwen3.8-Flash-Next - Avalon GGUF" model card, "Files / Main model": the
  routers and shared experts sit in the dense part; routed up/gate use a
  3.25-bpw codec with one scale per 256-weight block and per-32 sub-scales;
  down uses a 4-bit non-linear 32-weight codec; each expert is packed as
  up | gate | down, contiguous.
* "Betelgeuse" post (2026-11-01): all 10 routed experts are computed (no gate
  pruning) and router records are checked byte-for-byte.

The pages give no byte layout, codebook, router formula or activation; the
readings taken where they are silent are listed in the header of each module.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
something other than itself (hand-derived byte vectors and values stored under
``tests/golden/``, closed forms, library routines for special cases, brute force
on tiny inputs, invariants).  No function is "parity unpinned".
"""
