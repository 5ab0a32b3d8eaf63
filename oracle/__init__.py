"""ORACLE -- test infrastructure, not part of the library.

A plain, slow CPU implementation of one expert-parallel rank's share of the
Mixture-of-Experts layer described in "Hosting Qwen on Blackwell"
(Perplexity).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it.  It shares no code with the
HIP path and imports nothing from it.

Router logits are float32 in a fixed summation order (``router_logits.c``,
plain C); everything after them is float64 numpy (``moe.py``).  The MXFP8
variant of the expert GEMMs (the pages' deployed quantisation, OCP
Microscaling format) is ``mxfp8.py``.
"""
from .moe import (combine, dispatch, expert_ffn, moe_layer, moe_layer_rows, num_threads,  # noqa: F401
                  pack, route, router_logits, select_topk, silu, softmax, topk_weights)
from . import mxfp8  # noqa: F401
