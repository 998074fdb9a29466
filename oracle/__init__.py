"""CPU oracle for one pretraining step of the depth-parameterised GPT and its Muon update.

TEST INFRASTRUCTURE ONLY. Imported solely by tests/, by __graft_entry__.smoke()
and by the cpu_baseline leg of bench.py. The product path (the HIP library and
its Python binding) never imports, links or calls anything here, and nothing
here imports the product path.

The oracle is the plain definition of what the step computes, in NumPy, in the
floating-point type of its inputs (float64 for checks, float32 for timing). It
performs no blocking, fusion or reordering beyond what the definitions state.

Sources (cited by page title and section):
  [CT50]  dev.to, "Como treinar seu próprio ChatGPT por 50 dólares".
  [HADA]  GeekNews (hada.io) summary of the nanochat launch README.

Parity status of each function is stated in its module header.
"""
from .gpt import (  # noqa: F401
    EPS_NORM,
    attention_by_head,
    attention_by_head_bwd,
    ROPE_BASE,
    causal_attention,
    causal_attention_bwd,
    forward_backward,
    forward_logits,
    rms_norm,
    rms_norm_bwd,
    rope,
    rope_bwd,
    rope_tables,
)
from .adamw import adamw_step, adamw_update  # noqa: F401
from .muon import muon_step, newton_schulz, newton_schulz_svd  # noqa: F401
from .polar_express import greedy_minimax_triples  # noqa: F401
from .normuon import normuon_step, variance_reduction  # noqa: F401
from .packing import pack_best_fit  # noqa: F401
