"""MI355X-native (gfx950) row-wise RMSNorm and LayerNorm families behind a C ABI
(include/dnorm.h).

``dit_normalization_amd.dnorm`` is the thin binding of ``libdnorm.so``; its ``dn_*``
functions are re-exported here on first use.  Importing any of them without the built
library raises ImportError: there is no CPU fallback.
"""

__all__ = [
    "dn_rmsnorm", "dn_rmsnorm_quant", "dn_fused_add_rmsnorm", "dn_fused_add_rmsnorm_quant",
    "dn_fused_add_rmsnorm_fp8_block_quant", "dn_ada_rms_norm", "dn_gate_residual_ada_norm_fp8",
    "dn_train_forward", "dn_train_backward", "dn_train_backward_noalloc",
    "dn_train_backward_partials",
    "dn_train_backward_reduce", "dn_train_backward_workspace_bytes", "train_backward_workspace",
    "dn_layernorm", "dn_layernorm_quant", "dn_fused_dit_gate_residual_layernorm_gamma_beta",
    "dn_fused_dit_gate_residual_layernorm_scale_shift",
    "dn_fused_dit_residual_layernorm_scale_shift", "dn_fused_qk_rmsnorm_rope",
    "dn_fused_rmsnorm_silu", "dn_rmsnorm_sigmoid_gate", "dn_gated_residual_rmsnorm",
    "dn_gated_residual_next_rmsnorm",
    "dn_force_threads_per_row", "dn_max_hidden", "DnormError",
    "rmsnorm_train",
    "RMSNormTrainFunction",
]


def __getattr__(name):
    if name in ("rmsnorm_train", "RMSNormTrainFunction"):
        from . import autograd
        return getattr(autograd, name)
    if name in __all__:
        from . import dnorm
        return getattr(dnorm, name)
    raise AttributeError(name)
