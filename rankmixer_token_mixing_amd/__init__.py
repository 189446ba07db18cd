"""RankMixer block forward for MI355X (gfx950): token mixing, per-token FFN,
ReLU-gated per-token MoE, pad-split tokenizer and mean pooling, as HIP kernels
behind the C ABI of ``librankmixer.so`` (declared in include/rankmixer.h).

The Python names mirror the C entry points; they only marshal torch tensors
to pointers.  Importing this package does not load the library; the first
call does, and it raises if the library is missing.
"""
_BINDING_NAMES = (
    "RankMixerError", "lib_path", "load", "rm_block_fwd", "rm_model_fwd", "rm_moe_relu_fwd",
    "rm_moe_route", "rm_pffn_fwd", "rm_token_mix", "rm_tokenize_padsplit", "workspace_bytes",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
