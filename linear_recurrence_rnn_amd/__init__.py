"""MI355X (gfx950) per-channel linear recurrences: RWKV-4 WKV forward/backward and
real/complex diagonal scans with their adjoints, as hand-written HIP kernels behind a C ABI
(``include/linrec.h``).  The Python functions here marshal torch tensors to that ABI.

The binding is imported lazily so that ``linear_recurrence_rnn_amd.workloads`` (the seeded
input generators) can be used without loading the GPU library.
"""

__all__ = ["wkv4_forward", "wkv4_forward_noalloc", "wkv4_forward_ex", "wkv4_decode_step", "token_shift", "token_shift_backward", "wkv4_backward", "wkv4_backward_gated", "wkv4_backward_ex",
           "wkv4_forward_ckpt", "wkv4_backward_ckpt", "wkv4_forward_ckpt_ex", "wkv4_backward_ckpt_ex", "wkv4_checkpoint_size", "scan_real", "scan_complex", "scan_real_backward",
           "scan_complex_backward", "scan_mingru", "scan_minlstm", "scan_real_decay",
           "scan_complex_normalized", "scan_mingru_backward", "scan_minlstm_backward",
           "scan_real_decay_backward", "scan_complex_normalized_backward", "workspace_size", "LinrecError"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
