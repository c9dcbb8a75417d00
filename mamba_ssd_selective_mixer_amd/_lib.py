"""ctypes binding of libssd_mi355x.so (the C ABI in include/ssd_mi355x.h).

Loading needs no GPU; every compute entry needs one. There is no fallback:
if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssd_mi355x.so")

SSD_F32, SSD_BF16 = 0, 1
KERNELS = ("conv1d_silu", "conv_state", "gated_rmsnorm", "decode_step", "chunk_state",
           "state_pass", "chunk_out", "fused_chunk_state", "fused_state_pass",
           "fused_chunk_out_norm", "bwd_gated_norm", "bwd_chunk_z", "bwd_rev_pass", "bwd_chunk",
           "bwd_group_sum", "bwd_conv_du", "bwd_conv_dx", "bwd_y", "chunk_cb")
ENTRY = {"conv1d": 0, "chunk_scan": 1, "gated_rmsnorm": 2, "decode_step": 3, "mixer_prefill": 4}
STATUS = {0: "SSD_OK", -1: "SSD_ERR_NULL", -2: "SSD_ERR_SHAPE", -3: "SSD_ERR_UNSUPPORTED",
          -4: "SSD_ERR_DTYPE", -5: "SSD_ERR_ALIAS", -6: "SSD_ERR_WORKSPACE", -7: "SSD_ERR_HIP",
          -8: "SSD_ERR_ALIGN", -9: "SSD_ERR_TIMEOUT", -10: "SSD_ERR_NONFINITE",
          -11: "SSD_ERR_SCRATCH", -12: "SSD_ERR_VARLEN"}
SSD_FLAG_FP32_OPERANDS = 1

# every symbol the header declares
EXPORTS = ("ssd_conv_channels", "ssd_ssm_state_bytes", "ssd_conv_state_bytes", "ssd_validate",
           "ssd_status_str", "ssd_conv1d", "ssd_chunk_scan_workspace_bytes", "ssd_chunk_scan",
           "ssd_gated_rmsnorm", "ssd_decode_step", "ssd_mixer_prefill_workspace_bytes",
           "ssd_mixer_prefill", "ssd_mixer_prefill_packed", "ssd_decode_step_packed",
           "ssd_mixer_varlen_workspace_bytes", "ssd_mixer_varlen",
           "ssd_mixer_prefill_noalloc", "ssd_mixer_backward_workspace_bytes",
           "ssd_mixer_backward", "ssd_workspace_status", "ssd_set_exchange_spin_limit",
           "ssd_set_backward_chunk_heads", "ssd_set_output_norm_fusion",
           "ssd_profile_start", "ssd_profile_stop", "ssd_profile_set_mask", "ssd_profile_read",
           "ssd_kernel_name")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "seqlen", "nheads", "headdim", "ngroups", "dstate", "conv_width",
                 "chunk", "io_dtype", "flags")]


_lib = None


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library {LIB_PATH} is not built; run __graft_entry__.build() "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Dims)
    vp, i64, f32, sz, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_int
    sig = {
        "ssd_conv_channels": (i64, [P]),
        "ssd_ssm_state_bytes": (i64, [P]),
        "ssd_conv_state_bytes": (i64, [P, i32]),
        "ssd_validate": (i32, [i32, P]),
        "ssd_status_str": (ctypes.c_char_p, [i32]),
        "ssd_conv1d": (i32, [P, vp, i64, vp, vp, vp, vp, vp, i64, vp]),
        "ssd_chunk_scan_workspace_bytes": (sz, [P]),
        "ssd_chunk_scan": (i32, [P, vp, i64, vp, vp, vp, vp, vp, i64, vp, vp, f32, vp, vp, vp,
                                 vp, sz, vp]),
        "ssd_gated_rmsnorm": (i32, [P, vp, vp, vp, f32, vp, vp]),
        "ssd_decode_step": (i32, [P, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp]),
        "ssd_mixer_prefill_workspace_bytes": (sz, [P]),
        "ssd_mixer_prefill": (i32, [P, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp,
                                    vp, sz, vp]),
        "ssd_mixer_prefill_packed": (i32, [P, vp, i64, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp,
                                           vp, vp, vp, sz, vp]),
        "ssd_decode_step_packed": (i32, [P, vp, i64, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp,
                                         vp]),
        "ssd_mixer_varlen_workspace_bytes": (sz, [P, i32]),
        "ssd_mixer_varlen": (i32, [P, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp,
                                   vp, vp, sz, vp]),
        "ssd_mixer_prefill_noalloc": (i32, [P, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp,
                                            vp, vp, vp]),
        "ssd_mixer_backward_workspace_bytes": (sz, [P]),
        "ssd_mixer_backward": (i32, [P, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp,
                                     vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "ssd_workspace_status": (i32, [vp, vp]),
        "ssd_set_exchange_spin_limit": (i32, [i32]),
        "ssd_set_backward_chunk_heads": (i32, [i32]),
        "ssd_set_output_norm_fusion": (i32, [i32]),
        "ssd_profile_start": (i32, [i32]),
        "ssd_profile_stop": (i32, []),
        "ssd_profile_set_mask": (ctypes.c_uint64, [ctypes.c_uint64]),
        "ssd_profile_read": (i32, [i32, ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)]),
        "ssd_kernel_name": (ctypes.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_str(rc: int) -> str:
    return load().ssd_status_str(rc).decode()
