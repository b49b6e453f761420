"""ctypes binding of libvlm.so (include/vlm.h): same names, argument marshalling only.

Every computation runs in the library's HIP kernels; this module only
declares the C types and signatures and turns non-zero status codes into
exceptions. It fails loudly when the library has not been built.
"""
import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvlm.so")

VLM_OK, VLM_ERR_ARG, VLM_ERR_SHAPE, VLM_ERR_CAPACITY, VLM_ERR_COUNT_MISMATCH = 0, -1, -2, -3, -4
VLM_ERR_DTYPE, VLM_ERR_NONFINITE, VLM_ERR_HIP, VLM_ERR_UNSUPPORTED, VLM_ERR_WORKSPACE = -5, -6, -7, -8, -9
STATUS_NAMES = {0: "VLM_OK", -1: "VLM_ERR_ARG", -2: "VLM_ERR_SHAPE", -3: "VLM_ERR_CAPACITY",
                -4: "VLM_ERR_COUNT_MISMATCH", -5: "VLM_ERR_DTYPE", -6: "VLM_ERR_NONFINITE", -7: "VLM_ERR_HIP",
                -8: "VLM_ERR_UNSUPPORTED", -9: "VLM_ERR_WORKSPACE"}
VLM_F32, VLM_BF16 = 0, 1
VLM_BLOCK_DECODER, VLM_BLOCK_VIT, VLM_BLOCK_MLA = 0, 1, 2
VLM_MASK_CAUSAL, VLM_MASK_NONE, VLM_MASK_ADDITIVE, VLM_MASK_SEGMENT = 0, 1, 2, 3
KV_HEADER_BYTES = 256


class VlmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class ModelDesc(C.Structure):
    _fields_ = [("block_kind", C.c_int32), ("n_layers", C.c_int32), ("hidden", C.c_int32),
                ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("ffn", C.c_int32), ("vocab", C.c_int32), ("dtype", C.c_int32), ("qk_norm", C.c_int32),
                ("rope_segments", C.c_int32), ("norm_eps", C.c_float), ("rope_interleave", C.c_int32),
                ("q_lora_rank", C.c_int32), ("kv_lora_rank", C.c_int32), ("qk_rope_dim", C.c_int32),
                ("v_head_dim", C.c_int32)]


class Layer(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "attn_norm_b", "wqkv", "bqkv", "q_norm", "k_norm", "wo",
                                          "bo", "mlp_norm", "mlp_norm_b", "w1", "b1", "w2", "b2",
                                          "w_a", "q_a_norm", "q_b", "kv_a_norm", "kv_b")]


class Mask(C.Structure):
    _fields_ = [("kind", C.c_int32), ("ld_add", C.c_int32), ("add", C.c_void_p), ("seg", C.c_void_p)]


class Merger(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("merge", C.c_int32), ("merger_hidden", C.c_int32), ("out_dim", C.c_int32),
                ("dtype", C.c_int32), ("norm_eps", C.c_float)] + \
               [(n, C.c_void_p) for n in ("post_ln", "post_ln_b", "w1", "b1", "w2", "b2")]


class Sampling(C.Structure):
    _fields_ = [("temperature", C.c_float), ("top_k", C.c_int32), ("top_p", C.c_float),
                ("repetition_penalty", C.c_float)]


_P = C.c_void_p
_I = C.c_int32
_SIG = {
    "vlm_last_error": (C.c_char_p, []),
    "vlm_kv_bytes": (_I, [C.POINTER(ModelDesc), _I, C.POINTER(C.c_size_t)]),
    "vlm_kv_alloc": (_I, [C.POINTER(ModelDesc), _I, _P, C.c_size_t, _P, C.POINTER(_P)]),
    "vlm_kv_free": (_I, [_P]),
    "vlm_kv_len": (_I, [_P, C.POINTER(_I)]),
    "vlm_kv_truncate": (_I, [_P, _I, _P]),
    "vlm_kv_status": (_I, [_P, _P, C.POINTER(_I)]),
    "vlm_token_status": (_I, [_P, _P, C.POINTER(_I)]),
    "vlm_workspace_bytes": (_I, [C.POINTER(ModelDesc), _I, C.POINTER(C.c_size_t)]),
    "vlm_pack_qkv": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "vlm_pack_gate_up": (_I, [_P, _P, _I, _I, _I, _P, _P]),
    "vlm_rope_table": (_I, [_P, _I, _I, C.POINTER(_I), _I, _I, C.c_double, _P, _P, _P]),
    "vlm_rope_alpha_base": (_I, [C.c_double, C.c_double, _I, C.POINTER(C.c_double)]),
    "vlm_sample_logits": (_I, [_P, _I, C.POINTER(Sampling), _P, _I, _P, _P, _P]),
    "vlm_embed": (_I, [C.POINTER(ModelDesc), _P, _P, _I, _P, _P]),
    "vlm_inject_image_embeds": (_I, [C.POINTER(ModelDesc), _P, _I, C.POINTER(_I), _P, _I, _P, _I, _I, _P]),
    "vlm_prefill": (_I, [C.POINTER(ModelDesc), C.POINTER(Layer), _P, _I, _I, _P, _P, _I, C.POINTER(Mask), _I, _P,
                         _P, C.c_size_t, _P]),
    "vlm_lmhead_argmax": (_I, [C.POINTER(ModelDesc), _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "vlm_lmhead_argmax_noalloc": (_I, [C.POINTER(ModelDesc), _P, _P, _P, _P, _P, _P]),
    "vlm_lmhead_argmax_rows": (_I, [C.POINTER(ModelDesc), _P, _P, _P, _I, _P, _P, _P, C.c_size_t, _P]),
    "vlm_verify_commit": (_I, [_P, _I, C.POINTER(_I), _I, _P, _P, C.POINTER(_I), C.POINTER(_I)]),
    "vlm_decode_step": (_I, [C.POINTER(ModelDesc), C.POINTER(Layer), _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P,
                             _P, C.c_size_t, _P]),
    "vlm_decode_loop": (_I, [C.POINTER(ModelDesc), C.POINTER(Layer), _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _P,
                             C.c_size_t, _P]),
    "vlm_decode_loop_sampled": (_I, [C.POINTER(ModelDesc), C.POINTER(Layer), _P, _P, _P, _P, _P, _P, _P, _I, _P,
                                     C.POINTER(Sampling), _P, _I, _P, C.c_size_t, _P]),
    "vlm_vit_window_index": (_I, [_I, _I, _I, _I, C.POINTER(_I), C.POINTER(_I), C.POINTER(_I), C.POINTER(_I)]),
    "vlm_gather_rows": (_I, [_P, _I, _P, _I, _I, _P, _P]),
    "vlm_vit_merger": (_I, [C.POINTER(Merger), _P, _I, _P, _P, _P, C.c_size_t, _P]),
    "vlm_vit_merger_workspace_bytes": (_I, [C.POINTER(Merger), _I, C.POINTER(C.c_size_t)]),
    "vlm_decode_split_plan": (_I, [_I, _I, C.POINTER(_I), C.POINTER(_I)]),
    "vlm_launch_kernel": (_I, [C.POINTER(ModelDesc), C.POINTER(Layer), _P, _P, _P, _P, _P, _I, _I, _I, _P, _P,
                               C.c_size_t, _P]),
}
VLM_KERNEL_LMHEAD, VLM_KERNEL_QKV, VLM_KERNEL_O, VLM_KERNEL_GATE_UP, VLM_KERNEL_DOWN, VLM_KERNEL_ATTN = range(6)

_lib = None


def lib():
    """The loaded library; raises when libvlm.so is missing (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m decoder_prefill_decode_amd.build` "
                               "(there is no CPU fallback)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().vlm_last_error().decode()


def check(status: int):
    if status != VLM_OK:
        raise VlmError(status, last_error())


def call(name, *args):
    """Calls vlm_<name> and raises VlmError on a non-zero status."""
    check(getattr(lib(), name)(*args))
