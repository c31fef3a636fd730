"""ctypes binding of libfp8w8a8.so (argument marshalling only).

Every name here mirrors an ``extern "C"`` entry point of include/fp8w8a8.h.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8w8a8.so")

c_i32 = ctypes.c_int32
c_i64 = ctypes.c_int64
c_size = ctypes.c_size_t
c_vp = ctypes.c_void_p
c_f32 = ctypes.c_float

FP8_OK = 0
FP8_ERR_INVALID = -1
FP8_ERR_UNSUPPORTED = -2
FP8_ERR_WORKSPACE = -3
FP8_ERR_HIP = -4
# bytes of the library's static split-K scratch per device (fp8_scaled_mm_noalloc)
NOALLOC_SCRATCH_BYTES = (256 << 10) + (64 << 20)

KIND_CHANNELWISE = 0
KIND_BLOCKWISE = 1
KIND_BLOCKWISE_UE8M0 = 2

QUANT_FUSE_SILU_MUL = 1
QUANT_SCALE_UE8M0 = 2

VARIANTS = {"default": -1, "skinny": 0, "t64x64": 1, "t128x128": 2, "t256x128": 3, "t256x256": 4,
            "t256x256w8": 5, "t256x128w8": 6, "t128x128w8": 7, "t128x64k256": 8,
            "t64x128k256": 9, "t128x128k256": 10, "t256x256dma": 11, "t256x128dma": 12,
            "t128x128dma": 13, "t256x256panel": 14, "t256x128panel": 15,
            "t128x128panel": 16, "t128x64panel": 17, "t64x64panel": 18,
            "t64x64deep": 19, "t128x64deep": 20,
            "t128x128panel8": 21, "t128x64panel8": 22,
            "t32x32deep": 23, "t64x32deep": 24, "t256x256bw16": 25,
            "decode": 26}
VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}


class TileConfig(ctypes.Structure):
    _fields_ = [("variant", c_i32), ("bm", c_i32), ("bn", c_i32), ("bk", c_i32),
                ("split_k", c_i32), ("waves", c_i32)]

    def as_dict(self):
        return {"variant": VARIANT_NAMES.get(self.variant, self.variant), "bm": self.bm,
                "bn": self.bn, "bk": self.bk, "split_k": self.split_k, "waves": self.waves}


# name -> (restype, argtypes)
SIGNATURES = {
    "fp8_padded_rows": (c_i64, [c_i64, c_i32]),
    "fp8_quant_per_token": (c_i32, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_f32, c_vp]),
    "fp8_quant_per_token_group": (c_i32, [c_vp, c_i64, c_i64, c_i64, c_i32, c_i32, c_vp, c_i64,
                                          c_vp, c_f32, c_vp]),
    "fp8_quant_per_token_ex": (c_i32, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_f32, c_i32,
                                       c_vp]),
    "fp8_quant_per_token_group_ex": (c_i32, [c_vp, c_i64, c_i64, c_i64, c_i32, c_i32, c_vp, c_i64,
                                             c_vp, c_f32, c_i32, c_vp]),
    "fp8_quant_per_token_group_masked": (c_i32, [c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_i32, c_i32,
                                                 c_vp, c_i64, c_vp, c_f32, c_i32, c_vp]),
    "fp8_scaled_mm_blockwise_masked": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i64,
                                               c_i64, c_i64, c_i64, c_i64, c_i64, c_i32,
                                               ctypes.POINTER(TileConfig), c_vp]),
    "fp8_quant_static": (c_i32, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_i64, c_vp]),
    "fp8_scaled_mm_channelwise": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64,
                                          c_i64, c_i64, c_i64, c_vp, c_size, c_vp]),
    "fp8_scaled_mm_channelwise_ex": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64,
                                             c_i64, c_i64, c_i64, c_i64, c_vp, c_size,
                                             ctypes.POINTER(TileConfig), c_vp]),
    "fp8_scaled_mm_noalloc": (c_i32, [c_i32, c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i64,
                                      c_i64, c_i64, c_i64, c_i64, ctypes.POINTER(TileConfig), c_vp]),
    "fp8_scaled_mm_blockwise": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i64,
                                        c_i64, c_i64, c_i64, c_i64, c_vp, c_size, c_vp]),
    "fp8_scaled_mm_blockwise_ex": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_i64,
                                           c_i64, c_i64, c_i64, c_i64, c_i64, c_vp, c_size,
                                           ctypes.POINTER(TileConfig), c_vp]),
    "fp8_scaled_mm_blockwise_ue8m0": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_i64,
                                              c_i64, c_i64, c_i64, c_i64, c_i64, c_vp, c_size, c_vp]),
    "fp8_scaled_mm_blockwise_ue8m0_ex": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_i64,
                                                 c_i64, c_i64, c_i64, c_i64, c_i64, c_vp, c_size,
                                                 ctypes.POINTER(TileConfig), c_vp]),
    "fp8_scaled_mm_workspace_size": (c_size, [c_i32, c_i64, c_i64, c_i64,
                                              ctypes.POINTER(TileConfig)]),
    "fp8_linear_channelwise": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64,
                                       c_i64, c_i64, c_f32, c_vp, c_i64, c_vp, c_vp, c_size,
                                       ctypes.POINTER(TileConfig), c_vp]),
    "fp8_linear_blockwise": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64,
                                     c_i64, c_i64, c_i32, c_f32, c_vp, c_i64, c_vp, c_vp, c_size,
                                     ctypes.POINTER(TileConfig), c_vp]),
    "fp8_linear_channelwise_ex": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64,
                                          c_i64, c_i64, c_f32, c_vp, c_i64, c_vp, c_vp, c_size,
                                          ctypes.POINTER(TileConfig), c_i32, c_vp]),
    "fp8_linear_blockwise_ex": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64,
                                        c_i64, c_i64, c_i32, c_f32, c_vp, c_i64, c_vp, c_vp, c_size,
                                        ctypes.POINTER(TileConfig), c_i32, c_vp]),
    "fp8_linear_launches": (c_i32, [c_i32, c_i64, c_i64, c_i64, ctypes.POINTER(TileConfig)]),
    "fp8_linear_launches_ex": (c_i32, [c_i32, c_i64, c_i64, c_i64, ctypes.POINTER(TileConfig), c_i32]),
    "fp8_tile_config_lookup": (c_i32, [c_i32, c_i64, c_i64, c_i64, ctypes.POINTER(TileConfig)]),
    "fp8_tile_config_default": (c_i32, [c_i32, c_i64, c_i64, c_i64, ctypes.POINTER(TileConfig)]),
    "fp8_tile_config_set_dir": (c_i32, [ctypes.c_char_p]),
    "fp8_probe_stream_read": (c_i32, [c_vp, c_size, c_vp, c_i32, c_vp]),
    "fp8_probe_strided_read": (c_i32, [c_vp, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp]),
    "fp8_probe_l2_feed": (c_i32, [c_vp, c_size, c_i32, c_i32, c_vp, c_i32, c_vp]),
    "fp8_probe_panel_feed": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp]),
    "fp8_probe_mfma": (c_i32, [c_i32, c_vp, c_i32, c_vp]),
    "fp8_probe_wave_read": (c_i32, [c_vp, c_size, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp]),
    "fp8_probe_lds": (c_i32, [c_i32, c_i32, c_vp, c_i32, c_vp]),
    "fp8_probe_mfma_dot": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp]),
    "fp8_last_error": (ctypes.c_char_p, []),
    "fp8_version": (c_i32, []),
}

_lib = None


def load():
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m fp8_w8a8_quantized_token_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class Fp8Error(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"[{code}] {message}")
        self.code = code


def check(status):
    if status != FP8_OK:
        raise Fp8Error(status, load().fp8_last_error().decode())
    return status
