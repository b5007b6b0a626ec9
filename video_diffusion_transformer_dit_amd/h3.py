"""Thin ctypes binding of libh3block.so (include/h3block.h).

Argument marshalling only: every step of the block runs in the library's HIP
kernels. Tensors are torch tensors on the GPU (PyTorch supplies device memory
and streams); BF16 tensors are passed by their bit patterns. Each wrapper
raises H3Error on a non-zero status. If the library has not been built the
import of this module fails loudly; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libh3block.so")

H3_OK, H3_ERR_NULL, H3_ERR_SHAPE, H3_ERR_UNSUPPORTED, H3_ERR_ALIGN, H3_ERR_ALIAS, \
    H3_ERR_WORKSPACE, H3_ERR_DEVICE, H3_ERR_HIP = range(9)
H3_EPI_STORE, H3_EPI_RESIDUAL, H3_EPI_SWIGLU = range(3)
H3_WS_H, H3_WS_QKV, H3_WS_O, H3_WS_X1, H3_WS_H2, H3_WS_G, H3_WS_VT, H3_WS_GEMM = range(8)
H3_WS_COUNT = 8
H3_MXWS_HQ, H3_MXWS_HS, H3_MXWS_QKV, H3_MXWS_O, H3_MXWS_OQ, H3_MXWS_OS, H3_MXWS_X1, H3_MXWS_H2Q, H3_MXWS_H2S, \
    H3_MXWS_GQ, H3_MXWS_GS, H3_MXWS_VT, H3_MXWS_BLOCKS, H3_MXWS_COUNTS, H3_MXWS_SELECT = range(15)
H3_MXWS_COUNT = 15
H3_MAX_SEGMENTS = 4
H3_MAX_GROUPS = 8
H3_SPARSE_Q_BLOCK, H3_SPARSE_K_BLOCK, H3_SPARSE_MAX_KBLOCKS = 256, 64, 4096
H3_ATTENTION_SCRATCH_BYTES = 128 << 20
H3_CEIL_BF16, H3_CEIL_FP8 = 0, 1


class H3Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class Dims(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("rot_dim", C.c_int32), ("norm_type", C.c_int32), ("rope_pairing", C.c_int32),
                ("reserved", C.c_int32), ("rope_theta", C.c_float), ("eps", C.c_float)]


class BlockWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("w_qkv", "b_qkv", "q_gain", "k_gain", "w_o", "b_o", "w_up", "b_up",
                                          "w_down", "b_down")]


class BlockWeightsMx(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("w_qkv", "s_qkv", "w_o", "s_o", "w_up", "s_up", "w_down", "s_down",
                                          "b_qkv", "b_o", "b_up", "b_down", "q_gain", "k_gain")]


class KvSeg(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("ld", C.c_int64), ("begin", C.c_int64),
                ("len", C.c_int64), ("vt", C.c_void_p), ("kmax2", C.c_void_p)]


class QGroup(C.Structure):
    _fields_ = [("q_begin", C.c_int64), ("q_end", C.c_int64), ("n_seg", C.c_int32), ("reserved", C.c_int32),
                ("seg", KvSeg * H3_MAX_SEGMENTS)]


class KvExport(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("ld", C.c_int64), ("src_begin", C.c_int64),
                ("len", C.c_int64)]


def _load():
    # torch supplies device memory and streams, and ships its own HIP runtime
    # (libamdhip64, soname libamdhip64.so.7). Importing torch first makes the
    # library bind to that same runtime; loading the library first would bring
    # in a second HIP runtime that does not see torch's device state.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m video_diffusion_transformer_dit_amd.build`")
    lib = C.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
    sig = {
        "h3_block_forward": [C.POINTER(Dims), C.POINTER(BlockWeights), P, P, P, I32, P, P, I64, I64,
                             C.POINTER(QGroup), I32, C.POINTER(KvExport), P, SZ, P],
        "h3_check_block_forward": [C.POINTER(Dims), C.POINTER(BlockWeights), P, P, P, I32, P, P, I64, I64,
                                   C.POINTER(QGroup), I32, C.POINTER(KvExport), P, SZ],
        "h3_attention": [P, I64, P, I64, P, I64, P, I64, I64, I64, I32, I32, F32, C.POINTER(QGroup), I32, P, SZ,
                         P],
        "h3_check_attention": [P, I64, P, I64, P, I64, P, I64, I64, I64, I32, I32, F32, C.POINTER(QGroup), I32,
                               P, SZ],
        "h3_attention_workspace_bytes": [I64, I32, C.POINTER(QGroup), I32],
        "h3_kv_stage": [P, P, I64, I64, I32, I32, P, P, P],
        "h3_check_kv_stage": [P, P, I64, I64, I32, I32, P, P],
        "h3_kv_stage_bytes": [I64, I32],
        "h3_mfma_ceiling": [I32, I32, P, I64, C.POINTER(C.c_double), P],
        "h3_check_mfma_ceiling": [I32, I32, P, I64, C.POINTER(C.c_double)],
        "h3_attention_noalloc": [P, I64, P, I64, P, I64, P, I64, I64, I64, I32, I32, F32, C.POINTER(QGroup), I32,
                                 P],
        "h3_fused_modulate_norm": [P, I64, P, I64, P, P, P, I64, I32, P, P, I64, P, I64, I64, I64, I32, F32, I32, P],
        "h3_check_fused_modulate_norm": [P, I64, P, I64, P, P, P, I64, I32, P, I64, P, I64, I64, I64, I32, F32,
                                         I32],
        "h3_qk_norm_rope": [P, P, I64, P, P, P, I64, I64, I32, I32, I32, I32, F32, F32, P],
        "h3_check_qk_norm_rope": [P, P, I64, P, P, I64, I64, I32, I32, I32, I32, F32, F32],
        "h3_swiglu": [P, I64, P, I64, I64, I64, I32, P],
        "h3_check_swiglu": [P, I64, P, I64, I64, I64, I32],
        "h3_qk_norm_rope_lora": [P, P, P, I64, P, P, P, I64, P, P, P, I64, I64, I32, I32, I32, I32, F32, F32, P],
        "h3_check_qk_norm_rope_lora": [P, P, P, I64, P, P, P, I64, P, P, I64, I64, I32, I32, I32, I32, F32, F32],
        "h3_fused_modulate_norm_lora": [P, I64, P, I64, P, I64, P, P, P, I64, I32, P, P, I64, P, I64, I64, I64, I32,
                                        F32, I32, I32, P],
        "h3_check_fused_modulate_norm_lora": [P, I64, P, I64, P, I64, P, P, P, I64, I32, P, I64, P, I64, I64, I64,
                                              I32, F32, I32, I32],
        "h3_swiglu_lora": [P, I64, P, I64, P, I64, I64, I64, I32, P],
        "h3_check_swiglu_lora": [P, I64, P, I64, P, I64, I64, I64, I32],
        "h3_linear": [P, I64, P, I64, P, P, I64, I64, I64, I64, I64, I32, P, I64, P, I64, I32, P, P, SZ, P],
        "h3_check_linear": [P, I64, P, I64, P, P, I64, I64, I64, I64, I64, I32, P, I64, P, I64, I32, P, SZ],
        "h3_linear_workspace_bytes": [I64, I64, I64, I32],
        "h3_stack_forward": [C.POINTER(Dims), C.POINTER(BlockWeights), I32, P, P, I64, I32, P, P, I64, I64, P, SZ,
                             P],
        "h3_check_stack_forward": [C.POINTER(Dims), C.POINTER(BlockWeights), I32, P, P, I64, I32, P, P, I64, I64, P,
                                   SZ],
        "h3_block_workspace_bytes": [C.POINTER(Dims), I64, C.POINTER(QGroup), I32],
        "h3_block_workspace_layout": [C.POINTER(Dims), I64, C.POINTER(QGroup), I32, C.POINTER(I64),
                                      C.POINTER(I64)],
        "h3_block_forward_sparse": [C.POINTER(Dims), C.POINTER(BlockWeights), P, P, P, I32, P, P, I64, I64, I64,
                                    F32, P, SZ, P],
        "h3_check_block_forward_sparse": [C.POINTER(Dims), C.POINTER(BlockWeights), P, P, P, I32, P, P, I64, I64,
                                          I64, F32, P, SZ],
        "h3_block_sparse_workspace_bytes": [C.POINTER(Dims), I64, I64, I64],
        "h3_block_sparse_workspace_layout": [C.POINTER(Dims), I64, I64, I64, C.POINTER(I64), C.POINTER(I64)],
        "h3_sparse_select": [P, I64, P, I64, I64, I64, I32, I32, F32, P, P, P, SZ, P],
        "h3_check_sparse_select": [P, I64, P, I64, I64, I64, I32, I32, F32, P, P, P, SZ],
        "h3_sparse_select_workspace_bytes": [I64, I64, I32],
        "h3_sparse_attention": [P, I64, P, I64, P, I64, P, I64, I64, I64, I64, I32, I32, F32, P, P, P, SZ, P],
        "h3_check_sparse_attention": [P, I64, P, I64, P, I64, P, I64, I64, I64, I64, I32, I32, F32, P, P, P, SZ],
        "h3_sparse_attention_workspace_bytes": [I64, I64, I32],
        "h3_mxfp8_quantize": [P, I64, I64, I64, I64, P, I64, P, P],
        "h3_check_mxfp8_quantize": [P, I64, I64, I64, I64, P, I64, P],
        "h3_linear_mxfp8": [P, I64, P, I64, P, I64, P, P, P, I64, I64, I64, I64, I64, I32, P, I64, P, I64, I32, P,
                            P],
        "h3_check_linear_mxfp8": [P, I64, P, I64, P, I64, P, P, P, I64, I64, I64, I64, I64, I32, P, I64, P, I64,
                                  I32],
        "h3_fused_modulate_norm_mxfp8": [P, I64, P, I64, P, P, P, I64, I32, P, P, I64, P, I64, P, I64, I64, I32, F32,
                                         I32, P],
        "h3_check_fused_modulate_norm_mxfp8": [P, I64, P, I64, P, P, P, I64, I32, P, I64, P, I64, P, I64, I64, I32,
                                               F32, I32],
        "h3_block_forward_mxfp8": [C.POINTER(Dims), C.POINTER(BlockWeightsMx), P, P, P, I32, P, P, I64, I64, I64,
                                   F32, P, SZ, P],
        "h3_check_block_forward_mxfp8": [C.POINTER(Dims), C.POINTER(BlockWeightsMx), P, P, P, I32, P, P, I64, I64,
                                         I64, F32, P, SZ],
        "h3_block_mxfp8_workspace_bytes": [C.POINTER(Dims), I64, I64, I64],
        "h3_block_mxfp8_workspace_layout": [C.POINTER(Dims), I64, I64, I64, C.POINTER(I64)],
        "h3_status_string": [C.c_int],
        "h3_abi_version": [],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = C.c_int
    lib.h3_block_workspace_bytes.restype = C.c_size_t
    lib.h3_attention_workspace_bytes.restype = C.c_size_t
    lib.h3_linear_workspace_bytes.restype = C.c_size_t
    lib.h3_kv_stage_bytes.restype = C.c_size_t
    lib.h3_sparse_select_workspace_bytes.restype = C.c_size_t
    lib.h3_block_sparse_workspace_bytes.restype = C.c_size_t
    lib.h3_block_mxfp8_workspace_bytes.restype = C.c_size_t
    lib.h3_sparse_attention_workspace_bytes.restype = C.c_size_t
    lib.h3_status_string.restype = C.c_char_p
    return lib


LIB = _load()
EXPORTS = ["h3_block_forward", "h3_attention", "h3_fused_modulate_norm", "h3_qk_norm_rope", "h3_swiglu",
           "h3_linear", "h3_attention_workspace_bytes", "h3_block_workspace_bytes", "h3_block_workspace_layout", "h3_status_string",
           "h3_abi_version", "h3_check_block_forward", "h3_check_attention", "h3_check_fused_modulate_norm",
           "h3_check_qk_norm_rope", "h3_check_swiglu", "h3_check_linear", "h3_qk_norm_rope_lora",
           "h3_fused_modulate_norm_lora", "h3_swiglu_lora", "h3_check_qk_norm_rope_lora",
           "h3_check_fused_modulate_norm_lora", "h3_check_swiglu_lora", "h3_sparse_select", "h3_sparse_attention",
           "h3_sparse_select_workspace_bytes", "h3_sparse_attention_workspace_bytes", "h3_check_sparse_select",
           "h3_check_sparse_attention", "h3_block_forward_sparse", "h3_block_sparse_workspace_bytes",
           "h3_check_block_forward_sparse",
           "h3_block_sparse_workspace_layout", "h3_mxfp8_quantize", "h3_linear_mxfp8", "h3_check_mxfp8_quantize",
           "h3_check_linear_mxfp8", "h3_fused_modulate_norm_mxfp8", "h3_check_fused_modulate_norm_mxfp8",
           "h3_block_forward_mxfp8", "h3_check_block_forward_mxfp8", "h3_block_mxfp8_workspace_bytes",
           "h3_block_mxfp8_workspace_layout", "h3_stack_forward", "h3_check_stack_forward",
           "h3_attention_noalloc", "h3_linear_workspace_bytes", "h3_kv_stage", "h3_check_kv_stage",
           "h3_kv_stage_bytes", "h3_mfma_ceiling", "h3_check_mfma_ceiling"]


def status_string(s: int) -> str:
    return LIB.h3_status_string(int(s)).decode()


def _ok(s: int, where: str) -> None:
    if s != H3_OK:
        raise H3Error(s, where)


def _ptr(t):
    """Device (or host) address of a tensor, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _ld(t, default=None):
    if t is None:
        return 0 if default is None else default
    return t.stride(0) if t.dim() > 1 else t.shape[0]


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def make_dims(hidden, heads, ffn, head_dim=128, rot_dim=64, norm_type=0, rope_pairing=0, rope_theta=10000.0,
              eps=1e-6) -> Dims:
    return Dims(hidden, heads, head_dim, ffn, rot_dim, norm_type, rope_pairing, 0, rope_theta, eps)


def make_weights(w: dict) -> BlockWeights:
    return BlockWeights(*[_ptr(w.get(n)) for n in ("w_qkv", "b_qkv", "q_gain", "k_gain", "w_o", "b_o", "w_up",
                                                   "b_up", "w_down", "b_down")])


def make_groups(groups):
    """groups: list of (q_begin, q_end, segs) with segs a list of
    ('self', begin, len), (k_tensor, v_tensor, begin, len), or
    (k_tensor, v_tensor, begin, len, (vt, kmax2)) for a segment whose rows
    [begin, begin+len) were staged by kv_stage."""
    if groups is None:
        return None, 0
    arr = (QGroup * len(groups))()
    for i, (qb, qe, segs) in enumerate(groups):
        arr[i].q_begin, arr[i].q_end, arr[i].n_seg = qb, qe, len(segs)
        for j, s in enumerate(segs):
            if isinstance(s[0], str):
                arr[i].seg[j] = KvSeg(None, None, 0, s[1], s[2], None, None)
            else:
                k, v, b, ln = s[:4]
                vt, km = s[4] if len(s) > 4 else (None, None)
                arr[i].seg[j] = KvSeg(_ptr(k), _ptr(v), k.stride(0), b, ln, _ptr(vt), _ptr(km))
    return arr, len(groups)


def workspace_bytes(dims: Dims, L_buf: int, groups=None) -> int:
    garr, ng = make_groups(groups)
    return int(LIB.h3_block_workspace_bytes(C.byref(dims), L_buf, garr, ng))


def workspace_layout(dims: Dims, L_buf: int, groups=None):
    garr, ng = make_groups(groups)
    off = (C.c_int64 * H3_WS_COUNT)()
    lds = (C.c_int64 * H3_WS_COUNT)()
    _ok(LIB.h3_block_workspace_layout(C.byref(dims), L_buf, garr, ng, off, lds), "h3_block_workspace_layout")
    return list(off), list(lds)


def attention_workspace_bytes(valid_len: int, heads: int, groups=None) -> int:
    garr, ng = make_groups(groups)
    return int(LIB.h3_attention_workspace_bytes(valid_len, heads, garr, ng))


def block_forward(dims: Dims, weights: BlockWeights, x, y, mod, n_mod_groups, valid_len, workspace,
                  mod_idx=None, pos=None, groups=None, kv_export=None, stream=None):
    garr, ng = make_groups(groups)
    exp = None
    if kv_export is not None:
        k, v, src_begin, ln = kv_export
        exp = KvExport(_ptr(k), _ptr(v), k.stride(0), src_begin, ln)
    s = LIB.h3_block_forward(C.byref(dims), C.byref(weights), _ptr(x), _ptr(y), _ptr(mod), n_mod_groups,
                             _ptr(mod_idx), _ptr(pos), x.shape[0], valid_len, garr, ng,
                             C.byref(exp) if exp is not None else None, _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    _ok(s, "h3_block_forward")


def make_weight_stack(weight_sets) -> "C.Array":
    """ctypes array of BlockWeights, one per block, for stack_forward."""
    arr = (BlockWeights * len(weight_sets))()
    for i, w in enumerate(weight_sets):
        arr[i] = w
    return arr


def stack_forward(dims: Dims, weight_stack, x, mod, ld_mod_block, n_mod_groups, valid_len, workspace,
                  mod_idx=None, pos=None, stream=None):
    """h3_stack_forward: len(weight_stack) blocks in place on x; block b reads
    its modulation table at mod + b * ld_mod_block floats."""
    n = len(weight_stack)
    s = LIB.h3_stack_forward(C.byref(dims), weight_stack if n else None, n, _ptr(x), _ptr(mod), ld_mod_block,
                             n_mod_groups, _ptr(mod_idx), _ptr(pos), x.shape[0], valid_len, _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    _ok(s, "h3_stack_forward")


def block_sparse_workspace_bytes(dims: Dims, L_buf: int, valid_len: int, prefix_len: int) -> int:
    return int(LIB.h3_block_sparse_workspace_bytes(C.byref(dims), L_buf, valid_len, prefix_len))


def block_sparse_workspace_layout(dims: Dims, L_buf: int, valid_len: int, prefix_len: int):
    """(blocks_off, counts_off): where the block's selection lies in its workspace."""
    b, c = C.c_int64(), C.c_int64()
    _ok(LIB.h3_block_sparse_workspace_layout(C.byref(dims), L_buf, valid_len, prefix_len, C.byref(b), C.byref(c)),
        "h3_block_sparse_workspace_layout")
    return b.value, c.value


def block_forward_sparse(dims: Dims, weights: BlockWeights, x, y, mod, n_mod_groups, valid_len, prefix_len, tau,
                         workspace, mod_idx=None, pos=None, stream=None):
    s = LIB.h3_block_forward_sparse(C.byref(dims), C.byref(weights), _ptr(x), _ptr(y), _ptr(mod), n_mod_groups,
                                    _ptr(mod_idx), _ptr(pos), x.shape[0], valid_len, prefix_len, float(tau),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _ok(s, "h3_block_forward_sparse")


def attention(q, k, v, o, valid_len, heads, softmax_scale=0.0, groups=None, workspace=None, stream=None):
    """workspace: uint8 device tensor of at least attention_workspace_bytes(...)
    bytes, or None to allocate one here (torch's caching allocator)."""
    garr, ng = make_groups(groups)
    if workspace is None:
        import torch
        workspace = torch.empty(max(attention_workspace_bytes(valid_len, heads, groups), 1), dtype=torch.uint8,
                                device=q.device)
    s = LIB.h3_attention(_ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0), _ptr(o), o.stride(0),
                         q.shape[0], valid_len, heads, 128, softmax_scale, garr, ng, _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _stream(stream))
    _ok(s, "h3_attention")


def kv_stage_bytes(length: int, heads: int) -> int:
    return int(LIB.h3_kv_stage_bytes(length, heads))


def kv_stage(k, v, heads, vt=None, kmax2=None, stream=None):
    """Stage rows [0, k.shape[0]) of an external K/V segment once: returns
    (vt, kmax2) device tensors (allocated here unless given) to pass as a
    segment's staged form."""
    import torch
    n = k.shape[0]
    if vt is None:
        vt = torch.empty(max(kv_stage_bytes(n, heads), 16) // 2, dtype=torch.bfloat16, device=k.device)
    if kmax2 is None:
        kmax2 = torch.empty(heads, dtype=torch.float32, device=k.device)
    s = LIB.h3_kv_stage(_ptr(k), _ptr(v), k.stride(0), n, heads, 128, _ptr(vt), _ptr(kmax2), _stream(stream))
    _ok(s, "h3_kv_stage")
    return vt, kmax2


def mfma_ceiling(iters, sink, dtype=0, stream=None) -> float:
    """Launch the matrix-core ceiling probe (h3_mfma_ceiling; dtype
    H3_CEIL_BF16 or H3_CEIL_FP8) on `sink` (FP32 device tensor of at least
    256 floats per CU); returns the launch's flops."""
    fl = C.c_double(0.0)
    s = LIB.h3_mfma_ceiling(int(dtype), int(iters), _ptr(sink), sink.numel(), C.byref(fl), _stream(stream))
    _ok(s, "h3_mfma_ceiling")
    return fl.value


def attention_noalloc(q, k, v, o, valid_len, heads, softmax_scale=0.0, groups=None, stream=None):
    """h3_attention with the library's own fixed device workspace (no
    allocation anywhere, on either side of the boundary)."""
    garr, ng = make_groups(groups)
    s = LIB.h3_attention_noalloc(_ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0), _ptr(o),
                                 o.stride(0), q.shape[0], valid_len, heads, 128, softmax_scale, garr, ng,
                                 _stream(stream))
    _ok(s, "h3_attention_noalloc")


def fused_modulate_norm(x, shift, scale, h_out, valid_len, eps=1e-6, norm_type=0, branch=None, gate=None,
                        x1_out=None, ld_mod_group=0, n_mod_groups=1, mod_idx=None, stream=None):
    hidden = x.shape[1]
    s = LIB.h3_fused_modulate_norm(_ptr(x), x.stride(0), _ptr(branch), _ld(branch), _ptr(shift), _ptr(scale),
                                   _ptr(gate), ld_mod_group, n_mod_groups, _ptr(mod_idx), _ptr(x1_out),
                                   _ld(x1_out), _ptr(h_out), h_out.stride(0), x.shape[0], valid_len, hidden, eps,
                                   norm_type, _stream(stream))
    _ok(s, "h3_fused_modulate_norm")


def qk_norm_rope(q, k, q_gain, k_gain, valid_len, heads, rot_dim=64, pairing=0, theta=10000.0, eps=1e-6,
                 pos=None, stream=None):
    s = LIB.h3_qk_norm_rope(_ptr(q), _ptr(k), q.stride(0), _ptr(q_gain), _ptr(k_gain), _ptr(pos), q.shape[0],
                            valid_len, heads, 128, rot_dim, pairing, theta, eps, _stream(stream))
    _ok(s, "h3_qk_norm_rope")


def swiglu(u, g, valid_len, ffn, stream=None):
    s = LIB.h3_swiglu(_ptr(u), u.stride(0), _ptr(g), g.stride(0), u.shape[0], valid_len, ffn, _stream(stream))
    _ok(s, "h3_swiglu")


def qk_norm_rope_lora(q, k, dq, dk, q_gain, k_gain, valid_len, heads, v=None, dv=None, rot_dim=64, pairing=0,
                      theta=10000.0, eps=1e-6, pos=None, stream=None):
    s = LIB.h3_qk_norm_rope_lora(_ptr(q), _ptr(k), _ptr(v), q.stride(0), _ptr(dq), _ptr(dk), _ptr(dv), dq.stride(0),
                                 _ptr(q_gain), _ptr(k_gain), _ptr(pos), q.shape[0], valid_len, heads, 128, rot_dim,
                                 pairing, theta, eps, _stream(stream))
    _ok(s, "h3_qk_norm_rope_lora")


def fused_modulate_norm_lora(x, branch, delta, gate, x1_out, valid_len, shift=None, scale=None, h_out=None,
                             eps=1e-6, norm_type=0, gate_bf16=False, ld_mod_group=0, n_mod_groups=1, mod_idx=None,
                             stream=None):
    hidden = x.shape[1]
    s = LIB.h3_fused_modulate_norm_lora(_ptr(x), x.stride(0), _ptr(branch), branch.stride(0), _ptr(delta),
                                        delta.stride(0), _ptr(shift), _ptr(scale), _ptr(gate), ld_mod_group,
                                        n_mod_groups, _ptr(mod_idx), _ptr(x1_out), x1_out.stride(0), _ptr(h_out),
                                        _ld(h_out), x.shape[0], valid_len, hidden, eps, norm_type,
                                        1 if gate_bf16 else 0, _stream(stream))
    _ok(s, "h3_fused_modulate_norm_lora")


def swiglu_lora(u, du, g, valid_len, ffn, stream=None):
    s = LIB.h3_swiglu_lora(_ptr(u), u.stride(0), _ptr(du), du.stride(0), _ptr(g), g.stride(0), u.shape[0],
                           valid_len, ffn, _stream(stream))
    _ok(s, "h3_swiglu_lora")


def linear_workspace_bytes(M_valid: int, N: int, K: int, epilogue: int = H3_EPI_STORE) -> int:
    return int(LIB.h3_linear_workspace_bytes(M_valid, N, K, epilogue))


def linear(a, w, c, M_valid, epilogue=H3_EPI_STORE, bias=None, resid=None, gate=None, ld_gate_group=0,
           n_mod_groups=1, mod_idx=None, workspace=None, stream=None):
    """workspace: None (one workgroup per output tile) or a uint8 device tensor
    of at least linear_workspace_bytes(...) bytes for the stream-K tail."""
    N, K = w.shape
    s = LIB.h3_linear(_ptr(a), a.stride(0), _ptr(w), w.stride(0), _ptr(bias), _ptr(c), c.stride(0), a.shape[0],
                      M_valid, N, K, epilogue, _ptr(resid), _ld(resid), _ptr(gate), ld_gate_group, n_mod_groups,
                      _ptr(mod_idx), _ptr(workspace),
                      0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream))
    _ok(s, "h3_linear")


def sparse_geometry(valid_len: int, prefix_len: int):
    """(n_qb, n_kb): target query blocks and KV blocks of a block-sparse call."""
    T = max(valid_len - prefix_len, 0)
    return -(-T // H3_SPARSE_Q_BLOCK), -(-T // H3_SPARSE_K_BLOCK)


def sparse_select_workspace_bytes(valid_len: int, prefix_len: int, heads: int) -> int:
    return int(LIB.h3_sparse_select_workspace_bytes(valid_len, prefix_len, heads))


def sparse_attention_workspace_bytes(valid_len: int, prefix_len: int, heads: int) -> int:
    return int(LIB.h3_sparse_attention_workspace_bytes(valid_len, prefix_len, heads))


def sparse_select(q, k, valid_len, prefix_len, heads, tau, blocks, counts, workspace=None, stream=None):
    """blocks: uint16 (or int16) device tensor [heads, n_qb, n_kb]; counts: int32
    [heads, n_qb]. workspace: uint8 device tensor or None (allocated here)."""
    if workspace is None:
        import torch
        workspace = torch.empty(max(sparse_select_workspace_bytes(valid_len, prefix_len, heads), 1),
                                dtype=torch.uint8, device=q.device)
    s = LIB.h3_sparse_select(_ptr(q), q.stride(0), _ptr(k), k.stride(0), valid_len, prefix_len, heads, 128,
                             float(tau), _ptr(blocks), _ptr(counts), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    _ok(s, "h3_sparse_select")


def sparse_attention(q, k, v, o, valid_len, prefix_len, heads, blocks, counts, softmax_scale=0.0, workspace=None,
                     stream=None):
    if workspace is None:
        import torch
        workspace = torch.empty(max(sparse_attention_workspace_bytes(valid_len, prefix_len, heads), 1),
                                dtype=torch.uint8, device=q.device)
    s = LIB.h3_sparse_attention(_ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0), _ptr(o),
                                o.stride(0), q.shape[0], valid_len, prefix_len, heads, 128, softmax_scale,
                                _ptr(blocks), _ptr(counts), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _ok(s, "h3_sparse_attention")


def mx_scales_shape(rows: int, K: int):
    """Shape of an MXFP8 scale array: [K / 128, rows, 4] uint8."""
    return (K // 128, rows, 4)


def mxfp8_quantize(x, valid_len, q, scales, stream=None):
    """x [rows_buf, K] BF16 -> q [rows_buf, K] uint8 codes, scales [K/128, rows_buf, 4] uint8."""
    s = LIB.h3_mxfp8_quantize(_ptr(x), x.stride(0), x.shape[0], valid_len, x.shape[1], _ptr(q), q.stride(0),
                              _ptr(scales), _stream(stream))
    _ok(s, "h3_mxfp8_quantize")


def linear_mxfp8(a, a_scales, w, w_scales, c, M_valid, epilogue=H3_EPI_STORE, bias=None, resid=None, gate=None,
                 ld_gate_group=0, n_mod_groups=1, mod_idx=None, stream=None):
    """a [M_buf, K] / w [N, K] uint8 codes with scales [K/128, rows, 4]."""
    N, K = w.shape
    s = LIB.h3_linear_mxfp8(_ptr(a), a.stride(0), _ptr(a_scales), a_scales.shape[1], _ptr(w), w.stride(0),
                            _ptr(w_scales), _ptr(bias), _ptr(c), c.stride(0), a.shape[0], M_valid, N, K, epilogue,
                            _ptr(resid), _ld(resid), _ptr(gate), ld_gate_group, n_mod_groups, _ptr(mod_idx),
                            _stream(stream))
    _ok(s, "h3_linear_mxfp8")


def fused_modulate_norm_mxfp8(x, shift, scale, hq, hs, valid_len, eps=1e-6, norm_type=0, branch=None, gate=None,
                              x1_out=None, ld_mod_group=0, n_mod_groups=1, mod_idx=None, stream=None):
    """h written as MXFP8: hq [L_buf, hidden] uint8, hs [hidden/128, L_buf, 4] uint8."""
    s = LIB.h3_fused_modulate_norm_mxfp8(_ptr(x), x.stride(0), _ptr(branch), _ld(branch), _ptr(shift), _ptr(scale),
                                         _ptr(gate), ld_mod_group, n_mod_groups, _ptr(mod_idx), _ptr(x1_out),
                                         _ld(x1_out), _ptr(hq), hq.stride(0), _ptr(hs), x.shape[0], valid_len,
                                         x.shape[1], eps, norm_type, _stream(stream))
    _ok(s, "h3_fused_modulate_norm_mxfp8")


def make_weights_mx(wq: dict) -> BlockWeightsMx:
    """wq: w_qkv / w_o / w_up / w_down -> (codes, scales) pairs; b_* and q_gain / k_gain BF16 tensors."""
    f = {}
    for n, sname in (("w_qkv", "s_qkv"), ("w_o", "s_o"), ("w_up", "s_up"), ("w_down", "s_down")):
        f[n], f[sname] = _ptr(wq[n][0]), _ptr(wq[n][1])
    for n in ("b_qkv", "b_o", "b_up", "b_down", "q_gain", "k_gain"):
        f[n] = _ptr(wq.get(n))
    return BlockWeightsMx(**f)


def block_mxfp8_workspace_bytes(dims: Dims, L_buf: int, valid_len=None, prefix_len: int = -1) -> int:
    valid_len = L_buf if valid_len is None else valid_len
    return int(LIB.h3_block_mxfp8_workspace_bytes(C.byref(dims), L_buf, valid_len, prefix_len))


def block_mxfp8_workspace_layout(dims: Dims, L_buf: int, valid_len=None, prefix_len: int = -1):
    valid_len = L_buf if valid_len is None else valid_len
    off = (C.c_int64 * H3_MXWS_COUNT)()
    _ok(LIB.h3_block_mxfp8_workspace_layout(C.byref(dims), L_buf, valid_len, prefix_len, off),
        "h3_block_mxfp8_workspace_layout")
    return list(off)


def block_forward_mxfp8(dims: Dims, weights: BlockWeightsMx, x, y, mod, n_mod_groups, valid_len, workspace,
                        mod_idx=None, pos=None, prefix_len: int = -1, tau: float = 0.0, stream=None):
    """prefix_len < 0: dense attention; else Sol-Attn block-sparse attention with threshold tau."""
    s = LIB.h3_block_forward_mxfp8(C.byref(dims), C.byref(weights), _ptr(x), _ptr(y), _ptr(mod), n_mod_groups,
                                   _ptr(mod_idx), _ptr(pos), x.shape[0], valid_len, prefix_len, float(tau),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _ok(s, "h3_block_forward_mxfp8")
