"""Python binding of libtq: the randomized-Hadamard + Lloyd-Max codecs on MI355X.

Argument marshalling only. Every step of every codec runs in the HIP kernels of
libtq.so (built in-tree by ``build.py``); torch supplies device memory and the
current stream. There is no CPU fallback: importing this package without the
built library, or calling it with CPU tensors, raises.

Entry points (same names as the C ABI in include/tq.h):
  tq3_quantize(x)                  -> uint8 [..., D/128, 56] records
  tq3_dequantize(records, dtype)   -> [..., D/128 * 128] tensor
  tq3_quantize_split(x)            -> (packed [..., D/128, 48], norms, scales)
  tq3_dequantize_split(packed, norms, scales, dtype)
                                   -> the same codec on the three-array layout;
                                      tq3_quantize_dict / tq3_dequantize_dict wrap
                                      it in the TQ3 page's dict form
  orbit_quantize_weight(W, bits)   -> (packed uint8, row_norms fp32)
  orbit_dequantize(packed, norms, d, bits, rotated_only, dtype)
  tq3_decode_attention(q, k_records, v_records, n_kv_heads, signs, scale)
                                   -> [Hq, 128] attention output
  orbit_rotate(x, perm, signs)     -> rpbh_forward of activation rows (fp32/bf16/fp16)
  orbit_linear(x_rot, packed, norms, bits, codebook, bias)
                                   -> x_rot @ W'^T + bias (W' decoded on the fly)
  orbit_rotate_tiled, orbit_linear_tiled
                                   -> the same two steps through the matrix-core
                                      operand layout (bf16 / fp16)
  orbit_forward(x, packed, norms, perm, signs, bits, codebook, bias)
                                   -> the two above: the quantized layer's output
plus host helpers tq3_record_bytes, orbit_block_size, tq_gaussian_lloyd_max,
orbit_make_codebook.
"""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
TQ_MSB_FIRST, TQ_LSB_FIRST = 0, 1
TQ3_DIM, TQ3_RECORD_BYTES = 128, 56

_DTYPES = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16, torch.float16: TQ_F16}
_STATUS = {
    1: ValueError, 2: ValueError, 3: TypeError, 4: ValueError, 5: ValueError,
    6: ValueError, 7: RuntimeError, 8: ValueError, 9: ValueError,
}

_vp, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libtq.so not built at {LIB_PATH}; run `python -m randomized_hadamard_lloyd_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "tq3_quantize": [_vp, _int, _i64, _i64, _vp, _vp, _vp],
        "tq3_dequantize": [_vp, _i64, _vp, _vp, _int, _i64, _vp],
        "tq3_quantize_split": [_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp, _vp],
        "tq3_dequantize_split": [_vp, _vp, _vp, _i64, _vp, _vp, _int, _i64, _vp],
        "orbit_quantize_weight": [_vp, _i64, _i64, _int, _vp, _vp, _vp, _int, _vp, _vp, _vp],
        "orbit_dequantize": [_vp, _vp, _i64, _i64, _int, _vp, _vp, _vp, _int, _int, _vp,
                             _int, _vp],
        "tq_gaussian_lloyd_max": [_int, _int, _vp],
        "orbit_make_codebook": [_int, _i64, _vp],
        "orbit_rotate": [_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp],
        "orbit_linear": [_vp, _int, _i64, _i64, _vp, _vp, _i64, _int, _vp, _int, _vp, _vp, _vp],
        "orbit_rotate_tiled": [_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp],
        "orbit_linear_tiled": [_vp, _int, _i64, _i64, _vp, _vp, _i64, _int, _vp, _int, _vp, _vp,
                               _vp],
        "tq3_decode_attention": [_vp, _int, _int, _vp, _vp, _i64, _int, _vp, ctypes.c_float,
                                 _vp, ctypes.c_size_t, _vp, _int, _vp],
        "tq3_decode_attention_noalloc": [_vp, _int, _int, _vp, _vp, _i64, _int, _vp,
                                         ctypes.c_float, _vp, _int, _vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _int
    lib.tq3_record_bytes.argtypes = []
    lib.tq3_record_bytes.restype = ctypes.c_size_t
    lib.orbit_block_size.argtypes = [_i64]
    lib.orbit_block_size.restype = _i64
    lib.tq_status_str.argtypes = [_int]
    lib.tq_status_str.restype = ctypes.c_char_p
    lib.tq3_attention_workspace_bytes.argtypes = [_i64, _int, _int]
    lib.tq3_attention_workspace_bytes.restype = ctypes.c_size_t
    lib.tq3_attention_noalloc_max_bytes.argtypes = []
    lib.tq3_attention_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.orbit_tiled_bytes.argtypes = [_i64, _i64]
    lib.orbit_tiled_bytes.restype = ctypes.c_size_t
    return lib


lib = _load()

# the symbols include/tq.h declares
EXPORTS = ("tq3_quantize", "tq3_dequantize", "tq3_quantize_split", "tq3_dequantize_split",
           "orbit_quantize_weight", "orbit_dequantize", "tq3_record_bytes", "orbit_block_size", "tq_gaussian_lloyd_max",
           "orbit_make_codebook", "tq_status_str", "tq3_decode_attention",
           "tq3_attention_workspace_bytes", "orbit_rotate", "orbit_linear",
           "orbit_tiled_bytes", "orbit_rotate_tiled", "orbit_linear_tiled",
           "tq3_decode_attention_noalloc", "tq3_attention_noalloc_max_bytes")


def _check(status: int, what: str):
    if status != 0:
        exc = _STATUS.get(status, RuntimeError)
        raise exc(f"{what}: {lib.tq_status_str(status).decode()} (status {status})")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need_gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("libtq operates on GPU tensors only (no CPU fallback)")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _check_out(out, dtype, numel, device, what):
    """A caller-given output buffer must be exactly what the kernels write: the
    C entry points cannot see a buffer's size or type."""
    if (not isinstance(out, torch.Tensor) or out.dtype != dtype or not out.is_contiguous()
            or out.numel() != numel or out.device != device):
        raise ValueError(f"{what}: out must be a contiguous {dtype} tensor of {numel} "
                         f"elements on {device}")


# ------------------------------------------------------------------- TQ3 ---

def sign_mask(signs) -> bytes:
    """16-byte mask of a 128-entry +-1 sign vector: bit j set where s_j < 0."""
    s = np.asarray(signs.detach().cpu() if isinstance(signs, torch.Tensor) else signs,
                   dtype=np.float32).reshape(-1)
    if s.size != TQ3_DIM:
        raise ValueError("TQ3 sign vector must have 128 entries")
    return np.packbits(s < 0, bitorder="little").tobytes()


def tq3_record_bytes() -> int:
    return int(lib.tq3_record_bytes())


def tq3_quantize(x: torch.Tensor, signs, out: torch.Tensor = None) -> torch.Tensor:
    """x [..., D] (D a positive multiple of 128; fp32, bf16 or fp16, on the GPU)
    -> uint8 records [..., D/128, 56] (48 bytes of 3-bit indices, fp32 norm,
    fp32 scale). `signs` is the 128-entry +-1 vector or its 16-byte mask."""
    if not isinstance(x, torch.Tensor):
        raise TypeError("tq3_quantize expects a torch.Tensor input")
    if x.ndim == 0:
        raise ValueError("tq3_quantize expects at least one dimension")
    if x.shape[-1] <= 0 or x.shape[-1] % TQ3_DIM:
        raise ValueError(f"last dim must be a positive multiple of 128, got {x.shape[-1]}")
    if x.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {x.dtype}")
    nb = x.shape[-1] // TQ3_DIM
    n = x.numel() // TQ3_DIM
    if out is not None:
        _check_out(out, torch.uint8, n * TQ3_RECORD_BYTES, x.device, "tq3_quantize")
    _need_gpu(x)
    xv = x.reshape(-1, TQ3_DIM) if x.is_contiguous() else x.contiguous().reshape(-1, TQ3_DIM)
    if out is None:
        out = torch.empty((*x.shape[:-1], nb, TQ3_RECORD_BYTES), dtype=torch.uint8,
                          device=x.device)
    m = signs if isinstance(signs, (bytes, bytearray)) else sign_mask(signs)
    _check(lib.tq3_quantize(_ptr(xv), _DTYPES[x.dtype], n, xv.stride(0), m, _ptr(out),
                            _stream(x)), "tq3_quantize")
    return out


def tq3_dequantize(records: torch.Tensor, signs, dtype=torch.float32,
                   out: torch.Tensor = None) -> torch.Tensor:
    """uint8 records [..., nb, 56] -> [..., nb*128] of `dtype` (fp32 values,
    narrowed by round-to-nearest-even for bf16/fp16)."""
    if records.dtype != torch.uint8 or records.shape[-1] != TQ3_RECORD_BYTES:
        raise ValueError("records must be uint8 [..., 56]")
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    n = records.numel() // TQ3_RECORD_BYTES
    if out is not None:
        _check_out(out, dtype, n * TQ3_DIM, records.device, "tq3_dequantize")
    _need_gpu(records)
    rec = records.contiguous()
    lead = tuple(records.shape[:-2])
    nb = records.shape[-2] if records.ndim >= 2 else 1
    if out is None:
        out = torch.empty((*lead, nb * TQ3_DIM), dtype=dtype, device=records.device)
    m = signs if isinstance(signs, (bytes, bytearray)) else sign_mask(signs)
    _check(lib.tq3_dequantize(_ptr(rec), n, m, _ptr(out), _DTYPES[dtype], TQ3_DIM,
                              _stream(records)), "tq3_dequantize")
    return out


def tq3_quantize_split(x: torch.Tensor, signs, packed: torch.Tensor = None,
                       norms: torch.Tensor = None, scales: torch.Tensor = None):
    """x [..., D] -> (packed uint8 [..., D/128, 48], norms fp32 [..., D/128],
    scales fp32 [..., D/128]): tq3_quantize's fields in three arrays."""
    if not isinstance(x, torch.Tensor):
        raise TypeError("tq3_quantize expects a torch.Tensor input")
    if x.ndim == 0:
        raise ValueError("tq3_quantize expects at least one dimension")
    if x.shape[-1] <= 0 or x.shape[-1] % TQ3_DIM:
        raise ValueError(f"last dim must be a positive multiple of 128, got {x.shape[-1]}")
    if x.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {x.dtype}")
    _need_gpu(x)
    nb = x.shape[-1] // TQ3_DIM
    xv = x.reshape(-1, TQ3_DIM) if x.is_contiguous() else x.contiguous().reshape(-1, TQ3_DIM)
    n = xv.shape[0]
    lead = (*x.shape[:-1], nb)
    if packed is None:
        packed = torch.empty((*lead, 48), dtype=torch.uint8, device=x.device)
    if norms is None:
        norms = torch.empty(lead, dtype=torch.float32, device=x.device)
    if scales is None:
        scales = torch.empty(lead, dtype=torch.float32, device=x.device)
    for t, want, name in ((packed, torch.uint8, "packed"), (norms, torch.float32, "norms"),
                          (scales, torch.float32, "scales")):
        if t.dtype != want or not t.is_contiguous() or t.device != x.device:
            raise ValueError(f"{name} must be a contiguous {want} tensor on {x.device}")
    if packed.numel() != n * 48 or norms.numel() != n or scales.numel() != n:
        raise ValueError("output sizes do not match the input's vector count")
    m = signs if isinstance(signs, (bytes, bytearray)) else sign_mask(signs)
    _check(lib.tq3_quantize_split(_ptr(xv), _DTYPES[x.dtype], n, xv.stride(0), m, _ptr(packed),
                                  _ptr(norms), _ptr(scales), _stream(x)), "tq3_quantize_split")
    return packed, norms, scales


def tq3_dequantize_split(packed: torch.Tensor, norms: torch.Tensor, scales: torch.Tensor, signs,
                         dtype=torch.float32, out: torch.Tensor = None) -> torch.Tensor:
    """(packed uint8 [..., nb, 48], norms [..., nb], scales [..., nb], both fp32)
    -> [..., nb*128] of `dtype`."""
    if norms.shape != scales.shape:
        raise ValueError("TQ3 norms and scales must have identical shapes")
    if packed.dtype != torch.uint8 or packed.shape[:-1] != norms.shape or packed.shape[-1] != 48:
        raise ValueError("TQ3 packed must be uint8 with the shape of norms/scales + [48]")
    if norms.dtype != torch.float32 or scales.dtype != torch.float32:
        raise TypeError("TQ3 norms and scales must be float32")
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    n = norms.numel()
    if out is not None:
        _check_out(out, dtype, n * TQ3_DIM, packed.device, "tq3_dequantize_split")
    _need_gpu(packed, norms, scales)
    pk, nr, sc = packed.contiguous(), norms.contiguous(), scales.contiguous()
    lead = tuple(norms.shape[:-1])
    nb = norms.shape[-1] if norms.ndim >= 1 else 1
    if out is None:
        out = torch.empty((*lead, nb * TQ3_DIM), dtype=dtype, device=packed.device)
    m = signs if isinstance(signs, (bytes, bytearray)) else sign_mask(signs)
    _check(lib.tq3_dequantize_split(_ptr(pk), _ptr(nr), _ptr(sc), n, m, _ptr(out), _DTYPES[dtype],
                                    TQ3_DIM, _stream(packed)), "tq3_dequantize_split")
    return out


def tq3_quantize_dict(x: torch.Tensor, signs) -> dict:
    """The TQ3 page's return form: {"norms", "scales", "packed", "orig_shape"}."""
    packed, norms, scales = tq3_quantize_split(x, signs)
    return {"norms": norms, "scales": scales, "packed": packed, "orig_shape": x.shape}


def tq3_dequantize_dict(tq3: dict, signs, dtype=torch.float32) -> torch.Tensor:
    """A dict in the TQ3 page's form -> tensor of its orig_shape (fp32 unless
    `dtype` says otherwise). Missing keys raise KeyError, as on the page."""
    missing = {"norms", "scales", "packed", "orig_shape"}.difference(tq3)
    if missing:
        raise KeyError("TQ3 payload missing required keys: " + ", ".join(sorted(missing)))
    y = tq3_dequantize_split(tq3["packed"], tq3["norms"], tq3["scales"], signs, dtype)
    return y.reshape(tq3["orig_shape"])


def tq3_attention_workspace_bytes(n_tokens: int, n_q_heads: int, n_kv_heads: int) -> int:
    return int(lib.tq3_attention_workspace_bytes(n_tokens, n_q_heads, n_kv_heads))


def tq3_decode_attention(q: torch.Tensor, k_records: torch.Tensor, v_records: torch.Tensor,
                         n_kv_heads: int, signs, softmax_scale: float = None,
                         dtype=torch.float32, workspace: torch.Tensor = None,
                         out: torch.Tensor = None) -> torch.Tensor:
    """One decode step of attention over a TQ3-compressed KV cache.

    q [Hq, 128] (fp32/bf16/fp16); k_records, v_records uint8 [T, Hkv, 56] or
    [T * Hkv, 56], token-major; query head h reads KV head h // (Hq / Hkv).
    softmax_scale defaults to 1/sqrt(128). Returns [Hq, 128] of `dtype`.
    The workspace (uint8, tq3_attention_workspace_bytes) is allocated here
    when not given."""
    if q.dtype not in _DTYPES or dtype not in _DTYPES:
        raise TypeError("unsupported dtype")
    if q.ndim != 2 or q.shape[1] != TQ3_DIM:
        raise ValueError("q must be [n_q_heads, 128]")
    for r in (k_records, v_records):
        if r.dtype != torch.uint8 or r.shape[-1] != TQ3_RECORD_BYTES:
            raise ValueError("records must be uint8 [..., 56]")
    if k_records.numel() != v_records.numel():
        raise ValueError("K and V must hold the same number of records")
    hq, hkv = q.shape[0], int(n_kv_heads)
    if out is not None:
        _check_out(out, dtype, hq * TQ3_DIM, q.device, "tq3_decode_attention")
    if workspace is not None and (not isinstance(workspace, torch.Tensor)
                                  or not workspace.is_contiguous()
                                  or workspace.device != q.device):
        raise ValueError("tq3_decode_attention: workspace must be a contiguous tensor on "
                         f"{q.device}")
    _need_gpu(q, k_records, v_records)
    nrec = k_records.numel() // TQ3_RECORD_BYTES
    if hkv < 1 or nrec % hkv:
        raise ValueError("the records must split evenly over the KV heads")
    n_tok = nrec // hkv
    if softmax_scale is None:
        softmax_scale = TQ3_DIM ** -0.5
    qc, kc, vc = q.contiguous(), k_records.contiguous(), v_records.contiguous()
    need = tq3_attention_workspace_bytes(n_tok, hq, hkv)
    if need == 0:
        raise ValueError("unsupported sizes (need >= 1 token and Hq/Hkv in {1, 2, 4, 8})")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((hq, TQ3_DIM), dtype=dtype, device=q.device)
    m = signs if isinstance(signs, (bytes, bytearray)) else sign_mask(signs)
    _check(lib.tq3_decode_attention(_ptr(qc), _DTYPES[q.dtype], hq, _ptr(kc), _ptr(vc), n_tok,
                                    hkv, m, float(softmax_scale), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _ptr(out),
                                    _DTYPES[dtype], _stream(q)), "tq3_decode_attention")
    return out


def tq3_attention_noalloc_max_bytes() -> int:
    return int(lib.tq3_attention_noalloc_max_bytes())


def tq3_decode_attention_noalloc(q: torch.Tensor, k_records: torch.Tensor,
                                 v_records: torch.Tensor, n_kv_heads: int, signs,
                                 softmax_scale: float = None, dtype=torch.float32,
                                 out: torch.Tensor = None) -> torch.Tensor:
    """tq3_decode_attention with the library's own per-GPU scratch instead of a
    workspace (the C call allocates nothing; with `out` given, neither does
    this wrapper). Sizes needing more than tq3_attention_noalloc_max_bytes()
    of partial results raise ValueError. Calls that overlap in time on one GPU
    share the scratch and race."""
    if q.dtype not in _DTYPES or dtype not in _DTYPES:
        raise TypeError("unsupported dtype")
    if q.ndim != 2 or q.shape[1] != TQ3_DIM:
        raise ValueError("q must be [n_q_heads, 128]")
    for r in (k_records, v_records):
        if r.dtype != torch.uint8 or r.shape[-1] != TQ3_RECORD_BYTES:
            raise ValueError("records must be uint8 [..., 56]")
    if k_records.numel() != v_records.numel():
        raise ValueError("K and V must hold the same number of records")
    hq, hkv = q.shape[0], int(n_kv_heads)
    if out is not None:
        _check_out(out, dtype, hq * TQ3_DIM, q.device, "tq3_decode_attention_noalloc")
    _need_gpu(q, k_records, v_records)
    for t, name in ((q, "q"), (k_records, "k_records"), (v_records, "v_records")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (no copy is made)")
    nrec = k_records.numel() // TQ3_RECORD_BYTES
    if hkv < 1 or nrec % hkv:
        raise ValueError("the records must split evenly over the KV heads")
    if softmax_scale is None:
        softmax_scale = TQ3_DIM ** -0.5
    if out is None:
        out = torch.empty((hq, TQ3_DIM), dtype=dtype, device=q.device)
    m = signs if isinstance(signs, (bytes, bytearray)) else sign_mask(signs)
    _check(lib.tq3_decode_attention_noalloc(_ptr(q), _DTYPES[q.dtype], hq, _ptr(k_records),
                                            _ptr(v_records), nrec // hkv, hkv, m,
                                            float(softmax_scale), _ptr(out), _DTYPES[dtype],
                                            _stream(q)), "tq3_decode_attention_noalloc")
    return out


def tq3_memory_bytes(shape):
    """(compressed bytes, fp16 bytes, ratio) for a tensor shape [..., D]."""
    if not shape:
        raise ValueError("shape must be non-empty")
    if shape[-1] <= 0 or shape[-1] % TQ3_DIM:
        raise ValueError(f"last dim must be a positive multiple of 128, got {shape[-1]}")
    if any(d <= 0 for d in shape):
        raise ValueError(f"all dimensions must be positive, got {shape}")
    numel = 1
    for d in shape:
        numel *= d
    comp = numel // TQ3_DIM * tq3_record_bytes()
    return comp, numel * 2, numel * 2 / comp


# ------------------------------------------------------------ OrbitQuant ---

def orbit_block_size(d: int) -> int:
    return int(lib.orbit_block_size(d))


def tq_gaussian_lloyd_max(bits: int, iters: int = 200) -> torch.Tensor:
    out = (ctypes.c_double * (1 << bits))()
    _check(lib.tq_gaussian_lloyd_max(bits, iters, ctypes.cast(out, _vp)), "tq_gaussian_lloyd_max")
    return torch.tensor(list(out), dtype=torch.float64)


def orbit_make_codebook(bits: int, d: int) -> torch.Tensor:
    out = (ctypes.c_float * (1 << bits))()
    _check(lib.orbit_make_codebook(bits, d, ctypes.cast(out, _vp)), "orbit_make_codebook")
    return torch.tensor(list(out), dtype=torch.float32)


def _host_f32(cb) -> ctypes.Array:
    v = torch.as_tensor(cb).reshape(-1).to("cpu", torch.float32).tolist()
    return (ctypes.c_float * len(v))(*v)


def orbit_quantize_weight(W: torch.Tensor, bits: int, perm: torch.Tensor,
                          signs: torch.Tensor, codebook, bit_order: int = TQ_MSB_FIRST,
                          packed: torch.Tensor = None, row_norms: torch.Tensor = None):
    """fp32 W [rows, d] on the GPU -> (packed uint8 [rows, d*bits/8], row_norms fp32).
    perm: int32 [d], signs: int8 [d] (GPU); codebook: 2^bits fp32 (host values)."""
    if W.dtype != torch.float32 or W.ndim != 2:
        raise ValueError("W must be a 2-D fp32 tensor")
    _need_gpu(W, perm, signs)
    W = W.contiguous()
    rows, d = W.shape
    perm = perm.to(torch.int32).contiguous()
    signs = signs.to(torch.int8).contiguous()
    if packed is None:
        packed = torch.empty((rows, d * bits // 8), dtype=torch.uint8, device=W.device)
    if row_norms is None:
        row_norms = torch.empty((rows,), dtype=torch.float32, device=W.device)
    # caller-given buffers (requantize_ writes into the layer's own) must fit
    if (packed.dtype != torch.uint8 or not packed.is_contiguous() or not packed.is_cuda
            or packed.numel() != rows * d * bits // 8):
        raise ValueError("packed must be a contiguous uint8 GPU tensor of rows*d*bits/8 bytes")
    if (row_norms.dtype != torch.float32 or not row_norms.is_contiguous() or not row_norms.is_cuda
            or row_norms.numel() != rows):
        raise ValueError("row_norms must be a contiguous fp32 GPU tensor of `rows` values")
    cb = _host_f32(codebook)
    if len(cb) != (1 << bits):
        raise ValueError("codebook must hold 2**bits values")
    _check(lib.orbit_quantize_weight(_ptr(W), rows, d, bits, _ptr(perm), _ptr(signs),
                                     ctypes.cast(cb, _vp), bit_order, _ptr(packed),
                                     _ptr(row_norms), _stream(W)), "orbit_quantize_weight")
    return packed, row_norms


def orbit_rotate(x: torch.Tensor, perm: torch.Tensor, signs: torch.Tensor,
                 out: torch.Tensor = None) -> torch.Tensor:
    """rpbh_forward of activation rows x [..., d] (fp32, bf16 or fp16, GPU) ->
    the same shape and dtype; bf16 / fp16 round every stage to their format."""
    if x.dtype not in _DTYPES or x.ndim < 1:
        raise ValueError("x must be an fp32, bf16 or fp16 tensor")
    _need_gpu(x, perm, signs)
    d = x.shape[-1]
    xv = x.contiguous().reshape(-1, d)
    perm = perm.to(torch.int32).contiguous()
    signs = signs.to(torch.int8).contiguous()
    if out is None:
        out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    if out.dtype != x.dtype or not out.is_contiguous() or out.numel() != x.numel():
        raise ValueError("out must be a contiguous tensor of x's dtype and size")
    _check(lib.orbit_rotate(_ptr(xv), _DTYPES[x.dtype], xv.shape[0], d, _ptr(perm), _ptr(signs),
                            _ptr(out), _stream(x)), "orbit_rotate")
    return out


def _linear_weight_args(x, m, d_in, packed, row_norms, bits, codebook, bias, out, lead):
    """Checks shared by orbit_linear and orbit_linear_tiled -> (packed,
    norms, bias pointer, host codebook, out)."""
    d_out = row_norms.numel()
    if packed.numel() != d_out * d_in * bits // 8:
        raise ValueError("packed does not match d_out x d_in at this bit width")
    nr = row_norms.to(torch.float32).contiguous()
    pk = packed.contiguous()
    bp = None
    if bias is not None:
        if bias.dtype != x.dtype or bias.numel() != d_out:
            raise ValueError("bias must hold d_out values of the activations' dtype")
        bias = bias.contiguous()
        _need_gpu(bias)
        bp = _ptr(bias)
    cb = _host_f32(codebook)
    if len(cb) != (1 << bits):
        raise ValueError("codebook must hold 2**bits values")
    if out is None:
        out = torch.empty((*lead, d_out), dtype=x.dtype, device=x.device)
    if (out.dtype != x.dtype or not out.is_contiguous() or out.numel() != m * d_out
            or out.device != x.device):
        raise ValueError("out must be a contiguous [..., d_out] tensor of the activations' "
                         "dtype on their device")
    return pk, nr, bp, cb, out


def orbit_linear(x_rot: torch.Tensor, packed: torch.Tensor, row_norms: torch.Tensor, bits: int,
                 codebook, bias: torch.Tensor = None, bit_order: int = TQ_MSB_FIRST,
                 out: torch.Tensor = None) -> torch.Tensor:
    """x_rot [..., d_in] (fp32, bf16 or fp16) times the rotated-basis weight
    decoded from packed [d_out, d_in*bits/8] and row_norms [d_out], plus bias
    (same dtype as x_rot) -> [..., d_out] of x_rot's dtype."""
    if x_rot.dtype not in _DTYPES:
        raise ValueError("x_rot must be fp32, bf16 or fp16")
    _need_gpu(x_rot, packed, row_norms)
    d_in = x_rot.shape[-1]
    xv = x_rot.contiguous().reshape(-1, d_in)
    pk, nr, bp, cb, out = _linear_weight_args(x_rot, xv.shape[0], d_in, packed, row_norms, bits,
                                              codebook, bias, out, x_rot.shape[:-1])
    _check(lib.orbit_linear(_ptr(xv), _DTYPES[x_rot.dtype], xv.shape[0], d_in, _ptr(pk),
                            _ptr(nr), row_norms.numel(), bits,
                            ctypes.cast(cb, _vp), bit_order, bp, _ptr(out), _stream(x_rot)),
           "orbit_linear")
    return out


def orbit_tiled_bytes(m: int, d: int) -> int:
    return int(lib.orbit_tiled_bytes(m, d))


def orbit_rotate_tiled(x: torch.Tensor, perm: torch.Tensor, signs: torch.Tensor,
                       out: torch.Tensor = None) -> torch.Tensor:
    """orbit_rotate of bf16 / fp16 rows x [m, d] into the matrix-core operand
    layout orbit_linear_tiled reads (rows padded to a multiple of 16 with
    zeros) -> a flat tensor of x's dtype, orbit_tiled_bytes(m, d) bytes."""
    if x.dtype not in (torch.bfloat16, torch.float16) or x.ndim != 2:
        raise ValueError("x must be a 2-D bf16 or fp16 tensor")
    m, d = x.shape
    nbytes = orbit_tiled_bytes(m, d)
    if nbytes == 0 and m > 0:
        raise ValueError("d must be a positive multiple of 32, at most 16384")
    if out is None:
        out = torch.empty(nbytes // 2, dtype=x.dtype, device=x.device)
    _check_out(out, x.dtype, nbytes // 2, x.device, "orbit_rotate_tiled")
    _need_gpu(x, perm, signs)
    xv = x.contiguous()
    perm = perm.to(torch.int32).contiguous()
    signs = signs.to(torch.int8).contiguous()
    _check(lib.orbit_rotate_tiled(_ptr(xv), _DTYPES[x.dtype], m, d, _ptr(perm), _ptr(signs),
                                  _ptr(out), _stream(x)), "orbit_rotate_tiled")
    return out


def orbit_linear_tiled(x_tiled: torch.Tensor, m: int, packed: torch.Tensor,
                       row_norms: torch.Tensor, bits: int, codebook, bias: torch.Tensor = None,
                       bit_order: int = TQ_MSB_FIRST, out: torch.Tensor = None) -> torch.Tensor:
    """orbit_linear of m rows held in the tiled layout (orbit_rotate_tiled's
    output; d_in from packed and row_norms) -> [m, d_out] of x_tiled's dtype."""
    if x_tiled.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("x_tiled must be bf16 or fp16")
    d_out = row_norms.numel()
    if d_out < 1 or (packed.numel() * 8) % (bits * d_out):
        raise ValueError("packed does not hold d_out rows at this bit width")
    d_in = packed.numel() * 8 // (bits * d_out)
    if not x_tiled.is_contiguous() or x_tiled.numel() * 2 != orbit_tiled_bytes(m, d_in):
        raise ValueError("x_tiled must be a contiguous tiled [m, d_in] buffer")
    _need_gpu(x_tiled, packed, row_norms)
    pk, nr, bp, cb, out = _linear_weight_args(x_tiled, m, d_in, packed, row_norms, bits,
                                              codebook, bias, out, (m,))
    _check(lib.orbit_linear_tiled(_ptr(x_tiled), _DTYPES[x_tiled.dtype], m, d_in, _ptr(pk),
                                  _ptr(nr), d_out, bits, ctypes.cast(cb, _vp), bit_order, bp,
                                  _ptr(out), _stream(x_tiled)), "orbit_linear_tiled")
    return out


# the forward takes the tiled path above this many bf16 / fp16 rows (the
# few-rows kernels below read x_rot through LDS anyway)
_TILED_MIN_ROWS = 64


def orbit_forward(x: torch.Tensor, packed: torch.Tensor, row_norms: torch.Tensor,
                  perm: torch.Tensor, signs: torch.Tensor, bits: int, codebook,
                  bias: torch.Tensor = None, bit_order: int = TQ_MSB_FIRST) -> torch.Tensor:
    """The quantized layer's forward: orbit_linear(orbit_rotate(x), ...). For
    more than 64 bf16 / fp16 rows (and 64 <= d_in < 2^22) the rotation goes
    into the tiled layout and orbit_linear_tiled reads it: the same values."""
    d_in = x.shape[-1]
    rows = x.numel() // d_in if d_in else 0
    if (x.dtype in (torch.bfloat16, torch.float16) and rows > _TILED_MIN_ROWS
            and 64 <= d_in < (1 << 22) and d_in % 32 == 0):
        xv = x.reshape(rows, d_in)
        y = orbit_linear_tiled(orbit_rotate_tiled(xv, perm, signs), rows, packed, row_norms,
                               bits, codebook, bias, bit_order)
        return y.reshape(*x.shape[:-1], row_norms.numel())
    return orbit_linear(orbit_rotate(x, perm, signs), packed, row_norms, bits, codebook, bias,
                        bit_order)


def orbit_dequantize(packed: torch.Tensor, row_norms: torch.Tensor, d: int, bits: int,
                     inv_perm: torch.Tensor, signs: torch.Tensor, codebook,
                     bit_order: int = TQ_MSB_FIRST, rotated_only: bool = False,
                     dtype=torch.float32, out: torch.Tensor = None) -> torch.Tensor:
    """-> [rows, d] of `dtype`: the rotated-basis W' (rotated_only) or W."""
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    if bits not in (2, 3, 4):
        raise ValueError("bits must be 2, 3 or 4")
    rows = row_norms.numel()
    if packed.dtype != torch.uint8 or packed.numel() != rows * d * bits // 8:
        raise ValueError("packed must be uint8 holding rows * d * bits / 8 bytes")
    cb = _host_f32(codebook)
    if len(cb) != (1 << bits):
        raise ValueError("codebook must hold 2**bits values")
    for t, name in ((inv_perm, "inv_perm"), (signs, "signs")):
        if t is None:
            if not rotated_only:
                raise ValueError(f"{name} is needed unless rotated_only")
        elif t.numel() != d:
            raise ValueError(f"{name} must hold d = {d} entries")
    if out is not None:
        _check_out(out, dtype, rows * d, packed.device, "orbit_dequantize")
    _need_gpu(packed, row_norms)
    packed = packed.contiguous()
    row_norms = row_norms.to(torch.float32).contiguous()
    if out is None:
        out = torch.empty((rows, d), dtype=dtype, device=packed.device)
    ip = inv_perm.to(torch.int32).contiguous() if inv_perm is not None else None
    sg = signs.to(torch.int8).contiguous() if signs is not None else None
    for t in (ip, sg):
        if t is not None:
            _need_gpu(t)
    _check(lib.orbit_dequantize(_ptr(packed), _ptr(row_norms), rows, d, bits,
                                _ptr(ip) if ip is not None else None,
                                _ptr(sg) if sg is not None else None,
                                ctypes.cast(cb, _vp), bit_order, int(bool(rotated_only)),
                                _ptr(out), _DTYPES[dtype], _stream(packed)), "orbit_dequantize")
    return out
