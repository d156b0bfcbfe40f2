"""ctypes binding of libasv.so: argument marshalling only.

Every function here has the name of the C entry point it calls (without the
``asv_`` prefix), converts tensors to device addresses and torch streams to
``hipStream_t`` handles, and raises ``AsvError`` on a non-zero return code.
No step of the computation runs in Python. When libasv.so is missing the
first call raises: there is no fallback.
"""

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libasv.so")

ABI_VERSION = 4
HIDDEN = 2048
CONV_IN = 6144
Q_HEADS = 32
KV_HEADS = 8
HEAD_DIM = 64
TILE_ROWS = 16
KEY_BLOCK = 32
MAX_ROWS = 2048
MAX_KEYS = 131072
PARTIAL_FLOATS = 66

OK, E_ARG, E_SHAPE, E_UNSUPPORTED, E_CAPACITY, E_HIP = 0, -1, -2, -3, -4, -5

# every entry point include/asv.h declares
SYMBOLS = [
    "asv_abi_version", "asv_strerror", "asv_seg_table_build", "asv_block_table_build",
    "asv_table_upload",
    "asv_shared_conv", "asv_shared_attn", "asv_attn_merge", "asv_row_argmax_workspace",
    "asv_row_argmax", "asv_row_argmax_noalloc", "asv_draft_ids", "asv_markov_workspace",
    "asv_markov_pick", "asv_markov_pick_form",
    "asv_markov_pack_w2", "asv_shared_qk",
]

QKV_WIDTH = 3072

MARKOV_MAX_CHAINS = 32
MARKOV_MAX_DEPTH = 16
MARKOV_MAX_RANK = 256


class AsvError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} ({code})")


class StreamDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("key_count", ctypes.c_int32),
                ("kv_capacity", ctypes.c_int32)]


class MarkovChain(ctypes.Structure):
    _fields_ = [("row0", ctypes.c_int32), ("depth", ctypes.c_int32)]


class TableInfo(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32), ("n_streams", ctypes.c_int32),
        ("n_rows", ctypes.c_int32), ("n_tiles", ctypes.c_int32), ("n_work", ctypes.c_int32),
        ("n_conv_layers", ctypes.c_int32), ("n_attn_layers", ctypes.c_int32),
        ("max_tile_rows", ctypes.c_int32), ("partial_count", ctypes.c_int64),
        ("blob_bytes", ctypes.c_int64), ("off_segs", ctypes.c_int64),
        ("off_rows", ctypes.c_int64), ("off_tiles", ctypes.c_int64),
        ("off_work", ctypes.c_int64), ("off_conv_state", ctypes.c_int64),
        ("off_k", ctypes.c_int64), ("off_v", ctypes.c_int64),
    ]


# numpy views of the blob's arrays (layouts of include/asv.h)
SEG_DTYPE = np.dtype([("row0", "<i4"), ("rows", "<i4"), ("keys", "<i4"), ("cap", "<i4"),
                      ("split_keys", "<i4"), ("nsplit", "<i4"), ("poff", "<i8"),
                      ("split_tail", "<i4"), ("nbig", "<i4"), ("reserved", "<i4", (2,))])
ROW_DTYPE = np.dtype([("stream", "<i4"), ("pos", "<i4"), ("nkeys", "<i4"), ("tile", "<i4")])
TILE_DTYPE = np.dtype([("stream", "<i4"), ("row0", "<i4"), ("nrows", "<i4"), ("pos0", "<i4")])
WORK_DTYPE = np.dtype([("tile", "<i4"), ("head", "i1"), ("ntiles", "i1"), ("stream", "<i2"),
                       ("split", "<i4"), ("keys", "<i4")])

_lib = None


def lib():
    """Load libasv.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m attention_stream_verify_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.asv_abi_version.restype = ctypes.c_int
        L.asv_abi_version.argtypes = []
        L.asv_strerror.restype = ctypes.c_char_p
        L.asv_strerror.argtypes = [ctypes.c_int]
        L.asv_seg_table_build.restype = ctypes.c_int
        L.asv_seg_table_build.argtypes = [ctypes.POINTER(StreamDesc), i32, ctypes.POINTER(vp), i32,
                                          ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp, sz,
                                          ctypes.POINTER(TableInfo)]
        L.asv_block_table_build.restype = ctypes.c_int
        L.asv_block_table_build.argtypes = L.asv_seg_table_build.argtypes
        L.asv_table_upload.restype = ctypes.c_int
        L.asv_table_upload.argtypes = [vp, sz, vp, vp]
        L.asv_shared_conv.restype = ctypes.c_int
        L.asv_shared_conv.argtypes = [ctypes.POINTER(TableInfo), vp, i32, vp, vp, vp, vp]
        L.asv_shared_attn.restype = ctypes.c_int
        L.asv_shared_attn.argtypes = [ctypes.POINTER(TableInfo), vp, i32, vp, vp, vp]
        L.asv_attn_merge.restype = ctypes.c_int
        L.asv_attn_merge.argtypes = [ctypes.POINTER(TableInfo), vp, vp, vp, vp]
        L.asv_row_argmax_workspace.restype = sz
        L.asv_row_argmax_workspace.argtypes = [i64, i64]
        L.asv_row_argmax.restype = ctypes.c_int
        L.asv_row_argmax.argtypes = [vp, i64, i64, i64, vp, vp, vp, sz, vp]
        L.asv_row_argmax_noalloc.restype = ctypes.c_int
        L.asv_row_argmax_noalloc.argtypes = [vp, i64, i64, i64, vp, vp, vp]
        L.asv_draft_ids.restype = ctypes.c_int
        L.asv_draft_ids.argtypes = [vp, i32, vp, vp, i64, i64, vp, i64, vp, vp]
        L.asv_markov_workspace.restype = sz
        L.asv_markov_workspace.argtypes = [i64]
        L.asv_markov_pick.restype = ctypes.c_int
        L.asv_markov_pick.argtypes = [vp, i64, i64, ctypes.POINTER(MarkovChain), i32, vp, vp, vp,
                                      i64, i32, vp, vp, vp, sz, vp]
        L.asv_markov_pick_form.restype = ctypes.c_int
        L.asv_markov_pick_form.argtypes = [vp, i64, i64, ctypes.POINTER(MarkovChain), i32, vp, vp, vp,
                                           i64, i32, vp, vp, vp, sz, i32, vp]
        L.asv_shared_qk.restype = ctypes.c_int
        L.asv_shared_qk.argtypes = [ctypes.POINTER(TableInfo), vp, i32, vp, vp, vp, ctypes.c_double,
                                    ctypes.c_double, vp, vp]
        L.asv_markov_pack_w2.restype = ctypes.c_int
        L.asv_markov_pack_w2.argtypes = [vp, i64, i32, vp, vp]
        if L.asv_abi_version() != ABI_VERSION:
            raise RuntimeError("libasv.so has a different ABI version than this binding")
        _lib = L
    return _lib


def strerror(code):
    return lib().asv_strerror(int(code)).decode()


def abi_version():
    return int(lib().asv_abi_version())


def _check(code, where):
    if code != OK:
        raise AsvError(code, where)


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s):
    if s is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _ptr_array(rows):
    flat = [_addr(p) for layer in rows for p in layer]
    arr = (ctypes.c_void_p * max(1, len(flat)))(*flat)
    return arr


def time_table_build(streams, conv_state=(), k_cache=(), v_cache=(), reps=20, full=False):
    """Average host time of one table build call, in microseconds: the
    arguments are marshalled once, then the C call alone is timed."""
    import time
    L = lib()
    build = L.asv_block_table_build if full else L.asv_seg_table_build
    S = len(streams)
    descs = (StreamDesc * max(1, S))(*[StreamDesc(int(w), int(k), int(c)) for (w, k, c) in streams])
    n_conv, n_attn = len(conv_state), len(k_cache)
    cs = _ptr_array(conv_state) if n_conv else None
    kp = _ptr_array(k_cache) if n_attn else None
    vv = _ptr_array(v_cache) if n_attn else None
    info = TableInfo()
    _check(build(descs, S, cs, n_conv, kp, vv, n_attn, None, 0, ctypes.byref(info)), "table build")
    blob = np.zeros(int(info.blob_bytes), dtype=np.uint8)
    addr, nbytes = blob.ctypes.data, blob.nbytes
    t0 = time.perf_counter()
    for _ in range(reps):
        build(descs, S, cs, n_conv, kp, vv, n_attn, addr, nbytes, ctypes.byref(info))
    return (time.perf_counter() - t0) / reps * 1e6


def seg_table_build(streams, conv_state=(), k_cache=(), v_cache=(), blob=None, full=False):
    """Build the round's table on the host (full: block attention, every row
    seeing all of its stream's keys -- asv_block_table_build).

    streams: [(rows, key_count, kv_capacity)]; conv_state / k_cache / v_cache:
    per layer, a list with one tensor (or device address) per stream.
    Returns (info, blob) with blob a numpy uint8 array of info.blob_bytes
    (or the given ``blob`` buffer, a writable uint8 numpy array or pinned
    CPU tensor).
    """
    L = lib()
    build = L.asv_block_table_build if full else L.asv_seg_table_build
    name = "asv_block_table_build" if full else "asv_seg_table_build"
    S = len(streams)
    descs = (StreamDesc * max(1, S))(*[StreamDesc(int(w), int(k), int(c)) for (w, k, c) in streams])
    n_conv, n_attn = len(conv_state), len(k_cache)
    if len(v_cache) != n_attn:
        raise ValueError("k_cache and v_cache need the same number of layers")
    cs = _ptr_array(conv_state) if n_conv else None
    kp = _ptr_array(k_cache) if n_attn else None
    vv = _ptr_array(v_cache) if n_attn else None
    info = TableInfo()
    _check(build(descs, S, cs, n_conv, kp, vv, n_attn, None, 0, ctypes.byref(info)), name)
    if blob is None:
        blob = np.zeros(int(info.blob_bytes), dtype=np.uint8)
    if isinstance(blob, np.ndarray):
        addr, nbytes = blob.ctypes.data, blob.nbytes
    else:
        addr, nbytes = int(blob.data_ptr()), blob.numel() * blob.element_size()
    _check(build(descs, S, cs, n_conv, kp, vv, n_attn, addr, nbytes, ctypes.byref(info)), name)
    return info, blob


def table_arrays(info, blob):
    """numpy views of a host blob's arrays (segs, rows, tiles, work, addresses)."""
    b = blob if isinstance(blob, np.ndarray) else blob.numpy()
    b = b.view(np.uint8)
    S, R = info.n_streams, info.n_rows

    def take(off, dtype, n):
        return b[off:off + dtype.itemsize * n].view(dtype)

    return {
        "segs": take(info.off_segs, SEG_DTYPE, S),
        "rows": take(info.off_rows, ROW_DTYPE, R),
        "tiles": take(info.off_tiles, TILE_DTYPE, info.n_tiles),
        "work": take(info.off_work, WORK_DTYPE, info.n_work),
        "conv_state": take(info.off_conv_state, np.dtype("<u8"), info.n_conv_layers * S),
        "k": take(info.off_k, np.dtype("<u8"), info.n_attn_layers * S),
        "v": take(info.off_v, np.dtype("<u8"), info.n_attn_layers * S),
    }


def table_upload(blob, dev_blob, stream=None):
    if isinstance(blob, np.ndarray):
        addr, nbytes = blob.ctypes.data, blob.nbytes
    else:
        addr, nbytes = int(blob.data_ptr()), blob.numel() * blob.element_size()
    _check(lib().asv_table_upload(addr, nbytes, _addr(dev_blob), _stream(stream)),
           "asv_table_upload")


def shared_conv(info, dev_blob, layer, x, w, y, stream=None):
    _check(lib().asv_shared_conv(ctypes.byref(info), _addr(dev_blob), int(layer), _addr(x),
                                 _addr(w), _addr(y), _stream(stream)), "asv_shared_conv")


def shared_attn(info, dev_blob, layer, q, partials, stream=None):
    _check(lib().asv_shared_attn(ctypes.byref(info), _addr(dev_blob), int(layer), _addr(q),
                                 _addr(partials), _stream(stream)), "asv_shared_attn")


def attn_merge(info, dev_blob, partials, o, stream=None):
    _check(lib().asv_attn_merge(ctypes.byref(info), _addr(dev_blob), _addr(partials), _addr(o),
                                _stream(stream)), "asv_attn_merge")


def row_argmax_workspace(rows, vocab):
    return int(lib().asv_row_argmax_workspace(int(rows), int(vocab)))


def row_argmax(logits, rows, vocab, row_stride, pick, flag, workspace, stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().asv_row_argmax(_addr(logits), int(rows), int(vocab), int(row_stride), _addr(pick),
                                _addr(flag), _addr(workspace), nbytes, _stream(stream)),
           "asv_row_argmax")


ARGMAX_SCRATCH_BYTES = 4 << 20


def row_argmax_noalloc(logits, rows, vocab, row_stride, pick, flag, stream=None):
    """asv_row_argmax_noalloc: the same picks and flags, the workspace being
    the library's own device array (no allocation)."""
    _check(lib().asv_row_argmax_noalloc(_addr(logits), int(rows), int(vocab), int(row_stride),
                                        _addr(pick), _addr(flag), _stream(stream)),
           "asv_row_argmax_noalloc")


def draft_ids(spans, n_streams, pick, pick_flag, n_picks, vocab, ids, n_ids, fail, stream=None):
    """spans: device int32 [n_streams][3] (src, dst, count); the rest device
    tensors as in include/asv.h."""
    _check(lib().asv_draft_ids(_addr(spans), int(n_streams), _addr(pick), _addr(pick_flag),
                               int(n_picks), int(vocab), _addr(ids), int(n_ids), _addr(fail),
                               _stream(stream)), "asv_draft_ids")


def partial_floats(info):
    """floats of the partials buffer asv_shared_attn writes."""
    return int(info.partial_count) * PARTIAL_FLOATS


def markov_workspace(vocab):
    return int(lib().asv_markov_workspace(int(vocab)))


def markov_pack_w2(w2, vocab, rank, w2c, stream=None):
    """W2 [vocab][rank] bf16 -> the tiled layout markov_pick reads (64-token tiles, each [rank/8][tile][8])."""
    _check(lib().asv_markov_pack_w2(_addr(w2), int(vocab), int(rank), _addr(w2c), _stream(stream)),
           "asv_markov_pack_w2")


MARKOV_FORMS = {"auto": 0, "launches": 1, "resident": 2}


def markov_pick(base, rows, row_stride, chains, prev0, w1, w2c, vocab, rank, pick, flag, workspace,
                stream=None, form=None):
    """chains: host list of (row0, depth); the rest device tensors as in
    include/asv_draft.h. workspace: a device tensor of markov_workspace(vocab)
    bytes. form: None (asv_markov_pick) or "auto" / "launches" / "resident"
    (asv_markov_pick_form)."""
    n = len(chains)
    arr = (MarkovChain * max(1, n))(*[MarkovChain(int(r), int(d)) for (r, d) in chains])
    nbytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    args = (_addr(base), int(rows), int(row_stride), arr, n, _addr(prev0), _addr(w1), _addr(w2c), int(vocab),
            int(rank), _addr(pick), _addr(flag), _addr(workspace), nbytes)
    if form is None:
        _check(lib().asv_markov_pick(*args, _stream(stream)), "asv_markov_pick")
    else:
        _check(lib().asv_markov_pick_form(*args, MARKOV_FORMS[form], _stream(stream)), "asv_markov_pick_form")


def shared_qk(info, dev_blob, layer, qkv, q_gain, k_gain, theta, eps, q_out, stream=None):
    """qk stage of attention layer `layer`: q to q_out, k and v into the caches
    the table names."""
    _check(lib().asv_shared_qk(ctypes.byref(info), _addr(dev_blob), int(layer), _addr(qkv), _addr(q_gain),
                               _addr(k_gain), float(theta), float(eps), _addr(q_out), _stream(stream)),
           "asv_shared_qk")
