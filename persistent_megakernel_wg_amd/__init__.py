"""Python binding of libamk.so (the C ABI in include/amk.h).

Argument marshalling only: every step of the decode path runs in the
library's HIP kernels.  PyTorch supplies device memory and streams.  There
is no fallback: importing the binding fails when libamk.so is missing.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("AMK_LIB_PATH") or os.path.join(_HERE, "libamk.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "(the decode path has no CPU fallback)")

# torch brings its own HIP runtime (same soname as the system one).  Load it
# first so that libamk.so binds to that runtime instead of pulling a second
# HIP/HSA runtime into the process.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

# ---------------------------------------------------------------- types --

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_UNSAFE_SCHEDULE, ERR_OUT_OF_RANGE, ERR_HIP, \
    ERR_NOMEM, ERR_TIMEOUT = 0, -1, -2, -3, -4, -5, -6, -7
NOALLOC_SCRATCH_BYTES = 96 * 1024 * 1024  # AMK_NOALLOC_SCRATCH_BYTES
W_BF16, W_INT8_ROW, W_INT4_G128 = 0, 1, 2
WFMT = {"bf16": W_BF16, "int8": W_INT8_ROW, "int4": W_INT4_G128}
TASK_NOP, TASK_QKV, TASK_ATTN, TASK_MERGE, TASK_OPROJ, TASK_GATEUP, TASK_DOWN, TASK_LMHEAD = range(8)
TASK_NAMES = ["NOP", "QKV", "ATTN", "MERGE", "OPROJ", "GATEUP", "DOWN", "LMHEAD"]
BUF_WEIGHT, BUF_SCRATCH, BUF_OUTPUT, BUF_STATE, BUF_HISTORY = range(5)
ACCESS_READ, ACCESS_WRITE = 1, 2
V_OK, V_REF, V_THRESHOLD, V_CYCLE, V_QUEUE_ORDER, V_UNDER_JOINED, V_RACE, V_OUTPUT = range(8)
VERDICT_NAMES = ["OK", "REF", "THRESHOLD", "CYCLE", "QUEUE_ORDER", "UNDER_JOINED", "RACE", "OUTPUT"]
FUSE_DEFAULT = 0xF

_i32, _u32, _i64, _f32, _p = ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class ModelConfig(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim",
                                    "ffn", "vocab", "max_ctx")] + [
        ("rms_eps", _f32), ("rope_theta", _f32), ("tied_embeddings", _i32), ("attn_bias", _i32),
        ("mlp_bias", _i32), ("wfmt", _i32), ("act_bf16", _i32)]

    @classmethod
    def from_workload(cls, wl):
        return cls(wl.n_layers, wl.hidden, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.ffn,
                   wl.vocab, wl.max_ctx, wl.rms_eps, wl.rope_theta, int(wl.tied), 0, 0,
                   WFMT[wl.wfmt], int(wl.act_bf16))


class ScheduleConfig(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("num_cus", "wg_threads", "tiles_qkv", "tiles_o",
                                    "tiles_gateup", "tiles_down", "tiles_lm", "attn_splits",
                                    "cu_policy", "pipeline_depth")] + [("fuse_flags", _u32)] + [
        (n, _i32) for n in ("poll_mode", "release_mode", "prefetch_kb")] + [("xcd_weight", (_i32 * 8) * 5), ("merge_o_share", _i32),
        ("merge_place", _i32), ("prefetch_attn_kb", _i32), ("sync_mode", _i32)]

    def as_dict(self):
        return {n: ([list(r) for r in getattr(self, n)] if n == "xcd_weight" else getattr(self, n))
                for n, _ in self._fields_}


TASK_NAMES = ["NOP", "QKV", "ATTN", "MERGE", "OPROJ", "GATEUP", "DOWN", "LMHEAD"]
TASK_NTYPES = len(TASK_NAMES)


class RegionStat(ctypes.Structure):
    _fields_ = [("n_tasks", _i32), ("wait_us", ctypes.c_double), ("work_us", ctypes.c_double),
                ("signal_us", ctypes.c_double), ("span_us", ctypes.c_double)]


class TaskDesc(ctypes.Structure):
    _fields_ = [("type", _i32), ("cu", _i32), ("p", _i32 * 8)]


class WaitDesc(ctypes.Structure):
    _fields_ = [("counter", _i32), ("threshold", _u32)]


class AccessDesc(ctypes.Structure):
    _fields_ = [("buffer", _i32), ("mode", _i32), ("begin", _i64), ("end", _i64)]


class BufferDesc(ctypes.Structure):
    _fields_ = [("size", _i64), ("kind", _i32), ("reserved", _i32)]


class ScheduleDesc(ctypes.Structure):
    _fields_ = [("model", ModelConfig), ("config", ScheduleConfig), ("n_tasks", _i32),
                ("n_counters", _i32), ("n_buffers", _i32), ("n_cus", _i32),
                ("tasks", ctypes.POINTER(TaskDesc)),
                ("wait_off", ctypes.POINTER(_i32)), ("waits", ctypes.POINTER(WaitDesc)),
                ("sig_off", ctypes.POINTER(_i32)), ("sigs", ctypes.POINTER(_i32)),
                ("acc_off", ctypes.POINTER(_i32)), ("accesses", ctypes.POINTER(AccessDesc)),
                ("queue_off", ctypes.POINTER(_i32)), ("queue", ctypes.POINTER(_i32)),
                ("buffers", ctypes.POINTER(BufferDesc))]


class Verdict(ctypes.Structure):
    _fields_ = [("code", _i32), ("task", _i32), ("counter", _i32), ("aux", _i32)]

    def astuple(self):
        return (self.code, self.task, self.counter, self.aux)


class DeviceBuffers(ctypes.Structure):
    _fields_ = [("weights", ctypes.POINTER(_p)), ("n_weights", _i32), ("kv_cache", _p),
                ("logits", ctypes.POINTER(_f32))]


_SIGS = {
    "amk_default_schedule_config": ([ctypes.POINTER(ModelConfig), _i32, ctypes.POINTER(ScheduleConfig)], _i32),
    "amk_build_schedule": ([ctypes.POINTER(ModelConfig), ctypes.POINTER(ScheduleConfig), ctypes.POINTER(_p)], _i32),
    "amk_validate": ([_p, ctypes.POINTER(Verdict)], _i32),
    "amk_multistep_check": ([_p, ctypes.POINTER(_i32)], _i32),
    "amk_schedule_view": ([_p, ctypes.POINTER(ScheduleDesc)], _i32),
    "amk_schedule_from_desc": ([ctypes.POINTER(ScheduleDesc), ctypes.POINTER(_p)], _i32),
    "amk_schedule_free": ([_p], None),
    "amk_packed_count": ([ctypes.POINTER(ModelConfig), ctypes.POINTER(_i32)], _i32),
    "amk_packed_bytes": ([ctypes.POINTER(ModelConfig), _i32, ctypes.POINTER(ctypes.c_size_t)], _i32),
    "amk_pack_tensor": ([ctypes.POINTER(ModelConfig), _i32, ctypes.POINTER(_p), _p], _i32),
    "amk_unpack_tensor": ([ctypes.POINTER(ModelConfig), _i32, _i32, _p, _p, _p, _p], _i32),
    "amk_kv_bytes": ([ctypes.POINTER(ModelConfig), ctypes.POINTER(ctypes.c_size_t)], _i32),
    "amk_engine_create": ([_p, ctypes.POINTER(DeviceBuffers), ctypes.POINTER(_p)], _i32),
    "amk_engine_create_noalloc": ([_p, ctypes.POINTER(DeviceBuffers), ctypes.POINTER(_p)], _i32),
    "amk_decode_step": ([_p, _i32, _i32, _p], _i32),
    "amk_decode_steps": ([_p, _i32, _i32, _i32, _p, _p], _i32),
    "amk_engine_check": ([_p], _i32),
    "amk_engine_launch_empty": ([_p, _p], _i32),
    "amk_engine_set_spin_budget": ([_p, _i64], _i32),
    "amk_engine_set_kv_length": ([_p, _i32], _i32),
    "amk_engine_set_trace": ([_p, _i32], _i32),
    "amk_engine_read_trace": ([_p, _p, _i64, ctypes.POINTER(_i32)], _i32),
    "amk_engine_region_stats": ([_p, _p], _i32),
    "amk_engine_steps": ([_p, ctypes.POINTER(_i64)], _i32),
    "amk_engine_destroy": ([_p], _i32),
    "amk_stream_read_probe": ([_p, ctypes.c_size_t, _p, _i32, _p], _i32),
    "amk_status_string": ([_i32], ctypes.c_char_p),
    "amk_last_error": ([], ctypes.c_char_p),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = sorted(_SIGS)


class AmkError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.amk_last_error().decode(errors="replace")
        name = _lib.amk_status_string(status).decode()
        super().__init__(f"{where}: {name}: {msg}")


def _check(status, where):
    if status != OK:
        raise AmkError(status, where)


# --------------------------------------------------------- configuration --

def default_schedule_config(model, device_cus):
    out = ScheduleConfig()
    _check(_lib.amk_default_schedule_config(ctypes.byref(model), device_cus, ctypes.byref(out)),
           "amk_default_schedule_config")
    return out


class Schedule:
    """Owns an amk_schedule*."""

    def __init__(self, handle, keep=None):
        self._h = ctypes.c_void_p(handle)
        self._keep = keep

    @classmethod
    def build(cls, model, config):
        h = ctypes.c_void_p()
        _check(_lib.amk_build_schedule(ctypes.byref(model), ctypes.byref(config), ctypes.byref(h)),
               "amk_build_schedule")
        return cls(h.value)

    @property
    def handle(self):
        return self._h

    def validate(self):
        """Verdict tuple (code, task, counter, aux); code 0 means safe."""
        v = Verdict()
        st = _lib.amk_validate(self._h, ctypes.byref(v))
        if st not in (OK, ERR_UNSAFE_SCHEDULE):
            _check(st, "amk_validate")
        return v.astuple()

    def multistep_check(self):
        """(status, task) of amk_multistep_check: OK and -1 when greedy
        multi-step launches are safe, else the first task that happens-before
        no LM-head task (-2: there is none)."""
        t = _i32()
        st = _lib.amk_multistep_check(self._h, ctypes.byref(t))
        if st not in (OK, ERR_UNSUPPORTED):
            _check(st, "amk_multistep_check")
        return st, t.value

    def view(self):
        """Plain-Python copy of the flat schedule description."""
        d = ScheduleDesc()
        _check(_lib.amk_schedule_view(self._h, ctypes.byref(d)), "amk_schedule_view")
        return desc_to_dict(d)

    @classmethod
    def from_dict(cls, s):
        desc, keep = dict_to_desc(s)
        h = ctypes.c_void_p()
        _check(_lib.amk_schedule_from_desc(ctypes.byref(desc), ctypes.byref(h)), "amk_schedule_from_desc")
        return cls(h.value)

    def close(self):
        if self._h and self._h.value:
            _lib.amk_schedule_free(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _arr(ptr, n, ctype):
    if n == 0:
        return []
    return list((ctype * n).from_address(ctypes.addressof(ptr.contents)))


def desc_to_dict(d):
    nt, ncu, nb = d.n_tasks, d.n_cus, d.n_buffers
    wait_off = _arr(d.wait_off, nt + 1, _i32)
    sig_off = _arr(d.sig_off, nt + 1, _i32)
    acc_off = _arr(d.acc_off, nt + 1, _i32)
    q_off = _arr(d.queue_off, ncu + 1, _i32)
    waits = _arr(d.waits, wait_off[-1], WaitDesc) if wait_off[-1] else []
    sigs = _arr(d.sigs, sig_off[-1], _i32) if sig_off[-1] else []
    accs = _arr(d.accesses, acc_off[-1], AccessDesc) if acc_off[-1] else []
    queue = _arr(d.queue, q_off[-1], _i32) if q_off[-1] else []
    tasks = _arr(d.tasks, nt, TaskDesc)
    bufs = _arr(d.buffers, nb, BufferDesc)
    out = {
        "model": d.model, "config": d.config, "n_counters": d.n_counters,
        "buffers": [(b.size, b.kind) for b in bufs],
        "tasks": [],
        "queues": [queue[q_off[c]:q_off[c + 1]] for c in range(ncu)],
    }
    for i, t in enumerate(tasks):
        out["tasks"].append({
            "type": t.type, "cu": t.cu, "p": list(t.p),
            "waits": [(w.counter, w.threshold) for w in waits[wait_off[i]:wait_off[i + 1]]],
            "sigs": list(sigs[sig_off[i]:sig_off[i + 1]]),
            "acc": [(a.buffer, a.mode, a.begin, a.end) for a in accs[acc_off[i]:acc_off[i + 1]]],
        })
    return out


def dict_to_desc(s):
    """Build an amk_schedule_desc from the plain dict form (arrays kept alive)."""
    tasks = s["tasks"]
    nt = len(tasks)
    T = (TaskDesc * max(nt, 1))()
    wait_off, sig_off, acc_off = [0], [0], [0]
    waits, sigs, accs = [], [], []
    for i, t in enumerate(tasks):
        T[i].type = t["type"]
        T[i].cu = t["cu"]
        p = list(t.get("p", [])) + [0] * (8 - len(t.get("p", [])))
        for k in range(8):
            T[i].p[k] = p[k]
        waits += t.get("waits", [])
        sigs += t.get("sigs", [])
        accs += t.get("acc", [])
        wait_off.append(len(waits))
        sig_off.append(len(sigs))
        acc_off.append(len(accs))
    W = (WaitDesc * max(len(waits), 1))(*[WaitDesc(c, th & 0xFFFFFFFF) for c, th in waits])
    S = (_i32 * max(len(sigs), 1))(*sigs)
    A = (AccessDesc * max(len(accs), 1))(*[AccessDesc(b, m, bg, e) for b, m, bg, e in accs])
    queues = s["queues"]
    q_off = [0]
    flat = []
    for q in queues:
        flat += list(q)
        q_off.append(len(flat))
    Q = (_i32 * max(len(flat), 1))(*flat)
    QO = (_i32 * len(q_off))(*q_off)
    B = (BufferDesc * max(len(s["buffers"]), 1))(*[BufferDesc(sz, k, 0) for sz, k in s["buffers"]])
    WO = (_i32 * len(wait_off))(*wait_off)
    SO = (_i32 * len(sig_off))(*sig_off)
    AO = (_i32 * len(acc_off))(*acc_off)
    d = ScheduleDesc()
    d.model = s.get("model", ModelConfig())
    d.config = s.get("config", ScheduleConfig())
    d.n_tasks = nt
    d.n_counters = s["n_counters"]
    d.n_buffers = len(s["buffers"])
    d.n_cus = len(queues)
    d.tasks = ctypes.cast(T, ctypes.POINTER(TaskDesc))
    d.wait_off = ctypes.cast(WO, ctypes.POINTER(_i32))
    d.waits = ctypes.cast(W, ctypes.POINTER(WaitDesc))
    d.sig_off = ctypes.cast(SO, ctypes.POINTER(_i32))
    d.sigs = ctypes.cast(S, ctypes.POINTER(_i32))
    d.acc_off = ctypes.cast(AO, ctypes.POINTER(_i32))
    d.accesses = ctypes.cast(A, ctypes.POINTER(AccessDesc))
    d.queue_off = ctypes.cast(QO, ctypes.POINTER(_i32))
    d.queue = ctypes.cast(Q, ctypes.POINTER(_i32))
    d.buffers = ctypes.cast(B, ctypes.POINTER(BufferDesc))
    return d, (T, W, S, A, Q, QO, B, WO, SO, AO)


# -------------------------------------------------------------- weights --

def packed_count(model):
    n = _i32()
    _check(_lib.amk_packed_count(ctypes.byref(model), ctypes.byref(n)), "amk_packed_count")
    return n.value


def packed_bytes(model, k):
    n = ctypes.c_size_t()
    _check(_lib.amk_packed_bytes(ctypes.byref(model), k, ctypes.byref(n)), "amk_packed_bytes")
    return n.value


def kv_bytes(model):
    n = ctypes.c_size_t()
    _check(_lib.amk_kv_bytes(ctypes.byref(model), ctypes.byref(n)), "amk_kv_bytes")
    return n.value


def _canon_table(model, canonical):
    n = 3 + 9 * model.n_layers
    tbl = (_p * n)()
    keep = {}
    for k, arr in canonical.items():
        a = np.ascontiguousarray(arr, dtype=np.uint16)
        keep[k] = a
        tbl[k] = a.ctypes.data
    return tbl, keep


def pack_tensor(model, k, canonical, out=None):
    """Packed tensor k (host bytes, numpy uint8) from canonical bf16 tensors."""
    tbl, keep = _canon_table(model, canonical)
    nbytes = packed_bytes(model, k)
    if out is None:
        out = np.empty(nbytes, dtype=np.uint8)
    assert out.nbytes == nbytes and out.flags.c_contiguous
    _check(_lib.amk_pack_tensor(ctypes.byref(model), k, tbl, out.ctypes.data), "amk_pack_tensor")
    return out


def unpack_tensor(model, k, canonical_id, packed, rows, cols):
    """Canonical quantised values of one projection inside packed tensor k."""
    fmt = model.wfmt if k == 2 or (k >= 3 and (k - 3) % 6 in (1, 2, 4, 5)) else W_BF16
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    if fmt == W_BF16:
        q = np.empty((rows, cols), np.uint16)
        s = z = None
    elif fmt == W_INT8_ROW:
        q = np.empty((rows, cols), np.int8)
        s = np.empty(rows, np.float32)
        z = None
    else:
        q = np.empty((rows, cols // 2), np.uint8)
        s = np.empty((rows, cols // 128), np.uint16)
        z = np.empty((rows, cols // 128), np.uint16)
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    _check(_lib.amk_unpack_tensor(ctypes.byref(model), k, canonical_id, packed.ctypes.data,
                                  ptr(q), ptr(s), ptr(z)), "amk_unpack_tensor")
    return q, s, z


# --------------------------------------------------------------- engine --

class Engine:
    """amk_engine over torch-owned device buffers (weights, KV cache, logits)."""

    def __init__(self, schedule, weights, kv_cache, logits, noalloc=False):
        """noalloc: bind with amk_engine_create_noalloc (the library's static
        device scratch instead of allocations)."""
        import torch  # device memory only
        assert all(w.is_cuda for w in weights) and kv_cache.is_cuda and logits.is_cuda
        assert logits.dtype == torch.float32 and logits.is_contiguous()
        self._keep = (schedule, list(weights), kv_cache, logits)
        self._wp = (_p * len(weights))(*[w.data_ptr() for w in weights])
        bufs = DeviceBuffers(ctypes.cast(self._wp, ctypes.POINTER(_p)), len(weights),
                             kv_cache.data_ptr(), ctypes.cast(logits.data_ptr(), ctypes.POINTER(_f32)))
        h = ctypes.c_void_p()
        create = "amk_engine_create_noalloc" if noalloc else "amk_engine_create"
        _check(getattr(_lib, create)(schedule.handle, ctypes.byref(bufs), ctypes.byref(h)), create)
        self._h = h
        self.logits = logits
        self.kv_cache = kv_cache

    def decode_step(self, token, pos, stream=None):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        _check(_lib.amk_decode_step(self._h, int(token), int(pos), ctypes.c_void_p(s.cuda_stream)),
               "amk_decode_step")

    def decode_steps(self, token, pos, n_steps, tokens_out, stream=None):
        """Greedy decode of n_steps tokens in one launch (amk_decode_steps);
        tokens_out: a device int32 tensor of at least n_steps elements."""
        import torch
        assert tokens_out.dtype == torch.int32 and tokens_out.is_cuda and tokens_out.numel() >= n_steps
        s = stream if stream is not None else torch.cuda.current_stream()
        _check(_lib.amk_decode_steps(self._h, int(token), int(pos), int(n_steps),
                                     ctypes.c_void_p(tokens_out.data_ptr()), ctypes.c_void_p(s.cuda_stream)),
               "amk_decode_steps")

    def check(self):
        _check(_lib.amk_engine_check(self._h), "amk_engine_check")

    def launch_empty(self, stream=None):
        """One launch of the decode kernel with every queue empty (the
        cooperative-launch overhead of a step); nothing runs or changes."""
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        _check(_lib.amk_engine_launch_empty(self._h, ctypes.c_void_p(s.cuda_stream)), "amk_engine_launch_empty")

    def set_kv_length(self, n):
        _check(_lib.amk_engine_set_kv_length(self._h, int(n)), "amk_engine_set_kv_length")

    def set_trace(self, enable):
        _check(_lib.amk_engine_set_trace(self._h, int(bool(enable))), "amk_engine_set_trace")

    def read_trace(self, n_tasks):
        """(stamps uint64 [n_tasks][4], clock kHz) of the last traced launch."""
        out = np.empty((n_tasks, 4), dtype=np.uint64)
        khz = _i32()
        _check(_lib.amk_engine_read_trace(self._h, out.ctypes.data, out.size, ctypes.byref(khz)),
               "amk_engine_read_trace")
        return out, khz.value

    def region_stats(self):
        """Per task type of the last traced launch (amk_engine_region_stats):
        {name: {n_tasks, wait_us, work_us, signal_us, span_us}}."""
        out = (RegionStat * TASK_NTYPES)()
        _check(_lib.amk_engine_region_stats(self._h, ctypes.cast(out, _p)), "amk_engine_region_stats")
        return {TASK_NAMES[k]: {f: getattr(out[k], f) for f, _ in RegionStat._fields_}
                for k in range(TASK_NTYPES) if out[k].n_tasks}

    def set_spin_budget(self, microseconds):
        _check(_lib.amk_engine_set_spin_budget(self._h, int(microseconds)), "amk_engine_set_spin_budget")

    def steps(self):
        n = _i64()
        _check(_lib.amk_engine_steps(self._h, ctypes.byref(n)), "amk_engine_steps")
        return n.value

    def close(self):
        if self._h and self._h.value:
            _lib.amk_engine_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def stream_read_probe(src, out, blocks, stream=None):
    """Enqueue one plain streaming read of tensor `src` (see amk.h)."""
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    nbytes = src.numel() * src.element_size()
    _check(_lib.amk_stream_read_probe(ctypes.c_void_p(src.data_ptr()), nbytes - nbytes % 16,
                                      ctypes.c_void_p(out.data_ptr()), int(blocks),
                                      ctypes.c_void_p(s.cuda_stream)), "amk_stream_read_probe")


def upload_model(model, canonical, device="cuda"):
    """Pack every tensor on the host and copy it to device tensors (torch owns them)."""
    import torch
    n = packed_count(model)
    out = []
    for k in range(n):
        host = pack_tensor(model, k, canonical)
        out.append(torch.from_numpy(host).to(device))
    return out


def alloc_state(model, device="cuda"):
    import torch
    kv = torch.zeros(kv_bytes(model) // 2, dtype=torch.int16, device=device)
    logits = torch.zeros(model.vocab, dtype=torch.float32, device=device)
    return kv, logits
