"""MI355X-native recurrent core of Sparse Delta Memory (SDM).

Thin Python binding of libsdm.so, whose C ABI is declared in include/sdm.h.
This module only marshals arguments: torch tensors supply device memory and
the current HIP stream, and every step of the computation (selection, state
initialisation, forwarding plan, gated delta write, sparse read) runs in the
library's HIP kernels.  There is no fallback: if libsdm.so is missing or no
GPU is present, the calls raise.

    core = SDM(M0, W=64, R=64)            # M0: [H, N, d_v] float32 on the GPU
    Iw, kw, Ir, qw = core.select(kp, qp)  # kp, qp: [B, T, H, 2*sqrtN]
    y, M = core.forward(kp, qp, v, alpha, beta)
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["SDM", "SDMError", "lib", "lib_path", "F32", "BF16", "FP8_E4M3", "AUTO", "SERIAL", "TIMEPAR",
           "FLAG_CONTINUE", "EXPORTS", "NOALLOC_MAX_BYTES"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsdm.so")
_lib = None

F32, BF16, FP8_E4M3 = 0, 1, 2
AUTO, SERIAL, TIMEPAR = 0, 1, 2
FLAG_CONTINUE = 1
STATUS = {0: "SDM_OK", 1: "SDM_ERR_ARG", 2: "SDM_ERR_UNSUPPORTED", 3: "SDM_ERR_WORKSPACE",
          4: "SDM_ERR_HIP"}

# every function include/sdm.h declares
EXPORTS = ("sdm_backward", "sdm_backward_workspace_size", "sdm_backward_workspace_size_ex",
           "sdm_create", "sdm_create_ex", "sdm_create_fp8",
           "sdm_destroy", "sdm_workspace_size", "sdm_select", "sdm_forward",
           "sdm_forward_noalloc", "sdm_prepare", "sdm_apply", "sdm_write_histogram",
           "sdm_status_string", "sdm_last_error")
NOALLOC_MAX_BYTES = 64 << 20  # SDM_NOALLOC_MAX_BYTES: the static scratch of sdm_forward_noalloc


class SDMError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libsdm (ctypes), with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise SDMError(-1, f"{_LIB_PATH} is not built; run "
                               "`python -m sparse_memory_linear_select_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        p, i, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.sdm_create.argtypes = [p, i, i, i, i, i, ctypes.POINTER(p)]
        L.sdm_create_ex.argtypes = [p, i, i, i, i, i, i, ctypes.POINTER(p)]
        L.sdm_create_fp8.argtypes = [p, i, i, i, i, i, i, ctypes.POINTER(p)]
        L.sdm_destroy.argtypes = [p]
        L.sdm_workspace_size.argtypes = [p, i, i64, i, i, ctypes.POINTER(sz)]
        L.sdm_select.argtypes = [p, i, i64, p, p, i, p, p, p, p, p]
        L.sdm_forward.argtypes = [p, i, i64, p, p, p, p, p, i, i, ctypes.c_uint, p, sz, p, p, p]
        L.sdm_forward_noalloc.argtypes = [p, i, i64, p, p, p, p, p, i, i, ctypes.c_uint, p, p, p]
        L.sdm_prepare.argtypes = [p, i, i64, p, p, p, p, i, i, ctypes.c_uint, p, sz, p, p]
        L.sdm_apply.argtypes = [p, i, i64, p, i, i, p, sz, p, p, p]
        L.sdm_write_histogram.argtypes = [p, i, i64, p, i, p, p]
        L.sdm_backward_workspace_size.argtypes = [p, i, i64, i, ctypes.POINTER(sz)]
        L.sdm_backward_workspace_size_ex.argtypes = [p, i, i64, i, i, ctypes.POINTER(sz)]
        L.sdm_backward.argtypes = [p, i, i64, p, p, p, p, p, i, p, p, p, p, sz, p, p, p, p, p,
                                   p, p, p]
        for f in EXPORTS[:-2]:
            getattr(L, f).restype = ctypes.c_int
        L.sdm_status_string.argtypes = [i]
        L.sdm_status_string.restype = ctypes.c_char_p
        L.sdm_last_error.argtypes = []
        L.sdm_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def variant_name(core, B, T, dtype, variant) -> str:
    """Name of the schedule a call would use ("token-serial" or "time-parallel")."""
    if variant == SERIAL:
        return "token-serial"
    if variant == TIMEPAR or core.state != torch.float32:
        return "time-parallel"
    n_auto = core.workspace_size(B, T, dtype, AUTO)
    return "time-parallel" if n_auto == core.workspace_size(B, T, dtype, TIMEPAR) and \
        n_auto != core.workspace_size(B, T, dtype, SERIAL) else "token-serial"


def _check(status: int):
    if status != 0:
        raise SDMError(status, lib().sdm_last_error().decode())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev_tensor(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise SDMError(1, f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise SDMError(1, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise SDMError(1, f"{name} must be {dtype}, got {t.dtype}")
    return t


def _same_device(t: torch.Tensor, ref: torch.Tensor, name: str):
    if t.device != ref.device:
        raise SDMError(1, f"{name} is on {t.device}, the inputs on {ref.device}")
    return t


def _out_tensor(t, name: str, shape: tuple, dtype, ref: torch.Tensor):
    """A caller-supplied output: a contiguous GPU tensor of exactly this shape
    and dtype on the inputs' device (the kernels write through its pointer)."""
    _dev_tensor(t, name, dtype)
    _same_device(t, ref, name)
    if tuple(t.shape) != tuple(shape):
        raise SDMError(1, f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _workspace(ws, need: int, ref: torch.Tensor):
    """The caller's workspace (a contiguous uint8 GPU tensor on the inputs'
    device with at least `need` bytes), or a new one."""
    if ws is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=ref.device)
    _dev_tensor(ws, "workspace", torch.uint8)
    _same_device(ws, ref, "workspace")
    if ws.numel() < need:
        raise SDMError(3, f"workspace has {ws.numel()} bytes, needs {need}")
    return ws


def _in_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise SDMError(1, f"k', q', v must be float32 or bfloat16, got {t.dtype}")


class SDM:
    """One SDM layer shape bound to its shared initial state M_0 (borrowed).

    state: element type of the state M: torch.float32; torch.bfloat16; or
    torch.float8_e4m3fn, whose codes stand for their value times
    2^state_scale_log2 (M.float() * 2**state_scale_log2 gives the state).
    The narrower states need the time-parallel schedule.
    """

    def __init__(self, M0: torch.Tensor, W: int, R: int, state: torch.dtype = torch.float32,
                 state_scale_log2: int = 0):
        _dev_tensor(M0, "M0", torch.float32)
        if M0.dim() != 3:
            raise SDMError(1, "M0 must be [H, N, d_v]")
        if state not in (torch.float32, torch.bfloat16, torch.float8_e4m3fn):
            raise SDMError(1, "state must be torch.float32, torch.bfloat16 or "
                              f"torch.float8_e4m3fn, got {state}")
        H, N, d_v = M0.shape
        sqrtN = math.isqrt(N)
        if sqrtN * sqrtN != N:
            raise SDMError(1, f"N = {N} is not a perfect square")
        self.M0, self.H, self.sqrtN, self.N, self.d_v = M0, H, sqrtN, N, d_v
        self.W, self.R, self.state = int(W), int(R), state
        self.state_scale_log2 = int(state_scale_log2) if state == torch.float8_e4m3fn else 0
        h = ctypes.c_void_p()
        if state == torch.float8_e4m3fn:
            _check(lib().sdm_create_fp8(_ptr(M0), H, sqrtN, d_v, self.W, self.R,
                                        self.state_scale_log2, ctypes.byref(h)))
        else:
            _check(lib().sdm_create_ex(_ptr(M0), H, sqrtN, d_v, self.W, self.R,
                                       BF16 if state == torch.bfloat16 else F32, ctypes.byref(h)))
        self._h = h

    def state_values(self, M: torch.Tensor) -> torch.Tensor:
        """The float32 values a state tensor M of this layer holds."""
        if self.state == torch.float8_e4m3fn:
            return M.float() * (2.0 ** self.state_scale_log2)
        return M.float()

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().sdm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, B: int, T: int, dtype: int = F32, variant: int = AUTO) -> int:
        n = ctypes.c_size_t()
        _check(lib().sdm_workspace_size(self._h, B, T, dtype, variant, ctypes.byref(n)))
        return n.value

    def _shape_in(self, x: torch.Tensor, last: int, name: str):
        if x.dim() != 4 or x.shape[2] != self.H or x.shape[3] != last:
            raise SDMError(1, f"{name} must be [B, T, {self.H}, {last}], got {tuple(x.shape)}")
        return x.shape[0], x.shape[1]

    def select(self, kp: torch.Tensor, qp: torch.Tensor, out=None):
        """(Iw, kw, Ir, qw): write/read slots ([B,T,H,W|R] int32) and softmax weights."""
        _dev_tensor(kp, "kp")
        _dev_tensor(qp, "qp")
        B, T = self._shape_in(kp, 2 * self.sqrtN, "kp")
        if qp.shape != kp.shape or qp.dtype != kp.dtype:
            raise SDMError(1, "qp must match kp in shape and dtype")
        dev = kp.device
        _same_device(qp, kp, "qp")
        shp_w, shp_r = (B, T, self.H, self.W), (B, T, self.H, self.R)
        if out is None:
            Iw = torch.empty(shp_w, dtype=torch.int32, device=dev)
            kw = torch.empty(shp_w, dtype=torch.float32, device=dev)
            Ir = torch.empty(shp_r, dtype=torch.int32, device=dev)
            qw = torch.empty(shp_r, dtype=torch.float32, device=dev)
        else:
            Iw, kw, Ir, qw = out
            _out_tensor(Iw, "Iw", shp_w, torch.int32, kp)
            _out_tensor(kw, "kw", shp_w, torch.float32, kp)
            _out_tensor(Ir, "Ir", shp_r, torch.int32, kp)
            _out_tensor(qw, "qw", shp_r, torch.float32, kp)
        _check(lib().sdm_select(self._h, B, T, _ptr(kp), _ptr(qp), _in_dtype(kp), _ptr(Iw),
                                _ptr(kw), _ptr(Ir), _ptr(qw), _stream(dev)))
        return Iw, kw, Ir, qw

    def write_histogram(self, kp: torch.Tensor, counts: torch.Tensor | None = None):
        """Per head and slot, how many head-tokens wrote the slot ([H, N] int32 view of
        uint32 counts).  `counts` (if given) is accumulated into."""
        _dev_tensor(kp, "kp")
        B, T = self._shape_in(kp, 2 * self.sqrtN, "kp")
        if counts is None:
            counts = torch.zeros((self.H, self.N), dtype=torch.int32, device=kp.device)
        _out_tensor(counts, "counts", (self.H, self.N), torch.int32, kp)
        _check(lib().sdm_write_histogram(self._h, B, T, _ptr(kp), _in_dtype(kp), _ptr(counts),
                                         _stream(kp.device)))
        return counts

    def backward_workspace_size(self, B: int, T: int, dtype: int = F32, chunks: int = 0) -> int:
        """Bytes of workspace for sdm_backward run in `chunks` chunks of epochs
        (0: the least memory; 1: the whole sequence at once, the fastest)."""
        n = ctypes.c_size_t()
        _check(lib().sdm_backward_workspace_size_ex(self._h, B, T, dtype, chunks,
                                                    ctypes.byref(n)))
        return n.value

    def backward(self, kp, qp, v, alpha, beta, dy, dMT=None, Minit=None, workspace=None,
                  dM0: bool = True, chunks: int = 0) -> dict:
        """Gradients of the core for upstream gradients dy [B,T,H,d_v] (and dMT
        [B,H,N,d_v], None = zero), with the selections held fixed.  Minit is the
        state the forward started from (None: M_0).  Without a workspace, one
        for `chunks` chunks is allocated (0: the least memory).  Returns float32
        dkp, dqp [B,T,H,2 sqrtN], dv [B,T,H,d_v], dalpha, dbeta [B,T,H], dMinit
        [B,H,N,d_v] and (dM0=True) dM0 [H,N,d_v]."""
        for t, nm in ((kp, "kp"), (qp, "qp"), (v, "v")):
            _dev_tensor(t, nm)
        _dev_tensor(alpha, "alpha", torch.float32)
        _dev_tensor(beta, "beta", torch.float32)
        _dev_tensor(dy, "dy", torch.float32)
        B, T = self._shape_in(kp, 2 * self.sqrtN, "kp")
        if qp.shape != kp.shape or qp.dtype != kp.dtype or v.dtype != kp.dtype:
            raise SDMError(1, "kp, qp and v must share one dtype (and kp, qp one shape)")
        if tuple(v.shape) != (B, T, self.H, self.d_v) or tuple(dy.shape) != tuple(v.shape):
            raise SDMError(1, "v and dy must be [B, T, H, d_v]")
        if tuple(alpha.shape) != (B, T, self.H) or tuple(beta.shape) != (B, T, self.H):
            raise SDMError(1, "alpha and beta must be [B, T, H]")
        sshape = (B, self.H, self.N, self.d_v)
        for t, nm in ((qp, "qp"), (v, "v"), (alpha, "alpha"), (beta, "beta"), (dy, "dy"),
                      (self.M0, "M0")):
            _same_device(t, kp, nm)
        for t, nm in ((dMT, "dMT"), (Minit, "Minit")):
            if t is not None:
                _out_tensor(t, nm, sshape, torch.float32, kp)
        dev = kp.device
        dt = _in_dtype(kp)
        need = self.backward_workspace_size(B, T, dt, 0)
        if workspace is None:
            need = self.backward_workspace_size(B, T, dt, chunks)
        workspace = _workspace(workspace, need, kp)
        f32 = dict(dtype=torch.float32, device=dev)
        out = dict(dkp=torch.empty((B, T, self.H, 2 * self.sqrtN), **f32),
                   dqp=torch.empty((B, T, self.H, 2 * self.sqrtN), **f32),
                   dv=torch.empty((B, T, self.H, self.d_v), **f32),
                   dalpha=torch.empty((B, T, self.H), **f32), dbeta=torch.empty((B, T, self.H), **f32),
                   dMinit=torch.empty(sshape, **f32))
        if dM0:
            out["dM0"] = torch.empty((self.H, self.N, self.d_v), **f32)
        _check(lib().sdm_backward(
            self._h, B, T, _ptr(kp), _ptr(qp), _ptr(v), _ptr(alpha), _ptr(beta), dt, _ptr(Minit),
            _ptr(dy), _ptr(dMT), _ptr(workspace), workspace.numel(), _ptr(out["dkp"]),
            _ptr(out["dqp"]), _ptr(out["dv"]), _ptr(out["dalpha"]), _ptr(out["dbeta"]),
            _ptr(out["dMinit"]), _ptr(out.get("dM0")), _stream(dev)))
        return out

    def _forward_args(self, kp, qp, v, alpha, beta, y, M, cont):
        """Validated (B, T, input dtype code, y, M) of a forward call."""
        for t, n in ((kp, "kp"), (qp, "qp"), (v, "v")):
            _dev_tensor(t, n)
        _dev_tensor(alpha, "alpha", torch.float32)
        _dev_tensor(beta, "beta", torch.float32)
        B, T = self._shape_in(kp, 2 * self.sqrtN, "kp")
        if qp.shape != kp.shape or qp.dtype != kp.dtype or v.dtype != kp.dtype:
            raise SDMError(1, "kp, qp and v must share one dtype (and kp, qp one shape)")
        if tuple(v.shape) != (B, T, self.H, self.d_v):
            raise SDMError(1, f"v must be [B, T, H, d_v], got {tuple(v.shape)}")
        if tuple(alpha.shape) != (B, T, self.H) or tuple(beta.shape) != (B, T, self.H):
            raise SDMError(1, "alpha and beta must be [B, T, H]")
        for t, n in ((qp, "qp"), (v, "v"), (alpha, "alpha"), (beta, "beta"), (self.M0, "M0")):
            _same_device(t, kp, n)
        dev = kp.device
        if y is None:
            y = torch.empty((B, T, self.H, self.d_v), dtype=torch.float32, device=dev)
        if M is None:
            if cont:
                raise SDMError(1, "cont=True needs the state M")
            M = torch.empty((B, self.H, self.N, self.d_v), dtype=self.state, device=dev)
        _out_tensor(y, "y", (B, T, self.H, self.d_v), torch.float32, kp)
        _out_tensor(M, "M", (B, self.H, self.N, self.d_v), self.state, kp)
        return B, T, _in_dtype(kp), y, M

    def forward_noalloc(self, kp, qp, v, alpha, beta, y, M, variant: int = AUTO,
                        cont: bool = False):
        """sdm_forward_noalloc: as forward(), with the library's static scratch
        in place of a workspace, so the call allocates no device memory (y and
        M are the caller's).  For callers that cannot allocate: HIP graph
        capture, serving loops.  Raises SDMError (SDM_ERR_UNSUPPORTED) when the
        call needs more than NOALLOC_MAX_BYTES of scratch; calls that overlap
        on one GPU share the scratch and race."""
        B, T, dt, y, M = self._forward_args(kp, qp, v, alpha, beta, y, M, cont)
        flags = FLAG_CONTINUE if cont else 0
        _check(lib().sdm_forward_noalloc(self._h, B, T, _ptr(kp), _ptr(qp), _ptr(v), _ptr(alpha),
                                         _ptr(beta), dt, variant, flags, _ptr(y), _ptr(M),
                                         _stream(kp.device)))
        return y, M

    def forward(self, kp, qp, v, alpha, beta, variant: int = AUTO, y=None, M=None,
                workspace=None, cont: bool = False, staged: bool = False):
        """(y, M): outputs [B,T,H,d_v] and final state [B,H,N,d_v] (float32).

        With cont=True, M must hold the state to continue from (no M <- M_0).
        staged=True issues sdm_prepare + sdm_apply instead of sdm_forward
        (the same results on the same stream; for one token per sequence
        sdm_forward runs the whole step as one launch).
        """
        B, T, dt, y, M = self._forward_args(kp, qp, v, alpha, beta, y, M, cont)
        dev = kp.device
        workspace = _workspace(workspace, self.workspace_size(B, T, dt, variant), kp)
        flags = FLAG_CONTINUE if cont else 0
        if staged:
            _check(lib().sdm_prepare(self._h, B, T, _ptr(kp), _ptr(qp), _ptr(alpha), _ptr(beta),
                                     dt, variant, flags, _ptr(workspace), workspace.numel(),
                                     _ptr(M), _stream(dev)))
            _check(lib().sdm_apply(self._h, B, T, _ptr(v), dt, variant, _ptr(workspace),
                                   workspace.numel(), _ptr(y), _ptr(M), _stream(dev)))
            return y, M
        _check(lib().sdm_forward(self._h, B, T, _ptr(kp), _ptr(qp), _ptr(v), _ptr(alpha),
                                 _ptr(beta), dt, variant, flags, _ptr(workspace),
                                 workspace.numel(), _ptr(y), _ptr(M), _stream(dev)))
        return y, M
