"""ctypes binding of the C ABI in ``include/dg.h`` (argument marshalling only).

The raw functions keep the C names (``dg_create``, ``dg_plan``, ``dg_gemm``,
...).  ``Handle`` wraps a handle and marshals torch tensors (device pointers,
leading dimensions, the current HIP stream) into those calls; every step of
the computation runs in the library's HIP kernels.  There is no fallback: if
``libdg.so`` is missing or fails to load, every call raises.
"""
import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg.so")

# ------------------------------------------------------------------ enums
DG_OK, DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_ALIGNMENT, DG_ERR_NO_CANDIDATE, \
    DG_ERR_CONFLICT, DG_ERR_INVALID_STATE, DG_ERR_WORKSPACE, DG_ERR_HIP, DG_ERR_INTERNAL = range(10)
DG_F16, DG_BF16, DG_F32, DG_I8, DG_I32, DG_E2M1, DG_F8E4M3, DG_E8M0 = range(8)
DG_ROW_MAJOR, DG_COL_MAJOR = 0, 1
DG_EPI_NONE, DG_EPI_BIAS, DG_EPI_GELU_ERF, DG_EPI_BIAS_GELU_ERF, DG_EPI_REQUANT_I8, \
    DG_EPI_REQUANT_F16 = range(6)
DG_UNIT_AUTO, DG_UNIT_MFMA, DG_UNIT_VALU = 0, 1, 2
DG_PATH_AUTO, DG_PATH_TILED, DG_PATH_SKINNY = 0, 1, 2
DG_PROBE_STREAM, DG_PROBE_MFMA, DG_PROBE_LDS, DG_PROBE_MFMA_DATA = 0, 1, 2, 3

EPI = {"none": DG_EPI_NONE, "bias": DG_EPI_BIAS, "gelu_erf": DG_EPI_GELU_ERF,
       "bias_gelu_erf": DG_EPI_BIAS_GELU_ERF, "requant_i8": DG_EPI_REQUANT_I8,
       "requant_f16": DG_EPI_REQUANT_F16}
DTYPE = {"f16": DG_F16, "bf16": DG_BF16, "f32": DG_F32, "i8": DG_I8, "i32": DG_I32,
         "e2m1": DG_E2M1, "f8e4m3": DG_F8E4M3, "e8m0": DG_E8M0}


# ------------------------------------------------------------- structures
class dg_dtypes(C.Structure):
    _fields_ = [("a", C.c_int32), ("b", C.c_int32), ("c", C.c_int32), ("compute", C.c_int32)]


class dg_layouts(C.Structure):
    _fields_ = [("a", C.c_int32), ("b", C.c_int32), ("lda", C.c_int64), ("ldb", C.c_int64),
                ("ldc", C.c_int64), ("ldd", C.c_int64)]


class dg_epilogue(C.Structure):
    _fields_ = [("kind", C.c_int32), ("bias_type", C.c_int32), ("bias", C.c_void_p),
                ("scale", C.c_float)]


class dg_plan_opts(C.Structure):
    _fields_ = [("force_m_tile", C.c_int32), ("force_n_tile", C.c_int32),
                ("force_k_tile", C.c_int32), ("force_split_k", C.c_int32),
                ("force_path", C.c_int32), ("unit", C.c_int32), ("lds_limit_bytes", C.c_int32),
                ("target_occupancy", C.c_float), ("pad_k", C.c_int32),
                ("force_waves", C.c_int32), ("force_mfma", C.c_int32)]

    def __init__(self, **kw):
        super().__init__()
        for k, v in kw.items():
            setattr(self, k, v)


class dg_device_desc(C.Structure):
    _fields_ = [("arch", C.c_char * 32), ("cu_count", C.c_int32), ("xcd_count", C.c_int32),
                ("simd_per_cu", C.c_int32), ("wave_size", C.c_int32),
                ("lds_bytes_per_cu", C.c_int32), ("lds_bytes_per_wg", C.c_int32),
                ("vgpr_per_lane", C.c_int32), ("max_waves_per_simd", C.c_int32),
                ("clock_ghz", C.c_double), ("hbm_gbps", C.c_double),
                ("l2_bytes_per_xcd", C.c_double), ("mall_bytes", C.c_double),
                ("mfma_tflops_f16", C.c_double), ("launch_us", C.c_double),
                ("lds_conflict_stride_words", C.c_int32), ("calibrated", C.c_int32)]


class dg_plan_info(C.Structure):
    _fields_ = [("path", C.c_int32), ("unit", C.c_int32), ("mfma_m", C.c_int32),
                ("mfma_n", C.c_int32), ("mfma_k", C.c_int32), ("m_tile", C.c_int32),
                ("n_tile", C.c_int32), ("k_main", C.c_int32), ("n_main", C.c_int32),
                ("k_tail", C.c_int32), ("n_tail", C.c_int32), ("split_k", C.c_int32),
                ("k_slice", C.c_int32), ("waves_per_wg", C.c_int32), ("lds_bytes", C.c_int32),
                ("vgpr_est", C.c_int32), ("agpr_est", C.c_int32), ("waves_per_simd", C.c_int32),
                ("grid", C.c_int32), ("workspace_bytes", C.c_int64), ("est_us", C.c_double),
                ("est_roof_fraction", C.c_double), ("kernel_id", C.c_int32),
                ("kernel_name", C.c_char * 64)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["kernel_name"] = self.kernel_name.decode()
        return d


EXPORTS = ("dg_create", "dg_create_offline", "dg_default_device_desc", "dg_destroy", "dg_plan",
           "dg_plan_candidates", "dg_plan_range", "dg_gemm", "dg_gemm_noalloc", "dg_gemm_mx", "dg_quant_mx", "dg_set_stage_clock",
           "dg_probe", "dg_set_device_desc", "dg_load_device_json", "dg_get_device_desc", "dg_last_error",
           "dg_status_str")

_lib = None


def load():
    """Load libdg.so (raises if it is missing: there is no other implementation)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with tile_planned_generator_amd.build")
    lib = C.CDLL(LIB_PATH)
    H, P, i64, i32 = C.c_void_p, C.c_void_p, C.c_int64, C.c_int32
    S = C.c_int
    sig = {
        "dg_create": ([C.POINTER(H), C.c_int], S),
        "dg_create_offline": ([C.POINTER(H), C.POINTER(dg_device_desc)], S),
        "dg_default_device_desc": ([C.POINTER(dg_device_desc)], S),
        "dg_destroy": ([H], S),
        "dg_plan": ([H, i64, i64, i64, C.POINTER(dg_dtypes), C.POINTER(dg_layouts), i32, i32,
                     C.POINTER(dg_plan_opts), C.POINTER(dg_plan_info)], S),
        "dg_plan_candidates": ([H, i64, i64, i64, C.POINTER(dg_dtypes), C.POINTER(dg_layouts), i32,
                                i32, C.POINTER(dg_plan_opts), C.POINTER(dg_plan_info), i32,
                                C.POINTER(i32)], S),
        "dg_plan_range": ([H, i64, i64, i64, i64, C.POINTER(dg_dtypes), C.POINTER(dg_layouts), i32, i32,
                           C.POINTER(dg_plan_opts), C.POINTER(dg_plan_opts), C.POINTER(dg_plan_info),
                           C.POINTER(C.c_double)], S),
        "dg_gemm": ([H, i64, i64, i64, C.POINTER(dg_dtypes), C.POINTER(dg_layouts), P, P, P, i32,
                     P, P, P, P, C.POINTER(dg_epilogue), C.POINTER(dg_plan_opts), P, C.c_size_t,
                     P], S),
        "dg_gemm_noalloc": ([H, i64, i64, i64, C.POINTER(dg_dtypes), C.POINTER(dg_layouts), P, P, P, i32,
                             P, P, P, P, C.POINTER(dg_epilogue), C.POINTER(dg_plan_opts), P], S),
        "dg_gemm_mx": ([H, i64, i64, i64, P, i64, P, i64, P, i64, P, i64, P, i32, i64, C.c_float,
                        C.POINTER(dg_epilogue), C.POINTER(dg_plan_opts), P, C.c_size_t, P], S),
        "dg_quant_mx": ([H, i64, i64, P, i64, P, i64, P, i64, P], S),
        "dg_set_stage_clock": ([H, P, i64], S),
        "dg_probe": ([H, i32, P, C.c_size_t, i32, P, i32, P], S),
        "dg_set_device_desc": ([H, C.POINTER(dg_device_desc)], S),
        "dg_load_device_json": ([H, C.c_char_p], S),
        "dg_get_device_desc": ([H, C.POINTER(dg_device_desc)], S),
        "dg_last_error": ([], C.c_char_p),
        "dg_status_str": ([C.c_int], C.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


# raw C names
def dg_create(out, device):
    return load().dg_create(out, device)


def dg_create_offline(out, desc):
    return load().dg_create_offline(out, desc)


def dg_default_device_desc(out):
    return load().dg_default_device_desc(out)


def dg_destroy(h):
    return load().dg_destroy(h)


def dg_plan(*a):
    return load().dg_plan(*a)


def dg_plan_candidates(*a):
    return load().dg_plan_candidates(*a)


def dg_plan_range(*a):
    return load().dg_plan_range(*a)


def dg_gemm(*a):
    return load().dg_gemm(*a)


def dg_load_device_json(*a):
    return load().dg_load_device_json(*a)


def dg_get_device_desc(*a):
    return load().dg_get_device_desc(*a)


def dg_gemm_noalloc(*a):
    return load().dg_gemm_noalloc(*a)


def dg_gemm_mx(*a):
    return load().dg_gemm_mx(*a)


def dg_quant_mx(*a):
    return load().dg_quant_mx(*a)


def dg_set_stage_clock(h, buf, entries):
    return load().dg_set_stage_clock(h, buf, entries)


def dg_probe(h, kind, buf, nbytes, param, out, grid, stream):
    return load().dg_probe(h, kind, buf, nbytes, param, out, grid, stream)


def dg_set_device_desc(h, desc):
    return load().dg_set_device_desc(h, desc)


def dg_last_error():
    return load().dg_last_error().decode()


def dg_status_str(s):
    return load().dg_status_str(s).decode()


class DGError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{dg_status_str(status)}: {msg}")
        self.status = status


def check(status):
    if status != DG_OK:
        raise DGError(status, dg_last_error())


def default_device_desc():
    d = dg_device_desc()
    check(dg_default_device_desc(C.byref(d)))
    return d


# -------------------------------------------------- operand layout helpers
def pack_e2m1(codes_kn):
    """Logical e2m1 codes [K][N] (one per uint8) -> device layout [N][K/2]:
    column n's codes contiguous along K, two per byte, even k in the low nibble."""
    import torch
    t = codes_kn.t().contiguous().to(torch.uint8)          # [N][K]
    return (t[:, 0::2] & 0xF) | ((t[:, 1::2] & 0xF) << 4)


def scales_gn(scale_gn):
    """Logical group scales [K/32][N] -> device layout: group-major rows of N
    rounded up to even (the padding column is zero), contiguous."""
    import torch
    G, N = scale_gn.shape
    if N % 2 == 0:
        return scale_gn.contiguous()
    out = torch.zeros(G, N + 1, dtype=scale_gn.dtype, device=scale_gn.device)
    out[:, :N] = scale_gn
    return out


# ------------------------------------------------------------ torch wrapper
def _dtype_name(t):
    import torch
    return {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32", torch.int8: "i8",
            torch.int32: "i32"}[t.dtype]


class Handle:
    """A library handle.  ``Handle(device)`` opens HIP device ``device``;
    ``Handle(offline=desc)`` plans for a described device without a GPU."""

    def __init__(self, device=None, offline=None):
        self.h = C.c_void_p()
        if offline is not None:
            check(dg_create_offline(C.byref(self.h), C.byref(offline)))
        else:
            check(dg_create(C.byref(self.h), 0 if device is None else int(device)))

    def close(self):
        if self.h:
            check(dg_destroy(self.h))
            self.h = C.c_void_p()

    def set_device_desc(self, desc):
        """Plan with ``desc`` (a dg_device_desc, e.g. probe.load_desc(path)) from now on."""
        check(dg_set_device_desc(self.h, C.byref(desc)))

    def load_device_json(self, path):
        """Plan with the probe's JSON description at ``path`` (dg_load_device_json)."""
        check(dg_load_device_json(self.h, str(path).encode()))

    def device_desc(self):
        """The description the handle plans with (dg_get_device_desc)."""
        d = dg_device_desc()
        check(dg_get_device_desc(self.h, C.byref(d)))
        return d

    def set_stage_clock(self, buf):
        """Record per-workgroup stage clocks of tiled launches into ``buf`` (a
        device uint64/int64 tensor, 8 entries per workgroup), or stop (None)."""
        if buf is None:
            check(dg_set_stage_clock(self.h, None, 0))
        else:
            check(dg_set_stage_clock(self.h, C.c_void_p(buf.data_ptr()), buf.numel()))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def problem(a, b, c, b_layout=DG_ROW_MAJOR, lda=0, ldb=0, ldc=0, ldd=0):
        compute = DG_I32 if DTYPE[a] == DG_I8 else DG_F32
        dt = dg_dtypes(DTYPE[a], DTYPE[b], DTYPE[c], compute)
        lay = dg_layouts(DG_ROW_MAJOR, b_layout, lda, ldb, ldc, ldd)
        return dt, lay

    def quant_mx(self, X, codes, scales, stream=None):
        """MX quantiser through dg_quant_mx: X [M, K] fp16 -> codes [M, K] uint8
        (fp8 e4m3) and scales [K/32, M] uint8 (e8m0, group-major, the layout
        gemm_mx takes); rows may be padded."""
        import torch
        M, K = X.shape
        for t, nm in ((X, "X"), (codes, "codes"), (scales, "scales")):
            if t.dim() != 2 or t.stride(1) != 1:
                raise ValueError(f"{nm} must be a 2-D tensor with unit column stride")
        if stream is None:
            stream = torch.cuda.current_stream(X.device).cuda_stream
        check(dg_quant_mx(self.h, M, K, X.data_ptr(), X.stride(0), codes.data_ptr(), codes.stride(0),
                          scales.data_ptr(), scales.stride(0), stream))

    def gemm_mx(self, A, SA, B, SB, C_out, *, alpha=1.0, bias=None, epilogue="none", K=None,
                opts=None, workspace=None, stream=None, prepared=False):
        """C_out = act(alpha * (A.B) + bias) through dg_gemm_mx (``prepared``: as
        for gemm).

        A: [M, K] uint8 fp8 e4m3 codes; SA: [K/32, >= M] uint8 e8m0 scales,
        group-major; B: [N, K/2] uint8 packed e2m1 codes (pack_e2m1); SB:
        [K/32, >= N] uint8 e8m0 scales, group-major.  Rows may be padded (strides
        are the leading dimensions; scale strides multiples of 4).
        Returns the plan info.
        """
        import torch
        M, K_a = A.shape
        N = B.shape[0]
        K = K_a if K is None else K
        for t, nm in ((A, "A"), (SA, "SA"), (B, "B"), (SB, "SB"), (C_out, "C")):
            if t.dim() != 2 or t.stride(1) != 1:
                raise ValueError(f"{nm} must be a 2-D tensor with unit column stride")
        c = _dtype_name(C_out)
        epi = dg_epilogue(EPI[epilogue], DTYPE[_dtype_name(bias)] if bias is not None else 0,
                          bias.data_ptr() if bias is not None else None, 1.0)
        lda, ldb, ldc = A.stride(0), B.stride(0) * 2, C_out.stride(0)
        info = self.plan(M, N, K, "f8e4m3", "e2m1", c, DG_COL_MAJOR, epilogue, group_k=32, opts=opts,
                         lda=lda, ldb=ldb, ldc=ldc)
        if workspace is None and info.workspace_bytes > 0:
            workspace = torch.empty(info.workspace_bytes, dtype=torch.uint8, device=A.device)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        if stream is None:
            stream = torch.cuda.current_stream(A.device).cuda_stream
        args = (self.h, M, N, K, A.data_ptr(), lda, SA.data_ptr(), SA.stride(0), B.data_ptr(),
                ldb, SB.data_ptr(), SB.stride(0), C_out.data_ptr(), DTYPE[c], ldc, float(alpha),
                C.byref(epi), C.byref(opts) if opts is not None else None, ws_ptr, ws_bytes, stream)
        if prepared:
            return info, _prepared(load().dg_gemm_mx, args, (A, SA, B, SB, C_out, bias, workspace))
        check(dg_gemm_mx(*args))
        return info

    def plan(self, M, N, K, a="f16", b="f16", c="f16", b_layout=None, epilogue="none",
             group_k=0, opts=None, **ld):
        if b_layout is None:
            b_layout = DG_COL_MAJOR if b == "e2m1" else DG_ROW_MAJOR
        dt, lay = self.problem(a, b, c, b_layout, **ld)
        info = dg_plan_info()
        check(dg_plan(self.h, M, N, K, C.byref(dt), C.byref(lay), group_k or (32 if b == "e2m1" else 0),
                      EPI[epilogue], C.byref(opts) if opts is not None else None, C.byref(info)))
        return info

    def plan_range(self, M, N, K_min, K_max, a="f16", b="f16", c="f16", b_layout=None, epilogue="none",
                   group_k=0, opts=None, **ld):
        """dg_plan_range: (options pinning the variant for every K in the range,
        plan info at K_max, worst estimated-time ratio)."""
        if b_layout is None:
            b_layout = DG_COL_MAJOR if b == "e2m1" else DG_ROW_MAJOR
        dt, lay = self.problem(a, b, c, b_layout, **ld)
        ro, info, worst = dg_plan_opts(), dg_plan_info(), C.c_double()
        check(dg_plan_range(self.h, M, N, K_min, K_max, C.byref(dt), C.byref(lay),
                            group_k or (32 if b in ("e2m1",) else 0), EPI[epilogue],
                            C.byref(opts) if opts is not None else None, C.byref(ro), C.byref(info),
                            C.byref(worst)))
        return ro, info, worst.value

    def candidates(self, M, N, K, a="f16", b="f16", c="f16", b_layout=None, epilogue="none",
                   group_k=0, opts=None, cap=64, **ld):
        if b_layout is None:
            b_layout = DG_COL_MAJOR if b == "e2m1" else DG_ROW_MAJOR
        dt, lay = self.problem(a, b, c, b_layout, **ld)
        arr = (dg_plan_info * cap)()
        cnt = C.c_int32()
        check(dg_plan_candidates(self.h, M, N, K, C.byref(dt), C.byref(lay),
                                 group_k or (32 if b == "e2m1" else 0), EPI[epilogue],
                                 C.byref(opts) if opts is not None else None, arr, cap,
                                 C.byref(cnt)))
        return [arr[i] for i in range(min(cap, cnt.value))]

    def gemm(self, A, B, C_out, *, alpha=1.0, beta=0.0, D=None, bias=None, epilogue="none",
             b_scale=None, b_layout=None, K=None, requant_scale=1.0, opts=None, workspace=None,
             stream=None, noalloc=False, prepared=False):
        """C_out = act(alpha * A.B + beta * D + bias) through dg_gemm (through
        dg_gemm_noalloc, with the library's static scratch, when ``noalloc``).
        With ``prepared`` nothing is launched: returns (plan info, a function
        that enqueues the call with its arguments marshalled once).

        A: [M, K] (row-major, rows may be padded: A.stride(0) is lda).
        B: [K, N] row-major, or, with b_layout=DG_COL_MAJOR, [N, K]; for e2m1 the
           packed codes [N, K/2] (uint8) with ``b_scale`` the group-major fp16
           scales of scales_gn ([K/32][N rounded up to even]).
        Returns the plan info.  ``workspace``: a device tensor of at least the
        planned bytes (allocated here when None and the plan needs one).
        """
        import torch
        a = _dtype_name(A)
        e2m1 = B.dtype == torch.uint8
        b = "e2m1" if e2m1 else _dtype_name(B)
        if b_layout is None:
            b_layout = DG_COL_MAJOR if e2m1 else DG_ROW_MAJOR
        c = _dtype_name(C_out)
        M, Ka = A.shape
        if e2m1:
            N = B.shape[0]
            Kk = B.shape[1] * 2
        elif b_layout == DG_COL_MAJOR:
            N, Kk = B.shape
        else:
            Kk, N = B.shape
        K = Ka if K is None else K
        for t, nm in ((A, "A"), (B, "B"), (C_out, "C")):
            if t.dim() != 2 or t.stride(1) != 1:
                raise ValueError(f"{nm} must be a 2-D tensor with unit column stride")
        lda = A.stride(0)
        ldb = B.stride(0) * (2 if e2m1 else 1)
        ldc = C_out.stride(0)
        ldd = D.stride(0) if D is not None else 0
        dt, lay = self.problem(a, b, c, b_layout, lda, ldb, ldc, ldd)
        is_int = a == "i8"
        if is_int:
            al, be = C.c_int32(int(alpha)), C.c_int32(int(beta))
        else:
            al, be = C.c_float(float(alpha)), C.c_float(float(beta))
        epi = dg_epilogue(EPI[epilogue], DTYPE[_dtype_name(bias)] if bias is not None else 0,
                          bias.data_ptr() if bias is not None else None, float(requant_scale))
        if stream is None:
            stream = torch.cuda.current_stream(A.device).cuda_stream
        if noalloc:
            check(dg_gemm_noalloc(self.h, M, N, K, C.byref(dt), C.byref(lay), A.data_ptr(), B.data_ptr(),
                                  b_scale.data_ptr() if b_scale is not None else None, 32 if e2m1 else 0,
                                  D.data_ptr() if D is not None else None, C_out.data_ptr(), C.byref(al),
                                  C.byref(be), C.byref(epi), C.byref(opts) if opts is not None else None,
                                  stream))
            return None
        info = self.plan(M, N, K, a, b, c, b_layout, epilogue, opts=opts, lda=lda, ldb=ldb,
                         ldc=ldc, ldd=ldd)
        if workspace is None and info.workspace_bytes > 0:
            workspace = torch.empty(info.workspace_bytes, dtype=torch.uint8, device=A.device)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        args = (self.h, M, N, K, C.byref(dt), C.byref(lay), A.data_ptr(), B.data_ptr(),
                b_scale.data_ptr() if b_scale is not None else None, 32 if e2m1 else 0,
                D.data_ptr() if D is not None else None, C_out.data_ptr(), C.byref(al),
                C.byref(be), C.byref(epi), C.byref(opts) if opts is not None else None,
                ws_ptr, ws_bytes, stream)
        if prepared:
            return info, _prepared(load().dg_gemm, args, (A, B, C_out, D, bias, b_scale, workspace))
        check(dg_gemm(*args))
        return info


def _prepared(fn, args, keep):
    """A function enqueueing fn(*args); `keep` holds the tensors the arguments
    point into."""
    def call():
        s = fn(*args)
        if s != 0:
            check(s)
    call.keep = keep
    return call


def stage_cycles(rec, wgs):
    """Summarise stage-clock records ([wgs][8] int64, as written by
    dg_set_stage_clock): per-workgroup ticks of the prologue (entry to K-loop
    start), the K loop and the epilogue, as medians and maxima, plus the span
    from the earliest entry to the latest end.  Each die (XCC) counts on its own
    clock, so the span is taken per die and the largest is reported.  The K
    loop's real time comes from the 100 MHz counter in the high halves of
    entries 4 and 5; `k_loop_us` is its median and `tick_ghz` the median rate of
    the s_memtime counter over it (None when the records hold no real time)."""
    import numpy as np
    r = np.asarray(rec, dtype=np.int64).reshape(-1, 8)[:wgs]
    pro, loop, epi = r[:, 1] - r[:, 0], r[:, 2] - r[:, 1], r[:, 3] - r[:, 2]
    out = {}
    for name, v in (("prologue", pro), ("k_loop", loop), ("epilogue", epi)):
        out[name] = {"median": int(np.median(v)), "max": int(v.max())}
    die = r[:, 5] & 0xFFFFFFFF
    out["span"] = int(max(r[die == x, 3].max() - r[die == x, 0].min() for x in np.unique(die)))
    out["k_steps"] = int(np.median(r[:, 6]))
    rt = (((r[:, 5] >> 32) & 0xFFFFFFFF) - ((r[:, 4] >> 32) & 0xFFFFFFFF)) % (1 << 32)
    ok = rt > 0
    out["k_loop_us"] = round(float(np.median(rt[ok])) / 100.0, 3) if ok.any() else None
    out["tick_ghz"] = round(float(np.median(loop[ok] / (rt[ok] * 10.0))), 4) if ok.any() else None
    return out
