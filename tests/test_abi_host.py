"""The C ABI on the CPU: the libraries load, export every declared symbol, and
validate arguments exactly as documented, all without touching a device
(ccv_fwd_check / ccv_fwd_plan never dereference the pointers they are given)."""
import ctypes
import os
import re
import subprocess

import pytest

import causal_depthwise_conv1d_amd as ccv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = {"ccv.h": ccv.LIB_PATH, "ccv_calib.h": ccv.CALIB_LIB_PATH}


def declared_functions(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ccv_\w+)\s*\(", text, flags=re.M)


def test_every_header_is_covered():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == sorted(HEADERS)


@pytest.mark.parametrize("header", sorted(HEADERS))
def test_library_exports_every_declared_symbol(header):
    names = declared_functions(header)
    assert names, header
    lib = ctypes.CDLL(HEADERS[header])
    dyn = subprocess.run(["nm", "-D", "--defined-only", HEADERS[header]], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\S+)$", dyn, flags=re.M))
    for n in names:
        assert n in exported, (header, n)
        getattr(lib, n)


def test_abi_version_and_status_names():
    assert ccv.ccv_abi_version() == ccv.CCV_ABI_VERSION == 1
    for code, name in ccv.STATUS.items():
        assert ccv.ccv_status_str(code) == name
    assert ccv.ccv_status_str(12345) == "CCV_E_UNKNOWN"


# Fake, never-dereferenced device addresses (16-byte aligned unless stated).
X, W, BIAS, SEQ, INIT, FIN, OUT = (0x100000 * (i + 1) for i in range(7))


def args(B=2, C=64, L=1000, K=4, layout="cf", **over):
    a = ccv.ccv_fwd_args_t()
    a.B, a.C, a.L, a.K = B, C, L, K
    a.x_dtype = a.w_dtype = ccv.CCV_BF16
    a.activation = ccv.CCV_ACT_SILU
    a.x, a.weight, a.out = X, W, OUT
    st = (C * L, L, 1) if layout == "cf" else (L * C, 1, C)
    a.x_stride = type(a.x_stride)(*st)
    a.out_stride = type(a.out_stride)(*st)
    for k, v in over.items():
        if k.endswith("stride"):
            v = type(getattr(a, k))(*v)
        setattr(a, k, v)
    return a


def check(a):
    return ccv.STATUS[ccv.ccv_fwd_check(a)]


def test_valid_calls():
    assert check(args()) == "CCV_OK"
    assert check(args(layout="cl")) == "CCV_OK"
    assert check(args(bias=BIAS, seq_idx=SEQ)) == "CCV_OK"
    assert check(args(initial_states=INIT, init_stride=(64 * 3, 1, 64),
                      final_states_out=FIN, final_stride=(64 * 3, 1, 64))) == "CCV_OK"


def test_struct_size_mismatch():
    a = args()
    a.struct_size = 8
    assert check(a) == "CCV_E_ABI"


def test_shapes_and_k():
    assert check(args(B=-1)) == "CCV_E_SHAPE"
    assert check(args(L=-5)) == "CCV_E_SHAPE"
    assert check(args(C=2**31)) == "CCV_E_SHAPE"
    for K in (0, 1, 5, 8):
        assert check(args(K=K)) == "CCV_E_KSIZE"
    assert check(args(x_stride=(2**62, 1000, 1))) == "CCV_E_SHAPE"      # offsets overflow


def test_dtypes_and_activation():
    assert check(args(x_dtype=3)) == "CCV_E_DTYPE"
    assert check(args(w_dtype=-1)) == "CCV_E_DTYPE"
    assert check(args(activation=2)) == "CCV_E_UNSUPPORTED"


def test_null_pointers():
    assert check(args(x=None)) == "CCV_E_NULL"
    assert check(args(weight=None)) == "CCV_E_NULL"
    assert check(args(out=None)) == "CCV_E_NULL"
    assert ccv.lib().ccv_fwd_check(None) == -1


def test_seq_idx_with_states_is_accepted():
    # lifted version limit: the history is the first sequence's, final states the last's
    assert check(args(seq_idx=SEQ, initial_states=INIT, init_stride=(192, 1, 64))) == "CCV_OK"
    assert check(args(seq_idx=SEQ, final_states_out=FIN, final_stride=(192, 1, 64))) == "CCV_OK"


def test_aliasing():
    assert check(args(out=X)) == "CCV_E_ALIAS"
    assert check(args(initial_states=INIT, final_states_out=INIT, init_stride=(192, 1, 64),
                      final_stride=(192, 1, 64))) == "CCV_E_ALIAS"


def test_final_states_aliasing_x_or_out():
    fs = dict(final_states_out=X, final_stride=(192, 1, 64))
    assert check(args(**fs)) == "CCV_E_ALIAS"
    fs["final_states_out"] = OUT
    assert check(args(**fs)) == "CCV_E_ALIAS"
    # with L = 0 nothing of out is written, so only x is compared
    assert check(args(L=0, out=FIN, final_states_out=FIN, final_stride=(192, 1, 64))) == "CCV_OK"


def test_written_layouts_must_not_overlap():
    # out with a zero stride, or time steps landing on the next channel's elements
    assert check(args(out_stride=(64000, 0, 1))) == "CCV_E_LAYOUT"
    assert check(args(out_stride=(64000, 500, 1))) == "CCV_E_LAYOUT"
    assert check(args(layout="cl", out_stride=(64000, 1, 32))) == "CCV_E_LAYOUT"
    # final states whose entries of two channels coincide
    assert check(args(final_states_out=FIN, final_stride=(192, 0, 64))) == "CCV_E_LAYOUT"
    assert check(args(final_states_out=FIN, final_stride=(192, 2, 1))) == "CCV_E_LAYOUT"
    # a padded pitch is fine
    assert check(args(out_stride=(70000, 1024, 1))) == "CCV_OK"


def test_batch_times_channels_overflow():
    # zero batch and channel strides keep every offset small, but B*C overflows int64
    assert check(args(B=2**40, C=2**30, L=4, x_stride=(0, 0, 1))) == "CCV_E_SHAPE"


def test_layouts():
    # neither time nor channels unit-stride: the caller must copy
    assert check(args(x_stride=(64 * 1000 * 2, 2000, 2))) == "CCV_E_LAYOUT"
    # out unit-stride in the other dimension than x
    assert check(args(out_stride=(64000, 1, 64))) == "CCV_E_LAYOUT"
    assert check(args(x_stride=(64000, 1000, -1))) == "CCV_E_LAYOUT"
    # a slice of a wider channel-last buffer (s_L > C) is accepted as is
    assert check(args(layout="cl", x_stride=(1000 * 10240, 1, 10240))) == "CCV_OK"


def test_nothing_to_do_needs_no_pointers():
    for B, C, L in ((0, 4, 8), (2, 0, 8), (2, 4, 0)):
        a = args(B=B, C=C, L=L, x=None, weight=None, out=None)
        assert check(a) == "CCV_OK"
        st, p = ccv.ccv_fwd_plan(a)
        assert st == 0 and p.path == ccv.CCV_PATH_NONE


def test_empty_sequence_still_writes_final_states():
    a = args(L=0, x=None, weight=None, out=None, initial_states=INIT, init_stride=(192, 3, 1),
             final_states_out=FIN, final_stride=(192, 3, 1))
    st, p = ccv.ccv_fwd_plan(a)
    assert st == 0 and p.path != ccv.CCV_PATH_NONE and p.grid > 0


def test_plan_channel_first():
    st, p = ccv.ccv_fwd_plan(args(B=4, C=2048, L=4096))
    assert st == 0
    assert p.path == ccv.CCV_PATH_CHANNEL_FIRST and p.vector == 1 and p.elems_per_lane == 8
    seg = 64 * 8 * p.unroll                   # one wave-wide pass of 16-byte vectors
    assert p.span % seg == 0                  # a work item is a run of whole segments
    assert p.work_items == 4 * 2048 * -(-4096 // p.span)
    # bf16 + SiLU: a grid of 16 waves per CU (256 CUs), each walking several segments
    assert p.grid * p.waves_per_group == min(p.work_items, 256 * 16)


def test_plan_channel_first_short_last_segments_get_workgroups_of_their_own():
    # L not a multiple of the span: the whole segments keep their grid (16 waves per
    # CU for bf16 + SiLU), and one wave per row, in workgroups appended to the grid,
    # takes the row's last, shorter segment.
    rows = 4 * 2048
    _, p = ccv.ccv_fwd_plan(args(B=4, C=2048, L=4097))
    assert p.vector == 1 and p.work_items == rows * 3
    assert p.grid == min(rows * 2, 256 * 16) // p.waves_per_group + rows // p.waves_per_group
    # rows shorter than a span: only the appended workgroups
    a = args(B=8, C=1024, L=1001, activation=ccv.CCV_ACT_NONE)
    a.x_dtype = a.w_dtype = ccv.CCV_F32
    _, p = ccv.ccv_fwd_plan(a)
    assert p.span == 1024 and p.grid == 8 * 1024 // p.waves_per_group


def test_plan_grid_follows_the_cu_count_override(monkeypatch):
    # No launch has run in this process, so plans size the grid for 256 CUs;
    # CCV_CU_COUNT replaces the count (a partitioned or smaller part).
    _, p = ccv.ccv_fwd_plan(args(B=4, C=2048, L=4096))
    assert p.grid * p.waves_per_group == 256 * 16
    monkeypatch.setenv("CCV_CU_COUNT", "32")
    _, p = ccv.ccv_fwd_plan(args(B=4, C=2048, L=4096))
    assert p.grid * p.waves_per_group == 32 * 16
    monkeypatch.setenv("CCV_CU_COUNT", "0")              # not a count: ignored
    _, p = ccv.ccv_fwd_plan(args(B=4, C=2048, L=4096))
    assert p.grid * p.waves_per_group == 256 * 16


def test_plan_channel_first_light_calls_get_a_wave_per_segment():
    a = args(B=2, C=128, L=1 << 16, activation=ccv.CCV_ACT_NONE)
    a.x_dtype = a.w_dtype = ccv.CCV_F32
    st, p = ccv.ccv_fwd_plan(a)
    assert st == 0 and p.grid == -(-p.work_items // p.waves_per_group)


def test_plan_channel_first_long_rows_are_split():
    # 256 rows of 1M fp32 steps: many runs per row, each a whole number of segments
    a = args(B=2, C=128, L=1 << 20, x_dtype=ccv.CCV_F32)
    a.x_dtype = ccv.CCV_F32
    st, p = ccv.ccv_fwd_plan(a)
    assert st == 0 and p.path == ccv.CCV_PATH_CHANNEL_FIRST
    seg = 64 * 4 * p.unroll
    assert p.span % seg == 0 and p.span < (1 << 20)
    assert p.work_items == 256 * -(-(1 << 20) // p.span)
    assert p.work_items >= 16 * 256


def test_plan_channel_last_strided_view():
    st, p = ccv.ccv_fwd_plan(args(B=8, C=4096, L=8192, layout="cl", x_stride=(8192 * 10240, 1, 10240)))
    assert st == 0
    assert p.path == ccv.CCV_PATH_CHANNEL_LAST and p.vector == 1
    assert p.channels_per_item == 512
    assert p.work_items == 8 * (4096 // 512) * -(-8192 // p.span)


def test_plan_channel_last_lds_forms(monkeypatch):
    """CCV_CL_LDS picks the LDS-staged tile (1: 16 rows of 64 * V channels per wave)
    or the transposing tile (2: 256 channels by 64 rows for 16-bit data, one
    workgroup per item); an unaligned layout or an unknown value keeps the register
    tiles (32 rows)."""
    view = dict(B=8, C=4096, L=8192, layout="cl", x_stride=(8192 * 10240, 1, 10240))
    _, p0 = ccv.ccv_fwd_plan(args(**view))
    assert (p0.span, p0.channels_per_item) == (32, 512)
    monkeypatch.setenv("CCV_CL_LDS", "1")
    _, p = ccv.ccv_fwd_plan(args(**view))
    assert (p.span, p.unroll, p.channels_per_item, p.vector) == (16, 16, 512, 1)
    assert p.work_items == 8 * 8 * (8192 // 16)
    monkeypatch.setenv("CCV_CL_LDS", "2")
    _, p = ccv.ccv_fwd_plan(args(**view))
    assert (p.span, p.channels_per_item) == (64, 256)
    assert p.work_items == 8 * (4096 // 256) * (8192 // 64) == p.grid     # a workgroup per item
    _, p = ccv.ccv_fwd_plan(args(layout="cl", x_stride=(1000 * 67, 1, 67)))
    assert (p.vector, p.channels_per_item) == (1, 64 * 8)                    # unaligned rows: registers
    monkeypatch.setenv("CCV_CL_LDS", "7")
    _, p = ccv.ccv_fwd_plan(args(**view))
    assert (p.span, p.channels_per_item) == (p0.span, p0.channels_per_item)


def test_plan_channel_last_unaligned_rows_keep_16_byte_accesses(monkeypatch):
    # channel offset 3 in a bf16 buffer (base not 16-byte aligned) and an odd time
    # stride (every row after the first unaligned): whole channel vectors still take
    # 16-byte accesses; the LDS-staged forms need aligned rows and fall back to the
    # register tiles; CCV_FORCE_SCALAR selects the element path
    for kw in (dict(x=X + 6, x_stride=(1000 * 72, 1, 72)), dict(x_stride=(1000 * 67, 1, 67))):
        _, p = ccv.ccv_fwd_plan(args(layout="cl", **kw))
        assert p.vector == 1 and p.span == 32, kw
        for lds in ("1", "2"):
            monkeypatch.setenv("CCV_CL_LDS", lds)
            _, p = ccv.ccv_fwd_plan(args(layout="cl", **kw))
            assert p.vector == 1 and p.span == 32 and p.channels_per_item == 64 * 8, (kw, lds)
        monkeypatch.delenv("CCV_CL_LDS")
    monkeypatch.setenv("CCV_FORCE_SCALAR", "1")
    _, p = ccv.ccv_fwd_plan(args(layout="cl", x_stride=(1000 * 67, 1, 67)))
    assert p.vector == 0


def test_channel_first_takes_16_byte_accesses_at_any_alignment(monkeypatch):
    # Channel-first rows of any length and offset take the 16-byte path (the GPU
    # serves unaligned 16-byte accesses; the vector that straddles L goes element
    # by element); only CCV_FORCE_SCALAR selects the element path.
    for kw in (dict(x_stride=(64 * 1001, 1001, 1)), dict(seq_idx=SEQ + 4), dict(seq_idx=SEQ, L=1002),
               dict(x=X + 6), dict(L=3, x_stride=(192, 3, 1), out_stride=(192, 3, 1))):
        _, p = ccv.ccv_fwd_plan(args(layout="cf", **kw))
        assert p.path == ccv.CCV_PATH_CHANNEL_FIRST and p.vector == 1, kw
    monkeypatch.setenv("CCV_FORCE_SCALAR", "1")
    _, p = ccv.ccv_fwd_plan(args(layout="cf", x_stride=(64 * 1001, 1001, 1)))
    assert p.vector == 0


def test_size_one_dims_take_either_stride():
    # L == 1: any time stride; C == 1: any channel stride
    assert check(args(L=1, x_stride=(64, 1, 999), out_stride=(64, 1, 7))) == "CCV_OK"
    assert check(args(C=1, layout="cl", x_stride=(1000, 77, 1), out_stride=(1000, 5, 1))) == "CCV_OK"


def test_wrapper_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 8)
    w = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        ccv.causal_conv1d_fwd(x, w)


# ---- update (decode) -----------------------------------------------------------------

def uargs(B=2, C=64, L=1, K=4, state_layout="bci", **over):
    a = ccv.ccv_update_args_t()
    a.B, a.C, a.L, a.K = B, C, L, K
    a.x_dtype = a.w_dtype = ccv.CCV_BF16
    a.activation = ccv.CCV_ACT_SILU
    a.x, a.weight, a.state, a.out = X, W, INIT, OUT
    a.x_stride = type(a.x_stride)(C * L, L, 1)
    a.out_stride = type(a.out_stride)(C * L, L, 1)
    H = K - 1
    st = (C * H, H, 1) if state_layout == "bci" else (H * C, 1, C)
    a.state_stride = type(a.state_stride)(*st)
    for k, v in over.items():
        if k.endswith("stride"):
            v = type(getattr(a, k))(*v)
        setattr(a, k, v)
    return a


def ucheck(a):
    return ccv.STATUS[ccv.ccv_update_check(a)]


def test_update_valid_calls():
    assert ucheck(uargs()) == "CCV_OK"
    assert ucheck(uargs(state_layout="bic")) == "CCV_OK"
    assert ucheck(uargs(L=5, bias=BIAS, activation=ccv.CCV_ACT_NONE)) == "CCV_OK"
    # channel-last new steps and a state that is a slice of a longer per-row buffer
    assert ucheck(uargs(L=3, x_stride=(3 * 64, 1, 64), out_stride=(3 * 64, 1, 64),
                        state_stride=(64 * 8, 8, 1))) == "CCV_OK"
    # any dtype pair
    assert ucheck(uargs(x_dtype=ccv.CCV_F32, w_dtype=ccv.CCV_F16)) == "CCV_OK"


def test_update_argument_errors():
    a = uargs()
    a.struct_size = 8
    assert ucheck(a) == "CCV_E_ABI"
    assert ucheck(uargs(B=-1)) == "CCV_E_SHAPE"
    assert ucheck(uargs(L=-1)) == "CCV_E_SHAPE"
    for K in (1, 5):
        assert ucheck(uargs(K=K)) == "CCV_E_KSIZE"
    assert ucheck(uargs(x_dtype=7)) == "CCV_E_DTYPE"
    assert ucheck(uargs(activation=3)) == "CCV_E_UNSUPPORTED"
    for name in ("x", "weight", "state", "out"):
        assert ucheck(uargs(**{name: None})) == "CCV_E_NULL", name
    assert ccv.lib().ccv_update_check(None) == -1
    assert ucheck(uargs(state=X)) == "CCV_E_ALIAS"
    assert ucheck(uargs(out=X)) == "CCV_E_ALIAS"
    assert ucheck(uargs(state=OUT)) == "CCV_E_ALIAS"
    assert ucheck(uargs(state_stride=(192, 3, -1))) == "CCV_E_LAYOUT"
    assert ucheck(uargs(x_stride=(2**62, 1, 1), B=4)) == "CCV_E_SHAPE"


def test_update_written_layouts_must_not_overlap():
    # every batch row of the state at one address
    assert ucheck(uargs(state_stride=(0, 3, 1))) == "CCV_E_LAYOUT"
    # channels and history steps interleaved onto the same elements
    assert ucheck(uargs(state_stride=(192, 1, 1))) == "CCV_E_LAYOUT"
    assert ucheck(uargs(state_stride=(192, 2, 1))) == "CCV_E_LAYOUT"
    # out with two steps on one element
    assert ucheck(uargs(L=2, out_stride=(128, 2, 0))) == "CCV_E_LAYOUT"
    # x may overlap itself (it is only read): a broadcast input is fine
    assert ucheck(uargs(L=2, x_stride=(0, 1, 0))) == "CCV_OK"
    # size-1 dimensions never overlap, whatever their stride
    assert ucheck(uargs(B=1, state_stride=(0, 3, 1))) == "CCV_OK"


def test_update_nothing_to_do_needs_no_pointers():
    for B, C, L in ((0, 4, 1), (2, 0, 1), (2, 4, 0)):
        assert ucheck(uargs(B=B, C=C, L=L, x=None, weight=None, state=None, out=None)) == "CCV_OK"


def test_update_wrapper_refuses_cpu_tensors():
    import torch
    x = torch.zeros(2, 4)
    with pytest.raises(ValueError):
        ccv.causal_conv1d_update(x, torch.zeros(2, 4, 3), torch.zeros(4, 4))


def uplan(a):
    st, p = ccv.ccv_update_plan(a)
    assert st == 0, ccv.STATUS[st]
    return p


def test_update_plan_takes_16_byte_path_on_standard_layouts():
    p = uplan(uargs(B=4, C=512))                     # x [B, C], state [B, C, K-1] contiguous
    assert p.path == ccv.CCV_PATH_UPDATE and p.vector == 1 and p.elems_per_lane == 8
    assert p.grid == -(-4 * 512 // (256 * 8)) and p.work_items == 4 * 512
    p = uplan(uargs(C=64, L=3, x_stride=(3 * 64, 1, 64), out_stride=(3 * 64, 1, 64)))
    assert p.vector == 1                             # channel-last steps
    a = uargs(C=64)
    a.x_dtype = a.w_dtype = ccv.CCV_F32
    p = uplan(a)
    assert p.vector == 1 and p.elems_per_lane == 4


def test_update_plan_falls_back_to_element_path():
    assert uplan(uargs(state_layout="bic")).vector == 0            # channels-fastest state
    assert uplan(uargs(C=60)).vector == 0                          # C not a multiple of 8
    assert uplan(uargs(w_dtype=ccv.CCV_F32)).vector == 1           # weights of another dtype are fine
    assert uplan(uargs(w_dtype=ccv.CCV_F32, weight=W + 4)).vector == 0  # but not unaligned ones
    assert uplan(uargs(x=X + 2)).vector == 0                       # x not 16-byte aligned
    assert uplan(uargs(bias=BIAS + 2)).vector == 0
    assert uplan(uargs(L=3, x_stride=(192, 3, 1), out_stride=(192, 3, 1))).vector == 0
    p = uplan(uargs(C=60))
    assert p.elems_per_lane == 4 and p.grid == -(-2 * 60 // (256 * 4))
    assert uplan(uargs(L=0, x=None, weight=None, state=None, out=None)).path == ccv.CCV_PATH_NONE


# ---- backward ----------------------------------------------------------------------

DOUT, DX, DW, DB, DINIT, DFS, WS = (0x4000000 + 0x100000 * i for i in range(7))


def bargs(B=2, C=64, L=1000, K=4, layout="cf", ws=True, **over):
    a = ccv.ccv_bwd_args_t()
    a.B, a.C, a.L, a.K = B, C, L, K
    a.x_dtype = a.w_dtype = ccv.CCV_BF16
    a.activation = ccv.CCV_ACT_SILU
    st = (C * L, L, 1) if layout == "cf" else (L * C, 1, C)
    a.x, a.dout, a.dx = X, DOUT, DX
    a.x_stride = type(a.x_stride)(*st)
    a.dout_stride = type(a.dout_stride)(*st)
    a.dx_stride = type(a.dx_stride)(*st)
    a.weight, a.dweight = W, DW
    for k, v in over.items():
        if k.endswith("stride"):
            v = type(getattr(a, k))(*v)
        setattr(a, k, v)
    if ws:
        a.workspace, a.workspace_bytes = WS, ccv.ccv_bwd_workspace_size(a)
    return a


def bcheck(a):
    return ccv.STATUS[ccv.ccv_bwd_check(a)]


def test_bwd_workspace_size_is_the_partial_sums():
    # one fp32 row of (K + 1) * C partial sums per (b, tile group), plus the rows the
    # level kernels of the reduction tree write while more than 512 rows are left (the
    # final kernel sums up to 16 groups of 32 at once)
    # channel-first without seq_idx: the register path, a row per segment of 2048
    # (16-bit) or 1024 (fp32) steps
    a = bargs(B=3, C=100, L=1000, K=3, ws=False)
    assert ccv.ccv_bwd_workspace_size(a) == 3 * 100 * (3 + 1) * 4
    a = bargs(B=2, C=128, L=1 << 20, K=3, ws=False)
    a.x_dtype = ccv.CCV_F32
    parts = 2 * (1 << 20) // 1024                    # 2048 -> 64, then the final kernel
    assert ccv.ccv_bwd_workspace_size(a) == (parts + 64) * 128 * 4 * 4
    # channel-first with seq_idx: the register path as well
    a = bargs(B=3, C=100, L=1000, K=3, ws=False, seq_idx=SEQ)
    assert ccv.ccv_bwd_workspace_size(a) == 3 * 100 * (3 + 1) * 4
    # ... unless seq_idx is not 16-byte aligned: the LDS path, a row per tile of 32 steps
    a = bargs(B=3, C=100, L=1000, K=3, ws=False, seq_idx=SEQ + 4)
    parts = 3 * -(-1000 // 32)                       # 96 rows: the final kernel alone
    assert ccv.ccv_bwd_workspace_size(a) == parts * 100 * (3 + 1) * 4
    # channel-last: a row per group of 4 tiles
    a = bargs(B=3, C=100, L=1000, K=3, layout="cl", ws=False)
    parts = 3 * -(-(-(-1000 // 32)) // 4)            # 24 rows: one level
    assert ccv.ccv_bwd_workspace_size(a) == parts * 100 * (3 + 1) * 4
    assert ccv.ccv_bwd_workspace_size(bargs(B=2, C=5, L=0, ws=False)) == 2 * 1 * 5 * 5 * 4
    a = bargs(B=1, C=8, L=512 * 128, K=2, layout="cl", ws=False)   # 512 rows: the final kernel alone
    assert ccv.ccv_bwd_workspace_size(a) == 512 * 8 * 3 * 4
    a = bargs(B=1, C=8, L=513 * 128, K=2, layout="cl", ws=False)   # 513 rows -> 17 -> final
    assert ccv.ccv_bwd_workspace_size(a) == (513 + 17) * 8 * 3 * 4
    assert ccv.ccv_bwd_workspace_size(bargs(B=0, ws=False)) == 0
    assert ccv.ccv_bwd_workspace_size(bargs(K=5, ws=False)) == ccv.lib().ccv_bwd_check(bargs(K=5, ws=False))


def test_bwd_valid_calls():
    assert bcheck(bargs()) == "CCV_OK"
    assert bcheck(bargs(layout="cl")) == "CCV_OK"
    assert bcheck(bargs(bias=BIAS, dbias=DB, seq_idx=SEQ)) == "CCV_OK"
    assert bcheck(bargs(initial_states=INIT, init_stride=(192, 1, 64), dfinal_states=DFS,
                        dfinal_stride=(192, 3, 1), dinitial_states=DINIT,
                        dinit_stride=(192, 1, 64))) == "CCV_OK"
    # dx may be strided differently from x (any non-overlapping layout)
    assert bcheck(bargs(dx_stride=(64 * 1000, 1, 64))) == "CCV_OK"


def test_bwd_argument_errors():
    a = bargs()
    a.struct_size = 4
    assert bcheck(a) == "CCV_E_ABI"
    assert bcheck(bargs(K=1)) == "CCV_E_KSIZE"
    assert bcheck(bargs(w_dtype=9)) == "CCV_E_DTYPE"
    assert bcheck(bargs(activation=5)) == "CCV_E_UNSUPPORTED"
    assert bcheck(bargs(seq_idx=SEQ, initial_states=INIT, init_stride=(192, 3, 1))) == "CCV_OK"
    assert bcheck(bargs(seq_idx=SEQ, dfinal_states=DFS, dfinal_stride=(192, 3, 1))) == "CCV_OK"
    assert bcheck(bargs(dinitial_states=DINIT, dinit_stride=(192, 3, 1))) == "CCV_E_UNSUPPORTED"
    for name in ("x", "dout", "dx", "weight", "dweight"):
        assert bcheck(bargs(**{name: None})) == "CCV_E_NULL", name
    assert bcheck(bargs(dx=X)) == "CCV_E_ALIAS"
    assert bcheck(bargs(dx=DOUT)) == "CCV_E_ALIAS"
    assert bcheck(bargs(dweight=W)) == "CCV_E_ALIAS"
    assert bcheck(bargs(initial_states=INIT, init_stride=(192, 3, 1), dinitial_states=INIT,
                        dinit_stride=(192, 3, 1))) == "CCV_E_ALIAS"
    assert bcheck(bargs(dx_stride=(64000, 1000, 0))) == "CCV_E_LAYOUT"     # dx overlaps itself
    assert bcheck(bargs(x_stride=(64000, 1000, -1))) == "CCV_E_LAYOUT"


def test_bwd_workspace_errors():
    a = bargs(ws=False)
    assert bcheck(a) == "CCV_E_NULL"
    a.workspace, a.workspace_bytes = WS, ccv.ccv_bwd_workspace_size(a) - 4
    assert bcheck(a) == "CCV_E_SHAPE"
    a.workspace, a.workspace_bytes = WS + 4, ccv.ccv_bwd_workspace_size(a)
    assert bcheck(a) == "CCV_E_LAYOUT"


def test_bwd_empty_extents():
    # no channels: nothing to do, no pointer needed
    assert bcheck(bargs(C=0, x=None, dout=None, dx=None, weight=None, dweight=None, ws=False)) == "CCV_OK"
    # no rows: dweight (and dbias) are still written (as zeros); x / dout / dx unused
    a = bargs(B=0, x=None, dout=None, dx=None, ws=False)
    assert bcheck(a) == "CCV_OK"
    st, p = ccv.ccv_bwd_plan(a)
    assert st == 0 and p.path == ccv.CCV_PATH_BACKWARD and p.grid == 0


def test_bwd_plan():
    # aligned channel-first without seq_idx: the register-only kernel, one wave per
    # (b, c, segment of 2048 bf16 steps), in workgroups of 4
    st, p = ccv.ccv_bwd_plan(bargs(B=4, C=2048, L=4096))
    assert st == 0 and p.path == ccv.CCV_PATH_BACKWARD and p.vector == 3
    assert p.span == 2048 and p.unroll == 1 and p.elems_per_lane == 8
    assert p.work_items == 4 * 2048 * 2 and p.grid == 4 * 2048 * 2 // 4 and p.block == 256
    # with seq_idx: the register kernel too, its ids loaded beside x
    st, p = ccv.ccv_bwd_plan(bargs(B=4, C=2048, L=4096, seq_idx=SEQ))
    assert st == 0 and p.vector == 3 and p.span == 2048 and p.work_items == 4 * 2048 * 2
    # seq_idx not 16-byte aligned: the LDS-staged channel-first kernel, a 64-lane
    # workgroup per (b, tile of 32 steps, group of 64 channels)
    st, p = ccv.ccv_bwd_plan(bargs(B=4, C=2048, L=4096, seq_idx=SEQ + 4))
    assert st == 0 and p.vector == 1 and p.span == 32 and p.unroll == 1
    assert p.work_items == 4 * 128 * 32 and p.grid == p.work_items and p.block == 64
    # aligned channel-last: the LDS-staged channel-last kernel, 4 tiles per work item
    st, p = ccv.ccv_bwd_plan(bargs(B=4, C=2048, L=4096, layout="cl"))
    assert st == 0 and p.vector == 2 and p.unroll == 4 and p.work_items == 4 * 32 * 32
    # fp32: segments of 1024 steps on the register path, tiles of 32 on the LDS paths
    a = bargs(B=1, C=64, L=100, ws=False)
    a.x_dtype = ccv.CCV_F32
    a.workspace, a.workspace_bytes = WS, ccv.ccv_bwd_workspace_size(a)
    st, p = ccv.ccv_bwd_plan(a)
    assert st == 0 and p.span == 1024 and p.vector == 3 and p.work_items == 64 and p.grid == 16
    a.seq_idx = SEQ
    st, p = ccv.ccv_bwd_plan(a)
    assert st == 0 and p.span == 1024 and p.vector == 3
    a.seq_idx = SEQ + 4
    st, p = ccv.ccv_bwd_plan(a)
    assert st == 0 and p.span == 32 and p.vector == 1
    # channel-first rows that are not 16-byte aligned (L = 4095): the register kernel,
    # its vector that straddles L moving element by element
    odd = dict(B=4, C=2048, L=4095, x_stride=(2048 * 4095, 4095, 1), dout_stride=(2048 * 4095, 4095, 1),
               dx_stride=(2048 * 4095, 4095, 1))
    st, p = ccv.ccv_bwd_plan(bargs(**odd))
    assert st == 0 and p.vector == 3 and p.span == 2048 and p.work_items == 4 * 2048 * 2
    # ... with ids that are not 16-byte aligned either, and mixed layouts: the element
    # kernel, one lane per (b, tile, c)
    st, p = ccv.ccv_bwd_plan(bargs(seq_idx=SEQ + 4, **odd))
    assert st == 0 and p.vector == 0 and p.work_items == 4 * 128 * 2048 and p.grid == 4 * 128 * 2048 // 256
    assert ccv.ccv_bwd_plan(bargs(dx_stride=(64 * 1000, 1, 64)))[1].vector == 0


def test_bwd_static_refuses_calls_beyond_its_scratch():
    """ccv_bwd_static checks the partial-sum space it needs against its fixed array
    before touching any device."""
    a = ccv.ccv_bwd_args_t()
    a.B, a.C, a.L, a.K = 16, 8192, 8192, 4
    a.x_dtype = a.w_dtype = ccv.CCV_BF16
    a.x, a.dout, a.dx, a.weight, a.dweight = X, OUT, FIN, W, BIAS
    for f in ("x_stride", "dout_stride", "dx_stride"):
        setattr(a, f, type(getattr(a, f))(8192 * 8192, 1, 8192))
    assert ccv.ccv_bwd_workspace_size(a) > ccv.CCV_BWD_STATIC_SCRATCH_BYTES == 64 << 20
    static = ccv.lib().ccv_bwd_static
    assert ccv.STATUS[static(ctypes.byref(a), None)] == "CCV_E_SCRATCH"
    assert ccv.STATUS[static(None, None)] == "CCV_E_NULL"
    a.dx = X                                           # argument errors come first, as in ccv_bwd
    assert ccv.STATUS[static(ctypes.byref(a), None)] == "CCV_E_ALIAS"


def test_binding_refuses_non_contiguous_seq_idx():
    """The C ABI reads seq_idx as a contiguous [B, L] array, so the binding's argument
    builders refuse a view with other strides instead of passing its pointer on."""
    import torch

    import workloads as wl
    ids = wl.seq_idx_from_lengths([3, 5], 2)
    assert ids.is_contiguous() and ids.stride() == (8, 1)
    x = torch.zeros(2, 4, 8)
    wt = torch.zeros(4, 4)
    bad = torch.zeros(8, 2, dtype=torch.int32).t()
    with pytest.raises(ValueError, match="contiguous"):
        ccv.make_args(x, wt, x.clone(), seq_idx=bad)
    with pytest.raises(ValueError, match="contiguous"):
        ccv.make_bwd_args(x, wt, None, x, x.clone(), wt.clone(), seq_idx=bad)
    ccv.make_args(x, wt, x.clone(), seq_idx=bad.contiguous())


@pytest.mark.parametrize("K", [2, 3, 4])
def test_every_dtype_pair_takes_the_vector_paths(K):
    """Aligned channel-last calls take the straight-line tile path (two row batches in
    flight) and aligned decode calls the 16-byte update path for every pair of x and
    weight dtypes."""
    codes = (ccv.CCV_F32, ccv.CCV_F16, ccv.CCV_BF16)
    for xd in codes:
        for wd in codes:
            a = args(K=K, layout="cl", x_dtype=xd, w_dtype=wd, bias=BIAS,
                     initial_states=INIT, init_stride=(64 * (K - 1), 1, 64))
            st, p = ccv.ccv_fwd_plan(a)
            assert st == 0 and p.path == ccv.CCV_PATH_CHANNEL_LAST and p.vector == 1 and p.unroll == 8, (xd, wd)
            u = uargs(K=K, x_dtype=xd, w_dtype=wd)
            st, p = ccv.ccv_update_plan(u)
            assert st == 0 and p.vector == 1, (xd, wd)
    # an unaligned weight pointer sends whole tiles to the element path
    st, p = ccv.ccv_fwd_plan(args(layout="cl", weight=W + 2))
    assert st == 0 and p.vector == 1 and p.unroll == 4
