"""The C-ABI library loads, exports every function include/ssd.h declares, and
rejects bad arguments before touching the device (CPU only: no call here reaches
a kernel launch)."""
import ctypes
import os
import re

import pytest

import state_space_model_mamba_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssd.LIBRARY):
        pytest.fail("libssd.so is not built (run __graft_entry__.build())")
    return ssd.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(ssd.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.ssd_version() == 10200


def test_status_strings(lib):
    for code, name in ssd.STATUS.items():
        assert lib.ssd_status_string(code).decode().startswith(name)
    assert lib.ssd_status_string(99).decode() == "SSD_ERR_UNKNOWN"


def dims(**kw):
    base = dict(batch=4, seqlen=8192, nheads=80, headdim=64, dstate=128, ngroups=1, chunk=256,
                io_dtype=ssd.SSD_BF16)
    base.update(kw)
    return ssd.make_dims(**base)


def ws_size(lib, d):
    n = ctypes.c_size_t(0)
    rc = lib.ssd_chunk_scan_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return rc, n.value


def test_workspace_size_host_logic(lib):
    rc, n = ws_size(lib, dims())
    assert rc == 0 and n > 0
    # the segment states are fp32 P x N per (b, h, slot): a whole multiple of 32 KiB
    assert (n - n % 256) % (64 * 128 * 4) == 0 or n > 4 * 80 * 64 * 128 * 4
    assert ws_size(lib, dims(seqlen=0)) == (0, 0)
    assert ws_size(lib, dims(batch=0)) == (0, 0)
    assert ws_size(lib, dims(io_dtype=ssd.SSD_F32, headdim=16, dstate=16, chunk=64)) == (0, 0)
    assert ws_size(lib, dims(headdim=32))[0] == 3        # bf16 path needs P = 64, N = 128
    assert ws_size(lib, dims(chunk=96))[0] == 3          # Q must be a multiple of 64
    assert ws_size(lib, dims(chunk=1024))[0] == 3
    assert ws_size(lib, dims(ngroups=3))[0] == 2         # H % G != 0
    assert ws_size(lib, dims(nheads=0))[0] == 2
    assert ws_size(lib, dims(seqlen=-1))[0] == 2
    assert ws_size(lib, dims(io_dtype=7))[0] == 3
    d = dims()
    d.flags = 2                                          # unknown flag bit
    assert ws_size(lib, d)[0] == 2
    d.flags = ssd.SSD_DT_SOFTPLUS                        # the fused softplus is accepted
    assert ws_size(lib, d)[0] == 0
    assert lib.ssd_chunk_scan_workspace_size(None, ctypes.byref(ctypes.c_size_t())) == 1
    assert lib.ssd_chunk_scan_workspace_size(ctypes.byref(dims()), None) == 1


FAKE = 1 << 40   # a fake, well-aligned "device" address; never dereferenced here


def scan(lib, d, x=FAKE, dt=FAKE + (1 << 33), A=FAKE + (2 << 33), B=FAKE + (3 << 33),
         C=FAKE + (4 << 33), D=FAKE + (5 << 33), init=None, y=FAKE + (6 << 33),
         fin=FAKE + (7 << 33), ws=FAKE + (8 << 33), ws_bytes=1 << 40):
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    return lib.ssd_chunk_scan(ctypes.byref(d), p(x), p(dt), p(A), p(B), p(C), p(D), p(init),
                              p(y), p(fin), p(ws), ws_bytes, None)


def test_scan_validation(lib):
    d = dims()
    assert scan(lib, d, x=None) == 1
    assert scan(lib, d, fin=None) == 1
    assert scan(lib, d, ws=None) == 5
    assert scan(lib, d, ws_bytes=16) == 5
    assert scan(lib, d, y=FAKE + 64) == 4                 # y overlaps x
    assert scan(lib, d, y=FAKE + (8 << 33) + 1024) == 4   # y overlaps the workspace
    assert scan(lib, d, fin=FAKE + 256) == 4              # final state overlaps x
    assert scan(lib, d, init=FAKE + (7 << 33) + 4096) == 4  # partial init/final overlap
    assert scan(lib, d, x=FAKE + 2) == 7                  # misaligned
    assert scan(lib, dims(headdim=48)) == 3
    assert scan(lib, dims(ngroups=3)) == 2
    assert scan(lib, dims(batch=0), x=None, y=None, fin=None) == 0   # empty batch: no-op
    assert lib.ssd_chunk_scan(None, *([None] * 10), 0, None) == 1


def test_decode_validation(lib):
    p = ctypes.c_void_p
    d = dims()
    base = [p(FAKE + (k << 33)) for k in range(8)]

    def call(*over, **kw):
        args = list(base)
        for i, v in over:
            args[i] = v
        return lib.ssd_decode_step(ctypes.byref(kw.get("d", d)), *args, None)

    assert call((0, None)) == 1
    assert call((7, p(FAKE + (6 << 33) + 64))) == 4     # y overlaps the state
    assert call((6, p(FAKE + 64))) == 4                 # state overlaps x
    assert call(d=dims(dstate=96)) == 3
    assert call(d=dims(ngroups=7)) == 2
    assert call((6, p(FAKE + (6 << 33) + 4))) == 7      # misaligned state
    assert lib.ssd_decode_step(ctypes.byref(dims(batch=0)), *([None] * 8), None) == 0


def test_state_init_validation(lib):
    d = dims()
    assert lib.ssd_state_init(ctypes.byref(d), None, None, None) == 1
    assert lib.ssd_state_init(ctypes.byref(d), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 64), None) == 4
    assert lib.ssd_state_init(ctypes.byref(dims(batch=0)), None, None, None) == 0


def test_decode_steps_validation(lib):
    p = ctypes.c_void_p
    d = dims()
    # x, dt, A, B, C, D, state, y: 8 GiB apart, well beyond 1000 steps of the 2.7B shape
    base = [p(FAKE + (k << 33)) for k in range(8)]

    def call(*over, steps=1000, **kw):
        args = list(base)
        for i, v in over:
            args[i] = v
        return lib.ssd_decode_steps(ctypes.byref(kw.get("d", d)), ctypes.c_int64(steps), *args,
                                    None)

    assert call((0, None)) == 1
    assert call((7, None)) == 1
    assert call(steps=-1) == 2
    assert call((7, p(FAKE + (6 << 33) + 64))) == 4     # y overlaps the state
    assert call((6, p(FAKE + 64))) == 4                 # state overlaps x
    # y [S, B, H, P] bf16 spans S x 40960 bytes at batch 4: 1000 steps of it
    # (41 MB) reach x placed 16 MiB after it, where one step's slice ends well before
    assert call((7, p(FAKE + (1 << 32))), (0, p(FAKE + (1 << 32) + (1 << 24)))) == 4
    assert call((1, p(FAKE + (7 << 33) + 4096))) == 4   # dt inside y
    assert call(d=dims(dstate=96)) == 3
    assert call(d=dims(headdim=(1 << 24) + 1)) == 3
    assert call(d=dims(ngroups=7)) == 2
    assert call(steps=1 << 31) == 3
    assert call((6, p(FAKE + (6 << 33) + 4))) == 7      # misaligned state
    assert call((3, p(FAKE + (3 << 33) + 8))) == 7      # misaligned B
    assert call((0, p(FAKE + 1))) == 7                  # x not element-aligned
    assert lib.ssd_decode_steps(ctypes.byref(dims(batch=0)), ctypes.c_int64(5), *([None] * 8),
                                None) == 0
    assert lib.ssd_decode_steps(ctypes.byref(d), ctypes.c_int64(0), *([None] * 8), None) == 0
    assert lib.ssd_decode_steps(None, ctypes.c_int64(1), *([None] * 8), None) == 1


def test_dt_bias_validation(lib):
    """The fused step-size prep: the bias is 4-byte aligned and outside the outputs
    (every call here fails validation, so nothing is launched)."""
    p = lambda v: ctypes.c_void_p(v)
    d = dims()
    d.flags = ssd.SSD_DT_SOFTPLUS
    d.dt_bias = FAKE + (9 << 33) + 2
    assert scan(lib, d) == 7                              # misaligned bias
    d.dt_bias = FAKE + (6 << 33) + 64
    assert scan(lib, d) == 4                              # bias inside y
    d.dt_bias = FAKE + (7 << 33) + 64
    assert scan(lib, d) == 4                              # bias inside the final state
    base = [p(FAKE + (k << 33)) for k in range(8)]
    d.dt_bias = FAKE + (7 << 33) + 8                      # bias inside y of a decode step
    assert lib.ssd_decode_step(ctypes.byref(d), *base, None) == 4
    d.dt_bias = FAKE + (6 << 33) + 8                      # ... or inside the state
    assert lib.ssd_decode_steps(ctypes.byref(d), ctypes.c_int64(3), *base, None) == 4
    d.flags = 0                                           # without the flag the bias is not read
    d.dt_bias = FAKE + (6 << 33) + 2
    assert scan(lib, d, x=None) == 1


def test_varlen_host_logic(lib):
    """Packed variable-length batches: offsets are validated and the workspace is
    the largest of the equal-length runs' (CPU only, nothing launched)."""
    H, P, N, G, Q = 80, 64, 128, 1, 256

    def size(cu):
        arr = (ctypes.c_int64 * len(cu))(*cu)
        d = dims(batch=len(cu) - 1, seqlen=cu[-1], nheads=H, headdim=P, dstate=N, ngroups=G,
                 chunk=Q)
        n = ctypes.c_size_t(0)
        return lib.ssd_chunk_scan_varlen_workspace_size(ctypes.byref(d), arr, ctypes.byref(n)), n.value

    def run_ws(b, L):
        return ws_size(lib, dims(batch=b, seqlen=L, nheads=H, headdim=P, dstate=N, ngroups=G,
                                 chunk=Q))[1]

    # runs of equal length share one launch pair, each planning for its share of
    # the CUs with a workspace region of its own: at most the runs' own sizes summed
    rc, n = size([0, 8192, 8192 + 100, 8192 + 200, 8192 + 4296])
    assert rc == 0 and 0 < n <= run_ws(1, 8192) + run_ws(2, 100) + run_ws(1, 4096) + 3 * 256
    assert n % 256 == 0
    assert size([0, 4096, 8192, 12288, 16384]) == (0, run_ws(4, 4096))   # one run: the batched scan
    assert size([0, 0, 0])[0] == 0
    assert size([1, 5])[0] == 2                # cu[0] != 0
    assert size([0, 7, 5, 9])[0] == 2          # decreasing
    arr = (ctypes.c_int64 * 3)(0, 5, 9)
    d = dims(batch=2, seqlen=10)               # cu[S] != T
    assert lib.ssd_chunk_scan_varlen_workspace_size(ctypes.byref(d), arr,
                                                    ctypes.byref(ctypes.c_size_t())) == 2
    assert lib.ssd_chunk_scan_varlen_workspace_size(ctypes.byref(d), None,
                                                    ctypes.byref(ctypes.c_size_t())) == 1
    # a scan whose last run has a misaligned slice fails before anything is launched:
    # fp32 I/O with H = 5, P = 3 is 60 bytes of x per token; lengths 4, 5, 6 are three
    # runs starting at tokens 0, 4, 9, i.e. bytes 0, 240 (16-aligned) and 540 (not)
    arr = (ctypes.c_int64 * 4)(0, 4, 9, 15)
    d = dims(batch=3, seqlen=15, nheads=5, headdim=3, dstate=16, ngroups=1, chunk=64,
             io_dtype=ssd.SSD_F32)
    p = lambda v: ctypes.c_void_p(v)
    rc = lib.ssd_chunk_scan_varlen(ctypes.byref(d), arr, *[p(FAKE + (k << 33)) for k in range(6)],
                                   None, p(FAKE + (6 << 33)), p(FAKE + (7 << 33)), None, 0, None)
    assert rc == 7


def test_gdn_validation(lib):
    """ssd_gdn_decode_step rejects bad arguments before any launch (CPU only)."""
    p = ctypes.c_void_p

    def gd(**kw):
        base = dict(batch=4, qk_heads=16, v_heads=32, dk=128, dv=128, io_dtype=ssd.SSD_BF16,
                    reserved=0)
        base.update(kw)
        return ssd.SsdGdnDims(**base)

    args = [p(FAKE + (k << 33)) for k in range(7)]   # q, k, v, g, beta, state, o

    def call(d, *over):
        a = list(args)
        for i, v in over:
            a[i] = v
        return lib.ssd_gdn_decode_step(ctypes.byref(d), *a, None)

    assert lib.ssd_gdn_decode_step(None, *args, None) == 1
    assert call(gd(), (0, None)) == 1
    assert call(gd(v_heads=24, qk_heads=16)) == 2      # Hv % Hk != 0
    assert call(gd(reserved=1)) == 2
    assert call(gd(dk=96)) == 3
    assert call(gd(dv=512)) == 3
    assert call(gd(io_dtype=5)) == 3
    assert call(gd(), (5, p(FAKE + (5 << 33) + 8))) == 7          # misaligned state
    assert call(gd(), (6, p(FAKE + (5 << 33) + 64))) == 4         # o inside the state
    assert call(gd(), (5, p(FAKE + (2 << 33) + 64))) == 4         # state inside v
    assert call(gd(batch=0), *[(i, None) for i in range(7)]) == 0


def test_gdn_steps_validation(lib):
    p = ctypes.c_void_p
    d = ssd.SsdGdnDims(4, 16, 32, 128, 128, ssd.SSD_BF16, 0)
    args = [p(FAKE + (k << 33)) for k in range(7)]

    def call(steps, *over):
        a = list(args)
        for i, v in over:
            a[i] = v
        return lib.ssd_gdn_decode_steps(ctypes.byref(d), ctypes.c_int64(steps), *a, None)

    assert call(-1) == 2
    assert call(0, *[(i, None) for i in range(7)]) == 0
    assert call(5, (0, None)) == 1
    # o [S, B, Hv, dv] bf16 of 100 steps spans 100 x 32768 bytes: it reaches a
    # state placed 2 MiB after it
    assert call(100, (6, p(FAKE + (6 << 33))), (5, p(FAKE + (6 << 33) + (2 << 20)))) == 4
    assert call(1 << 31) == 3


def test_binding_rejects_host_tensors():
    """The binding hands data pointers to GPU kernels, so a host tensor must be
    refused before the C call (it would pass a host address to a kernel)."""
    import torch
    x = torch.zeros((1, 64, 4, 64), dtype=torch.bfloat16)
    dt = torch.zeros((1, 64, 4))
    A = torch.zeros(4)
    Bm = torch.zeros((1, 64, 1, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device"):
        ssd.ssd_chunk_scan(x, dt, A, Bm, Bm, A, 64)
    with pytest.raises(ValueError, match="device"):
        ssd.ssd_decode_step(x[:, 0], dt[:, 0], A, Bm[:, 0], Bm[:, 0], A,
                            torch.zeros((1, 4, 64, 128)))
    with pytest.raises(ValueError, match="device"):
        ssd.ssd_state_init(torch.zeros((1, 4, 64, 128)))


def test_noalloc_rejects_workspace_beyond_scratch(lib):
    """A problem whose workspace exceeds the no-alloc scratch array is refused
    with SSD_ERR_WORKSPACE before any device call (the pointers are never used)."""
    d = ssd.make_dims(16, 16384, 80, 64, 128, 1, 256, ssd.SSD_BF16)
    need = ssd.ssd_chunk_scan_workspace_size(16, 16384, 80, 64, 128, 1, 256)
    assert need > ssd.NOALLOC_SCRATCH_BYTES
    p = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(9)]
    assert lib.ssd_chunk_scan_noalloc(ctypes.byref(d), *p, None) == 5
    # unsupported shapes and bad dims are refused the same way
    d.headdim = 32
    assert lib.ssd_chunk_scan_noalloc(ctypes.byref(d), *p, None) == 3
    assert lib.ssd_chunk_scan_noalloc(None, *p, None) == 1


def test_planner_segment_counts(lib):
    """The planner's segment counts at the three layer shapes, read back from
    the workspace size (one state slot per unit of the first nseg - 1 segments,
    one unit each at these shapes, plus one spare: B*H*nseg*P*N*4 bytes plus
    the slots' decays, each part 256-byte aligned).  2.7B layer: 3 segments
    (240 scan work-groups); 130M layer: 5 (240); 131072 tokens in 8 groups: 10
    (240, the one-round maximum: 21 segments, a two-round plan, measured
    slower)."""
    def align(n):
        return (n + 255) // 256 * 256
    for (b, L, H, G, nseg) in ((4, 8192, 80, 1, 3), (8, 2048, 24, 1, 5), (1, 131072, 80, 8, 10)):
        slots = b * H * nseg
        want = align(slots * 64 * 128 * 4) + align(slots * 4)
        assert ssd.ssd_chunk_scan_workspace_size(b, L, H, 64, 128, G, 256) == want, (b, L, H, G)
