"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "packattn.h")
LIB = os.path.join(ROOT, "packed_variable_length_amd", "libpackattn.so")

PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_HEADDIM = 0, -1, -2, -3, -4
PA_ERR_MASK_MISMATCH, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_ALIGN = -5, -6, -7, -8


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__  # build on demand (loads build.py by path)
        __graft_entry__._build_module().build(verbose=False)
    from packed_variable_length_amd import packattn  # loads the library, checks signatures
    return packattn._lib


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\**([a-z_0-9]+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for want in ("seq_ids_from_valid_frames", "build_block_mask", "build_block_mask_bytes",
                 "attn_packed_fwd", "attn_packed_bwd", "attn_packed_bwd_workspace_bytes",
                 "pa_status_str", "masked_mse_fwd", "masked_mse_bwd", "masked_mse_fwd_bwd",
                 "masked_mse_workspace_bytes", "adaln_fwd", "adaln_bwd", "plan_token_packs",
                 "seq_ids_from_lengths", "length_bucket_batches", "dual_constraint_batch",
                 "fit_step_cost"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    from packed_variable_length_amd import packattn
    for code in (PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_HEADDIM,
                 PA_ERR_MASK_MISMATCH, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_ALIGN):
        s = packattn.pa_status_str(code)
        assert s and s != "unknown status"
    assert packattn.pa_status_str(-99) == "unknown status"


def test_mask_bytes_validation(lib):
    assert lib.build_block_mask_bytes(36864, 36864, 128, 128) > 0
    assert lib.build_block_mask_bytes(0, 10, 128, 128) == 0
    assert lib.build_block_mask_bytes(10, 10, 8, 128) == 0        # block too small
    assert lib.build_block_mask_bytes(10, 10, 128, 2048) == 0     # block too large
    assert lib.build_block_mask_bytes(16384 * 16 + 1, 10, 16, 16) == 0  # too many tiles
    assert lib.attn_packed_bwd_workspace_bytes(1, 100, 100, 2, 128) >= 800
    assert lib.attn_packed_bwd_workspace_bytes(1, 100, 100, 2, 96) == 0
    assert lib.attn_packed_bwd_workspace_bytes(7, 100, 100, 2, 128) == 0


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails first


def test_seq_ids_errors(lib):
    assert lib.seq_ids_from_valid_frames(None, 3, 8, 4, FAKE, None) == PA_ERR_NULL
    assert lib.seq_ids_from_valid_frames(FAKE, -1, 8, 4, FAKE, None) == PA_ERR_SHAPE
    assert lib.seq_ids_from_valid_frames(FAKE, 3, 0, 4, FAKE, None) == PA_ERR_SHAPE
    assert lib.seq_ids_from_valid_frames(FAKE, 3, 8, 0, FAKE, None) == PA_ERR_SHAPE
    assert lib.seq_ids_from_valid_frames(FAKE, 1 << 20, 1 << 10, 1 << 10, FAKE, None) == PA_ERR_SHAPE
    assert lib.seq_ids_from_valid_frames(None, 0, 8, 4, None, None) == PA_OK  # empty: no-op


def test_block_mask_errors(lib):
    from packed_variable_length_amd.packattn import PaBlockMask
    d = PaBlockMask()
    need = lib.build_block_mask_bytes(1000, 1000, 128, 128)
    args = lambda **kw: dict(dict(q=FAKE, nq=1000, k=FAKE, nkv=1000, bq=128, bkv=128,  # noqa: E731
                                  st=FAKE, nb=need, out=ctypes.byref(d)), **kw)
    call = lambda a: lib.build_block_mask(a["q"], a["nq"], a["k"], a["nkv"], a["bq"], a["bkv"],  # noqa: E731
                                          a["st"], a["nb"], a["out"], None)
    assert call(args(q=None)) == PA_ERR_NULL
    assert call(args(st=None)) == PA_ERR_NULL
    assert call(args(nq=0)) == PA_ERR_SHAPE
    assert call(args(bq=4)) == PA_ERR_SHAPE
    assert call(args(nb=need - 1)) == PA_ERR_WORKSPACE
    assert call(args(st=ctypes.c_void_p(0x100010))) == PA_ERR_ALIGN


def _fake_mask(nq, nkv, bq=128, bkv=128):
    from packed_variable_length_amd.packattn import PaBlockMask
    d = PaBlockMask()
    d.nq, d.nkv, d.block_q, d.block_kv = nq, nkv, bq, bkv
    d.nq_tiles, d.nkv_tiles = -(-nq // bq), -(-nkv // bkv)
    for f in ("tile_class", "q_ptr", "q_cols", "kv_ptr", "kv_rows", "q_order", "kv_order",
              "pair_off", "pair_len", "pair_ent"):
        setattr(d, f, 0x200000)
    return d


def _fwd(lib, dtype=1, nq=500, nkv=500, H=2, d=128, mask=None, q=FAKE, o=FAKE):
    m = _fake_mask(500, 500) if mask is None else mask
    return lib.attn_packed_fwd(dtype, nq, nkv, H, d, 0.1, q, FAKE, FAKE, FAKE, FAKE,
                               ctypes.byref(m), o, FAKE, None)


def test_attention_argument_errors(lib):
    assert _fwd(lib, dtype=5) == PA_ERR_DTYPE
    assert _fwd(lib, d=96) == PA_ERR_HEADDIM
    assert _fwd(lib, H=0) == PA_ERR_SHAPE
    assert _fwd(lib, q=None) == PA_ERR_NULL
    assert _fwd(lib, q=ctypes.c_void_p(0x100008)) == PA_ERR_ALIGN
    assert lib.attn_packed_fwd(1, 500, 500, 2, 128, 0.1, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                               FAKE, FAKE, None) == PA_ERR_NULL


def test_backward_stage_argument_errors(lib):
    # the three stage entry points check their arguments like attn_packed_bwd,
    # before anything is launched
    ws = lib.attn_packed_bwd_workspace_bytes(1, 500, 500, 2, 128)
    pre = lib.attn_packed_bwd_preprocess
    assert pre(1, 500, 2, 128, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == PA_ERR_WORKSPACE
    assert pre(1, 500, 2, 128, None, FAKE, FAKE, FAKE, ws, None) == PA_ERR_NULL
    assert pre(1, 500, 2, 128, FAKE, FAKE, None, FAKE, ws, None) == PA_ERR_NULL
    assert pre(1, 500, 2, 96, FAKE, FAKE, FAKE, FAKE, ws, None) == PA_ERR_HEADDIM
    assert pre(7, 500, 2, 128, FAKE, FAKE, FAKE, FAKE, ws, None) == PA_ERR_DTYPE
    assert pre(1, 0, 2, 128, FAKE, FAKE, FAKE, FAKE, ws, None) == PA_ERR_SHAPE
    assert pre(1, 500, 2, 128, FAKE, FAKE, FAKE, ctypes.c_void_p(0x200080), ws,
               None) == PA_ERR_ALIGN
    good, bad = _fake_mask(500, 500), _fake_mask(500, 600)

    def dq(mask, wsb, out=FAKE):
        return lib.attn_packed_bwd_dq(1, 500, 500, 2, 128, 0.1, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, FAKE, wsb, FAKE, FAKE, ctypes.byref(mask), out, None)

    def dkdv(mask, wsb, out=FAKE):
        return lib.attn_packed_bwd_dkdv(1, 500, 500, 2, 128, 0.1, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, wsb, FAKE, FAKE, ctypes.byref(mask), FAKE, out,
                                        None)
    for stage in (dq, dkdv):
        assert stage(bad, ws) == PA_ERR_MASK_MISMATCH
        assert stage(good, ws - 1) == PA_ERR_WORKSPACE
        assert stage(good, ws, out=None) == PA_ERR_NULL


def test_mask_shape_hazard_is_rejected(lib):
    # a mask built for another shape (the packing report's forward/backward
    # ordering hazard) is refused before anything runs
    assert _fwd(lib, mask=_fake_mask(400, 500)) == PA_ERR_MASK_MISMATCH
    assert _fwd(lib, mask=_fake_mask(500, 500, 64, 128)) == PA_ERR_MASK_MISMATCH   # bf16 needs 128
    assert _fwd(lib, dtype=0, mask=_fake_mask(500, 500, 48, 64)) == PA_ERR_MASK_MISMATCH
    m = _fake_mask(500, 500)
    m.nq_tiles = 3
    assert _fwd(lib, mask=m) == PA_ERR_MASK_MISMATCH
    ws = lib.attn_packed_bwd_workspace_bytes(1, 500, 500, 2, 128)
    bad = _fake_mask(500, 600)
    assert lib.attn_packed_bwd(1, 500, 500, 2, 128, 0.1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               FAKE, FAKE, ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, ws,
                               None) == PA_ERR_MASK_MISMATCH
    good = _fake_mask(500, 500)
    assert lib.attn_packed_bwd(1, 500, 500, 2, 128, 0.1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               FAKE, FAKE, ctypes.byref(good), FAKE, FAKE, FAKE, FAKE, ws - 1,
                               None) == PA_ERR_WORKSPACE


def test_noalloc_backward_argument_errors(lib):
    """The no-allocation backward checks its arguments like attn_packed_bwd and
    refuses sizes past its fixed array (8 bytes per head and query, 64 MiB) on
    the host: with no GPU here, getting past the checks would give PA_ERR_HIP."""
    assert lib.attn_packed_bwd_noalloc_max_bytes() == 64 << 20

    def call(nq, H, mask, dtype=1, d=128, out=FAKE):
        return lib.attn_packed_bwd_noalloc(dtype, nq, 256, H, d, 0.1, FAKE, FAKE, FAKE, FAKE,
                                           FAKE, FAKE, FAKE, FAKE, ctypes.byref(mask), out,
                                           FAKE, FAKE, None)
    H = 64
    nq = (64 << 20) // (8 * H) + 128  # one 128-row tile past the limit
    assert call(nq, H, _fake_mask(nq, 256)) == PA_ERR_WORKSPACE
    assert call(nq - 128, H, _fake_mask(nq - 128, 256)) == PA_ERR_HIP  # fits: no GPU here
    assert call(500, 2, _fake_mask(500, 600)) == PA_ERR_MASK_MISMATCH
    assert call(500, 2, _fake_mask(500, 256), out=None) == PA_ERR_NULL
    assert call(500, 2, _fake_mask(500, 256), d=96) == PA_ERR_HEADDIM
    assert call(500, 2, _fake_mask(500, 256), dtype=3) == PA_ERR_DTYPE


def test_tile_offset_identities():
    """The XOR forms of the LDS operand offsets equal the direct formulas
    (host re-implementation of the swizzle arithmetic in pa_tile.h)."""
    def swz(r):
        return ((r & 3) << 2) | ((r >> 2) & 3)

    def row_off(lane, kk):
        r = lane & 31
        return r * 256 + (((2 * kk + (lane >> 5)) ^ swz(r)) << 4)

    def tr_off(lane, db, s):
        L, h, gm = lane & 15, lane >> 5, (lane >> 4) & 1
        row = 4 * h + (L >> 2) + 8 * s
        col = 32 * db + 16 * gm + 4 * (L & 3)
        return row * 256 + (((col >> 3) ^ swz(row)) << 4) + ((col & 7) << 1)

    for lane in range(64):
        for kk in range(8):
            assert row_off(lane, kk) == row_off(lane, 0) ^ (32 * kk)
        for db in range(4):
            for s in range(2):
                assert tr_off(lane, db, s) == (tr_off(lane, 0, 0) ^ (64 * db + 32 * s)) + 2048 * s
    # conflict-freedom of the two read patterns (16-byte bank groups of a 256-byte row)
    for kk in range(8):
        for g16 in range(4):
            lanes = [16 * g16 + i for i in range(16)]
            assert len({(row_off(l, kk) % 256) // 16 for l in lanes}) == 16
    for db in range(4):
        for s in range(2):
            for half in range(2):
                lanes = range(32 * half, 32 * half + 32)
                banks = {(tr_off(l, db, s) % 1024) // 8 for l in lanes}
                assert len(banks) == 32  # 32 distinct 8-byte slots within 4 rows


def test_masked_loss_argument_errors(lib):
    ws = lib.masked_mse_workspace_bytes(1000)
    assert ws >= 8192 and lib.masked_mse_workspace_bytes(-1) == 0
    f = lambda **kw: lib.masked_mse_fwd(kw.get("dt", 1), kw.get("n", 1000), kw.get("c", 192),  # noqa: E731
                                        kw.get("p", FAKE), FAKE, kw.get("ids", FAKE), FAKE,
                                        kw.get("ws", FAKE), kw.get("nb", ws), None)
    assert f(dt=3) == PA_ERR_DTYPE
    assert f(c=100) == PA_ERR_SHAPE            # C must be a multiple of 8
    assert f(n=-1) == PA_ERR_SHAPE
    assert f(n=1 << 30, c=1 << 10) == PA_ERR_SHAPE
    assert f(ids=None) == PA_ERR_NULL
    assert f(p=ctypes.c_void_p(0x100008)) == PA_ERR_ALIGN
    assert f(nb=ws - 1) == PA_ERR_WORKSPACE
    assert f(ws=ctypes.c_void_p(0x100010)) == PA_ERR_ALIGN
    assert lib.masked_mse_bwd(1, 1000, 192, FAKE, FAKE, FAKE, None, 1.0, FAKE, None) == PA_ERR_NULL
    assert lib.masked_mse_bwd(1, 1000, 192, FAKE, FAKE, FAKE, FAKE, 1.0,
                              ctypes.c_void_p(0x100004), None) == PA_ERR_ALIGN
    assert lib.masked_mse_bwd(1, 0, 192, None, None, None, None, 1.0, None, None) == PA_OK
    assert lib.masked_mse_fwd_bwd(1, 1000, 192, FAKE, FAKE, FAKE, 1.0, FAKE, None, FAKE, ws,
                                  None) == PA_ERR_NULL
    assert lib.masked_mse_fwd_bwd(1, 1000, 192, FAKE, FAKE, FAKE, 1.0, FAKE, FAKE, FAKE, 16,
                                  None) == PA_ERR_WORKSPACE


def test_adaln_argument_errors(lib):
    assert lib.adaln_bwd_workspace_bytes(1000, 3072, 4) > 0
    assert lib.adaln_bwd_workspace_bytes(1000, 3076, 4) == 0     # D not a multiple of 8
    assert lib.adaln_bwd_workspace_bytes(1000, 4104, 4) == 0     # D > 4096
    assert lib.adaln_bwd_workspace_bytes(1000, 64, 2049) == 0    # too many segments
    f = lambda **kw: lib.adaln_fwd(kw.get("dt", 1), kw.get("n", 100), kw.get("d", 64),  # noqa: E731
                                   kw.get("s", 2), kw.get("eps", 1e-6), kw.get("x", FAKE), FAKE,
                                   kw.get("off", FAKE), FAKE, FAKE, kw.get("y", FAKE), FAKE,
                                   FAKE, None)
    assert f(dt=2) == PA_ERR_DTYPE
    assert f(d=60) == PA_ERR_SHAPE
    assert f(s=-1) == PA_ERR_SHAPE
    assert f(eps=-1.0) == PA_ERR_SHAPE
    assert f(eps=float("nan")) == PA_ERR_SHAPE
    assert f(off=None) == PA_ERR_NULL
    assert f(y=None) == PA_ERR_NULL
    assert f(x=ctypes.c_void_p(0x100004)) == PA_ERR_ALIGN
    ws = lib.adaln_bwd_workspace_bytes(100, 64, 2)
    g = lambda **kw: lib.adaln_bwd(1, 100, 64, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,  # noqa: E731
                                   FAKE, FAKE, FAKE, kw.get("ws", FAKE), kw.get("nb", ws), None)
    assert g(nb=ws - 1) == PA_ERR_WORKSPACE
    assert g(ws=ctypes.c_void_p(0x100010)) == PA_ERR_ALIGN
    assert g(ws=None) == PA_ERR_NULL


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits non-zero with a message,
    before anything touches a device."""
    import subprocess
    import sys
    bench = os.path.join(ROOT, "bench.py")
    r = subprocess.run([sys.executable, bench, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""
