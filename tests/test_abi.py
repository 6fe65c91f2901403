"""The C-ABI library loads, exports what include/q8kv.h declares, and rejects
bad arguments on the host before any HIP call (CPU only: no compute call is
made; every call here returns from argument validation)."""
import ctypes

import pytest

import decode_attention_int8_amd as q8

L = q8.lib
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
NUL = ctypes.c_void_p(0)


def test_exports_every_declared_symbol():
    names = q8.header_symbols()
    assert len(names) == 22
    for n in names:
        assert hasattr(L, n), n


def decode(**kw):
    a = dict(out=FAKE, q=FAKE, kp=FAKE, vp=FAKE, ks=FAKE, vs=FAKE, bt=FAKE, sl=FAKE,
             max_blocks=8, num_blocks=16, batch=2, n_q=8, n_kv=2, hd=128, kv_bs=16,
             scale=0.088, part=0)
    a.update(kw)
    return L.q8kv_decode_attn_split(a["out"], a["q"], a["kp"], a["vp"], a["ks"], a["vs"], a["bt"],
                                    a["sl"], a["max_blocks"], a["num_blocks"], a["batch"], a["n_q"],
                                    a["n_kv"], a["hd"], a["kv_bs"], a["scale"], a["part"], NUL)


def fp8_decode(**kw):
    a = dict(out=FAKE, q=FAKE, kp=FAKE, vp=FAKE, ks=FAKE, vs=FAKE, bt=FAKE, sl=FAKE,
             max_blocks=8, num_blocks=16, batch=2, n_q=8, n_kv=2, hd=128, kv_bs=16,
             scale=0.088, part=0)
    a.update(kw)
    return L.q8kv_fp8_decode_attn(a["out"], a["q"], a["kp"], a["vp"], a["ks"], a["vs"], a["bt"],
                                  a["sl"], a["max_blocks"], a["num_blocks"], a["batch"], a["n_q"],
                                  a["n_kv"], a["hd"], a["kv_bs"], a["scale"], a["part"], NUL)


@pytest.mark.parametrize("kw,code", [
    (dict(ks=NUL), q8.Q8KV_ENULL),
    (dict(vs=NUL), q8.Q8KV_ENULL),
    (dict(kp=NUL), q8.Q8KV_ENULL),
    (dict(sl=NUL), q8.Q8KV_ENULL),
    (dict(hd=96), q8.Q8KV_EINVAL),
    (dict(kv_bs=8), q8.Q8KV_EINVAL),
    (dict(n_q=18, n_kv=4), q8.Q8KV_EINVAL),
    (dict(scale=float("nan")), q8.Q8KV_EINVAL),
    (dict(part=48), q8.Q8KV_EINVAL),
])
def test_fp8_decode_rejects_before_any_hip_call(kw, code):
    assert fp8_decode(**kw) == code
    assert q8.last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(kp=NUL), q8.Q8KV_ENULL),
    (dict(ks=NUL), q8.Q8KV_ENULL),
    (dict(sm=NUL), q8.Q8KV_ENULL),
    (dict(n=-1), q8.Q8KV_EINVAL),
    (dict(hd=96), q8.Q8KV_EINVAL),
    (dict(dt=3), q8.Q8KV_EINVAL),
    (dict(num_blocks=0), q8.Q8KV_EINVAL),
])
def test_fp8_append_rejects_before_any_hip_call(kw, code):
    a = dict(kp=FAKE, vp=FAKE, ks=FAKE, vs=FAKE, kx=FAKE, vx=FAKE, dt=0, sm=FAKE, n=4, num_blocks=16,
             n_kv=2, hd=128, kv_bs=16)
    a.update(kw)
    rc = L.q8kv_fp8_append(a["kp"], a["vp"], a["ks"], a["vs"], a["kx"], a["vx"], a["dt"], a["sm"], a["n"],
                           a["num_blocks"], a["n_kv"], a["hd"], a["kv_bs"], NUL)
    assert rc == code
    assert q8.last_error() != ""


def append_decode(**kw):
    a = dict(out=FAKE, q=FAKE, kn=FAKE, vn=FAKE, dt=0, kp=FAKE, vp=FAKE, ks=FAKE, vs=FAKE, bt=FAKE,
             sl=FAKE, max_blocks=8, num_blocks=16, batch=2, n_q=8, n_kv=2, hd=128, kv_bs=16,
             scale=0.088, part=0)
    a.update(kw)
    return L.q8kv_append_decode_attn(a["out"], a["q"], a["kn"], a["vn"], a["dt"], a["kp"], a["vp"],
                                     a["ks"], a["vs"], a["bt"], a["sl"], a["max_blocks"],
                                     a["num_blocks"], a["batch"], a["n_q"], a["n_kv"], a["hd"],
                                     a["kv_bs"], a["scale"], a["part"], NUL)


@pytest.mark.parametrize("kw,code", [
    (dict(kn=NUL), q8.Q8KV_ENULL),
    (dict(vn=NUL), q8.Q8KV_ENULL),
    (dict(kp=NUL), q8.Q8KV_ENULL),
    (dict(out=NUL), q8.Q8KV_ENULL),
    (dict(dt=2), q8.Q8KV_EINVAL),
    (dict(dt=-1), q8.Q8KV_EINVAL),
    (dict(hd=80), q8.Q8KV_EINVAL),
    (dict(n_q=6, n_kv=4), q8.Q8KV_EINVAL),
    (dict(batch=0), q8.Q8KV_EINVAL),
    (dict(part=48), q8.Q8KV_EINVAL),
])
def test_append_decode_rejects_before_any_hip_call(kw, code):
    assert append_decode(**kw) == code
    assert q8.last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(out=NUL), q8.Q8KV_ENULL),
    (dict(q=NUL), q8.Q8KV_ENULL),
    (dict(kp=NUL), q8.Q8KV_ENULL),
    (dict(vs=NUL), q8.Q8KV_ENULL),
    (dict(bt=NUL), q8.Q8KV_ENULL),
    (dict(sl=NUL), q8.Q8KV_ENULL),
    (dict(batch=0), q8.Q8KV_EINVAL),
    (dict(batch=2049), q8.Q8KV_EINVAL),  # at most 2048 sequences per call
    (dict(n_q=0), q8.Q8KV_EINVAL),
    (dict(n_kv=0), q8.Q8KV_EINVAL),
    (dict(n_q=6, n_kv=4), q8.Q8KV_EINVAL),
    (dict(hd=80), q8.Q8KV_EINVAL),     # not a multiple of 32
    (dict(hd=0), q8.Q8KV_EINVAL),
    (dict(hd=288), q8.Q8KV_EINVAL),
    (dict(hd=512), q8.Q8KV_EINVAL),
    (dict(kv_bs=8), q8.Q8KV_EINVAL),
    (dict(kv_bs=48), q8.Q8KV_EINVAL),
    (dict(max_blocks=0), q8.Q8KV_EINVAL),
    (dict(max_blocks=1 << 30), q8.Q8KV_EINVAL),
    (dict(num_blocks=0), q8.Q8KV_EINVAL),
    (dict(num_blocks=1 << 30), q8.Q8KV_EINVAL),
    (dict(scale=float("inf")), q8.Q8KV_EINVAL),
    (dict(scale=float("nan")), q8.Q8KV_EINVAL),
    (dict(part=48), q8.Q8KV_EINVAL),
    (dict(part=-32), q8.Q8KV_EINVAL),
])
def test_decode_rejects_before_any_hip_call(kw, code):
    assert decode(**kw) == code
    assert q8.last_error() != ""


def test_append_rejects():
    def ap(**kw):
        a = dict(kp=FAKE, vp=FAKE, ks=FAKE, vs=FAKE, ksrc=FAKE, vsrc=FAKE, dt=0, sm=FAKE,
                 n=4, nb=8, n_kv=2, hd=128, kv_bs=16)
        a.update(kw)
        return L.q8kv_append(a["kp"], a["vp"], a["ks"], a["vs"], a["ksrc"], a["vsrc"], a["dt"],
                             a["sm"], a["n"], a["nb"], a["n_kv"], a["hd"], a["kv_bs"], NUL)
    assert ap(kp=NUL) == q8.Q8KV_ENULL
    assert ap(sm=NUL) == q8.Q8KV_ENULL
    assert ap(dt=2) == q8.Q8KV_EINVAL
    assert ap(n=-1) == q8.Q8KV_EINVAL
    assert ap(hd=100) == q8.Q8KV_EINVAL
    assert ap(hd=16) == q8.Q8KV_EINVAL
    assert ap(hd=288) == q8.Q8KV_EINVAL
    assert ap(kv_bs=24) == q8.Q8KV_EINVAL
    assert ap(nb=0) == q8.Q8KV_EINVAL
    assert ap(n=0) == q8.Q8KV_OK  # nothing to do: no launch


def test_debug_exports_reject():
    assert L.q8kv_debug_quantize_q(NUL, FAKE, FAKE, 4, 128, NUL) == q8.Q8KV_ENULL
    assert L.q8kv_debug_quantize_q(FAKE, FAKE, FAKE, 4, 100, NUL) == q8.Q8KV_EINVAL
    assert L.q8kv_debug_quantize_q(FAKE, FAKE, FAKE, 4, 96, NUL) == q8.Q8KV_EINVAL
    assert L.q8kv_debug_quantize_q(FAKE, FAKE, FAKE, 0, 128, NUL) == q8.Q8KV_OK
    assert L.q8kv_debug_block_dots(FAKE, 4, FAKE, FAKE, FAKE, FAKE, 4, 8, 1, 3, 2, 128, 16, NUL) == q8.Q8KV_EINVAL
    assert L.q8kv_debug_block_dots(NUL, 4, FAKE, FAKE, FAKE, FAKE, 4, 8, 1, 2, 2, 128, 16, NUL) == q8.Q8KV_ENULL


def test_set_wide_accepts_only_0_and_1():
    assert L.q8kv_debug_set_wide(2) == q8.Q8KV_EINVAL
    assert L.q8kv_debug_set_wide(-1) == q8.Q8KV_EINVAL
    assert L.q8kv_debug_set_wide(0) == q8.Q8KV_OK
    assert L.q8kv_debug_set_wide(1) == q8.Q8KV_OK  # the default again


def test_set_stage_accepts_only_0_and_1():
    assert L.q8kv_debug_set_stage(2) == q8.Q8KV_EINVAL
    assert L.q8kv_debug_set_stage(-1) == q8.Q8KV_EINVAL
    assert L.q8kv_debug_set_stage(1) == q8.Q8KV_OK
    assert L.q8kv_debug_set_stage(0) == q8.Q8KV_OK  # the default again


def test_stream_read_rejects():
    assert L.q8kv_debug_stream_read(NUL, 16, FAKE, 16, NUL) == q8.Q8KV_ENULL
    assert L.q8kv_debug_stream_read(FAKE, 17, FAKE, 16, NUL) == q8.Q8KV_EINVAL


def test_plan_counts_head_groups():
    """More than 8 query heads per kv head run as several head-group work
    items (the largest divisor of the group size up to 8 heads each), so the
    plan sees n_kv * groups item heads: 64 / 4 heads plan like 64 / 8."""
    assert q8.plan(1, 64, 4, 128, 64, 2048) == q8.plan(1, 64, 8, 128, 64, 2048)
    assert q8.plan(2, 36, 2, 128, 16, 256) == q8.plan(2, 36, 6, 128, 16, 256)   # 18 = 3 x 6
    assert q8.plan(1, 13, 1, 64, 16, 64) == q8.plan(1, 13, 13, 64, 16, 64)     # prime: 13 x 1


def test_plan_is_shape_only_and_sane():
    for shape in [(1, 32, 4, 128, 64, 2048), (1, 32, 32, 128, 16, 256), (16, 32, 8, 128, 16, 512),
                  (64, 64, 8, 128, 64, 512), (1, 1, 1, 128, 16, 32), (3, 8, 8, 64, 256, 1)]:
        pt, npart = q8.plan(*shape)
        max_tok = shape[4] * shape[5]
        assert pt % 128 == 0 and 128 <= pt and npart <= 256
        assert npart == -(-max_tok // pt)
        assert q8.plan(*shape) == (pt, npart)
    with pytest.raises(q8.Q8KVError):
        q8.plan(1, 3, 2, 128, 16, 4)


def test_release_without_workspace_is_ok():
    q8.release()


@pytest.mark.parametrize("kw,code", [
    (dict(sel=NUL), q8.Q8KV_ENULL),
    (dict(kmax=NUL), q8.Q8KV_ENULL),
    (dict(top_k=0), q8.Q8KV_EINVAL),
    (dict(max_blocks=5000), q8.Q8KV_EINVAL),
    (dict(n_q=18, n_kv=2), q8.Q8KV_EINVAL),
    (dict(n_q=6, n_kv=4), q8.Q8KV_EINVAL),
    (dict(hd=96), q8.Q8KV_EINVAL),
])
def test_quest_select_rejects_before_any_hip_call(kw, code):
    a = dict(sel=FAKE, sl_out=FAKE, q=FAKE, kmax=FAKE, kmin=FAKE, bt=FAKE, sl=FAKE, max_blocks=8,
             num_blocks=16, batch=2, n_q=8, n_kv=2, hd=128, kv_bs=16, top_k=4)
    a.update(kw)
    rc = L.q8kv_quest_select(a["sel"], a["sl_out"], a["q"], a["kmax"], a["kmin"], a["bt"], a["sl"],
                             a["max_blocks"], a["num_blocks"], a["batch"], a["n_q"], a["n_kv"], a["hd"],
                             a["kv_bs"], a["top_k"], NUL)
    assert rc == code
    assert q8.last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(kmax=NUL), q8.Q8KV_ENULL),
    (dict(kp=NUL), q8.Q8KV_ENULL),
    (dict(batch=0), q8.Q8KV_EINVAL),
    (dict(max_blocks=0), q8.Q8KV_EINVAL),
    (dict(kv_bs=24), q8.Q8KV_EINVAL),
    (dict(hd=96), q8.Q8KV_EINVAL),   # the QUEST kernels take 64, 128 or 256
])
def test_quest_metadata_rejects_before_any_hip_call(kw, code):
    a = dict(kmax=FAKE, kmin=FAKE, kp=FAKE, ks=FAKE, bt=FAKE, sl=FAKE, max_blocks=8, num_blocks=16, batch=2,
             n_kv=2, hd=128, kv_bs=16)
    a.update(kw)
    rc = L.q8kv_quest_metadata(a["kmax"], a["kmin"], a["kp"], a["ks"], a["bt"], a["sl"], a["max_blocks"],
                               a["num_blocks"], a["batch"], a["n_kv"], a["hd"], a["kv_bs"], NUL)
    assert rc == code
    assert q8.last_error() != ""


def test_decode_heads_rejects_before_any_hip_call():
    rc = L.q8kv_decode_attn_heads(FAKE, FAKE, FAKE, FAKE, FAKE, NUL, FAKE, FAKE, 8, 16, 2, 8, 2, 128, 16,
                                  0.088, 0, NUL)
    assert rc == q8.Q8KV_ENULL
    rc = L.q8kv_decode_attn_heads(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 2, 8, 2, 100, 16,
                                  0.088, 0, NUL)
    assert rc == q8.Q8KV_EINVAL


def import_pages(**kw):
    # destination at 0x100000.., sources 1 MB further on: 2 blocks x 2 kv heads
    # x 16 rows x 128 bytes = 8 KB of pages, 256 B of scales each
    a = dict(kp=0x100000, vp=0x110000, ks=0x120000, vs=0x130000,
             kr=0x200000, vr=0x210000, ksr=0x220000, vsr=0x230000,
             num_blocks=2, n_kv=2, hd=128, kv_bs=16)
    a.update(kw)
    p = [ctypes.c_void_p(a[k]) for k in ("kp", "vp", "ks", "vs", "kr", "vr", "ksr", "vsr")]
    return L.q8kv_import_pages(*p, a["num_blocks"], a["n_kv"], a["hd"], a["kv_bs"], NUL)


@pytest.mark.parametrize("kw,code", [
    (dict(kp=0), q8.Q8KV_ENULL),
    (dict(vsr=0), q8.Q8KV_ENULL),
    (dict(hd=80), q8.Q8KV_EINVAL),
    (dict(kv_bs=8), q8.Q8KV_EINVAL),
    (dict(num_blocks=0), q8.Q8KV_EINVAL),
    (dict(n_kv=0), q8.Q8KV_EINVAL),
    (dict(kr=0x100008), q8.Q8KV_EINVAL),        # misaligned source
    (dict(ks=0x120004), q8.Q8KV_EINVAL),        # misaligned destination
    (dict(kr=0x101000), q8.Q8KV_EINVAL),        # source inside k_pages
    (dict(vs=0x211f80), q8.Q8KV_EINVAL),        # v_scale runs into the end of v_rows
    (dict(ksr=0x1100f0), q8.Q8KV_EINVAL),       # k_row_scale inside v_pages
])
def test_import_pages_rejects_before_any_hip_call(kw, code):
    assert import_pages(**kw) == code
    assert q8.last_error() != ""


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """2048 sequences x 64 heads x 256 partitions of hd 256 need far more than
    the allocation-free entry's 32 MiB: rejected on the host, saying so."""
    rc = L.q8kv_decode_attn_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 131072, 2048, 64, 8,
                                    256, 256, 0.0625, 64, NUL)
    assert rc == q8.Q8KV_EINVAL
    assert "scratch" in q8.last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(kp=NUL), q8.Q8KV_ENULL),
    (dict(hd=80), q8.Q8KV_EINVAL),
    (dict(n_q=18, n_kv=4), q8.Q8KV_EINVAL),
    (dict(part=48), q8.Q8KV_EINVAL),
    (dict(scale=float("inf")), q8.Q8KV_EINVAL),
])
def test_noalloc_validates_like_split(kw, code):
    a = dict(out=FAKE, q=FAKE, kp=FAKE, vp=FAKE, ks=FAKE, vs=FAKE, bt=FAKE, sl=FAKE,
             max_blocks=8, num_blocks=16, batch=2, n_q=8, n_kv=2, hd=128, kv_bs=16, scale=0.088, part=0)
    a.update(kw)
    rc = L.q8kv_decode_attn_noalloc(a["out"], a["q"], a["kp"], a["vp"], a["ks"], a["vs"], a["bt"], a["sl"],
                                    a["max_blocks"], a["num_blocks"], a["batch"], a["n_q"], a["n_kv"], a["hd"],
                                    a["kv_bs"], a["scale"], a["part"], NUL)
    assert rc == code == decode(**kw)


def test_codec_paths_take_full_head_sizes_only():
    """The int8 cache takes any multiple of 32 up to 256 (padded pages); the
    FP8 and q4_0 kernels take 64, 128 or 256 and reject the rest on the host."""
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 16, 2, 8, 2, 96, 16, 0.088, 0, NUL)
    assert L.q8kv_q40_decode_attn(*args) == q8.Q8KV_EINVAL and "64, 128 or 256" in q8.last_error()
    assert L.q8kv_fp8_decode_attn(*args) == q8.Q8KV_EINVAL
    app = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 4, 16, 2, 96, 16, NUL)
    assert L.q8kv_q40_append(*app) == q8.Q8KV_EINVAL
    assert L.q8kv_fp8_append(*app) == q8.Q8KV_EINVAL
    assert L.q8kv_append(*app[:11], 80, 16, NUL) == q8.Q8KV_EINVAL
    assert "multiple of 32" in q8.last_error()


def test_padded_page_width():
    """int8 pages are the head size rounded up to 64, 128 or 256 wide; a
    wrapped pool names the head size it holds (host logic only)."""
    import torch
    assert [q8.page_hd(h) for h in (32, 64, 96, 128, 160, 192, 224, 256)] == [64, 64, 128, 128, 256, 256, 256, 256]
    kp = torch.zeros((2, 2, 16, 128), dtype=torch.int8)
    ks = torch.zeros((2, 2, 16), dtype=torch.float32)
    c = q8.PagedKVCache.wrap(kp, kp.clone(), ks, ks.clone(), hd=96)
    assert (c.hd, c.hp) == (96, 128)
    assert q8.PagedKVCache.wrap(kp, kp.clone(), ks, ks.clone()).hd == 128
    with pytest.raises(ValueError):
        q8.PagedKVCache.wrap(kp, kp.clone(), ks, ks.clone(), hd=64)


def test_load_probe_rejects_before_any_hip_call():
    p = lambda **kw: L.q8kv_debug_load_probe(*[kw.get(k, FAKE) for k in ("kp", "vp", "ks", "vs")],
                                             kw.get("n", 64), kw.get("hd", 128), kw.get("bs", 64),
                                             kw.get("item", 16), kw.get("pat", 0), NUL)
    assert p(kp=NUL) == q8.Q8KV_ENULL
    assert p(hd=96) == q8.Q8KV_EINVAL      # full page widths only
    assert p(bs=48) == q8.Q8KV_EINVAL
    assert p(pat=3) == q8.Q8KV_EINVAL
    assert p(n=60) == q8.Q8KV_EINVAL       # not a multiple of item_pages
    assert p(bs=16, item=4) == q8.Q8KV_EINVAL  # 64 tokens an item: not a multiple of 128
    assert p(n=0) == q8.Q8KV_EINVAL


def test_header_and_c_caller_compile_as_c(tmp_path):
    """include/q8kv.h is plain C: the C example that calls the library
    compiles and links with gcc -std=c11 -Wall -Wextra -Werror."""
    import importlib.util
    import os
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not installed")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("_q8kv_build_c", os.path.join(root, "decode_attention_int8_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    r = subprocess.run(b.example_command(str(tmp_path / "q8kv_example")), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
