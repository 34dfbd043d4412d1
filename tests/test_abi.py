"""The C ABI on the CPU: every function include/kvevict.h declares is exported,
argument validation rejects bad calls before anything is enqueued, and the
host-side filter tools agree with the oracle (Q-Filters page, "Calibrated",
"Key-SVD fallback", "Usage" and "Evidence")."""
import ctypes
import os
import re
import zipfile

import numpy as np
import pytest

from kv_cache_token_amd import _lib, api, synth
from kv_cache_token_amd._lib import KvxError
from oracle import calib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvevict.h")
D = 128


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"KVX_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 18, names
    L = _lib.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(api.exported_names()) == names
    assert L.kvx_abi_version() == 1


def _rc(fn, *args):
    rc = getattr(_lib.lib(), fn)(*args)
    return rc, _lib.lib().kvx_last_error().decode()


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first
C1, C2, C3, C4 = (ctypes.c_void_p(0x1000 * (i + 2)) for i in range(4))


def test_validation_rejects_bad_calls_without_launching():
    sh = api.make_shape(2, 1, 4, "bf16")
    ok = api.make_params(64, 4, 8, "low")
    cases = [
        ("kv_evict_topk", (FAKE, FAKE, sh, 0, 100, api.make_params(64, 60, 4, "low"), FAKE, None, 0, None), -1),
        ("kv_evict_topk", (FAKE, FAKE, sh, 65, 10, ok, FAKE, None, 0, None), -1),
        ("kv_evict_topk", (FAKE, FAKE, sh, 0, 10, api.make_params(64, 0, 0, 7), FAKE, None, 0, None), -1),
        ("kv_evict_topk", (FAKE, FAKE, sh, 0, 10, api.make_params((1 << 21) + 1, 4, 0, "low"), FAKE, None, 0, None), -2),
        ("kv_evict_topk", (FAKE, FAKE, sh, 1 << 21, (1 << 21) + 1, api.make_params(1 << 21, 4, 0, "low"), FAKE, None, 0,
                           None), -2),
        ("kv_evict_topk", (FAKE, FAKE, sh, 0, 300000, api.make_params(150000, 4, 0, "low"), FAKE, None, 0, None),
         -1),                                                                       # workspace missing
        ("kv_evict_topk", (FAKE, FAKE, api.KvxShape(2, 1, 4, 32, 1), 0, 10, ok, FAKE, None, 0, None), -1),
        ("kv_evict_topk", (FAKE, FAKE, api.KvxShape(2, 1, 4, 512, 1), 0, 10, ok, FAKE, None, 0, None), -1),
        ("kv_evict_topk", (FAKE, FAKE, api.KvxShape(2, 1, 4, 128, 5), 0, 10, ok, FAKE, None, 0, None), -1),
        ("kv_evict_topk", (FAKE, FAKE, api.KvxShape(2, 1, 4, 128, 3), 0, 10, ok, FAKE, None, 0, None), -1),
        ("kv_evict_topk", (FAKE, FAKE, sh, 0, -1, ok, FAKE, None, 0, None), -1),
        ("qf_score_keys", (FAKE, sh, 10, 1, None, 1, FAKE, None), -1),
        ("qf_score_keys", (FAKE, sh, 10, 1, FAKE, 2, FAKE, None), -1),
        ("qf_score_keys", (FAKE, sh, 10, 9, FAKE, 1, FAKE, None), -1),
        ("qf_score_keys", (FAKE, sh, 10, 0x200, FAKE, 1, FAKE, None), -1),
        ("qf_score_keys", (FAKE, sh, 10, 0x102, FAKE, 1, FAKE, None), -1),
        ("qf_score_keys", (FAKE, api.KvxShape(2, 1, 4, 128, 1), 2 ** 30, 0, None, 1, FAKE, None), -2),
        ("kv_compact_gather", (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, sh, 10, 10, ok,
                               FAKE, ctypes.c_void_p(0x2000), FAKE, FAKE, None), -1),      # partial alias
        ("kv_compact_gather", (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, sh, 60, 10, ok,
                               FAKE, FAKE, FAKE, FAKE, None), -1),                          # in place + evict
        ("kv_compact_gather", (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None, sh, 60, 10, ok,
                               ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000), ctypes.c_void_p(0x5000),
                               ctypes.c_void_p(0x6000), None), -1),                         # evict needs keep_idx
        ("kv_compact_gather", (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2 ** 31, FAKE, sh, 10, 10, ok,
                               FAKE, FAKE, FAKE, FAKE, None), -2),
        ("kv_evict_one_inplace", (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, sh, 65, ok, None), -1),
        ("kv_evict_one_inplace", (None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, sh, 64, ok, None), -1),
        ("kv_passthrough_append", (FAKE, FAKE, 10, 8, FAKE, FAKE, 1, sh, FAKE, FAKE, FAKE, 20, None), -1),
        ("kv_passthrough_append", (FAKE, FAKE, 5, 8, FAKE, FAKE, 4, sh, FAKE, FAKE, FAKE, 8, None), -1),
        ("kv_passthrough_append", (None, None, 5, 8, FAKE, FAKE, 1, sh, FAKE, FAKE, FAKE, 8, None), -1),
        ("kv_passthrough_append", (FAKE, FAKE, 5, 8, FAKE, FAKE, 1, sh, FAKE, FAKE, FAKE, 127, None), -1),  # overlap
        ("kv_passthrough_append", (None, None, 0, 0, FAKE, FAKE, 8, sh, FAKE, FAKE, FAKE, 8, None), -1),   # new = out
        ("kv_passthrough_append", (None, None, 0, 0, FAKE, FAKE, 1, api.KvxShape(2, 1, 4, 96, 1),
                                   FAKE, FAKE, FAKE, 8, None), -1),
        ("qf_filters_from_keys_device", (FAKE, 1, 4, 1, 8, 128, FAKE, FAKE, 100, None), -1),
        ("qf_filters_from_keys_device", (FAKE, 1, 4, 16, 8, 128, FAKE, FAKE, 100, None), -1),
        ("qf_filters_from_keys_device", (FAKE, 1, 4, 16, 16, 128, FAKE, FAKE, 0, None), -1),
        ("qf_filters_from_keys_device", (FAKE, 1, 4, 16, 16, 256, FAKE, FAKE, 100, None), -2),
        ("qf_filters_from_keys_device", (FAKE, 7, 4, 16, 16, 128, FAKE, FAKE, 100, None), -1),
        ("qf_filters_from_keys_device", (FAKE, 1, 4, 16, 16, 128, None, FAKE, 100, None), -1),
        ("qf_filters_from_queries_device", (FAKE, 1, 2, 6, 100, 128, 4, FAKE, FAKE, 100, None), -1),  # 6 % 4
        ("qf_filters_from_queries_device", (FAKE, 1, 2, 6, 0, 128, 2, FAKE, FAKE, 100, None), -1),
        ("qf_filters_from_queries_device", (FAKE, 1, 2, 6, 100, 256, 2, FAKE, FAKE, 100, None), -2),
        ("qf_filters_from_queries_device", (FAKE, 1, 2, 6, 100, 128, 2, FAKE, FAKE, 0, None), -1),
        ("qf_filters_from_queries_device", (None, 1, 2, 6, 100, 128, 2, FAKE, FAKE, 100, None), -1),
        ("kv_score_append", (FAKE, FAKE, sh, 10, 0, None, 1, 0, 60, ok, C1, C2, C3, C4, None, None), -1),  # evicts
        ("kv_score_append", (FAKE, FAKE, sh, 10, 1, None, 1, 0, 0, ok, C1, C2, C3, C4, None, None), -1),   # no filter
        ("kv_score_append", (FAKE, FAKE, sh, 10, 1, FAKE, 3, 0, 0, ok, C1, C2, C3, C4, None, None), -1),   # sign
        ("kv_score_append", (FAKE, FAKE, sh, 10, 7, FAKE, 1, 0, 0, ok, C1, C2, C3, C4, None, None), -1),   # mode
        ("kv_score_append", (FAKE, FAKE, sh, 10, 0, None, 1, 0, 0, ok, FAKE, C2, C3, C4, None, None), -1),  # alias
        ("kv_score_append", (FAKE, FAKE, sh, 10, 0, None, 1, 2 ** 31, 0, ok, C1, C2, C3, C4, None, None), -2),
        ("kv_score_append", (None, FAKE, sh, 10, 0, None, 1, 0, 0, ok, C1, C2, C3, C4, None, None), -1),   # NULL
    ]
    for fn, args, want in cases:
        rc, msg = _rc(fn, *args)
        assert rc == want, (fn, rc, msg)
        assert msg, fn
    # zero groups or zero rows: nothing to do, nothing launched
    assert _rc("qf_score_keys", None, api.KvxShape(0, 1, 4, 128, 1), 10, 0, None, 1, None, None)[0] == 0
    assert _rc("kv_evict_topk", None, None, sh, 0, 0, ok, None, None, 0, None)[0] == 0
    assert _rc("kv_passthrough_append", None, None, 0, 8, None, None, 0, sh, FAKE, FAKE, FAKE, 8, None)[0] == 0
    assert _rc("qf_filters_from_keys_device", None, 1, 0, 16, 16, 128, None, None, 100, None)[0] == 0
    assert _rc("kv_score_append", None, None, sh, 0, 0, None, 1, 0, 5, ok, None, None, None, None, None, None)[0] == 0
    n = ctypes.c_size_t(99)
    assert _rc("kv_evict_workspace_size", sh, 64, 1, ok, ctypes.byref(n))[0] == 0 and n.value == 0


def test_artifact_round_trip_and_mismatches(tmp_path):
    rng = np.random.default_rng(0)
    f = rng.standard_normal((3, 2, D)).astype(np.float32)
    p1 = str(tmp_path / "oracle_written.npz")
    calib.save_artifact(p1, f, "org/model-a", 3000, "pile-subset")
    got, ns = api.qf_filters_load(p1, 3, 2, "org/model-a")
    assert np.array_equal(got, f) and ns == 3000
    got, _ = api.qf_filters_load(p1, 3, 2, None)
    assert np.array_equal(got, f)
    p2 = str(tmp_path / "lib_written.npz")
    api.qf_filters_save(p2, f, "org/model-ü", 12, "synthetic")
    z = np.load(p2)
    assert np.array_equal(z["filters"], f) and str(z["model_id"]) == "org/model-ü"
    assert int(z["version"]) == 1 and int(z["n_samples"]) == 12 and str(z["dataset"]) == "synthetic"
    assert np.array_equal(api.qf_filters_load(p2, 3, 2, "org/model-ü")[0], f)
    expect = [
        (dict(L=3, H_kv=2, expect_model_id="org/other"), _lib.KVX_EMISMATCH),
        (dict(L=4, H_kv=2, expect_model_id=None), _lib.KVX_EMISMATCH),      # missing layer
        (dict(L=3, H_kv=4, expect_model_id=None), _lib.KVX_EMISMATCH),      # head layout
    ]
    for kw, code in expect:
        with pytest.raises(KvxError) as e:
            api.qf_filters_load(p1, **kw)
        assert e.value.code == code
    p3 = str(tmp_path / "v2.npz")
    np.savez(p3, filters=f, model_id=np.array("m"), version=np.array(2, np.int64),
             n_samples=np.array(1, np.int64), dataset=np.array("d"))
    with pytest.raises(KvxError) as e:
        api.qf_filters_load(p3, 3, 2)
    assert e.value.code == _lib.KVX_EMISMATCH
    p4 = str(tmp_path / "missing.npz")
    np.savez(p4, filters=f, model_id=np.array("m"), version=np.array(1, np.int64))
    with pytest.raises(KvxError) as e:
        api.qf_filters_load(p4, 3, 2)
    assert e.value.code == _lib.KVX_EIO
    p5 = str(tmp_path / "deflated.npz")
    np.savez_compressed(p5, filters=f, model_id=np.array("m"), version=np.array(1, np.int64),
                        n_samples=np.array(1, np.int64), dataset=np.array("d"))
    with pytest.raises(KvxError) as e:
        api.qf_filters_load(p5, 3, 2)
    assert e.value.code == _lib.KVX_EIO
    with pytest.raises(KvxError) as e:
        api.qf_filters_load(str(tmp_path / "absent.npz"), 3, 2)
    assert e.value.code == _lib.KVX_EIO
    assert zipfile.is_zipfile(p2)


def test_corrupt_artifacts_are_rejected(tmp_path):
    """A flipped byte in a member fails its CRC-32; offsets and sizes that point
    past the file (including ones that would wrap 64-bit arithmetic) and
    truncations are refused, never read."""
    import struct
    f = np.random.default_rng(2).standard_normal((3, 2, D)).astype(np.float32)
    good = str(tmp_path / "good.npz")
    api.qf_filters_save(good, f, "m", 1, "d")
    raw = bytearray(open(good, "rb").read())
    pos = raw.find(f.tobytes()[:16])
    assert pos > 0
    cases = {}
    flipped = bytearray(raw)
    flipped[pos + 100] ^= 0x01
    cases["flipped"] = flipped
    cases["truncated"] = raw[: len(raw) // 2]
    eocd = raw.rfind(b"PK\x05\x06")
    cd_off = struct.unpack_from("<I", raw, eocd + 16)[0]
    for name, field, value in (("cd_offset", eocd + 16, 0xFFFFFFF0), ("local_offset", cd_off + 42, 0xFFFFFFF0),
                               ("size", cd_off + 20, 0xFFFFFFF0)):
        b = bytearray(raw)
        struct.pack_into("<I", b, field, value)
        if name == "size":
            struct.pack_into("<I", b, cd_off + 24, value)
        cases[name] = b
    # a zip64 end record whose central directory offset wraps around 2^64
    b = bytearray(raw)
    struct.pack_into("<I", b, eocd + 16, 0xFFFFFFFF)
    loc = struct.pack("<IIQI", 0x07064B50, 0, eocd, 1)   # the zip64 record sits where the end record was
    z64 = struct.pack("<IQHHIIQQQQ", 0x06064B50, 44, 45, 45, 0, 0, 5, 5, 100, 2 ** 64 - 8)
    cases["zip64_wrap"] = bytes(b[:eocd]) + z64 + loc + bytes(b[eocd:])
    for name, data in cases.items():
        p = str(tmp_path / (name + ".npz"))
        open(p, "wb").write(bytes(data))
        with pytest.raises(KvxError) as e:
            api.qf_filters_load(p, 3, 2)
        assert e.value.code == _lib.KVX_EIO, name


def test_malformed_member_headers_are_rejected(tmp_path):
    """.npy headers cut off inside a field -- no value after 'fortran_order',
    an unclosed shape, an unclosed descr string -- in members whose CRC-32 is
    right: the reader refuses them with KVX_EIO (and does not abort)."""
    import struct
    import zipfile
    for name, header in (("fortran_cut", "{'descr': '<f4', 'fortran_order':   "),
                         ("shape_cut", "{'descr': '<f4', 'fortran_order': False, 'shape': (3, 2, "),
                         ("descr_cut", "{'descr': '<f4")):
        h = header.encode("latin-1")
        p = str(tmp_path / (name + ".npz"))
        with zipfile.ZipFile(p, "w", zipfile.ZIP_STORED) as z:
            z.writestr("filters.npy", b"\x93NUMPY\x01\x00" + struct.pack("<H", len(h)) + h)
        with pytest.raises(KvxError) as e:
            api.qf_filters_load(p, 3, 2)
        assert e.value.code == _lib.KVX_EIO and "not a valid .npy" in str(e.value), name


@pytest.mark.skipif("asan" in os.environ.get("LD_PRELOAD", ""),
                    reason="under AddressSanitizer a throwing operator new aborts on exhausted memory")
def test_host_estimators_report_exhausted_memory_as_a_status():
    """A host estimate whose working copy cannot be allocated (2^40 rows per
    head) returns KVX_ERANGE with a message, from the calling thread (one
    head) and from the worker threads (several heads); the inputs are not
    read before the allocation."""
    q = np.zeros(16, dtype=np.float32)
    out = np.zeros(4 * D, dtype=np.float32)
    for H_q in (1, 4):
        rc = _lib.lib().qf_filters_from_queries(q.ctypes.data, H_q, 1 << 40, D, 1, out.ctypes.data)
        assert rc == _lib.KVX_ERANGE and b"out of host memory" in _lib.lib().kvx_last_error(), H_q
        rc = _lib.lib().qf_filters_from_keys(q.ctypes.data, _lib.KVX_F32, H_q, 1 << 40, 1 << 40, D, out.ctypes.data)
        assert rc == _lib.KVX_ERANGE and b"out of host memory" in _lib.lib().kvx_last_error(), H_q


def test_query_filters_match_oracle():
    rng = np.random.default_rng(1)
    Hq, N, Hkv = 24, 600, 8
    mus = rng.standard_normal((Hq, D))
    mus /= np.linalg.norm(mus, axis=1, keepdims=True)
    q = (rng.uniform(0.5, 2, (Hq, N, 1)) * mus[:, None] + 0.5 * rng.standard_normal((Hq, N, D))).astype(np.float32)
    got = api.qf_filters_from_queries(q, Hkv)
    want = calib.average_gqa_filters(calib.compute_qfilters(q.astype(np.float64)), Hkv)
    cos = np.sum(got.astype(np.float64) * want, axis=1)
    assert np.all(np.abs(cos - 1) < 1e-6) and np.all(np.abs(np.linalg.norm(got, axis=1) - 1) < 1e-6)
    assert np.max(np.abs(got - want.astype(np.float32))) <= 1e-7
    with pytest.raises(KvxError):
        api.qf_filters_from_queries(q, 5)
    with pytest.raises(KvxError):
        api.qf_filters_from_queries(np.zeros((2, 10, D), np.float32), 1)


def test_key_filters_match_oracle_on_fallback_workload():
    cfg = synth.CONFIGS[5]
    groups = [0, 77, 255]
    K = np.stack([synth.group_chunk(cfg, g, 0)[0][:cfg.calib_tokens] for g in groups])
    got = api.qf_filters_from_keys(K, cfg.calib_tokens)
    kw = synth.bf16_bits_to_f32(K).astype(np.float64)
    want = np.stack([calib.estimate_filter_dir(kw[i]) for i in range(len(groups))])
    cos = np.sum(got.astype(np.float64) * want, axis=1)
    assert np.all(cos > 1 - 1e-6), cos
    for i in range(len(groups)):
        j = np.argmax(np.abs(got[i]))
        assert got[i, j] > 0
    # an interleaved stride reads only the first n rows of each group
    Kbig = np.stack([synth.group_chunk(cfg, g, 0)[0][:300] for g in groups])
    assert np.array_equal(api.qf_filters_from_keys(Kbig, cfg.calib_tokens), got)
    with pytest.raises(KvxError):
        api.qf_filters_from_keys(np.ones((1, 10, D), np.float32), 10)


def test_key_filters_read_f16_and_fp32_rows_like_bf16():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((2, 200, D)) * 0.5 + rng.standard_normal(D) * 0.2).astype(np.float32)
    for dt in ("f16", "bf16"):
        bits = synth.encode(x, dt)
        got = api.qf_filters_from_keys(bits, 128, dt)
        exact = api.qf_filters_from_keys(synth.bits_to_f32(bits, dt), 128)
        assert np.array_equal(got, exact)


def test_byte_accounting():
    st = api.kvx_stats(api.make_shape(28, 1, 8, "bf16"), 4096, 512, "proj")
    row = 2 * D * 2
    assert st["kept_bytes"] == 224 * 512 * row and st["full_seq_bytes"] == 224 * 4096 * row
    assert st["compression_ratio"] == 8.0 and st["filter_bytes"] == 28 * 8 * D * 4
    assert api.kvx_stats(api.make_shape(1, 1, 1, "f32"), 10, 10, "l2")["filter_bytes"] == 0
    assert api.kvx_stats(api.make_shape(1, 1, 1, "f16", 64), 10, 5, "l2")["kept_bytes"] == 5 * 2 * 64 * 2
    with pytest.raises(KvxError):
        api.kvx_stats(api.make_shape(1, 1, 1, "f32"), 10, 11, "l2")


def test_missing_library_fails_loudly(tmp_path):
    """No CPU fallback: without the built library every entry point raises."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from kv_cache_token_amd import _lib, api\n"
            "_lib.LIB_PATH = %r\n"
            "try:\n"
            "    api.kvx_stats(api.make_shape(1, 1, 1, 'bf16'), 1, 1, 'l2')\n"
            "except ImportError as e:\n"
            "    print('raised', e)\n" % (os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                           str(tmp_path / "absent.so")))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert "raised" in out.stdout and "not built" in out.stdout, out.stdout + out.stderr


def test_checked_build_exports_the_same_abi_and_only_it_takes_a_status_word():
    """libkvevict_check.so (-DKVX_CHECK) has every symbol of the header; the
    normal build refuses a status word, the checked one records where it is
    (nothing is launched either way)."""
    names = declared_functions()
    with _lib.checked() as L:
        for n in names:
            assert hasattr(L, n), n
        assert L.kvx_check_status_word(FAKE) == 0
        assert L.kvx_check_status_word(None) == 0
    assert _lib.lib().kvx_check_status_word(FAKE) == -1
    assert b"KVX_CHECK" in _lib.lib().kvx_last_error()
    assert _lib.lib().kvx_check_status_word(None) == 0


def test_library_path_follows_the_environment_override():
    """KVX_LIB / KVX_ORACLE_LIB (the sanitizer run) name the libraries that are
    loaded; without them the in-tree builds are."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from kv_cache_token_amd import _lib\n"
            "import oracle\n"
            "print(_lib.LIB_PATH); print(oracle._LIB)\n" % root)
    env = dict(os.environ, KVX_LIB="/x/a.so", KVX_ORACLE_LIB="/x/b.so")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, env=env)
    assert out.stdout.split() == ["/x/a.so", "/x/b.so"], out.stdout + out.stderr
    env.pop("KVX_LIB")
    env.pop("KVX_ORACLE_LIB")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, env=env)
    assert out.stdout.split() == [os.path.join(root, "kv_cache_token_amd", "libkvevict.so"),
                                  os.path.join(root, "oracle", "libkvx_oracle.so")]


def test_plain_c_caller(tmp_path):
    """include/kvevict.h compiles as strict C11 and the library links and
    answers from C (tests/abi_c/abi_check.c): host entry points, and device
    entry points refusing bad arguments before anything is enqueued."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = str(tmp_path / "abi_check")
    libdir = os.path.dirname(_lib.LIB_PATH)
    # a sanitized library (build.py --sanitize) links against the sanitizer runtime it preloads
    preload = os.environ.get("LD_PRELOAD", "")
    san_runtime = [preload] if "asan" in preload else []
    subprocess.check_call([gcc, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror",
                           "-I", os.path.join(root, "include"), os.path.join(root, "tests", "abi_c", "abi_check.c"),
                           "-o", exe, "-L", libdir, "-l:" + os.path.basename(_lib.LIB_PATH), "-lm",
                           "-Wl,-rpath," + libdir] + san_runtime)
    art = str(tmp_path / "filters.npz")
    out = subprocess.run([exe, art], capture_output=True, text=True, check=True).stdout
    got = dict(line.split(" ", 1) for line in out.strip().splitlines())
    want = {"abi_version": "1", "workspace_rc": "0", "workspace_onchip": "0",
            "workspace_multiblock": str(224 * (260 + 2 * 128) * 4),
            "topk_bad_params": str(_lib.KVX_EINVAL), "topk_null_idx": str(_lib.KVX_EINVAL),
            "score_bad_mode": str(_lib.KVX_EINVAL), "score_proj_no_filters": str(_lib.KVX_EINVAL),
            "score_bad_head_dim": str(_lib.KVX_EINVAL), "gather_partial_alias": str(_lib.KVX_EINVAL),
            "decode_position_range": str(_lib.KVX_ERANGE), "last_error_mentions_int32": "1",
            "save": "0", "load": "0", "load_same": "1", "load_other_model": str(_lib.KVX_EMISMATCH),
            "load_missing_layer": str(_lib.KVX_EMISMATCH), "from_queries": "0", "from_queries_unit": "1",
            "from_queries_axis": "1", "stats": "0", "stats_ratio": "8.0"}
    assert got == want
    z = np.load(art)
    assert z["filters"].shape == (2, 2, 4) and str(z["model_id"]) == "org/model" and int(z["n_samples"]) == 7
