"""CPU checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import block_diffusion_drafter_fuse_amd as dfa
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash_fuse.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dfa.LIB_PATH), reason="library not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b((?:dflash2?|dflow)_[a-z_]+)\s*\(", src)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert set(names) == set(dfa.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = dfa.lib()
    for n in declared_functions():
        assert hasattr(L, n), n


def _dims(**kw):
    d = synth.get_config("tiny").dims
    dims = dfa.make_dims(d, max_ctx=128, max_slots=2, max_batch=1)
    for k, v in kw.items():
        setattr(dims, k, v)
    return dims


def _q(dims):
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    return dfa.lib().dflash_query_sizes(ctypes.byref(dims), ctypes.byref(a), ctypes.byref(b)), a.value, b.value


def test_query_sizes_ok_and_monotone():
    rc, pool, ws = _q(_dims())
    assert rc == 0 and pool > 0 and ws > 0
    rc2, pool2, ws2 = _q(_dims(max_slots=4))
    assert rc2 == 0 and pool2 > pool and ws2 == ws
    rc3, _, ws3 = _q(_dims(max_batch=8))
    assert rc3 == 0 and ws3 > ws


def test_query_sizes_kv_pool_closed_form():
    """The pool holds max_slots * N * 2 * Hkv * ctx_pad * hd elements of K/V."""
    from synth.configs import QWEN3_8B
    dims = dfa.make_dims(QWEN3_8B, max_ctx=8192 + 16, max_slots=32, max_batch=32)
    rc, pool, ws = _q(dims)
    assert rc == 0
    ctx_pad = (8208 + 63) // 64 * 64
    kv = 32 * 5 * 2 * 8 * ctx_pad * 128 * 2
    assert kv <= pool < kv + 64 * 1024 * 1024


@pytest.mark.parametrize("field,value,code", [
    ("hd", 96, -2), ("B", 17, -2), ("B", 1, -2), ("dtype", 7, -2), ("D", 0, -1),
    ("Hkv", 3, -1), ("max_batch", 65, -2), ("D", 100, -2), ("V", 1000, -2), ("N", 17, -2),
])
def test_query_sizes_rejects(field, value, code):
    rc, _, _ = _q(_dims(**{field: value}))
    assert rc == code
    assert dfa.lib().dflash_last_error().decode() != ""


def test_query_sizes_null_outputs():
    dims = _dims()
    assert dfa.lib().dflash_query_sizes(ctypes.byref(dims), None, None) == -1
    assert dfa.lib().dflash_query_sizes(None, None, None) == -1


def test_create_rejects_before_any_gpu_call():
    L = dfa.lib()
    dims = _dims()
    h = ctypes.c_void_p()
    # NULL weights
    assert L.dflash_create(ctypes.byref(dims), None, 256, 1 << 20, 512, 1 << 20, ctypes.byref(h)) == -1
    layers = (dfa.dflash_layer_weights * dims.N)()
    for l in range(dims.N):
        for n in dfa.LAYER_FIELDS:
            setattr(layers[l], n, 4096)
    w = dfa.dflash_weights(4096, 4096, 4096, 4096, 4096, 4096, layers)
    # buffers too small -> ECAPACITY; misaligned -> EINVAL; NULL layer weight -> EINVAL
    assert L.dflash_create(ctypes.byref(dims), ctypes.byref(w), 256, 16, 512, 16, ctypes.byref(h)) == -3
    assert L.dflash_create(ctypes.byref(dims), ctypes.byref(w), 257, 1 << 40, 512, 1 << 40,
                           ctypes.byref(h)) == -1
    layers[1].w_up = None
    assert L.dflash_create(ctypes.byref(dims), ctypes.byref(w), 256, 1 << 40, 512, 1 << 40,
                           ctypes.byref(h)) == -1
    assert "layer 1" in L.dflash_last_error().decode()


def test_accept_argument_checks_without_gpu():
    L = dfa.lib()
    assert L.dflash_accept(None, 0, 16, None, 1, None, None, None) == 0
    assert L.dflash_accept(None, -1, 16, None, 1, None, None, None) == -1
    assert L.dflash_accept(None, 1, 16, 4096, 0, 4096, 4096, 4096) == -1
    assert L.dflash_accept(None, 1, 16, None, 1, 4096, 4096, 4096) == -1


def test_ctx_null_checks():
    L = dfa.lib()
    assert L.dflash_slot_reset(None, 0, 0) == -1
    v = ctypes.c_int32()
    assert L.dflash_slot_len(None, 0, ctypes.byref(v)) == -1
    assert L.dflash_fuse_ctx(None, None, 0, None, None, None) == -1
    assert L.dflash_draft_block(None, None, 0, None, None, 1, None, None, None) == -1
    assert L.dflash_read_cache(None, None, 0, 0, 0, 0, None, None) == -1


def test_strerror():
    L = dfa.lib()
    assert L.dflash_strerror(0) == b"ok"
    assert L.dflash_strerror(-3) == b"capacity exceeded"
    assert L.dflash_strerror(42) == b"unknown status"


def test_relay_rejects_null_ctx_and_arguments():
    L = dfa.lib()
    slots = (ctypes.c_int32 * 1)(0)
    nacc = (ctypes.c_int32 * 1)(3)
    rw = dfa.dflow_relay_weights(None, None)
    assert L.dflow_relay(None, None, 1, slots, nacc, None, 1, None, None, ctypes.byref(rw)) == -1
    n = ctypes.c_int32()
    assert L.dflow_read_relay(None, None, 0, None, ctypes.byref(n)) == -1


def test_spec_draft_static_rejects_bad_sizes_before_any_launch():
    """The allocation-free drafting call validates its sizes on the host (no
    GPU is touched for a rejected call)."""
    L = dfa.lib()
    f = L.dflash_spec_draft_static
    assert f(None, 65, 1024, 16, None, 1.0, 0, None, None, None) == -3       # n_req beyond 64
    assert f(None, 1, 262145, 16, None, 1.0, 0, None, None, None) == -3      # V beyond the scratch
    assert f(None, 1, 1024, 17, None, 1.0, 0, None, None, None) == -2        # B beyond 16
    assert f(None, 1, 1024, 16, None, 0.0, 0, None, None, None) == -1        # temperature
    assert f(None, 0, 1024, 16, None, 1.0, 0, None, None, None) == 0         # nothing to do
    assert f(None, 1, 1024, 16, None, 1.0, 0, None, None, None) == -1        # NULL logits


def test_header_compiles_as_c_and_links(tmp_path):
    """A C99 caller: the header is valid C, the library links by name, and the
    sizes it reports for the Qwen3-8B bs 32 shape equal the ctypes binding's."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "caller.c"
    src.write_text(r'''
#include <stdio.h>
#include "dflash_fuse.h"
int main(void) {
  dflash_dims d;
  size_t kv = 0, ws = 0;
  int rc;
  d.dtype = DFLASH_BF16; d.D = 4096; d.L = 5; d.Dt = 4096; d.N = 5; d.Hq = 32; d.Hkv = 8; d.hd = 128;
  d.I = 12288; d.V = 151936; d.B = 16; d.max_ctx = 8208; d.max_slots = 32; d.max_batch = 32;
  d.rope_base = 10000.0f; d.rms_eps = 1e-6f; d.use_rope = 1;
  rc = dflash_query_sizes(&d, &kv, &ws);
  printf("%d %zu %zu\n", rc, kv, ws);
  d.hd = 96;
  printf("%d %s\n", dflash_query_sizes(&d, &kv, &ws), dflash_strerror(DFLASH_EUNSUPPORTED));
  return rc;
}
''')
    exe = tmp_path / "caller"
    libdir = os.path.dirname(dfa.LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                        "-L", libdir, "-ldflash_fuse", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    first, second = out.stdout.splitlines()[:2]
    rc, kv, ws = (int(x) for x in first.split())
    d = synth.get_config("qwen3_8b_bs32").dims
    kv_py, ws_py = dfa.query_sizes(dfa.make_dims(d, 8208, 32, 32))
    assert rc == 0 and (kv, ws) == (kv_py, ws_py)
    assert second.split()[0] == "-2"
