"""The bench's per-workload tables agree with each other and with the
workload specs, and its default run names only known workloads (CPU only)."""
import os

import bench
import workloads


def test_every_workload_has_its_entries():
    for name in bench.RUNNERS:
        assert name in workloads.SPECS, name
        assert name in bench.UNITS and name in bench.DEFAULT_LAYERS, name
        assert name in bench.CALL_KERNELS and name in bench.KERNEL_SOURCES, name
        for f in bench.KERNEL_SOURCES[name]:
            assert os.path.exists(os.path.join(bench.CSRC, f)), (name, f)


def test_default_secondaries_are_known():
    src = open(bench.__file__).read()
    start = src.index('ap.add_argument("--secondary", default=')
    default = src[start:src.index("help=", start)]
    names = [n for n in bench.RUNNERS if n in default]
    assert set(names) >= {"extend_bf16", "long_decode_bf16", "decode_fp8", "sparse_decode_bf16"}
    for piece in default.split('"')[1::2]:
        for n in piece.split(","):
            if n and n != "--secondary":
                assert n in bench.RUNNERS, n
