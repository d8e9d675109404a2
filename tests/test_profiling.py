"""The bench's HBM-traffic figure comes from a committed counter profile and
is dropped (null) as soon as the kernel sources differ from the ones it was
measured on."""
import json

from matrix_aware_optimizer_libmuon_amd import profiling


def _profile(tmp_path, digest, value):
    p = tmp_path / "traffic.md"
    p.write_text("# t\n\n```json\n" + json.dumps(
        {"kernel_sources_sha256_16": digest, "traffic_bytes_per_launch": {"x_update": value}}) + "\n```\n")
    return str(p)


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(profiling, "TRAFFIC_PROFILE", _profile(tmp_path, profiling.kernel_sources_hash(), 123))
    assert profiling.current_traffic("x_update") == 123.0
    assert profiling.current_traffic("gram") is None
    monkeypatch.setattr(profiling, "TRAFFIC_PROFILE", _profile(tmp_path, "0" * 16, 123))
    assert profiling.current_traffic("x_update") is None
    monkeypatch.setattr(profiling, "TRAFFIC_PROFILE", str(tmp_path / "missing.md"))
    assert profiling.current_traffic("x_update") is None


def test_hash_covers_every_kernel_source():
    import os
    csrc = os.path.join(profiling.PKG, "csrc")
    kernels = {f for f in os.listdir(csrc) if f.endswith((".hip", ".h"))}
    assert kernels == set(profiling.KERNEL_SOURCES)
