"""GPU test helpers: tensor transfer (from synth.torch_io) and case banners."""
import sys

from synth.torch_io import dev, host_f64  # noqa: F401


def banner(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)
