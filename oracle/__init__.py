"""CPU oracle of the Whisper hot path: test infrastructure only.

Imported only by the tests, the package smoke check and the benchmark's
CPU-baseline leg. It shares no code with the GPU library.
"""
from . import whisper_oracle  # noqa: F401
