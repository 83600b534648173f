"""pytest plugin for the sanitizer run: point the ctypes binding at the host-only build
named by SS_SANITIZED_LIB (the C ABI's validation with stub launchers) before any test
loads the library."""
import os

from selective_state_space_85_amd import _lib

_lib.LIB_PATH = os.environ["SS_SANITIZED_LIB"]
_lib._lib = None
