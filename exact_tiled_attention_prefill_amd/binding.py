"""placeholder; replaced by the ctypes binding"""
class FaError(RuntimeError):
    pass
def _missing(*a, **k):
    raise FaError("libfa.so not built")
decode = decode_workspace_bytes = library_path = load_library = prefill = _missing
