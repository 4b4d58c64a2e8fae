"""Python binding placeholder (filled in with the C-ABI library)."""


class KvattnError(RuntimeError):
    pass


def _missing(*a, **k):
    raise KvattnError("libkvattn.so binding not built yet")


gqa_decode = mla_decode = gqa_workspace_bytes = mla_workspace_bytes = load_library = library_path = _missing
