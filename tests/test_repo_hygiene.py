"""Layout rules the repository keeps: committed code never refers to the
builder's scratch folder, and profiles/ holds short text summaries only
(raw profiler output stays out of the tree)."""
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SKIP_DIRS = {".git", "_work", "gpurun_out", "__pycache__", ".pytest_cache", "_build"}
CODE = (".py", ".hip", ".h", ".cpp", ".sh", ".txt", ".toml", ".cfg")


def _files():
    for d, dirs, files in os.walk(ROOT):
        dirs[:] = [x for x in dirs if x not in SKIP_DIRS]
        for f in files:
            yield os.path.join(d, f)


def test_code_does_not_use_the_scratch_folder():
    me = os.path.abspath(__file__)
    for p in _files():
        if p.endswith(CODE) and os.path.abspath(p) != me:
            with open(p, errors="replace") as f:
                assert "_work/" not in f.read(), p


def test_profiles_are_short_text_summaries():
    prof = os.path.join(ROOT, "profiles")
    for f in os.listdir(prof):
        p = os.path.join(prof, f)
        assert f.endswith((".md", ".txt", ".json")), f
        assert os.path.getsize(p) < 64 * 1024, f
