import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct MI355X (gfx950) device")


def pytest_sessionstart(session):
    """Builds the in-tree libraries only if they are missing (a build is
    otherwise the job of __graft_entry__.build())."""
    import oracle
    from vision_image_preprocessing_amd import build as libbuild

    if not os.path.exists(oracle._LIB_PATH):
        oracle.build()
    if not os.path.exists(libbuild.LIB_PATH):
        try:
            libbuild.build()
        except RuntimeError as e:  # no hipcc: the tests that need it fail loudly
            print("libmimopre.so not built:", e)
