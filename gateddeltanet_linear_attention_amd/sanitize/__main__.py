import sys

from . import build

print(build(*sys.argv[1:]))
