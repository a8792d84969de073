#!/bin/bash
# Builds libemb.so (gfx950) from the HIP/C++ sources in this directory.
set -euo pipefail
here="$(cd "$(dirname "${BASH_SOURCE[0]}")" && pwd)"
root="$(cd "$here/../.." && pwd)"
out="${1:-$here/../libemb.so}"
tmp="$out.tmp$$"
hipcc --offload-arch=gfx950 -O3 -std=c++17 -fPIC -shared \
    -Xclang -target-feature -Xclang -packed-fp32-ops \
    -Wall -Wno-unused-function \
    -I"$root/include" -I"$here" \
    "$here/plan.cpp" "$here/forward.hip" "$here/backward.hip" "$here/table.hip" "$here/noalloc.hip" "$here/copy.hip" \
    -o "$tmp"
mv -f "$tmp" "$out"
